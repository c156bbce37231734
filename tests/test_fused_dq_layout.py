"""Index math of the fused design's dQ product in the 256-key dK/dV kernel,
checked on the CPU.

Each wave writes the bf16 dS fragments it packs for dK^T (lane L = key
c + 32 g of its 32-key sub-column holds queries 16 tt + 4 g + 0..3 and
16 tt + 8 + 4 g + 0..3) into an LDS image: per 32-query block qb, 8 sub-tiles
of 32 keys (2 KiB, halves tt of 1 KiB), lane slot L ^ 4 (L >= 32) ^ 8 tt. The K
tile sits row-major in LDS with the row swizzle dma_swz (16-byte slot pos of
row r holds logical chunk pos ^ dma_swz(r)). Wave w then forms the 32 x 32
dQ unit (query block w // (d / 32), dim block w % (d / 32)) as sixteen
32x32x16 MFMAs: A = dS (query on the lane) and B = K (dim on the lane), both
from ds_read_b64_tr_b16 at the lane addresses the kernel computes. The test
replays the writes and the reads in numpy, with the MFMA's operand layout
(lane l: A[l % 32][8 (l // 32) + e], B[8 (l // 32) + e][l % 32]), and checks
every unit equals dS K; it also checks that every LDS access stays inside
its region and that the dS reads are free of bank conflicts (64 banks of 4
bytes, a 64-bit read serviced 32 lanes at a time). No GPU is used.
"""
import numpy as np
import pytest


def _dma_swz(d, r):
    if d >= 128:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    t = (r >> 1) & 7
    return ((t & 1) << 2) | (t >> 1)


def _tr_read(lds, addr, lo, hi):
    """ds_read_b64_tr_b16: lane i of each 16-lane group gets element i % 4 of
    the 8 bytes read by lanes 4 j + i // 4, as its element j."""
    out = np.zeros((64, 4))
    for grp in range(4):
        for i in range(16):
            for j in range(4):
                a = addr[16 * grp + 4 * j + i // 4]
                assert a % 8 == 0 and lo <= a and a + 8 <= hi, a
                out[16 * grp + i, j] = lds[a // 2 + i % 4]
    return out


@pytest.mark.parametrize("d,bm", [(128, 32), (64, 64)])
def test_fused_dq_units_equal_ds_times_k(d, bm):
    rng = np.random.default_rng(d)
    bn, kb_per_wave, nw = 256, 2, 4
    nqb, ndb, nkc, rb = bm // 32, d // 32, bn // 32, 2 * d
    kt, dsb = bn * rb, bm * bn * 2
    assert nqb * ndb == nw
    k = rng.standard_normal((bn, d))
    ds = rng.standard_normal((bm, bn))
    lds = np.full((kt + 2 * dsb) // 2, np.nan)
    lds_k, lds_s, par = 0, kt, dsb          # the odd step's image
    spr = d // 8
    for i in range(kt // (16 * 256)):       # K tile by 16-byte direct loads
        for w in range(nw):
            for lane in range(64):
                slot = (i * nw + w) * 64 + lane
                r, pos = slot // spr, slot % spr
                ch = pos ^ _dma_swz(d, r)
                dst = lds_k + slot * 16
                lds[dst // 2: dst // 2 + 8] = k[r, 8 * ch: 8 * ch + 8]
    for w in range(nw):                     # dS image from each wave's fragments
        for qb in range(nqb):
            for kb in range(kb_per_wave):
                for tt in range(2):
                    for ln in range(64):
                        key, g = 32 * (w * kb_per_wave + kb) + ln % 32, ln // 32
                        rows = [16 * tt + 4 * g + r for r in range(4)] + \
                               [16 * tt + 8 + 4 * g + r for r in range(4)]
                        dsw = lds_s + par + w * kb_per_wave * 2048 + ((ln ^ ((ln >> 5) << 2)) << 4)
                        a = (dsw ^ (128 * tt)) + qb * nkc * 2048 + kb * 2048 + tt * 1024
                        assert lds_s + par <= a and a + 16 <= lds_s + par + dsb
                        lds[a // 2: a // 2 + 8] = [ds[32 * qb + q, key] for q in rows]
    assert not np.isnan(lds[:kt // 2]).any()
    assert not np.isnan(lds[(lds_s + par) // 2:(lds_s + par + dsb) // 2]).any()
    dq = ds @ k
    for w in range(nw):
        qb_w, db_w = w // ndb, w % ndb
        ra, k0, k1 = [], [], []
        for ln in range(64):
            l16, lh, lg = ln & 15, (ln >> 4) & 1, ln >> 5
            sl = l16 & 1
            ra.append(lds_s + par + qb_w * nkc * 2048 + lh * 1024
                      + (32 * sl + ((4 * lg + (l16 >> 2)) ^ (4 * sl)) + 8 * lh) * 16
                      + ((l16 >> 1) & 1) * 8)
            lr, lc = 4 * lg + (l16 >> 2), 2 * lh + ((l16 & 3) >> 1)
            lt = lr * rb + 16 * (lc ^ _dma_swz(d, lr)) + 8 * (l16 & 1)
            k0.append(lds_k + (lt ^ (64 * db_w)))
            k1.append(lds_k + (lt ^ (64 * db_w + 32)) + 8 * rb)
        acc = np.zeros((32, 32))
        for jq in range(bn // 16):
            kc, tt = jq >> 1, jq & 1
            so, ko = kc * 2048 + 256 * tt, (kc * 32 + 16 * tt) * rb
            img = (lds_s + par, lds_s + par + dsb)
            a0, a1 = [x + so for x in ra], [(x ^ 128) + so for x in ra]
            for addr in (a0, a1):   # one 256-byte bank line per 32-lane pass
                for half in (addr[:32], addr[32:]):
                    assert len({(x % 256) // 8 for x in half}) == 32
            a_op = np.concatenate([_tr_read(lds, a0, *img), _tr_read(lds, a1, *img)], 1)
            b_op = np.concatenate([_tr_read(lds, [x + ko for x in k0], lds_k, lds_k + kt),
                                   _tr_read(lds, [x + ko for x in k1], lds_k, lds_k + kt)], 1)
            am, bmat = np.zeros((32, 16)), np.zeros((16, 32))
            for l in range(64):
                am[l % 32, 8 * (l // 32): 8 * (l // 32) + 8] = a_op[l]
                bmat[8 * (l // 32): 8 * (l // 32) + 8, l % 32] = b_op[l]
            acc += am @ bmat
        want = dq[32 * qb_w: 32 * qb_w + 32, 32 * db_w: 32 * db_w + 32]
        np.testing.assert_allclose(acc, want, rtol=0, atol=1e-10)


def test_fused_dq_lds_fits():
    """K tile + two dS images after the Q / dO ring (rounded to 1 KiB) fit the
    160 KiB of LDS a workgroup may use."""
    for d, bm in ((128, 32), (64, 64)):
        ring = 2 * 3 * bm * 2 * d + 3 * 2 * bm * 4
        total = (ring + 1023) // 1024 * 1024 + 256 * 2 * d + 2 * bm * 256 * 2
        assert total <= 160 * 1024, (d, total)
