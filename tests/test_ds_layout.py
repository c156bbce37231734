"""Index math of the stored-dS backward, checked on the CPU.

The dK/dV kernel stores each 32-query x 32-key dS sub-tile as two 1 KiB
fragments (16-query halves tt'): lane L = key c' + 32 g' writes its packed
dK^T B operand, 8 bf16 whose element e is query 16 tt' + 8 (e // 4) + 4 g' +
e % 4 (register 8 tt' + e of the S accumulator: row 8 (i // 4) + 4 g + i % 4),
at 16-byte slot L ^ 4 (L >= 32) ^ 8 tt'. The dQ kernel reads it back with
ds_read_b64_tr_b16, which gives lane i of each 16-lane group element i % 4 of
the 8 bytes addressed by lanes 4 j + i // 4, as its element j. These tests
replay both sides in numpy and check that every lane of every dQ^T B operand
receives dS[query][key] for its own query (16 dh + lane % 16) and the keys the
K^T A operand holds in the same k slots (16 tt + 4 g + j, then + 8), and that
the reads are free of bank conflicts: LDS has 64 banks of 4 bytes, and a
64-bit read is serviced 32 lanes at a time, so the 32 addresses of each half
of the wavefront must fall in distinct 8-byte slots of one 256-byte line (the
K^T reads of the same kernels are laid out that way, and measure no
conflicts). No GPU is used.
"""
import numpy as np


def _store_subtile(ds):
    """Bytes of one stored sub-tile (as uint16 words) from dS[query][key]."""
    words = np.full(1024, -1, dtype=np.int64)     # 2 KiB = 1024 bf16 words
    for tt in range(2):
        for lane in range(64):
            key, g = lane % 32, lane // 32
            slot = lane ^ (4 if lane >= 32 else 0) ^ (8 * tt)
            for e in range(8):
                q = 16 * tt + 8 * (e // 4) + 4 * g + e % 4
                words[(tt * 1024 + slot * 16 + 2 * e) // 2] = ds[q, key]
    return words


def _tr_read(words, addr):
    """ds_read_b64_tr_b16 over 64 lanes: addr[l] = byte address read by lane l."""
    out = np.zeros((64, 4), dtype=np.int64)
    for grp in range(4):
        for i in range(16):
            for j in range(4):
                src = 16 * grp + 4 * j + i // 4
                out[16 * grp + i, j] = words[(addr[src] + 2 * (i % 4)) // 2]
    return out


def _read_addresses(tt, hh):
    """Byte addresses the dQ kernel's lanes give the transposing read of
    16-key half tt, key group hh (0: slots 0..3, 1: slots 4..7): bt, or
    bt ^ 128 for hh = 1, plus 256 tt."""
    addr = []
    for lane in range(64):
        s16, dh, g = lane & 15, (lane >> 4) & 1, lane >> 5
        sl = s16 & 1
        b_t = dh * 1024 + (32 * sl + ((4 * g + (s16 >> 2)) ^ (4 * sl)) + 8 * dh) * 16 + \
            ((s16 >> 1) & 1) * 8
        addr.append((b_t ^ (128 * hh)) + 256 * tt)
    return addr


def _ways(addr):
    """Most distinct 8-byte words one bank pair serves in one 32-lane pass."""
    worst = 0
    for half in (addr[:32], addr[32:]):
        per = {}
        for a in half:
            per.setdefault((a % 256) // 8, set()).add(a // 8)
        worst = max(worst, max(len(v) for v in per.values()))
    return worst


def test_every_stored_element_lands_once():
    ds = np.arange(32 * 32).reshape(32, 32)
    words = _store_subtile(ds)
    assert (words >= 0).all()
    assert sorted(words.tolist()) == list(range(1024))


def test_transposing_reads_give_the_dq_b_operand():
    rng = np.random.default_rng(5)
    ds = rng.permutation(32 * 32).reshape(32, 32)     # distinct values: any mix-up shows
    words = _store_subtile(ds)
    for tt in range(2):
        frag = np.concatenate([_tr_read(words, _read_addresses(tt, hh)) for hh in range(2)], axis=1)
        for lane in range(64):
            q, g = lane % 32, lane // 32
            keys = [16 * tt + 4 * g + j for j in range(4)] + [16 * tt + 8 + 4 * g + j for j in range(4)]
            assert frag[lane].tolist() == [ds[q, k] for k in keys], (tt, lane)


def test_k_operand_uses_the_same_k_order():
    """The K^T operand's k slots (transposing read of the row-major K tile:
    lane s16 of group (g, dh) reads key row 4 g + s16 // 4, then + 8) hold
    keys 16 tt + 4 g + j and 16 tt + 8 + 4 g + j, the order the dS^T operand
    was checked against above."""
    for tt in range(2):
        for lane in range(64):
            g, i = lane // 32, lane & 15
            slots = []
            for hh in range(2):
                for j in range(4):
                    src = 4 * j + i // 4               # lane whose row lane i takes as element j
                    slots.append(16 * tt + 4 * g + (src >> 2) + 8 * hh)
            assert slots == [16 * tt + 4 * g + j for j in range(4)] + \
                            [16 * tt + 8 + 4 * g + j for j in range(4)]


def test_reads_are_bank_conflict_free():
    for tt in range(2):
        for hh in range(2):
            addr = _read_addresses(tt, hh)
            assert all(x % 8 == 0 for x in addr)
            for grp in range(4):
                a = addr[16 * grp:16 * grp + 16]
                assert len({(x % 128) // 8 for x in a}) == 16, (tt, hh, grp)
            for half in (addr[:32], addr[32:]):
                assert len({(x % 256) // 8 for x in half}) == 32, (tt, hh)
            assert _ways(addr) == 1


def test_without_the_half_swap_the_32_lane_passes_conflict():
    """The ^ 8 of the second 16-row half is what puts the dh = 0 and dh = 1
    groups of one 32-lane pass on different 128-byte halves of the bank
    line: read at the unswapped addresses every bank pair serves two words."""
    for tt in range(2):
        for hh in range(2):
            addr = []
            for lane in range(64):
                s16, dh, g = lane & 15, (lane >> 4) & 1, lane >> 5
                sl = s16 & 1
                b_t = dh * 1024 + (32 * sl + ((4 * g + (s16 >> 2)) ^ (4 * sl))) * 16 + \
                    ((s16 >> 1) & 1) * 8
                addr.append(b_t + 128 * hh + 256 * tt)
            assert _ways(addr) == 2


def test_without_the_lane_swap_the_reads_conflict():
    """The L ^ 4 store swap is what separates the two query-group halves by
    64 bytes: without it each 16-lane read hits only 8 distinct slots."""
    for tt in range(2):
        addr = []
        for lane in range(16):
            s16, sl = lane, lane & 1
            addr.append((32 * sl + (s16 >> 2)) * 16 + ((s16 >> 1) & 1) * 8 + 16 * tt * 16)
        assert len({(x % 128) // 8 for x in addr}) == 8
