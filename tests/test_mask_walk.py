"""The dK/dV kernel's walk over a block mask, modelled on the CPU.

A masked dK/dV workgroup (keys n0 .. n0 + BN - 1, query blocks of BM rows,
mask rows of 128 queries, so 128 / BM query blocks per mask row) lists the
(query head, mask row) pairs whose mask byte is set in one of its 128-key
columns, from the row of its first causal query block m_first on, head-major;
its step count is 128 / BM per listed pair, less the query blocks of the
first row before m_first and those of the last row past the sequence, and
its cursors step through the query blocks of each listed row. With more
pairs than the list holds it walks every (head, query block) step. These
tests replay that arithmetic (the kernel's own constants and formulas) and
check it against a brute-force enumeration of the steps with a visible
block, for random lengths, masks, tilings and causal offsets. No GPU is used.
"""
import random


def cdiv(a, b):
    return -(-a // b)


def walk(lq, lk, bm, bn, gs, causal, mask, n0, cap):
    """Steps (head, query block) the kernel's cursors visit for key block n0."""
    rpb = 128 // bm
    nm = cdiv(lq, bm)
    shift = lk - lq
    m_first = min(max(0, n0 - shift) // bm, nm) if causal else 0
    ncols = 2 if bn > 128 and n0 + 128 < lk else 1
    c0 = n0 // 128

    def vis(h, r):
        return any(mask[h][r][c0 + c] for c in range(ncols))

    n_steps = gs * (nm - m_first)
    if n_steps == 0:
        return [], None
    r0, nmr = m_first // rpb, cdiv(nm, rpb)
    nrows = nmr - r0
    dense = gs * nrows > cap
    if dense:
        rows, n_ent, h, m = None, gs, 0, m_first
    else:
        rows, nf, nl = [], 0, 0
        for e in range(gs * nrows):
            hh, rr = divmod(e, nrows)
            if vis(hh, r0 + rr):
                rows.append(hh << 16 | rr)
                nf += rr == 0
                nl += r0 + rr == nmr - 1
        n_ent = len(rows)
        n_steps = rpb * n_ent - nf * (m_first - r0 * rpb) - nl * (nmr * rpb - nm)
        if n_steps == 0:
            return [], rows
        h, m = rows[0] >> 16, max((r0 + (rows[0] & 0xFFFF)) * rpb, m_first)
    out, e = [], 0
    for _ in range(n_steps):
        out.append((h, m))
        m += 1
        if m == nm or (not dense and m % rpb == 0):
            e += 1
            if e < n_ent:
                if dense:
                    h, m = e, m_first
                else:
                    v = rows[e]
                    h, m = v >> 16, max((r0 + (v & 0xFFFF)) * rpb, m_first)
    return out, rows


def brute(lq, lk, bm, bn, gs, causal, mask, n0):
    nm = cdiv(lq, bm)
    shift = lk - lq
    m_first = min(max(0, n0 - shift) // bm, nm) if causal else 0
    ncols = 2 if bn > 128 and n0 + 128 < lk else 1
    c0 = n0 // 128
    return [(h, m) for h in range(gs) for m in range(m_first, nm)
            if any(mask[h][m * bm // 128][c0 + c] for c in range(ncols))]


def test_listed_walk_visits_exactly_the_visible_steps():
    rng = random.Random(71)
    for _ in range(1500):
        bm, bn = rng.choice([32, 64]), rng.choice([128, 256])
        lq, lk, gs = rng.randint(1, 1500), rng.randint(1, 1500), rng.randint(1, 4)
        causal, density = rng.random() < 0.6, rng.random()
        mask = [[[rng.random() < density for _ in range(cdiv(lk, 128))]
                 for _ in range(cdiv(lq, 128))] for _ in range(gs)]
        for n0 in range(0, lk, bn):
            got, rows = walk(lq, lk, bm, bn, gs, causal, mask, n0, cap=2048)
            assert got == brute(lq, lk, bm, bn, gs, causal, mask, n0), (lq, lk, bm, bn, n0)
            assert rows is None or all((v >> 16) < gs and (v & 0xFFFF) < 2048 for v in rows)


def test_dense_walk_covers_every_step_in_order():
    rng = random.Random(72)
    for _ in range(300):
        bm, bn = rng.choice([32, 64]), rng.choice([128, 256])
        lq, lk, gs = rng.randint(1, 1500), rng.randint(1, 600), rng.randint(1, 4)
        causal = rng.random() < 0.5
        mask = [[[rng.random() < 0.5 for _ in range(cdiv(lk, 128))]
                 for _ in range(cdiv(lq, 128))] for _ in range(gs)]
        for n0 in range(0, lk, bn):
            got, _ = walk(lq, lk, bm, bn, gs, causal, mask, n0, cap=0)
            nm = cdiv(lq, bm)
            m_first = min(max(0, n0 - (lk - lq)) // bm, nm) if causal else 0
            assert got == [(h, m) for h in range(gs) for m in range(m_first, nm)]
            assert set(brute(lq, lk, bm, bn, gs, causal, mask, n0)) <= set(got)


def test_a_planted_step_count_error_is_caught():
    """Dropping the last row's correction from the step count (a plausible
    slip) makes the walk disagree with the brute force on a ragged length."""
    lq, lk, bm, bn, gs = 650, 700, 32, 256, 1
    mask = [[[True] * cdiv(lk, 128) for _ in range(cdiv(lq, 128))]]
    n0 = 0
    want = brute(lq, lk, bm, bn, gs, True, mask, n0)
    nm, rpb = cdiv(lq, bm), 128 // bm
    wrong = rpb * cdiv(nm, rpb)    # no correction for the partial last row
    assert wrong != len(want)
    assert len(walk(lq, lk, bm, bn, gs, True, mask, n0, cap=2048)[0]) == len(want)
