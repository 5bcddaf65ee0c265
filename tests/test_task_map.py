"""CPU model of the prefill GEMM's block -> task map (host logic, no GPU).

The prefill kernels derive their task (expert, n-tile, m-tile) from the block
index and the expert segment sizes, with no host synchronisation. Block b
runs on XCD b % 8 in slot b // 8 (the hardware deals workgroups round-robin
to the 8 XCDs); XCD x then takes an equal contiguous share of the tasks that
exist, in one of three orders:
  lpt 0  expert-major: expert, then n-tile, then m-tile (weight-tile reuse);
  lpt 1  longest first, two classes: every full m-tile, then every partial one;
  lpt 2  longest first, four classes by filled 32-row sub-tiles (4, 3, 2, 1).
This model restates that arithmetic (gemm.hip: find_task_lpt, find_task_lpt4)
per block and checks, over random segment-size vectors, that every task runs
exactly once, that spare blocks find nothing, and that no XCD takes more than
one task of a class above another.
"""
import numpy as np
import pytest

BM = 128  # token rows per prefill block


def tasks_expected(cnt, NB):
    out = set()
    for e, c in enumerate(cnt):
        for nt in range(NB):
            for mi in range((c + BM - 1) // BM):
                out.add((e, mi * BM, min(BM, c - mi * BM), nt))
    return out


def offsets_of(cnt):
    return np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)


def lookup_lpt(cnt, NB, b, lpt):
    """find_task_lpt for block b: the (e, row0 - offsets[e], rows, n-tile)
    task, or None."""
    nfu = [(c // BM) * NB for c in cnt]
    npa = [NB if c % BM else 0 for c in cnt]
    F, P = sum(nfu), sum(npa)
    x, slot = b & 7, b >> 3
    if lpt == 0:
        TOT = F + P
        q8, r8 = TOT >> 3, TOT & 7
        n8 = q8 + (1 if x < r8 else 0)
        if slot >= n8:
            return None
        L = x * q8 + min(x, r8) + slot
        st = 0
        for e, c in enumerate(cnt):
            n = nfu[e] + npa[e]
            if st <= L < st + n:
                rel = L - st
                mt = (c + BM - 1) // BM
                mi = rel % mt
                return (e, mi * BM, min(BM, c - mi * BM), rel // mt)
            st += n
        return None
    qf, rf, qp, rp = F >> 3, F & 7, P >> 3, P & 7
    nf = qf + (1 if x < rf else 0)
    bf = x * qf + min(x, rf)
    np_ = qp + (1 if x >= 8 - rp else 0)
    bp = x * qp + max(0, x - (8 - rp))
    full = slot < nf
    if not (full or slot - nf < np_):
        return None
    L = bf + slot if full else bp + (slot - nf)
    sf = sp = 0
    for e, c in enumerate(cnt):
        st, n = (sf, nfu[e]) if full else (sp, npa[e])
        if st <= L < st + n:
            rel = L - st
            mf = c // BM
            mi = rel % mf if full else mf
            return (e, mi * BM, min(BM, c - mi * BM), rel // mf if full else rel)
        sf += nfu[e]
        sp += npa[e]
    return None


def lookup_lpt4(cnt, NB, b):
    """find_task_lpt4 for block b."""
    NC, SUB = 4, BM // 4
    ncl, cls = [], []
    for c in cnt:
        rem = c % BM
        k_ = NC - (rem + SUB - 1) // SUB if rem else 0
        v = [0] * NC
        v[0] = (c // BM) * NB
        if rem:
            v[k_] += NB
        ncl.append(v)
        cls.append(k_)
    tot = [sum(v[k] for v in ncl) for k in range(NC)]
    x, slot = b & 7, b >> 3
    rot = before = 0
    k_sel, L = -1, 0
    for k in range(NC):
        q, r = tot[k] >> 3, tot[k] & 7
        d = (x - rot + 8) & 7
        n = q + (1 if d < r else 0)
        ex = sum(1 for y in range(x) if ((y - rot + 8) & 7) < r)
        if k_sel < 0 and slot - before < n:
            k_sel, L = k, x * q + ex + (slot - before)
        before += n
        rot = (rot + r) & 7
    if k_sel < 0:
        return None
    st = 0
    for e, c in enumerate(cnt):
        n = ncl[e][k_sel]
        if st <= L < st + n:
            rel = L - st
            mf = c // BM
            if k_sel == 0:
                mt = mf + (1 if (c % BM) and cls[e] == 0 else 0)
                mi, nt = rel % mt, rel // mt
            else:
                mi, nt = mf, rel
            return (e, mi * BM, min(BM, c - mi * BM), nt)
        st += n
    return None


def grid_blocks(cnt, NB):
    """The launch's grid: an upper bound of the task count (the host cannot
    see the segment sizes) plus 16 spare blocks."""
    R, E = int(sum(cnt)), len(cnt)
    return ((R + BM - 1) // BM + min(R, E)) * NB + 16


def random_counts(rng, E, R):
    kind = rng.integers(0, 4)
    if kind == 0:   # uniform
        p = np.full(E, 1.0 / E)
    elif kind == 1:  # Zipf-skewed
        p = 1.0 / np.arange(1, E + 1) ** rng.uniform(0.3, 1.5)
        p = rng.permutation(p / p.sum())
    elif kind == 2:  # a few experts only
        p = np.zeros(E)
        p[rng.choice(E, size=max(1, E // 8), replace=False)] = 1.0
        p /= p.sum()
    else:            # multiples of BM and near-multiples
        return list(rng.choice([0, BM - 1, BM, BM + 1, 2 * BM, 3 * BM - 33, 97], size=E))
    return list(rng.multinomial(R, p))


CASES = [(8, 4096, 28), (8, 16384, 16), (64, 16384, 32), (256, 24576, 16), (256, 32768, 4),
         (8, 300, 7), (1, 5000, 3), (256, 100, 16)]


@pytest.mark.parametrize("E,R,NB", CASES)
@pytest.mark.parametrize("order", ["lpt0", "lpt1", "lpt4"])
def test_every_task_once(E, R, NB, order):
    rng = np.random.default_rng(E * 131 + R + NB)
    for _ in range(6 if E * R > 100000 else 20):
        cnt = [int(c) for c in random_counts(rng, E, R)]
        want = tasks_expected(cnt, NB)
        got, per_xcd = [], [[] for _ in range(8)]
        for b in range(grid_blocks(cnt, NB)):
            t = lookup_lpt4(cnt, NB, b) if order == "lpt4" else \
                lookup_lpt(cnt, NB, b, 0 if order == "lpt0" else 1)
            if t is not None:
                got.append(t)
                per_xcd[b & 7].append(t)
        assert len(got) == len(set(got)), "a task ran twice"
        assert set(got) == want, "a task was dropped"
        # shares: within a class no XCD runs more than one task above another
        if order == "lpt0":
            sizes = [len(v) for v in per_xcd]
            assert max(sizes) - min(sizes) <= 1
        else:
            ncls = 4 if order == "lpt4" else 2

            def klass(t):
                rows = t[2]
                if order == "lpt1":
                    return 0 if rows == BM else 1
                return 0 if rows > 3 * BM // 4 else 4 - (rows + BM // 4 - 1) // (BM // 4)
            for k in range(ncls):
                sizes = [sum(1 for t in v if klass(t) == k) for v in per_xcd]
                assert max(sizes) - min(sizes) <= 1, (k, sizes)


def test_longest_first_orders_slots():
    """lpt 1: on every XCD the full m-tiles occupy the earlier slots."""
    cnt = [700, 129, 1000, 64, 511, 256, 0, 3]
    NB = 8
    for x in range(8):
        rows = [lookup_lpt(cnt, NB, b, 1) for b in range(x, grid_blocks(cnt, NB), 8)]
        rows = [t[2] for t in rows if t is not None]
        full = [r == BM for r in rows]
        assert full == sorted(full, reverse=True)
