"""Pins of the oracle's cumulative mixture (C6c): per-update window counts
from the cycle's cumulative quotas.

NeuronSpark-Trainer README, Concepts: every update holds each source within
two samples of its recipe share, and every source's data are trained
(max_epochs 1).  The reading: after u updates source s has taken A_s(u)
windows, floor(u·B·w_s/W) ≤ A_s(u) ≤ ceil(u·B·w_s/W), never fewer than after
u−1 updates.  These tests pin the schedule by those requirements (checked in
exact integers), by exhaustive enumeration of every valid schedule on tiny
cases, and by closed forms (one source; shares that are whole windows, where
the schedule must equal the fixed apportionment)."""
import itertools

import numpy as np
import pytest

import oracle
from synth.corpus import random_small

pytestmark = pytest.mark.filterwarnings("ignore")


def _valid(A, B, w):
    """Quota at every boundary, monotone, B windows per update."""
    W = int(sum(int(x) for x in w))
    U = A.shape[0] - 1
    for u in range(U + 1):
        assert int(A[u].sum()) == u * B
        for s, ws in enumerate(w):
            q = u * B * int(ws)
            assert q // W <= int(A[u, s]) <= -(-q // W), (u, s, A[u].tolist())
    c = np.diff(A.astype(np.int64), axis=0)
    assert (c >= 0).all()
    for s, ws in enumerate(w):   # within two windows of the share, every update
        assert all(abs(int(x) * W - B * int(ws)) < 2 * W for x in c[:, s])


@pytest.mark.parametrize("seed", range(40))
def test_quota_monotone_random(seed):
    r = np.random.default_rng(seed)
    S = int(r.integers(1, 9))
    w = [int(r.choice([0, 1, 2, 3, 7, 100, int(r.integers(1, 10**9))])) for _ in range(S)]
    if sum(w) == 0:
        w[0] = 1
    B = int(r.choice([1, 2, 3, 5, 8, 64, 256]))
    U = int(r.integers(1, 120))
    got_U, A = oracle.cumulative(B, w, [10**9] * S, updates=U)
    assert got_U == U and A.shape == (U + 1, S)
    _valid(A, B, w)


def test_huge_weights_exact():
    """Weights near 2^64 in total: the quotas need 128-bit products."""
    w = [2**63 - 25, 2**62 + 7, 3, 2**61 + 1]
    _, A = oracle.cumulative(1024, w, [10**9] * 4, updates=50)
    _valid(A, 1024, w)


def _enumerate(B, w, U):
    """Every schedule of U updates that satisfies the requirements."""
    S = len(w)
    comps = [c for c in itertools.product(range(B + 1), repeat=S) if sum(c) == B]
    out = []
    W = sum(w)

    def rec(u, A, acc):
        if u == U:
            out.append(np.array(acc, np.uint32))
            return
        for c in comps:
            nxt = [A[s] + c[s] for s in range(S)]
            h = (u + 1) * B
            if all(h * w[s] // W <= nxt[s] <= -(-h * w[s] // W) for s in range(S)):
                rec(u + 1, nxt, acc + [nxt])

    rec(0, [0] * S, [[0] * S])
    return out


@pytest.mark.parametrize("B,w,U", [(1, [1, 1, 1], 5), (2, [1, 2, 4], 5), (3, [5, 1, 1], 5), (1, [3, 2], 6),
                                   (2, [1, 1, 1, 1], 4), (3, [2, 7, 11], 4), (1, [1, 9], 7)])
def test_valid_among_all_schedules(B, w, U):
    """Brute force: the oracle's schedule is one of the valid ones (which exist,
    as the quota method of Balinski and Young shows), and where the valid
    schedule is unique it is that one."""
    _, A = oracle.cumulative(B, w, [10**6] * len(w), updates=U)
    allv = _enumerate(B, w, U)
    assert allv, "no valid schedule"
    assert any(np.array_equal(A, v) for v in allv)
    if len(allv) == 1:
        assert np.array_equal(A, allv[0])


def test_one_source():
    _, A = oracle.cumulative(7, [5], [10**6], updates=9)
    assert A[:, 0].tolist() == [7 * u for u in range(10)]


@pytest.mark.parametrize("B,w", [(8, [1, 1, 2, 4]), (256, [3, 1]), (12, [1, 2, 3]), (4, [1, 1, 1, 1])])
def test_whole_window_shares(B, w):
    """B·w_s/W whole for every source: each update takes exactly that many."""
    _, A = oracle.cumulative(B, w, [10**6] * len(w), updates=20)
    c = np.diff(A.astype(np.int64), axis=0)
    W = sum(w)
    for s in range(len(w)):
        assert (c[:, s] == B * w[s] // W).all()


def test_small_share_gets_windows():
    """A share below one window per update: the fixed apportionment gives the
    source none; the cumulative quotas give it its windows over the cycle, each
    by the update at which its lower quota reaches it."""
    B, w = 4, [1, 99]
    assert oracle.apportion(B, w).tolist() == [0, 4]
    _, A = oracle.cumulative(B, w, [10**6, 10**6], updates=100)
    assert int(A[100, 0]) == 4                      # 100·4·1/100 windows: exact at the end
    for u in range(101):
        assert int(A[u, 0]) >= u * B // 100         # lower quota: the window comes in time
        assert int(A[u, 0]) <= -(-u * B // 100)


def test_updates_zero_takes_the_most_that_fit():
    B, w, rem = 8, [3, 5, 1], [40, 70, 9]
    U, A = oracle.cumulative(B, w, rem)
    assert U > 0
    assert all(int(A[U, s]) <= rem[s] for s in range(3))
    # one more update does not fit
    U2, A2 = oracle.cumulative(B, w, rem, updates=U + 1)
    assert U2 == U
    assert np.array_equal(A2[:U + 1], A)


def _corpus(seed, **kw):
    c = random_small(seed, n_docs=kw.pop("n_docs", 400), n_sources=kw.pop("S", 3), max_strata=2, T=64,
                     B=kw.pop("B", 5), max_len=150, bp_max=1500)
    return c.replace(cumulative=True, **kw)


@pytest.mark.parametrize("seed", range(6))
def test_cycle_uses_each_window_once(seed):
    c = _corpus(seed, S=1 + seed % 4, B=[1, 3, 5, 8, 2, 7][seed])
    op = oracle.Plan(c)
    ci = op.cycle(0)
    A = op.cumulative_taken()
    _valid(A, c.B, c.weight)
    assert ci.taken.tolist() == A[-1].astype(np.uint64).tolist()
    seen = {}
    for b in range(ci.n_updates):
        for j in range(c.B):
            g = op.window_of(b, j)
            seen[g] = seen.get(g, 0) + 1
    assert all(v == 1 for v in seen.values())
    expect = set()
    for s in range(c.n_sources):
        lo = int(op.src_win_start[s] + ci.start[s])
        expect.update(range(lo, lo + int(ci.taken[s])))
    assert set(seen) == expect
    # each update's slots hold that update's counts
    for b in range(ci.n_updates):
        srcs = [next(s for s in range(c.n_sources) if op.src_win_start[s] <= op.window_of(b, j) <
                     op.src_win_start[s + 1]) for j in range(c.B)]
        assert np.bincount(srcs, minlength=c.n_sources).tolist() == (A[b + 1] - A[b]).astype(int).tolist()


def test_cycles_chain_and_exhaust():
    c = _corpus(3, S=3, B=4).replace(updates_per_cycle=5)
    op = oracle.Plan(c)
    nxt = np.zeros(3, np.uint64)
    k = 0
    while True:
        try:
            ci = op.cycle(k)
        except oracle.OracleError as e:
            assert e.code == oracle.OR_E_EXHAUSTED
            break
        assert ci.start.tolist() == nxt.tolist()
        nxt = ci.start + ci.taken
        assert (ci.remaining == op.windows_per_source - nxt).all()
        k += 1
    assert k >= 2


def test_whole_shares_equal_fixed_plan():
    """With shares that are whole windows the cumulative plan emits the same
    batches as the fixed apportionment (the digest differs by the mode)."""
    c = _corpus(1, S=2, B=6).replace(weight=np.array([2, 1], np.uint64), updates_per_cycle=3)
    a = oracle.Plan(c)
    b = oracle.Plan(c.replace(cumulative=False))
    ia, ib = a.cycle(0), b.cycle(0)
    assert ia.n_updates == ib.n_updates == 3
    ba, bb = a.batch(0, 3), b.batch(0, 3)
    for k in ("tokens", "pos", "doc", "mask", "learned", "digests"):
        assert np.array_equal(ba[k], bb[k]), k
    assert ia.plan_digest != ib.plan_digest


def test_tiny_share_source_trained():
    """The fixed apportionment never trains a source below half a window per
    update; the cumulative one takes its windows."""
    c = _corpus(4, S=2, B=4).replace(weight=np.array([1, 60], np.uint64))
    fixed = oracle.Plan(c.replace(cumulative=False))
    cum = oracle.Plan(c)
    fi, ci = fixed.cycle(0), cum.cycle(0)
    assert int(fi.taken[0]) == 0
    assert int(ci.taken[0]) > 0
    W = 61
    assert int(ci.taken[0]) in (ci.n_updates * 4 * 1 // W, -(-ci.n_updates * 4 // W))


def test_read_random_with_cumulative():
    """The random read order permutes each source's cycle windows; counts stay."""
    c = _corpus(5, S=3, B=5)
    a = oracle.Plan(c)
    b = oracle.Plan(c.replace(read_random=True))
    ia, ib = a.cycle(0), b.cycle(0)
    assert ia.n_updates == ib.n_updates and ia.taken.tolist() == ib.taken.tolist()
    wa = sorted(a.window_of(u, j) for u in range(ia.n_updates) for j in range(c.B))
    wb = sorted(b.window_of(u, j) for u in range(ib.n_updates) for j in range(c.B))
    assert wa == wb
    assert ia.plan_digest != ib.plan_digest


@pytest.mark.parametrize("seed", range(6))
def test_schedule_prefix_does_not_depend_on_length(seed):
    """A window's due update is read from the continuing batches, not from the
    cycle's length: a shorter schedule is a prefix of a longer one."""
    r = np.random.default_rng(100 + seed)
    S = int(r.integers(2, 7))
    w = [int(x) for x in r.choice([1, 2, 3, 50, 1000], size=S)]
    B = int(r.choice([1, 3, 8, 64]))
    U2 = int(r.integers(20, 90))
    _, A2 = oracle.cumulative(B, w, [10**9] * S, updates=U2)
    for U1 in (1, 2, 5, U2 // 2):
        _, A1 = oracle.cumulative(B, w, [10**9] * S, updates=U1)
        assert np.array_equal(A1, A2[:U1 + 1]), U1


@pytest.mark.parametrize("ramp", [None, ((0, 128), (700, 320), (2000, 64))])
def test_cycle_schedule_prefix_with_updates_per_cycle(ramp):
    """updates_per_cycle cuts the same schedule shorter (ramped or not)."""
    base = _corpus(8, S=4, B=5 if ramp is None else 5).replace(weight=np.array([1, 3, 40, 7], np.uint64))
    if ramp is not None:
        base = base.replace(ramp=ramp)
    long = oracle.Plan(base)
    ci = long.cycle(0)
    A_long = long.cumulative_taken()
    for upc in (1, 2, 3, max(1, ci.n_updates // 2)):
        short = oracle.Plan(base.replace(updates_per_cycle=upc))
        short.cycle(0)
        assert np.array_equal(short.cumulative_taken(), A_long[:upc + 1]), upc


def test_tiny_share_limit_in_plans():
    """A plan with the cumulative mixture needs every nonzero share ≥ 2^-62."""
    c = _corpus(9, S=2, B=4).replace(weight=np.array([1, 2**62], np.uint64))
    with pytest.raises(oracle.OracleError) as e:
        oracle.Plan(c)
    assert e.value.code == oracle.OR_E_INVAL
    oracle.Plan(c.replace(weight=np.array([2, 2**62], np.uint64)))   # just above the limit
