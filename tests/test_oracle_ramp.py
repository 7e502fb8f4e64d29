"""Pins of the oracle's batch-size ramp (C6b).

NeuronSpark-Trainer README, Training, Updates: tokens_per_update is one number
or pieces by the tokens trained; the batch of an update is read at the data
line's token count (the cycle's start token plus its updates so far).
Reading: the count is the positions (B·T) of every earlier update, from 0 at
cycle 0, across cycles; an update starting at count t has tokens/T windows of
the last piece whose start is ≤ t.  The checks recompute the batches from that
definition, compare each update's counts with the apportionment of its own
batch (fixed) or with the quotas at the running seat count (cumulative), and
tie a one-piece ramp to the plan without a ramp."""
import itertools

import numpy as np
import pytest

import oracle
from synth.corpus import random_small


def _corpus(seed, ramp, B, **kw):
    c = random_small(seed, n_docs=kw.pop("n_docs", 700), n_sources=kw.pop("S", 3), max_strata=2, T=64, B=B,
                     max_len=150, bp_max=1500, prompts=kw.pop("prompts", False))
    return c.replace(ramp=ramp, **kw)


RAMPS = [((0, 128), (1000, 256), (3000, 512)), ((0, 512), (700, 64), (2000, 320)), ((0, 192),)]


def _expected_batches(ramp, T, t0, U):
    """Batches from the definition: piece of the count at each update's start."""
    out, t = [], t0
    for _ in range(U):
        k = max(i for i, (f, _) in enumerate(ramp) if f <= t)
        out.append(ramp[k][1] // T)
        t += out[-1] * T
    return out, t


@pytest.mark.parametrize("ri", range(len(RAMPS)))
@pytest.mark.parametrize("cumulative", [False, True])
def test_batches_follow_the_ramp_across_cycles(ri, cumulative):
    ramp = RAMPS[ri]
    B = max(t for _, t in ramp) // 64
    c = _corpus(10 + ri, ramp, B, updates_per_cycle=3, cumulative=cumulative)
    op = oracle.Plan(c)
    t = 0
    for k in range(6):
        try:
            ci = op.cycle(k)
        except oracle.OracleError as e:
            assert e.code == oracle.OR_E_EXHAUSTED and k >= 1
            break
        assert ci.tokens_start == t
        exp, t = _expected_batches(ramp, 64, t, ci.n_updates)
        assert ci.batches.tolist() == exp
        assert ci.positions == sum(exp) * 64


@pytest.mark.parametrize("seed", range(4))
def test_fixed_counts_are_each_batch_apportionment(seed):
    ramp = RAMPS[seed % 2]
    B = max(t for _, t in ramp) // 64
    c = _corpus(20 + seed, ramp, B, S=2 + seed % 3)
    op = oracle.Plan(c)
    ci = op.cycle(0)
    A = op.cumulative_taken()
    for b in range(ci.n_updates):
        counts = (A[b + 1] - A[b]).astype(int)
        assert counts.tolist() == oracle.apportion(int(ci.batches[b]), c.weight).tolist()
    # updates = 0: one more update would not fit
    nxt = oracle.apportion(_expected_batches(ramp, 64, 0, ci.n_updates + 1)[0][-1], c.weight)
    assert any(int(A[-1, s]) + int(nxt[s]) > int(op.windows_per_source[s]) for s in range(c.n_sources))


@pytest.mark.parametrize("seed", range(4))
def test_cumulative_quota_at_running_seat_count(seed):
    ramp = RAMPS[seed % 3]
    B = max(t for _, t in ramp) // 64
    c = _corpus(30 + seed, ramp, B, S=2 + seed % 3, cumulative=True)
    op = oracle.Plan(c)
    ci = op.cycle(0)
    A = op.cumulative_taken()
    W = int(sum(int(x) for x in c.weight))
    H = 0
    for u in range(ci.n_updates + 1):
        assert int(A[u].sum()) == H
        for s, w in enumerate(c.weight):
            q = H * int(w)
            assert q // W <= int(A[u, s]) <= -(-q // W)
        if u < ci.n_updates:
            assert (A[u + 1] >= A[u]).all()
            H += int(ci.batches[u])


def _enumerate(Bs, w):
    S, W = len(w), sum(w)
    out = []

    def rec(u, A, H, acc):
        if u == len(Bs):
            out.append(np.array(acc, np.uint32))
            return
        for c in itertools.product(range(Bs[u] + 1), repeat=S):
            if sum(c) != Bs[u]:
                continue
            nxt = [A[s] + c[s] for s in range(S)]
            h = H + Bs[u]
            if all(h * w[s] // W <= nxt[s] <= -(-h * w[s] // W) for s in range(S)):
                rec(u + 1, nxt, h, acc + [nxt])

    rec(0, [0] * S, 0, [[0] * S])
    return out


@pytest.mark.parametrize("Bs,w", [([1, 3, 2, 1], [1, 2, 4]), ([2, 2, 1, 3], [5, 1, 1]), ([3, 1, 1, 1, 2], [3, 2]),
                                  ([1, 1, 4, 2], [1, 1, 1, 1])])
def test_cumulative_ramp_among_all_valid_schedules(Bs, w):
    U, A = oracle.cumulative(max(Bs), w, [10**6] * len(w), updates=len(Bs), batches=Bs)
    assert U == len(Bs)
    allv = _enumerate(Bs, w)
    assert any(np.array_equal(A, v) for v in allv)
    if len(allv) == 1:
        assert np.array_equal(A, allv[0])


@pytest.mark.parametrize("cumulative", [False, True])
def test_one_piece_ramp_is_the_plain_plan(cumulative):
    """tokens_per_update = B·T from token 0: the same batches as without a ramp."""
    c = _corpus(40, None, 6, updates_per_cycle=4, cumulative=cumulative)
    a = oracle.Plan(c)
    b = oracle.Plan(c.replace(ramp=((0, 6 * 64),)))
    ia, ib = a.cycle(0), b.cycle(0)
    assert ia.n_updates == ib.n_updates and ia.taken.tolist() == ib.taken.tolist()
    ba, bb = a.batch(0, 4), b.batch(0, 4)
    for k in ("tokens", "pos", "doc", "mask", "digests"):
        assert np.array_equal(ba[k].reshape(-1), bb[k].reshape(-1)), k
    assert np.array_equal(ba["learned"], bb["learned"])
    assert ia.plan_digest != ib.plan_digest


@pytest.mark.parametrize("cumulative", [False, True])
def test_ramp_uses_each_window_once_and_slices_by_rank(cumulative):
    ramp = ((0, 128), (900, 256), (2500, 512))
    c = _corpus(50, ramp, 8, S=3, cumulative=cumulative)
    op = oracle.Plan(c)
    ci = op.cycle(0)
    seen = [op.window_of(b, j) for b in range(ci.n_updates) for j in range(int(ci.batches[b]))]
    assert len(seen) == len(set(seen))
    expect = set()
    for s in range(c.n_sources):
        lo = int(op.src_win_start[s] + ci.start[s])
        expect.update(range(lo, lo + int(ci.taken[s])))
    assert set(seen) == expect
    n = ci.n_updates
    whole = op.batch(0, n, world=1)
    parts = [op.batch(0, n, rank=r, world=2) for r in range(2)]
    # rank r holds the r-th half of each update's windows
    off, offs = 0, [0, 0]
    for b in range(n):
        Bb = int(ci.batches[b])
        for r in range(2):
            seg = parts[r]["tokens"][offs[r]:offs[r] + Bb // 2]
            assert np.array_equal(seg, whole["tokens"][off + r * (Bb // 2):off + (r + 1) * (Bb // 2)])
            offs[r] += Bb // 2
        off += Bb
    assert np.array_equal(parts[0]["learned"], whole["learned"])


def test_packed_rows_with_ramp():
    """Padding-free rows of a ramped cycle: each row is its update's windows without padding."""
    ramp = ((0, 128), (900, 256))
    c = _corpus(60, ramp, 4)
    op = oracle.Plan(c)
    ci = op.cycle(0)
    n = min(ci.n_updates, 12)
    pk = op.batch_packed(0, n, bucket=64)
    pad = op.batch(0, n, digests=False)
    w = 0
    for i in range(n):
        Bb = int(ci.batches[i])
        row = []
        for jj in range(Bb):
            real = int((pad["doc"][w] >= 0).sum())
            row.append(pad["tokens"][w][:real])
            w += 1
        row = np.concatenate(row)
        assert pk["row_start"][i][Bb] == row.size
        assert (pk["row_start"][i][Bb:] == row.size).all()
        assert np.array_equal(pk["tokens"][i][:row.size], row)


@pytest.mark.parametrize("ramp,B", [(((0, 100),), 2), (((5, 128),), 2), (((0, 128), (0, 256)), 4),
                                    (((0, 128), (10, 256)), 8)])
def test_bad_ramps_rejected(ramp, B):
    """Tokens not a multiple of T, a first piece not at 0, pieces not rising, or B
    other than the largest batch."""
    c = _corpus(70, ramp, B)
    with pytest.raises(oracle.OracleError) as e:
        oracle.Plan(c)
    assert e.value.code == oracle.OR_E_INVAL
