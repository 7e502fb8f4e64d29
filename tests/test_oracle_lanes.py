"""Pins of the oracle's lanes (C2l).

Zephon blog post, "lanes instead of ranks": the data are split into a fixed
number of logical streams, each with its own ordered samples and its own
packing state, and the ranks take whole lanes, so the global batches do not
depend on the rank count.  Reading: document d belongs to lane d mod L; each
(source, lane) is a stream planned as a source is; each update gives lane l
its B/L consecutive slots, apportioned over the sources like a batch of B/L.
The checks recompute each stream's order by brute force, rebuild every kept
document from the emitted windows, check the slot layout and counts per lane,
and tie L = 1 to the plan without lanes."""
import numpy as np
import pytest

import oracle
from synth.corpus import Corpus, random_small
from test_oracle_plan import _brute_order, _reconstruct_stream


def _corpus(seed, L, B=8, **kw):
    c = random_small(seed, n_docs=kw.pop("n_docs", 600), n_sources=kw.pop("S", 3), max_strata=3, T=64, B=B,
                     max_len=150, bp_max=2000, prompts=kw.pop("prompts", bool(seed % 2)))
    return c.replace(lanes=L, **kw)


def _streams_corpus(c):
    """The same documents with source s·L + d mod L (a stream per source and lane)."""
    L = c.lanes
    d = np.arange(c.n_docs)
    return Corpus(c.name, c.tokens, c.offsets, (c.source.astype(np.int64) * L + d % L).astype(np.uint16), c.stratum,
                  c.prompt_len, np.repeat(c.n_strata, L), np.repeat(c.weight, L), np.repeat(c.holdout_bp, L),
                  T=c.T, B=c.B, updates_per_cycle=c.updates_per_cycle, seed=c.seed, pad_token=c.pad_token)


@pytest.mark.parametrize("seed,L", [(0, 2), (1, 4), (2, 3), (3, 8)])
def test_stream_orders_match_bruteforce(seed, L):
    c = _corpus(seed, L, B=L * 2)
    p = oracle.Plan(c)
    keep, order = _brute_order(_streams_corpus(c))
    assert p.keep.tolist() == keep.tolist()
    assert p.order.tolist() == order
    for v in range(c.n_sources * L):  # stream v holds only its source's documents of lane v mod L
        docs = p.order[int(p.src_doc_start[v]):int(p.src_doc_start[v + 1])]
        assert all(int(c.source[d]) == v // L and int(d) % L == v % L for d in docs)


@pytest.mark.parametrize("seed,L,B", [(4, 2, 8), (5, 4, 12), (6, 3, 9)])
def test_lane_slots_and_counts(seed, L, B):
    c = _corpus(seed, L, B=B)
    p = oracle.Plan(c)
    per = B // L
    n = oracle.apportion(per, c.weight)
    for l in range(L):
        slots = p.slot_src[l * per:(l + 1) * per]
        assert all(int(v) % L == l for v in slots)
        assert np.bincount(slots // L, minlength=c.n_sources).tolist() == n.tolist()
    assert p.n_per_update.tolist() == np.repeat(n, L).tolist()


@pytest.mark.parametrize("seed,L", [(7, 2), (8, 4)])
def test_every_kept_token_once_and_lanes_in_their_slots(seed, L):
    c = _corpus(seed, L, B=2 * L)
    p = oracle.Plan(c)
    ci = p.cycle(0)
    all_windows = np.arange(p.n_windows)
    got = _reconstruct_stream(c, p, all_windows)
    kept = [d for d in range(c.n_docs) if p.keep[d]]
    assert sorted(got) == kept
    per = c.B // L
    for b in range(ci.n_updates):
        for j in range(c.B):
            tok, pos, doc, mask = p.emit_window(p.window_of(b, j))
            docs = set(int(x) for x in doc[doc >= 0])
            assert all(d % L == j // per for d in docs)


@pytest.mark.parametrize("cumulative", [False, True])
def test_one_lane_is_the_plain_plan(cumulative):
    c = _corpus(9, 1, B=6, cumulative=cumulative)
    a, b = oracle.Plan(c), oracle.Plan(c.replace(lanes=0))
    ia, ib = a.cycle(0), b.cycle(0)
    assert ia.plan_digest == ib.plan_digest
    ba, bb = a.batch(0, ia.n_updates), b.batch(0, ib.n_updates)
    for k in ("tokens", "digests", "learned"):
        assert np.array_equal(ba[k], bb[k])


@pytest.mark.parametrize("cumulative", [False, True])
def test_lanes_identical_at_any_rank_count(cumulative):
    L = 4
    c = _corpus(10, L, B=8, cumulative=cumulative)
    p = oracle.Plan(c)
    ci = p.cycle(0)
    n = min(ci.n_updates, 5)
    whole = p.batch(0, n)
    for world in (2, 4):
        parts = [p.batch(0, n, rank=r, world=world) for r in range(world)]
        for k in ("tokens", "doc", "digests"):
            assert np.array_equal(np.concatenate([x[k] for x in parts], axis=1), whole[k])


def test_cumulative_lanes_share_one_schedule():
    """Each lane takes the same counts: the per-lane schedule over the sources."""
    L, B = 3, 6
    c = _corpus(11, L, B=B, cumulative=True, S=3)
    c = c.replace(weight=np.array([1, 5, 30], np.uint64))
    p = oracle.Plan(c)
    ci = p.cycle(0)
    A = p.cumulative_taken()
    U = ci.n_updates
    W = 36
    for u in range(U + 1):
        for v in range(c.n_sources * L):
            q = u * (B // L) * int(c.weight[v // L])
            assert q // W <= int(A[u, v]) <= -(-q // W)
            assert A[u, v] == A[u, (v // L) * L]   # every lane of a source the same
    _, Aref = oracle.cumulative(B // L, c.weight, [10**6] * 3, updates=U)
    assert np.array_equal(A[:, ::L], Aref)


def test_lanes_with_ramp():
    c = _corpus(12, 2, B=8).replace(ramp=((0, 128), (800, 512)))
    p = oracle.Plan(c)
    ci = p.cycle(0)
    A = p.cumulative_taken()
    for b in range(ci.n_updates):
        per = int(ci.batches[b]) // 2
        n = oracle.apportion(per, c.weight)
        assert (A[b + 1] - A[b]).astype(int).tolist() == np.repeat(n, 2).tolist()


@pytest.mark.parametrize("L,B,ramp", [(3, 8, None), (2, 6, ((0, 64 * 6), (100, 64 * 3)))])
def test_bad_lane_counts_rejected(L, B, ramp):
    c = _corpus(13, L, B=B).replace(ramp=ramp)
    with pytest.raises(oracle.OracleError) as e:
        oracle.Plan(c)
    assert e.value.code == oracle.OR_E_INVAL
