"""Pins of the oracle's random read order of windows (NeuronSpark-Trainer
README, Concepts: the trainer reads each source's windows of a segment in a
random order).  Reading: a segment is a cycle; the U·n_s windows source s
gives a cycle are read in order of (key64, i), key64 = x1·2^32 + x0 of
Philox4x32-10(counter = (i, s, cycle, 0x57494E44), key = seed).  The keys are
recomputed here from the Philox primitive (pinned against rocRAND) and sorted
with Python's sorted, independently of the oracle's own sort."""
import hashlib

import numpy as np
import pytest

import oracle
from synth import make_corpus, random_small


def _key(seed, s, cyc, i):
    x = oracle.philox4x32_10([i, s, cyc, 0x57494E44], [seed & 0xFFFFFFFF, seed >> 32])
    return (int(x[1]) << 32) | int(x[0])


def _reads(p, c, U):
    """[U][B] global window of every slot of the current cycle."""
    return [[p.window_of(b, j) for j in range(c.B)] for b in range(U)]


@pytest.mark.parametrize("seed", range(6))
def test_read_order_is_the_sorted_philox_permutation(seed):
    c = random_small(1200 + seed, n_docs=400, n_sources=1 + seed % 3, T=64, B=2 + seed, max_len=80)
    c = c.replace(seed=0x123456789 * (seed + 1) & 0xFFFFFFFFFFFFFFFF)
    seq, rnd = oracle.Plan(c), oracle.Plan(c.replace(read_random=True))
    for cyc, u in enumerate((3, 2)):
        a, b = seq.cycle(cyc, updates_per_cycle=u), rnd.cycle(cyc, updates_per_cycle=u)
        assert a.n_updates == b.n_updates == u
        ra, rb = _reads(seq, c, u), _reads(rnd, c, u)
        for s in range(c.n_sources):
            n = int(seq.n_per_update[s])
            base = int(seq.src_win_start[s]) + int(a.start[s])
            # slot (update b, k-th window of s) reads the source's i-th cycle window, i = b·n + k
            want_perm = sorted(range(u * n), key=lambda i: (_key(c.seed, s, cyc, i), i))
            got = []
            for bb in range(u):
                got += [rb[bb][j] - base for j in range(c.B) if int(seq.slot_src[j]) == s]
            assert got == want_perm, (s, cyc)
            # the same windows as the sequential order, each once
            seq_got = sorted(ra[bb][j] - base for bb in range(u) for j in range(c.B) if int(seq.slot_src[j]) == s)
            assert seq_got == list(range(u * n))


def test_read_order_keeps_counts_and_changes_batches():
    c = make_corpus("tiny", 1.0)
    seq, rnd = oracle.Plan(c), oracle.Plan(c.replace(read_random=True))
    a, b = seq.cycle(0), rnd.cycle(0)
    assert a.n_updates == b.n_updates and a.real_tokens == b.real_tokens and a.learned_tokens == b.learned_tokens
    assert a.plan_digest != b.plan_digest
    x, y = seq.batch(0, 4), rnd.batch(0, 4)
    assert not np.array_equal(x["tokens"], y["tokens"])
    for i in range(4):  # every update still takes n_s windows of each source, in slot order
        for j in range(c.B):
            s = int(seq.slot_src[j])
            gw = rnd.window_of(i, j)
            assert int(seq.src_win_start[s]) <= gw < int(seq.src_win_start[s + 1])


def test_read_order_batches_identical_at_any_rank_count():
    c = make_corpus("tiny", 0.5).replace(read_random=True)
    ref = None
    for R in (1, 2, 4, 8):
        parts = []
        for r in range(R):
            p = oracle.Plan(c)
            p.cycle(0)
            parts.append(p.batch(0, 2, rank=r, world=R))
        cat = {k: np.concatenate([x[k] for x in parts], axis=1) for k in ("tokens", "pos", "doc", "mask", "digests")}
        plain = [hashlib.sha256(b"".join(cat[k][i].tobytes() for k in ("tokens", "pos", "doc", "mask"))).digest()
                 for i in range(2)]
        if ref is None:
            ref = (cat, plain)
        else:
            assert all(np.array_equal(cat[k], ref[0][k]) for k in cat) and plain == ref[1]
