"""Pins of the oracle's held-out (validation) stream.  NeuronSpark-Trainer
README, Concepts: each source's validation rows come from its held-out
documents of every stratum, and the validation mix weights the sources by the
recipe.  Reading: the same plan over the non-empty held-out documents instead
of the kept ones (PACK_FLAG_HELDOUT on the GPU side)."""
import numpy as np
import pytest

import oracle
from synth import random_small
from test_oracle_plan import _brute_order, _reconstruct_stream


@pytest.mark.parametrize("seed", range(8))
def test_heldout_stream_is_the_complement_of_training(seed):
    c = random_small(700 + seed, n_docs=120, n_sources=3, max_strata=3, max_len=120, bp_max=5000)
    tr, ho = oracle.Plan(c), oracle.Plan(c.replace(heldout=True))
    L = c.lengths()
    # every non-empty document is in exactly one of the two streams
    for d in range(c.n_docs):
        assert int(tr.keep[d]) + int(ho.keep[d]) == (1 if L[d] > 0 else 0), d
    assert np.array_equal(tr.hash, ho.hash)
    # the per-source statistics keep their meaning: held_* from the hash, kept_* = the stream
    assert np.array_equal(tr.held_docs, ho.held_docs) and np.array_equal(tr.held_tokens, ho.held_tokens)
    for s in range(c.n_sources):
        docs = [d for d in range(c.n_docs) if ho.keep[d] and c.source[d] == s]
        assert int(ho.kept_docs[s]) == len(docs) and int(ho.kept_tokens[s]) == int(sum(L[d] for d in docs))


@pytest.mark.parametrize("seed", range(8))
def test_heldout_order_matches_bruteforce(seed):
    c = random_small(800 + seed, n_docs=int(40 + 20 * seed), max_strata=4, bp_max=6000).replace(heldout=True)
    p = oracle.Plan(c)
    keep, order = _brute_order(c, heldout=True)
    assert p.keep.tolist() == keep.tolist()
    assert p.order.tolist() == order


@pytest.mark.parametrize("wrap", [False, True])
def test_heldout_emits_each_heldout_token_exactly_once(wrap):
    c = random_small(900, n_docs=300, T=64, max_len=150, prompts=True, bp_max=6000).replace(heldout=True, wrap=wrap)
    p = oracle.Plan(c)
    got = _reconstruct_stream(c, p, range(p.n_windows))
    sel = [d for d in range(c.n_docs) if p.keep[d]]
    assert sel and sorted(got) == sel
    for d in sel:
        assert got[d] == c.tokens[c.offsets[d]:c.offsets[d + 1]].tolist()


def test_heldout_stream_is_its_own_plan():
    c = random_small(950, n_docs=400, T=64, B=2, max_len=80, bp_max=6000)
    a = oracle.Plan(c).cycle(0, updates_per_cycle=1).plan_digest
    b = oracle.Plan(c.replace(heldout=True))
    b.cycle(0, updates_per_cycle=1)
    assert b.cycle_info.plan_digest != a
