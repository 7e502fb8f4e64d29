"""Pins of the oracle's stream starts (C5s): a context that cuts each stream
from a given token, the cycle numbering and token count going on.

NeuronSpark-Trainer README, Training: every update has one sequence length,
updates never span a cycle end or a change of length, and a branch forks from
the state after a trunk cycle.  Reading: a new context (another T, or the same
one) is planned over the same corpus with each stream starting at the token
where the previous context's next cycle would have begun.  Next-fit and wrap
windows depend only on the stream from their first piece, so with the same T
the new context's cycles are the old context's next cycles, bit for bit; with
another T every token after the cut is emitted once and none before it."""
import numpy as np
import pytest

import oracle
from synth.corpus import random_small

MODES = [dict(), dict(wrap=True), dict(read_random=True), dict(cumulative=True),
         dict(ramp=((0, 128), (900, 384), (2500, 192))), dict(lanes=2), dict(heldout=True, wrap=True),
         dict(cumulative=True, lanes=3, ramp=((0, 192), (1200, 384)), read_random=True)]


def _corpus(seed, **mode):
    B = 6
    held = mode.get("heldout", False)
    c = random_small(seed, n_docs=900, n_sources=3, max_strata=2, T=64, B=B, max_len=200, prompts=True,
                     bp_max=6000 if held else 1500)
    return c.replace(updates_per_cycle=3, **mode)


def _resumed(c, ci, cycle):
    """The context that goes on after `cycle`: each stream from its next token."""
    tokens = ci.tokens_start + ci.positions
    return c.replace(start_tokens=ci.stream_next.copy(), first_cycle=cycle + 1, tokens_start=tokens)


@pytest.mark.parametrize("mi", range(len(MODES)))
def test_same_T_resume_reproduces_the_next_cycles(mi):
    c = _corpus(20 + mi, **MODES[mi])
    a = oracle.Plan(c)
    infos = []
    for k in range(4):
        try:
            infos.append(a.cycle(k))
        except oracle.OracleError:
            break
    assert len(infos) >= 2
    for cut in range(len(infos) - 1):
        ref = oracle.Plan(c)
        for k in range(cut + 2):
            ri = ref.cycle(k)
        b = oracle.Plan(_resumed(c, infos[cut], cut))
        bi = b.cycle(cut + 1)
        assert bi.n_updates == ri.n_updates and bi.batches.tolist() == ri.batches.tolist()
        assert bi.taken.tolist() == ri.taken.tolist()
        assert bi.stream_next.tolist() == ri.stream_next.tolist()
        ba, bb = ref.batch(0, ri.n_updates), b.batch(0, bi.n_updates)
        for key in ("tokens", "pos", "doc", "mask", "learned", "digests"):
            assert np.array_equal(ba[key], bb[key]), (mi, cut, key)


def test_zero_starts_are_the_plain_plan():
    c = _corpus(30)
    a = oracle.Plan(c)
    b = oracle.Plan(c.replace(start_tokens=np.zeros(c.n_sources, np.uint64)))
    ia, ib = a.cycle(0), b.cycle(0)
    assert np.array_equal(a.batch(0, ia.n_updates)["digests"], b.batch(0, ib.n_updates)["digests"])
    assert ia.plan_digest != ib.plan_digest   # the starts are part of the plan


@pytest.mark.parametrize("wrap", [False, True])
@pytest.mark.parametrize("T2", [128, 64 * 5])
def test_new_length_emits_every_later_token_once(wrap, T2):
    """Re-cut with another T: each stream's tokens from its start on, each once, in
    order, with masks by the documents' own offsets; nothing before the start."""
    c = _corpus(31, wrap=wrap)
    a = oracle.Plan(c)
    ai = a.cycle(0)
    start = ai.stream_next
    b = oracle.Plan(c.replace(T=T2, start_tokens=start.copy(), first_cycle=1, tokens_start=ai.positions))
    L = c.lengths()
    first = {}  # document -> its first token to emit
    for s in range(c.n_sources):
        x = 0
        for d in a.order[int(a.src_doc_start[s]):int(a.src_doc_start[s + 1])]:
            d = int(d)
            o = max(0, int(start[s]) - x)
            if o < L[d]:
                first[d] = o
            x += int(L[d])
    got = {}
    for gw in range(b.n_windows):
        tok, pos, doc, mask = b.emit_window(gw)
        n_real = int((doc >= 0).sum())
        t = 0
        while t < n_real:
            d = int(doc[t])
            u = t
            while u < n_real and doc[u] == d and pos[u] == u - t:
                u += 1
            at = first[d] + len(got.setdefault(d, []))   # the document offset of this run
            got[d].extend(tok[t:u].tolist())
            pl = int(c.prompt_len[d])
            assert mask[t:u].tolist() == [1 if at + i >= pl else 0 for i in range(u - t)]
            t = u
    assert sorted(got) == sorted(first)
    for d, o in first.items():
        assert got[d] == c.tokens[int(c.offsets[d]) + o:int(c.offsets[d + 1])].tolist(), d


def test_stream_next_is_the_total_once_used_up():
    c = _corpus(32).replace(updates_per_cycle=0)
    a = oracle.Plan(c)
    ai = a.cycle(0)
    L = c.lengths()
    for s in range(c.n_sources):
        tot = sum(int(L[int(d)]) for d in a.order[int(a.src_doc_start[s]):int(a.src_doc_start[s + 1])])
        M = int(a.windows_per_source[s])
        if int(ai.taken[s]) == M:
            assert int(ai.stream_next[s]) == tot
        else:
            assert int(ai.stream_next[s]) < tot
