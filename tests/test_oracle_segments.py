"""Pins of the oracle's streamed corpora (C3a): documents arrive with the
cycles, each source's order goes arrival by arrival.

NeuronSpark-Trainer README, Concepts: a data line's cycles are each
downloaded, tokenized, trained on and deleted; a file's documents are shuffled
at tokenization; the files left open give the rest to the next cycles.
Reading: a document belongs to the arrival it came with; within a source each
arrival is shuffled and strata-merged on its own and the arrivals follow one
another, so the order of the arrivals so far never changes when more arrive.
With stream starts (C5s), a context per arrival that goes on where the
previous one stopped plans the same cycles as one context over every arrival."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth.corpus import Corpus, random_small


def _arrivals(seed, n_seg, n_docs=1600, even=False, **kw):
    """A corpus whose documents are sorted by arrival (indices grow with it); the
    arrivals are of random sizes, or of equal ones with `even`."""
    c = random_small(seed, n_docs=n_docs, n_sources=kw.pop("S", 3), max_strata=2, T=64, B=kw.pop("B", 6),
                     max_len=150, prompts=True, bp_max=1500)
    r = np.random.default_rng(seed + 7)
    c = _permuted(c, r.permutation(c.n_docs))   # the sources arrive mixed
    if even:
        cuts = np.arange(1, n_seg) * (c.n_docs // n_seg)
    else:
        cuts = np.sort(r.choice(np.arange(1, c.n_docs), size=n_seg - 1, replace=False))
    seg = np.zeros(c.n_docs, np.uint16)
    for k, x in enumerate(cuts):
        seg[x:] = k + 1
    return c.replace(segment=seg, n_segments=n_seg, **kw), np.concatenate([[0], cuts, [c.n_docs]])


def _permuted(c, perm):
    """The same documents, document i of the result being document perm[i]."""
    L = c.lengths()[perm]
    offsets = np.concatenate([[0], np.cumsum(L)]).astype(c.offsets.dtype)
    tokens = np.concatenate([c.tokens[int(c.offsets[d]):int(c.offsets[d + 1])] for d in perm]).astype(c.tokens.dtype)
    return Corpus(c.name, tokens, offsets, c.source[perm], c.stratum[perm],
                  None if c.prompt_len is None else c.prompt_len[perm], c.n_strata, c.weight, c.holdout_bp,
                  T=c.T, B=c.B, updates_per_cycle=c.updates_per_cycle, seed=c.seed, pad_token=c.pad_token)


def _prefix(c, n):
    """The corpus as it stood when its first n documents had arrived."""
    return Corpus(c.name, c.tokens, c.offsets[:n + 1], c.source[:n], c.stratum[:n],
                  None if c.prompt_len is None else c.prompt_len[:n], c.n_strata, c.weight, c.holdout_bp,
                  T=c.T, B=c.B, updates_per_cycle=c.updates_per_cycle, seed=c.seed, pad_token=c.pad_token,
                  wrap=c.wrap, segment=c.segment[:n], n_segments=c.n_segments)


@pytest.mark.parametrize("seed,n_seg", [(0, 2), (1, 3), (2, 5)])
def test_order_is_arrival_by_arrival(seed, n_seg):
    """Brute force: per source, per arrival, strata sorted by key and merged by
    least consumed fraction (Fractions), arrivals in order."""
    c, _ = _arrivals(seed, n_seg)
    p = oracle.Plan(c)
    L = c.lengths()
    order = []
    for s in range(c.n_sources):
        for g in range(n_seg):
            strata = []
            for k in range(int(c.n_strata[s])):
                docs = [d for d in range(c.n_docs) if p.keep[d] and c.source[d] == s and c.segment[d] == g
                        and c.stratum[d] == k]
                strata.append(sorted(docs, key=lambda d: (oracle.shuffle_key(c.seed, d), d)))
            A = [sum(int(L[d]) for d in st) for st in strata]
            head, a = [0] * len(strata), [0] * len(strata)
            while True:
                cand = [k for k in range(len(strata)) if head[k] < len(strata[k])]
                if not cand:
                    break
                k = min(cand, key=lambda k: (Fraction(a[k], A[k]), k))
                order.append(strata[k][head[k]])
                a[k] += int(L[strata[k][head[k]]])
                head[k] += 1
    assert p.order.tolist() == order


def test_one_arrival_is_the_plain_plan():
    c, _ = _arrivals(3, 2)
    a = oracle.Plan(c.replace(segment=np.zeros(c.n_docs, np.uint16)))
    b = oracle.Plan(c.replace(segment=None, n_segments=1))
    assert a.order.tolist() == b.order.tolist()


@pytest.mark.parametrize("seed,n_seg", [(4, 3), (5, 4)])
def test_earlier_arrivals_keep_their_order(seed, n_seg):
    c, cuts = _arrivals(seed, n_seg)
    full = oracle.Plan(c)
    for g in range(1, n_seg):
        part = oracle.Plan(_prefix(c, int(cuts[g])))
        for s in range(c.n_sources):
            a = part.order[int(part.src_doc_start[s]):int(part.src_doc_start[s + 1])].tolist()
            b = full.order[int(full.src_doc_start[s]):int(full.src_doc_start[s + 1])].tolist()
            assert b[:len(a)] == a


ARRIVAL_MODES = [dict(), dict(wrap=True), dict(cumulative=True), dict(lanes=2), dict(read_random=True),
                 dict(ramp=((0, 256), (1500, 512))), dict(cumulative=True, lanes=2, read_random=True, wrap=True)]


def arrival_corpus(seed, mode):
    """Four equal arrivals; B = 8 (the ramp's largest batch, two lanes of four)."""
    c, cuts = _arrivals(seed, 4, n_docs=2400, even=True, updates_per_cycle=4, B=8)
    return c.replace(**mode), cuts


@pytest.mark.parametrize("mi", range(len(ARRIVAL_MODES)))
def test_a_context_per_arrival_plans_the_same_cycles(mi):
    """Cycle c planned by a context over arrivals 0..c, going on from the previous
    context's stream tokens, next cycle number and tokens trained, equals cycle c
    of one context over every arrival, in every mode (the cycles here never reach
    a stream's still open last window)."""
    mode = ARRIVAL_MODES[mi]
    c, cuts = arrival_corpus(6, mode)
    full = oracle.Plan(c)
    nxt, tokens = None, 0
    for cyc in range(4):
        fi = full.cycle(cyc)
        cc = _prefix(c, int(cuts[cyc + 1])).replace(**mode)
        if cyc:
            cc = cc.replace(start_tokens=nxt, first_cycle=cyc, tokens_start=tokens)
        part = oracle.Plan(cc)
        pi = part.cycle(cyc)
        # the cycle stays clear of each stream's last (still open) window
        assert all(int(x) >= 1 for x in pi.remaining)
        assert pi.n_updates == fi.n_updates and pi.taken.tolist() == fi.taken.tolist()
        assert pi.batches.tolist() == fi.batches.tolist()
        a, b = full.batch(0, fi.n_updates), part.batch(0, pi.n_updates)
        for key in ("tokens", "pos", "doc", "mask", "digests", "learned"):
            assert np.array_equal(a[key], b[key]), (cyc, key)
        assert pi.stream_next.tolist() == fi.stream_next.tolist()
        nxt, tokens = pi.stream_next.copy(), pi.tokens_start + pi.positions


def test_bad_arrival_ids_rejected():
    c, _ = _arrivals(7, 2)
    seg = c.segment.copy()
    seg[5] = 9
    with pytest.raises(oracle.OracleError) as e:
        oracle.Plan(c.replace(segment=seg))
    assert e.value.code == oracle.OR_E_INVAL
