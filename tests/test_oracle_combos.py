"""Invariants of the oracle's cycles under seeded random combinations of every
mode (wrap packing, random read order, cumulative mixture, lanes, batch-size
ramp, held-out stream, arrivals, stream starts), checked without assuming the
order in which windows are read: padding only after a window's real
positions; every run of positions is a contiguous slice of its document's
tokens with position ids from 0; no document gives more tokens than it has;
an update holds the windows its batch says and learns Σ mask positions."""
import numpy as np
import pytest

import oracle
from _combos import combo_corpus


def _runs(tok, pos, doc, n_real):
    """Maximal runs (doc, start, end) of one piece each: the document id holds and
    position ids count up from 0."""
    t = 0
    while t < n_real:
        d = int(doc[t])
        assert pos[t] == 0
        u = t + 1
        while u < n_real and doc[u] == d and pos[u] == u - t:
            u += 1
        yield d, t, u
        t = u


def _is_slice(run, seq):
    n = len(run)
    return any(np.array_equal(seq[o:o + n], run) for o in range(len(seq) - n + 1))


@pytest.mark.parametrize("seed", range(24))
def test_combination_cycles_hold_the_invariants(seed):
    c, _ = combo_corpus(seed)
    cyc = int(getattr(c, "first_cycle", 0))
    p = oracle.Plan(c)
    try:
        ci = p.cycle(cyc)
    except oracle.OracleError as e:
        assert e.code == oracle.OR_E_EXHAUSTED
        return
    U = ci.n_updates
    b = p.batch(0, U)
    tok, pos, doc, mask = (x.reshape(-1, c.T) for x in (b["tokens"], b["pos"], b["doc"], b["mask"]))
    counts = [int(x) for x in ci.batches] if getattr(c, "ramp", None) is not None else [c.B] * U
    assert tok.shape[0] == sum(counts)
    emitted = {}
    for w in range(tok.shape[0]):
        real = doc[w] >= 0
        n_real = int(real.sum())
        assert real[:n_real].all() and not real[n_real:].any()
        assert (tok[w, n_real:] == c.pad_token).all() and (pos[w, n_real:] == 0).all()
        assert (mask[w, n_real:] == 0).all()
        for d, t, u in _runs(tok[w], pos[w], doc[w], n_real):
            assert p.keep[d]  # only documents of the planned stream
            seq = c.tokens[int(c.offsets[d]):int(c.offsets[d + 1])]
            assert _is_slice(tok[w, t:u], seq), (w, d)
            emitted[d] = emitted.get(d, 0) + (u - t)
    for d, n in emitted.items():
        assert n <= int(c.offsets[d + 1] - c.offsets[d]), d
    x = 0
    for i, k in enumerate(counts):
        assert int(b["learned"][i]) == int(mask[x:x + k].sum())
        x += k
