"""Seeded random combinations of every mode on small corpora (wrap packing,
random read order, cumulative mixture, lanes, batch-size ramp, held-out
stream, arrivals, stream starts, window lengths that are not multiples of
64, chunked window digests), for parity between the GPU and the oracle."""
import numpy as np

import oracle
from synth.corpus import random_small


def combo_corpus(seed, even=False):
    """(corpus, description): the modes drawn from the seed; with stream starts,
    the corpus goes on from the oracle's cycle 0 (first cycle 1).  even: every
    update's batch a multiple of 2·lanes and an even lane count (two ranks can
    split it), and a combination that runs out of data before its first cycle
    is drawn again (from the seed and the attempt), so every seed has batches."""
    if not even:
        return _draw(seed, seed, [4242, seed], False)
    for attempt in range(32):
        c, desc = _draw(seed + 10000 * attempt, seed, [4242, seed] + ([attempt] if attempt else []), True)
        try:
            oracle.Plan(c).cycle(int(c.first_cycle))
        except oracle.OracleError:
            continue
        if attempt:
            desc["redrawn"] = attempt
        return c, desc
    raise RuntimeError(f"no combination with batches for seed {seed}")


def _draw(corpus_seed, seed, seq, even):
    r = np.random.default_rng(np.random.SeedSequence(seq))
    L = int(r.choice([1, 1, 2, 4] if even else [1, 1, 2, 3]))
    ramp = r.random() < 0.3
    heldout = r.random() < 0.2
    T = 64 * int(r.choice([1, 2]))
    # about a third of the combinations take a window length that is not a multiple of 64 (nor of 4),
    # drawn from a stream of its own so the other draws stay as they were
    t_alt = np.random.default_rng(np.random.SeedSequence(seq + [77]))
    if t_alt.random() < 0.35:
        T = int(t_alt.choice([37, 100]))
    # about a third take chunked window digests, from a stream of their own as well
    chunked = bool(np.random.default_rng(np.random.SeedSequence(seq + [78])).random() < 0.35)
    m = 2 * L if even else L
    b = [m * int(x) for x in r.integers(1, 4, size=2)]
    B = max(b) if ramp else m * int(r.integers(1, 4))
    c = random_small(corpus_seed, n_docs=int(r.integers(400, 1400)), n_sources=int(r.integers(1, 5)),
                     max_strata=int(r.integers(1, 4)), T=T, B=B, max_len=int(r.integers(40, 400)),
                     prompts=bool(r.random() < 0.5), bp_max=6000 if heldout else 1500)
    mode = dict(digest_chunked=chunked, wrap=bool(r.random() < 0.4), read_random=bool(r.random() < 0.4),
                cumulative=bool(r.random() < 0.4), heldout=heldout, lanes=L,
                updates_per_cycle=0 if heldout else int(r.choice([0, 2, 3, 5])))
    if ramp:
        mode["ramp"] = ((0, b[0] * T), (int(r.integers(T, 40 * T)), b[1] * T))
    if r.random() < 0.3:
        n_seg = int(r.integers(2, 4))
        mode.update(segment=r.integers(0, n_seg, size=c.n_docs).astype(np.uint16), n_segments=n_seg)
    c = c.replace(**mode)
    desc = {k: v for k, v in mode.items() if k not in ("segment",) and v not in (False, None)}
    if r.random() < 0.25:
        try:
            ci = oracle.Plan(c).cycle(0)
            c = c.replace(start_tokens=ci.stream_next.copy(), first_cycle=1, tokens_start=ci.tokens_start + ci.positions)
            desc["resumed"] = True
        except oracle.OracleError:
            pass
    return c, desc
