"""Pins of the oracle's wrap packing (Zephon post, minimal example:
pack_flat(max_length, algorithm="wrap")).  Reading: per source, the merged
order's tokens form one stream cut every T tokens; a document crossing a cut
continues at the next window's first position with position ids restarting
at 0; only the stream's last window can be short (padded).  The checks below
rebuild each window from that definition directly (concatenate, slice) and
compare the oracle's emitted windows with it."""
import hashlib

import numpy as np
import pytest

import oracle
from synth import make_corpus, random_small
from test_oracle_plan import _reconstruct_stream, _single_source


def _stream_windows(c, p, s):
    """Windows of source s by the definition: the source's stream sliced
    every T tokens, with per-position doc id, position id and mask."""
    T = c.T
    docs = [int(d) for d in p.order[int(p.src_doc_start[s]):int(p.src_doc_start[s + 1])]]
    tok, doc, off = [], [], []
    for d in docs:
        a, b = int(c.offsets[d]), int(c.offsets[d + 1])
        tok.extend(c.tokens[a:b].tolist())
        doc.extend([d] * (b - a))
        off.extend(range(b - a))
    n = len(tok)
    out = []
    for w0 in range(0, n, T):
        w1 = min(w0 + T, n)
        t = np.full(T, c.pad_token, np.uint32)
        pos = np.zeros(T, np.int32)
        dc = np.full(T, -1, np.int32)
        mk = np.zeros(T, np.uint8)
        for x in range(w0, w1):
            i = x - w0
            t[i] = tok[x]
            dc[i] = doc[x]
            start = max(w0, x - off[x])  # where this document's run in the window starts
            pos[i] = x - start
            prompt = 0 if c.prompt_len is None else int(c.prompt_len[doc[x]])
            mk[i] = 1 if off[x] >= prompt else 0
        out.append((t, pos, dc, mk))
    return out


@pytest.mark.parametrize("seed", range(8))
def test_wrap_windows_are_the_stream_cut_every_T(seed):
    c = random_small(400 + seed, n_docs=60, n_sources=3, T=64, B=4, max_len=200, prompts=bool(seed % 2))
    c = c.replace(wrap=True)
    p = oracle.Plan(c)
    for s in range(c.n_sources):
        want = _stream_windows(c, p, s)
        w0, w1 = int(p.src_win_start[s]), int(p.src_win_start[s + 1])
        assert w1 - w0 == len(want)
        for k, (t, pos, dc, mk) in enumerate(want):
            gt, gp, gd, gm = p.emit_window(w0 + k)
            assert np.array_equal(gt, t) and np.array_equal(gp, pos), (s, k)
            assert np.array_equal(gd, dc) and np.array_equal(gm, mk), (s, k)
            real = int((dc >= 0).sum())
            assert int(p.win_real[w0 + k]) == real
            assert int(p.win_learn[w0 + k]) == int(mk.sum())
            if k < len(want) - 1:
                assert real == c.T  # only the stream's last window is short


@pytest.mark.parametrize("ell,n,T", [(1, 100, 64), (7, 50, 64), (33, 9, 64), (64, 5, 64), (21, 40, 128), (200, 3, 64)])
def test_wrap_window_count_closed_form(ell, n, T):
    p = oracle.Plan(_single_source([ell] * n, T).replace(wrap=True))
    assert p.n_windows == -(-(ell * n) // T)
    # pieces: one per (document, window) it touches
    touches = sum(((i * ell + ell - 1) // T) - ((i * ell) // T) + 1 for i in range(n))
    assert len(p.piece_doc) == touches


@pytest.mark.parametrize("seed", range(4))
def test_wrap_emits_every_kept_token_exactly_once(seed):
    c = random_small(500 + seed, n_docs=70, T=64, max_len=180, prompts=bool(seed % 2), bp_max=3000).replace(wrap=True)
    p = oracle.Plan(c)
    got = _reconstruct_stream(c, p, range(p.n_windows))
    kept = [d for d in range(c.n_docs) if p.keep[d]]
    assert sorted(got) == kept
    for d in kept:
        assert got[d] == c.tokens[c.offsets[d]:c.offsets[d + 1]].tolist()


def test_wrap_batches_identical_at_any_rank_count():
    c = make_corpus("tiny", 0.5).replace(wrap=True)
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


def test_wrap_is_part_of_the_plan_digest_and_keeps_the_order():
    c = random_small(600, n_docs=200, T=64, B=4, max_len=60)
    a, b = oracle.Plan(c), oracle.Plan(c.replace(wrap=True))
    assert np.array_equal(a.order, b.order) and np.array_equal(a.keep, b.keep)
    assert a.cycle(0, updates_per_cycle=1).plan_digest != b.cycle(0, updates_per_cycle=1).plan_digest
