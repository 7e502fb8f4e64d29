"""Pins of the oracle's plan, emission and cycles against the properties the
pages state and against brute force written differently from the oracle
(Fractions instead of 128-bit cross-multiplication, Python's sorted instead of
qsort, a characterisation instead of a second next-fit).  No GPU is used."""
import hashlib
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import make_corpus, random_small
from synth.corpus import Corpus

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=", 1)
                vals[k.strip()] = [int(x) for x in v.split()]
    return vals


# --------------------------------------------------------------- apportionment and slots

def test_apportion_worked_example():
    g = _read_golden("apportion_tiny.txt")
    n = oracle.apportion(g["B"][0], g["weights"])
    assert n.tolist() == g["n"]
    ss, sk = oracle.slot_table(g["B"][0], n)
    assert ss.tolist() == g["slot_source"]
    assert sk.tolist() == g["slot_k"]


def _check_hamilton(B, w, n):
    W = sum(w)
    q = [Fraction(B * x, W) for x in w]
    assert sum(n) == B
    for qs, ns in zip(q, n):
        assert qs.numerator // qs.denominator <= ns <= -((-qs.numerator) // qs.denominator)
    rem = [(B * x) % W for x in w]
    floors = [(B * x) // W for x in w]
    seated = [s for s in range(len(w)) if n[s] == floors[s] + 1]
    unseated = [s for s in range(len(w)) if n[s] == floors[s]]
    for a in seated:
        for b in unseated:
            assert rem[a] > rem[b] or (rem[a] == rem[b] and a < b)


def test_apportion_hamilton_properties():
    r = np.random.default_rng(21)
    for _ in range(300):
        S = int(r.integers(1, 20))
        B = int(r.integers(1, 2000))
        w = r.integers(0, 10**9, size=S).tolist()
        if sum(w) == 0:
            w[0] = 1
        if r.random() < 0.3:  # many exact ties
            w = [int(x) % 7 + 1 for x in w]
        n = oracle.apportion(B, w).tolist()
        _check_hamilton(B, w, n)


def test_slot_table_properties():
    r = np.random.default_rng(22)
    for _ in range(200):
        S = int(r.integers(1, 12))
        n = r.integers(0, 40, size=S)
        if n.sum() == 0:
            n[0] = 1
        B = int(n.sum())
        ss, sk = oracle.slot_table(B, n)
        items = list(zip(ss.tolist(), sk.tolist()))
        assert sorted(items) == sorted((s, k) for s in range(S) for k in range(int(n[s])))
        keys = [(Fraction(2 * k + 1, 2 * int(n[s])), s) for s, k in items]
        assert keys == sorted(keys)


def test_every_update_within_two_samples_of_share():
    # [NS] Concepts: every update holds each source within two samples of its
    # recipe share (the fixed apportionment is within one).
    r = np.random.default_rng(23)
    for _ in range(200):
        S = int(r.integers(1, 16))
        B = int(r.integers(1, 1025))
        w = (r.integers(1, 10**9, size=S)).tolist()
        n = oracle.apportion(B, w)
        W = sum(w)
        for s in range(S):
            assert abs(Fraction(int(n[s])) - Fraction(B * w[s], W)) < 1


# --------------------------------------------------------------- hold-out, shuffle and strata merge by brute force

def _brute_order(c: Corpus, heldout: bool = False):
    """Kept docs (with heldout, the non-empty held-out ones) and their
    per-source order, from the pinned primitives with Python big ints,
    Python's sorted and exact Fractions."""
    L = c.lengths()
    keep = []
    for d in range(c.n_docs):
        h = oracle.doc_hash(c.tokens[c.offsets[d]:c.offsets[d + 1]])
        held = ((h * 10000) >> 64) < int(c.holdout_bp[c.source[d]])
        keep.append((held if heldout else not held) and L[d] > 0)
    order = []
    for s in range(c.n_sources):
        strata = []
        for k in range(int(c.n_strata[s])):
            docs = [d for d in range(c.n_docs) if keep[d] and c.source[d] == s and c.stratum[d] == k]
            strata.append(sorted(docs, key=lambda d: (oracle.shuffle_key(c.seed, d), d)))
        A = [sum(int(L[d]) for d in st) for st in strata]
        head = [0] * len(strata)
        a = [0] * len(strata)
        while True:
            cand = [k for k in range(len(strata)) if head[k] < len(strata[k])]
            if not cand:
                break
            k = min(cand, key=lambda k: (Fraction(a[k], A[k]), k))
            d = strata[k][head[k]]
            order.append(d)
            a[k] += int(L[d])
            head[k] += 1
    return np.array(keep, dtype=np.uint8), order


@pytest.mark.parametrize("seed", range(12))
def test_plan_order_matches_bruteforce(seed):
    c = random_small(seed, n_docs=int(30 + 15 * seed), max_strata=4, bp_max=4000)
    p = oracle.Plan(c)
    keep, order = _brute_order(c)
    assert p.keep.tolist() == keep.tolist()
    assert p.order.tolist() == order


def test_merge_tracks_stratum_shares():
    # For every document-boundary prefix of a source and every stratum k:
    # |taken_k − (A_k/A)·taken| ≤ A_k · max_j(longest doc of j / A_j).
    c = make_corpus("pretrain", 0.002)
    p = oracle.Plan(c)
    L = c.lengths()
    for s in range(c.n_sources):
        docs = p.order[int(p.src_doc_start[s]):int(p.src_doc_start[s + 1])]
        K = int(c.n_strata[s])
        A = [int(L[docs[c.stratum[docs] == k]].sum()) for k in range(K)]
        lmax = [int(L[docs[c.stratum[docs] == k]].max()) if A[k] else 0 for k in range(K)]
        At = sum(A)
        bound = max(Fraction(lmax[j], A[j]) for j in range(K) if A[j])
        taken = [0] * K
        tot = 0
        for d in docs:
            k = int(c.stratum[d])
            taken[k] += int(L[d])
            tot += int(L[d])
            for j in range(K):
                if A[j]:
                    assert abs(taken[j] - Fraction(A[j] * tot, At)) <= A[j] * bound


def test_keep_is_independent_of_seed_and_order_follows_seed():
    c = random_small(3, n_docs=120)
    p0 = oracle.Plan(c)
    p1 = oracle.Plan(c.replace(seed=c.seed + 1))
    assert p0.keep.tolist() == p1.keep.tolist()
    assert p0.hash.tolist() == p1.hash.tolist()
    assert sorted(p0.order.tolist()) == sorted(p1.order.tolist())
    assert p0.order.tolist() != p1.order.tolist()


def test_shuffle_order_is_stable_under_holdout_changes():
    # keys depend only on (seed, d): raising a hold-out rate removes docs but
    # never reorders the docs that stay, within a (source, stratum) group.
    c = random_small(4, n_docs=150, bp_max=0)
    p0 = oracle.Plan(c)
    p1 = oracle.Plan(c.replace(holdout_bp=np.full(c.n_sources, 3000, np.uint32)))
    kept1 = set(p1.order.tolist())
    assert kept1 < set(p0.order.tolist())
    for s in range(c.n_sources):
        for k in range(int(c.n_strata[s])):
            g0 = [d for d in p0.order.tolist() if c.source[d] == s and c.stratum[d] == k and d in kept1]
            g1 = [d for d in p1.order.tolist() if c.source[d] == s and c.stratum[d] == k]
            assert g0 == g1


# --------------------------------------------------------------- pieces and next-fit

def _check_next_fit(c: Corpus, p):
    T = c.T
    L = c.lengths()
    # pieces: each doc of the order, in order, split at multiples of T
    q = 0
    for i, d in enumerate(p.order.tolist()):
        o = 0
        while o < L[d]:
            ln = min(T, int(L[d]) - o)
            assert (int(p.piece_doc[q]), int(p.piece_off[q]), int(p.piece_len[q])) == (d, o, ln)
            o += ln
            q += 1
    assert q == p.piece_doc.shape[0]
    # windows: contiguous pieces; fill ≤ T; offsets are running sums; and the
    # next window's first piece would not have fitted (this pins next-fit)
    for s in range(c.n_sources):
        w0, w1 = int(p.src_win_start[s]), int(p.src_win_start[s + 1])
        assert int(p.win_first[w0]) == int(p.src_piece_start[s])
        fills = []
        for w in range(w0, w1):
            a, b = int(p.win_first[w]), int(p.win_first[w + 1])
            assert b > a
            f = 0
            for qq in range(a, b):
                assert int(p.piece_woff[qq]) == f
                f += int(p.piece_len[qq])
            assert f <= T
            assert int(p.win_real[w]) == f
            fills.append(f)
        for w in range(w0, w1 - 1):
            assert fills[w - w0] + int(p.piece_len[int(p.win_first[w + 1])]) > T
        if w1 > w0:
            assert int(p.win_first[w1]) == int(p.src_piece_start[s + 1])


@pytest.mark.parametrize("seed", range(10))
def test_next_fit_characterisation(seed):
    c = random_small(100 + seed, n_docs=80, T=64, max_len=200)
    p = oracle.Plan(c)
    _check_next_fit(c, p)


def test_next_fit_characterisation_on_workload_shapes():
    for name, sc in [("tiny", 0.2), ("pretrain", 0.001), ("sft", 0.002), ("long", 0.002)]:
        c = make_corpus(name, sc)
        p = oracle.Plan(c)
        _check_next_fit(c, p)


def _single_source(lengths, T, B=1, prompt=None):
    L = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(L.shape[0] + 1, np.uint64)
    np.cumsum(L, out=off[1:])
    r = np.random.default_rng(0)
    return Corpus("t", r.integers(0, 1000, size=int(off[-1]), dtype=np.uint32), off,
                  np.zeros(L.shape[0], np.uint16), np.zeros(L.shape[0], np.uint16),
                  None if prompt is None else np.asarray(prompt, np.uint32),
                  np.array([1], np.uint32), np.array([1], np.uint64), np.array([0], np.uint32),
                  T=T, B=B, updates_per_cycle=0)


@pytest.mark.parametrize("ell,n,T", [(1, 100, 64), (7, 50, 64), (32, 9, 64), (33, 9, 64), (64, 5, 64), (21, 40, 128)])
def test_next_fit_equal_lengths_closed_form(ell, n, T):
    p = oracle.Plan(_single_source([ell] * n, T))
    per = T // ell
    assert p.n_windows == -(-n // per)


@pytest.mark.parametrize("L,T", [(1, 64), (64, 64), (65, 64), (1000, 64), (4096, 64), (4097, 64)])
def test_long_document_splits_into_ceil_L_over_T(L, T):
    p = oracle.Plan(_single_source([L], T))
    assert p.n_windows == -(-L // T)


# --------------------------------------------------------------- emission

def _reconstruct_stream(c: Corpus, p, windows):
    """Rebuild each document from emitted windows (pieces split where pos
    restarts at 0 or the doc id changes), checking padding and masks."""
    pl = c.prompt_len
    got = {}
    for gw in windows:
        tok, pos, doc, mask = p.emit_window(int(gw))
        assert tok.shape[0] == c.T
        real = doc >= 0
        n_real = int(real.sum())
        assert real[:n_real].all() and not real[n_real:].any()  # padding only at the end
        assert (tok[n_real:] == c.pad_token).all() and (pos[n_real:] == 0).all() and (mask[n_real:] == 0).all()
        t = 0
        while t < n_real:
            d = int(doc[t])
            assert pos[t] == 0  # a piece starts at position id 0
            u = t
            while u < n_real and doc[u] == d and pos[u] == u - t:
                u += 1
            seq = got.setdefault(d, [])
            start = len(seq)
            seq.extend(tok[t:u].tolist())
            prompt = 0 if pl is None else int(pl[d])
            want_mask = (np.arange(start, start + (u - t)) >= prompt).astype(np.uint8)
            assert mask[t:u].tolist() == want_mask.tolist()
            t = u
    return got


@pytest.mark.parametrize("seed", range(6))
def test_every_kept_token_emitted_exactly_once_over_the_streams(seed):
    c = random_small(200 + seed, n_docs=70, T=64, max_len=180, prompts=bool(seed % 2), bp_max=3000)
    p = oracle.Plan(c)
    got = _reconstruct_stream(c, p, range(p.n_windows))
    kept = [d for d in range(c.n_docs) if p.keep[d]]
    assert sorted(got) == kept
    for d in kept:
        assert got[d] == c.tokens[c.offsets[d]:c.offsets[d + 1]].tolist()
    held = [d for d in range(c.n_docs) if not p.keep[d]]
    assert not set(held) & set(got)


def test_learned_count_is_mask_sum_and_prompt_masked():
    c = make_corpus("sft", 0.0005)
    p = oracle.Plan(c)
    ci = p.cycle(0)
    b = p.batch(0, min(4, ci.n_updates))
    assert (b["learned"] == b["mask"].reshape(b["mask"].shape[0], -1).sum(axis=1)).all()
    # completion-only: the first prompt_len tokens of each document are not learned
    assert b["mask"].sum() < (b["doc"] >= 0).sum()


# --------------------------------------------------------------- cycles, elasticity, resume

def test_cycles_take_consecutive_disjoint_ranges_until_exhausted():
    c = random_small(300, n_docs=200, T=64, B=6, max_len=90)
    p = oracle.Plan(c)
    n = p.n_per_update.astype(np.int64)
    M = p.windows_per_source.astype(np.int64)
    used = np.zeros(c.n_sources, np.int64)
    for cyc in range(100):
        U = 3
        fits = all(used[s] + U * n[s] <= M[s] for s in range(c.n_sources))
        if not fits:
            with pytest.raises(oracle.OracleError) as e:
                p.cycle(cyc, updates_per_cycle=U)
            assert e.value.code == oracle.OR_E_EXHAUSTED
            break
        ci = p.cycle(cyc, updates_per_cycle=U)
        assert ci.start.tolist() == used.tolist()
        wins = [p.window_of(b, j) for b in range(U) for j in range(c.B)]
        assert len(set(wins)) == len(wins)
        for s in range(c.n_sources):
            mine = sorted(w - int(p.src_win_start[s]) for w in wins
                          if p.src_win_start[s] <= w < p.src_win_start[s + 1])
            assert mine == list(range(int(used[s]), int(used[s] + U * n[s])))
        used += U * n
    else:
        pytest.fail("never exhausted")


def test_cycle_out_of_order_is_refused():
    p = oracle.Plan(random_small(301, n_docs=100))
    with pytest.raises(oracle.OracleError) as e:
        p.cycle(1)
    assert e.value.code == oracle.OR_E_STATE


def test_max_updates_cycle_uses_binding_source():
    c = make_corpus("tiny")
    p = oracle.Plan(c)
    ci = p.cycle(0)
    n = p.n_per_update.astype(np.int64)
    M = p.windows_per_source.astype(np.int64)
    assert ci.n_updates == min(M[s] // n[s] for s in range(2) if n[s] > 0)
    with pytest.raises(oracle.OracleError):
        p.cycle(1)  # the binding source has fewer than n_s windows left


@pytest.mark.parametrize("name,scale,worlds", [("tiny", 0.5, [1, 2, 4, 8]),
                                               ("pretrain", 0.006, [1, 8, 16, 32, 64])])
def test_global_batches_identical_at_any_rank_count(name, scale, worlds):
    c = make_corpus(name, scale)
    if name == "pretrain":
        c = c.replace(updates_per_cycle=2)
    ref = None
    for R in worlds:
        parts = []
        for r in range(R):
            p = oracle.Plan(c)  # a fresh, independent plan per rank
            p.cycle(0)
            parts.append(p.batch(0, 2, rank=r, world=R))
        cat = {k: np.concatenate([x[k] for x in parts], axis=1) for k in ("tokens", "pos", "doc", "mask", "digests")}
        learned = parts[0]["learned"]
        assert all((x["learned"] == learned).all() for x in parts)
        plain = [hashlib.sha256(b"".join(cat[k][i].tobytes() for k in ("tokens", "pos", "doc", "mask"))).digest()
                 for i in range(2)]
        fps = [oracle.batch_fingerprint(cat["digests"][i]) for i in range(2)]
        if ref is None:
            ref = (cat, learned, plain, fps)
        else:
            for k in cat:
                assert np.array_equal(cat[k], ref[0][k]), (R, k)
            assert (learned == ref[1]).all() and plain == ref[2] and fps == ref[3]


def test_world_not_dividing_batch_is_rejected():
    c = make_corpus("tiny", 0.2)
    p = oracle.Plan(c)
    p.cycle(0)
    with pytest.raises(oracle.OracleError) as e:
        p.batch(0, 1, rank=0, world=3)
    assert e.value.code == oracle.OR_E_INVAL


def test_resume_reproduces_remaining_batches():
    c = random_small(302, n_docs=300, T=64, B=4, max_len=60)
    a = oracle.Plan(c)
    a.cycle(0, updates_per_cycle=2)
    a.cycle(1, updates_per_cycle=3)
    full = a.batch(0, 3)
    b = oracle.Plan(c)  # "restart": plan again, replay the cycle schedule, index the step
    b.cycle(0, updates_per_cycle=2)
    b.cycle(1, updates_per_cycle=3)
    tail = b.batch(1, 2)
    for k in ("tokens", "pos", "doc", "mask", "digests", "learned"):
        assert np.array_equal(full[k][1:], tail[k])


def test_plan_digest_tracks_recipe_and_corpus():
    c = random_small(303, n_docs=200, T=64, B=4, max_len=60)

    def dig(cc):
        p = oracle.Plan(cc)
        return p.cycle(0, updates_per_cycle=1).plan_digest

    base = dig(c)
    assert dig(c) == base
    tok2 = c.tokens.copy()
    tok2[5] ^= 1
    variants = [c.replace(seed=c.seed ^ 1), c.replace(T=128),
                c.replace(weight=c.weight + np.uint64(1)), c.replace(B=8), c.replace(tokens=tok2)]
    for v in variants:
        assert dig(v) != base
