"""Pin of the plan digest's byte layout, rebuilt independently of the oracle.

The plan digest identifies what a cycle was planned from, so that a resume
planned from another recipe, seed, corpus or sample order is refused
(NeuronSpark-Trainer README, Training).  The pages fix no layout: the layout
is the library's own definition, stated here field by field and rebuilt with
``struct.pack`` and ``hashlib`` from quantities this test derives itself:

- each stream's kept documents and tokens and the sum of the kept documents'
  hashes, from the corpus, the stream of each document (its source, or
  source·L + d mod L with lanes) and the keep flags;
- the order check, Σ_i mix64((i << 32) xor order[i]) mod 2^64, with mix64
  written here from the SplitMix64 paper and checked against its published
  first output;
- a stream record (60 bytes, little-endian): weight u64, hold-out rate u32,
  strata u32, windows per update u32, windows in the stream u64, kept
  documents u64, kept tokens u64, the cycle's first window u64, the stream's
  first token u64 (0 without stream starts);
- the message: "DPACKP", 'W' (wrap) or 'D' (next-fit), 'V' (held-out) or
  '1' (training); then, in this order and only when the mode is on, "RAND";
  "CUMU"; "RAMP" + pieces u32 + (from u64, tokens u64) per piece + tokens
  trained before the cycle u64; "LANE" + lanes u32; "STRT"; "SEGS" +
  arrivals u32; then T u32, B u32, seed u64, streams u32, pad token u32,
  cycle u32, updates u32, order check u64, hash check u64; then one 32-byte
  leaf per 8 streams: SHA-256 of those streams' records.

A one-byte change to a record field's width or order, to a mode word, or to
the leaf grouping in the oracle fails here.
"""
import hashlib
import struct

import numpy as np
import pytest

import oracle
from synth.corpus import random_small

M64 = (1 << 64) - 1


def mix64(z: int) -> int:
    """SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014)."""
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_mix64_published_value():
    # SplitMix64 from state 0: the first output is mix64(0x9E3779B97F4A7C15)
    assert mix64(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF


def rebuild(plan: "oracle.Plan", info: "oracle.CycleInfo") -> bytes:
    c = plan.corpus
    L = plan.lanes
    S = c.n_sources * L
    d_idx = np.arange(c.n_docs, dtype=np.int64)
    stream = c.source.astype(np.int64) * L + (d_idx % L if L > 1 else 0)
    lens = np.diff(c.offsets.astype(np.int64))
    keep = plan.keep.astype(bool)
    kept_docs = np.bincount(stream[keep], minlength=S)
    kept_tokens = np.bincount(stream[keep], weights=lens[keep].astype(np.float64), minlength=S)
    hash_check = sum(int(h) for h in plan.hash[keep]) & M64
    order_check = 0
    for i, d in enumerate(plan.order.tolist()):
        order_check = (order_check + mix64((i << 32) ^ d)) & M64
    windows = np.diff(plan.src_win_start.astype(np.int64))
    start_tok = c.start_tokens if c.start_tokens is not None else np.zeros(S, np.uint64)

    records = b"".join(
        struct.pack("<QIIIQQQQQ", int(c.weight[s // L]), int(c.holdout_bp[s // L]), int(c.n_strata[s // L]),
                    int(plan.n_per_update[s]), int(windows[s]), int(kept_docs[s]), int(kept_tokens[s]),
                    int(info.start[s]), int(start_tok[s]))
        for s in range(S))
    assert len(records) == 60 * S

    head = b"DPACKP" + (b"W" if c.wrap else b"D") + (b"V" if c.heldout else b"1")
    if c.read_random:
        head += b"RAND"
    if c.cumulative:
        head += b"CUMU"
    if c.ramp is not None:
        head += b"RAMP" + struct.pack("<I", len(c.ramp))
        for f, t in c.ramp:
            head += struct.pack("<QQ", int(f), int(t))
        head += struct.pack("<Q", int(info.tokens_start))
    if L > 1:
        head += b"LANE" + struct.pack("<I", L)
    if c.start_tokens is not None:
        head += b"STRT"
    if c.segment is not None and c.n_segments > 1:
        head += b"SEGS" + struct.pack("<I", c.n_segments)
    head += struct.pack("<IIQIIIIQQ", c.T, c.B, c.seed, S, c.pad_token, info.cycle, info.n_updates,
                        order_check, hash_check)
    leaves = b"".join(hashlib.sha256(records[60 * s0:60 * min(s0 + 8, S)]).digest() for s0 in range(0, S, 8))
    return hashlib.sha256(head + leaves).digest()


def _base(seed, n_sources=3, **kw):
    return random_small(seed, n_docs=kw.pop("n_docs", 400), n_sources=n_sources, T=64, B=kw.pop("B", 4),
                        max_len=120, **kw)


def _cases():
    c = _base(1)
    yield "plain", c
    yield "wrap", c.replace(wrap=True)
    yield "heldout", _base(2, bp_max=6000).replace(heldout=True)
    yield "read_random", c.replace(read_random=True)
    yield "cumulative", c.replace(cumulative=True)
    yield "ramp", _base(3, B=8).replace(ramp=((0, 4 * 64), (20 * 64, 8 * 64)))
    yield "lanes", _base(4, B=8).replace(lanes=4)
    seg = _base(5)
    yield "arrivals", seg.replace(segment=(np.arange(seg.n_docs) % 3).astype(np.uint16), n_segments=3)
    # more than 8 streams: several leaves, the last one partial
    yield "many_streams", _base(6, n_sources=37, n_docs=1500, B=40)
    yield "lanes_many_streams", _base(7, n_sources=9, n_docs=1500, B=16).replace(lanes=4, cumulative=True)
    # stream starts: go on from the tokens the first cycle reported
    r = _base(8)
    ci = oracle.Plan(r).cycle(0, updates_per_cycle=2)
    yield "stream_starts", r.replace(start_tokens=ci.stream_next.copy(), first_cycle=1,
                                     tokens_start=ci.tokens_start + ci.positions)
    yield "everything", _base(9, B=8).replace(wrap=True, read_random=True, cumulative=True, lanes=2,
                                              ramp=((0, 4 * 64), (10 * 64, 8 * 64)),
                                              segment=(np.arange(400) % 2).astype(np.uint16), n_segments=2)


@pytest.mark.parametrize("name,corpus", list(_cases()), ids=[n for n, _ in _cases()])
def test_plan_digest_layout(name, corpus):
    p = oracle.Plan(corpus)
    first = corpus.first_cycle
    for cyc in (first, first + 1):  # two cycles: the cycle number, start windows and ramp count move
        try:
            info = p.cycle(cyc, updates_per_cycle=2)
        except oracle.OracleError as e:
            assert cyc > first and e.code == oracle.OR_E_EXHAUSTED
            break
        assert info.plan_digest == rebuild(p, info), f"{name}: cycle {cyc}"


def test_plan_digest_fields_matter():
    """Every field the layout names moves the digest (a check that the rebuild
    above is not vacuous: it would also pass if a field were left out of both)."""
    c = _base(11)
    p = oracle.Plan(c)
    info = p.cycle(0, updates_per_cycle=2)
    base = rebuild(p, info)
    assert info.plan_digest == base
    for k, v in dict(seed=c.seed ^ 1, pad_token=c.pad_token + 1, holdout_bp=c.holdout_bp + np.uint32(1),
                     weight=c.weight + np.uint64(1), T=128, B=8).items():
        q = oracle.Plan(c.replace(**{k: v}))
        qi = q.cycle(0, updates_per_cycle=2)
        assert qi.plan_digest == rebuild(q, qi)
        assert qi.plan_digest != base, k
