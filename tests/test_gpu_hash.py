"""The document hash and hold-out decision on the GPU, against the oracle, on
corpora shaped to reach every path of the hash kernels (GPU).

The hash cuts the token range into tiles of 1,024 tokens, one per wavefront,
16 contiguous tokens per lane.  A tile inside one document, a tile of a few
documents, a tile of more documents than a wavefront has lanes, a lane that
crosses two or more document ends (empty documents among them), the last
partial tile, a token range that does not start at token 0 or ends before the
token buffer does, and per-source statistics with documents grouped by
source, interleaved, and with more sources than the statistics' LDS bins
hold: each corpus below takes one or more of these.  Compared bit for bit:
the per-document hash and keep arrays, and the kept and held-out counts."""
import numpy as np
import pytest

import deterministic_packing_amd as dp
import oracle
from synth.corpus import Corpus

from _gpu_parity import compare_cycle, compare_plan, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dp.load_library()
    yield
    torch.cuda.synchronize()


def _corpus(name, lengths, sources=None, lead=0, tail=0, tokens="uniform", bp=2500, seed=0):
    """Documents of the given lengths laid out from token `lead` on, `tail`
    unused tokens after the last; sources in document order (default: one)."""
    r = np.random.default_rng(seed)
    L = np.asarray(lengths, np.int64)
    D = L.shape[0]
    off = np.zeros(D + 1, np.uint64)
    np.cumsum(L, out=off[1:])
    off += np.uint64(lead)
    n = int(off[-1]) + tail
    if tokens == "max":
        tok = np.full(n, 0xFFFFFFFF, np.uint32)
    else:
        tok = r.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    src = np.zeros(D, np.uint16) if sources is None else np.asarray(sources, np.uint16)
    S = int(src.max()) + 1
    return Corpus(name, tok, off, src, np.zeros(D, np.uint16), None, np.ones(S, np.uint32),
                  np.ones(S, np.uint64), np.full(S, bp, np.uint32), T=64, B=1, updates_per_cycle=1, seed=seed,
                  pad_token=5)


def _lognormal(seed, n, median, sigma, lo, hi):
    r = np.random.default_rng(seed)
    return np.clip(np.round(r.lognormal(np.log(median), sigma, n)), lo, hi).astype(np.int64)


CASES = {
    # tiles inside one document; documents of exactly a tile and a tile + 1
    "long_documents": lambda: _corpus("long", [70000, 1024, 1025, 2048, 5000, 3000, 1023, 4097]),
    # a few documents per tile (lanes hold the tile's offsets)
    "documents_100_3000": lambda: _corpus("mid", _lognormal(1, 3000, 700, 0.8, 100, 3000), seed=1),
    # more documents in a tile than lanes (binary search), lanes crossing many ends
    "documents_0_12": lambda: _corpus("tiny", _lognormal(2, 20000, 5, 0.8, 0, 12), seed=2),
    # exactly 16, 64 documents a tile: every lane's partner is in the next document
    "documents_of_16": lambda: _corpus("d16", [16] * 3000, seed=3),
    "documents_of_17": lambda: _corpus("d17", [17] * 3000, seed=4),
    # short and empty documents among long ones, fewer than 64 a tile: lanes
    # crossing two and three document ends out of the lanes' offsets
    "short_and_empty_among_long": lambda: _corpus("mix", [3, 2, 1, 0, 0, 5, 300, 0, 1, 1, 700] * 300, seed=5),
    # token ranges: a multiple of the tile, one past, one short, not at token 0,
    # unused tokens after the last document
    "range_exact_tiles": lambda: _corpus("exact", [512] * 64, seed=6),
    "range_tile_plus_one": lambda: _corpus("plus1", [512] * 64 + [1], seed=7),
    "range_tile_minus_one": lambda: _corpus("minus1", [512] * 63 + [511], seed=8),
    "range_offset_start": lambda: _corpus("lead", _lognormal(9, 2000, 300, 1.0, 0, 2000), lead=777, tail=33, seed=9),
    "range_one_token": lambda: _corpus("one", [1], seed=10),
    # every token 2^32 - 1: the largest factors
    "tokens_all_max": lambda: _corpus("max", _lognormal(11, 1500, 200, 1.0, 1, 5000), tokens="max", seed=11),
    # statistics: sources interleaved document by document, and more sources than LDS bins
    "sources_interleaved": lambda: _corpus("inter", _lognormal(12, 4000, 50, 1.0, 0, 400),
                                           sources=np.arange(4000) % 5, seed=12),
    "sources_300": lambda: _corpus("s300", _lognormal(13, 6000, 40, 1.0, 0, 300),
                                   sources=np.random.default_rng(13).integers(0, 300, 6000), seed=13),
    "sources_grouped_all_held": lambda: _corpus("held", _lognormal(14, 3000, 400, 1.0, 1, 3000),
                                                sources=np.repeat(np.arange(3), 1000), bp=10000, seed=14),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_hash_and_hold_out_match_oracle(name):
    c = CASES[name]()
    say("hash", name, "docs", len(c.offsets) - 1, "tokens", int(c.offsets[-1] - c.offsets[0]))
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    assert np.array_equal(pk.inspect("hash"), np.asarray(op.hash, np.uint64))
    assert np.array_equal(pk.inspect("keep"), np.asarray(op.keep))
    compare_plan(pk, op)
    try:
        oi = op.cycle(0)
    except oracle.OracleError as e:  # everything held out: no stream to cut
        assert e.code == oracle.OR_E_EXHAUSTED
        with pytest.raises(dp.DpackError) as g:
            pk.cycle(0)
        assert g.value.code == dp.PACK_E_EXHAUSTED
    else:
        compare_cycle(pk.cycle(0), oi, op)
    pk.close()


def test_hash_of_one_document_is_the_pages_definition():
    """One document through the GPU equals the hash written out in Python from
    its definition (the oracle's doc_hash), independent of the plan."""
    c = CASES["long_documents"]()
    pk = dp.Packer(c)
    h = pk.inspect("hash")
    for d in range(len(c.offsets) - 1):
        assert int(h[d]) == oracle.doc_hash(c.tokens[int(c.offsets[d]):int(c.offsets[d + 1])]), d
    pk.close()
