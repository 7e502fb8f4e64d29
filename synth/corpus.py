"""Seeded synthetic corpora with the shapes of the packing workloads.

The pages measure on corpora that are not available here (MiniCPM data lines,
InfLLM-V2, Alpaca, FineWeb/DCLM evaluation sets).  These generators stand in
for them: they reproduce the number of documents, the length laws, the token
value laws, the source/stratum structure and the recipe of each workload, with
every draw seeded so that the same call always returns the same bytes.

Documents are laid out by (source, stratum), then in generation order.  Shares
are turned into integer weights here (round(share * 1e9)), so the packing code
never sees a float.

Nothing in this module packs, hashes, shuffles or apportions windows: it only
draws inputs.  Doc counts per source/stratum are split with a plain
floor-then-first-come rule that is unrelated to the packer's own
apportionment.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

WEIGHT_SCALE = 10**9  # share -> integer weight


@dataclasses.dataclass
class Corpus:
    """A corpus plus the recipe and packing parameters of one workload."""

    name: str
    tokens: np.ndarray          # uint32 [N]
    offsets: np.ndarray         # uint64 [D+1], offsets[0] == 0, monotone
    source: np.ndarray          # uint16 [D]
    stratum: np.ndarray         # uint16 [D]
    prompt_len: Optional[np.ndarray]  # uint32 [D] or None (pre-training)
    n_strata: np.ndarray        # uint32 [S]
    weight: np.ndarray          # uint64 [S] integer share weights
    holdout_bp: np.ndarray      # uint32 [S] hold-out rate in basis points
    T: int                      # window length in positions
    B: int                      # windows per update (global batch)
    updates_per_cycle: int      # 0 = as many as the data support
    seed: int = 0
    pad_token: int = 0
    meta: Dict = dataclasses.field(default_factory=dict)
    wrap: bool = False          # packing: False = next-fit cut at document ends, True = wrap
    heldout: bool = False       # stream: False = training documents, True = held-out (validation)
    read_random: bool = False   # each cycle's windows of a source read in a random order
    cumulative: bool = False    # per-update counts from the cycle's cumulative quotas
    ramp: Optional[Tuple[Tuple[int, int], ...]] = None  # batch-size ramp: ((from_tokens, tokens_per_update), ...)
    lanes: int = 1              # Zephon lanes: document d in lane d mod lanes
    start_tokens: Optional[np.ndarray] = None  # per stream: first token to cut (a resumed or re-cut stream)
    first_cycle: int = 0        # number of the first cycle planned
    tokens_start: int = 0       # tokens trained before the first cycle
    segment: Optional[np.ndarray] = None  # per document: the arrival it came with (streamed corpora)
    n_segments: int = 1         # arrivals
    digest_chunked: bool = False  # window digests chunk by chunk (4,096-byte chunks of the record)

    @property
    def n_docs(self) -> int:
        return int(self.source.shape[0])

    @property
    def n_sources(self) -> int:
        return int(self.weight.shape[0])

    @property
    def n_tokens(self) -> int:
        return int(self.tokens.shape[0])

    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets).astype(np.int64)

    def replace(self, **kw) -> "Corpus":
        return dataclasses.replace(self, **kw)


def recipe_from_shares(shares) -> np.ndarray:
    """Integer weights round(share * 1e9), at least 1 for a positive share."""
    w = [max(1, int(round(float(s) * WEIGHT_SCALE))) if s > 0 else 0 for s in shares]
    return np.asarray(w, dtype=np.uint64)


def _split_counts(total: int, ratios) -> np.ndarray:
    """Split `total` items by `ratios`: floors, then the leftover one each to the
    first entries.  Generator bookkeeping only."""
    r = np.asarray(ratios, dtype=np.float64)
    r = r / r.sum()
    c = np.floor(total * r).astype(np.int64)
    left = total - int(c.sum())
    i = 0
    while left > 0:
        c[i % len(c)] += 1
        left -= 1
        i += 1
    return c


def _rng(cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, stream]))


_CHUNK = 1 << 22  # fixed chunk of token draws: the byte stream never depends on memory size


def _uniform_tokens(rng: np.random.Generator, n: int, vocab: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = rng.integers(0, vocab, size=hi - lo, dtype=np.uint32)
    return out


_ZIPF_TABLE_BITS = 20


def _zipf_quantile_table(vocab: int, s: float) -> np.ndarray:
    """Token id for each of 2^20 equal-probability cells of P(k) ∝ (k+1)^-s:
    cell c holds the id whose CDF interval contains the cell's midpoint."""
    k = np.arange(vocab, dtype=np.float64)
    p = (k + 1.0) ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    n = 1 << _ZIPF_TABLE_BITS
    # number of cell midpoints (c + 0.5) / n below each cdf value
    below = np.floor(cdf * n - 0.5).astype(np.int64) + 1
    below = np.clip(below, 0, n)
    below[-1] = n
    counts = np.diff(np.concatenate([[0], below]))
    return np.repeat(np.arange(vocab, dtype=np.uint32), counts)


_ZIPF_CACHE: Dict = {}


def _zipf_tokens(rng: np.random.Generator, n: int, vocab: int, s: float) -> np.ndarray:
    key = (vocab, s)
    if key not in _ZIPF_CACHE:
        _ZIPF_CACHE[key] = _zipf_quantile_table(vocab, s)
    table = _ZIPF_CACHE[key]
    out = np.empty(n, dtype=np.uint32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        cell = rng.integers(0, 1 << _ZIPF_TABLE_BITS, size=hi - lo, dtype=np.uint32)
        out[lo:hi] = table[cell]
    return out


def _lognormal_lengths(rng, n, median, sigma, lo, hi) -> np.ndarray:
    z = rng.standard_normal(n)
    L = np.rint(np.exp(math.log(median) + sigma * z))
    return np.clip(L, lo, hi).astype(np.int64)


def _layout(doc_counts_per_group, n_strata, lengths):
    """source/stratum arrays for docs laid out group by group."""
    src, strat = [], []
    g = 0
    for s, K in enumerate(n_strata):
        for k in range(K):
            c = int(doc_counts_per_group[g])
            src.append(np.full(c, s, dtype=np.uint16))
            strat.append(np.full(c, k, dtype=np.uint16))
            g += 1
    source = np.concatenate(src) if src else np.zeros(0, np.uint16)
    stratum = np.concatenate(strat) if strat else np.zeros(0, np.uint16)
    assert source.shape[0] == lengths.shape[0]
    offsets = np.zeros(lengths.shape[0] + 1, dtype=np.uint64)
    np.cumsum(lengths, out=offsets[1:])
    return source, stratum, offsets


def _group_counts(n_docs, source_ratios, strata_ratios):
    per_src = _split_counts(n_docs, source_ratios)
    out = []
    for c in per_src:
        out.extend(_split_counts(int(c), strata_ratios).tolist())
    return np.asarray(out, dtype=np.int64)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def _tiny(scale: float) -> Corpus:
    cfg = 1
    per_src = max(1, int(round(2000 * scale)))
    n = 2 * per_src
    L = _rng(cfg, 0).geometric(1.0 / 300.0, size=n).astype(np.int64)
    L = np.clip(L, 1, 4096)
    source, stratum, offsets = _layout([per_src, per_src], [1, 1], L)
    tokens = _uniform_tokens(_rng(cfg, 1), int(offsets[-1]), 32000)
    return Corpus("tiny", tokens, offsets, source, stratum, None,
                  np.array([1, 1], np.uint32), recipe_from_shares([0.7, 0.3]),
                  np.array([100, 100], np.uint32), T=2048, B=8, updates_per_cycle=0,
                  meta=dict(lengths="geometric p=1/300 clip [1,4096]", vocab=32000,
                            token_law="uniform", shares=[0.7, 0.3]))


def _pretrain_like(cfg, n_docs, n_strata_each, strata_ratios, T, B, U, name, target_tokens=None):
    S = 15
    src_ratios = [1.0 / (s + 1) for s in range(S)]
    rng_len = _rng(cfg, 0)
    if target_tokens is None:
        L = _lognormal_lengths(rng_len, n_docs, 600.0, 1.2, 1, 65536)
    else:
        # draw docs until the running total reaches the target; truncate the last
        parts, total = [], 0
        while total < target_tokens:
            chunk = _lognormal_lengths(rng_len, 1 << 20, 600.0, 1.2, 1, 65536)
            cs = np.cumsum(chunk)
            need = target_tokens - total
            if cs[-1] >= need:
                k = int(np.searchsorted(cs, need, side="left"))
                chunk = chunk[: k + 1].copy()
                chunk[-1] -= int(cs[k] - need)
                parts.append(chunk)
                total = target_tokens
            else:
                parts.append(chunk)
                total += int(cs[-1])
        L = np.concatenate(parts)
        L = L[L > 0]
        n_docs = int(L.shape[0])
    counts = _group_counts(n_docs, src_ratios, strata_ratios)
    n_strata = np.full(S, n_strata_each, dtype=np.uint32)
    source, stratum, offsets = _layout(counts, n_strata, L)
    tokens = _zipf_tokens(_rng(cfg, 1), int(offsets[-1]), 65536, 1.1)
    shares = np.asarray(src_ratios) / np.sum(src_ratios)
    bp = np.full(S, 100, dtype=np.uint32)
    bp[S - 1] = 500
    return Corpus(name, tokens, offsets, source, stratum, None, n_strata,
                  recipe_from_shares(shares), bp, T=T, B=B, updates_per_cycle=U,
                  meta=dict(lengths="lognormal median 600 sigma 1.2 clip [1,65536]",
                            vocab=65536, token_law="zipf s=1.1 (2^20-cell quantile table)",
                            shares=shares.tolist(), strata_ratios=list(strata_ratios)))


def _pretrain(scale: float) -> Corpus:
    n = max(60, int(round(1_000_000 * scale)))
    return _pretrain_like(2, n, 4, [4, 3, 2, 1], 4096, 256, 200, "pretrain")


def _sft(scale: float) -> Corpus:
    cfg = 3
    n = max(1, int(round(500_000 * scale)))
    r = _rng(cfg, 0)
    prompt = _lognormal_lengths(r, n, 200.0, 1.0, 1, 2048)
    comp = np.rint(np.exp(math.log(300.0) + 1.0 * r.standard_normal(n)))
    comp = np.clip(comp, 1, 4096 - prompt).astype(np.int64)
    L = prompt + comp
    source, stratum, offsets = _layout([n], [1], L)
    tokens = _uniform_tokens(_rng(cfg, 1), int(offsets[-1]), 128256)
    return Corpus("sft", tokens, offsets, source, stratum, prompt.astype(np.uint32),
                  np.array([1], np.uint32), np.array([WEIGHT_SCALE], np.uint64),
                  np.array([0], np.uint32), T=4096, B=8, updates_per_cycle=0,
                  meta=dict(prompt="lognormal median 200 sigma 1.0 clip [1,2048]",
                            completion="lognormal median 300 sigma 1.0 clip [1,4096-prompt]",
                            vocab=128256, token_law="uniform"))


def _long(scale: float) -> Corpus:
    cfg = 4
    S = 8
    n = max(S, int(round(200_000 * scale)))
    shares = _rng(cfg, 3).dirichlet(np.ones(S))
    counts = _split_counts(n, shares)
    u = _rng(cfg, 0).random(n)
    a, lo, hi = 1.3, 1000.0, 200000.0
    L = np.floor(lo / (1.0 - u * (1.0 - (lo / hi) ** a)) ** (1.0 / a))
    L = np.clip(L, lo, hi).astype(np.int64)
    source, stratum, offsets = _layout(counts, [1] * S, L)
    tokens = _uniform_tokens(_rng(cfg, 1), int(offsets[-1]), 65536)
    return Corpus("long", tokens, offsets, source, stratum, None,
                  np.ones(S, np.uint32), recipe_from_shares(shares),
                  np.full(S, 100, np.uint32), T=32768, B=32, updates_per_cycle=0,
                  meta=dict(lengths="bounded pareto alpha 1.3 on [1000,200000]",
                            vocab=65536, token_law="uniform", shares=shares.tolist()))


def _full(scale: float) -> Corpus:
    target = max(1 << 20, int(round(2_000_000_000 * scale)))
    return _pretrain_like(5, 0, 8, list(range(8, 0, -1)), 4096, 1024, 0, "full",
                          target_tokens=target)


CONFIGS = {
    "tiny": _tiny,
    "pretrain": _pretrain,
    "sft": _sft,
    "long": _long,
    "full": _full,
}


def make_corpus(name: str, scale: float = 1.0, **overrides) -> Corpus:
    """Build one of the five workloads, optionally scaled down in documents
    (or tokens, for "full") and with recipe/packing fields overridden."""
    c = CONFIGS[name](scale)
    c.meta["scale"] = scale
    if overrides:
        c = c.replace(**overrides)
    return c


def random_small(seed: int, n_docs: int = 40, n_sources: int = 3, max_strata: int = 3,
                 T: int = 64, B: int = 4, max_len: int = 150, vocab: int = 1000,
                 prompts: bool = False, bp_max: int = 3000, zero_len_frac: float = 0.05,
                 updates_per_cycle: int = 0) -> Corpus:
    """Small random corpus for brute-force comparisons: mixed lengths (some
    zero, some longer than T), random strata counts, random recipe."""
    r = np.random.default_rng(np.random.SeedSequence([1000, seed]))
    S = n_sources
    n_strata = r.integers(1, max_strata + 1, size=S).astype(np.uint32)
    G = int(n_strata.sum())
    g_of_doc = np.sort(r.integers(0, G, size=n_docs))
    counts = np.bincount(g_of_doc, minlength=G)
    L = r.integers(1, max_len + 1, size=n_docs).astype(np.int64)
    L[r.random(n_docs) < zero_len_frac] = 0
    source, stratum, offsets = _layout(counts, n_strata, L)
    tokens = r.integers(0, vocab, size=int(offsets[-1]), dtype=np.uint32)
    prompt_len = None
    if prompts:
        prompt_len = np.minimum(r.integers(0, max_len + 1, size=n_docs), L + r.integers(0, 3, size=n_docs)).astype(np.uint32)
    w = r.integers(1, 1000, size=S).astype(np.uint64)
    bp = r.integers(0, bp_max + 1, size=S).astype(np.uint32)
    return Corpus(f"small{seed}", tokens, offsets, source, stratum, prompt_len, n_strata,
                  w, bp, T=T, B=B, updates_per_cycle=updates_per_cycle,
                  seed=int(r.integers(0, 2**63)), pad_token=int(r.integers(0, vocab)),
                  meta=dict(kind="random_small"))
