"""CPU oracle of deterministic packing — TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it; the two share no code.

This module only marshals arguments: every step of the method is computed by
the plain sequential C in ``oracle.c`` (built here with gcc), which cites the
page and section each step follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OR_OK, OR_E_INVAL, OR_E_NOMEM, OR_E_EXHAUSTED, OR_E_STATE, OR_E_RANGE = 0, -2, -3, -5, -6, -7


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what}: error {code}")
        self.code = code


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no vectorising
    flags beyond the default)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = C.CDLL(build())
        u64, u32, i32, vp = C.c_uint64, C.c_uint32, C.c_int, C.c_void_p
        lib.or_mix64.restype = u64
        lib.or_mix64.argtypes = [u64]
        lib.or_doc_hash.restype = u64
        lib.or_doc_hash.argtypes = [vp, u64]
        lib.or_held.restype = i32
        lib.or_held.argtypes = [u64, u32]
        lib.or_philox4x32_10.restype = None
        lib.or_philox4x32_10.argtypes = [vp, vp, vp]
        lib.or_shuffle_key.restype = u64
        lib.or_shuffle_key.argtypes = [u64, u64]
        lib.or_sha256.restype = None
        lib.or_sha256.argtypes = [vp, u64, vp]
        lib.or_apportion.restype = i32
        lib.or_apportion.argtypes = [u32, u32, vp, vp]
        lib.or_slot_table.restype = i32
        lib.or_slot_table.argtypes = [u32, u32, vp, vp, vp]
        lib.or_plan_build.restype = vp
        lib.or_plan_build.argtypes = [vp, C.POINTER(C.c_int)]
        lib.or_plan_free.restype = None
        lib.or_plan_free.argtypes = [vp]
        lib.or_plan_sizes.restype = u64
        lib.or_plan_sizes.argtypes = [vp, C.POINTER(u64), C.POINTER(u64), C.POINTER(u64)]
        lib.or_plan_export.restype = None
        lib.or_plan_export.argtypes = [vp] * 19
        lib.or_cycle.restype = i32
        lib.or_cycle.argtypes = [vp, u32, u32]
        lib.or_cycle_state.restype = u32
        lib.or_cycle_state.argtypes = [vp, C.POINTER(C.c_int64), vp, vp]
        lib.or_cum_export.restype = i32
        lib.or_cum_export.argtypes = [vp, vp]
        lib.or_cumulative.restype = i32
        lib.or_cumulative.argtypes = [u32, u32, vp, vp, u64, u64, vp, C.POINTER(u64)]
        lib.or_cumulative_b.restype = i32
        lib.or_cumulative_b.argtypes = [u32, vp, u32, vp, vp, u64, u64, vp, C.POINTER(u64)]
        lib.or_cycle_batches.restype = u64
        lib.or_cycle_batches.argtypes = [vp, vp]
        lib.or_cycle_stream_next.restype = i32
        lib.or_cycle_stream_next.argtypes = [vp, vp]
        lib.or_window_of.restype = u64
        lib.or_window_of.argtypes = [vp, u64, u32]
        lib.or_emit_window.restype = None
        lib.or_emit_window.argtypes = [vp, u64, vp, vp, vp, vp]
        lib.or_window_digest.restype = None
        lib.or_window_digest.argtypes = [u32, vp, vp, vp, vp, vp]
        lib.or_window_digests_chunked.restype = i32
        lib.or_window_digests_chunked.argtypes = [u32, u64, vp, vp, vp, vp, vp]
        lib.or_batch.restype = i32
        lib.or_batch.argtypes = [vp, u32, u32, u32, u32, vp, vp, vp, vp, vp, vp]
        lib.or_batch_packed.restype = i32
        lib.or_batch_packed.argtypes = [vp, u32, u32, u32, u32, u32, vp, vp, vp, vp, vp, vp]
        lib.or_plan_digest.restype = i32
        lib.or_plan_digest.argtypes = [vp, vp]
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


# ---------------------------------------------------------------- primitives

def mix64(x: int) -> int:
    return int(_load().or_mix64(x & 0xFFFFFFFFFFFFFFFF))


def doc_hash(tokens) -> int:
    t = np.ascontiguousarray(tokens, dtype=np.uint32)
    return int(_load().or_doc_hash(_ptr(t), t.shape[0]))


def held(h: int, bp: int) -> bool:
    return bool(_load().or_held(h, bp))


def philox4x32_10(counter, key):
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def shuffle_key(seed: int, d: int) -> int:
    return int(_load().or_shuffle_key(seed, d))


def sha256(data: bytes) -> bytes:
    buf = np.frombuffer(bytes(data), dtype=np.uint8) if len(data) else np.zeros(1, np.uint8)
    out = np.zeros(32, dtype=np.uint8)
    _load().or_sha256(_ptr(buf), len(data), _ptr(out))
    return out.tobytes()


def apportion(B: int, weights) -> np.ndarray:
    w = np.ascontiguousarray(weights, dtype=np.uint64)
    n = np.zeros(w.shape[0], dtype=np.uint32)
    rc = _load().or_apportion(B, w.shape[0], _ptr(w), _ptr(n))
    if rc:
        raise OracleError(rc, "apportion")
    return n


def cumulative(B: int, weights, remaining, updates: int = 0, cap: Optional[int] = None, batches=None):
    """C6c on its own: (U, A [U+1, S]) for B windows per update (or
    batches[u] windows in update u), integer weights and each source's
    remaining windows; updates = 0 takes the most that fit."""
    w = np.ascontiguousarray(weights, np.uint64)
    rem = np.ascontiguousarray(remaining, np.uint64)
    S = w.shape[0]
    if batches is not None:
        bs = np.ascontiguousarray(batches, np.uint32)
        cap = bs.shape[0] if cap is None else cap
        assert bs.shape[0] >= cap
    elif cap is None:
        cap = updates if updates else int(rem.sum()) // B
    A = np.zeros((cap + 1, S), np.uint32)
    U = C.c_uint64()
    if batches is not None:
        rc = _load().or_cumulative_b(B, _ptr(bs), S, _ptr(w), _ptr(rem), updates, cap, _ptr(A), C.byref(U))
    else:
        rc = _load().or_cumulative(B, S, _ptr(w), _ptr(rem), updates, cap, _ptr(A), C.byref(U))
    if rc:
        raise OracleError(rc, "cumulative")
    return int(U.value), A[:U.value + 1].copy()


def slot_table(B: int, n) -> tuple:
    n = np.ascontiguousarray(n, dtype=np.uint32)
    ss = np.zeros(B, dtype=np.uint32)
    sk = np.zeros(B, dtype=np.uint32)
    rc = _load().or_slot_table(B, n.shape[0], _ptr(n), _ptr(ss), _ptr(sk))
    if rc:
        raise OracleError(rc, "slot_table")
    return ss, sk


def window_digest(tok, pos, doc, mask) -> bytes:
    T = tok.shape[-1]
    out = np.zeros(32, dtype=np.uint8)
    tok = np.ascontiguousarray(tok, np.uint32)
    pos = np.ascontiguousarray(pos, np.int32)
    doc = np.ascontiguousarray(doc, np.int32)
    mask = np.ascontiguousarray(mask, np.uint8)
    _load().or_window_digest(T, _ptr(tok), _ptr(pos), _ptr(doc), _ptr(mask), _ptr(out))
    return out.tobytes()


def window_digests_chunked(tok, pos, doc, mask) -> np.ndarray:
    """Chunked window digests of windows laid out [..., T]: [..., 32]."""
    T = tok.shape[-1]
    lead = tok.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    out = np.zeros(lead + (32,), dtype=np.uint8)
    tok = np.ascontiguousarray(tok, np.uint32)
    pos = np.ascontiguousarray(pos, np.int32)
    doc = np.ascontiguousarray(doc, np.int32)
    mask = np.ascontiguousarray(mask, np.uint8)
    rc = _load().or_window_digests_chunked(T, n, _ptr(tok), _ptr(pos), _ptr(doc), _ptr(mask), _ptr(out))
    if rc:
        raise OracleError(rc, "window_digests_chunked")
    return out


def batch_fingerprint(window_digests: np.ndarray) -> bytes:
    """SHA-256 over the B window digests of one global batch, in slot order."""
    d = np.ascontiguousarray(window_digests, dtype=np.uint8).reshape(-1)
    return sha256(d.tobytes())


# ---------------------------------------------------------------- the plan

class _OrCorpus(C.Structure):
    _fields_ = [
        ("tokens", C.c_void_p), ("n_tokens", C.c_uint64),
        ("offsets", C.c_void_p), ("n_docs", C.c_uint64),
        ("source", C.c_void_p), ("stratum", C.c_void_p), ("prompt_len", C.c_void_p),
        ("n_sources", C.c_uint32), ("n_strata", C.c_void_p), ("weight", C.c_void_p),
        ("bp", C.c_void_p), ("T", C.c_uint32), ("B", C.c_uint32), ("seed", C.c_uint64),
        ("pad_token", C.c_uint32), ("wrap", C.c_uint32), ("heldout", C.c_uint32), ("read_random", C.c_uint32),
        ("cumulative", C.c_uint32),
        ("n_ramp", C.c_uint32), ("ramp_from", C.c_void_p), ("ramp_tokens", C.c_void_p),
        ("lanes", C.c_uint32), ("start_tokens", C.c_void_p), ("first_cycle", C.c_uint32),
        ("tokens_start", C.c_uint64), ("segment", C.c_void_p), ("n_segments", C.c_uint32),
    ]


@dataclass
class CycleInfo:
    cycle: int
    n_updates: int
    start: np.ndarray        # [S] first window of the cycle in each source's stream
    taken: np.ndarray        # [S] windows the cycle takes from each source
    remaining: np.ndarray    # [S] windows left after the cycle
    real_tokens: int
    learned_tokens: int
    positions: int
    plan_digest: bytes
    batches: np.ndarray = None     # [U] windows of each update (B, or the ramp's batch)
    tokens_start: int = 0          # tokens trained before the cycle
    stream_next: np.ndarray = None # [streams] token where each stream's next cycle starts


class Plan:
    """The oracle's plan of one corpus (hash, hold-out, shuffle, strata merge,
    pieces, next-fit or wrap windows, apportionment, slot table), plus cycle
    state."""

    def __init__(self, corpus):
        lib = _load()
        c = corpus
        self.corpus = c
        self._keep = dict(
            tokens=np.ascontiguousarray(c.tokens, np.uint32),
            offsets=np.ascontiguousarray(c.offsets, np.uint64),
            source=np.ascontiguousarray(c.source, np.uint16),
            stratum=np.ascontiguousarray(c.stratum, np.uint16),
            prompt_len=None if c.prompt_len is None else np.ascontiguousarray(c.prompt_len, np.uint32),
            n_strata=np.ascontiguousarray(c.n_strata, np.uint32),
            weight=np.ascontiguousarray(c.weight, np.uint64),
            bp=np.ascontiguousarray(c.holdout_bp, np.uint32),
            ramp_from=None if getattr(c, "ramp", None) is None else
            np.ascontiguousarray([int(f) for f, _ in c.ramp], np.uint64),
            ramp_tokens=None if getattr(c, "ramp", None) is None else
            np.ascontiguousarray([int(t) for _, t in c.ramp], np.uint64),
            start_tokens=None if getattr(c, "start_tokens", None) is None else
            np.ascontiguousarray(c.start_tokens, np.uint64),
            segment=None if getattr(c, "segment", None) is None else np.ascontiguousarray(c.segment, np.uint16),
        )
        k = self._keep
        D, S = k["source"].shape[0], k["weight"].shape[0]
        self.lanes = max(1, int(getattr(c, "lanes", 1) or 1))
        if k["offsets"].shape[0] != D + 1 or np.any(np.diff(k["offsets"].astype(np.int64)) < 0):
            raise OracleError(OR_E_INVAL, "offsets")
        if D and (int(k["source"].max()) >= S or np.any(k["stratum"] >= k["n_strata"][k["source"]])):
            raise OracleError(OR_E_INVAL, "source/stratum ids")
        if int(k["offsets"][-1]) > k["tokens"].shape[0]:
            raise OracleError(OR_E_INVAL, "offsets beyond tokens")
        self._cs = _OrCorpus(
            _ptr(k["tokens"]) if k["tokens"].shape[0] else None, k["tokens"].shape[0],
            _ptr(k["offsets"]), D, _ptr(k["source"]) if D else None, _ptr(k["stratum"]) if D else None,
            _ptr(k["prompt_len"]), S, _ptr(k["n_strata"]), _ptr(k["weight"]), _ptr(k["bp"]),
            c.T, c.B, c.seed & 0xFFFFFFFFFFFFFFFF, c.pad_token, 1 if getattr(c, "wrap", False) else 0,
            1 if getattr(c, "heldout", False) else 0, 1 if getattr(c, "read_random", False) else 0,
            1 if getattr(c, "cumulative", False) else 0,
            0 if k["ramp_from"] is None else k["ramp_from"].shape[0], _ptr(k["ramp_from"]), _ptr(k["ramp_tokens"]),
            self.lanes, _ptr(k["start_tokens"]), int(getattr(c, "first_cycle", 0)),
            int(getattr(c, "tokens_start", 0)), _ptr(k["segment"]), int(getattr(c, "n_segments", 1) or 1))
        err = C.c_int(0)
        self._p = lib.or_plan_build(C.byref(self._cs), C.byref(err))
        if not self._p:
            raise OracleError(err.value, "plan")
        nk, npc, nw = C.c_uint64(), C.c_uint64(), C.c_uint64()
        lib.or_plan_sizes(self._p, C.byref(nk), C.byref(npc), C.byref(nw))
        nk, npc, nw = nk.value, npc.value, nw.value
        S = S * self.lanes  # with lanes every per-source array is per stream (source s, lane l) = s·L + l
        self.hash = np.zeros(D, np.uint64)
        self.keep = np.zeros(D, np.uint8)
        self.order = np.zeros(nk, np.uint32)
        self.src_doc_start = np.zeros(S + 1, np.uint64)
        self.piece_doc = np.zeros(npc, np.uint32)
        self.piece_off = np.zeros(npc, np.uint32)
        self.piece_len = np.zeros(npc, np.uint32)
        self.piece_woff = np.zeros(npc, np.uint32)
        self.src_piece_start = np.zeros(S + 1, np.uint64)
        self.win_first = np.zeros(nw + 1, np.uint64)
        self.src_win_start = np.zeros(S + 1, np.uint64)
        self.win_real = np.zeros(nw, np.uint64)
        self.win_learn = np.zeros(nw, np.uint64)
        self.n_per_update = np.zeros(S, np.uint32)
        self.slot_src = np.zeros(c.B, np.uint32)
        self.slot_k = np.zeros(c.B, np.uint32)
        stats = np.zeros((4, S), np.uint64)
        checks = np.zeros(2, np.uint64)
        lib.or_plan_export(self._p, *[_ptr(a) for a in (
            self.hash, self.keep, self.order, self.src_doc_start, self.piece_doc, self.piece_off,
            self.piece_len, self.piece_woff, self.src_piece_start, self.win_first, self.src_win_start,
            self.win_real, self.win_learn, self.n_per_update, self.slot_src, self.slot_k, stats, checks)])
        self.kept_docs, self.kept_tokens, self.held_docs, self.held_tokens = stats
        self.order_check, self.hash_check = int(checks[0]), int(checks[1])
        self.windows_per_source = np.diff(self.src_win_start)
        self.cycle_info: Optional[CycleInfo] = None

    def __del__(self):
        if getattr(self, "_p", None):
            _load().or_plan_free(self._p)
            self._p = None

    @property
    def n_windows(self) -> int:
        return int(self.win_first.shape[0] - 1)

    def cycle(self, c: int, updates_per_cycle: Optional[int] = None) -> CycleInfo:
        lib = _load()
        U_cfg = self.corpus.updates_per_cycle if updates_per_cycle is None else updates_per_cycle
        rc = lib.or_cycle(self._p, c, U_cfg)
        if rc:
            raise OracleError(rc, "cycle")
        S = self.corpus.n_sources * self.lanes
        start = np.zeros(S, np.uint64)
        cyc = C.c_int64()
        taken = np.zeros(S, np.uint64)
        U = int(lib.or_cycle_state(self._p, C.byref(cyc), _ptr(start), _ptr(taken)))
        remaining = self.windows_per_source - start - taken
        batches = np.zeros(max(U, 1), np.uint32)
        t0 = int(lib.or_cycle_batches(self._p, _ptr(batches)))
        batches = batches[:U]
        nslots = int(batches.sum())
        wins = [self.window_of(b, j) for b in range(U) for j in range(int(batches[b]))] if nslots <= 2_000_000 else None
        if wins is not None:
            wins = np.asarray(wins, dtype=np.int64)
            real = int(self.win_real[wins].sum()) if wins.size else 0
            learned = int(self.win_learn[wins].sum()) if wins.size else 0
        else:
            real = learned = -1
        dig = np.zeros(32, np.uint8)
        rc = lib.or_plan_digest(self._p, _ptr(dig))
        if rc:
            raise OracleError(rc, "plan_digest")
        nxt = np.zeros(S, np.uint64)
        rc = lib.or_cycle_stream_next(self._p, _ptr(nxt))
        if rc:
            raise OracleError(rc, "stream_next")
        self.cycle_info = CycleInfo(c, U, start, taken, remaining, real, learned,
                                    nslots * self.corpus.T, dig.tobytes(), batches, t0, nxt)
        return self.cycle_info

    def cumulative_taken(self) -> np.ndarray:
        """With the cumulative mixture: A [U+1, S], windows of each source taken
        before each update of the current cycle (row U: the cycle's totals)."""
        S = self.corpus.n_sources * self.lanes
        A = np.zeros((self.cycle_info.n_updates + 1, S), np.uint32)
        rc = _load().or_cum_export(self._p, _ptr(A))
        if rc:
            raise OracleError(rc, "cum_export")
        return A

    def window_of(self, b: int, j: int) -> int:
        return int(_load().or_window_of(self._p, b, j))

    def emit_window(self, gw: int):
        T = self.corpus.T
        tok = np.zeros(T, np.uint32)
        pos = np.zeros(T, np.int32)
        doc = np.zeros(T, np.int32)
        mask = np.zeros(T, np.uint8)
        _load().or_emit_window(self._p, gw, _ptr(tok), _ptr(pos), _ptr(doc), _ptr(mask))
        return tok, pos, doc, mask

    def batch(self, step: int, n_steps: int = 1, rank: int = 0, world: int = 1,
              digests: bool = True, learned: bool = True) -> dict:
        """This rank's windows of updates [step, step+n_steps): [n, B/world, T]
        arrays, or with a batch-size ramp [Σ B_b/world, T] (update after update)."""
        B, T = self.corpus.B, self.corpus.T
        if world <= 0 or B % world:
            raise OracleError(OR_E_INVAL, "batch world")
        ramp = getattr(self.corpus, "ramp", None) is not None
        if ramp:
            bs = self.cycle_info.batches[step:step + n_steps]
            if len(bs) != n_steps:
                raise OracleError(OR_E_RANGE, "batch range")
            shape = (int(bs.sum()) // world,)
        else:
            shape = (n_steps, B // world)
        tok = np.zeros(shape + (T,), np.uint32)
        pos = np.zeros(shape + (T,), np.int32)
        doc = np.zeros(shape + (T,), np.int32)
        mask = np.zeros(shape + (T,), np.uint8)
        lrn = np.zeros(n_steps, np.int64) if learned else None
        dig = np.zeros(shape + (32,), np.uint8) if digests else None
        chunked = digests and getattr(self.corpus, "digest_chunked", False)
        rc = _load().or_batch(self._p, step, n_steps, rank, world, _ptr(tok), _ptr(pos), _ptr(doc),
                              _ptr(mask), _ptr(lrn), _ptr(None if chunked else dig))
        if rc:
            raise OracleError(rc, "batch")
        if chunked:  # the same records, digested chunk by chunk
            dig = window_digests_chunked(tok, pos, doc, mask)
        return dict(tokens=tok, pos=pos, doc=doc, mask=mask, learned=lrn, digests=dig)

    def batch_packed(self, step: int, n_steps: int = 1, rank: int = 0, world: int = 1, bucket: int = 256) -> dict:
        """Padding-free rows: one packed row per update of this rank's windows'
        real positions, its length rounded up to a multiple of bucket."""
        B, T = self.corpus.B, self.corpus.T
        if world <= 0 or B % world:
            raise OracleError(OR_E_INVAL, "batch world")
        per = B // world
        tok = np.zeros((n_steps, per * T), np.uint32)
        pos = np.zeros((n_steps, per * T), np.int32)
        doc = np.zeros((n_steps, per * T), np.int32)
        mask = np.zeros((n_steps, per * T), np.uint8)
        row_start = np.zeros((n_steps, per + 1), np.int64)
        length = np.zeros(n_steps, np.int64)
        rc = _load().or_batch_packed(self._p, step, n_steps, rank, world, bucket, _ptr(tok), _ptr(pos), _ptr(doc),
                                     _ptr(mask), _ptr(row_start), _ptr(length))
        if rc:
            raise OracleError(rc, "batch_packed")
        return dict(tokens=tok, pos=pos, doc=doc, mask=mask, row_start=row_start, length=length)
