"""Deterministic, elastically reproducible packing on MI355X — Python binding.

A thin ctypes layer over the C ABI in ``include/dpack.h`` (libdpack.so, built
from ``csrc/`` with hipcc for gfx950).  Functions keep the C names
(``pack_init``, ``pack_cycle``, ``pack_batch``, ``pack_fingerprint``,
``pack_inspect``, ``pack_destroy``); :class:`Packer` bundles them with torch
device tensors.  Only argument marshalling happens here: every step of the
path runs in the library's HIP kernels.  There is no CPU fallback — when the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

__all__ = [
    "DpackError", "load_library", "pack_init", "pack_init_noalloc", "pack_cycle", "pack_batch", "pack_batch_packed", "pack_fingerprint",
    "pack_fingerprint_steps", "pack_inspect", "pack_get_timings", "pack_status", "pack_test_option", "pack_destroy",
    "pack_strerror", "Packer", "INSPECT", "SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdpack.so")
ABI_VERSION = 2

PACK_OK, PACK_E_ABI, PACK_E_INVAL, PACK_E_NOMEM, PACK_E_HIP = 0, -1, -2, -3, -4
PACK_E_EXHAUSTED, PACK_E_STATE, PACK_E_RANGE, PACK_E_INTERNAL = -5, -6, -7, -8
PACK_TEST_WAIT_GIVE_UP, PACK_TEST_CYCLE_FAULT, PACK_TEST_SORT_INSERTION, PACK_TEST_DIGEST_SLICES = 1, 2, 3, 4

SYMBOLS = ("pack_init", "pack_init_noalloc", "pack_cycle", "pack_batch", "pack_batch_packed", "pack_fingerprint",
           "pack_fingerprint_steps", "pack_inspect", "pack_get_timings", "pack_status", "pack_test_option",
           "pack_destroy", "pack_strerror", "pack_last_error")

PACK_FLAG_TIMING = 1
PACK_FLAG_WRAP = 2
PACK_FLAG_HELDOUT = 4
PACK_FLAG_READ_RANDOM = 8
PACK_FLAG_CUMULATIVE = 16
PACK_FLAG_TIMING_BATCH = 32
PACK_FLAG_DIGEST_CHUNKED = 64
PHASES = ("validate", "hash", "keys", "sort", "merge", "pieces", "cut", "windows", "mixture",
          "cycle", "emit", "learned", "digest", "fingerprint")

# what -> (numpy dtype, length key)
INSPECT = {
    "hash": (1, np.uint64), "keep": (2, np.uint8), "order": (3, np.uint32),
    "src_doc_start": (4, np.uint64), "piece_doc": (5, np.uint32), "piece_off": (6, np.uint32),
    "piece_len": (7, np.uint32), "piece_woff": (8, np.uint32), "src_piece_start": (9, np.uint64),
    "win_first": (10, np.uint64), "src_win_start": (11, np.uint64), "win_real": (12, np.uint64),
    "win_learn": (13, np.uint64), "per_update": (14, np.uint32), "slot_src": (15, np.uint32),
    "slot_k": (16, np.uint32), "counts": (17, np.uint64),
    "cum_taken": (18, np.uint32), "update_batch": (19, np.uint32),
}


class DpackError(RuntimeError):
    def __init__(self, code: int, call: str, msg: str = ""):
        super().__init__(f"{call} failed: {code} ({_strerror(code)}){': ' + msg if msg else ''}")
        self.code = code


class PackConfig(C.Structure):
    _fields_ = [
        ("abi_version", C.c_uint32), ("flags", C.c_uint32),
        ("tokens", C.c_void_p), ("n_tokens", C.c_uint64),
        ("doc_offsets", C.c_void_p), ("n_docs", C.c_uint64),
        ("doc_source", C.c_void_p), ("doc_stratum", C.c_void_p), ("doc_prompt_len", C.c_void_p),
        ("n_sources", C.c_uint32), ("n_strata", C.c_void_p), ("share_weight", C.c_void_p),
        ("holdout_bp", C.c_void_p), ("window_tokens", C.c_uint32), ("global_batch", C.c_uint32),
        ("updates_per_cycle", C.c_uint32), ("pad_token", C.c_uint32), ("seed", C.c_uint64),
        ("rank", C.c_uint32), ("world", C.c_uint32), ("stream", C.c_void_p),
        ("n_ramp", C.c_uint32), ("ramp_from", C.c_void_p), ("ramp_tokens", C.c_void_p),
        ("n_lanes", C.c_uint32), ("start_tokens", C.c_void_p), ("first_cycle", C.c_uint32),
        ("tokens_start", C.c_uint64), ("doc_segment", C.c_void_p), ("n_segments", C.c_uint32),
    ]


class PackCycleInfo(C.Structure):
    _fields_ = [
        ("cycle", C.c_uint32), ("n_updates", C.c_uint32), ("real_tokens", C.c_uint64),
        ("learned_tokens", C.c_uint64), ("positions", C.c_uint64), ("plan_digest", C.c_uint8 * 32),
        ("windows_start", C.c_void_p), ("windows_taken", C.c_void_p), ("windows_remaining", C.c_void_p),
        ("kept_docs", C.c_void_p), ("kept_tokens", C.c_void_p), ("held_docs", C.c_void_p),
        ("held_tokens", C.c_void_p), ("per_update", C.c_void_p), ("stream_next_token", C.c_void_p),
    ]


class PackTimings(C.Structure):
    _fields_ = [("ms", C.c_double * len(PHASES)), ("calls", C.c_uint64 * len(PHASES))]


class PackOut(C.Structure):
    _fields_ = [
        ("tokens", C.c_void_p), ("pos", C.c_void_p), ("doc", C.c_void_p), ("mask", C.c_void_p),
        ("learned", C.c_void_p), ("digests", C.c_void_p),
    ]


class PackOutPacked(C.Structure):
    _fields_ = [
        ("tokens", C.c_void_p), ("pos", C.c_void_p), ("doc", C.c_void_p), ("mask", C.c_void_p),
        ("row_start", C.c_void_p), ("length", C.c_void_p), ("learned", C.c_void_p), ("bucket", C.c_uint32),
    ]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libdpack.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libdpack.so not found at {p}: build it with "
                           "`python -m deterministic_packing_amd.build` (hipcc, gfx950)")
    lib = C.CDLL(p)
    vp, i32, u32 = C.c_void_p, C.c_int, C.c_uint32
    lib.pack_init.restype = i32
    lib.pack_init.argtypes = [C.POINTER(PackConfig), C.POINTER(vp)]
    lib.pack_init_noalloc.restype = i32
    lib.pack_init_noalloc.argtypes = [C.POINTER(PackConfig), C.POINTER(vp)]
    lib.pack_cycle.restype = i32
    lib.pack_cycle.argtypes = [vp, u32, C.POINTER(PackCycleInfo)]
    lib.pack_batch.restype = i32
    lib.pack_batch.argtypes = [vp, u32, u32, C.POINTER(PackOut)]
    lib.pack_batch_packed.restype = i32
    lib.pack_batch_packed.argtypes = [vp, u32, u32, C.POINTER(PackOutPacked)]
    lib.pack_fingerprint.restype = i32
    lib.pack_fingerprint.argtypes = [vp, vp, u32, vp]
    lib.pack_fingerprint_steps.restype = i32
    lib.pack_fingerprint_steps.argtypes = [vp, u32, u32, vp, vp]
    lib.pack_inspect.restype = i32
    lib.pack_inspect.argtypes = [vp, u32, vp, C.c_uint64, C.POINTER(C.c_uint64)]
    lib.pack_get_timings.restype = i32
    lib.pack_get_timings.argtypes = [vp, C.POINTER(PackTimings), i32]
    lib.pack_status.restype = i32
    lib.pack_status.argtypes = [vp]
    lib.pack_test_option.restype = i32
    lib.pack_test_option.argtypes = [vp, u32, u32]
    lib.pack_destroy.restype = None
    lib.pack_destroy.argtypes = [vp]
    lib.pack_strerror.restype = C.c_char_p
    lib.pack_strerror.argtypes = [i32]
    lib.pack_last_error.restype = C.c_char_p
    lib.pack_last_error.argtypes = [vp]
    if path is None:
        _lib = lib
    return lib


def _strerror(code: int) -> str:
    try:
        return load_library().pack_strerror(code).decode()
    except Exception:
        return "unknown"


def pack_strerror(code: int) -> str:
    return load_library().pack_strerror(code).decode()


def _check(rc: int, call: str, ctx=None):
    if rc != PACK_OK:
        msg = load_library().pack_last_error(ctx).decode()
        raise DpackError(rc, call, msg)


def pack_init(cfg: PackConfig) -> int:
    ctx = C.c_void_p()
    _check(load_library().pack_init(C.byref(cfg), C.byref(ctx)), "pack_init")
    return ctx.value


def pack_init_noalloc(cfg: PackConfig) -> int:
    ctx = C.c_void_p()
    _check(load_library().pack_init_noalloc(C.byref(cfg), C.byref(ctx)), "pack_init_noalloc")
    return ctx.value


def pack_cycle(ctx: int, cycle: int, info: Optional[PackCycleInfo] = None) -> PackCycleInfo:
    info = info or PackCycleInfo()
    _check(load_library().pack_cycle(ctx, cycle, C.byref(info)), "pack_cycle", ctx)
    return info


def pack_batch(ctx: int, step: int, n_steps: int, out: PackOut) -> None:
    _check(load_library().pack_batch(ctx, step, n_steps, C.byref(out)), "pack_batch", ctx)


def pack_batch_packed(ctx: int, step: int, n_steps: int, out: PackOutPacked) -> None:
    _check(load_library().pack_batch_packed(ctx, step, n_steps, C.byref(out)), "pack_batch_packed", ctx)


def pack_fingerprint(ctx: int, digests_ptr: int, n_batches: int, out_ptr: int) -> None:
    _check(load_library().pack_fingerprint(ctx, digests_ptr, n_batches, out_ptr), "pack_fingerprint", ctx)


def pack_fingerprint_steps(ctx: int, step: int, n_steps: int, digests_ptr: int, out_ptr: int) -> None:
    _check(load_library().pack_fingerprint_steps(ctx, step, n_steps, digests_ptr, out_ptr),
           "pack_fingerprint_steps", ctx)


def pack_inspect(ctx: int, what: str) -> np.ndarray:
    code, dtype = INSPECT[what]
    lib = load_library()
    need = C.c_uint64(0)
    rc = lib.pack_inspect(ctx, code, None, 0, C.byref(need))
    if rc not in (PACK_OK, PACK_E_RANGE):
        _check(rc, "pack_inspect", ctx)
    out = np.zeros(max(1, need.value // np.dtype(dtype).itemsize), dtype=dtype)
    _check(lib.pack_inspect(ctx, code, out.ctypes.data, out.nbytes, C.byref(need)), "pack_inspect", ctx)
    return out[: need.value // np.dtype(dtype).itemsize]


def pack_get_timings(ctx: int, reset: bool = False) -> dict:
    """Phase -> (milliseconds summed, intervals) since the last reset."""
    t = PackTimings()
    _check(load_library().pack_get_timings(ctx, C.byref(t), 1 if reset else 0), "pack_get_timings", ctx)
    return {name: (t.ms[i], int(t.calls[i])) for i, name in enumerate(PHASES)}


def pack_status(ctx: int) -> None:
    """Synchronize and raise if a kernel of an earlier asynchronous call failed."""
    _check(load_library().pack_status(ctx), "pack_status", ctx)


def pack_test_option(ctx: int, what: int, value: int) -> None:
    _check(load_library().pack_test_option(ctx, what, value), "pack_test_option", ctx)


def pack_destroy(ctx: int) -> None:
    if ctx:
        load_library().pack_destroy(ctx)


class Packer:
    """One packing context over a corpus held in torch device tensors.

    ``corpus`` provides numpy arrays (tokens, offsets, source, stratum,
    prompt_len) and the recipe (n_strata, weight, holdout_bp, T, B,
    updates_per_cycle, seed, pad_token); they are copied to ``device`` once
    (or pass ``device_tensors`` to reuse resident ones).  ``timing``: True
    times every kernel phase, "batch" only the phases of batch and
    fingerprint calls (read with ``timings``)."""

    def __init__(self, corpus, rank: int = 0, world: int = 1, device: str = "cuda",
                 device_tensors: Optional[dict] = None, stream=None, timing=False,
                 noalloc: bool = False):
        import torch

        self.torch = torch
        self.corpus = corpus
        self.rank, self.world = rank, world
        if device_tensors is None:
            device_tensors = upload_corpus(corpus, device)
        self.dev = device_tensors
        self.stream = stream if stream is not None else torch.cuda.current_stream(device=self.dev["tokens"].device)
        S = corpus.n_sources
        self._host = dict(
            n_strata=np.ascontiguousarray(corpus.n_strata, np.uint32),
            weight=np.ascontiguousarray(corpus.weight, np.uint64),
            bp=np.ascontiguousarray(corpus.holdout_bp, np.uint32),
        )
        assert self._host["weight"].shape[0] == S
        ramp = getattr(corpus, "ramp", None)
        if ramp is not None:
            self._host["ramp_from"] = np.ascontiguousarray([int(f) for f, _ in ramp], np.uint64)
            self._host["ramp_tokens"] = np.ascontiguousarray([int(t) for _, t in ramp], np.uint64)
        self.ramp = ramp is not None
        self.lanes = max(1, int(getattr(corpus, "lanes", 1) or 1))
        st0 = getattr(corpus, "start_tokens", None)
        if st0 is not None:
            self._host["start_tokens"] = np.ascontiguousarray(st0, np.uint64)
            assert self._host["start_tokens"].shape[0] == S * self.lanes
        d = self.dev
        self.cfg = PackConfig(
            ABI_VERSION, (PACK_FLAG_TIMING_BATCH if timing == "batch" else PACK_FLAG_TIMING if timing else 0)
            | (PACK_FLAG_WRAP if getattr(corpus, "wrap", False) else 0)
            | (PACK_FLAG_HELDOUT if getattr(corpus, "heldout", False) else 0)
            | (PACK_FLAG_READ_RANDOM if getattr(corpus, "read_random", False) else 0)
            | (PACK_FLAG_CUMULATIVE if getattr(corpus, "cumulative", False) else 0)
            | (PACK_FLAG_DIGEST_CHUNKED if getattr(corpus, "digest_chunked", False) else 0),
            d["tokens"].data_ptr() if d["tokens"].numel() else None, int(d["tokens"].numel()),
            d["offsets"].data_ptr(), int(d["source"].numel()),
            d["source"].data_ptr(), d["stratum"].data_ptr() if d.get("stratum") is not None else None,
            d["prompt_len"].data_ptr() if d.get("prompt_len") is not None else None,
            S, self._host["n_strata"].ctypes.data, self._host["weight"].ctypes.data,
            self._host["bp"].ctypes.data, corpus.T, corpus.B, corpus.updates_per_cycle,
            corpus.pad_token, corpus.seed & 0xFFFFFFFFFFFFFFFF, rank, world, self.stream.cuda_stream,
            len(ramp) if ramp is not None else 0,
            self._host["ramp_from"].ctypes.data if ramp is not None else None,
            self._host["ramp_tokens"].ctypes.data if ramp is not None else None,
            self.lanes, self._host["start_tokens"].ctypes.data if st0 is not None else None,
            int(getattr(corpus, "first_cycle", 0)), int(getattr(corpus, "tokens_start", 0)),
            d["segment"].data_ptr() if d.get("segment") is not None else None,
            int(getattr(corpus, "n_segments", 1) or 1))
        self.ctx = pack_init_noalloc(self.cfg) if noalloc else pack_init(self.cfg)
        self.per = corpus.B // world
        self.batches = None  # windows of each update of the current cycle (all ranks)

    def close(self):
        if getattr(self, "ctx", None):
            pack_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def cycle(self, c: int) -> dict:
        S = self.corpus.n_sources * self.lanes  # with lanes: one entry per stream (source, lane)
        arrs = {k: np.zeros(S, np.uint64) for k in ("windows_start", "windows_taken", "windows_remaining",
                                                     "kept_docs", "kept_tokens", "held_docs", "held_tokens")}
        arrs["per_update"] = np.zeros(S, np.uint32)
        arrs["stream_next_token"] = np.zeros(S, np.uint64)
        info = PackCycleInfo()
        for k, v in arrs.items():
            setattr(info, k, v.ctypes.data)
        pack_cycle(self.ctx, c, info)
        # each update's batch: B without a ramp, else the library's per-update table
        self.batches = (pack_inspect(self.ctx, "update_batch") if self.ramp
                        else np.full(info.n_updates, self.corpus.B, np.uint32))
        out = dict(cycle=info.cycle, n_updates=info.n_updates, real_tokens=info.real_tokens,
                   learned_tokens=info.learned_tokens, positions=info.positions,
                   plan_digest=bytes(info.plan_digest), batches=self.batches)
        out.update(arrs)
        return out

    def windows_of(self, step: int, n_steps: int) -> int:
        """This rank's windows of updates [step, step+n_steps)."""
        if not self.ramp:
            return n_steps * self.per
        return int(self.batches[step:step + n_steps].sum()) // self.world

    def alloc_out(self, n_steps: int, digests: bool = True, learned: bool = True, step: int = 0) -> dict:
        """Output buffers: [n_steps, B/world, ...], or with a ramp [windows, ...]
        for the windows of updates [step, step+n_steps), update after update."""
        t = self.torch
        dev = self.dev["tokens"].device
        lead = (self.windows_of(step, n_steps),) if self.ramp else (n_steps, self.per)
        shape = lead + (self.corpus.T,)
        return dict(
            tokens=t.empty(shape, dtype=t.int32, device=dev),  # uint32 bits
            pos=t.empty(shape, dtype=t.int32, device=dev),
            doc=t.empty(shape, dtype=t.int32, device=dev),
            mask=t.empty(shape, dtype=t.uint8, device=dev),
            learned=t.empty((n_steps,), dtype=t.int64, device=dev) if learned else None,
            digests=t.empty(lead + (32,), dtype=t.uint8, device=dev) if digests else None,
        )

    def batch_into(self, step: int, n_steps: int, out: dict) -> dict:
        po = PackOut(out["tokens"].data_ptr(), out["pos"].data_ptr(), out["doc"].data_ptr(),
                     out["mask"].data_ptr(),
                     out["learned"].data_ptr() if out.get("learned") is not None else None,
                     out["digests"].data_ptr() if out.get("digests") is not None else None)
        pack_batch(self.ctx, step, n_steps, po)
        return out

    def batch(self, step: int, n_steps: int = 1, digests: bool = True, learned: bool = True) -> dict:
        """pack_batch into new buffers, then pack_status (synchronous)."""
        out = self.batch_into(step, n_steps, self.alloc_out(n_steps, digests, learned, step))
        pack_status(self.ctx)
        return out

    def alloc_out_packed(self, n_steps: int, learned: bool = True) -> dict:
        t = self.torch
        dev = self.dev["tokens"].device
        cap = self.per * self.corpus.T
        return dict(tokens=t.empty((n_steps, cap), dtype=t.int32, device=dev),
                    pos=t.empty((n_steps, cap), dtype=t.int32, device=dev),
                    doc=t.empty((n_steps, cap), dtype=t.int32, device=dev),
                    mask=t.empty((n_steps, cap), dtype=t.uint8, device=dev),
                    row_start=t.empty((n_steps, self.per + 1), dtype=t.int64, device=dev),
                    length=t.empty(n_steps, dtype=t.int64, device=dev),
                    learned=t.empty(n_steps, dtype=t.int64, device=dev) if learned else None)

    def batch_packed_into(self, step: int, n_steps: int, out: dict, bucket: int = 256) -> dict:
        po = PackOutPacked(out["tokens"].data_ptr(), out["pos"].data_ptr(), out["doc"].data_ptr(),
                           out["mask"].data_ptr(), out["row_start"].data_ptr(), out["length"].data_ptr(),
                           out["learned"].data_ptr() if out.get("learned") is not None else None, bucket)
        pack_batch_packed(self.ctx, step, n_steps, po)
        return out

    def batch_packed(self, step: int, n_steps: int = 1, bucket: int = 256, learned: bool = True) -> dict:
        """Padding-free rows: update i's windows' real positions in row i."""
        return self.batch_packed_into(step, n_steps, self.alloc_out_packed(n_steps, learned), bucket)

    def fingerprint(self, digests) -> "torch.Tensor":
        """digests: device uint8 [n][B][32] (all ranks' slices in rank order)."""
        t = self.torch
        n = int(digests.shape[0])
        out = t.empty((n, 32), dtype=t.uint8, device=digests.device)
        pack_fingerprint(self.ctx, digests.data_ptr(), n, out.data_ptr())
        return out

    def fingerprint_steps(self, step: int, n_steps: int, digests) -> "torch.Tensor":
        """digests: device uint8, the B_b digests of updates [step, step+n_steps)
        one after another (every rank's slice of an update in rank order)."""
        t = self.torch
        out = t.empty((n_steps, 32), dtype=t.uint8, device=digests.device)
        pack_fingerprint_steps(self.ctx, step, n_steps, digests.data_ptr(), out.data_ptr())
        return out

    def inspect(self, what: str) -> np.ndarray:
        return pack_inspect(self.ctx, what)

    def timings(self, reset: bool = False) -> dict:
        return pack_get_timings(self.ctx, reset)

    def status(self) -> None:
        pack_status(self.ctx)

    def test_option(self, what: int, value: int) -> None:
        pack_test_option(self.ctx, what, value)


def upload_corpus(corpus, device: str = "cuda") -> dict:
    """Copy a corpus's arrays to the device as torch tensors (uint16/uint32/uint64
    carried in same-width signed dtypes: only the bits matter to the library)."""
    import torch

    def t(a, dt):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

    return dict(tokens=t(corpus.tokens, np.int32), offsets=t(corpus.offsets, np.int64),
                source=t(corpus.source, np.int16), stratum=t(corpus.stratum, np.int16),
                prompt_len=t(corpus.prompt_len, np.int32),
                segment=t(getattr(corpus, "segment", None), np.int16))
