"""Helpers for GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded corpus, compare bit for bit."""
import sys

import numpy as np

import deterministic_packing_amd as dp
import oracle

PLAN_ARRAYS = {
    # inspect name -> oracle Plan attribute
    "hash": "hash", "keep": "keep", "order": "order", "src_doc_start": "src_doc_start",
    "piece_doc": "piece_doc", "piece_off": "piece_off", "piece_len": "piece_len",
    "piece_woff": "piece_woff", "src_piece_start": "src_piece_start", "win_first": "win_first",
    "src_win_start": "src_win_start", "win_real": "win_real", "win_learn": "win_learn",
    "per_update": "n_per_update", "slot_src": "slot_src", "slot_k": "slot_k",
}


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def compare_plan(pk: "dp.Packer", op: "oracle.Plan"):
    for name, attr in PLAN_ARRAYS.items():
        g = pk.inspect(name)
        o = np.asarray(getattr(op, attr))
        assert g.shape == o.shape, (name, g.shape, o.shape)
        if not np.array_equal(g.astype(np.uint64), o.astype(np.uint64)):
            bad = np.nonzero(g.astype(np.uint64) != o.astype(np.uint64))[0]
            raise AssertionError(f"plan array {name}: {bad.size} mismatches, first at {bad[:5]}: "
                                 f"gpu {g[bad[:5]]} oracle {o[bad[:5]]}")


def to_np(out: dict) -> dict:
    r = {}
    for k, v in out.items():
        if v is None:
            r[k] = None
            continue
        a = v.cpu().numpy()
        if k == "tokens":
            a = a.view(np.uint32)
        r[k] = a
    return r


def compare_batch(g: dict, o: dict, what=""):
    for k in ("tokens", "pos", "doc", "mask", "learned", "digests"):
        if g.get(k) is None or o.get(k) is None:
            continue
        a, b = np.asarray(g[k]), np.asarray(o[k])
        assert a.shape == b.shape, (what, k, a.shape, b.shape)
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{what} {k}: {len(bad)} mismatches, first {bad[:3].tolist()}")


def compare_cycle(gi: dict, oi: "oracle.CycleInfo", op: "oracle.Plan"):
    assert gi["n_updates"] == oi.n_updates
    assert gi["plan_digest"] == oi.plan_digest
    assert gi["windows_start"].tolist() == oi.start.tolist()
    assert gi["windows_taken"].tolist() == oi.taken.tolist()
    assert gi["windows_remaining"].tolist() == oi.remaining.tolist()
    assert gi["per_update"].tolist() == op.n_per_update.tolist()
    assert gi["kept_docs"].tolist() == op.kept_docs.tolist()
    assert gi["kept_tokens"].tolist() == op.kept_tokens.tolist()
    assert gi["held_docs"].tolist() == op.held_docs.tolist()
    assert gi["held_tokens"].tolist() == op.held_tokens.tolist()
    if oi.real_tokens >= 0:
        assert gi["real_tokens"] == oi.real_tokens
        assert gi["learned_tokens"] == oi.learned_tokens
    assert gi["positions"] == oi.positions
    assert np.asarray(gi["batches"]).tolist() == [int(x) for x in oi.batches]
    if getattr(oi, "stream_next", None) is not None:
        assert gi["stream_next_token"].tolist() == oi.stream_next.tolist()


def oracle_digests(op: "oracle.Plan", steps, rank: int = 0, world: int = 1, threads: int = 0) -> np.ndarray:
    """The oracle's window digests of the given updates, [len(steps), B/world, 32]
    (updates of B windows each).  Each update is one call of the oracle's batch
    function; the calls run on a thread pool (the C oracle keeps no shared
    mutable state and ctypes releases the interpreter lock during a call)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    steps = list(steps)
    n = threads or min(16, len(os.sched_getaffinity(0)))

    def one(b):
        return op.batch(b, 1, rank=rank, world=world, digests=True, learned=False)["digests"][0]

    with ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        return np.stack(list(ex.map(one, steps))) if steps else np.zeros((0, 0, 32), np.uint8)
