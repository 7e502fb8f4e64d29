"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (every update of the cycle emitted by one pack_batch call with learned
counts and digests).  The oracle computes the whole plan; outputs are compared
on every window's digest of the cycle (the SHA-256 of its whole record, or
with chunked digests of its chunks' digests, so every output byte), sampled windows' contents, whole sampled batches
(fingerprints) and every learned count, and checked on the GPU for properties
that hold everywhere (padding at the end, position ids, masks agreeing with the
learned counts).  The full-cycle workload is also re-derived at emulated rank
counts 1/8/16/32/64, one fresh context per rank."""
import numpy as np
import pytest

import deterministic_packing_amd as dp
import oracle
from synth import make_corpus

from _gpu_parity import compare_cycle, compare_plan, oracle_digests, say

pytestmark = pytest.mark.gpu

_CACHE = {}


def _setup(name):
    if name not in _CACHE:
        _CACHE.clear()  # one workload's buffers at a time
        import torch
        torch.cuda.empty_cache()
        say("generate", name)
        mode, _, base = name.partition("-") if "-" in name else ("", "", name)
        c = make_corpus(base).replace(wrap=mode == "wrap", heldout=mode == "heldout", read_random=mode == "random",
                                      cumulative=mode == "cum")
        if mode == "ramp":  # 128 windows per update until 10^8 tokens, then 256: both within cycle 0
            c = c.replace(ramp=((0, 128 * c.T), (100_000_000, 256 * c.T)))
        if mode == "lanes":  # 8 lanes: 120 streams of (source, lane)
            c = c.replace(lanes=8)
        if mode == "arrivals":  # 8 arrivals, seeded uniform labels: 480 (source, arrival, stratum) groups
            r = np.random.default_rng(np.random.SeedSequence([7, 8]))
            c = c.replace(segment=r.integers(0, 8, size=c.n_docs).astype(np.uint16), n_segments=8)
        if mode == "heldout":
            c = c.replace(updates_per_cycle=0)  # the 1-5 % held out cannot supply 200 updates
        if mode == "chunked":  # window digests over 4,096-byte chunks of each record
            c = c.replace(digest_chunked=True)
        say("oracle plan", name, c.n_docs, "docs", c.n_tokens, "tokens")
        op = oracle.Plan(c)
        oi = op.cycle(0)
        say("gpu plan", name)
        tensors = dp.upload_corpus(c)
        pk = dp.Packer(c, device_tensors=tensors)
        gi = pk.cycle(0)
        _CACHE[name] = (c, op, oi, tensors, pk, gi)
    return _CACHE[name]


# (workload, updates emitted per call: None = the whole cycle in one call, as the
# bench does; else the first a and the last b updates of the cycle).  The full
# workload's call holds 581,632 windows (2,272 workgroups of the emission-and-
# digest kernel, nine CU-loads); wrap-pretrain is the pre-train workload with
# wrap packing, heldout-pretrain its held-out (validation) stream,
# random-pretrain with each cycle's windows read in a random order,
# cum-pretrain with per-update counts from the cycle's cumulative quotas,
# lanes-pretrain with 8 lanes, arrivals-pretrain with its documents labelled
# with 8 arrivals, chunked-pretrain and chunked-long with chunked window digests.
FULL = [("tiny", None), ("pretrain", None), ("sft", None), ("long", None), ("full", None),
        ("wrap-pretrain", None), ("heldout-pretrain", None), ("random-pretrain", None), ("cum-pretrain", None),
        ("lanes-pretrain", None), ("arrivals-pretrain", None), ("chunked-pretrain", None), ("chunked-long", None)]


def _window_digest(c, tok, pos, dc, mask):
    if c.digest_chunked:
        return oracle.window_digests_chunked(tok, pos, dc, mask).tobytes()
    return oracle.window_digest(tok, pos, dc, mask)


@pytest.mark.parametrize("name,cap", FULL)
def test_full_size_parity(name, cap):
    import torch
    c, op, oi, tensors, pk, gi = _setup(name)
    say("compare plan", name)
    compare_plan(pk, op)
    compare_cycle(gi, oi, op)
    if c.cumulative:
        assert np.array_equal(pk.inspect("cum_taken"), op.cumulative_taken().ravel())
    U = oi.n_updates
    B, T = c.B, c.T
    r = np.random.default_rng(7)
    # emit in one call per contiguous range (bench: the whole cycle in one call)
    ranges = [(0, U)] if cap is None else [(0, min(cap[0], U)), (max(U - cap[1], 0), min(cap[1], U))]
    outs = []
    for s0, cnt in ranges:
        say("emit", name, "steps", s0, "+", cnt)
        outs.append((s0, pk.batch(s0, cnt)))
    torch.cuda.synchronize()
    for s0, g in outs:
        cnt = g["tokens"].shape[0]
        # every window digest of the call against the oracle's
        say("oracle digests", name, cnt, "updates")
        exp = oracle_digests(op, range(s0, s0 + cnt))
        got = g["digests"].cpu().numpy()
        if not np.array_equal(got, exp):
            bad = np.argwhere((got != exp).any(axis=2))
            raise AssertionError(f"{name}: {len(bad)} window digests differ, first (update, slot) {bad[:3].tolist()}")
        # learned counts of every update in the call
        learned = g["learned"].cpu().numpy()
        for i in range(cnt):
            exp = sum(int(op.win_learn[op.window_of(s0 + i, j)]) for j in range(B))
            assert learned[i] == exp, (name, s0 + i)
        # properties of every window of the call, on the GPU
        doc = g["doc"]
        real = doc >= 0
        n_real = real.sum(dim=2)
        idx = torch.arange(T, device=doc.device).view(1, 1, T)
        assert bool((real == (idx < n_real.unsqueeze(2))).all()), "padding only at the end of a window"
        # (no boolean-mask indexing: the full cycle has more than 2^31 positions)
        assert bool(((g["pos"] == 0) | real).all()) and bool(((g["mask"] == 0) | real).all())
        assert bool(((g["tokens"] == c.pad_token) | real).all())
        assert bool((g["mask"].sum(dim=(1, 2)).cpu() == g["learned"].cpu()).all()), "learned = sum of mask"
        exp_real = np.array([[int(op.win_real[op.window_of(s0 + i, j)]) for j in range(B)] for i in range(cnt)])
        assert np.array_equal(n_real.cpu().numpy(), exp_real)
        # sampled windows: whole content and digest vs the oracle
        picks = [(int(r.integers(cnt)), int(r.integers(B))) for _ in range(48)] + [(0, 0), (cnt - 1, B - 1)]
        for i, j in picks:
            gw = op.window_of(s0 + i, j)
            tok, pos, dc, mask = op.emit_window(gw)
            assert np.array_equal(g["tokens"][i, j].cpu().numpy().view(np.uint32), tok), (name, s0 + i, j)
            assert np.array_equal(g["pos"][i, j].cpu().numpy(), pos)
            assert np.array_equal(g["doc"][i, j].cpu().numpy(), dc)
            assert np.array_equal(g["mask"][i, j].cpu().numpy(), mask)
            assert g["digests"][i, j].cpu().numpy().tobytes() == _window_digest(c, tok, pos, dc, mask)
        # whole sampled batches: every window digest and the batch fingerprint
        for i in sorted({0, cnt - 1}):
            o = op.batch(s0 + i, 1)
            assert np.array_equal(g["digests"][i].cpu().numpy(), o["digests"][0]), (name, s0 + i)
            fp = pk.fingerprint(g["digests"][i:i + 1]).cpu().numpy()[0].tobytes()
            assert fp == oracle.batch_fingerprint(o["digests"][0])
    outs.clear()
    _CACHE.clear()
    torch.cuda.empty_cache()


def test_full_size_ramp_parity():
    """The pre-train workload with a batch-size ramp (128 windows per update until
    10^8 tokens, then 256): the whole cycle in one call, ragged layout."""
    import torch
    name = "ramp-pretrain"
    c, op, oi, tensors, pk, gi = _setup(name)
    compare_plan(pk, op)
    compare_cycle(gi, oi, op)
    assert gi["batches"].tolist() == oi.batches.tolist()
    assert len(set(oi.batches.tolist())) == 2, "both pieces within the cycle"
    U, T = oi.n_updates, c.T
    slot0 = np.concatenate([[0], np.cumsum(oi.batches.astype(np.int64))])
    say("emit", name, "steps 0 +", U)
    g = pk.batch(0, U)
    torch.cuda.synchronize()
    learned = g["learned"].cpu().numpy()
    for b in range(U):
        exp = sum(int(op.win_learn[op.window_of(b, j)]) for j in range(int(oi.batches[b])))
        assert learned[b] == exp, b
    doc = g["doc"]
    real = doc >= 0
    n_real = real.sum(dim=1)
    idx = torch.arange(T, device=doc.device).view(1, T)
    assert bool((real == (idx < n_real.unsqueeze(1))).all()), "padding only at the end of a window"
    assert bool(((g["pos"] == 0) | real).all()) and bool(((g["mask"] == 0) | real).all())
    exp_real = np.array([int(op.win_real[op.window_of(b, j)]) for b in range(U) for j in range(int(oi.batches[b]))])
    assert np.array_equal(n_real.cpu().numpy(), exp_real)
    r = np.random.default_rng(8)
    picks = [(int(r.integers(U)), None) for _ in range(40)] + [(0, 0), (U - 1, None)]
    for b, j in picks:
        j = int(r.integers(int(oi.batches[b]))) if j is None else j
        x = int(slot0[b]) + j
        tok, pos, dc, mask = op.emit_window(op.window_of(b, j))
        assert np.array_equal(g["tokens"][x].cpu().numpy().view(np.uint32), tok), (b, j)
        assert np.array_equal(g["pos"][x].cpu().numpy(), pos)
        assert np.array_equal(g["doc"][x].cpu().numpy(), dc)
        assert np.array_equal(g["mask"][x].cpu().numpy(), mask)
        assert g["digests"][x].cpu().numpy().tobytes() == oracle.window_digest(tok, pos, dc, mask)
    switch = int(np.argmax(oi.batches != oi.batches[0]))
    for b in sorted({0, switch - 1, switch, U - 1}):
        o = op.batch(b, 1)
        d = g["digests"][int(slot0[b]):int(slot0[b + 1])]
        assert np.array_equal(d.cpu().numpy(), o["digests"]), b
        fp = pk.fingerprint_steps(b, 1, d).cpu().numpy()[0].tobytes()
        assert fp == oracle.batch_fingerprint(o["digests"])
    del g
    _CACHE.clear()
    torch.cuda.empty_cache()


def test_full_size_new_length_after_a_cycle():
    """The pre-train workload, 100 updates in cycle 0 at T = 4096, then a context
    that goes on at T = 8192 (128 windows per update, the same tokens) from the
    stream tokens the GPU reports: plan, cycle and sampled windows vs the oracle."""
    import torch
    _CACHE.clear()
    c = make_corpus("pretrain").replace(updates_per_cycle=100)
    say("generate", "pretrain for the re-cut")
    tensors = dp.upload_corpus(c)
    pk = dp.Packer(c, device_tensors=tensors)
    gi = pk.cycle(0)
    pk.close()
    c2 = c.replace(T=8192, B=128, start_tokens=gi["stream_next_token"].copy(), first_cycle=1,
                   tokens_start=int(gi["positions"]))
    say("oracle plan", "re-cut at T 8192")
    op = oracle.Plan(c2)
    oi = op.cycle(1)
    p2 = dp.Packer(c2, device_tensors=tensors)
    compare_plan(p2, op)
    compare_cycle(p2.cycle(1), oi, op)
    n = oi.n_updates
    say("emit", "re-cut", n, "updates")
    g = p2.batch(0, n)
    torch.cuda.synchronize()
    r = np.random.default_rng(9)
    for _ in range(24):
        i, j = int(r.integers(n)), int(r.integers(c2.B))
        tok, pos, dc, mask = op.emit_window(op.window_of(i, j))
        assert np.array_equal(g["tokens"][i, j].cpu().numpy().view(np.uint32), tok), (i, j)
        assert np.array_equal(g["mask"][i, j].cpu().numpy(), mask)
        assert g["digests"][i, j].cpu().numpy().tobytes() == oracle.window_digest(tok, pos, dc, mask)
    o = op.batch(n - 1, 1)
    assert np.array_equal(g["digests"][n - 1].cpu().numpy(), o["digests"][0])
    p2.close()
    torch.cuda.empty_cache()


def test_full_cycle_fingerprints_at_emulated_rank_counts():
    """The full-cycle workload at full size (2·10^9 tokens, B = 1024): for each
    rank count R in 1, 8, 16, 32, 64, every rank's slice of the cycle's first,
    middle and last update is emitted by a fresh context of its own over the
    resident corpus; the slices side by side must give the oracle's window
    digests, and the batch fingerprint the oracle's (Zephon blog post, resume
    of a 16-GPU run on 8/32/64 GPUs: every global batch's SHA-256 equal byte
    for byte)."""
    import torch
    c, op, oi, tensors, pk, gi = _setup("full")
    U, B = oi.n_updates, c.B
    steps = [0, U // 2, U - 1]
    say("oracle digests", "full", steps)
    exp = oracle_digests(op, steps)
    exp_fp = [oracle.batch_fingerprint(exp[k]) for k in range(len(steps))]
    for R in (1, 8, 16, 32, 64):
        per = B // R
        dig = torch.empty((len(steps), B, 32), dtype=torch.uint8, device=tensors["tokens"].device)
        say("emulated ranks", R)
        for r in range(R):
            p = dp.Packer(c, rank=r, world=R, device_tensors=tensors)
            info = p.cycle(0)
            assert info["plan_digest"] == oi.plan_digest and info["n_updates"] == U, (R, r)
            for k, b in enumerate(steps):
                out = p.alloc_out(1)
                p.batch_into(b, 1, out)
                dig[k, r * per:(r + 1) * per] = out["digests"][0]
            p.status()
            p.close()
        got = dig.cpu().numpy()
        for k, b in enumerate(steps):
            assert np.array_equal(got[k], exp[k]), (R, b)
        fps = pk.fingerprint(dig).cpu().numpy()
        for k, b in enumerate(steps):
            assert fps[k].tobytes() == exp_fp[k], (R, b)
    _CACHE.clear()
    torch.cuda.empty_cache()
