#!/usr/bin/env python3
"""Packed tokens/s of the whole deterministic-packing path on one MI355X.

One step = one pass of the whole path over the resident synthetic corpus:
pack_init (validation, hash + hold-out, keys, sort, strata merge, pieces,
next-fit cut, window table, mixture) + pack_cycle(0) + pack_batch of every
update of the cycle with learned counts and per-window SHA-256 digests +
pack_destroy.  The corpus is in HBM and the output buffers are allocated
before the timed region.  value = real (non-padding) tokens emitted per second.
The default workload is the full cycle: 2·10^9 tokens resident, 15 sources x
8 strata, T = 4096, B = 1024, every update of the longest cycle.

Per-kernel times come from HIP events the library records on its stream.
Inside the timed steps only the batch's kernels are timed
(PACK_FLAG_TIMING_BATCH: two events around the dominant kernel per step); the
plan's phases are timed in a second pass of the same steps after the timed
region (PACK_FLAG_TIMING), since an event costs several microseconds of stream
time.  The roofline object is reported for the kernel that takes the most
time, and every phase is listed under "kernels".  The emission kernel without
digests (the packing kernel on its own, HBM-bound) is timed the same way in a
separate pass over the same cycle and reported as roofline_emit.  The CPU baseline is the oracle (plain
sequential C) timed on this host on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0                      # MI355X HBM3E, 8 TB/s
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12  # 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz = 39.3 T int32 ops/s
SHA_OPS_PER_BLOCK = 1400                    # int32 VALU ops per SHA-256 compression on gfx950
METRIC = "packed tokens/s and achieved HBM GB/s (% of peak), 1 MI355X, bit-exact vs oracle"

WORKLOAD_TEXT = {
    "pretrain": "pre-train mix: 15 sources x 4 strata, 1M docs, lognormal lengths (median 600, sigma 1.2, "
                "max 65536), Zipf(1.1) ids over 65,536, hold-out 1% (5% source 14), T=4096, B=256, 200 updates",
    "tiny": "tiny: 2 sources x 2,000 docs, geometric lengths mean 300, T=2048, B=8, max updates",
    "sft": "SFT: 500k prompt/completion pairs, T=4096, B=8, completion-only mask, max updates",
    "long": "long-context: 8 sources, 200k Pareto(1.3) docs 1k-200k, T=32768, B=32, max updates",
    "full": "full cycle: 2B tokens, 15 sources x 8 strata, T=4096, B=1024, max updates",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def digest_blocks(T: int, chunked: bool) -> int:
    """SHA-256 compressions per window digest: the record's 13·T bytes and their
    padding, or, chunked, every 4,096-byte chunk with its padding and then the
    digest of the chunk digests (32 bytes each)."""
    n = 13 * T
    if not chunked:
        return (n + 72) // 64
    full, last = divmod(n, 4096)
    blocks = full * ((4096 + 72) // 64) + ((last + 72) // 64 if last else 0)
    return blocks + (32 * (full + (1 if last else 0)) + 72) // 64


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 PMC runs, if a committed
    summary exists for this kernel and workload (profiles/<kernel>_<workload>
    _pmc.md, the workload with a _packed suffix for padding-free rows) and the
    kernel's source is unchanged since (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    src = fields.get("source file")
    if not src or "traffic bytes per launch" not in fields:
        return None
    cur = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
    if cur != fields.get("source sha256"):
        return None
    return float(fields["traffic bytes per launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="full", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--scale", type=float, default=1.0, help="fraction of the workload (1.0 = as specified)")
    ap.add_argument("--cpu-sample-seconds", type=float, default=12.0,
                    help="the oracle emits (with digests) whole updates from update 0 until this much time has "
                         "passed, for the CPU baseline (the plan is always whole)")
    ap.add_argument("--cpu-sample-updates", type=int, default=0,
                    help="emit exactly this many updates for the CPU baseline instead (0: by time)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy", action="store_true", help="skip the plain D2D copy used as calibration/ceiling")
    ap.add_argument("--no-per-call", action="store_true",
                    help="skip the latency of one update per pack_batch call (kernel traces of the step alone)")
    ap.add_argument("--wrap", action="store_true", help="wrap packing (PACK_FLAG_WRAP) instead of next-fit")
    ap.add_argument("--packed", action="store_true",
                    help="emit padding-free rows (pack_batch_packed, bucket 256) instead of padded windows and digests")
    ap.add_argument("--lanes", type=int, default=1, help="Zephon lanes (document d in lane d mod lanes)")
    ap.add_argument("--ramp", action="store_true",
                    help="batch-size ramp: B/2 windows per update until 10^8 tokens, then B (pre-train: 128 -> 256)")
    ap.add_argument("--cumulative", action="store_true",
                    help="per-update window counts from each cycle's cumulative quotas (PACK_FLAG_CUMULATIVE)")
    ap.add_argument("--read-random", action="store_true",
                    help="each cycle's windows of a source read in a random order (PACK_FLAG_READ_RANDOM)")
    ap.add_argument("--heldout", action="store_true",
                    help="the held-out (validation) stream instead of the training one, cycle of maximal length")
    ap.add_argument("--arrivals", type=int, default=1,
                    help="streamed corpus: each document carries one of N arrivals (seeded uniform labels)")
    ap.add_argument("--resume", action="store_true",
                    help="time cycle 1 of a context that starts each stream at the token cycle 0 reported")
    ap.add_argument("--digest-chunked", action="store_true",
                    help="window digests over the digests of 4,096-byte chunks of each record "
                         "(PACK_FLAG_DIGEST_CHUNKED)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import deterministic_packing_amd as dp
    from synth import make_corpus

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dp.load_library()

    t0 = time.time()
    corpus = make_corpus(args.workload, args.scale).replace(wrap=args.wrap, read_random=args.read_random,
                                                             cumulative=args.cumulative,
                                                             digest_chunked=args.digest_chunked)
    if args.ramp:
        corpus = corpus.replace(ramp=((0, corpus.B // 2 * corpus.T), (100_000_000, corpus.B * corpus.T)))
    if args.lanes > 1:
        corpus = corpus.replace(lanes=args.lanes)
    if args.heldout:
        corpus = corpus.replace(heldout=True, updates_per_cycle=0)
    if args.arrivals > 1:
        r = np.random.default_rng(np.random.SeedSequence([7, args.arrivals]))
        corpus = corpus.replace(segment=r.integers(0, args.arrivals, size=corpus.n_docs).astype(np.uint16),
                                n_segments=args.arrivals)
    log(f"corpus {args.workload} scale {args.scale}: {corpus.n_docs} docs, {corpus.n_tokens} tokens "
        f"({time.time() - t0:.1f}s)")
    tensors = dp.upload_corpus(corpus)
    torch.cuda.synchronize()
    log("corpus resident in HBM")

    if args.resume:
        # each stream from the token where cycle 0 left it: a context for cycle 1 on
        first = dp.Packer(corpus, device_tensors=tensors)
        i0 = first.cycle(0)
        corpus = corpus.replace(start_tokens=i0["stream_next_token"].copy(), first_cycle=1,
                                tokens_start=int(i0["positions"]))
        first.close()
    cyc = corpus.first_cycle
    probe = dp.Packer(corpus, device_tensors=tensors)
    try:
        U = probe.cycle(cyc)["n_updates"]
    except dp.DpackError as e:
        if e.code != dp.PACK_E_EXHAUSTED or args.scale == 1.0:
            raise
        # a scaled-down corpus cannot supply the configured updates: take the most it supports
        probe.close()
        corpus = corpus.replace(updates_per_cycle=0)
        probe = dp.Packer(corpus, device_tensors=tensors)
        U = probe.cycle(cyc)["n_updates"]
    probe.close()
    B, T = corpus.B, corpus.T
    batches = [int(x) for x in probe.batches]  # windows of each update of the timed cycle
    # output buffers outside the timed region
    out = dp.Packer.alloc_out_packed(probe, U) if args.packed else dp.Packer.alloc_out(probe, U)
    torch.cuda.synchronize()
    log(f"cycle {cyc}: {U} updates x {B if not args.ramp else sorted(set(batches))} windows x {T} positions")

    def one_step(timing):
        pk = dp.Packer(corpus, device_tensors=tensors, timing=timing)
        info = pk.cycle(cyc)
        if args.packed:
            pk.batch_packed_into(0, info["n_updates"], out)
        else:
            pk.batch_into(0, info["n_updates"], out)
        tm = pk.timings(reset=True)
        pk.status()  # a failure inside the batch kernels raises here
        pk.close()
        return info, tm

    # the timed steps record events only around the batch's kernels (the
    # dominant kernel's launch time): an event costs several microseconds of
    # stream time, which the plan's dozen phases would add to every step
    for w in range(args.warmup):
        one_step("batch")
        log(f"warmup {w + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    phase_ms = {}
    phase_calls = {}
    t_start = time.perf_counter()
    for s in range(args.steps):
        info, tm = one_step("batch")
        for k, (ms, n) in tm.items():
            phase_ms[k] = phase_ms.get(k, 0.0) + ms
            phase_calls[k] = phase_calls.get(k, 0) + n
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    # the plan's phases: the same steps again after the timed region, every phase timed
    for s in range(args.steps):
        _, tm = one_step(True)
        for k, (ms, n) in tm.items():
            if k not in ("emit", "learned", "digest", "fingerprint"):
                phase_ms[k] = phase_ms.get(k, 0.0) + ms
                phase_calls[k] = phase_calls.get(k, 0) + n
    real = info["real_tokens"]
    positions = info["positions"]
    value = real / (ms_per_step / 1e3)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value:.4g} packed tokens/s")

    # per-kernel figures (averaged per launch: the batch's over the timed steps,
    # the plan's over the instrumented pass)
    n_windows = sum(batches)
    # read every real token once, write 13 bytes per output position (padded
    # windows: U·B·T; padding-free rows: the rows' lengths, bucket padding included)
    row_positions = int(out["length"].sum().item()) if args.packed else positions
    emit_bytes = 4.0 * real + 13.0 * row_positions
    fused = phase_calls.get("emit", 0) == 0     # emission ran inside the digest kernel
    algo = {
        "emit": ("hbm", emit_bytes, "GB/s"),
        # hash: read every token once + per document offsets/source in, hash/keep out
        "hash": ("hbm", 4.0 * corpus.n_tokens + 19.0 * corpus.n_docs, "GB/s"),
        # window SHA-256: (13T/64 + 1) compressions per window; chunked, each chunk's blocks and
        # padding, then the SHA-256 of the chunk digests
        "digest": ("alu", SHA_OPS_PER_BLOCK * n_windows * digest_blocks(T, args.digest_chunked), "TOP/s"),
    }
    # bytes the digest kernel moves: the emission when fused, a 32-byte digest per window, and the
    # 13T-byte records read back where the paired kernel hashes them from the outputs (launches of
    # 513 to 1,024 waves of 64 windows; the ring pairs and the own-record kernel read nothing back)
    waves = (n_windows + 63) // 64
    read_back = 512 < waves <= 1024 or args.digest_chunked
    digest_bytes = (13.0 * positions if read_back else 0.0) + (emit_bytes if fused else 0.0) + 32.0 * n_windows
    kernels = {}
    for k in phase_ms:
        if phase_calls[k] == 0:
            continue
        per_step = phase_ms[k] / args.steps
        entry = {"ms_per_step": round(per_step, 4), "launch_groups_per_step": phase_calls[k] / args.steps}
        if k in algo:
            bound, work, unit = algo[k]
            per_launch_ms = phase_ms[k] / phase_calls[k]
            ach = work / (per_launch_ms / 1e3) / 1e9 if unit == "GB/s" else work / (per_launch_ms / 1e3) / 1e12
            peak = HBM_PEAK_GBPS if unit == "GB/s" else VALU_PEAK_TOPS
            entry.update(bound=bound, achieved=round(ach, 2), peak=round(peak, 1), unit=unit,
                         frac=round(ach / peak, 4), work_per_launch=work)
            if k == "digest":
                entry.update(emission_inside=fused, bytes_per_launch=digest_bytes,
                             achieved_GBps=round(digest_bytes / (per_launch_ms / 1e3) / 1e9, 1))
        kernels[k] = entry
    # profiles are taken per kernel and workload, with and without padding-free rows, in the
    # plain mode only: another mode can run another kernel (the held-out stream's few windows
    # take the ring kernel) or other bytes, so it reports no traffic; the hash does not depend
    # on how the windows are emitted
    moded = (args.wrap or args.lanes > 1 or args.ramp or args.cumulative or args.read_random or args.heldout
             or args.arrivals > 1 or args.resume or args.digest_chunked or args.scale != 1.0)

    def traffic_of(k):
        if moded:
            return None
        return traffic_from_profile(k, args.workload if k == "hash" else
                                    args.workload + ("_packed" if args.packed else ""))

    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dom = kernels[dominant]
    roofline = None
    if "bound" in dom:
        traffic = traffic_of(dominant)
        roofline = {"kernel": dominant, "bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                    "unit": dom["unit"], "frac": dom["frac"], "traffic": traffic}
    # the HBM-bound kernels, each against the HBM roofline
    side = {}
    for k in ("hash", "emit"):
        e = kernels.get(k, {})
        if "achieved" in e:
            side[k] = {"kernel": k, "bound": "hbm", "achieved": e["achieved"], "peak": HBM_PEAK_GBPS,
                       "unit": "GB/s", "frac": e["frac"], "traffic": traffic_of(k)}
    if "emit" not in side:
        # the emission kernel on its own (pack_batch without digests over the
        # same cycle, into the same buffers), timed by the library's events
        pk2 = dp.Packer(corpus, device_tensors=tensors, timing="batch")
        pk2.cycle(cyc)
        nod = dict(out, digests=None)
        pk2.batch_into(0, U, nod)  # warm-up
        pk2.timings(reset=True)
        reps = 3
        for _ in range(reps):
            pk2.batch_into(0, U, nod)
        ms_e, n_e = pk2.timings(reset=True)["emit"]
        pk2.status()
        pk2.close()
        per_launch_ms = ms_e / n_e
        ach = emit_bytes / (per_launch_ms / 1e3) / 1e9
        side["emit"] = {"kernel": "emit", "bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                        "traffic": traffic_of("emit"),
                        "ms_per_launch": round(per_launch_ms, 4), "work_per_launch": emit_bytes,
                        "measured": f"pack_batch without digests over the whole cycle, {reps} launches"}
        log(f"emission alone: {per_launch_ms:.3f} ms per cycle, {ach:.1f} GB/s")

    # latency of one update per call (pack_batch of a single update), with and
    # without the window digests, on a context whose cycle is planned: GPU time
    # between events on the context's stream, and host wall time to completion
    per_call = None
    if not args.packed and not args.ramp and not args.no_per_call:
        pk1 = dp.Packer(corpus, device_tensors=tensors)
        pk1.cycle(cyc)
        n_calls = min(20, U)
        per_call = {"calls": n_calls, "windows_per_call": B}
        for dg in (False, True):
            o1 = pk1.alloc_out(1, digests=dg)
            gpu, wall = [], []
            for s_ in range(n_calls):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                t_a = time.perf_counter()
                e0.record()
                pk1.batch_into(s_, 1, o1)
                e1.record()
                torch.cuda.synchronize()
                wall.append((time.perf_counter() - t_a) * 1e3)
                gpu.append(e0.elapsed_time(e1))
            tag = "with_digests" if dg else "without_digests"
            per_call[tag + "_gpu_ms"] = round(float(np.median(gpu)), 4)
            per_call[tag + "_wall_ms"] = round(float(np.median(wall)), 4)
        pk1.close()
        log(f"one update per call: {per_call}")

    # plain device-to-device copy of 1 GiB: practical HBM ceiling and the
    # known-size kernel the PMC byte counters are calibrated against
    copy = None
    if not args.no_copy:
        n = 1 << 28
        a = torch.empty(n, dtype=torch.int32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        copy = {"bytes_per_copy": 2 * 4 * n, "ms": round(ms, 4), "GBps": round(2 * 4 * n / (ms / 1e3) / 1e9, 1)}
        del a, b

    # CPU baseline: the oracle on this host (whole plan, then whole updates
    # from update 0 until the time budget is spent), and a bit-exact check of
    # the GPU's outputs of the last timed step on every sampled update
    cpu = None
    sample_check = None
    if not args.no_cpu_baseline:
        import platform
        import oracle
        oracle.build()
        t_a = time.perf_counter()
        op = oracle.Plan(corpus)
        t_b = time.perf_counter()
        oi = op.cycle(cyc)
        t_c = time.perf_counter()
        first_win = np.concatenate([[0], np.cumsum(batches)]).astype(np.int64)
        n_s, t_emit, mism = 0, 0.0, 0
        while n_s < U and ((args.cpu_sample_updates == 0 and t_emit < args.cpu_sample_seconds)
                           or n_s < args.cpu_sample_updates):
            t_x = time.perf_counter()
            ob = op.batch_packed(n_s, 1) if args.packed else op.batch(n_s, 1, digests=True)
            t_emit += time.perf_counter() - t_x
            if args.packed:
                ln = int(ob["length"][0])
                mism += int(int(out["length"][n_s].item()) != ln)
                mism += int((out["row_start"][n_s].cpu().numpy() != ob["row_start"][0]).sum())
                for key in ("tokens", "pos", "doc", "mask"):
                    g = out[key][n_s, :ln].cpu().numpy()
                    if key == "tokens":
                        g = g.view(np.uint32)
                    mism += int((g != ob[key][0, :ln]).sum())
                mism += int(int(out["learned"][n_s].item()) != int(op.batch(n_s, 1, digests=False)["learned"][0]))
            else:
                for key in ("tokens", "pos", "doc", "mask", "digests"):
                    if args.ramp:  # flat [windows, ...]: this update's windows
                        g = out[key][int(first_win[n_s]):int(first_win[n_s + 1])].cpu().numpy()
                    else:
                        g = out[key][n_s].cpu().numpy()
                    if key == "tokens":
                        g = g.view(np.uint32)
                    mism += int((g != ob[key].reshape(g.shape)).sum())
                mism += int(int(out["learned"][n_s].item()) != int(ob["learned"][0]))
            n_s += 1
        est = (t_b - t_a) + (t_c - t_b) + t_emit * sum(batches) / sum(batches[:n_s])
        model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")),
                     platform.processor())
        cpu = {"value": round(real / est, 1), "unit": "packed tokens/s", "cores": 1, "kind": "oracle",
               "host": {"nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "cpu_model": model},
               "sample": (f"whole plan of the corpus ({t_b - t_a:.2f}s) + cycle ({t_c - t_b:.2f}s) + "
                          + ("padding-free rows" if args.packed else "emission with SHA-256")
                          + f" of updates 0..{n_s - 1} of {U} ({t_emit:.2f}s), scaled to the cycle's "
                          f"{sum(batches)} windows: {est:.2f}s per step; single-threaded C on one core")}
        log(f"cpu baseline {cpu['value']:.4g} tokens/s ({est:.1f}s per step) on {model}")
        mism += int(oi.plan_digest != info["plan_digest"])
        sample_check = {"updates_compared": n_s, "windows_compared": int(sum(batches[:n_s])), "mismatches": mism}
        log(f"bit-exact check on {n_s} updates: {mism} mismatches")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "packed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload] + ("" if args.scale == 1.0 else f" (scale {args.scale})")
                   + (", wrap packing" if args.wrap else "") + (", random read order" if args.read_random else "")
                   + (", per-update counts from cumulative quotas" if args.cumulative else "")
                   + (f", batch-size ramp {B // 2} -> {B} windows per update at 10^8 tokens" if args.ramp else "")
                   + (f", {args.lanes} lanes" if args.lanes > 1 else "")
                   + (", held-out (validation) stream, cycle of maximal length" if args.heldout else "")
                   + (f", {args.arrivals} arrivals" if args.arrivals > 1 else "")
                   + (", cycle 1 of a context resumed at cycle 0's stream tokens" if args.resume else "")
                   + (", padding-free rows" if args.packed else "")
                   + (", chunked window digests (4,096-byte chunks)" if args.digest_chunked else ""),
                   "docs": corpus.n_docs, "tokens": corpus.n_tokens, "T": T, "B": B, "updates": U,
                   "real_tokens_per_step": real, "positions_per_step": row_positions,
                   "step": ("pack_init + pack_cycle + pack_batch_packed(all updates, learned, bucket 256) + pack_destroy"
                            if args.packed else
                            "pack_init + pack_cycle + pack_batch(all updates, learned, digests) + pack_destroy")},
        "roofline": roofline,
        "roofline_hash": side.get("hash"),
        "roofline_emit": side.get("emit"),
        "cpu_baseline": cpu,
        "kernels": kernels,
        "copy_ceiling": copy,
        "per_call_batch": per_call,
        "bit_exact_sample": sample_check,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
