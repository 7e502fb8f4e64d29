"""Parity of the HIP path (through the C ABI) with the CPU oracle, bit for bit,
on seeded corpora of every workload shape, plus error paths and determinism."""
import numpy as np
import pytest

import deterministic_packing_amd as dp
import oracle
from synth import make_corpus, random_small
from synth.corpus import Corpus

from _gpu_parity import compare_batch, compare_cycle, compare_plan, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dp.load_library()
    yield
    torch.cuda.synchronize()


SMALL_CASES = [("small", s) for s in range(8)] + [
    ("tiny", 1.0), ("sft", 0.004), ("long", 0.01), ("pretrain", 0.006), ("full", 0.002)]


def _corpus(kind, arg):
    if kind == "small":
        s = int(arg)
        return random_small(s, n_docs=60 + 40 * s, n_sources=1 + s % 4, max_strata=1 + s % 3, T=64 * (1 + s % 2),
                            B=[1, 2, 4, 6, 8, 3, 5, 7][s], max_len=[40, 150, 300, 90, 64, 200, 20, 500][s],
                            prompts=bool(s % 2), bp_max=2000)
    if kind == "tinydocs":  # documents of 1-5 tokens: windows of many pieces, short source tails
        s = int(arg)
        return random_small(50 + s, n_docs=40 + 30 * s, n_sources=1 + s % 3, max_strata=2, T=64, B=1 + s,
                            max_len=5, prompts=bool(s % 2), bp_max=1000)
    c = make_corpus(kind, arg)
    if kind == "pretrain":
        c = c.replace(updates_per_cycle=0)  # a scaled-down corpus cannot supply 200 updates
    return c


@pytest.mark.parametrize("kind,arg", SMALL_CASES)
def test_plan_cycle_batch_parity(kind, arg):
    _parity_run(_corpus(kind, arg), kind, arg)


@pytest.mark.parametrize("kind,arg", SMALL_CASES)
def test_wrap_plan_cycle_batch_parity(kind, arg):
    """The same cases with wrap packing (PACK_FLAG_WRAP)."""
    _parity_run(_corpus(kind, arg).replace(wrap=True), "wrap-" + kind, arg)


@pytest.mark.parametrize("kind,arg", SMALL_CASES)
def test_read_random_parity(kind, arg):
    """The same cases with each cycle's windows read in a random order (PACK_FLAG_READ_RANDOM)."""
    _parity_run(_corpus(kind, arg).replace(read_random=True), "random-order-" + kind, arg)


PACKED_CASES = ([("small", s, b, w, False) for s, b, w in [(0, 256, 1), (1, 64, 1), (3, 1, 2), (4, 256, 4),
                                                            (5, 256, 1), (7, 0, 7)]]
                + [("tinydocs", s, b, 1, wr) for s, b in [(0, 1), (1, 256), (2, 3), (3, 0)] for wr in (False, True)]
                + [("small", 2, 256, 1, True), ("sft", 0.004, 256, 1, False), ("pretrain", 0.006, 256, 8, False),
                   ("long", 0.01, 256, 2, False)])


NODIG_CASES = [("small", s) for s in range(8)] + [("tinydocs", 3), ("sft", 0.004), ("long", 0.01), ("full", 0.004)]


@pytest.mark.parametrize("kind,arg", NODIG_CASES)
@pytest.mark.parametrize("wrap", [False, True])
def test_batch_without_digests_parity(kind, arg, wrap):
    """pack_batch without digests (the emission kernel alone): padded windows whose
    four-position groups lie in one piece take one 16-byte token load, the others
    (piece ends, padding, the corpus end) go element by element."""
    c = _corpus(kind, arg).replace(wrap=wrap, updates_per_cycle=0)  # the longest cycle the corpus supports
    op = oracle.Plan(c)
    oi = op.cycle(0)
    n = min(4, oi.n_updates)
    say("no digests", kind, arg, "wrap", wrap)
    pk = dp.Packer(c)
    pk.cycle(0)
    compare_batch(to_np(pk.batch(0, n, digests=False)), op.batch(0, n, digests=False), f"{kind}{arg} no digests")
    pk.close()


@pytest.mark.parametrize("kind,arg,bucket,world,wrap", PACKED_CASES)
def test_padding_free_rows_parity(kind, arg, bucket, world, wrap):
    """pack_batch_packed against the oracle's padding-free rows (rank 0 and the last rank).
    Row starts fall anywhere, so windows begin and end inside 16-byte store groups."""
    c = _corpus(kind, arg).replace(wrap=wrap)
    if c.B % world:
        c = c.replace(B=world * max(1, c.B // world))
    op = oracle.Plan(c)
    try:
        oi = op.cycle(0)
    except oracle.OracleError:
        pytest.skip("corpus exhausted at this size")
    n = min(3, oi.n_updates)
    for rank in sorted({0, world - 1}):
        say("packed", kind, arg, "bucket", bucket, "world", world, "rank", rank)
        pk = dp.Packer(c, rank=rank, world=world)
        pk.cycle(0)
        g = {k: (v.cpu().numpy() if v is not None else None) for k, v in pk.batch_packed(0, n, bucket).items()}
        o = op.batch_packed(0, n, rank=rank, world=world, bucket=bucket)
        assert np.array_equal(g["row_start"], o["row_start"]) and np.array_equal(g["length"], o["length"])
        for i in range(n):
            L = int(o["length"][i])
            for k in ("tokens", "pos", "doc", "mask"):
                a = g[k][i, :L].view(np.uint32) if k == "tokens" else g[k][i, :L]
                assert np.array_equal(a, o[k][i, :L]), (i, k)
        assert np.array_equal(g["learned"], op.batch(0, n, digests=False)["learned"])
        pk.close()


@pytest.mark.parametrize("kind,arg", SMALL_CASES)
def test_cumulative_parity(kind, arg):
    """The same cases with per-update counts from the cycle's cumulative quotas (PACK_FLAG_CUMULATIVE)."""
    _parity_run(_corpus(kind, arg).replace(cumulative=True), "cumulative-" + kind, arg)


CUM_MODES = [(s, wrap, rr, held) for s, (wrap, rr, held) in enumerate(
    [(False, False, False), (True, False, False), (False, True, False), (False, False, True), (True, True, True),
     (False, True, True), (True, False, False), (False, False, False)])]


@pytest.mark.parametrize("seed,wrap,read_random,heldout", CUM_MODES)
def test_cumulative_with_other_modes(seed, wrap, read_random, heldout):
    """Cumulative quotas with wrap packing, the random read order and the held-out stream;
    recipes with shares below one window per update."""
    r = np.random.default_rng(500 + seed)
    S = 2 + seed % 4
    c = random_small(600 + seed, n_docs=700 + 150 * seed, n_sources=S, max_strata=1 + seed % 3, T=64,
                     B=[1, 3, 4, 7, 8, 5, 16, 2][seed], max_len=130, prompts=bool(seed % 2),
                     bp_max=6000 if heldout else 1500)
    w = r.integers(1, 50, size=S).astype(np.uint64)
    w[0] = 1 if seed % 2 else w[0]                     # a small share
    w[-1] = 40 * int(w.sum()) if seed % 3 == 0 else w[-1]  # a dominant one
    c = c.replace(weight=w, wrap=wrap, read_random=read_random, heldout=heldout, cumulative=True)
    _parity_run(c, "cumulative-modes", seed)


@pytest.mark.parametrize("upc,ramp", [(1, None), (2, None), (3, None), (2, ((0, 128), (700, 320), (2000, 64))),
                                      (5, ((0, 128), (700, 320), (2000, 64)))])
def test_cumulative_short_cycles(upc, ramp):
    """Short cycles of the cumulative schedule: windows due after a cycle's last
    update still order the seats by their true due updates, cycle after cycle."""
    c = random_small(900 + upc, n_docs=900, n_sources=4, T=64, B=5, max_len=120, prompts=True, bp_max=1000)
    c = c.replace(weight=np.array([1, 3, 40, 7], np.uint64), cumulative=True, updates_per_cycle=upc, ramp=ramp)
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    for cyc in range(6):
        try:
            oi = op.cycle(cyc)
        except oracle.OracleError as e:
            with pytest.raises(dp.DpackError) as ge:
                pk.cycle(cyc)
            assert ge.value.code == e.code
            break
        say("short cycles", upc, "cycle", cyc)
        gi = pk.cycle(cyc)
        compare_cycle(gi, oi, op)
        assert np.array_equal(pk.inspect("cum_taken"), op.cumulative_taken().ravel())
        compare_batch(to_np(pk.batch(0, oi.n_updates)), op.batch(0, oi.n_updates), f"short {upc} cycle {cyc}")
    pk.close()


@pytest.mark.parametrize("S,B", [(70, 128), (130, 64)])
def test_cumulative_many_sources(S, B):
    """More sources than one wavefront holds: the schedule runs on a whole workgroup."""
    c = random_small(700, n_docs=6000, n_sources=S, max_strata=2, T=64, B=B, max_len=60, bp_max=500)
    _parity_run(c.replace(cumulative=True), "cumulative-many-sources", S)


MANY_SOURCE_SCHEDULES = [
    # (S, B, ramp, updates per cycle, tiny shares): schedules of many updates on the several-wavefront path
    (70, 50, None, 0, False),
    (130, 96, None, 0, True),
    (257, 200, ((0, 120 * 64), (40 * 120 * 64, 200 * 64)), 0, True),
    (1024, 300, None, 0, True),
    (1024, 1500, None, 12, False),
]


@pytest.mark.parametrize("case", range(len(MANY_SOURCE_SCHEDULES)))
def test_cumulative_many_sources_long_schedules(case):
    """More sources than a wavefront over a cycle of many updates: weights near
    each source's share of the tokens (so the schedule runs until the corpus is
    nearly used), some of them tiny (windows due thousands of updates ahead),
    with a batch-size ramp, up to 1,024 sources, and a cycle cut by its update
    count; the per-update table, batches and fingerprints equal the oracle's."""
    S, B, ramp, upc, tiny = MANY_SOURCE_SCHEDULES[case]
    c = random_small(800 + case, n_docs=min(200 * S, 100000), n_sources=S, max_strata=2, T=64, B=B, max_len=100,
                     bp_max=300, updates_per_cycle=upc)
    r = np.random.default_rng(810 + case)
    L = np.diff(c.offsets.astype(np.int64))
    tok = np.bincount(c.source.astype(np.int64), weights=L, minlength=S)
    w = np.round(tok * r.uniform(0.8, 1.2, size=S)).astype(np.uint64)
    if tiny:
        w[r.choice(S, size=max(2, S // 16), replace=False)] = 1
    w[tok == 0] = 0
    c = c.replace(weight=w, cumulative=True, ramp=ramp)
    _parity_run(c, "cumulative-many-sources-long", case)


def test_cumulative_small_share_parity():
    """A source below half a window per update: no windows under the fixed
    apportionment, its windows under the cumulative quotas."""
    c = _explicit([40, 20, 64, 10, 30] * 60, 64, 4, sources=[0, 1, 1, 1, 1] * 60, weights=[1, 60])
    op = oracle.Plan(c.replace(cumulative=True))
    assert op.cycle(0).taken[0] > 0
    _parity_run(c.replace(cumulative=True), "cumulative-small-share", 0)


INTEGRAL_CASES = [
    # (seed, sources, weights, B, ramp, lanes, updates per cycle): every update's seats times every weight
    # a multiple of the weights' sum, so every cumulative quota is an integer
    (0, 1, [5], 5, None, 1, 0),
    (1, 3, [1, 1, 2], 8, None, 1, 0),
    (2, 2, [1, 3], 16, ((0, 256), (700, 512), (2000, 1024)), 1, 0),
    (3, 2, [1, 1], 8, None, 2, 0),
    (4, 2, [1, 1], 6, None, 1, 3),
    (5, 3, [0, 2, 2], 4, None, 1, 2),
    (6, 1, [7], 3, ((0, 192), (900, 64)), 1, 4),
]


@pytest.mark.parametrize("case", range(len(INTEGRAL_CASES)))
def test_cumulative_integral_quotas(case):
    """Cumulative quotas that are integers every update (one source, or shares
    dividing every batch): the schedule's closed form, cycle after cycle until
    a source runs out, with a ramp, lanes and fixed cycle lengths."""
    seed, S, w, B, ramp, L, upc = INTEGRAL_CASES[case]
    c = random_small(950 + seed, n_docs=800, n_sources=S, max_strata=2, T=64, B=B, max_len=150,
                     prompts=bool(seed % 2), bp_max=1000)
    c = c.replace(weight=np.array(w, np.uint64), cumulative=True, ramp=ramp, lanes=L, updates_per_cycle=upc)
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    for cyc in range(4):
        try:
            oi = op.cycle(cyc)
        except oracle.OracleError as e:
            with pytest.raises(dp.DpackError) as ge:
                pk.cycle(cyc)
            assert ge.value.code == e.code
            break
        say("integral quotas", case, "cycle", cyc, "updates", oi.n_updates)
        compare_cycle(pk.cycle(cyc), oi, op)
        assert np.array_equal(pk.inspect("cum_taken"), op.cumulative_taken().ravel())
        n = oi.n_updates
        compare_batch(to_np(pk.batch(0, n)), op.batch(0, n), f"integral {case} cycle {cyc}")
    pk.close()


RAMP_CASES = [
    # (seed, ramp pieces (from tokens, tokens per update), B, cumulative, read_random, wrap, updates per cycle)
    (0, ((0, 128), (1000, 256), (3000, 512)), 8, False, False, False, 3),
    (1, ((0, 128), (1000, 256), (3000, 512)), 8, True, False, False, 3),
    (2, ((0, 512), (700, 64), (2000, 320)), 8, False, True, False, 0),
    (3, ((0, 512), (700, 64), (2000, 320)), 8, True, True, True, 0),
    (4, ((0, 64), (640, 192), (5000, 384)), 6, True, False, True, 5),
    (5, ((0, 256),), 4, False, False, False, 4),
    (6, ((0, 256), (900, 128), (2600, 512)), 8, True, True, True, 0),
]


def _ramp_corpus(seed, ramp, B, cumulative, read_random, wrap, upc):
    c = random_small(800 + seed, n_docs=900, n_sources=2 + seed % 3, max_strata=2, T=64, B=B, max_len=150,
                     prompts=bool(seed % 2), bp_max=1500)
    return c.replace(ramp=ramp, cumulative=cumulative, read_random=read_random, wrap=wrap, updates_per_cycle=upc)


@pytest.mark.parametrize("case", range(len(RAMP_CASES)))
def test_ramp_parity(case):
    """Batch-size ramp: every cycle's batches, counts, digest and outputs (ragged
    layout), learned counts and fingerprints against the oracle, across cycles."""
    seed, ramp, B, cum, rr, wrap, upc = RAMP_CASES[case]
    c = _ramp_corpus(seed, ramp, B, cum, rr, wrap, upc)
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    compare_plan(pk, op)
    for cyc in range(4):
        try:
            oi = op.cycle(cyc)
        except oracle.OracleError as e:
            with pytest.raises(dp.DpackError) as ge:
                pk.cycle(cyc)
            assert ge.value.code == e.code
            break
        say("ramp", case, "cycle", cyc, "U", oi.n_updates, "batches", oi.batches.tolist()[:8])
        gi = pk.cycle(cyc)
        compare_cycle(gi, oi, op)
        assert gi["batches"].tolist() == oi.batches.tolist()
        assert np.array_equal(pk.inspect("cum_taken"), op.cumulative_taken().ravel())
        U = oi.n_updates
        for st in sorted({0, max(0, U // 2 - 1), max(0, U - 2)}):
            n = min(2, U - st)
            o = op.batch(st, n)
            g = to_np(pk.batch(st, n))
            compare_batch(g, o, f"ramp{case} cycle {cyc} step {st}")
            fp = pk.fingerprint_steps(st, n, pk.batch(st, n)["digests"]).cpu().numpy()
            x = 0
            for i in range(n):
                Bb = int(oi.batches[st + i])
                assert fp[i].tobytes() == oracle.batch_fingerprint(o["digests"][x:x + Bb])
                x += Bb
    pk.close()


@pytest.mark.parametrize("case", [0, 1, 6])  # every piece's batch even: two ranks
def test_ramp_rank_slices_and_packed_rows(case):
    """Each rank's slice of every update (world 2) and padding-free rows of a ramped cycle."""
    seed, ramp, B, cum, rr, wrap, upc = RAMP_CASES[case]
    c = _ramp_corpus(seed, ramp, B, cum, rr, wrap, upc)
    op = oracle.Plan(c)
    oi = op.cycle(0)
    n = min(6, oi.n_updates)
    for rank in range(2):
        say("ramp-ranks", case, "rank", rank)
        pk = dp.Packer(c, rank=rank, world=2)
        pk.cycle(0)
        compare_batch(to_np(pk.batch(0, n)), op.batch(0, n, rank=rank, world=2), f"ramp{case} rank {rank}")
        g = {k: (v.cpu().numpy() if v is not None else None) for k, v in pk.batch_packed(0, n, 64).items()}
        o = op.batch_packed(0, n, rank=rank, world=2, bucket=64)
        assert np.array_equal(g["row_start"], o["row_start"]) and np.array_equal(g["length"], o["length"])
        for i in range(n):
            L = int(o["length"][i])
            for k in ("tokens", "pos", "doc", "mask"):
                a = g[k][i, :L].view(np.uint32) if k == "tokens" else g[k][i, :L]
                assert np.array_equal(a, o[k][i, :L]), (i, k)
        pk.close()


def test_ramp_fingerprint_needs_steps():
    """pack_fingerprint cannot tell a ramp's batch sizes apart: it refuses."""
    seed, ramp, B, cum, rr, wrap, upc = RAMP_CASES[0]
    c = _ramp_corpus(seed, ramp, B, cum, rr, wrap, upc)
    pk = dp.Packer(c)
    pk.cycle(0)
    d = pk.batch(0, 1)["digests"]
    with pytest.raises(dp.DpackError) as e:
        pk.fingerprint(d.reshape(1, -1, 32))
    assert e.value.code == dp.PACK_E_STATE
    pk.close()


LANE_CASES = [
    # (seed, lanes, B, cumulative, ramp, wrap, read_random, heldout)
    (0, 2, 8, False, None, False, False, False),
    (1, 4, 8, False, None, True, False, False),
    (2, 3, 9, True, None, False, True, False),
    (3, 8, 16, False, None, False, False, True),
    (4, 2, 8, True, ((0, 256), (900, 512)), False, False, False),
    (5, 4, 8, False, ((0, 256), (600, 512), (2400, 256)), True, True, False),
    (6, 2, 6, True, None, True, True, True),
]


def _lane_corpus(seed, L, B, cum, ramp, wrap, rr, held):
    c = random_small(1200 + seed, n_docs=1200, n_sources=2 + seed % 3, max_strata=3, T=64, B=B, max_len=130,
                     prompts=bool(seed % 2), bp_max=6000 if held else 1500)
    return c.replace(lanes=L, cumulative=cum, ramp=ramp, wrap=wrap, read_random=rr, heldout=held)


@pytest.mark.parametrize("case", range(len(LANE_CASES)))
def test_lanes_parity(case):
    """Zephon lanes: streams per (source, lane), per-lane slots, with the other modes."""
    c = _lane_corpus(*LANE_CASES[case])
    if c.ramp is None:
        _parity_run(c, "lanes", case)
        return
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    compare_plan(pk, op)
    oi = op.cycle(0)
    gi = pk.cycle(0)
    compare_cycle(gi, oi, op)
    assert np.array_equal(pk.inspect("cum_taken"), op.cumulative_taken().ravel())
    n = min(4, oi.n_updates)
    compare_batch(to_np(pk.batch(0, n)), op.batch(0, n), f"lanes{case}")
    pk.close()


@pytest.mark.parametrize("case", [0, 1, 4])
def test_lanes_each_rank_takes_whole_lanes(case):
    """Every rank count dividing the lanes gives the same global batches."""
    c = _lane_corpus(*LANE_CASES[case])
    op = oracle.Plan(c)
    oi = op.cycle(0)
    n = min(3, oi.n_updates)
    for world in sorted({1, 2, c.lanes}):
        for rank in sorted({0, world - 1}):
            say("lanes-ranks", case, "world", world, "rank", rank)
            pk = dp.Packer(c, rank=rank, world=world)
            pk.cycle(0)
            compare_batch(to_np(pk.batch(0, n)), op.batch(0, n, rank=rank, world=world), f"lanes{case} {rank}/{world}")
            pk.close()


RESUME_MODES = [dict(), dict(wrap=True), dict(read_random=True), dict(cumulative=True),
                dict(ramp=((0, 128), (900, 384), (2500, 192))), dict(lanes=2), dict(heldout=True, wrap=True),
                dict(cumulative=True, lanes=3, ramp=((0, 192), (1200, 384)), read_random=True)]


def _resume_corpus(seed, **mode):
    held = mode.get("heldout", False)
    c = random_small(1300 + seed, n_docs=900, n_sources=3, max_strata=2, T=64, B=6, max_len=200, prompts=True,
                     bp_max=6000 if held else 1500)
    return c.replace(updates_per_cycle=3, **mode)


@pytest.mark.parametrize("mi", range(len(RESUME_MODES)))
def test_resume_at_reported_tokens(mi):
    """A context cut from the tokens the GPU reports after a cycle goes on where the
    first one would have: the same T gives its next cycle byte for byte; another T
    matches the oracle's re-cut."""
    c = _resume_corpus(mi, **RESUME_MODES[mi])
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    oi0 = op.cycle(0)
    gi0 = pk.cycle(0)
    compare_cycle(gi0, oi0, op)
    oi1 = op.cycle(1)
    gi1 = pk.cycle(1)
    nxt = gi0["stream_next_token"].copy()
    cr = c.replace(start_tokens=nxt, first_cycle=1, tokens_start=int(gi0["positions"]))
    say("resume", mi, "same T")
    pb = dp.Packer(cr)
    ob = oracle.Plan(cr)
    compare_plan(pb, ob)
    gb = pb.cycle(1)
    compare_cycle(gb, ob.cycle(1), ob)
    assert gb["n_updates"] == gi1["n_updates"] and gb["windows_taken"].tolist() == gi1["windows_taken"].tolist()
    n = gb["n_updates"]
    compare_batch(to_np(pb.batch(0, n)), to_np(pk.batch(0, n)), f"resume {mi}: next cycle")
    pb.close()
    for T2 in ((128, 320) if c.ramp is None else ()):  # a ramp's tokens per update are multiples of its T
        say("resume", mi, "T", T2)
        c2 = cr.replace(T=T2)
        o2 = oracle.Plan(c2)
        try:
            oi2 = o2.cycle(1)
        except oracle.OracleError as e:
            with pytest.raises(dp.DpackError) as ge:
                dp.Packer(c2).cycle(1)
            assert ge.value.code == e.code
            continue
        p2 = dp.Packer(c2)
        compare_plan(p2, o2)
        compare_cycle(p2.cycle(1), oi2, o2)
        m = min(3, oi2.n_updates)
        compare_batch(to_np(p2.batch(0, m)), o2.batch(0, m), f"resume {mi} T {T2}")
        p2.close()
    pk.close()


SEG_CASES = [(0, 2, dict()), (1, 3, dict(wrap=True)), (2, 5, dict(lanes=2)), (3, 3, dict(cumulative=True)),
             (4, 4, dict(read_random=True, ramp=((0, 128), (1500, 384)))), (5, 2, dict(heldout=True))]


@pytest.mark.parametrize("case", range(len(SEG_CASES)))
def test_arrivals_parity(case):
    """Streamed corpora: documents ordered arrival by arrival, with the other modes."""
    from test_oracle_segments import _arrivals
    seed, n_seg, mode = SEG_CASES[case]
    c, _ = _arrivals(1400 + seed, n_seg)
    if mode.get("heldout"):
        c = c.replace(holdout_bp=np.full(c.n_sources, 5000, np.uint32))
    _parity_run(c.replace(**mode), "arrivals", case)


@pytest.mark.parametrize("mi", range(7))
def test_a_context_per_arrival_on_the_gpu(mi):
    """A context per arrival, each going on from the tokens the previous GPU context
    reported, plans the cycles one context over every arrival plans, in every mode."""
    from test_oracle_segments import ARRIVAL_MODES, _prefix, arrival_corpus
    mode = ARRIVAL_MODES[mi]
    c, cuts = arrival_corpus(1500 + mi, mode)
    full = dp.Packer(c)
    nxt, tokens = None, 0
    for cyc in range(4):
        fi = full.cycle(cyc)
        cc = _prefix(c, int(cuts[cyc + 1])).replace(**mode)
        if cyc:
            cc = cc.replace(start_tokens=nxt, first_cycle=cyc, tokens_start=tokens)
        say("arrival", cyc, "mode", mode)
        part = dp.Packer(cc)
        pi = part.cycle(cyc)
        assert pi["n_updates"] == fi["n_updates"] and pi["windows_taken"].tolist() == fi["windows_taken"].tolist()
        assert pi["batches"].tolist() == fi["batches"].tolist()
        n = pi["n_updates"]
        compare_batch(to_np(part.batch(0, n)), to_np(full.batch(0, n)), f"arrival {cyc}")
        assert pi["stream_next_token"].tolist() == fi["stream_next_token"].tolist()
        nxt, tokens = pi["stream_next_token"].copy(), int(tokens + pi["positions"])
        part.close()
    full.close()


def test_bad_arrival_id_is_an_error():
    from test_oracle_segments import _arrivals
    c, _ = _arrivals(1600, 2)
    seg = c.segment.copy()
    seg[3] = 7
    with pytest.raises(dp.DpackError) as e:
        dp.Packer(c.replace(segment=seg))
    assert e.value.code == dp.PACK_E_INVAL and "arrival" in str(e.value)


PACKED_SHORT = {
    # windows of 1-3 real positions, many of them inside one 16-byte store group of the row
    "split_130": (lambda: _explicit([130] * 20, 64, 3), 1),
    "split_66": (lambda: _explicit([66] * 31, 64, 5), 1),
    "mixed_prompts": (lambda: _explicit([130, 3, 1, 2, 67] * 12, 64, 4, prompts=[5, 0, 1, 0, 70] * 12), 2),
}


@pytest.mark.parametrize("name", sorted(PACKED_SHORT))
def test_padding_free_rows_short_windows(name):
    """Every update of a cycle whose windows are shorter than a store group."""
    make, world = PACKED_SHORT[name]
    c = make()
    op = oracle.Plan(c)
    n = op.cycle(0).n_updates
    for rank in sorted({0, world - 1}):
        say("packed-short", name, "world", world, "rank", rank)
        pk = dp.Packer(c, rank=rank, world=world)
        pk.cycle(0)
        g = {k: (v.cpu().numpy() if v is not None else None) for k, v in pk.batch_packed(0, n, 8).items()}
        o = op.batch_packed(0, n, rank=rank, world=world, bucket=8)
        lens = np.diff(o["row_start"], axis=1)
        assert ((lens > 0) & (lens < 4)).any()
        assert np.array_equal(g["row_start"], o["row_start"]) and np.array_equal(g["length"], o["length"])
        for i in range(n):
            L = int(o["length"][i])
            for k in ("tokens", "pos", "doc", "mask"):
                a = g[k][i, :L].view(np.uint32) if k == "tokens" else g[k][i, :L]
                assert np.array_equal(a, o[k][i, :L]), (i, k)
        pk.close()


HELDOUT_CASES = [(s, w) for s in range(6) for w in (False, True)]


@pytest.mark.parametrize("seed,wrap", HELDOUT_CASES)
def test_heldout_stream_parity(seed, wrap):
    """The held-out (validation) stream, PACK_FLAG_HELDOUT, with both packings."""
    c = random_small(1000 + seed, n_docs=300 + 100 * seed, n_sources=1 + seed % 3, max_strata=1 + seed % 3,
                     T=64, B=1 + seed % 4, max_len=120, prompts=bool(seed % 2), bp_max=6000)
    _parity_run(c.replace(heldout=True, wrap=wrap), "heldout" + ("-wrap" if wrap else ""), seed)


def _parity_run(c, kind, arg):
    say("plan/cycle/batch", kind, arg, "docs", c.n_docs, "T", c.T, "B", c.B)
    cyc = int(getattr(c, "first_cycle", 0))  # the first cycle the context plans
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    compare_plan(pk, op)
    try:
        oi = op.cycle(cyc)
    except oracle.OracleError as e:
        with pytest.raises(dp.DpackError) as ge:
            pk.cycle(cyc)
        assert ge.value.code == e.code
        return
    gi = pk.cycle(cyc)
    compare_cycle(gi, oi, op)
    # the library's per-update batches (the binding reads them only with a ramp)
    assert pk.inspect("update_batch").tolist() == [int(x) for x in oi.batches]
    if getattr(c, "cumulative", False):
        assert np.array_equal(pk.inspect("cum_taken"), op.cumulative_taken().ravel())
    U = oi.n_updates
    steps = list(range(0, U, max(1, U // 6)))[:6]
    for st in steps:
        n = min(3, U - st)
        say("batch", kind, arg, "step", st, "n", n)
        o = op.batch(st, n)
        g = to_np(pk.batch(st, n))
        compare_batch(g, o, f"{kind}{arg} step {st}")
        if getattr(c, "ramp", None) is None:
            fp = pk.fingerprint(pk.batch(st, n)["digests"]).cpu().numpy()
            for i in range(n):
                assert fp[i].tobytes() == oracle.batch_fingerprint(o["digests"][i])
        else:  # batches of a ramp: each update's own digests
            fp = pk.fingerprint_steps(st, n, pk.batch(st, n)["digests"]).cpu().numpy()
            x = 0
            for i in range(n):
                Bb = int(oi.batches[st + i])
                assert fp[i].tobytes() == oracle.batch_fingerprint(o["digests"][x:x + Bb])
                x += Bb
    pk.close()


@pytest.mark.parametrize("seed", range(24))
def test_mode_combinations(seed):
    """Seeded random combinations of every mode (wrap, random read order,
    cumulative mixture, lanes, batch-size ramp, held-out stream, arrivals,
    stream starts) on small corpora: plan, cycle, batches and fingerprints
    against the oracle."""
    from _combos import combo_corpus
    c, desc = combo_corpus(seed)
    say("combination", seed, desc)
    _parity_run(c, "combo", seed)


@pytest.mark.parametrize("seed", range(24))
def test_mode_combinations_two_ranks(seed):
    """The combinations with even batches and even lane counts at world 2: each
    rank's slice equals the oracle's, and the two slices side by side equal the
    world-1 batch (tokens, document ids and window digests)."""
    from _combos import combo_corpus
    c, desc = combo_corpus(seed, even=True)
    ramp = getattr(c, "ramp", None)
    L = max(1, int(getattr(c, "lanes", 1) or 1))
    assert L == 1 or L % 2 == 0, "ranks take whole lanes"
    cyc = int(getattr(c, "first_cycle", 0))
    op = oracle.Plan(c)
    oi = op.cycle(cyc)
    n = min(3, oi.n_updates)
    whole = op.batch(0, n)
    parts = []
    for r in range(2):
        say("combination", seed, desc, "rank", r)
        pk = dp.Packer(c, rank=r, world=2)
        pk.cycle(cyc)
        g = to_np(pk.batch(0, n))
        compare_batch(g, op.batch(0, n, rank=r, world=2), f"combo {seed} rank {r}")
        parts.append(g)
        pk.close()
    if ramp is None:  # [n, B/2, T] side by side
        for k in ("tokens", "doc", "digests"):
            assert np.array_equal(np.concatenate([x[k] for x in parts], axis=1), whole[k])
    else:  # each update's windows: rank 0's half, then rank 1's
        off, offs = 0, [0, 0]
        for b in range(n):
            Bb = int(oi.batches[b])
            for r in range(2):
                for k in ("tokens", "doc", "digests"):
                    seg = parts[r][k][offs[r]:offs[r] + Bb // 2]
                    assert np.array_equal(seg, whole[k][off + r * (Bb // 2):off + (r + 1) * (Bb // 2)]), (b, r, k)
                offs[r] += Bb // 2
            off += Bb


@pytest.mark.parametrize("kind,arg,worlds", [("tiny", 0.5, [1, 2, 4, 8]), ("pretrain", 0.006, [1, 8, 16, 32, 64]),
                                             ("small", 4, [1, 2, 4, 8]), ("wrap-pretrain", 0.006, [1, 8, 64]),
                                             ("heldout", 1100, [1, 2, 4, 8]), ("random-tiny", 0.5, [1, 2, 4, 8]),
                                             ("cum-pretrain", 0.006, [1, 8, 64]), ("cum-tiny", 0.5, [1, 2, 8])])
def test_elastic_rank_counts_identical(kind, arg, worlds):
    if kind == "heldout":  # a held-out stream large enough for B = 8
        c = random_small(arg, n_docs=2000, n_sources=2, T=64, B=8, max_len=60, bp_max=6000).replace(heldout=True)
    else:
        mode, _, base = kind.partition("-") if "-" in kind else ("", "", kind)
        c = _corpus(base, arg).replace(wrap=mode == "wrap", read_random=mode == "random", cumulative=mode == "cum")
    if kind == "small":
        c = c.replace(B=8)
    if kind.endswith("pretrain"):
        c = c.replace(updates_per_cycle=2)
    op = oracle.Plan(c)
    op.cycle(0)
    n = min(2, op.cycle_info.n_updates)
    ref = op.batch(0, n)
    ref_fp = [oracle.batch_fingerprint(ref["digests"][i]) for i in range(n)]
    tensors = dp.upload_corpus(c)
    for R in worlds:
        say("elastic", kind, arg, "world", R)
        parts = []
        for r in range(R):
            pk = dp.Packer(c, rank=r, world=R, device_tensors=tensors)  # an independent context per rank
            pk.cycle(0)
            parts.append(to_np(pk.batch(0, n)))
            pk.close()
        cat = {k: np.concatenate([p[k] for p in parts], axis=1) for k in ("tokens", "pos", "doc", "mask", "digests")}
        cat["learned"] = parts[0]["learned"]
        for p in parts:
            assert np.array_equal(p["learned"], ref["learned"])
        compare_batch(cat, ref, f"world {R}")
        fps = [oracle.batch_fingerprint(cat["digests"][i]) for i in range(n)]
        assert fps == ref_fp


def test_world_not_dividing_batch_fails_at_init():
    c = make_corpus("tiny", 0.2)
    for R in (3, 16, 64):
        with pytest.raises(dp.DpackError) as e:
            dp.Packer(c, rank=0, world=R)
        assert e.value.code == dp.PACK_E_INVAL


@pytest.mark.parametrize("read_random,cumulative", [(False, False), (True, False), (False, True), (True, True)])
def test_cycles_until_exhausted_match_oracle(read_random, cumulative):
    c = random_small(40, n_docs=400, n_sources=3, T=64, B=6, max_len=100, prompts=True, updates_per_cycle=2)
    c = c.replace(read_random=read_random, cumulative=cumulative)
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    compare_plan(pk, op)
    for cyc in range(100):
        try:
            oi = op.cycle(cyc)
        except oracle.OracleError as e:
            assert e.code == oracle.OR_E_EXHAUSTED
            with pytest.raises(dp.DpackError) as ge:
                pk.cycle(cyc)
            assert ge.value.code == dp.PACK_E_EXHAUSTED
            break
        say("cycle", cyc)
        compare_cycle(pk.cycle(cyc), oi, op)
        if cumulative:
            assert np.array_equal(pk.inspect("cum_taken"), op.cumulative_taken().ravel())
        compare_batch(to_np(pk.batch(0, oi.n_updates)), op.batch(0, oi.n_updates), f"cycle {cyc}")
    else:
        pytest.fail("never exhausted")
    pk.close()


def test_call_order_errors():
    c = random_small(41, n_docs=200, T=64, B=4, max_len=80)
    pk = dp.Packer(c)
    with pytest.raises(dp.DpackError) as e:
        pk.batch(0, 1)
    assert e.value.code == dp.PACK_E_STATE
    with pytest.raises(dp.DpackError) as e:
        pk.cycle(1)
    assert e.value.code == dp.PACK_E_STATE
    info = pk.cycle(0)
    with pytest.raises(dp.DpackError) as e:
        pk.batch(info["n_updates"], 1)
    assert e.value.code == dp.PACK_E_RANGE
    with pytest.raises(dp.DpackError) as e:
        pk.batch(0, 0)
    assert e.value.code == dp.PACK_E_RANGE
    pk.close()


def _bad_corpus(kind):
    c = random_small(42, n_docs=50, T=64, B=2, max_len=40, zero_len_frac=0.0)
    if kind == "offsets":
        off = c.offsets.copy()
        off[11] = off[10] - 1  # document 10 gets a negative length
        return c.replace(offsets=off)
    if kind == "source":
        src = c.source.copy()
        src[7] = c.n_sources
        return c.replace(source=src)
    if kind == "stratum":
        st = c.stratum.copy()
        st[5] = c.n_strata[c.source[5]]
        return c.replace(stratum=st)
    if kind == "tokens":
        return c.replace(tokens=c.tokens[:-5].copy())
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["offsets", "source", "stratum", "tokens"])
def test_invalid_corpus_rejected_by_validation_kernel(kind):
    c = _bad_corpus(kind)
    say("invalid corpus", kind)
    with pytest.raises(dp.DpackError) as e:
        dp.Packer(c)
    assert e.value.code == dp.PACK_E_INVAL


def test_all_held_out_is_exhausted_not_a_fault():
    c = random_small(43, n_docs=100, T=64, B=2, max_len=50)
    c = c.replace(holdout_bp=np.full(c.n_sources, 10000, np.uint32))
    op = oracle.Plan(c)
    assert op.order.size == 0
    pk = dp.Packer(c)
    compare_plan(pk, op)
    with pytest.raises(dp.DpackError) as e:
        pk.cycle(0)
    assert e.value.code == dp.PACK_E_EXHAUSTED


def _explicit(lengths, T, B, sources=None, strata=None, n_strata=None, weights=None, prompts=None, bp=None):
    L = np.asarray(lengths, np.int64)
    D = L.shape[0]
    off = np.zeros(D + 1, np.uint64)
    np.cumsum(L, out=off[1:])
    r = np.random.default_rng(D)
    src = np.zeros(D, np.uint16) if sources is None else np.asarray(sources, np.uint16)
    S = int(src.max()) + 1 if D else 1
    st = np.zeros(D, np.uint16) if strata is None else np.asarray(strata, np.uint16)
    ns = np.ones(S, np.uint32) if n_strata is None else np.asarray(n_strata, np.uint32)
    w = np.ones(S, np.uint64) if weights is None else np.asarray(weights, np.uint64)
    return Corpus("edge", r.integers(0, 50000, size=int(off[-1]), dtype=np.uint32), off, src, st,
                  None if prompts is None else np.asarray(prompts, np.uint32), ns, w,
                  np.zeros(S, np.uint32) if bp is None else np.asarray(bp, np.uint32), T=T, B=B,
                  updates_per_cycle=0, seed=7, pad_token=99)


EDGE = {
    "exact_T": lambda: _explicit([64] * 10 + [128, 192, 1], 64, 2),
    "one_token_docs": lambda: _explicit([1] * 300, 64, 1),
    "one_long_doc": lambda: _explicit([64 * 37 + 5], 64, 1),
    "ragged_many_pieces": lambda: _explicit([1, 2, 3, 600, 1, 63, 65, 2] * 40, 64, 4),
    "empty_docs_and_source": lambda: _explicit([0, 5, 0, 70, 3, 0] * 20, 64, 2,
                                              sources=[0, 0, 2, 2, 0, 2] * 20, weights=[3, 0, 5]),
    "empty_stratum": lambda: _explicit([10, 20, 30, 40] * 30, 64, 2, strata=[0, 2, 0, 2] * 30, n_strata=[3]),
    "tiny_share_zero_seats": lambda: _explicit([30] * 200, 64, 4, sources=[0, 1] * 100, weights=[1000, 1]),
    "prompt_beyond_doc": lambda: _explicit([10, 100, 200] * 30, 64, 2, prompts=[50, 3, 150] * 30),
    "many_pieces_window": lambda: _explicit([1] * 5000, 4096, 1),
    "single_document": lambda: _explicit([37], 64, 1),
    "one_nonempty_among_empty": lambda: _explicit([0, 0, 0, 130, 0, 0], 64, 1),
    "prompts_cover_everything": lambda: _explicit([10, 70, 200, 3] * 20, 64, 2, prompts=[10, 80, 200, 9] * 20),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases(name):
    _edge_run(EDGE[name](), name)


@pytest.mark.parametrize("name", sorted(EDGE))
def test_wrap_edge_cases(name):
    _edge_run(EDGE[name]().replace(wrap=True), "wrap-" + name)


def _edge_run(c, name):
    say("edge", name)
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    compare_plan(pk, op)
    try:
        oi = op.cycle(0)
    except oracle.OracleError as e:
        with pytest.raises(dp.DpackError) as ge:
            pk.cycle(0)
        assert ge.value.code == e.code
        return
    gi = pk.cycle(0)
    compare_cycle(gi, oi, op)
    n = min(oi.n_updates, 8)
    compare_batch(to_np(pk.batch(0, n)), op.batch(0, n), name)


def _max_case(name):
    """Corpora at the limits the library documents (sources, groups, token ids,
    window length, windows per update), small enough for the oracle."""
    r = np.random.default_rng(np.random.SeedSequence([31, len(name)]))
    vocab = 50000
    if name == "max_sources":  # 4,096 sources: per-source statistics past the LDS bins
        S, D, T, B = 4096, 60000, 64, 64
        L = r.integers(1, 200, size=D)
        src = r.integers(0, S, size=D).astype(np.uint16)
        st, ns = np.zeros(D, np.uint16), np.ones(S, np.uint32)
        w, bp = r.integers(1, 1000, size=S).astype(np.uint64), r.integers(0, 3000, size=S).astype(np.uint32)
    elif name == "max_groups":  # 16 sources x 4,096 strata = 65,536 groups, most of them empty
        S, D, T, B = 16, 40000, 64, 16
        L = r.integers(1, 150, size=D)
        src, st = r.integers(0, S, size=D).astype(np.uint16), r.integers(0, 4096, size=D).astype(np.uint16)
        ns = np.full(S, 4096, np.uint32)
        w, bp = r.integers(1, 100, size=S).astype(np.uint64), np.full(S, 100, np.uint32)
    elif name == "full_range_tokens":  # token ids over all of [0, 2^32)
        S, D, T, B = 3, 3000, 128, 4
        L = r.integers(0, 700, size=D)
        src, st, ns = r.integers(0, S, size=D).astype(np.uint16), np.zeros(D, np.uint16), np.ones(S, np.uint32)
        w, bp = np.array([5, 3, 2], np.uint64), np.array([500, 100, 2000], np.uint32)
        vocab = 2**32
    elif name == "long_windows":  # T = 65,536: 13,313 compressions per window record
        S, D, T, B = 2, 400, 65536, 2
        L = r.integers(1, 150000, size=D)
        src, st, ns = r.integers(0, S, size=D).astype(np.uint16), np.zeros(D, np.uint16), np.ones(S, np.uint32)
        w, bp = np.array([1, 1], np.uint64), np.array([100, 100], np.uint32)
    elif name == "max_arrivals":  # 30,000 arrivals of one source: 30,001 group bases staged at init
        S, D, T, B = 1, 60000, 64, 8
        L = r.integers(1, 120, size=D)
        src, st, ns = np.zeros(D, np.uint16), np.zeros(D, np.uint16), np.ones(S, np.uint32)
        w, bp = np.array([1], np.uint64), np.array([300], np.uint32)
    else:  # wide_update: 65,536 windows in one update, three updates in one emission-and-digest
        # launch (196,608 windows: 768 workgroups, three times as many as the CUs)
        S, D, T, B = 2, 230000, 64, 65536
        L = r.integers(20, 64, size=D)
        src, st, ns = r.integers(0, S, size=D).astype(np.uint16), np.zeros(D, np.uint16), np.ones(S, np.uint32)
        w, bp = np.array([1, 1], np.uint64), np.zeros(S, np.uint32)
    order = np.lexsort((st, src))
    src, st, L = src[order], st[order], L[order]
    off = np.zeros(D + 1, np.uint64)
    np.cumsum(L, out=off[1:])
    tok = r.integers(0, vocab, size=int(off[-1]), dtype=np.uint64).astype(np.uint32)
    pl = np.minimum(r.integers(0, 100, size=D), L).astype(np.uint32)
    c = Corpus(name, tok, off, src, st, pl, ns, w, bp, T=T, B=B, updates_per_cycle=0, seed=11, pad_token=7)
    if name == "max_arrivals":
        c = c.replace(segment=r.integers(0, 30000, size=D).astype(np.uint16), n_segments=30000)
    return c


@pytest.mark.parametrize("name", ["max_sources", "max_groups", "max_arrivals", "full_range_tokens", "long_windows",
                                  "wide_update"])
def test_maximum_sizes(name):
    _edge_run(_max_case(name), name)


def test_two_contexts_on_two_streams():
    """Two contexts alive at once, each on its own stream, their batches issued
    interleaved: each equals what a context alone emits (own workspace each,
    stream-ordered work only)."""
    import torch
    ca, cb = make_corpus("sft", 0.003), random_small(77, n_docs=900, n_sources=3, max_strata=2, T=128, B=4,
                                                      max_len=300, prompts=True, bp_max=1500)
    ref = {}
    for name, c in (("a", ca), ("b", cb)):
        pk = dp.Packer(c)
        n = min(pk.cycle(0)["n_updates"], 6)
        ref[name] = (n, to_np(pk.batch(0, n)))
        pk.close()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ta, tb = dp.upload_corpus(ca), dp.upload_corpus(cb)
    torch.cuda.synchronize()  # the corpora are resident before other streams read them
    pa, pb = dp.Packer(ca, stream=sa, device_tensors=ta), dp.Packer(cb, stream=sb, device_tensors=tb)
    pa.cycle(0)
    pb.cycle(0)
    outs = {"a": pa.alloc_out(ref["a"][0]), "b": pb.alloc_out(ref["b"][0])}
    torch.cuda.synchronize()
    for i in range(max(ref["a"][0], ref["b"][0])):  # one update at a time, alternating streams
        for name, pk in (("a", pa), ("b", pb)):
            if i < ref[name][0]:
                one = {k: (v[i:i + 1] if v is not None else None) for k, v in outs[name].items()}
                pk.batch_into(i, 1, one)
    torch.cuda.synchronize()
    for name in ("a", "b"):
        got = to_np(outs[name])
        for k, v in ref[name][1].items():
            assert np.array_equal(got[k], v), (name, k)
    pa.close()
    pb.close()


def test_reemission_and_reinit_are_bytewise_identical():
    c = make_corpus("sft", 0.002)
    a = dp.Packer(c)
    a.cycle(0)
    x = to_np(a.batch(1, 3))
    y = to_np(a.batch(1, 3))
    b = dp.Packer(c)
    b.cycle(0)
    z = to_np(b.batch(1, 3))
    for k in x:
        assert np.array_equal(x[k], y[k]) and np.array_equal(x[k], z[k]), k


def test_timing_flags_change_no_output():
    """PACK_FLAG_TIMING times every phase, PACK_FLAG_TIMING_BATCH only the batch
    and fingerprint calls' phases; neither changes an output byte."""
    c = make_corpus("sft", 0.002)
    outs, tms = {}, {}
    for timing in (False, True, "batch"):
        pk = dp.Packer(c, timing=timing)
        pk.cycle(0)
        outs[timing] = to_np(pk.batch(0, 2))
        tms[timing] = pk.timings(reset=True)
        pk.close()
    for k in outs[False]:
        assert np.array_equal(outs[False][k], outs[True][k]) and np.array_equal(outs[False][k], outs["batch"][k]), k
    plan = ("validate", "hash", "keys", "sort", "merge", "pieces", "cut", "windows", "mixture", "cycle")
    assert all(tms[True][p][1] > 0 for p in plan), tms[True]
    assert all(tms["batch"][p][1] == 0 for p in plan), tms["batch"]
    for t in (True, "batch"):
        ms, n = tms[t]["digest"]
        assert n == 1 and ms > 0, tms[t]


# Window lengths that are not multiples of 64 (1, 3 and 17 not even of 4):
# padded windows that start off 16-byte boundaries go through the span writer,
# and the digests come from the emitted outputs, hashed by their own kernel.
ANY_T_CASES = [(1, 4), (3, 3), (17, 5), (60, 4), (100, 4), (130, 2), (1000, 3), (4095, 2), (4097, 2)]


def _any_t(T, B, wrap):
    return random_small(80 + T % 97, n_docs=90, n_sources=2, max_strata=2, T=T, B=B, max_len=max(3, 2 * T),
                        prompts=True, bp_max=1500).replace(wrap=wrap)


@pytest.mark.parametrize("T,B", ANY_T_CASES)
@pytest.mark.parametrize("wrap", [False, True])
def test_any_window_length_parity(T, B, wrap):
    _parity_run(_any_t(T, B, wrap), ("wrap-" if wrap else "") + f"T{T}", B)


@pytest.mark.parametrize("T,B", [(3, 4), (100, 4), (4095, 2)])
def test_any_window_length_without_digests_and_padding_free(T, B):
    """The emission kernel alone, padded and in padding-free rows of two ranks."""
    c = _any_t(T, B, False)
    op = oracle.Plan(c)
    oi = op.cycle(0)
    n = min(4, oi.n_updates)
    say("any T, no digests", T, B)
    pk = dp.Packer(c)
    pk.cycle(0)
    compare_batch(to_np(pk.batch(0, n, digests=False)), op.batch(0, n, digests=False), f"T{T} no digests")
    pk.close()
    for rank in (0, 1):
        say("any T, padding-free rows", T, B, "rank", rank)
        pk = dp.Packer(c, rank=rank, world=2)
        pk.cycle(0)
        g = {k: (v.cpu().numpy() if v is not None else None) for k, v in pk.batch_packed(0, n, 8).items()}
        o = op.batch_packed(0, n, rank=rank, world=2, bucket=8)
        assert np.array_equal(g["row_start"], o["row_start"]) and np.array_equal(g["length"], o["length"])
        for i in range(n):
            L = int(o["length"][i])
            for k in ("tokens", "pos", "doc", "mask"):
                a = g[k][i, :L].view(np.uint32) if k == "tokens" else g[k][i, :L]
                assert np.array_equal(a, o[k][i, :L]), (i, k)
        pk.close()


@pytest.mark.parametrize("T", [4000, 4100])
@pytest.mark.parametrize("wrap", [False, True])
def test_any_window_length_every_digest_of_a_cycle(T, wrap):
    """The pre-train mix at 20,000 documents with T not a multiple of 64: every
    window digest of the cycle (the emission, then the digests from the
    outputs) against the oracle's, and the first and last updates whole."""
    from _gpu_parity import oracle_digests
    c = make_corpus("pretrain", 0.02, T=T, updates_per_cycle=0).replace(wrap=wrap)
    op = oracle.Plan(c)
    oi = op.cycle(0)
    say("any T, whole cycle", T, "wrap", wrap, "updates", oi.n_updates)
    pk = dp.Packer(c)
    compare_cycle(pk.cycle(0), oi, op)
    U = oi.n_updates
    got = pk.batch(0, U)["digests"].cpu().numpy()
    assert np.array_equal(got, oracle_digests(op, range(U)))
    for st in sorted({0, U - 1}):
        compare_batch(to_np(pk.batch(st, 1)), op.batch(st, 1), f"T{T} update {st}")
    pk.close()


# ---------------------------------------------------------------- chunked window digests
CHUNKED_CASES = [("small", 0), ("small", 3), ("small", 5), ("tinydocs", 2), ("sft", 0.004), ("long", 0.01),
                 ("pretrain", 0.006), ("full", 0.002)]


@pytest.mark.parametrize("kind,arg", CHUNKED_CASES)
def test_chunked_digest_parity(kind, arg):
    """PACK_FLAG_DIGEST_CHUNKED: every output and each window's digest over its
    record's 4,096-byte chunk digests equal the oracle's, and so do the batch
    fingerprints taken over them."""
    _parity_run(_corpus(kind, arg).replace(digest_chunked=True), "chunked-" + kind, arg)


@pytest.mark.parametrize("T", [1, 37, 100, 315, 316, 1000, 1024, 1500, 3072, 5000])
def test_chunked_digest_any_window_length(T):
    """Window lengths whose records are one chunk (T ≤ 315), one byte more, whose
    chunks straddle tok, pos, doc and mask (T not a multiple of 1,024: the word by
    word kernel) or lie in one array each (1,024, 3,072: the line kernel)."""
    c = random_small(1200 + T, n_docs=200, n_sources=2, max_strata=2, T=T, B=3, max_len=max(8, 2 * T),
                     prompts=True, bp_max=1000)
    _parity_run(c.replace(digest_chunked=True), "chunked-T", T)


@pytest.mark.parametrize("T", [2048, 1000])
def test_chunked_digests_in_slices(T):
    """With PACK_TEST_DIGEST_SLICES the chunk digests go through slices of three
    windows (a partial last one): the digests are those of one slice and the
    oracle's; the same context without digests emits the same arrays."""
    c = random_small(1300 + T, n_docs=400, n_sources=3, T=T, B=4, max_len=3 * T, bp_max=500).replace(
        digest_chunked=True)
    op = oracle.Plan(c)
    oi = op.cycle(0)
    n = min(4, oi.n_updates)
    o = op.batch(0, n)
    pk = dp.Packer(c)
    pk.cycle(0)
    one = to_np(pk.batch(0, n))
    pk.test_option(dp.PACK_TEST_DIGEST_SLICES, 1)
    sliced = to_np(pk.batch(0, n))
    pk.test_option(dp.PACK_TEST_DIGEST_SLICES, 0)
    plain = to_np(pk.batch(0, n, digests=False))
    assert np.array_equal(one["digests"], sliced["digests"])
    compare_batch(sliced, o, f"chunked slices T={T}")
    for k in ("tokens", "pos", "doc", "mask"):
        assert np.array_equal(plain[k], one[k]), k
    pk.close()


def test_chunked_and_whole_record_digests_differ_arrays_equal():
    """The flag changes the digests only: the same corpus with and without it
    emits the same arrays, and every digest differs."""
    c = _corpus("small", 1)
    a, b = dp.Packer(c), dp.Packer(c.replace(digest_chunked=True))
    a.cycle(0)
    b.cycle(0)
    x, y = to_np(a.batch(0, 2)), to_np(b.batch(0, 2))
    for k in ("tokens", "pos", "doc", "mask", "learned"):
        assert np.array_equal(x[k], y[k]), k
    dx, dy = x["digests"].reshape(-1, 32), y["digests"].reshape(-1, 32)
    assert all(dx[i].tobytes() != dy[i].tobytes() for i in range(dx.shape[0]))
    a.close()
    b.close()
