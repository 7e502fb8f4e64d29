"""pack_init_noalloc against pack_init (GPU).

pack_init_noalloc builds the plan in the device's static scratch instead of an
allocated workspace.  Two calls in a row, the second with a smaller corpus
(the scratch then still holds the first plan's bytes): each context's plan
arrays, cycle information, batches, learned counts, window digests and
fingerprints must equal, bit for bit, those of a pack_init context over the
same corpus, and the oracle's.  While a no-alloc context is alive a second one
on the same device is refused."""
import numpy as np
import pytest

import deterministic_packing_amd as dp
import oracle
from synth import make_corpus, random_small

from _gpu_parity import PLAN_ARRAYS, compare_batch, compare_cycle, compare_plan, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dp.load_library()
    yield
    torch.cuda.synchronize()


def _run(c, tensors, noalloc):
    pk = dp.Packer(c, device_tensors=tensors, noalloc=noalloc)
    plan = {name: pk.inspect(name) for name in PLAN_ARRAYS}
    cycles = []
    for cyc in (0, 1):
        info = pk.cycle(cyc)
        n = info["n_updates"]
        out = pk.batch(0, n)
        fp = pk.fingerprint_steps(0, n, out["digests"].reshape(-1, 32)).cpu().numpy()
        cycles.append((info, to_np(out), fp))
    return pk, plan, cycles


def _check(name, c):
    import torch
    say("no-alloc", name, c.n_docs, "docs", c.n_tokens, "tokens")
    t = dp.upload_corpus(c)
    torch.cuda.synchronize()
    ref_pk, ref_plan, ref_cycles = _run(c, t, noalloc=False)
    ref_pk.close()
    pk, plan, cycles = _run(c, t, noalloc=True)
    with pytest.raises(dp.DpackError) as e:  # one no-alloc context per device at a time
        dp.Packer(c, device_tensors=t, noalloc=True)
    assert e.value.code == dp.PACK_E_STATE
    op = oracle.Plan(c)
    compare_plan(pk, op)
    for k in plan:
        assert np.array_equal(plan[k], ref_plan[k]), (name, k)
    for cyc, ((info, out, fp), (rinfo, rout, rfp)) in enumerate(zip(cycles, ref_cycles)):
        for k in ("n_updates", "real_tokens", "learned_tokens", "positions", "plan_digest"):
            assert info[k] == rinfo[k], (name, cyc, k)
        for k in ("windows_start", "windows_taken", "windows_remaining", "per_update", "stream_next_token"):
            assert np.array_equal(info[k], rinfo[k]), (name, cyc, k)
        compare_batch(out, rout, f"{name} cycle {cyc} vs pack_init")
        assert np.array_equal(fp, rfp), (name, cyc)
        oi = op.cycle(cyc)
        compare_cycle(info, oi, op)
        compare_batch(out, op.batch(0, oi.n_updates), f"{name} cycle {cyc} vs oracle")
    pk.close()


def test_noalloc_equals_pack_init_twice_smaller_second():
    first = make_corpus("tiny").replace(cumulative=True, read_random=True, updates_per_cycle=20)
    second = random_small(404, n_docs=700, n_sources=3, max_strata=2, T=128, B=6, max_len=260, prompts=True,
                          bp_max=1200).replace(wrap=True, ramp=((0, 3 * 128), (4 * 3 * 128, 6 * 128)),
                                               updates_per_cycle=5)
    assert second.n_docs < first.n_docs and second.n_tokens < first.n_tokens
    _check("tiny, cumulative, random read order", first)
    _check("smaller, wrap, batch-size ramp", second)


def test_noalloc_chunked_digests_one_stream():
    """Chunked window digests (the emission, then the chunk digests from the
    outputs) in the static scratch: the no-alloc context equals a pack_init
    context and the oracle, across a batch-size ramp."""
    c = random_small(405, n_docs=900, n_sources=3, max_strata=2, T=1024, B=4, max_len=2500, prompts=True,
                     bp_max=800).replace(digest_chunked=True, ramp=((0, 2 * 1024), (6 * 2 * 1024, 4 * 1024)),
                                         updates_per_cycle=4)
    _check("chunked digests, batch-size ramp", c)
