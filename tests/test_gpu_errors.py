"""Internal failures inside the kernels reach the caller, and rare code paths
run, forced by the library's test options (GPU).

The window digests of pack_batch wait, boundedly, for the emitting waves
beside them; if such a wait gives up, the call's digests are not valid and
pack_status must say so.  A cycle kernel that finds the plan inconsistent must
make pack_cycle fail and leave no cycle current.  Both conditions are forced
from the host with the library's test options, so every kernel still runs to
its end: the wait asks for a block count no wave publishes and gives up after
one poll; the cycle kernel raises the flag without touching anything else."""
import numpy as np
import pytest

import deterministic_packing_amd as dp
import oracle
from synth import random_small

from _gpu_parity import compare_batch, compare_cycle, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dp.load_library()
    yield
    torch.cuda.synchronize()


def _corpus(seed, **mode):
    c = random_small(seed, n_docs=900, n_sources=3, max_strata=2, T=128, B=8, max_len=300, prompts=True,
                     bp_max=1500)
    return c.replace(**mode)


def _large_corpus(seed, **mode):  # a launch of 513 to 1,024 waves: the paired kernel
    c = random_small(seed, n_docs=40000, n_sources=3, max_strata=2, T=64, B=640, max_len=120, bp_max=500)
    return c.replace(**mode)


@pytest.mark.parametrize("mode,large", [({}, False), ({"wrap": True, "read_random": True}, False), ({}, True)])
def test_digest_wait_that_gives_up_is_reported(mode, large):
    """Both kernels with bounded waits: the ring pairs (launches of at most 512
    waves) and the paired kernel (513 to 1,024 waves, here 600)."""
    c = _large_corpus(505, **mode) if large else _corpus(501, **mode)
    upc = 60 if large else 3
    say("digest wait give-up", mode, "large" if large else "small")
    op = oracle.Plan(c)
    oi = op.cycle(0, updates_per_cycle=upc)
    if large:
        assert 512 * 64 < oi.n_updates * c.B <= 1024 * 64
    pk = dp.Packer(c.replace(updates_per_cycle=upc))
    pk.cycle(0)
    n = oi.n_updates
    good = to_np(pk.batch(0, n))  # batch() ends with pack_status: no failure
    compare_batch(good, op.batch(0, n), "before")

    pk.test_option(dp.PACK_TEST_WAIT_GIVE_UP, 1)
    out = pk.alloc_out(n)
    pk.batch_into(0, n, out)  # asynchronous: accepted
    with pytest.raises(dp.DpackError) as e:
        pk.status()
    assert e.value.code == dp.PACK_E_INTERNAL
    pk.status()  # reported once, then cleared

    pk.test_option(dp.PACK_TEST_WAIT_GIVE_UP, 0)
    again = to_np(pk.batch(0, n))
    compare_batch(again, op.batch(0, n), "after")
    pk.close()


@pytest.mark.parametrize("mode", [{}, {"cumulative": True}, {"ramp": ((0, 4 * 128), (2 * 4 * 128 + 1, 8 * 128))}])
def test_cycle_kernel_failure_fails_the_cycle(mode):
    c = _corpus(502, **mode).replace(updates_per_cycle=2)
    say("cycle fault", {k: v for k, v in mode.items()})
    op = oracle.Plan(c)
    o0 = op.cycle(0)
    pk = dp.Packer(c)
    compare_cycle(pk.cycle(0), o0, op)

    pk.test_option(dp.PACK_TEST_CYCLE_FAULT, 1)
    with pytest.raises(dp.DpackError) as e:
        pk.cycle(1)
    assert e.value.code == dp.PACK_E_INTERNAL
    with pytest.raises(dp.DpackError) as e:  # no cycle is current after the failure
        pk.batch(0, 1)
    assert e.value.code == dp.PACK_E_STATE
    with pytest.raises(dp.DpackError) as e:  # the failed cycle is still the one to plan
        pk.cycle(2)
    assert e.value.code == dp.PACK_E_STATE

    pk.test_option(dp.PACK_TEST_CYCLE_FAULT, 0)
    o1 = op.cycle(1)
    compare_cycle(pk.cycle(1), o1, op)
    n = o1.n_updates
    compare_batch(to_np(pk.batch(0, n)), op.batch(0, n), "cycle 1 after the failed attempt")
    pk.close()


def test_exhaustion_leaves_no_current_cycle():
    c = _corpus(503, cumulative=True, ramp=((0, 4 * 128), (10 * 128, 8 * 128)))
    op = oracle.Plan(c)
    oi = op.cycle(0)
    pk = dp.Packer(c)
    compare_cycle(pk.cycle(0), oi, op)
    with pytest.raises(oracle.OracleError) as oe:
        op.cycle(1)
    assert oe.value.code == oracle.OR_E_EXHAUSTED
    with pytest.raises(dp.DpackError) as e:
        pk.cycle(1)
    assert e.value.code == dp.PACK_E_EXHAUSTED
    with pytest.raises(dp.DpackError) as e:
        pk.batch(0, 1)
    assert e.value.code == dp.PACK_E_STATE
    pk.close()


def test_test_options_change_no_output_byte_when_off():
    c = _corpus(504)
    pk = dp.Packer(c.replace(updates_per_cycle=2))
    pk.cycle(0)
    a = to_np(pk.batch(0, 2))
    pk.test_option(dp.PACK_TEST_WAIT_GIVE_UP, 0)
    pk.test_option(dp.PACK_TEST_CYCLE_FAULT, 0)
    b = to_np(pk.batch(0, 2))
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    with pytest.raises(dp.DpackError) as e:
        pk.test_option(99, 1)
    assert e.value.code == dp.PACK_E_INVAL
    pk.close()


@pytest.mark.parametrize("mode", [{}, {"cumulative": True}, {"lanes": 2}])
def test_sort_insertion_path_gives_the_same_read_order(mode):
    """The sort's insertion path (buckets above 16 elements, which uniform keys
    almost never fill) forced for every bucket of the cycles' random read order:
    the read order, and so every batch, still equal the oracle's."""
    c = _corpus(506, read_random=True, **mode).replace(updates_per_cycle=3)
    say("sort insertion path", mode)
    op = oracle.Plan(c)
    pk = dp.Packer(c)
    pk.test_option(dp.PACK_TEST_SORT_INSERTION, 1)
    for cyc in range(3):
        oi = op.cycle(cyc)
        compare_cycle(pk.cycle(cyc), oi, op)
        n = oi.n_updates
        compare_batch(to_np(pk.batch(0, n)), op.batch(0, n), f"insertion sort cycle {cyc}")
    pk.close()
