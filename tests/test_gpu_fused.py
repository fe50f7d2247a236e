"""GPU parity of gdn_replay_verify_flush (flush folded into the next verify)
against the oracle's flush-then-verify, through the C ABI."""
import numpy as np
import pytest
import torch

from gated_deltanet_state_replayssm_amd import synth
from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device
from tests.gpu_harness import Pair, run_schedule, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_replayssm_amd import binding
    binding.load()


def test_fused_r8_multi_step():
    wl = synth.Workload("r8f", 8, 12, 32, 16, 128, 128, 32, 16, synth.BF16, 16, 2,
                        "clipnormal:12:3", "uniform:0:15")
    say("case fused r8 x 12 slots, 2 layers x 6 steps, flush every 16")
    pairs = run_schedule(wl, 6, 78, layers=2, label="r8f", fused=True)
    assert sum(p.flushed_count for p in pairs) > 0
    say(f"  worst {[p.worst for p in pairs]}")


def test_fused_pages_point_full_size_sampled():
    wl = W["r32_hv32_hk16_d128_f16"]
    say("case fused r32_hv32_hk16_d128_f16 full size, sampled")
    rng = np.random.default_rng(13)
    sample = rng.choice(wl.num_slots, 6, replace=False)
    pairs = run_schedule(wl, 5, synth.seed_for(wl.name, 0, 1), oracle_slots=sample,
                         label="c2f", fused=True)
    assert pairs[0].flushed_count > 0
    say(f"  worst {pairs[0].worst}")


@pytest.mark.parametrize("hv,hk", [(32, 16), (16, 4), (8, 8)])
def test_fused_draft_wraps_onto_folded_rows(hv, hk):
    """Every slot due with len = C or C - 1: the draft append wraps onto ring rows
    that the key head's other value heads fold in the same call."""
    C, D = 32, 16
    wl = synth.Workload("wrap", 6, 6, hv, hk, 128, 128, C, D, synth.BF16, 16, 1, "uniform",
                        "uniform:31:32")
    say(f"case fused wrap HV={hv} HK={hk}")
    rng = np.random.default_rng(hv * 10 + hk)
    init = synth.make_cache_init(wl, rng)
    p = Pair(wl, init)
    slots = synth.make_slot_idx(wl, rng)
    p.verify_flush(slots, 16, synth.make_draft(wl, rng), "wrap")
    assert p.flushed_count == wl.num_reqs
    p.rollback(slots, D, synth.sample_accepted(wl, rng), "wrap")
    p.verify_flush(slots, 16, synth.make_draft(wl, rng), "wrap2")


def test_fused_other_shapes_run_flush_then_verify():
    """Shapes without the one-kernel path (fp32 or small dims, capacity > 32)."""
    for dk, dt, C, D, F in ((32, synth.BF16, 12, 5, 4), (16, synth.F32, 12, 5, 4),
                            (128, synth.BF16, 80, 16, 64)):
        wl = synth.Workload("o", 3, 5, 4, 2, dk, dk, C, D, dt, F, 1, "clipnormal:12:3",
                            f"uniform:0:{C - D}")
        say(f"case fused fallback d={dk} {dt} C={C}")
        run_schedule(wl, 4, 300 + dk + C, label=f"fb{dk}", fused=True)


def test_fused_min_len_zero_and_edges():
    """min_len <= 1 folds every slot with len >= 1; len = 0 slots only verify."""
    wl = synth.Workload("ml", 4, 6, 4, 2, 64, 64, 32, 16, synth.BF16, 0, 1, "uniform",
                        "uniform:0:16")
    say("case fused min_len 0 / len 0, d=64")
    rng = np.random.default_rng(21)
    init = synth.make_cache_init(wl, rng)
    init["len"][:] = [0, 1, 16, 32, 5, 0]
    p = Pair(wl, init)
    slots = np.array([0, 1, 2, 3], np.int32)
    p.verify_flush(slots, 0, synth.make_draft(wl, rng), "ml0")
    assert p.flushed_count == 3


def test_fused_device_errors():
    wl = synth.Workload("fe", 4, 6, 4, 2, 128, 128, 32, 16, synth.BF16, 16, 1, "uniform",
                        "uniform:0:4")
    say("case fused device errors")
    rng = np.random.default_rng(22)
    init = synth.make_cache_init(wl, rng)
    init["len"][:] = [3, 17, 20, 0, 2, 1]   # slot 1 due (17 + 16 > 32 is fine), 2 due
    init["head"][5] = 40                    # slot 5: POINTER
    p = Pair(wl, init)
    slots = np.array([0, 1, 9, 5], np.int32)  # 9: SLOT
    p.verify_flush(slots, 18, synth.make_draft(wl, rng), "errors")   # slot 1 not due: CAPACITY
    assert int(p.gpu.err.item()) == 1 | 4 | 8
    p.gpu.err.zero_()
    p.orc.err = 0
    p.verify_flush(np.array([2, 3], np.int32), 18, synth.make_draft(wl, rng, num_reqs=2), "due")
    assert int(p.gpu.err.item()) == 0


def test_fused_equals_flush_then_verify_bitwise():
    """One kernel gives the same bits as the two separate calls."""
    wl = W["r32_hv32_hk16_d128_f16"]
    say("case fused vs flush + verify, bitwise, r32")
    rng = np.random.default_rng(23)
    init = synth.make_cache_init(wl, rng, init_len=rng.integers(0, 33, wl.num_slots))
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    slots = to_device(synth.make_slot_idx(wl, rng))
    oa = a.verify_flush(slots, 16, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
    b.flush(slots, 16)
    ob = b.verify(slots, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
    torch.cuda.synchronize()
    assert int(a.err.item()) == 0 and int(b.err.item()) == 0
    assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
    for name in ("state", "head", "len", "ring_k", "ring_v", "ring_alpha", "ring_beta", "ring_q"):
        x, y = getattr(a, name), getattr(b, name)
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        elif x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), name
    assert not a.sync.any()


def test_fused_stress_batch_sampled():
    """128 requests: more workgroups than fit on the GPU at once, and the due
    ordering counted in rounds of 64 requests."""
    wl = W["r128_hv32_hk16_d128_f16"]
    say("case fused r128_hv32_hk16_d128_f16, sampled")
    rng = np.random.default_rng(24)
    sample = rng.choice(wl.num_slots, 5, replace=False)
    pairs = run_schedule(wl, 4, synth.seed_for(wl.name, 0, 1), oracle_slots=sample,
                         label="c4f", fused=True)
    say(f"  worst {pairs[0].worst}")


@pytest.mark.parametrize("hv,hk", [(64, 8), (64, 32), (16, 2)])
def test_fused_gva_shapes_and_xcd_placement(hv, hk):
    """Value heads per key head G = 8, 2, 8 at HV = 64, 64, 16: the workgroups of
    a key head's value heads are placed 8 apart (one XCD) when HV is a multiple
    of 8 G, in order otherwise; the fused and separate orders both checked."""
    wl = synth.Workload("gva", 3, 4, hv, hk, 64, 64, 32, 8, synth.BF16, 16, 1,
                        "clipnormal:6:2", "uniform:0:23")
    say(f"case gva HV={hv} HK={hk}")
    run_schedule(wl, 4, 660 + hv + hk, label=f"gva{hv}_{hk}", fused=True)
    run_schedule(wl, 3, 670 + hv + hk, label=f"gvas{hv}_{hk}", fused=False)
