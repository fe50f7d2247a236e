"""GPU parity of gdn_replay_verify_flush for replays of several chunks (ring
capacity above 32: the flush folded into the next verify, chunk by chunk)
against the oracle's flush-then-verify, through the C ABI; and bit for bit
against the two separate calls."""
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


@pytest.mark.parametrize("d,C,F", [(128, 80, 64), (64, 48, 24), (128, 256, 200)])
def test_long_multi_step(d, C, F):
    """Folds of up to 3 (C = 80), 2 (C = 48) and 7 (C = 256) chunks, 2 layers."""
    D = 16
    wl = synth.Workload("lg", 6, 9, 8, 4, d, d, C, D, synth.BF16, F, 2, "clipnormal:12:3",
                        f"uniform:0:{C - D}")
    say(f"case long fused d={d} C={C} F={F}")
    pairs = run_schedule(wl, 6, 600 + C + d, layers=2, label=f"lg{C}", fused=True)
    assert sum(p.flushed_count for p in pairs) > 0
    say(f"  worst {[p.worst for p in pairs]}")


@pytest.mark.parametrize("hv,hk", [(32, 16), (16, 4), (8, 8)])
def test_long_draft_wraps_onto_folded_rows(hv, hk):
    """Every slot due with len = C or C - 1 (three chunks to fold): the draft
    append wraps onto committed key rows that the key head's other value heads
    fold in the same call."""
    C, D = 80, 16
    wl = synth.Workload("lwrap", 5, 5, hv, hk, 128, 128, C, D, synth.BF16, 64, 1, "uniform",
                        f"uniform:{C - 1}:{C}")
    say(f"case long wrap HV={hv} HK={hk}")
    rng = np.random.default_rng(610 + hv + hk)
    init = synth.make_cache_init(wl, rng)
    p = Pair(wl, init)
    slots = synth.make_slot_idx(wl, rng)
    p.verify_flush(slots, 64, synth.make_draft(wl, rng), "wrap")
    assert p.flushed_count == wl.num_reqs
    p.rollback(slots, D, synth.sample_accepted(wl, rng), "wrap")
    p.verify_flush(slots, 64, synth.make_draft(wl, rng), "wrap2")


def test_long_varlen_with_empty_drafts():
    """Per-request lengths 0..16 at C = 80: due slots without a draft fold only."""
    wl = synth.Workload("lvl", 6, 8, 4, 2, 128, 128, 80, 16, synth.BF16, 48, 1,
                        "clipnormal:12:3", "uniform:30:64", "uniform:0:16")
    say("case long varlen")
    run_schedule(wl, 6, 620, label="lvl", fused=True)


def test_long_errors_and_min_len_edges():
    wl = synth.Workload("lerr", 5, 7, 4, 2, 64, 64, 48, 8, synth.BF16, 1, 1, "uniform",
                        "uniform:0:4")
    say("case long errors, min_len 0")
    rng = np.random.default_rng(621)
    init = synth.make_cache_init(wl, rng)
    init["len"][:] = [0, 1, 33, 45, 41, 2, 40]  # 3: 45 + 8 > 48 but due; 4: not due below
    init["head"][5] = 60                         # POINTER
    p = Pair(wl, init)
    slots = np.array([0, 1, 2, 3, 5], np.int32)
    p.verify_flush(slots, 0, synth.make_draft(wl, rng), "min_len 0")
    assert int(p.gpu.err.item()) == 8
    p.gpu.err.zero_()
    p.orc.err = 0
    slots = np.array([4, 6, 11], np.int32)         # 4: 41 + 8 > 48, not due at 42: CAPACITY
    p.verify_flush(slots, 42, synth.make_draft(wl, rng, num_reqs=3), "capacity")
    assert int(p.gpu.err.item()) == 1 | 4


def test_long_c3_full_size_sampled():
    wl = W["r32_hv32_hk16_d128_f64"]
    say("case long r32_hv32_hk16_d128_f64 full size, sampled")
    rng = np.random.default_rng(630)
    sample = rng.choice(wl.num_slots, 6, replace=False)
    pairs = run_schedule(wl, 5, synth.seed_for(wl.name, 0, 1), oracle_slots=sample,
                         label="c3f", fused=True)
    say(f"  worst {pairs[0].worst}")


def test_long_equals_flush_then_verify_bitwise():
    wl = W["r32_hv32_hk16_d128_f64"]
    say("case long fused vs flush + verify, bitwise, C = 80")
    rng = np.random.default_rng(631)
    init = synth.make_cache_init(wl, rng, init_len=rng.integers(0, 65, wl.num_slots))
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    slots = to_device(synth.make_slot_idx(wl, rng))
    oa = a.verify_flush(slots, 40, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
    b.flush(slots, 40)
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
    assert int((a.len == 0).sum()) > 0


@pytest.mark.parametrize("varlen", [False, True])
def test_long_one_call_step(varlen):
    """rollback_verify_flush at C = 80 (one kernel: the previous draft's
    rollback, the chunked fold and the verify) against the oracle's rollback
    then verify_flush; requests leaving and joining the batch."""
    wl = synth.Workload("lstep", 6, 9, 8, 4, 128, 128, 80, 16, synth.BF16, 48, 2,
                        "clipnormal:12:3", "uniform:0:64",
                        "uniform:0:16" if varlen else "fixed")
    say(f"case long one-call step varlen={varlen}")
    pairs = run_schedule(wl, 6, 640 + varlen, layers=2, label="lstep", one_call=True)
    assert sum(p.flushed_count for p in pairs) > 0


def test_long_one_call_step_bitwise():
    wl = W["r32_hv32_hk16_d128_f64"]
    say("case long one-call step vs rollback + verify_flush, bitwise, C = 80")
    rng = np.random.default_rng(650)
    init = synth.make_cache_init(wl, rng, init_len=rng.integers(0, 49, wl.num_slots))
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    slots = to_device(synth.make_slot_idx(wl, rng))
    acc = to_device(rng.integers(0, wl.draft + 1, wl.num_reqs).astype(np.int32))
    oa = a.rollback_verify_flush(slots, acc, wl.draft, 56, dr["q"], dr["k"], dr["v"],
                                 dr["alpha"], dr["beta"])
    b.rollback(slots, wl.draft, acc)
    ob = b.verify_flush(slots, 56, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
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


@pytest.mark.parametrize("R,one_call", [(64, False), (65, False), (64, True)])
def test_long_work_order_at_the_lane_limit(R, one_call):
    """64 requests (the ordering pass ranks them by fold chunks in one wave's
    lanes) and 65 (the pass over rounds of 64, due first), with committed
    counts that give every chunk class (none to three fold chunks)."""
    wl = synth.Workload("lord", R, R + 8, 2, 1, 64, 64, 80, 16, synth.BF16, 48, 1,
                        "clipnormal:12:3", "uniform:0:64")
    say(f"case long work order R={R} one_call={one_call}")
    pairs = run_schedule(wl, 3, 640 + R, label=f"lord{R}", fused=not one_call, one_call=one_call)
    assert sum(p.flushed_count for p in pairs) > 0
