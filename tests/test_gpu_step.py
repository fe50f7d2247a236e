"""GPU parity of gdn_replay_rollback_verify_flush (the previous draft's rollback
and the periodic flush folded into the next verify, one call per layer and
step) against the oracle's rollback followed by its verify_flush, through the
C ABI; and bit-for-bit against the two separate calls."""
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


@pytest.mark.parametrize("d,slots", [(128, 12), (64, 8)])
def test_step_multi_step(d, slots):
    """8 requests per step over 12 slots (a slot leaving the batch gets its
    rollback from a call of its own; new ones pass per-request previous
    lengths) or over 8 (every request has a previous draft of the fixed
    length), 2 layers, flush every 16."""
    wl = synth.Workload("st", 8, slots, 8, 4, d, d, 32, 16, synth.BF16, 16, 2,
                        "clipnormal:12:3", "uniform:0:15")
    say(f"case step d={d}, 8 of {slots} slots, 2 layers x 6 steps")
    pairs = run_schedule(wl, 6, 700 + d, layers=2, label=f"st{d}", one_call=True)
    assert sum(p.flushed_count for p in pairs) > 0
    say(f"  worst {[p.worst for p in pairs]}")


def test_step_varlen_multi_step():
    """Per-request lengths 0..16 in both the previous and this step's draft."""
    wl = synth.Workload("stv", 6, 8, 4, 2, 128, 128, 32, 16, synth.BF16, 16, 2,
                        "clipnormal:12:3", "uniform:0:15", "uniform:0:16")
    say("case step varlen")
    pairs = run_schedule(wl, 6, 711, layers=2, label="stv", one_call=True)
    say(f"  worst {pairs[0].worst}")


def test_step_pages_point_sampled():
    wl = W["r32_hv32_hk16_d128_f16"]
    say("case step r32_hv32_hk16_d128_f16 full size, sampled")
    rng = np.random.default_rng(712)
    sample = rng.choice(wl.num_slots, 6, replace=False)
    pairs = run_schedule(wl, 5, synth.seed_for(wl.name, 0, 1), oracle_slots=sample,
                         label="c2s", one_call=True)
    say(f"  worst {pairs[0].worst}")


def test_step_other_shapes_run_the_calls_back_to_back():
    """Shapes without the one-kernel path (fp32, small dims, capacity > 32)."""
    for dk, dt, C, D, F in ((32, synth.BF16, 12, 5, 4), (16, synth.F32, 12, 5, 4),
                            (128, synth.BF16, 80, 16, 64)):
        wl = synth.Workload("o", 3, 5, 4, 2, dk, dk, C, D, dt, F, 1, "clipnormal:12:3",
                            f"uniform:0:{C - 2 * D}")
        say(f"case step fallback d={dk} {dt} C={C}")
        run_schedule(wl, 4, 720 + dk + C, label=f"sfb{dk}", one_call=True)


def test_step_device_errors():
    """The rollback's own errors (ACCEPT, DRAFT, CAPACITY) leave len as it was
    and the request still goes through verify_flush; with slot and pointer
    errors, the error word is the OR of both calls'."""
    wl = synth.Workload("se", 6, 8, 4, 2, 128, 128, 32, 8, synth.BF16, 16, 1, "uniform",
                        "uniform:0:4")
    say("case step device errors")
    rng = np.random.default_rng(713)
    init = synth.make_cache_init(wl, rng)
    init["len"][:] = [3, 20, 30, 10, 2, 1, 0, 0]
    init["head"][5] = 40                       # slot 5: POINTER
    p = Pair(wl, init)
    slots = np.array([0, 1, 2, 3, 5, 11], np.int32)   # 11: SLOT
    acc = np.array([9, 2, 5, 4, 0, 0], np.int32)       # 0: a > D (ACCEPT); 2: 30 + 5 > 32
    p.rollback_verify_flush(slots, acc, 8, 16, synth.make_draft(wl, rng), "errors")
    assert int(p.gpu.err.item()) == 1 | 2 | 4 | 8
    p.gpu.err.zero_()
    p.orc.err = 0
    # per-request previous lengths: 9 > prev_draft (DRAFT), a > its length (ACCEPT)
    slots = np.array([0, 1, 3, 4], np.int32)
    p.rollback_verify_flush(slots, np.array([1, 1, 2, 0], np.int32), 8, 16,
                            synth.make_draft(wl, rng, num_reqs=4), "errors2",
                            prev_lens=np.array([9, 0, 2, 8], np.int32))
    assert int(p.gpu.err.item()) == 2 | 16


@pytest.mark.parametrize("varlen", [False, True])
def test_step_equals_rollback_then_verify_flush_bitwise(varlen):
    """One kernel gives the same bits as gdn_replay_rollback followed by
    gdn_replay_verify_flush, at 32 requests x 32 heads."""
    wl = W["r32_hv32_hk16_d128_f16"]
    say(f"case step vs rollback + verify_flush, bitwise, r32, varlen={varlen}")
    rng = np.random.default_rng(714 + varlen)
    init = synth.make_cache_init(wl, rng, init_len=rng.integers(0, 17, wl.num_slots))
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    slots = to_device(synth.make_slot_idx(wl, rng))
    R = wl.num_reqs
    plens = lens = None
    if varlen:
        plens = to_device(rng.integers(0, wl.draft + 1, R).astype(np.int32))
        lens = to_device(rng.integers(0, wl.draft + 1, R).astype(np.int32))
        acc = to_device((rng.random(R) * (plens.cpu().numpy() + 1)).astype(np.int32))
    else:
        acc = to_device(rng.integers(0, wl.draft + 1, R).astype(np.int32))
    oa = a.rollback_verify_flush(slots, acc, wl.draft, 16, dr["q"], dr["k"], dr["v"], dr["alpha"],
                                 dr["beta"], prev_draft_lens=plens, draft_lens=lens)
    b.rollback(slots, wl.draft, acc, draft_lens=plens)
    ob = b.verify_flush(slots, 16, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"],
                        draft_lens=lens)
    torch.cuda.synchronize()
    assert int(a.err.item()) == 0 and int(b.err.item()) == 0
    if varlen:   # rows past a request's length are not written by either call
        keep = torch.arange(wl.draft, device="cuda")[None, :] < lens[:, None]
        oa, ob = oa[keep], ob[keep]
    assert torch.equal(oa.view(torch.int32), ob.view(torch.int32))
    for name in ("state", "head", "len", "ring_k", "ring_v", "ring_alpha", "ring_beta", "ring_q"):
        x, y = getattr(a, name), getattr(b, name)
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        elif x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), name
    assert not a.sync.any()
    assert int((a.len == 0).sum()) > 0       # some slots were flushed


@pytest.mark.parametrize("C", [32, 48])
@pytest.mark.parametrize("R", [65, 200, 300])
def test_step_ordering_rounds(R, C):
    """More than 64 requests: the ordering pass in rounds of 64 with every
    round's values kept in lanes (up to 256 requests), and in reloaded rounds
    beyond; bad slots and pointers in the batch; one-chunk (C = 32) and
    multi-chunk (C = 48) replays."""
    wl = synth.Workload("rounds", R, R + 20, 2, 1, 64, 64, C, 8, synth.BF16, 16, 1,
                        "clipnormal:6:3", "uniform:0:23")
    say(f"case step ordering rounds R={R} C={C}")
    rng = np.random.default_rng(740 + R)
    init = synth.make_cache_init(wl, rng)
    init["head"][3] = 77                       # POINTER for whoever gets slot 3
    p = Pair(wl, init)
    prev = {}
    for step in range(3):
        slots = synth.make_slot_idx(wl, rng)
        if step == 1:
            slots[R // 2] = wl.num_slots + 5   # SLOT
        acc = synth.sample_accepted(wl, rng)
        pa = np.array([prev.get(int(s), 0) for s in slots], np.int32)
        p.rollback_verify_flush(slots, pa, wl.draft, wl.flush_min_len, synth.make_draft(wl, rng),
                                f"rounds{R} step{step}")
        prev = {int(s): int(acc[i]) for i, s in enumerate(slots)}
    assert p.flushed_count > 0


def test_step_equals_rollback_then_verify_flush_bitwise_r128():
    wl = W["r128_hv32_hk16_d128_f16"]
    say("case step vs rollback + verify_flush, bitwise, r128")
    rng = np.random.default_rng(750)
    init = synth.make_cache_init(wl, rng, init_len=rng.integers(0, 17, wl.num_slots))
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    slots = to_device(synth.make_slot_idx(wl, rng))
    acc = to_device(rng.integers(0, wl.draft + 1, wl.num_reqs).astype(np.int32))
    oa = a.rollback_verify_flush(slots, acc, wl.draft, 16, dr["q"], dr["k"], dr["v"], dr["alpha"],
                                 dr["beta"])
    b.rollback(slots, wl.draft, acc)
    ob = b.verify_flush(slots, 16, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
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
