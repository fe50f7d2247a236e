"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Sizes span several tiles and ragged buffers; full-size workloads are checked on
sampled requests (requests are independent, so a sample is an exact check of
those requests at the real batch size and launch configuration).
"""
import numpy as np
import pytest
import torch

from gated_deltanet_state_replayssm_amd import synth
from gated_deltanet_state_replayssm_amd.cache import to_device
from tests.gpu_harness import Pair, run_schedule, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_replayssm_amd import binding
    binding.load()


def test_tiny_one_step():
    wl = W["tiny_r1_h1_d16"]
    say("case tiny_r1_h1_d16 one step")
    rng = np.random.default_rng(synth.seed_for(wl.name, 0, 0))
    p = Pair(wl, synth.make_cache_init(wl, rng))
    slots = np.array([0], np.int32)
    p.verify(slots, synth.make_draft(wl, rng), "tiny")
    p.rollback(slots, wl.draft, synth.sample_accepted(wl, rng), "tiny")
    p.flush(slots, wl.flush_min_len, "tiny")
    assert p.flushed_count == 1


def test_r8_one_step():
    wl = W["r8_hv32_hk16_d128"]
    say("case r8_hv32_hk16_d128 one step")
    pairs = run_schedule(wl, 1, synth.seed_for(wl.name, 0, 0), label="r8")
    say(f"  worst {pairs[0].worst}")


def test_r8_multi_step_with_flushes():
    wl = synth.Workload("r8s", 8, 12, 32, 16, 128, 128, 32, 16, synth.BF16, 16, 2,
                        "clipnormal:12:3", "uniform:0:15")
    say("case r8 x 12 slots, 2 layers x 6 steps, flush every 16")
    pairs = run_schedule(wl, 6, 77, layers=2, label="r8s")
    assert sum(p.flushed_count for p in pairs) > 0
    say(f"  worst {[p.worst for p in pairs]}")


def test_small_dims_and_fp32_inputs():
    for dk in (16, 32, 64):
        for dt in (synth.F32, synth.BF16):
            wl = synth.Workload("s", 3, 5, 4, 2, dk, dk, 12, 5, dt, 4, 1, "uniform",
                                "uniform:0:7")
            say(f"case d={dk} {dt}")
            run_schedule(wl, 4, 1000 + dk, label=f"d{dk}{dt}")


def test_without_ring_q():
    wl = synth.Workload("nq", 4, 4, 8, 4, 128, 128, 32, 16, synth.BF16, 8, 1, "uniform",
                        "uniform:0:15")
    say("case ring_q = NULL")
    run_schedule(wl, 3, 5, with_q=False, label="noq")


def test_pages_point_full_size_sampled():
    """32 requests x 32 value heads x 128^2, flush every 16: full batch on the GPU,
    oracle on 6 sampled slots, several steps so flushes happen."""
    wl = W["r32_hv32_hk16_d128_f16"]
    say("case r32_hv32_hk16_d128_f16 full size, sampled")
    rng = np.random.default_rng(3)
    sample = rng.choice(wl.num_slots, 6, replace=False)
    pairs = run_schedule(wl, 4, synth.seed_for(wl.name, 0, 0), oracle_slots=sample, label="c2")
    assert pairs[0].flushed_count > 0


def test_flush_heavy_long_buffers():
    """Capacity 80, flush every 64: buffers of up to 63 committed tokens."""
    wl = synth.Workload("fh", 4, 4, 32, 16, 128, 128, 80, 16, synth.BF16, 64, 1,
                        "clipnormal:12:3", "fixed:0")
    say("case flush-heavy C=80 F=64")
    rng = np.random.default_rng(31)
    for B in (0, 8, 16, 32, 48, 63, 64):
        init = synth.make_cache_init(wl, rng, init_len=[B] * wl.num_slots)
        p = Pair(wl, init)
        slots = synth.make_slot_idx(wl, rng)
        p.verify(slots, synth.make_draft(wl, rng), f"B={B}")
        p.rollback(slots, wl.draft, synth.sample_accepted(wl, rng), f"B={B}")
        p.flush(slots, 1, f"B={B}")


@pytest.mark.parametrize("d", [128, 64])
def test_long_rings_many_chunks(d):
    """Ring capacity 256 with a 32-token draft: replays of up to 8 chunks, with
    chunk boundaries inside the committed tokens and right before the draft."""
    C, D = 256, 32
    wl = synth.Workload("lr", 2, 2, 4, 2, d, d, C, D, synth.BF16, 1, 1, "fixed:7",
                        "fixed:0")
    rng = np.random.default_rng(41 + d)
    for B in (0, 1, 31, 32, 33, 100, 224):
        say(f"case long ring d={d} C={C} D={D} B={B}")
        init = synth.make_cache_init(wl, rng, init_len=[B] * wl.num_slots)
        p = Pair(wl, init)
        slots = synth.make_slot_idx(wl, rng)
        p.verify(slots, synth.make_draft(wl, rng), f"B={B}")
        p.rollback(slots, wl.draft, synth.sample_accepted(wl, rng), f"B={B}")
        p.flush(slots, 1, f"B={B}")


def test_stress_batch_sampled():
    wl = W["r128_hv32_hk16_d128_f16"]
    say("case r128_hv32_hk16_d128_f16, sampled")
    rng = np.random.default_rng(4)
    sample = rng.choice(wl.num_slots, 5, replace=False)
    run_schedule(wl, 3, synth.seed_for(wl.name, 0, 0), oracle_slots=sample, label="c4")


def test_edge_draft_lengths_and_full_ring():
    """D = 1, D = C with an empty buffer, len = C - D exactly, all-reject, all-accept."""
    for C, D, B, a in ((8, 1, 0, 1), (8, 8, 0, 8), (12, 5, 7, 0), (12, 5, 7, 5), (16, 16, 0, 0)):
        wl = synth.Workload("e", 2, 3, 4, 2, 32, 32, C, D, synth.BF16, 1, 1, f"fixed:{a}",
                            f"fixed:{B}")
        say(f"case edge C={C} D={D} B={B} a={a}")
        rng = np.random.default_rng(C * 100 + D * 10 + B)
        p = Pair(wl, synth.make_cache_init(wl, rng))
        slots = synth.make_slot_idx(wl, rng)
        p.verify(slots, synth.make_draft(wl, rng), "edge")
        p.rollback(slots, D, synth.sample_accepted(wl, rng), "edge")
        p.flush(slots, 1, "edge")


def test_device_errors_skip_requests():
    """Out-of-range slot, capacity overflow, invalid accept count and corrupt
    pointers set the sticky bits and leave the offending requests untouched."""
    wl = synth.Workload("err", 4, 6, 4, 2, 16, 16, 8, 4, synth.BF16, 1, 1, "uniform",
                        "uniform:0:4")
    say("case device errors")
    rng = np.random.default_rng(9)
    init = synth.make_cache_init(wl, rng)
    init["len"][:] = [1, 5, 2, 0, 3, 1]          # slot 1: 5 + 4 > 8 -> CAPACITY
    init["head"][5] = 9                          # slot 5: head >= C -> POINTER
    p = Pair(wl, init)
    slots = np.array([0, 1, 9, 5], np.int32)     # 9 is out of range -> SLOT
    out = p.verify(slots, synth.make_draft(wl, rng), "errors")
    assert int(p.gpu.err.item()) == 1 | 4 | 8
    acc = np.array([5, 1, 0, 0], np.int32)       # 5 > D -> ACCEPT
    p.rollback(slots, wl.draft, acc, "errors")
    assert int(p.gpu.err.item()) == 1 | 2 | 4 | 8
    p.flush(slots, 1, "errors")
    # a clean request in the same call still went through
    p2slots = np.array([2, 3], np.int32)
    p.verify(p2slots, synth.make_draft(wl, rng, num_reqs=2), "clean")


def test_skipped_request_outputs_untouched():
    wl = synth.Workload("sk", 2, 2, 4, 2, 16, 16, 8, 4, synth.BF16, 1, 1, "uniform", "fixed:6")
    say("case skipped outputs untouched")
    rng = np.random.default_rng(10)
    p = Pair(wl, synth.make_cache_init(wl, rng))
    dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    out = torch.full((2, 4, 4, 16), 7.0, device="cuda")
    p.gpu.verify(to_device(np.array([0, 1], np.int32)), dr["q"], dr["k"], dr["v"], dr["alpha"],
                 dr["beta"], out=out)
    torch.cuda.synchronize()
    assert int(p.gpu.err.item()) == 1
    assert bool((out == 7.0).all())


def test_zero_requests_noop():
    wl = synth.Workload("z", 2, 2, 4, 2, 16, 16, 8, 4, synth.BF16, 1, 1, "uniform", "fixed:1")
    say("case zero requests")
    rng = np.random.default_rng(11)
    p = Pair(wl, synth.make_cache_init(wl, rng))
    before = p.gpu.to_numpy()
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng, num_reqs=0).items()}
    p.gpu.verify(e, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
    p.gpu.rollback(e, 4, e)
    p.gpu.flush(e, 1)
    torch.cuda.synchronize()
    after = p.gpu.to_numpy()
    for k in before:
        if before[k] is not None:
            assert np.array_equal(before[k], after[k]), k


def test_deterministic_bitwise():
    wl = W["r8_hv32_hk16_d128"]
    say("case determinism")
    outs = []
    for _ in range(2):
        rng = np.random.default_rng(5)
        init = synth.make_cache_init(wl, rng)
        p = Pair(wl, init, oracle_slots=[])
        slots = synth.make_slot_idx(wl, rng)
        o = p.verify(slots, synth.make_draft(wl, rng), "det")
        p.rollback(slots, wl.draft, synth.sample_accepted(wl, rng), "det")
        p.flush(slots, 1, "det")
        outs.append((o.cpu().numpy().view(np.uint32), p.gpu.state.cpu().numpy().view(np.uint32)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_checkpoint_save_restore_resume():
    """Saving the cache tensors mid-run and restoring them into a fresh cache
    continues bit-exactly."""
    wl = synth.Workload("ck", 4, 4, 8, 4, 64, 64, 32, 16, synth.BF16, 16, 1, "clipnormal:12:3",
                        "uniform:0:15")
    say("case save/restore")
    rng = np.random.default_rng(12)
    init = synth.make_cache_init(wl, rng)
    a = Pair(wl, init, oracle_slots=[])
    slots = synth.make_slot_idx(wl, rng)
    a.verify(slots, synth.make_draft(wl, rng))
    a.rollback(slots, wl.draft, synth.sample_accepted(wl, rng))
    saved = a.gpu.to_numpy()
    b = Pair(wl, saved, oracle_slots=[])
    dr = synth.make_draft(wl, rng)
    for p in (a, b):
        p.flush(slots, 1)
    oa = a.verify(slots, dr)
    ob = b.verify(slots, dr)
    assert int(a.gpu.err.item()) == 0 and int(b.gpu.err.item()) == 0
    assert torch.equal(oa, ob) and torch.equal(a.gpu.state, b.gpu.state)


def test_degenerate_decays_and_write_strengths():
    """alpha = 0 (full reset), alpha = 1, tiny alpha, beta = 0 and beta = 1 in the
    committed buffer and the draft; the oracle replays them exactly."""
    for cap in (32, 80):
        wl = synth.Workload("dg", 4, 4, 4, 2, 128, 128, cap, 16, synth.BF16, 1, 1, "uniform",
                            "uniform:8:15")
        say(f"case degenerate decays C={cap}")
        rng = np.random.default_rng(41 + cap)
        init = synth.make_cache_init(wl, rng)
        special = np.array([0.0, 1.0, 1e-30, 0.5], np.float32)
        init["ring_alpha"] = rng.choice(special, init["ring_alpha"].shape).astype(np.float32)
        init["ring_beta"] = rng.choice(np.array([0.0, 1.0, 0.3], np.float32),
                                       init["ring_beta"].shape).astype(np.float32)
        p = Pair(wl, init)
        slots = synth.make_slot_idx(wl, rng)
        dr = synth.make_draft(wl, rng)
        dr["alpha"] = rng.choice(special, dr["alpha"].shape).astype(np.float32)
        dr["beta"] = rng.choice(np.array([0.0, 1.0, 0.7], np.float32), dr["beta"].shape).astype(np.float32)
        p.verify(slots, dr, "degenerate")
        p.rollback(slots, wl.draft, synth.sample_accepted(wl, rng), "degenerate")
        p.flush(slots, 1, "degenerate")
        say(f"  worst {p.worst}")
