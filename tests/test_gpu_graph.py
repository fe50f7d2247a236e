"""HIP-graph capture of the calls that are replayed from graphs (verify_flush +
rollback, rollback_verify_flush, the step with the gated RMSNorm + FP8 in its
epilogue, gated RMSNorm + FP8, the causal convolution):
each graph is replayed several times with new inputs copied into its buffers,
with eager work and synchronisations between the replays, and every replay is
compared bit for bit with the same calls made eagerly on a twin."""
import numpy as np
import pytest
import torch

from gated_deltanet_state_replayssm_amd import synth
from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CACHE_FIELDS = ("state", "head", "len", "ring_k", "ring_v", "ring_alpha", "ring_beta", "ring_q",
                "sync", "err")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_replayssm_amd import binding
    binding.load()


def _bits(t):
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t


def _same(x, y, what):
    assert torch.equal(_bits(x), _bits(y)), what


def _eager_work():
    """Unrelated eager work between replays (a reduction over many blocks)."""
    x = torch.randn(1 << 20, device="cuda")
    float(x.abs().sum().item())
    torch.cuda.synchronize()


@pytest.mark.parametrize("workload", ["r32_hv32_hk16_d128_f16", "r32_hv32_hk16_d128_f64"])
@pytest.mark.parametrize("path", ["fused", "step"])
def test_replay_graph_matches_eager(path, workload):
    """32 requests x 32 heads, 6 replays: the draft, the slot permutation and
    the accept counts change at every replay; flushes fall due on the way
    (ring capacity 32: one-chunk replays; 80: several chunks)."""
    wl = W[workload]
    D, F = wl.draft, wl.flush_min_len
    say(f"case graph replay {path}, {workload}")
    rng = np.random.default_rng(800 + (path == "step") + 10 * (wl.cap > 32))
    init = synth.make_cache_init(wl, rng)
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    names = ("q", "k", "v", "alpha", "beta")
    buf = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    slots_buf = to_device(synth.make_slot_idx(wl, rng))
    acc_buf = torch.zeros(wl.num_reqs, dtype=torch.int32, device="cuda")
    out_a = torch.empty((wl.num_reqs, D, wl.hv, wl.dv), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        if path == "fused":
            b.verify_flush(slots_buf, F, *(buf[x] for x in names), out=out_b)
            b.rollback(slots_buf, D, acc_buf)
        else:
            b.rollback_verify_flush(slots_buf, acc_buf, D, F, *(buf[x] for x in names), out=out_b)
    torch.cuda.synchronize()
    prev = {}                      # step path: slot -> accepted count of its last draft
    flushed = 0
    for step in range(6):
        slots = synth.make_slot_idx(wl, rng)
        acc = synth.sample_accepted(wl, rng)
        dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
        sd = to_device(slots)
        head_before = a.head.clone()
        if path == "fused":
            a.verify_flush(sd, F, *(dr[x] for x in names), out=out_a)
            a.rollback(sd, D, to_device(acc))
            acc_now = acc
        else:
            acc_now = np.array([prev.get(int(s), 0) for s in slots], np.int32)
            a.rollback_verify_flush(sd, to_device(acc_now), D, F, *(dr[x] for x in names),
                                    out=out_a)
            prev = {int(s): int(acc[i]) for i, s in enumerate(slots)}
        slots_buf.copy_(sd)
        acc_buf.copy_(to_device(acc_now))
        for x in names:
            buf[x].copy_(dr[x])
        g.replay()
        _eager_work()
        flushed += int((a.head != head_before).sum())   # a flush moves head
        _same(out_a, out_b, f"out, replay {step}")
        for name in CACHE_FIELDS:
            _same(getattr(a, name), getattr(b, name), f"{name}, replay {step}")
        assert int(a.err.item()) == 0
    assert flushed > 0
    del g


def test_step_varlen_graph_matches_eager():
    """rollback_verify_flush with per-request lengths for the previous and the
    current draft (zeros included), both read from device buffers that change
    between replays; 32 requests x 32 heads, 6 replays."""
    wl = W["r32_hv32_hk16_d128_f16"]
    D, F = wl.draft, wl.flush_min_len
    say("case graph replay step, per-request lengths")
    rng = np.random.default_rng(807)
    init = synth.make_cache_init(wl, rng)
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    names = ("q", "k", "v", "alpha", "beta")
    R = wl.num_reqs
    buf = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    slots_buf = to_device(synth.make_slot_idx(wl, rng))
    acc_buf = torch.zeros(R, dtype=torch.int32, device="cuda")
    plen_buf = torch.zeros(R, dtype=torch.int32, device="cuda")
    len_buf = torch.zeros(R, dtype=torch.int32, device="cuda")
    out_a = torch.zeros((R, D, wl.hv, wl.dv), dtype=torch.float32, device="cuda")
    out_b = torch.zeros_like(out_a)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.rollback_verify_flush(slots_buf, acc_buf, D, F, *(buf[x] for x in names), out=out_b,
                                prev_draft_lens=plen_buf, draft_lens=len_buf)
    torch.cuda.synchronize()
    prev = {}                      # slot -> (accepted, length) of its last draft
    flushed = 0
    for step in range(6):
        slots = synth.make_slot_idx(wl, rng)
        lens = rng.integers(0, D + 1, R).astype(np.int32)
        acc = synth.sample_accepted(wl, rng, draft_lens=lens)
        pa = np.array([prev.get(int(s), (0, 0))[0] for s in slots], np.int32)
        pl = np.array([prev.get(int(s), (0, 0))[1] for s in slots], np.int32)
        dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
        sd = to_device(slots)
        head_before = a.head.clone()
        a.rollback_verify_flush(sd, to_device(pa), D, F, *(dr[x] for x in names), out=out_a,
                                prev_draft_lens=to_device(pl), draft_lens=to_device(lens))
        prev = {int(s): (int(acc[i]), int(lens[i])) for i, s in enumerate(slots)}
        slots_buf.copy_(sd)
        acc_buf.copy_(to_device(pa))
        plen_buf.copy_(to_device(pl))
        len_buf.copy_(to_device(lens))
        for x in names:
            buf[x].copy_(dr[x])
        g.replay()
        _eager_work()
        flushed += int((a.head != head_before).sum())
        _same(out_a, out_b, f"out, replay {step}")
        for name in CACHE_FIELDS:
            _same(getattr(a, name), getattr(b, name), f"{name}, replay {step}")
        assert int(a.err.item()) == 0
    assert flushed > 0
    del g


@pytest.mark.parametrize("write_out", [True, False])
def test_step_norm_graph_matches_eager(write_out):
    """gdn_replay_step_norm_fp8 at 32 requests x 32 heads, 5 replays with a new
    draft, gate, slot permutation and accept counts each time; out written or
    left out (codes and scales only)."""
    wl = W["r32_hv32_hk16_d128_f16"]
    D, F = wl.draft, wl.flush_min_len
    say(f"case graph replay step_norm, write_out={write_out}")
    rng = np.random.default_rng(805 + write_out)
    init = synth.make_cache_init(wl, rng)
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    names = ("q", "k", "v", "alpha", "beta")
    R, HV, dv = wl.num_reqs, wl.hv, wl.dv
    buf = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    slots_buf = to_device(synth.make_slot_idx(wl, rng))
    acc_buf = torch.zeros(R, dtype=torch.int32, device="cuda")
    z_buf = torch.zeros((R, D, HV, dv), dtype=torch.bfloat16, device="cuda")
    w = to_device(rng.uniform(0.5, 1.5, dv).astype(np.float32))
    mk = lambda: (torch.empty((R, D, HV, dv), dtype=torch.float32, device="cuda"),
                  torch.empty((R, D, HV, dv), dtype=torch.uint8, device="cuda"),
                  torch.empty((R, D, HV), dtype=torch.float32, device="cuda"))
    out_a, q_a, s_a = mk()
    out_b, q_b, s_b = mk()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.step_norm_fp8(slots_buf, acc_buf, D, F, *(buf[x] for x in names), z_buf, w, 1e-6,
                        out=out_b if write_out else None, codes=q_b, scale=s_b,
                        write_out=write_out)
    torch.cuda.synchronize()
    prev = {}
    flushed = 0
    for step in range(5):
        slots = synth.make_slot_idx(wl, rng)
        acc = synth.sample_accepted(wl, rng)
        acc_now = np.array([prev.get(int(s), 0) for s in slots], np.int32)
        dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
        z = torch.randn((R, D, HV, dv), device="cuda").to(torch.bfloat16)
        sd = to_device(slots)
        head_before = a.head.clone()
        a.step_norm_fp8(sd, to_device(acc_now), D, F, *(dr[x] for x in names), z, w, 1e-6,
                        out=out_a if write_out else None, codes=q_a, scale=s_a,
                        write_out=write_out)
        prev = {int(s): int(acc[i]) for i, s in enumerate(slots)}
        slots_buf.copy_(sd)
        acc_buf.copy_(to_device(acc_now))
        z_buf.copy_(z)
        for x in names:
            buf[x].copy_(dr[x])
        g.replay()
        _eager_work()
        flushed += int((a.head != head_before).sum())
        if write_out:
            _same(out_a, out_b, f"out, replay {step}")
        _same(q_a, q_b, f"codes, replay {step}")
        _same(s_a, s_b, f"scales, replay {step}")
        for name in CACHE_FIELDS:
            _same(getattr(a, name), getattr(b, name), f"{name}, replay {step}")
        assert int(a.err.item()) == 0
    assert flushed > 0
    del g


def test_norm_graph_matches_eager():
    from gated_deltanet_state_replayssm_amd.norm import gated_rmsnorm_fp8
    say("case graph replay gated RMSNorm + FP8")
    rows, H, dv = 64, 8, 128
    torch.manual_seed(801)
    w = torch.rand(dv, device="cuda") + 0.5
    o_buf = torch.randn((rows, H, dv), device="cuda")
    z_buf = torch.randn((rows, H, dv), device="cuda").to(torch.bfloat16)
    q_b = torch.empty((rows, H, dv), dtype=torch.uint8, device="cuda")
    s_b = torch.empty((rows, H), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gated_rmsnorm_fp8(o_buf, z_buf, w, 1e-6, q_b, s_b)
    torch.cuda.synchronize()
    for it in range(4):
        o = torch.randn((rows, H, dv), device="cuda") * (it + 1)
        z = torch.randn((rows, H, dv), device="cuda").to(torch.bfloat16)
        q_a, s_a = gated_rmsnorm_fp8(o, z, w, 1e-6)
        o_buf.copy_(o)
        z_buf.copy_(z)
        g.replay()
        _eager_work()
        _same(q_a, q_b, f"codes, replay {it}")
        _same(s_a, s_b, f"scales, replay {it}")
    del g


def test_conv_graph_matches_eager():
    """The pointers the convolution reads change between replays (written in
    place, as the recurrence's calls would)."""
    from gated_deltanet_state_replayssm_amd.conv import ConvRing
    say("case graph replay causal convolution")
    S, R, D, C, CH, K = 8, 6, 5, 16, 96, 4
    rng = np.random.default_rng(802)
    caches = [ReplayCache(S, 1, 1, 16, 16, C, synth.BF16) for _ in range(2)]
    rings = [ConvRing(c, CH, K) for c in caches]
    init_ring = torch.randn((S, C, CH), device="cuda").to(torch.bfloat16)
    for r in rings:
        r.ring.copy_(init_ring)
    w = torch.randn((CH, K), device="cuda") * 0.5
    bias = torch.randn((CH,), device="cuda")
    slots_buf = torch.zeros(R, dtype=torch.int32, device="cuda")
    x_buf = torch.zeros((R, D, CH), dtype=torch.bfloat16, device="cuda")
    y_b = torch.empty_like(x_buf)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rings[1].update(slots_buf, x_buf, w, bias, y_b)
    torch.cuda.synchronize()
    for it in range(4):
        head = to_device(rng.integers(0, C, S).astype(np.int32))
        length = to_device(rng.integers(0, C - D + 1, S).astype(np.int32))
        for c in caches:
            c.head.copy_(head)
            c.len.copy_(length)
        slots = to_device(rng.permutation(S)[:R].astype(np.int32))
        x = torch.randn((R, D, CH), device="cuda").to(torch.bfloat16)
        y_a = rings[0].update(slots, x, w, bias)
        slots_buf.copy_(slots)
        x_buf.copy_(x)
        g.replay()
        _eager_work()
        _same(y_a, y_b, f"outputs, replay {it}")
        _same(rings[0].ring, rings[1].ring, f"ring, replay {it}")
        assert int(caches[0].err.item()) == 0 and int(caches[1].err.item()) == 0
    del g
