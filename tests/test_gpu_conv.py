"""GPU parity of gdn_causal_conv_update (the causal convolution before the
recurrence, history in a ring that shares the recurrence's pointers) against the
fp64 oracle, through the C ABI, over multi-step schedules with rollbacks and
flushes driven by the recurrence's own calls.

Outputs are bf16: each must be the oracle's value rounded to nearest even,
except where the oracle's value lies within the fp32 error bound of the
kernel's sum (1e-6 of |b| + sum |w x|, four times the bound of a 4-term fp32
sum, plus 1e-6 of |y| for the exponential)
from a rounding midpoint, where any bf16 value between the roundings of the
window's ends is accepted. The ring is compared bit for bit."""
import numpy as np
import pytest
import torch

from gated_deltanet_state_replayssm_amd import synth
from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device, to_host
from gated_deltanet_state_replayssm_amd.conv import ConvRing
from oracle import conv_oracle as co
from oracle import gdn_oracle as go
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu



@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_replayssm_amd import binding
    binding.load()


def _bf16(v64):
    return synth.f32_to_bf16_bits(np.asarray(v64, dtype=np.float64).astype(np.float32))


def _check_out(got_bits, ref, mag):
    ok = ~np.isnan(ref)
    eps = 1e-6 * np.nan_to_num(mag) + 1e-6 * np.abs(np.nan_to_num(ref))
    lo, hi = _bf16(ref - eps), _bf16(ref + eps)
    exact = ok & (lo == hi)
    assert np.array_equal(got_bits[exact], lo[exact]), (
        f"{int((got_bits[exact] != lo[exact]).sum())} outputs differ away from rounding midpoints")
    amb = ok & ~exact
    val = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32)
    g, a, c = val(got_bits[amb]), val(lo[amb]), val(hi[amb])
    assert ((a <= g) & (g <= c)).all(), "outputs outside the rounding of the error window"
    assert amb.sum() <= max(0.05 * ok.sum(), 1)
    return int(amb.sum())


def _run(wl, CH, K, steps, seed, with_bias=True, fused=False):
    rng = np.random.default_rng(seed)
    init = synth.make_cache_init(wl, rng)
    cache = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    conv = ConvRing(cache, CH, K)
    orc_ptr = go.ReplayOracle(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, mode="replay")
    orc = co.ConvOracle(np.zeros((wl.num_slots, wl.cap, CH), np.uint16), wl.cap)
    w = rng.standard_normal((CH, K)).astype(np.float32) * 0.5
    bias = rng.standard_normal(CH).astype(np.float32) if with_bias else None
    wd = to_device(w)
    bd = None if bias is None else to_device(bias)
    amb = 0
    for step in range(steps):
        slots = synth.make_slot_idx(wl, rng)
        x = synth.f32_to_bf16_bits(rng.standard_normal((wl.num_reqs, wl.draft, CH)).astype(np.float32))
        dr = synth.make_draft(wl, rng)
        acc = synth.sample_accepted(wl, rng)
        sd = to_device(slots)
        y = conv.update(sd, to_device(x), wd, bd)
        ref, mag = orc.update(orc_ptr.head.copy(), orc_ptr.len.copy(), slots, x, w, bias,
                              magnitudes=True)
        # the recurrence's step moves the shared pointers
        dd = {k: to_device(v) for k, v in dr.items()}
        if fused:
            cache.verify_flush(sd, wl.flush_min_len, dd["q"], dd["k"], dd["v"], dd["alpha"],
                               dd["beta"])
            orc_ptr.flush(slots, wl.flush_min_len)
        else:
            cache.verify(sd, dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"])
        cache.rollback(sd, wl.draft, to_device(acc))
        orc_ptr.rollback(slots, wl.draft, acc)
        if not fused:
            cache.flush(sd, wl.flush_min_len)
            orc_ptr.flush(slots, wl.flush_min_len)
        torch.cuda.synchronize()
        amb += _check_out(to_host(y), ref, mag)
        assert np.array_equal(to_host(conv.ring), orc.ring), f"conv ring differs at step {step}"
        assert np.array_equal(to_host(cache.head), orc_ptr.head.astype(np.int32))
        assert np.array_equal(to_host(cache.len), orc_ptr.len.astype(np.int32))
        assert int(cache.err.item()) == 0 and orc.err == 0
    return amb


# channels a multiple of 8 take the 16-byte kernel (groups of 4 draft tokens;
# drafts of 5 and 7 leave a ragged group), the others the 4-byte one
@pytest.mark.parametrize("K,CH,fused,D", [(4, 256, False, 4), (4, 1024, True, 4), (2, 66, False, 4),
                                          (1, 8, True, 4), (8, 130, False, 4), (8, 136, False, 5),
                                          (3, 24, True, 7)])
def test_conv_schedule(K, CH, fused, D):
    wl = synth.Workload("cv", 5, 7, 4, 2, 32, 32, 16, D, synth.BF16, 6, 1, "uniform",
                        "uniform:0:5")
    say(f"case conv K={K} CH={CH} fused={fused} D={D}")
    amb = _run(wl, CH, K, 12, 700 + K * 10 + CH, with_bias=(K % 2 == 0), fused=fused)
    say(f"  {amb} outputs at a bf16 rounding midpoint")


def test_conv_pages_point():
    """32 requests, D = 16, q/k/v channels of 16 key heads x 128 (x2) and 32 value
    heads x 128, K = 4, ring capacity 32 shared with the recurrence's cache."""
    wl = synth.Workload("cvp", 32, 32, 32, 16, 128, 128, 32, 16, synth.BF16, 16, 1,
                        "clipnormal:12:3", "fixed:0")
    say("case conv pages' point")
    _run(wl, 2 * 16 * 128 + 32 * 128, 4, 3, 710, fused=True)


def test_conv_device_errors():
    wl = synth.Workload("cve", 4, 5, 4, 2, 32, 32, 12, 4, synth.BF16, 1, 1, "uniform", "fixed:0")
    rng = np.random.default_rng(711)
    init = synth.make_cache_init(wl, rng)
    init["len"][:] = [9, 1, 2, 3, 0]        # slot 0: 9 + 4 > 12 is fine here
    init["head"][3] = 20                    # slot 3: POINTER
    cache = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    conv = ConvRing(cache, 16, 3)
    x = to_device(synth.f32_to_bf16_bits(np.ones((4, 4, 16), np.float32)))
    y = torch.full((4, 4, 16), 7.0, dtype=torch.bfloat16, device="cuda")
    conv.update(to_device(np.array([0, 3, 9, 1], np.int32)), x,
                to_device(np.ones((16, 3), np.float32)), y=y)
    torch.cuda.synchronize()
    assert int(cache.err.item()) == 4 | 8
    yh = y.float().cpu().numpy()
    assert (yh[1:3] == 7.0).all() and (yh[[0, 3]] != 7.0).all()
    ring = to_host(conv.ring)
    assert not ring[[2, 3]].any() and ring[0].any() and ring[1].any()


def _run_one_call(wl, CH, K, steps, seed, bad_accept=False):
    """The convolution composed with the one-call step: per step, the
    convolution (given the step's pending rollback) and then
    gdn_replay_rollback_verify_flush, on one cache; the oracle side commits the
    previous draft's accepted prefix first and evaluates the convolution from
    the committed count that gives, then runs verify_flush. With bad_accept, one
    request per step passes an accepted count above its previous draft's length:
    the step keeps its len (and flags ACCEPT), and so must the convolution."""
    rng = np.random.default_rng(seed)
    init = synth.make_cache_init(wl, rng)
    cache = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    conv = ConvRing(cache, CH, K)
    orc_ptr = go.ReplayOracle(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, mode="replay")
    orc = co.ConvOracle(np.zeros((wl.num_slots, wl.cap, CH), np.uint16), wl.cap)
    w = rng.standard_normal((CH, K)).astype(np.float32) * 0.5
    bias = rng.standard_normal(CH).astype(np.float32)
    wd, bd = to_device(w), to_device(bias)
    D = wl.draft
    pending = {}
    amb = 0
    for step in range(steps):
        slots = synth.make_slot_idx(wl, rng)
        lens = rng.integers(0, D + 1, wl.num_reqs).astype(np.int32)
        acc = synth.sample_accepted(wl, rng, draft_lens=lens)
        pa = np.array([pending.get(int(s), (0, 0))[0] for s in slots], np.int32)
        pl = np.array([pending.get(int(s), (0, 0))[1] for s in slots], np.int32)
        if bad_accept and step > 0:
            pa[0] = pl[0] + 1
        x = synth.f32_to_bf16_bits(rng.standard_normal((wl.num_reqs, D, CH)).astype(np.float32))
        dr = synth.make_draft(wl, rng)
        say(f"  step {step} pa={list(pa)} pl={list(pl)} lens={list(lens)}")
        sd, pad, pld, ld = to_device(slots), to_device(pa), to_device(pl), to_device(lens)
        y = conv.update(sd, to_device(x), wd, bd, num_accepted=pad, prev_draft=D,
                        prev_draft_lens=pld)
        dd = {k: to_device(v) for k, v in dr.items()}
        cache.rollback_verify_flush(sd, pad, D, wl.flush_min_len, dd["q"], dd["k"], dd["v"],
                                    dd["alpha"], dd["beta"], prev_draft_lens=pld, draft_lens=ld)
        torch.cuda.synchronize()
        orc_ptr.rollback(slots, D, pa, draft_lens=pl)
        ref, mag = orc.update(orc_ptr.head.copy(), orc_ptr.len.copy(), slots, x, w, bias,
                              magnitudes=True)
        orc_ptr.verify_flush(slots, wl.flush_min_len,
                             *(dr[k] for k in ("q", "k", "v", "alpha", "beta")), draft_lens=lens)
        # rows past a request's draft length are computed by the convolution
        # (it takes the fixed block) and compared too
        amb += _check_out(to_host(y), ref, mag)
        assert np.array_equal(to_host(conv.ring), orc.ring), f"conv ring differs at step {step}"
        assert np.array_equal(to_host(cache.head), orc_ptr.head.astype(np.int32))
        assert np.array_equal(to_host(cache.len), orc_ptr.len.astype(np.int32))
        assert int(cache.err.item()) == orc_ptr.err
        pending = {int(s): (int(acc[i]), int(lens[i])) for i, s in enumerate(slots)}
    return amb


@pytest.mark.parametrize("bad_accept", [False, True])
def test_conv_composes_with_the_one_call_step(bad_accept):
    """Convolution then rollback_verify_flush, every step, per-request draft
    lengths, ring capacity 32 shared by both rings, flush every 8."""
    wl = synth.Workload("cv1", 6, 8, 4, 2, 64, 64, 32, 8, synth.BF16, 8, 1, "uniform",
                        "uniform:0:15")
    say(f"case conv + one-call step, bad_accept={bad_accept}")
    amb = _run_one_call(wl, 384, 4, 10, 740 + bad_accept, bad_accept=bad_accept)
    say(f"  {amb} outputs at a bf16 rounding midpoint")
