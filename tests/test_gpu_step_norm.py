"""GPU parity of gdn_replay_step_norm_fp8 (the one-call step with the gated
RMSNorm + FP8 of its outputs in the same kernel), through the C ABI:

* out, state, ring, pointers and error word bit for bit against
  gdn_replay_rollback_verify_flush on a twin cache (itself checked against the
  oracle's rollback then verify_flush);
* codes and scales against the fp64 norm oracle evaluated on the kernel's own
  fp32 outputs: scales within 1e-5 relative, codes exact away from a rounding
  midpoint (either neighbour within a relative 1e-5 of one);
* the whole chain against the fp64 oracles (verify, then norm) with a bound
  that covers the output tolerance and half an E4M3 step;
* out = NULL gives the same codes and scales; rows past a request's draft
  length and skipped requests are left untouched."""
import numpy as np
import pytest
import torch

from gated_deltanet_state_replayssm_amd import synth
from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device
from oracle import gdn_oracle as go
from oracle import norm_oracle as no
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
DELTA = 1e-5
EPS = 1e-6
CANARY_Q = 0x5A
CANARY_S = -7.0
FIELDS = ("state", "head", "len", "ring_k", "ring_v", "ring_alpha", "ring_beta", "ring_q",
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


def _norm_inputs(wl, rng):
    z = synth.f32_to_bf16_bits((rng.standard_normal((wl.num_reqs, wl.draft, wl.hv, wl.dv)) * 2)
                               .astype(np.float32))
    w = rng.uniform(0.5, 1.5, wl.dv).astype(np.float32)
    return z, w


def _zf(zb):
    return (np.asarray(zb).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check_codes(o, zb, w, q, s, rows):
    """Boundary-aware check of the groups in `rows` ([R, D] bool) against the
    oracle evaluated on o (the kernel's fp32 outputs)."""
    y, s_ref, c_ref = no.gated_rmsnorm_fp8(o[rows].astype(np.float64), _zf(zb[rows]),
                                           w.astype(np.float64), EPS)
    qs, ss = q[rows], s[rows]
    nz = s_ref != 1.0
    np.testing.assert_allclose(ss[nz], s_ref[nz], rtol=DELTA, atol=0)
    assert (ss[~nz] == 1.0).all()
    x = y / s_ref[..., None]
    lo = no.e4m3_encode(x * (1 - DELTA))
    hi = no.e4m3_encode(x * (1 + DELTA))
    exact = lo == hi
    assert np.array_equal(qs[exact], c_ref[exact]), (
        f"{int((qs[exact] != c_ref[exact]).sum())} codes differ away from rounding midpoints")
    amb = ~exact
    assert ((qs[amb] == lo[amb]) | (qs[amb] == hi[amb])).all()
    assert amb.mean() < 1e-3
    return int(amb.sum())


def _check_chain(o_ref, zb, w, q, s, rows):
    """Codes * scale against the fp64 chain (oracle outputs, then the norm
    oracle): within half an E4M3 step (2^-4 relative, 2^-10 * scale absolute
    for subnormal codes) plus what the output tolerance can move."""
    y, s_ref, _ = no.gated_rmsnorm_fp8(o_ref[rows], _zf(zb[rows]), w.astype(np.float64), EPS)
    deq = no.e4m3_decode(q[rows]) * s[rows][..., None]
    amax = np.abs(y).max(axis=-1, keepdims=True)
    bound = 2.0 ** -4 * np.abs(y) + 2.0 ** -10 * s_ref[..., None] + 1e-2 * amax
    assert (np.abs(deq - y) <= bound).all(), float(np.max(np.abs(deq - y) - bound))


def _step_pair(wl, seed, steps, varlen_lens=False, with_oracle=False, write_out=True):
    rng = np.random.default_rng(seed)
    init = synth.make_cache_init(wl, rng)
    a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    orc = go.ReplayOracle(dict(init), wl.hv, wl.hk, wl.dk, wl.dv, wl.cap) if with_oracle else None
    R, D = wl.num_reqs, wl.draft
    prev = {}
    ambig = 0
    for step in range(steps):
        slots = synth.make_slot_idx(wl, rng)
        lens = rng.integers(0, D + 1, R).astype(np.int32) if varlen_lens else None
        acc = synth.sample_accepted(wl, rng, draft_lens=lens)
        pa = np.array([prev.get(int(s), (0, 0))[0] for s in slots], np.int32)
        pl = np.array([prev.get(int(s), (0, 0))[1] for s in slots], np.int32)
        dr = synth.make_draft(wl, rng)
        zb, w = _norm_inputs(wl, rng)
        dd = {k: to_device(v) for k, v in dr.items()}
        args = (to_device(slots), to_device(pa), D, wl.flush_min_len, dd["q"], dd["k"], dd["v"],
                dd["alpha"], dd["beta"])
        kw = dict(prev_draft_lens=to_device(pl), draft_lens=None if lens is None else to_device(lens))
        codes = torch.full((R, D, wl.hv, wl.dv), CANARY_Q, dtype=torch.uint8, device="cuda")
        scale = torch.full((R, D, wl.hv), CANARY_S, dtype=torch.float32, device="cuda")
        out_a = torch.full((R, D, wl.hv, wl.dv), 3.0, dtype=torch.float32, device="cuda")
        say(f"  step {step} lens={None if lens is None else list(lens[:8])} prev_acc={list(pa[:8])}")
        o_a, q, s = a.step_norm_fp8(*args, to_device(zb), to_device(w), EPS,
                                    out=out_a if write_out else None, codes=codes, scale=scale,
                                    write_out=write_out, **kw)
        out_b = torch.full_like(out_a, 3.0)
        b.rollback_verify_flush(*args, out=out_b, **kw)
        torch.cuda.synchronize()
        for name in FIELDS:
            assert torch.equal(_bits(getattr(a, name)), _bits(getattr(b, name))), name
        ob = out_b.cpu().numpy()
        Ds = np.full(R, D) if lens is None else lens
        rows = np.arange(D)[None, :] < Ds[:, None]          # draft rows of every request
        if write_out:
            # the fused kernel places the draft at fixed rows of its chunk (a
            # split output chunk), which changes the rounding order only; rows
            # past a request's draft keep their canary in both
            oa_h = o_a.cpu().numpy()
            assert np.array_equal(oa_h[~rows], ob[~rows]) and (ob[~rows] == 3.0).all(), "out rows"
            scale = max(float(np.abs(ob[rows]).max()), 1e-30)
            assert np.abs(oa_h[rows] - ob[rows]).max() <= 2e-4 * scale, "out"
        else:
            assert o_a is None
        qn, sn = q.cpu().numpy(), s.cpu().numpy()
        # the boundary-aware check runs on the fused kernel's own outputs (its
        # rounding order is not the separate step's); without them, the codes
        # are checked against a run that writes them (and the fp64 chain)
        if write_out:
            ambig += _check_codes(oa_h, zb, w, qn, sn, rows)
        assert (qn[~rows] == CANARY_Q).all() and (sn[~rows] == CANARY_S).all()
        if orc is not None:
            orc.rollback(slots, D, pa, draft_lens=pl)
            ref = orc.verify_flush(slots, wl.flush_min_len,
                                   *(dr[x] for x in ("q", "k", "v", "alpha", "beta")),
                                   draft_lens=lens)
            assert not np.isnan(ref[rows]).any()
            _check_chain(ref, zb, w, qn, sn, rows)
        prev = {int(sl): (int(acc[i]), int(Ds[i])) for i, sl in enumerate(slots)}
        yield step, qn, sn
    assert int(a.err.item()) == 0
    say(f"  {ambig} codes at a rounding midpoint (either neighbour accepted)")


# draft 16 and a flush every 16: the split output chunk (draft rows from row
# 16); a flush every 24 (up to 23 committed rows) or a draft of 20: the plain
# layout for those slots
@pytest.mark.parametrize("d,varlen,draft,flush", [(128, False, 16, 16), (128, True, 16, 16),
                                                  (64, False, 16, 16), (64, True, 16, 16),
                                                  (128, False, 8, 24), (128, True, 20, 12)])
def test_step_norm_parity(d, varlen, draft, flush):
    wl = synth.Workload("sn", 6, 8, 8, 4, d, d, 32, draft, synth.BF16, flush, 1,
                        "clipnormal:12:3", f"uniform:0:{min(flush, 32 - draft) - 1}")
    say(f"case step_norm d={d} varlen={varlen} draft={draft} flush={flush}")
    for _ in _step_pair(wl, 900 + d + varlen + draft, 5, varlen_lens=varlen, with_oracle=True):
        pass


def test_step_norm_pages_point():
    """32 requests x 32 heads x 128, 3 steps: the boundary-aware check of the
    codes on the kernel's own outputs, and the fp64 chain (the oracle's
    rollback and verify_flush, then the norm oracle) on every request."""
    wl = W["r32_hv32_hk16_d128_f16"]
    say("case step_norm r32 full size, fp64 chain on every request")
    for _ in _step_pair(wl, 910, 3, with_oracle=True):
        pass


def test_step_norm_without_out_gives_the_same_codes():
    wl = synth.Workload("sn0", 6, 8, 8, 4, 128, 128, 32, 16, synth.BF16, 16, 1, "clipnormal:12:3",
                        "uniform:0:15")
    say("case step_norm out = NULL")
    with_out = [(q, s) for _, q, s in _step_pair(wl, 920, 4, varlen_lens=True)]
    without = [(q, s) for _, q, s in _step_pair(wl, 920, 4, varlen_lens=True, write_out=False)]
    for (q1, s1), (q2, s2) in zip(with_out, without):
        assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.int32), s2.view(np.int32))


def test_step_norm_skipped_requests_untouched():
    """A bad slot and bad pointers: no codes or scales for those requests, the
    others normalised as usual; error word as the step's."""
    wl = synth.Workload("sne", 4, 6, 4, 2, 64, 64, 32, 8, synth.BF16, 16, 1, "uniform",
                        "uniform:0:4")
    say("case step_norm device errors")
    rng = np.random.default_rng(930)
    init = synth.make_cache_init(wl, rng)
    init["head"][3] = 99                      # slot 3: POINTER
    c = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
    slots = np.array([0, 9, 3, 1], np.int32)  # 9: SLOT
    dr = {k: to_device(v) for k, v in synth.make_draft(wl, rng).items()}
    zb, w = _norm_inputs(wl, rng)
    codes = torch.full((4, 8, wl.hv, wl.dv), CANARY_Q, dtype=torch.uint8, device="cuda")
    scale = torch.full((4, 8, wl.hv), CANARY_S, dtype=torch.float32, device="cuda")
    out, q, s = c.step_norm_fp8(to_device(slots), to_device(np.zeros(4, np.int32)), 8, 16,
                                dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"],
                                to_device(zb), to_device(w), EPS, codes=codes, scale=scale)
    torch.cuda.synchronize()
    assert int(c.err.item()) == go.ERR_SLOT | go.ERR_POINTER
    qn, sn = q.cpu().numpy(), s.cpu().numpy()
    assert (qn[[1, 2]] == CANARY_Q).all() and (sn[[1, 2]] == CANARY_S).all()
    rows = np.zeros((4, 8), bool)
    rows[[0, 3]] = True
    _check_codes(out.cpu().numpy(), zb, w, qn, sn, rows)
