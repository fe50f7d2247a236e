"""GPU parity of gdn_gated_rmsnorm_fp8 against the fp64 oracle, through the C ABI.

Scales within 1e-5 relative. Codes: the oracle's exact value x = y / s decides
each code; where x lies within a relative 1e-5 of the midpoint between two codes
(closer than the fp32 arithmetic of the kernel can resolve) either neighbour is
accepted, everywhere else the code must be the oracle's exactly."""
import numpy as np
import pytest
import torch

from gated_deltanet_state_replayssm_amd import synth
from gated_deltanet_state_replayssm_amd.cache import to_device
from gated_deltanet_state_replayssm_amd.norm import gated_rmsnorm_fp8
from oracle import norm_oracle as no
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

DELTA = 1e-5


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_state_replayssm_amd import binding
    binding.load()


def _inputs(rng, rows, H, dv):
    """o with per-group magnitudes over six decades, a bf16 gate, a weight; a few
    special groups: zero rows, zero gates, one dominant value, tiny values."""
    o = rng.standard_normal((rows, H, dv)) * 10.0 ** rng.uniform(-3, 3, (rows, H, 1))
    o = o.astype(np.float32)
    z = (rng.standard_normal((rows, H, dv)) * 2.0).astype(np.float32)
    w = rng.uniform(0.5, 1.5, dv).astype(np.float32)
    if rows >= 2 and H >= 2:
        o[0, 0] = 0.0                      # all-zero group
        z[0, 1] = 0.0                      # zero gate
        o[1, 0] *= 1e-3
        o[1, 0, 3] = 50.0                  # one dominant value: most codes subnormal or 0
        o[1, 1] = np.float32(1e-30) * o[1, 1]
    zb = synth.f32_to_bf16_bits(z)
    return o, zb, w


def _check(o, zb, w, eps, q, s):
    zf = (zb.astype(np.uint32) << 16).view(np.float32)
    y, s_ref, c_ref = no.gated_rmsnorm_fp8(o.astype(np.float64), zf.astype(np.float64),
                                           w.astype(np.float64), eps)
    nz = s_ref != 1.0
    np.testing.assert_allclose(s[nz], s_ref[nz], rtol=DELTA, atol=0)
    assert (s[~nz] == 1.0).all()
    x = y / s_ref[..., None]
    lo = no.e4m3_encode(x * (1 - DELTA))
    hi = no.e4m3_encode(x * (1 + DELTA))
    exact = lo == hi
    assert np.array_equal(q[exact], c_ref[exact]), (
        f"{int((q[exact] != c_ref[exact]).sum())} codes differ away from rounding midpoints")
    amb = ~exact
    assert ((q[amb] == lo[amb]) | (q[amb] == hi[amb])).all()
    assert amb.mean() < 1e-3, f"too many near-midpoint values: {amb.mean():.2e}"
    return int(amb.sum()), q.size


@pytest.mark.parametrize("rows,H,dv", [(512, 32, 128), (37, 5, 128), (64, 8, 64), (33, 3, 32),
                                       (20, 4, 16)])
def test_gated_rmsnorm_fp8_parity(rows, H, dv):
    say(f"case norm rows={rows} H={H} dv={dv}")
    rng = np.random.default_rng(rows * 1000 + H * 10 + dv)
    o, zb, w = _inputs(rng, rows, H, dv)
    eps = 1e-6
    q, s = gated_rmsnorm_fp8(to_device(o), to_device(zb), to_device(w), eps)
    torch.cuda.synchronize()
    amb, n = _check(o, zb, w, eps, q.cpu().numpy(), s.cpu().numpy())
    say(f"  {amb} of {n} codes at a rounding midpoint (either neighbour accepted)")


def test_gated_rmsnorm_fp8_on_verify_outputs_shape_and_zero_rows():
    """The verify output layout [R][D][HV][dv] is taken as rows = R * D; zero rows
    launch nothing and leave the outputs untouched."""
    rng = np.random.default_rng(9)
    o, zb, w = _inputs(rng, 4 * 16, 32, 128)
    o4 = to_device(o.reshape(4, 16, 32, 128))
    z4 = to_device(zb.reshape(4, 16, 32, 128))
    q, s = gated_rmsnorm_fp8(o4, z4, to_device(w), 1e-5)
    torch.cuda.synchronize()
    assert q.shape == (4, 16, 32, 128) and s.shape == (4, 16, 32)
    _check(o, zb, w, 1e-5, q.cpu().numpy().reshape(64, 32, 128), s.cpu().numpy().reshape(64, 32))
    qe = torch.full((0, 32, 128), 7, dtype=torch.uint8, device="cuda")
    se = torch.full((0, 32), 7.0, device="cuda")
    gated_rmsnorm_fp8(torch.empty((0, 32, 128), device="cuda"),
                      torch.empty((0, 32, 128), dtype=torch.bfloat16, device="cuda"),
                      to_device(w), 1e-5, qe, se)
    torch.cuda.synchronize()
