"""Pins of the gated RMSNorm + FP8 (OCP E4M3) oracle against the format's
definition and the mathematics, independent of its own formulas."""
import numpy as np
import pytest

from oracle import norm_oracle as no


def test_e4m3_known_codes():
    """Values fixed by the E4M3 definition (sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 is subnormal; 0x7F is NaN)."""
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xC0: -2.0, 0xB8: -1.0}
    for c, v in table.items():
        assert no.e4m3_decode(np.array([c]))[0] == v, hex(c)
    assert np.isnan(no.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert np.signbit(no.e4m3_decode(np.array([0x80]))[0])


def test_e4m3_round_trip_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(no.e4m3_encode(no.e4m3_decode(codes)), codes)


def _brute_encode(x):
    """argmin over all finite codes of |value - x|, ties to the code whose
    mantissa LSB is 0; saturation at the largest finite magnitude."""
    codes = np.array([c for c in range(128) if c != 0x7F])
    vals = no.e4m3_decode(codes)
    out = []
    for xi in np.asarray(x, dtype=np.float64):
        a = min(abs(xi), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else [b for b in best if codes[b] % 2 == 0][0]
        out.append(codes[c] | (0x80 if np.signbit(xi) else 0))
    return np.array(out, dtype=np.uint8)


def test_e4m3_rounding_matches_brute_force():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(2000) * 50, rng.standard_normal(500) * 1e-2,
                        rng.standard_normal(200) * 1e4])
    # exact midpoints between neighbouring codes: ties go to the even code
    v = no.e4m3_decode(np.arange(0x7E))
    mids = (v[:-1] + v[1:]) / 2
    x = np.concatenate([x, mids, -mids, [0.0, -0.0, 448.0, 449.0, 464.0, 1e30, -1e30]])
    assert np.array_equal(no.e4m3_encode(x), _brute_encode(x))
    assert no.e4m3_encode(np.array([1.0625]))[0] == 0x38      # 1 + 1/16: tie -> 1.0 (even)
    assert no.e4m3_encode(np.array([1.1875]))[0] == 0x3A      # 1 + 3/16: tie -> 1.25 (even)


def test_silu_identities():
    x = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(no.silu(x) - no.silu(-x), x, rtol=0, atol=1e-12)
    assert no.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(no.silu(np.array([1.0]))[0], 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)


def test_gated_rmsnorm_invariants():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((5, 3, 64))
    z = rng.standard_normal((5, 3, 64))
    w = rng.uniform(0.5, 1.5, 64)
    y = no.gated_rmsnorm(o, z, w, 0.0)
    # scale invariance in o (eps = 0) and linearity in the weight
    np.testing.assert_allclose(no.gated_rmsnorm(7.5 * o, z, w, 0.0), y, rtol=1e-13, atol=0)
    np.testing.assert_allclose(no.gated_rmsnorm(o, z, 2 * w, 0.0), 2 * y, rtol=1e-13, atol=0)
    # the normalised vector has unit root mean square
    u = y / (w * no.silu(z))
    np.testing.assert_allclose(np.mean(u * u, axis=-1), 1.0, rtol=1e-13)
    # zero gate gives zero; signs multiply
    assert (no.gated_rmsnorm(o, np.zeros_like(z), w, 0.0) == 0).all()
    assert (np.sign(y) == np.sign(o) * np.sign(no.silu(z))).all()
    # eps: a constant row c has r = sqrt(c^2 + eps)
    c = 0.25
    yc = no.gated_rmsnorm(np.full((1, 8), c), np.full((1, 8), 3.0), np.ones(8), 1e-2)
    np.testing.assert_allclose(yc, c / np.sqrt(c * c + 1e-2) * no.silu(np.array(3.0)), rtol=1e-14)


def test_group_scale_and_codes():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((4, 2, 128))
    z = rng.standard_normal((4, 2, 128))
    w = rng.uniform(0.5, 1.5, 128)
    y, s, c = no.gated_rmsnorm_fp8(o, z, w, 1e-6)
    # the largest magnitude of every group lands on +-448
    i = np.argmax(np.abs(y), axis=-1)
    top = np.take_along_axis(c, i[..., None], axis=-1)[..., 0]
    assert np.isin(top, [0x7E, 0xFE]).all()
    # dequantised values are within half a code step of y (3 mantissa bits)
    deq = no.e4m3_decode(c) * s[..., None]
    step = np.maximum(np.abs(y), 2.0 ** -6 * s[..., None]) * 2.0 ** -3
    assert (np.abs(deq - y) <= step / 2 + 1e-12).all()
    # all-zero group (zero gate): scale 1, codes +-0 (the sign of o is kept)
    y0, s0, c0 = no.gated_rmsnorm_fp8(o[:1], np.zeros_like(z[:1]), w, 1e-6)
    assert (s0 == 1.0).all() and ((c0 & 0x7F) == 0).all()
    assert ((c0 == 0x80) == (o[:1] < 0)).all()


@pytest.mark.parametrize("bad", ["ties_away", "bias8"])
def test_planted_encoder_mistakes_are_caught(bad, monkeypatch):
    """Mistakes in the encoder (ties away from zero, the FNUZ bias) fail the
    pins above."""
    if bad == "ties_away":
        def enc(x):
            x = np.asarray(x, dtype=np.float64)
            a = np.minimum(np.abs(x), 448.0)
            lo = np.searchsorted(no._POS, a, side="right") - 1
            hi = np.minimum(lo + 1, 0x7E)
            up = (no._POS[hi] - a) <= (a - no._POS[lo])
            code = np.where(up & (hi != lo), hi, lo)
            return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
        monkeypatch.setattr(no, "e4m3_encode", enc)
        with pytest.raises(AssertionError):
            test_e4m3_rounding_matches_brute_force()
    else:
        orig = no.e4m3_decode
        monkeypatch.setattr(no, "E4M3_BIAS", 8)
        with pytest.raises(AssertionError):
            test_e4m3_known_codes()
        assert orig is no.e4m3_decode
