"""Pins of the bf16 handling that every bf16 workload goes through.

bf16 is the storage format of the q, k, v inputs ("The inference stack behind
OCRia", section on workload-aware quantization, which keeps BF16 among the
formats it serves; "Inference Engineering", chapter 5, section 5.1.1, number
formats). The format is fixed by its definition: 1 sign bit, 8 exponent bits
with bias 127, 7 fraction bits, i.e. the upper half of an IEEE binary32. The
pins below check

* the oracle's decode (bf16_bits_to_f64, and to_f64 on bf16 bits) against a
  table of patterns whose values the format fixes, and exhaustively against a
  decode of the three fields with integer arithmetic and ldexp (no bit
  reinterpretation, so it shares nothing with the decoder under test);
* the host encoder that rounds the synthetic inputs (and the convolution's
  expected outputs) to bf16 against round-to-nearest-even: hand-picked ties
  and carries, and a brute-force nearest-value search on random inputs;
* conv_oracle.silu against closed-form values.
"""
import math

import numpy as np

from gated_deltanet_state_replayssm_amd import synth
from oracle import conv_oracle as co
from oracle import gdn_oracle as go

# bit pattern -> value fixed by the format (sign, exponent - 127, 1.fraction)
BF16_TABLE = [
    (0x0000, 0.0),
    (0x3F80, 1.0),
    (0xBF80, -1.0),
    (0xC000, -2.0),
    (0x3F00, 0.5),
    (0x4049, 3.140625),                        # 2 * (1 + 73/128)
    (0x4120, 10.0),                            # 8 * (1 + 32/128)
    (0x3DCD, 0.10009765625),                   # 2^-4 * (1 + 77/128)
    (0x0080, 2.0 ** -126),                     # smallest normal
    (0x0001, 2.0 ** -133),                     # smallest subnormal: 2^-126 * 1/128
    (0x007F, 127 * 2.0 ** -133),               # largest subnormal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0xFF7F, -(2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
]


def _decode_fields(bits: int) -> float:
    """bf16 value from its fields, as the format defines it."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        return math.nan if m else sign * math.inf
    if e == 0:
        return sign * math.ldexp(m, -126 - 7)
    return sign * math.ldexp(128 + m, e - 127 - 7)


def test_bf16_decode_table():
    bits = np.array([b for b, _ in BF16_TABLE], dtype=np.uint16)
    want = np.array([v for _, v in BF16_TABLE], dtype=np.float64)
    got = go.bf16_bits_to_f64(bits)
    assert got.dtype == np.float64
    assert np.array_equal(got, want)
    # the dispatch used on every oracle input: uint16 arrays are bf16 bits
    assert np.array_equal(go.to_f64(bits), want)
    # negative zero keeps its sign
    assert math.copysign(1.0, float(go.bf16_bits_to_f64(np.array([0x8000], np.uint16))[0])) == -1.0


def test_bf16_decode_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):   # NaN patterns
        got = go.bf16_bits_to_f64(bits)
    want = np.array([_decode_fields(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_to_f64_keeps_fp32_values():
    x = np.array([1.0, -0.1, 3.0e-39, 1.0e30], dtype=np.float32)
    got = go.to_f64(x)
    assert got.dtype == np.float64
    assert np.array_equal(got, x.astype(np.float64))


def _f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


# fp32 bit pattern -> bf16 bit pattern under round-to-nearest-even
RNE_TABLE = [
    (0x3F800000, 0x3F80),  # exact
    (0x3F807FFF, 0x3F80),  # just below the midpoint
    (0x3F808000, 0x3F80),  # tie, even neighbour below
    (0x3F808001, 0x3F81),  # just above the midpoint
    (0x3F818000, 0x3F82),  # tie, even neighbour above
    (0xBF818000, 0xBF82),  # the same tie, negative
    (0xBF808000, 0xBF80),
    (0x3FFF8000, 0x4000),  # tie that carries into the exponent
    (0x3FFFFFFF, 0x4000),
    (0x00008000, 0x0000),  # subnormal tie, even below
    (0x00018000, 0x0002),  # subnormal tie, even above
    (0x7F7F7FFF, 0x7F7F),  # rounds down to the largest finite
    (0x7F7F8000, 0x7F80),  # tie above the largest finite rounds to infinity (odd fraction)
]


def test_bf16_encode_ties_and_carries():
    src = _f32([a for a, _ in RNE_TABLE])
    want = np.array([b for _, b in RNE_TABLE], dtype=np.uint16)
    got = synth.f32_to_bf16_bits(src)
    assert got.dtype == np.uint16
    assert np.array_equal(got, want), [(hex(a), hex(b), hex(int(g)))
                                       for (a, b), g in zip(RNE_TABLE, got) if b != g]


def test_bf16_encode_is_nearest_even_brute_force():
    rng = np.random.default_rng(7)
    # finite fp32 below the largest bf16 midpoint, every exponent, plus exact ties
    u = rng.integers(0, 0x7F7F8000, 20000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 0x7F7F, 2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, u | 0x80000000])
    x = u.view(np.float32)
    got = synth.f32_to_bf16_bits(x)
    for xi, gi in zip(x.astype(np.float64), got):
        down = (int(np.float32(xi).view(np.uint32)) >> 16)  # toward zero
        cands = [down, down + 1]
        vals = [_decode_fields(c) for c in cands]
        d = [abs(v - xi) for v in vals]
        if d[0] < d[1]:
            best = cands[0]
        elif d[1] < d[0]:
            best = cands[1]
        else:
            best = cands[0] if cands[0] % 2 == 0 else cands[1]
        assert int(gi) == best, (float(xi), hex(int(gi)), hex(best))


def test_conv_silu_closed_forms():
    ln3 = math.log(3.0)
    x = np.array([0.0, ln3, -ln3, 1.0, 40.0, -40.0])
    got = co.silu(x)
    # sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4, sigma(1) = e / (1 + e)
    want = np.array([0.0, 0.75 * ln3, -0.25 * ln3, math.e / (1.0 + math.e), 40.0,
                     -40.0 * math.exp(-40.0)])
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=0)
    z = np.linspace(-6, 6, 49)
    np.testing.assert_allclose(co.silu(z) - co.silu(-z), z, rtol=0, atol=1e-13)
