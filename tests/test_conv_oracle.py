"""Pins of the causal-convolution oracle (ring history, pointer-only rollback)
against closed forms and a plain causal convolution over the committed stream."""
import numpy as np
import pytest
from numpy.lib.stride_tricks import sliding_window_view

from gated_deltanet_state_replayssm_amd import synth
from oracle import bookkeeping as bk
from oracle import conv_oracle as co
from oracle import gdn_oracle as go


def _silu(x):
    return x * (1.0 / (1.0 + np.exp(-x)))


def test_identity_and_shift_kernels():
    """w = e_{K-1}: y = silu(x) of the same token; w = e_0: y_j = silu(x_{j-K+1}),
    the first K - 1 outputs coming from the committed history, oldest first."""
    K, C, CH, D = 4, 16, 8, 5
    rng = np.random.default_rng(1)
    ring = np.zeros((2, C, CH), np.float32)
    hist = rng.standard_normal((3, CH)).astype(np.float32)
    head, length = np.array([14, 0]), np.array([3, 0])
    for m in range(3):                       # committed inputs at 14, 15, 0
        ring[0, (14 + m) % C] = hist[m]
    x = rng.standard_normal((1, D, CH)).astype(np.float32)
    w_id = np.zeros((CH, K)); w_id[:, K - 1] = 1
    orc = co.ConvOracle(ring, C)
    y = orc.update(head, length, [0], x, w_id)
    np.testing.assert_allclose(y[0], _silu(x[0].astype(np.float64)), rtol=1e-15)
    w_sh = np.zeros((CH, K)); w_sh[:, 0] = 1
    orc = co.ConvOracle(ring, C)
    y = orc.update(head, length, [0], x, w_sh)
    expect = np.concatenate([hist, x[0, :D - 3]]).astype(np.float64)
    np.testing.assert_allclose(y[0], _silu(expect), rtol=1e-15)
    # the draft was appended behind the committed inputs
    for j in range(D):
        assert np.array_equal(orc.ring[0, (14 + 3 + j) % C], x[0, j])
    # a fresh slot reads zeros: y_0 = silu(b) with the shift kernel
    orc = co.ConvOracle(ring, C)
    y = orc.update(head, length, [1], x, w_sh, bias=np.full(CH, 0.5))
    np.testing.assert_allclose(y[0, :3], _silu(np.full((3, CH), 0.5)), rtol=1e-15)


@pytest.mark.parametrize("K", [2, 4])
def test_schedule_equals_plain_causal_conv(K):
    """Many steps of update -> rollback (len += a) -> flush of the due slots: every
    draft output equals a plain causal convolution (zero padded) over the slot's
    committed inputs followed by the draft."""
    wl = synth.Workload("cv", 3, 4, 1, 1, 8, 8, 24, 6, synth.BF16, 7, 1, "uniform", "fixed:0")
    CH = 12
    rng = np.random.default_rng(10 + K)
    ring = np.zeros((wl.num_slots, wl.cap, CH), np.uint16)
    ptr = bk.RingPointers(rng.integers(0, wl.cap, wl.num_slots), [0] * wl.num_slots, wl.cap)
    orc = co.ConvOracle(ring, wl.cap)
    w = rng.standard_normal((CH, K))
    b = rng.standard_normal(CH)
    committed = {s: [] for s in range(wl.num_slots)}
    for step in range(25):
        slots = synth.make_slot_idx(wl, rng)
        x = synth.f32_to_bf16_bits(rng.standard_normal((wl.num_reqs, wl.draft, CH)).astype(np.float32))
        y = orc.update(np.array(ptr.head), np.array(ptr.len), slots, x, w, b)
        acc = synth.sample_accepted(wl, rng)
        for i, s in enumerate(slots):
            seq = np.array(committed[s] + [go.to_f64(x[i, j]) for j in range(wl.draft)])
            padded = np.concatenate([np.zeros((K - 1, CH)), seq])
            win = sliding_window_view(padded, K, axis=0)          # [T, CH, K]
            full = _silu((win * w[None]).sum(-1) + b)
            np.testing.assert_allclose(y[i], full[-wl.draft:], rtol=1e-13, atol=1e-13)
            committed[s] += [go.to_f64(x[i, j]) for j in range(int(acc[i]))]
        ptr.rollback(slots, wl.draft, acc)
        ptr.flush(slots, wl.flush_min_len)       # slots with len >= 7 only
    assert orc.err == 0 and ptr.err == 0


def test_errors_skip_the_request():
    C, CH, D = 8, 4, 4
    ring = np.zeros((2, C, CH), np.float32)
    orc = co.ConvOracle(ring, C)
    x = np.ones((2, D, CH), np.float32)
    y = orc.update(np.array([0, 9]), np.array([5, 0]), [1, 7], x, np.ones((CH, 4)))
    assert orc.err == go.ERR_POINTER | go.ERR_SLOT
    assert np.isnan(y).all() and not orc.ring.any()


def test_long_committed_window_keeps_the_history():
    """len + D > C is fine for the convolution: the draft overwrites committed
    inputs older than the K - 1 it reads, and the next step still reads the
    right ones (the shift kernel returns the inputs K - 1 tokens back)."""
    K, C, CH, D = 4, 8, 2, 4
    rng = np.random.default_rng(5)
    orc = co.ConvOracle(np.zeros((1, C, CH), np.float32), C)
    w = np.zeros((CH, K)); w[:, 0] = 1
    head, n = np.array([0]), np.array([7])
    stream = rng.standard_normal((7, CH)).astype(np.float32)
    for t in range(7):
        orc.ring[0, t] = stream[t]
    x = rng.standard_normal((1, D, CH)).astype(np.float32)
    y = orc.update(head, n, [0], x, w)
    assert orc.err == 0
    np.testing.assert_allclose(y[0], _silu(np.concatenate([stream[4:], x[0, :1]]).astype(np.float64)),
                               rtol=1e-15)
    # the 7 committed tokens were folded (head 7, len 0) and all D accepted
    # (len 4): the next history is x[1:], at positions 0..2 now
    x2 = rng.standard_normal((1, D, CH)).astype(np.float32)
    y2 = orc.update(np.array([7]), np.array([4]), [0], x2, w)
    assert orc.err == 0
    np.testing.assert_allclose(y2[0], _silu(np.concatenate([x[0, 1:], x2[0, :1]]).astype(np.float64)),
                               rtol=1e-15)


def test_planted_history_mistake_is_caught(monkeypatch):
    """Reading the history one position late (the newest committed input twice)
    fails the schedule pin."""
    orig = co.ConvOracle.update

    def late(self, head, length, slot_idx, x, weight, bias=None):
        return orig(self, np.asarray(head) + 1, length, slot_idx, x, weight, bias)

    monkeypatch.setattr(co.ConvOracle, "update", late)
    with pytest.raises(AssertionError):
        test_schedule_equals_plain_causal_conv(4)
