"""The benchmark's algorithmic byte counts (the numerator of its roofline
figure) against a count made unit by unit, request by request, from what each
call reads and writes: the state once per (request, value head) that replays,
the committed ring rows of the replay, the draft read and appended, the outputs
written, and a folded slot's state written once."""
import numpy as np
import pytest

import bench
from gated_deltanet_state_replayssm_amd import synth


def _row_bytes(wl):
    """Bytes of one token: key and query rows per key head, value row, alpha and
    beta (fp32) per value head."""
    ib = wl.in_bytes
    k = wl.hk * wl.dk * ib
    q = wl.hk * wl.dk * ib
    v = wl.hv * wl.dv * ib
    ab = wl.hv * 4 * 2
    return k, q, v, ab


def _count_separate(wl, lens, drafts, folded_lens):
    """verify (every request with a draft replays its n committed tokens and its
    draft from the checkpoint), then flush of the folded slots."""
    k, q, v, ab = _row_bytes(wl)
    state = wl.hv * wl.dk * wl.dv * 4
    total_v = 0
    for n, d in zip(lens, drafts):
        if d == 0:
            continue
        total_v += state                       # checkpoint read
        total_v += n * (k + v + ab)            # committed rows (no query needed)
        total_v += d * (k + q + v + ab)        # draft read
        total_v += d * (k + q + v + ab)        # draft appended to the ring
        total_v += d * wl.hv * wl.dv * 4       # fp32 outputs
    total_f = 0
    for n in folded_lens:
        total_f += 2 * state                   # read and write the checkpoint
        total_f += n * (k + v + ab)            # the folded rows
    return total_v, total_f


def _count_fused(wl, lens, drafts):
    """verify_flush: a due slot folds its n committed rows into the state it
    reads once and writes once, then verifies its draft from it (no committed
    rows left); another slot with a draft replays as verify does."""
    k, q, v, ab = _row_bytes(wl)
    state = wl.hv * wl.dk * wl.dv * 4
    mn = max(wl.flush_min_len, 1)
    total = 0
    for n, d in zip(lens, drafts):
        due = n >= mn
        if not due and d == 0:
            continue
        total += state                         # one read serves fold and verify
        total += n * (k + v + ab)              # committed rows, read once
        if due:
            total += state                     # folded state written once
        total += d * 2 * (k + q + v + ab)      # draft read and appended
        total += d * wl.hv * wl.dv * 4         # outputs
    return total


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F32])
def test_byte_models_match_a_unit_count(seed, dtype):
    rng = np.random.default_rng(4000 + seed)
    wl = synth.Workload("bytes", 9, 12, 8, 4, 64, 32, 48, 6, dtype, 10, 1, "uniform",
                        "uniform:0:40")
    lens = rng.integers(0, 43, wl.num_reqs)
    drafts = rng.integers(0, wl.draft + 1, wl.num_reqs)
    drafts[:2] = 0                             # requests without a draft
    lens[0] = 20                               # ... one of them due (fold only)
    lens[1] = 3                                # ... one not due (nothing to do)
    due = lens >= wl.flush_min_len
    folded = [int(n) for n in lens[due]]

    v_bytes, f_bytes = bench.byte_model(wl, lens, folded, drafts)
    assert (v_bytes, f_bytes) == _count_separate(wl, lens, drafts, folded)

    fused = bench.byte_model_fused(wl, lens, folded, drafts)
    assert fused == _count_fused(wl, lens, drafts)
    # the fused call saves one state read per folded slot with a draft and the
    # second read of its committed rows, and nothing else
    k, q, v, ab = _row_bytes(wl)
    state = wl.hv * wl.dk * wl.dv * 4
    saved = sum(state + int(n) * (k + v + ab) for n, d in zip(lens, drafts)
                if n >= wl.flush_min_len and d > 0)
    assert v_bytes + f_bytes - fused == saved


def test_byte_model_fixed_drafts_default():
    """drafts=None means every request drafts the workload's D."""
    wl = synth.WORKLOADS["r32_hv32_hk16_d128_f16"]
    lens = np.arange(wl.num_reqs) % 20
    folded = [int(n) for n in lens if n >= wl.flush_min_len]
    assert bench.byte_model(wl, lens, folded) == bench.byte_model(
        wl, lens, folded, np.full(wl.num_reqs, wl.draft))
    assert bench.byte_model_fused(wl, lens, folded) == _count_fused(
        wl, lens, np.full(wl.num_reqs, wl.draft))
