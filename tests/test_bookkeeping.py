"""Ring-pointer bookkeeping: hand-worked walk, integer model vs oracle, window contents."""
import os

import numpy as np

from gated_deltanet_state_replayssm_amd import synth
from oracle import bookkeeping as bk
from oracle import gdn_oracle as go

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pointer_walk.txt")


def _walk():
    ops = []
    start = None
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("start"):
            start = tuple(int(x) for x in line.split()[1:])
            continue
        op, ptr, pos, err = (p.strip() for p in line.split("|"))
        name, *args = op.split()
        ops.append((name, [int(a) for a in args], tuple(int(x) for x in ptr.split()),
                    None if pos == "-" else [int(x) for x in pos.split()], int(err)))
    return start, ops


def test_pointer_walk_on_integer_model():
    (head, length), ops = _walk()
    m = bk.RingPointers([head], [length], 8)
    for name, args, (eh, el), pos, err in ops:
        if name == "verify":
            w = m.verify([0], args[0])
            assert w.get(0) == pos
        elif name == "rollback":
            m.rollback([0], args[0], [args[1]])
        else:
            m.flush([0], args[0])
        assert (m.head[0], m.len[0], m.err) == (eh, el, err), (name, args)


def test_pointer_walk_on_oracle():
    """The same walk through the fp64 oracle: pointers, error word, and exactly the
    listed ring positions rewritten by each verify."""
    (head, length), ops = _walk()
    wl = synth.Workload("walk", 1, 1, 1, 1, 4, 4, 8, 4, synth.F32, 1, 1, "fixed:0", "fixed:0")
    rng = np.random.default_rng(21)
    init = synth.make_cache_init(wl, rng, init_len=[length])
    init["head"][:] = head
    for mode in ("replay", "snapshot"):
        orc = go.ReplayOracle(init, 1, 1, 4, 4, 8, mode=mode)
        for name, args, (eh, el), pos, err in ops:
            if name == "verify":
                before = orc.ring_v.copy()
                dr = synth.make_draft(wl, rng, draft=args[0])
                orc.verify([0], dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
                changed = [p for p in range(8) if not np.array_equal(before[0, :, p], orc.ring_v[0, :, p])]
                assert sorted(changed) == sorted(pos or [])
                if pos:
                    for j, p in enumerate(pos):
                        assert np.array_equal(orc.ring_v[0, :, p], dr["v"][0, j])
            elif name == "rollback":
                orc.rollback([0], args[0], [args[1]])
            else:
                orc.flush([0], args[0])
            assert (int(orc.head[0]), int(orc.len[0]), orc.err) == (eh, el, err), (mode, name, args)


def test_integer_model_matches_oracle_on_random_schedules():
    wl = synth.Workload("t", 4, 6, 2, 1, 4, 4, 12, 5, synth.F32, 6, 1, "uniform", "uniform:0:7")
    rng = np.random.default_rng(22)
    init = synth.make_cache_init(wl, rng)
    orc = go.ReplayOracle(init, 2, 1, 4, 4, wl.cap, mode="replay")
    m = bk.RingPointers(init["head"], init["len"], wl.cap)
    for step in range(60):
        slots = synth.make_slot_idx(wl, rng)
        if step % 7 == 3:                      # plant an out-of-range slot now and then
            slots = slots.copy()
            slots[0] = wl.num_slots + 2
        D = int(rng.integers(1, wl.draft + 1))
        dr = synth.make_draft(wl, rng, draft=D)
        orc.verify(slots, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
        m.verify(slots, D)
        acc = rng.integers(-1, D + 2, len(slots))      # includes invalid counts
        orc.rollback(slots, D, acc)
        m.rollback(slots, D, acc)
        fl = int(rng.integers(0, 9))
        orc.flush(slots, fl)
        m.flush(slots, fl)
        assert list(orc.head) == m.head and list(orc.len) == m.len and orc.err == m.err


def test_committed_window_holds_accepted_tokens_in_order():
    wl = synth.Workload("t", 3, 3, 2, 1, 4, 4, 16, 4, synth.BF16, 9, 1, "uniform", "fixed:0")
    rng = np.random.default_rng(23)
    init = synth.make_cache_init(wl, rng)
    orc = go.ReplayOracle(init, 2, 1, 4, 4, wl.cap, mode="replay")
    hist = {s: [] for s in range(3)}
    for _ in range(25):
        slots = synth.make_slot_idx(wl, rng)
        dr = synth.make_draft(wl, rng)
        acc = synth.sample_accepted(wl, rng)
        orc.verify(slots, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"])
        orc.rollback(slots, wl.draft, acc)
        for i, s in enumerate(slots):
            hist[s] += [dr["k"][i, j] for j in range(acc[i])]
        n_before = orc.len.copy()
        orc.flush(slots, wl.flush_min_len)
        for s in range(3):
            if orc.len[s] == 0 and n_before[s] > 0:
                hist[s] = []
            assert orc.len[s] == len(hist[s])
            for t, rec in enumerate(hist[s]):
                pos = (int(orc.head[s]) + t) % wl.cap
                assert np.array_equal(orc.ring_k[s, :, pos], rec)


def test_verify_flush_is_flush_then_verify_on_the_model():
    """The fused call's pointer rule on the integer model: a due slot is folded
    (head += len, len = 0) and the draft lands right behind the new head; a slot
    that is not due and has len + D > C is rejected without any change."""
    m = bk.RingPointers([3, 5, 0, 7], [6, 2, 7, 1], 8)
    folded, written = m.verify_flush([0, 1, 2, 3], 2, 6)
    assert folded == {0: 6, 2: 7}
    assert m.head == [1, 5, 7, 7] and m.len == [0, 2, 0, 1]
    assert written == {0: [1, 2], 1: [7, 0], 2: [7, 0], 3: [0, 1]}
    assert m.err == 0
    m2 = bk.RingPointers([0], [7], 8)
    folded, written = m2.verify_flush([0], 2, 8)    # not due, 7 + 2 > 8
    assert folded == {} and written == {} and m2.err == 1
    assert m2.head == [0] and m2.len == [7]


def test_integer_model_matches_oracle_with_per_request_draft_lengths():
    """Per-request draft lengths (including 0 and out-of-range values): the
    integer model and the oracle agree on pointers and error bits, through
    both the separate and the fused order."""
    wl = synth.Workload("t", 4, 6, 2, 1, 4, 4, 12, 5, synth.F32, 6, 1, "uniform", "uniform:0:7")
    rng = np.random.default_rng(23)
    init = synth.make_cache_init(wl, rng)
    orc = go.ReplayOracle(init, 2, 1, 4, 4, wl.cap, mode="replay")
    m = bk.RingPointers(init["head"], init["len"], wl.cap)
    for step in range(80):
        slots = synth.make_slot_idx(wl, rng)
        dmax = int(rng.integers(1, wl.draft + 1))
        dl = rng.integers(-1, dmax + 2, len(slots)).astype(np.int32)   # includes invalid
        dr = synth.make_draft(wl, rng, draft=dmax)
        fl = int(rng.integers(0, 9))
        if step % 2:
            orc.verify_flush(slots, fl, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"],
                             draft_lens=dl)
            m.verify_flush(slots, list(dl), fl, dmax)
        else:
            orc.verify(slots, dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"], draft_lens=dl)
            m.verify(slots, list(dl), dmax)
        acc = rng.integers(-1, dmax + 2, len(slots))
        orc.rollback(slots, dmax, acc, draft_lens=dl)
        m.rollback(slots, list(dl), acc, dmax)
        if step % 2 == 0:
            orc.flush(slots, fl)
            m.flush(slots, fl)
        assert list(orc.head) == m.head and list(orc.len) == m.len and orc.err == m.err
    assert orc.err & bk.ERR_DRAFT


def test_per_request_written_positions():
    m = bk.RingPointers([3, 10, 0], [2, 1, 5], 12)
    w = m.verify([0, 1, 2], [4, 3, 0], 4)
    assert w == {0: [5, 6, 7, 8], 1: [11, 0, 1], 2: []} and m.err == 0
    w = m.verify([0, 1], [5, -1], 4)
    assert w == {} and m.err == bk.ERR_DRAFT
