"""Runs the HIP path (through the C ABI) and the fp64 oracle side by side on the
same seeded inputs and compares them after every call.

Bars:
  * outputs and flushed states: max |x_gpu - x_ref| <= 2e-3 * max |x_ref| over
    the call's whole tensor (outputs) / the flushed slots' state (states);
  * bit-exact: head, len, error word, sync counters, the whole ring (written
    window and canaries), the state bytes of slots not flushed, and the state
    bytes after verify / rollback (unchanged).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from gated_deltanet_state_replayssm_amd import synth
from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device
from oracle import gdn_oracle as go

TOL = 2e-3
CANARY = 12345.0  # pre-filled output value that a row no call writes keeps


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x_gpu: np.ndarray, x_ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(x_ref))) if x_ref.size else 0.0
    diff = float(np.max(np.abs(x_gpu.astype(np.float64) - x_ref))) if x_ref.size else 0.0
    return diff / scale if scale > 0 else diff


class Pair:
    """GPU cache + oracle for one layer, driven by the same calls."""

    def __init__(self, wl: synth.Workload, init: dict, with_q=True, mode="replay",
                 oracle_slots=None):
        self.wl = wl
        self.gpu = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap,
                                          wl.in_dtype, with_q=with_q)
        oinit = dict(init)
        if not with_q:
            oinit["ring_q"] = None
        self.orc = go.ReplayOracle(oinit, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, mode=mode)
        # which slots the oracle follows (None = all): requests are independent,
        # so a sample of slots can be checked at full batch size
        self.oracle_slots = None if oracle_slots is None else set(int(s) for s in oracle_slots)
        self.worst = {"out": 0.0, "state": 0.0}
        self.flushed_count = 0

    def _sel(self, slot_idx):
        idx = np.arange(len(slot_idx))
        if self.oracle_slots is None:
            return idx
        return np.array([i for i in idx if int(slot_idx[i]) in self.oracle_slots], dtype=np.int64)

    def _check_common(self, host):
        o = self.orc
        slots = list(range(self.wl.num_slots)) if self.oracle_slots is None else sorted(self.oracle_slots)
        assert np.array_equal(host["len"][slots], o.len[slots].astype(np.int32)), (host["len"], o.len)
        assert np.array_equal(host["head"][slots], o.head[slots].astype(np.int32)), (host["head"], o.head)
        if self.oracle_slots is None:
            assert int(host["err"][0]) == o.err, (int(host["err"][0]), o.err)
        assert not host["sync"].any()
        for s in slots:
            assert np.array_equal(host["ring_k"][s], o.ring_k[s]), f"ring_k slot {s}"
            assert np.array_equal(host["ring_v"][s], o.ring_v[s]), f"ring_v slot {s}"
            assert np.array_equal(host["ring_alpha"][s], o.ring_alpha[s]), f"ring_alpha slot {s}"
            assert np.array_equal(host["ring_beta"][s], o.ring_beta[s]), f"ring_beta slot {s}"
            if host["ring_q"] is not None:
                assert np.array_equal(host["ring_q"][s], o.ring_q[s]), f"ring_q slot {s}"

    def _out_buffer(self, dr):
        R, D = dr["alpha"].shape[:2]
        return torch.full((R, D, self.wl.hv, self.wl.dv), CANARY, dtype=torch.float32,
                          device="cuda")

    def _check_out(self, got, ref, what):
        """Rows the oracle wrote (not NaN): within the bar over the call's
        tensor; rows it did not write (skipped requests, rows past a request's
        draft length): still holding the canary."""
        written = ~np.isnan(ref)
        if written.any():
            e = rel_err(got[written], ref[written])
            self.worst["out"] = max(self.worst["out"], e)
            assert e <= TOL, f"{what} outputs: rel err {e:.3e} > {TOL}"
        assert (got[~written] == CANARY).all(), f"{what} wrote rows it should not have"

    def _lens_dev(self, lens):
        return None if lens is None else to_device(np.asarray(lens, np.int32))

    def verify(self, slot_idx, dr, label="", lens=None):
        say(f"  verify {label} R={len(slot_idx)} D={dr['alpha'].shape[1]}"
            + ("" if lens is None else f" lens={list(lens)[:8]}"))
        before = self.gpu.state.clone()
        dev = {k: to_device(v) for k, v in dr.items()}
        out = self.gpu.verify(to_device(slot_idx), dev["q"], dev["k"], dev["v"], dev["alpha"],
                              dev["beta"], out=self._out_buffer(dr), draft_lens=self._lens_dev(lens))
        torch.cuda.synchronize()
        sel = self._sel(slot_idx)
        ref = self.orc.verify(slot_idx[sel], *(dr[x][sel] for x in ("q", "k", "v", "alpha", "beta")),
                              draft_lens=None if lens is None else np.asarray(lens)[sel])
        self._check_out(out.cpu().numpy()[sel], ref, "verify")
        assert torch.equal(before, self.gpu.state), "verify modified the state"
        host = self.gpu.to_numpy()
        self._check_common(host)
        return out

    def _check_flushed(self, host, before, slot_idx, sel, min_len, len_before):
        ref_state = self.orc.state_abi()
        flushed = [int(slot_idx[i]) for i in sel
                   if 0 <= slot_idx[i] < self.wl.num_slots and
                   len_before[slot_idx[i]] >= max(min_len, 1) and self.orc.len[slot_idx[i]] == 0]
        if flushed:
            e = rel_err(host["state"][flushed], ref_state[flushed])
            self.worst["state"] = max(self.worst["state"], e)
            assert e <= TOL, f"flushed states: rel err {e:.3e} > {TOL}"
            self.flushed_count += len(flushed)
        others = [s for s in range(self.wl.num_slots) if s not in set(flushed)
                  and (self.oracle_slots is None or s in self.oracle_slots)]
        assert np.array_equal(host["state"][others].view(np.uint32),
                              before[others].view(np.uint32)), "unflushed slot state changed"

    def verify_flush(self, slot_idx, min_len, dr, label="", lens=None):
        say(f"  verify_flush {label} R={len(slot_idx)} D={dr['alpha'].shape[1]} min_len={min_len}"
            + ("" if lens is None else f" lens={list(lens)[:8]}"))
        before = self.gpu.state.cpu().numpy()
        len_before = self.orc.len.copy()
        dev = {k: to_device(v) for k, v in dr.items()}
        out = self.gpu.verify_flush(to_device(slot_idx), min_len, dev["q"], dev["k"], dev["v"],
                                    dev["alpha"], dev["beta"], out=self._out_buffer(dr),
                                    draft_lens=self._lens_dev(lens))
        torch.cuda.synchronize()
        sel = self._sel(slot_idx)
        ref = self.orc.verify_flush(slot_idx[sel], min_len,
                                    *(dr[x][sel] for x in ("q", "k", "v", "alpha", "beta")),
                                    draft_lens=None if lens is None else np.asarray(lens)[sel])
        self._check_out(out.cpu().numpy()[sel], ref, "verify_flush")
        host = self.gpu.to_numpy()
        self._check_common(host)
        self._check_flushed(host, before, slot_idx, sel, min_len, len_before)
        return out

    def rollback_verify_flush(self, slot_idx, acc, prev_draft, min_len, dr, label="",
                              prev_lens=None, lens=None):
        """The one-call step; the oracle side is its rollback, then its
        verify_flush, on the same requests."""
        say(f"  rollback_verify_flush {label} R={len(slot_idx)} D={dr['alpha'].shape[1]} "
            f"prev={prev_draft} min_len={min_len} acc={list(acc)[:8]}"
            + ("" if lens is None else f" lens={list(lens)[:8]}")
            + ("" if prev_lens is None else f" prev_lens={list(prev_lens)[:8]}"))
        before = self.gpu.state.cpu().numpy()
        dev = {k: to_device(v) for k, v in dr.items()}
        out = self.gpu.rollback_verify_flush(
            to_device(slot_idx), to_device(np.asarray(acc, np.int32)), prev_draft, min_len,
            dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], out=self._out_buffer(dr),
            prev_draft_lens=self._lens_dev(prev_lens), draft_lens=self._lens_dev(lens))
        torch.cuda.synchronize()
        sel = self._sel(slot_idx)
        self.orc.rollback(slot_idx[sel], prev_draft, np.asarray(acc)[sel],
                          draft_lens=None if prev_lens is None else np.asarray(prev_lens)[sel])
        len_before = self.orc.len.copy()
        ref = self.orc.verify_flush(slot_idx[sel], min_len,
                                    *(dr[x][sel] for x in ("q", "k", "v", "alpha", "beta")),
                                    draft_lens=None if lens is None else np.asarray(lens)[sel])
        self._check_out(out.cpu().numpy()[sel], ref, "rollback_verify_flush")
        host = self.gpu.to_numpy()
        self._check_common(host)
        self._check_flushed(host, before, slot_idx, sel, min_len, len_before)
        return out

    def rollback(self, slot_idx, draft_len, acc, label="", lens=None):
        say(f"  rollback {label}")
        before = self.gpu.state.clone()
        self.gpu.rollback(to_device(slot_idx), draft_len, to_device(acc),
                          draft_lens=self._lens_dev(lens))
        torch.cuda.synchronize()
        sel = self._sel(slot_idx)
        self.orc.rollback(slot_idx[sel], draft_len, acc[sel],
                          draft_lens=None if lens is None else np.asarray(lens)[sel])
        assert torch.equal(before, self.gpu.state), "rollback modified the state"
        self._check_common(self.gpu.to_numpy())

    def flush(self, slot_idx, min_len, label=""):
        say(f"  flush {label} min_len={min_len}")
        before = self.gpu.state.cpu().numpy()
        len_before = self.orc.len.copy()
        self.gpu.flush(to_device(slot_idx), min_len)
        torch.cuda.synchronize()
        sel = self._sel(slot_idx)
        self.orc.flush(slot_idx[sel], min_len)
        host = self.gpu.to_numpy()
        self._check_common(host)
        self._check_flushed(host, before, slot_idx, sel, min_len, len_before)


def run_schedule(wl: synth.Workload, steps: int, seed: int, layers: int = 1, with_q=True,
                 oracle_slots=None, label="", fused=False, one_call=False):
    """verify -> rollback -> flush for `steps` steps over `layers` independent caches
    (fused: verify_flush -> rollback, the flush folded into the next verify;
    one_call: rollback_verify_flush, the previous step's rollback folded in too).

    With one_call a request carries the accepted count of the draft it appended
    in the previous step; a slot that had a draft and is not in this step's
    batch gets a rollback call of its own first, a slot new to the batch
    passes 0."""
    rng = np.random.default_rng(seed)
    pairs = []
    for L in range(layers):
        init = synth.make_cache_init(wl, rng)
        pairs.append(Pair(wl, init, with_q=with_q, oracle_slots=oracle_slots))
    pending = {}   # slot -> (accepted, that draft's length), one_call only
    for step in range(steps):
        slots = synth.make_slot_idx(wl, rng)
        lens = synth.sample_draft_lens(wl, rng)   # None: every request drafts wl.draft
        acc = synth.sample_accepted(wl, rng, draft_lens=lens)
        if one_call:
            gone = np.array([s for s in pending if s not in set(int(x) for x in slots)], np.int32)
            if len(gone):
                ga = np.array([pending[int(s)][0] for s in gone], np.int32)
                gl = np.array([pending[int(s)][1] for s in gone], np.int32)
                for L, p in enumerate(pairs):
                    p.rollback(gone, wl.draft, ga, f"{label} L{L} step{step} gone", lens=gl)
            pa = np.array([pending.get(int(s), (0, 0))[0] for s in slots], np.int32)
            pl = np.array([pending.get(int(s), (0, 0))[1] for s in slots], np.int32)
            # fixed previous length when every request had one (and this is not the first step)
            prev_lens = None if (lens is None and step > 0 and
                                 all(int(s) in pending for s in slots)) else pl
        for L, p in enumerate(pairs):
            dr = synth.make_draft(wl, rng)
            tag = f"{label} L{L} step{step}"
            if one_call:
                p.rollback_verify_flush(slots, pa, wl.draft, wl.flush_min_len, dr, tag,
                                        prev_lens=prev_lens, lens=lens)
            elif fused:
                p.verify_flush(slots, wl.flush_min_len, dr, tag, lens=lens)
            else:
                p.verify(slots, dr, tag, lens=lens)
        if one_call:
            pending = {int(s): (int(acc[i]), wl.draft if lens is None else int(lens[i]))
                       for i, s in enumerate(slots)}
            continue
        for L, p in enumerate(pairs):
            p.rollback(slots, wl.draft, acc, f"{label} L{L} step{step}", lens=lens)
        if not fused:
            for L, p in enumerate(pairs):
                p.flush(slots, wl.flush_min_len, f"{label} L{L} step{step}")
    return pairs
