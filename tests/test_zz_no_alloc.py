"""gdn_replay_rollback_verify_flush_noalloc (the one-call step for callers that
cannot allocate: its arrival counters live in a library-owned device array)
against gdn_replay_rollback_verify_flush with the caller's counter buffer,
through the C ABI, on twin caches built from the same seeded inputs:

* out, state, ring, head, len and err bit for bit equal after every call, and
  the outputs and flushed states within 2e-3 * max |ref| of the fp64 oracle's
  rollback then verify_flush;
* calls in a row whose counter layouts differ: a cache of 12 slots, then a
  smaller one (4 slots, fewer requests), then the first again, so each call
  relies on the previous one having left the shared counters at zero;
* the caller's counter fields are ignored (NULL and 0 here).
"""
import ctypes

import numpy as np
import pytest
import torch

from gated_deltanet_state_replayssm_amd import binding, synth
from gated_deltanet_state_replayssm_amd.cache import ReplayCache, to_device
from oracle import gdn_oracle as go
from tests.gpu_harness import TOL, rel_err, say

pytestmark = pytest.mark.gpu

FIELDS = ("state", "head", "len", "ring_k", "ring_v", "ring_alpha", "ring_beta", "ring_q", "err")


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def _bits(t):
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t


class Twin:
    def __init__(self, wl, seed):
        self.wl = wl
        self.rng = np.random.default_rng(seed)
        init = synth.make_cache_init(wl, self.rng)
        self.a = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
        self.b = ReplayCache.from_numpy(init, wl.hv, wl.hk, wl.dk, wl.dv, wl.cap, wl.in_dtype)
        self.orc = go.ReplayOracle(dict(init), wl.hv, wl.hk, wl.dk, wl.dv, wl.cap)
        self.pending = {}
        # the no-alloc call's struct: the caller's counter fields left empty
        sa = self.a.struct()
        self.sa = binding.GdnReplayCache(*[getattr(sa, f) for f, _ in sa._fields_])
        self.sa.sync = None
        self.sa.sync_len = 0

    def step(self, label):
        wl, rng = self.wl, self.rng
        slots = synth.make_slot_idx(wl, rng)
        acc = synth.sample_accepted(wl, rng)
        pa = np.array([self.pending.get(int(s), 0) for s in slots], np.int32)
        pl = np.array([wl.draft if int(s) in self.pending else 0 for s in slots], np.int32)
        dr = synth.make_draft(wl, rng)
        dd = {k: to_device(v) for k, v in dr.items()}
        R, D = wl.num_reqs, wl.draft
        out_a = torch.full((R, D, wl.hv, wl.dv), 7.0, dtype=torch.float32, device="cuda")
        out_b = torch.full_like(out_a, 7.0)
        sl, pa_d, pl_d = to_device(slots), to_device(pa), to_device(pl)
        dp = tuple(dd[x].data_ptr() for x in ("q", "k", "v", "alpha", "beta"))
        say(f"  {label}: R={R} slots={wl.num_slots} lens={list(self.orc.len[:8])}")
        st = binding.rollback_verify_flush_noalloc_raw(
            self.sa, R, sl.data_ptr(), pa_d.data_ptr(), pl_d.data_ptr(), D, None, D,
            wl.flush_min_len, *dp, out_a.data_ptr(), None)
        assert st == binding.GDN_OK, st
        st = binding.rollback_verify_flush_raw(
            self.b.struct(), R, sl.data_ptr(), pa_d.data_ptr(), pl_d.data_ptr(), D, None, D,
            wl.flush_min_len, *dp, out_b.data_ptr(), None)
        assert st == binding.GDN_OK, st
        torch.cuda.synchronize()
        assert torch.equal(_bits(out_a), _bits(out_b)), f"{label}: out"
        for name in FIELDS:
            assert torch.equal(_bits(getattr(self.a, name)), _bits(getattr(self.b, name))), \
                f"{label}: {name}"
        assert not self.b.sync.any()
        # the oracle: rollback, then verify_flush
        self.orc.rollback(slots, D, pa, draft_lens=pl)
        due = [int(s) for s in slots if self.orc.len[s] >= wl.flush_min_len]
        ref = self.orc.verify_flush(slots, wl.flush_min_len,
                                    *(dr[x] for x in ("q", "k", "v", "alpha", "beta")))
        e = rel_err(out_a.cpu().numpy(), ref)
        assert e <= TOL, f"{label}: outputs rel err {e:.3e}"
        host = self.a.to_numpy()
        assert np.array_equal(host["len"], self.orc.len.astype(np.int32))
        assert np.array_equal(host["head"], self.orc.head.astype(np.int32))
        assert int(host["err"][0]) == self.orc.err == 0
        if due:
            es = rel_err(host["state"][due], self.orc.state_abi()[due])
            assert es <= TOL, f"{label}: flushed states rel err {es:.3e}"
        self.pending = {int(s): int(acc[i]) for i, s in enumerate(slots)}
        return len(due)


def test_noalloc_step_matches_the_step_with_a_counter_buffer():
    big = synth.Workload("na", 8, 12, 32, 16, 128, 128, 32, 16, synth.BF16, 16, 1,
                         "clipnormal:12:3", "uniform:0:31")
    small = synth.Workload("nb", 3, 4, 8, 4, 64, 64, 32, 8, synth.BF16, 8, 1,
                           "clipnormal:6:2", "uniform:0:23")
    say("case no-alloc step: 12-slot cache, then a 4-slot one, then the first again")
    t1, t2 = Twin(big, 1500), Twin(small, 1501)
    folded = 0
    for i in range(3):
        folded += t1.step(f"big step {i}")
        folded += t2.step(f"small step {i}")
    assert folded > 0


def test_noalloc_step_refuses_caches_past_its_counter_array():
    """Host-side: more slots than the library's counter array covers."""
    c = ReplayCache(8, 4, 2, 64, 64, 32, synth.BF16)
    s = c.struct()
    big = binding.GdnReplayCache(*[getattr(s, f) for f, _ in s._fields_])
    big.num_slots = 1 << 16            # 32 * (2^16 + 1) + 2^17 > 65536 counters
    big.sync, big.sync_len = None, 0
    f = 1 << 20
    st = binding.rollback_verify_flush_noalloc_raw(big, 2, f, f, None, 4, None, 4, 16, f, f, f, f,
                                                   f, f, None)
    assert st == binding.GDN_EUNSUPPORTED
