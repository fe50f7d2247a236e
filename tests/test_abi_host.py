"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and host validation rejects bad arguments synchronously,
before any HIP call (so nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

from gated_deltanet_state_replayssm_amd import binding as b

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gdn_replay.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = b.load()
    declared = _declared_functions()
    assert set(declared) == set(b.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_strerror():
    assert b.version() == 7
    for st in (b.GDN_OK, b.GDN_EINVAL, b.GDN_EUNSUPPORTED, b.GDN_EHIP):
        assert b.load().gdn_replay_strerror(st)
    assert b.load().gdn_replay_strerror(12345) == b"unknown status"


FAKE = 1 << 20  # a non-NULL, 16-byte-aligned address that is never dereferenced


def _cache(**over):
    kw = dict(num_slots=4, num_v_heads=4, num_k_heads=2, d_k=16, d_v=16, ring_cap=8,
              in_dtype=b.GDN_BF16, sync_len=b.sync_entries(4, 2), state=FAKE, ring_q=None, ring_k=FAKE,
              ring_v=FAKE, ring_alpha=FAKE, ring_beta=FAKE, head=FAKE, len=FAKE, sync=FAKE,
              err=FAKE)
    kw.update(over)
    return b.GdnReplayCache(**kw)


def _verify(c, num_reqs=2, draft=4, **ptrs):
    p = dict(slot=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, be=FAKE, out=FAKE)
    p.update(ptrs)
    return b.verify_raw(c, num_reqs, p["slot"], draft, p["q"], p["k"], p["v"], p["a"], p["be"],
                        p["out"], None)


def _verify_flush(c, num_reqs=2, draft=4, min_len=1, **ptrs):
    p = dict(slot=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, be=FAKE, out=FAKE)
    p.update(ptrs)
    return b.verify_flush_raw(c, num_reqs, p["slot"], draft, min_len, p["q"], p["k"], p["v"],
                              p["a"], p["be"], p["out"], None)


def test_null_cache_rejected():
    lib = b.load()
    assert lib.gdn_replay_verify(None, 1, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == b.GDN_EINVAL
    assert lib.gdn_replay_rollback(None, 1, FAKE, 1, FAKE, None) == b.GDN_EINVAL
    assert lib.gdn_replay_flush(None, 1, FAKE, 1, None) == b.GDN_EINVAL
    assert lib.gdn_replay_verify_flush(None, 1, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == b.GDN_EINVAL


@pytest.mark.parametrize("over,status", [
    (dict(num_slots=0), b.GDN_EINVAL),
    (dict(num_v_heads=0), b.GDN_EINVAL),
    (dict(num_k_heads=3), b.GDN_EINVAL),          # 4 % 3 != 0
    (dict(d_k=48, d_v=48), b.GDN_EUNSUPPORTED),
    (dict(d_k=128, d_v=64), b.GDN_EUNSUPPORTED),
    (dict(d_k=256, d_v=256), b.GDN_EUNSUPPORTED),
    (dict(in_dtype=7), b.GDN_EINVAL),
    (dict(ring_cap=0), b.GDN_EINVAL),
    (dict(ring_cap=257), b.GDN_EUNSUPPORTED),
    (dict(state=None), b.GDN_EINVAL),
    (dict(ring_k=None), b.GDN_EINVAL),
    (dict(sync=None), b.GDN_EINVAL),
    (dict(len=None), b.GDN_EINVAL),
    (dict(state=FAKE + 4), b.GDN_EINVAL),          # misaligned
    (dict(ring_v=FAKE + 2), b.GDN_EINVAL),
    (dict(num_v_heads=8192, num_k_heads=8192), b.GDN_EUNSUPPORTED),
    # the counter buffer's declared size: one entry short, none, negative
    (dict(sync_len=b.sync_entries(4, 2) - 1), b.GDN_EINVAL),
    (dict(sync_len=0), b.GDN_EINVAL),
    (dict(sync_len=-1), b.GDN_EINVAL),
    # more counters than an int32 count can describe
    (dict(num_slots=1 << 30, sync_len=(1 << 31) - 1), b.GDN_EUNSUPPORTED),
])
def test_cache_validation(over, status):
    c = _cache(**over)
    assert _verify(c) == status
    assert b.rollback_raw(c, 2, FAKE, 4, FAKE, None) == status
    assert b.flush_raw(c, 2, FAKE, 1, None) == status
    assert _verify_flush(c) == status


def test_call_validation():
    c = _cache()
    assert _verify(c, num_reqs=-1) == b.GDN_EINVAL
    assert _verify(c, num_reqs=5) == b.GDN_EINVAL            # more requests than slots
    assert _verify(c, draft=0) == b.GDN_EINVAL
    assert _verify(c, draft=9) == b.GDN_EINVAL               # D > C
    assert _verify(c, q=None) == b.GDN_EINVAL
    assert _verify(c, out=None) == b.GDN_EINVAL
    assert _verify(c, out=FAKE + 4) == b.GDN_EINVAL
    assert _verify(c, slot=FAKE + 2) == b.GDN_EINVAL
    assert b.rollback_raw(c, 2, FAKE, 0, FAKE, None) == b.GDN_EINVAL
    assert b.rollback_raw(c, 2, FAKE, 4, None, None) == b.GDN_EINVAL
    assert b.flush_raw(c, -3, FAKE, 1, None) == b.GDN_EINVAL
    assert b.flush_raw(c, 2, None, 1, None) == b.GDN_EINVAL
    for kw in (dict(num_reqs=-1), dict(num_reqs=5), dict(draft=0), dict(draft=9),
               dict(k=None), dict(be=None), dict(out=FAKE + 4),
               dict(slot=None)):
        assert _verify_flush(c, **kw) == b.GDN_EINVAL, kw


def _verify_varlen(c, num_reqs=2, dmax=4, lens=FAKE, **ptrs):
    p = dict(slot=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, be=FAKE, out=FAKE)
    p.update(ptrs)
    return b.verify_varlen_raw(c, num_reqs, p["slot"], lens, dmax, p["q"], p["k"], p["v"], p["a"],
                               p["be"], p["out"], None)


def _verify_flush_varlen(c, num_reqs=2, dmax=4, lens=FAKE, min_len=1, **ptrs):
    p = dict(slot=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, be=FAKE, out=FAKE)
    p.update(ptrs)
    return b.verify_flush_varlen_raw(c, num_reqs, p["slot"], lens, dmax, min_len, p["q"], p["k"],
                                     p["v"], p["a"], p["be"], p["out"], None)


def test_varlen_call_validation():
    """Per-request draft lengths: the lengths pointer is required (and 4-byte
    aligned), the maximum obeys the fixed-length call's bounds; the cache
    checks apply unchanged; zero requests launch nothing."""
    c = _cache()
    for fn in (_verify_varlen, _verify_flush_varlen):
        assert fn(c, lens=None) == b.GDN_EINVAL
        assert fn(c, lens=FAKE + 2) == b.GDN_EINVAL
        assert fn(c, dmax=0) == b.GDN_EINVAL
        assert fn(c, dmax=9) == b.GDN_EINVAL              # max_draft > C
        assert fn(c, num_reqs=5) == b.GDN_EINVAL
        assert fn(c, out=None) == b.GDN_EINVAL
        assert fn(_cache(d_k=48, d_v=48)) == b.GDN_EUNSUPPORTED
        assert fn(c, num_reqs=0, lens=None, q=None) == b.GDN_OK
    rb = b.rollback_varlen_raw
    assert rb(c, 2, FAKE, None, 4, FAKE, None) == b.GDN_EINVAL
    assert rb(c, 2, FAKE, FAKE, 0, FAKE, None) == b.GDN_EINVAL
    assert rb(c, 2, FAKE, FAKE, 4, None, None) == b.GDN_EINVAL
    assert rb(_cache(ring_cap=0), 2, FAKE, FAKE, 4, FAKE, None) == b.GDN_EINVAL
    assert rb(c, 0, None, None, 4, None, None) == b.GDN_OK
    lib = b.load()
    assert lib.gdn_replay_verify_varlen(None, 1, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, None) == b.GDN_EINVAL


def _step(c, num_reqs=2, acc=FAKE, plens=None, pdraft=4, lens=None, draft=4, **ptrs):
    p = dict(slot=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, be=FAKE, out=FAKE)
    p.update(ptrs)
    return b.rollback_verify_flush_raw(c, num_reqs, p["slot"], acc, plens, pdraft, lens, draft, 1,
                                       p["q"], p["k"], p["v"], p["a"], p["be"], p["out"], None)


def test_step_call_validation():
    """The one-call step checks what both of its calls check: the accepted
    counts are required, the previous (maximum) length is in 1..C, optional
    length arrays are 4-byte aligned; nothing is launched on a bad argument."""
    c = _cache()
    assert _step(c, acc=None) == b.GDN_EINVAL
    assert _step(c, acc=FAKE + 2) == b.GDN_EINVAL
    assert _step(c, pdraft=0) == b.GDN_EINVAL
    assert _step(c, pdraft=9) == b.GDN_EINVAL             # previous draft > C
    assert _step(c, plens=FAKE + 1) == b.GDN_EINVAL
    assert _step(c, lens=FAKE + 2) == b.GDN_EINVAL
    assert _step(c, draft=0) == b.GDN_EINVAL
    assert _step(c, draft=9) == b.GDN_EINVAL
    assert _step(c, num_reqs=5) == b.GDN_EINVAL
    assert _step(c, k=None) == b.GDN_EINVAL
    assert _step(c, out=FAKE + 4) == b.GDN_EINVAL
    assert _step(_cache(d_k=48, d_v=48)) == b.GDN_EUNSUPPORTED
    assert _step(c, num_reqs=0, acc=None, q=None) == b.GDN_OK
    assert b.load().gdn_replay_rollback_verify_flush(None, 1, FAKE, FAKE, None, 4, None, 4, 1,
                                                     FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                     None) == b.GDN_EINVAL


def _step_norm(c, num_reqs=2, acc=FAKE, pdraft=4, draft=4, out=FAKE, norm="ok", **ptrs):
    p = dict(slot=FAKE, q=FAKE, k=FAKE, v=FAKE, a=FAKE, be=FAKE)
    p.update(ptrs)
    if norm == "ok":
        norm = b.GdnNormFp8(FAKE, FAKE, 1e-6, FAKE, FAKE)
    return b.step_norm_fp8_raw(c, num_reqs, p["slot"], acc, None, pdraft, None, draft, 1, p["q"],
                               p["k"], p["v"], p["a"], p["be"], out, norm, None)


def test_step_norm_call_validation():
    """The one-kernel shapes only (no fallback, no scratch); out may be NULL;
    the norm's arguments are checked as gdn_gated_rmsnorm_fp8 checks them."""
    c = _cache(d_k=64, d_v=64, ring_cap=32)
    assert _step_norm(c, num_reqs=0, acc=None, q=None) == b.GDN_OK
    assert _step_norm(_cache(), num_reqs=0) == b.GDN_EUNSUPPORTED          # d = 16
    assert _step_norm(_cache(d_k=64, d_v=64, ring_cap=40)) == b.GDN_EUNSUPPORTED   # C > 32
    assert _step_norm(_cache(d_k=64, d_v=64, ring_cap=32, in_dtype=b.GDN_F32)) == b.GDN_EUNSUPPORTED
    assert _step_norm(c, norm=None) == b.GDN_EINVAL
    for eps in (0.0, -1.0, float("nan"), 2.0):
        assert _step_norm(c, norm=b.GdnNormFp8(FAKE, FAKE, eps, FAKE, FAKE)) == b.GDN_EINVAL, eps
    for i in range(4):
        ptrs = [FAKE, FAKE, FAKE, FAKE]
        ptrs[i] = None
        assert _step_norm(c, norm=b.GdnNormFp8(ptrs[0], ptrs[1], 1e-6, ptrs[2], ptrs[3])) \
            == b.GDN_EINVAL, i
    assert _step_norm(c, norm=b.GdnNormFp8(FAKE + 2, FAKE, 1e-6, FAKE, FAKE)) == b.GDN_EINVAL
    assert _step_norm(c, norm=b.GdnNormFp8(FAKE, FAKE + 4, 1e-6, FAKE, FAKE)) == b.GDN_EINVAL
    assert _step_norm(c, norm=b.GdnNormFp8(FAKE, FAKE, 1e-6, FAKE + 1, FAKE)) == b.GDN_EINVAL
    assert _step_norm(c, norm=b.GdnNormFp8(FAKE, FAKE, 1e-6, FAKE, FAKE + 2)) == b.GDN_EINVAL
    assert _step_norm(c, acc=None) == b.GDN_EINVAL
    assert _step_norm(c, pdraft=0) == b.GDN_EINVAL
    assert _step_norm(c, draft=33) == b.GDN_EINVAL
    assert _step_norm(c, out=FAKE + 4) == b.GDN_EINVAL
    assert _step_norm(c, k=None) == b.GDN_EINVAL


def test_norm_call_validation():
    """gdn_gated_rmsnorm_fp8: sizes, supported head dims, eps, NULL and
    misaligned pointers are rejected before any launch; zero rows is a no-op."""
    f = b.gated_rmsnorm_fp8_raw
    ok = dict(rows=4, num_heads=2, d_v=128, o=FAKE, z=FAKE, weight=FAKE, eps=1e-6, q=FAKE,
              scale=FAKE, stream=None)

    def call(**over):
        kw = dict(ok)
        kw.update(over)
        return f(**kw)

    assert call(rows=-1) == b.GDN_EINVAL
    assert call(num_heads=0) == b.GDN_EINVAL
    assert call(d_v=48) == b.GDN_EUNSUPPORTED
    assert call(d_v=256) == b.GDN_EUNSUPPORTED
    assert call(eps=-1.0) == b.GDN_EINVAL
    assert call(eps=0.0) == b.GDN_EINVAL
    assert call(eps=float("nan")) == b.GDN_EINVAL
    for name in ("o", "z", "weight", "q", "scale"):
        assert call(**{name: None}) == b.GDN_EINVAL, name
    assert call(o=FAKE + 8) == b.GDN_EINVAL
    assert call(z=FAKE + 2) == b.GDN_EINVAL
    assert call(z=FAKE + 4) == b.GDN_EINVAL
    assert call(weight=FAKE + 8) == b.GDN_EINVAL
    assert call(q=FAKE + 2) == b.GDN_EINVAL
    assert call(rows=1 << 30, num_heads=4096) == b.GDN_EUNSUPPORTED
    assert call(rows=0, o=None, q=None) == b.GDN_OK


def test_conv_call_validation():
    """gdn_causal_conv_update: cache checks, channel count, width, D + K - 1 <= C,
    bf16 inputs only, NULL / misaligned pointers; zero requests is a no-op."""
    f = b.causal_conv_update_raw
    c = _cache(ring_cap=8)
    ok = dict(conv_ring=FAKE, channels=64, width=4, num_reqs=2, slot_idx=FAKE, draft_len=4,
              x=FAKE, weight=FAKE, bias=None, y=FAKE, stream=None)

    def call(cache=c, **over):
        kw = dict(ok)
        kw.update(over)
        return f(cache, **kw)

    assert call(cache=_cache(num_slots=0)) == b.GDN_EINVAL
    assert call(channels=63) == b.GDN_EINVAL
    assert call(channels=0) == b.GDN_EINVAL
    assert call(width=0) == b.GDN_EUNSUPPORTED
    assert call(width=9) == b.GDN_EUNSUPPORTED
    assert call(draft_len=6) == b.GDN_EINVAL            # 6 + 4 - 1 > 8
    assert call(draft_len=0) == b.GDN_EINVAL
    assert call(num_reqs=5) == b.GDN_EINVAL
    assert call(cache=_cache(ring_cap=8, in_dtype=b.GDN_F32)) == b.GDN_EUNSUPPORTED
    for name in ("conv_ring", "slot_idx", "x", "weight", "y"):
        assert call(**{name: None}) == b.GDN_EINVAL, name
    assert call(x=FAKE + 2) == b.GDN_EINVAL
    assert call(bias=FAKE + 2) == b.GDN_EINVAL
    assert call(num_reqs=0, x=None, conv_ring=None) == b.GDN_OK
    # the pending rollback of the one-call step: its previous length in 1..C,
    # aligned counts
    assert call(num_accepted=FAKE, prev_draft=0) == b.GDN_EINVAL
    assert call(num_accepted=FAKE, prev_draft=9) == b.GDN_EINVAL
    assert call(num_accepted=FAKE + 2, prev_draft=4) == b.GDN_EINVAL
    assert call(num_accepted=FAKE, prev_draft=4, prev_draft_lens=FAKE + 1) == b.GDN_EINVAL


def test_grids_past_the_dispatch_limit_are_refused():
    """num_reqs * HV workgroups of 256 threads must fit a dispatch's 32-bit
    work-item count; the norm takes 32 work-items per (row, head) group."""
    c = _cache(num_slots=4096, num_v_heads=4096, num_k_heads=1, d_k=64, d_v=64,
               ring_cap=32, sync_len=b.sync_entries(4096, 1))
    assert _verify(c, num_reqs=2048) == b.GDN_EUNSUPPORTED      # 2048 * 4096 * 256 = 2^31
    assert _verify_flush(c, num_reqs=2048) == b.GDN_EUNSUPPORTED
    assert b.flush_raw(c, 2048, FAKE, 1, None) == b.GDN_EUNSUPPORTED
    assert _verify(c, num_reqs=2047, q=None) == b.GDN_EINVAL    # within the limit: next check
    assert b.gated_rmsnorm_fp8_raw(1 << 23, 8, 128, FAKE, FAKE, FAKE, 1e-6, FAKE, FAKE,
                                   None) == b.GDN_EUNSUPPORTED  # 2^26 groups * 32 = 2^31


def test_zero_requests_is_a_noop_without_launch():
    c = _cache()
    assert _verify(c, num_reqs=0, q=None, k=None) == b.GDN_OK
    assert b.rollback_raw(c, 0, None, 4, None, None) == b.GDN_OK
    assert b.flush_raw(c, 0, None, 1, None) == b.GDN_OK
    assert _verify_flush(c, num_reqs=0, q=None, out=None) == b.GDN_OK


def test_norm_struct_layout_matches_header():
    # two pointers, a float (padded to 8), two pointers
    assert ctypes.sizeof(b.GdnNormFp8) == 40
    assert b.GdnNormFp8.eps.offset == 16 and b.GdnNormFp8.q.offset == 24


def test_struct_layout_matches_header():
    # 8 int32 then 10 pointers
    assert ctypes.sizeof(b.GdnReplayCache) == 8 * 4 + 10 * 8
    assert b.GdnReplayCache.state.offset == 32
    assert b.GdnReplayCache.err.offset == 32 + 9 * 8


def test_noalloc_step_host_checks():
    """The no-alloc one-call step: the caller's counter fields are ignored (NULL
    and 0 accepted), every other check is the one-call step's, and a cache whose
    counters do not fit the library's array is refused; all before any HIP call."""
    f = FAKE
    c = _cache(d_k=64, d_v=64, ring_cap=32, sync=None, sync_len=0)
    call = lambda cache, **kw: b.rollback_verify_flush_noalloc_raw(
        cache, kw.get("n", 2), f, kw.get("acc", f), None, 4, None, kw.get("d", 4), 16, f, f, f, f,
        f, kw.get("out", f), None)
    assert b.load().gdn_replay_rollback_verify_flush_noalloc(
        None, 1, f, f, None, 4, None, 4, 16, f, f, f, f, f, f, None) == b.GDN_EINVAL
    assert call(c, n=0) == b.GDN_OK                       # no request: nothing to do
    assert call(c, acc=None) == b.GDN_EINVAL
    assert call(c, d=0) == b.GDN_EINVAL
    assert call(c, out=f + 4) == b.GDN_EINVAL
    assert call(_cache(d_k=48, d_v=48, sync=None, sync_len=0)) == b.GDN_EUNSUPPORTED
    big = _cache(num_slots=2000, num_v_heads=32, num_k_heads=16, d_k=128, d_v=128, ring_cap=32,
                 sync=None, sync_len=0)
    assert b.sync_entries(2000, 16) > b.NOALLOC_SYNC_ENTRIES
    assert call(big) == b.GDN_EUNSUPPORTED
