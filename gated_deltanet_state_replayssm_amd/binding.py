"""Thin ctypes binding of libgdnreplay.so (include/gdn_replay.h).

Argument marshalling only: every step of verify / rollback / flush runs in the
HIP kernels behind the C ABI. PyTorch provides device memory and the stream.
If the library is missing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdnreplay.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EHIP = 0, -1, -2, -3
GDN_BF16, GDN_F32 = 0, 1
GDN_DERR_CAPACITY, GDN_DERR_ACCEPT, GDN_DERR_SLOT, GDN_DERR_POINTER = 1, 2, 4, 8
GDN_DERR_DRAFT = 16

EXPORTED = ("gdn_replay_verify", "gdn_replay_rollback", "gdn_replay_flush",
            "gdn_replay_verify_flush", "gdn_replay_verify_varlen",
            "gdn_replay_verify_flush_varlen", "gdn_replay_rollback_varlen",
            "gdn_replay_rollback_verify_flush", "gdn_replay_rollback_verify_flush_noalloc",
            "gdn_replay_sync_entries",
            "gdn_replay_step_norm_fp8",
            "gdn_gated_rmsnorm_fp8", "gdn_causal_conv_update", "gdn_replay_strerror",
            "gdn_replay_version")


class GdnNormFp8(ctypes.Structure):
    """Mirror of gdn_norm_fp8."""
    _fields_ = [("z", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("q", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class GdnReplayCache(ctypes.Structure):
    """Mirror of gdn_replay_cache."""
    _fields_ = [
        ("num_slots", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("num_k_heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("ring_cap", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("sync_len", ctypes.c_int32),
        ("state", ctypes.c_void_p),
        ("ring_q", ctypes.c_void_p),
        ("ring_k", ctypes.c_void_p),
        ("ring_v", ctypes.c_void_p),
        ("ring_alpha", ctypes.c_void_p),
        ("ring_beta", ctypes.c_void_p),
        ("head", ctypes.c_void_p),
        ("len", ctypes.c_void_p),
        ("sync", ctypes.c_void_p),
        ("err", ctypes.c_void_p),
    ]


_lib = None


def load(path: str = None):
    """Load the library (once) and declare the signatures. Raises if absent.
    The in-tree build is used unless GDN_REPLAY_LIB names another build."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("GDN_REPLAY_LIB", LIB_PATH)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run gated_deltanet_state_replayssm_amd.build")
    # PyTorch ships its own HIP runtime. Load it first when it is installed, so
    # that the library binds to the same runtime as the tensors it is handed
    # (two runtimes in one process do not share devices).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I32, VP = ctypes.POINTER(GdnReplayCache), ctypes.c_int32, ctypes.c_void_p
    lib.gdn_replay_verify.argtypes = [P, I32, VP, I32, VP, VP, VP, VP, VP, VP, VP]
    lib.gdn_replay_verify.restype = ctypes.c_int
    lib.gdn_replay_rollback.argtypes = [P, I32, VP, I32, VP, VP]
    lib.gdn_replay_rollback.restype = ctypes.c_int
    lib.gdn_replay_flush.argtypes = [P, I32, VP, I32, VP]
    lib.gdn_replay_flush.restype = ctypes.c_int
    lib.gdn_replay_verify_flush.argtypes = [P, I32, VP, I32, I32, VP, VP, VP, VP, VP, VP, VP]
    lib.gdn_replay_verify_flush.restype = ctypes.c_int
    lib.gdn_replay_verify_varlen.argtypes = [P, I32, VP, VP, I32, VP, VP, VP, VP, VP, VP, VP]
    lib.gdn_replay_verify_varlen.restype = ctypes.c_int
    lib.gdn_replay_verify_flush_varlen.argtypes = [P, I32, VP, VP, I32, I32, VP, VP, VP, VP, VP,
                                                   VP, VP]
    lib.gdn_replay_verify_flush_varlen.restype = ctypes.c_int
    lib.gdn_replay_rollback_varlen.argtypes = [P, I32, VP, VP, I32, VP, VP]
    lib.gdn_replay_rollback_varlen.restype = ctypes.c_int
    lib.gdn_replay_rollback_verify_flush.argtypes = [P, I32, VP, VP, VP, I32, VP, I32, I32, VP,
                                                     VP, VP, VP, VP, VP, VP]
    lib.gdn_replay_rollback_verify_flush.restype = ctypes.c_int
    lib.gdn_replay_rollback_verify_flush_noalloc.argtypes = \
        lib.gdn_replay_rollback_verify_flush.argtypes
    lib.gdn_replay_rollback_verify_flush_noalloc.restype = ctypes.c_int
    lib.gdn_replay_step_norm_fp8.argtypes = [P, I32, VP, VP, VP, I32, VP, I32, I32, VP, VP, VP,
                                             VP, VP, VP, ctypes.POINTER(GdnNormFp8), VP]
    lib.gdn_replay_step_norm_fp8.restype = ctypes.c_int
    lib.gdn_replay_sync_entries.argtypes = [I32, I32]
    lib.gdn_replay_sync_entries.restype = ctypes.c_int64
    lib.gdn_gated_rmsnorm_fp8.argtypes = [I32, I32, I32, VP, VP, VP, ctypes.c_float, VP, VP, VP]
    lib.gdn_gated_rmsnorm_fp8.restype = ctypes.c_int
    lib.gdn_causal_conv_update.argtypes = [P, VP, I32, I32, I32, VP, VP, VP, I32, I32, VP, VP,
                                           VP, VP, VP]
    lib.gdn_causal_conv_update.restype = ctypes.c_int
    lib.gdn_replay_strerror.argtypes = [ctypes.c_int]
    lib.gdn_replay_strerror.restype = ctypes.c_char_p
    lib.gdn_replay_version.argtypes = []
    lib.gdn_replay_version.restype = ctypes.c_int
    _lib = lib
    return lib


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().gdn_replay_strerror(status).decode()
        super().__init__(f"{fn} returned {status}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != GDN_OK:
        raise GdnError(fn, status)


def verify_raw(cache: GdnReplayCache, num_reqs, slot_idx, draft_len, q, k, v, alpha, beta,
               out, stream) -> int:
    return load().gdn_replay_verify(ctypes.byref(cache), num_reqs, slot_idx, draft_len, q, k, v,
                                    alpha, beta, out, stream)


def rollback_raw(cache: GdnReplayCache, num_reqs, slot_idx, draft_len, num_accepted,
                 stream) -> int:
    return load().gdn_replay_rollback(ctypes.byref(cache), num_reqs, slot_idx, draft_len,
                                      num_accepted, stream)


def flush_raw(cache: GdnReplayCache, num_reqs, slot_idx, min_len, stream) -> int:
    return load().gdn_replay_flush(ctypes.byref(cache), num_reqs, slot_idx, min_len, stream)


def verify_flush_raw(cache: GdnReplayCache, num_reqs, slot_idx, draft_len, min_len, q, k, v,
                     alpha, beta, out, stream) -> int:
    return load().gdn_replay_verify_flush(ctypes.byref(cache), num_reqs, slot_idx, draft_len,
                                          min_len, q, k, v, alpha, beta, out, stream)


def verify_varlen_raw(cache: GdnReplayCache, num_reqs, slot_idx, draft_lens, max_draft, q, k, v,
                      alpha, beta, out, stream) -> int:
    return load().gdn_replay_verify_varlen(ctypes.byref(cache), num_reqs, slot_idx, draft_lens,
                                           max_draft, q, k, v, alpha, beta, out, stream)


def verify_flush_varlen_raw(cache: GdnReplayCache, num_reqs, slot_idx, draft_lens, max_draft,
                            min_len, q, k, v, alpha, beta, out, stream) -> int:
    return load().gdn_replay_verify_flush_varlen(ctypes.byref(cache), num_reqs, slot_idx,
                                                 draft_lens, max_draft, min_len, q, k, v, alpha,
                                                 beta, out, stream)


def rollback_varlen_raw(cache: GdnReplayCache, num_reqs, slot_idx, draft_lens, max_draft,
                        num_accepted, stream) -> int:
    return load().gdn_replay_rollback_varlen(ctypes.byref(cache), num_reqs, slot_idx, draft_lens,
                                             max_draft, num_accepted, stream)


def rollback_verify_flush_raw(cache: GdnReplayCache, num_reqs, slot_idx, num_accepted,
                              prev_draft_lens, prev_draft, draft_lens, draft_len, min_len, q, k,
                              v, alpha, beta, out, stream) -> int:
    return load().gdn_replay_rollback_verify_flush(ctypes.byref(cache), num_reqs, slot_idx,
                                                   num_accepted, prev_draft_lens, prev_draft,
                                                   draft_lens, draft_len, min_len, q, k, v, alpha,
                                                   beta, out, stream)


def rollback_verify_flush_noalloc_raw(cache: GdnReplayCache, num_reqs, slot_idx, num_accepted,
                                      prev_draft_lens, prev_draft, draft_lens, draft_len, min_len,
                                      q, k, v, alpha, beta, out, stream) -> int:
    return load().gdn_replay_rollback_verify_flush_noalloc(
        ctypes.byref(cache), num_reqs, slot_idx, num_accepted, prev_draft_lens, prev_draft,
        draft_lens, draft_len, min_len, q, k, v, alpha, beta, out, stream)


NOALLOC_SYNC_ENTRIES = 65536   # GDN_REPLAY_NOALLOC_SYNC_ENTRIES


def step_norm_fp8_raw(cache: GdnReplayCache, num_reqs, slot_idx, num_accepted, prev_draft_lens,
                      prev_draft, draft_lens, draft_len, min_len, q, k, v, alpha, beta, out,
                      norm: GdnNormFp8 | None, stream) -> int:
    return load().gdn_replay_step_norm_fp8(ctypes.byref(cache), num_reqs, slot_idx, num_accepted,
                                           prev_draft_lens, prev_draft, draft_lens, draft_len,
                                           min_len, q, k, v, alpha, beta, out,
                                           None if norm is None else ctypes.byref(norm), stream)


def verify(cache, num_reqs, slot_idx, draft_len, q, k, v, alpha, beta, out, stream) -> None:
    _check("gdn_replay_verify",
           verify_raw(cache, num_reqs, slot_idx, draft_len, q, k, v, alpha, beta, out, stream))


def rollback(cache, num_reqs, slot_idx, draft_len, num_accepted, stream) -> None:
    _check("gdn_replay_rollback",
           rollback_raw(cache, num_reqs, slot_idx, draft_len, num_accepted, stream))


def flush(cache, num_reqs, slot_idx, min_len, stream) -> None:
    _check("gdn_replay_flush", flush_raw(cache, num_reqs, slot_idx, min_len, stream))


def verify_flush(cache, num_reqs, slot_idx, draft_len, min_len, q, k, v, alpha, beta, out,
                 stream) -> None:
    _check("gdn_replay_verify_flush",
           verify_flush_raw(cache, num_reqs, slot_idx, draft_len, min_len, q, k, v, alpha, beta,
                            out, stream))


def verify_varlen(cache, num_reqs, slot_idx, draft_lens, max_draft, q, k, v, alpha, beta, out,
                  stream) -> None:
    _check("gdn_replay_verify_varlen",
           verify_varlen_raw(cache, num_reqs, slot_idx, draft_lens, max_draft, q, k, v, alpha,
                             beta, out, stream))


def verify_flush_varlen(cache, num_reqs, slot_idx, draft_lens, max_draft, min_len, q, k, v, alpha,
                        beta, out, stream) -> None:
    _check("gdn_replay_verify_flush_varlen",
           verify_flush_varlen_raw(cache, num_reqs, slot_idx, draft_lens, max_draft, min_len, q, k,
                                   v, alpha, beta, out, stream))


def rollback_varlen(cache, num_reqs, slot_idx, draft_lens, max_draft, num_accepted,
                    stream) -> None:
    _check("gdn_replay_rollback_varlen",
           rollback_varlen_raw(cache, num_reqs, slot_idx, draft_lens, max_draft, num_accepted,
                               stream))


def rollback_verify_flush(cache, num_reqs, slot_idx, num_accepted, prev_draft_lens, prev_draft,
                          draft_lens, draft_len, min_len, q, k, v, alpha, beta, out,
                          stream) -> None:
    _check("gdn_replay_rollback_verify_flush",
           rollback_verify_flush_raw(cache, num_reqs, slot_idx, num_accepted, prev_draft_lens,
                                     prev_draft, draft_lens, draft_len, min_len, q, k, v, alpha,
                                     beta, out, stream))


def step_norm_fp8(cache, num_reqs, slot_idx, num_accepted, prev_draft_lens, prev_draft,
                  draft_lens, draft_len, min_len, q, k, v, alpha, beta, out, norm,
                  stream) -> None:
    _check("gdn_replay_step_norm_fp8",
           step_norm_fp8_raw(cache, num_reqs, slot_idx, num_accepted, prev_draft_lens, prev_draft,
                             draft_lens, draft_len, min_len, q, k, v, alpha, beta, out, norm,
                             stream))


def gated_rmsnorm_fp8_raw(rows, num_heads, d_v, o, z, weight, eps, q, scale, stream) -> int:
    return load().gdn_gated_rmsnorm_fp8(rows, num_heads, d_v, o, z, weight, eps, q, scale, stream)


def gated_rmsnorm_fp8(rows, num_heads, d_v, o, z, weight, eps, q, scale, stream) -> None:
    _check("gdn_gated_rmsnorm_fp8",
           gated_rmsnorm_fp8_raw(rows, num_heads, d_v, o, z, weight, eps, q, scale, stream))


def causal_conv_update_raw(cache: GdnReplayCache, conv_ring, channels, width, num_reqs, slot_idx,
                           draft_len, x, weight, bias, y, stream, num_accepted=None,
                           prev_draft_lens=None, prev_draft=0) -> int:
    return load().gdn_causal_conv_update(ctypes.byref(cache), conv_ring, channels, width, num_reqs,
                                         slot_idx, num_accepted, prev_draft_lens, prev_draft,
                                         draft_len, x, weight, bias, y, stream)


def causal_conv_update(cache, conv_ring, channels, width, num_reqs, slot_idx, draft_len, x, weight,
                       bias, y, stream, num_accepted=None, prev_draft_lens=None,
                       prev_draft=0) -> None:
    _check("gdn_causal_conv_update",
           causal_conv_update_raw(cache, conv_ring, channels, width, num_reqs, slot_idx, draft_len,
                                  x, weight, bias, y, stream, num_accepted, prev_draft_lens,
                                  prev_draft))


def sync_entries(num_slots: int, num_k_heads: int) -> int:
    """Entries of the cache's int32 arrival-counter buffer."""
    return int(load().gdn_replay_sync_entries(num_slots, num_k_heads))


def version() -> int:
    return load().gdn_replay_version()
