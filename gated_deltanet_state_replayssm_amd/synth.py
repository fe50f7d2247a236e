"""Seeded synthetic workloads for the GDN replay verify / rollback / flush path.

This module only draws random inputs and fixes their layout. It holds none of
the method's arithmetic, so both the HIP path and the CPU oracle may use it.

Value distributions (every workload):
  q, k   : N(0, 1) per element, L2-normalised over d_k per (token, key head),
           then rounded once to bf16 (round-to-nearest-even) unless the
           workload keeps fp32 inputs.
  v      : N(0, 1), rounded to bf16 the same way.
  alpha  : U[0.9, 1.0], fp32.   beta : U[0, 1), fp32.
  state  : N(0, 0.1^2) per element, fp32.
  ring   : every one of the C positions holds a random record drawn as above;
           positions outside the committed window act as canaries.
  head   : U{0..C-1} so that wrap-around is exercised.

Layouts (row-major, all contiguous):
  state       [num_slots][HV][d_k][d_v]  fp32, element (i, j) = S[j][i]
  ring_q/k    [num_slots][HK][C][d_k]    bf16 bits (uint16) or fp32
  ring_v      [num_slots][HV][C][d_v]    bf16 bits (uint16) or fp32
  ring_alpha/beta [num_slots][HV][C]     fp32
  head, len   [num_slots]                int32
  draft q/k   [num_reqs][D][HK][d_k]
  draft v     [num_reqs][D][HV][d_v]
  draft alpha/beta [num_reqs][D][HV]     fp32

Workloads follow the serving point described in "The inference stack behind
OCRia" (LlamaIndex), section "Making speculative verification cheaper":
32 concurrent requests, 24 GDN layers, block drafts with a mean accepted
length above 12 (section on speculative decoding of the same page).
"""
from __future__ import annotations

import dataclasses

import numpy as np

BF16 = "bf16"
F32 = "f32"


# ---------------------------------------------------------------------------
# bf16 bit handling (input preparation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns uint16 bits.

    Inputs are finite by construction, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_reqs: int
    num_slots: int
    hv: int
    hk: int
    dk: int
    dv: int
    cap: int            # ring capacity C per slot
    draft: int          # draft block D
    in_dtype: str       # BF16 or F32
    flush_min_len: int  # flush folds slots whose committed length >= this
    layers: int
    accept: str         # "fixed:<a>", "uniform", "clipnormal:<mu>:<sd>", "uniform_forced"
    init_len: str       # "fixed:<b>", "uniform:<lo>:<hi>"
    draft_lens: str = "fixed"  # "fixed" (every request drafts `draft`) or "uniform:<lo>:<hi>"

    @property
    def in_bytes(self) -> int:
        return 2 if self.in_dtype == BF16 else 4


WORKLOADS = {
    # one request, one head, d=16, fp32 inputs: 4 committed + 4 draft, accept 2
    "tiny_r1_h1_d16": Workload("tiny_r1_h1_d16", 1, 1, 1, 1, 16, 16, 8, 4, F32,
                               1, 1, "fixed:2", "fixed:4"),
    # 8 requests, 32 value / 16 key heads, d=128, buffer U{0..15}, accept U{0..16}
    "r8_hv32_hk16_d128": Workload("r8_hv32_hk16_d128", 8, 8, 32, 16, 128, 128, 32, 16,
                                  BF16, 1, 1, "uniform", "uniform:0:15"),
    # the pages' profiled point: 32 requests, 24 layers, flush every 16 accepted
    "r32_hv32_hk16_d128_f16": Workload("r32_hv32_hk16_d128_f16", 32, 32, 32, 16, 128, 128,
                                       32, 16, BF16, 16, 24, "clipnormal:12:3", "fixed:0"),
    # flush-heavy: buffer grows to 64 before a flush
    "r32_hv32_hk16_d128_f64": Workload("r32_hv32_hk16_d128_f64", 32, 32, 32, 16, 128, 128,
                                       80, 16, BF16, 64, 24, "clipnormal:12:3", "fixed:0"),
    # stress batch: 128 requests, accept U{0..16} with all-reject / all-accept rows forced
    "r128_hv32_hk16_d128_f16": Workload("r128_hv32_hk16_d128_f16", 128, 128, 32, 16, 128,
                                        128, 32, 16, BF16, 16, 24, "uniform_forced",
                                        "fixed:0"),
    # plain decode (no speculation): one token per request and step, always kept
    "r32_hv32_hk16_d128_d1": Workload("r32_hv32_hk16_d128_d1", 32, 32, 32, 16, 128, 128, 32,
                                      1, BF16, 16, 24, "fixed:1", "fixed:0"),
    # per-request draft lengths U{1..16} (adaptive speculation), accept clipped to each
    "r32_hv32_hk16_d128_varlen": Workload("r32_hv32_hk16_d128_varlen", 32, 32, 32, 16, 128,
                                          128, 32, 16, BF16, 16, 24, "clipnormal:12:3",
                                          "fixed:0", "uniform:1:16"),
}

# index used in the per-workload seed formula
WORKLOAD_INDEX = {name: i for i, name in enumerate(WORKLOADS)}


def seed_for(workload: str, layer: int, step: int) -> int:
    return 1000 * WORKLOAD_INDEX[workload] + 100 * layer + step


def _qk(rng: np.random.Generator, shape, in_dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape).astype(np.float64)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    x = x.astype(np.float32)
    return f32_to_bf16_bits(x) if in_dtype == BF16 else x


def _vv(rng: np.random.Generator, shape, in_dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape).astype(np.float32)
    return f32_to_bf16_bits(x) if in_dtype == BF16 else x


def _alpha(rng, shape):
    return rng.uniform(0.9, 1.0, shape).astype(np.float32)


def _beta(rng, shape):
    return rng.uniform(0.0, 1.0, shape).astype(np.float32)


def sample_init_len(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    kind, *args = wl.init_len.split(":")
    if kind == "fixed":
        return np.full(wl.num_slots, int(args[0]), dtype=np.int32)
    lo, hi = int(args[0]), int(args[1])
    return rng.integers(lo, hi + 1, wl.num_slots).astype(np.int32)


def make_cache_init(wl: Workload, rng: np.random.Generator, init_len=None) -> dict:
    """Initial cache contents: checkpoint, full ring (committed + canaries), pointers."""
    S, HV, HK, C = wl.num_slots, wl.hv, wl.hk, wl.cap
    state = (0.1 * rng.standard_normal((S, HV, wl.dk, wl.dv))).astype(np.float32)
    ring_q = _qk(rng, (S, HK, C, wl.dk), wl.in_dtype)
    ring_k = _qk(rng, (S, HK, C, wl.dk), wl.in_dtype)
    ring_v = _vv(rng, (S, HV, C, wl.dv), wl.in_dtype)
    ring_alpha = _alpha(rng, (S, HV, C))
    ring_beta = _beta(rng, (S, HV, C))
    head = rng.integers(0, C, S).astype(np.int32)
    length = sample_init_len(wl, rng) if init_len is None else np.asarray(init_len, np.int32)
    return dict(state=state, ring_q=ring_q, ring_k=ring_k, ring_v=ring_v,
                ring_alpha=ring_alpha, ring_beta=ring_beta, head=head,
                len=length.astype(np.int32).copy())


def make_draft(wl: Workload, rng: np.random.Generator, num_reqs=None, draft=None) -> dict:
    R = wl.num_reqs if num_reqs is None else num_reqs
    D = wl.draft if draft is None else draft
    return dict(
        q=_qk(rng, (R, D, wl.hk, wl.dk), wl.in_dtype),
        k=_qk(rng, (R, D, wl.hk, wl.dk), wl.in_dtype),
        v=_vv(rng, (R, D, wl.hv, wl.dv), wl.in_dtype),
        alpha=_alpha(rng, (R, D, wl.hv)),
        beta=_beta(rng, (R, D, wl.hv)),
    )


def make_slot_idx(wl: Workload, rng: np.random.Generator, num_reqs=None) -> np.ndarray:
    """A random injection of the requests into the slots (slot indirection)."""
    R = wl.num_reqs if num_reqs is None else num_reqs
    return rng.permutation(wl.num_slots)[:R].astype(np.int32)


def sample_draft_lens(wl: Workload, rng: np.random.Generator, num_reqs=None):
    """Per-request draft lengths, or None when every request drafts wl.draft."""
    R = wl.num_reqs if num_reqs is None else num_reqs
    kind, *args = wl.draft_lens.split(":")
    if kind == "fixed":
        return None
    if kind == "uniform":
        lo, hi = int(args[0]), int(args[1])
        return rng.integers(lo, hi + 1, R).astype(np.int32)
    raise ValueError(wl.draft_lens)


def sample_accepted(wl: Workload, rng: np.random.Generator, num_reqs=None, draft=None,
                    draft_lens=None):
    """Accepted counts a_i in [0, D_i] (D_i = draft_lens[i] when given)."""
    R = wl.num_reqs if num_reqs is None else num_reqs
    D = wl.draft if draft is None else draft
    if draft_lens is not None:
        D = np.asarray(draft_lens, dtype=np.int64)
    kind, *args = wl.accept.split(":")
    if kind == "fixed":
        a = np.minimum(np.full(R, int(args[0])), D)
    elif kind == "uniform":
        a = rng.integers(0, np.asarray(D) + 1, R)
    elif kind == "uniform_forced":
        a = rng.integers(0, np.asarray(D) + 1, R)
        if R >= 2:
            i, j = rng.choice(R, 2, replace=False)
            a[i], a[j] = 0, np.broadcast_to(D, (R,))[j]
    elif kind == "clipnormal":
        mu, sd = float(args[0]), float(args[1])
        a = np.clip(np.rint(rng.normal(mu, sd, R)), 0, D)
    else:
        raise ValueError(wl.accept)
    return np.asarray(a).astype(np.int32)


def canonical(workload: str) -> Workload:
    return WORKLOADS[workload]
