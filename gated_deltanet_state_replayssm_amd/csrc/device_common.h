// Device helpers shared by the replay kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn_replay.h"

namespace gdnr {

// q/k/v element loads: bf16 bits (upcast is exact) or fp32.
template <bool F32IN>
__device__ __forceinline__ float ld_in(const void *p, int64_t i) {
  if constexpr (F32IN) {
    return static_cast<const float *>(p)[i];
  } else {
    const uint32_t b = static_cast<const uint16_t *>(p)[i];
    return __uint_as_float(b << 16);
  }
}

// Bit copy of one q/k/v element (ring append keeps the caller's bits).
template <bool F32IN>
__device__ __forceinline__ void copy_in(void *dst, int64_t di, const void *src, int64_t si) {
  if constexpr (F32IN) {
    static_cast<uint32_t *>(dst)[di] = static_cast<const uint32_t *>(src)[si];
  } else {
    static_cast<uint16_t *>(dst)[di] = static_cast<const uint16_t *>(src)[si];
  }
}

// v moved by the DPP control CTRL within the rows enabled by ROW_MASK; lanes
// with no source (and rows not enabled) get identity.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or(float identity, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v),
                                                    CTRL, ROW_MASK, 0xf, false));
}

__device__ __forceinline__ void raise_err(int32_t *err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// Draft length of request r: dmax for every request when lens is null, else the
// request's own length; -1 when that is outside [0, dmax]. Draft rows keep the
// stride dmax either way (request r's rows start at r * dmax).
__device__ __forceinline__ int request_draft(const int32_t *lens, int r, int dmax) {
  if (!lens) return dmax;
  const int d = lens[r];
  return (d < 0 || d > dmax) ? -1 : d;
}

// Committed count of a slot once the accepted prefix of the previous draft is
// committed (a rollback folded into a later call): len + a when the previous
// draft's length `bound` is in [0, prev_draft], a in [0, bound] and
// len + a <= cap; otherwise len, with the rollback's error bit in *bad (as a
// separate rollback call would skip the request and flag it).
__device__ __forceinline__ int rolled_from(int len, int a, int bound, int prev_draft, int cap,
                                          int *bad) {
  *bad = 0;
  if (bound < 0 || bound > prev_draft)
    *bad = GDN_DERR_DRAFT;
  else if (a < 0 || a > bound)
    *bad = GDN_DERR_ACCEPT;
  else if (len + a > cap)
    *bad = GDN_DERR_CAPACITY;
  return *bad ? len : len + a;
}

}  // namespace gdnr
