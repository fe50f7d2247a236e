// Token-by-token replay kernels (fp32 VALU), one lane per state column.
//
// Gated delta rule (Yang et al., "Gated Delta Networks", 2025) in rank-1 form,
// on the stored checkpoint H = S^T (d_k rows of d_v floats):
//     y = H^T k,  u = beta (v - alpha y),  H <- alpha H + k u^T,  o = H^T q.
// Lane j of a workgroup owns column j of H (all d_k rows in registers), so
// y and o are per-lane dot products and no cross-lane reduction is needed;
// the loads of a row are 64 consecutive floats per wave.
//
// ReplaySSM bookkeeping ("The inference stack behind OCRia", section "Making
// speculative verification cheaper"): verify replays checkpoint + committed
// ring tokens + draft without writing the state; flush folds the committed
// tokens into the checkpoint and moves the ring pointer.
#include "device_common.h"
#include "internal.h"

namespace gdnr {

namespace {

constexpr int kLanes = 64;

template <int DK, bool F32IN>
__device__ __forceinline__ void stage_vec(float *dst, const void *src, int64_t off) {
#pragma unroll
  for (int i = threadIdx.x; i < DK; i += kLanes) dst[i] = ld_in<F32IN>(src, off + i);
}

// one recurrence step on this lane's column
template <int DK>
__device__ __forceinline__ void step_col(float (&H)[DK], const float *ks, float al, float be,
                                         float vj) {
  float y = 0.f;
#pragma unroll
  for (int i = 0; i < DK; ++i) y = fmaf(H[i], ks[i], y);
  const float u = be * (vj - al * y);
#pragma unroll
  for (int i = 0; i < DK; ++i) H[i] = fmaf(al, H[i], ks[i] * u);
}

template <int DK>
__device__ __forceinline__ float dot_col(const float (&H)[DK], const float *qs) {
  float o = 0.f;
#pragma unroll
  for (int i = 0; i < DK; ++i) o = fmaf(H[i], qs[i], o);
  return o;
}

// grid (num_reqs, HV, ceil(DV/64)), block 64
template <int DK, int DV, bool F32IN>
__global__ __launch_bounds__(kLanes) void verify_recurrent(VerifyArgs a) {
  const CacheView &c = a.c;
  const int r = blockIdx.x, h = blockIdx.y, tile = blockIdx.z;
  const int lane = threadIdx.x;
  const int j = tile * kLanes + lane;
  const bool col = j < DV;
  const bool lead = (h == 0 && tile == 0 && lane == 0);
  const int s = a.slot_idx[r];
  if (s < 0 || s >= c.num_slots) {
    if (lead) raise_err(c.err, GDN_DERR_SLOT);
    return;
  }
  const int C = c.cap, Dmax = a.draft;
  const int head = c.head[s], n = c.len[s];
  if (head < 0 || head >= C || n < 0 || n > C) {
    if (lead) raise_err(c.err, GDN_DERR_POINTER);
    return;
  }
  const int D = request_draft(a.draft_lens, r, Dmax);
  if (D < 0) {
    if (lead) raise_err(c.err, GDN_DERR_DRAFT);
    return;
  }
  if (D == 0) return;  // no draft: nothing to emit or append
  if (n + D > C) {
    if (lead) raise_err(c.err, GDN_DERR_CAPACITY);
    return;
  }
  const int HV = c.hv, HK = c.hk, G = HV / HK, kh = h / G;
  __shared__ float ks[DK], qs[DK];

  float H[DK];
  const float *st = c.state + ((int64_t)s * HV + h) * DK * DV;
#pragma unroll
  for (int i = 0; i < DK; ++i) H[i] = col ? st[(int64_t)i * DV + j] : 0.f;

  const int64_t ring_kq = ((int64_t)s * HK + kh) * C;   // token row base of ring_k/q
  const int64_t ring_vh = ((int64_t)s * HV + h) * C;    // token row base of ring_v/alpha/beta
  for (int t = 0; t < n; ++t) {
    const int pos = (head + t) % C;
    __syncthreads();
    stage_vec<DK, F32IN>(ks, c.ring_k, (ring_kq + pos) * DK);
    __syncthreads();
    const float vj = col ? ld_in<F32IN>(c.ring_v, (ring_vh + pos) * DV + j) : 0.f;
    step_col<DK>(H, ks, c.ring_alpha[ring_vh + pos], c.ring_beta[ring_vh + pos], vj);
  }
  for (int jd = 0; jd < D; ++jd) {
    const int64_t tok = (int64_t)r * Dmax + jd;
    __syncthreads();
    stage_vec<DK, F32IN>(ks, a.k, (tok * HK + kh) * DK);
    stage_vec<DK, F32IN>(qs, a.q, (tok * HK + kh) * DK);
    __syncthreads();
    const float vj = col ? ld_in<F32IN>(a.v, (tok * HV + h) * DV + j) : 0.f;
    step_col<DK>(H, ks, a.alpha[tok * HV + h], a.beta[tok * HV + h], vj);
    const float o = dot_col<DK>(H, qs);
    if (col) a.out[(tok * HV + h) * DV + j] = o;
  }

  // tentative append of the draft behind the committed window
  for (int jd = 0; jd < D; ++jd) {
    const int64_t tok = (int64_t)r * Dmax + jd;
    const int pos = (head + n + jd) % C;
    if (col) copy_in<F32IN>(c.ring_v, (ring_vh + pos) * DV + j, a.v, (tok * HV + h) * DV + j);
    if (tile == 0 && lane == 0) {
      c.ring_alpha[ring_vh + pos] = a.alpha[tok * HV + h];
      c.ring_beta[ring_vh + pos] = a.beta[tok * HV + h];
    }
    if (tile == 0 && h % G == 0) {
      for (int i = lane; i < DK; i += kLanes) {
        copy_in<F32IN>(c.ring_k, (ring_kq + pos) * DK + i, a.k, (tok * HK + kh) * DK + i);
        if (c.ring_q)
          copy_in<F32IN>(c.ring_q, (ring_kq + pos) * DK + i, a.q, (tok * HK + kh) * DK + i);
      }
    }
  }
}

// grid (num_reqs, HV, ceil(DV/64)), block 64
template <int DK, int DV, bool F32IN>
__global__ __launch_bounds__(kLanes) void flush_recurrent(FlushArgs a) {
  const CacheView &c = a.c;
  const int r = blockIdx.x, h = blockIdx.y, tile = blockIdx.z;
  const int lane = threadIdx.x;
  const int j = tile * kLanes + lane;
  const bool col = j < DV;
  const int s = a.slot_idx[r];
  if (s < 0 || s >= c.num_slots) {
    if (h == 0 && tile == 0 && lane == 0) raise_err(c.err, GDN_DERR_SLOT);
    return;
  }
  const int C = c.cap;
  const int head = c.head[s], n = c.len[s];
  if (head < 0 || head >= C || n < 0 || n > C) {
    if (h == 0 && tile == 0 && lane == 0) raise_err(c.err, GDN_DERR_POINTER);
    return;
  }
  if (n < max(a.min_len, 1)) return;  // not due: nothing is written
  // verify_flush run as two calls: a request with a bad draft length is not flushed
  if (a.draft_lens && request_draft(a.draft_lens, r, a.max_draft) < 0) return;
  const int HV = c.hv, HK = c.hk, G = HV / HK, kh = h / G;
  __shared__ float ks[DK];

  float H[DK];
  float *st = c.state + ((int64_t)s * HV + h) * DK * DV;
#pragma unroll
  for (int i = 0; i < DK; ++i) H[i] = col ? st[(int64_t)i * DV + j] : 0.f;
  const int64_t ring_kq = ((int64_t)s * HK + kh) * C;
  const int64_t ring_vh = ((int64_t)s * HV + h) * C;
  for (int t = 0; t < n; ++t) {
    const int pos = (head + t) % C;
    __syncthreads();
    stage_vec<DK, F32IN>(ks, c.ring_k, (ring_kq + pos) * DK);
    __syncthreads();
    const float vj = col ? ld_in<F32IN>(c.ring_v, (ring_vh + pos) * DV + j) : 0.f;
    step_col<DK>(H, ks, c.ring_alpha[ring_vh + pos], c.ring_beta[ring_vh + pos], vj);
  }
  if (col) {
#pragma unroll
    for (int i = 0; i < DK; ++i) st[(int64_t)i * DV + j] = H[i];
  }

  // The last workgroup of this slot to arrive moves the pointers. Every
  // workgroup's head/len loads were consumed (by the branches above) before
  // its arrival, so none can observe the update; no memory fence is needed.
  __syncthreads();
  if (lane == 0) {
    const int total = HV * (int)gridDim.z;
    const int prev = atomicAdd(slot_counter(c, s), 1);
    if (prev == total - 1) {
      c.head[s] = (head + n) % C;
      c.len[s] = 0;
      *slot_counter(c, s) = 0;
    }
  }
}

template <int DK, bool F32IN>
hipError_t launch_verify_t(const VerifyArgs &a, hipStream_t stream) {
  dim3 grid(a.num_reqs, a.c.hv, (DK + kLanes - 1) / kLanes);
  hipLaunchKernelGGL((verify_recurrent<DK, DK, F32IN>), grid, dim3(kLanes), 0, stream, a);
  return hipGetLastError();
}

template <int DK, bool F32IN>
hipError_t launch_flush_t(const FlushArgs &a, hipStream_t stream) {
  dim3 grid(a.num_reqs, a.c.hv, (DK + kLanes - 1) / kLanes);
  hipLaunchKernelGGL((flush_recurrent<DK, DK, F32IN>), grid, dim3(kLanes), 0, stream, a);
  return hipGetLastError();
}

template <bool F32IN>
hipError_t dispatch_verify(const VerifyArgs &a, hipStream_t stream) {
  switch (a.c.dk) {
    case 16: return launch_verify_t<16, F32IN>(a, stream);
    case 32: return launch_verify_t<32, F32IN>(a, stream);
    case 64: return launch_verify_t<64, F32IN>(a, stream);
    case 128: return launch_verify_t<128, F32IN>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <bool F32IN>
hipError_t dispatch_flush(const FlushArgs &a, hipStream_t stream) {
  switch (a.c.dk) {
    case 16: return launch_flush_t<16, F32IN>(a, stream);
    case 32: return launch_flush_t<32, F32IN>(a, stream);
    case 64: return launch_flush_t<64, F32IN>(a, stream);
    case 128: return launch_flush_t<128, F32IN>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_verify_recurrent(const VerifyArgs &a, bool in_f32, hipStream_t stream) {
  return in_f32 ? dispatch_verify<true>(a, stream) : dispatch_verify<false>(a, stream);
}

hipError_t launch_flush_recurrent(const FlushArgs &a, bool in_f32, hipStream_t stream) {
  return in_f32 ? dispatch_flush<true>(a, stream) : dispatch_flush<false>(a, stream);
}

}  // namespace gdnr
