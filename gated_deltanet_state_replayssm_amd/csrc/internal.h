// Internal launch interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "../../include/gdn_replay.h"

namespace gdnr {

// Everything a kernel needs about one layer's cache, passed by value.
struct CacheView {
  int32_t num_slots, hv, hk, dk, dv, cap;
  float *state;
  void *ring_q, *ring_k, *ring_v;
  float *ring_alpha, *ring_beta;
  int32_t *head, *len, *sync, *err;
};

// Arrival counters in CacheView::sync (int32, zero between calls): [0] the
// grid counter, [kSyncStride * (1 + i)] the counter of slot i (flush) or of the
// i-th request in the fused kernel's order, each on a 128-byte line of its own
// (atomics on one line are served one after another), then the per-(slot, key
// head) counters at [kSyncStride * (1 + num_slots) + s * HK + kh].
constexpr int kSyncStride = 32;

__host__ __device__ inline int64_t sync_entries(int num_slots, int hk) {
  return (int64_t)kSyncStride * (num_slots + 1) + (int64_t)num_slots * hk;
}

__device__ inline int32_t *slot_counter(const CacheView &c, int i) {
  return c.sync + (int64_t)kSyncStride * (1 + i);
}

__device__ inline int32_t *group_counter(const CacheView &c, int s, int kh) {
  return c.sync + (int64_t)kSyncStride * (1 + c.num_slots) + (int64_t)s * c.hk + kh;
}

struct VerifyArgs {
  CacheView c;
  int32_t num_reqs, draft;       // draft: D, or D_max with per-request lengths
  const int32_t *slot_idx;
  const int32_t *draft_lens;     // per-request lengths in [0, draft], or null
  // rollback of the previous draft folded into this call (verify_flush only):
  // accepted counts (null: none), the previous draft's length or per-request
  // lengths (null: prev_draft for every request)
  const int32_t *prev_accepted;
  const int32_t *prev_draft_lens;
  int32_t prev_draft;
  // gated RMSNorm + FP8 of the draft outputs in the same kernel (fused kernel
  // with the rollback only; norm_q null: none). out may then be null.
  const void *norm_z;            // [R][draft][HV][d_v] bf16 gate
  const float *norm_w;           // [d_v]
  float norm_eps;
  uint8_t *norm_q;               // [R][draft][HV][d_v] E4M3 codes
  float *norm_scale;             // [R][draft][HV]
  const void *q, *k, *v;
  const float *alpha, *beta;
  float *out;
};

struct RollbackArgs {
  CacheView c;
  int32_t num_reqs, draft;
  const int32_t *slot_idx;
  const int32_t *draft_lens;     // as in VerifyArgs
  const int32_t *num_accepted;
};

struct FlushArgs {
  CacheView c;
  int32_t num_reqs, min_len;
  const int32_t *slot_idx;
  // verify_flush run as two calls with per-request draft lengths: a request
  // whose length is outside [0, max_draft] is not flushed (null: no check)
  const int32_t *draft_lens;
  int32_t max_draft;
};

// Tokens per chunk of the chunked (MFMA) replay kernels, and the widest causal
// convolution built.
constexpr int kChunkTokens = 32;
constexpr int kMaxConvWidth = 8;

// Launchers return hipSuccess or the launch error. in_f32 selects fp32 inputs.
// Chunked MFMA kernels (bf16 inputs, d_k = d_v in {64, 128}, draft <= 32):
inline bool chunked_supported(int dk, int dv, bool in_f32, int draft) {
  return !in_f32 && dk == dv && (dk == 64 || dk == 128) && draft <= kChunkTokens;
}
hipError_t launch_verify_chunked(const VerifyArgs &a, hipStream_t stream);
hipError_t launch_flush_chunked(const FlushArgs &a, hipStream_t stream);
// Flush fused into verify in one kernel (chunked shapes, ring capacity <= 32).
inline bool fused_supported(int dk, int dv, bool in_f32, int draft, int cap) {
  return chunked_supported(dk, dv, in_f32, draft) && cap <= kChunkTokens;
}
// The same for replays of several chunks (ring capacity above 32).
inline bool fused_long_supported(int dk, int dv, bool in_f32, int draft, int cap) {
  return chunked_supported(dk, dv, in_f32, draft) && cap > kChunkTokens;
}
hipError_t launch_verify_flush_long(const VerifyArgs &a, int min_len, hipStream_t stream);
hipError_t launch_verify_flush_fused(const VerifyArgs &a, int min_len, hipStream_t stream);
// (a.prev_accepted non-null: the previous draft's rollback first, in the same kernel)
// Token-by-token fp32 kernels (every built shape, bf16 or fp32 inputs):
hipError_t launch_verify_recurrent(const VerifyArgs &a, bool in_f32, hipStream_t stream);
hipError_t launch_flush_recurrent(const FlushArgs &a, bool in_f32, hipStream_t stream);
hipError_t launch_rollback(const RollbackArgs &a, hipStream_t stream);

// Gated RMSNorm + FP8 quantisation of groups of d_v values (norm.hip).
struct NormArgs {
  int64_t groups;        // rows * heads
  const float *o;        // [groups][d_v] fp32
  const void *z;         // [groups][d_v] bf16 (gate)
  const float *weight;   // [d_v] fp32
  float eps;
  uint8_t *q;            // [groups][d_v] OCP E4M3 codes
  float *scale;          // [groups] fp32
};
inline bool norm_supported(int dv) { return dv == 16 || dv == 32 || dv == 64 || dv == 128; }
hipError_t launch_gated_rmsnorm_fp8(const NormArgs &a, int dv, hipStream_t stream);

// Causal convolution of a draft block with its input ring (conv.hip); the ring
// shares head / len / capacity with the cache c.
struct ConvArgs {
  CacheView c;
  int32_t num_reqs, draft, channels;
  const int32_t *slot_idx;
  // the previous draft's rollback, not yet applied to len (the one-call step
  // runs after this call): accepted counts (null: none) and the previous
  // drafts' lengths (null: prev_draft for every request)
  const int32_t *prev_accepted;
  const int32_t *prev_draft_lens;
  int32_t prev_draft;
  void *ring;            // [num_slots][C][channels] bf16
  const void *x;         // [num_reqs][draft][channels] bf16
  const float *weight;   // [channels][width]
  const float *bias;     // [channels] or null
  void *y;               // [num_reqs][draft][channels] bf16
};
inline bool conv_width_supported(int k) { return k >= 1 && k <= kMaxConvWidth; }
hipError_t launch_causal_conv_update(const ConvArgs &a, int width, hipStream_t stream);

// gdn_replay_rollback_verify_flush with every host check; with check_only set
// it returns after the checks (GDN_OK when the call would be launched) and
// enqueues nothing.
int rollback_verify_flush_call(const gdn_replay_cache *c, int32_t num_reqs,
                               const int32_t *slot_idx, const int32_t *num_accepted,
                               const int32_t *prev_draft_lens, int32_t prev_draft,
                               const int32_t *draft_lens, int32_t draft_len, int32_t min_len,
                               const void *q, const void *k, const void *v, const float *alpha,
                               const float *beta, float *out, hipStream_t stream, bool check_only);

// head dims with a compiled kernel
inline bool dims_supported(int dk, int dv) {
  return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

}  // namespace gdnr
