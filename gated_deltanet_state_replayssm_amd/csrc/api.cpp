// C-ABI entry points of libgdnreplay.so: synchronous host validation, then
// asynchronous launches on the caller's stream. No allocation, no host/device sync.
#include <stdint.h>

#include <climits>

#include "internal.h"

namespace {

using gdnr::CacheView;

constexpr int32_t kMaxRingCap = 256;
constexpr int32_t kMaxHeads = 4096;  // grid.y limit headroom
// A dispatch counts the work-items of each grid dimension in 32 bits: the
// replay kernels launch num_reqs * HV workgroups of (at most) 256 threads.
constexpr int64_t kMaxWorkItems = INT32_MAX;

bool replay_grid_ok(int64_t num_reqs, const gdn_replay_cache *c) {
  return num_reqs * c->num_v_heads * 256 <= kMaxWorkItems;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by all three calls.
int check_cache(const gdn_replay_cache *c) {
  if (!c) return GDN_EINVAL;
  if (c->num_slots < 1 || c->num_v_heads < 1 || c->num_k_heads < 1 || c->d_k < 1 ||
      c->d_v < 1 || c->ring_cap < 1)
    return GDN_EINVAL;
  if (c->num_v_heads % c->num_k_heads != 0) return GDN_EINVAL;
  if (c->num_v_heads > kMaxHeads) return GDN_EUNSUPPORTED;
  if (c->in_dtype != GDN_BF16 && c->in_dtype != GDN_F32) return GDN_EINVAL;
  if (!gdnr::dims_supported(c->d_k, c->d_v)) return GDN_EUNSUPPORTED;
  if (c->ring_cap > kMaxRingCap) return GDN_EUNSUPPORTED;
  if (!c->state || !c->ring_k || !c->ring_v || !c->ring_alpha || !c->ring_beta || !c->head ||
      !c->len || !c->sync)
    return GDN_EINVAL;
  // the counter buffer must hold every counter a launch may touch
  const int64_t need = gdnr::sync_entries(c->num_slots, c->num_k_heads);
  if (need > INT32_MAX) return GDN_EUNSUPPORTED;
  if (c->sync_len < need) return GDN_EINVAL;
  if (!aligned(c->state, 16) || !aligned(c->ring_k, 16) || !aligned(c->ring_v, 16) ||
      (c->ring_q && !aligned(c->ring_q, 16)) || !aligned(c->ring_alpha, 4) ||
      !aligned(c->ring_beta, 4) || !aligned(c->head, 4) || !aligned(c->len, 4) ||
      !aligned(c->sync, 4) || (c->err && !aligned(c->err, 4)))
    return GDN_EINVAL;
  return GDN_OK;
}

CacheView view_of(const gdn_replay_cache *c) {
  CacheView v;
  v.num_slots = c->num_slots;
  v.hv = c->num_v_heads;
  v.hk = c->num_k_heads;
  v.dk = c->d_k;
  v.dv = c->d_v;
  v.cap = c->ring_cap;
  v.state = c->state;
  v.ring_q = c->ring_q;
  v.ring_k = c->ring_k;
  v.ring_v = c->ring_v;
  v.ring_alpha = c->ring_alpha;
  v.ring_beta = c->ring_beta;
  v.head = c->head;
  v.len = c->len;
  v.sync = c->sync;
  v.err = c->err;
  return v;
}

// Validation and argument packing shared by verify and verify_flush (varlen:
// draft_lens non-null, draft_len is the maximum).
int verify_args(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                int32_t draft_len, const void *q, const void *k, const void *v, const float *alpha,
                const float *beta, float *out, gdnr::VerifyArgs *a, bool varlen = false,
                const int32_t *draft_lens = nullptr, bool out_optional = false) {
  int st = check_cache(c);
  if (st != GDN_OK) return st;
  if (num_reqs < 0 || num_reqs > c->num_slots) return GDN_EINVAL;
  if (draft_len < 1 || draft_len > c->ring_cap) return GDN_EINVAL;
  if (!replay_grid_ok(num_reqs, c)) return GDN_EUNSUPPORTED;
  if (num_reqs == 0) return GDN_OK;
  if (!slot_idx || !q || !k || !v || !alpha || !beta || (!out && !out_optional))
    return GDN_EINVAL;
  if (varlen && (!draft_lens || !aligned(draft_lens, 4))) return GDN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(alpha, 4) ||
      !aligned(beta, 4) || !aligned(out, 16) || !aligned(slot_idx, 4))
    return GDN_EINVAL;
  a->c = view_of(c);
  a->num_reqs = num_reqs;
  a->draft = draft_len;
  a->slot_idx = slot_idx;
  a->draft_lens = varlen ? draft_lens : nullptr;
  a->prev_accepted = nullptr;
  a->prev_draft_lens = nullptr;
  a->prev_draft = 0;
  a->norm_z = nullptr;
  a->norm_w = nullptr;
  a->norm_eps = 0.f;
  a->norm_q = nullptr;
  a->norm_scale = nullptr;
  a->q = q;
  a->k = k;
  a->v = v;
  a->alpha = alpha;
  a->beta = beta;
  a->out = out;
  return GDN_OK;
}

int launch_verify(const gdn_replay_cache *c, const gdnr::VerifyArgs &a, hipStream_t stream) {
  const bool f32 = c->in_dtype == GDN_F32;
  const hipError_t e = gdnr::chunked_supported(c->d_k, c->d_v, f32, a.draft)
                           ? gdnr::launch_verify_chunked(a, stream)
                           : gdnr::launch_verify_recurrent(a, f32, stream);
  return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

gdnr::FlushArgs flush_args(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                           int32_t min_len) {
  gdnr::FlushArgs a;
  a.c = view_of(c);
  a.num_reqs = num_reqs;
  a.min_len = min_len;
  a.slot_idx = slot_idx;
  a.draft_lens = nullptr;
  a.max_draft = 0;
  return a;
}

int launch_flush(const gdn_replay_cache *c, const gdnr::FlushArgs &a, hipStream_t stream) {
  const bool f32 = c->in_dtype == GDN_F32;
  const hipError_t e = gdnr::chunked_supported(c->d_k, c->d_v, f32, 0)
                           ? gdnr::launch_flush_chunked(a, stream)
                           : gdnr::launch_flush_recurrent(a, f32, stream);
  return e == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // namespace

extern "C" {

int gdn_replay_verify(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                      int32_t draft_len, const void *q, const void *k, const void *v,
                      const float *alpha, const float *beta, float *out, hipStream_t stream) {
  gdnr::VerifyArgs a;
  const int st = verify_args(c, num_reqs, slot_idx, draft_len, q, k, v, alpha, beta, out, &a);
  if (st != GDN_OK || num_reqs == 0) return st;
  return launch_verify(c, a, stream);
}

int gdn_replay_verify_varlen(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                             const int32_t *draft_lens, int32_t max_draft, const void *q,
                             const void *k, const void *v, const float *alpha, const float *beta,
                             float *out, hipStream_t stream) {
  gdnr::VerifyArgs a;
  const int st = verify_args(c, num_reqs, slot_idx, max_draft, q, k, v, alpha, beta, out, &a,
                             true, draft_lens);
  if (st != GDN_OK || num_reqs == 0) return st;
  return launch_verify(c, a, stream);
}

}  // extern "C"

namespace {

int verify_flush_impl(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                      int32_t draft_len, int32_t min_len, const void *q, const void *k,
                      const void *v, const float *alpha, const float *beta, float *out,
                      hipStream_t stream, bool varlen, const int32_t *draft_lens) {
  gdnr::VerifyArgs a;
  const int st = verify_args(c, num_reqs, slot_idx, draft_len, q, k, v, alpha, beta, out, &a,
                             varlen, draft_lens);
  if (st != GDN_OK || num_reqs == 0) return st;
  const bool f32 = c->in_dtype == GDN_F32;
  if (gdnr::fused_supported(c->d_k, c->d_v, f32, draft_len, c->ring_cap))
    return gdnr::launch_verify_flush_fused(a, min_len, stream) == hipSuccess ? GDN_OK : GDN_EHIP;
  if (gdnr::fused_long_supported(c->d_k, c->d_v, f32, draft_len, c->ring_cap))
    return gdnr::launch_verify_flush_long(a, min_len, stream) == hipSuccess ? GDN_OK : GDN_EHIP;
  // Other shapes: the same result from the two calls back to back. With
  // per-request lengths a request whose length is out of range must not be
  // flushed, so the flush checks the lengths too.
  gdnr::FlushArgs fa = flush_args(c, num_reqs, slot_idx, min_len);
  fa.draft_lens = a.draft_lens;
  fa.max_draft = draft_len;
  const int fs = launch_flush(c, fa, stream);
  return fs != GDN_OK ? fs : launch_verify(c, a, stream);
}

int rollback_impl(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                  int32_t draft_len, const int32_t *num_accepted, hipStream_t stream, bool varlen,
                  const int32_t *draft_lens) {
  int st = check_cache(c);
  if (st != GDN_OK) return st;
  if (num_reqs < 0 || num_reqs > c->num_slots) return GDN_EINVAL;
  if (draft_len < 1 || draft_len > c->ring_cap) return GDN_EINVAL;
  if (num_reqs == 0) return GDN_OK;
  if (!slot_idx || !num_accepted) return GDN_EINVAL;
  if (!aligned(slot_idx, 4) || !aligned(num_accepted, 4)) return GDN_EINVAL;
  if (varlen && (!draft_lens || !aligned(draft_lens, 4))) return GDN_EINVAL;
  gdnr::RollbackArgs a;
  a.c = view_of(c);
  a.num_reqs = num_reqs;
  a.draft = draft_len;
  a.slot_idx = slot_idx;
  a.draft_lens = varlen ? draft_lens : nullptr;
  a.num_accepted = num_accepted;
  return gdnr::launch_rollback(a, stream) == hipSuccess ? GDN_OK : GDN_EHIP;
}

}  // namespace

extern "C" {

int gdn_replay_verify_flush(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                            int32_t draft_len, int32_t min_len, const void *q, const void *k,
                            const void *v, const float *alpha, const float *beta, float *out,
                            hipStream_t stream) {
  return verify_flush_impl(c, num_reqs, slot_idx, draft_len, min_len, q, k, v, alpha, beta, out,
                           stream, false, nullptr);
}

int gdn_replay_verify_flush_varlen(const gdn_replay_cache *c, int32_t num_reqs,
                                   const int32_t *slot_idx, const int32_t *draft_lens,
                                   int32_t max_draft, int32_t min_len, const void *q,
                                   const void *k, const void *v, const float *alpha,
                                   const float *beta, float *out, hipStream_t stream) {
  return verify_flush_impl(c, num_reqs, slot_idx, max_draft, min_len, q, k, v, alpha, beta, out,
                           stream, true, draft_lens);
}

int gdn_replay_rollback_verify_flush(const gdn_replay_cache *c, int32_t num_reqs,
                                     const int32_t *slot_idx, const int32_t *num_accepted,
                                     const int32_t *prev_draft_lens, int32_t prev_draft,
                                     const int32_t *draft_lens, int32_t draft_len,
                                     int32_t min_len, const void *q, const void *k, const void *v,
                                     const float *alpha, const float *beta, float *out,
                                     hipStream_t stream) {
  return gdnr::rollback_verify_flush_call(c, num_reqs, slot_idx, num_accepted, prev_draft_lens,
                                          prev_draft, draft_lens, draft_len, min_len, q, k, v,
                                          alpha, beta, out, stream, false);
}

}  // extern "C"

namespace gdnr {

int rollback_verify_flush_call(const gdn_replay_cache *c, int32_t num_reqs,
                               const int32_t *slot_idx, const int32_t *num_accepted,
                               const int32_t *prev_draft_lens, int32_t prev_draft,
                               const int32_t *draft_lens, int32_t draft_len, int32_t min_len,
                               const void *q, const void *k, const void *v, const float *alpha,
                               const float *beta, float *out, hipStream_t stream, bool check_only) {
  gdnr::VerifyArgs a;
  const bool varlen = draft_lens != nullptr;
  int st = verify_args(c, num_reqs, slot_idx, draft_len, q, k, v, alpha, beta, out, &a, varlen,
                       draft_lens);
  if (st != GDN_OK || num_reqs == 0) return st;
  if (prev_draft < 1 || prev_draft > c->ring_cap) return GDN_EINVAL;
  if (!num_accepted || !aligned(num_accepted, 4)) return GDN_EINVAL;
  if (prev_draft_lens && !aligned(prev_draft_lens, 4)) return GDN_EINVAL;
  if (check_only) return GDN_OK;
  const bool f32 = c->in_dtype == GDN_F32;
  const bool one_chunk = gdnr::fused_supported(c->d_k, c->d_v, f32, draft_len, c->ring_cap);
  if (one_chunk || gdnr::fused_long_supported(c->d_k, c->d_v, f32, draft_len, c->ring_cap)) {
    a.prev_accepted = num_accepted;
    a.prev_draft_lens = prev_draft_lens;
    a.prev_draft = prev_draft;
    const hipError_t e = one_chunk ? gdnr::launch_verify_flush_fused(a, min_len, stream)
                                   : gdnr::launch_verify_flush_long(a, min_len, stream);
    return e == hipSuccess ? GDN_OK : GDN_EHIP;
  }
  // Other shapes: the rollback, then verify_flush, as separate launches.
  st = rollback_impl(c, num_reqs, slot_idx, prev_draft, num_accepted, stream,
                     prev_draft_lens != nullptr, prev_draft_lens);
  if (st != GDN_OK) return st;
  return verify_flush_impl(c, num_reqs, slot_idx, draft_len, min_len, q, k, v, alpha, beta, out,
                           stream, varlen, draft_lens);
}

}  // namespace gdnr

extern "C" {

int gdn_replay_step_norm_fp8(const gdn_replay_cache *c, int32_t num_reqs,
                             const int32_t *slot_idx, const int32_t *num_accepted,
                             const int32_t *prev_draft_lens, int32_t prev_draft,
                             const int32_t *draft_lens, int32_t draft_len, int32_t min_len,
                             const void *q, const void *k, const void *v, const float *alpha,
                             const float *beta, float *out, const gdn_norm_fp8 *norm,
                             hipStream_t stream) {
  gdnr::VerifyArgs a;
  const bool varlen = draft_lens != nullptr;
  int st = verify_args(c, num_reqs, slot_idx, draft_len, q, k, v, alpha, beta, out, &a, varlen,
                       draft_lens, /*out_optional=*/true);
  if (st != GDN_OK) return st;
  if (!gdnr::fused_supported(c->d_k, c->d_v, c->in_dtype == GDN_F32, draft_len, c->ring_cap))
    return GDN_EUNSUPPORTED;
  if (!norm || !(norm->eps > 0.f) || norm->eps > 1.f) return GDN_EINVAL;  // also rejects NaN
  if (num_reqs == 0) return GDN_OK;
  if (prev_draft < 1 || prev_draft > c->ring_cap) return GDN_EINVAL;
  if (!num_accepted || !aligned(num_accepted, 4)) return GDN_EINVAL;
  if (prev_draft_lens && !aligned(prev_draft_lens, 4)) return GDN_EINVAL;
  if (!norm->z || !norm->weight || !norm->q || !norm->scale) return GDN_EINVAL;
  if (!aligned(norm->z, 4) || !aligned(norm->weight, 8) || !aligned(norm->q, 2) ||
      !aligned(norm->scale, 4))
    return GDN_EINVAL;
  a.prev_accepted = num_accepted;
  a.prev_draft_lens = prev_draft_lens;
  a.prev_draft = prev_draft;
  a.norm_z = norm->z;
  a.norm_w = norm->weight;
  a.norm_eps = norm->eps;
  a.norm_q = norm->q;
  a.norm_scale = norm->scale;
  return gdnr::launch_verify_flush_fused(a, min_len, stream) == hipSuccess ? GDN_OK : GDN_EHIP;
}

int gdn_replay_rollback(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                        int32_t draft_len, const int32_t *num_accepted, hipStream_t stream) {
  return rollback_impl(c, num_reqs, slot_idx, draft_len, num_accepted, stream, false, nullptr);
}

int gdn_replay_rollback_varlen(const gdn_replay_cache *c, int32_t num_reqs,
                               const int32_t *slot_idx, const int32_t *draft_lens,
                               int32_t max_draft, const int32_t *num_accepted, hipStream_t stream) {
  return rollback_impl(c, num_reqs, slot_idx, max_draft, num_accepted, stream, true, draft_lens);
}

int gdn_replay_flush(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                     int32_t min_len, hipStream_t stream) {
  int st = check_cache(c);
  if (st != GDN_OK) return st;
  if (num_reqs < 0 || num_reqs > c->num_slots) return GDN_EINVAL;
  if (!replay_grid_ok(num_reqs, c)) return GDN_EUNSUPPORTED;
  if (num_reqs == 0) return GDN_OK;
  if (!slot_idx || !aligned(slot_idx, 4)) return GDN_EINVAL;
  return launch_flush(c, flush_args(c, num_reqs, slot_idx, min_len), stream);
}

int gdn_gated_rmsnorm_fp8(int32_t rows, int32_t num_heads, int32_t d_v, const float *o,
                          const void *z, const float *weight, float eps, uint8_t *q, float *scale,
                          hipStream_t stream) {
  if (rows < 0 || num_heads < 1 || d_v < 1) return GDN_EINVAL;
  if (!gdnr::norm_supported(d_v)) return GDN_EUNSUPPORTED;
  // 8 groups per workgroup of 256 threads: 32 work-items per group
  if ((int64_t)rows * num_heads * 32 > kMaxWorkItems) return GDN_EUNSUPPORTED;
  if (!(eps > 0.f) || eps > 1.f) return GDN_EINVAL;  // also rejects NaN
  if (rows == 0) return GDN_OK;
  if (!o || !z || !weight || !q || !scale) return GDN_EINVAL;
  if (!aligned(o, 16) || !aligned(z, 8) || !aligned(weight, 16) || !aligned(q, 4) ||
      !aligned(scale, 4))
    return GDN_EINVAL;
  gdnr::NormArgs a;
  a.groups = (int64_t)rows * num_heads;
  a.o = o;
  a.z = z;
  a.weight = weight;
  a.eps = eps;
  a.q = q;
  a.scale = scale;
  return gdnr::launch_gated_rmsnorm_fp8(a, d_v, stream) == hipSuccess ? GDN_OK : GDN_EHIP;
}

int gdn_causal_conv_update(const gdn_replay_cache *c, void *conv_ring, int32_t channels,
                           int32_t width, int32_t num_reqs, const int32_t *slot_idx,
                           const int32_t *num_accepted, const int32_t *prev_draft_lens,
                           int32_t prev_draft, int32_t draft_len, const void *x,
                           const float *weight, const float *bias, void *y, hipStream_t stream) {
  int st = check_cache(c);
  if (st != GDN_OK) return st;
  if (channels < 2 || channels % 2 != 0) return GDN_EINVAL;
  if (!gdnr::conv_width_supported(width)) return GDN_EUNSUPPORTED;
  if (c->in_dtype != GDN_BF16) return GDN_EUNSUPPORTED;
  if (num_reqs < 0 || num_reqs > c->num_slots) return GDN_EINVAL;
  if (draft_len < 1 || draft_len + width - 1 > c->ring_cap) return GDN_EINVAL;
  if ((channels / 2 + 255) / 256 > 65535 || num_reqs > 65535) return GDN_EUNSUPPORTED;  // grid
  if (draft_len > 65535) return GDN_EUNSUPPORTED;
  if (num_reqs == 0) return GDN_OK;
  if (!conv_ring || !slot_idx || !x || !weight || !y) return GDN_EINVAL;
  if (num_accepted) {  // the previous draft's rollback is still pending
    if (prev_draft < 1 || prev_draft > c->ring_cap) return GDN_EINVAL;
    if (!aligned(num_accepted, 4) || (prev_draft_lens && !aligned(prev_draft_lens, 4)))
      return GDN_EINVAL;
  }
  if (!aligned(conv_ring, 4) || !aligned(slot_idx, 4) || !aligned(x, 4) || !aligned(weight, 4) ||
      (bias && !aligned(bias, 4)) || !aligned(y, 4))
    return GDN_EINVAL;
  gdnr::ConvArgs a;
  a.c = view_of(c);
  a.num_reqs = num_reqs;
  a.draft = draft_len;
  a.channels = channels;
  a.slot_idx = slot_idx;
  a.prev_accepted = num_accepted;
  a.prev_draft_lens = num_accepted ? prev_draft_lens : nullptr;
  a.prev_draft = num_accepted ? prev_draft : 0;
  a.ring = conv_ring;
  a.x = x;
  a.weight = weight;
  a.bias = bias;
  a.y = y;
  return gdnr::launch_causal_conv_update(a, width, stream) == hipSuccess ? GDN_OK : GDN_EHIP;
}

int64_t gdn_replay_sync_entries(int32_t num_slots, int32_t num_k_heads) {
  if (num_slots < 0 || num_k_heads < 0) return 0;
  return gdnr::sync_entries(num_slots, num_k_heads);
}

const char *gdn_replay_strerror(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument";
    case GDN_EUNSUPPORTED: return "unsupported configuration (head dims, dtype or ring capacity)";
    case GDN_EHIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int gdn_replay_version(void) { return GDN_REPLAY_VERSION; }

}  // extern "C"
