/*
 * gdn_replay.h — C ABI of libgdnreplay.so: ReplaySSM verify / rollback / flush
 * for Gated DeltaNet (GDN) layers under block speculative decoding, MI355X
 * (gfx950).
 *
 * The scheme is the one described in "The inference stack behind OCRia"
 * (LlamaIndex), section "Making speculative verification cheaper": a GDN layer
 * summarises its history in a fixed-size recurrent state; instead of writing
 * that state back per token and restoring it when a speculative token is
 * rejected, each (request, value head) keeps a state checkpoint plus a small
 * buffer of recent inputs. Outputs are computed from the checkpoint and the
 * buffered inputs, the full checkpoint is rewritten only at a periodic flush,
 * and a rejection only moves the buffer pointer so the accepted prefix is kept.
 *
 * The recurrence replayed is the gated delta rule (Yang et al., "Gated Delta
 * Networks", 2025), per value head, with S of shape d_v x d_k:
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t   (output after the update).
 * No q scaling and no normalisation happen inside: the caller passes final
 * q, k, alpha (multiplicative decay) and beta (write strength).
 *
 * Memory: every pointer below is a DEVICE pointer unless stated otherwise. The
 * caller owns all memory. The library allocates nothing, keeps no pointer after
 * a call returns and holds no global state; calls are reentrant.
 *
 * Ordering: every call only enqueues work on `stream` (no host/device
 * synchronisation). Stream order gives verify -> rollback -> flush, or
 * verify_flush -> rollback with the flush folded into the next step's verify.
 *
 * Errors: host-side validation is synchronous: a non-zero gdn_status is
 * returned and nothing is enqueued. Contract violations that only the device
 * can see (they depend on device-resident pointers) skip the offending
 * request with no writes at all and OR a GDN_DERR_* bit into *err (a sticky
 * word the caller clears). A failed kernel launch returns GDN_EHIP.
 * Calls whose launch would exceed a dispatch's 32-bit work-item count return
 * GDN_EUNSUPPORTED: num_reqs * HV * 256 must stay below 2^31 for the replay
 * calls, rows * num_heads * 32 for gdn_gated_rmsnorm_fp8.
 */
#ifndef GDN_REPLAY_H
#define GDN_REPLAY_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_REPLAY_VERSION 7

typedef enum {
  GDN_OK = 0,
  GDN_EINVAL = -1,        /* bad argument: NULL, negative size, D outside 1..C, ... */
  GDN_EUNSUPPORTED = -2,  /* valid but not built: head dims, dtype, ring capacity   */
  GDN_EHIP = -3           /* the HIP runtime refused the launch                     */
} gdn_status;

typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype; /* dtype of q, k, v (ring and draft) */

/* sticky device error bits */
enum {
  GDN_DERR_CAPACITY = 1,  /* verify: len + D > C;  rollback: len + a > C  */
  GDN_DERR_ACCEPT = 2,    /* rollback: a outside [0, D]                  */
  GDN_DERR_SLOT = 4,      /* slot index outside [0, num_slots)           */
  GDN_DERR_POINTER = 8,   /* head outside [0, C) or len outside [0, C]   */
  GDN_DERR_DRAFT = 16     /* *_varlen: draft_lens[i] outside [0, max_draft] */
};

/*
 * One layer's replay cache. Host struct describing caller-owned device memory.
 * All arrays are dense row-major.
 *
 *   state      [num_slots][HV][d_k][d_v] fp32. Element (i, j) holds S[j][i]:
 *              the checkpoint is stored as H = S^T (d_k rows of d_v floats).
 *              16-byte aligned.
 *   ring_q     [num_slots][HK][C][d_k] in_dtype, or NULL. Written by verify
 *              (draft append), never read: a buffered token's q is not needed
 *              because its output was already emitted.
 *   ring_k     [num_slots][HK][C][d_k] in_dtype.
 *   ring_v     [num_slots][HV][C][d_v] in_dtype.
 *   ring_alpha [num_slots][HV][C] fp32, ring_beta [num_slots][HV][C] fp32.
 *   head       [num_slots] int32: ring position of the first committed token.
 *   len        [num_slots] int32: committed tokens not yet in the checkpoint.
 *              The committed tokens sit at (head + t) mod C, t < len.
 *   sync       int32 arrival counters, zero when created; every completed call
 *              leaves them zero. They let the last workgroup of a slot (flush)
 *              or of the grid (verify_flush) move the pointers once every
 *              workgroup has read them. At least
 *              gdn_replay_sync_entries(num_slots, HK) entries (32 * (num_slots
 *              + 1) + num_slots * HK: the counters that many workgroups hit sit
 *              128 bytes apart, since atomics on one cache line are served one
 *              after another); 128-byte alignment keeps each on a line of its
 *              own.
 *   sync_len   number of int32 entries the caller allocated at sync. Every call
 *              returns GDN_EINVAL, with nothing enqueued, when it is below
 *              gdn_replay_sync_entries(num_slots, HK); GDN_EUNSUPPORTED when
 *              that count does not fit in an int32.
 *   err        [1] int32 sticky error word, or NULL to drop device errors.
 *
 * Value head h reads key head h / (HV / HK) (consecutive grouping, HV % HK == 0).
 * Built head dims: d_k = d_v in {16, 32, 64, 128}. Ring capacity 1..256.
 */
typedef struct {
  int32_t num_slots;
  int32_t num_v_heads;  /* HV */
  int32_t num_k_heads;  /* HK */
  int32_t d_k;
  int32_t d_v;
  int32_t ring_cap;     /* C */
  int32_t in_dtype;     /* gdn_dtype */
  int32_t sync_len;     /* entries of sync */
  float *state;
  void *ring_q;
  void *ring_k;
  void *ring_v;
  float *ring_alpha;
  float *ring_beta;
  int32_t *head;
  int32_t *len;
  int32_t *sync;
  int32_t *err;
} gdn_replay_cache;

/*
 * gdn_replay_verify — outputs of a draft block, computed from the checkpoint and
 * the buffered inputs without writing the state back ("Making speculative
 * verification cheaper", as above).
 *
 * For request i with slot s = slot_idx[i] and every value head h: start from
 * the checkpoint S_c[s, h], replay the len[s] committed ring tokens in order,
 * then draft tokens j = 0..D-1, and write
 *     out[i][j][h][:] = S q_j   for the state after draft token j.
 * The draft (q if ring_q != NULL, k, v, alpha, beta) is appended to ring
 * positions (head + len + j) mod C, so that a later rollback only has to move
 * a pointer. state, head and len are NOT modified.
 *
 *   num_reqs   >= 0 (0 is a no-op returning GDN_OK).
 *   slot_idx   [num_reqs] int32, unique within the call (caller's guarantee).
 *   draft_len  D, 1..C.
 *   q, k       [num_reqs][D][HK][d_k] in_dtype;  v [num_reqs][D][HV][d_v] in_dtype.
 *   alpha,beta [num_reqs][D][HV] fp32.
 *   out        [num_reqs][D][HV][d_v] fp32; must not alias any input.
 * Device errors: len + D > C -> CAPACITY; slot out of range -> SLOT; head or len
 * of the slot out of range -> POINTER. The request is skipped: its out rows and
 * its ring are left untouched.
 */
int gdn_replay_verify(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                      int32_t draft_len, const void *q, const void *k, const void *v,
                      const float *alpha, const float *beta, float *out, hipStream_t stream);

/*
 * gdn_replay_rollback — keep the accepted prefix by moving the buffer pointer
 * only ("Making speculative verification cheaper": rejection adjusts the buffer
 * pointer, no full-state restore). The first a = num_accepted[i] tokens of the
 * draft last appended by verify become committed: len[s] += a. Tokens after the
 * first rejection are dropped ("Inference Engineering", chapter 5, section 5.2:
 * a rejected draft token rejects all later ones), so a in [0, D] says it all.
 *
 *   num_accepted [num_reqs] int32 (device).
 * Device errors: a outside [0, D] -> ACCEPT; len + a > C -> CAPACITY; slot out
 * of range -> SLOT; head or len out of range -> POINTER (request skipped).
 */
int gdn_replay_rollback(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                        int32_t draft_len, const int32_t *num_accepted, hipStream_t stream);

/*
 * gdn_replay_flush — the periodic checkpoint update ("Making speculative
 * verification cheaper": the full checkpoint is only updated at a periodic
 * flush). For every slot s = slot_idx[i] with len[s] >= max(min_len, 1): fold
 * its len[s] committed tokens into state[s] (all value heads), then
 * head[s] = (head[s] + len[s]) mod C and len[s] = 0. Other slots are untouched
 * (their state bytes are not rewritten).
 *
 * Device errors: slot out of range -> SLOT; head or len out of range -> POINTER
 * (request skipped).
 */
int gdn_replay_flush(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                     int32_t min_len, hipStream_t stream);

/*
 * gdn_replay_verify_flush — gdn_replay_flush(min_len) followed by
 * gdn_replay_verify, in one pass over the state: the periodic flush ("Making
 * speculative verification cheaper", as above) is folded into the next
 * verify, so the state of a due slot is read once and written once.
 *
 * For request i with slot s = slot_idx[i]: if len[s] >= max(min_len, 1), fold the
 * len[s] committed tokens into state[s], head[s] = (head[s] + len[s]) mod C and
 * len[s] = 0 (exactly as gdn_replay_flush); then verify the draft exactly as
 * gdn_replay_verify, from the resulting checkpoint, pointers and ring. Arguments
 * as for gdn_replay_verify plus min_len. bf16 inputs with d_k = d_v in
 * {64, 128} and D <= 32 run as one kernel (a replay of one chunk of 32 tokens
 * for ring capacity <= 32, of several above); other shapes run the two calls
 * back to back on the stream.
 * Device errors: slot out of range -> SLOT; head or len out of range -> POINTER;
 * a slot that is not due with len + D > C -> CAPACITY. The request is skipped
 * with no writes at all (no flush either).
 */
int gdn_replay_verify_flush(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                            int32_t draft_len, int32_t min_len, const void *q, const void *k,
                            const void *v, const float *alpha, const float *beta, float *out,
                            hipStream_t stream);

/*
 * Per-request draft lengths. Speculative decoding drafts a block of tokens per
 * request and keeps the prefix up to the first rejected one ("Inference
 * Engineering", chapter 5, section 5.2); here each request i drafts its own
 * D_i = draft_lens[i] tokens, 0 <= D_i <= max_draft. D_i = 1 with every token
 * accepted is plain (non-speculative) decode; D_i = 0 gives the request no
 * draft this step (nothing appended or emitted; verify_flush still flushes it).
 *
 * The draft arrays keep the layout of the fixed-length calls with
 * D = max_draft: request i's tokens are rows 0 .. D_i - 1 of its max_draft-row
 * block of q, k, v, alpha, beta and out, so all num_reqs * max_draft rows must
 * be allocated. Rows D_i .. max_draft - 1 are never written and their values
 * are never used (verify_flush may load them into cache ahead of use).
 *
 *   draft_lens [num_reqs] int32 (device).   max_draft: 1..C (host value).
 * Device errors as for the fixed-length calls, plus DRAFT when D_i is outside
 * [0, max_draft] (request skipped with no writes; verify_flush does not flush
 * it either). Checks run in the order slot, pointers, draft length, then
 * capacity or accept count. rollback_varlen needs a in [0, D_i].
 */
int gdn_replay_verify_varlen(const gdn_replay_cache *c, int32_t num_reqs, const int32_t *slot_idx,
                             const int32_t *draft_lens, int32_t max_draft, const void *q,
                             const void *k, const void *v, const float *alpha, const float *beta,
                             float *out, hipStream_t stream);
int gdn_replay_verify_flush_varlen(const gdn_replay_cache *c, int32_t num_reqs,
                                   const int32_t *slot_idx, const int32_t *draft_lens,
                                   int32_t max_draft, int32_t min_len, const void *q,
                                   const void *k, const void *v, const float *alpha,
                                   const float *beta, float *out, hipStream_t stream);
int gdn_replay_rollback_varlen(const gdn_replay_cache *c, int32_t num_reqs,
                               const int32_t *slot_idx, const int32_t *draft_lens,
                               int32_t max_draft, const int32_t *num_accepted, hipStream_t stream);

/*
 * gdn_replay_rollback_verify_flush — the whole step of a layer in one call: the
 * rollback of the previous draft (pointer only, "Making speculative
 * verification cheaper"), then verify_flush of this step's draft. Its result
 * (out, state, ring, head, len, err) is exactly that of
 *     gdn_replay_rollback[_varlen](slot_idx, prev_draft[_lens], num_accepted)
 *     gdn_replay_verify_flush[_varlen](slot_idx, draft_len[s], min_len, ...)
 * on the same requests. Request i therefore both commits num_accepted[i]
 * tokens of the draft it appended in the previous step and verifies its new
 * draft; a request new to the batch passes num_accepted[i] = 0. With the
 * rollback folded in, the pointer moves of both calls are made once, by the
 * last workgroup of the kernel, and a due slot is flushed together with the
 * tokens it has just accepted.
 *
 *   num_accepted    [num_reqs] int32 (device).
 *   prev_draft_lens [num_reqs] int32 (device) lengths of the previous drafts,
 *                   or NULL: every previous draft had prev_draft tokens.
 *   prev_draft      1..C (host): the previous drafts' (maximum) length.
 *   draft_lens      [num_reqs] int32 (device) lengths of this step's drafts,
 *                   or NULL: every draft has draft_len tokens.
 *   draft_len       1..C (host): this step's (maximum) draft length.
 *   other arguments as for gdn_replay_verify_flush.
 * Device errors: those of the two calls. A request whose rollback fails (DRAFT
 * for a previous length out of range, ACCEPT, CAPACITY) keeps its len, as the
 * rollback call would leave it, and goes on to verify_flush. Shapes the fused
 * kernel does not take run the two calls back to back on the stream.
 */
int gdn_replay_rollback_verify_flush(const gdn_replay_cache *c, int32_t num_reqs,
                                     const int32_t *slot_idx, const int32_t *num_accepted,
                                     const int32_t *prev_draft_lens, int32_t prev_draft,
                                     const int32_t *draft_lens, int32_t draft_len,
                                     int32_t min_len, const void *q, const void *k, const void *v,
                                     const float *alpha, const float *beta, float *out,
                                     hipStream_t stream);

/*
 * gdn_replay_step_norm_fp8 — gdn_replay_rollback_verify_flush with the gated
 * RMSNorm + FP8 of its outputs in the same kernel: the draft outputs go
 * through the norm while still in registers ("The inference stack behind
 * OCRia", section on fusing kernels: avoid HBM round trips between the
 * producer of a tensor and its normalisation and quantisation), so the fp32
 * outputs need not be written or read back.
 *
 * Result: out (if not NULL), state, ring, head, len and err exactly as
 * gdn_replay_rollback_verify_flush with the same arguments; norm->q and
 * norm->scale as gdn_gated_rmsnorm_fp8 over the draft rows of out (the
 * [num_reqs * D][HV] groups, D = draft_len), i.e. for request i, draft token
 * j < D_i, value head h: the group out[i][j][h][:] with gate z[i][j][h][:].
 * Rows j >= D_i and skipped requests (device errors) are left untouched in
 * q and scale, as in out. Arithmetic in fp32 as gdn_gated_rmsnorm_fp8 (the sums
 * are taken in another order, so a code can differ from that call's where the
 * value lies at a rounding midpoint).
 *
 *   out   [num_reqs][D][HV][d_v] fp32, or NULL: outputs not stored.
 *   norm  z [num_reqs][D][HV][d_v] bf16 (4-byte aligned), weight [d_v] fp32
 *         (8-byte aligned), eps in (0, 1], q [num_reqs][D][HV][d_v] uint8
 *         (2-byte aligned), scale [num_reqs][D][HV] fp32.
 *   other arguments as for gdn_replay_rollback_verify_flush.
 * Only the one-kernel shapes (bf16 inputs, d_k = d_v in {64, 128}, ring
 * capacity <= 32, D <= 32) are taken: GDN_EUNSUPPORTED otherwise (the
 * library allocates no scratch for a fallback; use the separate calls).
 * Performance: the norm lengthens every workgroup's life, so this pays off
 * when the launch is one generation of workgroups (num_reqs * HV up to about
 * 4 per CU); for larger batches the two separate calls are faster.
 */
typedef struct gdn_norm_fp8 {
  const void *z;
  const float *weight;
  float eps;
  uint8_t *q;
  float *scale;
} gdn_norm_fp8;

int gdn_replay_step_norm_fp8(const gdn_replay_cache *c, int32_t num_reqs,
                             const int32_t *slot_idx, const int32_t *num_accepted,
                             const int32_t *prev_draft_lens, int32_t prev_draft,
                             const int32_t *draft_lens, int32_t draft_len, int32_t min_len,
                             const void *q, const void *k, const void *v, const float *alpha,
                             const float *beta, float *out, const gdn_norm_fp8 *norm,
                             hipStream_t stream);

/*
 * gdn_gated_rmsnorm_fp8 — the step after the recurrence: gated RMSNorm of the
 * GDN output followed by FP8 quantisation, in one kernel ("The inference stack
 * behind OCRia", section on fusing kernels: the gated RMSNorm and the FP8
 * quantisation of its result run as one kernel so that the normalised values
 * never go through HBM). For every (row t, head h) group of d_v values:
 *     r = sqrt(mean_j o[t][h][j]^2 + eps)
 *     y_j = o[t][h][j] / r * weight[j] * silu(z[t][h][j]),  silu(x) = x / (1 + e^-x)
 *     scale[t][h] = max_j |y_j| / 448   (1 when every y_j is 0)
 *     q[t][h][j] = E4M3(y_j / scale[t][h])
 * E4M3 is the OCP 8-bit float (sign, 4 exponent bits, bias 7, 3 mantissa bits,
 * largest finite 448), rounded to nearest even and saturating; a group
 * dequantises as q * scale. Computed in fp32.
 *
 *   rows >= 0 (0 is a no-op), num_heads >= 1, d_v in {16, 32, 64, 128}.
 *   o      [rows][num_heads][d_v] fp32 (e.g. the out of gdn_replay_verify with
 *          rows = num_reqs * D), 16-byte aligned.
 *   z      [rows][num_heads][d_v] bf16 gate, 8-byte aligned.
 *   weight [d_v] fp32, shared by the heads, 16-byte aligned.   eps in (0, 1] (an
 *          all-zero group then normalises to zeros).
 *   q      [rows][num_heads][d_v] uint8 codes (4-byte aligned); scale
 *          [rows][num_heads] fp32. Outputs must not alias inputs.
 * Errors: synchronous only (EINVAL / EUNSUPPORTED / EHIP); nothing is enqueued
 * on error.
 */
int gdn_gated_rmsnorm_fp8(int32_t rows, int32_t num_heads, int32_t d_v, const float *o,
                          const void *z, const float *weight, float eps, uint8_t *q, float *scale,
                          hipStream_t stream);

/*
 * gdn_causal_conv_update — the step before the recurrence: the short causal
 * convolution of a GDN layer over a draft block, with its state kept the
 * ReplaySSM way. GDN layers convolve their q, k, v projections causally before
 * the recurrence ("The inference stack behind OCRia", LlamaIndex, which lists a
 * faster causal convolution for GDN layers among its kernels); the state is the
 * last K - 1 inputs of the committed stream, and, as for the recurrence's
 * inputs ("Making speculative verification cheaper"), it lives in a ring whose
 * pointers move instead of being restored:
 *   conv_ring [num_slots][C][channels] bf16, caller-owned, zero when a slot starts;
 *             it shares num_slots, C, head, len and err with the cache c.
 * For request i (slot s = slot_idx[i], h = head[s], n = len[s]) and channel ch:
 *   y[i][j][ch] = silu(bias[ch] + sum_{t<K} weight[ch][t] * x_{j-K+1+t}[ch]),
 * where x_{-m} (m >= 1) is conv_ring[s][(h + n - m) mod C][ch]; then the draft x
 * is appended at conv_ring[s][(h + n + j) mod C] (where gdn_replay_verify appends
 * its rows). Pointers are not changed: gdn_replay_rollback and gdn_replay_flush
 * (or verify_flush) move them for both rings. Call it before the step's verify,
 * with the same slots and D.
 *
 * Which len: with num_accepted == NULL, len[s] as it stands, i.e. after the
 * previous draft's rollback (the separate calls: verify, rollback, flush per
 * step, or verify_flush then rollback). With the one-call step
 * (gdn_replay_rollback_verify_flush, gdn_replay_step_norm_fp8), whose rollback
 * of the previous draft happens inside the step after this call, pass the
 * step's num_accepted, prev_draft_lens and prev_draft: n is then len[s] + a,
 * exactly the committed count that step works from (len[s] where the step's
 * rollback fails: a outside [0, previous length], a previous length outside
 * [0, prev_draft], or len + a > C; the step raises those errors, this call
 * does not). Either way the draft lands where the step's verify appends its
 * rows, and its history is the last K - 1 tokens the step has committed.
 *   num_accepted    [num_reqs] int32 (device) or NULL; prev_draft_lens
 *                   [num_reqs] int32 or NULL (every previous draft had
 *                   prev_draft tokens); prev_draft 1..C (host) when
 *                   num_accepted is given, ignored otherwise.
 *   channels even >= 2; width K in 1..8; D >= 1 with D + K - 1 <= C (the draft
 *   never overwrites the history it reads); inputs bf16 only (in_dtype).
 *   x, y      [num_reqs][D][channels] bf16 (y rounded to nearest even), 4-byte aligned.
 *   weight    [channels][K] fp32;  bias [channels] fp32 or NULL.
 * Only the last K - 1 committed inputs are read, so len + D may exceed C (the
 * draft then overwrites inputs no step reads again): the call can run before a
 * gdn_replay_verify_flush that folds the due slots in the same step.
 * Device errors: SLOT, POINTER as for verify: the request is skipped with no
 * writes.
 */
int gdn_causal_conv_update(const gdn_replay_cache *c, void *conv_ring, int32_t channels,
                           int32_t width, int32_t num_reqs, const int32_t *slot_idx,
                           const int32_t *num_accepted, const int32_t *prev_draft_lens,
                           int32_t prev_draft, int32_t draft_len, const void *x,
                           const float *weight, const float *bias, void *y, hipStream_t stream);

/*
 * gdn_replay_rollback_verify_flush_noalloc — for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops that must not
 * allocate, harnesses that forbid it. The same call, with the same result, as
 * gdn_replay_rollback_verify_flush, except that the arrival counters come from
 * a library-owned device array instead of c->sync: c->sync and c->sync_len are
 * ignored (they may be NULL and 0); the other fields and arguments are as for
 * gdn_replay_rollback_verify_flush.
 *
 * Limit: gdn_replay_sync_entries(num_slots, HK) must not exceed
 * GDN_REPLAY_NOALLOC_SYNC_ENTRIES (e.g. num_slots <= 1364 at HK = 16); larger
 * caches get GDN_EUNSUPPORTED, with nothing enqueued, and must use
 * gdn_replay_rollback_verify_flush with a counter buffer of their own.
 * The array (GDN_REPLAY_NOALLOC_SYNC_ENTRIES int32, 256 KiB) exists once per
 * GPU the library runs on and stays until the process ends; the first call on
 * a device looks up its address (call with the stream's device current). Every
 * call on a GPU shares that GPU's array: calls that overlap in time on one GPU
 * (on other streams or threads) race on it and must not be issued. The
 * counters are zero at load and every completed call leaves them zero. Nothing
 * is allocated, by the library or on its behalf, in any call.
 */
#define GDN_REPLAY_NOALLOC_SYNC_ENTRIES 65536
int gdn_replay_rollback_verify_flush_noalloc(const gdn_replay_cache *c, int32_t num_reqs,
                                             const int32_t *slot_idx, const int32_t *num_accepted,
                                             const int32_t *prev_draft_lens, int32_t prev_draft,
                                             const int32_t *draft_lens, int32_t draft_len,
                                             int32_t min_len, const void *q, const void *k,
                                             const void *v, const float *alpha, const float *beta,
                                             float *out, hipStream_t stream);

/* Human-readable text of a gdn_status (static storage). */
const char *gdn_replay_strerror(int status);

/* Number of int32 entries of gdn_replay_cache::sync for num_slots slots and
 * num_k_heads key heads (0 for a negative argument). */
int64_t gdn_replay_sync_entries(int32_t num_slots, int32_t num_k_heads);

/* GDN_REPLAY_VERSION of the built library. */
int gdn_replay_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_REPLAY_H */
