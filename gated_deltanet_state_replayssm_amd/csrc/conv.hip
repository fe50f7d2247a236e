// Short causal convolution of GDN layers (depthwise, width K, silu) for a draft
// block, with its input history in a ring that shares the recurrence's head/len.
//
// "The inference stack behind OCRia" (LlamaIndex): GDN layers convolve the q, k,
// v projections causally before the recurrence, and under speculation the
// section "Making speculative verification cheaper" keeps state in buffers
// whose pointer moves on rejection. The convolution's state is the last K - 1
// inputs of the committed stream; they sit in the ring at
// (head + len - K + 1 + m) mod C, the draft is appended at (head + len + j) mod C
// (where the recurrence appends its rows), so a rollback (len += a) and a flush
// (head += len) need no work here. When the previous draft's rollback is still
// to come (it is folded into the one-call step that runs after this kernel),
// len + a of that rollback stands for len.
//
// One thread per pair of channels of a group of draft tokens of one request
// (coalesced rows: consecutive threads take consecutive channels). fp32
// arithmetic, bf16 in and out (round to nearest even). Memory-bound: per
// channel and draft token 2 bytes read from HBM and 4 written, plus the K - 1
// history tokens read.
#include "device_common.h"
#include "internal.h"

namespace gdnr {

namespace {

constexpr int kMaxWidth = kMaxConvWidth;

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// grid (ceil(channels / 2 / 256), ceil(D / kTok), num_reqs), block 256: one
// thread per (request, group of kTok draft tokens, channel pair). A thread loads
// its two channels' weights once, gathers the K - 1 + kTok inputs of its group's
// windows (earlier draft rows, or the ring for the committed ones before the
// draft) with the loads issued together, then writes kTok outputs and appends
// its kTok inputs. The K - 1 rows before a group are read by two groups (the
// repeats are served by L2); the ring positions read (before the draft) never
// meet those written (D + K - 1 <= C). Groups of 4 tokens: measured against 2,
// 8 and 16 (and against 2 or 4 channel pairs per thread), the most threads in
// flight for the fewest repeated history reads.
constexpr int kTok = 4;

template <int K>
__global__ __launch_bounds__(256) void causal_conv_update_kernel(ConvArgs a) {
  const int r = blockIdx.z, j0 = blockIdx.y * kTok;
  const int cp = blockIdx.x * 256 + threadIdx.x;  // channel pair
  const int CH = a.channels;
  const bool lead = blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0;
  const CacheView &c = a.c;
  const int s = a.slot_idx[r];
  if (s < 0 || s >= c.num_slots) {
    if (lead) raise_err(c.err, GDN_DERR_SLOT);
    return;
  }
  const int C = c.cap;
  const int head = c.head[s], n0 = c.len[s];
  if (head < 0 || head >= C || n0 < 0 || n0 > C) {
    if (lead) raise_err(c.err, GDN_DERR_POINTER);
    return;
  }
  // The committed count the step that follows works from: with the previous
  // draft's rollback still pending (folded into the one-call step), len + a
  // under that step's checks (a failed rollback keeps len; the step flags it).
  int n = n0;
  if (a.prev_accepted) {
    int bad;
    const int bound = a.prev_draft_lens ? a.prev_draft_lens[r] : a.prev_draft;
    n = rolled_from(n0, a.prev_accepted[r], bound, a.prev_draft, C, &bad);
  }
  // D + K - 1 <= C (host-checked): the draft never reaches the history it
  // reads; committed inputs older than that are never read again, so len + D
  // may exceed C here (a verify_flush later in the step folds those slots).
  const int D = a.draft;
  const int CP = CH / 2;
  if (cp >= CP) return;
  const int c0 = 2 * cp;

  float w0[K], w1[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    w0[i] = a.weight[(int64_t)c0 * K + i];
    w1[i] = a.weight[(int64_t)(c0 + 1) * K + i];
  }
  const float b0 = a.bias ? a.bias[c0] : 0.f, b1 = a.bias ? a.bias[c0 + 1] : 0.f;

  const uint32_t *xin = static_cast<const uint32_t *>(a.x);
  uint32_t *ring = static_cast<uint32_t *>(a.ring);  // bf16 pairs
  const int64_t slot_row0 = (int64_t)s * C;
  const int64_t xrow0 = (int64_t)r * D;
  // inputs of tokens j0 - K + 1 .. j0 + kTok - 1 (past the draft: unused zeros)
  uint32_t v[K - 1 + kTok];
#pragma unroll
  for (int u = 0; u < K - 1 + kTok; ++u) {
    const int t = j0 - (K - 1) + u;
    if (t >= D) {
      v[u] = 0u;
    } else if (t >= 0) {
      v[u] = xin[(xrow0 + t) * CP + cp];
    } else {
      int pos = head + n + t;  // in [-(K - 1), 2 C), and K - 1 < C
      pos += pos < 0 ? C : 0;
      pos -= pos >= C ? C : 0;
      v[u] = ring[(slot_row0 + pos) * CP + cp];
    }
  }
  uint32_t *yout = static_cast<uint32_t *>(a.y);
#pragma unroll
  for (int q = 0; q < kTok; ++q) {
    const int j = j0 + q;
    if (j >= D) break;
    float acc0 = b0, acc1 = b1;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      acc0 = fmaf(w0[i], __uint_as_float(v[q + i] << 16), acc0);
      acc1 = fmaf(w1[i], __uint_as_float(v[q + i] & 0xffff0000u), acc1);
    }
    const float y0 = acc0 / (1.f + __expf(-acc0));
    const float y1 = acc1 / (1.f + __expf(-acc1));
    yout[(xrow0 + j) * CP + cp] = bf16_rne(y0) | (bf16_rne(y1) << 16);
    // head < C, len <= C and j < D <= C: head + len + j < 3 C
    ring[(slot_row0 + (head + n + j) % C) * CP + cp] = v[q + K - 1];
  }
}

template <int K>
hipError_t launch_k(const ConvArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.channels / 2 + 255) / 256), (unsigned)((a.draft + kTok - 1) / kTok),
                  (unsigned)a.num_reqs);
  hipLaunchKernelGGL(causal_conv_update_kernel<K>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_causal_conv_update(const ConvArgs &a, int width, hipStream_t stream) {
  switch (width) {
    case 1: return launch_k<1>(a, stream);
    case 2: return launch_k<2>(a, stream);
    case 3: return launch_k<3>(a, stream);
    case 4: return launch_k<4>(a, stream);
    case 5: return launch_k<5>(a, stream);
    case 6: return launch_k<6>(a, stream);
    case 7: return launch_k<7>(a, stream);
    case 8: return launch_k<8>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdnr
