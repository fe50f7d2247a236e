// Chunked (WY / UT form) replay kernels for gfx950: verify and flush.
//
// Math (gated delta rule, Yang et al., "Gated Delta Networks", 2025; per value
// head, S is d_v x d_k, stored as H = S^T). For a chunk of T tokens replayed
// from a state S_0, with gamma_t = alpha_0 ... alpha_t (chunk-local) and
// L[t][i] = alpha_{i+1} ... alpha_t (i <= t):
//     Y = K S_0^T,  X_t = beta_t (v_t - gamma_t Y_t),
//     A_ti = beta_t L[t][i] (k_t . k_i) for i < t,   W = (I + A)^-1 X,
//     S_T = gamma_{T-1} S_0 + sum_t L[T-1][t] w_t k_t^T              (fold)
//     o_t = gamma_t S_0 q_t + sum_{i<=t} L[t][i] (q_t . k_i) w_i      (outputs)
// so the only contractions with the d_k x d_v state are K H, Q H and the
// rank-T update K^T W'. Those run on MFMA (v_mfma_f32_16x16x32_bf16): k and q
// are bf16 inputs (exact operands) and every fp32 operand (state, X, W, the
// T x T matrices) is split into hi + lo bf16 halves, so the products keep
// ~2^-16 relative accuracy with fp32 accumulation. The T x T work (decay
// table, Gram matrices, unit-lower-triangular inverse) is tiny and runs on VALU.
//
// ReplaySSM ("The inference stack behind OCRia", section "Making speculative
// verification cheaper"): verify replays checkpoint + committed ring tokens +
// draft and never writes the state; flush folds the committed tokens into the
// checkpoint. Tokens are processed in chunks of 32; every chunk but verify's
// last is folded into the on-chip state.
//
// Layout: one workgroup per (request, value head); wave w owns 16*NT state
// columns. Lane l (g = l / 16, l16 = l % 16) holds, for every 16-row tile mt
// of the state and every column tile nt, the entries
//     H[16 mt + 4 g + i][c0 + NT l16 + nt],  i = 0..3,
// i.e. the MFMA 16x16 accumulator layout of column tile nt, with the NT
// columns of a row contiguous (one NT-float global load or store per row). Because an MFMA
// operand may use any k-order that A and B share, the same registers are the
// B operand of K H: k-step s takes rows 32 s + 4 g + {0..3} and
// 32 s + 16 + 4 g + {0..3}, and the key rows are read from LDS in that order.
// Token-indexed accumulators (Y, W) chain the same way into the next product.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace gdnr {

namespace {

constexpr int kCh = 32;    // tokens per chunk
constexpr int kPadK = 8;   // bf16 padding per token row of K / Q in LDS
constexpr int kPadT = 8;   // bf16 padding per row of K^T
constexpr int kPadF = 4;   // fp32 padding per row of the 32 x 32 matrices

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in fp32)
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)x[j];
    hi[j] = h;
    lo[j] = (__bf16)(x[j] - (float)h);
  }
}

// Same split with hi = x truncated to bf16 (|x - hi| < 2^-7 |x|, lo keeps the
// pair within ~2^-16 |x|). Used for a second pass over the state so that its
// split is not shared with (and kept alive from) the first pass.
__device__ __forceinline__ void split8_trunc(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t b = __float_as_uint(x[j]) & 0xffff0000u;
    hi[j] = __builtin_bit_cast(__bf16, (uint16_t)(b >> 16));
    lo[j] = (__bf16)(x[j] - __uint_as_float(b));
  }
}

// the NT consecutive state columns of one lane: fp32 values and bf16 bits
template <int N>
struct Cols {
  typedef float F __attribute__((ext_vector_type(N)));
  typedef uint16_t U __attribute__((ext_vector_type(N)));
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int DK, int DV>
struct Smem {
  uint16_t k[kCh][DK + kPadK];     // chunk keys, token-major (bf16 bits)
  union {
    uint16_t q[kCh][DK + kPadK];   // output chunk: queries (draft rows, zero elsewhere)
    uint16_t kt[DK][kCh + kPadT];  // folded chunk: keys, transposed
  };
  uint16_t v[kCh][DV + kPadK];     // chunk values, token-major (bf16 bits)
  float T[kCh][kCh + kPadF];       // A = beta_t L[t][i] (k_t . k_i) (strictly lower),
                                   // then (I + A)^-1 in place
  float Cm[kCh][kCh + kPadF];      // L[t][i] (q_t . k_i), lower incl. diagonal
  float gam[kCh], bet[kCh], alp[kCh];
  float lg[kCh];                   // log2(alpha_0 ... alpha_t), each log clamped at -126
  float lgc[kCh];                  // the same, from the scan of the wave that builds Cm
};

// 8 bf16 of a token row in k-step s order: columns 32s+4g+{0..3}, 32s+16+4g+{0..3}
template <int W>
__device__ __forceinline__ bf16x8 rd_row(const uint16_t (*m)[W], int row, int col0) {
  const uint16_t *p = &m[row][col0];
  const uint2 a = *reinterpret_cast<const uint2 *>(p);
  const uint2 b = *reinterpret_cast<const uint2 *>(p + 16);
  const uint4 v = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, v);
}

// 8 fp32 of a 32 x 32 matrix row in token-slot order: 4g+{0..3}, 16+4g+{0..3}
__device__ __forceinline__ void rd_frow(const float (*m)[kCh + kPadF], int row, int g,
                                        float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(&m[row][4 * g]);
  const float4 b = *reinterpret_cast<const float4 *>(&m[row][16 + 4 * g]);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// B operand of a token-indexed accumulator pair (rows 4g+i and 16+4g+i)
__device__ __forceinline__ void tok_operand(const f32x4 &m0, const f32x4 &m1, bf16x8 &hi,
                                            bf16x8 &lo) {
  const float x[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
  split8(x, hi, lo);
}

// Value head of the j-th workgroup of a request's HV consecutive workgroups.
// Workgroups are dealt to the 8 XCDs in turn (block b on XCD b mod 8), and the G
// value heads of a key head read the same key and query rows: when HV is a
// multiple of 8 G they take positions 8 apart, so that they run on one XCD and
// share its L2 (j = 8 (G a + b) + x -> key head 8 a + x, value head G kh + b).
__device__ __forceinline__ int head_of(int j, int HV, int G) {
  if (HV % (8 * G) != 0) return j;
  const int x = j & 7, m = j >> 3, a = m / G, b = m - a * G;
  return G * (8 * a + x) + b;
}

struct Unit {
  int r, h, s, kh, head, B, T, C;
};

// Raw buffer accesses: a uniform resource (base address and size in bytes)
// plus a 32-bit per-lane byte offset. An offset at or past the size reads as
// zero and drops a store, which the staging uses for rows that a resource does
// not hold (ring vs draft rows, chunk padding) instead of branches or selects
// of 64-bit addresses.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource's end
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) 32-bit data, as every gfx9 buffer access
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Cache policy bits of an access (gfx950: sc0 = 1, nt = 2, sc1 = 16).
// kStream: data read once (the state tile, the draft).
// kWriteOut: data written once and not read again by this kernel (outputs, ring
// appends, the folded state). Plain write-back stores leave these lines dirty
// in the XCD's L2, where the end-of-kernel release writes them back after all
// the loads; written through, they reach memory while the loads still stream.
constexpr int kStream = 2;
constexpr int kWriteOut = 19;

template <typename T, int AUX = 0>
__device__ __forceinline__ T bload(Rsrc r, uint32_t voff, uint32_t soff = 0) {
  if constexpr (sizeof(T) == 4)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
  else if constexpr (sizeof(T) == 8)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX));
  else
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}

template <typename T, int AUX = kWriteOut>
__device__ __forceinline__ void bstore(const T &v, Rsrc r, uint32_t voff, uint32_t soff = 0) {
  if constexpr (sizeof(T) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, voff, soff, AUX);
  else if constexpr (sizeof(T) == 4)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, AUX);
  else if constexpr (sizeof(T) == 8)
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, soff, AUX);
  else
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, AUX);
}

// One row from the ring or from the draft: a divergent pair of loads into one
// destination (rows in neither read as zero through the draft resource). The
// draft is read once, non-temporally; the differing policy bits also keep the
// compiler from merging the two loads into one with a per-lane resource.
template <typename T>
__device__ __forceinline__ T bload_rd(bool in_ring, Rsrc ring, uint32_t roff, Rsrc draft,
                                      uint32_t doff) {
  T x;
  if (in_ring)
    x = bload<T, 0>(ring, roff);
  else
    x = bload<T, kStream>(draft, doff);
  return x;
}

template <typename T>
__device__ __forceinline__ T bits_or(const T &a, const T &b) {
  if constexpr (sizeof(T) == 4)
    return __builtin_bit_cast(T, __builtin_bit_cast(uint32_t, a) | __builtin_bit_cast(uint32_t, b));
  else if constexpr (sizeof(T) == 8)
    return __builtin_bit_cast(T, __builtin_bit_cast(u32x2, a) | __builtin_bit_cast(u32x2, b));
  else
    return __builtin_bit_cast(T, __builtin_bit_cast(u32x4, a) | __builtin_bit_cast(u32x4, b));
}

// The d_k x d_v state tile of one (slot, value head): lane (g, l16) of wave w
// holds rows 16 mt + 4 g + i, columns colL .. colL + NT - 1 (colL = 16 NT w +
// NT l16). voff = byte offset of row 4 g, column colL; the 16-row step goes in
// the scalar offset and the row step i in the instruction's immediate.
template <int DK, int DV, int NT>
__device__ __forceinline__ void load_state(Rsrc st, uint32_t voff,
                                           typename Cols<NT>::F (&H)[DK / 16][4]) {
  typedef typename Cols<NT>::F F;
#pragma unroll
  for (int mt = 0; mt < DK / 16; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) H[mt][i] = bload<F, kStream>(st, voff + i * DV * 4, mt * 16 * DV * 4);
}
template <int DK, int DV, int NT>
__device__ __forceinline__ void store_state(Rsrc st, uint32_t voff,
                                            const typename Cols<NT>::F (&H)[DK / 16][4]) {
#pragma unroll
  for (int mt = 0; mt < DK / 16; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) bstore(H[mt][i], st, voff + i * DV * 4, mt * 16 * DV * 4);
}

// Per-workgroup resources of everything a chunk reads or appends: the ring rows
// of this (slot, key head) and (slot, value head), the draft rows of this
// (request, key head) and (request, value head) with their row strides.
struct Srcs {
  Rsrc rk, rq, rv, ra, rb;  // ring k / q / v / alpha / beta (rq: appended only, may be empty)
  Rsrc dk, dq, dv, da, db;  // draft k / q / v / alpha / beta
  uint32_t dk_row, dv_row, dab_row;  // draft row strides in bytes
};

template <int DK, int DV>
__device__ __forceinline__ Srcs make_srcs(const CacheView &c, const Unit &u, const VerifyArgs *va,
                                          bool verify) {
  const int C = u.C, HV = c.hv, HK = c.hk;
  const int64_t kq_row0 = (int64_t)(u.s * HK + u.kh) * C;
  const int64_t vh_row0 = (int64_t)(u.s * HV + u.h) * C;
  Srcs b;
  b.rk = make_rsrc(static_cast<uint16_t *>(c.ring_k) + kq_row0 * DK, C * DK * 2);
  b.rq = c.ring_q ? make_rsrc(static_cast<uint16_t *>(c.ring_q) + kq_row0 * DK, C * DK * 2)
                  : make_rsrc(nullptr, 0);
  b.rv = make_rsrc(static_cast<uint16_t *>(c.ring_v) + vh_row0 * DV, C * DV * 2);
  b.ra = make_rsrc(c.ring_alpha + vh_row0, C * 4);
  b.rb = make_rsrc(c.ring_beta + vh_row0, C * 4);
  b.dk_row = HK * DK * 2;
  b.dv_row = HV * DV * 2;
  b.dab_row = HV * 4;
  if (verify) {
    // this request's draft length; rows are va->draft apart. A fused verify of a
    // due slot without a draft stages zero rows: resources of one row then.
    const int D = max(u.T - u.B, 1);
    const int64_t d0 = (int64_t)u.r * va->draft;
    const uint32_t kq_bytes = (D - 1) * b.dk_row + DK * 2;
    b.dk = make_rsrc(static_cast<const uint16_t *>(va->k) + (d0 * HK + u.kh) * DK, kq_bytes);
    b.dq = make_rsrc(static_cast<const uint16_t *>(va->q) + (d0 * HK + u.kh) * DK, kq_bytes);
    b.dv = make_rsrc(static_cast<const uint16_t *>(va->v) + (d0 * HV + u.h) * DV,
                     (D - 1) * b.dv_row + DV * 2);
    b.da = make_rsrc(va->alpha + d0 * HV + u.h, (D - 1) * b.dab_row + 4);
    b.db = make_rsrc(va->beta + d0 * HV + u.h, (D - 1) * b.dab_row + 4);
  } else {
    b.dk = b.dq = b.dv = b.da = b.db = make_rsrc(nullptr, 0);
  }
  return b;
}

// The thread index through an empty volatile asm: values derived from it are
// recomputed after each call instead of being hoisted out of loops and held in
// registers (the chunk loop's body is register-bound).
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Where chunk row t (token t0 + t of the stream: B committed ring tokens, then
// the draft when verifying) lives: its ring slot (head + token) mod C and its
// draft index. Byte offsets for rows of the given sizes; kOOB where absent.
template <bool VERIFY>
struct RowAt {
  uint32_t ring, draft, append;  // ring read, draft read, ring append (draft rows)
  __device__ __forceinline__ RowAt(const Unit &u, int t0, int t, int Treal, uint32_t ring_row,
                                   uint32_t draft_row) {
    const int tok = t0 + t;
    const bool real = t < Treal;
    const bool in_ring = !VERIFY || tok < u.B;
    int pos = u.head + tok;
    pos -= pos >= u.C ? u.C : 0;  // head < C and tok < C for real rows
    const uint32_t at = (uint32_t)pos * ring_row;
    ring = (real && in_ring) ? at : kOOB;
    append = (real && !in_ring) ? at : kOOB;
    draft = (real && !in_ring) ? (uint32_t)(tok - u.B) * draft_row : kOOB;
  }
};

// Chunk rows [t0, t0 + Treal) of the token stream. load() issues the loads of
// k (and q), v, alpha and beta into registers; store() writes them to LDS rows
// 0 .. 31 (rows past Treal read as zero). The output chunk (verify's last, which
// holds the whole draft) stages the queries; a folded chunk stages the
// transposed keys instead. append() copies the draft rows from LDS into the
// ring once the chunk is done.
template <int DK, int DV, int NT, bool VERIFY, int STAGERS = 64 * (DV / (16 * NT))>
struct Stage {
  static constexpr int THREADS = STAGERS;
  static constexpr int PK = DK / 8, PV = DV / 8;  // 16-byte pieces per k / v row
  static constexpr int IK = kCh * PK / THREADS, IV = kCh * PV / THREADS;
  static_assert(kCh * PK % THREADS == 0 && kCh * PV % THREADS == 0, "pieces per thread");

  u32x4 kv[IK], qv[IK], vv[IV];
  float al, be;

  __device__ __forceinline__ void load(const Srcs &sr, const Unit &u, int t0, int Treal,
                                       bool out_chunk) {
    const int tid = opaque_tid();
#pragma unroll
    for (int it = 0; it < IK; ++it) {
      const int p = tid + it * THREADS, t = p / PK, part = p % PK;
      const RowAt<VERIFY> at(u, t0, t, Treal, DK * 2, sr.dk_row);
      if constexpr (VERIFY) {
        kv[it] = bload_rd<u32x4>(at.ring != kOOB, sr.rk, at.ring + part * 16, sr.dk,
                                 at.draft + part * 16);
        // queries of committed rows are never read: those rows stay zero
        if (out_chunk) qv[it] = bload<u32x4, kStream>(sr.dq, at.draft + part * 16);
      } else {
        kv[it] = bload<u32x4>(sr.rk, at.ring + part * 16);
      }
    }
#pragma unroll
    for (int it = 0; it < IV; ++it) {
      const int p = tid + it * THREADS, t = p / PV, part = p % PV;
      const RowAt<VERIFY> at(u, t0, t, Treal, DV * 2, sr.dv_row);
      if constexpr (VERIFY)
        vv[it] = bload_rd<u32x4>(at.ring != kOOB, sr.rv, at.ring + part * 16, sr.dv,
                                 at.draft + part * 16);
      else
        vv[it] = bload<u32x4>(sr.rv, at.ring + part * 16);
    }
    const int t = tid & (kCh - 1);
    const RowAt<VERIFY> at(u, t0, t, Treal, 4, sr.dab_row);
    if constexpr (VERIFY) {
      al = bload_rd<float>(at.ring != kOOB, sr.ra, at.ring, sr.da, at.draft);
      be = bload_rd<float>(at.ring != kOOB, sr.rb, at.ring, sr.db, at.draft);
    } else {
      al = bload<float>(sr.ra, at.ring);
      be = bload<float>(sr.rb, at.ring);
    }
  }

  __device__ __forceinline__ void store(Smem<DK, DV> &sm, int Treal, bool out_chunk) {
    const int tid = opaque_tid();
#pragma unroll
    for (int it = 0; it < IK; ++it) {
      const int p = tid + it * THREADS, t = p / PK, part = p % PK;
      const u32x4 k = kv[it];
      *reinterpret_cast<u32x4 *>(&sm.k[t][part * 8]) = k;
      if (out_chunk) {
        *reinterpret_cast<u32x4 *>(&sm.q[t][part * 8]) = qv[it];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.kt[part * 8 + 2 * e][t] = (uint16_t)(k[e] & 0xffffu);
          sm.kt[part * 8 + 2 * e + 1][t] = (uint16_t)(k[e] >> 16);
        }
      }
    }
#pragma unroll
    for (int it = 0; it < IV; ++it) {
      const int p = tid + it * THREADS, t = p / PV, part = p % PV;
      *reinterpret_cast<u32x4 *>(&sm.v[t][part * 8]) = vv[it];
    }
    if ((tid & (kCh - 1)) >= Treal) al = 1.f;  // padding rows: alpha = 1, beta = 0 (read as 0)
    if (tid < kCh) {
      sm.alp[tid] = al;
      sm.bet[tid] = be;
    }
  }

  // Verify's output chunk: write the draft rows to ring slots (head + B + j) mod C,
  // from LDS (one workgroup per key head writes k and q).
  __device__ __forceinline__ void append(const Smem<DK, DV> &sm, const Srcs &sr, const Unit &u,
                                         int t0, int Treal, bool kq_writer) const {
    const int tid = opaque_tid();
    // Recompute the row offsets here rather than keep those of the loads alive
    // in registers through the whole kernel: the copy of the unit is opaque to
    // the compiler, so it cannot reuse them.
    Unit u2 = u;
    asm volatile("" : "+v"(u2.head));
    if (kq_writer) {
#pragma unroll
      for (int it = 0; it < IK; ++it) {
        const int p = tid + it * THREADS, t = p / PK, part = p % PK;
        const RowAt<VERIFY> at(u2, t0, t, Treal, DK * 2, sr.dk_row);
        bstore(*reinterpret_cast<const u32x4 *>(&sm.k[t][part * 8]), sr.rk, at.append + part * 16);
        bstore(*reinterpret_cast<const u32x4 *>(&sm.q[t][part * 8]), sr.rq, at.append + part * 16);
      }
    }
#pragma unroll
    for (int it = 0; it < IV; ++it) {
      const int p = tid + it * THREADS, t = p / PV, part = p % PV;
      const RowAt<VERIFY> at(u2, t0, t, Treal, DV * 2, sr.dv_row);
      bstore(*reinterpret_cast<const u32x4 *>(&sm.v[t][part * 8]), sr.rv, at.append + part * 16);
    }
    if (tid < kCh) {
      const RowAt<VERIFY> at(u2, t0, tid, Treal, 4, sr.dab_row);
      bstore(sm.alp[tid], sr.ra, at.append);
      bstore(sm.bet[tid], sr.rb, at.append);
    }
  }
};

// Inclusive scan over lanes 0..31 of a wave with DPP row shifts (within rows of
// 16 lanes) and a row broadcast of lane 15 into the second row. Lanes 32..63 get
// their own scan of lanes 32..63.
__device__ __forceinline__ float scan32_add(float v) {
  v += dpp_or<0x111, 0xf>(0.f, v);  // row_shr:1
  v += dpp_or<0x112, 0xf>(0.f, v);  // row_shr:2
  v += dpp_or<0x114, 0xf>(0.f, v);  // row_shr:4
  v += dpp_or<0x118, 0xf>(0.f, v);  // row_shr:8
  v += dpp_or<0x142, 0xa>(0.f, v);  // row_bcast:15 into rows 1 and 3
  return v;
}
__device__ __forceinline__ float scan32_mul(float v) {
  v *= dpp_or<0x111, 0xf>(1.f, v);
  v *= dpp_or<0x112, 0xf>(1.f, v);
  v *= dpp_or<0x114, 0xf>(1.f, v);
  v *= dpp_or<0x118, 0xf>(1.f, v);
  v *= dpp_or<0x142, 0xa>(1.f, v);
  return v;
}

// Decays of the chunk from this lane's staged alpha (token lane % 32):
// gamma_t = alpha_0 ... alpha_t (product scan) and lg_t = log2 gamma_t (sum scan
// of log2 alpha, each clamped at -126 so that a zero alpha stays finite), so
// that L[t][j] = alpha_{j+1} ... alpha_t = 2^(lg_t - lg_j).
struct Decay {
  float lg, gm;
};
__device__ __forceinline__ Decay chunk_decay(float al_staged) {
  Decay d;
  d.lg = scan32_add(fmaxf(__log2f(al_staged), -126.f));
  d.gm = scan32_mul(al_staged);
  return d;
}

// 16 x 16 tiles (0,0), (1,0), (1,1) of a Gram matrix P Q^T of two 32-token row
// blocks in LDS (exact bf16 products, fp32 sums); tile b holds rows
// 16 ta + 4 g + i, column 16 tb + l16. One k-step's operands are live at a time.
template <int DK, int W>
__device__ __forceinline__ void gram3(const uint16_t (*p)[W], const uint16_t (*q)[W], int g,
                                      int l16, f32x4 (&G)[3]) {
#pragma unroll
  for (int b = 0; b < 3; ++b) G[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DK / 32; ++ks) {
    const bf16x8 p0 = rd_row(p, l16, 32 * ks + 4 * g), p1 = rd_row(p, 16 + l16, 32 * ks + 4 * g);
    const bf16x8 q0 = p == q ? p0 : rd_row(q, l16, 32 * ks + 4 * g);
    const bf16x8 q1 = p == q ? p1 : rd_row(q, 16 + l16, 32 * ks + 4 * g);
    G[0] = mfma(q0, p0, G[0]);
    G[1] = mfma(q1, p0, G[1]);
    G[2] = mfma(q1, p1, G[2]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// L[t][j] for the three tiles of gram3, zero above the diagonal
__device__ __forceinline__ void decay_tiles(const float *lg, int g, int l16, float (&Lv)[3][4]) {
  float lgv[2][4], lgc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    lgc[a] = lg[16 * a + l16];
#pragma unroll
    for (int i = 0; i < 4; ++i) lgv[a][i] = lg[16 * a + 4 * g + i];
  }
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ta = b == 0 ? 0 : 1, tb = b == 2 ? 1 : 0;
      const int t = 16 * ta + 4 * g + i, j = 16 * tb + l16;
      Lv[b][i] = (j <= t) ? exp2f(lgv[ta][i] - lgc[tb]) : 0.f;
    }
}

// C = L o (Q K^T), lower triangle including the diagonal (output chunk only).
// Built by another wave than A and its inverse, from its own decay scan (kept
// in sm.lgc), so the two run side by side; it writes only sm.Cm and sm.lgc.
template <int DK, int DV>
__device__ __forceinline__ void build_c(Smem<DK, DV> &sm, float al_staged, int lane, int g, int l16) {
  // issue priority meanwhile, as build_tt
  __builtin_amdgcn_s_setprio(3);
  {
    const Decay d = chunk_decay(al_staged);
    if (lane < kCh) sm.lgc[lane] = d.lg;
  }
  f32x4 Pm[3];
  gram3<DK>(sm.k, sm.q, g, l16, Pm);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  float Lv[3][4];
  decay_tiles(sm.lgc, g, l16, Lv);
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ta = (b == 1 || b == 2) ? 1 : 0, tb = b >= 2 ? 1 : 0;
      const int t = 16 * ta + 4 * g + i, j = 16 * tb + l16;
      float c = 0.f;
      if (b < 3) c = Lv[b < 3 ? b : 0][i] * Pm[b < 3 ? b : 0][i];
      sm.Cm[t][j] = c;
    }
  __builtin_amdgcn_s_setprio(0);
}

// A = beta L o (K K^T) strictly lower, then (I + A)^-1 in sm.T, plus the decay vectors
// gamma and lg, built by one wave (no workgroup barriers inside: each step reads
// only what this wave wrote, in program order). al_staged is this lane's staged
// alpha, of token lane % 32.
template <int DK, int DV>
__device__ __forceinline__ void build_tt(Smem<DK, DV> &sm, float al_staged, int lane, int g, int l16) {
  // The T x T matrices are one wave's work on every workgroup's critical path;
  // the wave takes issue priority over the other waves of its SIMD meanwhile.
  __builtin_amdgcn_s_setprio(3);
  {
    const Decay d = chunk_decay(al_staged);
    if (lane < kCh) {
      sm.lg[lane] = d.lg;
      sm.gam[lane] = d.gm;
    }
  }
  f32x4 Gm[3];
  gram3<DK>(sm.k, sm.k, g, l16, Gm);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  {
    float Lv[3][4], bv[2][4];
    decay_tiles(sm.lg, g, l16, Lv);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[a][i] = sm.bet[16 * a + 4 * g + i];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ta = (b == 1 || b == 2) ? 1 : 0, tb = b >= 2 ? 1 : 0;
        const int t = 16 * ta + 4 * g + i, j = 16 * tb + l16;
        float v = 0.f;
        if (b < 3 && j < t) v = bv[ta][i] * Lv[b < 3 ? b : 0][i] * Gm[b < 3 ? b : 0][i];
        sm.T[t][j] = v;
      }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // ---- (I + A)^-1 in place, by recursive 2 x 2 blocking: T = [[T00, 0], [T10, T11]]
  // with T10 = -T11 (A10 T00). 4 x 4 diagonal blocks by forward substitution, then
  // 8 x 8 and 16 x 16 blocks on VALU, then the 32 x 32 level on MFMA. Each level
  // overwrites the A10 block it has read with T10; the A10 T00 products of the
  // VALU levels go to the (zero) upper-right block, which is cleared after use.
  // Every step reads everything it needs before it writes (one wave, LDS
  // accesses in program order).
  {
    // 4 x 4 diagonal blocks q = 0..7: lane = (q, column cc)
    const int q = (lane >> 2) & 7, cc = lane & 3, r0 = 4 * q;
    const float a10 = sm.T[r0 + 1][r0], a20 = sm.T[r0 + 2][r0], a21 = sm.T[r0 + 2][r0 + 1];
    const float a30 = sm.T[r0 + 3][r0], a31 = sm.T[r0 + 3][r0 + 1], a32 = sm.T[r0 + 3][r0 + 2];
    const float x0 = cc == 0 ? 1.f : 0.f;
    const float x1 = cc == 1 ? 1.f : (cc < 1 ? -a10 * x0 : 0.f);
    const float x2 = cc == 2 ? 1.f : (cc < 2 ? -(a20 * x0 + a21 * x1) : 0.f);
    const float x3 = cc == 3 ? 1.f : -(a30 * x0 + a31 * x1 + a32 * x2);
    if (lane < 32) {
      sm.T[r0][r0 + cc] = x0;
      sm.T[r0 + 1][r0 + cc] = x1;
      sm.T[r0 + 2][r0 + cc] = x2;
      sm.T[r0 + 3][r0 + cc] = x3;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  {
    // 8 x 8 blocks p = 0..3: lane = (p, i, j) over the 4 x 4 lower-left block
    const int p = lane >> 4, i = (lane >> 2) & 3, j = lane & 3, r0 = 8 * p;
    float av[4], tv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      av[k] = sm.T[r0 + 4 + i][r0 + k];
      tv[k] = sm.T[r0 + k][r0 + j];
    }
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = fmaf(av[k], tv[k], m);
    sm.T[r0 + i][r0 + 4 + j] = m;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    float t11[4], mv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      t11[k] = sm.T[r0 + 4 + i][r0 + 4 + k];
      mv[k] = sm.T[r0 + k][r0 + 4 + j];
    }
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) t = fmaf(t11[k], mv[k], t);
    sm.T[r0 + 4 + i][r0 + j] = -t;
    sm.T[r0 + i][r0 + 4 + j] = 0.f;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  {
    // 16 x 16 blocks b = 0, 1: lane = (b, i, j0) over the 8 x 8 lower-left block,
    // two columns j0 and j0 + 4 per lane
    const int b = lane >> 5, i = (lane >> 2) & 7, j0 = lane & 3, r0 = 16 * b;
    float av[8], tv[2][8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      av[k] = sm.T[r0 + 8 + i][r0 + k];
      tv[0][k] = sm.T[r0 + k][r0 + j0];
      tv[1][k] = sm.T[r0 + k][r0 + j0 + 4];
    }
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      m0 = fmaf(av[k], tv[0][k], m0);
      m1 = fmaf(av[k], tv[1][k], m1);
    }
    sm.T[r0 + i][r0 + 8 + j0] = m0;
    sm.T[r0 + i][r0 + 12 + j0] = m1;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    float t11[8], mv[2][8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      t11[k] = sm.T[r0 + 8 + i][r0 + 8 + k];
      mv[0][k] = sm.T[r0 + k][r0 + 8 + j0];
      mv[1][k] = sm.T[r0 + k][r0 + 12 + j0];
    }
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      t0 = fmaf(t11[k], mv[0][k], t0);
      t1 = fmaf(t11[k], mv[1][k], t1);
    }
    sm.T[r0 + 8 + i][r0 + j0] = -t0;
    sm.T[r0 + 8 + i][r0 + j0 + 4] = -t1;
    sm.T[r0 + i][r0 + 8 + j0] = 0.f;
    sm.T[r0 + i][r0 + 12 + j0] = 0.f;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  {
    // 16 x 16 products on MFMA with k = 4g + j (slots 4..7 zero), fp32
    // operands split into hi + lo bf16
    float xa[8], xb[8];
    const float4 arow = *reinterpret_cast<const float4 *>(&sm.T[16 + l16][4 * g]);
    const float4 trow = *reinterpret_cast<const float4 *>(&sm.T[16 + l16][16 + 4 * g]);
    float tcol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tcol[j] = sm.T[4 * g + j][l16];
    xa[0] = arow.x; xa[1] = arow.y; xa[2] = arow.z; xa[3] = arow.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) xb[j] = tcol[j];
#pragma unroll
    for (int j = 4; j < 8; ++j) xa[j] = xb[j] = 0.f;
    bf16x8 ah, al, bh, bl;
    split8(xa, ah, al);
    split8(xb, bh, bl);
    f32x4 M = {0.f, 0.f, 0.f, 0.f};  // A10 T0, rows 4g+i, column l16
    M = mfma(ah, bh, M);
    M = mfma(ah, bl, M);
    M = mfma(al, bh, M);
    xa[0] = trow.x; xa[1] = trow.y; xa[2] = trow.z; xa[3] = trow.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) xb[j] = M[j];
    split8(xa, ah, al);
    split8(xb, bh, bl);
    f32x4 T1 = {0.f, 0.f, 0.f, 0.f};
    T1 = mfma(ah, bh, T1);
    T1 = mfma(ah, bl, T1);
    T1 = mfma(al, bh, T1);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.T[16 + 4 * g + i][l16] = -T1[i];
  }
  
  __builtin_amdgcn_s_setprio(0);
}


enum { kY = 1, kZ = 2 };

// Y = K H and/or Z = Q H over d_k on MFMA, the state split into hi + lo bf16.
// Both products share one split per k-step; a Z-only pass splits with
// truncation so that it is never merged with (and kept alive from) a Y pass.
template <int DK, int DV, int NT, int WHAT>
__device__ __forceinline__ void contract(const Smem<DK, DV> &sm,
                                         const typename Cols<NT>::F (&H)[DK / 16][4], int g,
                                         int l16, f32x4 (&Y)[2][NT], f32x4 (&Z)[2][NT]) {
  constexpr int KS = DK / 32;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Y[a][nt] = Z[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 k0, k1, q0, q1;
    if constexpr ((WHAT & kY) != 0) {
      k0 = rd_row(sm.k, l16, 32 * ks + 4 * g);
      k1 = rd_row(sm.k, 16 + l16, 32 * ks + 4 * g);
    }
    if constexpr ((WHAT & kZ) != 0) {
      q0 = rd_row(sm.q, l16, 32 * ks + 4 * g);
      q1 = rd_row(sm.q, 16 + l16, 32 * ks + 4 * g);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float x[8] = {H[2 * ks][0][nt],     H[2 * ks][1][nt],     H[2 * ks][2][nt],
                          H[2 * ks][3][nt],     H[2 * ks + 1][0][nt], H[2 * ks + 1][1][nt],
                          H[2 * ks + 1][2][nt], H[2 * ks + 1][3][nt]};
      bf16x8 hh, hl;
      if constexpr (WHAT == kZ)
        split8_trunc(x, hh, hl);
      else
        split8(x, hh, hl);
      if constexpr ((WHAT & kY) != 0) {
        Y[0][nt] = mfma(k0, hh, Y[0][nt]);
        Y[0][nt] = mfma(k0, hl, Y[0][nt]);
        Y[1][nt] = mfma(k1, hh, Y[1][nt]);
        Y[1][nt] = mfma(k1, hl, Y[1][nt]);
      }
      if constexpr ((WHAT & kZ) != 0) {
        Z[0][nt] = mfma(q0, hh, Z[0][nt]);
        Z[0][nt] = mfma(q0, hl, Z[0][nt]);
        Z[1][nt] = mfma(q1, hh, Z[1][nt]);
        Z[1][nt] = mfma(q1, hl, Z[1][nt]);
      }
    }
  }
}

// X = beta (V - gamma Y), then W = (I + A)^-1 X (3-pass split product); this
// lane's v entries are rows 16 a + 4 g + i, columns colL .. colL + NT - 1.
template <int DK, int DV, int NT>
__device__ __forceinline__ void solve_w(const Smem<DK, DV> &sm, const f32x4 (&Y)[2][NT], int colL,
                                        int g, int l16, f32x4 (&Wm)[2][NT]) {
  typedef typename Cols<NT>::U U;
  bf16x8 xh[NT], xl[NT];
  {
    float be[2][4], ga[2][4];
    U vv[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        be[a][i] = sm.bet[16 * a + 4 * g + i];
        ga[a][i] = sm.gam[16 * a + 4 * g + i];
        vv[a][i] = *reinterpret_cast<const U *>(&sm.v[16 * a + 4 * g + i][colL]);
      }
    f32x4 X[2][NT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          X[a][nt][i] = be[a][i] * (bf16_to_f32(vv[a][i][nt]) - ga[a][i] * Y[a][nt][i]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tok_operand(X[0][nt], X[1][nt], xh[nt], xl[nt]);
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    float trow[8];
    rd_frow(sm.T, 16 * a + l16, g, trow);
    bf16x8 th, tl;
    split8(trow, th, tl);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma(th, xh[nt], acc);
      acc = mfma(th, xl[nt], acc);
      acc = mfma(tl, xh[nt], acc);
      Wm[a][nt] = acc;
    }
  }
}

// out[r][0..D-1][h][0..DV-1] of one (request, value head), rows HV DV floats apart;
// D >= 1 is the request's draft length (request r's rows start at r * va.draft)
__device__ __forceinline__ Rsrc out_rsrc(const VerifyArgs &va, int r, int h, int DV, int D) {
  const int HV = va.c.hv;
  return make_rsrc(va.out + ((int64_t)r * va.draft * HV + h) * DV, ((D - 1) * HV * DV + DV) * 4);
}

// Draft outputs O = gamma Z + C W of chunk rows t (token t0 + t >= B, t < Treal).
// out holds out[r][0..D-1][h][*] (rows row_bytes apart); col_off = 4 colL.
template <int DK, int DV, int NT>
__device__ __forceinline__ void emit_outputs(const Smem<DK, DV> &sm, const f32x4 (&Z)[2][NT],
                                             const f32x4 (&Wm)[2][NT], int g, int l16, int t0,
                                             int Treal, int B, Rsrc out, uint32_t col_off,
                                             uint32_t row_bytes) {
  typedef typename Cols<NT>::F F;
  asm volatile("" : "+v"(B));  // recompute the row offsets here (see Stage::append)
  bf16x8 wh[NT], wl[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tok_operand(Wm[0][nt], Wm[1][nt], wh[nt], wl[nt]);
  float crow[2][8], ga[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    rd_frow(sm.Cm, 16 * a + l16, g, crow[a]);
#pragma unroll
    for (int i = 0; i < 4; ++i) ga[a][i] = sm.gam[16 * a + 4 * g + i];
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    bf16x8 chh, chl;
    split8(crow[a], chh, chl);
    f32x4 O[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = ga[a][i] * Z[a][nt][i];
      acc = mfma(chh, wh[nt], acc);
      acc = mfma(chh, wl[nt], acc);
      acc = mfma(chl, wh[nt], acc);
      O[nt] = acc;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * a + 4 * g + i;
      const int tok = t0 + t;
      F o;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] = O[nt][i];
      bstore(o, out, (t < Treal && tok >= B) ? (uint32_t)(tok - B) * row_bytes + col_off : kOOB);
    }
  }
}

// The gate and weight a lane needs for the gated RMSNorm + FP8 of its draft
// rows (t = 16 a + 4 g + i, columns col, col + 1), loaded ahead of the outputs.
struct Gate {
  uint32_t z[2][4];  // bf16 pairs (zero for rows that are not draft rows)
  float w[2];
};

// Per-request resources of the norm's gate, codes and scales (rows of request
// r, value head h, at most D rows).
struct NormRsrc {
  Rsrc z, q, scale;
};

__device__ __forceinline__ NormRsrc norm_rsrc(const VerifyArgs &va, int r, int h, int DV, int D) {
  const int HV = va.c.hv;
  const int64_t row0 = (int64_t)r * va.draft * HV + h;  // (row r * draft, head h)
  NormRsrc n;
  n.z = make_rsrc(static_cast<const uint16_t *>(va.norm_z) + row0 * DV,
                  ((D - 1) * HV * DV + DV) * 2);
  n.q = make_rsrc(va.norm_q + row0 * DV, (D - 1) * HV * DV + DV);
  n.scale = make_rsrc(va.norm_scale + row0, ((D - 1) * HV + 1) * 4);
  return n;
}

template <int DV, int NT>
__device__ __forceinline__ Gate load_gate(const VerifyArgs &va, const NormRsrc &nr, int col, int g,
                                          int B, int Treal) {
  static_assert(NT == 2, "a lane's two columns are one bf16 pair");
  Gate gt;
  const uint32_t row_bytes = va.c.hv * DV * 2;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * a + 4 * g + i;
      gt.z[a][i] = bload<uint32_t, kStream>(
          nr.z, (t < Treal && t >= B) ? (uint32_t)(t - B) * row_bytes + col * 2 : kOOB);
    }
  const float2 w = *reinterpret_cast<const float2 *>(va.norm_w + col);
  gt.w[0] = w.x;
  gt.w[1] = w.y;
  return gt;
}

// Sum / maximum over the 16 lanes of a DPP row (lanes 16 g .. 16 g + 15): the
// total ends in the row's last lane.
template <bool MAX>
__device__ __forceinline__ float row16_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  v = op(v, dpp_or<0x111, 0xf>(0.f, v));  // row_shr:1
  v = op(v, dpp_or<0x112, 0xf>(0.f, v));  // row_shr:2
  v = op(v, dpp_or<0x114, 0xf>(0.f, v));  // row_shr:4
  v = op(v, dpp_or<0x118, 0xf>(0.f, v));  // row_shr:8
  return v;
}

// Draft outputs as emit_outputs (stored to out unless its resource is empty),
// then the gated RMSNorm + FP8 of each draft row (token, value head), per
// "The inference stack behind OCRia" (section on fusing kernels: the gated
// RMSNorm and the FP8 quantisation of its result in one kernel), here fused
// with the recurrence that produces the row as well:
//     r = sqrt(mean_j o_j^2 + eps),  y_j = o_j / r * w_j * silu(z_j),
//     s = max_j |y_j| / 448 (1 for an all-zero row),  c_j = E4M3(y_j / s)
// (OCP E4M3, round to nearest even, saturating). A row's DV values lie in one
// DPP row (16 lanes) of each wave: sums and maxima are reduced over the lanes
// with DPP moves, then across the waves through red[2][32][4] in LDS.
template <int DK, int DV, int NT>
__device__ __forceinline__ void emit_outputs_norm(const Smem<DK, DV> &sm,
                                                  const f32x4 (&Z)[2][NT],
                                                  const f32x4 (&Wm)[2][NT], int g, int l16,
                                                  int wave, int Treal, int B, Rsrc out, int col,
                                                  const VerifyArgs &va, const NormRsrc &nr,
                                                  const Gate &gt, float (*red)[kCh][4]) {
  typedef typename Cols<NT>::F F;
  constexpr int WAVES = DV / (16 * NT);
  constexpr float kE4M3Max = 448.f;
  const uint32_t out_row = va.c.hv * DV * 4, q_row = va.c.hv * DV, s_row = va.c.hv * 4;
  bf16x8 wh[NT], wl[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tok_operand(Wm[0][nt], Wm[1][nt], wh[nt], wl[nt]);
  f32x4 O[2][NT];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    float crow[8], ga[4];
    rd_frow(sm.Cm, 16 * a + l16, g, crow);
#pragma unroll
    for (int i = 0; i < 4; ++i) ga[i] = sm.gam[16 * a + 4 * g + i];
    bf16x8 chh, chl;
    split8(crow, chh, chl);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = ga[i] * Z[a][nt][i];
      acc = mfma(chh, wh[nt], acc);
      acc = mfma(chh, wl[nt], acc);
      acc = mfma(chl, wh[nt], acc);
      O[a][nt] = acc;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * a + 4 * g + i;
      F o;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt] = O[a][nt][i];
      bstore(o, out, (t < Treal && t >= B) ? (uint32_t)(t - B) * out_row + col * 4 : kOOB);
    }
  }
  // Row slot (a, i) of a lane holds rows 16 a + 4 g + i, g = 0..3: a slot with
  // no draft row in any of them (the same in every wave) is skipped whole.
  auto slot_live = [&](int a, int i) {
    const int t0 = 16 * a + i;
    return (t0 + 12 >= B) && (t0 < Treal) &&
           ((t0 >= B && t0 < Treal) || (t0 + 4 >= B && t0 + 4 < Treal) ||
            (t0 + 8 >= B && t0 + 8 < Treal) || (t0 + 12 >= B && t0 + 12 < Treal));
  };
  // Mean square of each row: the rows' reductions are independent chains. 1/r
  // comes from the hardware reciprocal square root (1 ulp) and the gate's
  // 1/(1 + e^-z) and 1/max|y| from the hardware reciprocal: r only sets the
  // scale (the codes are y / max|y|, where it cancels), and all three sit far
  // inside the scale's and the codes' tolerance.
  float acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!slot_live(a, i)) continue;
      float ss = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) ss = fmaf(O[a][nt][i], O[a][nt][i], ss);
      acc[a][i] = row16_reduce<false>(ss);
      if (l16 == 15) red[0][16 * a + 4 * g + i][wave] = acc[a][i];
    }
  __syncthreads();
  float y[2][NT][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!slot_live(a, i)) continue;
      const float4 p = *reinterpret_cast<const float4 *>(red[0][16 * a + 4 * g + i]);
      const float tot = WAVES == 4 ? (p.x + p.y) + (p.z + p.w) : p.x + p.y;
      const float rinv =
          __builtin_amdgcn_rsqf(fmaxf(fmaf(tot, 1.f / DV, va.norm_eps), 1.17549435e-38f));
      float amax = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t zb = gt.z[a][i];
        const float zf = __uint_as_float(nt == 0 ? zb << 16 : zb & 0xffff0000u);
        const float gate = zf * __builtin_amdgcn_rcpf(1.f + __expf(-zf));
        y[a][nt][i] = O[a][nt][i] * rinv * gt.w[nt] * gate;
        amax = fmaxf(amax, fabsf(y[a][nt][i]));
      }
      acc[a][i] = row16_reduce<true>(amax);
      if (l16 == 15) red[1][16 * a + 4 * g + i][wave] = acc[a][i];
    }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!slot_live(a, i)) continue;
      const int t = 16 * a + 4 * g + i;
      const bool row = t < Treal && t >= B;
      const float4 p = *reinterpret_cast<const float4 *>(red[1][t]);
      const float amax = WAVES == 4 ? fmaxf(fmaxf(p.x, p.y), fmaxf(p.z, p.w)) : fmaxf(p.x, p.y);
      float scale = 1.f, inv = 1.f;
      if (amax >= 0x1p-126f) {
        scale = amax * (1.f / kE4M3Max);
        inv = kE4M3Max * __builtin_amdgcn_rcpf(amax);
      } else if (amax > 0.f) {  // a subnormal maximum: exact quotients
        scale = amax / kE4M3Max;
        inv = kE4M3Max / amax;
      }
      // clamp first: the conversion then never sees a value past the largest code
      const float c0 = fminf(fmaxf(y[a][0][i] * inv, -kE4M3Max), kE4M3Max);
      const float c1 = fminf(fmaxf(y[a][1][i] * inv, -kE4M3Max), kE4M3Max);
      const uint32_t packed = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
      bstore((uint16_t)(packed & 0xffff), nr.q, row ? (uint32_t)(t - B) * q_row + col : kOOB);
      if (wave == 0 && l16 == 0)
        bstore(scale, nr.scale, row ? (uint32_t)(t - B) * s_row : kOOB);
    }
}

// Fold the chunk into the state: H <- gamma_T H + K^T (L[T-1] o W).
template <int DK, int DV, int NT>
__device__ __forceinline__ void fold_state(const Smem<DK, DV> &sm, const f32x4 (&Wm)[2][NT], int g,
                                           int l16, typename Cols<NT>::F (&H)[DK / 16][4]) {
  constexpr int MT = DK / 16;
  const float gT = sm.gam[kCh - 1], lg31 = sm.lg[kCh - 1];
  bf16x8 wh[NT], wl[NT];
  {
    float lt[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) lt[a][i] = exp2f(lg31 - sm.lg[16 * a + 4 * g + i]);
    f32x4 Wp[2][NT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) Wp[a][nt][i] = lt[a][i] * Wm[a][nt][i];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tok_operand(Wp[0][nt], Wp[1][nt], wh[nt], wl[nt]);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const bf16x8 kt = rd_row(sm.kt, 16 * mt + l16, 4 * g);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = {H[mt][0][nt] * gT, H[mt][1][nt] * gT, H[mt][2][nt] * gT, H[mt][3][nt] * gT};
      acc = mfma(kt, wh[nt], acc);
      acc = mfma(kt, wl[nt], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) H[mt][i][nt] = acc[i];
    }
  }
}

// One workgroup per (request, value head), any ring capacity. VERIFY: outputs of
// the draft, state untouched. !VERIFY (flush): fold all committed tokens, write
// the state back, move the pointers. The token stream (B committed ring tokens,
// then the draft when verifying) is cut into chunks of 32 from its end, so the
// last chunk (verify's output chunk) holds the whole draft (D <= 32); every other
// chunk is folded into the state held in registers.
//
// Chunk 0 is staged by waves 0..SW-1 while waves SW.. load their state columns
// (as in replay_single); later chunks are staged by all waves. Per chunk: wave 0
// builds the decays, A and (I + A)^-1, wave 1 the output chunk's C, one barrier,
// then every wave contracts its state columns and forms W and either the
// outputs or the fold. The chunk loop is not unrolled: its body is the
// register-bound part, and one copy of it keeps the kernel at 4 workgroups per CU.
template <int DK, int DV, int NT, bool VERIFY, bool VARLEN>
__global__ __launch_bounds__(64 * (DV / (16 * NT)), 4) void replay_chunked(VerifyArgs va,
                                                                           FlushArgs fa) {
  constexpr int WAVES = DV / (16 * NT);
  constexpr int MT = DK / 16;
  static_assert(DK % 32 == 0 && DV % (16 * NT) == 0 && (NT == 2 || NT == 4), "tile shape");
  static_assert(WAVES >= 2, "the T x T matrices are built by waves 0 and 1");
  typedef typename Cols<NT>::F F;
  __shared__ Smem<DK, DV> sm;

  const CacheView &c = VERIFY ? va.c : fa.c;
  const int HV = c.hv;
  const int r = blockIdx.x / HV, h = head_of(blockIdx.x % HV, HV, HV / c.hk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = (tid >> 4) & 3, l16 = tid & 15;  // bit fields of the thread index: cheap to recompute
  const bool lead = (h == 0 && tid == 0);
  // this lane's first state column and its byte offset in the state tile,
  // recomputed where used from an opaque copy of the thread index
  auto col_of = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return (t / 64) * 16 * NT + NT * (t & 15);
  };
  auto st_off_of = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return (uint32_t)((4 * ((t & 63) >> 4) * DV + (t / 64) * 16 * NT + NT * (t & 15)) * 4);
  };

  const int s = VERIFY ? va.slot_idx[r] : fa.slot_idx[r];
  if (s < 0 || s >= c.num_slots) {
    if (lead) raise_err(c.err, GDN_DERR_SLOT);
    return;
  }
  const int C = c.cap;
  const int head = c.head[s], n = c.len[s];
  if (head < 0 || head >= C || n < 0 || n > C) {
    if (lead) raise_err(c.err, GDN_DERR_POINTER);
    return;
  }
  int T;
  if constexpr (VERIFY) {
    // this request's draft length (per-request lengths: a separate instantiation)
    const int D = VARLEN ? request_draft(va.draft_lens, r, va.draft) : va.draft;
    if (VARLEN && D < 0) {
      if (lead) raise_err(c.err, GDN_DERR_DRAFT);
      return;
    }
    if (VARLEN && D == 0) return;  // no draft: nothing to emit or append
    if (n + D > C) {
      if (lead) raise_err(c.err, GDN_DERR_CAPACITY);
      return;
    }
    T = n + D;
    // opaque past the checks: value facts drawn from them made the register
    // allocation of the chunk loop spill
    asm volatile("" : "+s"(T));
  } else {
    if (n < max(fa.min_len, 1)) return;  // not due: nothing is written
    // verify_flush run as two calls: a request with a bad draft length is not flushed
    if (fa.draft_lens && request_draft(fa.draft_lens, r, fa.max_draft) < 0) return;
    T = n;
  }
  const Unit u{r, h, s, h / (HV / c.hk), head, n, T, C};
  const int nchunks = (T + kCh - 1) / kCh;
  const int T0 = T - kCh * (nchunks - 1);  // tokens in the first chunk (1..32)
  const Rsrc st = make_rsrc(c.state + ((int64_t)s * HV + h) * DK * DV, DK * DV * 4);
  const Srcs sr = make_srcs<DK, DV>(c, u, &va, VERIFY);
  const bool kq_writer = h % (HV / c.hk) == 0;

  constexpr int SW = WAVES >= 4 ? 2 : WAVES;
  F H[MT][4];
  float al;  // staged alpha of token lane % 32 of the current chunk (waves 0 and 1)
  {
    Stage<DK, DV, NT, VERIFY, 64 * SW> sg0;
    const bool out0 = VERIFY && nchunks == 1;
    if (wave >= SW) {
      load_state<DK, DV, NT>(st, st_off_of(), H);
      al = 1.f;
    } else {
      sg0.load(sr, u, 0, T0, out0);
      sg0.store(sm, T0, out0);
      al = sg0.al;
      __builtin_amdgcn_sched_barrier(0);
      load_state<DK, DV, NT>(st, st_off_of(), H);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }

  // every chunk but verify's last: fold into the state
  const int nfold = VERIFY ? nchunks - 1 : nchunks;
#pragma nounroll
  for (int ch = 0; ch < nfold; ++ch) {
    const int lane = opaque_tid() % 64, g = lane >> 4, l16 = lane & 15;
    const int t0 = ch == 0 ? 0 : T0 + kCh * (ch - 1);
    const int Treal = ch == 0 ? T0 : kCh;
    if (ch > 0) {
      Stage<DK, DV, NT, VERIFY> sg;
      sg.load(sr, u, t0, Treal, false);
      sg.store(sm, Treal, false);
      al = sg.al;
      __syncthreads();
    }
    if (wave == 0) build_tt<DK, DV>(sm, al, lane, g, l16);
    __syncthreads();  // T x T matrices complete
    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, DV, NT, kY>(sm, H, g, l16, Y, Z);
    solve_w<DK, DV, NT>(sm, Y, col_of(), g, l16, Wm);
    fold_state<DK, DV, NT>(sm, Wm, g, l16, H);
    __syncthreads();  // LDS is rewritten by the next chunk
  }

  if constexpr (VERIFY) {
    // the output chunk: the draft and the committed tokens before it
    const int t0 = nchunks == 1 ? 0 : T0 + kCh * (nchunks - 2);
    const int Treal = nchunks == 1 ? T0 : kCh;
    if (nchunks > 1) {
      Stage<DK, DV, NT, VERIFY> sg;
      sg.load(sr, u, t0, Treal, true);
      sg.store(sm, Treal, true);
      al = sg.al;
      __syncthreads();
    }
    if (wave == 0)
      build_tt<DK, DV>(sm, al, lane, g, l16);
    else if (wave == 1)
      build_c<DK, DV>(sm, al, lane, g, l16);
    __syncthreads();  // T x T matrices complete
    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, DV, NT, kY | kZ>(sm, H, g, l16, Y, Z);
    solve_w<DK, DV, NT>(sm, Y, col_of(), g, l16, Wm);
    emit_outputs<DK, DV, NT>(sm, Z, Wm, g, l16, t0, Treal, u.B, out_rsrc(va, r, h, DV, T - u.B),
                             col_of() * 4, HV * DV * 4);
    // the draft rows, from LDS; the thread mapping is that of the stage type
    if (nchunks == 1) {
      if (wave < SW) Stage<DK, DV, NT, VERIFY, 64 * SW>{}.append(sm, sr, u, t0, Treal, kq_writer);
    } else {
      Stage<DK, DV, NT, VERIFY>{}.append(sm, sr, u, t0, Treal, kq_writer);
    }
  }

  if constexpr (!VERIFY) {
    store_state<DK, DV, NT>(st, st_off_of(), H);
    // The last workgroup of this slot to arrive moves the pointers. Every
    // workgroup's head/len loads were consumed (by the branches above) before
    // its arrival, so none can observe the update; no memory fence is needed
    // (an agent-scope fence would write back this XCD's whole L2).
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(slot_counter(c, s), 1);
      if (prev == HV - 1) {
        c.head[s] = (head + n) % C;
        c.len[s] = 0;
        *slot_counter(c, s) = 0;
      }
    }
  }
}


// Ring capacity <= 32, so every replay is a single chunk (T = len [+ D] <= 32).
// Waves 2 and 3 load their state columns first; waves 0 and 1 stage the
// chunk's inputs, load theirs, then build the T x T matrices (wave 0: A and its
// inverse; wave 1: C) while the state streams in. Verify takes Y = K H and
// Z = Q H in one pass, so its state registers die right after it.
template <int DK, int DV, int NT, bool VERIFY, bool VARLEN>
__global__ __launch_bounds__(64 * (DV / (16 * NT)), 4) void replay_single(VerifyArgs va,
                                                                          FlushArgs fa) {
  constexpr int WAVES = DV / (16 * NT);
  constexpr int MT = DK / 16;
  static_assert(DK % 32 == 0 && DV % (16 * NT) == 0 && (NT == 2 || NT == 4), "tile shape");
  typedef typename Cols<NT>::F F;
  __shared__ Smem<DK, DV> sm;

  const CacheView &c = VERIFY ? va.c : fa.c;
  const int HV = c.hv;
  const int r = blockIdx.x / HV, h = head_of(blockIdx.x % HV, HV, HV / c.hk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = (tid >> 4) & 3, l16 = tid & 15;  // bit fields of the thread index: cheap to recompute
  const int colL = wave * 16 * NT + NT * l16;
  const bool lead = (h == 0 && tid == 0);

  const int s = VERIFY ? va.slot_idx[r] : fa.slot_idx[r];
  if (s < 0 || s >= c.num_slots) {
    if (lead) raise_err(c.err, GDN_DERR_SLOT);
    return;
  }
  const int C = c.cap;
  const int head = c.head[s], n = c.len[s];
  if (head < 0 || head >= C || n < 0 || n > C) {
    if (lead) raise_err(c.err, GDN_DERR_POINTER);
    return;
  }
  int T;
  if constexpr (VERIFY) {
    // this request's draft length (per-request lengths: a separate instantiation)
    const int D = VARLEN ? request_draft(va.draft_lens, r, va.draft) : va.draft;
    if (VARLEN && D < 0) {
      if (lead) raise_err(c.err, GDN_DERR_DRAFT);
      return;
    }
    if (VARLEN && D == 0) return;  // no draft: nothing to emit or append
    if (n + D > C) {
      if (lead) raise_err(c.err, GDN_DERR_CAPACITY);
      return;
    }
    T = n + D;
    // opaque past the checks: value facts drawn from them made the register
    // allocation of the chunk loop spill
    asm volatile("" : "+s"(T));
  } else {
    if (n < max(fa.min_len, 1)) return;  // not due: nothing is written
    // verify_flush run as two calls: a request with a bad draft length is not flushed
    if (fa.draft_lens && request_draft(fa.draft_lens, r, fa.max_draft) < 0) return;
    T = n;
  }
  const Unit u{r, h, s, h / (HV / c.hk), head, n, T, C};
  const Rsrc st = make_rsrc(c.state + ((int64_t)s * HV + h) * DK * DV, DK * DV * 4);
  const uint32_t st_off = (4 * g * DV + colL) * 4;

  const Srcs sr = make_srcs<DK, DV>(c, u, &va, VERIFY);
  // Waves SW.. issue their state loads first; waves 0..SW-1 stage the chunk's
  // inputs, then load their state columns (loads complete in issue order, so a
  // wave that must wait for its staged inputs must not have its state loads
  // ahead of them).
  constexpr int SW = WAVES >= 4 ? 2 : WAVES;
  Stage<DK, DV, NT, VERIFY, 64 * SW> sg;
  F H[MT][4];
  if (wave >= SW) {
    load_state<DK, DV, NT>(st, st_off, H);
  } else {
    sg.load(sr, u, 0, T, VERIFY);
    sg.store(sm, T, VERIFY);
    __builtin_amdgcn_sched_barrier(0);
    load_state<DK, DV, NT>(st, st_off, H);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  if (wave == 0) {
    build_tt<DK, DV>(sm, sg.al, lane, g, l16);
    if (WAVES == 1 && VERIFY) build_c<DK, DV>(sm, sg.al, lane, g, l16);
  } else if (wave == 1 && VERIFY) {
    build_c<DK, DV>(sm, sg.al, lane, g, l16);
  }
  __syncthreads();  // T x T matrices complete

  f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
  contract<DK, DV, NT, VERIFY ? (kY | kZ) : kY>(sm, H, g, l16, Y, Z);
  solve_w<DK, DV, NT>(sm, Y, colL, g, l16, Wm);
  if constexpr (VERIFY) {
    emit_outputs<DK, DV, NT>(sm, Z, Wm, g, l16, 0, T, u.B, out_rsrc(va, r, h, DV, T - u.B),
                             colL * 4, HV * DV * 4);
    if (wave < SW) sg.append(sm, sr, u, 0, T, h % (HV / c.hk) == 0);
  } else {
    fold_state<DK, DV, NT>(sm, Wm, g, l16, H);
    store_state<DK, DV, NT>(st, st_off, H);
    // The last workgroup of this slot to arrive moves the pointers. Every
    // workgroup's head/len loads were consumed (by the branches above) before
    // its arrival, so none can observe the update; no memory fence is needed
    // (an agent-scope fence would write back this XCD's whole L2).
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(slot_counter(c, s), 1);
      if (prev == HV - 1) {
        c.head[s] = (head + n) % C;
        c.len[s] = 0;
        *slot_counter(c, s) = 0;
      }
    }
  }
}

// Request of rank q in the order [due requests..., other requests...], where a
// request is due when its slot is valid and len >= mn, with its slot and that
// slot's pointers (head and len are meaningful only for a valid slot); every
// lane of the wave returns the same values. Up to 64 requests take one pass:
// each lane loads one request's slot and pointers, a ballot orders them, and the
// chosen lane's values are read across the wave, so the state address is known
// after two dependent loads. More requests are counted in rounds of 64 and the
// chosen one's slot and pointers are loaded again. The order depends only on
// slot_idx and len, which the fused kernel leaves unchanged until its last
// workgroup.
__device__ __forceinline__ int nth_bit(uint64_t m, int n) {
  for (int t = 0; t < n; ++t) m &= m - 1;
  return __builtin_ctzll(m);
}

struct Req {
  int r, s, head, len;  // len: committed count after the folded rollback, if any
  int raw_len;          // len as stored
  int due;              // number of due requests in the call
  int roll_err;         // the folded rollback's error bit for this request (0: none)
};

// Committed count of request i once the accepted prefix of the previous draft
// is committed (the rollback folded into this call): len + a when the previous
// length is in [0, prev_draft], a in [0, that length] and len + a <= C;
// otherwise len, with the rollback's error bit in *bad (as a separate rollback
// call would skip the request and flag it).
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

__device__ __forceinline__ int rolled_len(const VerifyArgs &va, int i, int len, int cap,
                                          int *bad) {
  const int bound = va.prev_draft_lens ? va.prev_draft_lens[i] : va.prev_draft;
  return rolled_from(len, va.prev_accepted[i], bound, va.prev_draft, cap, bad);
}

// The pointer move of one request at the end of the call: slot (-1: none), new
// head (-1: unchanged) and new len.
struct Move {
  int slot, head, len;
};

// With at most 64 requests, the lanes of the ordering pass hold every
// request's slot and pointers; wave 0 also works out each request's pointer
// move from them (exactly as the end-of-grid loop below would) and leaves it in
// moves[], so that the last workgroup only stores. The values are those at the
// start of the call, which is what the end-of-grid loop reads too: no pointer
// changes before the last workgroup.
template <bool ROLLBACK, bool VARLEN>
__device__ Req ordered_request(const VerifyArgs &va, int mn, int q, int lane, Move *moves) {
  const int R = va.num_reqs;
  const CacheView &c = va.c;
  auto lanes = [&](int j) -> uint64_t {
    const int m = min(64, R - 64 * j);
    return m == 64 ? ~0ull : ((1ull << m) - 1);
  };
  // committed count the call works from: the stored len, or len + a with the
  // previous draft's rollback folded in (when the pointers are valid)
  auto eff = [&](int i, int h, int n) {
    if (!ROLLBACK || h < 0 || h >= c.cap || n < 0 || n > c.cap) return n;
    int bad;
    return rolled_len(va, i, n, c.cap, &bad);
  };
  // the folded rollback's inputs of request i, loaded beside slot_idx[i] (they
  // do not depend on the slot), and the committed count they give
  auto roll_in = [&](int i, int *a, int *bound) {
    *a = va.prev_accepted[i];
    *bound = va.prev_draft_lens ? va.prev_draft_lens[i] : va.prev_draft;
  };
  auto eff_from = [&](int h, int n, int a, int bound, int *bad) {
    *bad = 0;
    if (!ROLLBACK || h < 0 || h >= c.cap || n < 0 || n > c.cap) return n;
    return rolled_from(n, a, bound, va.prev_draft, c.cap, bad);
  };
  if (R <= 64) {
    int si = -1, hi = 0, ni = 0, ne = 0, ai = 0, bi = 0, bad = 0;
    if (lane < R) {
      if constexpr (ROLLBACK) roll_in(lane, &ai, &bi);
      si = va.slot_idx[lane];
      if (si >= 0 && si < c.num_slots) {
        hi = c.head[si];
        ni = c.len[si];
        ne = eff_from(hi, ni, ai, bi, &bad);
      }
    }
    const uint64_t dm = __ballot(si >= 0 && si < c.num_slots && ne >= mn);
    if (moves && lane < R) {
      Move mv{-1, -1, 0};
      if (si >= 0 && si < c.num_slots && hi >= 0 && hi < c.cap && ni >= 0 && ni <= c.cap) {
        // a request with a bad draft length is not flushed (a folded rollback stands)
        const bool skip = VARLEN && request_draft(va.draft_lens, lane, va.draft) < 0;
        if (ne >= mn && !skip)
          mv = Move{si, hi + ne - (hi + ne >= c.cap ? c.cap : 0), 0};
        else if (ROLLBACK && ne != ni)
          mv = Move{si, -1, ne};
      }
      moves[lane] = mv;
    }
    const int nd = __popcll(dm);
    const int r = q < nd ? nth_bit(dm, q) : nth_bit(~dm & lanes(0), q - nd);
    return Req{r,
               __builtin_amdgcn_readlane(si, r),
               __builtin_amdgcn_readlane(hi, r),
               __builtin_amdgcn_readlane(ne, r),
               __builtin_amdgcn_readlane(ni, r),
               nd,
               ROLLBACK ? __builtin_amdgcn_readlane(bad, r) : 0};
  }
  // Up to 4 rounds of 64: every lane keeps its requests' slot and pointers, so
  // the chosen request's come from a readlane instead of reloads, and each
  // round's loads are issued once.
  constexpr int kRounds = 4;
  if (R <= 64 * kRounds) {
    int si[kRounds], hi[kRounds], ni[kRounds], ne[kRounds], bad[kRounds];
    uint64_t dm[kRounds];
    int nd = 0;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int i = 64 * j + lane;
      si[j] = -1;
      hi[j] = ni[j] = ne[j] = bad[j] = 0;
      if (i < R) {
        int ai = 0, bi = 0;
        if constexpr (ROLLBACK) roll_in(i, &ai, &bi);
        si[j] = va.slot_idx[i];
        if (si[j] >= 0 && si[j] < c.num_slots) {
          hi[j] = c.head[si[j]];
          ni[j] = c.len[si[j]];
          ne[j] = eff_from(hi[j], ni[j], ai, bi, &bad[j]);
        }
      }
      dm[j] = __ballot(si[j] >= 0 && si[j] < c.num_slots && ne[j] >= mn);
      nd += __popcll(dm[j]);
    }
    const bool want_due = q < nd;
    int left = want_due ? q : q - nd;
    Req o{0, -1, 0, 0, 0, nd, 0};
    bool found = false;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const uint64_t all = 64 * j < R ? lanes(j) : 0ull;
      const uint64_t m = want_due ? dm[j] : (~dm[j] & all);
      const int cnt = __popcll(m);
      if (!found && left < cnt) {
        const int l = nth_bit(m, left);
        o.r = 64 * j + l;
        o.s = __builtin_amdgcn_readlane(si[j], l);
        o.head = __builtin_amdgcn_readlane(hi[j], l);
        o.len = __builtin_amdgcn_readlane(ne[j], l);
        o.raw_len = __builtin_amdgcn_readlane(ni[j], l);
        if constexpr (ROLLBACK) o.roll_err = __builtin_amdgcn_readlane(bad[j], l);
        found = true;
      } else if (!found) {
        left -= cnt;
      }
    }
    return o;
  }
  auto due_mask = [&](int j) -> uint64_t {
    const int i = 64 * j + lane;
    bool d = false;
    if (i < R) {
      const int si = va.slot_idx[i];
      d = si >= 0 && si < c.num_slots && eff(i, c.head[si], c.len[si]) >= mn;
    }
    return __ballot(d);
  };
  const int chunks = (R + 63) / 64;
  int nd = 0;
  for (int j = 0; j < chunks; ++j) nd += __popcll(due_mask(j));
  const bool want_due = q < nd;
  int left = want_due ? q : q - nd;
  int r = q;  // replaced below: the two classes cover every request
  for (int j = 0; j < chunks; ++j) {
    uint64_t m = due_mask(j);
    if (!want_due) m = ~m & lanes(j);
    const int cnt = __popcll(m);
    if (left < cnt) {
      r = 64 * j + nth_bit(m, left);
      break;
    }
    left -= cnt;
  }
  Req o{r, va.slot_idx[r], 0, 0, 0, nd, 0};
  if (o.s >= 0 && o.s < c.num_slots) {
    o.head = c.head[o.s];
    o.raw_len = c.len[o.s];
    o.len = o.raw_len;
    if (ROLLBACK && o.head >= 0 && o.head < c.cap && o.raw_len >= 0 && o.raw_len <= c.cap)
      o.len = rolled_len(va, r, o.raw_len, c.cap, &o.roll_err);
  }
  return o;
}

// End of a fused launch. Every workgroup counts itself in (after a barrier, so
// that all its waves have read the pointers): HV per request rank on that
// rank's counter, then the last of those on the grid counter. The grid's last
// workgroup moves the pointers: a due slot's head += len, len = 0; with a
// folded rollback, len += a for the others. With no due request and no
// rollback nothing moves and no count is taken (every workgroup sees the same
// count, as no pointer changes during the call).
template <bool ROLLBACK, bool VARLEN>
__device__ __forceinline__ void end_of_grid(const VerifyArgs &va, const Req &rq, int mn,
                                            int32_t *rank_ctr, int32_t *grid_ctr,
                                            const Move *moves, int *grid_rank, int tid) {
  const CacheView &c = va.c;
  const int HV = c.hv;
  if (!ROLLBACK && rq.due == 0) return;  // a folded rollback moves len in any case
  __syncthreads();
  if (tid == 0) {
    int last = 0;
    if (atomicAdd(rank_ctr, 1) == HV - 1) {
      *rank_ctr = 0;
      last = atomicAdd(grid_ctr, 1) == va.num_reqs - 1;
    }
    *grid_rank = last;
  }
  __syncthreads();
  if (!*grid_rank) return;
  if (va.num_reqs <= 64) {  // moves worked out by the ordering pass
    if (tid < va.num_reqs) {
      const Move mv = moves[tid];
      if (mv.slot >= 0) {
        if (mv.head >= 0) c.head[mv.slot] = mv.head;
        c.len[mv.slot] = mv.len;
      }
    }
    if (tid == 0) *grid_ctr = 0;
    return;
  }
  for (int i = tid; i < va.num_reqs; i += blockDim.x) {
    const int si = va.slot_idx[i];
    if (si < 0 || si >= c.num_slots) continue;
    const int hs = c.head[si], n0 = c.len[si];
    if (hs < 0 || hs >= c.cap || n0 < 0 || n0 > c.cap) continue;
    int ns = n0;
    if constexpr (ROLLBACK) {
      int bad;
      ns = rolled_len(va, i, n0, c.cap, &bad);
    }
    // a request with a bad draft length is not flushed (its rollback stands)
    const bool skip = VARLEN && request_draft(va.draft_lens, i, va.draft) < 0;
    if (ns >= mn && !skip) {
      c.head[si] = hs + ns - (hs + ns >= c.cap ? c.cap : 0);
      c.len[si] = 0;
    } else if (ROLLBACK && ns != n0) {
      c.len[si] = ns;
    }
  }
  if (tid == 0) *grid_ctr = 0;
}

// Flush fused into verify, ring capacity <= 32. A slot with len >= max(min_len,
// 1) first folds its len committed tokens into the checkpoint and writes it
// back, then verifies the draft from the new checkpoint; other slots verify as
// replay_single does. One state read serves both, and a due slot's state is
// written once.
//
// Work order: units of due requests (about twice the work) come first, so that
// the dispatch, which spreads consecutive workgroups over the CUs, gives every
// CU a similar share of them. Every workgroup derives the order from each
// request's len, so len must not change while a workgroup may still read it:
// the pointers of the due slots (head += len, len = 0) are moved by the last
// workgroup of the grid to finish. It is found in two levels, so that no
// counter sees more than one arrival per workgroup of a request group: the
// HV workgroups of request rank q count in at that rank's counter (a 128-byte
// line of its own), the last of them at the grid counter.
//
// The draft is appended at (new head + j) mod C, which may wrap onto committed
// key rows that the other value heads of the same key head are still reading
// for their fold. So each workgroup of a due slot counts itself in at the
// (slot, key head) counter once its fold inputs are staged, and the last
// one of the key head's group appends k and q (the others have read by then).
template <int DK, int DV, int NT, bool VARLEN, bool ROLLBACK, bool NORM>
__global__ __launch_bounds__(64 * (DV / (16 * NT)), 4) void replay_fused(VerifyArgs va,
                                                                         int min_len) {
  constexpr int WAVES = DV / (16 * NT);
  constexpr int MT = DK / 16;
  static_assert(DK % 32 == 0 && DV % (16 * NT) == 0 && (NT == 2 || NT == 4), "tile shape");
  typedef typename Cols<NT>::F F;
  __shared__ Smem<DK, DV> sm;
  __shared__ int group_rank, grid_rank;
  __shared__ Move moves[64];

  const CacheView &c = va.c;
  const int HV = c.hv, G = HV / c.hk;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane >> 4, l16 = lane & 15;
  // This lane's first state column and its byte offset in the state tile, taken
  // from an opaque copy of the thread index at each use, so that they are
  // recomputed there instead of being held in registers through the kernel.
  auto col_of = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return (t / 64) * 16 * NT + NT * (t & 15);
  };
  auto st_off_of = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return (uint32_t)((4 * ((t & 63) >> 4) * DV + (t / 64) * 16 * NT + NT * (t & 15)) * 4);
  };
  const int mn = max(min_len, 1);
  const Req rq = ordered_request<ROLLBACK, VARLEN>(va, mn, blockIdx.x / HV, lane,
                                                  wave == 0 ? moves : nullptr);
  const int r = rq.r, h = head_of(blockIdx.x % HV, HV, G);
  const bool lead = (h == 0 && tid == 0);
  int32_t *grid_ctr = c.sync;
  int32_t *rank_ctr = slot_counter(c, blockIdx.x / HV);

  // every workgroup counts itself in at its end; the grid's last moves the pointers
  auto finish = [&]() {
    end_of_grid<ROLLBACK, VARLEN>(va, rq, mn, rank_ctr, grid_ctr, moves, &grid_rank, tid);
  };

  const int s = rq.s;
  if (s < 0 || s >= c.num_slots) {
    if (lead) raise_err(c.err, GDN_DERR_SLOT);
    finish();
    return;
  }
  const int C = c.cap;
  const int head = rq.head, n = rq.len;
  if (head < 0 || head >= C || rq.raw_len < 0 || rq.raw_len > C) {
    if (lead) raise_err(c.err, GDN_DERR_POINTER);
    finish();
    return;
  }
  // the folded rollback's own error, as a rollback call would flag it
  if (ROLLBACK && lead && rq.roll_err) raise_err(c.err, rq.roll_err);
  // this request's draft length (the per-request lengths are a separate
  // instantiation, so that the fixed-length kernel carries none of their code)
  const int D = VARLEN ? request_draft(va.draft_lens, r, va.draft) : va.draft;
  if (VARLEN && D < 0) {
    if (lead) raise_err(c.err, GDN_DERR_DRAFT);
    finish();
    return;
  }
  const bool due = n >= mn;
  if (!due && ((VARLEN && D == 0) || n + D > C)) {  // capacity error, or nothing to do
    if (lead && D > 0) raise_err(c.err, GDN_DERR_CAPACITY);
    finish();
    return;
  }
  const int kh = h / G;
  const Rsrc st = make_rsrc(c.state + ((int64_t)s * HV + h) * DK * DV, DK * DV * 4);
  int32_t *group_ctr = group_counter(c, s, kh);

  // Waves SW.. issue their state loads first; waves 0..SW-1 stage the inputs of
  // the first replay, then load their state columns (loads complete in issue
  // order, so a wave that waits for staged inputs must not have state loads
  // ahead of them).
  constexpr int SW = WAVES >= 4 ? 2 : WAVES;
  F H[MT][4];
  int hd = head, B = n;  // ring start and committed count of the verify below
  if (due) {
    // ---- flush: fold the n committed tokens
    const Unit uf{r, h, s, kh, head, n, n, C};
    Stage<DK, DV, NT, false, 64 * SW> sgf;
    if (wave >= SW) {
      load_state<DK, DV, NT>(st, st_off_of(), H);
    } else {
      const Srcs sf = make_srcs<DK, DV>(c, uf, nullptr, false);
      sgf.load(sf, uf, 0, n, false);
      sgf.store(sm, n, false);
      __builtin_amdgcn_sched_barrier(0);
      load_state<DK, DV, NT>(st, st_off_of(), H);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // the committed rows are read (and staged)
    if (tid == 0) group_rank = atomicAdd(group_ctr, 1);
    if (wave == 0) build_tt<DK, DV>(sm, sgf.al, lane, g, l16);
    __syncthreads();
    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, DV, NT, kY>(sm, H, g, l16, Y, Z);
    solve_w<DK, DV, NT>(sm, Y, col_of(), g, l16, Wm);
    fold_state<DK, DV, NT>(sm, Wm, g, l16, H);
    store_state<DK, DV, NT>(st, st_off_of(), H);
    hd = head + n - (head + n >= C ? C : 0);
    B = 0;
    __syncthreads();  // LDS is staged again below
  }

  // ---- verify the draft from checkpoint H plus B committed tokens at hd. A due
  // slot's state is live here, so all waves stage (fewer rows each); otherwise
  // waves 0..SW-1 stage while the others' state loads stream in.
  const Unit u{r, h, s, kh, hd, B, B + D, C};
  const Srcs sr = make_srcs<DK, DV>(c, u, &va, true);
  Stage<DK, DV, NT, true> sga;
  Stage<DK, DV, NT, true, 64 * SW> sgs;
  float al;  // this lane's staged alpha (token lane % 32)
  if (due) {
    sga.load(sr, u, 0, u.T, true);
    sga.store(sm, u.T, true);
    al = sga.al;
  } else {
    if (wave >= SW) {
      load_state<DK, DV, NT>(st, st_off_of(), H);
      al = 1.f;
    } else {
      sgs.load(sr, u, 0, u.T, true);
      sgs.store(sm, u.T, true);
      al = sgs.al;
      __builtin_amdgcn_sched_barrier(0);
      load_state<DK, DV, NT>(st, st_off_of(), H);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  if (wave == 0) {
    build_tt<DK, DV>(sm, al, lane, g, l16);
    if (WAVES == 1) build_c<DK, DV>(sm, al, lane, g, l16);
  } else if (wave == 1) {
    build_c<DK, DV>(sm, al, lane, g, l16);
  }
  __syncthreads();  // T x T matrices complete

  f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
  contract<DK, DV, NT, kY | kZ>(sm, H, g, l16, Y, Z);
  if constexpr (NORM) {
    // the gate and weight load while W is solved; out may be absent
    const NormRsrc nr = norm_rsrc(va, r, h, DV, max(D, 1));
    const Gate gt = load_gate<DV, NT>(va, nr, col_of(), g, u.B, u.T);
    solve_w<DK, DV, NT>(sm, Y, col_of(), g, l16, Wm);
    __shared__ __align__(16) float nred[2][kCh][4];
    emit_outputs_norm<DK, DV, NT>(
        sm, Z, Wm, g, l16, wave, u.T, u.B,
        va.out ? out_rsrc(va, r, h, DV, max(D, 1)) : make_rsrc(nullptr, 0), col_of(), va, nr, gt,
        nred);
  } else {
    solve_w<DK, DV, NT>(sm, Y, col_of(), g, l16, Wm);
    emit_outputs<DK, DV, NT>(sm, Z, Wm, g, l16, 0, u.T, u.B, out_rsrc(va, r, h, DV, max(D, 1)),
                             col_of() * 4, HV * DV * 4);
  }
  const bool kq_writer = due ? group_rank == G - 1 : h % G == 0;
  if (due)
    sga.append(sm, sr, u, 0, u.T, kq_writer);
  else if (wave < SW)
    sgs.append(sm, sr, u, 0, u.T, kq_writer);
  if (due && kq_writer && tid == 0) *group_ctr = 0;  // every member has counted in
  finish();
}

// Flush fused into verify when a replay takes several chunks (ring capacity
// above 32). A due slot folds its n committed tokens chunk by chunk, writes the
// folded state once and verifies the draft from it (one chunk, B = 0); any
// other slot replays its committed tokens and the draft as replay_chunked's
// verify does. The work order (due requests first), the draft append of a due
// slot's key and query rows (by the last workgroup of the key head to have
// staged all its fold inputs) and the end-of-grid pointer move are those of
// replay_fused.
template <int DK, int DV, int NT, bool VARLEN, bool ROLLBACK>
__global__ __launch_bounds__(64 * (DV / (16 * NT)), 4) void replay_fused_long(VerifyArgs va,
                                                                              int min_len) {
  constexpr int WAVES = DV / (16 * NT);
  constexpr int MT = DK / 16;
  static_assert(DK % 32 == 0 && DV % (16 * NT) == 0 && (NT == 2 || NT == 4), "tile shape");
  static_assert(WAVES >= 2, "the T x T matrices are built by waves 0 and 1");
  typedef typename Cols<NT>::F F;
  __shared__ Smem<DK, DV> sm;
  __shared__ int group_rank, grid_rank;
  __shared__ Move moves[64];

  const CacheView &c = va.c;
  const int HV = c.hv, G = HV / c.hk;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane >> 4, l16 = lane & 15;
  auto col_of = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return (t / 64) * 16 * NT + NT * (t & 15);
  };
  auto st_off_of = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return (uint32_t)((4 * ((t & 63) >> 4) * DV + (t / 64) * 16 * NT + NT * (t & 15)) * 4);
  };
  const int mn = max(min_len, 1);
  const Req rq = ordered_request<ROLLBACK, VARLEN>(va, mn, blockIdx.x / HV, lane,
                                                   wave == 0 ? moves : nullptr);
  const int r = rq.r, h = head_of(blockIdx.x % HV, HV, G);
  const bool lead = (h == 0 && tid == 0);
  int32_t *grid_ctr = c.sync;
  int32_t *rank_ctr = slot_counter(c, blockIdx.x / HV);
  auto finish = [&]() {
    end_of_grid<ROLLBACK, VARLEN>(va, rq, mn, rank_ctr, grid_ctr, moves, &grid_rank, tid);
  };

  const int s = rq.s;
  if (s < 0 || s >= c.num_slots) {
    if (lead) raise_err(c.err, GDN_DERR_SLOT);
    finish();
    return;
  }
  const int C = c.cap;
  const int head = rq.head, n = rq.len;  // n: after the folded rollback, if any
  if (head < 0 || head >= C || rq.raw_len < 0 || rq.raw_len > C) {
    if (lead) raise_err(c.err, GDN_DERR_POINTER);
    finish();
    return;
  }
  // the folded rollback's own error, as a rollback call would flag it
  if (ROLLBACK && lead && rq.roll_err) raise_err(c.err, rq.roll_err);
  const int D = VARLEN ? request_draft(va.draft_lens, r, va.draft) : va.draft;
  if (VARLEN && D < 0) {
    if (lead) raise_err(c.err, GDN_DERR_DRAFT);
    finish();
    return;
  }
  const bool due = n >= mn;
  if (!due && ((VARLEN && D == 0) || n + D > C)) {  // capacity error, or nothing to do
    if (lead && D > 0) raise_err(c.err, GDN_DERR_CAPACITY);
    finish();
    return;
  }
  const int kh = h / G;
  const Rsrc st = make_rsrc(c.state + ((int64_t)s * HV + h) * DK * DV, DK * DV * 4);
  int32_t *group_ctr = group_counter(c, s, kh);
  constexpr int SW = WAVES >= 4 ? 2 : WAVES;
  F H[MT][4];
  float al;  // staged alpha of token lane % 32 of the current chunk

  // One chunk loop and one output stage serve both kinds of slot (two copies of
  // the register-bound body do not fit the registers). The stream u1 starts at
  // head with the n committed tokens: a due slot's stream is those n tokens,
  // all folded (its state is then written and the draft verified from it as a
  // stream of its own, B = 0); any other slot's is the n tokens and the draft,
  // whose last chunk is the output chunk.
  const Unit u1{r, h, s, kh, head, n, due ? n : n + D, C};
  const Srcs s1 = due ? make_srcs<DK, DV>(c, u1, nullptr, false)
                      : make_srcs<DK, DV>(c, u1, &va, true);
  const int nch = (u1.T + kCh - 1) / kCh, T0 = u1.T - kCh * (nch - 1);
  const int nfold = due ? nch : nch - 1;
  const bool out0 = !due && nch == 1;  // chunk 0 is the output chunk
  {
    // waves SW.. load their state first; waves 0..SW-1 stage chunk 0, then load
    Stage<DK, DV, NT, true, 64 * SW> sg0;
    if (wave >= SW) {
      load_state<DK, DV, NT>(st, st_off_of(), H);
      al = 1.f;
    } else {
      sg0.load(s1, u1, 0, T0, out0);
      sg0.store(sm, T0, out0);
      al = sg0.al;
      __builtin_amdgcn_sched_barrier(0);
      load_state<DK, DV, NT>(st, st_off_of(), H);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }
  // The thread index comes through an opaque copy so that the per-thread row
  // offsets are recomputed in every iteration rather than held in registers.
#pragma nounroll
  for (int ch = 0; ch < nfold; ++ch) {
    const int lane = opaque_tid() % 64, g = lane >> 4, l16 = lane & 15;
    if (ch > 0) {
      Stage<DK, DV, NT, true> sg;
      sg.load(s1, u1, T0 + kCh * (ch - 1), kCh, false);
      sg.store(sm, kCh, false);
      al = sg.al;
      __syncthreads();
    }
    // a due slot's fold inputs are all read: count in for the key rows' append
    if (due && ch == nfold - 1 && tid == 0) group_rank = atomicAdd(group_ctr, 1);
    if (wave == 0) build_tt<DK, DV>(sm, al, lane, g, l16);
    __syncthreads();  // T x T matrices complete
    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, DV, NT, kY>(sm, H, g, l16, Y, Z);
    solve_w<DK, DV, NT>(sm, Y, col_of(), g, l16, Wm);
    fold_state<DK, DV, NT>(sm, Wm, g, l16, H);
    __syncthreads();  // LDS is rewritten by the next chunk
  }

  // ---- the output chunk
  Unit uo = u1;
  int t0 = nch == 1 ? 0 : T0 + kCh * (nch - 2), Treal = nch == 1 ? T0 : kCh;
  if (due) {
    store_state<DK, DV, NT>(st, st_off_of(), H);
    const int hd = head + n - (head + n >= C ? C : 0);
    uo = Unit{r, h, s, kh, hd, 0, D, C};
    t0 = 0;
    Treal = D;
  }
  const Srcs so = due ? make_srcs<DK, DV>(c, uo, &va, true) : s1;
  if (!out0) {
    Stage<DK, DV, NT, true> sg;
    sg.load(so, uo, t0, Treal, true);
    sg.store(sm, Treal, true);
    al = sg.al;
    __syncthreads();
  }
  if (wave == 0)
    build_tt<DK, DV>(sm, al, lane, g, l16);
  else if (wave == 1)
    build_c<DK, DV>(sm, al, lane, g, l16);
  __syncthreads();  // T x T matrices complete
  {
    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, DV, NT, kY | kZ>(sm, H, g, l16, Y, Z);
    solve_w<DK, DV, NT>(sm, Y, col_of(), g, l16, Wm);
    emit_outputs<DK, DV, NT>(sm, Z, Wm, g, l16, t0, Treal, uo.B,
                             out_rsrc(va, r, h, DV, max(D, 1)), col_of() * 4, HV * DV * 4);
  }
  const bool kq_writer = due ? group_rank == G - 1 : h % G == 0;
  // the draft rows, from LDS, with the thread mapping of the stage that wrote them
  if (out0) {
    if (wave < SW) Stage<DK, DV, NT, true, 64 * SW>{}.append(sm, so, uo, t0, Treal, kq_writer);
  } else {
    Stage<DK, DV, NT, true>{}.append(sm, so, uo, t0, Treal, kq_writer);
  }
  if (due && kq_writer && tid == 0) *group_ctr = 0;  // every member has counted in
  finish();
}

template <int DK, int DV, bool VERIFY, bool VARLEN>
hipError_t launch_t(const VerifyArgs &va, const FlushArgs &fa, int num_reqs, int hv, int cap,
                    hipStream_t stream) {
  constexpr int NT = 2;
  const dim3 grid(num_reqs * hv), block(64 * (DV / (16 * NT)));
  if (cap <= kCh)
    hipLaunchKernelGGL((replay_single<DK, DV, NT, VERIFY, VARLEN>), grid, block, 0, stream, va,
                       fa);
  else
    hipLaunchKernelGGL((replay_chunked<DK, DV, NT, VERIFY, VARLEN>), grid, block, 0, stream, va,
                       fa);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_flush_fused(const VerifyArgs &a, int min_len, hipStream_t stream) {
  constexpr int NT = 2;
  const dim3 grid(a.num_reqs * a.c.hv);
  const bool varlen = a.draft_lens != nullptr, rollback = a.prev_accepted != nullptr;
  const bool norm = a.norm_q != nullptr;
  if (norm && !rollback) return hipErrorInvalidValue;  // the norm rides on the one-call step
  auto go = [&](auto kernel, int dv) {
    hipLaunchKernelGGL(kernel, grid, dim3(64 * (dv / (16 * NT))), 0, stream, a, min_len);
  };
  // (VARLEN, ROLLBACK, NORM) instantiations; the kernel without the rollback
  // and the norm keeps its own code
  auto pick = [&](auto dk) {
    constexpr int D = decltype(dk)::value;
    if (norm)
      varlen ? go(replay_fused<D, D, NT, true, true, true>, D)
             : go(replay_fused<D, D, NT, false, true, true>, D);
    else if (rollback)
      varlen ? go(replay_fused<D, D, NT, true, true, false>, D)
             : go(replay_fused<D, D, NT, false, true, false>, D);
    else
      varlen ? go(replay_fused<D, D, NT, true, false, false>, D)
             : go(replay_fused<D, D, NT, false, false, false>, D);
  };
  if (a.c.dk == 128)
    pick(std::integral_constant<int, 128>());
  else if (a.c.dk == 64)
    pick(std::integral_constant<int, 64>());
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_verify_flush_long(const VerifyArgs &a, int min_len, hipStream_t stream) {
  constexpr int NT = 2;
  const dim3 grid(a.num_reqs * a.c.hv);
  const bool varlen = a.draft_lens != nullptr, rollback = a.prev_accepted != nullptr;
  if (a.norm_q) return hipErrorInvalidValue;  // the norm rides on single-chunk replays only
  auto go = [&](auto kernel, int dv) {
    hipLaunchKernelGGL(kernel, grid, dim3(64 * (dv / (16 * NT))), 0, stream, a, min_len);
  };
  auto pick = [&](auto dk) {
    constexpr int D = decltype(dk)::value;
    if (rollback)
      varlen ? go(replay_fused_long<D, D, NT, true, true>, D)
             : go(replay_fused_long<D, D, NT, false, true>, D);
    else
      varlen ? go(replay_fused_long<D, D, NT, true, false>, D)
             : go(replay_fused_long<D, D, NT, false, false>, D);
  };
  if (a.c.dk == 128)
    pick(std::integral_constant<int, 128>());
  else if (a.c.dk == 64)
    pick(std::integral_constant<int, 64>());
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

bool fused_long_supported(int dk, int dv, bool in_f32, int draft, int cap) {
  return chunked_supported(dk, dv, in_f32, draft) && cap > kCh;
}

bool fused_supported(int dk, int dv, bool in_f32, int draft, int cap) {
  return chunked_supported(dk, dv, in_f32, draft) && cap <= kCh;
}

bool chunked_supported(int dk, int dv, bool in_f32, int draft) {
  return !in_f32 && dk == dv && (dk == 64 || dk == 128) && draft <= kCh;
}

hipError_t launch_verify_chunked(const VerifyArgs &a, hipStream_t stream) {
  FlushArgs none{};
  const int R = a.num_reqs, HV = a.c.hv, C = a.c.cap;
  if (a.draft_lens) {
    if (a.c.dk == 128) return launch_t<128, 128, true, true>(a, none, R, HV, C, stream);
    if (a.c.dk == 64) return launch_t<64, 64, true, true>(a, none, R, HV, C, stream);
  } else {
    if (a.c.dk == 128) return launch_t<128, 128, true, false>(a, none, R, HV, C, stream);
    if (a.c.dk == 64) return launch_t<64, 64, true, false>(a, none, R, HV, C, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_flush_chunked(const FlushArgs &a, hipStream_t stream) {
  VerifyArgs none{};
  if (a.c.dk == 128)
    return launch_t<128, 128, false, false>(none, a, a.num_reqs, a.c.hv, a.c.cap, stream);
  if (a.c.dk == 64)
    return launch_t<64, 64, false, false>(none, a, a.num_reqs, a.c.hv, a.c.cap, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdnr
