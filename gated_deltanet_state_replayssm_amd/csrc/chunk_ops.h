// Building blocks of the chunked (WY / UT form) replay kernels for gfx950.
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
#pragma once

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace gdnr {

namespace {


constexpr int kCh = kChunkTokens;  // tokens per chunk
// Split output chunk: when a single-chunk replay has at most 16 committed
// tokens and at most 16 draft tokens, the committed rows sit at rows 0 .. B - 1,
// the draft at rows 16 .. 16 + D - 1, and the rows between are empty (k = q =
// v = 0, beta = 0, alpha = 1): such a row adds nothing to A, W, the decays or
// the products, so every output is unchanged, and the draft's outputs lie in
// the second 16-row tile: the output products and the fused norm's per-row
// reductions skip the first.
constexpr int kGapRow = kCh / 2;
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

// The LDS of the long replays: the arrays of Smem as LDS variables of their
// own, seen through a view per key buffer. Keys, values, alpha and beta arrive
// by LDS DMA while other arrays are read; the compiler waits for an LDS DMA
// before every LDS access it cannot tell apart from the DMA's writes, and it
// tells accesses to other variables apart, so each DMA target is a variable of
// its own. Two key buffers (each chunk's keys land in one while the previous
// chunk reads the other); the fold reads the transposed keys straight from the
// token-major rows (rd_kt_tr), so there is no transposed copy, and the output
// chunk's queries take the key buffer the chunk does not use.
struct SmemMats {
  float T[kCh][kCh + kPadF];
  float Cm[kCh][kCh + kPadF];
  float gam[kCh];
  float lg[kCh];
  float lgc[kCh];
};
template <int DK, int DV>
struct SmemLong {
  uint16_t (&k)[kCh][DK + kPadK];
  uint16_t (&q)[kCh][DK + kPadK];
  uint16_t (&v)[kCh][DV + kPadK];
  float (&T)[kCh][kCh + kPadF];
  float (&Cm)[kCh][kCh + kPadF];
  float (&gam)[kCh];
  float (&bet)[kCh];
  float (&alp)[kCh];
  float (&lg)[kCh];
  float (&lgc)[kCh];
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

// The A operand of K^T for key columns 16 mt + l16 (rows of the fold's
// product) in the token order of tok_operand (tokens 4g + {0..3}, then
// 16 + 4g + {0..3}), read from token-major key rows by two transposing LDS
// reads (ds_read_b64_tr_b16). Within each 16-lane group, lane a passes the
// address of 4 keys (row 4g + a / 4, columns 16 mt + 4 (a mod 4) ..); lane i
// receives element i mod 4 of lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4, i.e. column 16 mt + i of rows 4g .. 4g + 3.
template <int W>
__device__ __forceinline__ bf16x8 rd_kt_tr(const uint16_t (*m)[W], int mt, int g, int l16) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 *lds_ptr;
  const int r = 4 * g + (l16 >> 2), c = 16 * mt + 4 * (l16 & 3);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)&m[r][c]);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)&m[16 + r][c]);
  const s16x4 v[2] = {a, b};
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
                                   uint32_t draft_row, bool gap = false) {
    int tok = t0 + t;
    bool real = t < Treal;
    if (gap) {  // split output chunk (t0 = 0): see kGapRow
      const bool dr = t >= kGapRow;
      tok = dr ? t - kGapRow + u.B : t;
      real = dr ? tok < u.T : t < u.B;
    }
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
                                       bool out_chunk, bool gap = false) {
    const int tid = opaque_tid();
#pragma unroll
    for (int it = 0; it < IK; ++it) {
      const int p = tid + it * THREADS, t = p / PK, part = p % PK;
      const RowAt<VERIFY> at(u, t0, t, Treal, DK * 2, sr.dk_row, gap);
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
      const RowAt<VERIFY> at(u, t0, t, Treal, DV * 2, sr.dv_row, gap);
      if constexpr (VERIFY)
        vv[it] = bload_rd<u32x4>(at.ring != kOOB, sr.rv, at.ring + part * 16, sr.dv,
                                 at.draft + part * 16);
      else
        vv[it] = bload<u32x4>(sr.rv, at.ring + part * 16);
    }
    const int t = tid & (kCh - 1);
    const RowAt<VERIFY> at(u, t0, t, Treal, 4, sr.dab_row, gap);
    if constexpr (VERIFY) {
      al = bload_rd<float>(at.ring != kOOB, sr.ra, at.ring, sr.da, at.draft);
      be = bload_rd<float>(at.ring != kOOB, sr.rb, at.ring, sr.db, at.draft);
    } else {
      al = bload<float>(sr.ra, at.ring);
      be = bload<float>(sr.rb, at.ring);
    }
  }

  // KT: write the transposed keys of a folded chunk (kernels whose fold reads
  // them from the rows do not keep them)
  // (gapB >= 0: a split output chunk with gapB committed and gapD draft rows)
  template <bool KT = true, class SM>
  __device__ __forceinline__ void store(SM &sm, int Treal, bool out_chunk, int gapB = -1,
                                        int gapD = 0) {
    const int tid = opaque_tid();
#pragma unroll
    for (int it = 0; it < IK; ++it) {
      const int p = tid + it * THREADS, t = p / PK, part = p % PK;
      const u32x4 k = kv[it];
      *reinterpret_cast<u32x4 *>(&sm.k[t][part * 8]) = k;
      if (out_chunk) {
        *reinterpret_cast<u32x4 *>(&sm.q[t][part * 8]) = qv[it];
      } else if constexpr (KT) {
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
    {  // padding rows (and a split chunk's empty rows): alpha = 1, beta = 0 (read as 0)
      const int t = tid & (kCh - 1);
      const bool pad = gapB < 0 ? t >= Treal : (t < kGapRow ? t >= gapB : t - kGapRow >= gapD);
      if (pad) al = 1.f;
    }
    if (tid < kCh) {
      sm.alp[tid] = al;
      sm.bet[tid] = be;
    }
  }

  // Verify's output chunk: write the draft rows to ring slots (head + B + j) mod C,
  // from LDS (one workgroup per key head writes k and q).
  template <class SM>
  __device__ __forceinline__ void append(const SM &sm, const Srcs &sr, const Unit &u,
                                         int t0, int Treal, bool kq_writer,
                                         bool gap = false, int tid0 = 0) const {
    const int tid = opaque_tid() - tid0;  // threads tid0 .. tid0 + THREADS - 1
    // Recompute the row offsets here rather than keep those of the loads alive
    // in registers through the whole kernel: the copy of the unit is opaque to
    // the compiler, so it cannot reuse them.
    Unit u2 = u;
    asm volatile("" : "+v"(u2.head));
    if (kq_writer) {
#pragma unroll
      for (int it = 0; it < IK; ++it) {
        const int p = tid + it * THREADS, t = p / PK, part = p % PK;
        const RowAt<VERIFY> at(u2, t0, t, Treal, DK * 2, sr.dk_row, gap);
        bstore(*reinterpret_cast<const u32x4 *>(&sm.k[t][part * 8]), sr.rk, at.append + part * 16);
        bstore(*reinterpret_cast<const u32x4 *>(&sm.q[t][part * 8]), sr.rq, at.append + part * 16);
      }
    }
#pragma unroll
    for (int it = 0; it < IV; ++it) {
      const int p = tid + it * THREADS, t = p / PV, part = p % PV;
      const RowAt<VERIFY> at(u2, t0, t, Treal, DV * 2, sr.dv_row, gap);
      bstore(*reinterpret_cast<const u32x4 *>(&sm.v[t][part * 8]), sr.rv, at.append + part * 16);
    }
    if (tid < kCh) {
      const RowAt<VERIFY> at(u2, t0, tid, Treal, 4, sr.dab_row, gap);
      bstore(sm.alp[tid], sr.ra, at.append);
      bstore(sm.bet[tid], sr.rb, at.append);
    }
  }
};

// ---- Staging the next chunk while the current one is computed (long replays)
//
// A barrier for LDS traffic only: this wave's LDS accesses are complete
// (lgkmcnt) and no wave passes before all arrive. __syncthreads() also waits
// for every LDS DMA this wave has in flight (its workgroup-scope release covers
// writes to LDS by DMA), which would end the overlap the DMA is for. The
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One LDS DMA load: 16 bytes per lane from a buffer resource straight into LDS,
// lane l writing bytes [16 l, 16 l + 16) from lds (uniform across the wave); no
// registers are written and the wave runs on. An offset past the resource's
// end writes zeros; lanes switched off leave LDS untouched.
template <int AUX>
__device__ __forceinline__ void dma16(Rsrc r, char *lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                           voff, 0, 0, AUX);
}

// Rows 0 .. kCh - 1 of a padded token-major bf16 array [kCh][W + kPadK] in LDS
// by LDS DMA, the instructions dealt to waves [0, NW) (wv: the caller's wave,
// uniform). Instruction i writes the array's bytes [1024 i, 1024 i + 1024):
// lane l the 16-byte piece p = 64 i + l, which is piece p mod PR of row p / PR
// (PR pieces per row, the last one the row's padding: data = false, read from
// nowhere). Lanes past the array's end are switched off. src(t, pc, dst, data)
// issues the load of piece pc of row t.
template <int W, int NW, typename F>
__device__ __forceinline__ void dma_rows(uint16_t (*rows)[W + kPadK], int wv, int lane, F &&src) {
  static_assert((W + kPadK) % 8 == 0, "rows of whole 16-byte pieces");
  constexpr int PR = (W + kPadK) / 8, NP = kCh * PR, NI = (NP + 63) / 64;
  char *base = reinterpret_cast<char *>(&rows[0][0]);
  // every instruction's LDS address a constant offset into the array, so that
  // the compiler sees which LDS reads the DMA cannot touch (it waits for the
  // DMA before any LDS access it cannot tell apart)
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i % NW == wv) {
      const int p = 64 * i + lane;
      if (NP % 64 == 0 || i < NI - 1 || p < NP) {
        const int t = p / PR, pc = p - t * PR;
        src(t, pc, base + 1024 * i, pc < PR - 1);
      }
    }
  }
}

// One LDS DMA load of 4 bytes per lane (lane l writes lds + 4 l).
template <int AUX>
__device__ __forceinline__ void dma4(Rsrc r, char *lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4,
                                           voff, 0, 0, AUX);
}

// The staging of one chunk (rows [t0, t0 + Treal) of a token stream) issued
// while the previous chunk is computed, all of it by LDS DMA (no registers stay
// in flight across the chunk loop): keys, beta and alpha into the buffers the
// current chunk does not use, values once W has read the previous values,
// queries (output chunk) once the last fold has read the keys in their buffer.
// Rows past Treal, and committed rows' queries, come in as zeros (a reader
// takes alpha = 1 past Treal). The caller's barriers while the DMA is in flight
// are lds_barrier(); the next __syncthreads() waits for it.
// RING: every row of the chunk is a committed ring row (a folded chunk: the
// draft is always in the stream's last chunk), so each piece has one source
// and no lane takes the draft's branch.
template <int DK, int DV, int NW>
struct Prefetch {
  template <bool RING = false, class SM>
  __device__ __forceinline__ void issue_k(SM &sm, const Srcs &sr, const Unit &u, int t0,
                                          int Treal) const {
    const int tid = opaque_tid(), lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    dma_rows<DK, NW>(sm.k, wv, lane, [&](int t, int pc, char *dst, bool data) {
      const RowAt<true> at(u, t0, t, Treal, DK * 2, sr.dk_row);
      if constexpr (RING)
        dma16<0>(sr.rk, dst, data ? at.ring + pc * 16 : kOOB);
      else if (data && at.ring != kOOB)
        dma16<0>(sr.rk, dst, at.ring + pc * 16);
      else
        dma16<kStream>(sr.dk, dst, data ? at.draft + pc * 16 : kOOB);
    });
  }

  template <bool RING = false, class SM>
  __device__ __forceinline__ void issue_v(SM &sm, const Srcs &sr, const Unit &u, int t0,
                                          int Treal) const {
    const int tid = opaque_tid(), lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    dma_rows<DV, NW>(sm.v, wv, lane, [&](int t, int pc, char *dst, bool data) {
      const RowAt<true> at(u, t0, t, Treal, DV * 2, sr.dv_row);
      if constexpr (RING)
        dma16<0>(sr.rv, dst, data ? at.ring + pc * 16 : kOOB);
      else if (data && at.ring != kOOB)
        dma16<0>(sr.rv, dst, at.ring + pc * 16);
      else
        dma16<kStream>(sr.dv, dst, data ? at.draft + pc * 16 : kOOB);
    });
  }

  // beta then alpha of the chunk's rows (sm.bet and sm.alp adjacent): lane
  // l < 32 beta of row l, lane 32 + l alpha of row l; by the last wave
  template <bool RING = false, class SM>
  __device__ __forceinline__ void issue_ab(SM &sm, const Srcs &sr, const Unit &u, int t0,
                                           int Treal) const {
    const int tid = opaque_tid(), lane = tid & 63;
    if (__builtin_amdgcn_readfirstlane(tid >> 6) == NW - 1) {
      const int t = lane & (kCh - 1);
      const RowAt<true> at(u, t0, t, Treal, 4, sr.dab_row);
      char *dst = reinterpret_cast<char *>(&sm.bet[0]);
      if (RING || at.ring != kOOB) {
        if (lane < kCh)
          dma4<0>(sr.rb, dst, at.ring);
        else
          dma4<0>(sr.ra, dst, at.ring);
      } else {
        if (lane < kCh)
          dma4<kStream>(sr.db, dst, at.draft);
        else
          dma4<kStream>(sr.da, dst, at.draft);
      }
    }
  }

  // the output chunk's queries (draft rows only)
  template <class SM>
  __device__ __forceinline__ void issue_q(SM &sm, const Srcs &sr, const Unit &u, int t0,
                                          int Treal) const {
    const int tid = opaque_tid(), lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    dma_rows<DK, NW>(sm.q, wv, lane, [&](int t, int pc, char *dst, bool data) {
      const RowAt<true> at(u, t0, t, Treal, DK * 2, sr.dk_row);
      dma16<kStream>(sr.dq, dst, data ? at.draft + pc * 16 : kOOB);
    });
  }
};

// A chunk's keys, beta and alpha from the buffers the DMA fills to those the
// chunk is computed from, by the NTHR threads j = 0 .. NTHR - 1 of the caller's
// numbering (16 bytes a copy).
template <int DK, int NTHR>
__device__ __forceinline__ void copy_chunk_keys(const uint16_t (&kn)[kCh][DK + kPadK],
                                                uint16_t (&kc)[kCh][DK + kPadK],
                                                const float (&abn)[2][kCh], float (&abc)[2][kCh],
                                                int j) {
  constexpr int PK = (DK + kPadK) / 8, NK = kCh * PK, NA = 2 * kCh / 4;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(&kn[0][0]);
  u32x4 *dst = reinterpret_cast<u32x4 *>(&kc[0][0]);
#pragma unroll
  for (int it = 0; it < (NK + NTHR - 1) / NTHR; ++it) {
    const int p = j + it * NTHR;
    if (NK % NTHR == 0 || p < NK) dst[p] = src[p];
  }
  if (j < NA)
    reinterpret_cast<u32x4 *>(&abc[0][0])[j] = reinterpret_cast<const u32x4 *>(&abn[0][0])[j];
}

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

// 2^x by the hardware instruction (v_exp_f32). The decays' exponents are
// differences of clamped log2 prefix sums, x <= 0 up to rounding; results below
// 2^-126 (flushed or denormal) are negligible next to the terms they multiply.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

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
      Lv[b][i] = (j <= t) ? exp2_hw(lgv[ta][i] - lgc[tb]) : 0.f;
    }
}

// C = L o (Q K^T), lower triangle including the diagonal (output chunk only).
// Built by another wave than A and its inverse, from its own decay scan (kept
// in sm.lgc), so the two run side by side; it writes only sm.Cm and sm.lgc.
template <int DK, int DV, class SM>
__device__ __forceinline__ void build_c(SM &sm, float al_staged, int lane, int g, int l16) {
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
template <int DK, int DV, class SM>
__device__ __forceinline__ void build_tt(SM &sm, float al_staged, int lane, int g, int l16) {
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
  // ---- (I + A)^-1 in place, as T = [[T00, 0], [T10, T11]] with T00, T11 the
  // inverses of the 16 x 16 diagonal blocks and T10 = -T11 (A10 T00).
  // The diagonal blocks by forward substitution, one lane per column (lane
  // 16 b + c: column c of block b): x_r = [r == c] - sum_{m < r} A[r][m] x_m,
  // with x_m = 0 above the diagonal, so every lane runs the same unrolled
  // recurrence. The rows of A are read (broadcast) before the block is
  // overwritten (one wave, LDS accesses in program order).
  if (lane < 2 * 16) {
    const int b = lane >> 4, c = lane & 15, r0 = 16 * b;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float row[16];
#pragma unroll
      for (int q = 0; q < (r + 3) / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(&sm.T[r0 + r][r0 + 4 * q]);
        row[4 * q] = v.x;
        row[4 * q + 1] = v.y;
        row[4 * q + 2] = v.z;
        row[4 * q + 3] = v.w;
      }
      // two partial sums halve the dependent chain
      float s0 = r == c ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) {
        if (m & 1)
          s1 = fmaf(-row[m], x[m], s1);
        else
          s0 = fmaf(-row[m], x[m], s0);
      }
      x[r] = s0 + s1;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.T[r0 + r][r0 + c] = x[r];
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
// (A split output chunk needs only Z's second tile; skipping the first, at run
// time or in a second pass, measured no faster and the second pass spilled.)
template <int DK, int DV, int NT, int WHAT, class SM>
__device__ __forceinline__ void contract(const SM &sm,
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
template <int DK, int DV, int NT, class SM>
__device__ __forceinline__ void solve_w(const SM &sm, const f32x4 (&Y)[2][NT], int colL,
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

// The output chunk's outputs need W only through C W = C (I + A)^-1 diag(beta)
// (V - diag(gamma) Y): M = C (I + A)^-1 diag(beta) depends on the inputs alone,
// so it is formed once the T x T matrices are built (ahead of the state) and
// then O = gamma Z + M X' with X' = V - diag(gamma) Y, one product after the
// contraction instead of two. build_m: one wave, M into sm.Cm (in place: every
// read of Cm and T precedes the writes, LDS accesses of a wave in program
// order). Tiles (0,0), (1,0), (1,1) (tile (0,1) of C, and so of M, is zero);
// fp32 operands split into hi + lo bf16 as in the other products.
template <int DK, int DV, class SM>
__device__ __forceinline__ void build_m(SM &sm, int g, int l16) {
  bf16x8 ch[2], cl[2], th[2], tl[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    float crow[8], tcol[8];
    rd_frow(sm.Cm, 16 * a + l16, g, crow);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tcol[j] = sm.T[4 * g + j][16 * a + l16];
      tcol[4 + j] = sm.T[16 + 4 * g + j][16 * a + l16];
    }
    split8(crow, ch[a], cl[a]);
    split8(tcol, th[a], tl[a]);
  }
  float bcol[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) bcol[b] = sm.bet[16 * b + l16];
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int ta = b == 0 ? 0 : 1, tb = b == 2 ? 1 : 0;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma(ch[ta], th[tb], acc);
    acc = mfma(ch[ta], tl[tb], acc);
    acc = mfma(cl[ta], th[tb], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.Cm[16 * ta + 4 * g + i][16 * tb + l16] = acc[i] * bcol[tb];
  }
}

// X' = V - gamma Y (the output chunk's operand of M); this lane's entries as in
// solve_w.
template <int DK, int DV, int NT, class SM>
__device__ __forceinline__ void x_prime(const SM &sm, const f32x4 (&Y)[2][NT], int colL, int g,
                                        f32x4 (&Xm)[2][NT]) {
  typedef typename Cols<NT>::U U;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ga = sm.gam[16 * a + 4 * g + i];
      const U vv = *reinterpret_cast<const U *>(&sm.v[16 * a + 4 * g + i][colL]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Xm[a][nt][i] = bf16_to_f32(vv[nt]) - ga * Y[a][nt][i];
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
template <int DK, int DV, int NT, class SM>
__device__ __forceinline__ void emit_outputs(const SM &sm, const f32x4 (&Z)[2][NT],
                                             const f32x4 (&Wm)[2][NT], int g, int l16, int t0,
                                             int Treal, int B, Rsrc out, uint32_t col_off,
                                             uint32_t row_bytes, int a0 = 0) {
  typedef typename Cols<NT>::F F;
  asm volatile("" : "+v"(B));  // recompute the row offsets here (see Stage::append)
  bf16x8 wh[NT], wl[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tok_operand(Wm[0][nt], Wm[1][nt], wh[nt], wl[nt]);
  float crow[2][8], ga[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (a < a0) continue;  // a split chunk: no draft rows in tile 0
    rd_frow(sm.Cm, 16 * a + l16, g, crow[a]);
#pragma unroll
    for (int i = 0; i < 4; ++i) ga[a][i] = sm.gam[16 * a + 4 * g + i];
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (a < a0) continue;  // a split chunk: no draft rows in tile 0
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

// Fold the chunk into the state: H <- gamma_T H + K^T (L[T-1] o W).
// TR: the transposed keys come from the key rows by transposing reads (no kt).
template <int DK, int DV, int NT, bool TR = false, class SM>
__device__ __forceinline__ void fold_state(const SM &sm, const f32x4 (&Wm)[2][NT], int g,
                                           int l16, typename Cols<NT>::F (&H)[DK / 16][4]) {
  constexpr int MT = DK / 16;
  const float gT = sm.gam[kCh - 1], lg31 = sm.lg[kCh - 1];
  bf16x8 wh[NT], wl[NT];
  {
    float lt[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) lt[a][i] = exp2_hw(lg31 - sm.lg[16 * a + 4 * g + i]);
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
    bf16x8 kt;
    if constexpr (TR)
      kt = rd_kt_tr(sm.k, mt, g, l16);
    else
      kt = rd_row(sm.kt, 16 * mt + l16, 4 * g);
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

}  // namespace

}  // namespace gdnr
