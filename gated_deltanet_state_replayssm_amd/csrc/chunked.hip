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

template <int DK>
struct Smem {
  uint16_t k[kCh][DK + kPadK];     // chunk keys, token-major (bf16 bits)
  union {
    uint16_t q[kCh][DK + kPadK];   // output chunk: queries (draft rows, zero elsewhere)
    uint16_t kt[DK][kCh + kPadT];  // folded chunk: keys, transposed
  };
  float A[kCh][kCh + kPadF];       // beta_t L[t][i] (k_t . k_i), strictly lower;
                                   // its upper-right block is scratch for the inverse
  float Ti[kCh][kCh + kPadF];      // (I + A)^-1
  float Cm[kCh][kCh + kPadF];      // L[t][i] (q_t . k_i), lower incl. diagonal
  float gam[kCh], bet[kCh], alp[kCh];
  float lg[kCh];                   // log2(alpha_0 ... alpha_t), each log clamped at -126
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

struct Unit {
  int r, h, s, kh, head, B, T, C;
};

// Chunk rows [t0, t0 + Treal) of the token stream (B committed ring tokens,
// then the draft when verifying), loaded in two phases: load() issues every
// global load into registers, store() writes LDS rows 0 .. Treal-1 (zero rows
// after) and, for verify, appends the draft rows to the ring. The output chunk
// (verify's last, which holds the whole draft) stages the queries; a folded
// chunk stages the transposed keys instead. v stays in registers: each lane
// keeps its NT columns of its 8 token rows 16 a + 4 g + i.
// Per-workgroup base pointers of everything a chunk reads or appends (uniform,
// computed once); rows are then addressed with 32-bit element offsets.
struct Bases {
  const uint16_t *rk, *rv, *dk, *dq, *dv;  // ring k / v rows; draft k / q / v rows
  uint16_t *wk, *wq, *wv;                  // ring rows written by the append
  const float *ra, *rb, *da, *db;          // ring / draft alpha and beta
  float *wa, *wb;
  int dk_stride, dv_stride, dab_stride;    // draft row strides (elements)
};

template <int DK, int DV>
__device__ __forceinline__ Bases make_bases(const CacheView &c, const Unit &u,
                                            const VerifyArgs *va, bool verify) {
  const int C = u.C, HV = c.hv, HK = c.hk;
  Bases b;
  const int64_t kq_row0 = (int64_t)(u.s * HK + u.kh) * C;
  const int64_t vh_row0 = (int64_t)(u.s * HV + u.h) * C;
  b.wk = static_cast<uint16_t *>(c.ring_k) + kq_row0 * DK;
  b.wq = c.ring_q ? static_cast<uint16_t *>(c.ring_q) + kq_row0 * DK : nullptr;
  b.wv = static_cast<uint16_t *>(c.ring_v) + vh_row0 * DV;
  b.wa = c.ring_alpha + vh_row0;
  b.wb = c.ring_beta + vh_row0;
  b.rk = b.wk;
  b.rv = b.wv;
  b.ra = b.wa;
  b.rb = b.wb;
  b.dk = b.dq = b.dv = nullptr;
  b.da = b.db = nullptr;
  b.dk_stride = HK * DK;
  b.dv_stride = HV * DV;
  b.dab_stride = HV;
  if (verify) {
    const int64_t d0 = (int64_t)u.r * va->draft;
    b.dk = static_cast<const uint16_t *>(va->k) + (d0 * HK + u.kh) * DK;
    b.dq = static_cast<const uint16_t *>(va->q) + (d0 * HK + u.kh) * DK;
    b.dv = static_cast<const uint16_t *>(va->v) + (d0 * HV + u.h) * DV;
    b.da = va->alpha + d0 * HV + u.h;
    b.db = va->beta + d0 * HV + u.h;
  }
  return b;
}

// Chunk rows [t0, t0 + Treal) of the token stream (B committed ring tokens,
// then the draft when verifying), loaded in two phases: load() issues every
// global load into registers, store() writes LDS rows 0 .. Treal-1 (zero rows
// after) and, for verify, appends the draft rows to the ring. The output chunk
// (verify's last, which holds the whole draft) stages the queries; a folded
// chunk stages the transposed keys instead. v stays in registers: each lane
// keeps its NT columns of its 8 token rows 16 a + 4 g + i.
template <int DK, int DV, int NT, bool VERIFY>
struct Stage {
  static constexpr int THREADS = 64 * (DV / (16 * NT));
  static constexpr int PARTS = DK / 8;  // 16-byte pieces per key row
  static constexpr int ITER = kCh * PARTS / THREADS;
  static_assert(kCh * PARTS % THREADS == 0, "key pieces per thread");
  typedef typename Cols<NT>::U U;

  uint4 kv[ITER], qv[ITER];
  float al, be;
  U vv[2][4];
  uint32_t ok_k, ok_q, ok_v;  // per-item "real row" bits (padding rows are zero)
  bool ok_a;

  // Chunk token t as a source: ring position (committed) or draft index.
  // Padding rows (t >= Treal) read token 0 of the stream, which always exists,
  // so every load below is unconditional and in bounds.
  struct Src {
    bool ring;
    int pos, j;
  };
  __device__ __forceinline__ static Src src_of(const Unit &u, int t0, int t, int Treal) {
    const int tok = (t < Treal) ? t0 + t : 0;
    Src r;
    r.ring = !VERIFY || tok < u.B;
    const int pos = u.head + tok;
    r.pos = pos - (pos >= u.C ? u.C : 0);
    r.j = r.ring ? 0 : tok - u.B;
    return r;
  }

  __device__ __forceinline__ void load(const Bases &bs, const Unit &u, int t0, int Treal,
                                       bool out_chunk, int colL, int g) {
    const int tid = threadIdx.x;
    ok_k = ok_q = ok_v = 0u;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int p = tid + it * THREADS, t = p / PARTS, part = p % PARTS;
      const Src sr = src_of(u, t0, t, Treal);
      const uint16_t *src = bs.rk + sr.pos * DK + part * 8;
      if constexpr (VERIFY) {
        const int doff = sr.j * bs.dk_stride + part * 8;
        if (!sr.ring) src = bs.dk + doff;
        if (out_chunk) {
          qv[it] = *reinterpret_cast<const uint4 *>(bs.dq + doff);
          ok_q |= (t < Treal && !sr.ring) ? (1u << it) : 0u;
        }
      }
      kv[it] = *reinterpret_cast<const uint4 *>(src);
      ok_k |= (t < Treal) ? (1u << it) : 0u;
    }
    {
      const int t = tid & (kCh - 1);
      const Src sr = src_of(u, t0, t, Treal);
      const float *pa = bs.ra + sr.pos, *pb = bs.rb + sr.pos;
      if constexpr (VERIFY) {
        if (!sr.ring) {
          pa = bs.da + sr.j * bs.dab_stride;
          pb = bs.db + sr.j * bs.dab_stride;
        }
      }
      al = *pa;
      be = *pb;
      ok_a = t < Treal;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * a + 4 * g + i;
        const Src sr = src_of(u, t0, t, Treal);
        const uint16_t *src = bs.rv + sr.pos * DV + colL;
        if constexpr (VERIFY) {
          if (!sr.ring) src = bs.dv + sr.j * bs.dv_stride + colL;
        }
        vv[a][i] = *reinterpret_cast<const U *>(src);
        ok_v |= (t < Treal) ? (1u << (4 * a + i)) : 0u;
      }
    }
  }

  // Zero the padding rows and write LDS; verify appends the draft rows it holds.
  __device__ __forceinline__ void store(Smem<DK> &sm, const Bases &bs, const Unit &u, int t0,
                                        int Treal, bool out_chunk, int colL, int g, int G) {
    const int tid = threadIdx.x;
    const uint4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int p = tid + it * THREADS, t = p / PARTS, part = p % PARTS;
      const uint4 k = (ok_k >> it & 1u) ? kv[it] : zero;
      *reinterpret_cast<uint4 *>(&sm.k[t][part * 8]) = k;
      if (out_chunk) {
        const uint4 q = (ok_q >> it & 1u) ? qv[it] : zero;
        *reinterpret_cast<uint4 *>(&sm.q[t][part * 8]) = q;
        if constexpr (VERIFY) {  // one workgroup per key head appends k and q
          if ((ok_q >> it & 1u) && u.h % G == 0) {
            const Src sr = src_of(u, t0, t, Treal);
            const int off = sr.pos * DK + part * 8;
            *reinterpret_cast<uint4 *>(bs.wk + off) = k;
            if (bs.wq) *reinterpret_cast<uint4 *>(bs.wq + off) = q;
          }
        }
      } else {
        const uint32_t w[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.kt[part * 8 + 2 * e][t] = (uint16_t)(w[e] & 0xffffu);
          sm.kt[part * 8 + 2 * e + 1][t] = (uint16_t)(w[e] >> 16);
        }
      }
    }
    if (!ok_a) {
      al = 1.f;  // padding rows: alpha = 1, beta = 0
      be = 0.f;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!(ok_v >> (4 * a + i) & 1u)) vv[a][i] = (U)0;
    if (tid < kCh) {
      sm.alp[tid] = al;
      sm.bet[tid] = be;
    }
    if constexpr (VERIFY) {
      if (out_chunk) {
        if (tid < kCh) {
          const Src sr = src_of(u, t0, tid, Treal);
          if (ok_a && !sr.ring) {
            bs.wa[sr.pos] = al;
            bs.wb[sr.pos] = be;
          }
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * a + 4 * g + i;
            const Src sr = src_of(u, t0, t, Treal);
            if ((ok_v >> (4 * a + i) & 1u) && !sr.ring)
              *reinterpret_cast<U *>(bs.wv + sr.pos * DV + colL) = vv[a][i];
          }
      }
    }
  }
};

// Inclusive scan over lanes 0..31 of a wave with DPP row shifts (within rows of
// 16 lanes) and a row broadcast of lane 15 into the second row. Lanes 32..63 get
// their own scan of lanes 32..63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or(float identity, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v),
                                                    CTRL, ROW_MASK, 0xf, false));
}
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

// The chunk's T x T matrices, built by one wave (no workgroup barriers inside:
// each step reads only what this wave wrote, in program order): decay table
// gamma and log2 gamma, A = beta L o (K K^T), C = L o (Q K^T) (output chunk) and
// (I + A)^-1. al_staged is this lane's staged alpha, of token lane % 32.
template <int DK>
__device__ __forceinline__ void build_tt(Smem<DK> &sm, float al_staged, int lane, int g, int l16,
                                         bool out_chunk) {
  constexpr int KS = DK / 32;
  // Reads, arithmetic and writes of each step below are kept in separate
  // groups: LDS reads are then issued back to back instead of one by one.
  //
  // ---- decays: gamma_t = alpha_0 ... alpha_t (product scan) and
  // lg_t = log2 gamma_t (sum scan of log2 alpha, clamped at -126 so that a zero
  // alpha stays finite); L[t][j] = alpha_{j+1} ... alpha_t = 2^(lg_t - lg_j).
  {
    const float lg2a = fmaxf(__log2f(al_staged), -126.f);
    const float lg = scan32_add(lg2a);
    const float gm = scan32_mul(al_staged);
    if (lane < kCh) {
      sm.lg[lane] = lg;
      sm.gam[lane] = gm;
    }
  }
  // ---- Gram matrices K K^T and Q K^T (exact bf16 products, fp32 sums)
  f32x4 Gm[3], Pm[3];  // tiles (0,0), (1,0), (1,1)
  {
    bf16x8 kr[KS][2], qr[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kr[ks][0] = rd_row(sm.k, l16, 32 * ks + 4 * g);
      kr[ks][1] = rd_row(sm.k, 16 + l16, 32 * ks + 4 * g);
      if (out_chunk) {
        qr[ks][0] = rd_row(sm.q, l16, 32 * ks + 4 * g);
        qr[ks][1] = rd_row(sm.q, 16 + l16, 32 * ks + 4 * g);
      }
    }
#pragma unroll
    for (int b = 0; b < 3; ++b) Gm[b] = Pm[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Gm[0] = mfma(kr[ks][0], kr[ks][0], Gm[0]);
      Gm[1] = mfma(kr[ks][1], kr[ks][0], Gm[1]);
      Gm[2] = mfma(kr[ks][1], kr[ks][1], Gm[2]);
      if (out_chunk) {
        Pm[0] = mfma(qr[ks][0], kr[ks][0], Pm[0]);
        Pm[1] = mfma(qr[ks][1], kr[ks][0], Pm[1]);
        Pm[2] = mfma(qr[ks][1], kr[ks][1], Pm[2]);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // ---- A = beta L o (K K^T) strictly lower, C = L o (Q K^T) lower; tile b of
  // (0,0), (1,0), (1,1) holds rows 16 ta + 4 g + i, column 16 tb + l16
  {
    float Lv[3][4], bv[2][4], lgv[2][4], lgc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      lgc[a] = sm.lg[16 * a + l16];
#pragma unroll
      for (int i = 0; i < 4; ++i) lgv[a][i] = sm.lg[16 * a + 4 * g + i];
    }
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ta = b == 0 ? 0 : 1, tb = b == 2 ? 1 : 0;
        const int t = 16 * ta + 4 * g + i, j = 16 * tb + l16;
        Lv[b][i] = (j <= t) ? exp2f(lgv[ta][i] - lgc[tb]) : 0.f;
      }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[a][i] = sm.bet[16 * a + 4 * g + i];
    float Av[4][4], Cv[4][4];
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ta = b == 0 ? 0 : 1, tb = b == 2 ? 1 : 0;
        const int t = 16 * ta + 4 * g + i, j = 16 * tb + l16;
        Av[b][i] = (j < t) ? bv[ta][i] * Lv[b][i] * Gm[b][i] : 0.f;
        Cv[b][i] = (j <= t) ? Lv[b][i] * Pm[b][i] : 0.f;
      }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ta = (b == 1 || b == 2) ? 1 : 0, tb = b >= 2 ? 1 : 0;
        const int t = 16 * ta + 4 * g + i, j = 16 * tb + l16;
        sm.A[t][j] = b == 3 ? 0.f : Av[b][i];
        if (out_chunk) sm.Cm[t][j] = b == 3 ? 0.f : Cv[b][i];
      }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // ---- (I + A)^-1 by recursive 2 x 2 blocking, T = [[T00, 0], [T10, T11]] with
  // T10 = -T11 (A10 T00): 4 x 4 diagonal blocks by forward substitution, then
  // 8 x 8 and 16 x 16 blocks on VALU, then the 32 x 32 level on MFMA. The
  // strictly upper triangle of A (zero, never read) holds the A10 T00 products.
  {
    // 4 x 4 diagonal blocks q = 0..7: lane = (q, column cc)
    const int q = (lane >> 2) & 7, cc = lane & 3, r0 = 4 * q;
    const float a10 = sm.A[r0 + 1][r0], a20 = sm.A[r0 + 2][r0], a21 = sm.A[r0 + 2][r0 + 1];
    const float a30 = sm.A[r0 + 3][r0], a31 = sm.A[r0 + 3][r0 + 1], a32 = sm.A[r0 + 3][r0 + 2];
    const float x0 = cc == 0 ? 1.f : 0.f;
    const float x1 = cc == 1 ? 1.f : (cc < 1 ? -a10 * x0 : 0.f);
    const float x2 = cc == 2 ? 1.f : (cc < 2 ? -(a20 * x0 + a21 * x1) : 0.f);
    const float x3 = cc == 3 ? 1.f : -(a30 * x0 + a31 * x1 + a32 * x2);
    if (lane < 32) {
      sm.Ti[r0][r0 + cc] = x0;
      sm.Ti[r0 + 1][r0 + cc] = x1;
      sm.Ti[r0 + 2][r0 + cc] = x2;
      sm.Ti[r0 + 3][r0 + cc] = x3;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  {
    // 8 x 8 blocks p = 0..3: lane = (p, i, j) over the 4 x 4 lower-left block
    const int p = lane >> 4, i = (lane >> 2) & 3, j = lane & 3, r0 = 8 * p;
    float av[4], tv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      av[k] = sm.A[r0 + 4 + i][r0 + k];
      tv[k] = sm.Ti[r0 + k][r0 + j];
    }
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = fmaf(av[k], tv[k], m);
    sm.A[r0 + i][r0 + 4 + j] = m;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    float t11[4], mv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      t11[k] = sm.Ti[r0 + 4 + i][r0 + 4 + k];
      mv[k] = sm.A[r0 + k][r0 + 4 + j];
    }
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) t = fmaf(t11[k], mv[k], t);
    sm.Ti[r0 + 4 + i][r0 + j] = -t;
    sm.Ti[r0 + i][r0 + 4 + j] = 0.f;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  {
    // 16 x 16 blocks b = 0, 1: lane = (b, i, j0) over the 8 x 8 lower-left block,
    // two columns j0 and j0 + 4 per lane
    const int b = lane >> 5, i = (lane >> 2) & 7, j0 = lane & 3, r0 = 16 * b;
    float av[8], tv[2][8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      av[k] = sm.A[r0 + 8 + i][r0 + k];
      tv[0][k] = sm.Ti[r0 + k][r0 + j0];
      tv[1][k] = sm.Ti[r0 + k][r0 + j0 + 4];
    }
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      m0 = fmaf(av[k], tv[0][k], m0);
      m1 = fmaf(av[k], tv[1][k], m1);
    }
    sm.A[r0 + i][r0 + 8 + j0] = m0;
    sm.A[r0 + i][r0 + 12 + j0] = m1;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    float t11[8], mv[2][8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      t11[k] = sm.Ti[r0 + 8 + i][r0 + 8 + k];
      mv[0][k] = sm.A[r0 + k][r0 + 8 + j0];
      mv[1][k] = sm.A[r0 + k][r0 + 12 + j0];
    }
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      t0 = fmaf(t11[k], mv[0][k], t0);
      t1 = fmaf(t11[k], mv[1][k], t1);
    }
    sm.Ti[r0 + 8 + i][r0 + j0] = -t0;
    sm.Ti[r0 + 8 + i][r0 + j0 + 4] = -t1;
    sm.Ti[r0 + i][r0 + 8 + j0] = 0.f;
    sm.Ti[r0 + i][r0 + 12 + j0] = 0.f;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  {
    // 16 x 16 products on MFMA with k = 4g + j (slots 4..7 zero), fp32
    // operands split into hi + lo bf16
    float xa[8], xb[8];
    const float4 arow = *reinterpret_cast<const float4 *>(&sm.A[16 + l16][4 * g]);
    const float4 trow = *reinterpret_cast<const float4 *>(&sm.Ti[16 + l16][16 + 4 * g]);
    float tcol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tcol[j] = sm.Ti[4 * g + j][l16];
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
    for (int i = 0; i < 4; ++i) sm.Ti[16 + 4 * g + i][l16] = -T1[i];
    *reinterpret_cast<float4 *>(&sm.Ti[l16][16 + 4 * g]) = float4{0.f, 0.f, 0.f, 0.f};
  }
  
}


enum { kY = 1, kZ = 2 };

// Y = K H and/or Z = Q H over d_k on MFMA, the state split into hi + lo bf16.
// Both products share one split per k-step; a Z-only pass splits with
// truncation so that it is never merged with (and kept alive from) a Y pass.
template <int DK, int NT, int WHAT>
__device__ __forceinline__ void contract(const Smem<DK> &sm,
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

// X = beta (V - gamma Y), then W = (I + A)^-1 X (3-pass split product).
template <int DK, int NT>
__device__ __forceinline__ void solve_w(const Smem<DK> &sm, const f32x4 (&Y)[2][NT],
                                        const typename Cols<NT>::U (&vv)[2][4], int g, int l16,
                                        f32x4 (&Wm)[2][NT]) {
  bf16x8 xh[NT], xl[NT];
  {
    float be[2][4], ga[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        be[a][i] = sm.bet[16 * a + 4 * g + i];
        ga[a][i] = sm.gam[16 * a + 4 * g + i];
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
  float trow[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a) rd_frow(sm.Ti, 16 * a + l16, g, trow[a]);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    bf16x8 th, tl;
    split8(trow[a], th, tl);
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

// Draft outputs O = gamma Z + C W of chunk rows t (token t0 + t >= B, t < Treal);
// out_base points at out[r][0][h][colL], rows D apart by tok_stride floats.
template <int DK, int NT>
__device__ __forceinline__ void emit_outputs(const Smem<DK> &sm, const f32x4 (&Z)[2][NT],
                                             const f32x4 (&Wm)[2][NT], int g, int l16, int t0,
                                             int Treal, int B, float *out_base,
                                             int64_t tok_stride) {
  typedef typename Cols<NT>::F F;
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
      if (t < Treal && tok >= B) {
        F o;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt] = O[nt][i];
        *reinterpret_cast<F *>(out_base + (tok - B) * tok_stride) = o;
      }
    }
  }
}

// Fold the chunk into the state: H <- gamma_T H + K^T (L[T-1] o W).
template <int DK, int NT>
__device__ __forceinline__ void fold_state(const Smem<DK> &sm, const f32x4 (&Wm)[2][NT], int g,
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

// One workgroup per (request, value head). VERIFY: outputs of the draft, state
// untouched. !VERIFY (flush): fold all committed tokens, write the state back,
// move the pointers. Chunks are cut from the end of the token stream so the
// last one (verify's output chunk) holds the whole draft (D <= 32).
//
// Per chunk: all threads stage the chunk's inputs; wave 0 builds the T x T
// matrices (decay table, Gram matrices, (I + A)^-1) using only wave-local LDS
// ordering while every wave computes Y = K H; after one barrier every wave
// forms X, W and either the draft outputs or the fold of its state columns.
template <int DK, int DV, int NT, bool VERIFY>
__global__ __launch_bounds__(64 * (DV / (16 * NT)), 2) void replay_chunked(VerifyArgs va,
                                                                           FlushArgs fa) {
  constexpr int WAVES = DV / (16 * NT);
  constexpr int MT = DK / 16;   // 16-row tiles of the state
  constexpr int KS = DK / 32;   // k-steps of a contraction over d_k
  static_assert(DK % 32 == 0 && DV % (16 * NT) == 0 && (NT == 2 || NT == 4), "tile shape");
  static_assert(WAVES >= 1, "at least one wave");
  typedef typename Cols<NT>::F F;
  __shared__ Smem<DK> sm;

  const CacheView &c = VERIFY ? va.c : fa.c;
  const int HV = c.hv;
  const int r = blockIdx.x / HV, h = blockIdx.x % HV;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane >> 4, l16 = lane & 15;
  const int colL = wave * 16 * NT + NT * l16;  // this lane's first state column
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
    if (n + va.draft > C) {
      if (lead) raise_err(c.err, GDN_DERR_CAPACITY);
      return;
    }
    T = n + va.draft;
  } else {
    if (n < max(fa.min_len, 1)) return;  // not due: nothing is written
    T = n;
  }
  const Unit u{r, h, s, h / (HV / c.hk), head, n, T, C};
  const int nchunks = (T + kCh - 1) / kCh;
  const int T0 = T - kCh * (nchunks - 1);  // tokens in the first chunk (1..32)
  float *st = c.state + ((int64_t)s * HV + h) * DK * DV;

  // ---- first chunk's small inputs, then the whole state tile: waiting for the
  // former (loads complete in issue order) leaves the state loads in flight
  const Bases bs = make_bases<DK, DV>(c, u, &va, VERIFY);
  const int Ggrp = HV / c.hk;
  Stage<DK, DV, NT, VERIFY> sg;
  sg.load(bs, u, 0, T0, VERIFY && nchunks == 1, colL, g);
  __builtin_amdgcn_sched_barrier(0);
  // H[mt][i][nt] = state[16 mt + 4 g + i][colL + nt]: kept in the layout of the
  // loads so that nothing has to wait for them before it is used
  F H[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      H[mt][i] = *reinterpret_cast<const F *>(st + (int64_t)(16 * mt + 4 * g + i) * DV + colL);
  __builtin_amdgcn_sched_barrier(0);

  // One chunk; the first is peeled off the loop below so that the state loads
  // can still be in flight while its inputs are staged and its matrices built.
  auto chunk = [&](int ch) {
    const int t0 = ch == 0 ? 0 : T0 + kCh * (ch - 1);
    const int Treal = ch == 0 ? T0 : kCh;
    const bool out_chunk = VERIFY && (ch + 1 == nchunks);  // holds the draft
    if (ch > 0) sg.load(bs, u, t0, Treal, out_chunk, colL, g);
    sg.store(sm, bs, u, t0, Treal, out_chunk, colL, g, Ggrp);
    __syncthreads();

    if (wave == 0) build_tt<DK>(sm, sg.al, lane, g, l16, out_chunk);

    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, NT, kY>(sm, H, g, l16, Y, Z);
    __syncthreads();  // T x T matrices complete
    solve_w<DK, NT>(sm, Y, sg.vv, g, l16, Wm);
    if (out_chunk) {
      contract<DK, NT, kZ>(sm, H, g, l16, Y, Z);
      emit_outputs<DK, NT>(sm, Z, Wm, g, l16, t0, Treal, u.B,
                           va.out + ((int64_t)r * va.draft * HV + h) * DV + colL,
                           (int64_t)HV * DV);
    } else {
      fold_state<DK, NT>(sm, Wm, g, l16, H);
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  };
  chunk(0);
  for (int ch = 1; ch < nchunks; ++ch) chunk(ch);

  if constexpr (!VERIFY) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<F *>(st + (int64_t)(16 * mt + 4 * g + i) * DV + colL) = H[mt][i];
    // The last workgroup of this slot to arrive moves the pointers. Every
    // workgroup's head/len loads were consumed (by the branches above) before
    // its arrival, so none can observe the update; no memory fence is needed
    // (an agent-scope fence would write back this XCD's whole L2).
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&c.sync[s], 1);
      if (prev == HV - 1) {
        c.head[s] = (head + n) % C;
        c.len[s] = 0;
        c.sync[s] = 0;
      }
    }
  }
}


// Ring capacity <= 32, so every replay is a single chunk (T = len [+ D] <= 32).
// Waves 1.. issue their state loads as soon as the inputs are staged, while
// wave 0 builds the T x T matrices and only then loads its own state columns:
// the state is never live next to the matrix-building temporaries, which lets
// four workgroups share a CU. Verify takes Y = K H and Z = Q H in one pass, so
// its state registers die right after it.
template <int DK, int DV, int NT, bool VERIFY>
__global__ __launch_bounds__(64 * (DV / (16 * NT)), 4) void replay_single(VerifyArgs va,
                                                                          FlushArgs fa) {
  constexpr int MT = DK / 16;
  static_assert(DK % 32 == 0 && DV % (16 * NT) == 0 && (NT == 2 || NT == 4), "tile shape");
  typedef typename Cols<NT>::F F;
  __shared__ Smem<DK> sm;

  const CacheView &c = VERIFY ? va.c : fa.c;
  const int HV = c.hv;
  const int r = blockIdx.x / HV, h = blockIdx.x % HV;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane >> 4, l16 = lane & 15;
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
    if (n + va.draft > C) {
      if (lead) raise_err(c.err, GDN_DERR_CAPACITY);
      return;
    }
    T = n + va.draft;
  } else {
    if (n < max(fa.min_len, 1)) return;  // not due: nothing is written
    T = n;
  }
  const Unit u{r, h, s, h / (HV / c.hk), head, n, T, C};
  float *st = c.state + ((int64_t)s * HV + h) * DK * DV;

  const Bases bs = make_bases<DK, DV>(c, u, &va, VERIFY);
  Stage<DK, DV, NT, VERIFY> sg;
  sg.load(bs, u, 0, T, VERIFY, colL, g);
  sg.store(sm, bs, u, 0, T, VERIFY, colL, g, HV / c.hk);
  __syncthreads();

  if (wave == 0) build_tt<DK>(sm, sg.al, lane, g, l16, VERIFY);
  __builtin_amdgcn_sched_barrier(0);
  F H[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      H[mt][i] = *reinterpret_cast<const F *>(st + (int64_t)(16 * mt + 4 * g + i) * DV + colL);
  __syncthreads();  // T x T matrices complete

  f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
  contract<DK, NT, VERIFY ? (kY | kZ) : kY>(sm, H, g, l16, Y, Z);
  solve_w<DK, NT>(sm, Y, sg.vv, g, l16, Wm);
  if constexpr (VERIFY) {
    emit_outputs<DK, NT>(sm, Z, Wm, g, l16, 0, T, u.B,
                         va.out + ((int64_t)r * va.draft * HV + h) * DV + colL,
                         (int64_t)HV * DV);
  } else {
    fold_state<DK, NT>(sm, Wm, g, l16, H);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<F *>(st + (int64_t)(16 * mt + 4 * g + i) * DV + colL) = H[mt][i];
    // The last workgroup of this slot to arrive moves the pointers. Every
    // workgroup's head/len loads were consumed (by the branches above) before
    // its arrival, so none can observe the update; no memory fence is needed
    // (an agent-scope fence would write back this XCD's whole L2).
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&c.sync[s], 1);
      if (prev == HV - 1) {
        c.head[s] = (head + n) % C;
        c.len[s] = 0;
        c.sync[s] = 0;
      }
    }
  }
}

template <int DK, int DV, bool VERIFY>
hipError_t launch_t(const VerifyArgs &va, const FlushArgs &fa, int num_reqs, int hv, int cap,
                    hipStream_t stream) {
  constexpr int NT = 2;
  const dim3 grid(num_reqs * hv), block(64 * (DV / (16 * NT)));
  if (cap <= kCh)
    hipLaunchKernelGGL((replay_single<DK, DV, NT, VERIFY>), grid, block, 0, stream, va, fa);
  else
    hipLaunchKernelGGL((replay_chunked<DK, DV, NT, VERIFY>), grid, block, 0, stream, va, fa);
  return hipGetLastError();
}

}  // namespace

bool chunked_supported(int dk, int dv, bool in_f32, int draft) {
  return !in_f32 && dk == dv && (dk == 64 || dk == 128) && draft <= kCh;
}

hipError_t launch_verify_chunked(const VerifyArgs &a, hipStream_t stream) {
  FlushArgs none{};
  if (a.c.dk == 128) return launch_t<128, 128, true>(a, none, a.num_reqs, a.c.hv, a.c.cap, stream);
  if (a.c.dk == 64) return launch_t<64, 64, true>(a, none, a.num_reqs, a.c.hv, a.c.cap, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_flush_chunked(const FlushArgs &a, hipStream_t stream) {
  VerifyArgs none{};
  if (a.c.dk == 128) return launch_t<128, 128, false>(none, a, a.num_reqs, a.c.hv, a.c.cap, stream);
  if (a.c.dk == 64) return launch_t<64, 64, false>(none, a, a.num_reqs, a.c.hv, a.c.cap, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdnr
