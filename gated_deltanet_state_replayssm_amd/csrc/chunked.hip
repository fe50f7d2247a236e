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
// of the state and every column tile nt, the accumulator entries
//     H[16 mt + 4 g + i][c0 + NT l16 + nt],  i = 0..3,
// i.e. exactly the MFMA 16x16 accumulator layout, with the NT columns of a row
// contiguous (one NT-float global load or store per row). Because an MFMA
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

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DK>
struct Smem {
  uint16_t k[kCh][DK + kPadK];   // chunk keys, token-major (bf16 bits)
  uint16_t q[kCh][DK + kPadK];   // chunk queries: draft rows only, zero elsewhere
  uint16_t kt[DK][kCh + kPadT];  // chunk keys, transposed
  float L[kCh][kCh + kPadF];     // decay ratios L[t][i], 0 above the diagonal
  float A[kCh][kCh + kPadF];     // beta_t L[t][i] (k_t . k_i), strictly lower
  float Ti[kCh][kCh + kPadF];    // (I + A)^-1
  float Cm[kCh][kCh + kPadF];    // L[t][i] (q_t . k_i), lower incl. diagonal
  float gam[kCh], bet[kCh], alp[kCh];
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

// Stage chunk rows [t0, t0 + 32) of the token stream (B committed ring tokens,
// then the draft when verifying) into LDS; verify also appends the draft rows it
// stages to the ring. Returns this lane's values of v for its 8 token rows.
template <int DK, int DV, int NT, bool VERIFY>
__device__ __forceinline__ void stage_chunk(Smem<DK> &sm, const CacheView &c, const Unit &u,
                                            const VerifyArgs *va, int t0, int Treal,
                                            int colL, int g, uint32_t (&vv)[2][4]) {
  constexpr int THREADS = 64 * (DV / (16 * NT));
  constexpr int PARTS = DK / 8;  // 16-byte pieces per key row
  const int tid = threadIdx.x;
  const int C = u.C, HV = c.hv, HK = c.hk, G = HV / HK;
  const bool kq_writer = VERIFY && (u.h % G == 0);
  // keys and queries
  for (int p = tid; p < kCh * PARTS; p += THREADS) {
    const int t = p / PARTS, part = p % PARTS;
    uint4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
    if (t < Treal) {
      const int tok = t0 + t;
      if (tok < u.B) {
        const int pos = (u.head + tok) % C;
        kv = *reinterpret_cast<const uint4 *>(
            static_cast<const uint16_t *>(c.ring_k) + ((int64_t)(u.s * HK + u.kh) * C + pos) * DK + part * 8);
      } else if constexpr (VERIFY) {
        const int j = tok - u.B;
        const int64_t src = ((int64_t)(u.r * va->draft + j) * HK + u.kh) * DK + part * 8;
        kv = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(va->k) + src);
        qv = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(va->q) + src);
        if (kq_writer) {
          const int pos = (u.head + tok) % C;
          const int64_t dst = ((int64_t)(u.s * HK + u.kh) * C + pos) * DK + part * 8;
          *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(c.ring_k) + dst) = kv;
          if (c.ring_q) *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(c.ring_q) + dst) = qv;
        }
      }
    }
    *reinterpret_cast<uint4 *>(&sm.k[t][part * 8]) = kv;
    *reinterpret_cast<uint4 *>(&sm.q[t][part * 8]) = qv;
    const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.kt[part * 8 + 2 * e][t] = (uint16_t)(w[e] & 0xffffu);
      sm.kt[part * 8 + 2 * e + 1][t] = (uint16_t)(w[e] >> 16);
    }
  }
  // decays and write strengths (padding rows: alpha = 1, beta = 0)
  if (tid < kCh) {
    const int t = tid;
    float al = 1.f, be = 0.f;
    if (t < Treal) {
      const int tok = t0 + t;
      if (tok < u.B) {
        const int64_t i = (int64_t)(u.s * HV + u.h) * C + (u.head + tok) % C;
        al = c.ring_alpha[i];
        be = c.ring_beta[i];
      } else if constexpr (VERIFY) {
        const int64_t i = (int64_t)(u.r * va->draft + (tok - u.B)) * HV + u.h;
        al = va->alpha[i];
        be = va->beta[i];
        const int64_t d = (int64_t)(u.s * HV + u.h) * C + (u.head + tok) % C;
        c.ring_alpha[d] = al;
        c.ring_beta[d] = be;
      }
    }
    sm.alp[t] = al;
    sm.bet[t] = be;
  }
  // this lane's v: rows 16 mt + 4 g + i, columns colL .. colL + 1
  static_assert(NT == 2, "v staging packs two bf16 columns per row");
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * mt + 4 * g + i;
      uint32_t w = 0u;
      if (t < Treal) {
        const int tok = t0 + t;
        if (tok < u.B) {
          const int pos = (u.head + tok) % C;
          w = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(c.ring_v) +
                                                  ((int64_t)(u.s * HV + u.h) * C + pos) * DV + colL);
        } else if constexpr (VERIFY) {
          const int j = tok - u.B;
          w = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(va->v) +
                                                  ((int64_t)(u.r * va->draft + j) * HV + u.h) * DV + colL);
          const int pos = (u.head + tok) % C;
          *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(c.ring_v) +
                                        ((int64_t)(u.s * HV + u.h) * C + pos) * DV + colL) = w;
        }
      }
      vv[mt][i] = w;
    }
  }
}

// One workgroup per (request, value head). VERIFY: outputs of the draft, state
// untouched. !VERIFY (flush): fold all committed tokens, write the state back,
// move the pointers.
template <int DK, int DV, int NT, bool VERIFY>
__global__ __launch_bounds__(64 * (DV / (16 * NT))) void replay_chunked(VerifyArgs va,
                                                                        FlushArgs fa) {
  constexpr int WAVES = DV / (16 * NT);
  constexpr int MT = DK / 16;   // 16-row tiles of the state
  constexpr int KS = DK / 32;   // k-steps of a contraction over d_k
  static_assert(DK % 32 == 0 && DV % (16 * NT) == 0, "tile shape");
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
  Unit u{r, h, s, h / (HV / c.hk), head, n, T, C};
  const int nchunks = (T + kCh - 1) / kCh;
  float *st = c.state + ((int64_t)s * HV + h) * DK * DV;

  // ---- first chunk's small inputs, then the whole state tile, in that order so
  // that waiting for the former leaves the state loads in flight
  uint32_t vv[2][4];
  stage_chunk<DK, DV, NT, VERIFY>(sm, c, u, &va, 0, min(kCh, T), colL, g, vv);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 H[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 x = *reinterpret_cast<const float2 *>(st + (int64_t)(16 * mt + 4 * g + i) * DV + colL);
      H[mt][0][i] = x.x;
      H[mt][1][i] = x.y;
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * kCh;
    const int Treal = min(kCh, T - t0);
    if (ch > 0) stage_chunk<DK, DV, NT, VERIFY>(sm, c, u, &va, t0, Treal, colL, g, vv);
    __syncthreads();

    const bool has_draft = VERIFY && (t0 + Treal > u.B);
    const bool fold = !VERIFY || (ch + 1 < nchunks);

    // ---- decay table (wave 0) and Gram matrices (last wave)
    f32x4 Gm[2][2], Pm[2][2];
    if (wave == 0) {
      if (lane < kCh) {
        const int t = lane;
        float prod = 1.f;
#pragma unroll
        for (int i = kCh - 1; i >= 0; --i) {
          sm.L[t][i] = (i <= t) ? prod : 0.f;
          if (i >= 1 && i <= t) prod *= sm.alp[i];
        }
        sm.gam[t] = prod * sm.alp[0];
      }
    }
    if (wave == WAVES - 1) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) Gm[a][b] = Pm[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 k0 = rd_row(sm.k, l16, 32 * ks + 4 * g);
        const bf16x8 k1 = rd_row(sm.k, 16 + l16, 32 * ks + 4 * g);
        Gm[0][0] = mfma(k0, k0, Gm[0][0]);
        Gm[1][0] = mfma(k1, k0, Gm[1][0]);
        Gm[1][1] = mfma(k1, k1, Gm[1][1]);
        if (has_draft) {
          const bf16x8 q0 = rd_row(sm.q, l16, 32 * ks + 4 * g);
          const bf16x8 q1 = rd_row(sm.q, 16 + l16, 32 * ks + 4 * g);
          Pm[0][0] = mfma(q0, k0, Pm[0][0]);
          Pm[1][0] = mfma(q1, k0, Pm[1][0]);
          Pm[1][1] = mfma(q1, k1, Pm[1][1]);
        }
      }
    }
    __syncthreads();
    if (wave == WAVES - 1) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * a + 4 * g + i, j = 16 * b + l16;
            const float Ltj = sm.L[t][j];
            sm.A[t][j] = (b <= a && j < t) ? sm.bet[t] * Ltj * Gm[a][b][i] : 0.f;
            sm.Cm[t][j] = (b <= a && j <= t) ? Ltj * Pm[a][b][i] : 0.f;
          }
    }
    __syncthreads();

    // ---- (I + A)^-1 by columns (wave 0, lanes 0..31), overlapping the others' contraction
    if (wave == 0 && lane < kCh) {
      const int col = lane;
      float x[kCh];
#pragma unroll
      for (int t = 0; t < kCh; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < t; ++i) acc = fmaf(sm.A[t][i], x[i], acc);
        x[t] = (t < col) ? 0.f : (t == col ? 1.f : -acc);
        sm.Ti[t][col] = x[t];
      }
    }

    // ---- Y = K H and Z = Q H on MFMA (state split into hi + lo bf16)
    f32x4 Y[2][NT], Z[2][NT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Y[a][nt] = Z[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 k0 = rd_row(sm.k, l16, 32 * ks + 4 * g);
      const bf16x8 k1 = rd_row(sm.k, 16 + l16, 32 * ks + 4 * g);
      bf16x8 q0, q1;
      if (has_draft) {
        q0 = rd_row(sm.q, l16, 32 * ks + 4 * g);
        q1 = rd_row(sm.q, 16 + l16, 32 * ks + 4 * g);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 hh, hl;
        tok_operand(H[2 * ks][nt], H[2 * ks + 1][nt], hh, hl);
        Y[0][nt] = mfma(k0, hh, Y[0][nt]);
        Y[0][nt] = mfma(k0, hl, Y[0][nt]);
        Y[1][nt] = mfma(k1, hh, Y[1][nt]);
        Y[1][nt] = mfma(k1, hl, Y[1][nt]);
        if (has_draft) {
          Z[0][nt] = mfma(q0, hh, Z[0][nt]);
          Z[0][nt] = mfma(q0, hl, Z[0][nt]);
          Z[1][nt] = mfma(q1, hh, Z[1][nt]);
          Z[1][nt] = mfma(q1, hl, Z[1][nt]);
        }
      }
    }
    __syncthreads();  // (I + A)^-1 ready

    // ---- X = beta (V - gamma Y), then W = (I + A)^-1 X (3-pass split product)
    bf16x8 xh[NT], xl[NT];
    {
      f32x4 X[2][NT];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * a + 4 * g + i;
          const float be = sm.bet[t], ga = sm.gam[t];
          const float v0 = bf16lo(vv[a][i]), v1 = bf16hi(vv[a][i]);
          X[a][0][i] = be * (v0 - ga * Y[a][0][i]);
          X[a][1][i] = be * (v1 - ga * Y[a][1][i]);
        }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) tok_operand(X[0][nt], X[1][nt], xh[nt], xl[nt]);
    }
    f32x4 Wm[2][NT];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      float trow[8];
      rd_frow(sm.Ti, 16 * a + l16, g, trow);
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

    // ---- draft outputs: O = gamma Z + C W
    if (has_draft) {
      bf16x8 wh[NT], wl[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) tok_operand(Wm[0][nt], Wm[1][nt], wh[nt], wl[nt]);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float crow[8];
        rd_frow(sm.Cm, 16 * a + l16, g, crow);
        bf16x8 chh, chl;
        split8(crow, chh, chl);
        f32x4 O[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 acc;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = sm.gam[16 * a + 4 * g + i] * Z[a][nt][i];
          acc = mfma(chh, wh[nt], acc);
          acc = mfma(chh, wl[nt], acc);
          acc = mfma(chl, wh[nt], acc);
          O[nt] = acc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * a + 4 * g + i;
          const int tok = t0 + t;
          if (t < Treal && tok >= u.B) {
            const int j = tok - u.B;
            float2 o2 = {O[0][i], O[1][i]};
            *reinterpret_cast<float2 *>(
                va.out + ((int64_t)(r * va.draft + j) * HV + h) * DV + colL) = o2;
          }
        }
      }
    }

    // ---- fold the chunk into the on-chip state: H <- gamma_T H + K^T (L[T-1] W)
    if (fold) {
      const float gT = sm.gam[kCh - 1];
      bf16x8 wh[NT], wl[NT];
      {
        f32x4 Wp[2][NT];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lt = sm.L[kCh - 1][16 * a + 4 * g + i];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) Wp[a][nt][i] = lt * Wm[a][nt][i];
          }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) tok_operand(Wp[0][nt], Wp[1][nt], wh[nt], wl[nt]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 kt = rd_row(sm.kt, 16 * mt + l16, 4 * g);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 acc = H[mt][nt] * gT;
          acc = mfma(kt, wh[nt], acc);
          acc = mfma(kt, wl[nt], acc);
          H[mt][nt] = acc;
        }
      }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }

  if constexpr (!VERIFY) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float2 x = {H[mt][0][i], H[mt][1][i]};
        *reinterpret_cast<float2 *>(st + (int64_t)(16 * mt + 4 * g + i) * DV + colL) = x;
      }
    // the last workgroup of this slot moves the pointers; every workgroup of the
    // slot read head/len before its own arrival
    __syncthreads();
    if (tid == 0) {
      __threadfence();
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
hipError_t launch_t(const VerifyArgs &va, const FlushArgs &fa, int num_reqs, int hv,
                    hipStream_t stream) {
  constexpr int NT = 2;
  dim3 grid(num_reqs * hv);
  hipLaunchKernelGGL((replay_chunked<DK, DV, NT, VERIFY>), grid, dim3(64 * (DV / (16 * NT))), 0,
                     stream, va, fa);
  return hipGetLastError();
}

}  // namespace

bool chunked_supported(int dk, int dv, bool in_f32) {
  return !in_f32 && dk == dv && (dk == 64 || dk == 128);
}

hipError_t launch_verify_chunked(const VerifyArgs &a, hipStream_t stream) {
  FlushArgs none{};
  if (a.c.dk == 128) return launch_t<128, 128, true>(a, none, a.num_reqs, a.c.hv, stream);
  if (a.c.dk == 64) return launch_t<64, 64, true>(a, none, a.num_reqs, a.c.hv, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_flush_chunked(const FlushArgs &a, hipStream_t stream) {
  VerifyArgs none{};
  if (a.c.dk == 128) return launch_t<128, 128, false>(none, a, a.num_reqs, a.c.hv, stream);
  if (a.c.dk == 64) return launch_t<64, 64, false>(none, a, a.num_reqs, a.c.hv, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdnr
