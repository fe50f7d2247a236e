// Fused replay kernels for gfx950: the periodic flush folded into the next
// verify (replay_fused for one-chunk replays, ring capacity <= 32;
// replay_fused_long for several chunks), optionally with the previous draft's
// rollback and the gated RMSNorm + FP8 of the outputs in the same kernel. The
// building blocks and the chunked form are in chunk_ops.h.
#include "chunk_ops.h"

namespace gdnr {

namespace {

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
template <int DK, int DV, int NT, class SM>
__device__ __forceinline__ void emit_outputs_norm(const SM &sm,
                                                  const f32x4 (&Z)[2][NT],
                                                  const f32x4 (&Wm)[2][NT], int g, int l16,
                                                  int wave, int Treal, int B, Rsrc out, int col,
                                                  const VerifyArgs &va, const NormRsrc &nr,
                                                  const Gate &gt, float (*red)[kCh][4],
                                                  int a0 = 0) {
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
    if (a < a0) {  // a split chunk: no draft rows in tile 0
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) O[a][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      continue;
    }
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
  // One pass over each row, one exchange between the waves: the mean square
  // and the largest |u_j|, u_j = o_j w_j silu(z_j). Since y_j = u_j / r, the
  // row's max |y| is max |u| / r and the codes y_j / s = 448 u_j / max|u| need
  // no r at all; r sets only the scale s = max|u| / (448 r). 1/r comes from the
  // hardware reciprocal square root (1 ulp) and the gate's 1/(1 + e^-z) and
  // 1/max|u| from the hardware reciprocal, all far inside the scale's and the
  // codes' tolerance. The rows' reductions are independent chains.
  float u[2][NT][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!slot_live(a, i)) continue;
      float ss = 0.f, mx = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ss = fmaf(O[a][nt][i], O[a][nt][i], ss);
        const uint32_t zb = gt.z[a][i];
        const float zf = __uint_as_float(nt == 0 ? zb << 16 : zb & 0xffff0000u);
        const float gate = zf * __builtin_amdgcn_rcpf(1.f + __expf(-zf));
        u[a][nt][i] = O[a][nt][i] * gt.w[nt] * gate;
        mx = fmaxf(mx, fabsf(u[a][nt][i]));
      }
      ss = row16_reduce<false>(ss);
      mx = row16_reduce<true>(mx);
      if (l16 == 15) {
        red[0][16 * a + 4 * g + i][wave] = ss;
        red[1][16 * a + 4 * g + i][wave] = mx;
      }
    }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!slot_live(a, i)) continue;
      const int t = 16 * a + 4 * g + i;
      const bool row = t < Treal && t >= B;
      const float4 p = *reinterpret_cast<const float4 *>(red[0][t]);
      const float4 m = *reinterpret_cast<const float4 *>(red[1][t]);
      const float tot = WAVES == 4 ? (p.x + p.y) + (p.z + p.w) : p.x + p.y;
      const float umax = WAVES == 4 ? fmaxf(fmaxf(m.x, m.y), fmaxf(m.z, m.w)) : fmaxf(m.x, m.y);
      const float rinv =
          __builtin_amdgcn_rsqf(fmaxf(fmaf(tot, 1.f / DV, va.norm_eps), 1.17549435e-38f));
      const float amax = umax * rinv;  // max |y|
      float scale = 1.f, inv = 1.f;    // inv: 448 / max|u|
      if (amax >= 0x1p-126f) {
        scale = amax * (1.f / kE4M3Max);
      } else if (amax > 0.f) {  // a subnormal maximum: the exact quotient
        scale = amax / kE4M3Max;
      }
      if (umax >= 0x1p-126f)
        inv = kE4M3Max * __builtin_amdgcn_rcpf(umax);
      else if (umax > 0.f)
        inv = kE4M3Max / umax;
      // clamp first: the conversion then never sees a value past the largest code
      const float c0 = fminf(fmaxf(u[a][0][i] * inv, -kE4M3Max), kE4M3Max);
      const float c1 = fminf(fmaxf(u[a][1][i] * inv, -kE4M3Max), kE4M3Max);
      const uint32_t packed = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
      // write-back stores: the four waves' 32-byte pieces of a row's 128 code
      // bytes meet in L2 and leave it as one line (written through, each piece
      // went to memory on its own: 20 us of 135 at 128 requests)
      bstore<uint16_t, 0>((uint16_t)(packed & 0xffff), nr.q,
                          row ? (uint32_t)(t - B) * q_row + col : kOOB);
      if (wave == 0 && l16 == 0)
        bstore<float, 0>(scale, nr.scale, row ? (uint32_t)(t - B) * s_row : kOOB);
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
//
// CHAINS (several-chunk replays, up to 64 requests): requests in the order of
// the chunks their workgroups fold (three or more, two, fewer), due first
// within each class, so that the long chains come first and are spread over
// the CUs (36.9 -> 36.2 us per launch at 32 requests, capacity 80, with two
// classes; with three, and the three-chunk chains' state loaded first, 35.6).
template <bool ROLLBACK, bool VARLEN, bool CHAINS = false>
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
    int r;
    if constexpr (CHAINS) {
      int nf = 0;  // fold chunks of this lane's request (the stream less its output chunk)
      if (lane < R && si >= 0 && si < c.num_slots) {
        const int dl = VARLEN ? max(request_draft(va.draft_lens, lane, va.draft), 0) : va.draft;
        const bool du = ne >= mn;
        const int nch = ((du ? ne : ne + dl) + kCh - 1) / kCh;
        nf = du ? nch : nch - 1;
      }
      const uint64_t all = lanes(0);
      const uint64_t c3 = __ballot(nf >= 3), c2 = __ballot(nf == 2);
      const uint64_t c1 = all & ~c3 & ~c2;
      const uint64_t ms[6] = {c3 & dm, c3 & ~dm, c2 & dm, c2 & ~dm, c1 & dm, c1 & ~dm};
      int left = q;
      r = 0;
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const int cnt = __popcll(ms[k]);
        if (left >= 0 && left < cnt) r = nth_bit(ms[k], left);
        left -= cnt;
      }
    } else {
      r = q < nd ? nth_bit(dm, q) : nth_bit(~dm & lanes(0), q - nd);
    }
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

// Arrival count of a fused launch. The pointers (head, len) may move only once
// every workgroup has read them, and a workgroup reads them in its ordering
// pass only. So each workgroup counts itself in right after that pass (after a
// barrier, so that all its waves have read): HV per request rank on that
// rank's counter, then the last of those on the grid counter, and the
// workgroup that brings the grid count to num_reqs moves the pointers at its
// end (a due slot's head += len, len = 0; with a folded rollback, len += a for
// the others). The atomics' returns are read where waiting for them costs
// nothing: the rank count once the first staged inputs have arrived (it was
// issued before them; loads and atomics return in issue order), the grid count
// after the last contraction, whose result is read at the end. Neither count
// sits at the end of a workgroup's life, where it would lengthen the launch's
// tail. With no due request and no rollback nothing moves and no count is
// taken (every workgroup sees the same count, as no pointer changes during the
// call). Every counter is reset by its last arrival.
template <bool ROLLBACK, bool VARLEN>
struct Arrival {
  bool counting;   // uniform: the call moves pointers
  bool taken;      // uniform: the rank count has been read
  bool gridded;    // uniform: the grid count has been taken (if this is the rank's last)
  bool rank_last;  // wave 0, after take_rank(): last of its request rank to count in
  int ticket;      // lane 0 of wave 0: the rank counter's value before this arrival
  int gticket;     // lane 0 of wave 0: the grid counter's value before it (rank_last)

  __device__ __forceinline__ void count_in(const Req &rq, int32_t *rank_ctr, int tid) {
    counting = ROLLBACK || rq.due > 0;
    taken = gridded = rank_last = false;
    ticket = 0;
    if (!counting) return;
    __syncthreads();  // every wave has read the pointers
    if (tid == 0) ticket = atomicAdd(rank_ctr, 1);
  }

  // Wave 0 reads its rank count; called by every wave at the same point.
  __device__ __forceinline__ void take_rank(int HV, int32_t *rank_ctr, int tid) {
    if (!counting || taken) return;
    taken = true;
    if (__builtin_amdgcn_readfirstlane(tid) >= 64) return;  // (uniform: the wave's first lane)
    rank_last = __builtin_amdgcn_readfirstlane(ticket) == HV - 1;
    if (rank_last && tid == 0) *rank_ctr = 0;  // every arrival of the rank is in
  }

  // The last of a rank counts in at the grid counter. DEFER: the return is
  // awaited where it is read, at the end (a buffer atomic at an opaque per-lane
  // offset; at a uniform address the compiler rewrites the atomic as a
  // wave-wide one and waits for its return at once, which also waits for every
  // store issued before it).
  template <bool DEFER = false>
  __device__ __forceinline__ void grid_in(int HV, int32_t *rank_ctr, int32_t *grid_ctr,
                                          int tid) {
    if (!counting || gridded) return;
    take_rank(HV, rank_ctr, tid);
    gridded = true;
    if constexpr (DEFER) {
      int off = 0;
      asm volatile("" : "+v"(off));
      gticket = -1;
      if (rank_last && tid == 0)
        gticket =
            __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, make_rsrc(grid_ctr, 4), off, 0, 0);
    } else {
      gticket = (rank_last && tid == 0) ? atomicAdd(grid_ctr, 1) : -1;
    }
  }

  // End of the workgroup: the grid's last arrival moves the pointers (wave 0).
  __device__ __forceinline__ void finish(const VerifyArgs &va, int mn, int32_t *rank_ctr,
                                         int32_t *grid_ctr, const Move *moves, int tid) {
    const CacheView &c = va.c;
    if (!counting) return;
    grid_in(c.hv, rank_ctr, grid_ctr, tid);
    if (__builtin_amdgcn_readfirstlane(tid) >= 64 || !rank_last) return;
    if (__builtin_amdgcn_readfirstlane(gticket) != va.num_reqs - 1) return;
    const int lane = tid;
    if (va.num_reqs <= 64) {  // moves worked out by the ordering pass
      if (lane < va.num_reqs) {
        const Move mv = moves[lane];
        if (mv.slot >= 0) {
          if (mv.head >= 0) c.head[mv.slot] = mv.head;
          c.len[mv.slot] = mv.len;
        }
      }
      if (lane == 0) *grid_ctr = 0;
      return;
    }
    for (int i = lane; i < va.num_reqs; i += 64) {
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
    if (lane == 0) *grid_ctr = 0;
  }
};

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
// workgroup to count in after its ordering pass (Arrival). It is found in two
// levels, so that no counter sees more than one arrival per workgroup of a
// request group: the HV workgroups of request rank q count in at that rank's
// counter (a 128-byte line of its own), the last of them at the grid counter.
//
// The draft is appended at (new head + j) mod C, which may wrap onto committed
// key rows that the other value heads of the same key head are still reading
// for their fold. So each workgroup of a due slot counts itself in at the
// (slot, key head) counter once its fold inputs are staged, and the last
// one of the key head's group appends k and q (the others have read by then).
// Warms L2 with one dword of every 128-byte line of a request's draft rows
// (keys and queries of key head kh, values, alpha and beta of value head h),
// one line per thread: issued at the start, when memory is quiet, by the
// workgroup at the request's unordered position. The workgroup that stages
// those rows after the ordering pass has the same value head and, with HV a
// multiple of 8, runs on the same XCD (position mod 8), so its reads then hit
// that L2 instead of queueing behind the state stream. Returns the OR of the
// loaded words, for the caller to consume at its end.
template <int DK, int DV>
__device__ __forceinline__ uint32_t warm_draft(const VerifyArgs &va, int rn, int h, int kh,
                                               int tid) {
  constexpr int KL = DK * 2 / 128, VL = DV * 2 / 128;  // lines per key / value row
  const int HV = va.c.hv, HK = va.c.hk, D = va.draft;
  const int64_t d0 = (int64_t)rn * D;
  int t = tid, a = 0;
  if (t >= D * KL) { t -= D * KL; a = 1; }
  if (a == 1 && t >= D * KL) { t -= D * KL; a = 2; }
  if (a == 2 && t >= D * VL) { t -= D * VL; a = 3; }
  if (a == 3 && t >= D) { t -= D; a = 4; }
  if (a == 4 && t >= D) return 0u;  // past the request's lines
  const uint32_t kq_bytes = (D - 1) * HK * DK * 2 + DK * 2;
  Rsrc r;
  uint32_t off;
  if (a <= 1) {
    r = make_rsrc(static_cast<const uint16_t *>(a == 0 ? va.k : va.q) + (d0 * HK + kh) * DK,
                  kq_bytes);
    off = (uint32_t)(t / KL) * HK * DK * 2 + (t % KL) * 128;
  } else if (a == 2) {
    r = make_rsrc(static_cast<const uint16_t *>(va.v) + (d0 * HV + h) * DV,
                  (D - 1) * HV * DV * 2 + DV * 2);
    off = (uint32_t)(t / VL) * HV * DV * 2 + (t % VL) * 128;
  } else {
    r = make_rsrc((a == 3 ? va.alpha : va.beta) + d0 * HV + h, (D - 1) * HV * 4 + 4);
    off = (uint32_t)t * HV * 4;
  }
  return bload<uint32_t>(r, off);
}

template <int DK, int DV, int NT, bool VARLEN, bool ROLLBACK, bool NORM>
__global__ __launch_bounds__(64 * (DV / (16 * NT)), 4) void replay_fused(VerifyArgs va,
                                                                         int min_len) {
  constexpr int WAVES = DV / (16 * NT);
  constexpr int MT = DK / 16;
  static_assert(DK % 32 == 0 && DV % (16 * NT) == 0 && (NT == 2 || NT == 4), "tile shape");
  typedef typename Cols<NT>::F F;
  __shared__ Smem<DK, DV> sm;
  __shared__ int group_rank;
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
  const int h = head_of(blockIdx.x % HV, HV, G);
  // (the first generation of workgroups only, 256 CUs x 4: later ones start
  // with memory busy, where the extra requests measured 1 % slower)
  uint32_t warm = 0u;
  if (blockIdx.x < 1024) warm = warm_draft<DK, DV>(va, blockIdx.x / HV, h, h / G, tid);
  if constexpr (NORM) {
    // and the gate rows the norm reads (two lines of bf16 per row at d_v 128)
    constexpr int ZL = DV * 2 / 128;
    const int t = tid - 128;
    if (blockIdx.x < 1024 && t >= 0 && t < va.draft * ZL) {
      const NormRsrc nr = norm_rsrc(va, blockIdx.x / HV, h, DV, va.draft);
      warm |= bload<uint32_t>(nr.z, (uint32_t)(t / ZL) * HV * DV * 2 + (t % ZL) * 128);
    }
  }
  const Req rq = ordered_request<ROLLBACK, VARLEN>(va, mn, blockIdx.x / HV, lane,
                                                  wave == 0 ? moves : nullptr);
  const int r = rq.r;
  const bool lead = (h == 0 && tid == 0);
  int32_t *grid_ctr = c.sync;
  int32_t *rank_ctr = slot_counter(c, blockIdx.x / HV);
  // every workgroup counts itself in once its pointers are read; the grid's
  // last arrival moves the pointers at its end
  Arrival<ROLLBACK, VARLEN> arr;
  arr.count_in(rq, rank_ctr, tid);
  auto finish = [&]() { arr.finish(va, mn, rank_ctr, grid_ctr, moves, tid); };

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
    arr.take_rank(HV, rank_ctr, tid);
    // count in for the key rows' append; the last wave waits for the return,
    // which comes after its state loads, not the builder
    if (tid == 64 * (WAVES - 1)) group_rank = atomicAdd(group_ctr, 1);
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
  // With the norm, a split output chunk (kGapRow: committed rows from 0, draft
  // rows from 16) when both fit; its draft rows are the chunk's rows [ob, oT).
  // The norm's per-row reductions then cover one 16-row tile instead of two
  // (1 us less per launch at 32 requests); without the norm the split measured
  // 0.2 us slower, and the plain step keeps the layout of the separate verify.
  const bool split = NORM && B <= kGapRow && D <= kGapRow;
  const int ob = split ? kGapRow : B, oT = split ? kGapRow + D : B + D;
  const int gB = split ? B : -1;
  Stage<DK, DV, NT, true> sga;
  Stage<DK, DV, NT, true, 64 * SW> sgs;
  float al;  // this lane's staged alpha (token lane % 32)
  if (due) {
    sga.load(sr, u, 0, u.T, true, split);
    sga.store(sm, u.T, true, gB, D);
    al = sga.al;
  } else {
    if (wave >= SW) {
      load_state<DK, DV, NT>(st, st_off_of(), H);
      al = 1.f;
    } else {
      sgs.load(sr, u, 0, u.T, true, split);
      sgs.store(sm, u.T, true, gB, D);
      al = sgs.al;
      __builtin_amdgcn_sched_barrier(0);
      load_state<DK, DV, NT>(st, st_off_of(), H);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  // The draft rows go to the ring now, off the launch's tail, by the waves
  // that build nothing.
  constexpr int AW = WAVES >= 4 ? 2 : 1;  // appending waves: the last AW
  const bool kq_writer = due ? group_rank == G - 1 : h % G == 0;
  if (wave >= WAVES - AW)
    Stage<DK, DV, NT, true, 64 * AW>{}.append(sm, sr, u, 0, u.T, kq_writer, split,
                                              64 * (WAVES - AW));
  arr.take_rank(HV, rank_ctr, tid);
  if (wave == 0) {
    build_tt<DK, DV>(sm, al, lane, g, l16);
    if (WAVES == 1) build_c<DK, DV>(sm, al, lane, g, l16);
  } else if (wave == 1) {
    build_c<DK, DV>(sm, al, lane, g, l16);
  }
  __syncthreads();  // T x T matrices complete
  if (wave == (WAVES > 1 ? 1 : 0)) build_m<DK, DV>(sm, g, l16);

  f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
  if constexpr (NORM) {
    // the gate and weight load while the state is contracted and W solved
    // (issued after the contraction, their round trip fell into the launch's
    // tail; issued before the T x T build, they spill); out may be absent
    const NormRsrc nr = norm_rsrc(va, r, h, DV, max(D, 1));
    const Gate gt = load_gate<DV, NT>(va, nr, col_of(), g, ob, oT);
    contract<DK, DV, NT, kY | kZ>(sm, H, g, l16, Y, Z);
    arr.grid_in(HV, rank_ctr, grid_ctr, tid);
    lds_barrier();  // M complete (LDS only)
    x_prime<DK, DV, NT>(sm, Y, col_of(), g, Wm);
    // the norm's cross-wave partials in the T x T array: (I + A)^-1 has no
    // reader after M (an array of their own took the LDS past 4 workgroups
    // per CU: 39.4 KB)
    float(*nred)[kCh][4] = reinterpret_cast<float(*)[kCh][4]>(&sm.T[0][0]);
    static_assert(sizeof(sm.T) >= 2 * kCh * 4 * sizeof(float), "partials fit");
    emit_outputs_norm<DK, DV, NT>(
        sm, Z, Wm, g, l16, wave, oT, ob,
        va.out ? out_rsrc(va, r, h, DV, max(D, 1)) : make_rsrc(nullptr, 0), col_of(), va, nr, gt,
        nred, split ? 1 : 0);
  } else {
    contract<DK, DV, NT, kY | kZ>(sm, H, g, l16, Y, Z);
    arr.grid_in(HV, rank_ctr, grid_ctr, tid);
    lds_barrier();  // M complete (LDS only)
    x_prime<DK, DV, NT>(sm, Y, col_of(), g, Wm);
    emit_outputs<DK, DV, NT>(sm, Z, Wm, g, l16, 0, oT, ob, out_rsrc(va, r, h, DV, max(D, 1)),
                             col_of() * 4, HV * DV * 4, split ? 1 : 0);
  }
  if (due && kq_writer && tid == 0) *group_ctr = 0;  // every member has counted in
  asm volatile("" ::"v"(warm));  // (the warming loads' results, consumed)
  finish();
}

// Flush fused into verify when a replay takes several chunks (ring capacity
// above 32). A due slot folds its n committed tokens chunk by chunk, writes the
// folded state once and verifies the draft from it (one chunk, B = 0); any
// other slot replays its committed tokens and the draft as replay_chunked's
// verify does. The work order puts requests with more fold chunks first (up to
// 64 requests; then due first, as replay_fused). The draft append of a
// due slot's key and query rows (by the last workgroup of the key head to have
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
  __shared__ __align__(16) uint16_t lds_kn[kCh][DK + kPadK];
  __shared__ __align__(16) uint16_t lds_kc[kCh][DK + kPadK];
  __shared__ __align__(16) uint16_t lds_v[kCh][DV + kPadK];
  __shared__ __align__(16) SmemMats lds_m;
  __shared__ __align__(16) float lds_abn[2][kCh];  // beta, alpha (filled by one DMA)
  __shared__ __align__(16) float lds_abc[2][kCh];
  // A chunk arrives in the "n" buffers (keys, beta, alpha) and is copied to
  // the "c" buffers while wave 0 builds its T x T matrices from the n ones;
  // then the next chunk's DMA refills the n buffers while the contraction, W
  // and the fold read the c ones. The output chunk stays in the n buffers, its
  // queries in keys buffer c.
  const SmemLong<DK, DV> smn{lds_kn,    lds_kc,     lds_v,      lds_m.T,  lds_m.Cm,
                             lds_m.gam, lds_abn[0], lds_abn[1], lds_m.lg, lds_m.lgc};
  const SmemLong<DK, DV> smc{lds_kc,    lds_kn,     lds_v,      lds_m.T,  lds_m.Cm,
                             lds_m.gam, lds_abc[0], lds_abc[1], lds_m.lg, lds_m.lgc};
  __shared__ int group_rank;
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
  const Req rq = ordered_request<ROLLBACK, VARLEN, true>(va, mn, blockIdx.x / HV, lane,
                                                   wave == 0 ? moves : nullptr);
  const int r = rq.r, h = head_of(blockIdx.x % HV, HV, G);
  const bool lead = (h == 0 && tid == 0);
  int32_t *grid_ctr = c.sync;
  int32_t *rank_ctr = slot_counter(c, blockIdx.x / HV);
  Arrival<ROLLBACK, VARLEN> arr;
  arr.count_in(rq, rank_ctr, tid);
  auto finish = [&]() { arr.finish(va, mn, rank_ctr, grid_ctr, moves, tid); };

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
  // opaque past the checks: value facts drawn from them made the register
  // allocation of the chunk loop spill
  int Dq = D;
  asm volatile("" : "+s"(Dq));
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
  // stream of its own, B = 0, from where the folded tokens end); any other
  // slot's is the n tokens and the draft, whose last chunk is the output chunk.
  const Unit u1{r, h, s, kh, head, n, due ? n : n + Dq, C};
  const int hd = head + n - (head + n >= C ? C : 0);
  const Unit ud{r, h, s, kh, hd, 0, Dq, C};
  const Srcs s1 = due ? make_srcs<DK, DV>(c, u1, nullptr, false)
                      : make_srcs<DK, DV>(c, u1, &va, true);
  // The output chunk's resources (draft rows sized for Dq), built where they
  // are used: kept across the chunk loop, they took scalar registers the loop
  // needs and it spilled. The draft pointers come through opaque copies so
  // that the compiler does not hoist the resources out of the loop.
  auto out_srcs = [&]() {
    VerifyArgs v2 = va;
    const void *pk = va.k, *pq = va.q, *pv = va.v;
    const float *pa = va.alpha, *pb = va.beta;
    asm volatile("" : "+s"(pk), "+s"(pq), "+s"(pv), "+s"(pa), "+s"(pb));
    v2.k = pk;
    v2.q = pq;
    v2.v = pv;
    v2.alpha = pa;
    v2.beta = pb;
    return make_srcs<DK, DV>(c, due ? ud : u1, &v2, true);
  };
  const int nch = (u1.T + kCh - 1) / kCh, T0 = u1.T - kCh * (nch - 1);
  const int nfold = due ? nch : nch - 1;
  // A workgroup issues at a priority that grows with the fold chunks it has
  // left (2 for two or more, 1 for one, 0 in the output stage) over the other
  // workgroups on its SIMDs, so that the longest remaining chains go first. The
  // T x T builds raise it to 3 and drop it to 0; it is set again after each.
  // 39.6-39.8 -> 37.0-37.2 us per launch at 32 requests, capacity 80 (a fixed
  // 2 for workgroups with two fold chunks or more: 38.3-38.6; for the due
  // slots alone: no gain).
  auto chain_prio = [&](int left) {
    if (left >= 2)
      __builtin_amdgcn_s_setprio(2);
    else if (left == 1)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  };
  chain_prio(nfold);
  const bool out0 = !due && nch == 1;  // chunk 0 is the output chunk
  // the output chunk: the draft of a due slot, else the stream's last chunk
  const Unit uo = due ? ud : u1;
  const int t0 = due ? 0 : (nch == 1 ? 0 : T0 + kCh * (nch - 2));
  const int Treal = due ? Dq : (nch == 1 ? T0 : kCh);
  {
    // Waves 0..SW-1 stage chunk 0, then load their state. In a workgroup with
    // three fold chunks or more (the launch's longest chains) waves SW.. load
    // their state at once; in one with a shorter chain they wait until chunk 0
    // is staged, so that the longest chains' inputs and states enter the
    // memory queues ahead of theirs (at 32 requests, capacity 80, a threshold
    // of two chunks saved 1 us per launch, and three another 0.4 us with the
    // wave priorities below). One load_state for both, so that the state is
    // assigned its registers once (two call sites met at the chunk loop with
    // two assignments, and the copies between them spilled). The barriers wait
    // for LDS only.
    al = 1.f;
    if (wave < SW) {
      Stage<DK, DV, NT, true, 64 * SW> sg0;
      sg0.load(s1, u1, 0, T0, out0);
      sg0.template store<false>(smn, T0, out0);
      al = sg0.al;
    }
    if (nfold < 3) lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    load_state<DK, DV, NT>(st, st_off_of(), H);
    __builtin_amdgcn_sched_barrier(0);
    if (nfold >= 3) lds_barrier();
  }
  // A fold chunk 0 has its T x T matrices built (and its keys copied) while the
  // state loads are in flight, ahead of the loop: the state's registers are
  // copied into the loop's at its entry, and those copies wait for the loads.
  if (nfold > 0) {
    if (wave == 0)
      build_tt<DK, DV>(smn, al, lane, g, l16);
    else
      copy_chunk_keys<DK, 64 * (WAVES - 1)>(lds_kn, lds_kc, lds_abn, lds_abc, opaque_tid() - 64);
  }
  chain_prio(nfold);
  arr.take_rank(HV, rank_ctr, tid);
  // Every chunk after the first is staged by LDS DMA while its predecessor is
  // computed: its keys, beta and alpha once the predecessor's T x T matrices
  // are built (and its keys copied), its values once W has read the previous
  // values. While DMA is in flight the barriers are lds_barrier(): a
  // __syncthreads() waits for it. The one at a chunk's end does wait (with the
  // values' DMA left in flight across the loop's back edge, the compiler waits
  // for it before the next chunk's first LDS read anyway).
  Prefetch<DK, DV, WAVES> pf;
#pragma nounroll
  for (int ch = 0; ch < nfold; ++ch) {
    // the thread index through an opaque copy: the per-thread offsets are
    // recomputed in every chunk rather than held in registers
    const int lane = opaque_tid() % 64, g = lane >> 4, l16 = lane & 15;
    const bool last = ch == nfold - 1;
    // a due slot's fold inputs are all read: count in for the key rows' append
    // (the last wave waits for the return, which comes after its state loads)
    if (due && last && tid == 64 * (WAVES - 1)) group_rank = atomicAdd(group_ctr, 1);
    if (ch > 0) {
      chain_prio(nfold - ch);
      if (wave == 0) {
        al = smn.alp[lane & (kCh - 1)];
        build_tt<DK, DV>(smn, al, lane, g, l16);
        chain_prio(nfold - ch);
      } else {
        copy_chunk_keys<DK, 64 * (WAVES - 1)>(lds_kn, lds_kc, lds_abn, lds_abc, opaque_tid() - 64);
      }
    }
    lds_barrier();  // T x T matrices built, keys, beta and alpha copied
    // the next chunk: the stream's next fold chunk, or the output chunk
    if (!last) {
      pf.template issue_k<true>(smn, s1, u1, T0 + kCh * ch, kCh);
      pf.template issue_ab<true>(smn, s1, u1, T0 + kCh * ch, kCh);
    } else {
      const Srcs so = out_srcs();
      pf.issue_k(smn, so, uo, t0, Treal);
      pf.issue_ab(smn, so, uo, t0, Treal);
    }
    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, DV, NT, kY>(smc, H, g, l16, Y, Z);
    solve_w<DK, DV, NT>(smc, Y, col_of(), g, l16, Wm);
    lds_barrier();  // every wave has read the values
    if (!last)
      pf.template issue_v<true>(smn, s1, u1, T0 + kCh * ch, kCh);
    else
      pf.issue_v(smn, out_srcs(), uo, t0, Treal);
    fold_state<DK, DV, NT, true>(smc, Wm, g, l16, H);
    __syncthreads();  // (waits for the next chunk's DMA)
  }

  // ---- the output chunk (in the n buffers)
  const SmemLong<DK, DV> &sm = smn;
  const Srcs so = out_srcs();
  // its queries into keys buffer c, which the last fold has finished reading
  if (!out0) pf.issue_q(sm, so, uo, t0, Treal);
  // waits for the output chunk's DMA or, with one chunk, for the state
  __syncthreads();
  if (!out0) {
    const int t = lane & (kCh - 1);
    al = t < Treal ? sm.alp[t] : 1.f;
  }
  // The folded state is written after the last wait for loads: the memory
  // counter retires in issue order, so any later wait would wait for these
  // stores too. Past this point the barriers wait for LDS only and the grid
  // count's return is awaited at the end.
  if (due) store_state<DK, DV, NT>(st, st_off_of(), H);
  if (wave == 0)
    build_tt<DK, DV>(sm, al, lane, g, l16);
  else if (wave == 1)
    build_c<DK, DV>(sm, al, lane, g, l16);
  lds_barrier();  // T x T matrices complete
  if (wave == 1) build_m<DK, DV>(sm, g, l16);
  {
    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, DV, NT, kY | kZ>(sm, H, g, l16, Y, Z);
    arr.template grid_in<true>(HV, rank_ctr, grid_ctr, tid);  // (the state's stores in flight)
    lds_barrier();  // M complete (LDS only)
    x_prime<DK, DV, NT>(sm, Y, col_of(), g, Wm);
    emit_outputs<DK, DV, NT>(sm, Z, Wm, g, l16, t0, Treal, uo.B,
                             out_rsrc(va, r, h, DV, max(Dq, 1)), col_of() * 4, HV * DV * 4);
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

}  // namespace gdnr
