// Chunked replay kernels for gfx950: verify (replay_single for ring capacity
// <= 32, one chunk; replay_chunked above) and flush (the same kernels with
// VERIFY = false). The building blocks and the chunked form are in chunk_ops.h.
#include "chunk_ops.h"

namespace gdnr {

namespace {

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
    if (wave == 1) build_m<DK, DV>(sm, g, l16);
    f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
    contract<DK, DV, NT, kY | kZ>(sm, H, g, l16, Y, Z);
    lds_barrier();  // M complete (LDS only)
    x_prime<DK, DV, NT>(sm, Y, col_of(), g, Wm);
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
  if constexpr (VERIFY) {
    if (wave == (WAVES > 1 ? 1 : 0)) build_m<DK, DV>(sm, g, l16);
  }

  f32x4 Y[2][NT], Z[2][NT], Wm[2][NT];
  contract<DK, DV, NT, VERIFY ? (kY | kZ) : kY>(sm, H, g, l16, Y, Z);
  if constexpr (VERIFY) {
    lds_barrier();  // M complete (LDS only)
    x_prime<DK, DV, NT>(sm, Y, colL, g, Wm);
  } else
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
