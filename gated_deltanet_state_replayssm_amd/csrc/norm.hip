// Gated RMSNorm of the GDN output followed by FP8 quantisation, in one kernel.
//
// "The inference stack behind OCRia" (LlamaIndex), section on fusing kernels to
// avoid HBM round trips: the gated RMSNorm is fused with the FP8 quantisation
// of its result. Per (token, value head) group of d_v outputs o:
//     r = sqrt(mean_j o_j^2 + eps),  y_j = o_j / r * w_j * silu(z_j),
//     s = max_j |y_j| / 448 (1 for an all-zero group),  c_j = E4M3(y_j / s)
// with OCP E4M3 codes (bias 7, largest finite 448), round to nearest even,
// saturating. Each half of a wave (32 lanes) takes one group: a lane holds
// EPL consecutive values; the sum of squares and the maximum are reduced across
// the half with DPP moves; the codes are written as EPL bytes per lane and the
// scale by the half's first lane. Memory-bound: 4 + 2 bytes read and 1 byte
// written per value.
#include "device_common.h"
#include "internal.h"

namespace gdnr {

namespace {

constexpr float kE4M3Max = 448.f;

// Sum / maximum over each half (32 lanes) of a wave with DPP moves: row shifts
// within rows of 16 lanes, then a broadcast of lane 15 into rows 1 and 3; lanes
// 31 and 63 end with the totals of the two halves, read across the wave.
template <bool MAX>
__device__ __forceinline__ float half_reduce(float v, bool upper) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  v = op(v, dpp_or<0x111, 0xf>(0.f, v));  // row_shr:1
  v = op(v, dpp_or<0x112, 0xf>(0.f, v));  // row_shr:2
  v = op(v, dpp_or<0x114, 0xf>(0.f, v));  // row_shr:4
  v = op(v, dpp_or<0x118, 0xf>(0.f, v));  // row_shr:8
  v = op(v, dpp_or<0x142, 0xa>(0.f, v));  // row_bcast:15 into rows 1 and 3
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return upper ? hi : lo;
}

// grid: ceil(groups / 8) workgroups of 4 waves; each half of a wave (32 lanes)
// handles one group (one (token, head) row of DV values): wave w of workgroup b
// takes groups 8 b + 2 w (lanes 0..31) and 8 b + 2 w + 1 (lanes 32..63). A lane
// holds EPL = DV / 32 consecutive values (16-byte loads of o at DV = 128).
template <int DV>
__global__ __launch_bounds__(256) void gated_rmsnorm_fp8_kernel(NormArgs a) {
  constexpr int EPL = DV >= 32 ? DV / 32 : 1;  // values per lane
  constexpr int LANES = DV / EPL;              // lanes of a half holding values
  static_assert(EPL == 1 || EPL == 2 || EPL == 4, "values per lane");
  const int lane = threadIdx.x & 63;
  const bool upper = lane >= 32;
  const int hl = lane & 31;
  const int64_t grp = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + (upper ? 1 : 0);
  if (((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 >= a.groups) return;  // whole wave
  const bool act = hl < LANES && grp < a.groups;
  const int hcol = hl * EPL;  // column of this lane's first value (weight index)
  const int64_t base = grp * DV + hcol;

  float o[EPL], zf[EPL], w[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = zf[e] = w[e] = 0.f;
  if (act) {
    if constexpr (EPL == 4) {
      const float4 ov = *reinterpret_cast<const float4 *>(a.o + base);
      const uint2 zb = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.z) + base);
      const float4 wv = *reinterpret_cast<const float4 *>(a.weight + hcol);
      o[0] = ov.x; o[1] = ov.y; o[2] = ov.z; o[3] = ov.w;
      zf[0] = __uint_as_float(zb.x << 16); zf[1] = __uint_as_float(zb.x & 0xffff0000u);
      zf[2] = __uint_as_float(zb.y << 16); zf[3] = __uint_as_float(zb.y & 0xffff0000u);
      w[0] = wv.x; w[1] = wv.y; w[2] = wv.z; w[3] = wv.w;
    } else if constexpr (EPL == 2) {
      const float2 ov = *reinterpret_cast<const float2 *>(a.o + base);
      const uint32_t zb = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(a.z) + base);
      const float2 wv = *reinterpret_cast<const float2 *>(a.weight + hcol);
      o[0] = ov.x; o[1] = ov.y;
      zf[0] = __uint_as_float(zb << 16); zf[1] = __uint_as_float(zb & 0xffff0000u);
      w[0] = wv.x; w[1] = wv.y;
    } else {
      o[0] = a.o[base];
      zf[0] = __uint_as_float((uint32_t)static_cast<const uint16_t *>(a.z)[base] << 16);
      w[0] = a.weight[hcol];
    }
  }

  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) ss = fmaf(o[e], o[e], ss);
  ss = half_reduce<false>(ss, upper);
  const float rinv = 1.f / sqrtf(ss * (1.f / DV) + a.eps);

  float y[EPL], amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float g = zf[e] / (1.f + __expf(-zf[e]));  // silu
    y[e] = o[e] * rinv * w[e] * g;
    amax = fmaxf(amax, fabsf(y[e]));
  }
  amax = half_reduce<true>(amax, upper);
  const float scale = amax > 0.f ? amax / kE4M3Max : 1.f;
  const float inv = amax > 0.f ? kE4M3Max / amax : 1.f;

  if (act) {
    // clamp first: the conversion then never sees a value past the largest code
    float c[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < EPL; ++e) c[e] = fminf(fmaxf(y[e] * inv, -kE4M3Max), kE4M3Max);
    uint32_t packed = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    if constexpr (EPL == 4) {
      packed = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)packed, true);
      *reinterpret_cast<uint32_t *>(a.q + base) = packed;
    } else if constexpr (EPL == 2) {
      *reinterpret_cast<uint16_t *>(a.q + base) = (uint16_t)(packed & 0xffff);
    } else {
      a.q[base] = (uint8_t)(packed & 0xff);
    }
    if (hl == 0) a.scale[grp] = scale;
  }
}

template <int DV>
hipError_t launch_dv(const NormArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.groups + 7) / 8));
  hipLaunchKernelGGL(gated_rmsnorm_fp8_kernel<DV>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_rmsnorm_fp8(const NormArgs &a, int dv, hipStream_t stream) {
  switch (dv) {
    case 16: return launch_dv<16>(a, stream);
    case 32: return launch_dv<32>(a, stream);
    case 64: return launch_dv<64>(a, stream);
    case 128: return launch_dv<128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdnr
