// common.hpp -- device helpers shared by the CSA2 FP4-cache kernels (gfx950).
//
// Formats (from "DeepSeek-V4.1-Flash, expliqué pas à pas", FP4 KV cache section):
//   E2M1  : 1 sign, 2 exponent, 1 mantissa bit; magnitudes {0,.5,1,1.5,2,3,4,6};
//           code = 8*sign + magnitude index.
//   E4M3FN: OCP 8-bit float, bias 7, largest finite 448, no infinities.
//   E8M0  : OCP power-of-two scale 2^(u-127).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CSA2_DEV __device__ __forceinline__

namespace csa2 {

constexpr int kLatentDim = 512;
constexpr int kIndexDim = 128;
constexpr int kPage = 64;
constexpr int kMainRowBytes = 256;  // 512 codes
constexpr int kMainScaleBytes = 32;
constexpr int kIdxRowBytes = 64;  // 128 codes
constexpr int kIdxScaleBytes = 4;

CSA2_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// E4M3FN byte -> value (exact in fp32).
CSA2_DEV float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float mag = (e == 0) ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
  return (b & 0x80u) ? -mag : mag;
}

// E4M3FN byte of the value nearest to v >= 0 (round to nearest, ties to even),
// saturating at 448.  Every rescaling below is by a power of two, hence exact, and
// rintf rounds to nearest-even.
CSA2_DEV uint32_t e4m3_from_nonneg(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  int e = (v < 0.015625f) ? -6 : (int)((__float_as_uint(v) >> 23) & 0xFFu) - 127;
  float r = rintf(ldexpf(v, 3 - e));
  int byte = ((e + 7) << 3) + (int)r - 8;
  return (uint32_t)(byte > 0x7E ? 0x7E : byte);
}

// E2M1 code of x for a positive scale s: nearest of {0,.5,1,1.5,2,3,4,6}*s to |x|,
// ties to the even magnitude index, values beyond 6s clip to 6s, sign bit copied.
// Every threshold t*s is exact in fp32 (t has <= 3 and s <= 4 significant bits).
CSA2_DEV uint32_t e2m1_code(float x, float s) {
  float m = fabsf(x);
  uint32_t idx = (uint32_t)(m > 0.25f * s) + (uint32_t)(m >= 0.75f * s) + (uint32_t)(m > 1.25f * s) +
                 (uint32_t)(m >= 1.75f * s) + (uint32_t)(m > 2.5f * s) + (uint32_t)(m >= 3.5f * s) +
                 (uint32_t)(m > 5.0f * s);
  return idx | ((__float_as_uint(x) >> 28) & 8u);
}

// OCP MX shared exponent of a 32-element block from its largest magnitude:
// u = floor(log2 amax) - 2 + 127, clamped to [0, 254]; amax == 0 (or subnormal) -> 0.
CSA2_DEV uint32_t mx_exponent(float amax) {
  int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu);  // amax >= 0
  if (E == 0) return 0u;
  int u = E - 2;
  return (uint32_t)(u < 0 ? 0 : (u > 254 ? 254 : u));
}

// Signed E2M1 value times 2, an integer in [-12, 12]:
// magnitude index 0..7 -> 0 1 2 3 4 6 8 12.
CSA2_DEV int e2m1_twice(uint32_t c) {
  uint32_t i = c & 7u;
  int v = (i < 2u) ? (int)i : (int)((2u + (i & 1u)) << ((i >> 1) - 1u));
  return (c & 8u) ? -v : v;
}

// Order-preserving key of an fp32 score (larger score -> larger key); -0 and +0
// map to the same key so the comparison is numeric.
CSA2_DEV uint32_t score_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also waits for
// every outstanding global load, which would stall loads issued ahead of time to
// hide memory latency; this one leaves them in flight.
CSA2_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


// ---- cross-lane helpers (one wavefront of 64 lanes) --------------------------

// Max / sum over the lanes l, l^16, l^32, l^48 with the VALU lane swaps of gfx950:
// permlane16_swap(v, v) leaves the values of 16-lane rows 2i and 2i+1 in the two
// results, in that order, in every lane of both rows; permlane32_swap(v, v) does the
// same for the two halves.  Every lane combines the same operands in the same order.
CSA2_DEV float max_rows(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
CSA2_DEV float sum_rows(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// DPP lane exchanges within 16-lane rows (quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror): after the four steps every lane of a row holds the
// row's max / sum, combined in the same order in every lane.
template <int kCtrl>
CSA2_DEV float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, true));
}
CSA2_DEV float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return max_rows(v);
}
CSA2_DEV float wave_sum(float v) {
  v = v + dpp_f<0xB1>(v);
  v = v + dpp_f<0x4E>(v);
  v = v + dpp_f<0x141>(v);
  v = v + dpp_f<0x140>(v);
  return sum_rows(v);
}

// DPP row shift / row broadcast of a u32 (0 where the source lane is outside the
// row, or the lane's row is masked off).
template <int kCtrl, int kRowMask = 0xF>
CSA2_DEV uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 within each 16-lane
// row, then lane 15 of rows 0 / 2 into rows 1 / 3 and lane 31 into rows 2 and 3.
CSA2_DEV uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_u32<0x111>(v);
  v += dpp_u32<0x112>(v);
  v += dpp_u32<0x114>(v);
  v += dpp_u32<0x118>(v);
  v += dpp_u32<0x142, 0xA>(v);
  v += dpp_u32<0x143, 0xC>(v);
  return v;
}

}  // namespace csa2
