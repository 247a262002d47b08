// cache_write.hip -- fp4_cache_write: bf16 entries -> FP4 main cache + MXFP4 keys.
//
// Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", FP4 KV cache section (main
// entries: E2M1 with one E4M3 scale per 16 channels, no global scale; indexer keys:
// OCP MXFP4, E2M1 with one E8M0 scale per 32 channels; one format for all channels).
//
// One wavefront per entry.  Lane l owns latent channels 8l .. 8l+7 (one 16-byte
// load, half of a 16-channel scale block) and key channels 2l, 2l+1 (a 32-channel
// block spans 16 lanes).  Block maxima are wave shuffles; codes are written as one
// dword (main) and one byte (key) per lane, so every store is coalesced.
#include "common.hpp"
#include "host_common.hpp"

namespace csa2 {

__global__ __launch_bounds__(256) void cache_write_kernel(uint8_t* __restrict__ main_codes,
                                                          uint8_t* __restrict__ main_scales,
                                                          uint8_t* __restrict__ idx_codes,
                                                          uint8_t* __restrict__ idx_scales,
                                                          const uint16_t* __restrict__ latent,
                                                          const uint16_t* __restrict__ idx_key,
                                                          const int64_t* __restrict__ slot, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;  // uniform per wavefront
  const int64_t s = slot[row];

  // ---- main entry: 32 blocks of 16 channels, two lanes per block
  const uint4 raw = *reinterpret_cast<const uint4*>(latent + row * kLatentDim + lane * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  // nearest E4M3 to amax/6: fl32(amax/6) cannot cross or land on an E4M3 midpoint
  // unless amax/6 itself does (amax has 8 significant bits, a midpoint 5), so the
  // correctly rounded quotient gives the exact answer.
  const uint32_t sb = e4m3_from_nonneg(amax / 6.0f);
  const float sc = e4m3_value(sb);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t c = (sc == 0.0f) ? ((__float_as_uint(v[i]) >> 28) & 8u) : e2m1_code(v[i], sc);
    packed |= c << (4 * i);
  }
  reinterpret_cast<uint32_t*>(main_codes + s * kMainRowBytes)[lane] = packed;
  if ((lane & 1) == 0) main_scales[s * kMainScaleBytes + (lane >> 1)] = (uint8_t)sb;

  // ---- indexer key: 4 blocks of 32 channels, 16 lanes per block
  const uint32_t kr = reinterpret_cast<const uint32_t*>(idx_key + row * kIndexDim)[lane];
  const float k0 = bf16_to_f32(kr & 0xFFFFu), k1 = bf16_to_f32(kr >> 16);
  float kmax = fmaxf(fabsf(k0), fabsf(k1));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, o));
  const uint32_t u = mx_exponent(kmax);
  const float X = ldexpf(1.0f, (int)u - 127);
  const uint32_t kb = e2m1_code(k0, X) | (e2m1_code(k1, X) << 4);
  idx_codes[s * kIdxRowBytes + lane] = (uint8_t)kb;
  if ((lane & 15) == 0) idx_scales[s * kIdxScaleBytes + (lane >> 4)] = (uint8_t)u;
}

// ---- FP8 window rows -------------------------------------------------------
// "DeepSeek-V4.1-Flash, expliqué pas à pas", FP4 KV cache section: the window KV
// stays in FP8.  Format (the pages give none): E4M3FN codes and one E8M0 scale per
// 512-channel row, X = the smallest power of two with amax <= 448 X (no code
// saturates), code = nearest E4M3FN value to x / X with ties to even, sign copied;
// amax = 0 gives X = 2^-127.  One wavefront per row, lane l owns channels 8l..8l+7.
__global__ __launch_bounds__(256) void swa_fp8_write_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wavefront
  const uint4 raw = *reinterpret_cast<const uint4*>(x + row * kLatentDim + lane * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  // amax = m 2^ex with m in [1/2, 1): 448 X >= amax first holds at X = 2^(ex - 9)
  // when 2m <= 1.75, else at 2^(ex - 8)
  int e = -127;
  if (amax > 0.0f) {
    int ex;
    const float m = frexpf(amax, &ex);
    e = max(ex - 9 + (2.0f * m > 1.75f ? 1 : 0), -127);
  }
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = e4m3_from_nonneg(ldexpf(fabsf(v[i]), -e)) | ((__float_as_uint(v[i]) >> 24) & 0x80u);
    c[i >> 2] |= code << (8 * (i & 3));
  }
  *reinterpret_cast<uint2*>(codes + row * kLatentDim + lane * 8) = make_uint2(c[0], c[1]);
  if (lane == 0) scales[row] = (uint8_t)(e + 127);
}

}  // namespace csa2

using namespace csa2;

extern "C" int swa_fp8_write(const uint16_t* rows, int64_t n, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (n < 0) return CSA2_ERR_SHAPE;
  if (n == 0) return CSA2_OK;
  if (!rows || !codes || !scales) return CSA2_ERR_NULL;
  hipLaunchKernelGGL(swa_fp8_write_kernel, dim3(ceil_div(n, 4)), dim3(256), 0, stream, rows, n, codes, scales);
  return launch_status();
}

extern "C" int fp4_cache_write(const csa2_fp4_cache* cache, const uint16_t* latent, const uint16_t* idx_key,
                               const int64_t* slot, int64_t n, hipStream_t stream) {
  if (!cache_ok(cache)) return CSA2_ERR_NULL;
  if (!cache_shape_ok(cache) || n < 0) return CSA2_ERR_SHAPE;
  if (n == 0) return CSA2_OK;
  if (!latent || !idx_key || !slot) return CSA2_ERR_NULL;
  hipLaunchKernelGGL(cache_write_kernel, dim3(ceil_div(n, 4)), dim3(256), 0, stream, cache->main_codes,
                     cache->main_scales, cache->idx_codes, cache->idx_scales, latent, idx_key, slot, n);
  return launch_status();
}
