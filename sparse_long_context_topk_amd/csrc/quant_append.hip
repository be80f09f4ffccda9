// quant_append.hip -- write rows into the CSA2 FP4 main-KV cache (gfx950).
//
// The main KV is stored as E2M1 values with one E4M3 scale per 16 channels,
// NVFP4-style but without the global scale: "DeepSeek AI выпустила
// DeepSeek-V4.1-Flash с контекстом в 1 млн токенов, KV-кэшем FP4 ..."
// (wire.sakhanda.co), section "FP4 KV, ограниченное повторное проигрывание и
// другие расширения".  Record layout and rounding rules: csa2.h.
//
// One wave per row; lane l owns channels 8l..8l+7 (half of group l/2), so a
// row is one coalesced 1 KiB (bf16) or 2 KiB (fp32) read and a 256 B + 32 B
// write.  The scale is amax/6 rounded to E4M3 from the correctly rounded fp32
// quotient (no E4M3 midpoint can be crossed by that rounding: 6*midpoint is
// exact in fp32 and any other amax differs from it by more than the fp32
// quotient's half-ulp); the E2M1 codes come from exact comparisons of |x| with
// scale*midpoint (products of <= 4 and <= 3 significant bits, exact in fp32).
#include "csa2_device.h"

namespace csa2 {

// Nearest E4M3 (OCP FN) code to a non-negative q, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float q) {
  if (!(q < 448.0f)) return 0x7Eu;
  if (q < 0.015625f) return (uint32_t)rintf(q * 512.0f);  // subnormal: m * 2^-9 (m = 8 -> 0x08)
  uint32_t u = __float_as_uint(q);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  u &= 0xFFF00000u;
  const uint32_t e = (u >> 23) - 120u;  // (E + 127) - 127 + 7
  const uint32_t code = (e << 3) | ((u >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

__global__ __launch_bounds__(256) void k_quant_append(const void* x, int x_dtype, int64_t n_rows,
                                                      const int64_t* dst_row, uint8_t* cache,
                                                      int64_t cache_rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int64_t d = dst_row[row];
  if (d < 0 || d >= cache_rows) return;
  float v[8];
  if (x_dtype == CSA2_F32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + row * 512 + 8 * lane);
    const float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row * 512 + 8 * lane);
    const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(wd[j] << 16);
      v[2 * j + 1] = __uint_as_float(wd[j] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  const uint32_t sc = e4m3_rne_sat(__fdiv_rn(amax, 6.0f));
  const float s = e4m3_to_f32(sc);
  uint32_t packed = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = fabsf(v[j]);
    uint32_t mag = 0;
    if (s > 0.0f) {
      mag = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) + (a > 2.5f * s) +
            (a >= 3.5f * s) + (a > 5.0f * s);
    }
    const uint32_t code = mag | ((__float_as_uint(v[j]) >> 28) & 8u);
    packed |= code << (4 * j);
  }
  uint8_t* rec = cache + d * CSA2_KV_RECORD_BYTES;
  *reinterpret_cast<uint32_t*>(rec + 4 * lane) = packed;
  // one scale byte per group; the even lane of each pair stores it
  if ((lane & 1) == 0) rec[256 + (lane >> 1)] = (uint8_t)sc;
}

}  // namespace csa2

extern "C" csa2_status csa2_quant_append(const void* x, int x_dtype, int64_t n_rows, const int64_t* dst_row,
                                         uint8_t* cache, int64_t cache_rows, void* stream) {
  csa2::set_last_hip_error(0);
  if (n_rows < 0 || cache_rows < 0) return CSA2_E_INVAL;
  if (x_dtype != CSA2_F32 && x_dtype != CSA2_BF16) return CSA2_E_INVAL;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !dst_row || !cache) return CSA2_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(dst_row) & 7) ||
      (reinterpret_cast<uintptr_t>(cache) & 3))
    return CSA2_E_INVAL;
  if (n_rows > ((int64_t)1 << 40)) return CSA2_E_INVAL;
  const int64_t blocks = (n_rows + 3) / 4;
  if (blocks > 0x7FFFFFFF) return CSA2_E_INVAL;
  hipLaunchKernelGGL(csa2::k_quant_append, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     x, x_dtype, n_rows, dst_row, cache, cache_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    csa2::set_last_hip_error((int)e);
    return CSA2_E_HIP;
  }
  return CSA2_OK;
}
