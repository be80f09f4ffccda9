// index_keys_fp8.hip -- FP8 storage of the indexer keys (gfx950), the
// low-precision indexer-key variant.
//
// The pages give the global KV per token (890 bytes for the whole model) and
// the main KV's FP4 format, but not the indexer key's precision ("DeepSeek AI
// выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн токенов, KV-кэшем FP4
// ..." (wire.sakhanda.co), opening paragraph and section "FP4 KV,
// ограниченное повторное проигрывание и другие расширения").  This variant
// stores each key row as OCP E4M3FN codes with one power-of-two scale:
//   E    = the smallest integer with amax <= 448 * 2^E, at least -124;
//   code = the E4M3FN value nearest to k / 2^E (ties to the even code, sign
//          copied from k, so -0 gives 0x80);
//   exponent byte = E + 127 (the biased exponent of the fp32 2^E).
// The stored key code * 2^E has at most 4 significant bits and a quantum of
// at least 2^-133, so it is a bf16 value: the variant's score is the ordinary
// score of the stored keys (csa2.h), 129 bytes per 128-dim key instead of 256.
//
// 16 lanes per row (4 rows per wave): lane l of a row owns dims D/16 l ..,
// the row's largest magnitude comes from a 16-lane max, and every step is
// exact fp32 arithmetic (frexp, ldexp by powers of two, rint = round to
// nearest even).
#include "csa2_device.h"

#include "../../include/csa2.h"

namespace csa2 {

constexpr int kKeyThreads = 256;

// E4M3FN magnitude code nearest to y in [0, 448], ties to even.
__device__ __forceinline__ uint32_t e4m3_code_rne(float y) {
  if (y < 0.015625f) return (uint32_t)rintf(y * 512.0f);   // quantum 2^-9; 8 is 2^-6 = code 0x08
  const int e = __builtin_amdgcn_frexp_expf(y) - 1;          // y in [2^e, 2^(e+1))
  int m = (int)rintf(ldexpf(y, 3 - e));                      // 8 .. 16, exact quotient
  int ee = e;
  if (m == 16) {
    m = 8;
    ee += 1;
  }
  return (uint32_t)(((ee + 7) << 3) | (m - 8));
}

template <int D>
__global__ __launch_bounds__(kKeyThreads) void k_index_keys_fp8(const uint16_t* ik, int64_t rows, uint8_t* codes,
                                                               uint8_t* exps) {
  constexpr int EPL = D / 16;   // dims per lane
  const int64_t row = (int64_t)blockIdx.x * (kKeyThreads / 16) + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  if (row >= rows) return;   // whole 16-lane groups
  float v[EPL];
  const uint16_t* src = ik + (size_t)row * D + EPL * l;
  if constexpr (EPL == 8) {
    const uint4 r = *reinterpret_cast<const uint4*>(src);
    const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(wd[j] << 16);
      v[2 * j + 1] = __uint_as_float(wd[j] & 0xFFFF0000u);
    }
  } else {
    const uint2 r = *reinterpret_cast<const uint2*>(src);
    const uint32_t wd[2] = {r.x, r.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v[2 * j] = __uint_as_float(wd[j] << 16);
      v[2 * j + 1] = __uint_as_float(wd[j] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  // E: 448 2^E = 1.75 2^(E+8) >= amax = f 2^u with f in [1, 2)
  int E = -124;
  if (amax > 0.0f) {
    const float f = 2.0f * __builtin_amdgcn_frexp_mantf(amax);
    const int u = __builtin_amdgcn_frexp_expf(amax) - 1;
    E = max(f <= 1.75f ? u - 8 : u - 7, -124);
  }
  uint32_t packed[EPL / 4];
#pragma unroll
  for (int w = 0; w < EPL / 4; ++w) packed[w] = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const uint32_t sign = (__float_as_uint(v[j]) >> 24) & 0x80u;
    const uint32_t c = e4m3_code_rne(ldexpf(fabsf(v[j]), -E)) | sign;
    packed[j >> 2] |= c << (8 * (j & 3));
  }
  uint8_t* dst = codes + (size_t)row * D + EPL * l;
  if constexpr (EPL == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
  else *reinterpret_cast<uint32_t*>(dst) = packed[0];
  if (l == 0) exps[row] = (uint8_t)(E + 127);
}

}  // namespace csa2

extern "C" csa2_status csa2_index_keys_fp8(const uint16_t* ik, int d_i, int64_t rows, uint8_t* codes,
                                           uint8_t* exps, void* stream) {
  csa2::set_last_hip_error(0);
  if (rows < 0) return CSA2_E_INVAL;
  if (d_i != 64 && d_i != 128) return CSA2_E_UNSUPPORTED;
  if (rows == 0) return CSA2_OK;
  if (!ik || !codes || !exps) return CSA2_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(ik) & 15) || (reinterpret_cast<uintptr_t>(codes) & 7)) return CSA2_E_INVAL;
  const int64_t blocks = (rows + csa2::kKeyThreads / 16 - 1) / (csa2::kKeyThreads / 16);
  if (blocks > 0x7FFFFFFF) return CSA2_E_INVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d_i == 128)
    hipLaunchKernelGGL(csa2::k_index_keys_fp8<128>, dim3((unsigned)blocks), dim3(csa2::kKeyThreads), 0, st, ik, rows,
                       codes, exps);
  else
    hipLaunchKernelGGL(csa2::k_index_keys_fp8<64>, dim3((unsigned)blocks), dim3(csa2::kKeyThreads), 0, st, ik, rows,
                       codes, exps);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    csa2::set_last_hip_error((int)e);
    return CSA2_E_HIP;
  }
  return CSA2_OK;
}
