// window_append.hip -- append rows to a layer's sliding-window KV (gfx950).
//
// Every layer attends over its own 128-token sliding window besides the
// selected FP4 entries, and keeps that window KV itself ("DeepSeek AI
// выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн токенов, KV-кэшем FP4
// ..." (wire.sakhanda.co), sections "Каузальный энкодер-декодер" and "Сжатое
// разреженное внимание 2 (CSA2)").  The pages give the window's length but not
// its precision; it is kept in bf16 (only the main KV is said to be FP4).
//
// A decode step writes each layer's new window row into a ring of 128 rows per
// (layer, sequence): position p goes to ring row p mod 128, so the ring always
// holds the last min(L, 128) positions and the attention reads its first
// min(L, 128) rows (a softmax does not depend on the order of its keys).
//
// One wave per row; lane l owns channels 8l .. 8l+7: one coalesced 1 KiB
// (bf16) or 2 KiB (fp32) read and a 1 KiB write.  fp32 input is rounded to the
// nearest bf16, ties to even.
#include "csa2_device.h"

#include "../../include/csa2.h"

namespace csa2 {

__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) {
  const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  const uint32_t ra = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
  const uint32_t rb = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  return ra | (rb << 16);
}

__global__ __launch_bounds__(256) void k_window_append(const void* __restrict__ x, int x_f32, int64_t n_rows,
                                                     const int64_t* __restrict__ dst_row,
                                                     uint16_t* __restrict__ swa, int64_t swa_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  const int64_t d = dst_row[r];
  if (d < 0 || d >= swa_rows) return;
  uint4 v;
  if (x_f32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + r * CSA2_KV_CH) + 2 * lane;
    const float4 a = src[0], b = src[1];
    v = make_uint4(bf16_pair_rne(a.x, a.y), bf16_pair_rne(a.z, a.w), bf16_pair_rne(b.x, b.y),
                   bf16_pair_rne(b.z, b.w));
  } else {
    v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + r * CSA2_KV_CH)[lane];
  }
  reinterpret_cast<uint4*>(swa + d * CSA2_KV_CH)[lane] = v;
}

}  // namespace csa2

extern "C" csa2_status csa2_window_append(const void* x, int x_dtype, int64_t n_rows, const int64_t* dst_row,
                                          uint16_t* swa, int64_t swa_rows, void* stream) {
  csa2::set_last_hip_error(0);
  if (n_rows < 0 || swa_rows < 0) return CSA2_E_INVAL;
  if (x_dtype != CSA2_F32 && x_dtype != CSA2_BF16) return CSA2_E_INVAL;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !dst_row || !swa) return CSA2_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(dst_row) & 7) ||
      (reinterpret_cast<uintptr_t>(swa) & 15))
    return CSA2_E_INVAL;
  if (n_rows > ((int64_t)1 << 33)) return CSA2_E_INVAL;
  const int64_t blocks = (n_rows + 3) / 4;
  hipLaunchKernelGGL(csa2::k_window_append, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     x, x_dtype == CSA2_F32 ? 1 : 0, n_rows, dst_row, swa, swa_rows);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    csa2::set_last_hip_error((int)e);
    return CSA2_E_HIP;
  }
  return CSA2_OK;
}
