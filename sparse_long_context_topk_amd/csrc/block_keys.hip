// block_keys.hip -- stored block keys for the pool-based Full variant (gfx950).
//
// The hierarchical indexer groups positions into blocks of 8 and keeps at most
// 2048 of them ("DeepSeek AI выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн
// токенов, KV-кэшем FP4 ..." (wire.sakhanda.co), section "Сжатое разреженное
// внимание 2 (CSA2)").  When the Full layer picks its Top-512 inside its own
// pool, it scores blocks from a stored key per block instead of reading every
// token key: the block key is the mean of the member keys (fp32 sum from +0 in
// ascending position order, IEEE division by the member count, nearest-even to
// bf16; a partial last block averages its members).  The block scan itself is
// csa2_index_topk run over these keys.
//
// One thread per (block, 8 dims): it reads the members' 16-byte pieces (a
// wave covers whole 256-byte rows, so the reads are coalesced), sums them in
// order, divides and writes one 16-byte piece of the block key.  HBM-bound:
// 8 * 2 * d_i bytes read and 2 * d_i written per block.
#include "csa2_device.h"

#include "../../include/csa2.h"

namespace csa2 {

constexpr int kBlockKeyThreads = 256;

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;   // finite inputs (NaN/Inf are outside the contract)
}

__global__ __launch_bounds__(kBlockKeyThreads) void k_block_keys(const uint16_t* __restrict__ ik, int d_i,
                                                                const int64_t* __restrict__ seq_base,
                                                                const int32_t* __restrict__ seq_len,
                                                                const int32_t* __restrict__ blk_from,
                                                                int max_blocks, uint16_t* __restrict__ kbar,
                                                                const int64_t* __restrict__ kbar_base) {
  const int pieces = d_i >> 3;   // 16-byte pieces per key
  const int64_t t = (int64_t)blockIdx.x * kBlockKeyThreads + threadIdx.x;
  const int64_t lb = t / pieces;
  const int pc = (int)(t - lb * pieces);
  const int s = blockIdx.y;
  if (lb >= max_blocks) return;
  const int len = seq_len[s];
  const int64_t b = (int64_t)(blk_from ? blk_from[s] : 0) + lb;
  const int64_t nb = ((int64_t)len + 7) >> 3;
  if (b < 0 || b >= nb) return;
  const int64_t t0 = 8 * b;
  const int n = (int)min<int64_t>(8, (int64_t)len - t0);
  const uint4* src = reinterpret_cast<const uint4*>(ik + (size_t)(seq_base[s] + t0) * d_i) + pc;
  const size_t pitch = (size_t)pieces;   // uint4 per row
  uint4 r[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) r[m] = m < n ? src[m * pitch] : make_uint4(0, 0, 0, 0);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < n) {
      const uint32_t wd[4] = {r[m].x, r[m].y, r[m].z, r[m].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = acc[2 * j] + __uint_as_float(wd[j] << 16);
        acc[2 * j + 1] = acc[2 * j + 1] + __uint_as_float(wd[j] & 0xFFFF0000u);
      }
    }
  }
  const float cnt = (float)n;
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // n = 8: a multiplication by 1/8 rounds exactly as the division does
    const float lo = n == 8 ? acc[2 * j] * 0.125f : acc[2 * j] / cnt;
    const float hi = n == 8 ? acc[2 * j + 1] * 0.125f : acc[2 * j + 1] / cnt;
    o[j] = bf16_rne(lo) | (bf16_rne(hi) << 16);
  }
  reinterpret_cast<uint4*>(kbar + (size_t)(kbar_base[s] + b) * d_i)[pc] = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace csa2

extern "C" csa2_status csa2_block_keys(const uint16_t* ik, int d_i, const int64_t* seq_base, const int32_t* seq_len,
                                       const int32_t* blk_from, int n_seq, int max_blocks, uint16_t* kbar,
                                       const int64_t* kbar_base, void* stream) {
  csa2::set_last_hip_error(0);
  if (n_seq < 0 || max_blocks < 0) return CSA2_E_INVAL;
  if (d_i < 8 || d_i > 1024 || (d_i & 7)) return CSA2_E_UNSUPPORTED;
  if (n_seq == 0 || max_blocks == 0) return CSA2_OK;
  if (!ik || !seq_base || !seq_len || !kbar || !kbar_base) return CSA2_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(ik) & 15) || (reinterpret_cast<uintptr_t>(kbar) & 15) ||
      (reinterpret_cast<uintptr_t>(seq_base) & 7) || (reinterpret_cast<uintptr_t>(kbar_base) & 7) ||
      (reinterpret_cast<uintptr_t>(seq_len) & 3) || (reinterpret_cast<uintptr_t>(blk_from) & 3))
    return CSA2_E_INVAL;
  if (n_seq > 65535) return CSA2_E_INVAL;
  const int64_t threads = (int64_t)max_blocks * (d_i >> 3);
  const int64_t grid = (threads + csa2::kBlockKeyThreads - 1) / csa2::kBlockKeyThreads;
  if (grid > 0x7FFFFFFF) return CSA2_E_INVAL;
  hipLaunchKernelGGL(csa2::k_block_keys, dim3((unsigned)grid, (unsigned)n_seq), dim3(csa2::kBlockKeyThreads), 0,
                     static_cast<hipStream_t>(stream), ik, d_i, seq_base, seq_len, blk_from, max_blocks, kbar,
                     kbar_base);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    csa2::set_last_hip_error((int)e);
    return CSA2_E_HIP;
  }
  return CSA2_OK;
}
