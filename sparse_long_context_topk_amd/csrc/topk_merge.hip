// topk_merge.hip -- exact Top-K of a query among given candidate positions
// (gfx950): the merge step of a context split over several devices.
//
// Split into position ranges, every shard can run the exact index call on
// its range and keep its local Top-K; the global Top-K lies in the union of
// the local ones, and a position's score does not depend on the shard that
// computed it (the score is fixed to the bit per (query, key)), so the exact
// Top-K among the union's positions is the whole context's Top-K.  The pages
// fix Top-512 by (score, position) over the context ("DeepSeek AI выпустила
// DeepSeek-V4.1-Flash с контекстом в 1 млн токенов, KV-кэшем FP4 ..."
// (wire.sakhanda.co), section "Сжатое разреженное внимание 2 (CSA2)").
//
// How: the candidates' keys are gathered into a contiguous row per query in
// the workspace (k_merge_gather), the exact selection runs over that short
// "sequence" (MFMA scores, bound, exact rescoring), and the chosen local
// indices are mapped back to positions (k_merge_remap).  Up to 16,384
// candidates the selection is csa2_reindex_topk over the pool of all the
// row's blocks of 8 (its one-work-group select: three launches in all);
// beyond, csa2_index_topk's multi-kernel select.
// Candidates are ascending, so a lower local index is a lower position and
// ties resolve as over the whole context.
#include "csa2_device.h"

#include "../../include/csa2.h"

namespace csa2 {

constexpr int kMergeThreads = 256;

// one 16-byte piece of a candidate key per thread; empty candidates give zero
// keys (they are past the query's candidate count and never scored)
__global__ __launch_bounds__(kMergeThreads) void k_merge_gather(const uint16_t* __restrict__ ik, int d_i,
                                                                const int32_t* __restrict__ q_seq,
                                                                const int64_t* __restrict__ seq_base,
                                                                const int32_t* __restrict__ cand, int n_cand,
                                                                uint16_t* __restrict__ keys,
                                                                int32_t* __restrict__ nvalid,
                                                                int32_t* __restrict__ ident,
                                                                int64_t* __restrict__ kbase,
                                                                int32_t* __restrict__ pool, int nb) {
  const int pieces = d_i >> 3;
  const int per_block = kMergeThreads / pieces;
  const int c = blockIdx.x * per_block + threadIdx.x / pieces;
  const int pc = threadIdx.x % pieces;
  const int q = blockIdx.y;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ident[q] = q;
    kbase[q] = (int64_t)q * n_cand;
  }
  if (c >= n_cand) return;
  if (pool && pc == 0 && (c & 7) == 0) pool[(size_t)q * nb + (c >> 3)] = c >> 3;   // every block of the row
  const int32_t* cq = cand + (size_t)q * n_cand;
  const int32_t pos = cq[c];
  // the candidate count: the list is -1 padded at its end only
  if (pc == 0) {
    if (c == 0 && pos < 0) nvalid[q] = 0;
    if (pos >= 0 && (c + 1 == n_cand || cq[c + 1] < 0)) nvalid[q] = c + 1;
  }
  uint4 v = make_uint4(0, 0, 0, 0);
  if (pos >= 0) v = reinterpret_cast<const uint4*>(ik + (size_t)(seq_base[q_seq[q]] + pos) * d_i)[pc];
  reinterpret_cast<uint4*>(keys + ((size_t)q * n_cand + c) * d_i)[pc] = v;
}

__global__ __launch_bounds__(kMergeThreads) void k_merge_remap(const int32_t* __restrict__ local, int k,
                                                               const int32_t* __restrict__ cand, int n_cand,
                                                               int32_t* __restrict__ idx_out) {
  const int r = blockIdx.x * kMergeThreads + threadIdx.x;
  const int q = blockIdx.y;
  if (r >= k) return;
  const int32_t l = local ? local[(size_t)q * k + r] : -1;   // no local list: no candidates
  idx_out[(size_t)q * k + r] = l >= 0 ? cand[(size_t)q * n_cand + l] : -1;
}

}  // namespace csa2

namespace {

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMergeSmall = 16384;   // candidates up to which the Reindex select runs

struct MergeLayout {
  size_t keys, nvalid, ident, kbase, local, pool, inner, total;
};

MergeLayout merge_layout(int n_q, int n_cand, int d_i, int k, int h_i) {
  MergeLayout L;
  size_t o = 0;
  L.keys = o;   o = a256(o + (size_t)n_q * n_cand * d_i * 2);
  L.nvalid = o; o = a256(o + (size_t)n_q * 4);
  L.ident = o;  o = a256(o + (size_t)n_q * 4);
  L.kbase = o;  o = a256(o + (size_t)n_q * 8);
  L.local = o;  o = a256(o + (size_t)n_q * k * 4);
  const int nb = (n_cand + 7) / 8;
  const bool small = n_cand <= kMergeSmall;
  L.pool = o;   o = a256(o + (small ? (size_t)n_q * nb * 4 : 0));
  L.inner = o;
  o = a256(o + (small ? csa2_reindex_topk_ws_bytes(n_q, h_i, d_i, k, 8, nb)
                      : csa2_index_topk_ws_bytes(n_q, n_cand, h_i, d_i, k, 8, 0)));
  L.total = o;
  return L;
}

}  // namespace

extern "C" size_t csa2_topk_merge_ws_bytes(int n_q, int n_cand, int h_i, int d_i, int k) {
  if (n_q <= 0 || n_cand <= 0 || d_i <= 0 || k <= 0) return 0;
  return merge_layout(n_q, n_cand, d_i, k, h_i).total;
}

extern "C" csa2_status csa2_topk_merge(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                       const int32_t* q_seq, const uint16_t* ik, const int64_t* seq_base,
                                       const int32_t* cand, int n_cand, int k, int32_t* idx_out, void* ws,
                                       size_t ws_bytes, void* stream) {
  csa2::set_last_hip_error(0);
  if (n_q < 0 || n_cand < 0 || k < 1 || k > 2048) return CSA2_E_INVAL;
  if (d_i != 64 && d_i != 128) return CSA2_E_UNSUPPORTED;
  if (n_cand > (1 << 25)) return CSA2_E_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!iq || !w || !q_seq || !ik || !seq_base || !idx_out || !ws || (n_cand > 0 && !cand)) return CSA2_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(ik) & 15) || (reinterpret_cast<uintptr_t>(ws) & 255)) return CSA2_E_INVAL;
  if (n_q > 65535) return CSA2_E_INVAL;
  const int nc = n_cand > 0 ? n_cand : 1;
  const MergeLayout L = merge_layout(n_q, nc, d_i, k, h_i);
  if (ws_bytes < L.total) return CSA2_E_WORKSPACE;
  char* w8 = static_cast<char*>(ws);
  uint16_t* keys = reinterpret_cast<uint16_t*>(w8 + L.keys);
  int32_t* nvalid = reinterpret_cast<int32_t*>(w8 + L.nvalid);
  int32_t* ident = reinterpret_cast<int32_t*>(w8 + L.ident);
  int64_t* kbase = reinterpret_cast<int64_t*>(w8 + L.kbase);
  int32_t* local = reinterpret_cast<int32_t*>(w8 + L.local);
  const bool small = n_cand <= kMergeSmall;
  const int nb = (n_cand + 7) / 8;
  int32_t* pool = small ? reinterpret_cast<int32_t*>(w8 + L.pool) : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 gremap((k + csa2::kMergeThreads - 1) / csa2::kMergeThreads, n_q);
  hipError_t e;
  if (n_cand == 0) {   // no candidates: every output is padding
    hipLaunchKernelGGL(csa2::k_merge_remap, gremap, dim3(csa2::kMergeThreads), 0, st,
                       static_cast<const int32_t*>(nullptr), k, static_cast<const int32_t*>(nullptr), 0, idx_out);
    e = hipGetLastError();
    if (e != hipSuccess) {
      csa2::set_last_hip_error((int)e);
      return CSA2_E_HIP;
    }
    return CSA2_OK;
  }
  const int per_block = csa2::kMergeThreads / (d_i >> 3);
  hipLaunchKernelGGL(csa2::k_merge_gather, dim3((n_cand + per_block - 1) / per_block, n_q),
                     dim3(csa2::kMergeThreads), 0, st, ik, d_i, q_seq, seq_base, cand, n_cand, keys, nvalid, ident,
                     kbase, pool, nb);
  e = hipGetLastError();
  if (e != hipSuccess) {
    csa2::set_last_hip_error((int)e);
    return CSA2_E_HIP;
  }
  const csa2_status s =
      small ? csa2_reindex_topk(iq, w, n_q, h_i, d_i, ident, nvalid, keys, kbase, pool, 8, nb, k, local, w8 + L.inner,
                                L.total - L.inner, stream)
            : csa2_index_topk(iq, w, n_q, h_i, d_i, ident, nvalid, n_cand, keys, kbase, k, local, 8, 0, nullptr,
                              w8 + L.inner, L.total - L.inner, stream);
  if (s != CSA2_OK) return s;
  hipLaunchKernelGGL(csa2::k_merge_remap, gremap, dim3(csa2::kMergeThreads), 0, st, local, k, cand, n_cand,
                     idx_out);
  e = hipGetLastError();
  if (e != hipSuccess) {
    csa2::set_last_hip_error((int)e);
    return CSA2_E_HIP;
  }
  return CSA2_OK;
}
