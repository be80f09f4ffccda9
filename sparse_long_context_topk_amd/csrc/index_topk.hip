// index_topk.hip -- CSA2 lightning-indexer scan and exact Top-K for gfx950.
//
// What is computed (csa2.h states the full contract): for each query, the
// indexer score of every candidate position, score = sum_h w_h ReLU(q_h . k),
// defined to the bit as an fp32 fma chain over d and then over h; the Top-K
// positions by (score desc, position asc).  Full layers score every visible
// position and may also build the hierarchical pool (blocks of 8, block key =
// bf16 mean key, Top-keep_blocks blocks); Reindex layers score the positions
// of a pool.  Sources: "DeepSeek AI выпустила DeepSeek-V4.1-Flash с
// контекстом в 1 млн токенов, KV-кэшем FP4 ..." (wire.sakhanda.co), section
// "Сжатое разреженное внимание 2 (CSA2)": the Full / Reindex / Reuse modes,
// Top-512, and the pool of up to 2048 blocks of 8 positions.
//
// How (one pass over the keys at HBM speed, exact result):
//  1. k_prologue  zeroes per-problem counters and histograms, and computes
//                 QW = sum_h |w_h| ||q_h|| for the rounding bound.
//  2. k_scan      streams the indexer keys once.  Scores come from bf16 MFMA
//                 (v_mfma_f32_16x16x32_bf16: 16 heads x 16 positions x 32
//                 dims per instruction, the query held in registers); each
//                 work-group keeps a 4096-bin histogram of the top 12 bits of
//                 the scores in LDS and the largest squared key norm.  With a
//                 pool, block keys are averaged in LDS from the keys already
//                 loaded and scored by MFMA as well, so the pool costs no
//                 extra HBM traffic.  The last work-group of a query turns the
//                 histogram into a threshold below which no Top-K member can
//                 lie: T = (lowest value of the bin holding the K-th score) -
//                 2*Delta, where Delta bounds |MFMA score - exact score| for
//                 every key:  Delta = C * QW * max||k|| (Cauchy-Schwarz on
//                 the dot-product rounding error, ReLU is 1-Lipschitz, plus
//                 the head-sum rounding), C from the fp32 error constants with
//                 a 2x safety factor.
//  3. k_compact   keeps the candidates with approximate score >= T in
//                 position order; its last work-group finds the exact K-th
//                 approximate score a_K (radix select) and narrows the band
//                 to a >= a_K - 2*Delta.  Every exact Top-K member is in this
//                 band (it has exact score >= the K-th exact score >= a_K -
//                 Delta, hence approximate score >= a_K - 2*Delta).
//  4. k_rescore   recomputes the band's scores with the exact fp32 chain
//                 (one lane per head, then one lane for the head sum); its
//                 last work-group selects the Top-K by (score desc, position
//                 asc) with a radix select on the exact scores and writes the
//                 positions in ascending order.
// Degenerate inputs (ties everywhere) only make the band large; the result
// stays exact.
#include "csa2_device.h"

namespace csa2 {
namespace idx {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kNBins = 4096;
constexpr int kBinShift = 20;
constexpr int kCmpChunk = 4096;
constexpr int kCmpPerThread = kCmpChunk / kThreads;
constexpr int kRescoreWGs = 32;

struct Meta {
  uint32_t scan_done, cmp_done, rs_done, maxk2;
  float qw, wabs, thr, delta;
  int32_t nc, nband, nband2, pad0;
  uint32_t pad[4];
};
static_assert(sizeof(Meta) == 64, "Meta is one 64-byte line");

struct Entry {
  int32_t cand;
  float s;
};

struct Params {
  const uint16_t* iq;
  const float* w;
  int n_q, h_i, d_i;
  const int32_t* q_seq;
  const int32_t* q_nvis;
  const uint16_t* ik;
  const int64_t* seq_base;
  const int32_t* pool_in;  // Reindex: [n_q][keep_in]
  int keep_in;
  int k;                   // Top-K of the token problem
  int keep_blocks;         // Top-K of the block problem (0: none)
  int32_t* idx_out;
  int32_t* pool_out;
  int nprob;
  int reindex;
  int scan_chunk;
  int64_t stride;          // slots per problem in scores / band arrays
  int nchunk_cmp;
  float bound_c;
  float* scores;
  uint32_t* hist;
  Meta* meta;
  uint32_t* chunk_cnt;
  Entry* band_a;
  Entry* band_b;
};

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float delta_of(const Meta& m, float bound_c, int d_i) {
  float kn = sqrtf(__uint_as_float(m.maxk2));
  return bound_c * m.qw * kn * (1.0f + 0.0009765625f) + m.wabs * (float)d_i * 7.8886e-31f;
}

// Band threshold below a value v: v - 2*Delta with room for the rounding of
// this subtraction itself.
__device__ __forceinline__ float band_below(float v, float delta) {
  return v - 2.0f * delta * (1.0f + 0.00390625f) - fabsf(v) * 9.5367431640625e-07f;
}

// Exclusive prefix sum over the work-group (256 threads); returns the
// exclusive offset of this thread and writes the total to *total.
__device__ __forceinline__ uint32_t wg_exclusive_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    uint32_t t = s_tmp[i];
    if (i < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// K-th largest of the sortable keys key_of(i), i < n (1 <= K <= n), by a
// most-significant-digit radix select with 8-bit digits.  Returns the key and
// in *ties the number of entries equal to it that belong to the Top-K.
template <typename KeyOf>
__device__ uint32_t wg_kth_largest(int n, int K, KeyOf key_of, uint32_t* s_hist /*256*/,
                                   uint32_t* s_tmp, uint32_t* ties) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    s_hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      uint32_t key = key_of(i);
      if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // suffix sums: S[d] = sum_{d' >= d} hist[d'] ; thread tid owns digit 255 - tid
    uint32_t v = s_hist[255 - tid];
    uint32_t tot;
    uint32_t excl = wg_exclusive_scan(v, s_tmp, &tot);  // sum over digits above
    uint32_t incl = excl + v;
    if (excl < remaining && incl >= remaining) {
      s_tmp[8] = 255u - tid;
      s_tmp[9] = excl;
    }
    __syncthreads();
    uint32_t d = s_tmp[8];
    remaining -= s_tmp[9];
    prefix |= d << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  *ties = remaining;
  return prefix;
}

__device__ __forceinline__ int cand_pos(const Params& P, int q, int kind, int cand) {
  if (P.reindex) {
    int b = P.pool_in[(size_t)q * P.keep_in + (cand >> 3)];
    return b * 8 + (cand & 7);
  }
  (void)kind;
  return cand;
}

// ---------------------------------------------------------------- 1. prologue
__global__ __launch_bounds__(kThreads) void k_prologue(Params P) {
  const int p = blockIdx.x, q = p % P.n_q, kind = p / P.n_q;
  uint32_t* h = P.hist + (size_t)p * kNBins;
  for (int i = threadIdx.x; i < kNBins; i += kThreads) h[i] = 0;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    float qn = 0.0f, wa = 0.0f;
    if (lane < P.h_i) {
      const uint16_t* qh = P.iq + ((size_t)q * P.h_i + lane) * P.d_i;
      float ss = 0.0f;
      for (int d = 0; d < P.d_i; ++d) {
        float v = bf16_to_f32(qh[d]);
        ss = fmaf(v, v, ss);
      }
      wa = fabsf(P.w[(size_t)q * P.h_i + lane]);
      qn = wa * sqrtf(ss);
    }
    qn = wave_sum(qn);
    wa = wave_sum(wa);
    if (lane == 0) {
      Meta m;
      m.scan_done = m.cmp_done = m.rs_done = m.maxk2 = 0;
      m.qw = qn * (1.0f + 0.0009765625f);
      m.wabs = wa;
      m.thr = -INFINITY;
      m.delta = 0.0f;
      int nvis = P.q_nvis[q];
      m.nc = P.reindex ? 8 * P.keep_in : (kind == 0 ? nvis : (nvis + 7) / 8);
      m.nband = m.nband2 = m.pad0 = 0;
      for (int i = 0; i < 4; ++i) m.pad[i] = 0;
      P.meta[p] = m;
    }
  }
}

// Threshold from the global histogram of problem p (run by one work-group).
__device__ void wg_threshold(const Params& P, int p, int K, uint32_t* s_tmp) {
  const int tid = threadIdx.x;
  const uint32_t* h = P.hist + (size_t)p * kNBins;
  constexpr int kPer = kNBins / kThreads;  // 16 bins per thread
  // thread tid owns bins [kNBins - kPer*(tid+1), kNBins - kPer*tid): highest first
  const int b_hi = kNBins - kPer * tid - 1;
  uint32_t loc = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) loc += h[b_hi - j];
  uint32_t tot;
  uint32_t above = wg_exclusive_scan(loc, s_tmp, &tot);
  const Meta m = P.meta[p];
  const float delta = delta_of(m, P.bound_c, P.d_i);
  if (tid == 0 && tot <= (uint32_t)K) {
    P.meta[p].thr = -INFINITY;
    P.meta[p].delta = delta;
  }
  if (tot > (uint32_t)K && above < (uint32_t)K && above + loc >= (uint32_t)K) {
    uint32_t run = above;
    int bstar = b_hi;
    for (int j = 0; j < kPer; ++j) {
      run += h[b_hi - j];
      if (run >= (uint32_t)K) {
        bstar = b_hi - j;
        break;
      }
    }
    float t0 = unsortable((uint32_t)bstar << kBinShift);
    P.meta[p].thr = band_below(t0, delta);
    P.meta[p].delta = delta;
  }
}

// ---------------------------------------------------------------- 2. scan
template <int D, int MT, bool POOL, bool INDIRECT>
__global__ __launch_bounds__(kThreads) void k_scan(Params P) {
  constexpr int KS = D / 32;   // MFMA k-steps; also 16-byte loads per lane per key
  constexpr int DPL = D / 4;   // key dims held by one lane (one quarter of the key)
  constexpr int U4 = D / 8;    // 16-byte words per key row
  __shared__ uint32_t s_hist[kNBins];
  __shared__ uint32_t s_hist_b[POOL ? kNBins : 1];
  __shared__ uint4 s_stage[POOL ? kWaves * 16 * U4 : 1];
  __shared__ uint4 s_bkey[POOL ? kWaves * 16 * U4 : 1];
  __shared__ uint32_t s_tmp[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int q = blockIdx.y;
  const int p = q;                 // token problem
  const int pb = P.n_q + q;        // block problem (POOL)
  const int nvis = P.q_nvis[q];
  const int64_t base = P.seq_base[P.q_seq[q]];
  const int nc = INDIRECT ? 8 * P.keep_in : nvis;
  const int nblk = (nvis + 7) >> 3;
  const int c0 = blockIdx.x * P.scan_chunk;

  for (int i = tid; i < kNBins; i += kThreads) {
    s_hist[i] = 0;
    if (POOL) s_hist_b[i] = 0;
  }

  // query (A operand): lane (n, g) holds head 16*mt + n, dims g*DPL + 8*ks .. +7
  bf16x8 qa[MT][KS];
  float wr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = 16 * mt + n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (head < P.h_i)
        v = *reinterpret_cast<const uint4*>(P.iq + ((size_t)q * P.h_i + head) * D + g * DPL + 8 * ks);
      qa[mt][ks] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * mt + 4 * g + i;
      wr[mt][i] = hh < P.h_i ? P.w[(size_t)q * P.h_i + hh] : 0.0f;
    }
  }
  __syncthreads();

  float mk2 = 0.0f, mk2b = 0.0f;
  float* sc = P.scores + (size_t)p * P.stride;
  float* scb = P.scores + (size_t)pb * P.stride;
  const int nslots = min(P.scan_chunk, max(nc - c0, 0));
  const int ngroups = (nslots + 15) >> 4;
  int batch_slot = 0;   // POOL: groups collected in the current block batch
  int batch_first = 0;  // POOL: loop index of the batch's first group

  auto score_tile = [&](const uint4* kb, f32x4* acc) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 b = __builtin_bit_cast(bf16x8, kb[ks]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], b, acc[mt], 0, 0, 0);
    }
    float part = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(wr[mt][i], fmaxf(acc[mt][i], 0.0f), part);
    part += __shfl_xor(part, 16, kWave);
    part += __shfl_xor(part, 32, kWave);
    return part;
  };
  auto norm2 = [&](const uint4* kb) {
    float k2 = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t wds[4] = {kb[ks].x, kb[ks].y, kb[ks].z, kb[ks].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo = __uint_as_float(wds[j] << 16), hi = __uint_as_float(wds[j] & 0xFFFF0000u);
        k2 = fmaf(lo, lo, k2);
        k2 = fmaf(hi, hi, k2);
      }
    }
    k2 += __shfl_xor(k2, 16, kWave);
    k2 += __shfl_xor(k2, 32, kWave);
    return k2;
  };

  // Block batch: 8 groups -> 16 block keys in s_bkey[wave], scored by one MFMA tile.
  auto flush_blocks = [&](int nfill) {
    if constexpr (POOL) {
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      __builtin_amdgcn_wave_barrier();
      // slot n = (group t = n/2 of the batch, block j = n%2)
      const int t = n >> 1, j = n & 1;
      const int gi = wave + kWaves * (batch_first + t);
      const int blk = (c0 >> 3) + 2 * gi + j;
      const bool valid = t < nfill && blk < nblk;
      uint4 kb[KS];
      const uint4* row = s_bkey + (wave * 16 + n) * U4 + g * KS;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[ks] = row[ks];
      f32x4 acc[MT];
      float a = score_tile(kb, acc);
      float k2 = norm2(kb);
      if (valid) {
        if (g == 0) {
          scb[blk] = a;
          atomicAdd(&s_hist_b[sortable(a) >> kBinShift], 1u);
        }
        mk2b = fmaxf(mk2b, k2);
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      __builtin_amdgcn_wave_barrier();
    }
  };

  for (int it = 0;; ++it) {
    const int gi = wave + kWaves * it;
    if (gi >= ngroups) break;
    const int cand = c0 + 16 * gi + n;
    bool valid;
    int pos;
    if (INDIRECT) {
      const int b = cand < nc ? P.pool_in[(size_t)q * P.keep_in + (cand >> 3)] : -1;
      pos = b * 8 + (cand & 7);
      valid = b >= 0 && pos < nvis;
    } else {
      pos = cand;
      valid = cand < nc;
    }
    uint4 kb[KS];
    const uint4* src = reinterpret_cast<const uint4*>(P.ik + (size_t)(base + (valid ? pos : 0)) * D + g * DPL);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = valid ? src[ks] : make_uint4(0, 0, 0, 0);
    f32x4 acc[MT];
    float a = score_tile(kb, acc);
    float k2 = norm2(kb);
    if (g == 0 && cand < nc) {
      sc[cand] = valid ? a : -INFINITY;
      if (valid) atomicAdd(&s_hist[sortable(a) >> kBinShift], 1u);
    }
    if (valid) mk2 = fmaxf(mk2, k2);

    if constexpr (POOL) {
      // stage the 16 keys (natural dim order) and average each block of 8
      uint4* st = s_stage + (wave * 16 + n) * U4 + g * KS;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) st[ks] = kb[ks];
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      __builtin_amdgcn_wave_barrier();
      const int j = lane >> 5;                 // block of the group
      const int first = c0 + 16 * gi + 8 * j;  // its first position
      const int nb = min(max(nvis - first, 0), 8);
      const float inv_cnt = (float)nb;
      const uint16_t* stage16 = reinterpret_cast<const uint16_t*>(s_stage + wave * 16 * U4);
      uint16_t* bk16 = reinterpret_cast<uint16_t*>(s_bkey + (wave * 16 + 2 * batch_slot + j) * U4);
      constexpr int DPB = D / 32;  // dims per lane for the block mean
#pragma unroll
      for (int e = 0; e < DPB; ++e) {
        const int d = (lane & 31) * DPB + e;
        float s = 0.0f;
        for (int t = 0; t < nb; ++t) s = s + bf16_to_f32(stage16[(8 * j + t) * D + d]);
        uint32_t kbar = nb ? f32_to_bf16_rne(__fdiv_rn(s, inv_cnt)) : 0u;
        bk16[d] = (uint16_t)kbar;
      }
      ++batch_slot;
      if (batch_slot == 8) {
        flush_blocks(8);
        batch_slot = 0;
        batch_first = it + 1;
      }
    }
  }
  if constexpr (POOL) {
    if (batch_slot > 0) flush_blocks(batch_slot);
  }

  // ---- publish histograms and key norms
  __syncthreads();
  {
    uint32_t* gh = P.hist + (size_t)p * kNBins;
    for (int i = tid; i < kNBins; i += kThreads) {
      uint32_t c = s_hist[i];
      if (c) atomicAdd(&gh[i], c);
      if (POOL) {
        uint32_t cb = s_hist_b[i];
        if (cb) atomicAdd(&P.hist[(size_t)pb * kNBins + i], cb);
      }
    }
    mk2 = wave_max(mk2);
    mk2b = wave_max(mk2b);
    if (lane == 0) {
      s_tmp[wave] = __float_as_uint(mk2);
      s_tmp[4 + wave] = __float_as_uint(mk2b);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t m0 = 0, m1 = 0;
      for (int i = 0; i < kWaves; ++i) {
        m0 = max(m0, s_tmp[i]);
        m1 = max(m1, s_tmp[4 + i]);
      }
      if (m0) atomicMax(&P.meta[p].maxk2, m0);
      if (POOL && m1) atomicMax(&P.meta[pb].maxk2, m1);
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t prev = atomic_inc_acq_rel(&P.meta[p].scan_done);
    s_tmp[12] = (prev == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_tmp[12]) return;
  __threadfence();
  wg_threshold(P, p, P.k, s_tmp);
  if (POOL) {
    __syncthreads();
    wg_threshold(P, pb, P.keep_blocks, s_tmp);
  }
}

// ---------------------------------------------------------------- 3. compaction
__global__ __launch_bounds__(kThreads) void k_compact(Params P) {
  __shared__ uint32_t s_tmp[16];
  __shared__ uint32_t s_hist[256];
  const int tid = threadIdx.x;
  const int p = blockIdx.y, chunk = blockIdx.x;
  const float thr = P.meta[p].thr;
  const int nc = P.meta[p].nc;
  const int c0 = chunk * kCmpChunk;
  const int my0 = c0 + tid * kCmpPerThread;
  const float* sc = P.scores + (size_t)p * P.stride;
  float v[kCmpPerThread];
  uint32_t flags = 0;
  if (my0 < nc) {
    const float4* s4 = reinterpret_cast<const float4*>(sc + my0);
#pragma unroll
    for (int j = 0; j < kCmpPerThread / 4; ++j) {
      float4 t = s4[j];
      v[4 * j] = t.x;
      v[4 * j + 1] = t.y;
      v[4 * j + 2] = t.z;
      v[4 * j + 3] = t.w;
    }
#pragma unroll
    for (int j = 0; j < kCmpPerThread; ++j) {
      bool keep = (my0 + j < nc) && v[j] != -INFINITY && v[j] >= thr;
      flags |= (keep ? 1u : 0u) << j;
    }
  }
  uint32_t total;
  uint32_t off = wg_exclusive_scan(__popc(flags), s_tmp, &total);
  Entry* dst = P.band_a + (size_t)p * P.stride + c0;
#pragma unroll
  for (int j = 0; j < kCmpPerThread; ++j)
    if (flags & (1u << j)) dst[off++] = Entry{my0 + j, v[j]};
  if (tid == 0) P.chunk_cnt[(size_t)p * P.nchunk_cmp + chunk] = total;

  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t prev = atomic_inc_acq_rel(&P.meta[p].cmp_done);
    s_tmp[12] = (prev == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_tmp[12]) return;
  __threadfence();

  // ---- last work-group: gather the band in position order
  const int nch = gridDim.x;
  uint32_t* cnt = P.chunk_cnt + (size_t)p * P.nchunk_cmp;
  uint32_t carry = 0;
  for (int t0 = 0; t0 < nch; t0 += kThreads) {
    const int c = t0 + tid;
    uint32_t cv = c < nch ? cnt[c] : 0u;
    uint32_t tt;
    uint32_t ex = wg_exclusive_scan(cv, s_tmp, &tt);
    if (c < nch) cnt[c] = carry + ex;   // now the exclusive offset
    carry += tt;
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();
  const uint32_t nband = carry;
  Entry* ba = P.band_a + (size_t)p * P.stride;
  Entry* bb = P.band_b + (size_t)p * P.stride;
  for (int c = tid; c < nch; c += kThreads) {
    const uint32_t o = cnt[c];
    const uint32_t e = (c + 1 < nch) ? cnt[c + 1] : nband;
    const Entry* src = ba + (size_t)c * kCmpChunk;
    for (uint32_t i = 0; i < e - o; ++i) bb[o + i] = src[i];
  }
  __threadfence_block();
  __syncthreads();

  const int kind = p / P.n_q;
  const int K = (kind == 1) ? P.keep_blocks : P.k;
  uint32_t n2 = 0;
  if (nband > (uint32_t)K) {
    uint32_t ties;
    uint32_t kth = wg_kth_largest((int)nband, K, [&](int i) { return sortable(bb[i].s); }, s_hist,
                                  s_tmp, &ties);
    const float thr2 = band_below(unsortable(kth), P.meta[p].delta);
    // order-preserving compaction bb -> ba of entries >= thr2
    for (uint32_t t0 = 0; t0 < nband; t0 += kThreads) {
      const uint32_t i = t0 + tid;
      Entry e = i < nband ? bb[i] : Entry{0, 0.0f};
      const uint32_t keep = (i < nband && e.s >= thr2) ? 1u : 0u;
      uint32_t tt;
      uint32_t ex = wg_exclusive_scan(keep, s_tmp, &tt);
      if (keep) ba[n2 + ex] = e;
      n2 += tt;
    }
  } else {
    for (uint32_t i = tid; i < nband; i += kThreads) ba[i] = bb[i];
    n2 = nband;
  }
  if (tid == 0) {
    P.meta[p].nband = (int)nband;
    P.meta[p].nband2 = (int)n2;
  }
}

// ---------------------------------------------------------------- 4. rescoring
template <int D>
__global__ __launch_bounds__(kThreads) void k_rescore(Params P) {
  constexpr int DW = D / 2;  // packed bf16 pairs per head row
  __shared__ float s_key[kWaves][D];
  __shared__ float s_r[kWaves][64];
  __shared__ float s_w[64];
  __shared__ uint32_t s_tmp[16];
  __shared__ uint32_t s_hist[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = blockIdx.y, q = p % P.n_q, kind = p / P.n_q;
  const int nvis = P.q_nvis[q];
  const int64_t base = P.seq_base[P.q_seq[q]];
  const int n2 = P.meta[p].nband2;
  Entry* ba = P.band_a + (size_t)p * P.stride;

  if (tid < 64) s_w[tid] = tid < P.h_i ? P.w[(size_t)q * P.h_i + tid] : 0.0f;
  uint32_t qrow[DW];
  {
    const int hh = lane < P.h_i ? lane : 0;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(P.iq + ((size_t)q * P.h_i + hh) * D);
#pragma unroll
    for (int i = 0; i < DW; ++i) qrow[i] = src[i];
  }
  __syncthreads();

  const int stride_w = gridDim.x * kWaves;
  for (int j = blockIdx.x * kWaves + wave; j < n2; j += stride_w) {
    const int cand = ba[j].cand;
    if (kind == 1) {
      // block key: sequential fp32 sum of the visible keys, / count, bf16 nearest-even
      const int first = cand * 8;
      const int nb = min(nvis - first, 8);
      for (int d = lane; d < D; d += 64) {
        float s = 0.0f;
        for (int t = 0; t < nb; ++t) s = s + bf16_to_f32(P.ik[(size_t)(base + first + t) * D + d]);
        s_key[wave][d] = bf16_to_f32(f32_to_bf16_rne(__fdiv_rn(s, (float)nb)));
      }
    } else {
      const int pos = cand_pos(P, q, kind, cand);
      for (int d = lane; d < D; d += 64) s_key[wave][d] = bf16_to_f32(P.ik[(size_t)(base + pos) * D + d]);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < DW; ++i) {
      acc = fmaf(__uint_as_float(qrow[i] << 16), s_key[wave][2 * i], acc);
      acc = fmaf(__uint_as_float(qrow[i] & 0xFFFF0000u), s_key[wave][2 * i + 1], acc);
    }
    s_r[wave][lane] = acc > 0.0f ? acc : 0.0f;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) {
      float s = 0.0f;
      for (int h = 0; h < P.h_i; ++h) s = fmaf(s_w[h], s_r[wave][h], s);
      ba[j].s = s;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }

  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t prev = atomic_inc_acq_rel(&P.meta[p].rs_done);
    s_tmp[12] = (prev == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_tmp[12]) return;
  __threadfence();

  // ---- last work-group: exact Top-K of the band, ascending positions
  const int K = (kind == 1) ? P.keep_blocks : P.k;
  int32_t* out = (kind == 1) ? P.pool_out + (size_t)q * P.keep_blocks : P.idx_out + (size_t)q * P.k;
  uint32_t kth = 0, ties = 0;
  const bool all = n2 <= K;
  if (!all) kth = wg_kth_largest(n2, K, [&](int i) { return sortable(ba[i].s); }, s_hist, s_tmp, &ties);
  uint32_t nsel = 0, nties = 0;
  for (int t0 = 0; t0 < n2; t0 += kThreads) {
    const int i = t0 + tid;
    uint32_t key = 0;
    int cand = 0;
    if (i < n2) {
      key = sortable(ba[i].s);
      cand = ba[i].cand;
    }
    const uint32_t is_tie = (!all && i < n2 && key == kth) ? 1u : 0u;
    uint32_t tt;
    const uint32_t tie_rank = nties + wg_exclusive_scan(is_tie, s_tmp, &tt);
    nties += tt;
    const uint32_t keep = (i < n2 && (all || key > kth || (is_tie && tie_rank < ties))) ? 1u : 0u;
    uint32_t kt;
    const uint32_t ex = wg_exclusive_scan(keep, s_tmp, &kt);
    if (keep) out[nsel + ex] = (kind == 1) ? cand : cand_pos(P, q, kind, cand);
    nsel += kt;
  }
  for (int i = (int)nsel + tid; i < K; i += kThreads) out[i] = -1;
}

}  // namespace idx
}  // namespace csa2

// ======================================================================
// Host side
// ======================================================================
using namespace csa2;
using namespace csa2::idx;

namespace {

thread_local int g_last_hip_error = 0;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t scores, hist, meta, chunk_cnt, band_a, band_b, total;
};

Layout make_layout(int nprob, int64_t stride, int nchunk_cmp) {
  Layout L;
  size_t o = 0;
  L.scores = o;
  o = align256(o + (size_t)nprob * stride * sizeof(float));
  L.hist = o;
  o = align256(o + (size_t)nprob * kNBins * sizeof(uint32_t));
  L.meta = o;
  o = align256(o + (size_t)nprob * sizeof(Meta));
  L.chunk_cnt = o;
  o = align256(o + (size_t)nprob * nchunk_cmp * sizeof(uint32_t));
  L.band_a = o;
  o = align256(o + (size_t)nprob * stride * sizeof(Entry));
  L.band_b = o;
  o = align256(o + (size_t)nprob * stride * sizeof(Entry));
  L.total = o;
  return L;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

double gamma_n(double n, double u) { return n * u / (1.0 - n * u); }

// Delta = C * QW * max||k||: C covers the fp32 fma chain of the exact score
// (unit roundoff 2^-24) and any MFMA accumulation order or truncation (2^-23),
// for the d_i-term dot products and the head sum, doubled for safety.
float bound_constant(int h_i, int d_i) {
  const double u = std::ldexp(1.0, -24), u2 = std::ldexp(1.0, -23);
  const double gd = gamma_n(d_i, u), gm = gamma_n(d_i + 2, u2);
  const double gh = gamma_n(std::max(h_i, 66), u);
  return (float)(2.0 * (gd + gm + gh * (2.0 + gd + gm)));
}

bool launch_ok() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return false;
  }
  return true;
}

template <int D>
void launch_scan(const Params& P, int mt, bool pool, bool indirect, dim3 grid, hipStream_t s) {
#define CSA2_SCAN(MTV)                                                                   \
  if (mt == MTV) {                                                                       \
    if (indirect) hipLaunchKernelGGL((k_scan<D, MTV, false, true>), grid, dim3(kThreads), 0, s, P);  \
    else if (pool) hipLaunchKernelGGL((k_scan<D, MTV, true, false>), grid, dim3(kThreads), 0, s, P); \
    else hipLaunchKernelGGL((k_scan<D, MTV, false, false>), grid, dim3(kThreads), 0, s, P);         \
    return;                                                                              \
  }
  CSA2_SCAN(1) CSA2_SCAN(2) CSA2_SCAN(3) CSA2_SCAN(4)
#undef CSA2_SCAN
}

csa2_status run_pipeline(Params P, int64_t max_slots, void* ws, size_t ws_bytes, hipStream_t s,
                         size_t need) {
  if (ws_bytes < need) return CSA2_E_WORKSPACE;
  const Layout L = make_layout(P.nprob, P.stride, P.nchunk_cmp);
  char* w = static_cast<char*>(ws);
  P.scores = reinterpret_cast<float*>(w + L.scores);
  P.hist = reinterpret_cast<uint32_t*>(w + L.hist);
  P.meta = reinterpret_cast<Meta*>(w + L.meta);
  P.chunk_cnt = reinterpret_cast<uint32_t*>(w + L.chunk_cnt);
  P.band_a = reinterpret_cast<Entry*>(w + L.band_a);
  P.band_b = reinterpret_cast<Entry*>(w + L.band_b);
  P.bound_c = bound_constant(P.h_i, P.d_i);

  const int mt = (P.h_i + 15) / 16;
  const bool pool = !P.reindex && P.keep_blocks > 0;
  hipLaunchKernelGGL(k_prologue, dim3(P.nprob), dim3(kThreads), 0, s, P);
  if (!launch_ok()) return CSA2_E_HIP;
  const int nx = (int)std::max<int64_t>(1, (max_slots + P.scan_chunk - 1) / P.scan_chunk);
  const dim3 gscan(nx, P.n_q);
  if (P.d_i == 128) launch_scan<128>(P, mt, pool, P.reindex, gscan, s);
  else launch_scan<64>(P, mt, pool, P.reindex, gscan, s);
  if (!launch_ok()) return CSA2_E_HIP;
  hipLaunchKernelGGL(k_compact, dim3(P.nchunk_cmp, P.nprob), dim3(kThreads), 0, s, P);
  if (!launch_ok()) return CSA2_E_HIP;
  if (P.d_i == 128) hipLaunchKernelGGL(k_rescore<128>, dim3(kRescoreWGs, P.nprob), dim3(kThreads), 0, s, P);
  else hipLaunchKernelGGL(k_rescore<64>, dim3(kRescoreWGs, P.nprob), dim3(kThreads), 0, s, P);
  if (!launch_ok()) return CSA2_E_HIP;
  return CSA2_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool shape_ok(int h_i, int d_i) { return h_i >= 1 && h_i <= 64 && (d_i == 64 || d_i == 128); }

}  // namespace

extern "C" int csa2_internal_last_hip_error_index(void) { return g_last_hip_error; }

extern "C" size_t csa2_index_topk_ws_bytes(int n_q, int32_t max_nvis, int h_i, int d_i, int k,
                                           int block, int keep_blocks) {
  (void)h_i; (void)d_i; (void)k; (void)block;
  if (n_q <= 0) return 0;
  const int nprob = n_q * (keep_blocks > 0 ? 2 : 1);
  const int64_t stride = round_up(std::max<int64_t>(max_nvis, 1), kCmpChunk);
  return make_layout(nprob, stride, (int)(stride / kCmpChunk)).total;
}

extern "C" size_t csa2_reindex_topk_ws_bytes(int n_q, int h_i, int d_i, int k, int block, int keep_blocks) {
  (void)h_i; (void)d_i; (void)k; (void)block;
  if (n_q <= 0) return 0;
  const int64_t stride = round_up(std::max<int64_t>(8LL * keep_blocks, 1), kCmpChunk);
  return make_layout(n_q, stride, (int)(stride / kCmpChunk)).total;
}

extern "C" csa2_status csa2_index_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                       const int32_t* q_seq, const int32_t* q_nvis, int32_t max_nvis,
                                       const uint16_t* ik, const int64_t* seq_base, int k,
                                       int32_t* idx_out, int block, int keep_blocks, int32_t* pool_out,
                                       void* ws, size_t ws_bytes, void* stream) {
  if (n_q < 0 || max_nvis < 0 || max_nvis > 0x7FFFFFF0 || k < 1 || k > 2048 || keep_blocks < 0 ||
      keep_blocks > 4096)
    return CSA2_E_INVAL;
  if (!shape_ok(h_i, d_i)) return CSA2_E_UNSUPPORTED;
  if (keep_blocks > 0 && block != 8) return CSA2_E_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!iq || !w || !q_seq || !q_nvis || !ik || !seq_base || !idx_out || !ws) return CSA2_E_INVAL;
  if (keep_blocks > 0 && !pool_out) return CSA2_E_INVAL;
  if (!aligned(iq, 16) || !aligned(ik, 16) || !aligned(w, 4) || !aligned(ws, 256)) return CSA2_E_INVAL;
  Params P{};
  P.iq = iq; P.w = w; P.n_q = n_q; P.h_i = h_i; P.d_i = d_i;
  P.q_seq = q_seq; P.q_nvis = q_nvis; P.ik = ik; P.seq_base = seq_base;
  P.pool_in = nullptr; P.keep_in = 0; P.k = k; P.keep_blocks = keep_blocks;
  P.idx_out = idx_out; P.pool_out = pool_out;
  P.nprob = n_q * (keep_blocks > 0 ? 2 : 1);
  P.reindex = 0;
  P.scan_chunk = 4096;
  P.stride = round_up(std::max<int64_t>(max_nvis, 1), kCmpChunk);
  P.nchunk_cmp = (int)(P.stride / kCmpChunk);
  const size_t need = csa2_index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, block, keep_blocks);
  return run_pipeline(P, max_nvis, ws, ws_bytes, static_cast<hipStream_t>(stream), need);
}

extern "C" csa2_status csa2_reindex_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                         const int32_t* q_seq, const int32_t* q_nvis, const uint16_t* ik,
                                         const int64_t* seq_base, const int32_t* pool_blocks, int block,
                                         int keep_blocks, int k, int32_t* idx_out, void* ws,
                                         size_t ws_bytes, void* stream) {
  if (n_q < 0 || k < 1 || k > 2048 || keep_blocks < 1 || keep_blocks > 4096) return CSA2_E_INVAL;
  if (!shape_ok(h_i, d_i)) return CSA2_E_UNSUPPORTED;
  if (block != 8) return CSA2_E_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!iq || !w || !q_seq || !q_nvis || !ik || !seq_base || !pool_blocks || !idx_out || !ws)
    return CSA2_E_INVAL;
  if (!aligned(iq, 16) || !aligned(ik, 16) || !aligned(w, 4) || !aligned(ws, 256)) return CSA2_E_INVAL;
  Params P{};
  P.iq = iq; P.w = w; P.n_q = n_q; P.h_i = h_i; P.d_i = d_i;
  P.q_seq = q_seq; P.q_nvis = q_nvis; P.ik = ik; P.seq_base = seq_base;
  P.pool_in = pool_blocks; P.keep_in = keep_blocks; P.k = k; P.keep_blocks = 0;
  P.idx_out = idx_out; P.pool_out = nullptr;
  P.nprob = n_q;
  P.reindex = 1;
  P.scan_chunk = 512;
  const int64_t slots = 8LL * keep_blocks;
  P.stride = round_up(slots, kCmpChunk);
  P.nchunk_cmp = (int)(P.stride / kCmpChunk);
  const size_t need = csa2_reindex_topk_ws_bytes(n_q, h_i, d_i, k, block, keep_blocks);
  return run_pipeline(P, slots, ws, ws_bytes, static_cast<hipStream_t>(stream), need);
}
