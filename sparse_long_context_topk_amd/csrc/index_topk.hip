// index_topk.hip -- CSA2 lightning-indexer scan and exact Top-K for gfx950.
//
// What is computed (csa2.h states the full contract): for each query, the
// indexer score of every candidate position, score = sum_h w_h ReLU(q_h . k),
// defined to the bit as an fp32 fma chain over d and then over h; the Top-K
// positions by (score desc, position asc).  Full layers score every visible
// position and may also build the hierarchical pool (blocks of 8 scored by
// their mean key, Top-keep_blocks blocks); Reindex layers score the positions
// of a pool.  Source: "DeepSeek AI выпустила DeepSeek-V4.1-Flash с контекстом
// в 1 млн токенов, KV-кэшем FP4 ..." (wire.sakhanda.co), section "Сжатое
// разреженное внимание 2 (CSA2)": the Full / Reindex / Reuse modes, Top-512,
// and the pool of up to 2048 blocks of 8 positions.
//
// How (one pass over the keys at HBM speed, exact result):
//  1. k_prologue   zeroes the problem's histograms and Meta.
//  2. k_scan       streams the indexer keys once (up to 8192 keys per
//                  work-group, fewer when that keeps 512 work-groups busy;
//                  NBUF - 1 groups of 16 keys per wave in flight ahead of the
//                  math, scores staged in LDS and written once at the end).
//                  Scores come from bf16 MFMA
//                  (v_mfma_f32_16x16x32_bf16, S^T = K Q^T: 16 positions x 16
//                  heads x 32 dims, the query held in registers).  A block's
//                  per-head dot product is the mean of its members'
//                  (linearity), so block scores come from the same accumulators
//                  with a DPP butterfly: the pool costs no extra HBM traffic and
//                  no extra MFMA.  Work-groups add into a 4096-bin histogram of
//                  the top 12 bits of the scores' sortable keys and track the
//                  largest key magnitude t_k = sum_d u_d |k_d| (u_frag).
//  3. k_finehist   every work-group finds the coarse bin holding the K-th
//                  score, then histograms bits 19..8 of the keys in that bin:
//                  the K-th approximate score a_K is located in a fine bin
//                  [L, U].
//  4. k_compact    every work-group derives the band from the fine histogram
//                  and the rounding bound Delta = C * max t_k (each per-head
//                  dot's rounding is at most a constant times
//                  sum_d |q_hd k_d|, ReLU is 1-Lipschitz, plus the head-sum
//                  and block-mean roundings; C from the fp32 error constants
//                  with a 2x margin):
//                  every exact Top-K member has approximate score >= L - 2 Delta
//                  (it is >= the K-th exact score >= a_K - Delta); a member with
//                  approximate score > U + 2 Delta is certainly in (only members
//                  above a_K1 <= U can reach its exact score).  The band is
//                  written per chunk in position order, certain members flagged,
//                  the uncertain ones listed.
//  5. k_rescore    recomputes the uncertain members' scores with the exact fp32
//                  chains (one lane per head; a block runs its eight member
//                  chains and divides their sum by the member count).
//  6. k_final      one work-group per problem: the certain members plus the
//                  best uncertain ones by (exact score desc, position asc) --
//                  pairwise ranks of (score, index) composites, or a radix
//                  select when the uncertain set is large -- written as
//                  ascending positions, -1 padded.
// Degenerate inputs (ties everywhere) only make the band large; the result
// stays exact.
// A Reindex pool of at most 16,384 slots skips steps 1 and 3-6: its scan keeps
// each work-group's largest key magnitude t_k instead of histograms, and one
// work-group per query (section 7) selects from the scores it holds in
// registers.  A Full call without a pool whose contexts are all that short
// takes the same path over every block of the context (a null pool).
#include "csa2_device.h"

#include <algorithm>
#include <type_traits>
#include <cmath>
#include <mutex>

namespace csa2 {
namespace idx {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kNBins = 4096;
constexpr int kBinShift = 20;
constexpr int kCmpChunk = 4096;
constexpr double kLargeSelBytes = 1024.0 * 1048576.0;
constexpr int kLargeChunks = 8;   // large mode without a block problem: chunks per fine-histogram work-group   // token score bytes from which the selection runs in its large mode
constexpr int kCmpPerThread = kCmpChunk / kThreads;
constexpr int kMaxChunksLds = 8192;   // compaction chunks per problem (max_nvis <= 2^25)
constexpr int kRescoreWGs = 768;   // rescoring work-groups per launch (all queries): three per CU
#ifndef CSA2_SCAN_NBUF_FP8
#define CSA2_SCAN_NBUF_FP8 5
#endif
#ifndef CSA2_SCAN_NBUF
#define CSA2_SCAN_NBUF 3
#endif
#ifndef CSA2_SCAN_CHUNK
#define CSA2_SCAN_CHUNK 8192
#endif
constexpr int kMaxScanChunk = CSA2_SCAN_CHUNK;   // keys per scan work-group (Full layers)
constexpr int kBandLds = 12288;      // band entries the final kernel keeps in LDS (96 KiB)
constexpr int kUncLds = 4096;        // uncertain members whose keys the final kernel keeps in LDS
constexpr int kRankMax = 1024;       // uncertain members the final kernel ranks pairwise
constexpr uint32_t kCertain = 0x80000000u;
constexpr uint32_t kAll = 0xFFFFFFFFu;

struct Meta {
  uint32_t maxt;    // scan (token problem): largest key magnitude t_k = sum_d u_d |k_d|, float bits
  uint32_t bin;     // coarse bin holding the K-th score; kAll: every candidate is kept
  uint32_t above;   // valid candidates in coarse bins above `bin`
  uint32_t total;   // valid candidates
  float wabs;       // sum_h |w_h| (the bound's underflow term)
  float delta;      // rounding bound of the scores
  float keep_thr;   // band: approximate score >= keep_thr
  float in_thr;     // certainly selected: approximate score > in_thr
  int32_t nc;       // candidate slots
  uint32_t pad[7];
};
static_assert(sizeof(Meta) == 64, "Meta is one 64-byte line");

struct Entry {
  uint32_t cand;  // candidate index; top bit set = certainly selected
  float s;        // approximate score, replaced by the exact one when rescored
};

struct Params {
  const uint16_t* iq;
  const float* w;
  int n_q, h_i, d_i;
  const int32_t* q_seq;
  const int32_t* q_nvis;
  const uint16_t* ik;
  // FP8 keys (the low-precision indexer-key variant), used instead of ik when
  // set: E4M3 codes [rows][d_i] and one exponent byte per row (scale 2^(e - 127))
  const uint8_t* ik8;
  const uint8_t* ik8e;
  const int64_t* seq_base;
  const int32_t* pool_in;  // Reindex: [n_q][keep_in]; null: every block 0 .. keep_in-1 in order
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
  int rs_tok;              // rescoring work-groups per query given to the token problem (the rest: blocks)
  int rs_pool;             // the block work-groups of all queries share one member list
  int64_t base0;           // chunk calls (q_seq == nullptr): every query's sequence starts at key row base0
  float bound_tok, bound_blk;
  float* scores;
  uint32_t* hist;       // [nprob][kNBins] coarse histogram (top 12 bits of the key)
  uint32_t* hist2;      // [nprob][kNBins] fine histogram inside the coarse bin `bin`
  Meta* meta;
  uint32_t* chunk_cnt;  // [nprob][nchunk_cmp] band members per chunk
  uint32_t* chunk_unc;  // [nprob][nchunk_cmp] uncertain members per chunk
  Entry* band;          // [nprob][stride] band members, chunk c at c*kCmpChunk, in position order
  uint2* unc;           // [nprob][stride] uncertain members: {chunk-local index, candidate}
  uint16_t* gkey;       // [n_q][stride / 16] top 16 bits of the sortable key of the largest score of each
                        // 16-score group of a token (or Reindex) row (large mode)
  int large_sel;        // large problems: the coarse bin and the band are computed once per problem (k_coarse,
                        // k_band) and the selection kernels skip groups whose largest score is below them
  float* kpart;         // Reindex scan: [n_q][scan work-groups] largest key magnitude t_k of each
};

// ---------------------------------------------------------------- helpers
// v - 2*Delta and v + 2*Delta with room for the rounding of these operations.
__device__ __forceinline__ float band_below(float v, float delta) {
  return v - 2.0f * delta * (1.0f + 0.00390625f) - fabsf(v) * 9.5367431640625e-07f;
}
__device__ __forceinline__ float band_above(float v, float delta) {
  return v + 2.0f * delta * (1.0f + 0.00390625f) + fabsf(v) * 9.5367431640625e-07f;
}

__device__ __forceinline__ float dpp_f(float v, int ctrl) {
  // the DPP control must be a constant: dispatch on the three patterns used
  int x = __float_as_int(v);
  int r;
  if (ctrl == 0xB1) r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);        // quad xor 1
  else if (ctrl == 0x4E) r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad xor 2
  else r = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);                    // half-row mirror
  return __int_as_float(r);
}

// Sum over the 8 lanes of each half row (lanes 8j..8j+7 of every 16).
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f(v, 0xB1);
  v += dpp_f(v, 0x4E);
  v += dpp_f(v, 0x141);
  return v;
}

// Sum over the 16 lanes of each row.
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// max(x, 0) of an approximate (MFMA) dot as one integer max of its bits: a
// float with the sign bit set is a negative integer, any other orders as its
// bits.  Equals fmaxf(x, 0) for every non-NaN x (and -0 gives +0), without
// the NaN-quieting max the compiler puts in front of a float max.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// An all-zero key row (the largest row of any supported key layout, 256
// bytes) and exponent byte: a scan slot without a key loads it, so that its
// products, block sums and t_k come out zero without masking the loaded
// words.  Never written.
static __device__ __align__(256) uint8_t g_zero_key[256];
typedef __attribute__((address_space(1))) const uint8_t gbyte;   // global memory
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes from global memory (p 16-byte aligned)
__device__ __forceinline__ uint4 gload16(const gbyte* p) {
  const u32x4_t t = *(__attribute__((address_space(1))) const u32x4_t*)p;
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// The rounding bound's key magnitude.  For a query with heads q_h and weights
// w_h, every per-head dot product's rounding error (exact chain or MFMA) is at
// most a constant times sum_d |q_hd k_d|, so the score's error is at most a
// constant times t_k = sum_h |w_h| sum_d |q_hd| |k_d| = sum_d u_d |k_d| with
// u_d = sum_h |w_h| |q_hd|.  (t_k <= QW ||k|| by Cauchy-Schwarz, QW =
// sum_h |w_h| ||q_h||; on Gaussian data it is about two thirds of it.)
//
// u_frag: this lane's 32 dims of u (lane (n, g) of an MFMA key fragment
// holds dims 32 ks + 8 g .. +7), from the query fragments qb (lane (n, g):
// head 16 mt + n, the same dims) -- a sum over the 16 lanes of the row and
// over mt -- rounded up to bf16 and packed in pairs, so that an upper bound
// stays an upper bound.
template <int MT, int KS>
__device__ __forceinline__ void u_frag(const bf16x8 (&qb)[MT][KS], const float (&wr)[MT], uint32_t (&up)[KS][4]) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t pk = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float a = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint4 u4 = __builtin_bit_cast(uint4, qb[mt][ks]);
          const uint32_t wd = jj == 0 ? u4.x : jj == 1 ? u4.y : jj == 2 ? u4.z : u4.w;
          const float qv = e == 0 ? __uint_as_float(wd << 16) : __uint_as_float(wd & 0xFFFF0000u);
          a = fmaf(fabsf(wr[mt]), fabsf(qv), a);
        }
        a = sum16(a);
        const uint32_t bits = (__float_as_uint(a) + 0xFFFFu) & 0xFFFF0000u;   // bf16, rounded up (a >= 0)
        pk |= e == 0 ? (bits >> 16) : bits;
      }
      up[ks][jj] = pk;
    }
  }
}

// Sum over the four rows of the wave (lanes l, l^16, l^32, l^48 -- the four
// lane groups holding parts of one MFMA column), in every lane: two VALU lane
// permutes (rows 0<->1, 2<->3, then the halves).
__device__ __forceinline__ float sum_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// v + the value of lane l ^ 16 (rows 0 <-> 1 and 2 <-> 3 of the wave), with
// one VALU lane permute instead of an LDS permute.
__device__ __forceinline__ float add_xor16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// Exclusive prefix sum over the NT-thread work-group (s_tmp: >= NT / 64
// entries); returns this thread's offset and writes the total.
template <int NT = kThreads>
__device__ __forceinline__ uint32_t wg_exclusive_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t x = wave_incl_scan_u32(v);   // DPP row shifts and broadcasts
  if (lane == 63) s_tmp[wave] = x;
  lds_barrier();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    uint32_t t = s_tmp[i];
    if (i < wave) before += t;
    all += t;
  }
  lds_barrier();
  *total = all;
  return before + x - v;
}

// K-th largest of the sortable keys key_of(i), i < n (1 <= K <= n): a
// most-significant-digit radix select with 8-bit digits.  Band keys share
// their leading bits, so the digits start at the highest bit where the
// smallest and largest key differ: the first histogram then spreads over many
// bins instead of piling every LDS atomic onto one.  Returns the key; in
// *ties the number of entries equal to it that belong to the Top-K.  NT >= 256
// threads; s_tmp holds >= 2 NT / 64 + 2 entries.
template <int NT = kThreads, typename KeyOf>
__device__ uint32_t wg_kth_largest(int n, int K, KeyOf key_of, uint32_t* s_hist /*256*/,
                                   uint32_t* s_tmp, uint32_t* ties) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = tid; i < n; i += NT) {
    const uint32_t key = key_of(i);
    lo = min(lo, key);
    hi = max(hi, key);
  }
  lo = wave_min_u32(lo);
  hi = wave_max(hi);
  if ((tid & 63) == 0) {
    s_tmp[tid >> 6] = lo;
    s_tmp[NW + (tid >> 6)] = hi;
  }
  lds_barrier();
  lo = s_tmp[0];
  hi = s_tmp[NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    lo = min(lo, s_tmp[i]);
    hi = max(hi, s_tmp[NW + i]);
  }
  lds_barrier();
  if (lo == hi) {
    *ties = (uint32_t)K;
    return lo;
  }
  const int top = 31 - __clz(lo ^ hi);          // highest differing bit
  uint32_t mask = top == 31 ? 0u : (0xFFFFFFFFu << (top + 1));
  uint32_t prefix = lo & mask;
  uint32_t remaining = (uint32_t)K;
  for (int shift = top - 7;; shift -= 8) {
    const int sh = shift < 0 ? 0 : shift;
    const int width = shift < 0 ? 8 + shift : 8;   // last digit may be narrower
    const uint32_t dmask = (1u << width) - 1u;
    if (tid < 256) s_hist[tid] = 0;
    lds_barrier();
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = key_of(i);
      if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
    }
    lds_barrier();
    // thread tid < 256 owns digit 255 - tid; the exclusive scan counts larger digits
    const uint32_t v = tid < 256 ? s_hist[255 - tid] : 0u;
    uint32_t tot;
    const uint32_t excl = wg_exclusive_scan<NT>(v, s_tmp, &tot);
    if (excl < remaining && excl + v >= remaining) {
      s_tmp[2 * NW] = 255u - tid;
      s_tmp[2 * NW + 1] = excl;
    }
    lds_barrier();
    const uint32_t d = s_tmp[2 * NW];
    remaining -= s_tmp[2 * NW + 1];
    prefix |= d << sh;
    mask |= dmask << sh;
    lds_barrier();
    if (sh == 0) break;
  }
  *ties = remaining;
  return prefix;
}

// First key row of query q's sequence.
__device__ __forceinline__ int64_t seq_base_of(const Params& P, int q) {
  return P.q_seq ? P.seq_base[P.q_seq[q]] : P.base0;
}

// Compaction chunks of a problem: the block problem's rows hold 1/8 of the
// candidates.  (Its chunk counters keep the token problem's row pitch.)
__device__ __forceinline__ int nchunks_of(const Params& P, int kind) {
  return kind == 1 ? (P.nchunk_cmp + 7) >> 3 : P.nchunk_cmp;
}

// Grid of the per-chunk kernels: x covers the token (or Reindex) problem's
// chunks, then the block problem's; y is the query.
__device__ __forceinline__ void grid_chunk(const Params& P, int* p, int* chunk) {
  const bool blk = (int)blockIdx.x >= P.nchunk_cmp;
  *p = (blk ? P.n_q : 0) + (int)blockIdx.y;
  *chunk = blk ? (int)blockIdx.x - P.nchunk_cmp : (int)blockIdx.x;
}

// Large mode without a block problem: fine-histogram work-group (x, q) takes
// the kLargeChunks chunks from x kLargeChunks of query q's row.
__device__ __forceinline__ bool large_multi(const Params& P) {
  return P.large_sel && (P.reindex || P.keep_blocks == 0);
}

// Candidates of problem p (what the prologue records in Meta.nc), from the
// query's visible length.
__device__ __forceinline__ int cands_of(const Params& P, int kind, int nvis) {
  return P.reindex ? 8 * P.keep_in : (kind == 0 ? nvis : (nvis + 7) >> 3);
}

__device__ __forceinline__ int cand_pos(const Params& P, int q, int kind, uint32_t cand) {
  cand &= ~kCertain;
  if (P.reindex) {
    const int b = P.pool_in ? P.pool_in[(size_t)q * P.keep_in + (cand >> 3)] : (int)(cand >> 3);
    return b * 8 + (int)(cand & 7);
  }
  (void)kind;
  return (int)cand;
}

// Dims 2 p and 2 p + 1 of key row `row` as a bf16 pair (low half: dim 2 p).
// FP8 keys decode exactly: v_cvt_scalef32_pk_bf16_fp8 multiplies by the power
// of two of its scale argument, and an E4M3 value times the row's scale
// 2^E (E >= -124) is a bf16 value.
template <int D>
__device__ __forceinline__ uint32_t key_pair(const Params& P, int64_t row, int p) {
  if (P.ik8) {
    const uint32_t c = reinterpret_cast<const uint16_t*>(P.ik8 + (size_t)row * D)[p];
    const float sc = __uint_as_float((uint32_t)P.ik8e[row] << 23);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, sc, false));
  }
  return reinterpret_cast<const uint32_t*>(P.ik + (size_t)row * D)[p];
}

// Scores of one scan chunk (n of them from LDS `src`, positions c0 .. c0 + n
// - 1 of row `row`, c0 a multiple of 256) to global memory as whole 256-score
// groups, one per wave at a time (each lane four consecutive scores), with the
// top 16 bits of the sortable key of the largest score of every 16 scores in
// `gk` (scores c0 + 16 g .. c0 + 16 g + 15 at gk[(c0 >> 4) + g]; a DPP maximum
// over a lane quad's sortable keys, which order as the scores do): a group
// whose value there is below a threshold key's top 16 bits holds no score at or
// above the threshold.  Without `with_max`, one score per thread and step.
template <int NWAVES>
__device__ __forceinline__ void store_scores(float* row, uint16_t* gk, const float* src, int c0, int n, int wave,
                                             int lane, bool with_max) {
  if (!with_max) {   // the plain write-out
    for (int i = 64 * wave + lane; i < n; i += 64 * NWAVES) row[c0 + i] = src[i];
    return;
  }
  const int ng = (n + 255) >> 8;
  for (int gi = wave; gi < ng; gi += NWAVES) {
    const int i0 = (gi << 8) + 4 * lane;
    float m = -INFINITY;
    if (i0 + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(&src[i0]);
      *reinterpret_cast<float4*>(&row[c0 + i0]) = v;
      m = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i0 + e < n) {
          const float v = src[i0 + e];
          row[c0 + i0 + e] = v;
          m = fmaxf(m, v);
        }
    }
    if (with_max) {   // lane quad r covers the group's scores 16 r .. 16 r + 15
      uint32_t mk = sortable(m);
      mk = max(mk, dpp0<0xB1>(mk));   // quad_perm [1,0,3,2]
      mk = max(mk, dpp0<0x4E>(mk));   // quad_perm [2,3,0,1]
      if ((lane & 3) == 0) gk[(c0 >> 4) + 16 * gi + (lane >> 2)] = (uint16_t)(mk >> 16);
    }
  }
}

// ---------------------------------------------------------------- 1. prologue
template <int D>
__global__ __launch_bounds__(kThreads) void k_prologue(Params P) {
  const int p = blockIdx.x, q = p % P.n_q, kind = p / P.n_q;
  uint4* h = reinterpret_cast<uint4*>(P.hist + (size_t)p * kNBins);
  uint4* h2 = reinterpret_cast<uint4*>(P.hist2 + (size_t)p * kNBins);
  for (int i = threadIdx.x; i < kNBins / 4; i += kThreads) {
    h[i] = make_uint4(0, 0, 0, 0);
    h2[i] = make_uint4(0, 0, 0, 0);
  }
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    float wa = lane < P.h_i ? fabsf(P.w[(size_t)q * P.h_i + lane]) : 0.0f;
    wa = wave_sum(wa);
    if (lane == 0) {
      Meta m;
      m.maxt = 0;
      m.bin = kAll;
      m.above = m.total = 0;
      m.wabs = wa;
      m.delta = 0.0f;
      m.keep_thr = m.in_thr = -INFINITY;
      const int nvis = P.q_nvis[q];
      m.nc = P.reindex ? 8 * P.keep_in : (kind == 0 ? nvis : (nvis + 7) / 8);
      for (int i = 0; i < 7; ++i) m.pad[i] = 0;
      P.meta[p] = m;
    }
  }
}

// Coarse step of the threshold: the bin of the coarse histogram that holds
// the K-th score (kAll when at most K candidates exist), computed by every
// work-group that needs it; the publishing one also records it, with the
// rounding bound Delta and the count above the bin, in the problem's Meta.
// hv: this thread's 16 bins of the coarse histogram, highest first (bins
// 4095 - 16 tid down to 4080 - 16 tid), loaded by the caller; maxt (the
// largest key magnitude t_k, see u_frag) and wabs feed the published bound.
constexpr int kHPer = kNBins / kThreads;   // histogram bins per thread

__device__ __forceinline__ void load_hist16(const uint32_t* h, uint32_t hv[kHPer]) {
  const int b_hi = kNBins - kHPer * (int)threadIdx.x - 1;
#pragma unroll
  for (int j = 0; j < kHPer; ++j) hv[j] = h[b_hi - j];
}

__device__ uint32_t wg_coarse_bin(const Params& P, int p, const uint32_t hv[kHPer], bool publish, float maxt,
                                  float wabs, uint32_t* s_tmp /*>= 12*/) {
  const int tid = threadIdx.x;
  const int kind = p / P.n_q;
  const int K = kind == 1 ? P.keep_blocks : P.k;
  constexpr int kPer = kHPer;
  const int b_hi = kNBins - kPer * tid - 1;
  if (tid == 0) s_tmp[10] = kAll;          // ordered before its readers by the scan's barriers
  uint32_t loc = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) loc += hv[j];
  uint32_t tot;
  const uint32_t above = wg_exclusive_scan(loc, s_tmp, &tot);
  if (publish && tid == 0) {
    // the token problem's scan holds the largest t_k; blocks use it too
    const float bound = kind == 1 ? P.bound_blk : P.bound_tok;
    P.meta[p].delta = bound * maxt * (1.0f + 0.0009765625f) + wabs * (float)P.d_i * 7.8886e-31f;
    P.meta[p].total = tot;
  }
  if (tot > (uint32_t)K && above < (uint32_t)K && above + loc >= (uint32_t)K) {
    uint32_t run = above;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (run + hv[j] >= (uint32_t)K) {
        s_tmp[10] = (uint32_t)(b_hi - j);
        if (publish) {
          P.meta[p].bin = (uint32_t)(b_hi - j);
          P.meta[p].above = run;
        }
        break;
      }
      run += hv[j];
    }
  }
  lds_barrier();
  const uint32_t bin = s_tmp[10];
  lds_barrier();
  return bin;
}

// ---------------------------------------------------------------- 2. scan
// POOL: also score the 8-position blocks (Full layers building a pool).
// INDIRECT: candidates are the slots of a pool (Reindex layers).
// HIST: build the coarse score histograms (and the largest t_k) that the
// multi-kernel selection uses; without it the scan records each work-group's
// largest t_k for the single-work-group selection.
template <int D, int MT, bool POOL, bool INDIRECT, bool HIST, bool FP8>
__global__ __launch_bounds__(kThreads) void k_scan(Params P) {
  constexpr int KS = D / 32;   // MFMA k-steps; also 16-byte loads per lane per key
  // key groups in registers: one being multiplied, NBUF - 2 loaded or in
  // flight behind it, one being loaded (FP8 keys hold half the bytes per
  // group, so more groups fly)
  constexpr int NBUF = FP8 ? CSA2_SCAN_NBUF_FP8 : CSA2_SCAN_NBUF;
  __shared__ uint32_t s_hist[HIST ? kNBins : 1];
  __shared__ uint32_t s_hist_b[POOL ? kNBins : 1];
  __shared__ int32_t s_pool[INDIRECT ? 512 : 1];
  // the chunk's scores stay in LDS until the end: the hot loop then issues
  // only loads, and the results leave as one coalesced write
  __shared__ __attribute__((aligned(16))) float s_sc[kMaxScanChunk];
  __shared__ float s_scb[POOL ? kMaxScanChunk / 8 : 1];
  __shared__ uint32_t s_tmp[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int q = blockIdx.y;
  const int p = q;             // token problem
  const int pb = P.n_q + q;    // block problem (POOL)
  const int nvis = P.q_nvis[q];
  const int64_t base = seq_base_of(P, q);
  const int nc = INDIRECT ? 8 * P.keep_in : nvis;
  const int nblk = (nvis + 7) >> 3;
  const int c0 = blockIdx.x * P.scan_chunk;
  // a chunk past the query's visible keys (the grid spans the longest
  // context) has no score, block or histogram count to publish
  if constexpr (HIST) {
    if (c0 >= nc) return;
  }

  if constexpr (HIST) {
    for (int i = tid; i < kNBins; i += kThreads) {
      s_hist[i] = 0;
      if (POOL) s_hist_b[i] = 0;
    }
  }
  if constexpr (INDIRECT) {
    // block ids of this chunk's pool slots (scan_chunk / 8 <= 512 of them)
    for (int i = tid; i < P.scan_chunk / 8; i += kThreads) {
      const int slot = c0 / 8 + i;
      s_pool[i] = slot < P.keep_in ? (P.pool_in ? P.pool_in[(size_t)q * P.keep_in + slot] : slot) : -1;
    }
  }

  // Q^T as the MFMA B operand: lane (n, g) holds head 16*mt + n, dims dim0(ks) .. +7
  // (bf16 keys: the natural k-layout 32 ks + 8 g, for each k-step the four
  // lane groups cover 64 contiguous bytes of a row, so every key load
  // instruction reads whole lines; FP8 keys: 16 g + 8 ks for ks < 2 and
  // 64 + 16 g + 8 (ks - 2) after, so that a lane's 32 code bytes are two
  // 16-byte loads, each instruction covering 64 contiguous bytes of a row --
  // any k-order gives the same products, and the bound holds for any order)
  auto dim0 = [&](int ks) { return FP8 ? (ks < 2 ? 16 * g + 8 * ks : 64 + 16 * g + 8 * (ks - 2)) : 32 * ks + 8 * g; };
  bf16x8 qb[MT][KS];
  float wr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = 16 * mt + n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (head < P.h_i)
        v = *reinterpret_cast<const uint4*>(P.iq + ((size_t)q * P.h_i + head) * D + dim0(ks));
      qb[mt][ks] = __builtin_bit_cast(bf16x8, v);
    }
    wr[mt] = head < P.h_i ? P.w[(size_t)q * P.h_i + head] : 0.0f;
  }
  uint32_t up[KS][4];   // this lane's dims of u (the bound's key magnitude), set below

  float mk2 = 0.0f;   // largest key magnitude t_k of the chunk
  float* sc = P.scores + (size_t)p * P.stride;
  float* scb = P.scores + (size_t)pb * P.stride;
  const int nslots = min(P.scan_chunk, max(nc - c0, 0));
  const int ngroups = (nslots + 15) >> 4;
  const int my_groups = ngroups > wave ? (ngroups - wave + kWaves - 1) / kWaves : 0;

  // Row of the key that lane (n, g) loads for local group `it` (the wave's
  // it-th group); `valid` says whether the slot holds a key.  A slot without
  // one loads the zero row instead (a pool slot's loads run even for a
  // sequence with no visible position, whose base row may lie past the
  // array's end), so every load is in bounds and unconditional and the key
  // contributes nothing.
  auto key_row = [&](int it, bool& valid) -> int64_t {
    const int cand = c0 + 16 * (wave + kWaves * it) + n;
    int pos;
    if (INDIRECT) {
      const int b = cand < nc ? s_pool[(cand - c0) >> 3] : -1;
      pos = b * 8 + (cand & 7);
      valid = b >= 0 && pos < nvis;
    } else {
      pos = cand;
      valid = cand < nc;
    }
    return base + pos;
  };
  // bf16 keys: 16 bytes (dims 32 ks + 8 g .. + 7) per k-step; FP8 keys: the
  // code bytes of dims 16 g .. + 15 in kb[0] and 64 + 16 g .. + 15 in kb[1]
  // (k-steps 0, 1 and 2, 3: see dim0), the row's exponent byte in kb[2].x
  // the zero row's address, taken once and held in scalar registers (the
  // empty asm keeps the compiler from fetching it again in the loop); the
  // loads go through global-address-space pointers, so that a select between
  // a key row and the zero row still compiles to global loads
  const gbyte* zrow = (const gbyte*)(g_zero_key);
  asm volatile("" : "+s"(zrow));
  auto load = [&](int it, uint4* kb) {
    bool v;
    const int64_t row = key_row(min(it, my_groups - 1), v);
    if constexpr (FP8) {
      const gbyte* src = (v ? (const gbyte*)(P.ik8 + (size_t)row * D) : zrow) + 16 * g;
      kb[0] = gload16(src);
      kb[1] = gload16(src + 64);
      kb[2].x = *(v ? (const gbyte*)(P.ik8e + row) : zrow);
    } else {
      const gbyte* src = (v ? (const gbyte*)(P.ik + (size_t)row * D) : zrow) + 16 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[ks] = gload16(src + 64 * ks);
    }
  };

  // k-step ks of a loaded key group as a bf16 MFMA fragment (FP8 codes
  // decoded exactly; a slot without a key loaded the zero row, nothing to
  // mask)
  auto fragment = [&](const uint4* kin, int ks) -> uint4 {
    if constexpr (FP8) {
      const float sc = __uint_as_float(kin[2].x << 23);
      const uint4 r = kin[ks >> 1];
      const uint32_t lo = (ks & 1) ? r.z : r.x, hi = (ks & 1) ? r.w : r.y;
      const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false));
      const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true));
      const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false));
      const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true));
      return make_uint4(a, b, c, d);
    } else {
      return kin[ks];
    }
  };
  // k-step ks of a group's products S (16 keys x 16 heads per tile) = K . Q^T
  // -- lane (n, g) gets keys 4g+i, head 16*mt+n -- and of its keys'
  // magnitudes t_k = |K| . u, one more MFMA whose B operand is the lane's u
  // fragment in every column (lane (n, g) gets t of keys 4g+i; the products
  // are exact in fp32, the sums of non-negative terms round by far less than
  // the final factor 1 + 2^-10 covers)
  auto kstep = [&](const uint4& kb, int ks, f32x4 (&acc)[MT], f32x4& t) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, kb);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[mt][ks], ks == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : acc[mt],
                                                        0, 0, 0);
    const uint4 ab = make_uint4(kb.x & 0x7FFF7FFFu, kb.y & 0x7FFF7FFFu, kb.z & 0x7FFF7FFFu, kb.w & 0x7FFF7FFFu);
    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ab),
                                                __builtin_bit_cast(bf16x8, make_uint4(up[ks][0], up[ks][1], up[ks][2], up[ks][3])),
                                                ks == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : t, 0, 0, 0);
  };
  // the largest of a lane's four t_k (non-negative floats order as their bits)
  auto tmax4 = [](const f32x4& t) {
    return __uint_as_float(max(max(__float_as_uint(t[0]), __float_as_uint(t[1])),
                               max(__float_as_uint(t[2]), __float_as_uint(t[3]))));
  };

  // One pipeline step: the next group's products (kin -> accn, when
  // NEXT) in KS slices, each slice's MFMAs followed by a slice of the VALU
  // work that finishes local group `it` (the wave's it-th group) from its
  // products accp, so that every MFMA runs on the matrix core while VALU
  // instructions issue; then group it's scores and block scores go to LDS.
  // What the histograms count is returned for count(), which issues the
  // atomics.
  struct Counted {
    float si, bs;
    bool cvalid, bvalid;
  };
  auto step = [&](auto next, int it, const f32x4 (&accp)[MT], const uint4* kin, f32x4 (&accn)[MT]) -> Counted {
    constexpr bool NEXT = decltype(next)::value;
    const int gi = wave + kWaves * it;
    // block j = g/2 of the group holds keys 8j..8j+7 = rows 4g+i of lane groups g and g^1
    const int blk = ((c0 + 16 * gi) >> 3) + (g >> 1);
    float s[4];      // token scores of keys 4g..4g+3 (all 16 lanes of the row)
    float pt[MT];    // block score terms, relu(mean per head)
    f32x4 t;         // t_k of the next group's keys 4g..4g+3
    float inv = 0.125f;
    if constexpr (POOL) {
      const int nb = min(max(nvis - 8 * blk, 0), 8);
      inv = nb == 8 ? 0.125f : __builtin_amdgcn_rcpf((float)max(nb, 1));
    }
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      if constexpr (NEXT) {
        kstep(fragment(kin, c), c, accn, t);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = c; i < 4; i += KS) {
        float v = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) v = fmaf(wr[mt], relu_bits(accp[mt][i]), v);
        s[i] = sum16(v);
      }
      if constexpr (POOL) {
#pragma unroll
        for (int mt = c; mt < MT; mt += KS)
          pt[mt] = relu_bits(add_xor16((accp[mt][0] + accp[mt][1]) + (accp[mt][2] + accp[mt][3])) * inv);
      }
      if constexpr (NEXT) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) mk2 = fmaxf(mk2, tmax4(t));
    // every lane stores one score: lanes n, n+4, n+8, n+12 write the same value
    Counted r;
    const int i0 = n & 3;
    const int cand = c0 + 16 * gi + 4 * g + i0;
    r.si = i0 == 0 ? s[0] : i0 == 1 ? s[1] : i0 == 2 ? s[2] : s[3];
    if (INDIRECT) {
      const int b = cand < nc ? s_pool[(cand - c0) >> 3] : -1;
      r.cvalid = b >= 0 && b * 8 + (cand & 7) < nvis;
    } else {
      r.cvalid = cand < nc;
    }
    s_sc[cand - c0] = r.cvalid ? r.si : -INFINITY;
    r.bs = 0.0f;
    r.bvalid = false;
    if constexpr (POOL) {
      float v = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) v = fmaf(wr[mt], pt[mt], v);
      r.bs = sum16(v);
      r.bvalid = blk < nblk;
      // lanes of both lane groups of the block write the same value
      s_scb[blk - (c0 >> 3)] = r.bvalid ? r.bs : -INFINITY;
    }
    return r;
  };
  auto count = [&](const Counted& r) {
    if constexpr (HIST) {
      if (n < 4 && r.cvalid) atomicAdd(&s_hist[sortable(r.si) >> kBinShift], 1u);
    }
    if constexpr (POOL) {
      // one lane per block (lanes 0 and 32) counts it
      if ((lane & 31) == 0 && r.bvalid) atomicAdd(&s_hist_b[sortable(r.bs) >> kBinShift], 1u);
    }
  };

  // Software pipeline over this wave's groups, group g in buf[g % NBUF].
  // Step s loads group s + NBUF - 1, issues the MFMAs of group s + 1 and
  // finishes group s, so the matrix cores work one group ahead of the VALU
  // code that consumes their results and NBUF - 2 loaded groups wait behind
  // the one in use.  The steady state is straight-line code (every load and
  // store issued unconditionally; past the wave's last group the loads and
  // products repeat that group and are not finished), so the compiler waits
  // only for the group it is about to use; the tail has no loads left to
  // issue.
  uint4 buf[NBUF][KS];
  f32x4 acc[MT];
  auto first_loads = [&]() {
    if (my_groups > 0) {
#pragma unroll
      for (int b = 0; b < NBUF - 1; ++b) {
        load(b, buf[b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // a Full scan's first loads go out before the bound's setup, which waits
  // for the query; a Reindex scan's need the pool ids in LDS first
  if constexpr (!INDIRECT) first_loads();
  u_frag<MT, KS>(qb, wr, up);
  // LDS-only barrier: orders the histogram clear and the pool ids before any
  // wave uses them, without waiting for the query and key loads in flight
  lds_barrier();
  if constexpr (INDIRECT) first_loads();
  if (my_groups > 0) {
    f32x4 t;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kstep(fragment(buf[0], ks), ks, acc, t);
    mk2 = fmaxf(mk2, tmax4(t));
  }
  using with_next = std::integral_constant<bool, true>;
  using last = std::integral_constant<bool, false>;
  int it = 0;
  for (; it + NBUF <= my_groups; it += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      load(it + b + NBUF - 1, buf[(b + NBUF - 1) % NBUF]);
      // keep the loads in issue order (vmcnt retires in order: a group loaded
      // later must not be scheduled ahead of the one needed next)
      __builtin_amdgcn_sched_barrier(0);
      f32x4 nxt[MT];
      count(step(with_next{}, it + b, acc, buf[(b + 1) % NBUF], nxt));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = nxt[mt];
    }
  }
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b) {
    if (it + b < my_groups) {
      f32x4 nxt[MT] = {};
      if (it + b + 1 < my_groups) count(step(with_next{}, it + b, acc, buf[(b + 1) % NBUF], nxt));
      else count(step(last{}, it + b, acc, buf[(b + 1) % NBUF], nxt));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = nxt[mt];
    }
  }

  // ---- publish scores, histograms and the largest t_k
  lds_barrier();
  store_scores<kWaves>(sc, P.gkey + (size_t)p * (P.stride >> 4), s_sc, c0, nslots, wave, lane, P.large_sel != 0);
  if constexpr (POOL) {
    const int nbs = min((nslots + 7) >> 3, max(nblk - (c0 >> 3), 0));
    for (int i = tid; i < nbs; i += kThreads) scb[(c0 >> 3) + i] = s_scb[i];
  }
  if constexpr (!HIST) {
    mk2 = wave_max(mk2);
    if (lane == 0) s_tmp[wave] = __float_as_uint(mk2);
    lds_barrier();
    if (tid == 0) {
      uint32_t m0 = 0;
      for (int i = 0; i < kWaves; ++i) m0 = max(m0, s_tmp[i]);
      P.kpart[(size_t)q * gridDim.x + blockIdx.x] = __uint_as_float(m0);
    }
  } else {
    uint32_t* gh = P.hist + (size_t)p * kNBins;
    for (int i = tid; i < kNBins; i += kThreads) {
      const uint32_t c = s_hist[i];
      if (c) atomicAdd(&gh[i], c);
      if (POOL) {
        const uint32_t cb = s_hist_b[i];
        if (cb) atomicAdd(&P.hist[(size_t)pb * kNBins + i], cb);
      }
    }
    mk2 = wave_max(mk2);
    if (lane == 0) s_tmp[wave] = __float_as_uint(mk2);
    lds_barrier();
    if (tid == 0) {
      uint32_t m0 = 0;
      for (int i = 0; i < kWaves; ++i) m0 = max(m0, s_tmp[i]);
      if (m0) atomicMax(&P.meta[p].maxt, m0);   // non-negative floats order as their bits
    }
  }
}

// ---------------------------------------------------------------- 2b. chunk scan
// The queries of one sequence's chunk (encoder-side chunked prefill: many
// causal queries over the same keys): every work-group scores QB consecutive
// queries against one range of keys, so each key group it loads feeds QB
// queries' MFMAs (the keys' bytes are read once per QB queries instead of
// once per query).  The MFMA computes S = Q . K^T (heads x keys, the
// transpose of k_scan's tile): lane (key n, group g) then holds 4 heads of each
// 16-head tile for one key, so the weighted ReLU head sum runs in registers and
// two lane permutes finish it across the four lane groups.  The products and
// their k-order are those of k_scan; only the order of the head sum differs,
// which the rounding bound covers (it holds for any summation order).
// Positions at or past a query's own visible length are not scores.  One
// coarse histogram per query.
constexpr int kChunkKeys = 4096;   // keys per chunk-scan work-group

template <int D, int MT, int QB>
__global__ __launch_bounds__(kThreads, QB <= 2 ? 2 : 1) void k_scan_chunk(Params P) {   // two waves per SIMD up to QB = 2
  static_assert(QB >= 1 && QB <= 4, "lane group g stores query g's scores");
  constexpr int KS = D / 32;
  constexpr int NBUF = 2;           // one key group in flight, one in use (registers go to the queries)
  __shared__ uint32_t s_hist[QB][kNBins];
  __shared__ __attribute__((aligned(16))) float s_sc[QB][kChunkKeys];
  __shared__ uint32_t s_tmp[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  // x: the query group (the fast dimension of the launch order), y: the key
  // range -- the work-groups resident together, spread over the XCDs, then
  // share one 1 MiB key range, which each XCD's L2 holds
  const int q0 = blockIdx.x * QB;
  const int nq = min(QB, P.n_q - q0);
  const int c0 = blockIdx.y * kChunkKeys;
  int nvis[QB];
  int nmax = 0;
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    nvis[qq] = qq < nq ? P.q_nvis[q0 + qq] : 0;
    nmax = max(nmax, nvis[qq]);
  }
  const int64_t base = P.base0;   // one sequence
  for (int i = tid; i < QB * kNBins; i += kThreads) (&s_hist[0][0])[i] = 0;

  // Q as the MFMA A operand: lane (n, g) holds head 16*mt + n, dims 32*ks + 8*g .. +7;
  // wq: the weights of the heads this lane's accumulators hold (16*mt + 4*g + i)
  bf16x8 qb[QB][MT][KS];
  float wq[QB][MT][4];
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    const int q = min(q0 + qq, P.n_q - 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int head = 16 * mt + n;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (head < P.h_i)
          v = *reinterpret_cast<const uint4*>(P.iq + ((size_t)q * P.h_i + head) * D + 32 * ks + 8 * g);
        qb[qq][mt][ks] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hw = 16 * mt + 4 * g + i;
        wq[qq][mt][i] = hw < P.h_i ? P.w[(size_t)q * P.h_i + hw] : 0.0f;
      }
    }
  }
  // the bound's key magnitude with the block's largest u (dim by dim over its
  // queries, each u from its fragments and the weights of heads 16 mt + n):
  // an upper bound of every query's own t_k, for one dot per key
  uint32_t up[KS][4];
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    const int q = min(q0 + qq, P.n_q - 1);
    float wn[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) wn[mt] = 16 * mt + n < P.h_i ? P.w[(size_t)q * P.h_i + 16 * mt + n] : 0.0f;
    uint32_t uq[KS][4];
    u_frag<MT, KS>(qb[qq], wn, uq);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // bf16 pairs of non-negative values: the larger of each half
        const uint32_t a = qq ? up[ks][j] : 0u, b = uq[ks][j];
        up[ks][j] = max(a & 0xFFFF0000u, b & 0xFFFF0000u) | max(a & 0xFFFFu, b & 0xFFFFu);
      }
  }
  lds_barrier();   // the histogram clear; the query loads stay in flight

  float mk2 = 0.0f;   // the largest key magnitude (block's u) of the chunk
  const int nslots = min(kChunkKeys, max(nmax - c0, 0));
  const int ngroups = (nslots + 15) >> 4;
  const int my_groups = ngroups > wave ? (ngroups - wave + kWaves - 1) / kWaves : 0;
  auto key_row = [&](int it, bool& valid) -> int64_t {
    const int cand = c0 + 16 * (wave + kWaves * it) + n;
    valid = cand < nmax;
    return base + (valid ? cand : 0);
  };
  auto load = [&](int it, uint4* kb) {
    bool v;
    const uint4* src = reinterpret_cast<const uint4*>(P.ik + (size_t)key_row(min(it, my_groups - 1), v) * D + 8 * g);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kb[ks] = src[4 * ks];
  };
  auto process = [&](int it, const uint4 (&kb)[KS]) {
    const int gi = wave + kWaves * it;
    // no masking: a slot past the visible keys loaded the sequence's first key
    // (key_row), whose t_k belongs to the maximum anyway and whose scores are
    // not stored
    {
      // t_k = |K| . u by one more MFMA (u, the lane's fragment, in every row
      // of the A operand; lane (n, g) gets t of key n), as in k_scan
      f32x4 t = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 ab = make_uint4(kb[ks].x & 0x7FFF7FFFu, kb[ks].y & 0x7FFF7FFFu, kb[ks].z & 0x7FFF7FFFu,
                                    kb[ks].w & 0x7FFF7FFFu);
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, make_uint4(up[ks][0], up[ks][1], up[ks][2], up[ks][3])),
            __builtin_bit_cast(bf16x8, ab), t, 0, 0, 0);
      }
      mk2 = fmaxf(mk2, t[0]);
    }
    const int cand = c0 + 16 * gi + n;   // this lane's key
    float sq[QB];
#pragma unroll
    for (int qq = 0; qq < QB; ++qq) {
      f32x4 acc[MT];   // acc[mt][i]: head 16*mt + 4*g + i, key n
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, kb[ks]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[qq][mt][ks], b, acc[mt], 0, 0, 0);
      }
      float v = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wq[qq][mt][i], relu_bits(acc[mt][i]), v);
      sq[qq] = sum_rows4(v);   // + the other three lane groups' heads
    }
    // lane group g stores query g's score and counts it: one store and one
    // LDS atomic instruction for the QB queries
    if (g < QB) {
      float si = sq[0];
      int nv = nvis[0];
#pragma unroll
      for (int qq = 1; qq < QB; ++qq) {
        si = g == qq ? sq[qq] : si;
        nv = g == qq ? nvis[qq] : nv;
      }
      const bool cvalid = cand < nv;
      s_sc[g][cand - c0] = cvalid ? si : -INFINITY;
      if (cvalid) atomicAdd(&s_hist[g][sortable(si) >> kBinShift], 1u);
    }
  };

  uint4 buf[NBUF][KS];
  if (my_groups > 0) {
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) {
      load(b, buf[b]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  int it = 0;
  for (; it + NBUF <= my_groups; it += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      load(it + b + NBUF - 1, buf[(b + NBUF - 1) % NBUF]);
      __builtin_amdgcn_sched_barrier(0);
      process(it + b, buf[b]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b)
    if (it + b < my_groups) process(it + b, buf[b]);

  // ---- publish: each query's scores and histogram, the largest t_k
  lds_barrier();
#pragma unroll
  for (int qq = 0; qq < QB; ++qq) {
    if (qq < nq) {
      const int q = q0 + qq;
      const int ns = min(kChunkKeys, max(nvis[qq] - c0, 0));
      store_scores<kWaves>(P.scores + (size_t)q * P.stride, P.gkey + (size_t)q * (P.stride >> 4), s_sc[qq], c0,
                           ns, wave, lane, P.large_sel != 0);
      uint32_t* gh = P.hist + (size_t)q * kNBins;
      for (int i = tid; i < kNBins; i += kThreads) {
        const uint32_t c = s_hist[qq][i];
        if (c) atomicAdd(&gh[i], c);
      }
    }
  }
  mk2 = wave_max(mk2);
  if (lane == 0) s_tmp[wave] = __float_as_uint(mk2);
  lds_barrier();
  if (tid < nq) {
    uint32_t m0 = 0;
    for (int i = 0; i < kWaves; ++i) m0 = max(m0, s_tmp[i]);
    if (m0) atomicMax(&P.meta[q0 + tid].maxt, m0);   // an upper bound of each query's own largest t_k
  }
}

// 16 consecutive scores of one compaction chunk per thread (my0 + 15 <
// stride: the load stays inside the problem's row; entries at or past the
// candidate count are not counted, see count16).
__device__ __forceinline__ void load16(const Params& P, int p, int my0, float* v) {
  const float4* s4 = reinterpret_cast<const float4*>(P.scores + (size_t)p * P.stride + my0);
#pragma unroll
  for (int j = 0; j < kCmpPerThread / 4; ++j) {
    const float4 t = s4[j];
    v[4 * j] = t.x;
    v[4 * j + 1] = t.y;
    v[4 * j + 2] = t.z;
    v[4 * j + 3] = t.w;
  }
}
__device__ __forceinline__ int count16(int nc, int my0) { return max(0, min(kCmpPerThread, nc - my0)); }

// ---------------------------------------------------------------- 3. fine histogram
// Histogram of bits 19..8 of the keys that fall into the coarse bin: the K-th
// score is then located to 2^-15 of its value.  Every work-group first finds
// the coarse bin itself (kernel boundaries make the scan's histograms
// visible); chunk 0 publishes it.
__global__ __launch_bounds__(kThreads) void k_finehist(Params P) {
  __shared__ uint32_t s_h[kNBins];
  __shared__ uint32_t s_tmp[16];
  const int tid = threadIdx.x;
  if (P.large_sel) {
    // Large problems: k_coarse published the bin, so each thread works alone
    // (no barrier): a token thread whose 16 scores stay below the bin
    // loads nothing, and the few scores inside the bin go straight to the
    // problem's fine histogram.
    int p, chunk0, nch = 1;
    if (large_multi(P)) {
      p = blockIdx.y;
      chunk0 = blockIdx.x * kLargeChunks;
      nch = min(kLargeChunks, P.nchunk_cmp - chunk0);
    } else {
      grid_chunk(P, &p, &chunk0);
    }
    const int q = p % P.n_q, kind = p / P.n_q;
    // every load that does not depend on another goes out first: the visible
    // length, the bin and the 16-bit group keys of all the thread's chunks
    // (one 2-byte key per chunk); only the rare groups reaching the bin then
    // load their scores
    const int nvis = P.q_nvis[q];
    const uint32_t bin = P.meta[p].bin;
    uint32_t gk[kLargeChunks];
#pragma unroll
    for (int c = 0; c < kLargeChunks; ++c) {
      const int chunk = min(chunk0 + c, P.nchunk_cmp - 1);   // in bounds; chunks past nch are not used
      gk[c] = kind == 0 ? P.gkey[(size_t)p * (P.stride >> 4) + ((chunk * kCmpChunk + tid * kCmpPerThread) >> 4)] : 0xFFFFu;
    }
    const int nc = cands_of(P, kind, nvis);
    if (bin == kAll) return;
    uint32_t* gh = P.hist2 + (size_t)p * kNBins;
#pragma unroll
    for (int c = 0; c < kLargeChunks; ++c) {
      if (c >= nch) break;
      const int chunk = chunk0 + c;
      if (chunk > 0 && chunk * kCmpChunk >= nc) break;
      const int my0 = chunk * kCmpChunk + tid * kCmpPerThread;
      if ((gk[c] >> (kBinShift - 16)) < bin) continue;
      float v[kCmpPerThread];
      load16(P, p, my0, v);
      const int m = count16(nc, my0);
#pragma unroll
      for (int j = 0; j < kCmpPerThread; ++j) {
        if (j < m && v[j] != -INFINITY) {
          const uint32_t key = sortable(v[j]);
          if ((key >> kBinShift) == bin) atomicAdd(&gh[(key >> 8) & (kNBins - 1)], 1u);
        }
      }
    }
    return;
  }
  int p, chunk;
  grid_chunk(P, &p, &chunk);
  const int q = p % P.n_q, kind = p / P.n_q;
  // the visible length first: a chunk past the problem's candidates (the grid
  // spans the longest context; shorter ones leave most chunks empty) leaves
  // before loading anything.
  const int nc = cands_of(P, kind, P.q_nvis[q]);
  if (chunk > 0 && chunk * kCmpChunk >= nc) return;
  const int my0 = chunk * kCmpChunk + tid * kCmpPerThread;
  // Then every load goes out at once: the chunk's scores (inside the
  // problem's row), the coarse histogram and the bound's inputs
  float v[kCmpPerThread];
  load16(P, p, my0, v);
  uint32_t hv[kHPer];
  load_hist16(P.hist + (size_t)p * kNBins, hv);
  const float maxt = __uint_as_float(P.meta[q].maxt), wabs = P.meta[p].wabs;
  for (int i = tid; i < kNBins; i += kThreads) s_h[i] = 0;
  const uint32_t bin = wg_coarse_bin(P, p, hv, chunk == 0, maxt, wabs, s_tmp);   // its barriers order the clear
  if (bin == kAll || chunk * kCmpChunk >= nc) return;
  const int m = count16(nc, my0);
#pragma unroll
  for (int j = 0; j < kCmpPerThread; ++j) {
    if (j < m && v[j] != -INFINITY) {
      const uint32_t key = sortable(v[j]);
      if ((key >> kBinShift) == bin) atomicAdd(&s_h[(key >> 8) & (kNBins - 1)], 1u);
    }
  }
  lds_barrier();
  uint32_t* gh = P.hist2 + (size_t)p * kNBins;
  for (int i = tid; i < kNBins; i += kThreads) {
    const uint32_t c = s_h[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Band thresholds, computed by every compaction work-group from the fine
// histogram: with the fine bin [L, U] that holds the K-th approximate score
// a_K (so L <= a_K and U >= a_K >= a_K1), keep a >= L - 2 Delta (every exact
// Top-K member) and call a > U + 2 Delta certain.  No bin (at most K
// candidates): keep everything, all certain.
// hv: this thread's 16 bins of the fine histogram (as load_hist16); bin,
// above and delta: the problem's Meta fields.
__device__ void wg_band_thresholds(const Params& P, int p, const uint32_t hv[kHPer], uint32_t m_bin,
                                   uint32_t m_above, float m_delta, bool publish, uint32_t* s_tmp /*>= 16*/,
                                   float* keep_thr, float* in_thr) {
  const int tid = threadIdx.x;
  const int kind = p / P.n_q;
  const int K = (kind == 1) ? P.keep_blocks : P.k;
  struct {
    uint32_t bin, above;
    float delta;
  } m = {m_bin, m_above, m_delta};
  if (m.bin == kAll) {
    *keep_thr = *in_thr = -INFINITY;
    if (publish && tid == 0) P.meta[p].keep_thr = P.meta[p].in_thr = -INFINITY;
    return;
  }
  const uint32_t need = (uint32_t)K - m.above;   // >= 1
  constexpr int kPer = kHPer;
  const int f_hi = kNBins - kPer * tid - 1;
  if (tid == 0) s_tmp[12] = s_tmp[13] = __float_as_uint(-INFINITY);   // ordered by the scan's barriers
  uint32_t loc = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) loc += hv[j];
  uint32_t tot;
  const uint32_t above = wg_exclusive_scan(loc, s_tmp, &tot);
  if (above < need && above + loc >= need) {
    uint32_t run = above;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (run + hv[j] >= need) {
        const uint32_t lo_key = (m.bin << kBinShift) | ((uint32_t)(f_hi - j) << 8);
        const float kt = band_below(unsortable(lo_key), m.delta);
        const float it = band_above(unsortable(lo_key + 255u), m.delta);
        s_tmp[12] = __float_as_uint(kt);
        s_tmp[13] = __float_as_uint(it);
        if (publish) {
          P.meta[p].keep_thr = kt;
          P.meta[p].in_thr = it;
        }
        break;
      }
      run += hv[j];
    }
  }
  lds_barrier();
  *keep_thr = __uint_as_float(s_tmp[12]);
  *in_thr = __uint_as_float(s_tmp[13]);
  lds_barrier();
}

// Large problems (thousands of selection work-groups per problem): the coarse
// bin with the bound, and then the band, once per problem in one work-group
// each, instead of in every selection work-group from the whole histogram.
__global__ __launch_bounds__(kThreads) void k_coarse(Params P) {
  __shared__ uint32_t s_tmp[16];
  const int p = blockIdx.x, q = p % P.n_q;
  uint32_t hv[kHPer];
  load_hist16(P.hist + (size_t)p * kNBins, hv);
  const float maxt = __uint_as_float(P.meta[q].maxt), wabs = P.meta[p].wabs;
  (void)wg_coarse_bin(P, p, hv, true, maxt, wabs, s_tmp);
}

__global__ __launch_bounds__(kThreads) void k_band(Params P) {
  __shared__ uint32_t s_tmp[16];
  const int p = blockIdx.x;
  uint32_t hv[kHPer];
  load_hist16(P.hist2 + (size_t)p * kNBins, hv);
  float keep_thr, in_thr;
  wg_band_thresholds(P, p, hv, P.meta[p].bin, P.meta[p].above, P.meta[p].delta, true, s_tmp, &keep_thr, &in_thr);
}

// ---------------------------------------------------------------- 4. compaction
// Band members of one chunk, in position order, flagged certain or not; the
// uncertain ones are also listed (chunk-local index) for the rescoring.
//
// Large problems (k_band published the band): one wave per chunk, four
// chunks per work-group and no barrier.  Lane l holds the chunk's scores
// 64 l .. 64 l + 63, four groups of the scan's group maxima, and loads a
// group only when its maximum reaches the band (a block chunk, which has no
// maxima, always loads); a DPP scan over the lanes of the kept and uncertain
// counts places the entries exactly where the per-work-group kernel below
// puts them.
constexpr int kCmpLanePer = kCmpChunk / kWave;   // scores per lane (64)

__global__ __launch_bounds__(kThreads) void k_compact_large(Params P) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int pool = P.keep_blocks > 0 && !P.reindex;
  const int nblk_ch = pool ? (P.nchunk_cmp + 7) >> 3 : 0;
  const int f = (int)blockIdx.x * kWaves + wave;   // chunk of this wave: the token row's, then the block row's
  if (f >= P.nchunk_cmp + nblk_ch) return;
  const int kind = f >= P.nchunk_cmp ? 1 : 0;
  const int chunk = kind ? f - P.nchunk_cmp : f;
  const int q = blockIdx.y, p = kind * P.n_q + q;
  const int c0 = chunk * kCmpChunk;
  const int my0 = c0 + lane * kCmpLanePer;
  // the independent loads first (visible length, band, the lane's four
  // 16-bit group keys), then the scores that can reach the band
  const int nvis = P.q_nvis[q];
  const float keep_thr = P.meta[p].keep_thr, in_thr = P.meta[p].in_thr;
  uint2 gk = make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu);
  if (kind == 0) gk = *reinterpret_cast<const uint2*>(P.gkey + (size_t)p * (P.stride >> 4) + (my0 >> 4));
  const int nc = cands_of(P, kind, nvis);
  if (chunk > 0 && c0 >= nc) {
    if (lane == 0) {
      P.chunk_cnt[(size_t)p * P.nchunk_cmp + chunk] = 0;
      P.chunk_unc[(size_t)p * P.nchunk_cmp + chunk] = 0;
    }
    return;
  }
  const int m = max(0, min(kCmpLanePer, nc - my0));
  // the lane's four 16-score groups: each is loaded only if it holds a
  // candidate and (token rows) its largest key reaches the band's
  uint32_t need = 0;
  {
    const uint32_t thr16 = sortable(keep_thr) >> 16;
    const uint32_t k16[4] = {gk.x & 0xFFFFu, gk.x >> 16, gk.y & 0xFFFFu, gk.y >> 16};
#pragma unroll
    for (int g = 0; g < 4; ++g) need |= (16 * g < m && k16[g] >= thr16 ? 1u : 0u) << g;
  }
  float v[kCmpLanePer];
  const float4* s4 = reinterpret_cast<const float4*>(P.scores + (size_t)p * P.stride + my0);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if ((need >> g) & 1u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 t = s4[4 * g + j];
        v[16 * g + 4 * j] = t.x;
        v[16 * g + 4 * j + 1] = t.y;
        v[16 * g + 4 * j + 2] = t.z;
        v[16 * g + 4 * j + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[16 * g + j] = -INFINITY;
    }
  }
  uint64_t keep = 0, cert = 0;
#pragma unroll
  for (int j = 0; j < kCmpLanePer; ++j) {
    const bool k_ = j < m && v[j] != -INFINITY && v[j] >= keep_thr;
    keep |= (k_ ? 1ull : 0ull) << j;
    cert |= ((k_ && v[j] > in_thr) ? 1ull : 0ull) << j;
  }
  // both counts in one scan (each at most kCmpChunk, so the halves never carry)
  const uint32_t mine = (uint32_t)__popcll(keep) | ((uint32_t)__popcll(keep & ~cert) << 16);
  const uint32_t incl = wave_incl_scan_u32(mine);
  const uint32_t both = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  uint32_t off = (incl - mine) & 0xFFFFu, uoff = (incl - mine) >> 16;
  Entry* dst = P.band + (size_t)p * P.stride + c0;
  uint2* udst = P.unc + (size_t)p * P.stride + c0;
  // the few kept scores are read again (cached) rather than picked out of
  // the registers by a run-time index, which would move them to scratch
  const float* row = P.scores + (size_t)p * P.stride;
  while (keep) {
    const int j = __builtin_ctzll(keep);
    keep &= keep - 1;
    const bool c_ = (cert >> j) & 1ull;
    dst[off] = Entry{(uint32_t)(my0 + j) | (c_ ? kCertain : 0u), row[my0 + j]};
    if (!c_) udst[uoff++] = make_uint2(off, (uint32_t)(my0 + j));
    ++off;
  }
  if (lane == 0) {
    P.chunk_cnt[(size_t)p * P.nchunk_cmp + chunk] = both & 0xFFFFu;
    P.chunk_unc[(size_t)p * P.nchunk_cmp + chunk] = both >> 16;
  }
}

// Per-work-group mode.
__global__ __launch_bounds__(kThreads) void k_compact(Params P) {
  __shared__ uint32_t s_tmp[16];
  const int tid = threadIdx.x;
  auto chunk_body = [&](int p, int chunk) {
    const int q = p % P.n_q, kind = p / P.n_q;
    const int c0 = chunk * kCmpChunk;
    // the visible length first: a chunk past the problem's candidates only
    // records empty counts (the later kernels sum the counts of every chunk of
    // the row) and loads nothing.  Then every load goes out at once: the
    // chunk's scores, the fine histogram and the Meta fields the fine
    // histogram kernel published
    const int nc = cands_of(P, kind, P.q_nvis[q]);
    if (chunk > 0 && c0 >= nc) {
      if (tid == 0) {
        P.chunk_cnt[(size_t)p * P.nchunk_cmp + chunk] = 0;
        P.chunk_unc[(size_t)p * P.nchunk_cmp + chunk] = 0;
      }
      return;
    }
    const int my0 = c0 + tid * kCmpPerThread;
    float v[kCmpPerThread];
    load16(P, p, my0, v);
    uint32_t hv[kHPer];
    load_hist16(P.hist2 + (size_t)p * kNBins, hv);
    const uint32_t m_bin = P.meta[p].bin, m_above = P.meta[p].above;
    const float m_delta = P.meta[p].delta;
    float keep_thr = -INFINITY, in_thr = -INFINITY;
    if (chunk == 0 || c0 < nc) wg_band_thresholds(P, p, hv, m_bin, m_above, m_delta, chunk == 0, s_tmp, &keep_thr, &in_thr);
    const int m = count16(nc, my0);
    uint32_t keep = 0, cert = 0;
#pragma unroll
    for (int j = 0; j < kCmpPerThread; ++j) {
      const bool k_ = j < m && v[j] != -INFINITY && v[j] >= keep_thr;
      keep |= (k_ ? 1u : 0u) << j;
      cert |= ((k_ && v[j] > in_thr) ? 1u : 0u) << j;
    }
    // one scan for both counts (each at most kCmpChunk, so the halves never carry)
    uint32_t both;
    const uint32_t ob = wg_exclusive_scan(__popc(keep) | ((uint32_t)__popc(keep & ~cert) << 16), s_tmp, &both);
    uint32_t off = ob & 0xFFFFu, uoff = ob >> 16;
    const uint32_t total = both & 0xFFFFu, utotal = both >> 16;
    Entry* dst = P.band + (size_t)p * P.stride + c0;
    uint2* udst = P.unc + (size_t)p * P.stride + c0;
#pragma unroll
    for (int j = 0; j < kCmpPerThread; ++j) {
      if (keep & (1u << j)) {
        const bool c_ = (cert >> j) & 1u;
        dst[off] = Entry{(uint32_t)(my0 + j) | (c_ ? kCertain : 0u), v[j]};
        if (!c_) udst[uoff++] = make_uint2(off, (uint32_t)(my0 + j));
        ++off;
      }
    }
    if (tid == 0) {
      P.chunk_cnt[(size_t)p * P.nchunk_cmp + chunk] = total;
      P.chunk_unc[(size_t)p * P.nchunk_cmp + chunk] = utotal;
    }
  };
  int p, chunk;
  grid_chunk(P, &p, &chunk);
  chunk_body(p, chunk);
}

// Exclusive prefix of a problem's per-chunk counts into LDS (s[0..nch]).
template <int NT = kThreads>
__device__ __forceinline__ void chunk_prefix(const uint32_t* cnt, int nch, uint32_t* s, uint32_t* s_tmp) {
  uint32_t carry = 0;
  for (int t0 = 0; t0 < nch; t0 += NT) {
    const int c = t0 + threadIdx.x;
    const uint32_t cv = c < nch ? cnt[c] : 0u;
    uint32_t tt;
    const uint32_t ex = wg_exclusive_scan<NT>(cv, s_tmp, &tt);
    if (c < nch) s[c] = carry + ex;
    carry += tt;
  }
  if (threadIdx.x == 0) s[nch] = carry;
  lds_barrier();
}

// Largest c in [0, nch) with s[c] <= j.
__device__ __forceinline__ int chunk_of(const uint32_t* s, int nch, uint32_t j) {
  int lo = 0, hi = nch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s[mid] <= j) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- 5. rescoring
// Exact scores of the uncertain band members, one member per wave, one lane
// per head.  The lane's query row is held in registers; the member keys
// (wave-uniform) are converted to fp32 once into the wave's LDS slot and read
// back as broadcast 16-byte reads, four chain steps per read, the next four
// dimensions of all eight members loading while the current ones are used.
// The next member's keys are loaded while the current one is scored.  A block
// runs its eight member chains interleaved.
//
// Work-groups [0, rs_tok) of grid row q serve query q's token (or Reindex)
// problem, their waves striding over its members.  The other work-groups
// serve the block problems.  With rs_pool set, the block waves of every row
// form one pool: each query gets waves in proportion to its undecided blocks
// (contiguous ranges of `per` members, from a prefix over every query's chunk
// counts), so that the long contexts of a mixed batch, which hold nearly all
// of its block band, spread over the whole grid; without it, row q's block
// work-groups serve query q alone.  A wave never leaves its query.
constexpr int kPoolMaxQ = 256;   // queries of a pooled block rescoring

template <int D>
__global__ __launch_bounds__(kThreads) void k_rescore(Params P) {
  constexpr int DW = D / 2;            // packed bf16 pairs per key row
  constexpr int KPER = 8 * DW / 64;    // key dwords of 8 members per lane
  __shared__ uint32_t s_tmp[16];
  __shared__ uint32_t s_uoff[kMaxChunksLds + 1];
  __shared__ uint32_t s_woff[kPoolMaxQ + 1];
  __shared__ __attribute__((aligned(16))) float s_kf[kWaves][8][D];
  __shared__ __attribute__((aligned(16))) float s_w[kWaves][kWave];
  __shared__ __attribute__((aligned(16))) float s_r[kWaves][kWave];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kind = (int)blockIdx.x < P.rs_tok ? 0 : 1;
  const bool pooled = kind == 1 && P.rs_pool != 0;
  const int nbw = (int)gridDim.x - P.rs_tok;   // block work-groups per grid row
  // segments of the member list: one problem's chunks, or every query's block chunks
  const int nchk = nchunks_of(P, kind);
  const int nseg = pooled ? P.n_q * nchk : nchk;
  const int wg = pooled ? (int)blockIdx.y * nbw + ((int)blockIdx.x - P.rs_tok)
                        : (kind ? (int)blockIdx.x - P.rs_tok : (int)blockIdx.x);
  const int nwg = pooled ? P.n_q * nbw : (kind ? nbw : P.rs_tok);
  // exclusive prefix of the segments' uncertain counts into s_uoff[0 .. nseg]
  {
    uint32_t carry = 0;
    for (int t0 = 0; t0 < nseg; t0 += kThreads) {
      const int f = t0 + tid;
      uint32_t cv = 0;
      if (f < nseg) {
        const int qf = pooled ? f / nchk : (int)blockIdx.y, c = pooled ? f - qf * nchk : f;
        cv = P.chunk_unc[(size_t)(kind * P.n_q + qf) * P.nchunk_cmp + c];
      }
      uint32_t tt;
      const uint32_t ex = wg_exclusive_scan(cv, s_tmp, &tt);
      if (f < nseg) s_uoff[f] = carry + ex;
      carry += tt;
    }
    if (tid == 0) s_uoff[nseg] = carry;
    lds_barrier();
  }
  const int nwaves = nwg * kWaves, v = wg * kWaves + wave;
  int q, j, j_end, stride_w;
  if (pooled) {
    // query qq gets ceil(n_qq / per) waves; per leaves one spare wave per
    // query for the rounding up, so every query's members are covered
    const int nu = (int)s_uoff[nseg];
    const int per = max(1, (nu + nwaves - P.n_q - 1) / (nwaves - P.n_q));
    uint32_t wc = 0;
    if (tid < P.n_q) wc = (s_uoff[(tid + 1) * nchk] - s_uoff[tid * nchk] + per - 1) / per;
    uint32_t wt;
    const uint32_t wo = wg_exclusive_scan(wc, s_tmp, &wt);
    if (tid < P.n_q) s_woff[tid] = wo;
    if (tid == 0) s_woff[P.n_q] = wt;
    lds_barrier();
    if (v >= (int)wt) return;
    q = __builtin_amdgcn_readfirstlane(chunk_of(s_woff, P.n_q, (uint32_t)v));
    const int m0 = (int)s_uoff[q * nchk], m1 = (int)s_uoff[(q + 1) * nchk];
    j = __builtin_amdgcn_readfirstlane(m0 + (v - (int)s_woff[q]) * per);
    j_end = __builtin_amdgcn_readfirstlane(min(m1, j + per));
    stride_w = 1;
  } else {
    q = blockIdx.y;
    j = v;
    j_end = (int)s_uoff[nseg];
    stride_w = nwaves;
  }
  if (j >= j_end) return;
  const int p = kind * P.n_q + q;
  const int nvis = P.q_nvis[q];
  const int64_t base = seq_base_of(P, q);
  Entry* band = P.band + (size_t)p * P.stride;
  const uint2* unc = P.unc + (size_t)p * P.stride;
  // this problem's segments: s_uoff[seg0 .. seg0 + nchk]
  const int seg0 = pooled ? q * nchk : 0;

  // the head weights in the wave's own LDS row (wave-private: no barrier)
  s_w[wave][lane] = lane < P.h_i ? P.w[(size_t)q * P.h_i + lane] : 0.0f;
  uint32_t qrow[DW];   // the lane's query row, packed bf16 pairs
  {
    const int hh = lane < P.h_i ? lane : 0;
    const uint4* src = reinterpret_cast<const uint4*>(P.iq + ((size_t)q * P.h_i + hh) * D);
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
      const uint4 vv = src[i];
      qrow[4 * i] = vv.x;
      qrow[4 * i + 1] = vv.y;
      qrow[4 * i + 2] = vv.z;
      qrow[4 * i + 3] = vv.w;
    }
  }
  auto qv = [&](int d) {   // query element d as fp32
    return (d & 1) ? __uint_as_float(qrow[d >> 1] & 0xFFFF0000u) : __uint_as_float(qrow[d >> 1] << 16);
  };
  float* kf = &s_kf[wave][0][0];

  // Ordered head sum s = fma(w_h, r_h, s), h ascending, from LDS (every lane
  // runs the same chain on broadcast reads).  Entries h >= h_i hold w = 0 and
  // a finite r, so fma(0, r, s) returns s exactly: running all 64 equals the
  // chain over h < h_i.
  auto head_sum = [&](float r) {
    s_r[wave][lane] = r;   // wave-private row: LDS keeps the wave's order
    float sc = 0.0f;
#pragma unroll 2
    for (int h4 = 0; h4 < 16; ++h4) {   // partial unroll: few reads in flight, few VGPRs
      const f32x4 wv = *reinterpret_cast<const f32x4*>(&s_w[wave][4 * h4]);
      const f32x4 rv = *reinterpret_cast<const f32x4*>(&s_r[wave][4 * h4]);
      sc = fmaf(wv.x, rv.x, sc);
      sc = fmaf(wv.y, rv.y, sc);
      sc = fmaf(wv.z, rv.z, sc);
      sc = fmaf(wv.w, rv.w, sc);
    }
    return sc;
  };

  // candidate jj of this problem: its band slot, first member and member count
  struct Cand {
    uint32_t slot;
    int first, nmem;
  };
  // members are visited in ascending order: a pooled wave finds its first
  // segment by a search and walks forward from there
  int f_cur = seg0 + (pooled ? chunk_of(s_uoff + seg0, nchk, (uint32_t)j) : 0);
  auto locate = [&](int jj) {
    int f;
    if (pooled) {
      f = f_cur;
      while (s_uoff[f + 1] <= (uint32_t)jj) ++f;
      f = __builtin_amdgcn_readfirstlane(f);
      f_cur = f;
    } else {
      f = chunk_of(s_uoff, nseg, (uint32_t)jj);
    }
    const int c = f - seg0;
    const uint2 u = unc[(size_t)c * kCmpChunk + (jj - s_uoff[f])];
    const uint32_t cand = __builtin_amdgcn_readfirstlane(u.y);
    Cand r;
    r.slot = (uint32_t)c * kCmpChunk + __builtin_amdgcn_readfirstlane(u.x);
    if (kind == 1) {
      r.first = (int)cand * 8;
      r.nmem = min(nvis - r.first, 8);
    } else {
      r.first = cand_pos(P, q, kind, cand);
      r.nmem = 1;
    }
    return r;
  };
  // dword e of the 8-member key block (member e / DW, dword e % DW) goes to
  // lane e % 64, register e / 64; rows past the member count read member 0
  auto load_keys = [&](const Cand& c, uint32_t* wv) {
#pragma unroll
    for (int k = 0; k < KPER; ++k) {
      const int e = lane + 64 * k, t = e / DW, d2 = e % DW;
      const int tt = t < c.nmem ? t : 0;
      wv[k] = key_pair<D>(P, base + c.first + tt, d2);
    }
  };
  auto stage_keys = [&](const Cand& c, const uint32_t* wv) {
#pragma unroll
    for (int k = 0; k < KPER; ++k) {
      const int e = lane + 64 * k, t = e / DW, d2 = e % DW;
      const uint32_t x = t < c.nmem ? wv[k] : 0u;
      *reinterpret_cast<f32x2*>(&kf[t * D + 2 * d2]) = f32x2{__uint_as_float(x << 16), __uint_as_float(x & 0xFFFF0000u)};
    }
  };

  Cand cur = locate(j);
  uint32_t wv[KPER];
  load_keys(cur, wv);
  for (;;) {
    stage_keys(cur, wv);
    const int jn = j + stride_w;
    const bool more = jn < j_end;
    Cand nxt = cur;
    if (more) {
      nxt = locate(jn);
      load_keys(nxt, wv);   // in flight while the chains below run
    }
    float r;
    if (kind == 1) {
      // the query row's fp32 values are formed per block rather than held
      // across the loop: 64 registers fewer, three waves per SIMD
#pragma unroll
      for (int i = 0; i < DW; ++i) asm volatile("" : "+v"(qrow[i]));
      float a[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) a[t] = 0.0f;
      f32x4 kb[2][8];
#pragma unroll
      for (int t = 0; t < 8; ++t) kb[0][t] = *reinterpret_cast<const f32x4*>(&kf[t * D]);
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        if (d4 + 1 < D / 4) {
#pragma unroll
          for (int t = 0; t < 8; ++t) kb[(d4 + 1) & 1][t] = *reinterpret_cast<const f32x4*>(&kf[t * D + 4 * d4 + 4]);
        }
        const float q0 = qv(4 * d4), q1 = qv(4 * d4 + 1), q2 = qv(4 * d4 + 2), q3 = qv(4 * d4 + 3);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const f32x4 k4 = kb[d4 & 1][t];
          a[t] = fmaf(q0, k4.x, a[t]);
          a[t] = fmaf(q1, k4.y, a[t]);
          a[t] = fmaf(q2, k4.z, a[t]);
          a[t] = fmaf(q3, k4.w, a[t]);
        }
      }
      float sum = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (t < cur.nmem) sum = sum + a[t];
      const float mean = __fdiv_rn(sum, (float)cur.nmem);
      r = mean > 0.0f ? mean : 0.0f;
    } else {
      float acc = 0.0f;
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(&kf[4 * d4]);
        acc = fmaf(qv(4 * d4), k4.x, acc);
        acc = fmaf(qv(4 * d4 + 1), k4.y, acc);
        acc = fmaf(qv(4 * d4 + 2), k4.z, acc);
        acc = fmaf(qv(4 * d4 + 3), k4.w, acc);
      }
      r = acc > 0.0f ? acc : 0.0f;
    }
    const float sc = head_sum(r);
    if (lane == 0) band[cur.slot].s = sc;
    if (!more) break;
    // the prefetched words become visible only here, so their wait stays
    // below the chains
#pragma unroll
    for (int k = 0; k < KPER; ++k) asm volatile("" : "+v"(wv[k]));
    cur = nxt;
    j = jn;
  }
}

// ---------------------------------------------------------------- 6. final
// One work-group per problem: the certain members plus the best rescored
// ones (exact score desc, position asc), written as ascending positions and
// padded with -1.  The band is read in position order through the chunk
// prefix; bands up to kBandLds entries are staged in LDS first.  1024 threads:
// only a few problems run, so each gets a whole CU.
constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(kFinalThreads) void k_final(Params P) {
  constexpr int NT = kFinalThreads;
  __shared__ uint32_t s_tmp[2 * NT / kWave + 2];
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_off[kMaxChunksLds + 1];
  __shared__ uint32_t s_key[kBandLds];
  __shared__ uint32_t s_cand[kBandLds];
  // the radix path keys the uncertain members, the pairwise path ranks
  // (key, index) composites: the two never coexist
  __shared__ __attribute__((aligned(16))) uint32_t s_ukey[kUncLds];
  uint64_t* s_ucomp = reinterpret_cast<uint64_t*>(s_ukey);
  __shared__ uint32_t s_rank[kRankMax];
  const int tid = threadIdx.x;
  const int p = blockIdx.x, q = p % P.n_q, kind = p / P.n_q;
  const int nch = nchunks_of(P, kind);
  const Entry* band = P.band + (size_t)p * P.stride;
  const int K = (kind == 1) ? P.keep_blocks : P.k;
  int32_t* out = (kind == 1) ? P.pool_out + (size_t)q * P.keep_blocks : P.idx_out + (size_t)q * P.k;

  chunk_prefix<NT>(P.chunk_cnt + (size_t)p * P.nchunk_cmp, nch, s_off, s_tmp);
  const int n2 = (int)s_off[nch];
  // per-thread contiguous segment of the position-ordered band
  const int per = (n2 + NT - 1) / NT;
  const int i0 = min(n2, tid * per), i1 = min(n2, i0 + per);
  const bool in_lds = n2 <= kBandLds;
  auto entry_at = [&](int i) {
    const int c = chunk_of(s_off, nch, (uint32_t)i);
    return band[(size_t)c * kCmpChunk + (i - s_off[c])];
  };
  if (in_lds && i0 < i1) {
    // this thread's segment: one search for its first chunk, then a forward
    // walk; batches of U loads are in flight together
    constexpr int U = 12;
    int c = chunk_of(s_off, nch, (uint32_t)i0);
    for (int b0 = i0; b0 < i1; b0 += U) {
      Entry e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = b0 + u;
        if (i < i1) {
          while (s_off[c + 1] <= (uint32_t)i) ++c;
          e[u] = band[(size_t)c * kCmpChunk + (i - s_off[c])];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = b0 + u;
        if (i < i1) {
          s_key[i] = sortable(e[u].s);
          s_cand[i] = e[u].cand;
        }
      }
    }
  }
  lds_barrier();
  auto key = [&](int i) { return in_lds ? s_key[i] : sortable(entry_at(i).s); };
  auto cand_of = [&](int i) { return in_lds ? s_cand[i] : entry_at(i).cand; };

  // uncertain members in position order: count per segment, scan, collect keys
  uint32_t cu = 0;
  for (int i = i0; i < i1; ++i) cu += (cand_of(i) & kCertain) ? 0u : 1u;
  uint32_t nu;
  const uint32_t u_first = wg_exclusive_scan<NT>(cu, s_tmp, &nu);
  const int nin = n2 - (int)nu;
  const int need = K - nin;
  const bool take_none = need <= 0;
  const bool take_all = !take_none && (int)nu <= need;
  const bool cut = !take_all && !take_none;
  const bool u_lds = (int)nu <= kUncLds - 4;
  // up to kRankMax uncertain members: rank each against all (larger exact
  // score first, then lower position, i.e. lower index in this list)
  const bool pairwise = cut && (int)nu <= kRankMax;
  if (cut && u_lds) {
    uint32_t uo = u_first;
    for (int i = i0; i < i1; ++i)
      if (!(cand_of(i) & kCertain)) {
        if (pairwise) s_ucomp[uo] = ((uint64_t)key(i) << 32) | (uint64_t)(0xFFFFFFFFu - uo);
        else s_ukey[uo] = key(i);
        ++uo;
      }
    if (pairwise && tid < 4) s_ucomp[nu + tid] = 0;   // padding: below every member
  }
  if (pairwise)
    for (int i = tid; i < (int)nu; i += NT) s_rank[i] = 0;
  lds_barrier();
  uint32_t kth = 0, ties = 0;
  if (pairwise) {
    // composite (key, complement of the list index): a larger composite is a
    // larger exact score, or an equal one at a lower position; all distinct.
    // The list is cut into R slices of four-entry groups and thread t counts
    // the composites above member t % nu in slice t / nu, so that about all
    // NT threads share the nu * nu comparisons.
    const int ng = ((int)nu + 3) >> 2;                  // four-entry groups
    const int R = max(1, min(NT / (int)nu, ng));        // slices
    const int gps = (ng + R - 1) / R;                   // groups per slice
    if (tid < R * (int)nu) {
      const int i = tid % (int)nu, sl = tid / (int)nu;
      const uint64_t ci = s_ucomp[i];
      const int j0 = 4 * sl * gps, j1 = min(4 * ng, j0 + 4 * gps);
      uint32_t r = 0;
      for (int j = j0; j < j1; j += 4) {
        const uint64_t c0 = s_ucomp[j], c1 = s_ucomp[j + 1], c2 = s_ucomp[j + 2], c3 = s_ucomp[j + 3];
        r += (c0 > ci ? 1u : 0u) + (c1 > ci ? 1u : 0u) + (c2 > ci ? 1u : 0u) + (c3 > ci ? 1u : 0u);
      }
      if (r) atomicAdd(&s_rank[i], r);
    }
    lds_barrier();
  } else if (cut) {
    if (u_lds) {
      kth = wg_kth_largest<NT>((int)nu, need, [&](int i) { return s_ukey[i]; }, s_hist, s_tmp, &ties);
    } else {
      // degenerate: many uncertain members; select over the band, certain ones count as ineligible
      kth = wg_kth_largest<NT>(n2, need, [&](int i) { return (cand_of(i) & kCertain) ? 0u : key(i); },
                               s_hist, s_tmp, &ties);
    }
  }
  // Radix-select path: pass 1 counts the entries tied at the cut, pass 2 the
  // kept ones, pass 3 writes; a tied entry's rank among tied entries follows
  // position order, so the lower positions win the ties.
  auto decide = [&](int i, uint32_t& u, uint32_t& rank) {
    const uint32_t c = cand_of(i);
    if (c & kCertain) return true;
    const uint32_t ui = u++;
    if (take_none) return false;
    if (take_all) return true;
    if (pairwise) return s_rank[ui] < (uint32_t)need;
    const uint32_t kk = key(i);
    if (kk > kth) return true;
    if (kk == kth) return rank++ < ties;
    return false;
  };
  uint32_t nt = 0;
  if (cut && !pairwise)
    for (int i = i0; i < i1; ++i) nt += (!(cand_of(i) & kCertain) && key(i) == kth) ? 1u : 0u;
  uint32_t tot_t;
  const uint32_t tie_base = wg_exclusive_scan<NT>(nt, s_tmp, &tot_t);
  uint32_t cnt = 0, rank = tie_base, u = u_first;
  for (int i = i0; i < i1; ++i) cnt += decide(i, u, rank) ? 1u : 0u;
  uint32_t tot;
  uint32_t o = wg_exclusive_scan<NT>(cnt, s_tmp, &tot);
  rank = tie_base;
  u = u_first;
  for (int i = i0; i < i1; ++i) {
    if (decide(i, u, rank)) {
      const uint32_t cand = cand_of(i) & ~kCertain;
      out[o++] = (kind == 1) ? (int)cand : cand_pos(P, q, kind, cand);
    }
  }
  for (int i = (int)tot + tid; i < K; i += NT) out[i] = -1;
}

// ---------------------------------------------------------------- 7. small problems
// A problem with at most kSmallMax candidates (a Reindex layer's pool) is
// selected by one work-group per query that holds every approximate score:
// thread t owns the contiguous slots [32 t, 32 t + 32), keys in registers.  A
// radix select gives the K-th approximate score a_K exactly, and a_K1 (the
// (K+1)-th) from its tie count; every exact Top-K member has approximate score
// >= a_K - 2 Delta and a member above a_K1 + 2 Delta is certainly in (at most K
// members have approximate score > a_K1, and only they can reach its exact
// score).  The members in between are rescored with the exact fp32 chains
// (one wave per member, one lane per head); among them the final choice is by
// (exact score desc, position asc).  Slots are in position order (pool blocks
// ascending), so a prefix sum over the threads' segments places the output.
constexpr int kSmallMax = 16384;
constexpr int kSmallThreads = 512;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallPer = kSmallMax / kSmallThreads;   // slots per thread

// Exclusive prefix sum over the 512-thread work-group (s_tmp: >= 8 entries).
__device__ __forceinline__ uint32_t wg8_exclusive_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t x = wave_incl_scan_u32(v);
  if (lane == 63) s_tmp[wave] = x;
  lds_barrier();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSmallWaves; ++i) {
    const uint32_t t = s_tmp[i];
    if (i < wave) before += t;
    all += t;
  }
  lds_barrier();
  *total = all;
  return before + x - v;
}

// K-th largest of the register keys for which elig(key) holds (1 <= K <=
// their count): most-significant-digit radix select, 8-bit digits starting at
// the highest bit where the smallest and largest eligible key differ; one
// 256-bin histogram per wave.  *ties = how many keys equal to the result
// belong to the Top-K, *eq = how many eligible keys equal it.
//
// With stop_bits > 0 the search may end once at most stop_bits low bits are
// undetermined: the result r then satisfies r <= K-th largest <= r | *span
// (*span = the undetermined low-bit mask; 0 when exact), and *ties / *eq are
// not meaningful.
template <typename Elig>
__device__ uint32_t small_kth(const uint32_t key[kSmallPer], Elig elig, int K, uint32_t* s_h /*8*256*/,
                              uint32_t* s_tmp /*>= 24*/, uint32_t* ties, uint32_t* eq, int stop_bits = 0,
                              uint32_t* span = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, c = 0;
#pragma unroll
  for (int j = 0; j < kSmallPer; ++j) {
    const bool e = elig(key[j]);
    lo = e ? min(lo, key[j]) : lo;
    hi = e ? max(hi, key[j]) : hi;
    c += e ? 1u : 0u;
  }
  lo = wave_min_u32(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    s_tmp[wave] = lo;
    s_tmp[8 + wave] = hi;
  }
  lds_barrier();
  lo = 0xFFFFFFFFu;
  hi = 0u;
#pragma unroll
  for (int i = 0; i < kSmallWaves; ++i) {
    lo = min(lo, s_tmp[i]);
    hi = max(hi, s_tmp[8 + i]);
  }
  lds_barrier();
  if (span) *span = 0u;
  if (lo == hi) {
    uint32_t tot;
    (void)wg8_exclusive_scan(c, s_tmp, &tot);
    *ties = (uint32_t)K;
    *eq = tot;
    return lo;
  }
  const int top = 31 - __clz(lo ^ hi);
  uint32_t mask = top == 31 ? 0u : (0xFFFFFFFFu << (top + 1));
  uint32_t prefix = lo & mask;
  uint32_t remaining = (uint32_t)K;
  uint32_t cnt_digit = 0;
  for (int shift = top - 7;; shift -= 8) {
    const int sh = shift < 0 ? 0 : shift;
    const int width = shift < 0 ? 8 + shift : 8;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = tid; i < kSmallWaves * 256; i += kSmallThreads) s_h[i] = 0;
    lds_barrier();
    uint32_t* h = s_h + wave * 256;
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j)
      if (elig(key[j]) && (key[j] & mask) == prefix) atomicAdd(&h[(key[j] >> sh) & dmask], 1u);
    lds_barrier();
    // thread tid < 256 owns digit 255 - tid; the exclusive scan counts larger digits
    uint32_t v = 0;
    const int dg = 255 - tid;
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < kSmallWaves; ++w) v += s_h[w * 256 + dg];
    }
    uint32_t tot;
    const uint32_t excl = wg8_exclusive_scan(v, s_tmp, &tot);
    if (tid < 256 && excl < remaining && excl + v >= remaining) {
      s_tmp[16] = (uint32_t)dg;
      s_tmp[17] = excl;
      s_tmp[18] = v;
    }
    lds_barrier();
    const uint32_t d = s_tmp[16];
    remaining -= s_tmp[17];
    cnt_digit = s_tmp[18];
    prefix |= d << sh;
    mask |= dmask << sh;
    lds_barrier();
    if (sh == 0) break;
    if (sh <= stop_bits) {
      *span = (1u << sh) - 1u;
      return prefix;
    }
  }
  *ties = remaining;
  *eq = cnt_digit;   // the last digit's bucket holds exactly the keys equal to the result
  return prefix;
}

// Slot states in the key registers: 0 = no candidate or out of the band,
// kSure = certainly selected, anything else = a key to be ranked.
constexpr uint32_t kSure = 0xFFFFFFFFu;   // above every finite score's sortable key

constexpr int kPend = 4096;      // keys near the K-th that the fast path keeps in LDS
constexpr int kPairMax = 256;    // pending keys ranked pairwise (larger lists: radix select)
constexpr int kRsMembers = 4;    // uncertain members one wave rescores at a time

template <int D>
__global__ __launch_bounds__(kSmallThreads) void k_select_small(Params P) {
  // One buffer, two layouts: the general path's per-slot arrays, or the fast
  // path's list of pending keys (those near the K-th approximate score)
  __shared__ __attribute__((aligned(16))) uint32_t s_big[kSmallMax + kSmallMax / 2];
  uint32_t* s_key = s_big;                                                   // general: exact keys by slot
  uint16_t* s_ul = reinterpret_cast<uint16_t*>(s_big + kSmallMax);           // general: uncertain slots
  uint32_t* s_pk = s_big;                                                    // fast: pending keys (exact once rescored)
  uint16_t* s_ps = reinterpret_cast<uint16_t*>(s_big + kPend);               // fast: pending slots
  uint16_t* s_pu = reinterpret_cast<uint16_t*>(s_big + kPend + kPend / 2);   // fast: uncertain pending indices
  uint8_t* s_pst = reinterpret_cast<uint8_t*>(s_big + 2 * kPend);            // fast: pending states
  __shared__ __attribute__((aligned(16))) float s_kf[kSmallWaves][kRsMembers][D];   // member keys being rescored
  __shared__ __attribute__((aligned(16))) float s_r[kSmallWaves][kRsMembers][kWave];
  __shared__ int32_t s_pool[kSmallMax / 8];
  __shared__ uint32_t s_h[kSmallWaves * 256];
  __shared__ uint32_t s_selw[kSmallThreads];   // fast path: chosen pending slots, one word per thread
  __shared__ uint32_t s_tmp[32];
  __shared__ float s_par[4];
  __shared__ __attribute__((aligned(16))) float s_w[kWave];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = blockIdx.x;
  const int K = P.k;
  const int nc = 8 * P.keep_in;
  s_selw[tid] = 0;
  const int64_t base = seq_base_of(P, q);
  const float* sc = P.scores + (size_t)q * P.stride;
  int32_t* out = P.idx_out + (size_t)q * K;
  const int s0 = tid * kSmallPer;   // this thread's first slot

  // every load of the prologue is issued before any of them is used; indices
  // are clamped so that no load is conditional
  const int nwg = (nc + P.scan_chunk - 1) / P.scan_chunk;   // <= 64
  float4 raw[kSmallPer / 4];
#pragma unroll
  for (int j4 = 0; j4 < kSmallPer / 4; ++j4)
    raw[j4] = *reinterpret_cast<const float4*>(sc + min(s0 + 4 * j4, nc - 4));   // nc is a multiple of 8
  int32_t praw[kSmallMax / 8 / kSmallThreads];
#pragma unroll
  for (int k = 0; k < kSmallMax / 8 / kSmallThreads; ++k)
    praw[k] = P.pool_in ? P.pool_in[(size_t)q * P.keep_in + min(tid + kSmallThreads * k, P.keep_in - 1)]
                        : min(tid + kSmallThreads * k, P.keep_in - 1);
  const float wraw = P.w[(size_t)q * P.h_i + min(tid & 63, P.h_i - 1)];
  const float kraw = P.kpart[(size_t)q * nwg + min(tid & 63, nwg - 1)];

  // approximate scores -> sortable keys in registers (0: no candidate); the
  // smallest and largest key and their count
  uint32_t key[kSmallPer];
  uint32_t klo = 0xFFFFFFFFu, khi = 0u, nv_loc = 0;
#pragma unroll
  for (int j4 = 0; j4 < kSmallPer / 4; ++j4) {
    const bool in = s0 + 4 * j4 < nc;
    const float vv[4] = {raw[j4].x, raw[j4].y, raw[j4].z, raw[j4].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = in && vv[u] != -INFINITY;
      const uint32_t k = ok ? sortable(vv[u]) : 0u;
      key[4 * j4 + u] = k;
      klo = ok ? min(klo, k) : klo;
      khi = max(khi, k);
      nv_loc += ok ? 1u : 0u;
    }
  }
  // the smallest of the threads' largest keys: at least kSmallThreads keys
  // (one per thread) are >= it, so for K <= kSmallThreads it is <= the K-th
  // largest key and the histogram below needs only the keys above it
  uint32_t tmin = 0u;
#pragma unroll
  for (int j = 0; j < kSmallPer; ++j) tmin = max(tmin, key[j]);
  klo = wave_min_dpp(klo);
  khi = wave_max_dpp(khi);
  nv_loc = wave_sum_dpp(nv_loc);
  tmin = wave_min_dpp(tmin);
  if (lane == 0) {
    s_tmp[wave] = klo;
    s_tmp[8 + wave] = khi;
    s_tmp[16 + wave] = nv_loc;
    s_tmp[24 + wave] = tmin;
  }
#pragma unroll
  for (int k = 0; k < kSmallMax / 8 / kSmallThreads; ++k)
    if (tid + kSmallThreads * k < nc / 8) s_pool[tid + kSmallThreads * k] = praw[k];
  if (tid < kWave) s_w[tid] = tid < P.h_i ? wraw : 0.0f;
  // rounding bound Delta = C * max t_k over the pool's keys (the scan's
  // work-groups each left the largest key magnitude they saw), as the
  // multi-kernel path
  if (wave == 0) {
    const uint32_t mk = wave_max_dpp(lane < nwg ? __float_as_uint(kraw) : 0u);   // non-negative floats order as integers
    const float wa = wave_sum(fabsf(wraw) * (lane < P.h_i ? 1.0f : 0.0f));
    if (lane == 0)
      s_par[0] = P.bound_tok * __uint_as_float(mk) * (1.0f + 0.0009765625f) + wa * (float)P.d_i * 7.8886e-31f;
  }
  lds_barrier();   // every wave's range and count, the pool ids, the weights
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, nv = 0, floor_k = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kSmallWaves; ++i) {
    lo = min(lo, s_tmp[i]);
    hi = max(hi, s_tmp[8 + i]);
    nv += s_tmp[16 + i];
    floor_k = min(floor_k, s_tmp[24 + i]);
  }
  // (a thread without candidates has largest key 0, which disables the floor)
  if (K <= kSmallThreads && floor_k != 0u && floor_k > lo) lo = floor_k;
  lds_barrier();   // publishes s_par; s_tmp is free again
  const float delta = s_par[0];

  auto is_real = [](uint32_t k) { return k != 0u && k != kSure; };
  uint32_t sel = 0;   // bit j: slot s0 + j is selected
  // ---- fast path: a linear histogram of the values, then only the keys near
  // the K-th (a short list in LDS) are examined further
  const float vlo = unsortable(lo), vhi = unsortable(hi);
  const float rng = vhi - vlo;
  const bool linear = (int)nv > K && lo != hi && rng >= 1e-30f && rng <= 3.0e38f;
  bool fast = false;
  int np = 0, n_cert = 0, p_first = 0;
  uint32_t pend = 0;   // bit j: slot s0 + j is pending
  if (linear) {
    const float scale = 256.0f / rng;
    // bin of a key: monotone in the value (each rounding step is monotone)
    auto lbin = [vlo, scale](uint32_t k) { return (uint32_t)fminf((unsortable(k) - vlo) * scale, 255.0f); };
    for (int i = tid; i < kSmallWaves * 256; i += kSmallThreads) s_h[i] = 0;
    lds_barrier();
    uint32_t* hw = s_h + wave * 256;
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j)
      if (key[j] >= lo && key[j] != 0u) atomicAdd(&hw[lbin(key[j])], 1u);
    lds_barrier();
    // thread tid < 256 owns bin 255 - tid; the exclusive scan counts higher bins
    uint32_t v = 0;
    const int dg = 255 - tid;
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < kSmallWaves; ++w) v += s_h[w * 256 + dg];
    }
    uint32_t tot;
    const uint32_t excl = wg8_exclusive_scan(v, s_tmp, &tot);
    if (tid < 256 && excl < (uint32_t)K && excl + v >= (uint32_t)K) s_tmp[24] = (uint32_t)dg;
    lds_barrier();
    const uint32_t bk = s_tmp[24];
    // [e_lo, e_hi] holds every value of bin bk (the bin's edges widened by far
    // more than the rounding of the bin computation), so e_lo <= a_K <= e_hi:
    // a key below band_below(e_lo) is out, one above band_above(e_hi) is
    // certainly in, whatever a_K is inside the bin; the rest is pending.  The
    // comparisons run on the sortable keys, which order as the values do.
    const float wdt = rng * 0.00390625f;
    const float slack = (fabsf(vlo) + fabsf(vhi)) * 6.103515625e-05f + wdt * 0.0078125f;
    const float e_lo = bk == 0 ? vlo : vlo + (float)bk * wdt - slack;
    const float e_hi = bk == 255 ? vhi : vlo + (float)(bk + 1) * wdt + slack;
    const uint32_t k_keep0 = sortable(band_below(e_lo, delta)), k_in0 = sortable(band_above(e_hi, delta));
    uint32_t cert = 0;
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j) {
      const uint32_t k = key[j];   // 0 (no candidate) is below every finite threshold's key
      cert |= (k > k_in0 ? 1u : 0u) << j;
      pend |= (k >= k_keep0 && k <= k_in0 ? 1u : 0u) << j;
    }
    uint32_t all;
    const uint32_t before = wg8_exclusive_scan(__popc(pend) | ((uint32_t)__popc(cert) << 16), s_tmp, &all);
    np = (int)(all & 0xFFFFu);
    n_cert = (int)(all >> 16);
    p_first = (int)(before & 0xFFFFu);
    fast = np <= kPend;
    if (fast) {
      sel = cert;
      int po = p_first;
#pragma unroll
      for (int j = 0; j < kSmallPer; ++j) {
        if ((pend >> j) & 1u) {
          s_pk[po] = key[j];
          s_ps[po] = (uint16_t)(s0 + j);
          ++po;
        }
      }
    }
  }

  // the query row of head `lane` for the rescoring (packed bf16 pairs): its
  // loads overlap the selection steps below
  constexpr int DW = D / 2;
  uint32_t qrow[DW];
  {
    const uint4* src = reinterpret_cast<const uint4*>(P.iq + ((size_t)q * P.h_i + min(lane, P.h_i - 1)) * D);
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
      const uint4 v = src[i];
      qrow[4 * i] = v.x;
      qrow[4 * i + 1] = v.y;
      qrow[4 * i + 2] = v.z;
      qrow[4 * i + 3] = v.w;
    }
  }

  int nu = 0, need = 0;
  if (fast) {
    if (np <= kPairMax && tid < 8) s_pk[np + tid] = 0u;   // padding for four-wide reads (0: below every key)
    lds_barrier();
    // a_K exactly: the (K - n_cert)-th largest pending key (keys above the
    // pending range are above a_K, keys below it below, and a_K is pending)
    const int kp = K - n_cert;
    uint32_t kK;
    if (np <= kPairMax) {
      // pairwise: entry i holds it when (#keys > key_i) < kp <= (#keys >= key_i).
      // Threads t = i + npr * sl count slice sl of the list for entry i; the
      // counts gather in s_h (greater: [0, 256), greater or equal: [256, 512))
      const int npr = (np + 63) & ~63;                 // entries rounded to whole waves
      const int R = kSmallThreads / npr;               // slices: 2 .. 8
      const int per = ((np + R - 1) / R + 3) & ~3;     // list entries per slice, four-aligned
      if (tid < 512) s_h[tid] = 0;
      lds_barrier();
      const int i = tid % npr, sl = tid / npr;
      if (i < np && sl < R) {
        const uint32_t ki = s_pk[i];
        uint32_t gt = 0, ge = 0;
        const int j0 = sl * per, j1 = min(np, j0 + per);
        for (int j = j0; j < j1; j += 4) {   // entries past np read the zero padding
          const uint4 k4 = *reinterpret_cast<const uint4*>(&s_pk[j]);
          gt += (k4.x > ki ? 1u : 0u) + (k4.y > ki ? 1u : 0u) + (k4.z > ki ? 1u : 0u) + (k4.w > ki ? 1u : 0u);
          ge += (k4.x >= ki ? 1u : 0u) + (k4.y >= ki ? 1u : 0u) + (k4.z >= ki ? 1u : 0u) + (k4.w >= ki ? 1u : 0u);
        }
        if (gt) atomicAdd(&s_h[i], gt);
        if (ge) atomicAdd(&s_h[256 + i], ge);
      }
      lds_barrier();
      if (tid < np && s_h[tid] < (uint32_t)kp && (uint32_t)kp <= s_h[256 + tid]) s_tmp[24] = s_pk[tid];   // one key
      lds_barrier();
      kK = s_tmp[24];
    } else {
      uint32_t ties;
      kK = wg_kth_largest<kSmallThreads>(np, kp, [&](int i) { return s_pk[i]; }, s_h, s_tmp, &ties);
    }
    // classify the pending keys against the exact bracket [a_K, a_K]; the
    // uncertain ones are listed in pending (= slot) order
    const uint32_t k_keep1 = sortable(band_below(unsortable(kK), delta));
    const uint32_t k_in1 = sortable(band_above(unsortable(kK), delta));
    const int ppt = (np + kSmallThreads - 1) / kSmallThreads;
    const int i0 = min(np, tid * ppt), i1 = min(np, i0 + ppt);
    uint32_t c2 = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = s_pk[i];
      const uint8_t st = k < k_keep1 ? 0 : (k > k_in1 ? 1 : 2);
      s_pst[i] = st;
      c2 += st == 1 ? 0x10000u : (st == 2 ? 1u : 0u);
    }
    uint32_t all;
    uint32_t uo = wg8_exclusive_scan(c2, s_tmp, &all) & 0xFFFFu;
    nu = (int)(all & 0xFFFFu);
    need = K - (n_cert + (int)(all >> 16));
    for (int i = i0; i < i1; ++i)
      if (s_pst[i] == 2) s_pu[uo++] = (uint16_t)i;
    lds_barrier();
  } else {
    // ---- general path: bracket the K-th approximate score by a radix select
    // over all register keys (L <= a_K and U >= a_K >= a_K1, the last 8 bits of
    // the key -- 2^-15 of the value -- left open)
    if ((int)nv > K) {
      uint32_t ties, eq, span;
      const uint32_t kL = small_kth(key, is_real, K, s_h, s_tmp, &ties, &eq, 8, &span);
      const uint32_t kK = kL, kK1 = kL | span;
      const float keep_thr = band_below(unsortable(kK), delta);    // L - 2 Delta
      const float in_thr = band_above(unsortable(kK1), delta);     // U + 2 Delta
#pragma unroll
      for (int j = 0; j < kSmallPer; ++j) {
        const float v = unsortable(key[j]);
        key[j] = key[j] == 0u || !(v >= keep_thr) ? 0u : (v > in_thr ? kSure : key[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSmallPer; ++j) key[j] = key[j] != 0u ? kSure : 0u;
    }
    // uncertain list (slot order)
    uint32_t cu = 0, ci = 0;
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j) {
      cu += is_real(key[j]) ? 1u : 0u;
      ci += key[j] == kSure ? 1u : 0u;
      sel |= (key[j] == kSure ? 1u : 0u) << j;
    }
    uint32_t all;
    uint32_t uo = wg8_exclusive_scan(cu | (ci << 16), s_tmp, &all) & 0xFFFFu;
    nu = (int)(all & 0xFFFFu);
    need = K - (int)(all >> 16);
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j)
      if (is_real(key[j])) s_ul[uo++] = (uint16_t)(s0 + j);
    lds_barrier();
  }
  // member j of the uncertain list: its slot, and where its exact key goes
  auto u_slot = [&](int j) -> int { return fast ? (int)s_ps[s_pu[j]] : (int)s_ul[j]; };
  auto u_store = [&](int j, uint32_t k) {
    if (fast) s_pk[s_pu[j]] = k;
    else s_key[s_ul[j]] = k;
  };
  auto u_exact = [&](int j) -> uint32_t { return fast ? s_pk[s_pu[j]] : s_key[s_ul[j]]; };

  // exact scores of the uncertain members, kRsMembers per wave at a time, one
  // lane per head: the members' key rows are staged in LDS as fp32 and read
  // back as broadcasts, the lane's query row sits in registers; the head sums
  // run one member per lane.  Rows h >= h_i compute a finite throwaway value.
  const bool choose = nu > 0 && need > 0 && nu > need;   // otherwise no ranking is needed
  if (choose) {
    // each batch's key rows are loaded while the previous batch is computed
    uint32_t kw[kRsMembers];
    auto load_batch = [&](int j0) {
      const int nm = min(kRsMembers, nu - j0);
#pragma unroll
      for (int m = 0; m < kRsMembers; ++m) {
        const int slot = u_slot(j0 + min(m, nm - 1));
        const int64_t row = base + (int64_t)s_pool[slot >> 3] * 8 + (slot & 7);
        kw[m] = key_pair<D>(P, row, lane < DW ? lane : 0);
      }
    };
    if (wave * kRsMembers < nu) load_batch(wave * kRsMembers);
    for (int jb = wave * kRsMembers; jb < nu; jb += kSmallWaves * kRsMembers) {
      const int nm = min(kRsMembers, nu - jb);
#pragma unroll
      for (int m = 0; m < kRsMembers; ++m)
        if (lane < DW)
          *reinterpret_cast<f32x2*>(&s_kf[wave][m][2 * lane]) =
              f32x2{__uint_as_float(kw[m] << 16), __uint_as_float(kw[m] & 0xFFFF0000u)};
      if (jb + kSmallWaves * kRsMembers < nu) load_batch(jb + kSmallWaves * kRsMembers);
      // per head h = lane: fp32 fma chains over d ascending (the oracle's order)
      float acc[kRsMembers];
#pragma unroll
      for (int m = 0; m < kRsMembers; ++m) acc[m] = 0.0f;
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const float q0 = __uint_as_float(qrow[2 * d4] << 16), q1 = __uint_as_float(qrow[2 * d4] & 0xFFFF0000u);
        const float q2 = __uint_as_float(qrow[2 * d4 + 1] << 16), q3 = __uint_as_float(qrow[2 * d4 + 1] & 0xFFFF0000u);
#pragma unroll
        for (int m = 0; m < kRsMembers; ++m) {
          const f32x4 kv = *reinterpret_cast<const f32x4*>(&s_kf[wave][m][4 * d4]);
          acc[m] = fmaf(q0, kv.x, acc[m]);
          acc[m] = fmaf(q1, kv.y, acc[m]);
          acc[m] = fmaf(q2, kv.z, acc[m]);
          acc[m] = fmaf(q3, kv.w, acc[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < kRsMembers; ++m) s_r[wave][m][lane] = acc[m] > 0.0f ? acc[m] : 0.0f;
      // ordered head sum s = fma(w_h, r_h, s), h ascending, member m in lane m;
      // entries h >= h_i hold w = 0 and a finite r, which leave s unchanged
      if (lane < kRsMembers) {
        const float* rr = &s_r[wave][lane][0];
        float sv = 0.0f;
#pragma unroll 4
        for (int h4 = 0; h4 < 16; ++h4) {
          const f32x4 wv = *reinterpret_cast<const f32x4*>(&s_w[4 * h4]);
          const f32x4 r4 = *reinterpret_cast<const f32x4*>(rr + 4 * h4);
          sv = fmaf(wv.x, r4.x, sv);
          sv = fmaf(wv.y, r4.y, sv);
          sv = fmaf(wv.z, r4.z, sv);
          sv = fmaf(wv.w, r4.w, sv);
        }
        if (lane < nm) u_store(jb + lane, sortable(sv));
      }
    }
  }
  lds_barrier();

  // final choice among the uncertain members: the best `need` by (exact score
  // desc, position asc).  u_decide records a member's decision where the
  // write-back below finds it.
  auto u_decide = [&](int j, bool take) {
    if (fast) s_pst[s_pu[j]] = take ? 1 : 0;
    else s_key[s_ul[j]] = take ? kSure : 0u;
  };
  if (!choose) {
    for (int jj = tid; jj < nu; jj += kSmallThreads) u_decide(jj, need > 0);   // all in, or all out
  } else if (nu <= kWave) {
    // one wave ranks (exact key, complement of slot) composites pairwise
    if (wave == 0) {
      uint64_t comp = 0;
      if (lane < nu) comp = ((uint64_t)u_exact(lane) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)u_slot(lane));
      uint32_t r = 0;
      for (int jj = 0; jj < nu; ++jj) {
        const uint32_t clo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)comp, jj);
        const uint32_t chi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(comp >> 32), jj);
        r += ((((uint64_t)chi << 32) | clo) > comp) ? 1u : 0u;
      }
      if (lane < nu) u_decide(lane, r < (uint32_t)need);
    }
  } else {
    // radix select on the exact keys; ties at the cut go to the lower slots
    // (the list is in slot order).  Keys are kept inside [1, kSure - 1].
    auto xk = [&](int i) { return min(max(u_exact(i), 1u), kSure - 1u); };
    uint32_t ties;
    const uint32_t kth = wg_kth_largest<kSmallThreads>(nu, need, xk, s_h, s_tmp, &ties);
    const int upt = (nu + kSmallThreads - 1) / kSmallThreads;
    const int j0 = min(nu, tid * upt), j1 = min(nu, j0 + upt);
    uint32_t tl = 0;
    for (int jj = j0; jj < j1; ++jj) tl += xk(jj) == kth ? 1u : 0u;
    uint32_t ttot;
    uint32_t tr = wg8_exclusive_scan(tl, s_tmp, &ttot);
    for (int jj = j0; jj < j1; ++jj) {
      const uint32_t k = xk(jj);
      const bool tie = k == kth;
      u_decide(jj, k > kth || (tie && tr < ties));
      tr += tie ? 1u : 0u;
    }
  }
  lds_barrier();
  // decisions into the selection mask
  if (fast) {
    // chosen pending entries set their slot's bit in the owning thread's word
    // (slot s lives in thread s / 32, bit s % 32)
    for (int i = tid; i < np; i += kSmallThreads)
      if (s_pst[i] == 1) {
        const uint32_t slot = s_ps[i];
        atomicOr(&s_selw[slot >> 5], 1u << (slot & 31));
      }
    lds_barrier();
    sel |= s_selw[tid];
  } else {
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j)
      if (is_real(key[j])) sel |= (s_key[s0 + j] == kSure ? 1u : 0u) << j;
  }
  // selected slots in position order: a prefix sum over the threads' segments
  uint32_t tot;
  uint32_t o = wg8_exclusive_scan((uint32_t)__popc(sel), s_tmp, &tot);
  for (uint32_t m = sel; m; m &= m - 1) {
    const int slot = s0 + __builtin_ctz(m);
    out[o++] = s_pool[slot >> 3] * 8 + (slot & 7);
  }
  for (int i = (int)tot + tid; i < K; i += kSmallThreads) out[i] = -1;
}

}  // namespace idx
}  // namespace csa2

// ======================================================================
// Host side
// ======================================================================
using namespace csa2;
using namespace csa2::idx;

namespace {

// Keys per scan work-group: the largest power of two up to kMaxScanChunk that
// still gives at least two work-groups per CU (512), down to 1024 keys, so
// that short contexts (or the block keys of the pool-based variant) still fill
// the 256 CUs.
int scan_chunk_for(int n_q, int64_t max_nvis) {
  int chunk = kMaxScanChunk;
  while (chunk > 1024 && (int64_t)n_q * ((max_nvis + chunk - 1) / chunk) < 512) chunk >>= 1;
  return chunk;
}

// Pool slots per Reindex scan work-group: 256, doubled up to 2048 while that
// still leaves at least 512 work-groups (large batches amortise each
// work-group's query load and bound setup over more keys).
int reindex_chunk_for(int n_q, int64_t slots) {
  int chunk = 256;
  while (chunk < 2048 && (int64_t)n_q * ((slots + 2 * chunk - 1) / (2 * chunk)) >= 512) chunk <<= 1;
  return chunk;
}

thread_local hipEvent_t g_scan_ev_start = nullptr;
thread_local hipEvent_t g_scan_ev_stop = nullptr;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t scores, hist, hist2, meta, chunk_cnt, chunk_unc, band, unc, kpart, gkey, total;
};

Layout make_layout(int nprob, int64_t stride, int nchunk_cmp) {
  Layout L;
  size_t o = 0;
  L.scores = o;
  o = align256(o + (size_t)nprob * stride * sizeof(float));
  L.hist = o;
  o = align256(o + (size_t)nprob * kNBins * sizeof(uint32_t));
  L.hist2 = o;
  o = align256(o + (size_t)nprob * kNBins * sizeof(uint32_t));
  L.meta = o;
  o = align256(o + (size_t)nprob * sizeof(Meta));
  L.chunk_cnt = o;
  o = align256(o + (size_t)nprob * nchunk_cmp * sizeof(uint32_t));
  L.chunk_unc = o;
  o = align256(o + (size_t)nprob * nchunk_cmp * sizeof(uint32_t));
  L.band = o;
  o = align256(o + (size_t)nprob * stride * sizeof(Entry));
  L.unc = o;
  o = align256(o + (size_t)nprob * stride * sizeof(uint2));
  L.kpart = o;   // one float per Reindex scan work-group (256 slots each)
  o = align256(o + (size_t)nprob * (size_t)(stride / 256) * sizeof(float));
  L.gkey = o;    // 16 bits per 16 scores
  o = align256(o + (size_t)nprob * (size_t)(stride / 16) * sizeof(uint16_t));
  L.total = o;
  return L;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

double gamma_n(double n, double u) { return n * u / (1.0 - n * u); }

// Delta = C * max_k t_k.  Per head, the exact fp32 chain (unit roundoff 2^-24)
// and any MFMA accumulation order or truncation (2^-23) of the d_i-term dot
// products each err by at most gamma * sum_d |q_hd k_d|; weighted by |w_h|
// and summed over heads this is gamma * t_k, to which the two head sums' and,
// for blocks, the 8-term member sums' and the division's roundings add.  C
// covers all of these, doubled for safety.
float bound_constant(int d_i, bool block) {
  const double u = std::ldexp(1.0, -24), u2 = std::ldexp(1.0, -23);
  double e = gamma_n(d_i, u) + gamma_n(d_i + 2, u2);
  if (block) e += 2.0 * gamma_n(8, u) + 8.0 * u;
  const double gh = gamma_n(66, u);
  return (float)(2.0 * (e + gh * (2.0 + e)));
}

bool launch_ok() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_last_hip_error((int)e);
    return false;
  }
  return true;
}

template <int D, bool FP8>
void launch_scan_t(const Params& P, int mt, bool pool, bool indirect, bool hist, dim3 grid, hipStream_t s) {
#define CSA2_SCAN(MTV)                                                                                            \
  if (mt == MTV) {                                                                                                \
    if (indirect && hist) hipLaunchKernelGGL((k_scan<D, MTV, false, true, true, FP8>), grid, dim3(kThreads), 0, s, P); \
    else if (indirect) hipLaunchKernelGGL((k_scan<D, MTV, false, true, false, FP8>), grid, dim3(kThreads), 0, s, P);  \
    else if (pool) hipLaunchKernelGGL((k_scan<D, MTV, true, false, true, FP8>), grid, dim3(kThreads), 0, s, P);       \
    else hipLaunchKernelGGL((k_scan<D, MTV, false, false, true, FP8>), grid, dim3(kThreads), 0, s, P);                \
    return;                                                                                                       \
  }
  CSA2_SCAN(1) CSA2_SCAN(2) CSA2_SCAN(3) CSA2_SCAN(4)
#undef CSA2_SCAN
}

// FP8 keys are built for d_i = 128 only (the entry points check it).
template <int D>
void launch_scan(const Params& P, int mt, bool pool, bool indirect, bool hist, dim3 grid, hipStream_t s) {
  if constexpr (D == 128) {
    if (P.ik8) {
      launch_scan_t<D, true>(P, mt, pool, indirect, hist, grid, s);
      return;
    }
  }
  launch_scan_t<D, false>(P, mt, pool, indirect, hist, grid, s);
}

#ifndef CSA2_CHUNK_QB
#define CSA2_CHUNK_QB 2
#endif
constexpr int kChunkQB = CSA2_CHUNK_QB;   // queries per chunk-scan work-group

template <int D>
void launch_scan_chunk(const Params& P, int mt, dim3 grid, hipStream_t s) {
#define CSA2_SCANC(MTV) \
  if (mt == MTV) { hipLaunchKernelGGL((k_scan_chunk<D, MTV, kChunkQB>), grid, dim3(kThreads), 0, s, P); return; }
  CSA2_SCANC(1) CSA2_SCANC(2) CSA2_SCANC(3) CSA2_SCANC(4)
#undef CSA2_SCANC
}

csa2_status run_pipeline(Params P, int64_t max_slots, void* ws, size_t ws_bytes, hipStream_t s, size_t need,
                         bool chunk = false) {
  if (ws_bytes < need) return CSA2_E_WORKSPACE;
  const Layout L = make_layout(P.nprob, P.stride, P.nchunk_cmp);
  char* w = static_cast<char*>(ws);
  P.scores = reinterpret_cast<float*>(w + L.scores);
  P.hist = reinterpret_cast<uint32_t*>(w + L.hist);
  P.hist2 = reinterpret_cast<uint32_t*>(w + L.hist2);
  P.meta = reinterpret_cast<Meta*>(w + L.meta);
  P.chunk_cnt = reinterpret_cast<uint32_t*>(w + L.chunk_cnt);
  P.chunk_unc = reinterpret_cast<uint32_t*>(w + L.chunk_unc);
  P.band = reinterpret_cast<Entry*>(w + L.band);
  P.unc = reinterpret_cast<uint2*>(w + L.unc);
  P.kpart = reinterpret_cast<float*>(w + L.kpart);
  P.gkey = reinterpret_cast<uint16_t*>(w + L.gkey);
  // the selection's large mode pays once it has thousands of work-groups per
  // problem and reads gigabytes of scores (the encoder chunk: 4096 queries x
  // 512 K scores, 44.97 -> 43.99 ms per step); on a 64-query decode step
  // (256 MB) its two extra launches and round trips cost more than they save
  P.large_sel = (double)P.n_q * (double)P.stride * sizeof(float) >= kLargeSelBytes ? 1 : 0;
  P.bound_tok = bound_constant(P.d_i, false);
  P.bound_blk = bound_constant(P.d_i, true);

  const int mt = (P.h_i + 15) / 16;
  const bool pool = !P.reindex && P.keep_blocks > 0;
  if (P.reindex && 8 * P.keep_in <= kSmallMax) {
    // small problem: the scan, then one work-group per query selects in LDS
    const int nx = (int)std::max<int64_t>(1, (max_slots + P.scan_chunk - 1) / P.scan_chunk);
    hipEvent_t ev0 = g_scan_ev_start, ev1 = g_scan_ev_stop;
    g_scan_ev_start = g_scan_ev_stop = nullptr;
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return CSA2_E_HIP;
    if (P.d_i == 128) launch_scan<128>(P, mt, false, true, false, dim3(nx, P.n_q), s);
    else launch_scan<64>(P, mt, false, true, false, dim3(nx, P.n_q), s);
    if (!launch_ok()) return CSA2_E_HIP;
    if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return CSA2_E_HIP;
    if (P.d_i == 128) hipLaunchKernelGGL(k_select_small<128>, dim3(P.n_q), dim3(kSmallThreads), 0, s, P);
    else hipLaunchKernelGGL(k_select_small<64>, dim3(P.n_q), dim3(kSmallThreads), 0, s, P);
    if (!launch_ok()) return CSA2_E_HIP;
    return CSA2_OK;
  }
  if (P.d_i == 128) hipLaunchKernelGGL(k_prologue<128>, dim3(P.nprob), dim3(kThreads), 0, s, P);
  else hipLaunchKernelGGL(k_prologue<64>, dim3(P.nprob), dim3(kThreads), 0, s, P);
  if (!launch_ok()) return CSA2_E_HIP;
  const int nx = (int)std::max<int64_t>(1, (max_slots + P.scan_chunk - 1) / P.scan_chunk);
  const dim3 gscan(nx, P.n_q);
  hipEvent_t ev0 = g_scan_ev_start, ev1 = g_scan_ev_stop;
  g_scan_ev_start = g_scan_ev_stop = nullptr;
  if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return CSA2_E_HIP;
  if (chunk) {
    const dim3 gch((unsigned)((P.n_q + kChunkQB - 1) / kChunkQB),
                   (unsigned)std::max<int64_t>(1, (max_slots + kChunkKeys - 1) / kChunkKeys));
    if (P.d_i == 128) launch_scan_chunk<128>(P, mt, gch, s);
    else launch_scan_chunk<64>(P, mt, gch, s);
  } else if (P.d_i == 128) {
    launch_scan<128>(P, mt, pool, P.reindex, true, gscan, s);
  } else {
    launch_scan<64>(P, mt, pool, P.reindex, true, gscan, s);
  }
  if (!launch_ok()) return CSA2_E_HIP;
  if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return CSA2_E_HIP;
  // per-chunk kernels: the token (or Reindex) problem's chunks, then the block problem's
  const dim3 gchunk(P.nchunk_cmp + (pool ? (P.nchunk_cmp + 7) / 8 : 0), P.n_q);
  // the fine histogram in large mode without a block problem: kLargeChunks
  // chunks per work-group (its threads work alone; the compaction's chunks,
  // each a chain of dependent steps, keep a work-group each)
  const bool multi = P.large_sel && !pool;
  const dim3 gfine(multi ? (P.nchunk_cmp + kLargeChunks - 1) / kLargeChunks : gchunk.x, P.n_q);
  if (P.large_sel) {
    hipLaunchKernelGGL(k_coarse, dim3(P.nprob), dim3(kThreads), 0, s, P);
    if (!launch_ok()) return CSA2_E_HIP;
  }
  hipLaunchKernelGGL(k_finehist, gfine, dim3(kThreads), 0, s, P);
  if (!launch_ok()) return CSA2_E_HIP;
  if (P.large_sel) {
    hipLaunchKernelGGL(k_band, dim3(P.nprob), dim3(kThreads), 0, s, P);
    if (!launch_ok()) return CSA2_E_HIP;
  }
  if (P.large_sel) {
    const dim3 gwave((unsigned)((gchunk.x + kWaves - 1) / kWaves), P.n_q);   // one wave per chunk
    hipLaunchKernelGGL(k_compact_large, gwave, dim3(kThreads), 0, s, P);
  } else {
    hipLaunchKernelGGL(k_compact, gchunk, dim3(kThreads), 0, s, P);
  }
  if (!launch_ok()) return CSA2_E_HIP;
  // One resident round (three work-groups per CU at this kernel's register
  // and LDS use): about kRescoreWGs work-groups in all, a query's share split 1:7
  // between its token and block problems (blocks have about ten times more
  // undecided members, each eight chains).  Every wave strides over its
  // problem's members, so any split stays correct.  The block work-groups of
  // all queries share one member list when its chunk counts fit in LDS.
  const int per_q = std::min(128, std::max(pool ? 8 : 1, kRescoreWGs / P.n_q));
  P.rs_tok = pool ? std::max(1, per_q / 8) : per_q;
  P.rs_pool = pool && P.n_q <= kPoolMaxQ && (int64_t)P.n_q * ((P.nchunk_cmp + 7) >> 3) <= kMaxChunksLds ? 1 : 0;
  if (P.d_i == 128) hipLaunchKernelGGL(k_rescore<128>, dim3(per_q, P.n_q), dim3(kThreads), 0, s, P);
  else hipLaunchKernelGGL(k_rescore<64>, dim3(per_q, P.n_q), dim3(kThreads), 0, s, P);
  if (!launch_ok()) return CSA2_E_HIP;
  hipLaunchKernelGGL(k_final, dim3(P.nprob), dim3(kFinalThreads), 0, s, P);
  if (!launch_ok()) return CSA2_E_HIP;
  return CSA2_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool shape_ok(int h_i, int d_i) { return h_i >= 1 && h_i <= 64 && (d_i == 64 || d_i == 128); }

}  // namespace

extern "C" void csa2_record_scan_events(void* start, void* stop) {
  g_scan_ev_start = static_cast<hipEvent_t>(start);
  g_scan_ev_stop = static_cast<hipEvent_t>(stop);
}

extern "C" size_t csa2_index_topk_ws_bytes(int n_q, int32_t max_nvis, int h_i, int d_i, int k, int block,
                                           int keep_blocks) {
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

namespace {

// Keys of an index call: bf16 rows (ik) or FP8 rows with their exponent
// bytes (ik8, ik8e; d_i = 128 only).  Returns false when the pointers do not
// fit the contract.
bool keys_ok(int d_i, const uint16_t* ik, const uint8_t* ik8, const uint8_t* ik8e) {
  if (ik8) return d_i == 128 && ik8e && !ik && aligned(ik8, 8);
  return ik && !ik8e && aligned(ik, 16);
}

csa2_status index_call(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i, const int32_t* q_seq,
                       const int32_t* q_nvis, int32_t max_nvis, const uint16_t* ik, const uint8_t* ik8,
                       const uint8_t* ik8e, const int64_t* seq_base, int k, int32_t* idx_out, int block,
                       int keep_blocks, int32_t* pool_out, void* ws, size_t ws_bytes, void* stream) {
  csa2::set_last_hip_error(0);
  if (n_q < 0 || max_nvis < 0 || k < 1 || k > 2048 || keep_blocks < 0 || keep_blocks > 4096)
    return CSA2_E_INVAL;
  if ((int64_t)max_nvis > (int64_t)kMaxChunksLds * kCmpChunk) return CSA2_E_UNSUPPORTED;
  if (!shape_ok(h_i, d_i)) return CSA2_E_UNSUPPORTED;
  if (ik8 && d_i != 128) return CSA2_E_UNSUPPORTED;
  if (keep_blocks > 0 && block != 8) return CSA2_E_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!iq || !w || !q_seq || !q_nvis || !seq_base || !idx_out || !ws) return CSA2_E_INVAL;
  if (keep_blocks > 0 && !pool_out) return CSA2_E_INVAL;
  if (!keys_ok(d_i, ik, ik8, ik8e)) return CSA2_E_INVAL;
  if (!aligned(iq, 16) || !aligned(w, 4) || !aligned(ws, 256)) return CSA2_E_INVAL;
  Params P{};
  P.iq = iq; P.w = w; P.n_q = n_q; P.h_i = h_i; P.d_i = d_i;
  P.q_seq = q_seq; P.q_nvis = q_nvis; P.ik = ik; P.ik8 = ik8; P.ik8e = ik8e; P.seq_base = seq_base;
  if (keep_blocks == 0 && max_nvis <= kSmallMax) {
    // Short contexts without a pool: the Reindex path over every block of the
    // context in order (a null pool) -- the same exact Top-K over the positions
    // < q_nvis, from the scan and the one-work-group select (two launches
    // instead of six).  Its workspace (stride 8 ceil(max_nvis / 8) rounded up)
    // fits in this call's.
    P.pool_in = nullptr; P.keep_in = std::max(1, (max_nvis + 7) / 8); P.k = k; P.keep_blocks = 0;
    P.idx_out = idx_out; P.pool_out = nullptr;
    P.nprob = n_q;
    P.reindex = 1;
    const int64_t slots = 8LL * P.keep_in;
    P.scan_chunk = reindex_chunk_for(n_q, slots);
    P.stride = round_up(slots, kCmpChunk);
    P.nchunk_cmp = (int)(P.stride / kCmpChunk);
    const size_t need = csa2_index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, block, keep_blocks);
    return run_pipeline(P, slots, ws, ws_bytes, static_cast<hipStream_t>(stream), need);
  }
  P.pool_in = nullptr; P.keep_in = 0; P.k = k; P.keep_blocks = keep_blocks;
  P.idx_out = idx_out; P.pool_out = pool_out;
  P.nprob = n_q * (keep_blocks > 0 ? 2 : 1);
  P.reindex = 0;
  P.scan_chunk = scan_chunk_for(n_q, max_nvis);
  P.stride = round_up(std::max<int64_t>(max_nvis, 1), kCmpChunk);
  P.nchunk_cmp = (int)(P.stride / kCmpChunk);
  const size_t need = csa2_index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, block, keep_blocks);
  return run_pipeline(P, max_nvis, ws, ws_bytes, static_cast<hipStream_t>(stream), need);
}

csa2_status reindex_call(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i, const int32_t* q_seq,
                         const int32_t* q_nvis, const uint16_t* ik, const uint8_t* ik8, const uint8_t* ik8e,
                         const int64_t* seq_base, const int32_t* pool_blocks, int block, int keep_blocks, int k,
                         int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  csa2::set_last_hip_error(0);
  if (n_q < 0 || k < 1 || k > 2048 || keep_blocks < 1 || keep_blocks > 4096) return CSA2_E_INVAL;
  if (!shape_ok(h_i, d_i)) return CSA2_E_UNSUPPORTED;
  if (ik8 && d_i != 128) return CSA2_E_UNSUPPORTED;
  if (block != 8) return CSA2_E_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!iq || !w || !q_seq || !q_nvis || !seq_base || !pool_blocks || !idx_out || !ws) return CSA2_E_INVAL;
  if (!keys_ok(d_i, ik, ik8, ik8e)) return CSA2_E_INVAL;
  if (!aligned(iq, 16) || !aligned(w, 4) || !aligned(ws, 256)) return CSA2_E_INVAL;
  Params P{};
  P.iq = iq; P.w = w; P.n_q = n_q; P.h_i = h_i; P.d_i = d_i;
  P.q_seq = q_seq; P.q_nvis = q_nvis; P.ik = ik; P.ik8 = ik8; P.ik8e = ik8e; P.seq_base = seq_base;
  P.pool_in = pool_blocks; P.keep_in = keep_blocks; P.k = k; P.keep_blocks = 0;
  P.idx_out = idx_out; P.pool_out = nullptr;
  P.nprob = n_q;
  P.reindex = 1;
  const int64_t slots = 8LL * keep_blocks;
  P.scan_chunk = reindex_chunk_for(n_q, slots);
  P.stride = round_up(slots, kCmpChunk);
  P.nchunk_cmp = (int)(P.stride / kCmpChunk);
  const size_t need = csa2_reindex_topk_ws_bytes(n_q, h_i, d_i, k, block, keep_blocks);
  return run_pipeline(P, slots, ws, ws_bytes, static_cast<hipStream_t>(stream), need);
}

}  // namespace

extern "C" csa2_status csa2_index_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                       const int32_t* q_seq, const int32_t* q_nvis, int32_t max_nvis,
                                       const uint16_t* ik, const int64_t* seq_base, int k, int32_t* idx_out,
                                       int block, int keep_blocks, int32_t* pool_out, void* ws, size_t ws_bytes,
                                       void* stream) {
  return index_call(iq, w, n_q, h_i, d_i, q_seq, q_nvis, max_nvis, ik, nullptr, nullptr, seq_base, k, idx_out,
                    block, keep_blocks, pool_out, ws, ws_bytes, stream);
}

extern "C" csa2_status csa2_index_topk_fp8(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                           const int32_t* q_seq, const int32_t* q_nvis, int32_t max_nvis,
                                           const uint8_t* ik8, const uint8_t* ik8_exp, const int64_t* seq_base,
                                           int k, int32_t* idx_out, int block, int keep_blocks, int32_t* pool_out,
                                           void* ws, size_t ws_bytes, void* stream) {
  return index_call(iq, w, n_q, h_i, d_i, q_seq, q_nvis, max_nvis, nullptr, ik8, ik8_exp, seq_base, k, idx_out,
                    block, keep_blocks, pool_out, ws, ws_bytes, stream);
}

extern "C" csa2_status csa2_index_topk_chunk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                             const int32_t* q_nvis, int32_t max_nvis, const uint16_t* ik,
                                             int64_t ik_base, int k, int32_t* idx_out, void* ws, size_t ws_bytes,
                                             void* stream) {
  csa2::set_last_hip_error(0);
  if (n_q < 0 || max_nvis < 0 || k < 1 || k > 2048 || ik_base < 0) return CSA2_E_INVAL;
  if ((int64_t)max_nvis > (int64_t)kMaxChunksLds * kCmpChunk) return CSA2_E_UNSUPPORTED;
  if (!shape_ok(h_i, d_i)) return CSA2_E_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!iq || !w || !q_nvis || !ik || !idx_out || !ws) return CSA2_E_INVAL;
  if (!aligned(iq, 16) || !aligned(ik, 16) || !aligned(w, 4) || !aligned(ws, 256)) return CSA2_E_INVAL;
  Params P{};
  P.iq = iq; P.w = w; P.n_q = n_q; P.h_i = h_i; P.d_i = d_i;
  P.q_seq = nullptr; P.q_nvis = q_nvis; P.ik = ik; P.seq_base = nullptr; P.base0 = ik_base;
  P.pool_in = nullptr; P.keep_in = 0; P.k = k; P.keep_blocks = 0;
  P.idx_out = idx_out; P.pool_out = nullptr;
  P.nprob = n_q;
  P.reindex = 0;
  P.scan_chunk = kMaxScanChunk;
  P.stride = round_up(std::max<int64_t>(max_nvis, 1), kCmpChunk);
  P.nchunk_cmp = (int)(P.stride / kCmpChunk);
  const size_t need = csa2_index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, 8, 0);
  return run_pipeline(P, max_nvis, ws, ws_bytes, static_cast<hipStream_t>(stream), need, true);
}

extern "C" csa2_status csa2_reindex_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                         const int32_t* q_seq, const int32_t* q_nvis, const uint16_t* ik,
                                         const int64_t* seq_base, const int32_t* pool_blocks, int block,
                                         int keep_blocks, int k, int32_t* idx_out, void* ws, size_t ws_bytes,
                                         void* stream) {
  return reindex_call(iq, w, n_q, h_i, d_i, q_seq, q_nvis, ik, nullptr, nullptr, seq_base, pool_blocks, block,
                      keep_blocks, k, idx_out, ws, ws_bytes, stream);
}

extern "C" csa2_status csa2_reindex_topk_fp8(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                             const int32_t* q_seq, const int32_t* q_nvis, const uint8_t* ik8,
                                             const uint8_t* ik8_exp, const int64_t* seq_base,
                                             const int32_t* pool_blocks, int block, int keep_blocks, int k,
                                             int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  return reindex_call(iq, w, n_q, h_i, d_i, q_seq, q_nvis, nullptr, ik8, ik8_exp, seq_base, pool_blocks, block,
                      keep_blocks, k, idx_out, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- allocation-free Reindex
// A fixed scratch array in device memory, one per GPU the library runs on
// (held until the process ends), for callers that cannot allocate: the
// workspace of csa2_reindex_topk_noalloc.  Host code never passes `scratch`
// itself (in host code the name is a stand-in, not a device address): its
// device address is looked up once per device and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure,
// with the HIP error recorded).
void* scratch_for_current_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_last_hip_error((int)e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_last_hip_error((int)hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_last_hip_error((int)(e != hipSuccess ? e : hipErrorInvalidSymbol));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" csa2_status csa2_reindex_topk_noalloc(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                                 const int32_t* q_seq, const int32_t* q_nvis, const uint16_t* ik,
                                                 const int64_t* seq_base, const int32_t* pool_blocks, int block,
                                                 int keep_blocks, int k, int32_t* idx_out, void* stream) {
  csa2::set_last_hip_error(0);
  if (n_q < 0 || k < 1 || k > 2048 || keep_blocks < 1 || keep_blocks > 4096) return CSA2_E_INVAL;
  if (!shape_ok(h_i, d_i)) return CSA2_E_UNSUPPORTED;
  if (block != 8) return CSA2_E_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  const size_t need = csa2_reindex_topk_ws_bytes(n_q, h_i, d_i, k, block, keep_blocks);
  if (need > (size_t)CSA2_NOALLOC_SCRATCH_BYTES) return CSA2_E_WORKSPACE;
  void* ws = scratch_for_current_device();
  if (!ws) return CSA2_E_HIP;
  // the same kernels as csa2_reindex_topk; none of them needs the scratch
  // cleared beforehand (each launch writes what the next one reads, and the
  // multi-kernel path's first launch zeroes its histograms)
  return csa2_reindex_topk(iq, w, n_q, h_i, d_i, q_seq, q_nvis, ik, seq_base, pool_blocks, block, keep_blocks, k,
                           idx_out, ws, (size_t)CSA2_NOALLOC_SCRATCH_BYTES, stream);
}
