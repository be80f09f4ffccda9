// sparse_attn.hip -- CSA2 sparse attention over the selected FP4 main-KV
// entries merged with the layer's sliding-window rows (gfx950).
//
// Every decode layer attends over the Top-K entries chosen by its group's
// Full/Reindex layer (Reuse layers inherit that list) plus its own 128-row
// sliding window; the main KV is E2M1 with one E4M3 scale per 16 channels.
// Sources: "DeepSeek AI выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн
// токенов, KV-кэшем FP4 ..." (wire.sakhanda.co), sections "Каузальный
// энкодер-декодер" (128-token window in every layer), "Сжатое разреженное
// внимание 2 (CSA2)" (modes, own Q and window KV per layer) and "FP4 KV ..."
// (the cache format).
//
// Work decomposition: one work-group per (query, split of the key slots);
// slots [0, k) are the selected entries, [k, k + swa_len) the window rows.
// A split takes every nsplit-th 32-slot sub-tile (so the window's sub-tiles,
// whose rows are the largest, are spread over the splits).  The split's slot positions are
// staged in LDS first; then, double-buffered, the loads of sub-tile s+1 are
// in flight while the MFMA work of sub-tile s runs, and are decoded into the
// other LDS buffer after it.
// Per 32-slot sub-tile the whole work-group decodes the keys once into LDS,
// in two layouts (key-major for Q.K, channel-major for P.V), as fp16 -- an
// E2M1 value times an E4M3 scale has at most 6 significant bits and lies in
// [2^-10, 2688], so the decode is exact.  Each of the h/16 head waves then
// runs v_mfma_f32_16x16x32_f16:
//   S^T (32 keys x 16 heads) = K (32 x 512) . Q^T      (q in registers)
//   O  (16 heads x 512)     += P (16 x 32) . V (32 x 512)
// Computing S transposed leaves each lane with 8 key scores of one head, which
// is exactly the A-operand layout P needs, so P never moves between lanes.
// An online softmax (base-2 exponent, running max per head) carries across
// sub-tiles; splits are merged by k_merge with their (max, sum) pairs.
//
// Two kernels share this scheme: k_attn2 (bf16 queries) gives the loads and
// the decode to four waves of their own, so they overlap the multiply waves'
// MFMA work; k_attn<true> (fp32 queries, which carry a second fp16 term per
// channel and need the registers) runs both in its four waves, one after the
// other.
#include "csa2_device.h"

#include <type_traits>

namespace csa2 {
namespace attn {

constexpr int kThreads = 256;
constexpr int kSub = 32;            // key slots per sub-tile
constexpr int kKRow = 512 + 8;      // fp16 per key row in the key-major tile (16 B pad)
constexpr int kVRow = kSub + 4;     // fp16 per channel row in the channel-major tile (8 B pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSlotsWG = 3072;   // key slots one work-group stages: k <= 2048 plus a window <= 1024
constexpr int kMaxSplit = 64;       // splits per query (one wave merges their weights)

struct Params {
  const void* q;
  int n_q, h;
  const int32_t* q_seq;
  const uint8_t* cache;
  const int64_t* seq_base;
  const int32_t* idx;
  int k;
  const uint16_t* swa;
  // this call's new window rows (optional): swa_new[i] goes to row swa_dst[i]
  // of swa (written by work-group (i, 0)); a window slot on that row reads
  // swa_new[i] itself, so no work-group depends on the write
  const uint16_t* swa_new;
  const int64_t* swa_dst;
  uint16_t* swa_out;
  int64_t swa_rows;
  const int64_t* swa_row0;
  const int32_t* swa_len;
  float scale_log2;
  float* out;
  float* lse;
  int nsplit, nsub;
  _Float16* part_o;   // [n_q][nsplit][h][512]: each split's output / its l
  float* part_ml;     // [n_q][nsplit][h][2]: each split's (m, l)
};

// 8 E2M1 codes (one little-endian dword, channel 2i in the low nibble of byte
// i) times an E4M3 scale byte -> 4 packed fp16 pairs.  The scale goes to fp16
// by moving bits: (b & 0x7F) << 7 read as an fp16 is the E4M3 magnitude times
// 2^-8 (exponent bias 15 instead of 7, E4M3 subnormals landing on fp16
// subnormals); v_cvt_scalef32_pk_f16_fp4 turns a byte's two codes into fp16
// times 2^8 (a power-of-two scale argument is applied exactly), then one
// packed fp16 multiply.  Both factors are exact in fp16 and so is their
// product (an E2M1 value times an E4M3 scale has at most 6 significant bits
// and lies in [2^-10, 2688]).
__device__ __forceinline__ void decode8(uint32_t c, uint32_t sbyte, uint32_t out[4]) {
  const uint32_t sb = ((sbyte & 0x7Fu) << 7) | ((sbyte & 0x80u) << 8);
  const f16x2 s2 = __builtin_bit_cast(f16x2, sb | (sb << 16));
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 0) * s2);
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 1) * s2);
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 2) * s2);
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 256.0f, 3) * s2);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Raw words of one thread's share of a sub-tile (8 key slots x 8 channels),
// loaded one sub-tile ahead of the MFMA work and decoded after it.
struct Stage {
  uint32_t w[8][4];   // selected entry: codes dword, scale dword; window row: 8 bf16
  uint32_t valid;   // bit jj: slot 8*kq + jj holds a key
};

// Slot classes of a sub-tile: all selected entries, all window rows, or both.
__device__ __forceinline__ int sub_kind(int slot0, int k) {
  return slot0 + kSub <= k ? 0 : (slot0 >= k ? 1 : 2);
}

template <bool QF32>
__global__ __launch_bounds__(kThreads) void k_attn(Params P) {
  __shared__ __attribute__((aligned(16))) _Float16 s_k[2][kSub * kKRow];
  __shared__ __attribute__((aligned(16))) _Float16 s_v[2][512 * kVRow];
  __shared__ uint32_t s_valid[2][kSub];
  __shared__ int32_t s_pos[kMaxSlotsWG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int qi = blockIdx.x, split = blockIdx.y;
  const bool head_wave = 16 * wave < P.h;
  const int head = 16 * wave + n;
  const int64_t cbase = P.seq_base[P.q_seq[qi]];
  const int k = P.k;
  const int nswa = P.swa_len ? P.swa_len[qi] : 0;
  const int64_t srow0 = nswa ? P.swa_row0[qi] : 0;
  const int64_t wdst = P.swa_new ? P.swa_dst[qi] : -1;   // this call's new window row of the query
  // the window row `row` of this query, 8 channels from channel 8 cg
  auto win_src = [&](int64_t row, int cgi) -> const uint16_t* {
    return row == wdst ? P.swa_new + (size_t)qi * 512 + 8 * cgi : P.swa + (size_t)row * 512 + 8 * cgi;
  };
  if (wdst >= 0 && wdst < P.swa_rows && split == 0 && tid < 64)
    reinterpret_cast<uint4*>(P.swa_out + (size_t)wdst * 512)[tid] =
        reinterpret_cast<const uint4*>(P.swa_new + (size_t)qi * 512)[tid];
  // this split's sub-tiles: split, split + nsplit, split + 2 nsplit, ... (every
  // split gets its share of the window's sub-tiles, whose rows are the largest)
  const int ns = P.nsplit;
  const int nmine = split < P.nsub ? (P.nsub - split + ns - 1) / ns : 0;
  // fallback address for slots without a key: any readable bytes (the query)
  const uint8_t* fb = static_cast<const uint8_t*>(P.q);

  // selected positions of this split's sub-tiles: local sub-tile j at s_pos[32 j ..]
  for (int i = tid; i < nmine * kSub; i += kThreads) {
    const int slot = (split + (i / kSub) * ns) * kSub + (i % kSub);
    if (slot < k) s_pos[i] = P.idx[(size_t)qi * k + slot];
  }

  // decode assignment: thread -> key slots 8*kq .. 8*kq+7, channels 8*cg .. 8*cg+7
  const int kq = tid & 3, cg = tid >> 2;
  Stage st;

  // Global loads of a sub-tile, one loader per slot class.  Addresses of
  // empty slots point at the fallback bytes, so no load is conditional.
  auto load_sel_pos = [&](const int pos[8]) {   // all 32 slots are selected entries
    st.valid = 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint8_t* rec = pos[jj] >= 0 ? P.cache + (size_t)(cbase + pos[jj]) * CSA2_KV_RECORD_BYTES : fb;
      st.w[jj][0] = *reinterpret_cast<const uint32_t*>(rec + 4 * cg);
      st.w[jj][1] = *reinterpret_cast<const uint32_t*>(rec + 256 + 4 * (cg >> 3));
      st.valid |= (pos[jj] >= 0 ? 1u : 0u) << jj;
    }
  };
  auto load_sel = [&](int j) {        // local sub-tile j; positions from the LDS copy of the index list
    const int i0 = j * kSub + 8 * kq;   // multiple of 8: two 16-byte LDS reads
    const int4 pa = *reinterpret_cast<const int4*>(&s_pos[i0]);
    const int4 pb = *reinterpret_cast<const int4*>(&s_pos[i0 + 4]);
    const int pos[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    load_sel_pos(pos);
  };
  auto load_win = [&](int sub) {      // all 32 slots are window rows (or past the window)
    const int r0 = sub * kSub + 8 * kq - k;
    st.valid = 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const bool ok = r0 + jj < nswa;
      const uint16_t* src =
          ok ? win_src(srow0 + r0 + jj, cg) : reinterpret_cast<const uint16_t*>(fb) + 8 * cg;
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      st.w[jj][0] = v.x; st.w[jj][1] = v.y; st.w[jj][2] = v.z; st.w[jj][3] = v.w;
      st.valid |= (ok ? 1u : 0u) << jj;
    }
  };
  auto load_mixed = [&](int sub) {    // the one sub-tile that straddles slot k
    const int slot0 = sub * kSub + 8 * kq;
    st.valid = 0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int slot = slot0 + jj;
      st.w[jj][0] = st.w[jj][1] = st.w[jj][2] = st.w[jj][3] = 0u;
      if (slot < k) {
        const int pos = P.idx[(size_t)qi * k + slot];
        if (pos >= 0) {
          const uint8_t* rec = P.cache + (size_t)(cbase + pos) * CSA2_KV_RECORD_BYTES;
          st.w[jj][0] = *reinterpret_cast<const uint32_t*>(rec + 4 * cg);
          st.w[jj][1] = *reinterpret_cast<const uint32_t*>(rec + 256 + 4 * (cg >> 3));
          st.valid |= 1u << jj;
        }
      } else if (slot - k < nswa) {
        const uint4 v = *reinterpret_cast<const uint4*>(win_src(srow0 + slot - k, cg));
        st.w[jj][0] = v.x; st.w[jj][1] = v.y; st.w[jj][2] = v.z; st.w[jj][3] = v.w;
        st.valid |= 1u << jj;
      }
    }
  };

  // The first sub-tile's loads are issued before the query's: a selected
  // sub-tile takes its positions straight from the index list in global memory
  if (nmine > 0) {
    const int kind = sub_kind(split * kSub, k);
    if (kind == 0) {
      const int32_t* ip = P.idx + (size_t)qi * k + split * kSub + 8 * kq;
      int pos[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pos[jj] = ip[jj];
      load_sel_pos(pos);
    } else if (kind == 1) {
      load_win(split);
    } else {
      load_mixed(split);
    }
  }

  // Q^T as the B operand: lane (head n, group g) holds channels 32*ks + 8*g .. +7
  f16x8 qb[16];
  f16x8 ql[QF32 ? 16 : 1];
  if (head_wave) {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const size_t off = ((size_t)qi * P.h + head) * 512 + 32 * ks + 8 * g;
      float x[8];
      if (QF32) {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(P.q) + off);
        float4 a = src[0], b = src[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      } else {
        uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(P.q) + off);
        const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = __uint_as_float(wd[j] << 16);
          x[2 * j + 1] = __uint_as_float(wd[j] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        _Float16 hi = (_Float16)x[j];
        qb[ks][j] = hi;
        if constexpr (QF32) ql[ks][j] = (_Float16)(x[j] - (float)hi);
      }
    }
  }


  // Decode the loaded words to fp16 and write both LDS layouts of buffer b.
  auto store_stage = [&](int sub, int b) {
    const int slot0 = sub * kSub;
    const int sc_shift = 8 * ((cg >> 1) & 3);   // this thread's scale byte in the loaded scale dword
    uint32_t vals[8][4];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const bool is_sel = slot0 + 8 * kq + jj < k;
      const uint32_t keep = (st.valid >> jj) & 1u ? 0xFFFFFFFFu : 0u;
      uint32_t dv[4], sv[4];
      decode8(st.w[jj][0], (st.w[jj][1] >> sc_shift) & 0xFFu, dv);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sv[j] = pack_f16(__uint_as_float(st.w[jj][j] << 16), __uint_as_float(st.w[jj][j] & 0xFFFF0000u));
#pragma unroll
      for (int j = 0; j < 4; ++j) vals[jj][j] = (is_sel ? dv[j] : sv[j]) & keep;
      if (cg == 0) s_valid[b][8 * kq + jj] = keep & 1u;
      *reinterpret_cast<uint4*>(&s_k[b][(8 * kq + jj) * kKRow + 8 * cg]) =
          make_uint4(vals[jj][0], vals[jj][1], vals[jj][2], vals[jj][3]);
    }
    // channel-major copy: row (channel 8*cg + c) gets key slots 8*kq .. 8*kq+7
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t pk[4];
#pragma unroll
      for (int jp = 0; jp < 4; ++jp) {
        const uint32_t a = vals[2 * jp][c >> 1], bb = vals[2 * jp + 1][c >> 1];
        // take the low (c even) or high (c odd) fp16 of each
        pk[jp] = (c & 1) ? __builtin_amdgcn_perm(bb, a, 0x07060302u) : __builtin_amdgcn_perm(bb, a, 0x05040100u);
      }
      uint2* dst = reinterpret_cast<uint2*>(&s_v[b][(8 * cg + c) * kVRow + 8 * kq]);
      dst[0] = make_uint2(pk[0], pk[1]);
      dst[1] = make_uint2(pk[2], pk[3]);
    }
  };

  f32x4 o[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  if (nmine > 0) store_stage(split, 0);
  lds_barrier();   // s_pos and buffer 0

  auto compute = [&](int b) {
    if (head_wave) {
      // ---- S^T = K Q^T : lane (head n, g) gets keys 16*kt + 4*g + i
      // the two key tiles' chains interleaved (independent accumulators); each
      // k-step's fragments are read one k-step ahead of their MFMAs
      f32x4 sacc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
      const _Float16* krow0 = &s_k[b][n * kKRow + 8 * g];
      const _Float16* krow1 = &s_k[b][(16 + n) * kKRow + 8 * g];
      f16x8 n0 = *reinterpret_cast<const f16x8*>(krow0);
      f16x8 n1 = *reinterpret_cast<const f16x8*>(krow1);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const f16x8 a0 = n0, a1 = n1;
        if (ks + 1 < 16) {
          n0 = *reinterpret_cast<const f16x8*>(krow0 + 32 * (ks + 1));
          n1 = *reinterpret_cast<const f16x8*>(krow1 + 32 * (ks + 1));
        }
        sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qb[ks], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qb[ks], sacc[1], 0, 0, 0);
        if constexpr (QF32) {
          sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, ql[ks], sacc[0], 0, 0, 0);
          sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, ql[ks], sacc[1], 0, 0, 0);
        }
      }
      {
        constexpr int kM = QF32 ? 4 : 2;   // MFMAs per k-step
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int r = 0; r < 15; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, kM, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kM, 0);
      }
      float z[8];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * kt + 4 * g + i;
          const float v = s_valid[b][key] ? sacc[kt][i] * P.scale_log2 : -INFINITY;
          z[4 * kt + i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      // The running reference m_run moves only when a score exceeds it by more
      // than 8 (base 2): otherwise P = 2^(z - m_run) <= 256, still exact to
      // fp16's relative precision, and O and l keep their reference (the
      // softmax, and the merge of splits by their (m, l), do not depend on
      // which reference is used).  So the costly rescale of O is rare.
      const bool bump = mx > m_run + 8.0f;   // true on the first key (m_run = -inf)
      const float m_use = bump ? mx : m_run;
      float alpha, pv[8];
      if (m_use == -INFINITY) {
        alpha = 1.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = 0.0f;
      } else {
        alpha = bump ? exp2f(m_run - m_use) : 1.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = exp2f(z[j] - m_use);
      }
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ps += pv[j];
      l_run = l_run * alpha + ps;
      // rescale O rows (heads 4*g + i live in this lane's accumulators); a
      // wave whose references did not move, or whose O is still zero (no key
      // seen yet), skips it
      const bool rescale = bump && m_run != -INFINITY;
      m_run = m_use;
      if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
        float a4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
        for (int t = 0; t < 32; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[t][i] *= a4[i];
      }
      // P as the A operand: slots 0..3 = keys 4g+i, slots 4..7 = keys 16+4g+i
      f16x8 pa;
#pragma unroll
      for (int j = 0; j < 8; ++j) pa[j] = (_Float16)pv[j];
      // ---- O += P V  (each V fragment read one MFMA ahead)
      auto vfrag = [&](int t) {
        const _Float16* vrow = &s_v[b][(16 * t + n) * kVRow];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * g);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * g);
        return __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      };
      f16x8 nv = vfrag(0);
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        const f16x8 bv = nv;
        if (t + 1 < 32) nv = vfrag(t + 1);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bv, o[t], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int r = 0; r < 30; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };

  // Selected-entry sub-tiles (all but the last few) are prefetched: their
  // loads stay in flight during this sub-tile's MFMA work.  Window and
  // straddling sub-tiles load after it.
  for (int j = 0; j < nmine; ++j) {
    const int b = j & 1;
    const int nsub = split + (j + 1) * ns;   // the next sub-tile
    const int kind = j + 1 < nmine ? sub_kind(nsub * kSub, k) : 3;
    if (kind == 0) load_sel(j + 1);
    else if (kind == 1) load_win(nsub);
    compute(b);
    if (kind == 0 || kind == 1) {
      // the loaded words become visible to the decode only here, so the
      // compiler cannot hoist the decode (and its wait) above the MFMA work
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        asm volatile("" : "+v"(st.w[jj][0]), "+v"(st.w[jj][1]), "+v"(st.w[jj][2]), "+v"(st.w[jj][3]));
    }
    if (kind == 2) load_mixed(nsub);
    if (kind != 3) store_stage(nsub, b ^ 1);   // the other buffer: last read before the previous barrier
    lds_barrier();
  }

  if (!head_wave) return;
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  // per-row (head 4*g + i) values for this lane's accumulators
  float lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lrow[i] = __shfl(l_tot, 4 * g + i, kWave);
  if (P.nsplit == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * wave + 4 * g + i;
      const float inv = lrow[i] > 0.0f ? 1.0f / lrow[i] : 0.0f;
      float* dst = P.out + ((size_t)qi * P.h + hh) * 512 + n;
#pragma unroll
      for (int t = 0; t < 32; ++t) dst[16 * t] = o[t][i] * inv;
    }
    if (P.lse && g == 0)
      P.lse[(size_t)qi * P.h + head] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    // the split's output normalised by its own sum, rounded to fp16 (a convex
    // combination of fp16 values: in range, relative error 2^-11)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 16 * wave + 4 * g + i;
      const float inv = lrow[i] > 0.0f ? 1.0f / lrow[i] : 0.0f;
      _Float16* dst = P.part_o + (((size_t)qi * P.nsplit + split) * P.h + hh) * 512 + n;
#pragma unroll
      for (int t = 0; t < 32; ++t) dst[16 * t] = (_Float16)(o[t][i] * inv);
    }
    if (g == 0) {
      float* ml = P.part_ml + (((size_t)qi * P.nsplit + split) * P.h + head) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------- large batches
// k_attn2: the bf16-query kernel.  k_attn's four waves decode a sub-tile and
// then multiply it, in series, and its LDS leaves one work-group per CU.  Here
// a work-group has eight waves: waves 0-3 multiply as k_attn's do (16 heads
// each, the same MFMA shapes and online softmax; the LDS tiles are laid out
// differently, see key_row and v_addr), waves 4-7 only load and decode: while the multiply waves work on sub-tile j, the decode waves write
// sub-tile j + 1 into the other LDS buffer, with the loads of j + 2 and j + 3
// in flight.  One barrier per sub-tile; two waves per SIMD.  A SIMD's two
// waves share its VALU issue and the CU's LDS, which bound a sub-tile (about
// 5k cycles, a fifth of it MFMA work), so the decode is kept lean: a
// sub-tile's slot class is known before its decode and picks a decode without
// the other class's work, the FP4 scale is decoded by moving bits, and a
// gather address is one multiply-add from a per-thread base.
constexpr int kStages = 2;   // sub-tiles whose loads the decode waves keep in flight (3 or 4 time the same)
// read-only kernel inputs through the constant address space (scalar loads)
typedef __attribute__((address_space(4))) const int32_t ci32;
typedef __attribute__((address_space(4))) const int64_t ci64;
__device__ const int32_t kZeroI32 = 0;
// max / sum with the value of lane l ^ 16 (rows 0 <-> 1, 2 <-> 3) or l ^ 32
// (the wave's halves), by VALU lane swaps instead of LDS permutes
__device__ __forceinline__ float max_xor16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ const int64_t kZeroI64 = 0;
__device__ const int64_t kNoRowI64 = -1;
constexpr int kBuf2 = 3;     // k_attn2's key-major tiles: being decoded, multiplied (Q.K), multiplied (P.V)
constexpr int kPRow2 = kSub + 8;   // fp16 per head row of k_attn2's P tile (16-byte pad)
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
template <int NHT>
__global__ __launch_bounds__(2 * kThreads) void k_attn2(Params P) {
  __shared__ __attribute__((aligned(16))) _Float16 s_k[kBuf2][kSub * kKRow];   // key-major tiles, a ring of three
  __shared__ __attribute__((aligned(16))) _Float16 s_p[2][64 * kPRow2];        // P [head][key], double-buffered
  __shared__ __attribute__((aligned(16))) float s_alpha[2][64];                 // O rescale factor per head
  __shared__ float s_ml[64][2];                                                 // final (m, l) per head
  __shared__ int32_t s_pos[kMaxSlotsWG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int qi = blockIdx.x, split = blockIdx.y;
  // heads hbase .. hbase + 16 NHT - 1 (local rows 0 .. 16 NHT - 1)
  const int hbase = 16 * NHT * blockIdx.z;
  const bool mwave = wave < 4;   // multiply waves; waves 4-7 decode
  const bool qk_wave = wave < NHT;   // multiply waves that run Q.K and the softmax
  const bool head_wave = qk_wave && hbase + 16 * wave < P.h;
  const int lrow = 16 * wave + n;   // a Q.K wave's head, local row
  const int head = hbase + lrow;
  // Key-major tile: key slot s of a sub-tile sits in row key_row(s), so that
  // MFMA tile kt's row r holds key 8 (r >> 2) + 4 kt + (r & 3); keys 8 g ..
  // 8 g + 3 are rows 4 g .. 4 g + 3 and keys 8 g + 4 .. + 7 rows 16 + 4 g ..
  auto key_row = [](int s) { return 16 * ((s >> 2) & 1) + 4 * (s >> 3) + (s & 3); };
  // The query's window inputs, loaded without branches (an absent array
  // reads a constant) so that their loads are in flight together.
  const int k = P.k;
  const int nswa = *(P.swa_len ? (const ci32*)(P.swa_len + qi) : (const ci32*)&kZeroI32);
  const int64_t srow0 = *(P.swa_len ? (const ci64*)(P.swa_row0 + qi) : (const ci64*)&kZeroI64);   // used only when nswa > 0
  const int64_t wdst = *(P.swa_new ? (const ci64*)(P.swa_dst + qi) : (const ci64*)&kNoRowI64);   // this call's new window row of the query
  // The two window sources as values in scalar registers: a select between
  // the kernel-argument fields themselves may be compiled into a per-lane
  // load of the chosen field, a dependent round trip before every row load.
  const uint16_t* swa_p = P.swa;
  const uint16_t* swa_new_p = P.swa_new;
  asm volatile("" : "+s"(swa_p), "+s"(swa_new_p));
  auto win_src = [&](int64_t row, int cgi) -> const uint16_t* {
    return row == wdst ? swa_new_p + (size_t)qi * 512 + 8 * cgi : swa_p + (size_t)row * 512 + 8 * cgi;
  };
  const int ns = P.nsplit;
  const int nmine = split < P.nsub ? (P.nsub - split + ns - 1) / ns : 0;
  const uint8_t* fb = static_cast<const uint8_t*>(P.q);

  // ---- state of both roles.  Every wave runs the P.V of its channel eighth
  // (channels 64 wave .. 64 wave + 63) for the work-group's heads: O^T =
  // V^T P^T, where row m of channel tile t is channel 64 wave + 16 (m / 4) +
  // 4 t + m % 4, so o[mt][t] lane (local head 16 mt + n, g) holds channels
  // 64 wave + 16 g + 4 t .. + 3 of that head: the lane's sixteen are
  // consecutive.  The P.V of sub-tile j runs in step j + 1 (after the barrier
  // that publishes its P), reading P and the heads' rescale factors from LDS
  // (double-buffered) and V from the key-major tile (a ring of three: the
  // decode waves fill sub-tile j + 2 meanwhile).  Multiply waves 0 .. NHT - 1
  // also run Q.K and the online softmax of local heads 16 wave .. 16 wave +
  // 15, in one block with their P.V (the MFMAs of each cover the other's LDS
  // reads); heads past h are still multiplied (results dropped), so no branch
  // separates the MFMAs.
  f32x4 o[NHT][4];
#pragma unroll
  for (int mt = 0; mt < NHT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) o[mt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;
  // Q^T as the B operand, lane (head n, group g) holds channels 32*ks + 8*g
  // .. +7 (rounded to fp16, as k_attn); loaded by the multiply waves
  f16x8 qb[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qb[ks] = f16x8{};

  // One step: the P.V of sub-tile jp (tile buffer bp) when kPV, and the Q.K
  // and softmax of sub-tile jq (tile buffer bq) when kQK; the softmax leaves P
  // and the rescale factors of the wave's heads in LDS buffer jq & 1.
  auto step = [&](int jp, int bp, int jq, int bq, auto pv_flag, auto qk_flag) {
    constexpr bool kPV = decltype(pv_flag)::value, kQK = decltype(qk_flag)::value;
    f16x8 pa[NHT];
    if constexpr (kPV) {
      // P^T (B operand): lane (local head 16 mt + n, g) holds keys 8 g .. 8 g
      // + 7; O rows of heads whose reference moved are rescaled first
      float al[NHT];
      bool moved = false;
#pragma unroll
      for (int mt = 0; mt < NHT; ++mt) {
        al[mt] = s_alpha[jp & 1][16 * mt + n];
        pa[mt] = *reinterpret_cast<const f16x8*>(&s_p[jp & 1][(16 * mt + n) * kPRow2 + 8 * g]);
        moved |= al[mt] != 1.0f;
      }
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
        for (int mt = 0; mt < NHT; ++mt)
#pragma unroll
          for (int t = 0; t < 4; ++t) o[mt][t] *= al[mt];
      }
    }
    // S^T = K Q^T : tile kt's row r holds key 8 (r >> 2) + 4 kt + (r & 3), so
    // lane (head n, g) gets keys 8 g + 4 kt + i: eight consecutive keys.
    // V^T (A operand) of channel tile t: lane (row n, g) holds keys 8 g ..
    // 8 g + 7 of its channel by two transposed reads in which source lane n
    // reads key row 4 g + n / 4 (then 16 + 4 g + n / 4), channels 64 wave +
    // 16 (n & 3) + 4 t .. + 3.  k-step ks carries the two Q.K MFMAs of
    // channels 32 ks .. 32 ks + 31, and every (4 / NHT)-th k-step one of the
    // 4 NHT P.V MFMAs (channel tile by channel tile); each k-step's fragments
    // are read one k-step (V: one tile) ahead.
    constexpr int kPer = 4 / NHT;
    f32x4 sacc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
    const _Float16* krow0 = &s_k[bq][n * kKRow + 8 * g];
    const _Float16* krow1 = &s_k[bq][(16 + n) * kKRow + 8 * g];
    const _Float16* v0 = &s_k[bp][(4 * g + (n >> 2)) * kKRow + 64 * wave + 16 * (n & 3)];
    auto vread = [&](int t) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v0 + 4 * t));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v0 + 16 * kKRow + 4 * t));
      const uint2 va = __builtin_bit_cast(uint2, lo), vb = __builtin_bit_cast(uint2, hi);
      return __builtin_bit_cast(f16x8, make_uint4(va.x, va.y, vb.x, vb.y));
    };
    f16x8 n0{}, n1{}, bvn{}, bv{};
    if constexpr (kQK) {
      n0 = *reinterpret_cast<const f16x8*>(krow0);
      n1 = *reinterpret_cast<const f16x8*>(krow1);
    }
    if constexpr (kPV) bvn = vread(0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const f16x8 a0 = n0, a1 = n1;
      if constexpr (kQK) {
        if (ks + 1 < 16) {
          n0 = *reinterpret_cast<const f16x8*>(krow0 + 32 * (ks + 1));
          n1 = *reinterpret_cast<const f16x8*>(krow1 + 32 * (ks + 1));
        }
      }
      const int pvi = ks / kPer, pt = pvi / NHT, pmt = pvi % NHT;   // this k-step's P.V MFMA
      if constexpr (kPV) {
        if (ks % kPer == 0 && pmt == 0) {
          bv = bvn;
          if (pt + 1 < 4) bvn = vread(pt + 1);
        }
      }
      if constexpr (kQK) {
        sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qb[ks], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qb[ks], sacc[1], 0, 0, 0);
      }
      if constexpr (kPV) {
        if (ks % kPer == 0) o[pmt][pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv, pa[pmt], o[pmt][pt], 0, 0, 0);
      }
    }
    if constexpr (kQK) {
      // validity of keys 8 g .. 8 g + 7: a selected entry with a position,
      // or a window row the query has (the decode leaves finite values in
      // the other slots, which P = 0 then drops)
      const int sub0 = (split + jq * ns) * kSub;
      const int4 pa4 = *reinterpret_cast<const int4*>(&s_pos[jq * kSub + 8 * g]);
      const int4 pb4 = *reinterpret_cast<const int4*>(&s_pos[jq * kSub + 8 * g + 4]);
      const int pos8[8] = {pa4.x, pa4.y, pa4.z, pa4.w, pb4.x, pb4.y, pb4.z, pb4.w};
      bool ok[8];
      if (sub0 + kSub <= k) {   // selected entries only (uniform)
#pragma unroll
        for (int e = 0; e < 8; ++e) ok[e] = pos8[e] >= 0;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int slot = sub0 + 8 * g + e;
          ok[e] = slot < k ? pos8[e] >= 0 : slot - k < nswa;
        }
      }
      float z[8];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * kt + i;
          const float v = ok[e] ? sacc[kt][i] * P.scale_log2 : -INFINITY;
          z[e] = v;
          mx = fmaxf(mx, v);
        }
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      // The running reference m_run moves only when a score exceeds it by more
      // than 8 (base 2): otherwise P = 2^(z - m_run) <= 256, still exact to
      // fp16's relative precision, and O and l keep their reference (the
      // softmax, and the merge of splits by their (m, l), do not depend on
      // which reference is used).  So the rescale of O is rare.
      const bool bump = mx > m_run + 8.0f;   // true on the first key (m_run = -inf)
      const float m_use = bump ? mx : m_run;
      float alpha = 1.0f, pv[8];
      if (m_use == -INFINITY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = 0.0f;
      } else {
        // the hardware 2^x: results below 2^-126, flushed, are far below
        // what the fp16 P and the fp32 sum resolve
        if (bump && m_run != -INFINITY) alpha = __builtin_amdgcn_exp2f(m_run - m_use);
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(z[e] - m_use);
      }
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ps += pv[e];
      l_run = l_run * alpha + ps;
      m_run = m_use;
      // P (fp16) of head `head`, keys 8 g .. 8 g + 7, and the head's factor
      if (head_wave) {
        f16x8 pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) pw[e] = (_Float16)pv[e];
        *reinterpret_cast<f16x8*>(&s_p[jq & 1][lrow * kPRow2 + 8 * g]) = pw;
        if (g == 0) s_alpha[jq & 1][lrow] = alpha;
      }
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;

  // O / l (or the split's normalised partial) of the wave's channel eighth,
  // sixteen consecutive channels per lane (four lanes fill a head's 64), once
  // the heads' (m, l) are in s_ml
  auto write_out = [&]() {
    // every value is scaled (and packed) before the first store, so no store
    // waits for an earlier one to release its data registers
    float inv[NHT];
#pragma unroll
    for (int mt = 0; mt < NHT; ++mt) {
      const float l = s_ml[16 * mt + n][1];   // heads past h: read, never stored
      inv[mt] = l > 0.0f ? 1.0f / l : 0.0f;
    }
#pragma unroll
    for (int mt = 0; mt < NHT; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) o[mt][t] *= inv[mt];
    if (P.nsplit == 1) {
#pragma unroll
      for (int mt = 0; mt < NHT; ++mt) {
        if (hbase + 16 * mt >= P.h) continue;
        float* dst = P.out + ((size_t)qi * P.h + hbase + 16 * mt + n) * 512 + 64 * wave + 16 * g;
#pragma unroll
        for (int t = 0; t < 4; ++t) *reinterpret_cast<f32x4*>(dst + 4 * t) = o[mt][t];
      }
    } else {
      // the split's output normalised by its own sum, rounded to fp16 (a
      // convex combination of fp16 values: in range, relative error 2^-11)
      uint32_t w[NHT][8];
#pragma unroll
      for (int mt = 0; mt < NHT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          w[mt][2 * t] = pack_f16(o[mt][t][0], o[mt][t][1]);
          w[mt][2 * t + 1] = pack_f16(o[mt][t][2], o[mt][t][3]);
        }
#pragma unroll
      for (int mt = 0; mt < NHT; ++mt) {
        if (hbase + 16 * mt >= P.h) continue;
        _Float16* dst = P.part_o + (((size_t)qi * P.nsplit + split) * P.h + hbase + 16 * mt + n) * 512 +
                        64 * wave + 16 * g;
        *reinterpret_cast<uint4*>(dst) = make_uint4(w[mt][0], w[mt][1], w[mt][2], w[mt][3]);
        *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[mt][4], w[mt][5], w[mt][6], w[mt][7]);
      }
    }
  };

  // The two roles run separate loops; both pass one barrier after the
  // prologue, one per sub-tile and one before the output.
  if (!mwave) {
    // decode assignment as k_attn's: thread -> key slots 8*kq .. 8*kq+7,
    // channels 8*cg .. 8*cg+7
    const int dt = tid - kThreads;
    const int kq = dt & 3, cg = dt >> 2;
    // The index-list loads of the first sub-tiles (when they hold selected
    // entries only) go out before the query's row base, two dependent scalar
    // loads, is waited for.
    int first_pos[kStages][8];
#pragma unroll
    for (int x = 0; x < kStages; ++x) {
      const int sub = split + x * ns;
      if (x < nmine && sub_kind(sub * kSub, k) == 0) {
        const int32_t* ip = P.idx + (size_t)qi * k + sub * kSub + 8 * kq;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) first_pos[x][jj] = ip[jj];
      }
    }
    const int64_t cbase = P.seq_base[P.q_seq[qi]];
    // Global loads of a sub-tile, one loader per slot class.  Addresses of
    // empty slots point at the fallback bytes, so no load is conditional (any
    // bytes decode to finite values, and the softmax gives those slots P = 0).
    // cq: this thread's codes dword in the query's first record (fq: in the
    // fallback bytes); sdist: the distance from it to its scale dword
    const uint8_t* const cq = P.cache + (size_t)cbase * CSA2_KV_RECORD_BYTES + 4 * cg;
    const uint8_t* const fq = fb + 4 * cg;
    const int64_t sdist = 256 + 4 * (cg >> 3) - 4 * cg;
    auto load_sel_pos = [&](Stage& st, const int pos[8]) {   // all 32 slots are selected entries
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const uint8_t* rc = pos[jj] >= 0 ? cq + (uint64_t)(uint32_t)pos[jj] * CSA2_KV_RECORD_BYTES : fq;
        st.w[jj][0] = *reinterpret_cast<const uint32_t*>(rc);
        st.w[jj][1] = *reinterpret_cast<const uint32_t*>(rc + sdist);
      }
    };
    // this thread's eight positions of local sub-tile j from the LDS copy of
    // the index list (read ahead of their loads; j past the list reads entry 0)
    auto staged_pos = [&](int j, int pos[8]) {
      const int i0 = (j < nmine ? j : 0) * kSub + 8 * kq;   // multiple of 8: two 16-byte LDS reads
      const int4 pa = *reinterpret_cast<const int4*>(&s_pos[i0]);
      const int4 pb = *reinterpret_cast<const int4*>(&s_pos[i0 + 4]);
      pos[0] = pa.x; pos[1] = pa.y; pos[2] = pa.z; pos[3] = pa.w;
      pos[4] = pb.x; pos[5] = pb.y; pos[6] = pb.z; pos[7] = pb.w;
    };
    auto load_win = [&](Stage& st, int sub) {      // all 32 slots are window rows (or past the window)
      const int r0 = sub * kSub + 8 * kq - k;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const bool ok = r0 + jj < nswa;
        const uint16_t* src =
            ok ? win_src(srow0 + r0 + jj, cg) : reinterpret_cast<const uint16_t*>(fb) + 8 * cg;
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        st.w[jj][0] = v.x; st.w[jj][1] = v.y; st.w[jj][2] = v.z; st.w[jj][3] = v.w;
      }
    };
    auto load_mixed = [&](Stage& st, int sub) {    // the one sub-tile that straddles slot k (empty slots: zeros)
      const int slot0 = sub * kSub + 8 * kq;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int slot = slot0 + jj;
        st.w[jj][0] = st.w[jj][1] = st.w[jj][2] = st.w[jj][3] = 0u;
        if (slot < k) {
          const int pos = P.idx[(size_t)qi * k + slot];
          if (pos >= 0) {
            const uint8_t* rec = P.cache + (size_t)(cbase + pos) * CSA2_KV_RECORD_BYTES;
            st.w[jj][0] = *reinterpret_cast<const uint32_t*>(rec + 4 * cg);
            st.w[jj][1] = *reinterpret_cast<const uint32_t*>(rec + 256 + 4 * (cg >> 3));
          }
        } else if (slot - k < nswa) {
          const uint4 v = *reinterpret_cast<const uint4*>(win_src(srow0 + slot - k, cg));
          st.w[jj][0] = v.x; st.w[jj][1] = v.y; st.w[jj][2] = v.z; st.w[jj][3] = v.w;
        }
      }
    };

    auto load_first = [&](Stage& st, int x) {   // local sub-tile x < kStages
      const int sub = split + x * ns;
      const int kind = sub_kind(sub * kSub, k);
      if (kind == 0) {
        load_sel_pos(st, first_pos[x]);
      } else if (kind == 1) {
        load_win(st, sub);
      } else {
        load_mixed(st, sub);
      }
    };
    auto load_next = [&](Stage& st, int j, const int pos[8]) {   // local sub-tile j >= kStages; pos: staged_pos(j)
      const int sub = split + j * ns;
      const int kind = sub_kind(sub * kSub, k);
      if (kind == 0) load_sel_pos(st, pos);
      else if (kind == 1) load_win(st, sub);
      else load_mixed(st, sub);
    };
  // Decode the loaded words to fp16 and write the key-major tile of buffer b.
    // The slot class is a compile-time argument (0: selected entries only,
    // 1: window rows only, 2: both), so a sub-tile of one class runs only its
    // own decode: the decode waves' VALU issue, which they share with the
    // multiply waves on every SIMD, is what bounds a sub-tile.
    auto store_stage = [&](const Stage& st, int sub, int b, auto cls) {
      constexpr int kCls = decltype(cls)::value;
      const int slot0 = sub * kSub;
      const int sc_shift = 8 * ((cg >> 1) & 3);   // this thread's scale byte in the loaded scale dword
      uint32_t vals[8][4];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const bool is_sel = slot0 + 8 * kq + jj < k;
        uint32_t dv[4], sv[4];
        if constexpr (kCls != 1)
          decode8(st.w[jj][0], (st.w[jj][1] >> sc_shift) & 0xFFu, dv);
        if constexpr (kCls != 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sv[j] = pack_f16(__uint_as_float(st.w[jj][j] << 16), __uint_as_float(st.w[jj][j] & 0xFFFF0000u));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (kCls == 0) vals[jj][j] = dv[j];
          else if constexpr (kCls == 1) vals[jj][j] = sv[j];
          else vals[jj][j] = is_sel ? dv[j] : sv[j];
        }
        *reinterpret_cast<uint4*>(&s_k[b][key_row(8 * kq + jj) * kKRow + 8 * cg]) =
            make_uint4(vals[jj][0], vals[jj][1], vals[jj][2], vals[jj][3]);
      }
    };

    auto store_any = [&](const Stage& st, int sub, int b) {
      const int kind = sub_kind(sub * kSub, k);
      if (kind == 0) store_stage(st, sub, b, std::integral_constant<int, 0>{});
      else if (kind == 1) store_stage(st, sub, b, std::integral_constant<int, 1>{});
      else store_stage(st, sub, b, std::integral_constant<int, 2>{});
    };

    // sub-tile x's words sit in stg[x % kStages]: the loads of kStages sub-tiles
    // ahead of the one being decoded stay in flight
    Stage stg[kStages];
#pragma unroll
    for (int x = 0; x < kStages; ++x)
      if (x < nmine) load_first(stg[x], x);
    if (nmine > 0) store_any(stg[0], split, 0);
    lds_barrier();   // s_pos and buffer 0
    if (nmine > kStages) {
      int pos[8];
      staged_pos(kStages, pos);
      load_next(stg[0], kStages, pos);
    }
    // Local sub-tiles are in ascending slot order, so the selected-only ones
    // come first.  While the sub-tile being loaded is one of them, the loop
    // below issues only the branch-free gather loads: with no load under a
    // branch, the compiler's wait before a decode counts just the older loads
    // (the newer sub-tiles' loads stay in flight).
    const int k_full = k / kSub;   // sub-tiles below this hold selected entries only
    const int n_sel = split < k_full ? min(nmine, (k_full - split + ns - 1) / ns) : 0;
    const int n_a = max(0, n_sel - 1 - kStages) / kStages * kStages;   // j < n_a: sub-tile j + 1 + kStages is selected-only
    for (int j0 = 0; j0 < n_a; j0 += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        const int j = j0 + u;
        Stage& S = stg[(u + 1) % kStages];   // sub-tile j + 1
        int pos[8];
        staged_pos(j + 1 + kStages, pos);
        if (j > 0) step(j - 1, (j - 1) % kBuf2, 0, 0, yes{}, no{});
        store_stage(S, split + (j + 1) * ns, (j + 1) % kBuf2, std::integral_constant<int, 0>{});
        load_sel_pos(S, pos);
        lds_barrier();
      }
    }
    for (int j0 = n_a; j0 < nmine; j0 += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        const int j = j0 + u;
        if (j < nmine) {   // uniform
          int pos[8];
          staged_pos(j + 1 + kStages, pos);
          if (j > 0) step(j - 1, (j - 1) % kBuf2, 0, 0, yes{}, no{});
          if (j + 1 < nmine) {
            Stage& S = stg[(u + 1) % kStages];   // sub-tile j + 1
            store_any(S, split + (j + 1) * ns, (j + 1) % kBuf2);   // its buffer was last read before the previous barrier
            if (j + 1 + kStages < nmine) load_next(S, j + 1 + kStages, pos);
          }
          lds_barrier();
        }
      }
    }
    if (nmine > 0) step(nmine - 1, (nmine - 1) % kBuf2, 0, 0, yes{}, no{});
    lds_barrier();   // the heads' (m, l)
    write_out();
    return;
  }

  // ---- multiply waves.  Their prologue issues the query loads, the copy
  // of the index list into LDS (the decode waves read their first sub-tiles'
  // positions from global memory, so no wait of theirs is behind it) and
  // the load of the query's new window row, which is stored at the end.
  uint4 qraw[16];
  if (head_wave) {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qraw[ks] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(P.q) +
                                                 ((size_t)qi * P.h + head) * 512 + 32 * ks + 8 * g);
  }
  const bool copy_row = wdst >= 0 && wdst < P.swa_rows && split == 0 && blockIdx.z == 0 && tid < 64;
  uint4 new_row{};
  if (copy_row) new_row = reinterpret_cast<const uint4*>(P.swa_new + (size_t)qi * 512)[tid];
  for (int i = tid; i < nmine * kSub; i += kThreads) {
    const int slot = (split + (i / kSub) * ns) * kSub + (i % kSub);
    if (slot < k) s_pos[i] = P.idx[(size_t)qi * k + slot];
  }
  if (head_wave) {
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint32_t wd[4] = {qraw[ks].x, qraw[ks].y, qraw[ks].z, qraw[ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qb[ks][2 * e] = (_Float16)__uint_as_float(wd[e] << 16);
        qb[ks][2 * e + 1] = (_Float16)__uint_as_float(wd[e] & 0xFFFF0000u);
      }
    }
  }
  for (int i = tid; i < 2 * 16 * NHT; i += kThreads) {   // local rows of heads past h: P = 0, factor 1
    const int bi = i & 1, r = i >> 1;
    if (hbase + r >= P.h) {
      *reinterpret_cast<f16x8*>(&s_p[bi][r * kPRow2]) = f16x8{};
      *reinterpret_cast<f16x8*>(&s_p[bi][r * kPRow2 + 8]) = f16x8{};
      *reinterpret_cast<f16x8*>(&s_p[bi][r * kPRow2 + 16]) = f16x8{};
      *reinterpret_cast<f16x8*>(&s_p[bi][r * kPRow2 + 24]) = f16x8{};
      s_alpha[bi][r] = 1.0f;
    }
  }
  lds_barrier();   // s_pos, buffer 0 and the rows of heads past h
  if (qk_wave) {
    if (nmine > 0) {
      step(0, 0, 0, 0, no{}, yes{});
      lds_barrier();
    }
    for (int j = 1; j < nmine; ++j) {
      step(j - 1, (j - 1) % kBuf2, j, j % kBuf2, yes{}, yes{});
      lds_barrier();
    }
  } else {   // P.V only, as the decode waves
    if (nmine > 0) lds_barrier();
    for (int j = 1; j < nmine; ++j) {
      step(j - 1, (j - 1) % kBuf2, 0, 0, yes{}, no{});
      lds_barrier();
    }
  }
  if (nmine > 0) step(nmine - 1, (nmine - 1) % kBuf2, 0, 0, yes{}, no{});
  if (head_wave) {
    float l_tot = l_run;
    l_tot = add_xor32(add_xor16(l_tot));
    if (g == 0) {
      s_ml[lrow][0] = m_run;
      s_ml[lrow][1] = l_tot;
    }
  }
  lds_barrier();   // the heads' (m, l)
  write_out();
  if (copy_row) reinterpret_cast<uint4*>(P.swa_out + (size_t)wdst * 512)[tid] = new_row;
  if (tid < 16 * NHT && hbase + tid < P.h) {
    const float m = s_ml[tid][0], l = s_ml[tid][1];
    const int hh = hbase + tid;
    if (P.nsplit == 1) {
      if (P.lse) P.lse[(size_t)qi * P.h + hh] = l > 0.0f ? (m + log2f(l)) * kLn2 : -INFINITY;
    } else {
      float* ml = P.part_ml + (((size_t)qi * P.nsplit + split) * P.h + hh) * 2;
      ml[0] = m;
      ml[1] = l;
    }
  }
}

// Merge split partials: with each split's normalised output o_s = O_s / l_s,
// out = sum_s 2^(m_s - M) l_s o_s / sum_s 2^(m_s - M) l_s.  One wave per
// (query, head), four heads per work-group: every lane sums channels 8 lane ..
// 8 lane + 7 over the splits in ascending order (one 16-byte fp16 load of each
// split's partial row).  The first kB splits' partial loads are issued before
// anything else, then lane s reads split s's (m_s, l_s) and forms its weight,
// which the lanes take by broadcast; more splits follow kB at a time.
__global__ __launch_bounds__(kThreads) void k_merge(Params P) {
  const int lane = threadIdx.x & 63;
  const int qi = blockIdx.x, hh = blockIdx.y * (kThreads / kWave) + (threadIdx.x >> 6);
  if (hh >= P.h) return;   // whole wave
  const int ns = P.nsplit;
  const size_t row0 = (size_t)qi * ns * P.h + hh;   // row of split 0; split s adds s * h
  const uint4* po = reinterpret_cast<const uint4*>(P.part_o + row0 * 512) + lane;
  const size_t so = (size_t)P.h * 64;   // 16-byte pieces between splits
  constexpr int kB = 16;
  uint4 x[kB];
#pragma unroll
  for (int u = 0; u < kB; ++u)
    if (u < ns) x[u] = po[(size_t)u * so];   // uniform
  float m = -INFINITY, l = 0.0f;
  if (lane < ns) {
    const float2 v = *reinterpret_cast<const float2*>(P.part_ml + (row0 + (size_t)lane * P.h) * 2);
    m = v.x;
    l = v.y;
  }
  const float M = wave_max(m);
  const float w = (lane < ns && m != -INFINITY) ? exp2f(m - M) * l : 0.0f;
  const float L = wave_sum(w);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += kB) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (s0 + u < ns) x[u] = po[(size_t)(s0 + u) * so];   // uniform
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (s0 + u < ns) {
        const float wu = __shfl(w, s0 + u, kWave);
        const f16x8 xv = __builtin_bit_cast(f16x8, x[u]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wu, (float)xv[e], acc[e]);
      }
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float* dst = P.out + ((size_t)qi * P.h + hh) * 512 + 8 * lane;
  reinterpret_cast<float4*>(dst)[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  reinterpret_cast<float4*>(dst)[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if (P.lse && lane == 0) P.lse[(size_t)qi * P.h + hh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace attn
}  // namespace csa2

using namespace csa2;
using namespace csa2::attn;

namespace {

struct Split {
  int nsub, nsplit, per;
};

#ifndef CSA2_ATTN_WG_TARGET
#define CSA2_ATTN_WG_TARGET 256   // aim for about this many work-groups per call
#endif

Split choose_split(int n_q, int k, int w_max) {
  Split s;
  const int nslots = k + w_max;
  s.nsub = std::max(1, (nslots + kSub - 1) / kSub);
  const int target = std::max(
      1, std::min({s.nsub, kMaxSplit, (CSA2_ATTN_WG_TARGET + n_q - 1) / std::max(n_q, 1)}));
  s.per = (s.nsub + target - 1) / target;
  s.nsplit = (s.nsub + s.per - 1) / s.per;
  return s;
}

// The bf16-query kernel's launch: heads per work-group (16 nht) and slot
// splits.  Fewer heads per work-group spread one query over more CUs without
// splitting its slots (fewer partials, less merge) but repeat the key decode
// per head group; more splits cost the merge.  The estimate below, in
// microseconds from MI355X measurements of each head count (a work-group's
// fixed latency and output per 16 heads, a sub-tile's time -- MFMA-bound at
// 64 heads, decode-bound below -- and the merge's launch and partial bytes),
// over whole rounds of work-groups on the CUs, picks the cheapest.
struct Plan2 {
  int nht = 4, hgroups = 1;
  Split s;
};
Plan2 plan_bf16(int n_q, int h, int k, int w_max) {
  constexpr double kFixed = 4.6, kOutPerTile = 0.6, kMerge = 5.0, kMergePerMB = 0.12;
  constexpr double kTsub[5] = {0.0, 1.3, 1.4, 0.0, 2.06};   // by nht
  Plan2 best;
  double best_cost = 1e30;
  const int ntiles = (h + 15) / 16;
  for (int nht : {4, 2, 1}) {
#ifdef CSA2_ATTN_FORCE_NHT
    if (nht != CSA2_ATTN_FORCE_NHT) continue;
#endif
    Plan2 c;
    c.nht = nht;
    c.hgroups = (ntiles + nht - 1) / nht;
    c.s = choose_split(n_q * c.hgroups, k, w_max);
#ifdef CSA2_ATTN_FORCE_SPLIT
    c.s.per = (c.s.nsub + CSA2_ATTN_FORCE_SPLIT - 1) / CSA2_ATTN_FORCE_SPLIT;
    c.s.nsplit = (c.s.nsub + c.s.per - 1) / c.s.per;
#endif
    const double wgs = (double)n_q * c.hgroups * c.s.nsplit;
    const double rounds = std::ceil(wgs / CSA2_ATTN_WG_TARGET);
    const double part_mb = c.s.nsplit > 1 ? (double)n_q * c.s.nsplit * h * 1024.0 / 1048576.0 : 0.0;
    const double cost = rounds * (kFixed + kOutPerTile * nht + c.s.per * kTsub[nht]) +
                        (c.s.nsplit > 1 ? kMerge + kMergePerMB * part_mb : 0.0);
    if (cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ws_for(int n_q, int h, int nsplit) {
  if (nsplit == 1) return 256;
  return align256((size_t)n_q * nsplit * h * 512 * sizeof(_Float16)) +
         align256((size_t)n_q * nsplit * h * 2 * sizeof(float));
}

}  // namespace

extern "C" size_t csa2_sparse_attn_ws_bytes(int n_q, int h, int k, int w_max) {
  if (n_q <= 0 || h <= 0) return 0;
  // the larger of the fp32-query and bf16-query launches' needs
  return std::max(ws_for(n_q, h, choose_split(n_q, k, w_max).nsplit),
                  ws_for(n_q, h, plan_bf16(n_q, h, k, w_max).s.nsplit));
}

namespace {

csa2_status attn_call(const void* q, int q_dtype, int n_q, int h, int d, const int32_t* q_seq,
                      const uint8_t* cache, const int64_t* seq_base, const int32_t* idx, int k,
                      const uint16_t* swa, const int64_t* swa_row0, const int32_t* swa_len, int w_max,
                      float softmax_scale, float* out, float* lse, void* ws, size_t ws_bytes, void* stream,
                      const uint16_t* swa_new, const int64_t* swa_dst, int64_t swa_rows) {
  set_last_hip_error(0);
  if (n_q < 0 || k < 0 || k > 2048 || w_max < 0 || w_max > 1024) return CSA2_E_INVAL;
  if (q_dtype != CSA2_F32 && q_dtype != CSA2_BF16) return CSA2_E_INVAL;
  if (d != CSA2_KV_CH || h < 16 || h > 64 || h % 16 != 0) return CSA2_E_UNSUPPORTED;
  if (n_q == 0) return CSA2_OK;
  if (!q || !q_seq || !seq_base || !out || !ws) return CSA2_E_INVAL;
  if (k > 0 && (!idx || !cache)) return CSA2_E_INVAL;
  if (w_max > 0 && (!swa || !swa_row0 || !swa_len)) return CSA2_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(swa) & 15) ||
      (reinterpret_cast<uintptr_t>(cache) & 3) || (reinterpret_cast<uintptr_t>(ws) & 255) ||
      (reinterpret_cast<uintptr_t>(out) & 15))
    return CSA2_E_INVAL;
  if (swa_new && (!swa || !swa_dst || swa_rows < 0 || (reinterpret_cast<uintptr_t>(swa_new) & 15) ||
                  (reinterpret_cast<uintptr_t>(swa_dst) & 7)))
    return CSA2_E_INVAL;
  if (ws_bytes < csa2_sparse_attn_ws_bytes(n_q, h, k, w_max)) return CSA2_E_WORKSPACE;
  const Plan2 plan = plan_bf16(n_q, h, k, w_max);
  const Split s = q_dtype == CSA2_F32 ? choose_split(n_q, k, w_max) : plan.s;
  Params P{};
  P.q = q; P.n_q = n_q; P.h = h; P.q_seq = q_seq; P.cache = cache; P.seq_base = seq_base;
  P.idx = idx; P.k = k; P.swa = swa; P.swa_row0 = swa_row0; P.swa_len = w_max > 0 ? swa_len : nullptr;
  P.swa_new = swa_new; P.swa_dst = swa_dst; P.swa_out = const_cast<uint16_t*>(swa); P.swa_rows = swa_rows;
  P.scale_log2 = softmax_scale * kLog2e;
  P.out = out; P.lse = lse;
  P.nsplit = s.nsplit; P.nsub = s.nsub;
  char* w = static_cast<char*>(ws);
  P.part_o = reinterpret_cast<_Float16*>(w);
  P.part_ml = reinterpret_cast<float*>(w + align256((size_t)n_q * s.nsplit * h * 512 * sizeof(_Float16)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (q_dtype == CSA2_F32) {
    hipLaunchKernelGGL(k_attn<true>, dim3(n_q, s.nsplit), dim3(kThreads), 0, st, P);
  } else {
    const dim3 grid(n_q, s.nsplit, plan.hgroups);
    if (plan.nht == 4) hipLaunchKernelGGL(k_attn2<4>, grid, dim3(2 * kThreads), 0, st, P);
    else if (plan.nht == 2) hipLaunchKernelGGL(k_attn2<2>, grid, dim3(2 * kThreads), 0, st, P);
    else hipLaunchKernelGGL(k_attn2<1>, grid, dim3(2 * kThreads), 0, st, P);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_last_hip_error((int)e);
    return CSA2_E_HIP;
  }
  if (s.nsplit > 1) {
    hipLaunchKernelGGL(k_merge, dim3(n_q, (h + 3) / 4), dim3(kThreads), 0, st, P);
    e = hipGetLastError();
    if (e != hipSuccess) {
      set_last_hip_error((int)e);
      return CSA2_E_HIP;
    }
  }
  return CSA2_OK;
}

}  // namespace

extern "C" csa2_status csa2_sparse_attn(const void* q, int q_dtype, int n_q, int h, int d,
                                        const int32_t* q_seq, const uint8_t* cache, const int64_t* seq_base,
                                        const int32_t* idx, int k, const uint16_t* swa,
                                        const int64_t* swa_row0, const int32_t* swa_len, int w_max,
                                        float softmax_scale, float* out, float* lse, void* ws,
                                        size_t ws_bytes, void* stream) {
  return attn_call(q, q_dtype, n_q, h, d, q_seq, cache, seq_base, idx, k, swa, swa_row0, swa_len, w_max,
                   softmax_scale, out, lse, ws, ws_bytes, stream, nullptr, nullptr, 0);
}

extern "C" csa2_status csa2_sparse_attn_append(const void* q, int q_dtype, int n_q, int h, int d,
                                               const int32_t* q_seq, const uint8_t* cache, const int64_t* seq_base,
                                               const int32_t* idx, int k, uint16_t* swa, int64_t swa_rows,
                                               const int64_t* swa_row0, const int32_t* swa_len, int w_max,
                                               const uint16_t* swa_new, const int64_t* swa_dst,
                                               float softmax_scale, float* out, float* lse, void* ws,
                                               size_t ws_bytes, void* stream) {
  if (!swa_new) {
    set_last_hip_error(0);
    return CSA2_E_INVAL;
  }
  return attn_call(q, q_dtype, n_q, h, d, q_seq, cache, seq_base, idx, k, swa, swa_row0, swa_len, w_max,
                   softmax_scale, out, lse, ws, ws_bytes, stream, swa_new, swa_dst, swa_rows);
}
