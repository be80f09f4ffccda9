/*
 * csa2_ref.cpp -- plain, slow, obviously correct CPU oracle of the CSA2 decode
 * hot path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, by the smoke check and by the
 * CPU-baseline leg of the benchmark, never by the product path.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Built with g++ -O2 -ffp-contract=off -fno-fast-math: every rounding below is
 * the IEEE one written in the source; std::fma appears only where the score
 * definition says fused multiply-add.  OpenMP runs independent queries in
 * parallel, which cannot change any result.
 *
 * Sources:
 *   [W1] "DeepSeek AI выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн
 *        токенов, KV-кэшем FP4 и повторным использованием внимания между
 *        слоями" (wire.sakhanda.co).
 *   [W3] "DeepSeek-V4.1-Flash: Frontier Agents on a Smaller Memory Budget"
 *        (tgviewer.app).
 * Where the pages are silent the reading taken is stated next to the code.
 */
#include "csa2_ref.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

float bits_to_float(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

uint32_t float_to_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

void set_threads(int n_threads) {
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
}

}  // namespace

/* ======================================================================
 * Formats.  The main KV stores E2M1 values with one E4M3 scale per 16
 * channels, on the NVFP4 pattern without its second-level global scale
 * [W1, FP4 section].  E4M3 is read as the OCP "FN" variant (bias 7, no
 * infinities, only S.1111.111 is NaN, largest finite 448) because that is the
 * variant NVFP4 uses.
 * ====================================================================== */

/* E2M1: 1 sign bit (bit 3), 2 exponent bits (bias 1), 1 mantissa bit.
 * Exponent field 0 is subnormal: m * 2^-1.  Otherwise 2^(e-1) * (1 + m/2). */
double csa2_ref_e2m1_value(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? m * 0.5 : std::ldexp(1.0 + m * 0.5, e - 1);
  return s ? -mag : mag;
}

/* E4M3FN: 1 sign bit (bit 7), 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal: m/8 * 2^-6.  e = 15, m = 7 is NaN. */
double csa2_ref_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  double mag = (e == 0) ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* fp32 -> bf16 by the definition of round-to-nearest-even: take the two bf16
 * neighbours of x (same sign), pick the nearer, and on a tie the one whose
 * last significand bit is 0.  Distances are exact in double. */
uint16_t csa2_ref_bf16_bits(float x) {
  uint32_t u = float_to_bits(x);
  if (std::isnan(x)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lo_bits = u & 0xFFFF0000u;          /* toward zero */
  uint32_t hi_bits = lo_bits + 0x10000u;       /* away from zero */
  double ax = std::fabs((double)x);
  double lo = std::fabs((double)bits_to_float(lo_bits));
  double hi = ((hi_bits & 0x7FFFFFFFu) == 0x7F800000u) ? std::ldexp(1.0, 128)
                                                       : std::fabs((double)bits_to_float(hi_bits));
  if (std::isinf(x)) return (uint16_t)(u >> 16);
  double dlo = ax - lo, dhi = hi - ax;
  uint32_t pick;
  if (dlo < dhi) pick = lo_bits;
  else if (dhi < dlo) pick = hi_bits;
  else pick = ((lo_bits >> 16) & 1) ? hi_bits : lo_bits;
  return (uint16_t)(pick >> 16);
}

/* Scale of one 16-channel group: the E4M3 value nearest to amax/6, ties to
 * the even code, saturating at 448, never negative.  (The pages give no
 * scale rule; amax/6 maps the group maximum onto the largest E2M1 magnitude,
 * the usual NVFP4 choice.)  Written as exact threshold tests: amax/6 passes
 * the midpoint between codes c and c+1 iff amax > 6*mid, and on equality
 * rounds to whichever of c, c+1 is even.  6*mid is exact in double. */
int csa2_ref_e4m3_round_scale(float amax) {
  double a = (double)amax;
  int code = 0;
  for (int c = 0; c < 126; ++c) {
    double mid = 0.5 * (csa2_ref_e4m3_value(c) + csa2_ref_e4m3_value(c + 1));
    double t = 6.0 * mid;
    if (a > t || (a == t && ((c + 1) % 2 == 0))) code = c + 1;
    else break;
  }
  return code;
}

/* Magnitude code of |x|/s, nearest E2M1 magnitude, ties to the even code,
 * saturating at 6.  Threshold form again: |x|/s passes mid iff |x| > s*mid
 * (s*mid exact in double), with equality going to the even code. */
int csa2_ref_e2m1_round_mag(float ax, int scale_code) {
  double s = csa2_ref_e4m3_value(scale_code);
  if (!(s > 0.0)) return 0;
  double a = std::fabs((double)ax);
  int code = 0;
  for (int c = 0; c < 7; ++c) {
    double mid = 0.5 * (csa2_ref_e2m1_value(c) + csa2_ref_e2m1_value(c + 1));
    double t = s * mid;
    if (a > t || (a == t && ((c + 1) % 2 == 0))) code = c + 1;
    else break;
  }
  return code;
}

/* ======================================================================
 * a1: quantise one 512-channel row into a 288-byte record.
 * Layout (this implementation's choice): bytes [0,256) hold the codes, byte
 * j = channel 2j in the low nibble and channel 2j+1 in the high nibble;
 * bytes [256,288) hold the scale of group g (channels 16g..16g+15) at 256+g.
 * The sign nibble bit copies the sign of x, so -0 and values that round to a
 * zero magnitude keep their sign bit.
 * ====================================================================== */
static void quant_row(const float* x, uint8_t* rec) {
  for (int g = 0; g < CSA2_REF_CH / CSA2_REF_GROUP; ++g) {
    float amax = 0.0f;
    for (int i = 0; i < CSA2_REF_GROUP; ++i) amax = std::max(amax, std::fabs(x[g * 16 + i]));
    int sc = csa2_ref_e4m3_round_scale(amax);
    rec[256 + g] = (uint8_t)sc;
    for (int i = 0; i < CSA2_REF_GROUP; ++i) {
      int ch = g * 16 + i;
      int mag = csa2_ref_e2m1_round_mag(x[ch], sc);
      int code = (std::signbit(x[ch]) ? 8 : 0) | mag;
      if (ch % 2 == 0) rec[ch / 2] = (uint8_t)((rec[ch / 2] & 0xF0) | code);
      else rec[ch / 2] = (uint8_t)((rec[ch / 2] & 0x0F) | (code << 4));
    }
  }
}

int csa2_ref_quant_append(const void* x, int x_dtype, int64_t n_rows,
                          const int64_t* dst_row, uint8_t* cache, int64_t cache_rows) {
  if (n_rows < 0 || (x_dtype != 0 && x_dtype != 1)) return 1;
  if (n_rows > 0 && (!x || !dst_row || !cache)) return 1;
  std::vector<float> row(CSA2_REF_CH);
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t d = dst_row[r];
    if (d < 0 || d >= cache_rows) continue;
    for (int c = 0; c < CSA2_REF_CH; ++c) {
      if (x_dtype == 0) row[c] = ((const float*)x)[r * CSA2_REF_CH + c];
      else row[c] = bf16_to_float(((const uint16_t*)x)[r * CSA2_REF_CH + c]);
    }
    quant_row(row.data(), cache + d * CSA2_REF_RECORD);
  }
  return 0;
}

/* Dequantised value = E2M1(code) * E4M3(scale); the product has at most six
 * significant bits, so it is exact in float. */
void csa2_ref_dequant_record(const uint8_t* rec, float* out512) {
  for (int ch = 0; ch < CSA2_REF_CH; ++ch) {
    int byte = rec[ch / 2];
    int code = (ch % 2 == 0) ? (byte & 15) : (byte >> 4);
    double s = csa2_ref_e4m3_value(rec[256 + ch / 16]);
    out512[ch] = (float)(csa2_ref_e2m1_value(code) * s);
  }
}

/* ======================================================================
 * a2: indexer score of one key for one query.  The pages name the indexer
 * (a Full layer projects an indexer K and picks Top-512 with it; a Reindex
 * layer re-scores with its own indexer Q [W1, CSA2 section]) but give no
 * formula.  Reading: one key vector per token shared by all indexer heads;
 * score = sum over heads of w_h * ReLU(q_h . k).  The arithmetic order is
 * fixed so that the selected indices are defined to the bit:
 *   acc_h = +0; for d ascending: acc_h = fma(q_h[d], k[d], acc_h)
 *   r_h = acc_h > 0 ? acc_h : +0
 *   s = +0;     for h ascending: s = fma(w_h, r_h, s)
 * ====================================================================== */
/* One head's dot product q_h . k as the fp32 fma chain over d ascending. */
static float head_dot(const uint16_t* qh, const uint16_t* key, int d_i) {
  float acc = 0.0f;
  for (int d = 0; d < d_i; ++d) acc = std::fma(bf16_to_float(qh[d]), bf16_to_float(key[d]), acc);
  return acc;
}

float csa2_ref_index_score(const uint16_t* iq, const float* w, int h_i, int d_i,
                           const uint16_t* key) {
  float s = 0.0f;
  for (int h = 0; h < h_i; ++h) {
    float acc = head_dot(iq + (size_t)h * d_i, key, d_i);
    float r = (acc > 0.0f) ? acc : 0.0f;
    s = std::fma(w[h], r, s);
  }
  return s;
}

/* Score of one pool block: the members' per-head dots summed in fp32 in
 * ascending position order from +0, divided by the member count (IEEE),
 * then ReLU and the head fma chain as for a token (reading documented at
 * csa2_ref_index_topk below). */
float csa2_ref_block_score(const uint16_t* iq, const float* w, int h_i, int d_i,
                           const uint16_t* keys, int n_members) {
  const float cnt = (float)n_members;
  float s = 0.0f;
  for (int h = 0; h < h_i; ++h) {
    float sum = 0.0f;
    for (int t = 0; t < n_members; ++t) sum = sum + head_dot(iq + (size_t)h * d_i, keys + (size_t)t * d_i, d_i);
    float mean = sum / cnt;
    float r = (mean > 0.0f) ? mean : 0.0f;
    s = std::fma(w[h], r, s);
  }
  return s;
}

/* ======================================================================
 * a4: Top-K.  Order candidates by score descending, equal scores by the
 * lower position first (-0 and +0 compare equal); keep the first min(K, n);
 * emit the kept positions in ascending order and pad with -1 to K.
 * ====================================================================== */
void csa2_ref_topk(const float* scores, const int32_t* pos, int64_t n, int k, int32_t* out) {
  std::vector<std::pair<float, int32_t>> v((size_t)n);
  for (int64_t i = 0; i < n; ++i) v[(size_t)i] = {scores[i], pos ? pos[i] : (int32_t)i};
  std::sort(v.begin(), v.end(), [](const std::pair<float, int32_t>& a,
                                   const std::pair<float, int32_t>& b) {
    if (a.first != b.first) return a.first > b.first;
    return a.second < b.second;
  });
  int64_t keep = std::min<int64_t>(k, n);
  std::vector<int32_t> sel((size_t)keep);
  for (int64_t i = 0; i < keep; ++i) sel[(size_t)i] = v[(size_t)i].second;
  std::sort(sel.begin(), sel.end());
  for (int i = 0; i < k; ++i) out[i] = (i < keep) ? sel[(size_t)i] : -1;
}

/* ======================================================================
 * a2+a4 (Full) and a3 (hierarchical pool).
 * Full scores every visible position and keeps a fresh Top-K [W1, CSA2
 * section, Full mode].  With keep_blocks > 0 it also forms the candidate pool
 * of the hierarchical indexer: positions grouped into blocks of `block`
 * (8 on the pages, at most 2048 blocks kept, so at most 16384 positions
 * [W1, CSA2 section]).  Reading (the pages give no block key): a block is
 * scored as the indexer score of the mean of its visible members' keys, with
 * the mean kept exact.  Because a dot product is linear in the key, the
 * per-head dot product of the mean key is the mean of the members' per-head
 * dot products; it is evaluated as the fp32 sum of the members' head_dot
 * values in ascending position order from +0, divided by the member count
 * (IEEE), then ReLU and the head fma chain exactly as for a token.  The kept
 * blocks are the Top-keep_blocks blocks under the same order as tokens
 * (score desc, block id asc), emitted ascending and padded with -1.
 * ====================================================================== */
int csa2_ref_index_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                        const int32_t* q_seq, const int32_t* q_nvis,
                        const uint16_t* ik, const int64_t* seq_base,
                        int k, int32_t* idx_out,
                        int block, int keep_blocks, int32_t* pool_out, int n_threads) {
  if (n_q < 0 || h_i < 1 || d_i < 1 || k < 1 || keep_blocks < 0) return 1;
  if (keep_blocks > 0 && (block < 1 || !pool_out)) return 1;
  set_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int q = 0; q < n_q; ++q) {
    const uint16_t* qv = iq + (size_t)q * h_i * d_i;
    const float* wv = w + (size_t)q * h_i;
    int64_t nvis = q_nvis[q];
    const uint16_t* keys = ik + (size_t)seq_base[q_seq[q]] * d_i;
    std::vector<float> sc((size_t)nvis);
    for (int64_t t = 0; t < nvis; ++t)
      sc[(size_t)t] = csa2_ref_index_score(qv, wv, h_i, d_i, keys + (size_t)t * d_i);
    csa2_ref_topk(sc.data(), nullptr, nvis, k, idx_out + (size_t)q * k);
    if (keep_blocks > 0) {
      int64_t nb = (nvis + block - 1) / block;
      std::vector<float> bs((size_t)nb);
      for (int64_t b = 0; b < nb; ++b) {
        int64_t t0 = b * block, t1 = std::min<int64_t>(nvis, t0 + block);
        bs[(size_t)b] = csa2_ref_block_score(qv, wv, h_i, d_i, keys + (size_t)t0 * d_i, (int)(t1 - t0));
      }
      csa2_ref_topk(bs.data(), nullptr, nb, keep_blocks, pool_out + (size_t)q * keep_blocks);
    }
  }
  return 0;
}

/* ======================================================================
 * a5: Reindex.  Re-scores the keys of the last Full layer with this layer's
 * own indexer query [W1, CSA2 section, Reindex mode], restricted to the pool
 * (the positions of the kept blocks that are visible), then Top-K as in a4.
 * pool_blocks[q][keep_blocks]: block ids, -1 entries ignored.
 * ====================================================================== */
int csa2_ref_reindex_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                          const int32_t* q_seq, const int32_t* q_nvis,
                          const uint16_t* ik, const int64_t* seq_base,
                          const int32_t* pool_blocks, int block, int keep_blocks,
                          int k, int32_t* idx_out, int n_threads) {
  if (n_q < 0 || h_i < 1 || d_i < 1 || k < 1 || keep_blocks < 1 || block < 1) return 1;
  set_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int q = 0; q < n_q; ++q) {
    const uint16_t* qv = iq + (size_t)q * h_i * d_i;
    const float* wv = w + (size_t)q * h_i;
    int64_t nvis = q_nvis[q];
    const uint16_t* keys = ik + (size_t)seq_base[q_seq[q]] * d_i;
    std::vector<float> sc;
    std::vector<int32_t> pos;
    for (int j = 0; j < keep_blocks; ++j) {
      int32_t b = pool_blocks[(size_t)q * keep_blocks + j];
      if (b < 0) continue;
      for (int o = 0; o < block; ++o) {
        int64_t p = (int64_t)b * block + o;
        if (p >= nvis) break;
        pos.push_back((int32_t)p);
        sc.push_back(csa2_ref_index_score(qv, wv, h_i, d_i, keys + (size_t)p * d_i));
      }
    }
    csa2_ref_topk(sc.data(), pos.data(), (int64_t)sc.size(), k, idx_out + (size_t)q * k);
  }
  return 0;
}

/* ======================================================================
 * Block keys for the pool-based Full variant.  The hierarchical indexer
 * groups positions into blocks of 8 and keeps at most 2048 of them [W1, CSA2
 * section]; the pages do not say how a block is scored nor whether the Full
 * layer itself picks its Top-512 inside that pool.  In the variant where it
 * does, the Full layer must not read every token key, so a block is scored
 * from a stored key of its own.  Reading: the block key is the mean of the
 * member keys, summed in fp32 from +0 in ascending position order, divided by
 * the member count (IEEE), rounded to bf16 (nearest-even); a partial last
 * block averages its members.  The block's score is then the ordinary token
 * score (csa2_ref_index_score) of that key.
 * For sequence s, blocks b with blk_from[s] <= b < ceil(seq_len[s] / block)
 * and b - blk_from[s] < max_blocks are written to kbar[kbar_base[s] + b];
 * other blocks are left alone.
 * ====================================================================== */
int csa2_ref_block_keys(const uint16_t* ik, int d_i, const int64_t* seq_base, const int32_t* seq_len,
                        const int32_t* blk_from, int n_seq, int block, int max_blocks,
                        uint16_t* kbar, const int64_t* kbar_base) {
  if (d_i < 1 || n_seq < 0 || block < 1 || max_blocks < 0) return 1;
  for (int s = 0; s < n_seq; ++s) {
    const int64_t nb = ((int64_t)seq_len[s] + block - 1) / block;
    const int64_t b1 = std::min<int64_t>(nb, (int64_t)blk_from[s] + max_blocks);
    for (int64_t b = std::max<int64_t>(0, blk_from[s]); b < b1; ++b) {
      const int64_t t0 = b * block, t1 = std::min<int64_t>(seq_len[s], t0 + block);
      const float cnt = (float)(t1 - t0);
      for (int d = 0; d < d_i; ++d) {
        float sum = 0.0f;
        for (int64_t t = t0; t < t1; ++t) sum = sum + bf16_to_float(ik[(size_t)(seq_base[s] + t) * d_i + d]);
        kbar[(size_t)(kbar_base[s] + b) * d_i + d] = csa2_ref_bf16_bits(sum / cnt);
      }
    }
  }
  return 0;
}

/* ======================================================================
 * Low-precision indexer keys (a variant; the pages do not give the indexer
 * key's precision, only that the whole model's global KV is 890 bytes per
 * token and that the main KV is FP4 [W1, opening paragraph and FP4
 * section]).  Reading: each key row is stored as OCP E4M3FN codes with one
 * power-of-two scale per row.
 *   E = the smallest integer with amax <= 448 * 2^E (amax = the row's largest
 *       magnitude), raised to at least -124 (a zero row takes -124);
 *   code_d = the E4M3FN value nearest to k_d / 2^E, ties to the even code,
 *       sign copied from k_d (so -0 gives 0x80);
 *   exponent byte = E + 127.
 * The stored key is code_d * 2^E.  An E4M3 value has at most 4 significant
 * bits and its quantum is 2^-9, so with E >= -124 every stored key element is
 * a bf16 value: the variant's indexer score is the ordinary score of these
 * bf16 keys, and its Full and Reindex selections are csa2_ref_index_topk and
 * csa2_ref_reindex_topk on them.
 * ====================================================================== */
namespace {

/* nearest E4M3FN code (sign 0) to y in [0, 448], ties to even */
int e4m3_rne_mag(double y) {
  double q;
  int e = 0;
  if (y >= std::ldexp(1.0, -6)) {
    int ex;
    std::frexp(y, &ex);        /* y = f 2^ex, f in [0.5, 1) */
    e = ex - 1;                /* y in [2^e, 2^(e+1)) */
    q = std::ldexp(1.0, e - 3);
  } else {
    q = std::ldexp(1.0, -9);   /* subnormal quantum */
  }
  double m = std::nearbyint(y / q);   /* default rounding: ties to even; y / q is exact */
  if (q == std::ldexp(1.0, -9) && y < std::ldexp(1.0, -6)) return (int)m;   /* 0..8; 8 is 2^-6 (code 0x08) */
  if (m == 16.0) {
    m = 8.0;
    e += 1;
  }
  return ((e + 7) << 3) | ((int)m - 8);
}

int fp8_key_exponent(double amax) {
  if (amax == 0.0) return -124;
  int ex;
  const double f = 2.0 * std::frexp(amax, &ex);   /* amax = f 2^(ex-1), f in [1, 2) */
  const int u = ex - 1;
  int E = f <= 1.75 ? u - 8 : u - 7;               /* 448 2^E = 1.75 2^(E+8) */
  return E < -124 ? -124 : E;
}

}  // namespace

int csa2_ref_index_keys_fp8(const uint16_t* ik, int64_t rows, int d_i, uint8_t* codes, uint8_t* exps) {
  if (rows < 0 || d_i < 1) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* k = ik + (size_t)r * d_i;
    double amax = 0.0;
    for (int d = 0; d < d_i; ++d) amax = std::max(amax, std::fabs(bf16_to_double(k[d])));
    const int E = fp8_key_exponent(amax);
    exps[r] = (uint8_t)(E + 127);
    for (int d = 0; d < d_i; ++d) {
      const double x = bf16_to_double(k[d]);
      const double y = std::ldexp(std::fabs(x), -E);   /* exact */
      codes[(size_t)r * d_i + d] = (uint8_t)(e4m3_rne_mag(y) | (std::signbit(x) ? 0x80 : 0));
    }
  }
  return 0;
}

void csa2_ref_dequant_keys_fp8(const uint8_t* codes, const uint8_t* exps, int64_t rows, int d_i, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int E = (int)exps[r] - 127;
    for (int d = 0; d < d_i; ++d) {
      const double v = std::ldexp(csa2_ref_e4m3_value(codes[(size_t)r * d_i + d]), E);
      out[(size_t)r * d_i + d] = csa2_ref_bf16_bits((float)v);   /* exact: see above */
    }
  }
}

/* ======================================================================
 * a6+a7: attention of one decode query over the selected main-KV entries
 * merged with the layer's sliding-window rows.  Every layer runs a 128-token
 * sliding window [W1, encoder-decoder section] and keeps its own main Q and
 * SWA KV [W1, CSA2 section]; Reuse layers attend with the indices of the last
 * Full/Reindex layer (same call, different q and SWA).  Readings: one
 * 512-channel vector per entry is both key and value, shared by all heads;
 * the selected entries and the window rows enter one softmax as separate
 * keys (no de-duplication); no sink, no positional rotation.  Computed in
 * double from the exact inputs, rounded to float at the end.  No valid key:
 * out = 0, lse = -inf.
 * ====================================================================== */
int csa2_ref_sparse_attn(const void* q, int q_dtype, int n_q, int h, int d,
                         const int32_t* q_seq, const uint8_t* cache, const int64_t* seq_base,
                         const int32_t* idx, int k,
                         const uint16_t* swa, const int64_t* swa_row0, const int32_t* swa_len,
                         float softmax_scale, float* out, float* lse, int n_threads) {
  if (n_q < 0 || h < 1 || d != CSA2_REF_CH || k < 0 || (q_dtype != 0 && q_dtype != 1)) return 1;
  set_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int qi = 0; qi < n_q; ++qi) {
    std::vector<std::vector<double>> keys;
    std::vector<float> rowf(CSA2_REF_CH);
    for (int j = 0; j < k; ++j) {
      int32_t p = idx[(size_t)qi * k + j];
      if (p < 0) continue;
      const uint8_t* rec = cache + (size_t)(seq_base[q_seq[qi]] + p) * CSA2_REF_RECORD;
      csa2_ref_dequant_record(rec, rowf.data());
      keys.emplace_back(rowf.begin(), rowf.end());
    }
    int nw = swa_len ? swa_len[qi] : 0;
    for (int r = 0; r < nw; ++r) {
      const uint16_t* row = swa + (size_t)(swa_row0[qi] + r) * CSA2_REF_CH;
      std::vector<double> v(CSA2_REF_CH);
      for (int c = 0; c < CSA2_REF_CH; ++c) v[(size_t)c] = bf16_to_double(row[c]);
      keys.push_back(std::move(v));
    }
    size_t nk = keys.size();
    for (int hh = 0; hh < h; ++hh) {
      std::vector<double> qv(CSA2_REF_CH);
      for (int c = 0; c < CSA2_REF_CH; ++c) {
        size_t off = ((size_t)qi * h + hh) * CSA2_REF_CH + c;
        qv[(size_t)c] = (q_dtype == 0) ? (double)((const float*)q)[off]
                                       : bf16_to_double(((const uint16_t*)q)[off]);
      }
      float* o = out + ((size_t)qi * h + hh) * CSA2_REF_CH;
      if (nk == 0) {
        for (int c = 0; c < CSA2_REF_CH; ++c) o[c] = 0.0f;
        if (lse) lse[(size_t)qi * h + hh] = -std::numeric_limits<float>::infinity();
        continue;
      }
      std::vector<double> z(nk);
      double m = -std::numeric_limits<double>::infinity();
      for (size_t j = 0; j < nk; ++j) {
        double dot = 0.0;
        for (int c = 0; c < CSA2_REF_CH; ++c) dot += qv[(size_t)c] * keys[j][(size_t)c];
        z[j] = (double)softmax_scale * dot;
        m = std::max(m, z[j]);
      }
      double l = 0.0;
      std::vector<double> acc(CSA2_REF_CH, 0.0);
      for (size_t j = 0; j < nk; ++j) {
        double p = std::exp(z[j] - m);
        l += p;
        for (int c = 0; c < CSA2_REF_CH; ++c) acc[(size_t)c] += p * keys[j][(size_t)c];
      }
      for (int c = 0; c < CSA2_REF_CH; ++c) o[c] = (float)(acc[(size_t)c] / l);
      if (lse) lse[(size_t)qi * h + hh] = (float)(m + std::log(l));
    }
  }
  return 0;
}
