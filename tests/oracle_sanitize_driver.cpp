// Runs every entry point of the CPU oracle on small seeded inputs, including
// the edge cases (empty contexts, fewer candidates than K, padding entries,
// rows outside the cache, partial blocks), so that a build with AddressSanitizer
// and UndefinedBehaviorSanitizer can check the oracle's memory accesses and
// arithmetic.  Test infrastructure: built and run by
// tests/test_oracle_sanitizers.py; it computes nothing of the method itself
// (inputs from a fixed linear congruential generator, results only checked
// for shape-level sanity), and exits 0 when every call returned.
#include "csa2_ref.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

uint64_t g_state = 0x243F6A8885A308D3ull;
uint32_t next_u32() {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_state >> 32);
}
float next_normalish() {   // sum of uniforms, centred: enough spread for the scores
  float s = 0.0f;
  for (int i = 0; i < 4; ++i) s += (float)(next_u32() >> 8) * (1.0f / 16777216.0f);
  return (s - 2.0f) * 1.7f;
}
uint16_t bf16_of(float x) {   // truncation is enough for test inputs
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}
void fill_bf16(std::vector<uint16_t>& v) {
  for (auto& x : v) x = bf16_of(next_normalish());
}
void fill_f32(std::vector<float>& v, float lo, float hi) {
  for (auto& x : v) x = lo + (hi - lo) * (float)(next_u32() >> 8) * (1.0f / 16777216.0f);
}
int fails = 0;
void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "unexpected: %s\n", what);
    ++fails;
  }
}

}  // namespace

int main() {
  // ---- formats
  for (int c = 0; c < 16; ++c) expect(std::isfinite(csa2_ref_e2m1_value(c)), "e2m1 value finite");
  for (int c = 0; c < 256; ++c) (void)csa2_ref_e4m3_value(c);
  const float specials[] = {0.0f, -0.0f, 1.0f, -3.5f, 1e-40f, -1e-45f, 3.4e38f, INFINITY, -INFINITY, NAN};
  for (float x : specials) (void)csa2_ref_bf16_bits(x);
  for (float a : {0.0f, 1e-30f, 0.5f, 6.0f, 448.0f * 6.0f, 1e6f, INFINITY}) {
    const int s = csa2_ref_e4m3_round_scale(a);
    expect(s >= 0 && s < 256, "scale code in range");
    for (float x : {0.0f, 0.1f, 1.0f, 5.9f, 1e7f}) (void)csa2_ref_e2m1_round_mag(x, s);
  }

  // ---- a1: quantise-append, fp32 and bf16 rows, rows outside the cache skipped
  const int ch = CSA2_REF_CH;
  const int64_t cache_rows = 8;
  std::vector<uint8_t> cache(cache_rows * CSA2_REF_RECORD, 0);
  std::vector<float> x32(5 * ch);
  fill_f32(x32, -10.0f, 10.0f);
  for (int j = 0; j < ch; j += 16) x32[j] = 0.0f;   // a row group with a zero
  std::vector<uint16_t> x16(5 * ch);
  fill_bf16(x16);
  const int64_t dst[5] = {0, 7, -1, 8, 3};
  expect(csa2_ref_quant_append(x32.data(), 0, 5, dst, cache.data(), cache_rows) == 0, "quant fp32");
  expect(csa2_ref_quant_append(x16.data(), 1, 5, dst, cache.data(), cache_rows) == 0, "quant bf16");
  std::vector<float> deq(ch);
  for (int r = 0; r < cache_rows; ++r) csa2_ref_dequant_record(cache.data() + r * CSA2_REF_RECORD, deq.data());

  // ---- index keys and queries: 4 sequences, lengths 0, 1, 37 and 300
  const int h_i = 4, d_i = 64, n_q = 4, block = 8;
  const int lens[n_q] = {0, 1, 37, 300};
  int64_t total = 0;
  std::vector<int64_t> seq_base(n_q);
  for (int s = 0; s < n_q; ++s) {
    seq_base[s] = total;
    total += lens[s];
  }
  std::vector<uint16_t> ik(std::max<int64_t>(total, 1) * d_i);
  fill_bf16(ik);
  std::vector<uint16_t> iq(n_q * h_i * d_i);
  fill_bf16(iq);
  std::vector<float> w(n_q * h_i);
  fill_f32(w, 0.0f, 1.0f);
  std::vector<int32_t> q_seq(n_q), q_nvis(n_q);
  for (int q = 0; q < n_q; ++q) {
    q_seq[q] = q;
    q_nvis[q] = lens[q];
  }
  (void)csa2_ref_index_score(iq.data(), w.data(), h_i, d_i, ik.data());
  for (int m = 1; m <= block; ++m) (void)csa2_ref_block_score(iq.data(), w.data(), h_i, d_i, ik.data(), m);

  // ---- a4: Top-K with fewer candidates than K, ties and an empty set
  {
    std::vector<float> sc = {1.0f, 3.0f, 3.0f, -0.0f, 0.0f, 2.0f};
    std::vector<int32_t> pos = {5, 1, 9, 2, 3, 7}, out(8);
    csa2_ref_topk(sc.data(), pos.data(), (int64_t)sc.size(), 4, out.data());
    csa2_ref_topk(sc.data(), pos.data(), (int64_t)sc.size(), 8, out.data());
    csa2_ref_topk(sc.data(), pos.data(), 0, 8, out.data());
  }

  // ---- a2+a3+a4: Full layer with and without a pool; a5: Reindex over the pool
  const int k = 16, keep = 4;
  std::vector<int32_t> idx(n_q * k), pool(n_q * keep), idx2(n_q * k);
  expect(csa2_ref_index_topk(iq.data(), w.data(), n_q, h_i, d_i, q_seq.data(), q_nvis.data(), ik.data(),
                             seq_base.data(), k, idx.data(), block, 0, nullptr, 1) == 0, "full, no pool");
  expect(csa2_ref_index_topk(iq.data(), w.data(), n_q, h_i, d_i, q_seq.data(), q_nvis.data(), ik.data(),
                             seq_base.data(), k, idx.data(), block, keep, pool.data(), 2) == 0, "full, pool");
  for (int q = 0; q < n_q; ++q)
    for (int i = 0; i < k; ++i) expect(idx[q * k + i] >= -1 && idx[q * k + i] < lens[q], "index in range");
  expect(csa2_ref_reindex_topk(iq.data(), w.data(), n_q, h_i, d_i, q_seq.data(), q_nvis.data(), ik.data(),
                               seq_base.data(), pool.data(), block, keep, k, idx2.data(), 1) == 0, "reindex");

  // ---- pool-based Full variant: block keys from block 0 and from a later block
  {
    std::vector<int32_t> seq_len(lens, lens + n_q), blk_from = {0, 0, 2, 5};
    std::vector<int64_t> kbar_base(n_q);
    int64_t nb = 0;
    for (int s = 0; s < n_q; ++s) {
      kbar_base[s] = nb;
      nb += (lens[s] + block - 1) / block;
    }
    std::vector<uint16_t> kbar(std::max<int64_t>(nb, 1) * d_i, 0);
    expect(csa2_ref_block_keys(ik.data(), d_i, seq_base.data(), seq_len.data(), blk_from.data(), n_q, block, 64,
                               kbar.data(), kbar_base.data()) == 0, "block keys");
  }

  // ---- FP8 indexer keys: quantise and dequantise every row, a zero row included
  {
    std::vector<uint16_t> rows(ik.begin(), ik.begin() + 8 * d_i);
    for (int d = 0; d < d_i; ++d) rows[3 * d_i + d] = 0;
    std::vector<uint8_t> codes(8 * d_i), exps(8);
    std::vector<uint16_t> back(8 * d_i);
    expect(csa2_ref_index_keys_fp8(rows.data(), 8, d_i, codes.data(), exps.data()) == 0, "fp8 keys");
    csa2_ref_dequant_keys_fp8(codes.data(), exps.data(), 8, d_i, back.data());
  }

  // ---- a6+a7: sparse attention, fp32 and bf16 queries, padding and window rows
  {
    const int h = 16, ka = 6, na = 2;
    std::vector<int32_t> aq_seq = {0, 0}, aidx = {0, 7, -1, 3, 3, -1, -1, -1, -1, -1, -1, -1};
    std::vector<int64_t> abase = {0}, srow0 = {0, 2};
    std::vector<int32_t> slen = {2, 0};
    std::vector<uint16_t> swa(4 * ch);
    fill_bf16(swa);
    std::vector<float> q32(na * h * ch), out(na * h * ch), lse(na * h);
    fill_f32(q32, -1.0f, 1.0f);
    std::vector<uint16_t> q16(na * h * ch);
    fill_bf16(q16);
    expect(csa2_ref_sparse_attn(q32.data(), 0, na, h, ch, aq_seq.data(), cache.data(), abase.data(), aidx.data(), ka,
                                swa.data(), srow0.data(), slen.data(), 0.044f, out.data(), lse.data(), 1) == 0,
           "attention fp32");
    expect(csa2_ref_sparse_attn(q16.data(), 1, na, h, ch, aq_seq.data(), cache.data(), abase.data(), aidx.data(), ka,
                                swa.data(), srow0.data(), slen.data(), 0.044f, out.data(), nullptr, 2) == 0,
           "attention bf16");
    // the second query has no valid key at all: output 0, lse -inf
    expect(std::isinf(lse[h]) && lse[h] < 0.0f, "no key gives lse -inf");
  }

  std::printf("oracle sanitizer driver: %s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
