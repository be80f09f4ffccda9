/*
 * csa2_ref.h -- plain CPU oracle for the CSA2 decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load or call this library.  The
 * product path (the HIP library and its Python binding) never calls it, and
 * this code shares nothing with the HIP sources.
 *
 * Sources (cited by page title and section, no line numbers):
 *   [W1] "DeepSeek AI выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн
 *        токенов, KV-кэшем FP4 и повторным использованием внимания между
 *        слоями" (wire.sakhanda.co), sections "Каузальный энкодер-декодер",
 *        "Сжатое разреженное внимание 2 (CSA2)", "FP4 KV, ограниченное
 *        повторное проигрывание и другие расширения".
 *   [W3] "DeepSeek-V4.1-Flash: Frontier Agents on a Smaller Memory Budget"
 *        (tgviewer.app), the CSA2 bullet.
 *
 * Every function takes host memory and mirrors the argument meaning of the
 * corresponding csa2_* entry point of the HIP library (no workspace, no
 * stream).  Return value: 0 on success, 1 on invalid arguments.
 */
#ifndef CSA2_REF_H
#define CSA2_REF_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Record layout of one 512-channel main-KV entry (the pages fix E2M1 codes
 * with one E4M3 scale per 16 channels [W1, FP4 section]; 512 channels and the
 * byte order are this implementation's choice). */
#define CSA2_REF_CH 512
#define CSA2_REF_GROUP 16
#define CSA2_REF_RECORD 288

/* ---- formats (E2M1 / E4M3FN / bf16) ---------------------------------- */
double   csa2_ref_e2m1_value(int code);           /* code 0..15 */
double   csa2_ref_e4m3_value(int code);           /* code 0..255, NaN for 0x7F/0xFF */
uint16_t csa2_ref_bf16_bits(float x);             /* fp32 -> bf16, nearest-even */
int      csa2_ref_e4m3_round_scale(float amax);   /* nearest E4M3 to amax/6, ties even, saturating */
int      csa2_ref_e2m1_round_mag(float ax, int scale_code); /* magnitude code of |x| / scale */

/* ---- a1: quantise-and-append ----------------------------------------- */
/* x: [n_rows][512], x_dtype 0 = fp32, 1 = bf16 (uint16 bits).
 * Row i goes to record dst_row[i] of cache[cache_rows][288]; rows outside
 * [0, cache_rows) are skipped. */
int csa2_ref_quant_append(const void* x, int x_dtype, int64_t n_rows,
                          const int64_t* dst_row, uint8_t* cache, int64_t cache_rows);
void csa2_ref_dequant_record(const uint8_t* rec, float* out512);

/* ---- a2: canonical indexer score -------------------------------------- */
float csa2_ref_index_score(const uint16_t* iq, const float* w, int h_i, int d_i,
                           const uint16_t* key);

/* ---- a3: score of one pool block of n_members consecutive keys (the mean of
 *      the members' per-head dots, fp32 sum ascending, IEEE division) ------ */
float csa2_ref_block_score(const uint16_t* iq, const float* w, int h_i, int d_i,
                           const uint16_t* keys, int n_members);

/* ---- a4: Top-K by (score desc, position asc), output ascending, -1 pad - */
void csa2_ref_topk(const float* scores, const int32_t* pos, int64_t n, int k, int32_t* out);

/* ---- a2+a3+a4: Full layer --------------------------------------------- */
int csa2_ref_index_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                        const int32_t* q_seq, const int32_t* q_nvis,
                        const uint16_t* ik, const int64_t* seq_base,
                        int k, int32_t* idx_out,
                        int block, int keep_blocks, int32_t* pool_out, int n_threads);

/* ---- a5: Reindex layer ------------------------------------------------ */
int csa2_ref_reindex_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                          const int32_t* q_seq, const int32_t* q_nvis,
                          const uint16_t* ik, const int64_t* seq_base,
                          const int32_t* pool_blocks, int block, int keep_blocks,
                          int k, int32_t* idx_out, int n_threads);

/* ---- pool-based Full variant: stored block keys ------------------------
 * kbar[kbar_base[s] + b][d] = bf16(mean of the block's member keys, fp32 sum
 * in ascending order), for blocks blk_from[s] <= b < ceil(seq_len[s]/block),
 * at most max_blocks of them per sequence. */
int csa2_ref_block_keys(const uint16_t* ik, int d_i, const int64_t* seq_base, const int32_t* seq_len,
                        const int32_t* blk_from, int n_seq, int block, int max_blocks,
                        uint16_t* kbar, const int64_t* kbar_base);

/* ---- FP8 indexer keys (variant): per row, E = smallest integer with
 *      amax <= 448 * 2^E, at least -124; code = nearest E4M3FN to k / 2^E
 *      (ties even, sign copied); exps[r] = E + 127.  The stored key
 *      code * 2^E is a bf16 value. ------------------------------------------- */
int csa2_ref_index_keys_fp8(const uint16_t* ik, int64_t rows, int d_i, uint8_t* codes, uint8_t* exps);
void csa2_ref_dequant_keys_fp8(const uint8_t* codes, const uint8_t* exps, int64_t rows, int d_i, uint16_t* out);

/* ---- a6+a7(+a8): sparse attention over selected FP4 entries + SWA ------ */
int csa2_ref_sparse_attn(const void* q, int q_dtype, int n_q, int h, int d,
                         const int32_t* q_seq, const uint8_t* cache, const int64_t* seq_base,
                         const int32_t* idx, int k,
                         const uint16_t* swa, const int64_t* swa_row0, const int32_t* swa_len,
                         float softmax_scale, float* out, float* lse, int n_threads);

#ifdef __cplusplus
}
#endif
#endif
