/*
 * csa2.h -- C ABI of the CSA2 decode hot path for AMD Instinct MI355X (gfx950).
 *
 * CSA2 (Compressed Sparse Attention 2) gives every attention layer one of
 * three static modes.  A Full layer owns the main KV, projects an indexer key
 * from it and picks a fresh Top-512 set of positions; a Reindex layer keeps
 * the last Full layer's main KV and indexer keys but re-scores them with its
 * own indexer query; a Reuse layer takes both the main KV and the latest
 * Top-K list and skips the indexer.  Each layer keeps its own main query and
 * sliding-window (128-token) KV.  The main KV is stored as E2M1 values with
 * one E4M3 scale per 16 channels and no global scale.  In the decoder a
 * hierarchical indexer lets the Full layer build a pool of at most 2048
 * blocks of 8 positions that later Reindex layers score instead of the whole
 * context.
 *   Source: "DeepSeek AI выпустила DeepSeek-V4.1-Flash с контекстом в 1 млн
 *   токенов, KV-кэшем FP4 и повторным использованием внимания между слоями"
 *   (wire.sakhanda.co), sections "Сжатое разреженное внимание 2 (CSA2)",
 *   "FP4 KV, ограниченное повторное проигрывание и другие расширения" and
 *   "Каузальный энкодер-декодер"; also "DeepSeek-V4.1-Flash: Frontier Agents
 *   on a Smaller Memory Budget" (tgviewer.app), the CSA2 bullet.
 *
 * A decode step of one layer calls, in this order:
 *   Full:    csa2_quant_append (new rows) -> csa2_index_topk -> csa2_sparse_attn
 *   Reindex: csa2_reindex_topk -> csa2_sparse_attn
 *   Reuse:   csa2_sparse_attn with the idx of the group's Full/Reindex layer
 * with each layer's new window row written by csa2_window_append before its
 * csa2_sparse_attn (or both in one csa2_sparse_attn_append),
 * and, in the pool-based Full variant (see csa2_block_keys), a Full layer is
 *   csa2_quant_append -> csa2_block_keys (the appended position's block) ->
 *   csa2_index_topk over the block keys -> csa2_reindex_topk -> csa2_sparse_attn
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is DEVICE memory owned by the caller.  The library
 *    never allocates, frees or synchronises; scratch space is the caller's
 *    `ws` buffer of at least the size the matching *_ws_bytes function
 *    returns (its content on entry is irrelevant; it is clobbered).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; results are ready when the stream is.
 *  - Host-side argument checks fail with a status and enqueue nothing.
 *    Device-side data (positions, lengths, pool entries) is trusted to be in
 *    range; kernels clamp what they can, but out-of-range values give
 *    unspecified results.  NaN/Inf inputs are outside the contract.
 *  - Positions in idx and pool lists are relative to the sequence:
 *    0 <= p < nvis.  Row `seq_base[s] + p` addresses both the FP4 cache and
 *    the indexer-key array for position p of sequence s.
 *  - Outputs are written completely, including the -1 padding.
 *  - No device or host state is kept between calls, except two per-thread
 *    host slots: the HIP error behind the calling thread's most recent call
 *    (csa2_last_hip_error) and the measurement hook of the instrumentation
 *    section at the end (csa2_record_scan_events), which only a caller that
 *    sets it uses.  Calls on different streams may overlap if their outputs
 *    and workspaces are distinct.  No exception, abort or print ever leaves
 *    the library.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA2_OK = 0,
  CSA2_E_INVAL = 1,        /* null/unaligned pointer, negative or too large size */
  CSA2_E_UNSUPPORTED = 2,  /* shape outside the compiled set (see each call)     */
  CSA2_E_WORKSPACE = 3,    /* ws_bytes smaller than the *_ws_bytes result         */
  CSA2_E_HIP = 4           /* a HIP launch failed; see csa2_last_hip_error()      */
} csa2_status;

typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1 } csa2_dtype;

/* One main-KV entry: 512 channels quantised to E2M1 with one E4M3 (OCP FN,
 * max 448) scale per 16 channels.  288 bytes:
 *   [0, 256)   codes; byte j holds channel 2j in its low nibble and channel
 *              2j+1 in its high nibble; nibble = sign bit (bit 3) | magnitude
 *              code (0..7 = 0, .5, 1, 1.5, 2, 3, 4, 6)
 *   [256, 288) scale of group g (channels 16g..16g+15) at byte 256+g
 * The 512-channel width is this library's choice; the pages fix only the
 * formats and the 16-channel grouping. */
#define CSA2_KV_CH 512
#define CSA2_KV_GROUP 16
#define CSA2_KV_RECORD_BYTES 288

/* ------------------------------------------------------------------------
 * csa2_quant_append -- quantise rows into the FP4 main-KV cache (the write
 * side of the FP4 cache format; a Full layer owns and writes the main KV).
 *   x        [n_rows][512], fp32 (x_dtype = CSA2_F32) or bf16 bits (CSA2_BF16)
 *   dst_row  [n_rows] int64 record index of each row in `cache`; rows with an
 *            index outside [0, cache_rows) are skipped
 *   cache    [cache_rows][288] bytes, written in place
 * Per group: scale = E4M3 nearest to amax/6 (ties to even, saturating at
 * 448); code = E2M1 nearest to x/scale (ties to even, saturating at 6), sign
 * bit copied from x (so -0 gives 0x8); scale 0 gives zero magnitudes.
 * Alignment: x 16 B, dst_row 8 B, cache 4 B. */
csa2_status csa2_quant_append(const void* x, int x_dtype, int64_t n_rows,
                              const int64_t* dst_row, uint8_t* cache, int64_t cache_rows,
                              void* stream);

/* ------------------------------------------------------------------------
 * csa2_index_topk -- Full layer: indexer scan of every visible position,
 * exact Top-K, and optionally the hierarchical block pool.
 *   iq       [n_q][h_i][d_i] bf16 indexer query;  w [n_q][h_i] fp32 head weights
 *   q_seq    [n_q] sequence of each query; q_nvis [n_q] visible positions
 *            (0 <= q_nvis[i] <= max_nvis)
 *   ik       indexer keys, [rows][d_i] bf16, one key per position shared by
 *            all indexer heads; row = seq_base[q_seq[i]] + position
 *   score(p) = sum_h w[h] * ReLU(q_h . k_p), defined to the bit as:
 *            acc_h = fma chain over d ascending from +0 (fp32);
 *            s = fma chain over h ascending of w[h]*max(acc_h,0) from +0
 *   idx_out  [n_q][k]: the k positions with the largest scores (ties: lower
 *            position first), in ascending position order, -1 padded when
 *            q_nvis < k
 *   block, keep_blocks, pool_out: if keep_blocks > 0, also the pool: blocks
 *            of `block` positions (must be 8), scored as the indexer score of
 *            the mean of the block's visible keys.  Through linearity its
 *            per-head dot product is the mean of the members' per-head dot
 *            products, defined to the bit as: members' fma-chain dots summed
 *            in fp32 in ascending position from +0, divided by the member
 *            count (IEEE), then ReLU and the head fma chain as above;
 *            pool_out [n_q][keep_blocks] = the Top-keep_blocks block ids in
 *            ascending order (ties: lower id), -1 padded.  keep_blocks = 0:
 *            no pool (pool_out may be NULL).
 * The result is exact (bit-identical to the definition above) although the
 * scan runs on MFMA: candidates within a proven rounding bound of the cut
 * are re-scored with the exact fp32 chain before the final selection.
 * Supported: 1 <= h_i <= 64, d_i in {64, 128}, 1 <= k <= 2048,
 * 0 <= keep_blocks <= 4096, max_nvis <= 2^25 (32M positions).  Alignment: iq, ik 16 B. */
csa2_status csa2_index_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                            const int32_t* q_seq, const int32_t* q_nvis, int32_t max_nvis,
                            const uint16_t* ik, const int64_t* seq_base,
                            int k, int32_t* idx_out,
                            int block, int keep_blocks, int32_t* pool_out,
                            void* ws, size_t ws_bytes, void* stream);
size_t csa2_index_topk_ws_bytes(int n_q, int32_t max_nvis, int h_i, int d_i, int k,
                                int block, int keep_blocks);

/* ------------------------------------------------------------------------
 * csa2_index_topk_chunk -- Full layer for a chunk of queries of ONE sequence
 * (the encoder side: chunked prefill, where many causal queries index the same
 * keys; the encoder's CSA2 layers form groups of 1 Full + 5 Reuse at
 * compression ratio 2, source as above, section "Каузальный энкодер-декодер").
 * The same result as csa2_index_topk with every q_seq[i] naming one sequence
 * whose keys start at row ik_base, and no pool; the scan scores several
 * queries from each key group it loads, so the keys are read once per few
 * queries instead of once per query.
 *   iq, w, n_q, h_i, d_i, q_nvis, max_nvis, k, idx_out: as csa2_index_topk
 *   ik       indexer keys; query i sees rows ik_base .. ik_base + q_nvis[i] - 1
 *            (causal visibility: q_nvis per query, e.g. floor((t+1)/2) for a
 *            query at token t at compression ratio 2)
 *   ws       as csa2_index_topk with keep_blocks = 0
 *            (csa2_index_topk_ws_bytes(n_q, max_nvis, h_i, d_i, k, 8, 0))
 * Supported and alignment: as csa2_index_topk; ik_base >= 0. */
csa2_status csa2_index_topk_chunk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                  const int32_t* q_nvis, int32_t max_nvis, const uint16_t* ik,
                                  int64_t ik_base, int k, int32_t* idx_out,
                                  void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * csa2_reindex_topk -- Reindex layer: re-score the pool of the last Full
 * layer (its indexer keys `ik`) with this layer's own iq/w, exact Top-K.
 *   pool_blocks [n_q][keep_blocks] block ids as written by csa2_index_topk:
 *            ascending, distinct, -1 padded at the end.  Candidates are the
 *            positions block*8 .. block*8+7 that are < q_nvis.
 *   Other arguments and the score definition as in csa2_index_topk.
 *   idx_out  [n_q][k] ascending positions, -1 padded.
 * Supported: as csa2_index_topk, block = 8, 1 <= keep_blocks <= 4096. */
csa2_status csa2_reindex_topk(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                              const int32_t* q_seq, const int32_t* q_nvis,
                              const uint16_t* ik, const int64_t* seq_base,
                              const int32_t* pool_blocks, int block, int keep_blocks,
                              int k, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);
size_t csa2_reindex_topk_ws_bytes(int n_q, int h_i, int d_i, int k, int block, int keep_blocks);

/* ------------------------------------------------------------------------
 * csa2_reindex_topk_noalloc -- csa2_reindex_topk for callers that cannot
 * allocate device memory (code under HIP-graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and result without
 * ws / ws_bytes.  Its workspace is a fixed array of
 * CSA2_NOALLOC_SCRATCH_BYTES of device memory inside the library, one per GPU
 * it runs on, held until the process ends.  The call never allocates or
 * frees; its first call on a device (the device current on the calling
 * thread) looks up that device's array.
 *   Limit: csa2_reindex_topk_ws_bytes(n_q, h_i, d_i, k, block, keep_blocks)
 *   <= CSA2_NOALLOC_SCRATCH_BYTES (32 MiB: e.g. 64 queries at a 2048-block
 *   pool need 22 MiB, 47 queries at a 4096-block pool 31 MiB); larger calls
 *   return CSA2_E_WORKSPACE and enqueue nothing.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents: calls that overlap on one GPU (different streams or
 *   threads with no ordering between them) race and give wrong results.
 *   Calls on one stream are ordered and safe. */
#define CSA2_NOALLOC_SCRATCH_BYTES (32u << 20)
csa2_status csa2_reindex_topk_noalloc(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                      const int32_t* q_seq, const int32_t* q_nvis,
                                      const uint16_t* ik, const int64_t* seq_base,
                                      const int32_t* pool_blocks, int block, int keep_blocks,
                                      int k, int32_t* idx_out, void* stream);

/* ------------------------------------------------------------------------
 * Low-precision indexer keys (a variant).  The pages give the whole model's
 * global KV per token (890 bytes) and the main KV's FP4 format, not the
 * indexer key's precision (source as above: the opening paragraph and
 * section "FP4 KV, ограниченное повторное проигрывание и другие
 * расширения").  In this variant each key row is stored as OCP E4M3FN codes
 * with one power-of-two scale per row, 129 bytes per 128-dim key instead of
 * 256, and the score is the ordinary score (see csa2_index_topk) of the
 * stored keys, so the selections stay exact with respect to them.
 *
 * csa2_index_keys_fp8 -- quantise key rows:
 *   ik       [rows][d_i] bf16 keys;  codes [rows][d_i] E4M3FN bytes;
 *   exps     [rows] bytes, E + 127, where E is the smallest integer with
 *            max_d |ik[r][d]| <= 448 * 2^E, raised to at least -124 (a zero
 *            row takes -124);
 *   codes[r][d] = the E4M3FN value nearest to ik[r][d] / 2^E (ties to the
 *            even code, sign copied, so -0 gives 0x80).
 *   The stored key codes[r][d] * 2^E is a bf16 value (at most 4 significant
 *   bits, quantum >= 2^-133).
 * Supported: d_i in {64, 128}.  Alignment: ik 16 B, codes 8 B. */
csa2_status csa2_index_keys_fp8(const uint16_t* ik, int d_i, int64_t rows, uint8_t* codes, uint8_t* exps,
                                void* stream);

/* csa2_index_topk_fp8, csa2_reindex_topk_fp8 -- csa2_index_topk and
 * csa2_reindex_topk over FP8 keys: the same arguments, results and
 * workspace, with the key rows given as ik8 [rows][d_i] codes and ik8_exp
 * [rows] exponent bytes (as written by csa2_index_keys_fp8) instead of ik;
 * every score is that of the stored key ik8 * 2^(ik8_exp - 127).
 * Supported: d_i = 128.  Alignment: ik8 8 B. */
csa2_status csa2_index_topk_fp8(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                const int32_t* q_seq, const int32_t* q_nvis, int32_t max_nvis,
                                const uint8_t* ik8, const uint8_t* ik8_exp, const int64_t* seq_base,
                                int k, int32_t* idx_out, int block, int keep_blocks, int32_t* pool_out,
                                void* ws, size_t ws_bytes, void* stream);
csa2_status csa2_reindex_topk_fp8(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                                  const int32_t* q_seq, const int32_t* q_nvis, const uint8_t* ik8,
                                  const uint8_t* ik8_exp, const int64_t* seq_base,
                                  const int32_t* pool_blocks, int block, int keep_blocks, int k,
                                  int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * csa2_topk_merge -- exact Top-K of each query among given candidate
 * positions: the merge step of one context split over several devices.  Each
 * device runs csa2_index_topk on its position range and keeps its local
 * Top-K; the global Top-K lies in the union of the local ones and a
 * position's score does not depend on the device that computes it (defined to
 * the bit per (query, key)), so the exact Top-K among the union is the whole
 * context's (source as for csa2_index_topk: Top-512 by (score, position)).
 *   cand     [n_q][n_cand] positions of query i's sequence, ascending and
 *            distinct, -1 padded at the end (e.g. the shards' lists, each
 *            offset to global positions, concatenated in shard order)
 *   iq, w, h_i, d_i, q_seq, ik, seq_base, k: as csa2_index_topk
 *   idx_out  [n_q][k]: the k candidates with the largest scores (ties: lower
 *            position), ascending, -1 padded
 * ws: csa2_topk_merge_ws_bytes(n_q, n_cand, h_i, d_i, k) bytes (the
 * candidates' keys are gathered there, then selected exactly: by
 * csa2_reindex_topk over all their blocks of 8 when n_cand <= 16384, else by
 * csa2_index_topk; the result is the same Top-K either way).
 * Supported: as csa2_index_topk; n_cand <= 2^25, n_q <= 65535. */
csa2_status csa2_topk_merge(const uint16_t* iq, const float* w, int n_q, int h_i, int d_i,
                            const int32_t* q_seq, const uint16_t* ik, const int64_t* seq_base,
                            const int32_t* cand, int n_cand, int k, int32_t* idx_out, void* ws,
                            size_t ws_bytes, void* stream);
size_t csa2_topk_merge_ws_bytes(int n_q, int n_cand, int h_i, int d_i, int k);

/* ------------------------------------------------------------------------
 * csa2_block_keys -- stored block keys for the pool-based Full variant: a
 * Full layer that picks its Top-512 inside its own pool (the hierarchical
 * indexer's blocks of 8 positions, at most 2048 kept; source as above,
 * section "Сжатое разреженное внимание 2 (CSA2)").  Such a layer scores
 * blocks from one stored key per block instead of every token key:
 *   kbar[kbar_base[s] + b][d] = bf16_RNE( (sum over the block's positions
 *            8b .. min(8b+8, seq_len[s]) - 1, ascending, of float(ik[row][d]),
 *            fp32 from +0) / member count (IEEE) ),  row = seq_base[s] + position
 *   for every sequence s < n_seq and block b with blk_from[s] <= b <
 *   ceil(seq_len[s] / 8) and b - blk_from[s] < max_blocks; other rows of kbar
 *   are not touched.  blk_from may be NULL (every sequence from block 0).
 *   A decode step that appends position p refreshes block p / 8 only
 *   (blk_from[s] = p / 8, max_blocks = 1).
 * The variant's Full layer is then: csa2_index_topk over kbar (q_nvis =
 * ceil(visible positions / 8), seq_base = kbar_base, k = keep_blocks, no
 * pool) -> the pool's block ids, ascending; then csa2_reindex_topk with the
 * Full layer's own iq/w over that pool -> its Top-K.
 * Supported: d_i a multiple of 8 in [8, 1024], n_seq <= 65535.  Alignment:
 * ik, kbar 16 B; seq_base, kbar_base 8 B; seq_len, blk_from 4 B. */
csa2_status csa2_block_keys(const uint16_t* ik, int d_i, const int64_t* seq_base, const int32_t* seq_len,
                            const int32_t* blk_from, int n_seq, int max_blocks, uint16_t* kbar,
                            const int64_t* kbar_base, void* stream);

/* ------------------------------------------------------------------------
 * csa2_window_append -- write rows into a layer's sliding-window KV (every
 * layer keeps its own 128-token window KV; source as above, sections
 * "Каузальный энкодер-декодер" and "Сжатое разреженное внимание 2 (CSA2)").
 *   x        [n_rows][512], x_dtype CSA2_F32 (rounded to the nearest bf16,
 *            ties to even) or CSA2_BF16 (copied)
 *   dst_row  [n_rows] row of swa each row goes to; rows outside
 *            [0, swa_rows) are skipped
 *   swa      [swa_rows][512] bf16 window rows
 * Used as a ring of 128 rows per (layer, sequence): position p goes to ring
 * row p mod 128, so the ring holds the last min(L, 128) positions and
 * csa2_sparse_attn takes its first min(L, 128) rows as the window (the
 * softmax does not depend on the order of its keys).
 * Alignment: x, swa 16 B; dst_row 8 B. */
csa2_status csa2_window_append(const void* x, int x_dtype, int64_t n_rows, const int64_t* dst_row,
                               uint16_t* swa, int64_t swa_rows, void* stream);

/* ------------------------------------------------------------------------
 * csa2_sparse_attn -- gather + dequantise the selected FP4 entries and run
 * one softmax over them merged with the layer's sliding-window rows
 * (Full, Reindex and Reuse layers all use this call).
 *   q        [n_q][h][512] fp32 (q_dtype = CSA2_F32) or bf16 bits (CSA2_BF16)
 *   q_seq    [n_q]; cache [*][288] FP4 records; seq_base [n_seq] int64
 *   idx      [n_q][k] selected positions; entries < 0 are skipped
 *   swa      bf16 rows [*][512]; query i uses rows swa_row0[i] ..
 *            swa_row0[i] + swa_len[i] - 1 (0 <= swa_len[i] <= w_max)
 *   Each selected entry and each window row is one key whose vector is both
 *   key and value (shared by all heads).  For head j:
 *     z = softmax_scale * q_j . v,  out_j = sum softmax(z) v,
 *     lse_j = log sum exp(z)   (out = 0, lse = -inf when no key is valid)
 *   out [n_q][h][512] fp32; lse [n_q][h] fp32 or NULL.
 * Accuracy: main-KV values are decoded exactly; products run on fp16 MFMA
 * with fp32 accumulation (fp32 queries are split into two fp16 terms); when a
 * query's slots are split over several work-groups, each split's output,
 * normalised by its own softmax sum, is kept in fp16 (relative 2^-11) until
 * the fp32 merge;
 * bf16 queries and window rows must lie within the fp16 range (|x| < 65504).
 * Supported: d = 512, h in {16, 32, 48, 64}, 0 <= k <= 2048, 0 <= w_max <= 1024.
 * Alignment: q 16 B, swa 16 B, out 16 B, cache 4 B. */
csa2_status csa2_sparse_attn(const void* q, int q_dtype, int n_q, int h, int d,
                             const int32_t* q_seq, const uint8_t* cache, const int64_t* seq_base,
                             const int32_t* idx, int k,
                             const uint16_t* swa, const int64_t* swa_row0, const int32_t* swa_len,
                             int w_max, float softmax_scale, float* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);
/* ------------------------------------------------------------------------
 * csa2_sparse_attn_append -- csa2_window_append and csa2_sparse_attn in one
 * call (a decode step writes each layer's new window row and then attends
 * over the window that contains it; source as for both).  The same result as
 *   csa2_window_append(swa_new, CSA2_BF16, n_q, swa_dst, swa, swa_rows)
 *   followed by csa2_sparse_attn(... swa ...)
 * with one launch fewer: query i's new row swa_new[i] ([n_q][512] bf16) is
 * written to row swa_dst[i] of swa (skipped outside [0, swa_rows)), and a
 * window slot of query i on that row takes swa_new[i] directly.
 * Requirement beyond csa2_sparse_attn: a row written for query i is in no
 * other query's window of the same call (each query's ring is its own);
 * otherwise call the two entry points in order.
 * Other arguments, workspace, supported shapes and alignment: as
 * csa2_sparse_attn; swa_new 16 B, swa_dst 8 B aligned. */
csa2_status csa2_sparse_attn_append(const void* q, int q_dtype, int n_q, int h, int d,
                                    const int32_t* q_seq, const uint8_t* cache, const int64_t* seq_base,
                                    const int32_t* idx, int k, uint16_t* swa, int64_t swa_rows,
                                    const int64_t* swa_row0, const int32_t* swa_len, int w_max,
                                    const uint16_t* swa_new, const int64_t* swa_dst,
                                    float softmax_scale, float* out, float* lse, void* ws,
                                    size_t ws_bytes, void* stream);
size_t csa2_sparse_attn_ws_bytes(int n_q, int h, int k, int w_max);

/* ------------------------------------------------------------------------ */
const char* csa2_status_string(csa2_status s);
/* hipError_t behind the calling thread's most recent csa2_* call (any entry
 * point above): hipSuccess (0) unless that call returned CSA2_E_HIP.  One
 * slot per thread, cleared on entry to every call. */
int csa2_last_hip_error(void);

/* ========================================================================
 * Instrumentation (not part of the computation).
 *
 * csa2_record_scan_events -- measurement hook, the one piece of per-thread
 * state a caller sets.  The next csa2_index_topk, csa2_index_topk_chunk or
 * csa2_reindex_topk call made on the calling thread records the hipEvent_t
 * `start` right before and `stop` right after its indexer-scan kernel, on
 * that call's stream, and then forgets both (so the hook applies to exactly
 * one call).  Either may be NULL.  Lets a caller time the dominant kernel
 * with its own events while the whole step runs normally. */
void csa2_record_scan_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
