/* qsa.h — C ABI of the compressed block indexer of Qwen Sparse Attention (QSA) for AMD Instinct
 * MI355X (gfx950), built into the same library as gdn.h and sharing its status codes, dtype enum,
 * gdn_status_string() and gdn_last_error().
 *
 * What is computed (analysis notes "Qwen3.8-Flash-Next：架构、效率与技术谱系" §02 configuration
 * table, QSA indexer row, and §04 indexer data flow; paper summary "Qwen3.8-Flash-Next", QSA;
 * paper reading "On the Design of Qwen3.8-Next Architecture … 精读" §四 4.2). The indexer has
 * 4 query heads and one shared key head of dim 128 per token. For each sequence:
 *   1. compress: the keys of each complete micro-block of r = 4 tokens (tokens 4b .. 4b+3) are
 *      averaged, RMS-normalised with a gain w, and given partial RoPE at the block's first position
 *      4b -> kbar_b. Pooling comes before the rotation so that one compressed key has one position.
 *   2. score: a query at position i (its queries rotated at i) scores every block that is already
 *      complete (4b + 3 <= i) as I[i, b] = sum_h max(0, <q_ih, kbar_b>).
 *   3. select: the topk (512) highest-scoring blocks, i.e. a 2048-token budget, plus the tokens of
 *      the incomplete tail block [4 floor((i+1)/4), i], which every query keeps.
 * Readings where the pages are silent: RMSNorm is m / sqrt(mean(m^2) + norm_eps) * w; the rotary
 * part is the first rope_dims (64) dims, dim d paired with d + rope_dims/2 and turned by angle
 * pos * rope_base^(-2d/rope_dims); ties in the top-k go to the lower block index. Decode and
 * fp32-io scores are fp32 products of the rotated queries and the stored compressed keys; the bf16
 * prefill multiplies on bf16 MFMA (rotated queries rounded to bf16, fp32 accumulation). Rotation
 * angles are reduced in fp64, so they stay exact at 1M-token positions.
 *
 * Conventions are those of gdn.h (device pointers owned by the caller, work enqueued on the
 * caller's stream, host-side validation before any enqueue, 16-byte alignment, strides in
 * elements). Positions count from 0 at the first token of each sequence.
 *
 * Compressed-key cache: kbar is io [n_seqs][cap_blocks][128]; sequence n's block b is row
 * n * cap_blocks + b. cap_blocks must be at least floor(len / 4) of every sequence; blocks past
 * it are neither written nor scored. Pending keys: io [n_seqs][3][128], the keys of the current
 * incomplete block (len % 4 of them, oldest first).
 *
 * Limits: n_heads = 4, d = 128, block = 4, 1 <= topk <= 4096, rope_dims a multiple of 16 and
 * <= 128, and per query at most 16384 * floor(16384 / topk) complete blocks (2M tokens at
 * topk = 512). Selected block lists hold ascending block indices; entries past n_sel are -1.
 */
#ifndef QSA_H_
#define QSA_H_

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qsa_cfg {
  int32_t n_heads;   /* indexer query heads: 4                                   */
  int32_t d;         /* head dim of the queries and the shared key: 128          */
  int32_t block;     /* keys per micro-block (r): 4                              */
  int32_t topk;      /* blocks kept per query (K / r): 512                       */
  int32_t rope_dims; /* leading dims that are rotated: 64                        */
  int32_t io_dtype;  /* gdn_dtype of q, k, kbar and pending                      */
  float rope_base;   /* 10000                                                    */
  float norm_eps;    /* 1e-6                                                     */
} qsa_cfg;

/* Fills *cfg with the defaults above (bf16 io). */
void qsa_cfg_default(qsa_cfg* cfg);

/* Compressed keys of the packed sequences of a prefill (step 1), written into the cache.
 *   cu_seqlens       device int32 [n_seqs+1], as for gdn_prefill.
 *   cu_seqlens_host  optional host copy; when given, lengths are checked against cap_blocks
 *                    (GDN_E_SHAPE).
 *   k                io [T][128], row stride ld_k: the indexer key of every token.
 *   norm_w           fp32 [128]: RMSNorm gain.
 *   kbar             io [n_seqs][cap_blocks][128] out: blocks 0 .. floor(len/4) - 1 written.
 *   pending          io [n_seqs][3][128] out, or NULL: the len % 4 keys of the tail block.
 * n_seqs <= 65535. */
gdn_status qsa_compress(const qsa_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                        const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                        const void* k, int64_t ld_k, const float* norm_w,
                        void* kbar, int64_t cap_blocks, void* pending, void* hip_stream);

/* Bytes of workspace qsa_select and qsa_decode need to handle `rows` queries at once against
 * caches of cap_blocks blocks. Pure host computation. */
gdn_status qsa_workspace(const qsa_cfg* cfg, int64_t rows, int64_t cap_blocks, size_t* bytes);

/* Block selection for every token of a prefill (steps 2 and 3), from the cache qsa_compress filled.
 *   q        io [T][4][128], row stride ld_q (>= 512): the indexer queries, not yet rotated.
 *   sel      int32 [T][topk] out: the selected blocks of each token, ascending, -1 past n_sel.
 *   n_sel    int32 [T] out: min(topk, complete blocks).
 *   tail     int32 [T] out: first position of the token's incomplete tail block,
 *            4 floor((pos + 1) / 4); the tail is [tail, pos] (empty when tail = pos + 1).
 *   workspace  at least qsa_workspace(cfg, 1, cap_blocks) bytes; the tokens are processed in
 *            groups of as many as fit, so qsa_workspace(cfg, T, cap_blocks) bytes run them in one. */
gdn_status qsa_select(const qsa_cfg* cfg, int32_t n_seqs, int64_t total_tokens,
                      const int32_t* cu_seqlens, const void* q, int64_t ld_q,
                      const void* kbar, int64_t cap_blocks, int32_t* sel, int32_t* n_sel,
                      int32_t* tail, void* workspace, size_t workspace_bytes, void* hip_stream);

/* One decode step of the indexer for `batch` sequences, one new token each: the token's key joins
 * the pending block (and when it completes the block, the block is compressed into kbar), then
 * the token's queries select their blocks as in qsa_select.
 *   n_tok    device int32 [B]: tokens of each sequence including this one (its position + 1).
 *            Sequences with n_tok < 1 append nothing and select nothing.
 *   q        io [B][4][128], row stride ld_q;  k  io [B][128], row stride ld_k.
 *   norm_w   fp32 [128].
 *   pending  io [B][3][128], updated in place;  kbar  io [B][cap_blocks][128], updated in place.
 *   sel, n_sel, tail  as for qsa_select, one row per sequence.
 *   workspace  at least qsa_workspace(cfg, B, cap_blocks) bytes.
 * The call enqueues kernels only (no allocation, copy or memset), so a serving loop can capture it in a
 * HIP graph once and replay it with new n_tok, q and k in the same buffers. */
gdn_status qsa_decode(const qsa_cfg* cfg, int32_t batch, const int32_t* n_tok, const void* q, int64_t ld_q,
                      const void* k, int64_t ld_k, const float* norm_w, void* pending, void* kbar,
                      int64_t cap_blocks, int32_t* sel, int32_t* n_sel, int32_t* tail,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
