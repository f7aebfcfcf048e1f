/*
 * CPU oracle for single-query GQA decode attention — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 reference of what the decode path computes.  Only the
 * tests, the package smoke check and the benchmark's CPU-baseline leg may
 * load it; the product library never links or calls it.  It shares no code
 * with the GPU library: own types, own helpers, own constants.
 *
 * Sources (page titles as printed on each page):
 *  - "优化稀疏注意力中的令牌丢弃机制" (lzwjava.github.io), §2 attention output,
 *    §3 OAM score pseudo-code, §5 split-KV cross-shard online softmax, §6 INT8
 *    per-tensor / per-token-partition quantisation.
 *  - "注意力优化（Attention Optimization）" (learnagent.wiki), softmax(QK^T/sqrt(d_k))V
 *    formula, Flash Attention block pseudo-code, GQA repeat_interleave example.
 *  - "共同设计 AI 模型注意力…" (NVIDIA developer blog), decode FLOPs/bytes
 *    equations 5-7, G = query heads per KV head.
 *
 * All pointers are HOST pointers.  Every entry returns 0 on success and a
 * non-zero code for invalid arguments.
 */
#ifndef LCDG_ORACLE_H
#define LCDG_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_I8 = 2 };

/*
 * A decode problem.  Row (b, kh, t) of K (and of V) starts at element
 * seq_offset[b] + kh*stride_h + t*stride_t and holds D contiguous values.
 * Q is [B][KH*G][D]; query head qh = kh*G + g reads KV head kh = qh / G.
 * INT8 K: value = code * k_scale[(b*KH + kh)*k_scale_stride + t / k_part];
 * INT8 V: value = code * v_scale.
 * INT8 Q (q_type ORACLE_I8): value = code * q_scale[b*KH*G + qh].
 * If tok_idx is not NULL, (b, kh) attends only to the tokens
 * tok_idx[(b*KH + kh)*idx_stride + j], j < n_idx[b*KH + kh].
 */
typedef struct {
  int32_t B, KH, G, D;
  const int32_t *lens;
  const int64_t *seq_offset;
  int64_t stride_h, stride_t;
  int32_t q_type, kv_type;
  const void *q, *k, *v;
  const float *k_scale;
  int32_t k_part, k_scale_stride;
  float v_scale;
  double softmax_scale;
  const int32_t *tok_idx, *n_idx;
  int32_t idx_stride;
  const float *q_scale;
} oracle_problem;

/* Plain definition: out = sum_t softmax_t(s) v_t, lse = log sum_t exp(s_t). */
int oracle_attention_rows(const oracle_problem *p, int32_t nrows, const int32_t *row_b,
                          const int32_t *row_qh, double *out, double *lse, int32_t nthreads);

/* Second, independent form: the block-online recurrence (running m, l, O). */
int oracle_attention_rows_online(const oracle_problem *p, int32_t nrows, const int32_t *row_b,
                                 const int32_t *row_qh, int32_t block, double *out, double *lse);

/* Partial triple of one row over token positions [t0, t1) (positions index
 * the token list when tok_idx is set): m = max score, l = sum exp(s - m),
 * o = sum exp(s - m) v / l.  An empty range gives m = -inf, l = 0, o = 0. */
int oracle_partial(const oracle_problem *p, int32_t b, int32_t qh, int32_t t0, int32_t t1,
                   double *m, double *l, double *o);

/* Log-sum-exp merge of n partial triples (o is [n][D]). */
int oracle_merge(int32_t n, int32_t D, const double *m, const double *l, const double *o,
                 double *out, double *lse);

/* INT8, one scale per (b, kh, part-token partition aligned at token 0):
 * scale = fl32(max|x| / 127), code = clamp(rne(fl32(x / scale)), -127, 127).
 * codes use the same geometry as x; scales[(b*KH+kh)*scale_stride + t/part]. */
int oracle_quant_partitions(int32_t B, int32_t KH, int32_t D, const int32_t *lens,
                            const int64_t *seq_offset, int64_t stride_h, int64_t stride_t,
                            const uint16_t *x_bf16, int32_t part, int8_t *codes, float *scales,
                            int32_t scale_stride);

/* INT8 with one scale for the whole tensor (all b, kh, t < lens[b], d). */
int oracle_quant_tensor(int32_t B, int32_t KH, int32_t D, const int32_t *lens,
                        const int64_t *seq_offset, int64_t stride_h, int64_t stride_t,
                        const uint16_t *x_bf16, int8_t *codes, float *scale);

/* INT8 query of the page's Schemes A and B (§6: the query quantised in
 * per-token partitions).  A decode step has one token per sequence, so each
 * query row (b, qh) of D values is one partition: scales[r] = max|x_r| / 127
 * and codes by the rule above.  x_bf16 is [rows][D]. */
int oracle_quant_rows(int32_t rows, int32_t D, const uint16_t *x_bf16, int8_t *codes, float *scales);

/* INT8 codes of n values with a given (static, calibrated) per-tensor scale:
 * the page's baseline scheme; quotients beyond 127 clamp. */
int oracle_quant_static(int64_t n, const uint16_t *x_bf16, float scale, int8_t *codes);

/* OAM score of every token of (b, kh):
 * score_t = mean_g (q_g . k_t) * softmax_scale + beta * ln(||v_t||_2 + eps). */
int oracle_oam_scores(const oracle_problem *p, int32_t b, int32_t kh, double beta, double eps,
                      double *scores);

/* ln(||v_t||_2 + eps) of every token of (b, kh). */
int oracle_value_lognorm(const oracle_problem *p, int32_t b, int32_t kh, double eps, double *out);

/* Top-k by (score descending, index ascending); writes min(k, L) indices in
 * ascending order and returns that count (negative on error).  The first
 * form sorts everything; the second uses a selection followed by a sort. */
int32_t oracle_topk_sort(const double *scores, int32_t L, int32_t k, int32_t *idx_out);

/* Block-granular selection ("NSA" page §2.1, selected attention: the top-n
 * blocks of contiguous tokens by an importance shared by the GQA group).
 * The page's importance comes from a learned compression of each block;
 * with that compression taken as the mean over the block (a reading), a
 * block's score is the mean of its tokens' scores (token scores as in
 * oracle_oam_scores with the given beta and eps; beta = 0 gives the plain
 * routing logits).  Blocks are [j*block_tokens, min((j+1)*block_tokens, L))
 * of (b, kh); the n_blocks best by (score descending, block index ascending)
 * are kept, and their token indices are written to idx_out in ascending
 * order.  block_scores (optional) receives every block's score.  Returns
 * the number of kept tokens, or -1 on invalid arguments. */
int32_t oracle_block_select(const oracle_problem *p, int32_t b, int32_t kh, int32_t block_tokens, int32_t n_blocks,
                            double beta, double eps, int32_t *idx_out, double *block_scores);
int32_t oracle_topk_select(const double *scores, int32_t L, int32_t k, int32_t *idx_out);

#ifdef __cplusplus
}
#endif
#endif
