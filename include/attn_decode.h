/*
 * attn_decode.h — C ABI of the MI355X (gfx950) single-query GQA decode
 * attention library (libattn_decode.so).
 *
 * What the library computes, and where the pages define it:
 *  - Decode attention of one new query per head over a long KV cache,
 *    out = sum_t softmax_t(q.k_t / sqrt(d)) v_t ("优化稀疏注意力中的令牌丢弃机制"
 *    §2; "注意力优化（Attention Optimization）" 原理说明, softmax(QK^T/sqrt(d_k))V).
 *  - Grouped-query attention: G query heads share one KV head; query head
 *    qh = kh*G + g reads KV head kh ("注意力优化" 结构 2 and its GQA
 *    repeat_interleave example; the NVIDIA blog "共同设计 AI 模型注意力…",
 *    section 组规模, where G is the number of query heads per KV head).
 *  - Flash-style tiling with an online softmax (running max m, sum l,
 *    rescaled output) ("注意力优化" Flash Attention pseudo-code; NVIDIA blog,
 *    section on how FlashAttention kernels compute attention).
 *  - Split-KV: each sequence is cut into chunks processed in parallel whose
 *    partial (max, sum-exp, output) triples are merged with the log-sum-exp
 *    rule, with work balanced over variable-length sequences
 *    ("优化稀疏注意力中的令牌丢弃机制" §5, Split-KV method and its cross-shard
 *    online softmax).
 *  - INT8 KV: q_val = round(val/scale); K scale per token partition
 *    (scale = max|k| / 127 over the partition), V one per-tensor scale
 *    ("优化稀疏注意力中的令牌丢弃机制" §6, per-tensor baseline and Scheme A).
 *  - Output-aware token dropping (OAM): score_i = q.k_i/sqrt(d) +
 *    beta*log(||v_i|| + eps), keep the top-K, attend exactly to those
 *    ("优化稀疏注意力中的令牌丢弃机制" §3 pseudo-code and §7 composition).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless a comment says otherwise.  The caller
 *    owns every buffer, including workspaces; the library never allocates or
 *    frees device memory and keeps no pointer after a call returns (the one
 *    exception: attn_decode_splitkv_noalloc's static scratch array, which the
 *    library's code object holds on each GPU).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  Outputs are valid once the stream reaches that point.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    failed validation returns a status and enqueues nothing.  A failed
 *    launch returns ATTN_ERR_HIP.  attn_last_error() describes the most
 *    recent failure of the calling thread.  No C++ exception crosses the ABI.
 *  - Calls hold no global state besides a per-device cache of the compute
 *    unit count (and, for attn_decode_splitkv_noalloc, of its scratch
 *    address); they are safe to call from several host threads.  Calls that
 *    share a workspace must be ordered on one stream.
 *  - Non-finite inputs give undefined (but memory-safe) results.
 *  - Element types: ATTN_F32 = IEEE fp32, ATTN_BF16 = bfloat16,
 *    ATTN_I8 = int8 codes with fp32 scales.
 */
#ifndef LCDG_ATTN_DECODE_H
#define LCDG_ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *attn_stream_t; /* a hipStream_t */

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,
  ATTN_ERR_UNSUPPORTED = 2,
  ATTN_ERR_WORKSPACE_TOO_SMALL = 3,
  ATTN_ERR_HIP = 4
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_I8 = 2 } attn_dtype;

/* How the query enters the int8 matrix cores with ATTN_I8 KV
 * ("优化稀疏注意力中的令牌丢弃机制" §6, the scheme table: the baseline scheme
 * quantises Q with one static per-tensor scale, Schemes A and B in per-token
 * partitions). */
typedef enum {
  ATTN_QUANT_EXACT = 0,  /* no query quantisation (22-bit fixed point, below) */
  ATTN_QUANT_ROW = 1,    /* int8, one scale per query row (b, qh) */
  ATTN_QUANT_STATIC = 2  /* int8, one static per-tensor scale given by the caller */
} attn_q_quant;

/*
 * KV-cache geometry shared by all calls (the problem statement of the NVIDIA
 * blog's decode equations: batch DB = B, KV heads KH, head size Hsz = D,
 * per-sequence KV length).  Row (b, kh, t) of K (or V) holds D contiguous
 * elements starting at element seq_offset[b] + kh*stride_h + t*stride_t of
 * the tensor.  This covers [B][KH][L][D], packed token-major [sum L][KH][D]
 * and packed head-major [KH][sum L][D] caches.
 *   B, KH, D      host ints; B >= 0, KH >= 1, D in {64, 128} for bf16/int8
 *                 KV, D in [4, 256] and a multiple of 4 for fp32 KV
 *   max_seq_len   host int >= every seq_lens[b]; sizes workspaces and
 *                 scale tables (it is not checked against the device data)
 *   seq_lens      device int32[B], 0 <= L_b <= max_seq_len
 *   seq_offset    device int64[B], element offsets, >= 0
 *   stride_h, stride_t  element strides, >= D; every row must be 16-byte
 *                 aligned (so offsets and strides are multiples of 8 bf16 /
 *                 4 fp32 / 16 int8 elements)
 * Paged cache ("注意力优化" 结构 4, PagedAttention: the cache is cut into
 * fixed-size pages allocated on demand), optional: when block_table is not
 * NULL, row (b, kh, t) starts at element
 *   block_table[b*table_stride + t/page_tokens]*page_stride + kh*stride_h
 *   + (t % page_tokens)*stride_t
 * of a page pool, and seq_offset is ignored.
 *   block_table   device int32, page ids >= 0, table_stride >=
 *                 ceil(max_seq_len / page_tokens) entries per sequence
 *   page_tokens   tokens per page, a positive multiple of 32
 *   page_stride   elements between pages, > 0, 16-byte aligned
 * attn_decode_splitkv (bf16 or int8 KV, no token_idx), kv_quant_int8 (the
 * codes go to the same rows of a pool with the same geometry),
 * oam_value_lognorm and oam_score_topk read a paged cache; the decode's
 * indexed mode and fp32 KV return ATTN_ERR_UNSUPPORTED for one.  The
 * token-major pool [pages][page_tokens][KH][D] has stride_t = KH*D,
 * stride_h = D, page_stride = page_tokens*KH*D; the head-major pool
 * [pages][KH][page_tokens][D] has stride_t = D, stride_h = page_tokens*D,
 * page_stride = KH*page_tokens*D.
 */
typedef struct {
  int32_t B, KH, D, max_seq_len;
  const int32_t *seq_lens;
  const int64_t *seq_offset;
  int64_t stride_h, stride_t;
  const int32_t *block_table;
  int32_t page_tokens, table_stride;
  int64_t page_stride;
} attn_kv_geom;

/*
 * Arguments of one decode step.
 *   G           query heads per KV head, 1 <= G <= 64
 *   q_rows      query rows per sequence R (0 or 1: one).  R > 1 is the
 *               multi-row step of speculative decoding (NVIDIA blog, GEMM
 *               shapes: with D draft tokens GEMM-M = (1 + D) x G): the R query
 *               tokens are the last R tokens of each cache, so row r attends
 *               to the first L_b - (R - 1) + r tokens.  q, out and lse are
 *               then [B][R][KH*G][...].  R*G <= 64, bf16 or int8 KV, no
 *               token_idx.  The R*G rows of a KV head share each K/V load
 *               (G = 8, R = 2 fill the 16 matrix-core columns)
 *   q           [B][KH*G][D] in q_dtype (ATTN_BF16, or ATTN_F32 with fp32 KV);
 *               with ATTN_I8 KV the int8 matrix cores take each head's q as
 *               a 22-bit fixed-point value with its own scale (max|q_g| /
 *               2^22), error at most max|q_g| * 2^-23 per element
 *   k, v        KV cache in kv_dtype, geometry `kv`
 *   k_scale     ATTN_I8 only: fp32 scale of K row (b, kh, t) is
 *               k_scale[(b*KH + kh)*k_scale_stride + t / k_part_tokens];
 *               k_part_tokens is a multiple of 16 (64 or 128 on the page),
 *               k_scale_stride >= ceil(max_seq_len / k_part_tokens).
 *               k_part_tokens = 0 selects one per-tensor K scale, k_scale[0]
 *               (k_scale_stride is then ignored)
 *   v_scale     ATTN_I8 only: the per-tensor V scale (host value)
 *   q_quant     ATTN_I8 only, an attn_q_quant.  ATTN_QUANT_EXACT keeps the
 *               query as above.  ATTN_QUANT_ROW quantises each query row in
 *               the kernel: s = max|q_row| / 127 and code = clamp(rint(q / s),
 *               -127, 127), both in IEEE fp32 (correctly rounded divide,
 *               round half to even; s = 0 gives codes 0), so the scores use
 *               code * s.  ATTN_QUANT_STATIC uses the same rule with
 *               s = q_scale for every row (quotients beyond 127 clamp).
 *   q_scale     ATTN_QUANT_STATIC only: the static per-tensor query scale,
 *               finite and >= 0 (host value)
 *   token_idx   optional: when not NULL, (b, kh) attends only to the tokens
 *               token_idx[(b*KH + kh)*idx_stride + j], j < n_idx[b*KH + kh]
 *               (each < L_b; any order; n_idx <= idx_stride), e.g. the kept
 *               set written by oam_score_topk
 *   softmax_scale  multiplies q.k; 0 selects 1/sqrt(D)
 *   split_tokens   the split-KV granularity, a multiple of 32; 0 = library
 *               default.  bf16/int8 KV: the positions of all (b, kh) are laid
 *               end to end and cut into one equal contiguous range per
 *               decode worker, each range at least split_tokens positions
 *               long (fewer workers when there is less work); a (b, kh)
 *               then spans at most ceil(L_b / split_tokens) + 1 ranges, each
 *               giving one partial.  Default 4096 (with token_idx 512 kept
 *               tokens, up to 1024 for long lists; over token-major pages
 *               of a paged cache 2048, with twice the workers that fit at
 *               once).  With a given split_tokens the split depends only on
 *               the lengths, so equal split_tokens give bit-identical
 *               results over every cache layout.
 *               fp32 KV: chunks of split_tokens positions, default 256.
 *               attn_decode_split_tokens reports the choice
 *   workspace   caller-owned scratch of at least attn_decode_workspace_size()
 *               bytes, 256-byte aligned; holds the partials and, for
 *               bf16/int8 KV, one arrival counter per (b, kh).  It needs no
 *               initialisation: a counter word carries a 40-bit tag that
 *               changes with every call on the same counter array, a call
 *               leaves its counters at zero arrivals under the tag of the
 *               next call on that array, and a call's first arrival takes
 *               over a word without its own tag (whatever an earlier call
 *               left, finished or cut off, or other data, which matches a
 *               tag with probability 2^-40 per word).  The library keeps the
 *               tags of the last 64 counter arrays on the host.  Calls that
 *               run at the same time on one workspace race
 *   out         [B][KH*G][D] in out_dtype (ATTN_F32 or ATTN_BF16)
 *   lse         optional fp32 [B][KH*G]: natural-log log-sum-exp of the
 *               scaled scores (-inf for a sequence with no tokens)
 *   fixed_splits  0: the balanced split above (the default).  S >= 1 (bf16
 *               or int8 KV): the unbalanced schedule it replaces, kept for
 *               comparison: every (b, kh) is cut into S equal splits, one
 *               worker each, whatever its length, so with mixed lengths
 *               most workers idle while the longest sequence's finish
 *               ("优化稀疏注意力中的令牌丢弃机制" §5: 128K next to 512 tokens is
 *               250x the work).  S = 1 is one worker per (b, kh); split_tokens
 *               is then ignored
 * A sequence (or kept set) with no tokens gives out = 0.
 */
typedef struct {
  attn_kv_geom kv;
  int32_t G;
  int32_t q_rows;
  int32_t q_dtype, kv_dtype, out_dtype;
  const void *q;
  const void *k;
  const void *v;
  const float *k_scale;
  int32_t k_part_tokens, k_scale_stride;
  float v_scale;
  int32_t q_quant;
  float q_scale;
  const int32_t *token_idx;
  const int32_t *n_idx;
  int32_t idx_stride;
  float softmax_scale;
  int32_t split_tokens;
  void *workspace;
  size_t workspace_bytes;
  void *out;
  float *lse;
  int32_t fixed_splits;
} attn_decode_args;

/* Host-only: bytes of workspace attn_decode_splitkv needs for these args
 * (depends on B, KH, G, D, max_seq_len or idx_stride, split_tokens, dtypes
 * and the current device's compute-unit count).
 * Writes *bytes; returns ATTN_ERR_INVALID_ARG / ATTN_ERR_UNSUPPORTED for
 * arguments attn_decode_splitkv would reject. */
attn_status attn_decode_workspace_size(const attn_decode_args *args, size_t *bytes);

/* Host-only: the split granularity in tokens (split_tokens) attn_decode_splitkv
 * uses for these args: the given one, or for split_tokens = 0 the library's
 * default, chosen from the dtypes and, with token_idx, the list length.
 * Writes *split_tokens; same argument errors as attn_decode_workspace_size. */
attn_status attn_decode_split_tokens(const attn_decode_args *args, int32_t *split_tokens);

/*
 * Split-KV decode attention ("优化稀疏注意力中的令牌丢弃机制" §5 Split-KV;
 * "注意力优化" Flash Attention online softmax).  Every (b, kh) position range
 * is cut into tiles of 32 positions and all ranges are laid end to end; each
 * worker of a persistent grid streams an equal contiguous share of that tile
 * stream once.
 *  bf16/int8 KV: one launch.  A worker's part of a (b, kh) is one partial
 *      (m, l, o) per query head, written to the workspace; a worker holding
 *      a whole (b, kh) writes out and lse directly.  The last worker to finish
 *      a shared (b, kh) (an integer arrival counter) merges its partials by
 *      the log-sum-exp rule into out and lse inside the same launch.
 *  fp32 KV: a decode launch writes partials per chunk of split_tokens
 *      positions, and a second launch merges them (the operation
 *      attn_merge_lse exposes on its own).
 * Results are deterministic: no floating-point atomics are used, partials
 * are merged in a fixed order, and the work split depends only on the
 * lengths and the device's compute-unit count.
 */
attn_status attn_decode_splitkv(const attn_decode_args *args, attn_stream_t stream);

/*
 * attn_decode_splitkv plus timing marks: events[0..2] (hipEvent_t created by
 * the caller, any may be NULL) are recorded on `stream` before the decode
 * kernel, after it, and after the merge launch (for bf16/int8 KV the merge
 * runs inside the decode kernel, so the last two marks follow each other).
 * Same arguments and errors.
 */
attn_status attn_decode_splitkv_profiled(const attn_decode_args *args, attn_stream_t stream, void *const events[3]);

/*
 * attn_decode_splitkv for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that must not call hipMalloc, and
 * harnesses that forbid it.  The partials and arrival counters live in a
 * static device array of the library, ATTN_NOALLOC_SCRATCH_BYTES (64 MiB) on
 * each GPU it runs on, held until the process ends; the call allocates
 * nothing.  The caller still passes q, k, v, out, lse and the rest of args;
 * args->workspace must be NULL and args->workspace_bytes 0.
 *  - Arguments whose attn_decode_workspace_size exceeds the array return
 *    ATTN_ERR_WORKSPACE_TOO_SMALL and enqueue nothing (the 128K-token bf16
 *    step of 4 sequences x 8 KV heads needs about 4.4 MB, 32 sequences of up
 *    to 128K tokens about 35 MB).
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents.  Nothing in it needs clearing: partials are written
 *    before they are read, and the counters follow the rule described under
 *    attn_decode_args.workspace.  Calls that overlap on one GPU (several
 *    streams, or host threads without ordering) race on the array and give
 *    undefined results: order them on one stream.
 *  - The first call on a device looks up that device's copy of the array
 *    (hipGetSymbolAddress, with the device current); a failure there
 *    returns ATTN_ERR_HIP.
 * Results are those of attn_decode_splitkv with the same arguments, bit for
 * bit (same kernels, same work split).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
attn_status attn_decode_splitkv_noalloc(const attn_decode_args *args, attn_stream_t stream);

/*
 * Log-sum-exp merge of partial triples ("优化稀疏注意力中的令牌丢弃机制" §5,
 * cross-shard online softmax; read with the chunk term weighted by
 * exp(m_chunk - m_new), which makes the result independent of the split).
 * Row r (0 <= r < rows) owns partials row_split_start[r] ..
 * row_split_start[r+1]-1 (device int32, CSR, non-decreasing, starting at 0).
 * Partial i: m_part[i] = max scaled score (natural log units), l_part[i] =
 * sum exp(s - m_part[i]) >= 0, o_part[i*D .. i*D+D-1] = that chunk's
 * normalised output.  Partials with l_part = 0 are ignored.
 *   out[r*D + d] = sum_i exp(m_i - M) l_i o_i[d] / sum_i exp(m_i - M) l_i,
 *   lse[r] = M + ln(sum_i exp(m_i - M) l_i), M = max over partials with l > 0;
 * a row with no (non-empty) partial gets out = 0 and lse = -inf.
 * out_dtype is ATTN_F32 or ATTN_BF16; lse may be NULL.  1 <= D <= 256.
 */
attn_status attn_merge_lse(const float *o_part, const float *m_part, const float *l_part,
                           const int32_t *row_split_start, int32_t rows, int32_t D, int32_t out_dtype,
                           void *out, float *lse, attn_stream_t stream);

/* Host-only: workspace bytes for kv_quant_int8: 0 in per-partition mode; in
 * per-tensor mode 256 bytes plus one fp32 maximum per group of four row
 * blocks (a row block is 8192 elements: 64 rows at D = 128) per (b, kh), about
 * 1/8192 of the cache's bytes.  Validates the geometry's sizes. */
attn_status kv_quant_int8_workspace_size(const attn_kv_geom *geom, int32_t partition_tokens, size_t *bytes);

/*
 * INT8 quantisation of a bf16 K or V cache ("优化稀疏注意力中的令牌丢弃机制"
 * §6): q_val = round(val / scale), round half to even on the IEEE fp32
 * quotient, clamped to [-127, 127].
 *   partition_tokens > 0 (a multiple of 16; 64 or 128 on the page): Scheme A
 *     per-token-partition scales.  Partitions start at token 0 of every
 *     (b, kh); scale = fl32(max|x| / 127) over the partition's tokens and all
 *     D channels; it is written to scales[(b*KH + kh)*scale_stride + t/P]
 *     (scale_stride >= ceil(max_seq_len / P)).  An all-zero partition gets
 *     scale 0 and codes 0.
 *   partition_tokens == 0: one per-tensor scale over every valid row of every
 *     (b, kh), written to scales[0] (the page's per-tensor baseline, used for V).
 *   x_bf16   bf16 cache in geometry `geom`
 *   codes    int8 output in the same geometry (same offsets and strides, in
 *            elements); rows t >= L_b are not touched
 *   workspace  per-tensor mode only: >= kv_quant_int8_workspace_size() bytes
 * Run once when the cache is written, not per decode step.
 */
attn_status kv_quant_int8(const attn_kv_geom *geom, const void *x_bf16, int32_t partition_tokens,
                          int32_t scale_stride, int8_t *codes, float *scales, void *workspace,
                          size_t workspace_bytes, attn_stream_t stream);

/*
 * ln(||v_t||_2 + eps) of every V row, the value term of the OAM score
 * ("优化稀疏注意力中的令牌丢弃机制" §3: the natural log of the value's L2 norm
 * plus eps).  A row never
 * changes once appended, so this can be computed at append time and passed
 * to oam_score_topk.  vlog[(b*KH + kh)*vlog_stride + t] for t < L_b
 * (vlog_stride >= max_seq_len).  v_dtype is ATTN_BF16, or ATTN_I8 for an
 * INT8 cache whose rows are code * v_scale (the norm of those values; §7
 * stacks OAM on the INT8 cache).  Accumulates in fp32.
 */
attn_status oam_value_lognorm(const attn_kv_geom *geom, const void *v, int32_t v_dtype, float v_scale, float eps,
                              float *vlog, int32_t vlog_stride, attn_stream_t stream);

/*
 * Arguments of output-aware top-K token selection.
 *   q           bf16 [B][KH*G][D]; 1 <= G <= 16
 *   k           KV cache in kv_dtype and geometry `kv`; max_seq_len <= 2^21
 *               (ATTN_ERR_UNSUPPORTED otherwise)
 *   kv_dtype    ATTN_BF16, or ATTN_I8 to score an INT8 cache (the page's §7
 *               stack: OAM, then INT8 attention over the kept tokens) with
 *               the K scales of attn_decode_args: k_scale[(b*KH + kh)*
 *               k_scale_stride + t / k_part_tokens], k_part_tokens = 0 for
 *               one per-tensor scale k_scale[0]; v rows are code * v_scale
 *   v, vlog     the value term comes from vlog (fp32, layout of
 *               oam_value_lognorm, stride vlog_stride) when vlog != NULL,
 *               else it is computed from the rows of v (kv_dtype) on the fly
 *   softmax_scale  0 selects 1/sqrt(D); beta, eps as on the page
 *   top_k       >= 1 tokens kept per (b, kh); with block_tokens > 1, blocks
 *   block_tokens  0 or 1: token-granular selection.  A power of two in
 *               [16, 256]: block-granular selection ("原生稀疏注意力(NSA)"
 *               §2.1, selected attention: the top-n blocks of contiguous
 *               tokens, shared by the GQA group).  Blocks are [j*block_tokens,
 *               (j+1)*block_tokens) cut at L_b; a block's score is the mean of
 *               its tokens' scores (the page's learned block compression read
 *               as the mean over the block; beta = 0 gives the plain routing
 *               score); the top_k blocks by (score descending, block index
 *               ascending) are kept.  At most 8192 blocks per sequence
 *   idx_out     int32 [B][KH][top_k * max(block_tokens, 1)]: kept token
 *               indices in ascending order; entries past n_kept are -1
 *   n_kept      int32 [B][KH]: kept tokens, min(top_k, L_b) for tokens
 *   scores_out  optional fp32 [B][KH][max_seq_len]: the scores
 *   workspace   >= oam_score_topk_workspace_size() bytes, 256-byte aligned;
 *               needs no initialisation: the selection's histogram words
 *               carry a tag that changes with every call, so words left by
 *               an earlier call (or other data) count as zero.  Calls that
 *               share a workspace must be ordered on one stream
 */
typedef struct {
  attn_kv_geom kv;
  int32_t G;
  const void *q;
  const void *k;
  const void *v;
  int32_t kv_dtype;
  const float *k_scale;
  int32_t k_part_tokens, k_scale_stride;
  float v_scale;
  const float *vlog;
  int32_t vlog_stride;
  float softmax_scale, beta, eps;
  int32_t top_k;
  int32_t block_tokens;
  int32_t *idx_out;
  int32_t *n_kept;
  float *scores_out;
  void *workspace;
  size_t workspace_bytes;
} oam_topk_args;

/* Host-only: workspace bytes of oam_score_topk. */
attn_status oam_score_topk_workspace_size(const oam_topk_args *args, size_t *bytes);

/*
 * OAM scoring and top-K selection ("优化稀疏注意力中的令牌丢弃机制" §3: score
 * tokens by routing logit plus value magnitude and drop the lowest; §2 for
 * the classic q.k top-K it replaces).  For each (b, kh):
 *   score_t = mean_g (q_g . k_t) * softmax_scale + beta * ln(||v_t||_2 + eps)
 * (the mean over the G query heads gives one kept set per KV head; with
 * INT8 K the int8 matrix cores take the mean query as a 22-bit fixed-point
 * value, as attn_decode_splitkv does for its query), then the
 * top_k tokens by (score descending, index ascending) are kept.  Scores are
 * fp32; the selection is an exact radix select on order-preserving integer
 * keys of the fp32 scores.  Feed idx_out/n_kept to attn_decode_splitkv's
 * token_idx/n_idx for exact attention over the kept tokens (§7).
 */
attn_status oam_score_topk(const oam_topk_args *args, attn_stream_t stream);

/* Static description of a status code. */
const char *attn_status_string(attn_status status);

/* Message describing the calling thread's most recent failed call ("" if none). */
const char *attn_last_error(void);

/*
 * Measurement helpers (not part of the method): a plain device copy of
 * `bytes` (multiple of 16, 16-byte aligned pointers) and a read-only sweep
 * (non-temporal 16-byte loads, one contiguous chunk per workgroup) that
 * writes one checksum word per workgroup into sink (>= 4096 floats).  They
 * calibrate hardware byte counters and the achievable HBM bandwidth.
 * attn_util_read returns ATTN_ERR_UNSUPPORTED for 2^43 bytes or more (a
 * workgroup's chunk must stay under 2 GiB).
 */
attn_status attn_util_copy(void *dst, const void *src, size_t bytes, attn_stream_t stream);
attn_status attn_util_read(const void *src, size_t bytes, float *sink, attn_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LCDG_ATTN_DECODE_H */
