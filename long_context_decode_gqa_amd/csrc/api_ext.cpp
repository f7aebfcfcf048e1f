// C ABI: INT8 quantisation, OAM value norms and OAM top-K selection.
#include <math.h>

#include <string>

#include "common.hpp"

namespace lcdg {
attn_status api_fail(attn_status st, const char *msg);
attn_status api_fail_hip(hipError_t e, const char *where);
attn_status api_check_geom(const attn_kv_geom &g, int es, bool need_ptrs);
}  // namespace lcdg

using namespace lcdg;

extern "C" {

attn_status kv_quant_int8_workspace_size(const attn_kv_geom *geom, int32_t partition_tokens, size_t *bytes) {
  if (!geom || !bytes) return api_fail(ATTN_ERR_INVALID_ARG, "geom and bytes are required");
  if (partition_tokens < 0) return api_fail(ATTN_ERR_INVALID_ARG, "partition_tokens must be >= 0");
  if (partition_tokens == 0) {
    attn_status st = api_check_geom(*geom, 2, false);
    if (st != ATTN_OK) return st;
  }
  *bytes = partition_tokens == 0 ? quant_tensor_workspace_bytes(*geom) : 0;
  return ATTN_OK;
}

attn_status kv_quant_int8(const attn_kv_geom *geom, const void *x_bf16, int32_t partition_tokens,
                          int32_t scale_stride, int8_t *codes, float *scales, void *workspace,
                          size_t workspace_bytes, attn_stream_t stream) {
  if (!geom) return api_fail(ATTN_ERR_INVALID_ARG, "geom is NULL");
  attn_status st = api_check_geom(*geom, 2, true);
  if (st != ATTN_OK) return st;
  if (geom->D % 8 || geom->D > 4096) return api_fail(ATTN_ERR_UNSUPPORTED, "kv_quant_int8 needs D % 8 == 0");
  if (geom->stride_t % 8 || geom->stride_h % 8 || (geom->block_table && geom->page_stride % 8))
    return api_fail(ATTN_ERR_INVALID_ARG, "kv_quant_int8 needs strides that are multiples of 8 elements");
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % 16))
    return api_fail(ATTN_ERR_INVALID_ARG, "partition_tokens must be 0 or a positive multiple of 16");
  if (!scales) return api_fail(ATTN_ERR_INVALID_ARG, "scales is required");
  if (geom->B > 0 && (!x_bf16 || !codes)) return api_fail(ATTN_ERR_INVALID_ARG, "x_bf16 and codes are required");
  if (x_bf16 && (reinterpret_cast<uintptr_t>(x_bf16) & 15))
    return api_fail(ATTN_ERR_INVALID_ARG, "x_bf16 must be 16-byte aligned");
  if (codes && (reinterpret_cast<uintptr_t>(codes) & 7))
    return api_fail(ATTN_ERR_INVALID_ARG, "codes must be 8-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (partition_tokens > 0) {
    const int64_t need = ((int64_t)geom->max_seq_len + partition_tokens - 1) / partition_tokens;
    if (scale_stride < need || scale_stride < 1)
      return api_fail(ATTN_ERR_INVALID_ARG, "scale_stride must be >= ceil(max_seq_len / partition_tokens)");
    e = launch_quant_partitions(*geom, x_bf16, partition_tokens, scale_stride, codes, scales, s);
  } else {
    if (!workspace || workspace_bytes < quant_tensor_workspace_bytes(*geom) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255))
      return api_fail(ATTN_ERR_WORKSPACE_TOO_SMALL,
                      "per-tensor mode needs a 256-byte aligned workspace of kv_quant_int8_workspace_size() bytes");
    e = launch_quant_tensor(*geom, x_bf16, codes, scales, workspace, s);
  }
  return e == hipSuccess ? ATTN_OK : api_fail_hip(e, "quantisation launch");
}

attn_status oam_value_lognorm(const attn_kv_geom *geom, const void *v, int32_t v_dtype, float v_scale, float eps,
                              float *vlog, int32_t vlog_stride, attn_stream_t stream) {
  if (!geom) return api_fail(ATTN_ERR_INVALID_ARG, "geom is NULL");
  if (v_dtype != ATTN_BF16 && v_dtype != ATTN_I8) return api_fail(ATTN_ERR_INVALID_ARG, "v_dtype must be ATTN_BF16 or ATTN_I8");
  const bool i8 = v_dtype == ATTN_I8;
  attn_status st = api_check_geom(*geom, i8 ? 1 : 2, true);
  if (st != ATTN_OK) return st;
  if (geom->D != 64 && geom->D != 128 && geom->D != 256)
    return api_fail(ATTN_ERR_UNSUPPORTED, "oam_value_lognorm supports D = 64, 128 or 256");
  if (i8 && (geom->stride_t % 16 || geom->stride_h % 16))
    return api_fail(ATTN_ERR_INVALID_ARG, "int8 rows must be 16-byte aligned");
  if (i8 && !(fabsf(v_scale) < INFINITY)) return api_fail(ATTN_ERR_INVALID_ARG, "v_scale must be finite");
  if (!(eps >= 0.f) || !(eps < INFINITY)) return api_fail(ATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (vlog_stride < geom->max_seq_len) return api_fail(ATTN_ERR_INVALID_ARG, "vlog_stride must be >= max_seq_len");
  if (geom->B > 0 && (!v || !vlog)) return api_fail(ATTN_ERR_INVALID_ARG, "v and vlog are required");
  if (v && (reinterpret_cast<uintptr_t>(v) & 15)) return api_fail(ATTN_ERR_INVALID_ARG, "v must be 16-byte aligned");
  hipError_t e = launch_value_lognorm(*geom, v, v_dtype, v_scale, eps, vlog, vlog_stride,
                                      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : api_fail_hip(e, "value-norm launch");
}

}  // extern "C"

namespace {

struct OamLayout {
  size_t scores, vlog, hist, state, blk_gt, blk_nc, cand_key, cand_idx, bscores, total;
  int32_t bs_stride;
};

attn_status plan_oam(const oam_topk_args *a, OamLayout *L) {
  if (!a) return api_fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->kv_dtype != ATTN_BF16 && a->kv_dtype != ATTN_I8)
    return api_fail(ATTN_ERR_INVALID_ARG, "kv_dtype must be ATTN_BF16 or ATTN_I8");
  const bool i8 = a->kv_dtype == ATTN_I8;
  const int es = i8 ? 1 : 2;
  attn_status st = api_check_geom(a->kv, es, true);
  if (st != ATTN_OK) return st;
  const attn_kv_geom &g = a->kv;
  if (i8) {
    if (g.stride_t % 16 || g.stride_h % 16) return api_fail(ATTN_ERR_INVALID_ARG, "int8 rows must be 16-byte aligned");
    if (!a->k_scale) return api_fail(ATTN_ERR_INVALID_ARG, "int8 K needs k_scale");
    if (a->k_part_tokens != 0) {  // 0: one per-tensor K scale
      if (a->k_part_tokens < 16 || a->k_part_tokens % 16)
        return api_fail(ATTN_ERR_INVALID_ARG, "k_part_tokens must be 0 or a positive multiple of 16");
      const int64_t need = ((int64_t)g.max_seq_len + a->k_part_tokens - 1) / a->k_part_tokens;
      if (a->k_scale_stride < need || a->k_scale_stride < 1)
        return api_fail(ATTN_ERR_INVALID_ARG, "k_scale_stride must be >= ceil(max_seq_len / k_part_tokens)");
    }
    if (!(fabsf(a->v_scale) < INFINITY)) return api_fail(ATTN_ERR_INVALID_ARG, "v_scale must be finite");
  }
  if (g.D != 64 && g.D != 128) return api_fail(ATTN_ERR_UNSUPPORTED, "oam_score_topk supports D = 64 or 128");
  if (a->G < 1 || a->G > 16) return api_fail(ATTN_ERR_UNSUPPORTED, "oam_score_topk supports 1 <= G <= 16");
  if (a->top_k < 1) return api_fail(ATTN_ERR_INVALID_ARG, "top_k must be >= 1");
  const int bt = a->block_tokens;
  if (bt < 0 || (bt > 1 && (bt < 16 || bt > 256 || (bt & (bt - 1)))))
    return api_fail(ATTN_ERR_INVALID_ARG, "block_tokens must be 0, 1 or a power of two in [16, 256]");
  if (bt > 1 && ((int64_t)g.max_seq_len + bt - 1) / bt > oam_max_select_blocks())
    return api_fail(ATTN_ERR_UNSUPPORTED, "block-granular selection supports up to 8192 blocks per sequence");
  if (bt > 1 && (int64_t)a->top_k * bt >= (int64_t(1) << 31))
    return api_fail(ATTN_ERR_INVALID_ARG, "top_k * block_tokens must fit in int32");
  if (!(fabsf(a->softmax_scale) < INFINITY) || !(fabsf(a->beta) < INFINITY))
    return api_fail(ATTN_ERR_INVALID_ARG, "softmax_scale and beta must be finite");
  if (!(a->eps >= 0.f) || !(a->eps < INFINITY)) return api_fail(ATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  // the score pass reads a (sequence, KV head)'s rows, or a page's, through
  // one buffer resource with 32-bit offsets
  const int64_t span_rows = g.block_table ? (int64_t)g.page_tokens : (int64_t)g.max_seq_len + 64;
  if (span_rows * g.stride_t * es >= (int64_t(1) << 31))
    return api_fail(ATTN_ERR_UNSUPPORTED, "one (sequence, KV head) or page may span at most 2 GiB of rows");
  if (g.B > 0) {
    if (!a->q || !a->k) return api_fail(ATTN_ERR_INVALID_ARG, "q and k are required");
    if (!a->vlog && !a->v) return api_fail(ATTN_ERR_INVALID_ARG, "either vlog or v is required");
    if (!a->idx_out || !a->n_kept) return api_fail(ATTN_ERR_INVALID_ARG, "idx_out and n_kept are required");
    if ((reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->k)) & 15)
      return api_fail(ATTN_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
    if (!a->vlog && (reinterpret_cast<uintptr_t>(a->v) & 15))
      return api_fail(ATTN_ERR_INVALID_ARG, "v must be 16-byte aligned");
  }
  if (a->vlog && a->vlog_stride < g.max_seq_len) return api_fail(ATTN_ERR_INVALID_ARG, "vlog_stride must be >= max_seq_len");
  if (g.max_seq_len > oam_max_tokens())
    return api_fail(ATTN_ERR_UNSUPPORTED, "oam_score_topk supports max_seq_len up to 2^21 tokens");
  const int64_t npairs = (int64_t)g.B * g.KH;
  const int64_t stride = g.max_seq_len;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t off = 0;
  L->scores = off; off = al(off + (a->scores_out ? 0 : npairs * stride * sizeof(float)));
  L->vlog = off; off = al(off + (a->vlog ? 0 : npairs * stride * sizeof(float)));
  const size_t nblk_max = (size_t)oam_max_tokens() / 2048;
  L->hist = off; off = al(off + (size_t)npairs * 2048 * sizeof(uint64_t));
  L->state = off; off = al(off + (size_t)npairs * 8 * sizeof(int32_t));
  L->blk_gt = off; off = al(off + (size_t)npairs * nblk_max * sizeof(int32_t));
  L->blk_nc = off; off = al(off + (size_t)npairs * nblk_max * sizeof(int32_t));
  L->cand_key = off; off = al(off + (size_t)npairs * stride * sizeof(uint32_t));
  L->cand_idx = off; off = al(off + (size_t)npairs * stride * sizeof(int32_t));
  L->bs_stride = bt > 1 ? (int32_t)((g.max_seq_len + bt - 1) / bt) : 0;
  L->bscores = off; off = al(off + (size_t)npairs * L->bs_stride * sizeof(float));
  L->total = off;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status oam_score_topk_workspace_size(const oam_topk_args *args, size_t *bytes) {
  if (!bytes) return api_fail(ATTN_ERR_INVALID_ARG, "bytes is NULL");
  OamLayout L;
  attn_status st = plan_oam(args, &L);
  if (st != ATTN_OK) return st;
  *bytes = L.total;
  return ATTN_OK;
}

attn_status oam_score_topk(const oam_topk_args *a, attn_stream_t stream) {
  OamLayout L;
  attn_status st = plan_oam(a, &L);
  if (st != ATTN_OK) return st;
  if (a->kv.B == 0) return ATTN_OK;
  if (!a->workspace || (reinterpret_cast<uintptr_t>(a->workspace) & 255))
    return api_fail(ATTN_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
  if (a->workspace_bytes < L.total) return api_fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than required");
  char *ws = static_cast<char *>(a->workspace);
  OamPlan plan;
  plan.scores = a->scores_out ? a->scores_out : reinterpret_cast<float *>(ws + L.scores);
  plan.score_stride = a->kv.max_seq_len;
  plan.vlog = a->vlog ? const_cast<float *>(a->vlog) : reinterpret_cast<float *>(ws + L.vlog);
  plan.vlog_stride = a->vlog ? a->vlog_stride : a->kv.max_seq_len;
  plan.hist = reinterpret_cast<uint64_t *>(ws + L.hist);
  plan.blk_nc = reinterpret_cast<int32_t *>(ws + L.blk_nc);
  plan.bscores = reinterpret_cast<float *>(ws + L.bscores);
  plan.bs_stride = L.bs_stride;
  plan.state = reinterpret_cast<int32_t *>(ws + L.state);
  plan.blk_gt = reinterpret_cast<int32_t *>(ws + L.blk_gt);
  plan.cand_key = reinterpret_cast<uint32_t *>(ws + L.cand_key);
  plan.cand_idx = reinterpret_cast<int32_t *>(ws + L.cand_idx);
  hipError_t e = launch_oam(*a, plan, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : api_fail_hip(e, "oam launch");
}

}  // extern "C"
