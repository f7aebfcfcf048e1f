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
  *bytes = partition_tokens == 0 ? 256 : 0;
  return ATTN_OK;
}

attn_status kv_quant_int8(const attn_kv_geom *geom, const void *x_bf16, int32_t partition_tokens,
                          int32_t scale_stride, int8_t *codes, float *scales, void *workspace,
                          size_t workspace_bytes, attn_stream_t stream) {
  if (!geom) return api_fail(ATTN_ERR_INVALID_ARG, "geom is NULL");
  attn_status st = api_check_geom(*geom, 2, true);
  if (st != ATTN_OK) return st;
  if (geom->D % 8 || geom->D > 4096) return api_fail(ATTN_ERR_UNSUPPORTED, "kv_quant_int8 needs D % 8 == 0");
  if (geom->stride_t % 8 || geom->stride_h % 8)
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
    if (!workspace || workspace_bytes < 256 || (reinterpret_cast<uintptr_t>(workspace) & 255))
      return api_fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "per-tensor mode needs a 256-byte aligned workspace of 256 bytes");
    e = launch_quant_tensor(*geom, x_bf16, codes, scales, static_cast<uint32_t *>(workspace), s);
  }
  return e == hipSuccess ? ATTN_OK : api_fail_hip(e, "quantisation launch");
}

attn_status oam_value_lognorm(const attn_kv_geom *geom, const void *v_bf16, float eps, float *vlog,
                              int32_t vlog_stride, attn_stream_t stream) {
  if (!geom) return api_fail(ATTN_ERR_INVALID_ARG, "geom is NULL");
  attn_status st = api_check_geom(*geom, 2, true);
  if (st != ATTN_OK) return st;
  if (geom->D != 64 && geom->D != 128 && geom->D != 256)
    return api_fail(ATTN_ERR_UNSUPPORTED, "oam_value_lognorm supports D = 64, 128 or 256");
  if (!(eps >= 0.f) || !(eps < INFINITY)) return api_fail(ATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (vlog_stride < geom->max_seq_len) return api_fail(ATTN_ERR_INVALID_ARG, "vlog_stride must be >= max_seq_len");
  if (geom->B > 0 && (!v_bf16 || !vlog)) return api_fail(ATTN_ERR_INVALID_ARG, "v_bf16 and vlog are required");
  if (v_bf16 && (reinterpret_cast<uintptr_t>(v_bf16) & 15))
    return api_fail(ATTN_ERR_INVALID_ARG, "v_bf16 must be 16-byte aligned");
  hipError_t e = launch_value_lognorm(*geom, v_bf16, eps, vlog, vlog_stride, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : api_fail_hip(e, "value-norm launch");
}

attn_status oam_score_topk_workspace_size(const oam_topk_args *args, size_t *bytes) {
  (void)args;
  (void)bytes;
  return api_fail(ATTN_ERR_UNSUPPORTED, "oam_score_topk is not built yet");
}

attn_status oam_score_topk(const oam_topk_args *args, attn_stream_t stream) {
  (void)args;
  (void)stream;
  return api_fail(ATTN_ERR_UNSUPPORTED, "oam_score_topk is not built yet");
}

}  // extern "C"
