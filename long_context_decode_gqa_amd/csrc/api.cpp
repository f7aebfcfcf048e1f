// C ABI of libattn_decode.so: host-side validation, workspace layout and
// dispatch.  Nothing is enqueued until every argument check has passed.
#include <algorithm>
#include <math.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "common.hpp"

namespace lcdg {
namespace {

thread_local std::string g_last_error;

attn_status fail(attn_status st, const char *msg) {
  g_last_error = msg;
  return st;
}

attn_status fail_hip(hipError_t e, const char *where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return ATTN_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int elem_size(int dt) { return dt == ATTN_F32 ? 4 : dt == ATTN_BF16 ? 2 : 1; }

std::mutex g_cu_mutex;
int g_cu_cache[64] = {0};

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_cache[dev] = n;
  }
  return g_cu_cache[dev];
}

namespace {

// Validation shared by every call that takes a KV geometry.
attn_status check_geom(const attn_kv_geom &g, int es, bool need_ptrs) {
  if (g.B < 0 || g.KH < 1 || g.D < 1 || g.max_seq_len < 0)
    return fail(ATTN_ERR_INVALID_ARG, "geometry: need B >= 0, KH >= 1, D >= 1, max_seq_len >= 0");
  if ((int64_t)g.B * g.KH > (1 << 24)) return fail(ATTN_ERR_UNSUPPORTED, "geometry: B*KH above 2^24");
  if (g.stride_t < g.D || g.stride_h < g.D) return fail(ATTN_ERR_INVALID_ARG, "geometry: strides must be >= D");
  if ((g.stride_t * es) % 16 || (g.stride_h * es) % 16 || ((int64_t)g.D * es) % 4)
    return fail(ATTN_ERR_INVALID_ARG, "geometry: rows must be 16-byte aligned (stride_t, stride_h in bytes % 16)");
  if (need_ptrs && g.B > 0 && (!g.seq_lens || (!g.seq_offset && !g.block_table)))
    return fail(ATTN_ERR_INVALID_ARG, "geometry: seq_lens and seq_offset (or a block table) are required");
  if (g.block_table) {
    if (g.page_tokens < 32 || g.page_tokens % 32)
      return fail(ATTN_ERR_INVALID_ARG, "geometry: page_tokens must be a positive multiple of 32");
    if (g.table_stride < ((int64_t)g.max_seq_len + g.page_tokens - 1) / g.page_tokens)
      return fail(ATTN_ERR_INVALID_ARG, "geometry: table_stride must be >= ceil(max_seq_len / page_tokens)");
    if (g.page_stride <= 0 || (g.page_stride * es) % 16)
      return fail(ATTN_ERR_INVALID_ARG, "geometry: page_stride must be positive and 16-byte aligned");
  }
  return ATTN_OK;
}

struct DecodeLayout {
  size_t m, l, o, total;
  int64_t max_partials, max_chunks;
  int32_t split, ngb, max_tokens;
  int32_t cols;  // matrix-core columns per decode worker (16, or 32 for more than 16 rows per KV head)
  bool mfma;
};

attn_status plan_decode(const attn_decode_args *a, DecodeLayout *L) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  const attn_kv_geom &g = a->kv;
  if (a->kv_dtype != ATTN_F32 && a->kv_dtype != ATTN_BF16 && a->kv_dtype != ATTN_I8)
    return fail(ATTN_ERR_INVALID_ARG, "kv_dtype must be ATTN_F32, ATTN_BF16 or ATTN_I8");
  if (a->out_dtype != ATTN_F32 && a->out_dtype != ATTN_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "out_dtype must be ATTN_F32 or ATTN_BF16");
  if (a->q_dtype != ATTN_F32 && a->q_dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "q_dtype must be F32 or BF16");
  if (a->kv_dtype == ATTN_F32 && a->q_dtype != ATTN_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "fp32 KV needs fp32 Q");
  if (a->kv_dtype != ATTN_F32 && a->q_dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "bf16 and int8 KV need bf16 Q");
  attn_status st = check_geom(g, elem_size(a->kv_dtype), true);
  if (st != ATTN_OK) return st;
  if (a->G < 1 || a->G > 64) return fail(ATTN_ERR_UNSUPPORTED, "G must be in [1, 64]");
  const int R = a->q_rows > 1 ? a->q_rows : 1;
  if (a->q_rows < 0 || (int64_t)R * a->G > 64)
    return fail(ATTN_ERR_UNSUPPORTED, "q_rows must be >= 0 with q_rows * G <= 64");
  const bool mfma = a->kv_dtype != ATTN_F32;
  if (g.block_table && (!mfma || a->token_idx))
    return fail(ATTN_ERR_UNSUPPORTED, "a paged cache needs bf16 or int8 KV and no token_idx");
  if (R > 1 && (!mfma || a->token_idx))
    return fail(ATTN_ERR_UNSUPPORTED, "q_rows > 1 needs bf16 or int8 KV and no token_idx");
  if (mfma && g.D != 64 && g.D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "bf16/int8 KV supports head size D = 64 or 128");
  if (!mfma && (g.D < 4 || g.D > 256 || g.D % 4))
    return fail(ATTN_ERR_UNSUPPORTED, "fp32 KV supports D in [4, 256], a multiple of 4");
  if (a->kv_dtype == ATTN_I8 && (g.stride_t % 16 || g.stride_h % 16))
    return fail(ATTN_ERR_INVALID_ARG, "int8 KV rows must be 16-byte aligned");
  if (!(fabsf(a->softmax_scale) < INFINITY)) return fail(ATTN_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (a->split_tokens < 0 || (a->split_tokens && (a->split_tokens % 32 || a->split_tokens > (1 << 20))))
    return fail(ATTN_ERR_INVALID_ARG, "split_tokens must be 0 or a positive multiple of 32 (<= 2^20)");
  if (a->token_idx && (!a->n_idx || a->idx_stride < 0))
    return fail(ATTN_ERR_INVALID_ARG, "token_idx needs n_idx and idx_stride >= 0");
  if (a->q_quant != ATTN_QUANT_EXACT && a->q_quant != ATTN_QUANT_ROW && a->q_quant != ATTN_QUANT_STATIC)
    return fail(ATTN_ERR_INVALID_ARG, "q_quant must be ATTN_QUANT_EXACT, ATTN_QUANT_ROW or ATTN_QUANT_STATIC");
  if (a->q_quant != ATTN_QUANT_EXACT && a->kv_dtype != ATTN_I8)
    return fail(ATTN_ERR_UNSUPPORTED, "query quantisation needs int8 KV");
  if (a->q_quant == ATTN_QUANT_STATIC && !(a->q_scale >= 0.f && a->q_scale < INFINITY))
    return fail(ATTN_ERR_INVALID_ARG, "q_scale must be finite and >= 0");
  if (a->kv_dtype == ATTN_I8) {
    if (!a->k_scale) return fail(ATTN_ERR_INVALID_ARG, "int8 KV needs k_scale");
    if (a->k_part_tokens != 0) {  // 0: one per-tensor K scale
      if (a->k_part_tokens < 16 || a->k_part_tokens % 16)
        return fail(ATTN_ERR_INVALID_ARG, "k_part_tokens must be 0 or a positive multiple of 16");
      const int64_t need = ((int64_t)g.max_seq_len + a->k_part_tokens - 1) / a->k_part_tokens;
      if (a->k_scale_stride < need || a->k_scale_stride < 1)
        return fail(ATTN_ERR_INVALID_ARG, "k_scale_stride must be >= ceil(max_seq_len / k_part_tokens)");
    }
    if (!(fabsf(a->v_scale) < INFINITY)) return fail(ATTN_ERR_INVALID_ARG, "v_scale must be finite");
  }
  if (g.B > 0) {
    if (!a->q || !a->k || !a->v || !a->out) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and out are required");
    if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v))
      return fail(ATTN_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
  }
  L->mfma = mfma;
  // More than 16 query rows per KV head: each worker computes 32 columns
  // (two blocks sharing every K/V load) instead of streaming the cache once
  // per 16-column block.
  L->cols = (mfma && R * a->G > 16) ? 32 : 16;
  L->ngb = (R * a->G + L->cols - 1) / L->cols;
  L->max_tokens = a->token_idx ? a->idx_stride : g.max_seq_len;
  if (a->split_tokens) {
    L->split = a->split_tokens;
  } else if (!mfma) {
    L->split = 256;
  } else if (a->token_idx) {
    // Gathered runs are short and a worker's fixed costs weigh more: chunks
    // of at least 256 (bf16) or 128 (int8) and at most 1024 kept tokens
    // (4096 kept tokens per pair, bf16: 2048 two-tile workers took 26.6 us,
    // 512 eight-tile workers 23.3 us, 256 sixteen-tile workers 26.7 us;
    // int8: 27.6, 24.8 with four-tile workers, 26.1 us).
    const int64_t tiles = (int64_t)g.B * g.KH * L->ngb * (((int64_t)L->max_tokens + 31) / 32);
    const int64_t ct = std::min<int64_t>(std::max<int64_t>(tiles / 2048, a->kv_dtype == ATTN_I8 ? 4 : 8), 32);
    L->split = (int32_t)(32 * ct);
  } else {
    // About one chunk per worker, each worker streaming at least 32 tiles
    // when there are enough: every partial costs a write in the stream and
    // a read in the merge, and two one-wave workers per compute unit with
    // their register rings already keep HBM busy.  At most 2048 bf16
    // workers (two per SIMD) and 1024 int8 or 32-column workers (one per
    // SIMD); chunks of at most 4096 tokens.  The tile count is the bound
    // from max_seq_len (the lengths are on the device).  Measured on a
    // 256 MiB bf16 step (16384 tiles): 2048 workers 61 us, 512 workers
    // 52 us; on the 1 GiB int8 128K step: 2048 workers 205 us, 1024 with
    // 4096-token chunks 193 us; on the ragged bf16 batch: 2048-token chunks
    // 648 us, 4096-token 640 us.
    const int64_t tiles = (int64_t)g.B * g.KH * L->ngb * (((int64_t)L->max_tokens + 31) / 32);
    const bool one_per_simd = L->cols == 32 || a->kv_dtype == ATTN_I8;
    const int64_t wmax = one_per_simd ? 1024 : 2048;
    const int64_t workers = std::min<int64_t>(std::max<int64_t>(tiles / 32, 256), wmax);
    int64_t ct = std::min<int64_t>(std::max<int64_t>(tiles / workers, 1), 128);
    if (g.block_table) ct = std::min<int64_t>(ct, 2 * (int64_t)g.page_tokens);  // a chunk spans <= 64 pages
    L->split = (int32_t)(32 * ct);
  }
  if (mfma && ((int64_t)g.max_seq_len + 64) * g.stride_t * elem_size(a->kv_dtype) >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "one (sequence, KV head) may span at most 2 GiB of rows");
  if (mfma && a->token_idx && L->split > 1024)
    return fail(ATTN_ERR_UNSUPPORTED, "with token_idx, split_tokens must be <= 1024");
  if (g.block_table && (int64_t)L->split > 64 * (int64_t)g.page_tokens)
    return fail(ATTN_ERR_UNSUPPORTED, "with a paged cache, split_tokens must be <= 64 * page_tokens");
  L->max_chunks = ((int64_t)L->max_tokens + L->split - 1) / L->split;
  const int64_t QH = (int64_t)g.KH * a->G * R;
  L->max_partials = 2 * (int64_t)g.B * QH * L->max_chunks;
  const int64_t nlanes = (int64_t)g.B * g.KH * L->ngb;
  const int64_t max_tiles = nlanes * (((int64_t)L->max_tokens + 31) / 32);
  if (L->max_partials >= (int64_t(1) << 31) || max_tiles >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "too many split-KV partials (reduce max_seq_len or raise split_tokens)");
  size_t off = 0;
  L->m = off; off = align256(off + L->max_partials * sizeof(float));
  L->l = off; off = align256(off + L->max_partials * sizeof(float));
  L->o = off; off = align256(off + (size_t)L->max_partials * g.D * sizeof(float));
  L->total = off;
  return ATTN_OK;
}

}  // namespace

attn_status api_fail(attn_status st, const char *msg) { return fail(st, msg); }
attn_status api_fail_hip(hipError_t e, const char *where) { return fail_hip(e, where); }
attn_status api_check_geom(const attn_kv_geom &g, int es, bool need_ptrs) { return check_geom(g, es, need_ptrs); }

}  // namespace lcdg

using namespace lcdg;

extern "C" {

const char *attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *attn_last_error(void) { return g_last_error.c_str(); }

attn_status attn_decode_workspace_size(const attn_decode_args *args, size_t *bytes) {
  if (!bytes) return fail(ATTN_ERR_INVALID_ARG, "bytes is NULL");
  DecodeLayout L;
  attn_status st = plan_decode(args, &L);
  if (st != ATTN_OK) return st;
  *bytes = L.total;
  return ATTN_OK;
}

attn_status attn_decode_split_tokens(const attn_decode_args *args, int32_t *split_tokens) {
  if (!split_tokens) return fail(ATTN_ERR_INVALID_ARG, "split_tokens is NULL");
  DecodeLayout L;
  attn_status st = plan_decode(args, &L);
  if (st != ATTN_OK) return st;
  *split_tokens = L.split;
  return ATTN_OK;
}

static attn_status decode_impl(const attn_decode_args *a, attn_stream_t stream, void *const *events) {
  DecodeLayout L;
  attn_status st = plan_decode(a, &L);
  if (st != ATTN_OK) return st;
  if (a->kv.B == 0) return ATTN_OK;
  if (!a->workspace || (reinterpret_cast<uintptr_t>(a->workspace) & 255))
    return fail(ATTN_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
  if (a->workspace_bytes < L.total) return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than required");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(a->workspace);
  DecodeParams p;
  p.B = a->kv.B;
  p.KH = a->kv.KH;
  p.R = a->q_rows > 1 ? a->q_rows : 1;
  p.Gq = a->G;
  p.G = a->G * p.R;
  p.D = a->kv.D;
  p.QH = a->kv.KH * p.G;
  p.ngb = L.ngb;
  p.cols_per_wave = L.cols;
  p.seq_lens = a->kv.seq_lens;
  p.seq_offset = a->kv.seq_offset;
  p.stride_h = a->kv.stride_h;
  p.stride_t = a->kv.stride_t;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.k_scale = a->k_scale;
  // a per-tensor K scale is one partition longer than any sequence
  p.k_part = a->k_part_tokens > 0 ? a->k_part_tokens : (1 << 30);
  p.k_scale_stride = a->k_part_tokens > 0 ? a->k_scale_stride : 0;
  p.v_scale = a->v_scale;
  p.q_quant = a->q_quant;
  p.q_scale = a->q_scale;
  p.block_table = a->kv.block_table;
  p.page_tokens = a->kv.page_tokens;
  p.table_stride = a->kv.table_stride;
  p.page_stride = a->kv.page_stride;
  p.token_idx = a->token_idx;
  p.n_idx = a->n_idx;
  p.idx_stride = a->idx_stride;
  p.softmax_scale = a->softmax_scale != 0.f ? a->softmax_scale : 1.0f / sqrtf((float)a->kv.D);
  p.split = L.split;
  p.max_seq_len = a->kv.max_seq_len;
  p.max_chunks = (int32_t)L.max_chunks;
  {
    // persistent grid: the MFMA kernel runs one-wave workers, eight per compute
    // unit (two per SIMD, its register budget; four, one per SIMD, for
    // 32-column workers); the vector-ALU kernel four 256-thread workgroups
    // per unit; capped by the largest possible tile count
    const int cus = device_cu_count();
    const int64_t max_tiles = (int64_t)p.B * p.KH * L.ngb * (((int64_t)L.max_tokens + 31) / 32);
    int64_t grid = (int64_t)cus * (L.mfma ? (L.cols == 32 ? 4 : 8) : 4);
    if (grid > max_tiles) grid = max_tiles;
    // no more workers than ranges of at least one chunk (the kernel's own
    // rule), so the workers in use are the first ones dispatched
    const int64_t ct = L.split / 32;
    if (grid > (max_tiles + ct - 1) / ct) grid = (max_tiles + ct - 1) / ct;
    p.grid = (int)(grid < 1 ? 1 : grid);
  }
  p.wl.m_part = reinterpret_cast<float *>(ws + L.m);
  p.wl.l_part = reinterpret_cast<float *>(ws + L.l);
  p.wl.o_part = reinterpret_cast<float *>(ws + L.o);

  auto mark = [&](int i) -> hipError_t {
    if (events && events[i]) return hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s);
    return hipSuccess;
  };
  hipError_t e = mark(0);
  if (e != hipSuccess) return fail_hip(e, "event record");
  if (L.mfma) e = launch_decode_mfma(p, a->kv_dtype, s);
  else e = launch_decode_valu(p, a->q_dtype, a->kv_dtype, s);
  if (e != hipSuccess) return fail_hip(e, "decode launch");
  if ((e = mark(1)) != hipSuccess) return fail_hip(e, "event record");
  e = launch_merge_decode(p, a->out_dtype, a->out, a->lse, s);
  if (e != hipSuccess) return fail_hip(e, "merge launch");
  if ((e = mark(2)) != hipSuccess) return fail_hip(e, "event record");
  return ATTN_OK;
}

attn_status attn_decode_splitkv(const attn_decode_args *a, attn_stream_t stream) {
  return decode_impl(a, stream, nullptr);
}

attn_status attn_decode_splitkv_profiled(const attn_decode_args *a, attn_stream_t stream, void *const events[3]) {
  return decode_impl(a, stream, events);
}

attn_status attn_merge_lse(const float *o_part, const float *m_part, const float *l_part,
                           const int32_t *row_split_start, int32_t rows, int32_t D, int32_t out_dtype, void *out,
                           float *lse, attn_stream_t stream) {
  if (rows < 0) return fail(ATTN_ERR_INVALID_ARG, "rows must be >= 0");
  if (D < 1 || D > 256) return fail(ATTN_ERR_UNSUPPORTED, "D must be in [1, 256]");
  if (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "out_dtype must be ATTN_F32 or ATTN_BF16");
  if (rows == 0) return ATTN_OK;
  if (!o_part || !m_part || !l_part || !row_split_start || !out)
    return fail(ATTN_ERR_INVALID_ARG, "o_part, m_part, l_part, row_split_start and out are required");
  hipError_t e = launch_merge(o_part, m_part, l_part, row_split_start, rows, D, out_dtype, out, lse,
                              reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "merge launch");
  return ATTN_OK;
}

attn_status attn_util_copy(void *dst, const void *src, size_t bytes, attn_stream_t stream) {
  if (bytes % 16 || (bytes && (!dst || !src || !aligned16(dst) || !aligned16(src))))
    return fail(ATTN_ERR_INVALID_ARG, "copy: bytes % 16 == 0 and 16-byte aligned pointers required");
  hipError_t e = launch_copy(dst, src, bytes, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : fail_hip(e, "copy launch");
}

attn_status attn_util_read(const void *src, size_t bytes, float *sink, attn_stream_t stream) {
  if (bytes % 16 || (bytes && (!src || !sink || !aligned16(src))))
    return fail(ATTN_ERR_INVALID_ARG, "read: bytes % 16 == 0, aligned src and a sink are required");
  hipError_t e = launch_read(src, bytes, sink, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : fail_hip(e, "read launch");
}

}  // extern "C"
