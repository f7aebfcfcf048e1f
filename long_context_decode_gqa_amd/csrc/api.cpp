// C ABI of libattn_decode.so: host-side validation, workspace layout and
// dispatch.  Nothing is enqueued until every argument check has passed.
#include <algorithm>
#include <math.h>
#include <stdio.h>

#include <atomic>
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
  size_t m, l, o, ctr, total;
  int64_t max_partials, max_chunks, max_slots, lanes;
  int32_t split, ngb, max_tokens, grid;
  int32_t cols;  // matrix-core columns per decode wave: 16, 32 (more than 16 rows per KV head) or 64
  int32_t wpg;   // waves per decode worker (workgroup)
  bool mfma;     // matrix-core decode (bf16/int8 KV), whose launch also merges
  bool stream_nt;  // matrix-core decode: non-temporal K/V loads
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
  if (a->fixed_splits < 0 || a->fixed_splits > 65536)
    return fail(ATTN_ERR_INVALID_ARG, "fixed_splits must be in [0, 65536]");
  if (a->fixed_splits > 0 && a->kv_dtype == ATTN_F32)
    return fail(ATTN_ERR_UNSUPPORTED, "fixed_splits needs bf16 or int8 KV");
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
  // More than 16 query rows per KV head: each wave computes 32 columns
  // (two blocks sharing every K/V load) instead of streaming the cache once
  // per 16-column block.  More than 32 over a bf16 cache read by position:
  // 64 columns (four blocks) in one wave, so every wave of a worker streams
  // tiles of its own; two 32-column groups in one worker (int8, kept
  // tokens) load each tile once per group.
  const bool cols64 = mfma && R * a->G > 32 && a->kv_dtype == ATTN_BF16 && !a->token_idx;
  L->cols = cols64 ? 64 : (mfma && R * a->G > 16) ? 32 : 16;
  L->ngb = (R * a->G + L->cols - 1) / L->cols;
  L->max_tokens = a->token_idx ? a->idx_stride : g.max_seq_len;
  L->lanes = (int64_t)g.B * g.KH * (mfma ? 1 : L->ngb);
  const int64_t lane_tiles_max = ((int64_t)L->max_tokens + 31) / 32;
  const int64_t max_tiles = L->lanes * lane_tiles_max;
  if (max_tiles >= (int64_t(1) << 31)) return fail(ATTN_ERR_UNSUPPORTED, "too many positions in one call");
  // Workers: matrix-core waves run eight per compute unit (two per SIMD, the
  // register budget) for bf16 and four (one per SIMD) for int8 or 32-column
  // waves, in workers of four waves.  The vector-ALU kernel runs four
  // 256-thread workgroups per unit.
  L->wpg = mfma ? 4 : 1;
  const int cus = device_cu_count();
  const int waves_per_cu = (L->cols >= 32 || a->kv_dtype == ATTN_I8) ? 4 : 8;
  // A paged cache whose pages hold each token's heads together (token-major
  // pages: a KV head's rows stride_t > D apart): twice as many workers as fit
  // at once, over half-length ranges, so the workers active together cover
  // fewer sequences and the heads of one token are read close together in
  // time.  128K decode over scattered token-major 64-token pages: 377 ->
  // 366 us.  A contiguous token-major cache measured 373 -> 383 us with the
  // same grid, and contiguous head rows 1-8% slower, so they keep one
  // dispatch round.  Only the library's default split does this: with the
  // caller's split_tokens the split depends on the lengths alone, so equal
  // split_tokens give bit-identical results over any layout.
  const bool spread_rows =
      mfma && !a->token_idx && a->split_tokens == 0 && g.block_table && g.stride_t != g.D;
  const int64_t grid_cap =
      mfma ? (int64_t)cus * waves_per_cu / L->wpg * (spread_rows ? 2 : 1) : (int64_t)cus * 4;
  if (a->split_tokens) {
    L->split = a->split_tokens;
  } else if (!mfma) {
    L->split = 256;
  } else if (a->token_idx) {
    // Gathered runs are short and a worker's fixed costs (staging its index
    // list and query, the combine, a partial) weigh more: at least 512 and
    // at most 1024 kept tokens per four-wave worker (32 pairs x 4096 kept
    // tokens of 128K, bf16: 256 per worker 26.3 us, 512 24.5 us, 1024
    // 26.2 us, 2048 37.9 us; int8: 128 26.4 us, 256 26.3, 512 25.7, 1024
    // 28.7 us).
    const int64_t ct = std::min<int64_t>(std::max<int64_t>(max_tiles / 256, 16), 32);
    L->split = (int32_t)(32 * ct);
  } else {
    // Every wave streams at least 32 tiles when there are enough: each
    // worker's result costs a partial write and a read in the merge, and
    // the grid's waves with their register rings already keep HBM busy.
    L->split = 32 * (spread_rows ? 16 : 32) * L->wpg;
  }
  // Buffer resources use 32-bit offsets: over one (sequence, KV head), or
  // over one page of a paged cache.
  const int64_t span_rows = (g.block_table ? (int64_t)g.page_tokens : (int64_t)g.max_seq_len) + 64;
  if (mfma && span_rows * g.stride_t * elem_size(a->kv_dtype) >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "one (sequence, KV head) or page may span at most 2 GiB of rows");
  // The grid: at most grid_cap workers, and no more than ranges of at least
  // split_tokens positions (the kernel's own rule), so the workers in use
  // are the first ones dispatched.
  const int64_t ct = L->split / 32;
  L->grid = (int32_t)std::max<int64_t>(1, std::min<int64_t>(grid_cap, (max_tiles + ct - 1) / ct));
  if (a->fixed_splits > 0) {
    // the unbalanced schedule: one worker per split of every lane
    if (L->lanes * a->fixed_splits >= (int64_t(1) << 31))
      return fail(ATTN_ERR_UNSUPPORTED, "fixed_splits: too many workers");
    L->grid = (int32_t)(L->lanes * a->fixed_splits);
  }
  // Non-temporal K/V loads: a plain 4 GiB read through buffer loads with
  // the nt bit moved 7.0-7.1 TB/s against 6.1-6.3 TB/s without, and the
  // 128K decode steps went from 361 to 329 us (bf16) and 188 to 168 us
  // (int8).  Each such load takes longer, though: with few workers in flight
  // they lose (a 4-lane share of the 128K step: 54 -> 75 us), and so do two
  // column groups of one worker, which meet each tile in the caches (8
  // query rows per sequence: 448 -> 601 us).  So they are used where the
  // kernel's XCD-weighted split applies at the longest lengths the call
  // allows: one column group, and work for every worker.
  L->stream_nt = mfma && !a->token_idx && a->fixed_splits == 0 && L->ngb == 1 &&
                 max_tiles * 15 >= (int64_t)L->grid * 16 * ct;
  const int64_t QH = (int64_t)g.KH * a->G * R;
  if (mfma) {
    // A lane's workers: every worker's range is at least ct tiles (the
    // kernel's worker count ensures it), so a lane touches at most
    // ceil(tiles / ct) + 1 ranges, and there are at most grid workers.
    L->max_chunks = 0;
    L->max_slots = a->fixed_splits > 0 ? a->fixed_splits
                                       : std::min<int64_t>(L->grid, (lane_tiles_max + ct - 1) / ct + 1);
    L->max_partials = (int64_t)g.B * QH * L->max_slots;
  } else {
    L->max_chunks = ((int64_t)L->max_tokens + L->split - 1) / L->split;
    L->max_slots = 0;
    L->max_partials = 2 * (int64_t)g.B * QH * L->max_chunks;
  }
  if (L->max_partials >= (int64_t(1) << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "too many split-KV partials (reduce max_seq_len or raise split_tokens)");
  size_t off = 0;
  L->m = off; off = align256(off + L->max_partials * sizeof(float));
  L->l = off; off = align256(off + L->max_partials * sizeof(float));
  L->o = off; off = align256(off + (size_t)L->max_partials * g.D * sizeof(float));
  L->ctr = off;
  if (mfma) off = align256(off + (size_t)L->lanes * sizeof(uint64_t));
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

}  // extern "C"

namespace lcdg {

// The 40-bit tag of one call's arrival counters (or of the OAM selection's
// histogram words, which follow the same rule).  Each counter array (a
// workspace address and layout) gets the tag after the one its previous call
// used, which is the tag that call's last arrivals left in the words, so the
// common case costs one atomic add per arrival; an array not seen recently
// (64 remembered, replaced in turn) gets a fresh tag from a scrambled
// sequence, and its first arrivals take the words over.  Tags change with
// every call, so words left by any earlier call are never mistaken for live
// counts of this one.
uint64_t counter_tag_for(const void *ctr) {
  constexpr uint64_t kMask = (uint64_t(1) << 40) - 1;
  static std::mutex mu;
  static const void *addr[64] = {nullptr};
  static uint64_t tag[64];
  static unsigned victim = 0;
  static uint64_t fresh = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < 64; ++i)
    if (addr[i] == ctr) return tag[i] = (tag[i] + 1) & kMask;
  const unsigned i = victim++ % 64;
  addr[i] = ctr;
  tag[i] = ((++fresh) * 0x9E3779B97F4A7C15ull >> 24) & kMask;
  return tag[i];
}

// One decode call on a validated workspace: `workspace` / `workspace_bytes`
// take the place of the arguments' own (the no-allocation entry point passes
// its static scratch here).
attn_status decode_run(const attn_decode_args *a, void *workspace, size_t workspace_bytes, attn_stream_t stream,
                       void *const *events) {
  DecodeLayout L;
  attn_status st = plan_decode(a, &L);
  if (st != ATTN_OK) return st;
  if (a->kv.B == 0) return ATTN_OK;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(ATTN_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
  if (workspace_bytes < L.total) return fail(ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than required");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  DecodeParams p;
  p.B = a->kv.B;
  p.KH = a->kv.KH;
  p.R = a->q_rows > 1 ? a->q_rows : 1;
  p.Gq = a->G;
  p.G = a->G * p.R;
  p.D = a->kv.D;
  p.QH = a->kv.KH * p.G;
  p.ngb = L.ngb;
  p.lpp = L.mfma ? 1 : L.ngb;
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
  p.max_slots = (int32_t)L.max_slots;
  p.wpg = L.wpg;
  p.fixed_splits = a->fixed_splits;
  p.stream_nt = L.stream_nt ? 1 : 0;
  // the vector-ALU decode with one worker and one chunk per lane: every
  // lane's partial is its result, so the kernel writes out and lse and the
  // merge launch is skipped
  p.direct_out = (!L.mfma && L.grid == 1 && L.max_chunks == 1 && a->fixed_splits == 0) ? 1 : 0;
  p.grid = L.grid;
  p.wl.m_part = reinterpret_cast<float *>(ws + L.m);
  p.wl.l_part = reinterpret_cast<float *>(ws + L.l);
  p.wl.o_part = reinterpret_cast<float *>(ws + L.o);
  p.wl.ctr = L.mfma ? reinterpret_cast<uint64_t *>(ws + L.ctr) : nullptr;
  p.wl.ctr_tag = L.mfma ? counter_tag_for(p.wl.ctr) : 0;
  p.out_dtype = a->out_dtype;
  p.out = a->out;
  p.lse = a->lse;

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
  if (!L.mfma && !p.direct_out) {
    e = launch_merge_decode(p, a->out_dtype, a->out, a->lse, s);
    if (e != hipSuccess) return fail_hip(e, "merge launch");
  }
  if ((e = mark(2)) != hipSuccess) return fail_hip(e, "event record");
  return ATTN_OK;
}

}  // namespace lcdg

extern "C" {

attn_status attn_decode_splitkv(const attn_decode_args *a, attn_stream_t stream) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  return decode_run(a, a->workspace, a->workspace_bytes, stream, nullptr);
}

attn_status attn_decode_splitkv_profiled(const attn_decode_args *a, attn_stream_t stream, void *const events[3]) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  return decode_run(a, a->workspace, a->workspace_bytes, stream, events);
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
  if (bytes >= ((size_t)1 << 43)) return fail(ATTN_ERR_UNSUPPORTED, "read: at most 2^43 - 16 bytes");
  hipError_t e = launch_read(src, bytes, sink, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : fail_hip(e, "read launch");
}

}  // extern "C"
