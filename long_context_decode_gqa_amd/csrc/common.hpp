// Shared device/host definitions of the gfx950 decode-attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_decode.h"

namespace lcdg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48 end with the same result).  gfx950's row-swap permutes exchange whole
// rows between two registers without a trip through LDS: given x twice,
// the 16-lane swap returns rows (0,0,2,2) and (1,1,3,3), the 32-lane swap
// halves (lo,lo) and (hi,hi).
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Wave-uniform copies of values every lane holds alike: they then live in
// scalar registers, and a buffer resource built from them needs no per-lane
// (waterfall) loop around each load.
__device__ __forceinline__ int uniform_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- work split

// Split-KV partial buffers.  Pair (b, kh) = b*KH + kh owns 2*max_chunks slots,
// two per chunk of split_tokens positions: at most one worker-range boundary
// can fall inside a chunk, so slot 2j holds the part of chunk j before that
// boundary (or all of it) and slot 2j+1 the part after it (or an empty
// partial: m = -inf, l = 0).  The partial of head g in slot j is entry
// (pair*2*max_chunks + j)*G + g, so one worker's partials of a head group are
// contiguous.  Slots of chunks past the pair's own chunk count are never read.
struct WorkList {
  float *m_part;             // [max partials] natural-log max
  float *l_part;             // [max partials]
  float *o_part;             // [max partials][D]
};

struct DecodeParams {
  // G: query rows per KV head (the matrix-core columns), R * Gq; QH = KH * G
  int32_t B, KH, G, D, QH, ngb;
  int32_t Gq, R;  // query heads per KV head, query rows per sequence
  int32_t cols_per_wave;  // matrix-core columns a decode worker computes: 16, or 32 when G > 16
  const int32_t *seq_lens;
  const int64_t *seq_offset;
  int64_t stride_h, stride_t;
  const void *q, *k, *v;
  const float *k_scale;
  int32_t k_part, k_scale_stride;
  float v_scale;
  int32_t q_quant;  // attn_q_quant (int8 KV)
  float q_scale;    // static query scale (ATTN_QUANT_STATIC)
  const int32_t *block_table;  // paged cache (NULL: rows at seq_offset[b])
  int32_t page_tokens, table_stride;
  int64_t page_stride;
  const int32_t *token_idx, *n_idx;
  int32_t idx_stride;
  float softmax_scale;
  int32_t split;        // tokens per chunk (multiple of 32)
  int32_t max_seq_len;  // lengths are clamped to this bound
  int32_t max_chunks;   // chunks of the longest possible row
  int32_t grid;         // workgroups launched for the decode kernel
  WorkList wl;
};

// Row of q/out/lse ([B][R][KH*Gq]) of column gc (= r*Gq + g) of KV head kh.
__device__ __forceinline__ int64_t q_row_index(const DecodeParams &p, int b, int kh, int gc) {
  const int r = gc / p.Gq, g = gc - r * p.Gq;
  return ((int64_t)(b * p.R + r) * p.KH + kh) * p.Gq + g;
}

// A "lane" is (b, kh, query-head block of up to 16 heads): lane q belongs to
// pair q / ngb = b*KH + kh and covers ceil(n / 32) tiles of 32 positions,
// n = the sequence length (or kept-index count in indexed mode), clamped to
// the declared bounds.  All lanes' tiles are laid end to end in lane order;
// decode workers split that stream into equal contiguous ranges, so every
// worker streams the same number of K/V bytes whatever the length mix.
__device__ __forceinline__ int pair_positions(const DecodeParams &p, int pair) {
  const int b = pair / p.KH;
  const int L = min(max(p.seq_lens[b], 0), p.max_seq_len);
  if (p.token_idx) return L > 0 ? min(max(p.n_idx[pair], 0), p.idx_stride) : 0;
  return L;
}
__device__ __forceinline__ int pair_chunks(const DecodeParams &p, int pair) {
  return (pair_positions(p, pair) + p.split - 1) / p.split;
}
__device__ __forceinline__ int lane_tiles(const DecodeParams &p, int q) {
  return q < p.B * p.KH * p.ngb ? (pair_positions(p, q / p.ngb) + 31) / 32 : 0;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(v, o);
    if (lane >= o) v += x;
  }
  return v;
}

// Tiles of all lanes (wave-wide; every thread of the wave gets the total).
__device__ __forceinline__ int wave_total_tiles(const DecodeParams &p) {
  const int nl = p.B * p.KH * p.ngb;
  int acc = 0;
  for (int q = threadIdx.x & 63; q < nl; q += 64) acc += lane_tiles(p, q);
  return __builtin_amdgcn_readfirstlane(wave_sum_int(acc));
}

// The lane holding tile t (0 <= t < total) and that lane's first tile and tile
// count, by a scan over the lanes 64 at a time (wave-wide, uniform result).
struct LaneHit {
  int q, t0, nt;
};
__device__ __forceinline__ LaneHit wave_find_lane(const DecodeParams &p, int t) {
  const int lane = threadIdx.x & 63;
  const int nl = p.B * p.KH * p.ngb;
  LaneHit h = {0, 0, 0};
  int run = 0;
  for (int base = 0; base < nl; base += 64) {
    const int nt = lane_tiles(p, base + lane);
    const int incl = wave_incl_scan(nt);
    const int excl = run + incl - nt;
    const unsigned long long own = __ballot(nt > 0 && excl <= t && t < excl + nt);
    if (own) {
      const int src = __builtin_ctzll(own);
      h.q = base + src;
      h.t0 = __builtin_amdgcn_readlane(excl, src);
      h.nt = __builtin_amdgcn_readlane(nt, src);
      break;
    }
    run += __builtin_amdgcn_readlane(incl, 63);
  }
  return h;
}

// The lane after h that has tiles (its first tile follows h's last).
__device__ __forceinline__ LaneHit next_lane(const DecodeParams &p, LaneHit h) {
  const int nl = p.B * p.KH * p.ngb;
  LaneHit n = {h.q, h.t0 + h.nt, 0};
  while (n.nt == 0 && n.q + 1 < nl) {
    ++n.q;
    n.nt = __builtin_amdgcn_readfirstlane(lane_tiles(p, n.q));
  }
  return n;
}

// Workers that get a range: at most one per chunk's worth of tiles, so every
// range is at least one chunk long.
__device__ __forceinline__ int workers_for(const DecodeParams &p, int total_tiles) {
  return total_tiles == 0 ? 0 : min(p.grid, max(1, total_tiles / (p.split / 32)));
}

// Host-side launchers (each returns hipSuccess or the launch error).
hipError_t launch_merge_decode(const DecodeParams &p, int32_t out_dtype, void *out, float *lse, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeParams &p, int kv_dtype, hipStream_t s);
hipError_t launch_decode_valu(const DecodeParams &p, int q_dtype, int kv_dtype, hipStream_t s);
hipError_t launch_merge(const float *o_part, const float *m_part, const float *l_part, const int32_t *rss,
                        int32_t rows, int32_t D, int32_t out_dtype, void *out, float *lse, hipStream_t s);
hipError_t launch_quant_partitions(const attn_kv_geom &g, const void *x, int32_t part, int32_t scale_stride,
                                   int8_t *codes, float *scales, hipStream_t s);
hipError_t launch_quant_tensor(const attn_kv_geom &g, const void *x, int8_t *codes, float *scales, void *ws,
                               hipStream_t s);
size_t quant_tensor_workspace_bytes(const attn_kv_geom &g);
hipError_t launch_value_lognorm(const attn_kv_geom &g, const void *v, int32_t v_dtype, float v_scale, float eps,
                                float *vlog, int32_t stride, hipStream_t s);
hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s);
hipError_t launch_read(const void *src, size_t bytes, float *sink, hipStream_t s);

struct OamPlan {
  float *scores;         // [npairs][score_stride]
  int32_t score_stride;
  float *vlog;           // value log-norms: the caller's or computed into the workspace
  int32_t vlog_stride;
  uint32_t *hist;        // [npairs][2048] level-0 key histogram, followed by
  int32_t *state;        // [npairs][8] selection state
  int32_t *blk_gt;       // [npairs][oam_max_tokens() / 2048]
  int32_t *blk_off;      // [npairs][oam_max_tokens() / 2048]
  int32_t *blk_nc;       // [npairs][1024] candidates per block
  float *bscores;        // [npairs][bs_stride] block scores (block-granular selection)
  int32_t bs_stride;
  uint32_t *cand_key;    // [npairs][score_stride] per-block candidate regions
  int32_t *cand_idx;     // [npairs][score_stride]
};
hipError_t launch_oam(const oam_topk_args &a, const OamPlan &plan, hipStream_t s);
int oam_max_tokens();  // longest sequence oam_score_topk selects over
int oam_max_select_blocks();  // most token blocks per pair in block-granular selection

int device_cu_count();

}  // namespace lcdg
