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

// ---------------------------------------------------------------- work-list

// Device work-list shared by the decode kernels.
//
// A "lane" is (b, kh, query-head block of up to 16 heads); lane q covers
// ceil(n_q / 32) tiles of 32 token positions, and all lanes' tiles are laid
// end to end (lane q starts at tile_start[q]).  The decode grid splits this
// tile stream into equal contiguous ranges, one per workgroup, so every
// workgroup streams the same number of K/V bytes whatever the length mix.
// Each lane is also cut into chunks of split_tokens positions; a chunk owns
// two partial slots because at most one range boundary can fall inside it
// (ranges are at least one chunk long).  Slot 2j is the part of chunk j
// before that boundary (or all of it), slot 2j+1 the part after (or empty).
struct WorkList {
  int32_t *hdr;              // [0] tiles in total, [1] workgroups in use
  int32_t *tile_start;       // [nlanes + 1]
  int32_t *row_split_start;  // [B*QH + 1] first partial slot of each output row
  float *m_part;             // [max partials] natural-log max
  float *l_part;             // [max partials]
  float *o_part;             // [max partials][D]
};

struct DecodeParams {
  int32_t B, KH, G, D, QH, ngb;
  const int32_t *seq_lens;
  const int64_t *seq_offset;
  int64_t stride_h, stride_t;
  const void *q, *k, *v;
  const float *k_scale;
  int32_t k_part, k_scale_stride;
  float v_scale;
  const int32_t *token_idx, *n_idx;
  int32_t idx_stride;
  float softmax_scale;
  int32_t split;        // tokens per chunk (multiple of 32)
  int32_t max_seq_len;  // lengths are clamped to this bound
  int32_t grid;         // workgroups launched for the decode kernel
  WorkList wl;
};

// Host-side launchers (each returns hipSuccess or the launch error).
hipError_t launch_worklist(const DecodeParams &p, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeParams &p, int kv_dtype, hipStream_t s);
hipError_t launch_decode_valu(const DecodeParams &p, int q_dtype, int kv_dtype, hipStream_t s);
hipError_t launch_merge(const float *o_part, const float *m_part, const float *l_part, const int32_t *rss,
                        int32_t rows, int32_t D, int32_t out_dtype, void *out, float *lse, hipStream_t s);
hipError_t launch_quant_partitions(const attn_kv_geom &g, const void *x, int32_t part, int32_t scale_stride,
                                   int8_t *codes, float *scales, hipStream_t s);
hipError_t launch_quant_tensor(const attn_kv_geom &g, const void *x, int8_t *codes, float *scales,
                               uint32_t *ws, hipStream_t s);
hipError_t launch_value_lognorm(const attn_kv_geom &g, const void *v, float eps, float *vlog, int32_t stride,
                                hipStream_t s);
hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s);
hipError_t launch_read(const void *src, size_t bytes, float *sink, hipStream_t s);

struct OamPlan {
  float *scores;         // [npairs][score_stride]
  int32_t score_stride;
  float *vlog;           // value log-norms: the caller's or computed into the workspace
  int32_t vlog_stride;
  uint32_t *hist;        // [3][npairs][2048]
  int32_t *chunk_cnt;    // [npairs][nchunk][2]
  int32_t *offsets;      // [npairs][nchunk][2]
  int32_t *state;        // [npairs][4]
  int32_t nchunk;        // selection blocks per pair
};
hipError_t launch_oam(const oam_topk_args &a, const OamPlan &plan, hipStream_t s);
int oam_block_tokens();

int device_cu_count();

}  // namespace lcdg
