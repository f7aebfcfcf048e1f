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

// Split-KV partial buffers.  The matrix-core decode gives each pair (b, kh) =
// b*KH + kh max_slots slots: a lane's partial from its k-th worker goes to
// slot k, the entry of column g being (pair*max_slots + k)*G + g.  The
// vector-ALU decode gives each pair 2*max_chunks slots, two per chunk of
// split_tokens positions: at most one worker-range boundary can fall inside
// a chunk, so slot 2j holds the part of chunk j before that boundary (or all
// of it) and slot 2j+1 the part after it (or an empty partial: m = -inf,
// l = 0), at entry (pair*2*max_chunks + j)*G + g; its merge is a separate
// launch.
struct WorkList {
  float *m_part;             // [max partials] natural-log max
  float *l_part;             // [max partials]
  float *o_part;             // [max partials][D]
  // Merge inside the matrix-core decode launch: one arrival counter per lane.
  // A counter word holds (ctr_tag << 24) | arrivals, ctr_tag being a 40-bit
  // tag that changes with every call on the same counter array.  A call's
  // last arrivals leave their words at zero arrivals under the next call's
  // tag, and a word without this call's tag (left by an earlier call,
  // finished or cut off, or other data) is taken over by the call's first
  // arrival, so the workspace needs no clearing.
  uint64_t *ctr;             // [lanes] (matrix-core decode)
  uint64_t ctr_tag;          // < 2^40
};

struct DecodeParams {
  // G: query rows per KV head (the matrix-core columns), R * Gq; QH = KH * G
  // ngb: column blocks per KV head (16-row blocks for the vector-ALU decode,
  // 32-column groups of one worker for the matrix-core decode); lpp: lanes
  // per pair (ngb for the vector-ALU decode, 1 for the matrix-core decode)
  int32_t B, KH, G, D, QH, ngb, lpp;
  int32_t Gq, R;  // query heads per KV head, query rows per sequence
  int32_t cols_per_wave;  // matrix-core columns of a decode wave: 16, 32 when G > 16, 64 (bf16 by position) when G > 32
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
  int32_t max_chunks;   // chunks of the longest possible row (vector-ALU decode)
  int32_t max_slots;    // partial slots per pair (matrix-core decode)
  int32_t grid;         // workgroups launched for the decode kernel
  int32_t wpg;          // waves per decode workgroup (the MFMA kernel's workers)
  int32_t fixed_splits; // matrix-core decode: 0 = balanced split; S > 0 = each lane in S splits, one worker each
  int32_t stream_nt;    // matrix-core decode: non-temporal K/V loads (the launch streams over a full grid)
  int32_t direct_out;   // vector-ALU decode: one worker and one chunk per lane, so it writes out and lse itself
  WorkList wl;
  // outputs, written by the matrix-core decode launch
  int32_t out_dtype;
  void *out;
  float *lse;
};

// Row of q/out/lse ([B][R][KH*Gq]) of column gc (= r*Gq + g) of KV head kh.
__device__ __forceinline__ int64_t q_row_index(const DecodeParams &p, int b, int kh, int gc) {
  const int r = gc / p.Gq, g = gc - r * p.Gq;
  return ((int64_t)(b * p.R + r) * p.KH + kh) * p.Gq + g;
}

// A "lane" is (b, kh, query-head block) (the matrix-core decode: (b, kh)):
// lane q belongs to pair q / lpp = b*KH + kh and covers ceil(n / 32) tiles of
// 32 positions,
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
  return q < p.B * p.KH * p.lpp ? (pair_positions(p, q / p.lpp) + 31) / 32 : 0;
}

// Inclusive prefix sum over the 64 lanes of a wave, in six DPP moves (no
// trip through the LDS crossbar): shifts by 1, 2, 4 and 8 lanes inside each
// row of 16 lanes (a lane whose source lies before its row's start adds 0),
// then lane 15's sum into the next row for rows 1 and 3 (row_bcast:15), and
// lane 31's (rows 0-1) into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}
// The sum over the wave (uniform).
__device__ __forceinline__ int wave_sum_int(int v) { return __builtin_amdgcn_readlane(wave_incl_scan(v), 63); }

// Tiles of all nl lanes (wave-wide; every thread of the wave gets the total),
// tiles(q) giving lane q's tile count.
template <class F>
__device__ __forceinline__ int wave_total_tiles_of(int nl, F tiles) {
  int acc = 0;
  for (int q = threadIdx.x & 63; q < nl; q += 64) acc += tiles(q);
  return __builtin_amdgcn_readfirstlane(wave_sum_int(acc));
}
__device__ __forceinline__ int wave_total_tiles(const DecodeParams &p) {
  return wave_total_tiles_of(p.B * p.KH * p.lpp, [&](int q) { return lane_tiles(p, q); });
}

// The lane holding tile t (0 <= t < total) and that lane's first tile and tile
// count, by a scan over the lanes 64 at a time (wave-wide, uniform result).
struct LaneHit {
  int q, t0, nt;
};
template <class F>
__device__ __forceinline__ LaneHit wave_find_lane_of(int nl, int t, F tiles) {
  const int lane = threadIdx.x & 63;
  LaneHit h = {0, 0, 0};
  int run = 0;
  for (int base = 0; base < nl; base += 64) {
    const int nt = base + lane < nl ? tiles(base + lane) : 0;
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
__device__ __forceinline__ LaneHit wave_find_lane(const DecodeParams &p, int t) {
  return wave_find_lane_of(p.B * p.KH * p.lpp, t, [&](int q) { return lane_tiles(p, q); });
}

// The lane after h that has tiles (its first tile follows h's last).
template <class F>
__device__ __forceinline__ LaneHit next_lane_of(int nl, LaneHit h, F tiles) {
  LaneHit n = {h.q, h.t0 + h.nt, 0};
  while (n.nt == 0 && n.q + 1 < nl) {
    ++n.q;
    n.nt = __builtin_amdgcn_readfirstlane(tiles(n.q));
  }
  return n;
}
__device__ __forceinline__ LaneHit next_lane(const DecodeParams &p, LaneHit h) {
  return next_lane_of(p.B * p.KH * p.lpp, h, [&](int q) { return lane_tiles(p, q); });
}

// Workers that get a range: at most one per chunk's worth of tiles, so every
// range is at least one chunk long.
__device__ __forceinline__ int workers_for(const DecodeParams &p, int total_tiles) {
  return total_tiles == 0 ? 0 : min(p.grid, max(1, total_tiles / (p.split / 32)));
}

// Static split of the matrix-core decode's tile stream into one contiguous
// range per worker.  When the work fills the whole grid (every compute unit
// runs its full complement of workers) the split is XCD-aware: workgroup w
// runs on XCD w % 8 (workgroups are dealt to the eight XCDs in turn), and
// under that full load the odd-numbered XCDs stream about 6% slower than
// the even ones (measured per worker on several MI355X boxes, with the
// ranges rotated by one worker to show it follows the XCD, not the memory
// range), so a worker on an odd XCD gets weight 15 and one on an even XCD
// 16: worker w's range is [start(w), start(w+1)), start(w) = floor(T * S(w)
// / S(W)), S(w) = the sum of the weights of workers 0 .. w-1.  With fewer
// workers the XCDs do not contend, and with two column groups per worker
// (more than 32 query rows per KV head) each byte carries twice the matrix
// work and the weighted split measured 2% slower than the equal one; in
// both cases the split is equal, start(w) = floor(w * T / W).  Every range is at least ct = split / 32 tiles: the
// weighted split runs W = grid <= 15 T / (16 ct) workers, and start(w+1) -
// start(w) >= floor(15 T / (16 W)) >= ct; the equal one at most T / ct.  So
// no range is empty, and a lane of n tiles touches at most ceil(n / ct) + 1.
struct StreamSplit {
  int W;          // workers
  bool weighted;  // XCD-weighted (else equal)
};
// floor(n / d) for 0 <= n < 2^53 and d > 0, exactly, in fp64: an integer
// quotient is exact, and otherwise the correctly rounded quotient r of q =
// n / d stays in [floor(q), floor(q) + 1), because q lies at least 1/d below
// the next integer while |r - q| <= q * 2^-53 < 1/d.  About twenty fp64
// instructions, where a 64-bit integer division is a chain of more than a
// hundred (several per worker at every launch's start).
__device__ __forceinline__ int64_t floor_div53(int64_t n, int64_t d) {
  return (int64_t)((double)n / (double)d);
}
__device__ __forceinline__ int64_t xcd_weight_sum(int w) {
  const int r = w & 7;
  return (int64_t)(w >> 3) * (4 * 16 + 4 * 15) + (int64_t)((r + 1) / 2) * 16 + (int64_t)(r / 2) * 15;
}
__device__ __forceinline__ StreamSplit stream_split(const DecodeParams &p, int T, bool xcd_weights) {
  StreamSplit r = {0, false};
  if (T == 0) return r;
  const int ct = p.split / 32;
  // floor(15 T / (16 ct)) >= grid, without the division
  if (p.ngb == 1 && (int64_t)T * 15 >= (int64_t)p.grid * 16 * ct) {
    r.W = p.grid;
    r.weighted = xcd_weights;
  } else {
    r.W = min(p.grid, max(1, T / ct));
  }
  return r;
}
// The products below stay far under 2^53: T < 2^31 tiles and S(W) < 2^18.
__device__ __forceinline__ int range_start(int w, int T, StreamSplit sp) {
  if (sp.weighted) return (int)floor_div53((int64_t)T * xcd_weight_sum(w), xcd_weight_sum(sp.W));
  return (int)floor_div53((int64_t)w * T, sp.W);
}
// The worker whose range holds tile t (0 <= t < T): the largest w with
// start(w) <= t.  Equal split: w = floor(((t+1)*W - 1) / T).  Weighted: the
// largest w with T*S(w) < (t+1)*S(W), i.e. S(w) <= X = floor(((t+1)*S(W) - 1)
// / T); S(8k + r) = 124k + P(r) (124 = four weights of 16 and four of 15;
// P(r) = 0, 16, 31, 47, 62, 78, 93, 109), so w = 8k + r with k = X / 124 and r
// the largest with P(r) <= X - 124k.
__device__ __forceinline__ int worker_of(int t, int T, StreamSplit sp) {
  if (!sp.weighted) return (int)floor_div53((int64_t)(t + 1) * sp.W - 1, T);
  const int X = (int)floor_div53((int64_t)(t + 1) * xcd_weight_sum(sp.W) - 1, T);
  const int k = X / 124, rem = X - k * 124;
  const int r = (rem >= 16) + (rem >= 31) + (rem >= 47) + (rem >= 62) + (rem >= 78) + (rem >= 93) + (rem >= 109);
  return min(8 * k + r, sp.W - 1);
}

// One arrival on a counter word (see WorkList::ctr), in two halves so that
// several arrivals can be in flight together: counter_add issues the atomic
// add and returns the old word; counter_resolve turns that into the
// arrivals of this call so far, this one included.  With the call's tag in
// the old word that is the one atomic add.  An arrival that finds another
// tag (the first of each shared lane in a call) sets the word to the tagged
// count 1 by compare-and-swap, or, when another arrival did that first, adds
// itself again (its first add went into the old word); this loop ends
// because every failed exchange means another arrival changed the word.
// Relaxed at agent scope: the caller orders its own partial stores before
// the add (they are device-scope stores, complete once vmcnt drains) and
// issues the merge's loads only after the result returns.
__device__ __forceinline__ uint64_t counter_add(uint64_t *c) {
  return __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int counter_resolve(uint64_t *c, uint64_t old, uint64_t tag) {
  const uint64_t clean = tag << 24;
  if ((old >> 24) == tag) return (int)(old & 0xFFFFFFu) + 1;
  uint64_t cur = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if ((cur >> 24) == tag) {
      const uint64_t again = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return (int)(again & 0xFFFFFFu) + 1;
    }
    uint64_t expect = cur;
    if (__hip_atomic_compare_exchange_strong(c, &expect, clean | 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return 1;
    cur = expect;
  }
}

// The last arrival of a call leaves the counter at zero arrivals under the
// next tag, the one the next call on the same counter array uses.
__device__ __forceinline__ void counter_reset(uint64_t *c, uint64_t tag) {
  __hip_atomic_store(c, ((tag + 1) & ((1ull << 40) - 1)) << 24, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every vector-memory access this wave issued has completed; for
// device-scope (sc1) stores that means they are visible to every compute unit.
__device__ __forceinline__ void wait_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt left free
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Cache policy of the merge's buffer accesses: device scope (sc1), so stores
// write through to memory every XCD reads and loads fetch from there.
constexpr int kDeviceScope = 16;
// Cache policy of the K/V stream: non-temporal (nt).  Every cache row is read
// once per call, and a plain read of 4 GiB through buffer loads with this bit
// moved 7.0-7.1 TB/s on MI355X against 6.1-6.3 TB/s without it.
constexpr int kStream = 2;

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
  uint64_t *hist;        // [npairs][2048] level-0 key histogram, tagged words (tag << 24) | count
  int32_t *state;        // [npairs][8] selection state
  int32_t *blk_gt;       // [npairs][oam_max_tokens() / 2048]
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
// The tag of the next call on a tagged counter array (arrival counters, OAM histogram words).
uint64_t counter_tag_for(const void *ctr);

}  // namespace lcdg
