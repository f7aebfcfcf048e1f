// Output-aware token scoring and exact top-K selection
// ("优化稀疏注意力中的令牌丢弃机制" §3: rank tokens by q.k_i/sqrt(d_k) +
// beta*log(||v_i|| + eps) and drop the lowest; §2 for the q.k ranking it
// replaces).  For each (b, kh) the G query heads' routing logits are averaged,
// so the G heads of a KV head share one kept set.
//
// The K-th largest score is found by radix selection on order-preserving
// 32-bit keys of the fp32 scores: digits of 11, 11 and 10 bits from the top,
// then, among keys equal to the threshold T, the lowest indices are kept.
// Passes (each needs the previous one complete, so they are separate launches):
//   score      (token blocks x pairs) S = K Q^T on the matrix cores, mean over
//              the G heads, scale, + beta * vlog; write the fp32 score and
//              count the top 11 key bits into the pair's level-0 histogram.
//   candidates (2048-token blocks x pairs) every block reads the pair's
//              histogram and finds the threshold's top digit b0 (all blocks
//              find the same); it counts its keys above bin b0 and writes its
//              keys of bin b0, with their indices, to its own region of the
//              pair's candidate array, and their count.
//   select     (one workgroup per pair) gathers the candidates into LDS, then
//              finds the exact threshold key T and the last kept index I_T
//              among keys equal to T; then the output offset of every block.
//              (If there are more candidates than LDS holds - many equal
//              scores - it selects over the pair's scores directly.)
//   write      (2048-token blocks x pairs) ordered compaction of the kept
//              tokens, key > T or (key == T and index <= I_T), at the block's
//              offset, so idx_out is ascending.
// Only integer atomics (histogram counts) cross workgroups within a pass.
#include "common.hpp"

namespace lcdg {
namespace {

constexpr int kBins = 2048;       // 11-bit digits (the 10-bit ones use 1024)
constexpr int kBlockTok = 2048;   // tokens per workgroup of the candidate and write passes
constexpr int kCandCap = 12288;   // candidates the select pass holds in LDS (10 bytes each)
constexpr int kMaxBlocks = 1024;  // blocks of kBlockTok per pair (sequences up to 2M tokens)
constexpr int kMaxSelBlocks = 8192;  // token blocks per pair the block-granular select holds

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Per-pair selection state, passed from one pass to the next.
struct OamState {
  int32_t b0;        // top 11 bits of the threshold key
  int32_t need;      // keys of bin b0 to keep
  uint32_t T;        // threshold key
  int32_t I_T;       // last kept index among keys equal to T
  int32_t pad[4];
};

struct OamDev {
  int32_t B, KH, G, D, QH, L_max, L_cap, top_k;  // L_max: score row stride; L_cap: length bound
  const int32_t *seq_lens;
  const int64_t *seq_offset;
  int64_t stride_h, stride_t;
  const int32_t *block_table;  // paged cache (else null): page of row t of sequence b
  int32_t page_tokens, table_stride;
  int64_t page_stride;
  const uint16_t *q;
  const void *k;       // bf16 or int8 codes
  const float *k_scale;  // int8: scale of row t is k_scale[pair*k_scale_stride + t/k_part]
  int32_t k_part, k_scale_stride;
  const float *vlog;
  int32_t vlog_stride;
  float score_scale, beta;
  float *scores;       // [npairs][L_max]
  uint32_t *hist;      // [npairs][kBins]  level-0 histogram
  OamState *state;     // [npairs]
  int32_t *blk_gt;     // [npairs][kMaxBlocks]  keys above bin b0 per block
  int32_t *blk_off;    // [npairs][kMaxBlocks]  first output slot per block
  int32_t *blk_nc;     // [npairs][kMaxBlocks]  candidates (keys in bin b0) per block
  uint32_t *cand_key;  // [npairs][L_max]  block j's candidates at [j*kBlockTok, + blk_nc)
  int32_t *cand_idx;   // [npairs][L_max]
  int32_t *idx_out;    // [npairs][top_k * max(block_tokens, 1)]
  int32_t *n_kept;     // [npairs]
  int32_t block_tokens;  // > 1: block-granular selection of top_k blocks
  int32_t write_scores;  // token scores are written (token mode, or asked for)
  float *bscores;        // [npairs][bs_stride] block scores (block mode)
  int32_t bs_stride;
};

__device__ __forceinline__ int pair_len(const OamDev &o, int pair) {
  return min(max(o.seq_lens[pair / o.KH], 0), o.L_cap);
}

// Exclusive prefix sum of one value per thread over a 256-thread block;
// *total gets the sum.  Every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_tmp, int *total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o);
    if (lane >= o) incl += x;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_tmp[w];
  const int tot = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// In a histogram of nb bins (1024 or 2048), the bin holding the need-th
// largest entry (1 <= need <= entries): returns it and sets *above to the
// entries in higher bins.  All 256 threads call it; all get the result.
__device__ int select_bin(const uint32_t *hist, int nb, int need, int *above, int *s_tmp, int *s_res) {
  const int tid = threadIdx.x;
  const int per = nb / 256;  // bins per thread, taken from the top down
  int local = 0;
  for (int j = 0; j < per; ++j) local += (int)hist[nb - 1 - (tid * per + j)];
  int tot;
  const int before = block_exclusive_scan(local, s_tmp, &tot);
  if (before < need && need <= before + local) {
    int run = before;
    for (int j = 0; j < per; ++j) {
      const int bin = nb - 1 - (tid * per + j);
      const int h = (int)hist[bin];
      if (run < need && need <= run + h) {
        s_res[0] = bin;
        s_res[1] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  const int bin = s_res[0];
  *above = s_res[1];
  __syncthreads();
  return bin;
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// Score pass.  The mean query of the KV head's G heads, q_bar (fp32), is
// split into three bf16 parts hi + mid + lo (24 significant bits) placed in
// B-operand columns 4j, 4j+1, 4j+2 (column 4j+3 is zero), so one 16x16x32
// MFMA chain per 16 tokens gives, in every lane quad, the three partial dot
// products of its four tokens; two quad DPP adds finish q_bar . k_t.  For an
// INT8 cache the same columns hold the three int8 digits of q_bar as a 22-bit
// fixed-point integer, the int8 MFMA consumes the K codes as loaded, and the
// quad add recombines the digit sums (weights 1, 256, 65536) before the
// scale of q_bar and the K partition scale apply.  Each wave of the
// workgroup streams a quarter of its tokens in 32-token tiles.
constexpr int kScoreTok = 8192;   // tokens per workgroup of the score pass
constexpr int kScoreBufs = 3;     // tiles in the register ring of each wave

__device__ __forceinline__ float quad_sum3(float v) {
  // lane 4j gets v(4j) + v(4j+1) + v(4j+2); quad_perm(1,2,3,0) = 0x39, (2,3,0,1) = 0x4E
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x39, 0xF, 0xF, true));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v + a + b;
}

template <int D, int KVT, bool PAGED>
__global__ __launch_bounds__(256) void oam_score_kernel(OamDev o) {
  constexpr bool I8 = KVT == ATTN_I8;
  static_assert(D <= 256, "one thread per channel for the mean query");
  constexpr int KB = I8 ? D / 64 : D / 32;  // MFMAs per 16 tokens (16x16x64 int8 or 16x16x32 bf16)
  constexpr int ES = I8 ? 1 : 2;            // bytes per K element
  // an int8 tile carries half the bytes of a bf16 one: more tiles in flight
  constexpr int NBUF = I8 ? 5 : kScoreBufs;
  __shared__ uint32_t s_hist[kBins];
  __shared__ float s_qbar[D];
  __shared__ float s_sc[kScoreTok];
  // paged: the page ids under the workgroup's tokens (at most kScoreTok / 32
  // + 1 pages, as a page holds a positive multiple of 32 tokens)
  __shared__ int s_pages[PAGED ? kScoreTok / 32 + 1 : 1];
  const int pair = blockIdx.y;
  const int b = pair / o.KH, kh = pair - b * o.KH;
  const int tid = threadIdx.x, lane = tid & 63;
  // The set-up's loads (the length, the offset and the group's G <= 16
  // queries of channel tid) go out together, before the length is checked:
  // one memory latency instead of three in a row.
  const int len_raw = o.seq_lens[b];
  const int64_t seq_off = PAGED ? 0 : o.seq_offset[b];
  float qv[16];
  {
    const uint16_t *q0 = o.q + ((int64_t)b * o.QH + (int64_t)kh * o.G) * D + min(tid, D - 1);
#pragma unroll
    for (int g = 0; g < 16; ++g) qv[g] = bf16_bits_to_f32(q0[(int64_t)min(g, o.G - 1) * D]);
  }
  const int L = min(max(len_raw, 0), o.L_cap);
  const int blk0 = blockIdx.x * kScoreTok;
  if (blk0 >= L) return;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the tile loop is a scalar loop
  const int col = lane & 15, cg = lane >> 4;
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  typedef typename std::conditional<I8, i32x4_t, bf16x8_t>::type QOp;
  QOp qop[KB];
  const int part = col & 3;  // bf16: 0 hi, 1 mid, 2 lo; int8: digit plane 0, 1, 2; 3: zero
  float qscale = 1.f;        // int8: q_bar = qscale * (fixed-point integer)
  // int8: the integer digit sums recombine with weights 1, 256, 65536 in the quad add
  const float dweight = part == 0 ? 1.f : part == 1 ? 256.f : part == 2 ? 65536.f : 0.f;
  const int64_t head_off = seq_off + (int64_t)kh * o.stride_h;
  const uint32_t rs = (uint32_t)(o.stride_t * ES);
  const int nrec = (int)((uint32_t)(L - 1) * rs + D * ES);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)o.k + head_off * ES), (short)0, nrec, 0x00020000);
  // paged: the workgroup's page ids, staged once
  const int bpage0 = PAGED ? blk0 / o.page_tokens : 0;
  if constexpr (PAGED) {
    const int npg = min(kScoreTok / 32 + 1, (min(L, blk0 + kScoreTok) - 1) / o.page_tokens - bpage0 + 1);
    const int *tbl = o.block_table + (int64_t)b * o.table_stride + bpage0;
    for (int i = tid; i < npg; i += 256) s_pages[i] = max(tbl[i], 0);
    __syncthreads();
  }
  const __amdgpu_buffer_rsrc_t ksrs = __builtin_amdgcn_make_buffer_rsrc(
      I8 ? (void *)(o.k_scale + (int64_t)pair * o.k_scale_stride) : nullptr, (short)0,
      I8 ? max(o.k_scale_stride, 1) * 4 : 0, 0x00020000);
  const float *vl = o.vlog + (int64_t)pair * o.vlog_stride;
  float *sc = o.scores + (int64_t)pair * o.L_max;
  // the value term of the lane's four tokens (and an int8 tile's K scales)
  // are fetched with the tile: a load issued later would make the compiler
  // wait for the prefetch too
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vl, (short)0, L * 4, 0x00020000);
  struct KTile {
    u32x4_t k[2][KB];
    u32x4_t vl[2];
    float ks[2];
  };
  // Scores are collected in LDS and written out once, in full coalesced
  // lines, when the block's tiles are done: small scattered stores between
  // the K loads cost far more HBM time than their bytes.
  auto load = [&](KTile &R, int tile, bool valid) {
    const int t0 = blk0 + 32 * tile;
    const uint32_t oob = valid ? 0u : 0x80000000u;
    // a 32-token tile lies in one page: one resource over that page's valid
    // rows (rows past L read as zero), row t0 % page_tokens + i of it
    __amdgpu_buffer_rsrc_t tk = krs;
    int rbase = t0;
    if constexpr (PAGED) {
      const int pidx = t0 / o.page_tokens;
      const int pg = __builtin_amdgcn_readfirstlane(s_pages[min(max(pidx - bpage0, 0), kScoreTok / 32)]);
      const int prows = min(o.page_tokens, L - pidx * o.page_tokens);
      const int nrec_p = prows > 0 ? (int)((uint32_t)(prows - 1) * rs + D * ES) : 0;
      tk = __builtin_amdgcn_make_buffer_rsrc(
          (void *)((const char *)o.k + ((int64_t)pg * o.page_stride + head_off) * ES), (short)0, nrec_p, 0x00020000);
      rbase = t0 - pidx * o.page_tokens;
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const uint32_t off = ((uint32_t)(rbase + 16 * tb + col) * rs + 16 * cg) | oob;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) R.k[tb][kb] = __builtin_amdgcn_raw_buffer_load_b128(tk, off + 64 * kb, 0, 0);
      R.vl[tb] = __builtin_amdgcn_raw_buffer_load_b128(vrs, ((uint32_t)(t0 + 16 * tb + 4 * cg) * 4) | oob, 0, 0);
      if constexpr (I8) {
        // k_part is a multiple of 16, so a 16-token block has one scale
        const uint32_t pi = (uint32_t)((t0 + 16 * tb) / o.k_part);
        R.ks[tb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksrs, (4 * pi) | oob, 0, 0));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Lane (col = 4j + p, cg) ends with, for p == 0, the full q_bar . k of the
  // four tokens 4cg..4cg+3 of each 16-token block; it publishes token 4cg + j.
  const bool token_mode = o.block_tokens <= 1;
  const int jq = col >> 2;
  const bool leader = (col & 3) == 0;
  auto compute = [&](const KTile &R, int tile, bool valid) {
    const int t0 = blk0 + 32 * tile;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      float mult = o.score_scale;
      if constexpr (I8) {
        i32x4_t ai = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          ai = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, R.k[tb][kb]), qop[kb], ai, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = (float)ai[i] * dweight;
        mult = qscale * R.ks[tb] * o.score_scale;
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, R.k[tb][kb]), qop[kb], acc, 0, 0,
                                                        0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = quad_sum3(acc[i]);
      const float dot = jq == 0 ? acc[0] : jq == 1 ? acc[1] : jq == 2 ? acc[2] : acc[3];
      const uint32_t vw = jq == 0 ? R.vl[tb][0] : jq == 1 ? R.vl[tb][1] : jq == 2 ? R.vl[tb][2] : R.vl[tb][3];
      const int t = t0 + 16 * tb + 4 * cg + jq;
      const bool mine = valid && leader && t < L;
      const float sv = dot * mult + o.beta * __uint_as_float(vw);
      if (mine) {
        s_sc[t - blk0] = sv;
        if (token_mode) atomicAdd(&s_hist[order_key(sv) >> 21], 1u);
      }
    }
  };
  // The workgroup's tiles are dealt to its four waves in turn (wave w:
  // tiles w, w + 4, ...), so together they read one contiguous stream (one
  // stream per wave, 64 tiles each, measured 8 us slower on the 128K step).
  // Each wave's tiles pass through a ring of NBUF register buffers: its
  // j-th tile is loaded NBUF-1 tiles before it is scored.  The step count is
  // rounded up to a multiple of the ring; the extra steps load and publish
  // nothing.
  const int ntile = min(kScoreTok / 32, (L - blk0 + 31) / 32);
  const int ntw = max(0, (ntile - wave + 3) / 4);
  const int nst = (ntw + NBUF - 1) / NBUF * NBUF;
  auto tile_at = [&](int j) { return wave + 4 * j; };
  KTile buf[NBUF];
#pragma unroll
  for (int j = 0; j + 1 < NBUF; ++j) load(buf[j], tile_at(j), j < ntw);
  // The query operand is built while the first tiles are in flight (the
  // queries' loads went out first, so waiting for them leaves the tiles').
  // mean query of the group, in fp32, summed in head order
  if (tid < D) {
#pragma unroll
    for (int g = 0; g < 16; ++g) qv[g] = g < o.G ? qv[g] : 0.f;
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) acc += qv[g];  // adding the zeros past G changes nothing
    s_qbar[tid] = acc / (float)o.G;
  }
  __syncthreads();
  if constexpr (I8) {
    // q_bar as a 22-bit fixed-point integer n = rint(q_bar / s), s = max|q_bar| / 2^22,
    // in three balanced int8 digits n = 65536 d2 + 256 d1 + d0 (column part p holds digit p)
    float mx = 0.f;
    for (int d = 0; d < D; ++d) mx = fmaxf(mx, fabsf(s_qbar[d]));
    const float inv = mx > 0.f ? 4194304.0f / mx : 0.f;
    qscale = mx * (1.0f / 4194304.0f);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        uint32_t w = 0u;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int n = (int)__builtin_rintf(s_qbar[64 * kb + 16 * cg + 4 * j4 + y] * inv);
          const int d0 = (int)(int8_t)(n & 0xFF);
          const int r1 = (n - d0) >> 8;
          const int d1 = (int)(int8_t)(r1 & 0xFF);
          const int d2 = (r1 - d1) >> 8;
          const int dg = part == 0 ? d0 : part == 1 ? d1 : part == 2 ? d2 : 0;
          w |= (uint32_t)(dg & 0xFF) << (8 * y);
        }
        qop[kb][j4] = (int)w;
      }
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = s_qbar[8 * (4 * kb + cg) + j];
        const uint32_t hb = f32_to_bf16_bits(x);
        const float r1 = x - __uint_as_float(hb << 16);
        const uint32_t mb = f32_to_bf16_bits(r1);
        const float r2 = r1 - __uint_as_float(mb << 16);
        const uint32_t lb = f32_to_bf16_bits(r2);
        const uint32_t sel = part == 0 ? hb : part == 1 ? mb : part == 2 ? lb : 0u;
        qop[kb][j] = __builtin_bit_cast(__bf16, (uint16_t)sel);
      }
    }
  }
  for (int i = 0; i < nst; i += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      const int ahead = i + j + NBUF - 1;
      load(buf[(j + NBUF - 1) % NBUF], tile_at(ahead), ahead < ntw);
      compute(buf[j], tile_at(i + j), i + j < ntw);
    }
  }
  // the block's scores go out once, in full coalesced lines
  const int nblk_tok = min(kScoreTok, L - blk0);
  __syncthreads();
  if (o.write_scores)
    for (int i = tid; i < nblk_tok; i += 256) sc[blk0 + i] = s_sc[i];
  if (token_mode) {
    uint32_t *gh = o.hist + (size_t)pair * kBins;
    for (int i = tid; i < kBins; i += 256)
      if (s_hist[i]) atomicAdd(gh + i, s_hist[i]);
  } else {
    // block scores: the mean of each block's token scores (block_tokens is a
    // power of two dividing kScoreTok, so blocks never straddle workgroups)
    const int bt = o.block_tokens;
    const int nbb = (nblk_tok + bt - 1) / bt;
    float *bs = o.bscores + (int64_t)pair * o.bs_stride + blk0 / bt;
    for (int jb = wave; jb < nbb; jb += 4) {
      const int t0 = jb * bt, cnt = min(bt, nblk_tok - t0);
      float sum = 0.f;
      for (int i = lane; i < cnt; i += 64) sum += s_sc[t0 + i];
      sum = wave_sum(sum);
      if (lane == 0) bs[jb] = sum / (float)cnt;
    }
  }
}

// Exact selection inside bin b0 by the select pass: the
// need-th largest key T among the items of bin b0, and, among the items equal
// to T, the need'-th smallest index I_T (need' = how many of them are kept).
// Items come from the candidate list or, if it overflowed, from all scores.
// Calls f(key, idx) for the items 0..n-1, thread tid taking i = tid + 256 r:
// the candidate list in LDS, or the pair's whole score row, whose loads are
// issued 16 per thread before any is used.
template <bool FROM_LIST, typename F>
__device__ __forceinline__ void for_items(const uint32_t *ck, const int32_t *ci, const float *sc, int n, F &&f) {
  const int tid = threadIdx.x;
  if constexpr (FROM_LIST) {
    for (int i = tid; i < n; i += 256) f(ck[i], ci[i]);
  } else {
    constexpr int U = 16;
    for (int i0 = 0; i0 < n; i0 += 256 * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = sc[min(i0 + tid + 256 * u, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + tid + 256 * u;
        if (i < n) f(order_key(v[u]), i);
      }
    }
  }
}

template <bool FROM_LIST>
__device__ void select_threshold(const OamDev &o, int pair, int n, int b0, int need, const uint32_t *ck,
                                 const int32_t *ci, uint32_t *s_hist, int *s_tmp, int *s_res, uint32_t *T_out,
                                 int *I_out) {
  const int tid = threadIdx.x;
  const float *sc = o.scores + (int64_t)pair * o.L_max;
  int above;
  // digit 2: key bits 20..10 of the items with top digit b0
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  for_items<FROM_LIST>(ck, ci, sc, n, [&](uint32_t key, int idx) {
    if ((int)(key >> 21) == b0) atomicAdd(&s_hist[(key >> 10) & 0x7FFu], 1u);
  });
  __syncthreads();
  uint32_t prefix = ((uint32_t)b0 << 11) | (uint32_t)select_bin(s_hist, kBins, need, &above, s_tmp, s_res);
  need -= above;
  // digit 3: key bits 9..0
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  for_items<FROM_LIST>(ck, ci, sc, n, [&](uint32_t key, int idx) {
    if ((key >> 10) == prefix) atomicAdd(&s_hist[key & 0x3FFu], 1u);
  });
  __syncthreads();
  const uint32_t T = (prefix << 10) | (uint32_t)select_bin(s_hist, 1024, need, &above, s_tmp, s_res);
  need -= above;
  // When every key equal to T is kept (the usual case: T is a single key),
  // the index passes are not needed.
  const int n_eq = (int)s_hist[T & 0x3FFu];
  if (need == n_eq) {
    *T_out = T;
    *I_out = 0x7FFFFFFF;
    return;
  }
  __syncthreads();  // every thread has read n_eq before the histogram is cleared
  // among keys equal to T, the need-th smallest index: digits of 11 and 10
  // bits of the index, bins reversed so "largest bin" means smallest index
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  for_items<FROM_LIST>(ck, ci, sc, n, [&](uint32_t key, int idx) {
    if (key == T) atomicAdd(&s_hist[2047 - (idx >> 10)], 1u);
  });
  __syncthreads();
  const int ihi = 2047 - select_bin(s_hist, kBins, need, &above, s_tmp, s_res);
  need -= above;
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  for_items<FROM_LIST>(ck, ci, sc, n, [&](uint32_t key, int idx) {
    if (key == T && (idx >> 10) == ihi) atomicAdd(&s_hist[1023 - (idx & 0x3FF)], 1u);
  });
  __syncthreads();
  const int ilo = 1023 - select_bin(s_hist, 1024, need, &above, s_tmp, s_res);
  *T_out = T;
  *I_out = (ihi << 10) | ilo;
}

// Candidate pass: block j of pair p finds b0 from the pair's histogram,
// counts its keys above bin b0 and appends its keys of bin b0 to the pair's
// list.  Block 0 records b0 and how many keys of bin b0 are kept.
__global__ __launch_bounds__(256) void oam_candidate_kernel(OamDev o) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ int s_tmp[4], s_res[2];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int blk0 = blockIdx.x * kBlockTok;
  if (blk0 >= L || o.top_k >= L) return;  // top_k >= L: every token is kept
  const int tid = threadIdx.x;
  // The histogram loads go first, then the block's scores, which do not
  // depend on b0: loads complete in order, so the bin search waits for the
  // histogram only and the score loads' latency overlaps it.
  const float *sc = o.scores + (int64_t)pair * o.L_max;
  const int n = min(kBlockTok, L - blk0);
  uint32_t hv[kBins / 256];
#pragma unroll
  for (int j = 0; j < kBins / 256; ++j) hv[j] = o.hist[(size_t)pair * kBins + tid + 256 * j];
  // unconditional buffer loads (past n they read zero), so the wait for the
  // histogram can leave all eight in flight
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(sc + blk0), (short)0, n * 4, 0x00020000);
  float sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    sv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, (uint32_t)(tid + 256 * j) * 4u, 0, 0));
#pragma unroll
  for (int j = 0; j < kBins / 256; ++j) s_hist[tid + 256 * j] = hv[j];
  __syncthreads();
  int above;
  const int b0 = select_bin(s_hist, kBins, o.top_k, &above, s_tmp, s_res);
  if (blockIdx.x == 0 && tid == 0) {
    o.state[pair].b0 = b0;
    o.state[pair].need = o.top_k - above;
  }
  uint32_t keys[8];
  int gt = 0, nc = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = tid + 256 * j;
    keys[j] = i < n ? order_key(sv[j]) : 0u;
    const int d = (int)(keys[j] >> 21);
    gt += i < n && d > b0;
    nc += i < n && d == b0;
  }
  int tg, tc;
  block_exclusive_scan(gt, s_tmp, &tg);
  int pos = block_exclusive_scan(nc, s_tmp, &tc);
  if (tid == 0) {
    o.blk_gt[(size_t)pair * kMaxBlocks + blockIdx.x] = tg;
    o.blk_nc[(size_t)pair * kMaxBlocks + blockIdx.x] = tc;
  }
  // this block's region of the candidate array: its own token range
  uint32_t *ck = o.cand_key + (int64_t)pair * o.L_max + blk0;
  int32_t *ci = o.cand_idx + (int64_t)pair * o.L_max + blk0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = tid + 256 * j;
    if (i < n && (int)(keys[j] >> 21) == b0) {
      ck[pos] = keys[j];
      ci[pos] = blk0 + i;
      ++pos;
    }
  }
}

// Select pass, one workgroup per pair: T and I_T, then the output offset of
// every block (keys above bin b0 plus kept keys of bin b0 before it).
__global__ __launch_bounds__(256) void oam_select_kernel(OamDev o) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ int s_kept[kMaxBlocks];
  __shared__ int s_pre[kMaxBlocks + 1];
  __shared__ uint32_t s_ck[kCandCap];
  __shared__ int32_t s_ci[kCandCap];
  __shared__ uint16_t s_own[kCandCap];  // block of each gathered candidate
  __shared__ int s_tmp[4], s_res[2];
  const int pair = blockIdx.x;
  const int L = pair_len(o, pair);
  if (L == 0 || o.top_k >= L) return;
  const int tid = threadIdx.x;
  const int b0 = o.state[pair].b0, need = o.state[pair].need;
  const int nblk = (L + kBlockTok - 1) / kBlockTok;
  // where each block's candidates start in the gathered list
  int C = 0;
  for (int j0 = 0; j0 < nblk; j0 += 256) {
    const int j = j0 + tid;
    const int v = j < nblk ? o.blk_nc[(size_t)pair * kMaxBlocks + j] : 0;
    int tot;
    const int ex = block_exclusive_scan(v, s_tmp, &tot);
    if (j < nblk) s_pre[j] = C + ex;
    C += tot;
  }
  if (tid == 0) s_pre[nblk] = C;
  __syncthreads();
  uint32_t T;
  int I_T;
  const bool in_lds = C > 0 && C <= kCandCap;
  if (in_lds) {
    // Gather into LDS: item i lies in the block j with s_pre[j] <= i < s_pre[j+1].
    constexpr int kPer = 16;  // loads of one gather round per thread
    const uint32_t *gk = o.cand_key + (int64_t)pair * o.L_max;
    const int32_t *gi = o.cand_idx + (int64_t)pair * o.L_max;
    // Owner map first (LDS only): wave w writes block j's number over its
    // items, for blocks j = w, w+4, ...  Then each item costs two LDS reads
    // before its loads, and all of a thread's loads are in flight together
    // (clamped to the last item, so they are unconditional).
    const int wave = tid >> 6, lane = tid & 63;
    for (int j = wave; j < nblk; j += 4)
      for (int l = s_pre[j] + lane; l < s_pre[j + 1]; l += 64) s_own[l] = (uint16_t)j;
    __syncthreads();
    for (int i0 = 0; i0 < C; i0 += 256 * kPer) {
      uint32_t kr[kPer];
      int32_t ir[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = min(i0 + tid + 256 * r, C - 1);
        const int j = s_own[i];
        const int64_t src = (int64_t)j * kBlockTok + (i - s_pre[j]);
        kr[r] = gk[src];
        ir[r] = gi[src];
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = i0 + tid + 256 * r;
        if (i < C) {
          s_ck[i] = kr[r];
          s_ci[i] = ir[r];
        }
      }
    }
    __syncthreads();
    select_threshold<true>(o, pair, C, b0, need, s_ck, s_ci, s_hist, s_tmp, s_res, &T, &I_T);
  } else {
    select_threshold<false>(o, pair, L, b0, need, nullptr, nullptr, s_hist, s_tmp, s_res, &T, &I_T);
  }
  if (in_lds) {
    // the gathered list is in block order (block j's candidates are items
    // s_pre[j] .. s_pre[j+1]-1), so wave w counts blocks w, w+4, ... with
    // ballots: per-item atomics on one block's counter would serialise
    const int wave = tid >> 6, lane = tid & 63;
    for (int j = wave; j < nblk; j += 4) {
      int cnt = 0;
      for (int i0 = s_pre[j]; i0 < s_pre[j + 1]; i0 += 64) {
        const int i = i0 + lane;
        bool kept = false;
        if (i < s_pre[j + 1]) {
          const uint32_t key = s_ck[i];
          kept = key > T || (key == T && s_ci[i] <= I_T);
        }
        cnt += __popcll(__ballot(kept));
      }
      if (lane == 0) s_kept[j] = cnt;
    }
  } else {
    for (int j = tid; j < nblk; j += 256) s_kept[j] = 0;
    __syncthreads();
    const float *sc = o.scores + (int64_t)pair * o.L_max;
    for_items<false>(s_ck, s_ci, sc, L, [&](uint32_t key, int idx) {
      if ((int)(key >> 21) == b0 && (key > T || (key == T && idx <= I_T))) atomicAdd(&s_kept[idx / kBlockTok], 1);
    });
  }
  __syncthreads();
  int run = 0;
  for (int j0 = 0; j0 < nblk; j0 += 256) {
    const int j = j0 + tid;
    const int v = j < nblk ? o.blk_gt[(size_t)pair * kMaxBlocks + j] + s_kept[j] : 0;
    int tot;
    const int ex = block_exclusive_scan(v, s_tmp, &tot);
    if (j < nblk) o.blk_off[(size_t)pair * kMaxBlocks + j] = run + ex;
    run += tot;
  }
  if (tid == 0) {
    o.state[pair].T = T;
    o.state[pair].I_T = I_T;
  }
}

// Ordered compaction: the block's keys are staged in LDS with coalesced
// loads, then thread t takes tokens 8t..8t+7 of the block in order.
__global__ __launch_bounds__(256) void oam_write_kernel(OamDev o) {
  __shared__ uint32_t s_key[kBlockTok + kBlockTok / 8];  // one pad word per 8 keys
  __shared__ int s_tmp[4];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int tid = threadIdx.x;
  int32_t *out = o.idx_out + (int64_t)pair * o.top_k;
  const int nk = min(o.top_k, L);
  if (blockIdx.x == 0) {
    if (tid == 0) o.n_kept[pair] = nk;
    for (int i = nk + tid; i < o.top_k; i += 256) out[i] = -1;
  }
  const int blk0 = blockIdx.x * kBlockTok;
  if (blk0 >= L) return;
  const bool keep_all = o.top_k >= L;
  const float *sc = o.scores + (int64_t)pair * o.L_max;
  const int n = min(kBlockTok, L - blk0);
  if (keep_all) {
    for (int i = tid; i < n; i += 256) out[blk0 + i] = blk0 + i;
    return;
  }
  // the threshold and this block's offset are read first, then the scores
  // with unconditional buffer loads (past n they read zero), all in flight
  // together
  const uint32_t T = o.state[pair].T;
  const int I_T = o.state[pair].I_T;
  const int off0 = o.blk_off[(size_t)pair * kMaxBlocks + blockIdx.x];
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(sc + blk0), (short)0, n * 4, 0x00020000);
  float sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    sv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, (uint32_t)(tid + 256 * j) * 4u, 0, 0));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = tid + 256 * j;
    s_key[r + (r >> 3)] = order_key(sv[j]);
  }
  __syncthreads();
  bool keep[8];
  int kc = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * tid + j;
    const uint32_t key = s_key[r + (r >> 3)];
    keep[j] = r < n && (key > T || (key == T && blk0 + r <= I_T));
    kc += keep[j];
  }
  int tot;
  int pos = off0 + block_exclusive_scan(kc, s_tmp, &tot);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (keep[j]) out[pos++] = blk0 + 8 * tid + j;
}

// Block-granular select, one workgroup per pair: the top_k blocks by
// (block score descending, block index ascending), by radix selection on the
// order-preserving keys of the block scores (digits of 11, 11 and 10 bits;
// ties at the threshold go to the lowest block indices), then the kept
// blocks' tokens in ascending order, n_kept, and -1 past it.  Thread t owns
// the contiguous blocks [32t, 32t + 32), its keys held in registers.
__global__ __launch_bounds__(256) void oam_block_select_kernel(OamDev o) {
  constexpr int kPer = kMaxSelBlocks / 256;
  __shared__ uint32_t s_hist[kBins];
  __shared__ int s_kb[kMaxSelBlocks];  // kept blocks in ascending order
  __shared__ int s_tmp[4], s_res[2];
  const int pair = blockIdx.x;
  const int L = pair_len(o, pair);
  const int tid = threadIdx.x;
  const int bt = o.block_tokens;
  const int cap = o.top_k * bt;
  int32_t *out = o.idx_out + (int64_t)pair * cap;
  const int nb = (L + bt - 1) / bt;
  const int n = min(o.top_k, nb);
  const float *bsp = o.bscores + (int64_t)pair * o.bs_stride;
  uint32_t key[kPer];
  const int j0 = tid * kPer;
#pragma unroll
  for (int r = 0; r < kPer; ++r) key[r] = j0 + r < nb ? order_key(bsp[j0 + r]) : 0u;
  uint32_t T = 0u;
  int need = n;  // kept blocks still to place at the current prefix
  if (n > 0 && n < nb) {
    // three digit passes: prefix of the n-th largest key
    uint32_t prefix = 0u;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int d = 0; d < 3; ++d) {
      for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
      __syncthreads();
      const int sh = shifts[d];
      const uint32_t mask = (1u << widths[d]) - 1u;
#pragma unroll
      for (int r = 0; r < kPer; ++r)
        if (j0 + r < nb && (d == 0 || (key[r] >> (sh + widths[d])) == prefix))
          atomicAdd(&s_hist[(key[r] >> sh) & mask], 1u);
      __syncthreads();
      int above;
      const int bin = select_bin(s_hist, 1 << widths[d], need, &above, s_tmp, s_res);
      need -= above;
      prefix = (prefix << widths[d]) | (uint32_t)bin;
    }
    T = prefix;
  }
  // kept: key > T, or key == T among the first `need` such blocks by index
  // (all blocks when n == nb)
  int nt = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) nt += j0 + r < nb && key[r] == T;
  int ttot;
  int trank = block_exclusive_scan(nt, s_tmp, &ttot);
  int kc = 0;
  bool kept[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const bool live = j0 + r < nb;
    const bool tie = live && key[r] == T;
    kept[r] = n >= nb ? live : (live && (key[r] > T || (tie && trank < need)));
    trank += tie;
    kc += kept[r];
  }
  int ktot;
  int pos = block_exclusive_scan(kc, s_tmp, &ktot);
#pragma unroll
  for (int r = 0; r < kPer; ++r)
    if (kept[r]) s_kb[pos++] = j0 + r;
  __syncthreads();
  // tokens of the kept blocks; only the last block of the sequence is partial
  // and it is the last kept one if kept, so kept block q starts at q * bt
  const int last = ktot > 0 ? s_kb[ktot - 1] : 0;
  const int nk = ktot > 0 ? (ktot - 1) * bt + min(bt, L - last * bt) : 0;
  for (int e = tid; e < cap; e += 256) {
    const int q = e / bt, i = e - q * bt;
    int v = -1;
    if (e < nk) v = s_kb[q] * bt + i;
    out[e] = v;
  }
  if (tid == 0) o.n_kept[pair] = nk;
}

}  // namespace

template <bool PAGED>
static void launch_score(const OamDev &o, int kv_dtype, int D, dim3 grid, hipStream_t s) {
  const dim3 blk(256);
  if (kv_dtype == ATTN_I8) {
    if (D == 128) hipLaunchKernelGGL((oam_score_kernel<128, ATTN_I8, PAGED>), grid, blk, 0, s, o);
    else hipLaunchKernelGGL((oam_score_kernel<64, ATTN_I8, PAGED>), grid, blk, 0, s, o);
  } else {
    if (D == 128) hipLaunchKernelGGL((oam_score_kernel<128, ATTN_BF16, PAGED>), grid, blk, 0, s, o);
    else hipLaunchKernelGGL((oam_score_kernel<64, ATTN_BF16, PAGED>), grid, blk, 0, s, o);
  }
}

hipError_t launch_oam(const oam_topk_args &a, const OamPlan &plan, hipStream_t s) {
  const attn_kv_geom &g = a.kv;
  const int npairs = g.B * g.KH;
  if (npairs == 0) return hipSuccess;
  OamDev o;
  o.B = g.B;
  o.KH = g.KH;
  o.G = a.G;
  o.D = g.D;
  o.QH = g.KH * a.G;
  o.top_k = a.top_k;
  o.L_cap = g.max_seq_len;
  o.seq_lens = g.seq_lens;
  o.seq_offset = g.seq_offset;
  o.stride_h = g.stride_h;
  o.stride_t = g.stride_t;
  o.block_table = g.block_table;
  o.page_tokens = g.page_tokens;
  o.table_stride = g.table_stride;
  o.page_stride = g.page_stride;
  o.q = (const uint16_t *)a.q;
  o.k = a.k;
  // a per-tensor K scale is one partition longer than any sequence
  o.k_scale = a.k_scale;
  o.k_part = a.k_part_tokens > 0 ? a.k_part_tokens : (1 << 30);
  o.k_scale_stride = a.k_part_tokens > 0 ? a.k_scale_stride : 0;
  o.vlog = plan.vlog;
  o.vlog_stride = plan.vlog_stride;
  o.L_max = plan.score_stride;
  o.score_scale = a.softmax_scale != 0.f ? a.softmax_scale : 1.0f / sqrtf((float)g.D);
  o.beta = a.beta;
  o.scores = plan.scores;
  o.hist = plan.hist;
  o.blk_nc = plan.blk_nc;
  o.state = reinterpret_cast<OamState *>(plan.state);
  o.blk_gt = plan.blk_gt;
  o.blk_off = plan.blk_off;
  o.cand_key = plan.cand_key;
  o.cand_idx = plan.cand_idx;
  o.idx_out = a.idx_out;
  o.n_kept = a.n_kept;
  o.block_tokens = a.block_tokens;
  o.write_scores = a.block_tokens <= 1 || a.scores_out != nullptr;
  o.bscores = plan.bscores;
  o.bs_stride = plan.bs_stride;

  hipError_t e;
  const bool block_mode = a.block_tokens > 1;
  const int nblk = (g.max_seq_len + kBlockTok - 1) / kBlockTok;
  if (nblk > 0) {
    if (!block_mode) {
      // the histogram starts at zero (a fill kernel, not a memset)
      const size_t nz = (size_t)npairs * kBins;
      hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((nz + 255) / 256 < 128 ? (nz + 255) / 256 : 128)), dim3(256),
                         0, s, plan.hist, nz);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!a.vlog) {
      e = launch_value_lognorm(g, a.v, a.kv_dtype, a.v_scale, a.eps, plan.vlog, plan.vlog_stride, s);
      if (e != hipSuccess) return e;
    }
    dim3 sgrid((g.max_seq_len + kScoreTok - 1) / kScoreTok, npairs), blk(256);
    if (g.block_table) launch_score<true>(o, a.kv_dtype, g.D, sgrid, s);
    else launch_score<false>(o, a.kv_dtype, g.D, sgrid, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!block_mode) {
      hipLaunchKernelGGL(oam_candidate_kernel, dim3(nblk, npairs), blk, 0, s, o);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(oam_select_kernel, dim3(npairs), blk, 0, s, o);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  // the last pass also runs for empty caches: it sets n_kept and the -1 fill
  if (block_mode) hipLaunchKernelGGL(oam_block_select_kernel, dim3(npairs), dim3(256), 0, s, o);
  else hipLaunchKernelGGL(oam_write_kernel, dim3(nblk > 0 ? nblk : 1, npairs), dim3(256), 0, s, o);
  return hipGetLastError();
}

int oam_max_tokens() { return kMaxBlocks * kBlockTok; }
int oam_max_select_blocks() { return kMaxSelBlocks; }

}  // namespace lcdg
