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
//              The histogram's words carry a per-call tag (the rule of the
//              decode's arrival counters), so no pass has to clear them.
//   candidates (2048-token blocks x pairs) every block reads the pair's
//              histogram and finds the threshold's top digit b0 (all blocks
//              find the same); it counts its keys above bin b0 and writes its
//              keys of bin b0, with their indices, to its own region of the
//              pair's candidate array, and their count.
//   select and write (8192-token blocks x pairs) every block gathers the
//              pair's candidates (into LDS when they fit) and finds the exact
//              threshold key T and the last kept index I_T among keys equal to
//              T (all blocks of a pair find the same), then its output offset
//              (keys above bin b0 and kept candidates of the blocks before it)
//              and writes its kept tokens, key > T or (key == T and index <=
//              I_T), in index order, so idx_out is ascending.  Repeating the
//              selection in every block costs less than one more launch.
// Only integer atomics (histogram counts) cross workgroups within a pass.
#include "common.hpp"

namespace lcdg {
namespace {

constexpr int kBins = 2048;       // 11-bit digits (the 10-bit ones use 1024)
constexpr int kBlockTok = 2048;   // tokens per workgroup of the candidate and write passes
constexpr int kSWTok = 8192;      // tokens per workgroup of the select-and-write pass
constexpr int kSWCap = 12288;     // candidate keys a select-and-write workgroup holds in LDS
constexpr int kSWOwn = 8192;      // up to this many, an owner map (2 bytes per key) fits beside them
constexpr int kMaxBlocks = 1024;  // blocks of kBlockTok per pair (sequences up to 2M tokens)
constexpr int kMaxSelBlocks = 8192;  // token blocks per pair the block-granular select holds

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Per-pair selection state, passed from the candidate pass to the next.
struct OamState {
  int32_t b0;        // top 11 bits of the threshold key
  int32_t need;      // keys of bin b0 to keep
  int32_t pad[6];
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
  uint64_t *hist;      // [npairs][kBins]  level-0 histogram, words (hist_tag << 24) | count
  uint64_t hist_tag;   // this call's 40-bit tag; words with another tag count zero
  OamState *state;     // [npairs]
  int32_t *blk_gt;     // [npairs][kMaxBlocks]  keys above bin b0 per block
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

// Adds cnt to a histogram word of this call (tag): the arrival-counter rule
// with a count.  A word with another tag (left by an earlier call on the
// workspace, or other data) is taken over by compare-and-swap with the tagged
// count cnt; when another workgroup took it over first, cnt is added again
// (the first add went into the old word).  Every failed exchange means that
// another workgroup changed the word, so the loop ends.
__device__ __forceinline__ void tagged_add(uint64_t *w, uint32_t cnt, uint64_t tag) {
  const uint64_t old = __hip_atomic_fetch_add(w, (uint64_t)cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((old >> 24) == tag) return;
  uint64_t cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if ((cur >> 24) == tag) {
      __hip_atomic_fetch_add(w, (uint64_t)cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    uint64_t expect = cur;
    if (__hip_atomic_compare_exchange_strong(w, &expect, (tag << 24) | cnt, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return;
    cur = expect;
  }
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
//
// A pair's tokens are cut into ceil(L / kScoreTok) workgroup blocks on
// kScoreUnit-token boundaries, weighted by the XCD the workgroup runs on
// (workgroups are dealt to the eight XCDs in turn): 16 on an even XCD, 15 on
// an odd one, whose streams run about 6% slower under this cache policy
// when every compute unit streams.
constexpr int kScoreTok = 8192;   // average tokens per workgroup of the score pass
constexpr int kScoreUnit = 256;   // block boundaries fall on multiples of this many tokens
constexpr int kScoreMax = 8704;   // most tokens a workgroup takes: at most 34 units under the 16:15 weights
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
  __shared__ float s_sc[kScoreMax];
  // paged: the page ids under the workgroup's tokens (at most kScoreMax / 32
  // + 1 pages, as a page holds a positive multiple of 32 tokens)
  __shared__ int s_pages[PAGED ? kScoreMax / 32 + 1 : 1];
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
  // this block's tokens [blk0, blk_end): units [U S(x) / S(n), U S(x+1) / S(n)),
  // S(x) the weights of blocks 0..x-1 (block i runs on an odd XCD when
  // i + p0 is odd, p0 the parity of the pair's first workgroup)
  const int nact = (L + kScoreTok - 1) / kScoreTok;
  if ((int)blockIdx.x >= nact) return;
  const int p0 = (int)((blockIdx.y * gridDim.x) & 1u);
  auto wsum = [&](int x) { return 16 * x - (p0 ? (x + 1) / 2 : x / 2); };
  const int units = (L + kScoreUnit - 1) / kScoreUnit;
  const int S = wsum(nact);
  const int blk0 = (int)((int64_t)units * wsum(blockIdx.x) / S) * kScoreUnit;
  const int blk_end = min((int)((int64_t)units * wsum(blockIdx.x + 1) / S) * kScoreUnit, L);
  if (blk0 >= blk_end) return;
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
    const int npg = min(kScoreMax / 32 + 1, (blk_end - 1) / o.page_tokens - bpage0 + 1);
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
      const int pg = __builtin_amdgcn_readfirstlane(s_pages[min(max(pidx - bpage0, 0), kScoreMax / 32)]);
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
  const int ntile = (blk_end - blk0 + 31) / 32;  // at most kScoreMax / 32
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
  const int nblk_tok = blk_end - blk0;
  __syncthreads();
  if (o.write_scores)
    for (int i = tid; i < nblk_tok; i += 256) sc[blk0 + i] = s_sc[i];
  if (token_mode) {
    uint64_t *gh = o.hist + (size_t)pair * kBins;
    for (int i = tid; i < kBins; i += 256)
      if (s_hist[i]) tagged_add(gh + i, s_hist[i], o.hist_tag);
  } else {
    // block scores: the mean of each block's token scores (block_tokens is a
    // power of two dividing kScoreUnit, so blocks never straddle workgroups)
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

// The candidate block holding item i of a pair's gathered candidate list:
// the last block j with s_pre[j] <= i (s_pre: the blocks' first items,
// s_pre[nblk] the total; blocks without candidates start where the next one
// does, so the last such j is the one whose items include i).
__device__ __forceinline__ int block_of(const int *s_pre, int nblk, int i) {
  int lo = 0, hi = nblk - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Where the exact selection reads the candidates (keys of bin b0 and their
// indices): the keys gathered in LDS (no indices: the index passes, needed
// only when a group of equal keys is cut at the threshold, read global
// memory), or the pair's candidate regions in global memory (block j's
// items at j * kBlockTok, located through s_pre).
enum { kFromLds = 0, kFromGlobal = 1 };

// Calls f(key, idx) for the items 0..n-1 (idx is -1 from LDS), thread tid
// taking i = tid + 256 r; from global memory 16 items' loads per thread are
// issued before any is used.
template <int SRC, typename F>
__device__ __forceinline__ void for_items(const uint32_t *ck, const int32_t *ci, const int *s_pre, int nblk, int n,
                                          F &&f) {
  const int tid = threadIdx.x;
  if constexpr (SRC == kFromLds) {
    for (int i = tid; i < n; i += 256) f(ck[i], -1);
  } else {
    constexpr int U = 16;
    for (int i0 = 0; i0 < n; i0 += 256 * U) {
      uint32_t kr[U];
      int32_t ir[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = min(i0 + tid + 256 * u, n - 1);
        const int j = block_of(s_pre, nblk, i);
        const int64_t src = (int64_t)j * kBlockTok + (i - s_pre[j]);
        kr[u] = ck[src];
        ir[u] = ci[src];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + tid + 256 * u;
        if (i < n) f(kr[u], ir[u]);
      }
    }
  }
}

// Exact selection inside bin b0 over the pair's n >= need candidates: the
// need-th largest key T, and, among the candidates equal to T, the need'-th
// smallest index I_T (need' = how many of them are kept; I_T = INT_MAX when
// all of them are).  All 256 threads call it and get the result.
// The digit passes read the keys from SRC (ck: LDS keys, or the global
// list); the index passes read the global list (gk, gi).
template <int SRC>
__device__ void select_threshold(int n, int b0, int need, const uint32_t *ck, const uint32_t *gk, const int32_t *gi,
                                 const int *s_pre, int nblk, uint32_t *s_hist, int *s_tmp, int *s_res, uint32_t *T_out,
                                 int *I_out) {
  const int tid = threadIdx.x;
  int above;
  // digit 2: key bits 20..10 (every candidate has top digit b0)
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  for_items<SRC>(ck, gi, s_pre, nblk, n, [&](uint32_t key, int idx) { atomicAdd(&s_hist[(key >> 10) & 0x7FFu], 1u); });
  __syncthreads();
  uint32_t prefix = ((uint32_t)b0 << 11) | (uint32_t)select_bin(s_hist, kBins, need, &above, s_tmp, s_res);
  need -= above;
  // digit 3: key bits 9..0
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  for_items<SRC>(ck, gi, s_pre, nblk, n, [&](uint32_t key, int idx) {
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
  for_items<kFromGlobal>(gk, gi, s_pre, nblk, n, [&](uint32_t key, int idx) {
    if (key == T) atomicAdd(&s_hist[2047 - (idx >> 10)], 1u);
  });
  __syncthreads();
  const int ihi = 2047 - select_bin(s_hist, kBins, need, &above, s_tmp, s_res);
  need -= above;
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  for_items<kFromGlobal>(gk, gi, s_pre, nblk, n, [&](uint32_t key, int idx) {
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
  uint64_t hv[kBins / 256];
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
  // words without this call's tag count zero
#pragma unroll
  for (int j = 0; j < kBins / 256; ++j)
    s_hist[tid + 256 * j] = (hv[j] >> 24) == o.hist_tag ? (uint32_t)(hv[j] & 0xFFFFFFu) : 0u;
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

// Select-and-write pass, (kSWTok-token blocks) x pairs.  Block 0 of a pair
// sets n_kept and fills idx_out past it with -1, and leaves the pair's
// histogram words at zero counts under the next call's tag (the candidate
// pass, their last reader, is complete).  Each block then selects T and I_T
// from the pair's candidates, counts what the blocks before it keep, and
// writes its own kept tokens in order: thread t holds tokens 32t..32t+31 of
// the block.
__global__ __launch_bounds__(256) void oam_select_write_kernel(OamDev o) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ int s_pre[kMaxBlocks + 1];
  // the gathered keys; with at most kSWOwn of them, the candidate block of
  // each (the owner map) is kept in the words past kSWOwn
  __shared__ uint32_t s_ck[kSWCap];
  uint16_t *s_own = reinterpret_cast<uint16_t *>(s_ck + kSWOwn);
  static_assert(2 * kSWOwn <= 4 * (kSWCap - kSWOwn), "owner map beside kSWOwn keys");
  __shared__ int s_tmp[4], s_res[2];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int tid = threadIdx.x;
  int32_t *out = o.idx_out + (int64_t)pair * o.top_k;
  if (blockIdx.x == 0) {
    const int nk = min(o.top_k, L);
    if (tid == 0) o.n_kept[pair] = nk;
    for (int i = nk + tid; i < o.top_k; i += 256) out[i] = -1;
    uint64_t *gh = o.hist + (size_t)pair * kBins;
    const uint64_t next = ((o.hist_tag + 1) & ((1ull << 40) - 1)) << 24;
    for (int i = tid; i < kBins; i += 256) gh[i] = next;
  }
  const int blk0 = blockIdx.x * kSWTok;
  if (blk0 >= L) return;
  const int n = min(kSWTok, L - blk0);
  if (o.top_k >= L) {  // every token is kept
    for (int i = tid; i < n; i += 256) out[blk0 + i] = blk0 + i;
    return;
  }
  // this block's scores first (buffer loads past n read zero), so their
  // latency overlaps the selection
  const float *sc = o.scores + (int64_t)pair * o.L_max;
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(sc + blk0), (short)0, n * 4, 0x00020000);
  u32x4_t sv[kSWTok / 1024];
#pragma unroll
  for (int j = 0; j < kSWTok / 1024; ++j)
    sv[j] = __builtin_amdgcn_raw_buffer_load_b128(srs, (uint32_t)(kSWTok / 256 * tid + 4 * j) * 4u, 0, 0);
  const int b0 = o.state[pair].b0, need = o.state[pair].need;
  const int nblk = (L + kBlockTok - 1) / kBlockTok;
  const int jf = blk0 / kBlockTok;  // this block's first candidate block
  // where each candidate block's items start in the gathered list, and the
  // keys above bin b0 in the candidate blocks before jf
  int C = 0, gt_before = 0;
  for (int j0 = 0; j0 < nblk; j0 += 256) {
    const int j = j0 + tid;
    const int v = j < nblk ? o.blk_nc[(size_t)pair * kMaxBlocks + j] : 0;
    const int g = j < jf ? o.blk_gt[(size_t)pair * kMaxBlocks + j] : 0;
    int tot, gtot;
    const int ex = block_exclusive_scan(v, s_tmp, &tot);
    block_exclusive_scan(g, s_tmp, &gtot);
    if (j < nblk) s_pre[j] = C + ex;
    C += tot;
    gt_before += gtot;
  }
  if (tid == 0) s_pre[nblk] = C;
  __syncthreads();
  const uint32_t *gk = o.cand_key + (int64_t)pair * o.L_max;
  const int32_t *gi = o.cand_idx + (int64_t)pair * o.L_max;
  const int nbefore = s_pre[jf];  // candidates of the blocks before jf
  uint32_t T;
  int I_T, kc_before = 0;
  if (C <= kSWCap) {
    // Gather the keys into LDS.  With an owner map (built first, LDS only:
    // wave w writes block j's number over its items, for blocks j = w, w+4,
    // ...) each item costs two LDS reads before its load, else a binary
    // search over the block starts; all of a thread's loads are in flight
    // together (clamped to the last item, so they are unconditional).
    constexpr int kPer = 16;
    const bool own_map = C <= kSWOwn;
    if (own_map) {
      const int wave = tid >> 6, lane = tid & 63;
      for (int j = wave; j < nblk; j += 4)
        for (int l = s_pre[j] + lane; l < s_pre[j + 1]; l += 64) s_own[l] = (uint16_t)j;
      __syncthreads();
    }
    for (int i0 = 0; i0 < C; i0 += 256 * kPer) {
      uint32_t kr[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = min(i0 + tid + 256 * r, C - 1);
        const int j = own_map ? (int)s_own[i] : block_of(s_pre, nblk, i);
        kr[r] = gk[(int64_t)j * kBlockTok + (i - s_pre[j])];
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const int i = i0 + tid + 256 * r;
        if (i < C) s_ck[i] = kr[r];
      }
    }
    __syncthreads();
    select_threshold<kFromLds>(C, b0, need, s_ck, gk, gi, s_pre, nblk, s_hist, s_tmp, s_res, &T, &I_T);
  } else {
    select_threshold<kFromGlobal>(C, b0, need, gk, gk, gi, s_pre, nblk, s_hist, s_tmp, s_res, &T, &I_T);
  }
  // kept candidates of the blocks before this one: keys >= T when every key
  // equal to T is kept, else the indices of the keys equal to T decide
  if (C <= kSWCap && I_T == 0x7FFFFFFF) {
    for_items<kFromLds>(s_ck, gi, s_pre, nblk, nbefore, [&](uint32_t key, int idx) { kc_before += key >= T; });
  } else {
    for_items<kFromGlobal>(gk, gi, s_pre, nblk, nbefore,
                           [&](uint32_t key, int idx) { kc_before += key > T || (key == T && idx <= I_T); });
  }
  int kept_before;
  block_exclusive_scan(kc_before, s_tmp, &kept_before);
  // ordered compaction of this block's kept tokens; a key above bin b0 is
  // above T
  uint32_t km = 0u;
#pragma unroll
  for (int j = 0; j < kSWTok / 1024; ++j)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int r = kSWTok / 256 * tid + 4 * j + y;
      const uint32_t key = order_key(__uint_as_float(sv[j][y]));
      const bool keep = r < n && (key > T || (key == T && blk0 + r <= I_T));
      km |= (uint32_t)keep << (4 * j + y);
    }
  int tot;
  int pos = gt_before + kept_before + block_exclusive_scan(__popc(km), s_tmp, &tot);
  const int t0 = blk0 + kSWTok / 256 * tid;
  // (the slots past top_k are never reached when the candidate lists agree
  // with the histogram; the bound keeps every store inside the pair's row)
  while (km) {
    if (pos < o.top_k) out[pos] = t0 + __ffs(km) - 1;
    ++pos;
    km &= km - 1u;
  }
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
  o.hist_tag = block_mode ? 0 : counter_tag_for(plan.hist);
  const int nblk = (g.max_seq_len + kBlockTok - 1) / kBlockTok;
  if (nblk > 0) {
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
    }
  }
  // the last pass also runs for empty caches: it sets n_kept and the -1 fill
  if (block_mode) {
    hipLaunchKernelGGL(oam_block_select_kernel, dim3(npairs), dim3(256), 0, s, o);
  } else {
    const int nsw = (g.max_seq_len + kSWTok - 1) / kSWTok;
    hipLaunchKernelGGL(oam_select_write_kernel, dim3(nsw > 0 ? nsw : 1, npairs), dim3(256), 0, s, o);
  }
  return hipGetLastError();
}

int oam_max_tokens() { return kMaxBlocks * kBlockTok; }
int oam_max_select_blocks() { return kMaxSelBlocks; }

}  // namespace lcdg
