// Output-aware token scoring and exact top-K selection
// ("优化稀疏注意力中的令牌丢弃机制" §3: rank tokens by q.k_i/sqrt(d_k) +
// beta*log(||v_i|| + eps) and drop the lowest; §2 for the q.k ranking it
// replaces).  For each (b, kh) the G query heads' routing logits are averaged,
// so the G heads of a KV head share one kept set.
//
// Passes (grid = token blocks x (b, kh) pairs):
//   score    S = K Q^T on the matrix cores, mean over the G heads, scale,
//            + beta * vlog; write the fp32 score, and count the top 11 bits
//            of its order-preserving key into histogram level 0
//   level 1  keys whose top 11 bits are the threshold's: histogram of bits 20..10
//   level 2  keys matching the 22-bit prefix: histogram of bits 9..0
//            -> the K-th largest key T exactly, and how many keys equal to T
//            are kept (the lowest-index ones)
//   count    per block: keys > T and keys == T
//   write    per block: ordered compaction of the kept indices (ascending)
// Every pass recomputes the threshold digits from the histograms so no pass
// depends on a single-workgroup step.  Integer atomics only.
#include "common.hpp"

namespace lcdg {
namespace {

constexpr int kBlockTok = 2048;   // tokens per workgroup in every pass
constexpr int kBins = 2048;       // 11-bit digits (level 2 uses 1024)

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct OamDev {
  int32_t B, KH, G, D, QH, L_max, L_cap, top_k, nblk;  // L_max: score row stride; L_cap: length bound
  const int32_t *seq_lens;
  const int64_t *seq_offset;
  int64_t stride_h, stride_t;
  const uint16_t *q, *k;
  const float *vlog;
  int32_t vlog_stride;
  float score_scale, beta;
  float *scores;       // [npairs][L_max]
  uint32_t *hist;      // [3][npairs][kBins]
  int32_t *counts;     // [npairs][nblk][2]  per block: keys > T, keys == T
  int32_t *offsets;    // [npairs][nblk][2]  per block: kept before it, equal-to-T before it
  int32_t *state;      // [npairs][4]        prefix, need, keep_all
  int32_t *idx_out;    // [npairs][top_k]
  int32_t *n_kept;     // [npairs]
};

__device__ __forceinline__ int pair_len(const OamDev &o, int pair) {
  return min(max(o.seq_lens[pair / o.KH], 0), o.L_cap);
}

// Exclusive prefix sum of one value per thread over a 256-thread block.
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

// In a histogram of nb bins, the bin holding the need-th largest key
// (need >= 1): returns the bin and sets *above to the number of keys in
// higher bins.  All 256 threads call it; every thread gets the result.
__device__ int select_bin(const uint32_t *hist, int nb, int need, int *above, int *s_tmp, int *s_res) {
  const int tid = threadIdx.x;
  const int per = nb / 256;  // 8 or 4 bins per thread, taken from the top down
  int local = 0;
  for (int j = 0; j < per; ++j) local += (int)hist[nb - 1 - (tid * per + j)];
  int tot;
  const int before = block_exclusive_scan(local, s_tmp, &tot);
  if (tid == 0) s_res[0] = -1;
  __syncthreads();
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

// Threshold state of a pair after `levels` histogram levels: the key prefix
// found so far and how many keys equal to that prefix must still be kept.
struct Thresh {
  uint32_t prefix;  // digits found so far
  int need;         // keys to keep among those matching the prefix
  bool keep_all;
};

__device__ __forceinline__ Thresh load_state(const OamDev &o, int pair) {
  const int32_t *st = o.state + 4 * pair;
  Thresh th;
  th.prefix = (uint32_t)st[0];
  th.need = st[1];
  th.keep_all = st[2] != 0;
  return th;
}

// One workgroup per pair: fold histogram level LEVEL into the pair's
// threshold state (level 0 also initialises it).
template <int LEVEL>
__global__ __launch_bounds__(256) void oam_resolve_kernel(OamDev o) {
  __shared__ int s_tmp[4], s_res[2];
  const int pair = blockIdx.x;
  Thresh th;
  if (LEVEL == 0) {
    const int L = pair_len(o, pair);
    th.keep_all = o.top_k >= L;
    th.prefix = 0;
    th.need = min(o.top_k, L);
  } else {
    th = load_state(o, pair);
  }
  if (!th.keep_all) {
    const int npairs = o.B * o.KH;
    const uint32_t *h = o.hist + ((size_t)LEVEL * npairs + pair) * kBins;
    int above;
    const int bin = select_bin(h, LEVEL == 2 ? 1024 : kBins, th.need, &above, s_tmp, s_res);
    th.need -= above;
    th.prefix = LEVEL == 0 ? (uint32_t)bin : (LEVEL == 1 ? (th.prefix << 11) | bin : (th.prefix << 10) | bin);
  }
  if (threadIdx.x == 0) {
    int32_t *st = o.state + 4 * pair;
    st[0] = (int32_t)th.prefix;
    st[1] = th.need;
    st[2] = th.keep_all ? 1 : 0;
  }
}

// One workgroup per pair: exclusive prefix over its blocks of (kept, equal)
// counts, so each write block knows where its indices start.
__global__ __launch_bounds__(256) void oam_offsets_kernel(OamDev o) {
  __shared__ int s_tmp[4];
  const int pair = blockIdx.x;
  const Thresh th = load_state(o, pair);
  const int32_t *cnt = o.counts + (int64_t)pair * o.nblk * 2;
  int32_t *off = o.offsets + (int64_t)pair * o.nblk * 2;
  int run_k = 0, run_e = 0;
  for (int j0 = 0; j0 < o.nblk; j0 += 256) {
    const int j = j0 + threadIdx.x;
    const int g = j < o.nblk ? cnt[2 * j] : 0, e = j < o.nblk ? cnt[2 * j + 1] : 0;
    int te, tk;
    const int e_before = run_e + block_exclusive_scan(e, s_tmp, &te);
    const int take = th.keep_all ? 0 : min(e, max(0, th.need - e_before));
    const int k_before = run_k + block_exclusive_scan(g + take, s_tmp, &tk);
    if (j < o.nblk) {
      off[2 * j] = k_before;
      off[2 * j + 1] = e_before;
    }
    run_k += tk;
    run_e += te;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// Score pass.  The mean query of the KV head's G heads, q_bar (fp32), is
// split into three bf16 parts hi + mid + lo (24 significant bits) placed in
// B-operand columns 4j, 4j+1, 4j+2 (column 4j+3 is zero), so one 16x16x32
// MFMA chain per 16 tokens gives, in every lane quad, the three partial dot
// products of its four tokens; two quad DPP adds finish q_bar . k_t.  Wave w
// of the workgroup streams tiles [16w', 16w'+16) of 32 tokens, two in flight.
constexpr int kScoreTok = 8192;   // tokens per workgroup of the score pass

__device__ __forceinline__ float quad_sum3(float v) {
  // lane 4j gets v(4j) + v(4j+1) + v(4j+2); quad_perm(1,2,3,0) = 0x39, (2,3,0,1) = 0x4E
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x39, 0xF, 0xF, true));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v + a + b;
}

template <int D>
__global__ __launch_bounds__(256) void oam_score_kernel(OamDev o) {
  constexpr int KB = D / 32;
  constexpr int kTilesPerWave = kScoreTok / 32 / 4;
  __shared__ uint32_t s_hist[kBins];
  __shared__ float s_qbar[D];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int blk0 = blockIdx.x * kScoreTok;
  if (blk0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, cg = lane >> 4;
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  const int b = pair / o.KH, kh = pair - b * o.KH;
  // mean query of the group, in fp32
  for (int d = tid; d < D; d += 256) {
    const uint16_t *q0 = o.q + ((int64_t)b * o.QH + (int64_t)kh * o.G) * D + d;
    float acc = 0.f;
    for (int g = 0; g < o.G; ++g) acc += bf16_bits_to_f32(q0[(int64_t)g * D]);
    s_qbar[d] = acc / (float)o.G;
  }
  __syncthreads();
  bf16x8_t qop[KB];
  {
    const int part = col & 3;  // 0: hi, 1: mid, 2: lo, 3: zero
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
  const int64_t head_off = o.seq_offset[b] + (int64_t)kh * o.stride_h;
  const uint32_t rs = (uint32_t)(o.stride_t * 2);
  const int nrec = (int)((uint32_t)(L - 1) * rs + D * 2);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(o.k + head_off), (short)0, nrec, 0x00020000);
  const float *vl = o.vlog + (int64_t)pair * o.vlog_stride;
  float *sc = o.scores + (int64_t)pair * o.L_max;
  // the value term of the lane's four tokens is fetched with the tile (a
  // load issued later would make the compiler wait for the prefetch too)
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vl, (short)0, L * 4, 0x00020000);
  struct KTile {
    u32x4_t k[2][KB];
    u32x4_t vl[2];
  };
  auto load = [&](KTile &R, int tile, bool valid) {
    const int t0 = blk0 + 32 * tile;
    const uint32_t oob = valid ? 0u : 0x80000000u;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const uint32_t off = ((uint32_t)(t0 + 16 * tb + col) * rs + 16 * cg) | oob;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) R.k[tb][kb] = __builtin_amdgcn_raw_buffer_load_b128(krs, off + 64 * kb, 0, 0);
      R.vl[tb] = __builtin_amdgcn_raw_buffer_load_b128(vrs, ((uint32_t)(t0 + 16 * tb + 4 * cg) * 4) | oob, 0, 0);
    }
  };
  auto compute = [&](const KTile &R, int tile) {
    const int t0 = blk0 + 32 * tile;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, R.k[tb][kb]), qop[kb], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = quad_sum3(acc[i]);
      const int t = t0 + 16 * tb + 4 * cg;
      if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (t + i < L) {
            const float s = acc[i] * o.score_scale + o.beta * __uint_as_float(R.vl[tb][i]);
            sc[t + i] = s;
            atomicAdd(&s_hist[order_key(s) >> 21], 1u);
          }
        }
      }
    }
  };
  // this wave's tiles, stopping at the end of the sequence
  const int tw0 = kTilesPerWave * wave;
  const int ntw = max(0, min(kTilesPerWave, (L - blk0 - 32 * tw0 + 31) / 32));
  KTile ra, rb;
  load(ra, tw0, ntw > 0);
  for (int i = 0; i < ntw; i += 2) {
    load(rb, tw0 + i + 1, i + 1 < ntw);
    compute(ra, tw0 + i);
    load(ra, tw0 + i + 2, i + 2 < ntw);
    if (i + 1 < ntw) compute(rb, tw0 + i + 1);
  }
  __syncthreads();
  uint32_t *gh = o.hist + (size_t)pair * kBins;
  for (int i = tid; i < kBins; i += 256)
    if (s_hist[i]) atomicAdd(gh + i, s_hist[i]);
}

// Histogram levels 1 and 2 over the keys matching the prefix found so far.
template <int LEVEL>
__global__ __launch_bounds__(256) void oam_hist_kernel(OamDev o) {
  __shared__ uint32_t s_hist[kBins];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int blk0 = blockIdx.x * kBlockTok;
  if (blk0 >= L) return;
  const Thresh th = load_state(o, pair);
  if (th.keep_all) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  __syncthreads();
  const float *sc = o.scores + (int64_t)pair * o.L_max;
  const int n = min(kBlockTok, L - blk0);
  for (int i = tid; i < n; i += 256) {
    const uint32_t key = order_key(sc[blk0 + i]);
    if (LEVEL == 1) {
      if ((key >> 21) == th.prefix) atomicAdd(&s_hist[(key >> 10) & 0x7FFu], 1u);
    } else {
      if ((key >> 10) == th.prefix) atomicAdd(&s_hist[key & 0x3FFu], 1u);
    }
  }
  __syncthreads();
  const int npairs = o.B * o.KH;
  uint32_t *gh = o.hist + ((size_t)LEVEL * npairs + pair) * kBins;
  for (int i = tid; i < (LEVEL == 2 ? 1024 : kBins); i += 256)
    if (s_hist[i]) atomicAdd(gh + i, s_hist[i]);
}

// Keys above the threshold and keys equal to it, per block.
__global__ __launch_bounds__(256) void oam_count_kernel(OamDev o) {
  __shared__ int s_tmp[4];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int blk0 = blockIdx.x * kBlockTok;
  if (blk0 >= L) {
    if (threadIdx.x == 0) {
      int32_t *c = o.counts + ((int64_t)pair * o.nblk + blockIdx.x) * 2;
      c[0] = 0;
      c[1] = 0;
    }
    return;
  }
  const Thresh th = load_state(o, pair);
  const int tid = threadIdx.x;
  const float *sc = o.scores + (int64_t)pair * o.L_max;
  const int n = min(kBlockTok, L - blk0);
  int gt = 0, eq = 0;
  if (!th.keep_all) {
    for (int i = tid; i < n; i += 256) {
      const uint32_t key = order_key(sc[blk0 + i]);
      gt += key > th.prefix;
      eq += key == th.prefix;
    }
  }
  int tg, te;
  block_exclusive_scan(gt, s_tmp, &tg);
  block_exclusive_scan(eq, s_tmp, &te);
  if (tid == 0) {
    int32_t *c = o.counts + ((int64_t)pair * o.nblk + blockIdx.x) * 2;
    c[0] = th.keep_all ? n : tg;
    c[1] = th.keep_all ? 0 : te;
  }
}

// Ordered compaction: thread i of a block owns tokens 8i..8i+7 of it.
__global__ __launch_bounds__(256) void oam_write_kernel(OamDev o) {
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
  const Thresh th = load_state(o, pair);
  // kept and equal-to-threshold tokens in the blocks before this one
  const int32_t *off = o.offsets + ((int64_t)pair * o.nblk + blockIdx.x) * 2;
  const int kept_before = off[0], eq_before = off[1];
  const float *sc = o.scores + (int64_t)pair * o.L_max;
  const int n = min(kBlockTok, L - blk0);
  uint32_t keys[8];
  int eqc = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = 8 * tid + j;
    keys[j] = i < n ? order_key(sc[blk0 + i]) : 0u;
    eqc += (i < n) && !th.keep_all && keys[j] == th.prefix;
  }
  int tot;
  const int eq_rank0 = eq_before + block_exclusive_scan(eqc, s_tmp, &tot);
  bool keep[8];
  int kc = 0, er = eq_rank0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = 8 * tid + j;
    bool k = false;
    if (i < n) {
      if (th.keep_all) {
        k = true;
      } else if (keys[j] > th.prefix) {
        k = true;
      } else if (keys[j] == th.prefix) {
        k = er < th.need;
        ++er;
      }
    }
    keep[j] = k;
    kc += k;
  }
  int pos = kept_before + block_exclusive_scan(kc, s_tmp, &tot);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (keep[j]) out[pos++] = blk0 + 8 * tid + j;
}

}  // namespace

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
  o.nblk = plan.nchunk;
  o.seq_lens = g.seq_lens;
  o.seq_offset = g.seq_offset;
  o.stride_h = g.stride_h;
  o.stride_t = g.stride_t;
  o.q = (const uint16_t *)a.q;
  o.k = (const uint16_t *)a.k;
  o.vlog = plan.vlog;
  o.vlog_stride = plan.vlog_stride;
  o.L_max = plan.score_stride;
  o.score_scale = a.softmax_scale != 0.f ? a.softmax_scale : 1.0f / sqrtf((float)g.D);
  o.beta = a.beta;
  o.scores = plan.scores;
  o.hist = plan.hist;
  o.counts = plan.chunk_cnt;
  o.offsets = plan.offsets;
  o.state = plan.state;
  o.idx_out = a.idx_out;
  o.n_kept = a.n_kept;

  const size_t nhist = (size_t)3 * npairs * kBins;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((nhist + 255) / 256 < 4096 ? (nhist + 255) / 256 : 4096)), dim3(256),
                     0, s, plan.hist, nhist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.vlog) {
    e = launch_value_lognorm(g, a.v, a.eps, plan.vlog, plan.vlog_stride, s);
    if (e != hipSuccess) return e;
  }
  dim3 grid(plan.nchunk, npairs), blk(256), pgrid(npairs);
#define LCDG_CHECK_LAUNCH() if ((e = hipGetLastError()) != hipSuccess) return e
  if (plan.nchunk > 0) {
    dim3 sgrid((g.max_seq_len + kScoreTok - 1) / kScoreTok, npairs);
    if (g.D == 128) hipLaunchKernelGGL((oam_score_kernel<128>), sgrid, blk, 0, s, o);
    else hipLaunchKernelGGL((oam_score_kernel<64>), sgrid, blk, 0, s, o);
    LCDG_CHECK_LAUNCH();
    hipLaunchKernelGGL((oam_resolve_kernel<0>), pgrid, blk, 0, s, o);
    LCDG_CHECK_LAUNCH();
    hipLaunchKernelGGL((oam_hist_kernel<1>), grid, blk, 0, s, o);
    LCDG_CHECK_LAUNCH();
    hipLaunchKernelGGL((oam_resolve_kernel<1>), pgrid, blk, 0, s, o);
    LCDG_CHECK_LAUNCH();
    hipLaunchKernelGGL((oam_hist_kernel<2>), grid, blk, 0, s, o);
    LCDG_CHECK_LAUNCH();
    hipLaunchKernelGGL((oam_resolve_kernel<2>), pgrid, blk, 0, s, o);
    LCDG_CHECK_LAUNCH();
    hipLaunchKernelGGL(oam_count_kernel, grid, blk, 0, s, o);
    LCDG_CHECK_LAUNCH();
    hipLaunchKernelGGL(oam_offsets_kernel, pgrid, blk, 0, s, o);
    LCDG_CHECK_LAUNCH();
  }
#undef LCDG_CHECK_LAUNCH
  // the write pass also runs for empty caches: it sets n_kept and the -1 fill
  dim3 wgrid(plan.nchunk > 0 ? plan.nchunk : 1, npairs);
  hipLaunchKernelGGL(oam_write_kernel, wgrid, blk, 0, s, o);
  return hipGetLastError();
}

int oam_block_tokens() { return kBlockTok; }

}  // namespace lcdg
