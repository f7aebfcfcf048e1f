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
  int32_t *counts;     // [npairs][nblk][2]
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

__device__ Thresh resolve(const OamDev &o, int pair, int levels, int *s_tmp, int *s_res) {
  Thresh th;
  const int L = pair_len(o, pair);
  th.keep_all = o.top_k >= L;
  th.prefix = 0;
  th.need = min(o.top_k, L);
  if (th.keep_all) return th;
  const int npairs = o.B * o.KH;
  for (int lev = 0; lev < levels; ++lev) {
    const uint32_t *h = o.hist + ((size_t)lev * npairs + pair) * kBins;
    const int nb = lev == 2 ? 1024 : kBins;
    int above;
    const int bin = select_bin(h, nb, th.need, &above, s_tmp, s_res);
    th.need -= above;
    th.prefix = lev == 0 ? (uint32_t)bin : (lev == 1 ? (th.prefix << 11) | bin : (th.prefix << 10) | bin);
  }
  return th;
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// Score pass.  Wave w of the workgroup takes tiles [16w, 16w+16) of the
// block's 64 tiles of 32 tokens (contiguous rows, two loads in flight); the
// 16x16x32 MFMA gives S[t][g] (lane (c, n) holds tokens 4c..4c+3 of head n)
// and a 16-lane sum reduces over the heads.
template <int D>
__global__ __launch_bounds__(256) void oam_score_kernel(OamDev o) {
  constexpr int KB = D / 32;
  __shared__ uint32_t s_hist[kBins];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int blk0 = blockIdx.x * kBlockTok;
  if (blk0 >= L) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, cg = lane >> 4;
  for (int i = tid; i < kBins; i += 256) s_hist[i] = 0u;
  const int b = pair / o.KH, kh = pair - b * o.KH;
  const bool qvalid = col < o.G;

  bf16x8_t qop[KB];
  {
    const uint16_t *qrow = o.q + ((int64_t)b * o.QH + (int64_t)kh * o.G + (qvalid ? col : 0)) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      u32x4_t w = *(const u32x4_t *)(qrow + 8 * (4 * kb + cg));
      if (!qvalid) w = (u32x4_t){0u, 0u, 0u, 0u};
      qop[kb] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  const int64_t head_off = o.seq_offset[b] + (int64_t)kh * o.stride_h;
  const uint32_t rs = (uint32_t)(o.stride_t * 2);
  const int nrec = (int)((uint32_t)(L - 1) * rs + D * 2);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(o.k + head_off), (short)0, nrec, 0x00020000);
  const float *vl = o.vlog + (int64_t)pair * o.vlog_stride;
  float *sc = o.scores + (int64_t)pair * o.L_max;
  __syncthreads();

  typedef u32x4_t KTile[2][KB];
  auto load = [&](KTile &R, int tile) {
    const int t0 = blk0 + 32 * tile;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const uint32_t off = (uint32_t)(t0 + 16 * tb + col) * rs + 16 * cg;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) R[tb][kb] = __builtin_amdgcn_raw_buffer_load_b128(krs, off + 64 * kb, 0, 0);
    }
  };
  auto compute = [&](const KTile &R, int tile) {
    const int t0 = blk0 + 32 * tile;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, R[tb][kb]), qop[kb], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[i];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        acc[i] = v;
      }
      const int t = t0 + 16 * tb + 4 * cg;
      if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (t + i < L) {
            const float s = acc[i] * o.score_scale + o.beta * vl[t + i];
            sc[t + i] = s;
            atomicAdd(&s_hist[order_key(s) >> 21], 1u);
          }
        }
      }
    }
  };
  KTile ra, rb;
  const int tw0 = 16 * wave;
  load(ra, tw0);
  for (int i = 0; i < 16; i += 2) {
    load(rb, tw0 + i + 1);
    compute(ra, tw0 + i);
    load(ra, i + 2 < 16 ? tw0 + i + 2 : tw0);
    compute(rb, tw0 + i + 1);
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
  __shared__ int s_tmp[4], s_res[2];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int blk0 = blockIdx.x * kBlockTok;
  if (blk0 >= L) return;
  const Thresh th = resolve(o, pair, LEVEL, s_tmp, s_res);
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
  __shared__ int s_tmp[4], s_res[2];
  const int pair = blockIdx.y;
  const int L = pair_len(o, pair);
  const int blk0 = blockIdx.x * kBlockTok;
  if (blk0 >= L) return;
  const Thresh th = resolve(o, pair, 3, s_tmp, s_res);
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
  __shared__ int s_tmp[4], s_res[2];
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
  const Thresh th = resolve(o, pair, 3, s_tmp, s_res);
  // kept and equal-to-threshold tokens in the blocks before this one
  int kept_before = 0, eq_before = 0;
  const int32_t *cnt = o.counts + (int64_t)pair * o.nblk * 2;
  for (int j = 0; j < (int)blockIdx.x; ++j) {
    const int g = cnt[2 * j], e = cnt[2 * j + 1];
    const int take = th.keep_all ? 0 : min(e, max(0, th.need - eq_before));
    kept_before += g + take;
    eq_before += e;
  }
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
  const float ss = a.softmax_scale != 0.f ? a.softmax_scale : 1.0f / sqrtf((float)g.D);
  o.score_scale = ss / (float)a.G;
  o.beta = a.beta;
  o.scores = plan.scores;
  o.hist = plan.hist;
  o.counts = plan.chunk_cnt;
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
  dim3 grid(plan.nchunk, npairs), blk(256);
  if (plan.nchunk > 0) {
    if (g.D == 128) hipLaunchKernelGGL((oam_score_kernel<128>), grid, blk, 0, s, o);
    else hipLaunchKernelGGL((oam_score_kernel<64>), grid, blk, 0, s, o);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((oam_hist_kernel<1>), grid, blk, 0, s, o);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((oam_hist_kernel<2>), grid, blk, 0, s, o);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(oam_count_kernel, grid, blk, 0, s, o);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the write pass also runs for empty caches: it sets n_kept and the -1 fill
  dim3 wgrid(plan.nchunk > 0 ? plan.nchunk : 1, npairs);
  hipLaunchKernelGGL(oam_write_kernel, wgrid, blk, 0, s, o);
  return hipGetLastError();
}

int oam_block_tokens() { return kBlockTok; }

}  // namespace lcdg
