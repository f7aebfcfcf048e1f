// Work-list construction, log-sum-exp merge and measurement helpers.
#include "common.hpp"

namespace lcdg {
namespace {

// Ragged work-list ("优化稀疏注意力中的令牌丢弃机制" §5: long sequences are split
// across many workgroups so a 128K sequence next to a 512-token one does not
// leave compute units idle).  One workgroup scans the per-(b, kh) chunk
// counts and lays out: the first item of every pair, the partial slot of
// every (output row, chunk), the total item count; it also zeroes the claim
// counter, so a decode launch right after it starts from item 0.
__global__ __launch_bounds__(1024) void worklist_kernel(DecodeParams p) {
  __shared__ int s_sum[1024];
  const int tid = threadIdx.x;
  const int np = p.B * p.KH;
  const int per = (np + 1023) / 1024;
  const int q0 = min(np, tid * per), q1 = min(np, q0 + per);
  int local = 0;
  for (int q = q0; q < q1; ++q) {
    const int b = q / p.KH;
    const int L = min(max(p.seq_lens[b], 0), p.max_seq_len);
    int n = L;
    if (p.token_idx) n = L > 0 ? min(max(p.n_idx[q], 0), p.idx_stride) : 0;
    const int nc = (n + p.split - 1) / p.split;
    p.wl.chunks[q] = nc;
    local += nc;
  }
  s_sum[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? s_sum[tid - off] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  int run = s_sum[tid] - local;
  for (int q = q0; q < q1; ++q) {
    const int nc = p.wl.chunks[q];
    p.wl.item_start[q] = p.ngb * run;
    const int b = q / p.KH, kh = q - b * p.KH;
    for (int g = 0; g < p.G; ++g) p.wl.row_split_start[b * p.QH + kh * p.G + g] = p.G * run + g * nc;
    run += nc;
  }
  if (tid == 1023) {
    const int total = s_sum[1023];
    p.wl.item_start[np] = p.ngb * total;
    p.wl.row_split_start[p.B * p.QH] = p.G * total;
    *p.wl.total_items = p.ngb * total;
    *p.wl.counter = 0;
  }
}

// Log-sum-exp merge of partial triples, one wave per output row:
// M = max m_i, w_i = exp(m_i - M) l_i, out = sum w_i o_i / sum w_i,
// lse = M + ln(sum w_i).  Fixed summation order (deterministic).
template <int OUT>
__global__ __launch_bounds__(256) void merge_kernel(const float *o_part, const float *m_part, const float *l_part,
                                                    const int32_t *rss, int32_t rows, int32_t D, void *out,
                                                    float *lse) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float NEG_INF = -__builtin_huge_valf();
  const int s0 = rss[row], s1 = rss[row + 1];
  float M = NEG_INF;
  for (int i = s0 + lane; i < s1; i += 64)
    if (l_part[i] > 0.f) M = fmaxf(M, m_part[i]);
  M = wave_max(M);
  float Ls = 0.f;
  for (int i = s0 + lane; i < s1; i += 64) {
    const float l = l_part[i];
    if (l > 0.f) Ls += expf(m_part[i] - M) * l;
  }
  Ls = wave_sum(Ls);
  for (int d = lane; d < D; d += 64) {
    float acc = 0.f;
    for (int i = s0; i < s1; ++i) {
      const float l = l_part[i];
      if (l > 0.f) acc += expf(m_part[i] - M) * l * o_part[(int64_t)i * D + d];
    }
    const float o = (Ls > 0.f) ? acc / Ls : 0.f;
    if constexpr (OUT == ATTN_F32) {
      ((float *)out)[(int64_t)row * D + d] = o;
    } else {
      ((uint16_t *)out)[(int64_t)row * D + d] = (uint16_t)f32_to_bf16_bits(o);
    }
  }
  if (lane == 0 && lse) lse[row] = (Ls > 0.f) ? M + logf(Ls) : NEG_INF;
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4_t *dst, const u32x4_t *src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4_t *src, size_t n, float *sink) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const u32x4_t v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t s[256];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int i = 0; i < 256; ++i) x ^= s[i];
    sink[blockIdx.x] = __uint_as_float(x & 0x007FFFFFu);
  }
}

}  // namespace

hipError_t launch_worklist(const DecodeParams &p, hipStream_t s) {
  hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_merge(const float *o_part, const float *m_part, const float *l_part, const int32_t *rss,
                        int32_t rows, int32_t D, int32_t out_dtype, void *out, float *lse, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  dim3 g((rows + 3) / 4), blk(256);
  if (out_dtype == ATTN_F32)
    hipLaunchKernelGGL((merge_kernel<ATTN_F32>), g, blk, 0, s, o_part, m_part, l_part, rss, rows, D, out, lse);
  else
    hipLaunchKernelGGL((merge_kernel<ATTN_BF16>), g, blk, 0, s, o_part, m_part, l_part, rss, rows, D, out, lse);
  return hipGetLastError();
}

hipError_t launch_copy(void *dst, const void *src, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (!n) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const int grid = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, s, (u32x4_t *)dst, (const u32x4_t *)src, n);
  return hipGetLastError();
}

hipError_t launch_read(const void *src, size_t bytes, float *sink, hipStream_t s) {
  const size_t n = bytes / 16;
  if (!n) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const int grid = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, s, (const u32x4_t *)src, n, sink);
  return hipGetLastError();
}

}  // namespace lcdg
