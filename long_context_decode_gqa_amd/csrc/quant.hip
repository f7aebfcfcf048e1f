// INT8 KV quantisation ("优化稀疏注意力中的令牌丢弃机制" §6):
// q_val = round(val / scale), scale = max|x| / 127 per token partition
// (Scheme A, K) or per tensor (baseline, V).  The quotient is the IEEE fp32
// correctly rounded division and the rounding is half-to-even (v_rndne_f32),
// so codes match a CPU doing the same fp32 arithmetic bit for bit.
// Also: ln(||v||_2 + eps) per V row, the value term of the OAM score (§3).
#include "common.hpp"

namespace lcdg {
namespace {

__device__ __forceinline__ float absmax8(u32x4_t w) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
  return m;
}

__device__ __forceinline__ uint32_t code_of(float x, float scale) {
  if (scale == 0.f) return 0u;
  float q = __builtin_rintf(x / scale);
  q = fminf(127.f, fmaxf(-127.f, q));
  return (uint32_t)(int32_t)q & 0xFFu;
}

__device__ __forceinline__ u32x2_t codes8(u32x4_t w, float scale) {
  u32x2_t out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = w[2 * h], b = w[2 * h + 1];
    out[h] = code_of(bf16_lo(a), scale) | (code_of(bf16_hi(a), scale) << 8) | (code_of(bf16_lo(b), scale) << 16) |
             (code_of(bf16_hi(b), scale) << 24);
  }
  return out;
}

__device__ __forceinline__ float block_max(float v, float *s_red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float r = s_red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, s_red[w]);
  __syncthreads();
  return r;
}

// One workgroup per (partition, pair): max |x| over the partition's tokens and
// all channels, scale = fl32(max / 127), then the codes.
__global__ __launch_bounds__(256) void quant_partition_kernel(attn_kv_geom g, const uint16_t *x, int32_t part,
                                                              int32_t scale_stride, int8_t *codes, float *scales) {
  __shared__ float s_red[4];
  const int pair = blockIdx.y;
  const int b = pair / g.KH, kh = pair - b * g.KH;
  const int L = min(max(g.seq_lens[b], 0), g.max_seq_len);
  const int t0 = blockIdx.x * part;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + part);
  const int cpr = g.D / 8;  // 16-byte chunks per row
  const int n = (t1 - t0) * cpr;
  const int64_t base = g.seq_offset[b] + (int64_t)kh * g.stride_h;
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int t = t0 + i / cpr, c = i - (i / cpr) * cpr;
    m = fmaxf(m, absmax8(*(const u32x4_t *)(x + base + (int64_t)t * g.stride_t + 8 * c)));
  }
  m = block_max(m, s_red);
  const float scale = m / 127.0f;
  if (threadIdx.x == 0) scales[(int64_t)pair * scale_stride + blockIdx.x] = scale;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int t = t0 + i / cpr, c = i - (i / cpr) * cpr;
    const int64_t off = base + (int64_t)t * g.stride_t + 8 * c;
    *(u32x2_t *)(codes + off) = codes8(*(const u32x4_t *)(x + off), scale);
  }
}

__global__ void zero_word_kernel(uint32_t *w) { *w = 0u; }

constexpr int kRowsPerBlock = 64;

// Per-tensor max |x|: a grid-stride pass over every valid row of every
// (b, kh); workgroup maxima are combined with an integer atomic max on the
// fp32 bit pattern (non-negative floats order like their bit patterns).  The
// grid is bounded so the atomic is taken once per workgroup, a few thousand times.
__global__ __launch_bounds__(256) void tensor_absmax_kernel(attn_kv_geom g, const uint16_t *x, uint32_t *ws) {
  __shared__ float s_red[4];
  const int cpr = g.D / 8;
  const int npairs = g.B * g.KH;
  const int nblk_t = (g.max_seq_len + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t units = (int64_t)npairs * nblk_t;
  float m = 0.f;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int pair = (int)(u / nblk_t);
    const int t0 = (int)(u - (int64_t)pair * nblk_t) * kRowsPerBlock;
    const int b = pair / g.KH, kh = pair - b * g.KH;
    const int L = min(max(g.seq_lens[b], 0), g.max_seq_len);
    if (t0 >= L) continue;
    const int t1 = min(L, t0 + kRowsPerBlock);
    const int n = (t1 - t0) * cpr;
    const int64_t base = g.seq_offset[b] + (int64_t)kh * g.stride_h;
    for (int i = threadIdx.x; i < n; i += 256) {
      const int t = t0 + i / cpr, c = i - (i / cpr) * cpr;
      m = fmaxf(m, absmax8(*(const u32x4_t *)(x + base + (int64_t)t * g.stride_t + 8 * c)));
    }
  }
  m = block_max(m, s_red);
  if (threadIdx.x == 0) atomicMax(ws, __float_as_uint(m));
}

__global__ void tensor_scale_kernel(const uint32_t *ws, float *scales) { scales[0] = __uint_as_float(*ws) / 127.0f; }

__global__ __launch_bounds__(256) void tensor_codes_kernel(attn_kv_geom g, const uint16_t *x, const uint32_t *ws,
                                                           int8_t *codes) {
  const float scale = __uint_as_float(*ws) / 127.0f;
  const int pair = blockIdx.y;
  const int b = pair / g.KH, kh = pair - b * g.KH;
  const int L = min(max(g.seq_lens[b], 0), g.max_seq_len);
  const int t0 = blockIdx.x * kRowsPerBlock;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + kRowsPerBlock);
  const int cpr = g.D / 8;
  const int n = (t1 - t0) * cpr;
  const int64_t base = g.seq_offset[b] + (int64_t)kh * g.stride_h;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int t = t0 + i / cpr, c = i - (i / cpr) * cpr;
    const int64_t off = base + (int64_t)t * g.stride_t + 8 * c;
    *(u32x2_t *)(codes + off) = codes8(*(const u32x4_t *)(x + off), scale);
  }
}

// ln(||v_t||_2 + eps): one 16-byte chunk per lane (8 bf16 or 16 int8 values),
// LPR lanes per row, fp32 sums.  An int8 row's norm is v_scale * ||codes||
// (the integer sum of squares is exact).
template <int LPR, bool I8>
__global__ __launch_bounds__(256) void value_lognorm_kernel(attn_kv_geom g, const void *v, float v_scale, float eps,
                                                            float *out, int32_t stride) {
  constexpr int RPB = 256 / LPR;
  constexpr int EPC = I8 ? 16 : 8;  // elements per lane chunk
  const int pair = blockIdx.y;
  const int b = pair / g.KH, kh = pair - b * g.KH;
  const int L = min(max(g.seq_lens[b], 0), g.max_seq_len);
  const int t = blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float ss = 0.f;
  if (t < L) {
    const int64_t e0 = g.seq_offset[b] + (int64_t)kh * g.stride_h + (int64_t)t * g.stride_t + EPC * c;
    if constexpr (I8) {
      const u32x4_t w = *(const u32x4_t *)((const int8_t *)v + e0);
      int acc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int x = (int)(int8_t)(w[e] >> (8 * y));
          acc += x * x;
        }
      ss = (float)acc;
    } else {
      const u32x4_t w = *(const u32x4_t *)((const uint16_t *)v + e0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16_lo(w[e]), h = bf16_hi(w[e]);
        ss += a * a + h * h;
      }
    }
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (t < L && c == 0) out[(int64_t)pair * stride + t] = logf((I8 ? v_scale * sqrtf(ss) : sqrtf(ss)) + eps);
}

}  // namespace

hipError_t launch_quant_partitions(const attn_kv_geom &g, const void *x, int32_t part, int32_t scale_stride,
                                   int8_t *codes, float *scales, hipStream_t s) {
  const int nparts = (g.max_seq_len + part - 1) / part;
  if (g.B == 0 || nparts == 0) return hipSuccess;
  dim3 grid(nparts, g.B * g.KH);
  hipLaunchKernelGGL(quant_partition_kernel, grid, dim3(256), 0, s, g, (const uint16_t *)x, part, scale_stride, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(const attn_kv_geom &g, const void *x, int8_t *codes, float *scales, uint32_t *ws,
                               hipStream_t s) {
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = (g.max_seq_len + kRowsPerBlock - 1) / kRowsPerBlock;
  if (g.B > 0 && nblk > 0) {
    dim3 grid(nblk, g.B * g.KH);
    const int64_t units = (int64_t)nblk * g.B * g.KH;
    hipLaunchKernelGGL(tensor_absmax_kernel, dim3((unsigned)(units < 2048 ? units : 2048)), dim3(256), 0, s, g,
                       (const uint16_t *)x, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(tensor_codes_kernel, grid, dim3(256), 0, s, g, (const uint16_t *)x, ws, codes);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(1), 0, s, ws, scales);
  return hipGetLastError();
}

hipError_t launch_value_lognorm(const attn_kv_geom &g, const void *v, int32_t v_dtype, float v_scale, float eps,
                                float *vlog, int32_t stride, hipStream_t s) {
  if (g.B == 0 || g.max_seq_len == 0) return hipSuccess;
  const bool i8 = v_dtype == ATTN_I8;
  const int lpr = g.D / (i8 ? 16 : 8);
  const int rpb = 256 / lpr;
  dim3 grid((g.max_seq_len + rpb - 1) / rpb, g.B * g.KH), blk(256);
  if (i8) {
    if (lpr == 4) hipLaunchKernelGGL((value_lognorm_kernel<4, true>), grid, blk, 0, s, g, v, v_scale, eps, vlog, stride);
    else if (lpr == 8) hipLaunchKernelGGL((value_lognorm_kernel<8, true>), grid, blk, 0, s, g, v, v_scale, eps, vlog, stride);
    else if (lpr == 16) hipLaunchKernelGGL((value_lognorm_kernel<16, true>), grid, blk, 0, s, g, v, v_scale, eps, vlog, stride);
    else return hipErrorInvalidValue;
  } else {
    if (lpr == 8) hipLaunchKernelGGL((value_lognorm_kernel<8, false>), grid, blk, 0, s, g, v, v_scale, eps, vlog, stride);
    else if (lpr == 16) hipLaunchKernelGGL((value_lognorm_kernel<16, false>), grid, blk, 0, s, g, v, v_scale, eps, vlog, stride);
    else if (lpr == 32) hipLaunchKernelGGL((value_lognorm_kernel<32, false>), grid, blk, 0, s, g, v, v_scale, eps, vlog, stride);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lcdg
