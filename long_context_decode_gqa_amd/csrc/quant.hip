// INT8 KV quantisation ("优化稀疏注意力中的令牌丢弃机制" §6):
// q_val = round(val / scale), scale = max|x| / 127 per token partition
// (Scheme A, K) or per tensor (baseline, V).  The quotient is the IEEE fp32
// correctly rounded division and the rounding is half-to-even (v_rndne_f32),
// so codes match a CPU doing the same fp32 arithmetic bit for bit.
// Also: ln(||v||_2 + eps) per V row, the value term of the OAM score (§3).
#include "common.hpp"

namespace lcdg {
namespace {

// max |x| of 8 bf16 values on their bit patterns: with the sign bits
// cleared, non-negative bf16 values order like unsigned 16-bit integers, so
// two packed 16-bit maxima per word stand for 8 float compares.  The running
// maximum stays packed (two halves) until the end.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t absmax8_bits(u32x4_t w, uint32_t acc) {
  u16x2_t m = __builtin_bit_cast(u16x2_t, acc);
#pragma unroll
  for (int e = 0; e < 4; ++e) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[e] & 0x7FFF7FFFu));
  return __builtin_bit_cast(uint32_t, m);
}

// The larger half of a packed maximum, as the fp32 value of that bf16.
__device__ __forceinline__ float absmax_of_bits(uint32_t acc) {
  const uint32_t lo = acc & 0xFFFFu, hi = acc >> 16;
  return __uint_as_float((lo > hi ? lo : hi) << 16);
}

// The codes of one scale.  Each code needs rint(fl32(x / s)); a correctly
// rounded divide per element made these kernels ALU-bound, so the quotient
// is first taken as q = x * r with r = fl32(1 / s).  For |x| <= 127 s (true
// whenever s = fl32(max|x| / 127) over the same values), |x / s| < 127.0001,
// and q differs from x / s by at most two roundings of 2^-24 relative, i.e.
// by less than 2^-16; fl32(x / s) differs from x / s by at most half an ulp
// below 128, 2^-18.  So fl32(x / s) lies within 2^-15 of q, and whenever q
// is more than 2^-14 away from every half-integer, both round to the same
// integer.  Values nearer a half-integer (about one in 8000) and subnormal
// scales take the IEEE divide, so every code equals rint(fl32(x / s))
// exactly, ties to even included.
struct Quantiser {
  float scale, inv;
  bool fast;
};

__device__ __forceinline__ Quantiser make_quantiser(float scale) {
  Quantiser z;
  z.scale = scale;
  z.inv = scale > 0.f ? 1.0f / scale : 0.f;  // scale 0: every code is 0
  // a subnormal scale takes the divide: its products could meet flushed
  // subnormal operands, and its reciprocal may overflow
  z.fast = scale == 0.f || scale >= 0x1p-126f;
  return z;
}

// Adding M = 1.5 * 2^23 to |c| < 2^22 rounds c to an integer, half to even,
// and leaves that integer in the low mantissa bits: the low byte of the sum's
// bit pattern is the integer's two's-complement byte, and the sum minus M is
// the integer itself, exactly.
constexpr float kRoundMagic = 12582912.0f;

__device__ __forceinline__ u32x2_t codes8(u32x4_t w, const Quantiser &z) {
#pragma clang fp contract(off)
  float x[8], t[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(w[e]);
    x[2 * e + 1] = bf16_hi(w[e]);
  }
  bool near = !z.fast;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = x[i] * z.inv;
    t[i] = q + kRoundMagic;                                   // rint(q) + M
    near |= fabsf(q - (t[i] - kRoundMagic)) > 0.5f - 0x1p-14f;  // |q - rint(q)|, exact
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float c = z.scale > 0.f ? __builtin_rintf(x[i] / z.scale) : 0.f;
      t[i] = fminf(127.f, fmaxf(-127.f, c)) + kRoundMagic;
    }
  }
  // the low bytes of the eight sums, in order
  u32x2_t out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t[4 * h + 1]), __float_as_uint(t[4 * h]), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t[4 * h + 3]), __float_as_uint(t[4 * h + 2]), 0x0c0c0400u);
    out[h] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
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

// Element offset of row t of one (b, kh): contiguous caches add t rows to
// the sequence's offset; a paged cache looks the row's page up in the
// sequence's block-table row (the page holds page_tokens consecutive rows).
struct RowAddr {
  const int32_t *tbl;  // paged: block_table + b * table_stride; else null
  int64_t base;        // contiguous: seq_offset[b] + kh * stride_h; paged: kh * stride_h
  int64_t stride_t, page_stride;
  int page_tokens;
  __device__ __forceinline__ int64_t row(int t) const {
    if (tbl) {
      const int pg = tbl[t / page_tokens];
      return (int64_t)pg * page_stride + base + (int64_t)(t % page_tokens) * stride_t;
    }
    return base + (int64_t)t * stride_t;
  }
};

__device__ __forceinline__ RowAddr row_addr(const attn_kv_geom &g, int pair) {
  const int b = pair / g.KH, kh = pair - b * g.KH;
  RowAddr r;
  r.tbl = g.block_table ? g.block_table + (int64_t)b * g.table_stride : nullptr;
  r.base = (g.block_table ? 0 : g.seq_offset[b]) + (int64_t)kh * g.stride_h;
  r.stride_t = g.stride_t;
  r.page_stride = g.page_stride;
  r.page_tokens = g.page_tokens;
  return r;
}

// A row block of one wave: rows [t0, t1) of one (b, kh) as 16-byte chunks
// (8 bf16 values), row-major; chunk j of a lane is chunk lane + 64 j of the
// block.  CPR > 0 is the number of chunks per row known at compile time (a
// divisor of 64): the lane's chunk j is then row r0 + j * 64 / CPR, read and
// written through buffer resources over the block's rows (32-bit per-lane
// offsets, which the range check covers;
// the host checks that a block spans less than 2^30 elements), so chunks
// past the block's last row read as zeros and their stores are dropped by
// the hardware range check, with no branches.  CPR = 0 takes any D / 8 at
// run time, with 64-bit offsets and guarded accesses.
template <int CPR>
struct LaneChunks {
  int64_t blk;  // CPR > 0: element offset of the block's first row
  __amdgpu_buffer_rsrc_t src, dst;
  uint32_t off0, step;  // CPR > 0: lane's element offset from blk, step per j
  RowAddr ra;           // CPR = 0: rows through their (possibly paged) address
  int t0, cpr, n, rows, lane;
  __device__ __forceinline__ int64_t off(int j) const {
    const int i = lane + 64 * j, r = i / cpr;
    return ra.row(t0 + r) + 8 * (i - r * cpr);
  }
};

template <int CPR>
__device__ __forceinline__ LaneChunks<CPR> lane_chunks(const attn_kv_geom &g, const uint16_t *x, int8_t *codes,
                                                       int pair, int t0, int t1, int lane) {
  LaneChunks<CPR> c;
  c.ra = row_addr(g, pair);
  c.t0 = t0;
  c.cpr = g.D / 8;
  c.rows = t1 - t0;
  c.n = c.rows * c.cpr;
  c.lane = lane;
  if constexpr (CPR > 0) {  // contiguous caches only
    c.blk = c.ra.base + (int64_t)t0 * g.stride_t;
    const int span = (c.rows - 1) * (int)g.stride_t + g.D;  // elements from the first row to the end of the last
    c.src = __builtin_amdgcn_make_buffer_rsrc((void *)(x + c.blk), (short)0, 2 * span, 0x00020000);
    c.dst = __builtin_amdgcn_make_buffer_rsrc((void *)(codes + c.blk), (short)0, span, 0x00020000);
    c.off0 = (uint32_t)(lane / CPR) * (uint32_t)g.stride_t + 8u * (uint32_t)(lane % CPR);
    c.step = (uint32_t)(64 / CPR) * (uint32_t)g.stride_t;
  } else {
    c.blk = 0;
    c.off0 = c.step = 0u;
  }
  return c;
}

template <int CPR>
__device__ __forceinline__ bool lane_valid(const LaneChunks<CPR> &lc, int j) {
  return lc.lane + 64 * j < lc.n;
}

// All CPL chunks of the lane in flight before any is used (zeros past the block).
// The cache is streamed once, so loads (and the code stores) are
// non-temporal: K per partition 315 -> 287 us, V per tensor 501 -> 449 us on
// 1 GiB of bf16 each.
template <int CPL, int CPR>
__device__ __forceinline__ void load_chunks(const LaneChunks<CPR> &lc, const uint16_t *x, u32x4_t (&w)[CPL]) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    if constexpr (CPR > 0) {
      w[j] = __builtin_amdgcn_raw_buffer_load_b128(lc.src, 2u * (lc.off0 + (uint32_t)j * lc.step), 0, kStream);
    } else {
      w[j] = (u32x4_t){0u, 0u, 0u, 0u};
      if (lane_valid(lc, j)) w[j] = *(const u32x4_t *)(x + lc.off(j));
    }
  }
}

template <int CPL, int CPR>
__device__ __forceinline__ void store_codes(const LaneChunks<CPR> &lc, const u32x4_t (&w)[CPL], const Quantiser &z,
                                            int8_t *codes) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    if constexpr (CPR > 0) {
      __builtin_amdgcn_raw_buffer_store_b64(codes8(w[j], z), lc.dst, lc.off0 + (uint32_t)j * lc.step, 0, kStream);
    } else {
      if (lane_valid(lc, j)) *(u32x2_t *)(codes + lc.off(j)) = codes8(w[j], z);
    }
  }
}

// K per token partition.  One wave per (partition, pair), four waves per
// workgroup, no barriers: the partition (at most 64 * CPL chunks) is read
// once into registers, its max |x| reduced across the wave, scale =
// fl32(max / 127), then its codes written.  Many partitions per compute unit
// keep many loads in flight.
template <int CPL, int CPR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void quant_partition_wave_kernel(
    attn_kv_geom g, const uint16_t *x, int32_t part, int32_t nparts, int32_t scale_stride, int8_t *codes,
    float *scales) {
  const int lane = threadIdx.x & 63;
  const int pidx = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = blockIdx.y;
  const int L = min(max(g.seq_lens[pair / g.KH], 0), g.max_seq_len);
  const int t0 = pidx * part;
  if (pidx >= nparts || t0 >= L) return;  // the whole wave leaves together
  const LaneChunks<CPR> lc = lane_chunks<CPR>(g, x, codes, pair, t0, min(L, t0 + part), lane);
  u32x4_t w[CPL];
  load_chunks<CPL, CPR>(lc, x, w);
  uint32_t mb = 0u;
#pragma unroll
  for (int j = 0; j < CPL; ++j) mb = absmax8_bits(w[j], mb);
  const float m = wave_max(absmax_of_bits(mb));
  const float scale = m / 127.0f;
  if (lane == 0) scales[(int64_t)pair * scale_stride + pidx] = scale;
  store_codes<CPL, CPR>(lc, w, make_quantiser(scale), codes);
}

// Partitions of more than 1024 chunks: one workgroup each, read twice.
__global__ __launch_bounds__(256) void quant_partition_kernel(attn_kv_geom g, const uint16_t *x, int32_t part,
                                                              int32_t scale_stride, int8_t *codes, float *scales) {
  __shared__ float s_red[4];
  const int pair = blockIdx.y;
  const int b = pair / g.KH;
  const int L = min(max(g.seq_lens[b], 0), g.max_seq_len);
  const int t0 = blockIdx.x * part;
  if (t0 >= L) return;
  const int cpr = g.D / 8, n = (min(L, t0 + part) - t0) * cpr;
  const RowAddr ra = row_addr(g, pair);
  auto off = [&](int i) -> int64_t {
    const int r = i / cpr;
    return ra.row(t0 + r) + 8 * (i - r * cpr);
  };
  uint32_t mb = 0u;
  for (int i = threadIdx.x; i < n; i += 256) mb = absmax8_bits(*(const u32x4_t *)(x + off(i)), mb);
  const float m = block_max(absmax_of_bits(mb), s_red);
  const float scale = m / 127.0f;
  if (threadIdx.x == 0) scales[(int64_t)pair * scale_stride + blockIdx.x] = scale;
  const Quantiser z = make_quantiser(scale);
  for (int i = threadIdx.x; i < n; i += 256) {
    const int64_t o = off(i);
    *(u32x2_t *)(codes + o) = codes8(*(const u32x4_t *)(x + o), z);
  }
}

// Per-tensor passes work on wave row blocks of 1024 chunks (64 rows at
// D = 128), sixteen 16-byte loads per lane in flight; four waves per
// workgroup, each on its own block.
constexpr int kTensorCPL = 16;
__host__ __device__ __forceinline__ int tensor_block_rows(int D) {
  const int r = 64 * kTensorCPL / (D / 8);
  return r > 0 ? r : 1;
}

// Per-tensor max |x|, first level: one wave per row block, each workgroup
// writes the maximum of its four blocks to its own word of the workspace
// (no atomics; blocks past a sequence's end count as 0).
template <int CPR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void tensor_absmax_kernel(
    attn_kv_geom g, const uint16_t *x, float *wg_max) {
  __shared__ float s_red[4];
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.y;
  const int L = min(max(g.seq_lens[pair / g.KH], 0), g.max_seq_len);
  const int rows = tensor_block_rows(g.D);
  const int t0 = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * rows;
  uint32_t mb = 0u;
  if (t0 < L) {
    const LaneChunks<CPR> lc = lane_chunks<CPR>(g, x, nullptr, pair, t0, min(L, t0 + rows), lane);
    u32x4_t w[kTensorCPL];
    load_chunks<kTensorCPL, CPR>(lc, x, w);
#pragma unroll
    for (int j = 0; j < kTensorCPL; ++j) mb = absmax8_bits(w[j], mb);
  }
  const float m = block_max(absmax_of_bits(mb), s_red);
  if (threadIdx.x == 0) wg_max[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// Second level: one workgroup folds the n workgroup maxima (16 loads per
// thread in flight per round); scale = fl32(max / 127).
__global__ __launch_bounds__(256) void tensor_scale_kernel(const float *wg_max, int64_t n, float *scales) {
  __shared__ float s_red[4];
  constexpr int U = 16;
  float m = 0.f;
  for (int64_t i0 = 0; i0 < n; i0 += 256 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + threadIdx.x + 256 * u;
      v[u] = i < n ? wg_max[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) m = fmaxf(m, v[u]);
  }
  m = block_max(m, s_red);
  if (threadIdx.x == 0) scales[0] = m / 127.0f;
}

// One wave per row block of a (b, kh): the codes under the tensor's scale.
template <int CPR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void tensor_codes_kernel(
    attn_kv_geom g, const uint16_t *x, const float *scales, int8_t *codes) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.y;
  const int L = min(max(g.seq_lens[pair / g.KH], 0), g.max_seq_len);
  const int rows = tensor_block_rows(g.D);
  const int t0 = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * rows;
  if (t0 >= L) return;
  const LaneChunks<CPR> lc = lane_chunks<CPR>(g, x, codes, pair, t0, min(L, t0 + rows), lane);
  u32x4_t w[kTensorCPL];
  load_chunks<kTensorCPL, CPR>(lc, x, w);
  store_codes<kTensorCPL, CPR>(lc, w, make_quantiser(scales[0]), codes);
}

// ln(||v_t||_2 + eps): one 16-byte chunk per lane (8 bf16 or 16 int8 values),
// LPR lanes per row, fp32 sums.  An int8 row's norm is v_scale * ||codes||
// (the integer sum of squares is exact).  A workgroup covers kLognormRPT
// groups of 256 / LPR rows, each thread's loads all in flight at once, non-
// temporal (the rows are read once: 187 -> 174 us over 1 GiB of bf16).
constexpr int kLognormRPT = 8;

template <int LPR, bool I8>
__global__ __launch_bounds__(256) void value_lognorm_kernel(attn_kv_geom g, const void *v, float v_scale, float eps,
                                                            float *out, int32_t stride) {
  constexpr int RPB = 256 / LPR;
  constexpr int EPC = I8 ? 16 : 8;  // elements per lane chunk
  const int pair = blockIdx.y;
  const int b = pair / g.KH;
  const int L = min(max(g.seq_lens[b], 0), g.max_seq_len);
  const int tb = blockIdx.x * RPB * kLognormRPT + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  const RowAddr ra = row_addr(g, pair);
  u32x4_t w[kLognormRPT];
#pragma unroll
  for (int j = 0; j < kLognormRPT; ++j) {
    const int t = tb + RPB * j;
    w[j] = (u32x4_t){0u, 0u, 0u, 0u};
    if (t < L) {
      const int64_t e = ra.row(t) + EPC * c;
      if constexpr (I8) w[j] = __builtin_nontemporal_load((const u32x4_t *)((const int8_t *)v + e));
      else w[j] = __builtin_nontemporal_load((const u32x4_t *)((const uint16_t *)v + e));
    }
  }
#pragma unroll
  for (int j = 0; j < kLognormRPT; ++j) {
    float ss = 0.f;
    if constexpr (I8) {
      int acc = 0;  // exact: at most 16 * 127^2
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_sdot4((int)w[j][e], (int)w[j][e], acc, false);
      ss = (float)acc;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = bf16_lo(w[j][e]), h = bf16_hi(w[j][e]);
        ss += a * a + h * h;
      }
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const int t = tb + RPB * j;
    if (t < L && c == 0) out[(int64_t)pair * stride + t] = logf((I8 ? v_scale * sqrtf(ss) : sqrtf(ss)) + eps);
  }
}

}  // namespace

// Whether a block of `rows` rows spans less than 2^30 elements, so that the
// compile-time-geometry kernels may take 32-bit offsets within it (contiguous
// caches; a paged cache takes the run-time path, row by row).
static bool offsets_fit(const attn_kv_geom &g, int64_t rows) {
  return rows * g.stride_t + g.D < (int64_t(1) << 30);
}

template <int CPL>
static void launch_partition_wave(const attn_kv_geom &g, const uint16_t *x, int32_t part, int32_t nparts,
                                  int32_t scale_stride, int8_t *codes, float *scales, hipStream_t s) {
  dim3 grid((nparts + 3) / 4, g.B * g.KH), blk(256);
  // a lane's chunk offsets reach 64 * CPL chunks into the partition
  switch (!g.block_table && offsets_fit(g, 64 * CPL / (g.D / 8) + 1) ? g.D : 0) {
    case 64:
      hipLaunchKernelGGL((quant_partition_wave_kernel<CPL, 8>), grid, blk, 0, s, g, x, part, nparts, scale_stride,
                         codes, scales);
      break;
    case 128:
      hipLaunchKernelGGL((quant_partition_wave_kernel<CPL, 16>), grid, blk, 0, s, g, x, part, nparts, scale_stride,
                         codes, scales);
      break;
    case 256:
      hipLaunchKernelGGL((quant_partition_wave_kernel<CPL, 32>), grid, blk, 0, s, g, x, part, nparts, scale_stride,
                         codes, scales);
      break;
    default:
      hipLaunchKernelGGL((quant_partition_wave_kernel<CPL, 0>), grid, blk, 0, s, g, x, part, nparts, scale_stride,
                         codes, scales);
  }
}

hipError_t launch_quant_partitions(const attn_kv_geom &g, const void *x, int32_t part, int32_t scale_stride,
                                   int8_t *codes, float *scales, hipStream_t s) {
  const int nparts = (g.max_seq_len + part - 1) / part;
  if (g.B == 0 || nparts == 0) return hipSuccess;
  const int64_t n = (int64_t)part * (g.D / 8);  // chunks per partition
  const uint16_t *xs = (const uint16_t *)x;
  if (n <= 256) launch_partition_wave<4>(g, xs, part, nparts, scale_stride, codes, scales, s);
  else if (n <= 512) launch_partition_wave<8>(g, xs, part, nparts, scale_stride, codes, scales, s);
  else if (n <= 1024) launch_partition_wave<16>(g, xs, part, nparts, scale_stride, codes, scales, s);
  else hipLaunchKernelGGL(quant_partition_kernel, dim3(nparts, g.B * g.KH), dim3(256), 0, s, g, xs, part,
                          scale_stride, codes, scales);
  return hipGetLastError();
}

// Workgroups of the per-tensor passes: four row blocks each, per (b, kh).
static int64_t tensor_groups(const attn_kv_geom &g) {
  const int rows = tensor_block_rows(g.D);
  const int64_t nblk = ((int64_t)g.max_seq_len + rows - 1) / rows;
  return (nblk + 3) / 4;
}

size_t quant_tensor_workspace_bytes(const attn_kv_geom &g) {
  return 256 + 4 * (size_t)(tensor_groups(g) * (int64_t)g.B * g.KH);
}

template <int CPR>
static hipError_t launch_tensor_passes(const attn_kv_geom &g, const uint16_t *x, int8_t *codes, float *scales,
                                       float *wg_max, hipStream_t s) {
  const dim3 grid((unsigned)tensor_groups(g), g.B * g.KH);
  hipLaunchKernelGGL(tensor_absmax_kernel<CPR>, grid, dim3(256), 0, s, g, x, wg_max);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(256), 0, s, wg_max, (int64_t)grid.x * grid.y, scales);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(tensor_codes_kernel<CPR>, grid, dim3(256), 0, s, g, x, scales, codes);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(const attn_kv_geom &g, const void *x, int8_t *codes, float *scales, void *ws,
                               hipStream_t s) {
  if (g.B == 0 || g.max_seq_len == 0) {
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(256), 0, s, (const float *)ws, (int64_t)0, scales);
    return hipGetLastError();
  }
  const uint16_t *xs = (const uint16_t *)x;
  float *wg_max = (float *)((char *)ws + 256);
  switch (!g.block_table && offsets_fit(g, tensor_block_rows(g.D)) ? g.D : 0) {
    case 64: return launch_tensor_passes<8>(g, xs, codes, scales, wg_max, s);
    case 128: return launch_tensor_passes<16>(g, xs, codes, scales, wg_max, s);
    case 256: return launch_tensor_passes<32>(g, xs, codes, scales, wg_max, s);
    default: return launch_tensor_passes<0>(g, xs, codes, scales, wg_max, s);
  }
}

hipError_t launch_value_lognorm(const attn_kv_geom &g, const void *v, int32_t v_dtype, float v_scale, float eps,
                                float *vlog, int32_t stride, hipStream_t s) {
  if (g.B == 0 || g.max_seq_len == 0) return hipSuccess;
  const bool i8 = v_dtype == ATTN_I8;
  const int lpr = g.D / (i8 ? 16 : 8);
  const int rows = 256 / lpr * kLognormRPT;
  dim3 grid((g.max_seq_len + rows - 1) / rows, g.B * g.KH), blk(256);
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
