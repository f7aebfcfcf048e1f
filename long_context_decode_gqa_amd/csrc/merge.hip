// Log-sum-exp merge of split-KV partials, and measurement helpers.
#include "common.hpp"

namespace lcdg {
namespace {

constexpr int kMergeThreads = 512;
constexpr int kMergeWeights = 512;

__device__ __forceinline__ float block_reduce(float v, float *s_red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float r = s_red[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) r = is_max ? fmaxf(r, s_red[w]) : r + s_red[w];
  return r;
}

// Exclusive scan of one int per thread over the merge workgroup.
__device__ __forceinline__ int merge_scan(int v, int *s_red, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o);
    if (lane >= o) incl += x;
  }
  __syncthreads();
  if (lane == 63) s_red[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kMergeThreads / 64; ++w) {
    if (w < wave) base += s_red[w];
    tot += s_red[w];
  }
  *total = tot;
  return base + incl - v;
}

// The partials of output row `row`: index s0 + j*ss of slot j < n.  A decode
// call's row (b, kh, g) = pair*G + g owns the slots of its pair's chunks,
// laid out (pair, slot, head) so that one decode worker's partial of all the
// group's heads is one contiguous block; otherwise the caller's CSR offsets.
template <bool DECODE>
__device__ __forceinline__ void row_slots(int row, const int32_t *rss, const DecodeParams &dp, int *s0, int *n,
                                          int *ss) {
  if constexpr (DECODE) {
    const int pair = row / dp.G, g = row - pair * dp.G;
    *s0 = pair * 2 * dp.max_chunks * dp.G + g;
    *n = 2 * pair_chunks(dp, pair);
    *ss = dp.G;
  } else {
    *s0 = rss[row];
    *n = rss[row + 1] - *s0;
    *ss = 1;
  }
}

// Log-sum-exp merge of partial triples, one workgroup per output row:
// M = max m_i, w_i = exp(m_i - M) l_i, out = sum w_i o_i / sum w_i,
// lse = M + ln(sum w_i).  The row's non-empty partials are compacted into an
// LDS list (batches of 512), then spread over thread groups that each sum a
// strided subset with branch-free loads; the groups are added in a fixed
// order, so the result is deterministic.
//
template <int OUT, bool DECODE>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float *o_part, const float *m_part,
                                                              const float *l_part, const int32_t *rss,
                                                              DecodeParams dp, int32_t D, void *out, float *lse) {
  __shared__ float s_red[kMergeThreads / 64];
  __shared__ int s_cnt[kMergeThreads / 64];
  __shared__ float s_w[kMergeWeights];
  __shared__ int s_sl[kMergeWeights];
  __shared__ float s_acc[kMergeThreads * 4];
  const int row = blockIdx.x;
  // decode partials are laid out per (pair, column); the output row of a
  // column follows q's layout ([B][R][KH*Gq])
  int64_t orow = row;
  if constexpr (DECODE) {
    const int pair = row / dp.G;
    orow = q_row_index(dp, pair / dp.KH, pair % dp.KH, row - pair * dp.G);
  }
  const int tid = threadIdx.x;
  const float NEG_INF = -__builtin_huge_valf();
  int s0, n, ss;
  row_slots<DECODE>(row, rss, dp, &s0, &n, &ss);
  float M = NEG_INF;
  for (int i = tid; i < n; i += kMergeThreads)
    if (l_part[s0 + i * ss] > 0.f) M = fmaxf(M, m_part[s0 + i * ss]);
  M = block_reduce(M, s_red, true);

  const bool vec = (D & 3) == 0;
  const int nq = vec ? D / 4 : D;            // columns handled per group
  const int ngrp = kMergeThreads / nq;
  const int grp = tid / nq, q = tid - grp * nq;
  f32x4_t acc4 = {0.f, 0.f, 0.f, 0.f};
  float acc1 = 0.f, Lpart = 0.f;
  for (int base = 0; base < n; base += kMergeWeights) {
    const int i = base + tid;
    float w = 0.f;
    if (i < n) {
      const float l = l_part[s0 + i * ss];
      if (l > 0.f) w = expf(m_part[s0 + i * ss] - M) * l;
    }
    Lpart += w;
    int cnt;
    const int pos = merge_scan(w > 0.f ? 1 : 0, s_cnt, &cnt);
    if (w > 0.f) {
      s_w[pos] = w;
      s_sl[pos] = s0 + i * ss;
    }
    __syncthreads();
    if (grp < ngrp) {
      if (vec) {
#pragma unroll 4
        for (int k = grp; k < cnt; k += ngrp)
          acc4 += s_w[k] * *(const f32x4_t *)(o_part + (int64_t)s_sl[k] * D + 4 * q);
      } else {
        for (int k = grp; k < cnt; k += ngrp) acc1 += s_w[k] * o_part[(int64_t)s_sl[k] * D + q];
      }
    }
    __syncthreads();
  }
  const float Ls = block_reduce(Lpart, s_red, false);
  if (grp < ngrp) {
    if (vec) *(f32x4_t *)(s_acc + grp * D + 4 * q) = acc4;
    else s_acc[grp * D + q] = acc1;
  }
  __syncthreads();
  for (int d = tid; d < D; d += kMergeThreads) {
    float acc = 0.f;
    for (int g = 0; g < ngrp; ++g) acc += s_acc[g * D + d];
    const float o = (Ls > 0.f) ? acc / Ls : 0.f;
    if constexpr (OUT == ATTN_F32) {
      ((float *)out)[orow * D + d] = o;
    } else {
      ((uint16_t *)out)[orow * D + d] = (uint16_t)f32_to_bf16_bits(o);
    }
  }
  if (tid == 0 && lse) lse[orow] = (Ls > 0.f) ? M + logf(Ls) : NEG_INF;
}

// Single-pass merge for D % 4 == 0.  Workgroup (row, c) of csplit takes
// the row's channel slices [c*nq, (c+1)*nq), nq = D/4/csplit, with nq * ng
// threads, ng slot groups per slice (16, or 4 beyond 512 rows), so rows
// with many partials get more, smaller workgroups.  Thread (grp, q) owns
// the 16-byte column slice q and the slots grp, grp + ng, ... of the row
// (consecutive threads read consecutive slices of one slot), and folds them
// in order with a running maximum (online log-sum-exp: on a larger m the
// sums so far are rescaled), issuing U slots' loads before folding them, so
// a pass covers ng U slots in one round trip to memory.  Up to 512 rows, a
// decode call's first pass is addressed from the workspace layout alone and
// goes out together with the read of the sequence length that says how many
// of its slots count, and the 16 groups' states of a slice then meet in 16
// consecutive lanes (one transpose through LDS) and combine by a fixed
// butterfly (xor 8, 4, 2, 1); lane 0 of the 16 writes the slice.  Beyond
// 512 rows, thread q of the first nq combines its slice's groups in order.
// Neither csplit nor U changes which slots a thread folds, in what order, or
// how the groups combine, so the result depends only on the partials and on
// which side of 512 rows the call falls.
constexpr int kMergeV4Threads = 512;  // at most: D = 128 in one workgroup
constexpr int kMergeGroups = 16;      // slot groups per column slice (up to 512 rows)
constexpr int kMergeGroupsMany = 4;   // slot groups per column slice beyond 512 rows

// (m, l, acc) of a fold, rescaled to the larger maximum and added; an empty
// state has l = 0 and is the identity
__device__ __forceinline__ void merge_state(float &m, float &l, f32x4_t &acc, float m2, float l2, f32x4_t acc2) {
  if (l2 > 0.f) {
    if (l > 0.f) {
      const float M = fmaxf(m, m2);
      const float s1 = expf(m - M), s2 = expf(m2 - M);
      acc = s1 * acc + s2 * acc2;
      l = s1 * l + s2 * l2;
      m = M;
    } else {
      m = m2;
      l = l2;
      acc = acc2;
    }
  }
}

template <int OUT, bool DECODE, int U, bool FEW>
__global__ __launch_bounds__(kMergeV4Threads) void merge_v4_kernel(const float *o_part, const float *m_part,
                                                                 const float *l_part, const int32_t *rss,
                                                                 DecodeParams dp, int32_t D, int32_t csplit,
                                                                 void *out, float *lse) {
  const int row = blockIdx.x;
  // decode partials are laid out per (pair, column); the output row of a
  // column follows q's layout ([B][R][KH*Gq])
  int64_t orow = row;
  if constexpr (DECODE) {
    const int pair = row / dp.G;
    orow = q_row_index(dp, pair / dp.KH, pair % dp.KH, row - pair * dp.G);
  }
  const int tid = threadIdx.x;
  const float NEG_INF = -__builtin_huge_valf();
  constexpr int ng = FEW ? kMergeGroups : kMergeGroupsMany;
  const int nq = D / 4 / csplit;  // column slices of this workgroup
  const int grp = tid / nq, ql = tid - grp * nq;
  const int q = blockIdx.y * nq + ql;  // the row's slice
  float mt = NEG_INF, lt = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto fold = [&](float m, float l, f32x4_t o) {
    if (l > 0.f) {  // empty partials (l = 0) may hold any o
      if (m > mt) {
        const float sc = expf(mt - m);
        acc *= sc;
        lt *= sc;
        mt = m;
      }
      const float w = expf(m - mt) * l;
      acc += w * o;
      lt += w;
    }
  };
  int s0, n, ss;
  int first = 0;  // slots already folded
  if constexpr (DECODE && FEW) {
    // slot j of row (pair, g) is entry s0 + j*G, j < 2*max_chunks in the
    // workspace; the pair's own count n arrives with the first pass's loads
    const int pair = row / dp.G, g = row - pair * dp.G;
    s0 = pair * 2 * dp.max_chunks * dp.G + g;
    ss = dp.G;
    const int ncap = 2 * dp.max_chunks;
    constexpr int U1 = U < 16 ? U : 16;  // a first pass of 32 would spill
    if (ncap > 0) {
      float m[U1], l[U1];
      f32x4_t o[U1];
#pragma unroll
      for (int u = 0; u < U1; ++u) {
        const int sl = grp + u * ng;
        const int64_t i = s0 + (int64_t)(sl < ncap ? sl : 0) * ss;
        l[u] = l_part[i];
        m[u] = m_part[i];
        o[u] = *(const f32x4_t *)(o_part + i * D + 4 * q);
      }
      n = 2 * pair_chunks(dp, pair);
#pragma unroll
      for (int u = 0; u < U1; ++u) fold(m[u], grp + u * ng < n ? l[u] : 0.f, o[u]);
      first = ng * U1;
    } else {
      n = 0;
    }
  } else {
    row_slots<DECODE>(row, rss, dp, &s0, &n, &ss);
  }
  for (int base = first + grp; base < n; base += ng * U) {
    float m[U], l[U];
    f32x4_t o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sl = base + u * ng;
      const bool in = sl < n;
      const int64_t i = s0 + (int64_t)(in ? sl : 0) * ss;
      l[u] = in ? l_part[i] : 0.f;
      m[u] = m_part[i];
      o[u] = *(const f32x4_t *)(o_part + i * D + 4 * q);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) fold(m[u], l[u], o[u]);
  }
  __shared__ f32x4_t s_acc[kMergeV4Threads];
  __shared__ float s_m[kMergeV4Threads], s_l[kMergeV4Threads];
  s_acc[tid] = acc;
  s_m[tid] = mt;
  s_l[tid] = lt;
  __syncthreads();
  int qo;
  if constexpr (FEW) {
    // transpose: thread (slice tid / 16, group tid % 16) takes that state,
    // and the 16 lanes of a slice combine by the butterfly
    const int tq = tid / ng, tg = tid - tq * ng;
    const int src = tg * nq + tq;
    acc = s_acc[src];
    mt = s_m[src];
    lt = s_l[src];
#pragma unroll
    for (int off = ng / 2; off >= 1; off >>= 1) {
      const float m2 = __shfl_xor(mt, off, ng), l2 = __shfl_xor(lt, off, ng);
      f32x4_t a2;
#pragma unroll
      for (int i = 0; i < 4; ++i) a2[i] = __shfl_xor(acc[i], off, ng);
      merge_state(mt, lt, acc, m2, l2, a2);
    }
    if (tg != 0) return;
    qo = blockIdx.y * nq + tq;
  } else {
    // thread q of the first nq combines the 16 groups of its slice in order
    if (tid >= nq) return;
    mt = NEG_INF;
    lt = 0.f;
    acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < ng; ++g) merge_state(mt, lt, acc, s_m[g * nq + ql], s_l[g * nq + ql], s_acc[g * nq + ql]);
    qo = q;
  }
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const f32x4_t r = acc * inv;
  if constexpr (OUT == ATTN_F32) {
    *(f32x4_t *)((float *)out + orow * D + 4 * qo) = r;
  } else {
    uint16_t *po = (uint16_t *)out + orow * D + 4 * qo;
    const uint32_t w0 = f32_to_bf16_bits(r[0]) | (f32_to_bf16_bits(r[1]) << 16);
    const uint32_t w1 = f32_to_bf16_bits(r[2]) | (f32_to_bf16_bits(r[3]) << 16);
    *(uint32_t *)po = w0;
    *(uint32_t *)(po + 2) = w1;
  }
  if (qo == 0 && lse) lse[orow] = lt > 0.f ? mt + logf(lt) : NEG_INF;
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4_t *dst, const u32x4_t *src, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}

// One contiguous chunk per workgroup, read through a buffer resource with
// non-temporal loads, sixteen 16-byte loads per thread in flight: the fastest
// plain read measured on MI355X (7.0-7.1 TB/s over 4 GiB; the same sweep
// with the default cache policy 6.1-6.3 TB/s, and one grid-stride load per
// thread 5.2-6.4 TB/s depending on the grid).
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t *src, size_t n, float *sink) {
  constexpr int U = 16;
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t b0 = min(n, (size_t)blockIdx.x * per);
  const size_t b1 = min(n, b0 + per);
  const uint32_t cnt = (uint32_t)(b1 - b0);  // < 2^27 pieces: the launcher bounds the chunk
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(src + b0), (short)0, (int)(cnt * 16u), 0x00020000);
  uint32_t acc = 0;
  for (uint32_t i = threadIdx.x; i < cnt; i += 256 * U) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (i + 256u * u) * 16u, 0, kStream);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
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

// Channel split of the single-pass merge: a divisor of the D/4 slices with at
// most 32 slices (512 threads) per workgroup and at least 4 (one wave), as
// close as that allows to about 512 workgroups in all.
static int merge_csplit(int rows, int D) {
  const int nqt = D / 4;
  const int target = (512 + rows - 1) / rows;
  int best = 0;
  for (int c = 1; c <= nqt; ++c) {
    if (nqt % c || nqt / c > 32) continue;
    if (best == 0) best = c;                // the fewest workgroups that fit
    if (nqt / c < 4 && c > best) break;     // keep a full wave per workgroup
    best = c;
    if (c >= target) break;
  }
  return best;
}

template <int OUT, bool DECODE>
static void launch_merge_v4(const float *o_part, const float *m_part, const float *l_part, const int32_t *rss,
                            const DecodeParams &dp, int rows, int D, bool many_slots, void *out, float *lse,
                            hipStream_t s) {
  const int cs = merge_csplit(rows, D);
  const bool few = rows <= 512;
  const dim3 g(rows, cs), blk((D / 4 / cs) * (few ? kMergeGroups : kMergeGroupsMany));
  // Up to 512 rows the merge is a latency chain (a few hundred workgroups):
  // the speculative first pass and the butterfly shorten it.  With more rows
  // it is bound by the work of its many workgroups, where the lean serial
  // combine is faster and wasted speculative loads on short rows add up
  // (the 128K step's 256 rows: 9.8 vs 11.2 us; the ragged batch's 2048
  // rows: 15.6 vs 20.5 us); there each slice also has 4 slot groups
  // instead of 16, so short rows do not occupy 16 mostly idle groups.
#define LCDG_MERGE_V4(U_, FEW_)                                                                                  \
  hipLaunchKernelGGL((merge_v4_kernel<OUT, DECODE, U_, FEW_>), g, blk, 0, s, o_part, m_part, l_part, rss, dp, D, cs, \
                     out, lse)
  if (many_slots) {
    if (few) LCDG_MERGE_V4(32, true);
    else LCDG_MERGE_V4(32, false);
  } else {
    if (few) LCDG_MERGE_V4(8, true);
    else LCDG_MERGE_V4(8, false);
  }
#undef LCDG_MERGE_V4
}

hipError_t launch_merge(const float *o_part, const float *m_part, const float *l_part, const int32_t *rss,
                        int32_t rows, int32_t D, int32_t out_dtype, void *out, float *lse, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  DecodeParams none = {};
  const uintptr_t oa = reinterpret_cast<uintptr_t>(o_part), ua = reinterpret_cast<uintptr_t>(out);
  const bool v4 = D % 4 == 0 && oa % 16 == 0 && ua % (out_dtype == ATTN_F32 ? 16 : 4) == 0;
  if (v4 && out_dtype == ATTN_F32) {
    launch_merge_v4<ATTN_F32, false>(o_part, m_part, l_part, rss, none, rows, D, false, out, lse, s);
  } else if (v4) {
    launch_merge_v4<ATTN_BF16, false>(o_part, m_part, l_part, rss, none, rows, D, false, out, lse, s);
  } else {
    dim3 g(rows), blk(kMergeThreads);
    if (out_dtype == ATTN_F32)
      hipLaunchKernelGGL((merge_kernel<ATTN_F32, false>), g, blk, 0, s, o_part, m_part, l_part, rss, none, D, out, lse);
    else
      hipLaunchKernelGGL((merge_kernel<ATTN_BF16, false>), g, blk, 0, s, o_part, m_part, l_part, rss, none, D, out,
                         lse);
  }
  return hipGetLastError();
}

// The decode path's head sizes are multiples of 4 and its partials 16-byte
// aligned; the output may be less aligned, then the general kernel runs.
hipError_t launch_merge_decode(const DecodeParams &p, int32_t out_dtype, void *out, float *lse, hipStream_t s) {
  const int rows = p.B * p.QH;
  if (rows <= 0) return hipSuccess;
  const WorkList &w = p.wl;
  const uintptr_t ua = reinterpret_cast<uintptr_t>(out);
  if (p.D % 4 || ua % (out_dtype == ATTN_F32 ? 16 : 4)) {
    dim3 g(rows), blk(kMergeThreads);
    if (out_dtype == ATTN_F32)
      hipLaunchKernelGGL((merge_kernel<ATTN_F32, true>), g, blk, 0, s, w.o_part, w.m_part, w.l_part, nullptr, p, p.D,
                         out, lse);
    else
      hipLaunchKernelGGL((merge_kernel<ATTN_BF16, true>), g, blk, 0, s, w.o_part, w.m_part, w.l_part, nullptr, p, p.D,
                         out, lse);
    return hipGetLastError();
  }
  // two slots per chunk of the longest row; past 128 slots a pass takes 512
  const bool many = 2 * p.max_chunks > kMergeGroups * 8;
  if (out_dtype == ATTN_F32)
    launch_merge_v4<ATTN_F32, true>(w.o_part, w.m_part, w.l_part, nullptr, p, rows, p.D, many, out, lse, s);
  else
    launch_merge_v4<ATTN_BF16, true>(w.o_part, w.m_part, w.l_part, nullptr, p, rows, p.D, many, out, lse, s);
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
  // up to 4096 workgroups (the sink's length) of at least 4096 pieces each;
  // a chunk's byte count must fit the buffer resource's 31 bits
  const size_t want = (n + 4095) / 4096;
  const int grid = (int)(want < 4096 ? want : 4096);
  if ((n + grid - 1) / grid >= ((size_t)1 << 27)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, s, (const u32x4_t *)src, n, sink);
  return hipGetLastError();
}

}  // namespace lcdg
