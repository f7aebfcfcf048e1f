// Split-KV decode attention on the vector ALUs, for fp32 (or bf16) Q/K/V of
// any head size 4..256 and any group size.  Same work-list and partial format
// as the matrix-core kernel; used where the inputs are fp32 (no fp32 input
// path exists for the 16x16x32 MFMA) or the head size has no MFMA variant.
//
// Per work item, 256-token sub-tiles follow the online softmax of the
// Flash Attention block pseudo-code ("注意力优化（Attention Optimization）"):
// scores of the sub-tile -> new running max -> rescale (alpha) -> probabilities
// -> O = alpha*O + P V, with natural-log scores; the chunk's (m, l, O/l) is the
// partial triple of "优化稀疏注意力中的令牌丢弃机制" §5.
#include "common.hpp"

namespace lcdg {
namespace {

constexpr int kSub = 256;

template <int T>
__device__ __forceinline__ float load_elem(const void *base, int64_t i) {
  if constexpr (T == ATTN_F32) {
    return ((const float *)base)[i];
  } else {
    return bf16_bits_to_f32(((const uint16_t *)base)[i]);
  }
}

template <int QT, int KT>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeParams p) {
  __shared__ float s_q[16][257];
  __shared__ float s_p[16][kSub];
  __shared__ float s_m[16], s_l[16], s_alpha[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = p.D;
  const float NEG_INF = -__builtin_huge_valf();

  const int T = wave_total_tiles(p);
  const int nwg = workers_for(p, T);
  if ((int)blockIdx.x >= nwg) return;
  const int t_begin = (int)((int64_t)blockIdx.x * T / nwg);
  const int t_end = (int)((int64_t)(blockIdx.x + 1) * T / nwg);
  const int ct = p.split / 32;

  // every wave of the workgroup walks the lanes alike
  LaneHit hit = wave_find_lane(p, t_begin);
  for (int t = t_begin; t < t_end;) {
    if (hit.nt == 0) break;  // lane walk exhausted (cannot happen for t < total)
    const int q = hit.q;
    const int lane_t0 = hit.t0, lane_t1 = hit.t0 + hit.nt;
    const int run_end = min(t_end, lane_t1);
    const int pair = q / p.ngb, gb = q - pair * p.ngb;
    const int b = pair / p.KH, kh = pair - b * p.KH;
    const int L = min(max(p.seq_lens[b], 0), p.max_seq_len);
    int npos = L;
    const int *idxp = nullptr;
    if (p.token_idx) {
      npos = L > 0 ? min(max(p.n_idx[pair], 0), p.idx_stride) : 0;
      idxp = p.token_idx + (int64_t)pair * p.idx_stride;
    }
    const int g0 = gb * 16;
    const int gcount = min(16, p.G - g0);
    const int64_t head_off = p.seq_offset[b] + (int64_t)kh * p.stride_h;

    __syncthreads();
    for (int e = tid; e < gcount * D; e += 256) {
      const int g = e / D, d = e - g * D;
      s_q[g][d] = load_elem<QT>(p.q, ((int64_t)b * p.QH + (int64_t)kh * p.G + g0 + g) * D + d);
    }

    // one segment per chunk piece of this run
    for (int seg_t0 = t; seg_t0 < run_end;) {
      const int chunk = (seg_t0 - lane_t0) / ct;
      const int chunk_t1 = min(lane_t1, lane_t0 + (chunk + 1) * ct);
      const int seg_t1 = min(run_end, chunk_t1);
      const int pos0 = (seg_t0 - lane_t0) * 32;
      const int pos1 = min(npos, (seg_t1 - lane_t0) * 32);
      if (tid < 16) {
        s_m[tid] = NEG_INF;
        s_l[tid] = 0.f;
      }
      float o[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) o[k] = 0.f;
      __syncthreads();

      for (int sub0 = pos0; sub0 < pos1; sub0 += kSub) {
        const int n = min(kSub, pos1 - sub0);
        // scores of this sub-tile: thread tt owns token position sub0 + tt
        if (tid < n) {
          int tok = sub0 + tid;
          if (idxp) tok = min(max(idxp[tok], 0), L - 1);
          const int64_t row = head_off + (int64_t)tok * p.stride_t;
          float acc[16];
#pragma unroll
          for (int g = 0; g < 16; ++g) acc[g] = 0.f;
          for (int d = 0; d < D; ++d) {
            const float kv = load_elem<KT>(p.k, row + d);
#pragma unroll
            for (int g = 0; g < 16; ++g)
              if (g < gcount) acc[g] += s_q[g][d] * kv;
          }
#pragma unroll
          for (int g = 0; g < 16; ++g)
            if (g < gcount) s_p[g][tid] = acc[g] * p.softmax_scale;
        }
        __syncthreads();
        // running max, rescale factor and probabilities, one wave per head
        for (int g = wave; g < gcount; g += 4) {
          float mx = NEG_INF;
          for (int i = lane; i < n; i += 64) mx = fmaxf(mx, s_p[g][i]);
          mx = wave_max(mx);
          const float m_old = s_m[g];
          const float m_new = fmaxf(m_old, mx);
          float sum = 0.f;
          for (int i = lane; i < n; i += 64) {
            const float e = expf(s_p[g][i] - m_new);
            s_p[g][i] = e;
            sum += e;
          }
          sum = wave_sum(sum);
          if (lane == 0) {
            const float alpha = (m_old == NEG_INF) ? 0.f : expf(m_old - m_new);
            s_alpha[g] = alpha;
            s_l[g] = alpha * s_l[g] + sum;
            s_m[g] = m_new;
          }
        }
        __syncthreads();
        // O = alpha O + P V for the (g, d) outputs this thread owns
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int e = tid + 256 * k;
          if (e < gcount * D) {
            const int g = e / D, d = e - g * D;
            float acc = o[k] * s_alpha[g];
            for (int i = 0; i < n; ++i) {
              int tok = sub0 + i;
              if (idxp) tok = min(max(idxp[tok], 0), L - 1);
              acc += s_p[g][i] * load_elem<KT>(p.v, head_off + (int64_t)tok * p.stride_t + d);
            }
            o[k] = acc;
          }
        }
        __syncthreads();
      }

      const int half = (seg_t0 == lane_t0 + chunk * ct) ? 0 : 1;
      const bool fill_second = half == 0 && seg_t1 == chunk_t1;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = tid + 256 * k;
        if (e < gcount * D) {
          const int g = e / D, d = e - g * D;
          const int slot = (pair * 2 * p.max_chunks + 2 * chunk + half) * p.G + g0 + g;
          const float l = s_l[g];
          p.wl.o_part[(int64_t)slot * D + d] = (l > 0.f) ? o[k] / l : 0.f;
          if (d == 0) {
            p.wl.m_part[slot] = (l > 0.f) ? s_m[g] : NEG_INF;
            p.wl.l_part[slot] = l;
            if (fill_second) {
              p.wl.m_part[slot + p.G] = NEG_INF;
              p.wl.l_part[slot + p.G] = 0.f;
            }
          }
        }
      }
      __syncthreads();
      seg_t0 = seg_t1;
    }
    t = run_end;
    if (t < t_end) hit = next_lane(p, hit);
  }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams &p, int q_dtype, int kv_dtype, hipStream_t s) {
  dim3 g(p.grid), blk(256);
  if (q_dtype == ATTN_F32 && kv_dtype == ATTN_F32)
    hipLaunchKernelGGL((decode_valu_kernel<ATTN_F32, ATTN_F32>), g, blk, 0, s, p);
  else if (q_dtype == ATTN_BF16 && kv_dtype == ATTN_BF16)
    hipLaunchKernelGGL((decode_valu_kernel<ATTN_BF16, ATTN_BF16>), g, blk, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lcdg
