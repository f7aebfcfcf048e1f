// Split-KV GQA decode attention on gfx950 matrix cores (bf16 or int8 KV).
//
// One workgroup (4 waves) takes one work item = (sequence b, KV head kh,
// query-head block, chunk of split_tokens token positions) from the
// work-list, claimed with an integer atomic.  Each wave streams 32-token
// tiles of the chunk (tile w, w+4, ...), prefetching its next tile into
// registers while it computes the current one:
//
//   S^T[t][g]  = K[t][:] . Q[g][:]            v_mfma_f32_16x16x32_{bf16,f16}
//   online softmax per query head g (running max m, sum l; exp2 domain)
//   O^T[d][g] += V^T[d][t] . P^T[t][g]        same MFMA, P fed as hi + lo
//
// This is the FlashAttention block recurrence with one query row per head
// ("注意力优化（Attention Optimization）", Flash Attention pseudo-code; NVIDIA
// blog "共同设计 AI 模型注意力…", BMM1 -> online softmax -> BMM2), and the
// G query heads of a KV head share every K/V byte that is loaded (GQA head
// sharing on the same pages).  The chunk's partial (m, l, o) is written for
// the log-sum-exp merge ("优化稀疏注意力中的令牌丢弃机制" §5).
//
// Operand layouts (16x16x32 MFMA, lane = 16*c + r, c = lane/16, r = lane%16):
//  * A operand row r, k-slots 8c..8c+7 (8 consecutive elements of one lane).
//  * QK: A = K tile, row = token, k-slot 8c+j of block kb <-> channel
//    d = 8*(4*kb + c) + j (bf16) so each lane loads 16 contiguous bytes and a
//    token row's 4 lanes read 64 contiguous bytes per load.  B = Q^T in the
//    same channel order, column n = query head g (< G, others zero).
//  * C layout: lane (c, n) holds rows 4c..4c+3 of column n, i.e. the scores
//    of tokens 4c..4c+3 (block 0) and 16+4c..16+4c+3 (block 1) for head n.
//  * PV: contraction slot 8c+j <-> token j<4 ? 4c+j : 16+4c+j-4, which is
//    exactly the lane's own scores, so P^T needs no data movement.  Output
//    row m of block nb <-> channel d = NB*m + nb (NB = D/16): lane r then
//    needs channels NB*r .. NB*r+NB-1 of its 8 tokens, which is one natural,
//    fully coalesced load per token (16 lanes cover a 256-byte row), and the
//    V^T operand of block nb is element nb of those 8 loads (a register
//    permute, no LDS round trip).
//  * P is split as p = hi + lo with hi = bf16(p) and lo = bf16(p - hi); both
//    are multiplied into the same accumulator, so P carries ~16 bits.
#include "common.hpp"

namespace lcdg {
namespace {

constexpr int kTile = 32;
constexpr int kWaves = 4;

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int NW> struct VecW;
template <> struct VecW<1> { typedef uint32_t T; };
template <> struct VecW<2> { typedef u32x2_t T; };
template <> struct VecW<4> { typedef u32x4_t T; };

template <int NW>
__device__ __forceinline__ uint32_t word_of(const typename VecW<NW>::T &v, int i) {
  if constexpr (NW == 1) {
    return v;
  } else {
    return v[i];
  }
}

// Four int8 codes (bytes) -> their exact fp16 values: (0x6400 | (c ^ 0x80)) is
// 1152 + c in fp16, and subtracting 1152 is exact.
__device__ __forceinline__ uint32_t codes_to_f16x2(uint32_t pair_lo16_hi16) {
  f16x2_t h = __builtin_bit_cast(f16x2_t, pair_lo16_hi16 ^ 0x64806480u);
  const f16x2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
  h = h - off;
  return __builtin_bit_cast(uint32_t, h);
}

template <int D, int KVT>
struct Tile {
  static constexpr int ES = (KVT == ATTN_BF16) ? 2 : 1;
  static constexpr int KL = (KVT == ATTN_BF16) ? D / 32 : D / 64;  // 16-byte K loads per token block
  static constexpr int VW = (D / 16) * ES / 4;                      // V words per token per lane
  u32x4_t k[2][KL];
  typename VecW<VW>::T v[8];
};

template <int D, int KVT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_mfma_kernel(DecodeParams p) {
  typedef Tile<D, KVT> TileT;
  constexpr int NB = D / 16;
  constexpr int KB = D / 32;
  constexpr int ES = TileT::ES;
  constexpr int KL = TileT::KL;
  constexpr int VW = TileT::VW;
  typedef typename VecW<VW>::T VV;
  typedef typename std::conditional<KVT == ATTN_BF16, bf16x8_t, f16x8_t>::type OpT;

  __shared__ int s_info[2];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_o[kWaves][16][D + 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, cg = lane >> 4;
  const int npairs = p.B * p.KH;
  const float c1 = p.softmax_scale * kLog2e;
  const float NEG_INF = -__builtin_huge_valf();

  for (;;) {
    if (tid == 0) {
      const int item = atomicAdd(p.wl.counter, 1);
      int pair = -1, rel = 0;
      if (item < *p.wl.total_items) {
        int lo = 0, hi = npairs - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (p.wl.item_start[mid] <= item) lo = mid; else hi = mid - 1;
        }
        pair = lo;
        rel = item - p.wl.item_start[lo];
      }
      s_info[0] = pair;
      s_info[1] = rel;
    }
    __syncthreads();
    const int pair = s_info[0];
    const int rel = s_info[1];
    if (pair < 0) break;

    const int b = pair / p.KH, kh = pair - b * p.KH;
    const int gb = rel % p.ngb, chunk = rel / p.ngb;
    const int L = p.seq_lens[b];
    int npos = L;
    const int *idxp = nullptr;
    if (p.token_idx) {
      npos = L > 0 ? min(max(p.n_idx[pair], 0), p.idx_stride) : 0;
      idxp = p.token_idx + (int64_t)pair * p.idx_stride;
    }
    const int pos0 = chunk * p.split;
    const int pos1 = min(npos, pos0 + p.split);
    const int ntile = (pos1 - pos0 + kTile - 1) / kTile;
    const int g0 = gb * 16;
    const int gcount = min(16, p.G - g0);
    const bool qvalid = col < gcount;

    const int64_t head_off = p.seq_offset[b] + (int64_t)kh * p.stride_h;
    const char *kbase = (const char *)p.k + head_off * ES;
    const char *vbase = (const char *)p.v + head_off * ES;
    const int64_t rstride = p.stride_t * ES;

    // Q^T operand (B): column col = query head g0 + col, channels in K's order.
    OpT qop[KB];
    {
      const uint16_t *qrow = (const uint16_t *)p.q +
                             ((int64_t)b * p.QH + (int64_t)kh * p.G + g0 + (qvalid ? col : 0)) * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int d0 = (KVT == ATTN_BF16) ? 8 * (4 * kb + cg) : 64 * (kb >> 1) + 16 * cg + 8 * (kb & 1);
        u32x4_t w = *(const u32x4_t *)(qrow + d0);
        if (!qvalid) w = (u32x4_t){0u, 0u, 0u, 0u};
        if constexpr (KVT == ATTN_BF16) {
          qop[kb] = __builtin_bit_cast(bf16x8_t, w);
        } else {
          f16x8_t h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            h[2 * e] = (_Float16)bf16_lo(w[e]);
            h[2 * e + 1] = (_Float16)bf16_hi(w[e]);
          }
          qop[kb] = h;
        }
      }
    }

    auto row_of = [&](int pos) -> int {
      pos = min(pos, pos1 - 1);
      if (idxp) return min(max(idxp[pos], 0), L - 1);
      return pos;
    };

    auto load_tile = [&](TileT &R, int tile) {
      const int tpos = pos0 + tile * kTile;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const char *row = kbase + (int64_t)row_of(tpos + 16 * tb + col) * rstride;
#pragma unroll
        for (int kl = 0; kl < KL; ++kl) R.k[tb][kl] = *(const u32x4_t *)(row + 16 * (4 * kl + cg));
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int slot = (jj < 4) ? (4 * cg + jj) : (16 + 4 * cg + jj - 4);
        const char *row = vbase + (int64_t)row_of(tpos + slot) * rstride;
        R.v[jj] = *(const VV *)(row + col * VW * 4);
      }
    };

    f32x4_t O[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) O[nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    float m_run = NEG_INF, l_run = 0.f;

    auto compute_tile = [&](const TileT &R, int tile) {
      const int tpos = pos0 + tile * kTile;
      float s[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if constexpr (KVT == ATTN_BF16) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, R.k[tb][kb]), qop[kb], acc,
                                                          0, 0, 0);
          } else {
            const u32x4_t w = R.k[tb][kb >> 1];
            const uint32_t c0 = w[2 * (kb & 1)], c1w = w[2 * (kb & 1) + 1];
            u32x4_t hw;
            hw[0] = codes_to_f16x2((c0 & 0xFFu) | ((c0 & 0xFF00u) << 8));
            hw[1] = codes_to_f16x2(((c0 >> 16) & 0xFFu) | ((c0 >> 8) & 0xFF0000u));
            hw[2] = codes_to_f16x2((c1w & 0xFFu) | ((c1w & 0xFF00u) << 8));
            hw[3] = codes_to_f16x2(((c1w >> 16) & 0xFFu) | ((c1w >> 8) & 0xFF0000u));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, hw), qop[kb], acc, 0, 0, 0);
          }
        }
        float scale_tb = c1;
        if constexpr (KVT == ATTN_I8) {
          if (!idxp) {
            const int t = tpos + 16 * tb;
            scale_tb *= p.k_scale[(int64_t)pair * p.k_scale_stride + t / p.k_part];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = tpos + 16 * tb + 4 * cg + i;
          float sc = scale_tb;
          if constexpr (KVT == ATTN_I8) {
            if (idxp) sc *= p.k_scale[(int64_t)pair * p.k_scale_stride + row_of(pos) / p.k_part];
          }
          s[4 * tb + i] = (pos < pos1) ? acc[i] * sc : NEG_INF;
        }
      }
      float mt = s[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mt = fmaxf(mt, s[i]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      if (__any(m_new > m_run)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nb] *= alpha;
        m_run = m_new;
      }
      const float mref = (m_run == NEG_INF) ? 0.f : m_run;
      OpT phi, plo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float pv = __builtin_amdgcn_exp2f(s[i] - mref);
        pv = qvalid ? pv : 0.f;
        l_run += pv;
        if constexpr (KVT == ATTN_BF16) {
          const uint32_t hb = f32_to_bf16_bits(pv);
          const float hf = __uint_as_float(hb << 16);
          const uint32_t lb = f32_to_bf16_bits(pv - hf);
          phi[i] = __builtin_bit_cast(__bf16, (uint16_t)hb);
          plo[i] = __builtin_bit_cast(__bf16, (uint16_t)lb);
        } else {
          const _Float16 h = (_Float16)pv;
          phi[i] = h;
          plo[i] = (_Float16)(pv - (float)h);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        u32x4_t a;
        if constexpr (KVT == ATTN_BF16) {
          const int w = nb >> 1;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x = word_of<VW>(R.v[2 * q], w), y = word_of<VW>(R.v[2 * q + 1], w);
            a[q] = (nb & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
          }
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), phi, O[nb], 0, 0, 0);
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), plo, O[nb], 0, 0, 0);
        } else {
          const int w = nb >> 2, sh = 8 * (nb & 3);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x = word_of<VW>(R.v[2 * q], w), y = word_of<VW>(R.v[2 * q + 1], w);
            a[q] = codes_to_f16x2(((x >> sh) & 0xFFu) | (((y >> sh) & 0xFFu) << 16));
          }
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), phi, O[nb], 0, 0, 0);
          O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), plo, O[nb], 0, 0, 0);
        }
      }
    };

    // Wave w handles tiles w, w+4, ...; two register buffers alternate.
    {
      TileT ra, rb;
      int t = wave;
      if (t < ntile) load_tile(ra, t);
      while (t < ntile) {
        if (t + kWaves < ntile) load_tile(rb, t + kWaves);
        compute_tile(ra, t);
        t += kWaves;
        if (t >= ntile) break;
        if (t + kWaves < ntile) load_tile(ra, t + kWaves);
        compute_tile(rb, t);
        t += kWaves;
      }
    }

    // Combine the four waves' (m, l, O) and emit one partial per query head.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (cg == 0) {
      s_m[wave][col] = m_run;
      s_l[wave][col] = l_run;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[wave][col][NB * (4 * cg + i) + nb] = O[nb][i];
    __syncthreads();
    const float out_scale = (KVT == ATTN_I8) ? p.v_scale : 1.0f;
    for (int e = tid; e < gcount * D; e += 256) {
      const int g = e / D, d = e - g * D;
      float M = NEG_INF;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (s_l[w][g] > 0.f) M = fmaxf(M, s_m[w][g]);
      float Ls = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (s_l[w][g] > 0.f) {
          const float f = __builtin_amdgcn_exp2f(s_m[w][g] - M);
          Ls += f * s_l[w][g];
          acc += f * s_o[w][g][d];
        }
      }
      const int slot = p.wl.row_split_start[b * p.QH + kh * p.G + g0 + g] + chunk;
      p.wl.o_part[(int64_t)slot * D + d] = (Ls > 0.f) ? acc / Ls * out_scale : 0.f;
      if (d == 0) {
        p.wl.m_part[slot] = (Ls > 0.f) ? M * kLn2 : NEG_INF;
        p.wl.l_part[slot] = Ls;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams &p, int kv_dtype, int grid, hipStream_t s) {
  dim3 g(grid), blk(256);
  if (kv_dtype == ATTN_BF16) {
    if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_BF16>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_BF16>), g, blk, 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_I8>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_I8>), g, blk, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace lcdg
