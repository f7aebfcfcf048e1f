// Split-KV decode attention on the vector ALUs, for fp32 Q/K/V of any head
// size 4..256 (a multiple of 4) and any group size.  Same work split and
// partial format as the matrix-core kernel; used for fp32 inputs.
//
// One 256-thread workgroup per worker.  Each tile of a segment (64
// positions, 32 for head sizes above 128) is staged in LDS with coalesced
// 16-byte loads (K rows padded by 16 bytes, so lanes reading 16-byte pieces
// of different rows hit different banks), and the next two tiles' loads are
// in flight in registers while the current one is computed.  The tile then
// follows the online softmax of the Flash Attention block pseudo-code
// ("注意力优化（Attention Optimization）"): scores -> new running max ->
// rescale (alpha) -> probabilities -> O = alpha*O + P V, in natural-log
// units; the chunk's (m, l, O/l) is the partial triple of
// "优化稀疏注意力中的令牌丢弃机制" §5.  Thread (head g, position i) of a
// lane group (a wave, or half of one for 32-position tiles) computes that
// score and takes the head's running max and sum with shuffles inside the
// group, so the softmax needs no serial loop.
#include "common.hpp"

namespace lcdg {
namespace {

constexpr int kWT = 32;      // tokens per tile of the work split (the lane walk's unit)
constexpr int kVMaxD = 256;  // largest head size

// max / sum over the W lanes of a lane group (W = 32 or 64), every lane of the
// group getting the result: DPP moves inside each row of 16 lanes (swap
// neighbours, swap pairs, mirror each half-row, mirror the row), then the row
// swaps of gfx950 (rows 0<->1, 2<->3, and for W = 64 the two halves), with no
// trip through the LDS crossbar.
template <int C>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), C, 0xF, 0xF, false));
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_move<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_move<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_move<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_move<0x140>(v));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  if constexpr (W == 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  return v;
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x141>(v);
  v += dpp_move<0x140>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  if constexpr (W == 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  return v;
}

// DC: the head-size class (64, 128 or 256) that sizes the per-thread load
// registers; two tiles' loads are in flight while one is computed.  A
// compute tile holds TT = 64 positions (32 for head sizes above 128, which
// would not fit two tiles' loads in registers): the steps of a segment are a
// chain of dependent LDS phases and barriers, so fewer, larger steps finish
// it sooner.  IDX: positions go through the kept-token list.
template <int DC, bool IDX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_valu_kernel(DecodeParams p) {
  constexpr int TT = DC > 128 ? 32 : 64;         // positions per compute tile = lanes per head (scores)
  constexpr int NP = 16 * TT / 256;                // score passes over the 16 heads of a block
  constexpr int KO = 16 * DC / 256;                // (head, channel) outputs per thread
  constexpr int kVChunks = TT * DC / 4 / 256;      // 16-byte loads per thread for K (and V) of a tile
  constexpr int KR = DC + 4;                       // padded K row (floats)
  __shared__ __attribute__((aligned(16))) float s_q[16][DC];  // q * softmax_scale
  __shared__ __attribute__((aligned(16))) float s_k[TT][KR];  // K rows of the tile
  __shared__ __attribute__((aligned(16))) float s_v[TT][DC];
  __shared__ __attribute__((aligned(16))) float s_p[16][TT];  // probabilities (0 past the segment)
  __shared__ float s_alpha[16], s_m[16], s_l[16];

  const int tid = threadIdx.x;
  const int D = p.D;
  const int cpr = D / 4;  // 16-byte chunks per row
  const float NEG_INF = -__builtin_huge_valf();

  if (p.direct_out && blockIdx.x == 0) {
    // no merge follows: the lanes without positions get out = 0 and
    // lse = -inf here (every other lane is one segment of this worker)
    const int nlanes = p.B * p.KH * p.lpp;
    for (int q = 0; q < nlanes; ++q) {
      const int pair = q / p.lpp, gb = q - pair * p.lpp;
      const int b = pair / p.KH, kh = pair - b * p.KH;
      const int L = min(max(p.seq_lens[b], 0), p.max_seq_len);
      const int npos = IDX ? (L > 0 ? min(max(p.n_idx[pair], 0), p.idx_stride) : 0) : L;
      if (npos > 0) continue;
      const int g0 = gb * 16, gcount = min(16, p.G - g0);
      for (int e = tid; e < gcount * D; e += 256) {
        const int g = e / D, d = e - g * D;
        const int64_t orow = q_row_index(p, b, kh, g0 + g);
        if (p.out_dtype == ATTN_F32) ((float *)p.out)[orow * D + d] = 0.f;
        else ((uint16_t *)p.out)[orow * D + d] = 0u;
        if (d == 0 && p.lse) p.lse[orow] = NEG_INF;
      }
    }
  }

  const int T = wave_total_tiles(p);
  const int nwg = workers_for(p, T);
  if ((int)blockIdx.x >= nwg) return;
  const int t_begin = (int)((int64_t)blockIdx.x * T / nwg);
  const int t_end = (int)((int64_t)(blockIdx.x + 1) * T / nwg);
  const int ct = p.split / kWT;
  // score-phase roles: head tid / TT (+ 256 / TT per further pass), position tid % TT
  const int sg = tid / TT, si = tid % TT;

  // every wave of the workgroup walks the lanes alike
  LaneHit hit = wave_find_lane(p, t_begin);
  for (int t = t_begin; t < t_end;) {
    if (hit.nt == 0) break;  // lane walk exhausted (cannot happen for t < total)
    const int q = hit.q;
    const int lane_t0 = hit.t0, lane_t1 = hit.t0 + hit.nt;
    const int run_end = min(t_end, lane_t1);
    const int pair = q / p.lpp, gb = q - pair * p.lpp;
    const int b = pair / p.KH, kh = pair - b * p.KH;
    const int L = min(max(p.seq_lens[b], 0), p.max_seq_len);
    int npos = L;
    const int *idxp = nullptr;
    if constexpr (IDX) {
      npos = L > 0 ? min(max(p.n_idx[pair], 0), p.idx_stride) : 0;
      idxp = p.token_idx + (int64_t)pair * p.idx_stride;
    }
    const int g0 = gb * 16;
    const int gcount = min(16, p.G - g0);
    const int64_t head_off = p.seq_offset[b] + (int64_t)kh * p.stride_h;
    const float *kb = (const float *)p.k + head_off, *vb = (const float *)p.v + head_off;

    __syncthreads();
    for (int e = tid; e < gcount * D; e += 256) {
      const int g = e / D, d = e - g * D;
      s_q[g][d] = ((const float *)p.q)[((int64_t)b * p.QH + (int64_t)kh * p.G + g0 + g) * D + d] * p.softmax_scale;
    }

    // The K and V rows of the tile starting at position pos: chunk
    // c = tid + 256 j is row c / cpr, channels 4 (c % cpr) ...  The loads are
    // unconditional, so the compiler can wait for one tile's loads while the
    // next tile's stay in flight: a row at or past the segment's end (or past
    // the tile) reads the segment's last row instead, which is harmless, as
    // positions past the end get probability 0 and rows past the tile are
    // never staged.  pos_end > 0 whenever this is called.
    struct TileRegs {
      f32x4_t k[kVChunks], v[kVChunks];
    };
    auto load_tile = [&](TileRegs &R, int pos, int pos_end) {
      f32x4_t(&rk)[kVChunks] = R.k;
      f32x4_t(&rv)[kVChunks] = R.v;
#pragma unroll
      for (int j = 0; j < kVChunks; ++j) {
        const int c = tid + 256 * j, r = c / cpr;
        int tok = min(pos + min(r, TT - 1), pos_end - 1);
        if constexpr (IDX) tok = min(max(idxp[tok], 0), L - 1);
        const int64_t off = (int64_t)tok * p.stride_t + 4 * (c - r * cpr);
        rk[j] = *(const f32x4_t *)(kb + off);
        rv[j] = *(const f32x4_t *)(vb + off);
      }
    };
    auto store_tile = [&](const TileRegs &R) {
      const f32x4_t(&rk)[kVChunks] = R.k;
      const f32x4_t(&rv)[kVChunks] = R.v;
#pragma unroll
      for (int j = 0; j < kVChunks; ++j) {
        const int c = tid + 256 * j, r = c / cpr;
        if (r < TT) {
          const int d = 4 * (c - r * cpr);
          *(f32x4_t *)&s_k[r][d] = rk[j];
          *(f32x4_t *)&s_v[r][d] = rv[j];
        }
      }
    };

    // one segment per chunk piece of this run
    for (int seg_t0 = t; seg_t0 < run_end;) {
      const int chunk = (seg_t0 - lane_t0) / ct;
      const int chunk_t1 = min(lane_t1, lane_t0 + (chunk + 1) * ct);
      const int seg_t1 = min(run_end, chunk_t1);
      const int pos0 = (seg_t0 - lane_t0) * kWT;
      const int pos1 = min(npos, (seg_t1 - lane_t0) * kWT);
      // running max and sum of heads sg + (256 / TT) h (every lane of a head's
      // lane group holds that head's)
      float m_run[NP], l_run[NP];
#pragma unroll
      for (int h = 0; h < NP; ++h) {
        m_run[h] = NEG_INF;
        l_run[h] = 0.f;
      }
      float o[KO];
#pragma unroll
      for (int k = 0; k < KO; ++k) o[k] = 0.f;

      // tile tp: stage it (its loads were issued two tiles ago), issue the
      // loads of tile tp + 2 tiles into the same registers, compute
      auto step = [&](TileRegs &R, int tp) {
        if (tp >= pos1) return;
        __syncthreads();  // the previous tile's readers are done
        store_tile(R);
        load_tile(R, tp + 2 * TT, pos1);
        __syncthreads();
        const int n = min(TT, pos1 - tp);
#pragma unroll
        for (int h = 0; h < NP; ++h) {
          const int g = sg + (256 / TT) * h;
          if (g < gcount) {  // uniform over the lane group
            // 16-byte LDS reads: the head's query (one address for the
            // group) and this lane's K row
            const f32x4_t *qr = (const f32x4_t *)&s_q[g][0];
            const f32x4_t *kr = (const f32x4_t *)&s_k[si][0];
            f32x4_t a4 = {0.f, 0.f, 0.f, 0.f};
            int d4 = 0;
            for (; d4 + 4 <= cpr; d4 += 4) {
#pragma unroll
              for (int u = 0; u < 4; ++u) a4 += qr[d4 + u] * kr[d4 + u];
            }
            for (; d4 < cpr; ++d4) a4 += qr[d4] * kr[d4];
            const float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
            const float s = si < n ? acc : NEG_INF;
            const float m_new = fmaxf(m_run[h], group_max<TT>(s));  // finite: the tile has a token
            const float e = si < n ? expf(s - m_new) : 0.f;
            const float alpha = m_run[h] == NEG_INF ? 0.f : expf(m_run[h] - m_new);
            l_run[h] = alpha * l_run[h] + group_sum<TT>(e);
            m_run[h] = m_new;
            s_p[g][si] = e;
            if (si == 0) s_alpha[g] = alpha;
          }
        }
        __syncthreads();
        // O = alpha O + P V for the (g, d) outputs this thread owns
#pragma unroll
        for (int k = 0; k < KO; ++k) {
          const int e = tid + 256 * k;
          if (e < gcount * D) {
            const int g = e / D, d = e - g * D;
            float acc = o[k] * s_alpha[g];
#pragma unroll
            for (int i = 0; i < TT; i += 4) {
              const f32x4_t pp = *(const f32x4_t *)&s_p[g][i];
#pragma unroll
              for (int u = 0; u < 4; ++u) acc += pp[u] * s_v[i + u][d];
            }
            o[k] = acc;
          }
        }
      };
      TileRegs ra, rb;
      load_tile(ra, pos0, pos1);
      load_tile(rb, pos0 + TT, pos1);
      for (int tp = pos0; tp < pos1; tp += 2 * TT) {
        step(ra, tp);
        step(rb, tp + TT);
      }
#pragma unroll
      for (int h = 0; h < NP; ++h) {
        const int g = sg + (256 / TT) * h;
        if (g < gcount && si == 0) {
          s_m[g] = m_run[h];
          s_l[g] = l_run[h];
        }
      }
      __syncthreads();

      if (p.direct_out) {
        // the segment is the whole lane: out = O / l and lse = m + ln l
#pragma unroll
        for (int k = 0; k < KO; ++k) {
          const int e = tid + 256 * k;
          if (e < gcount * D) {
            const int g = e / D, d = e - g * D;
            const float l = s_l[g];
            const float ov = (l > 0.f) ? o[k] / l : 0.f;
            const int64_t orow = q_row_index(p, b, kh, g0 + g);
            if (p.out_dtype == ATTN_F32) ((float *)p.out)[orow * D + d] = ov;
            else ((uint16_t *)p.out)[orow * D + d] = (uint16_t)f32_to_bf16_bits(ov);
            if (d == 0 && p.lse) p.lse[orow] = (l > 0.f) ? s_m[g] + logf(l) : NEG_INF;
          }
        }
        seg_t0 = seg_t1;
        continue;
      }
      const int half = (seg_t0 == lane_t0 + chunk * ct) ? 0 : 1;
      const bool fill_second = half == 0 && seg_t1 == chunk_t1;
#pragma unroll
      for (int k = 0; k < KO; ++k) {
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
      seg_t0 = seg_t1;
    }
    t = run_end;
    if (t < t_end) hit = next_lane(p, hit);
  }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams &p, int q_dtype, int kv_dtype, hipStream_t s) {
  if (q_dtype != ATTN_F32 || kv_dtype != ATTN_F32 || p.D > kVMaxD || p.D % 4) return hipErrorInvalidValue;
  const bool idx = p.token_idx != nullptr;
  if (p.D <= 64) {
    if (idx) hipLaunchKernelGGL((decode_valu_kernel<64, true>), dim3(p.grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_valu_kernel<64, false>), dim3(p.grid), dim3(256), 0, s, p);
  } else if (p.D <= 128) {
    if (idx) hipLaunchKernelGGL((decode_valu_kernel<128, true>), dim3(p.grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_valu_kernel<128, false>), dim3(p.grid), dim3(256), 0, s, p);
  } else {
    if (idx) hipLaunchKernelGGL((decode_valu_kernel<256, true>), dim3(p.grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_valu_kernel<256, false>), dim3(p.grid), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace lcdg
