// Split-KV GQA decode attention on gfx950 matrix cores (bf16 or int8 KV).
//
// One wave is one worker of a persistent grid.  The 32-token tiles of every
// (sequence b, KV head kh, column block) are laid end to end and each wave
// streams one balanced contiguous range of them, cut into chunks of
// split_tokens positions, with its next tiles in flight in a register ring
// while it computes the current one:
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
//  * A KV head with more than 16 query rows runs 32-column workers (CB = 2):
//    two 16-column blocks whose MFMAs take the same K and V operands, so 32
//    rows share one read of the cache; such a wave holds twice the
//    accumulators and runs alone on its SIMD.
#include "common.hpp"

namespace lcdg {
namespace {

constexpr int kTile = 32;

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

// Registers of one 32-token tile: K in the MFMA operand layout, V as natural
// per-lane row pieces, and (int8) the K scales of the lane's scores.
template <int D, int KVT, bool IDX>
struct Tile {
  static constexpr int ES = (KVT == ATTN_BF16) ? 2 : 1;
  static constexpr int KL = (KVT == ATTN_BF16) ? D / 32 : D / 64;  // 16-byte K loads per token block
  static constexpr int VW = (D / 16) * ES / 4;                      // V words per token per lane
  static constexpr int NS = (KVT == ATTN_I8) ? (IDX ? 8 : 2) : 0;   // K scales per lane
  u32x4_t k[2][KL];
  typename VecW<VW>::T v[8];
  float ks[NS > 0 ? NS : 1];
};

// A pipeline step: TPS consecutive tiles, as many as fit a per-buffer
// register budget (64 VGPRs for bf16; 32 for int8, whose dequantisation needs
// more temporaries), so small tiles still keep more bytes in flight.
template <int D, int KVT, bool IDX, int CB>
struct Step {
  typedef Tile<D, KVT, IDX> TileT;
  static constexpr int kRegs = 2 * TileT::KL * 4 + 8 * TileT::VW;
  static constexpr int kBudget = KVT == ATTN_BF16 ? 64 : 32;
  static constexpr int TPS = kRegs >= kBudget ? 1 : kBudget / kRegs;
  // Steps in flight: NBUF register buffers rotate, so while one step is
  // consumed the next NBUF-1 are loading.  int8 starts a step's scores one
  // step early (its score chain, not its bytes, limits it), so the K of that
  // step has only NBUF-2 steps to arrive; it keeps four buffers where they
  // fit in registers (one-tile steps over the whole cache) and three where a
  // step holds two tiles or token indices take registers.
  // Two column blocks per wave (CB = 2) run one wave per SIMD with twice the
  // registers, so the ring is deeper to keep as many bytes in flight per SIMD.
  static constexpr int NBUF = CB == 2 ? (KVT == ATTN_BF16 ? 4 : (TPS == 1 && !IDX ? 6 : 4))
                                      : (KVT == ATTN_BF16 ? 2 : (TPS == 1 && !IDX ? 4 : 3));
  static constexpr bool PIPE = KVT == ATTN_I8;
  TileT t[TPS];
};

// Tokens per chunk of the indexed variant (its index list is staged in LDS).
constexpr int kMaxIdxChunk = 1024;
// Page ids a segment of the paged variant stages in LDS (a chunk may span at
// most 64 pages, so at most 65 are touched).
constexpr int kMaxSegPages = 72;

// One wave = one worker.  The work-list lays every (b, kh, head block) lane's
// tiles end to end; worker w streams the contiguous tile range
// [w*T/W, (w+1)*T/W), so all workers move the same number of K/V bytes
// whatever the mix of sequence lengths, with no atomics and no barriers in
// the loop.  A range is cut into runs (one lane each) and runs into segments
// (one chunk piece each); a segment's partial (m, l, o) goes straight from
// registers to its slot.
template <int D, int KVT, bool IDX, bool QI8, bool PAGED, int CB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(CB == 2 ? 1 : 2, CB == 2 ? 1 : 2))) void
decode_mfma_kernel(DecodeParams p) {
  static_assert(!(IDX && PAGED), "a paged cache is read by position");
  static_assert(CB == 1 || CB == 2, "one or two 16-column blocks per wave");
  typedef Tile<D, KVT, IDX> TileT;
  typedef Step<D, KVT, IDX, CB> StepT;
  constexpr int TPS = StepT::TPS;
  constexpr int NB = D / 16;
  constexpr int ES = TileT::ES;
  constexpr int KL = TileT::KL;
  constexpr int KB = D / 32;
  constexpr int VW = TileT::VW;
  typedef typename std::conditional<KVT == ATTN_BF16, bf16x8_t, f16x8_t>::type OpT;

  __shared__ int s_idx[IDX ? kMaxIdxChunk : 1];
  __shared__ int s_pages[PAGED ? kMaxSegPages : 1];  // page ids of the current segment
  // Q^T operand of the current run, 16*CB query rows x D channels, rows padded
  // by 16 bytes against bank conflicts: bf16 for bf16 KV; for int8 KV three
  // int8 digit planes of each row's 22-bit fixed-point query (see below).
  constexpr int kQRow = D * 2 + 16;
  constexpr int kQDRow = D + 16;
  constexpr int kQBytes = CB * (KVT == ATTN_I8 ? 3 * 16 * kQDRow : 16 * kQRow);
  __shared__ __attribute__((aligned(16))) unsigned char s_q[kQBytes];

  const int lane = threadIdx.x;
  const int col = lane & 15, cg = lane >> 4;
  const float c1 = p.softmax_scale * kLog2e;
  const float NEG_INF = -__builtin_huge_valf();

  const int T = wave_total_tiles(p);
  const int nworkers = workers_for(p, T);
  if ((int)blockIdx.x >= nworkers) return;
  const int t_begin = (int)((int64_t)blockIdx.x * T / nworkers);
  const int t_end = (int)((int64_t)(blockIdx.x + 1) * T / nworkers);
  const int ct = p.split / kTile;  // tiles per chunk

  // the lane (b, kh, query-head block) holding the first tile of the range;
  // each later run takes the next lane that has tiles
  LaneHit hit = wave_find_lane(p, t_begin);
  for (int t = t_begin; t < t_end;) {
    if (hit.nt == 0) break;  // lane walk exhausted (cannot happen for t < total)
    const int q = hit.q;
    const int lane_t0 = hit.t0, lane_t1 = hit.t0 + hit.nt;
    const int run_end = min(t_end, lane_t1);
    const int pair = q / p.ngb, gb = q - pair * p.ngb;
    const int b = pair / p.KH, kh = pair - b * p.KH;
    const int L = uniform_i32(min(max(p.seq_lens[b], 0), p.max_seq_len));
    int npos = L;
    if constexpr (IDX) npos = uniform_i32(L > 0 ? min(max(p.n_idx[pair], 0), p.idx_stride) : 0);
    // this lane's column of block cb is query row g0 + 16*cb + col of the KV head
    const int g0 = gb * 16 * CB;
    bool qvalid[CB];
    int col_end[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      qvalid[cb] = g0 + 16 * cb + col < p.G;
      // with R query rows per sequence, column gc is row r = gc / Gq, the token
      // at position L - R + r: it sees the first L - (R - 1) + r tokens
      col_end[cb] = p.R > 1 ? L - (p.R - 1) + (g0 + 16 * cb + col) / p.Gq : 0x7FFFFFFF;
    }

    // Buffer resources over this (b, kh)'s rows: 32-bit offsets, and rows at
    // or past L read as zero (their scores are masked), so no clamping.  A
    // paged cache gets one resource per tile instead (see load_tile).
    const int64_t head_off = PAGED ? 0 : uniform_i64(p.seq_offset[b]) + (int64_t)kh * p.stride_h;
    const char *kbase = (const char *)p.k + head_off * ES;
    const char *vbase = (const char *)p.v + head_off * ES;
    const uint32_t rs = (uint32_t)(p.stride_t * ES);
    const int nrec = L > 0 ? (int)((uint32_t)(L - 1) * rs + D * ES) : 0;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kbase, (short)0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vbase, (short)0, nrec, 0x00020000);
    // int8 K scales of this pair, read through a buffer resource as well, so
    // they are fetched in the same in-order stream as the tile they belong to
    // (a plain load sunk towards its use would make every wait drain the
    // tiles issued after it).
    const bool i8 = KVT == ATTN_I8;
    const __amdgpu_buffer_rsrc_t ksrs = __builtin_amdgcn_make_buffer_rsrc(
        i8 ? (void *)(p.k_scale + (int64_t)pair * p.k_scale_stride) : nullptr, (short)0,
        i8 ? max(p.k_scale_stride, 1) * 4 : 0, 0x00020000);

    // Stage Q (the 16 heads of this block, zero past G) in LDS in MFMA
    // operand form; tiles read their B operand from there.  The partial
    // slots of this lane's rows are loaded now as well: a global load inside
    // the segment loop would make the compiler wait for every load in
    // flight, the tile prefetch included.
    //
    // int8 KV: the scores run on the int8 matrix cores straight from the K
    // codes.  Head g's query becomes q = s_g * n with s_g = max|q_g| / 2^22
    // and n = rint(q / s_g) = 65536 d2 + 256 d1 + d0, d0, d1 in [-128, 127]
    // and |d2| <= 64 (|error| <= max|q_g| * 2^-23); each digit plane is one
    // int8 MFMA, and the three integer sums recombine exactly in fp32.  An
    // int8 query (QI8: per-row or static scale) is plane 0 alone.
    float qs[CB];  // int8: this lane's column scale s_col in each block
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) qs[cb] = 0.f;
    __syncthreads();
    if constexpr (KVT == ATTN_I8) {
      constexpr int CPL = D / 4;  // lane (col, cg) takes column col, channels [cg*CPL, cg*CPL + CPL)
      unsigned char *sq_blk = s_q;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb, sq_blk += 3 * 16 * kQDRow) {
        float qv[CPL];
        const uint16_t *qrow = (const uint16_t *)p.q + q_row_index(p, b, kh, g0 + 16 * cb + col) * D + cg * CPL;
#pragma unroll
        for (int x = 0; x < CPL / 8; ++x) {
          u32x4_t w = (u32x4_t){0u, 0u, 0u, 0u};
          if (qvalid[cb]) w = *(const u32x4_t *)(qrow + 8 * x);
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            qv[8 * x + 2 * y] = bf16_lo(w[y]);
            qv[8 * x + 2 * y + 1] = bf16_hi(w[y]);
          }
        }
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) mx = fmaxf(mx, fabsf(qv[j]));
        mx = rows_max(mx);  // the four lanes of column col hold all D channels
        if constexpr (QI8) {
          // int8 query (one digit plane): s = max|q_row| / 127, or the static
          // scale, and code = clamp(rint(q / s), -127, 127), in IEEE fp32
          // (correctly rounded divides, round half to even).
          const float sq = p.q_quant == ATTN_QUANT_ROW ? mx / 127.0f : p.q_scale;
          qs[cb] = sq;
#pragma unroll
          for (int x = 0; x < CPL / 16; ++x) {
            uint32_t w[4];
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
              uint32_t acc = 0u;
#pragma unroll
              for (int y = 0; y < 4; ++y) {
                float c = 0.f;
                if (sq > 0.f) c = fminf(127.f, fmaxf(-127.f, __builtin_rintf(qv[16 * x + 4 * j4 + y] / sq)));
                acc |= ((uint32_t)(int)c & 0xFFu) << (8 * y);
              }
              w[j4] = acc;
            }
            *(u32x4_t *)(sq_blk + col * kQDRow + cg * CPL + 16 * x) = (u32x4_t){w[0], w[1], w[2], w[3]};
          }
        } else {
          const float inv = mx > 0.f ? 4194304.0f / mx : 0.f;
          qs[cb] = mx * (1.0f / 4194304.0f);
          uint32_t dw[3][CPL / 4];
#pragma unroll
          for (int j4 = 0; j4 < CPL / 4; ++j4) {
            uint32_t w0 = 0u, w1 = 0u, w2 = 0u;
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              const int n = (int)__builtin_rintf(qv[4 * j4 + y] * inv);
              const int d0 = (int)(int8_t)(n & 0xFF);
              const int r1 = (n - d0) >> 8;
              const int d1 = (int)(int8_t)(r1 & 0xFF);
              const int d2 = (r1 - d1) >> 8;
              w0 |= (uint32_t)(d0 & 0xFF) << (8 * y);
              w1 |= (uint32_t)(d1 & 0xFF) << (8 * y);
              w2 |= (uint32_t)(d2 & 0xFF) << (8 * y);
            }
            dw[0][j4] = w0;
            dw[1][j4] = w1;
            dw[2][j4] = w2;
          }
#pragma unroll
          for (int dg = 0; dg < 3; ++dg)
#pragma unroll
            for (int x = 0; x < CPL / 16; ++x)
              *(u32x4_t *)(sq_blk + (dg * 16 + col) * kQDRow + cg * CPL + 16 * x) =
                  (u32x4_t){dw[dg][4 * x], dw[dg][4 * x + 1], dw[dg][4 * x + 2], dw[dg][4 * x + 3]};
        }
      }
    } else {
      for (int e = lane; e < 16 * CB * (D / 8); e += 64) {
        const int g = e / (D / 8), c8 = e - g * (D / 8);
        u32x4_t w = (u32x4_t){0u, 0u, 0u, 0u};
        if (g0 + g < p.G)
          w = *(const u32x4_t *)((const uint16_t *)p.q + q_row_index(p, b, kh, g0 + g) * D + 8 * c8);
        *(u32x4_t *)(s_q + g * kQRow + 16 * c8) = w;
      }
    }
    // partial (pair, slot j, column g) lives at (pair*2*max_chunks + j)*G + g
    const int slot_base = pair * 2 * p.max_chunks * p.G + g0 + col;
    __syncthreads();
    auto q_operand = [&](int cb, int kb) -> bf16x8_t {
      return __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(s_q + (16 * cb + col) * kQRow + 16 * (4 * kb + cg)));
    };
    // int8: digit plane dg of channels 64kb + 16cg .. + 15 of column col of block cb
    auto q_digits = [&](int cb, int dg, int kb) -> i32x4_t {
      return __builtin_bit_cast(i32x4_t,
                                *(const u32x4_t *)(s_q + ((3 * cb + dg) * 16 + col) * kQDRow + 64 * kb + 16 * cg));
    };

    // Positions of the current segment (IDX: its staged index list starts at
    // seg_pos0; PAGED: its staged page ids start at page seg_page0).
    int seg_pos0 = 0, seg_pos1 = 0, seg_page0 = 0;
    auto row_of = [&](int pos) -> int {
      if constexpr (IDX) return s_idx[min(pos, seg_pos1 - 1) - seg_pos0];
      return pos;
    };

    // Issue one tile's loads.  Every path through the loops issues the same
    // number of loads, so the compiler's wait counts never drain the tile in
    // flight; a tile that is not needed gets an out-of-range offset, which
    // the buffer unit answers with zeros and no memory traffic.
    auto load_tile = [&](TileT &R, int tile, bool valid) {
      const int tpos = (tile - lane_t0) * kTile;
      const uint32_t oob = valid ? 0u : 0x80000000u;
      __amdgpu_buffer_rsrc_t tk = krs, tv = vrs;
      int rshift = 0;  // row of position x in the resource: row_of(x) + rshift
      if constexpr (PAGED) {
        // page_tokens is a multiple of 32, so the tile lies in one page;
        // rows of that page at or past L read as zero
        const int pidx = tpos / p.page_tokens;
        const int pg = __builtin_amdgcn_readfirstlane(s_pages[min(max(pidx - seg_page0, 0), kMaxSegPages - 1)]);
        const int rows = min(p.page_tokens, L - pidx * p.page_tokens);
        const int nrec_p = rows > 0 ? (int)((uint32_t)(rows - 1) * rs + D * ES) : 0;
        const int64_t eoff = (int64_t)pg * p.page_stride + (int64_t)kh * p.stride_h;
        tk = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)p.k + eoff * ES), (short)0, nrec_p, 0x00020000);
        tv = __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)p.v + eoff * ES), (short)0, nrec_p, 0x00020000);
        rshift = -pidx * p.page_tokens;
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const uint32_t off = ((uint32_t)(row_of(tpos + 16 * tb + col) + rshift) * rs + 16 * cg) | oob;
#pragma unroll
        for (int kl = 0; kl < KL; ++kl) R.k[tb][kl] = __builtin_amdgcn_raw_buffer_load_b128(tk, off + 64 * kl, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int slot = (jj < 4) ? (4 * cg + jj) : (16 + 4 * cg + jj - 4);
        const uint32_t off = ((uint32_t)(row_of(tpos + slot) + rshift) * rs + col * VW * 4) | oob;
        if constexpr (VW == 4) R.v[jj] = __builtin_amdgcn_raw_buffer_load_b128(tv, off, 0, 0);
        else if constexpr (VW == 2) R.v[jj] = __builtin_amdgcn_raw_buffer_load_b64(tv, off, 0, 0);
        else R.v[jj] = __builtin_amdgcn_raw_buffer_load_b32(tv, off, 0, 0);
      }
      if constexpr (KVT == ATTN_I8) {
        const int last = max(npos - 1, 0);
        if constexpr (IDX) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t part = (uint32_t)(row_of(tpos + 16 * (i >> 2) + 4 * cg + (i & 3)) / p.k_part);
            R.ks[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksrs, (4 * part) | oob, 0, 0));
          }
        } else {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const uint32_t part = (uint32_t)(min(tpos + 16 * tb, last) / p.k_part);
            R.ks[tb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksrs, (4 * part) | oob, 0, 0));
          }
        }
      }
    };

    // a step = tiles tile0 .. tile0+TPS-1, each valid while below `limit`
    // The scheduling barrier keeps a step's loads (scales included) issued
    // as one group, in program order: the wait counts then stay the same on
    // every path into the loop, and a wait for one step never drains the
    // steps issued after it.
    auto load_step = [&](StepT &S, int tile0, int limit) {
#pragma unroll
      for (int j = 0; j < TPS; ++j) load_tile(S.t[j], tile0 + j, tile0 + j < limit);
      __builtin_amdgcn_sched_barrier(0);
    };

    // running output, max and sum of each column block
    f32x4_t O[CB][NB];
    float m_run[CB], l_run[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) O[cb][nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      m_run[cb] = NEG_INF;
      l_run[cb] = 0.f;
    }

    // Raw q.k of a tile's 8 scores of this lane in each column block (before
    // scale and mask).  The K operands as loaded serve every block.
    struct Raw {
      float v[CB][8];
    };
    auto qk_tile = [&](const TileT &R) -> Raw {
      Raw r;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
          if constexpr (KVT == ATTN_BF16) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, R.k[tb][kb]),
                                                            q_operand(cb, kb), acc, 0, 0, 0);
          } else {
            // the K codes as loaded are the int8 A operand (lane (col, cg):
            // token col, channels 64kb + 16cg .. + 15)
            i32x4_t a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0}, a2 = {0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < KL; ++kb) {
              const i32x4_t kop = __builtin_bit_cast(i32x4_t, R.k[tb][kb]);
              a0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, q_digits(cb, 0, kb), a0, 0, 0, 0);
              if constexpr (!QI8) {
                a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, q_digits(cb, 1, kb), a1, 0, 0, 0);
                a2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, q_digits(cb, 2, kb), a2, 0, 0, 0);
              }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[i] = QI8 ? (float)a0[i] : ((float)a2[i] * 65536.0f + (float)a1[i] * 256.0f) + (float)a0[i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) r.v[cb][4 * tb + i] = acc[i];
        }
      }
      return r;
    };

    // Online softmax and P.V of a tile whose raw scores are given; the V
    // operands are assembled once and serve every column block.
    auto finish_tile = [&](const TileT &R, int tile, const Raw &raw) {
      const int tpos = (tile - lane_t0) * kTile;
      OpT phi[CB], plo[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int lim = min(seg_pos1, col_end[cb]);
        float s[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = tpos + 16 * tb + 4 * cg + i;
            float sc = c1;
            if constexpr (KVT == ATTN_I8) sc *= qs[cb] * (IDX ? R.ks[4 * tb + i] : R.ks[tb]);
            s[4 * tb + i] = (pos < lim) ? raw.v[cb][4 * tb + i] * sc : NEG_INF;
          }
        float mt = s[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mt = fmaxf(mt, s[i]);
        mt = rows_max(mt);
        const float m_new = fmaxf(m_run[cb], mt);
        if (__any(m_new > m_run[cb])) {
          const float alpha = __builtin_amdgcn_exp2f(m_run[cb] - m_new);
          l_run[cb] *= alpha;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) O[cb][nb] *= alpha;
          m_run[cb] = m_new;
        }
        const float mref = (m_run[cb] == NEG_INF) ? 0.f : m_run[cb];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float pv = __builtin_amdgcn_exp2f(s[i] - mref);
          pv = qvalid[cb] ? pv : 0.f;
          l_run[cb] += pv;
          if constexpr (KVT == ATTN_BF16) {
            const uint32_t hb = f32_to_bf16_bits(pv);
            const float hf = __uint_as_float(hb << 16);
            const uint32_t lb = f32_to_bf16_bits(pv - hf);
            phi[cb][i] = __builtin_bit_cast(__bf16, (uint16_t)hb);
            plo[cb][i] = __builtin_bit_cast(__bf16, (uint16_t)lb);
          } else {
            const _Float16 h = (_Float16)pv;
            phi[cb][i] = h;
            plo[cb][i] = (_Float16)(pv - (float)h);
          }
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        u32x4_t a;
        if constexpr (KVT == ATTN_BF16) {
          const int w = nb >> 1;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const uint32_t x = word_of<VW>(R.v[2 * qq], w), y = word_of<VW>(R.v[2 * qq + 1], w);
            // the low (even nb) or high (odd nb) bf16 of tokens 2qq and 2qq+1
            a[qq] = __builtin_amdgcn_perm(y, x, (nb & 1) ? 0x07060302u : 0x05040100u);
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            O[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), phi[cb], O[cb][nb],
                                                                0, 0, 0);
            O[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), plo[cb], O[cb][nb],
                                                                0, 0, 0);
          }
        } else {
          const int w = nb >> 2;
          const uint32_t k = (uint32_t)(nb & 3);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            // byte k of tokens 2qq and 2qq+1 into the low byte of each half
            const uint32_t x = word_of<VW>(R.v[2 * qq], w), y = word_of<VW>(R.v[2 * qq + 1], w);
            a[qq] = codes_to_f16x2(__builtin_amdgcn_perm(y, x, 0x0c000c00u | k | ((4u + k) << 16)));
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            O[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), phi[cb], O[cb][nb],
                                                               0, 0, 0);
            O[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), plo[cb], O[cb][nb],
                                                               0, 0, 0);
          }
        }
      }
    };

    struct RawStep {
      Raw t[TPS];
    };
    auto qk_step = [&](const StepT &S) -> RawStep {
      RawStep r;
#pragma unroll
      for (int j = 0; j < TPS; ++j) r.t[j] = qk_tile(S.t[j]);
      return r;
    };
    auto finish_step = [&](const StepT &S, int tile0, const RawStep &r) {
#pragma unroll
      for (int j = 0; j < TPS; ++j) finish_tile(S.t[j], tile0 + j, r.t[j]);
    };

    // Segments: the run cut at chunk boundaries.  The NBUF register buffers
    // rotate statically: a segment takes a multiple of NBUF steps (the last
    // ones may be empty), and step s is loaded NBUF-1 steps before it is
    // consumed.  Loads issued past the segment's last step already fetch the
    // first steps of the next segment of the run (positions, not index
    // lists, so not in indexed mode), through one load site so that both
    // cases share the same registers.
    constexpr int NBUF = StepT::NBUF;
    StepT buf[NBUF];
    auto seg_end_of = [&](int s0) { return min(run_end, lane_t0 + ((s0 - lane_t0) / ct + 1) * ct); };
    if constexpr (!IDX && !PAGED) {
      const int t1 = seg_end_of(t);
#pragma unroll
      for (int j = 0; j + 1 < NBUF; ++j) load_step(buf[j], t + j * TPS, t1);
    }
    for (int seg_t0 = t; seg_t0 < run_end;) {
      const int seg_t1 = seg_end_of(seg_t0);
      const int chunk = (seg_t0 - lane_t0) / ct;
      const int chunk_t1 = min(lane_t1, lane_t0 + (chunk + 1) * ct);
      seg_pos0 = (seg_t0 - lane_t0) * kTile;
      seg_pos1 = min(npos, (seg_t1 - lane_t0) * kTile);
      if constexpr (IDX) {
        const int *src = p.token_idx + (int64_t)pair * p.idx_stride;
        __syncthreads();
        for (int i = lane; i < seg_pos1 - seg_pos0; i += 64) s_idx[i] = min(max(src[seg_pos0 + i], 0), L - 1);
        __syncthreads();
#pragma unroll
        for (int j = 0; j + 1 < NBUF; ++j) load_step(buf[j], seg_t0 + j * TPS, seg_t1);
      }
      if constexpr (PAGED) {
        // the page ids of this segment's positions (at most kMaxSegPages)
        seg_page0 = seg_pos0 / p.page_tokens;
        const int npg = (seg_pos1 - 1) / p.page_tokens - seg_page0 + 1;
        const int *tbl = p.block_table + (int64_t)b * p.table_stride + seg_page0;
        __syncthreads();
        for (int i = lane; i < min(npg, kMaxSegPages); i += 64) s_pages[i] = max(tbl[i], 0);
        __syncthreads();
#pragma unroll
        for (int j = 0; j + 1 < NBUF; ++j) load_step(buf[j], seg_t0 + j * TPS, seg_t1);
      }
      const int nsteps = (seg_t1 - seg_t0 + TPS - 1) / TPS;
      const int steps = (nsteps + NBUF - 1) / NBUF * NBUF;
      const int next_t1 = seg_end_of(seg_t1);
      auto issue = [&](StepT &S, int s) {
        const bool in_seg = s < steps;
        const int tn = in_seg ? seg_t0 + s * TPS : seg_t1 + (s - steps) * TPS;
        const int lim = in_seg ? seg_t1 : (IDX || PAGED ? 0 : next_t1);
        load_step(S, tn < lim ? tn : seg_t0, tn < lim ? lim : 0);
      };
      if constexpr (StepT::PIPE) {
        // the raw scores of step s + 1 are started before step s's softmax
        // and P.V, so the score MFMAs' latency overlaps that work
        RawStep pend = qk_step(buf[0]);
        for (int i = 0; i < steps; i += NBUF) {
#pragma unroll
          for (int j = 0; j < NBUF; ++j) {
            issue(buf[(j + NBUF - 1) % NBUF], i + j + NBUF - 1);
            const RawStep nxt = qk_step(buf[(j + 1) % NBUF]);
            finish_step(buf[j], seg_t0 + (i + j) * TPS, pend);
            pend = nxt;
          }
        }
      } else {
        for (int i = 0; i < steps; i += NBUF) {
#pragma unroll
          for (int j = 0; j < NBUF; ++j) {
            issue(buf[(j + NBUF - 1) % NBUF], i + j + NBUF - 1);
            finish_step(buf[j], seg_t0 + (i + j) * TPS, qk_step(buf[j]));
          }
        }
      }

      // Partial of this segment, straight from registers, for each column
      // block.  Lane (col, cg) holds channels NB*(4*cg + i) + nb =
      // 4*NB*cg + NB*i + nb of its column.
      const int half = (seg_t0 == lane_t0 + chunk * ct) ? 0 : 1;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float lsum = rows_sum(l_run[cb]);
        if (qvalid[cb]) {
          const int slot = slot_base + 16 * cb + (2 * chunk + half) * p.G;
          const float out_scale = (KVT == ATTN_I8) ? p.v_scale : 1.0f;
          const float inv = lsum > 0.f ? out_scale / lsum : 0.f;
          float *op = p.wl.o_part + (int64_t)slot * D + 4 * NB * cg;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int n4 = 0; n4 < NB / 4; ++n4) {
              const f32x4_t v = {O[cb][4 * n4][i] * inv, O[cb][4 * n4 + 1][i] * inv, O[cb][4 * n4 + 2][i] * inv,
                                 O[cb][4 * n4 + 3][i] * inv};
              *(f32x4_t *)(op + NB * i + 4 * n4) = v;
            }
          if (cg == 0) {
            p.wl.m_part[slot] = lsum > 0.f ? m_run[cb] * kLn2 : NEG_INF;
            p.wl.l_part[slot] = lsum;
            if (half == 0 && seg_t1 == chunk_t1) {
              p.wl.m_part[slot + p.G] = NEG_INF;
              p.wl.l_part[slot + p.G] = 0.f;
            }
          }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[cb][nb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        m_run[cb] = NEG_INF;
        l_run[cb] = 0.f;
      }
      seg_t0 = seg_t1;
    }
    t = run_end;
    if (t < t_end) hit = next_lane(p, hit);
  }
}

}  // namespace

template <bool IDX, bool PAGED, int CB>
static void launch_variant(const DecodeParams &p, int kv_dtype, dim3 g, hipStream_t s) {
  dim3 blk(64);
  if (kv_dtype == ATTN_BF16) {
    if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_BF16, IDX, false, PAGED, CB>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_BF16, IDX, false, PAGED, CB>), g, blk, 0, s, p);
  } else if (p.q_quant == ATTN_QUANT_EXACT) {
    if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_I8, IDX, false, PAGED, CB>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_I8, IDX, false, PAGED, CB>), g, blk, 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_I8, IDX, true, PAGED, CB>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_I8, IDX, true, PAGED, CB>), g, blk, 0, s, p);
  }
}

template <bool IDX, bool PAGED>
static void launch_cb(const DecodeParams &p, int kv_dtype, dim3 g, hipStream_t s) {
  if (p.cols_per_wave == 32) launch_variant<IDX, PAGED, 2>(p, kv_dtype, g, s);
  else launch_variant<IDX, PAGED, 1>(p, kv_dtype, g, s);
}

hipError_t launch_decode_mfma(const DecodeParams &p, int kv_dtype, hipStream_t s) {
  if (p.token_idx) {
    if (p.split > kMaxIdxChunk || p.block_table) return hipErrorInvalidValue;
    launch_cb<true, false>(p, kv_dtype, dim3(p.grid), s);
  } else if (p.block_table) {
    if (p.split > 64 * p.page_tokens) return hipErrorInvalidValue;
    launch_cb<false, true>(p, kv_dtype, dim3(p.grid), s);
  } else {
    launch_cb<false, false>(p, kv_dtype, dim3(p.grid), s);
  }
  return hipGetLastError();
}

}  // namespace lcdg
