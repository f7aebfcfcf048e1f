// Split-KV GQA decode attention on gfx950 matrix cores (bf16 or int8 KV).
//
// A workgroup of one or four waves is one worker of a persistent grid.  The
// 32-token tiles of every (sequence b, KV head kh, column block) are laid end
// to end and each worker streams one balanced contiguous range of them, with
// its next tiles in flight in a register ring while it computes the current
// one:
//
//   S^T[t][g]  = K[t][:] . Q[g][:]            v_mfma_f32_16x16x32_{bf16,f16}
//   online softmax per query head g (running max m, sum l; exp2 domain)
//   O^T[d][g] += V^T[d][t] . P^T[t][g]        same MFMA, P fed as hi + lo
//
// This is the FlashAttention block recurrence with one query row per head
// ("注意力优化（Attention Optimization）", Flash Attention pseudo-code; NVIDIA
// blog "共同设计 AI 模型注意力…", BMM1 -> online softmax -> BMM2), and the
// G query heads of a KV head share every K/V byte that is loaded (GQA head
// sharing on the same pages).  A worker's result over its part of a lane is
// a partial (m, l, o), merged with the lane's other partials by the
// log-sum-exp rule inside the same launch ("优化稀疏注意力中的令牌丢弃机制" §5).
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
// Online softmax: a column's reference maximum is raised only when a tile's
// scores exceed it by more than this (log2 units), so most tiles skip the
// rescale of the accumulators (every tile of a 32-column wave would
// otherwise pay it, as some column's maximum rises in nearly every tile).
constexpr float kLazyRescale = 8.0f;

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
  static constexpr int NBUF = CB == 4 ? 3 : CB == 2 ? (KVT == ATTN_BF16 ? 4 : (TPS == 1 && !IDX ? 6 : 4))
                                      : (KVT == ATTN_BF16 ? 2 : (TPS == 1 && !IDX ? 4 : 3));
  static constexpr bool PIPE = KVT == ATTN_I8;
  TileT t[TPS];
};

// Positions of an indexed segment (its index list is staged in LDS).
constexpr int kMaxIdxChunk = 1024;
// Page ids a segment of the paged variant stages in LDS (a segment spans at
// most 512 pages of tokens, so at most 513 are touched).
constexpr int kMaxSegPages = 520;

// A workgroup of WPG waves is one worker.  The work-list lays every (b, kh)
// lane's tiles end to end; worker w streams one contiguous tile range of a
// static split (XCD-weighted when the work fills the grid, see
// stream_split), so the workers' shares do not depend on the mix of sequence
// lengths, with no atomics and no barriers in the loop.  A range is cut into runs, one per lane it touches.  The waves of
// a worker take a run's steps in turn (wave i: steps i, i + WPG, ...), so
// together they read one contiguous stream; at the run's end they combine
// their (m, l, O) through LDS (one wave keeps its own in registers).
//
// A run that covers its whole lane is the lane's result: it goes straight to
// out and lse.  Otherwise it is one partial of the lane, in the slot given by
// the worker's position among the lane's workers, and the merge runs inside
// the launch: each worker arrives on the counters of its shared lanes (at
// most its first and last) when its partial stores are complete, and the
// arrival that completes a lane's count folds the lane's partials into out
// and lse by the log-sum-exp rule ("优化稀疏注意力中的令牌丢弃机制" §5,
// cross-shard online softmax).  Partials are stored and loaded at device
// scope (they write through to memory every XCD reads), and the merge reads
// only after its arrival returned the lane's full count.
constexpr int kWPG = 4;  // waves per worker

template <int D, int KVT, bool IDX, bool QI8, bool PAGED, int CB, bool STREAM>
__global__ __launch_bounds__(64 * kWPG) __attribute__((amdgpu_waves_per_eu(CB >= 2 ? 1 : 2, CB >= 2 ? 1 : 2))) void
decode_mfma_kernel(DecodeParams p) {
  static_assert(!(IDX && PAGED), "a paged cache is read by position");
  static_assert(CB == 1 || CB == 2 || (CB == 4 && KVT == ATTN_BF16), "one, two or (bf16) four 16-column blocks per wave");
  static_assert(!(STREAM && IDX), "gathered kept rows use the default cache policy");
  // K/V cache policy: non-temporal where the launch streams the whole cache
  // over a full grid (STREAM, chosen by the host), the default otherwise
  constexpr int kKVPol = STREAM ? kStream : 0;
  constexpr int WPG = kWPG;
  typedef Tile<D, KVT, IDX> TileT;
  typedef Step<D, KVT, IDX, CB> StepT;
  constexpr int TPS = StepT::TPS;
  constexpr int NB = D / 16;
  constexpr int ES = TileT::ES;
  constexpr int KL = TileT::KL;
  constexpr int KB = D / 32;
  constexpr int VW = TileT::VW;
  constexpr int NT = 64 * WPG;     // threads of a worker
  constexpr int kCols = 16 * CB;   // matrix-core columns of a wave
  constexpr int NQ = D / 4;        // 16-byte slices of a row
  typedef typename std::conditional<KVT == ATTN_BF16, bf16x8_t, f16x8_t>::type OpT;

  __shared__ int s_idx[IDX ? kMaxIdxChunk : 1];
  __shared__ int s_pages[PAGED ? kMaxSegPages : 1];  // page ids of the current segment
  // Q^T operand of the current run, 16*CB query rows x D channels, rows padded
  // by 16 bytes against bank conflicts: bf16 for bf16 KV; for int8 KV three
  // int8 digit planes of each row's 22-bit fixed-point query (see below).
  constexpr int kQRow = D * 2 + 16;
  constexpr int kQDRow = D + 16;
  constexpr int kQBytes = CB * (KVT == ATTN_I8 ? 3 * 16 * kQDRow : 16 * kQRow);  // one column group
  constexpr int kGroups = CB == 2 ? 2 : 1;  // column groups a worker can hold
  __shared__ __attribute__((aligned(16))) unsigned char s_q[kGroups * kQBytes];
  __shared__ float s_qs[KVT == ATTN_I8 ? kGroups * kCols : 1];  // int8: each column's query scale
  // combination of the waves' states at a segment's end (WPG > 1)
  __shared__ float s_cm[WPG * kCols], s_cl[WPG * kCols];
  __shared__ f32x4_t s_co[WPG * kCols * NQ];
  __shared__ int s_last;
  // The lane table: each lane's positions and each sequence's clamped length
  // and offset, staged once at the start with one round of loads, so the
  // work split, the lane walk and every run's set-up read LDS instead of a
  // chain of dependent global loads (worth several microseconds before the
  // first tile's loads could issue).  Batches with more than NT lanes read
  // them from global memory instead.
  __shared__ int s_np[NT];
  __shared__ int s_len[NT];
  __shared__ int64_t s_off[NT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, cg = lane >> 4;
  // More than 32 query rows per KV head: the waves form p.ngb = 2 column
  // groups of 32 columns, and wave wi of each group takes the same steps, so
  // both groups use every K/V tile while it is fresh in this compute unit's
  // caches and the cache streams from HBM once.
  const int S = WPG / p.ngb;                 // waves per column group
  const int gi = wv / S, wi = wv - gi * S;   // this wave's group and its turn in the group
  const int g0 = gi * kCols;                 // the group's first column
  const float c1 = p.softmax_scale * kLog2e;
  const float NEG_INF = -__builtin_huge_valf();

  // out row orow, channels 4*sl .. 4*sl+3 (fp32 or bf16, rounded to nearest
  // even); element stores where out is not aligned for the vector store
  const uintptr_t out_addr = reinterpret_cast<uintptr_t>(p.out);
  const bool out_vec = out_addr % (p.out_dtype == ATTN_F32 ? 16 : 4) == 0;
  auto store_out4 = [&](int64_t orow, int sl, f32x4_t v) {
    if (p.out_dtype == ATTN_F32) {
      float *po = (float *)p.out + orow * D + 4 * sl;
      if (out_vec) {
        *(f32x4_t *)po = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) po[i] = v[i];
      }
    } else {
      uint16_t *po = (uint16_t *)p.out + orow * D + 4 * sl;
      if (out_vec) {
        ((uint32_t *)po)[0] = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
        ((uint32_t *)po)[1] = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) po[i] = (uint16_t)f32_to_bf16_bits(v[i]);
      }
    }
  };
  // a pair's partials: entries pe0 .. pe0 + ne - 1 (max_slots * G of them)
  auto o_rsrc = [&](int64_t pe0, int ne) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)(p.wl.o_part + pe0 * D), (short)0, ne * D * 4, 0x00020000);
  };
  auto m_rsrc = [&](int64_t pe0, int ne) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)(p.wl.m_part + pe0), (short)0, ne * 4, 0x00020000);
  };
  auto l_rsrc = [&](int64_t pe0, int ne) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)(p.wl.l_part + pe0), (short)0, ne * 4, 0x00020000);
  };

  const int nl = p.B * p.KH;
  const bool cached = nl <= NT;  // then B <= NT as well
  if (cached) {
    // thread i: lane i's positions, and sequence i's length and offset.  The
    // loads go to clamped indices without a branch, so all of them are in
    // flight together (one memory latency, not one per array).
    const int qi = min(tid, nl - 1), bi = min(tid, p.B - 1);
    const int lq = p.seq_lens[qi / p.KH], lb = p.seq_lens[bi];
    const int nq = IDX ? p.n_idx[qi] : 0;
    const int64_t off = PAGED ? 0 : p.seq_offset[bi];
    const int Lq = min(max(lq, 0), p.max_seq_len);
    const int np = IDX ? (Lq > 0 ? min(max(nq, 0), p.idx_stride) : 0) : Lq;
    s_np[tid] = tid < nl ? np : 0;
    s_len[tid] = tid < p.B ? min(max(lb, 0), p.max_seq_len) : 0;
    s_off[tid] = tid < p.B ? off : 0;
  }
  __syncthreads();
  // positions and tiles of lane (pair) q < nl
  auto lane_pos = [&](int q) -> int { return cached ? s_np[q] : pair_positions(p, q); };
  auto tiles_of = [&](int q) -> int { return (lane_pos(q) + 31) / 32; };
  const int T = wave_total_tiles_of(nl, tiles_of);
  // fixed_splits = S > 0: the unbalanced schedule, worker w = q*S + s takes
  // split s of lane q; otherwise the balanced split of the whole stream
  const int FS = p.fixed_splits;
  // The XCD weights offset a slowness of the odd XCDs that the default
  // cache policy shows; with non-temporal loads the XCDs stream alike (per
  // worker clocks: with the weights, the even XCDs ended 6% later, the
  // weights' own ratio), so a streaming launch splits equally.
  const StreamSplit split = stream_split(p, T, !STREAM);
  const int nworkers = FS > 0 ? p.B * p.KH * FS : split.W;
  if (wv == 0) {
    // No worker visits a lane without positions, so its rows get out = 0 and
    // lse = -inf here; lane qq belongs to
    // workgroup qq % gridDim.x.
    for (int base = 0; base < nl; base += 64) {
      const int qq = base + lane;
      unsigned long long m = __ballot(qq < nl && qq % (int)gridDim.x == (int)blockIdx.x && tiles_of(qq) == 0);
      while (m) {
        const int pz = base + __builtin_ctzll(m);
        m &= m - 1;
        const int bz = pz / p.KH, khz = pz - bz * p.KH;
        for (int u = lane; u < p.G * NQ; u += 64) {
          const int c = u / NQ, sl = u - c * NQ;
          const int64_t orow = q_row_index(p, bz, khz, c);
          store_out4(orow, sl, (f32x4_t){0.f, 0.f, 0.f, 0.f});
          if (sl == 0 && p.lse) p.lse[orow] = NEG_INF;
        }
      }
    }
  }
  if ((int)blockIdx.x >= nworkers) return;

  // lanes this worker shares with others, whose arrivals wait for its end
  int npend = 0, pend_q0 = 0, pend_need0 = 0, pend_q1 = 0, pend_need1 = 0;

  // Merge inside the launch.  Only a worker's first and last runs can share
  // their lane with other workers (every run between covers a whole lane).
  // Once this worker's partial stores are complete it arrives on those
  // lanes' counters; the arrival that completes a lane's count folds the
  // lane's slots 0 .. need-1 in slot order (online log-sum-exp) into out
  // and lse.
  auto arrive_and_merge = [&]() {
  if (npend > 0) {
    wait_vmem();
    __syncthreads();
    if (tid == 0) {
      int last = 0;
      // both adds in flight together, then resolved
      const uint64_t o0 = counter_add(p.wl.ctr + pend_q0);
      const uint64_t o1 = npend > 1 ? counter_add(p.wl.ctr + pend_q1) : 0;
      if (counter_resolve(p.wl.ctr + pend_q0, o0, p.wl.ctr_tag) == pend_need0) {
        counter_reset(p.wl.ctr + pend_q0, p.wl.ctr_tag);
        last |= 1;
      }
      if (npend > 1 && counter_resolve(p.wl.ctr + pend_q1, o1, p.wl.ctr_tag) == pend_need1) {
        counter_reset(p.wl.ctr + pend_q1, p.wl.ctr_tag);
        last |= 2;
      }
      s_last = last;
    }
    __syncthreads();
    const int last = s_last;
    for (int i = 0; i < npend; ++i) {
      if (!((last >> i) & 1)) continue;
      const int pm = i == 0 ? pend_q0 : pend_q1, nm = i == 0 ? pend_need0 : pend_need1;
      const int bm = pm / p.KH, khm = pm - bm * p.KH;
      const int64_t pe0 = (int64_t)pm * p.max_slots * p.G;
      const int pne = p.max_slots * p.G;
      const __amdgpu_buffer_rsrc_t ors = o_rsrc(pe0, pne), mrs = m_rsrc(pe0, pne), lrs = l_rsrc(pe0, pne);
      constexpr int U = 8;
      for (int u = tid; u < p.G * NQ; u += NT) {
        const int c = u / NQ, sl = u - c * NQ;
        float mt = NEG_INF, lt = 0.f;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < nm; k0 += U) {
          float mv[U], lv[U];
          f32x4_t ov[U];
#pragma unroll
          for (int k = 0; k < U; ++k) {
            const uint32_t e = (uint32_t)(min(k0 + k, nm - 1) * p.G + c);
            const float l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lrs, e * 4, 0, kDeviceScope));
            lv[k] = k0 + k < nm ? l : 0.f;
            mv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mrs, e * 4, 0, kDeviceScope));
            ov[k] = __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ors, (e * D + 4 * sl) * 4, 0, kDeviceScope));
          }
#pragma unroll
          for (int k = 0; k < U; ++k) {
            if (lv[k] > 0.f) {  // an empty partial (l = 0) may hold any o
              if (mv[k] > mt) {
                const float sc = expf(mt - mv[k]);
                acc *= sc;
                lt *= sc;
                mt = mv[k];
              }
              const float w = expf(mv[k] - mt) * lv[k];
              acc += w * ov[k];
              lt += w;
            }
          }
        }
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        const int64_t orow = q_row_index(p, bm, khm, c);
        store_out4(orow, sl, acc * inv);
        if (sl == 0 && p.lse) p.lse[orow] = lt > 0.f ? mt + logf(lt) : NEG_INF;
      }
    }
  }
  };

  // The worker's range; each lane it touches is one run.
  int t_begin, t_end, fs_need = 0, fs_slot = 0;
  if (FS > 0) {
    // split s of lane q: [t0 + s*n/S, t0 + (s+1)*n/S) of the lane's n tiles,
    // t0 = the tiles of the lanes before q; the lane's non-empty splits are
    // its partials, in split order
    const int q = (int)blockIdx.x / FS, sp = (int)blockIdx.x - q * FS;
    int acc = 0;
    for (int qq = lane; qq < q; qq += 64) acc += tiles_of(qq);
    const int t0 = uniform_i32(wave_sum_int(acc)), n = uniform_i32(q < nl ? tiles_of(q) : 0);
    t_begin = t0 + (int)((int64_t)sp * n / FS);
    t_end = t0 + (int)((int64_t)(sp + 1) * n / FS);
    fs_need = min(FS, n);
    fs_slot = n < FS ? t_begin - t0 : sp;
  } else {
    t_begin = range_start(blockIdx.x, T, split);
    t_end = range_start(blockIdx.x + 1, T, split);
  }
  // the lane (b, kh) holding the first tile of the range; each later run
  // takes the next lane that has tiles
  LaneHit hit = wave_find_lane_of(nl, t_begin, tiles_of);
  for (int t = t_begin; t < t_end;) {
    if (hit.nt == 0) break;  // lane walk exhausted (cannot happen for t < total)
    const int q = hit.q;
    const int lane_t0 = hit.t0, lane_t1 = hit.t0 + hit.nt;
    const int run_end = min(t_end, lane_t1);
    // workers holding part of this lane, and this worker's slot among them
    int need = fs_need, slot = fs_slot;
    if (FS == 0) {
      const int w_first = worker_of(lane_t0, T, split);
      need = worker_of(lane_t1 - 1, T, split) - w_first + 1;
      slot = (int)blockIdx.x - w_first;
    }
    const int pair = q;
    const int b = pair / p.KH, kh = pair - b * p.KH;
    const int L = uniform_i32(cached ? s_len[b] : min(max(p.seq_lens[b], 0), p.max_seq_len));
    int npos = L;
    if constexpr (IDX) npos = uniform_i32(lane_pos(pair));
    // this lane's column of block cb is query row g0 + 16*cb + col of the KV head
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
    const int64_t head_off = PAGED ? 0 : uniform_i64(cached ? s_off[b] : p.seq_offset[b]) + (int64_t)kh * p.stride_h;
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
    // Q (the 16 heads of this block, zero past G) is staged in LDS in MFMA
    // operand form; tiles read their B operand from there.  A global load
    // inside the segment loop would make the compiler wait for every load in
    // flight, the tile prefetch included.  The query's loads are issued here,
    // and stage_q turns them into the LDS operand once the first segment's
    // tile loads are in flight, so their latencies overlap.
    //
    // int8 KV: the scores run on the int8 matrix cores straight from the K
    // codes.  Head g's query becomes q = s_g * n with s_g = max|q_g| / 2^22
    // and n = rint(q / s_g) = 65536 d2 + 256 d1 + d0, d0, d1 in [-128, 127]
    // and |d2| <= 64 (|error| <= max|q_g| * 2^-23); each digit plane is one
    // int8 MFMA, and the three integer sums recombine exactly in fp32.  An
    // int8 query (QI8: per-row or static scale) is plane 0 alone.
    constexpr int CPL = D / 4;  // int8: lane (col, cg) takes column col, channels [cg*CPL, cg*CPL + CPL)
    constexpr int kQL = KVT == ATTN_I8 ? CB * (CPL / 8) : (kGroups * kCols * (D / 8) + NT - 1) / NT;
    const int nqe = p.ngb * kCols * (D / 8);  // bf16: 16-byte pieces of the worker's query rows
    u32x4_t qraw[kQL];
    if constexpr (KVT == ATTN_I8) {
      // the first wave of each column group loads the group's query
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint16_t *qrow = (const uint16_t *)p.q + q_row_index(p, b, kh, g0 + 16 * cb + col) * D + cg * CPL;
#pragma unroll
        for (int x = 0; x < CPL / 8; ++x) {
          u32x4_t w = (u32x4_t){0u, 0u, 0u, 0u};
          if (wi == 0 && qvalid[cb]) w = *(const u32x4_t *)(qrow + 8 * x);
          qraw[cb * (CPL / 8) + x] = w;
        }
      }
    } else {
      // every column group's rows: column gc of the pair at row gc (a group
      // is kCols rows, kQBytes bytes)
#pragma unroll
      for (int j = 0; j < kQL; ++j) {
        const int e = tid + j * NT, gc = e / (D / 8), c8 = e - gc * (D / 8);
        u32x4_t w = (u32x4_t){0u, 0u, 0u, 0u};
        if (e < nqe && gc < p.G) w = *(const u32x4_t *)((const uint16_t *)p.q + q_row_index(p, b, kh, gc) * D + 8 * c8);
        qraw[j] = w;
      }
    }
    float qs[CB];  // int8: this lane's column scale s_col in each block
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) qs[cb] = 0.f;
    auto stage_q = [&]() {
    if constexpr (KVT == ATTN_I8) {
      if (wi == 0) {  // the first wave of each column group stages the group's query
        unsigned char *sq_blk = s_q + gi * kQBytes;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb, sq_blk += 3 * 16 * kQDRow) {
          // channel j of this lane's CPL, decoded where it is used (few
          // registers: the first segment's tile loads are in flight)
          auto qval = [&](int j) -> float {
            const uint32_t w = qraw[cb * (CPL / 8) + (j >> 3)][(j >> 1) & 3];
            return (j & 1) ? bf16_hi(w) : bf16_lo(w);
          };
          float mx = 0.f;
#pragma unroll
          for (int j = 0; j < CPL; ++j) mx = fmaxf(mx, fabsf(qval(j)));
          mx = rows_max(mx);  // the four lanes of column col hold all D channels
          float sc;
          if constexpr (QI8) {
            // int8 query (one digit plane): s = max|q_row| / 127, or the static
            // scale, and code = clamp(rint(q / s), -127, 127), in IEEE fp32
            // (correctly rounded divides, round half to even).
            const float sq = p.q_quant == ATTN_QUANT_ROW ? mx / 127.0f : p.q_scale;
            sc = sq;
#pragma unroll
            for (int x = 0; x < CPL / 16; ++x) {
              uint32_t w[4];
#pragma unroll
              for (int j4 = 0; j4 < 4; ++j4) {
                uint32_t acc = 0u;
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                  float c = 0.f;
                  if (sq > 0.f) c = fminf(127.f, fmaxf(-127.f, __builtin_rintf(qval(16 * x + 4 * j4 + y) / sq)));
                  acc |= ((uint32_t)(int)c & 0xFFu) << (8 * y);
                }
                w[j4] = acc;
              }
              *(u32x4_t *)(sq_blk + col * kQDRow + cg * CPL + 16 * x) = (u32x4_t){w[0], w[1], w[2], w[3]};
            }
          } else {
            const float inv = mx > 0.f ? 4194304.0f / mx : 0.f;
            sc = mx * (1.0f / 4194304.0f);
#pragma unroll
            for (int x = 0; x < CPL / 16; ++x) {
              // channels 16x .. 16x+15: one 16-byte piece of each digit plane
              uint32_t dw[3][4];
#pragma unroll
              for (int j4 = 0; j4 < 4; ++j4) {
                uint32_t w0 = 0u, w1 = 0u, w2 = 0u;
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                  const int n = (int)__builtin_rintf(qval(16 * x + 4 * j4 + y) * inv);
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
                *(u32x4_t *)(sq_blk + (dg * 16 + col) * kQDRow + cg * CPL + 16 * x) =
                    (u32x4_t){dw[dg][0], dw[dg][1], dw[dg][2], dw[dg][3]};
            }
          }
          if (cg == 0) s_qs[g0 + 16 * cb + col] = sc;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kQL; ++j) {
        const int e = tid + j * NT, gc = e / (D / 8), c8 = e - gc * (D / 8);
        if (e < nqe) *(u32x4_t *)(s_q + gc * kQRow + 16 * c8) = qraw[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) qs[cb] = KVT == ATTN_I8 ? s_qs[g0 + 16 * cb + col] : 0.f;
    };
    const unsigned char *sq = s_q + gi * kQBytes;  // this wave's column group
    auto q_operand = [&](int cb, int kb) -> bf16x8_t {
      return __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)(sq + (16 * cb + col) * kQRow + 16 * (4 * kb + cg)));
    };
    // int8: digit plane dg of channels 64kb + 16cg .. + 15 of column col of block cb
    auto q_digits = [&](int cb, int dg, int kb) -> i32x4_t {
      return __builtin_bit_cast(i32x4_t,
                                *(const u32x4_t *)(sq + ((3 * cb + dg) * 16 + col) * kQDRow + 64 * kb + 16 * cg));
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
        for (int kl = 0; kl < KL; ++kl) R.k[tb][kl] = __builtin_amdgcn_raw_buffer_load_b128(tk, off + 64 * kl, 0, kKVPol);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int slot = (jj < 4) ? (4 * cg + jj) : (16 + 4 * cg + jj - 4);
        const uint32_t off = ((uint32_t)(row_of(tpos + slot) + rshift) * rs + col * VW * 4) | oob;
        if constexpr (VW == 4) R.v[jj] = __builtin_amdgcn_raw_buffer_load_b128(tv, off, 0, kKVPol);
        else if constexpr (VW == 2) R.v[jj] = __builtin_amdgcn_raw_buffer_load_b64(tv, off, 0, kKVPol);
        else R.v[jj] = __builtin_amdgcn_raw_buffer_load_b32(tv, off, 0, kKVPol);
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
      // a tile below every column's end needs no position mask (the first
      // query row, r = 0, ends first)
      const bool full = tpos + kTile <= min(seg_pos1, p.R > 1 ? L - (p.R - 1) : seg_pos1);
      OpT phi[CB], plo[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float s[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float sc = c1;
            if constexpr (KVT == ATTN_I8) sc *= qs[cb] * (IDX ? R.ks[4 * tb + i] : R.ks[tb]);
            s[4 * tb + i] = raw.v[cb][4 * tb + i] * sc;
          }
        if (!full) {
          const int lim = min(seg_pos1, col_end[cb]);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (tpos + 16 * tb + 4 * cg + i >= lim) s[4 * tb + i] = NEG_INF;
        }
        float mt = s[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mt = fmaxf(mt, s[i]);
        mt = rows_max(mt);
        // The reference m_run moves only when the tile's maximum exceeds it
        // by more than kLazyRescale (log2 units): the weights exp2(s - m_run)
        // then stay at most 2^kLazyRescale, and the final (m, l, O) are the
        // same quantities for any reference.  A column whose reference does
        // not move keeps alpha = 1 exactly, so each column's arithmetic is
        // independent of the other columns of the wave.
        const bool up = mt > m_run[cb] + kLazyRescale;
        if (__any(up)) {
          const float m_new = up ? mt : m_run[cb];
          // a column with no position seen yet (m_run = -inf) holds zeros;
          // the rescale must not form exp2(-inf - -inf)
          const float alpha = m_run[cb] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(m_run[cb] - m_new);
          l_run[cb] *= alpha;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) O[cb][nb] *= alpha;
          m_run[cb] = m_new;
        }
        const float mref = (m_run[cb] == NEG_INF) ? 0.f : m_run[cb];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // (a column past the group's rows has a zero query: its weights
          // are finite and its sums are never read)
          const float pv = __builtin_amdgcn_exp2f(s[i] - mref);
          l_run[cb] += pv;
          if constexpr (KVT == ATTN_BF16) {
            // round to nearest even; pairs of these conversions become one
            // v_cvt_pk_bf16_f32
            const __bf16 h = (__bf16)pv;
            phi[cb][i] = h;
            plo[cb][i] = (__bf16)(pv - (float)h);
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

    // Segments of the run: the loads of a segment's positions go through
    // LDS-staged index lists (IDX, at most kMaxIdxChunk positions) or page
    // ids (PAGED, at most 512 pages), so those runs are cut into segments at
    // lane-relative multiples of cs tiles; a plain run is one segment.  The
    // running state carries across segments.  Local step s of this wave in
    // a segment starting at tile s0 is the segment's step s*S + wi; the
    // NBUF register buffers rotate statically, a segment takes a multiple of
    // NBUF local steps (the last ones may be empty), and local step s is
    // loaded NBUF-1 steps before it is consumed.
    constexpr int NBUF = StepT::NBUF;
    StepT buf[NBUF];
    const int cs = IDX ? kMaxIdxChunk / kTile : PAGED ? 16 * p.page_tokens : 0x40000000;
    auto seg_end_of = [&](int s0) {
      return (int)min((int64_t)run_end, (int64_t)lane_t0 + ((int64_t)(s0 - lane_t0) / cs + 1) * cs);
    };
    auto tile_of = [&](int s0, int s) { return s0 + (s * S + wi) * TPS; };
    // Opens the segment starting at tile s0 (its index list or page ids
    // staged, the loads of its first NBUF-1 local steps issued) and returns
    // its end.  The run's first segment is opened before the query is staged
    // (whose loads are then in flight with the tiles'), so the query's
    // registers are free before the steps begin.
    auto open_segment = [&](int seg_t0) -> int {
      const int seg_t1 = seg_end_of(seg_t0);
      seg_pos0 = (seg_t0 - lane_t0) * kTile;
      seg_pos1 = min(npos, (seg_t1 - lane_t0) * kTile);
      if constexpr (IDX) {
        const int *src = p.token_idx + (int64_t)pair * p.idx_stride;
        __syncthreads();
        for (int i = tid; i < seg_pos1 - seg_pos0; i += NT) s_idx[i] = min(max(src[seg_pos0 + i], 0), L - 1);
        __syncthreads();
      }
      if constexpr (PAGED) {
        // the page ids of this segment's positions (at most kMaxSegPages)
        seg_page0 = seg_pos0 / p.page_tokens;
        const int npg = (seg_pos1 - 1) / p.page_tokens - seg_page0 + 1;
        const int *tbl = p.block_table + (int64_t)b * p.table_stride + seg_page0;
        __syncthreads();
        for (int i = tid; i < min(npg, kMaxSegPages); i += NT) s_pages[i] = max(tbl[i], 0);
        __syncthreads();
      }
#pragma unroll
      for (int j = 0; j + 1 < NBUF; ++j) load_step(buf[j], tile_of(seg_t0, j), seg_t1);
      return seg_t1;
    };
    int seg_t0 = t;  // t < run_end
    int seg_t1 = open_segment(seg_t0);
    stage_q();
    for (;;) {
      const int nsteps = (seg_t1 - seg_t0 + TPS - 1) / TPS;
      const int wsteps = (nsteps + S - 1) / S;  // local steps of the busiest wave
      const int steps = (wsteps + NBUF - 1) / NBUF * NBUF;
      auto issue = [&](StepT &S, int s) {
        const int tn = tile_of(seg_t0, s);
        load_step(S, tn < seg_t1 ? tn : seg_t0, tn < seg_t1 ? seg_t1 : 0);
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
            finish_step(buf[j], tile_of(seg_t0, i + j), pend);
            pend = nxt;
          }
        }
      } else {
        for (int i = 0; i < steps; i += NBUF) {
#pragma unroll
          for (int j = 0; j < NBUF; ++j) {
            issue(buf[(j + NBUF - 1) % NBUF], i + j + NBUF - 1);
            finish_step(buf[j], tile_of(seg_t0, i + j), qk_step(buf[j]));
          }
        }
      }
      seg_t0 = seg_t1;
      if (seg_t0 >= run_end) break;
      seg_t1 = open_segment(seg_t0);
    }

    // The run's result for each column.  Lane (col, cg) holds channels
    // NB*(4*cg + i) + nb = 4*NB*cg + NB*i + nb of its column, i.e. the 16-byte
    // slices NB*(4*cg + i)/4 + n4.  The waves of a column group combine
    // through LDS: M = max of their maxima, each wave's sum and output
    // rescaled by exp2(m_w - M) and added in wave order.  A worker that holds
    // the whole lane writes out and lse; otherwise the run's partial
    // (m, l, o) goes to slot `slot` of the lane: entry slot*G + gc of the pair
    // for column gc.
    const float out_scale = (KVT == ATTN_I8) ? p.v_scale : 1.0f;
    const bool direct = need == 1;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float lsum = rows_sum(l_run[cb]);
      if (cg == 0) {
        s_cm[wv * kCols + 16 * cb + col] = m_run[cb];
        s_cl[wv * kCols + 16 * cb + col] = lsum;
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float M = NEG_INF;
#pragma unroll
      for (int j = 0; j < WPG; ++j)
        if (j < S) M = fmaxf(M, s_cm[(gi * S + j) * kCols + 16 * cb + col]);
      const float alpha = m_run[cb] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(m_run[cb] - M);
      f32x4_t *dst = s_co + (wv * kCols + 16 * cb + col) * NQ;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n4 = 0; n4 < NB / 4; ++n4)
          dst[(NB * (4 * cg + i)) / 4 + n4] =
              (f32x4_t){O[cb][4 * n4][i], O[cb][4 * n4 + 1][i], O[cb][4 * n4 + 2][i], O[cb][4 * n4 + 3][i]} * alpha;
    }
    __syncthreads();
    {
      const int64_t pe0 = (int64_t)pair * p.max_slots * p.G;
      const int pne = p.max_slots * p.G;
      for (int u = tid; u < p.G * NQ; u += NT) {
        const int gc = u / NQ, sl = u - gc * NQ;
        const int gu = gc / kCols, c = gc - gu * kCols;  // column group and column within it
        float M = NEG_INF;
#pragma unroll
        for (int j = 0; j < WPG; ++j)
          if (j < S) M = fmaxf(M, s_cm[(gu * S + j) * kCols + c]);
        float lt = 0.f;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < WPG; ++j) {
          if (j < S) {
            const int w = gu * S + j;
            const float mw = s_cm[w * kCols + c];
            lt += mw == NEG_INF ? 0.f : s_cl[w * kCols + c] * __builtin_amdgcn_exp2f(mw - M);
            acc += s_co[(w * kCols + c) * NQ + sl];
          }
        }
        const float inv = lt > 0.f ? out_scale / lt : 0.f;
        const f32x4_t o = acc * inv;
        if (direct) {
          const int64_t orow = q_row_index(p, b, kh, gc);
          store_out4(orow, sl, o);
          if (sl == 0 && p.lse) p.lse[orow] = lt > 0.f ? M * kLn2 + logf(lt) : NEG_INF;
        } else {
          const uint32_t e = (uint32_t)(slot * p.G + gc);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), o_rsrc(pe0, pne),
                                                 (e * D + 4 * sl) * 4, 0, kDeviceScope);
          if (sl == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lt > 0.f ? M * kLn2 : NEG_INF), m_rsrc(pe0, pne),
                                                  e * 4, 0, kDeviceScope);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lt), l_rsrc(pe0, pne), e * 4, 0, kDeviceScope);
          }
        }
      }
    }
    __syncthreads();  // the combine buffers are free again
    if (!direct) {
      if (npend == 0) {
        pend_q0 = q;
        pend_need0 = need;
      } else {
        pend_q1 = q;
        pend_need1 = need;
      }
      ++npend;
    }
    t = run_end;
    if (t < t_end) hit = next_lane_of(nl, hit, tiles_of);
  }
  arrive_and_merge();
}

}  // namespace

template <bool IDX, bool PAGED, int CB, bool STREAM>
static void launch_variant(const DecodeParams &p, int kv_dtype, dim3 g, hipStream_t s) {
  dim3 blk(64 * kWPG);
  if (kv_dtype == ATTN_BF16) {
    if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_BF16, IDX, false, PAGED, CB, STREAM>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_BF16, IDX, false, PAGED, CB, STREAM>), g, blk, 0, s, p);
  } else if (p.q_quant == ATTN_QUANT_EXACT) {
    if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_I8, IDX, false, PAGED, CB, STREAM>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_I8, IDX, false, PAGED, CB, STREAM>), g, blk, 0, s, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_I8, IDX, true, PAGED, CB, STREAM>), g, blk, 0, s, p);
    else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_I8, IDX, true, PAGED, CB, STREAM>), g, blk, 0, s, p);
  }
}

template <bool IDX, bool PAGED>
static void launch_cb(const DecodeParams &p, int kv_dtype, dim3 g, hipStream_t s) {
  if constexpr (!IDX) {
    if (p.stream_nt) {
      if (p.cols_per_wave == 32) launch_variant<IDX, PAGED, 2, true>(p, kv_dtype, g, s);
      else launch_variant<IDX, PAGED, 1, true>(p, kv_dtype, g, s);
      return;
    }
  }
  if (p.cols_per_wave == 32) launch_variant<IDX, PAGED, 2, false>(p, kv_dtype, g, s);
  else launch_variant<IDX, PAGED, 1, false>(p, kv_dtype, g, s);
}

// 64 columns per wave: bf16 caches read by position only (the host routes
// nothing else here)
template <bool PAGED, bool STREAM>
static void launch_cb4(const DecodeParams &p, dim3 g, hipStream_t s) {
  dim3 blk(64 * kWPG);
  if (p.D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, ATTN_BF16, false, false, PAGED, 4, STREAM>), g, blk, 0, s, p);
  else hipLaunchKernelGGL((decode_mfma_kernel<64, ATTN_BF16, false, false, PAGED, 4, STREAM>), g, blk, 0, s, p);
}

hipError_t launch_decode_mfma(const DecodeParams &p, int kv_dtype, hipStream_t s) {
  if (p.wpg != kWPG) return hipErrorInvalidValue;
  if (p.ngb < 1 || p.ngb > (p.cols_per_wave == 32 ? 2 : 1)) return hipErrorInvalidValue;
  if (!p.wl.ctr || p.max_slots < 1) return hipErrorInvalidValue;
  if (p.cols_per_wave == 64) {
    if (kv_dtype != ATTN_BF16 || p.token_idx) return hipErrorInvalidValue;
    if (p.block_table) {
      if (p.stream_nt) launch_cb4<true, true>(p, dim3(p.grid), s);
      else launch_cb4<true, false>(p, dim3(p.grid), s);
    } else {
      if (p.stream_nt) launch_cb4<false, true>(p, dim3(p.grid), s);
      else launch_cb4<false, false>(p, dim3(p.grid), s);
    }
    return hipGetLastError();
  }
  if (p.token_idx) {
    if (p.block_table) return hipErrorInvalidValue;
    launch_cb<true, false>(p, kv_dtype, dim3(p.grid), s);
  } else if (p.block_table) {
    launch_cb<false, true>(p, kv_dtype, dim3(p.grid), s);
  } else {
    launch_cb<false, false>(p, kv_dtype, dim3(p.grid), s);
  }
  return hipGetLastError();
}

}  // namespace lcdg
