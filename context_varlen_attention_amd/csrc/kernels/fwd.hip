// Forward attention kernels for gfx950.
//
// What is computed (DCP paper, background: block-wise masked attention with the
// online-softmax trick; MindSpeed RFC section 3.1: both local Q chunks of every
// sub-sequence in one fused call against their causal K/V prefix selected from
// the rank-major gathered K/V by a direct index):
//
//   for every scheduled (Q tile, head) and every non-empty K/V tile of its
//   segment, in order:  S = scale * Q K^T (fp32), masked on partial tiles,
//   m' = max(m, rowmax S), P = exp(S - m'), l = l e^(m-m') + rowsum P,
//   O = O e^(m-m') + P V;  finally O /= l, LSE = m + ln l.
//
// MFMA formulation.  A work-group is 8 waves in two groups of four that run the
// same steps one phase apart (below); each wave owns 32 query rows of one
// head.  The kernel computes the transposed scores S^T = K Q^T with
// v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q from registers), so every lane
// ends up holding 16 keys of ONE query column: the softmax statistics are
// lane-local, plus one v_permlane32_swap with the other half-wave.  The output
// is kept transposed too, O^T = V^T P^T, with P^T taken straight from the S^T
// accumulators (the MFMA's reduction slots are permuted to match the layout the
// accumulators already have) and the V^T operand read from row-major V tiles
// with the transposing LDS read ds_read_b64_tr_b16.
//
// Per K/V tile the vector ALU does only what the softmax needs:
//   * Q is pre-multiplied by scale*log2(e) when it is loaded, and the first
//     MFMA of every S^T chain takes a register block holding -base (the row's
//     exponent base) as its accumulator input, so P = exp2(acc) with no extra
//     arithmetic and no per-tile initialisation;
//   * P = exp2(acc) is formed at once; the row maximum (v_max3) is computed and
//     the base moved only when some P of the tile may exceed 2^8 (the sum of a
//     lane's P values exceeds 2^8) or the row has no base yet (lazy rescaling),
//     so both the maximum and the O rescale are rare;
//   * P is packed to 16 bits with v_cvt_pk; the row sum adds the fp32 P values
//     (at softmax scales beyond 1.5x the default, and at Q/K head dim 192, it
//     adds the packed values the PV MFMA consumes instead, unpacked with
//     integer operations -- v_dot2 would do that in one instruction, but it
//     issues many times slower while the other wave of the SIMD runs MFMAs);
//   * masking is a separate code path taken only on partial tiles.
// K/V rows are gathered through the prefix index straight into LDS with
// global_load_lds_dwordx4 (the index_select of the RFC, never materialised)
// through a 4-stage ring (3 at Q/K head dim 192), the tiles' indices fetched
// 2 x 4 tiles ahead.
//
// Attention dropout (MindSpeed RFC section 3.5.2.2) is a second instantiation
// of the per-item kernel: Q stays unscaled (the vector step forms
// S * scale * log2(e) - base with one fma per score), the row sum is that of the
// undropped P, the packed P is ANDed with the keep mask of the tile (bytes of
// Philox4x32-10 outputs, one generator call per 4 x 4 block of (query, key)
// positions, shared by the four lanes of a quad) and 1/l carries the
// 256 / (256 - t) scale of the kept values.
#include <cmath>
#include <type_traits>

#include "../host/plan.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace cva {

namespace {

constexpr int kThreads = 512;              // 8 waves: two ping-pong groups of 4
constexpr int kBN = 64;                    // keys per K/V tile
// lazy rescaling: the exponent base may lag the row maximum by up to 8 (log2
// units), i.e. a P value may reach 2^8 before the base moves
constexpr float kRescaleLimit = 256.0f;
constexpr int kReadAhead = 6;              // MFMAs between an LDS operand read and its use
constexpr int kXReadAhead = 3;             // MFMA pairs between an operand read and its use (Dqk == Dv)

// LDS layouts (16-byte chunks, XOR-swizzled so that the MFMA operand reads are
// bank-conflict free on gfx950's 64 x 4-byte-bank LDS, as measured with the
// SQ_LDS_BANK_CONFLICT counter):
//   K: row r, logical chunk c at physical chunk c ^ k_swz(r); read with
//      ds_read_b128, 32 consecutive rows per instruction (16 rows per pass).
//      Rows of 256 bytes start on the same bank, so the XOR takes r & 15; rows
//      of 128 or 384 bytes alternate bank halves, so it takes (r >> 1) & 7.
//   V: row r, logical 32-byte group G at physical group G ^ f(r) with
//      f(r) = (r & 3) ^ ((r & 1) << 2) for rows of 8+ groups (else r & 3); read
//      with ds_read_b64_tr_b16, which takes 4 consecutive rows x 32 bytes per
//      16 lanes.
template <int DQK>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (DQK == 128)
    return r & 15;
  else
    return (r >> 1) & 7;
}
// Per-lane K read offsets kept live: the swizzle permutes chunks inside aligned
// groups of 2*kKoff chunks.
template <int DQK>
constexpr int kKoff = (DQK == 128) ? 8 : 4;

template <int VCH>
__device__ __forceinline__ int v_swz(int r) {  // XOR applied to the 16-byte chunk index
  if constexpr (VCH >= 16)
    return 2 * ((r & 3) ^ ((r & 1) << 2));
  else
    return 2 * (r & 3);
}

constexpr int kMaxSpans = kFwdMaxSpans;  // spans per forward work item (checked by the plan builder)

// Cursor over the tiles of a work item: the spans' [t0, t1) ranges, in order.
// The span table sits in LDS (sp) so that advancing is a short, uniform read.
struct TileCursor {
  int sp, t, t_end, partial;
};

__device__ __forceinline__ TileCursor span_start(const int32_t* sp_tab, int sp) {
  const int4 r = *(const int4*)(sp_tab + 4 * sp);
  return TileCursor{sp, __builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                    __builtin_amdgcn_readfirstlane(r.z)};
}

__device__ __forceinline__ TileCursor next_tile(TileCursor c, const int32_t* sp_tab, int nspan) {
  ++c.t;
  if (c.t >= c.t_end) {
    ++c.sp;
    if (c.sp < nspan) c = span_start(sp_tab, c.sp);
  }
  return c;
}


template <int DQK, int DV, int NT>
struct TileLoader {
  static constexpr int kThreads = NT;              // threads that issue the tile loads
  static constexpr int KCH = DQK / 8, VCH = DV / 8;
  static constexpr int KN = kBN * KCH / kThreads;  // K slots per thread
  static constexpr int VN = kBN * VCH / kThreads;  // V slots per thread
  static constexpr bool kShared = (KCH == VCH);    // K and V slots cover the same rows
  static constexpr int NIDX = kShared ? KN : KN + VN;
  static_assert(kBN * KCH % kThreads == 0 && kBN * VCH % kThreads == 0, "tile / thread mismatch");

  __device__ static int krow(int i, int tid) { return (i * kThreads + tid) / KCH; }
  __device__ static int vrow(int i, int tid) { return (i * kThreads + tid) / VCH; }
  // byte offset of this thread's 16-byte chunk inside its row (swizzled position)
  __device__ static uint32_t kchunk(int i, int tid) {
    const int s = i * kThreads + tid;
    return (uint32_t)(((s % KCH) ^ k_swz<DQK>(s / KCH)) * 16);
  }
  __device__ static uint32_t vchunk(int i, int tid) {
    const int s = i * kThreads + tid;
    return (uint32_t)(((s % VCH) ^ v_swz<VCH>(s / VCH)) * 16);
  }

  // Prefix-index entries of the rows this thread loads (clamped into the prefix:
  // rows past it re-read the last key, which is masked).
  __device__ static void fetch_index(int (&idx)[NIDX], const int32_t* __restrict__ kvi, int kb0,
                                     int kv_len, int tid) {
#pragma unroll
    for (int i = 0; i < KN; ++i) idx[i] = kvi[min(kb0 + krow(i, tid), kv_len - 1)];
    if constexpr (!kShared) {
#pragma unroll
      for (int i = 0; i < VN; ++i) idx[KN + i] = kvi[min(kb0 + vrow(i, tid), kv_len - 1)];
    }
  }

  // The same entries, read from a tile's 64-entry index slot in LDS.
  __device__ static void read_index(int (&idx)[NIDX], const int32_t* sidx, int tid) {
#pragma unroll
    for (int i = 0; i < KN; ++i) idx[i] = sidx[krow(i, tid)];
    if constexpr (!kShared) {
#pragma unroll
      for (int i = 0; i < VN; ++i) idx[KN + i] = sidx[vrow(i, tid)];
    }
  }

  // Issue the direct-to-LDS loads of one K tile / one V tile.  kg / vg point at
  // the K/V head's first element; strides are bytes between gathered rows.
  // wave_off is the wave's first slot (uniform), so the LDS base is scalar.
  __device__ static void issue_k(uint16_t* sk, const char* kg, const int (&idx)[NIDX],
                                 uint32_t kstride, int tid, int wave_off) {
    const uint32_t kl = lds_addr(sk) + (uint32_t)wave_off * 16;
#pragma unroll
    for (int i = 0; i < KN; ++i)
      dma16(kg + ((uint64_t)(uint32_t)idx[i] * kstride + kchunk(i, tid)), kl + i * kThreads * 16);
  }
  __device__ static void issue_v(uint16_t* sv, const char* vg, const int (&idx)[NIDX],
                                 uint32_t vstride, int tid, int wave_off) {
    const uint32_t vl = lds_addr(sv) + (uint32_t)wave_off * 16;
#pragma unroll
    for (int i = 0; i < VN; ++i) {
      const int id = kShared ? idx[i] : idx[KN + i];
      dma16(vg + ((uint64_t)(uint32_t)id * vstride + vchunk(i, tid)), vl + i * kThreads * 16);
    }
  }
};

// Per-lane LDS byte offsets of the MFMA operand reads, relative to a tile buffer.
// The swizzles only permute 16-byte chunks inside aligned groups, so every read
// of a tile is one of a few per-lane offsets plus a compile-time constant.
//
// K (S^T A operand): step kt of 32-key block nb reads logical chunk 2kt + half of
// row nb*32 + col, i.e. byte  koff[kt % KO] + 32*KO*(kt / KO) + nb*32*rowbytes
// with KO = kKoff<DQK>.
template <int DQK>
__device__ __forceinline__ void k_offsets(uint32_t (&koff)[kKoff<DQK>], int col, int half) {
  const int sw = k_swz<DQK>(col);  // rows nb*32 + col share the swizzle of row col
#pragma unroll
  for (int u = 0; u < kKoff<DQK>; ++u)
    koff[u] = (uint32_t)(col * DQK * 2 + 16 * ((2 * u + half) ^ sw));
}

// V (PV A operand, transposing read): lane (s = lane & 15, g = lane >> 4) reads
// 8 bytes of row key0 + 4*half + (s >> 2) at logical column 32*blk + 16*(g&1) +
// 4*(s&3); for key0 a multiple of 8 the row's swizzle depends on the lane only,
// so the read is at  voff[blk] + key0*rowbytes.
template <int DV>
__device__ __forceinline__ void v_offsets(uint32_t (&voff)[DV / 32], int lane) {
  constexpr int VCH = DV / 8;
  const int s = lane & 15, g = lane >> 4;
  const int r = 4 * (g >> 1) + (s >> 2);  // row relative to key0 (half = g >> 1)
  const int sw = v_swz<VCH>(r);
#pragma unroll
  for (int blk = 0; blk < DV / 32; ++blk) {
    const int col = blk * 32 + 16 * (g & 1) + 4 * (s & 3);
    const int c = (col >> 3) ^ sw;
    voff[blk] = (uint32_t)(r * DV * 2 + c * 16 + (col & 7) * 2);
  }
}

__device__ __forceinline__ u32x4_t lds_read128(const uint16_t* base, uint32_t off) {
  return *(const u32x4_t*)((const char*)base + off);
}

__device__ __forceinline__ u32x2_t lds_read_tr(const uint16_t* base, uint32_t off) {
  return lds_read_tr16((const uint16_t*)((const char*)base + off));
}

__device__ __forceinline__ float wave_half_max(float x) {
  // max with the value the lane 32 apart holds
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float wave_half_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Per-lane state of the online softmax: exponent base (log2 units, shared by the
// two half-waves holding the same query), running sum and the O^T accumulators.
template <int DB>
struct SoftmaxState {
  float base, l;
  f32x16_t acc[DB];
};

// S^T = K (scaled Q)^T - base for the 64 keys of a tile (two 32-key blocks); the
// first MFMA of each chain takes its accumulator input from nbase (-base in every
// entry), so the scores never need initialising.
// (kFromBase = false: the chains start from s, which holds -base already.)
template <typename E, int DQK, bool kFromBase>
__device__ __forceinline__ void tile_scores(f32x16_t (&s)[2], const typename E::vec8 (&qf)[DQK / 16],
                                            const uint16_t* sk, const uint32_t (&koff)[kKoff<DQK>],
                                            const f32x16_t& nbase) {
  constexpr int KSTEPS = DQK / 16;
  constexpr int KO = kKoff<DQK>;
#pragma unroll
  for (int kt = 0; kt < KSTEPS; ++kt) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const u32x4_t x = lds_read128(sk + nb * 32 * DQK + (kt / KO) * 16 * KO, koff[kt % KO]);
      s[nb] = E::mfma32(as_vec8<E>(x), qf[kt], (kFromBase && kt == 0) ? nbase : s[nb]);
    }
  }
}

// Bits [a, b) of a 64-bit word (either end may lie outside [0, 64)).
__device__ __forceinline__ uint64_t range_bits64(int a, int b) {
  a = max(a, 0);
  b = min(b, 64);
  const uint64_t below_b = b >= 64 ? ~0ull : (b <= 0 ? 0ull : (1ull << b) - 1);
  const uint64_t below_a = a >= 64 ? ~0ull : (1ull << a) - 1;
  return below_b & ~below_a;
}

// Element-wise mask of a partial tile: lane (query column, half) holds keys
// kb0 + 32*nb + 8*(r/4) + 4*half + r%4; visible iff inside [lo1,hi1) or [lo2,hi2).
// The lane's visible keys of the tile become one 64-bit word; each score then
// takes two operations: its bit, sign-extended to a full word, selects between
// the score's bits and those of -inf.
__device__ __forceinline__ void tile_mask(f32x16_t (&s)[2], int kb0, int half, int lo1, int hi1,
                                          int lo2, int hi2) {
  const uint64_t m = (range_bits64(lo1 - kb0, hi1 - kb0) | range_bits64(lo2 - kb0, hi2 - kb0)) >> (4 * half);
  const uint32_t w[2] = {(uint32_t)m, (uint32_t)(m >> 32)};
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)w[nb], 8 * (r >> 2) + (r & 3), 1);
      const uint32_t x = __float_as_uint(s[nb][r]);
      s[nb][r] = __uint_as_float((x & keep) | (0xFF800000u & ~keep));
    }
  }
}

// Row max of a tile's scores relative to the base, both half-waves combined.
__device__ __forceinline__ float tile_max(const f32x16_t (&s)[2]) {
  float mx = -INFINITY;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(s[nb][r], s[nb][r + 1]));
  return wave_half_max(mx);
}

// P = exp2(S^T) for the 32 scores a lane holds, packed to 16 bits as the PV
// MFMA's operand; returns the lane's share of the row sum, in fp32, of exactly
// the rounded values the MFMA consumes (unpacked again with integer
// operations), so that O's weights sum to one and LSE matches them (EXACT:
// of the unrounded values instead, the softmax's own normaliser).  NPART
// partial sums shorten the dependent chain of adds (fewer save registers).
template <typename E, int NPART, bool EXACT = false>
__device__ __forceinline__ float exp_pack_tile(u32x4_t (&pk)[2][2], const f32x16_t (&s)[2]) {
  float part[NPART];
#pragma unroll
  for (int i = 0; i < NPART; ++i) part[i] = 0.f;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 8 * ks + 2 * j;
        const float e0 = __builtin_amdgcn_exp2f(s[nb][r]), e1 = __builtin_amdgcn_exp2f(s[nb][r + 1]);
        const uint32_t w = pack2<E>(e0, e1);
        pk[nb][ks][j] = w;
        if constexpr (EXACT) part[j % NPART] += e0 + e1;
        else part[j % NPART] += E::to_float((uint16_t)(w & 0xFFFFu)) + E::to_float((uint16_t)(w >> 16));
      }
  float l = part[0];
#pragma unroll
  for (int i = 1; i < NPART; ++i) l += part[i];
  return l;
}

// Forward work-group: 8 waves in two groups of 4 (group g = wave / 4; waves w and
// w + 4 share a SIMD).  Each wave owns 32 query rows of one head.  Both groups
// run the same sequence of steps, group 1 one phase behind group 0:
//     X(-1) = S(0), Y(0), X(0), Y(1), X(1), ..., Y(N-1), X(N-1)
// where X(n) = MFMA work (O += V(n)^T P(n), then the scores S(n+1) of the next
// tile) and Y(n) = vector work (mask, max, lazy rescale, P(n) = exp2 S(n), row
// sums).  A barrier ends every phase, so on every SIMD one wave is in an MFMA
// step while the other is in a vector step.
//
// The tiles stream through an NS-deep LDS ring, K(n+NS) into the slot K(n)
// used and V(n+NS-1) into the slot of V(n-1), with the prefix indices of tile
// n+2NS fetched into a small index ring; NS-2 batches stay in flight across
// every barrier.  When Dqk == Dv each group streams one operand inside its own
// MFMA steps (group 0 K, group 1 V, one load after every fourth MFMA pair of
// X(n)); group 0's first wave fetches the indices (for all eight waves, which
// read them after a barrier) and group 0 waits for K(n+2) at the end of
// Y(n+1), group 1 for V(n+1) at the end of X(n).  Otherwise group 0 streams both: K
// and the indices at the start of X(n), V after Y(n+1), then its wait.
template <int DQK>
constexpr int kStages = DQK > 128 ? 3 : 4;

template <typename E, int DQK, int DV, bool DROP, bool EXACT_SUM>
__global__ __launch_bounds__(kThreads, 1) void fwd_mfma_kernel(FwdParams P) {
  using TL = TileLoader<DQK, DV, kThreads / 2>;
  constexpr int KSTEPS = DQK / 16;  // 16-wide reduction steps of S^T
  constexpr int DB = DV / 32;       // 32-row blocks of O^T
  constexpr int NI = TL::NIDX;
  constexpr int NS = kStages<DQK>;
  constexpr int NIR = 2 * NS;       // index ring slots
  constexpr uint32_t KBUF = kBN * DQK * 2, VBUF = kBN * DV * 2;  // bytes per tile buffer
  // Dqk == Dv: each group streams one operand, its loads spread over its own
  // MFMA steps (group 0 K and the index ring, group 1 V); otherwise group 0
  // streams both in bursts
  constexpr bool kSpread = DQK == DV;
  __shared__ __attribute__((aligned(16))) uint16_t sK[NS][kBN * DQK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NS][kBN * DV];
  __shared__ __attribute__((aligned(16))) int32_t sIdx[NIR][kBN];
  __shared__ __attribute__((aligned(16))) int32_t sSpan[kMaxSpans * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, w4 = wave & 3;
  const int col = lane & 31, half = lane >> 5;
  const int ltid = w4 * 64 + lane;  // thread index inside the group

  const int tile = blockIdx.x / P.n_head_groups;
  const int hg = blockIdx.x % P.n_head_groups;
  const int32_t* tr = P.t.fwd_tiles + tile * 5;
  const int seg = tr[0], q0 = tr[1], rows = tr[2], span0 = tr[3], nspan = tr[4];
  const int32_t* sg = P.t.segs + seg * 8;
  const int kv_len = sg[3], q_row0 = sg[4], kv_off = sg[5];
  const int hpt = P.heads_per_tile;
  const int head = hg * hpt + (w4 % hpt);
  const int kvh = head / P.group;
  const int rowblk = w4 / hpt + grp * (4 / hpt);
  const int a = q0 + rowblk * 32 + col;  // segment-relative query index of this lane
  const int split_slot = P.slot != nullptr ? P.slot[tile] : -1;  // piece of a split K/V range
  const bool valid = a < q0 + rows;       // the tile's own rows (a tile may end inside its segment)
  const int row = q_row0 + a;             // local row
  [[maybe_unused]] const int seq = sg[0], qpos = sg[6] + a;  // sequence, in-sequence query position (dropout)

  const char* kg = (const char*)P.k + (int64_t)kvh * DQK * 2;
  const char* vg = (const char*)P.v + (int64_t)kvh * DV * 2;
  const uint32_t kstride = (uint32_t)P.hkv * DQK * 2, vstride = (uint32_t)P.hkv * DV * 2;
  const int32_t* __restrict__ kvi = P.t.kv_index + kv_off;

  if (nspan == 0) {  // no visible key for any row of the tile (unreachable for the supported masks)
    if (valid) {
      uint16_t* orow = (uint16_t*)P.o + ((int64_t)row * P.hq + head) * DV;
      for (int d = half; d < DV; d += 2) orow[d] = 0;
      if (half == 0) P.lse[(int64_t)head * P.t_loc + row] = -INFINITY;
    }
    return;
  }
  // The span table, then Q and the row intervals (they need only the tile
  // record and the segment), so that their latencies overlap: the wait before
  // the span table's LDS store leaves the later loads in flight.
  // (Lanes past the tile's rows load its first row, so that no load sits in a
  // branch, and drop the values below.)
  const int32_t span_w = P.t.fwd_spans[span0 * 4 + min(tid, 4 * nspan - 1)];
  __builtin_amdgcn_sched_barrier(0);  // the span load goes out first
  const int64_t lrow = valid ? (int64_t)row : (int64_t)(q_row0 + q0);
  u32x4_t qraw[KSTEPS];
  {
    const uint16_t* qrow = (const uint16_t*)P.q + (lrow * P.hq + head) * DQK + 8 * half;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) qraw[t] = *(const u32x4_t*)(qrow + 16 * t);
  }
  const int4 ivr = *(const int4*)(P.t.row_iv + lrow * 4);
  if (tid < 4 * nspan) sSpan[tid] = span_w;
  __syncthreads();
  int n_tiles = 0;
  for (int sp = 0; sp < nspan; ++sp) {
    const TileCursor c = span_start(sSpan, sp);
    n_tiles += c.t_end - c.t;
  }

  // ---- tile streaming (group 0) ----
  // batch(n), n >= -NS: K(n+NS), V(n+NS-1), indices of tile n+2NS-1 (each if it exists)
  TileCursor cI = span_start(sSpan, 0);  // next tile whose indices get fetched
  int next_idx = 0;                      // its number
  int bcount[NS];                        // loads per wave of the last batches (ring by n mod NS)
#pragma unroll
  for (int i = 0; i < NS; ++i) bcount[i] = 0;
  auto fetch_idx = [&]() {  // indices of tile next_idx into ring slot next_idx % NIR
    const int kb0 = cI.t * kBN;
    dma4(kvi + min(kb0 + lane, kv_len - 1), lds_addr(sIdx[next_idx % NIR]));
    ++next_idx;
    cI = next_tile(cI, sSpan, nspan);
  };
  // Indices of batch n's K and V tiles, read from the index ring ahead of the
  // batch (in the vector step before it) so that the loads issue at once.
  int idxK[NI], idxV[NI];
  auto prepare_batch = [&](int n) {
    const int mk = n + NS, mv = n + NS - 1;
    if (mk >= 0 && mk < n_tiles) TL::read_index(idxK, sIdx[mk % NIR], ltid);
    if (mv >= 0 && mv < n_tiles) TL::read_index(idxV, sIdx[mv % NIR], ltid);
  };
  // With a 4-deep ring a batch goes out in two parts: K and the indices at the
  // start of the MFMA step, V after the vector step (where the streaming group
  // has slack), so that neither step carries the whole issue cost.  With a
  // 3-deep ring V needs the earlier start and the batch goes out whole.
  constexpr bool kSplitIssue = NS >= 4;
  auto issue_k_part = [&](int n) {
    int cnt = 0;
    const int mk = n + NS, mi = n + 2 * NS;
    if (mk >= 0 && mk < n_tiles) {
      TL::issue_k(sK[mk % NS], kg, idxK, kstride, ltid, w4 * 64);
      cnt += TL::KN;
    }
    if (mi >= 2 * NS && mi < n_tiles) {  // earlier tiles' indices come with the prologue
      fetch_idx();
      cnt += 1;
    }
    bcount[(n + NS) % NS] = cnt;
  };
  auto issue_v_part = [&](int n) {
    const int mv = n + NS - 1;
    if (mv >= 0 && mv < n_tiles) {
      TL::issue_v(sV[mv % NS], vg, idxV, vstride, ltid, w4 * 64);
      bcount[(n + NS) % NS] += TL::VN;
    }
  };
  auto issue_batch = [&](int n) {
    issue_k_part(n);
    issue_v_part(n);
  };
  // after this, the loads needed by X(n+1) (batch n+2-NS) have landed
  auto wait_batch = [&](int n) {
    int allowed = 0;
#pragma unroll
    for (int b = 0; b < NS - 2; ++b) allowed += bcount[(n - b + NS) % NS];
    wait_vmem_le(allowed);
  };

  // ---- tile streaming by operand (kSpread) ----
  // Step n's own batch of a wave: group 0 K(n+NS), group 1 V(n+NS-1).  Batches
  // past the last tile are still issued (same rows as the wave's last real
  // batch, into a ring slot nobody reads any more), so that every step issues
  // the same number of loads and every wait count is a constant.
  int own_idx[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) own_idx[i] = 0;  // a valid row until the first batch's rows are read
  const char* own_g = grp == 0 ? kg : vg;
  const uint32_t own_stride = grp == 0 ? kstride : vstride;
  const uint32_t own_ring = grp == 0 ? lds_addr(sK) : lds_addr(sV);
  auto own_tile = [&](int n) { return grp == 0 ? n + NS : n + NS - 1; };
  auto read_own = [&](int n) {  // rows of step n's own batch, from the index ring
    const int m = own_tile(n);
    if (m >= 0 && m < n_tiles) TL::read_index(own_idx, sIdx[m % NIR], ltid);
  };
  auto issue_own = [&](int n, int l) {  // load l of step n's own batch
    const int m = own_tile(n);
    const uint32_t chunk = grp == 0 ? TL::kchunk(l, ltid) : TL::vchunk(l, ltid);
    dma16(own_g + ((uint64_t)(uint32_t)own_idx[l] * own_stride + chunk),
          own_ring + (uint32_t)(m % NS) * KBUF + (uint32_t)(w4 * 64 + l * TL::kThreads) * 16);
  };
  static_assert(!kSpread || (TL::kShared && KBUF == VBUF), "operand streams need equal K and V tiles");
  static_assert(!kSpread || NS == 4, "the operand streams' wait counts assume a 4-deep ring");
  // group 0, after the own batch of step n >= 0: the indices of tile n + 2NS
  // (a harmless re-fetch of the last prefix entry past the last tile)
  auto fetch_idx_step = [&]() {
    if (next_idx < n_tiles) fetch_idx();
    else dma4(kvi + (kv_len - 1), lds_addr(sIdx[next_idx++ % NIR]));
  };

  // group 0: indices of tiles 0 .. 2NS-1 first, so that they load together with Q
  if (grp == 0)
    if (!kSpread || w4 == 0)
      for (int m = 0; m < 2 * NS && m < n_tiles; ++m) fetch_idx();
  // Q fragments, pre-scaled by scale*log2(e): lane holds Q[row][16t + 8*half .. +7].
  // Q pre-scaled by scale * log2(e) and rounded back to 16 bits; with dropout
  // Q stays as given and the vector step scales the fp32 scores instead (the
  // dropout path keeps the softmax closer to its definition: with sharply
  // peaked rows the roundings of P's exponent and normaliser, amplified by the
  // dropped entries, would reach the 16-bit tolerance of the gradients)
  typename E::vec8 qf[KSTEPS];
  {
    const float c = P.scale_log2;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4_t x = qraw[t];
#pragma unroll
      for (int w = 0; w < 4; ++w) x[w] = valid ? x[w] : 0u;
      u32x4_t y = x;
      if constexpr (!DROP) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
          y[w] = pack2<E>(E::to_float((uint16_t)(x[w] & 0xFFFFu)) * c, E::to_float((uint16_t)(x[w] >> 16)) * c);
      }
      qf[t] = as_vec8<E>(y);
    }
  }
  const int lo1 = valid ? ivr.x : 0, hi1 = valid ? ivr.y : 0, lo2 = valid ? ivr.z : 0, hi2 = valid ? ivr.w : 0;
  wait_vmem_all();  // indices, Q and row intervals, before any tile load is in flight
  if constexpr (kSpread) {
    __syncthreads();  // the first tiles' indices are in LDS for both groups
    // own batches of steps -NS .. -2: K(0 .. NS-2), V(0 .. NS-3)
    for (int n = grp == 0 ? -NS : -NS + 1; n <= -2; ++n) {
      read_own(n);
#pragma unroll
      for (int l = 0; l < NI; ++l) issue_own(n, l);
    }
    if (grp == 0) wait_vmem_le((NS - 2) * NI);  // K(0)
    read_own(-1);
  } else if (grp == 0) {
    // batches -NS .. -2
    for (int n = -NS; n <= -2; ++n) {
      prepare_batch(n);
      issue_batch(n);
    }
    wait_batch(-2);  // batch -NS: K(0)
    prepare_batch(-1);
  }

  uint32_t koff[kKoff<DQK>], voff[DB];
  k_offsets<DQK>(koff, col, half);
  v_offsets<DV>(voff, lane);

  SoftmaxState<DB> st;
  st.base = 0.f;
  st.l = 0.f;
#pragma unroll
  for (int d = 0; d < DB; ++d) st.acc[d] = zero16();
  f32x16_t s[2];      // scores of a tile between its X step and its Y step
  u32x4_t pk[2][2];   // packed P of a tile between its Y step and its X step

  auto pv = [&](int n) {
    const uint16_t* sv = (const uint16_t*)((const char*)sV + (n % NS) * VBUF);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const typename E::vec8 bfrag = as_vec8<E>(pk[nb][ks]);
        const int key0 = nb * 32 + ks * 16;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const u32x2_t lo = lds_read_tr(sv + key0 * DV, voff[d]);
          const u32x2_t hi = lds_read_tr(sv + (key0 + 8) * DV, voff[d]);
          st.acc[d] = E::mfma32(as_vec8<E>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), bfrag, st.acc[d]);
        }
      }
  };
  // -base in every entry: the accumulator input of each score chain (for the
  // widest Q/K head dimension the registers are short, and the chains start from
  // scores initialised in the vector step instead)
  constexpr bool kFromBase = DQK <= 128;
  f32x16_t nbase;
#pragma unroll
  for (int r = 0; r < 16; ++r) nbase[r] = 0.f;
  auto scores = [&](int n) {  // S(n) - base from K ring slot n % NS
    tile_scores<E, DQK, kFromBase>(s, qf, (const uint16_t*)((const char*)sK + (n % NS) * KBUF), koff, nbase);
  };
  // X(n) when Dqk == Dv (as many score as PV MFMAs): the score MFMAs of tile n+1
  // and the PV MFMAs of tile n alternate, every LDS operand read issued AH MFMA
  // pairs ahead of its use and the order pinned pair by pair, so that the reads
  // are spread over the step and none is waited for right after its issue
  // K operand read i of X(n) (the scores of tile n+1)
  auto read_k_op = [&](int n, int i) {
    constexpr int KO = kKoff<DQK>;
    const uint16_t* skk = (const uint16_t*)((const char*)sK + ((n + 1) % NS) * KBUF);
    const int kt = i >> 1, nb = i & 1;
    return lds_read128(skk + nb * 32 * DQK + (kt / KO) * 16 * KO, koff[kt % KO]);
  };
  // The first K operand reads of the next MFMA step, issued by group 1 at the
  // end of the vector step before it (its copy of the tile was published by
  // group 0's waits and a barrier a phase earlier), so that the MFMA step does
  // not start with a full LDS latency after its barrier.  Group 0 reads them
  // at the start of its MFMA step: at the end of its vector step each of its
  // waves has waited only for its own share of the tile's loads, and the rows
  // of the other waves' shares are safe to read only after the barrier.
  u32x4_t kpre[kXReadAhead];
  auto prefetch_k = [&](int n) {
#pragma unroll
    for (int j = 0; j < kXReadAhead; ++j) kpre[j] = read_k_op(n, j);
  };
  auto x_step_interleaved = [&](int n) {
    constexpr int NP = 2 * KSTEPS;  // == 4 * DB
    constexpr int AH = kXReadAhead;
    const uint16_t* sv = (const uint16_t*)((const char*)sV + (n % NS) * VBUF);
    auto readk = [&](int i) { return read_k_op(n, i); };
    auto readv = [&](int i, u32x2_t& lo, u32x2_t& hi) {  // PV operand i: (nb, ks, d) = (i / 2DB, i / DB % 2, i % DB)
      const int key0 = (i / (2 * DB)) * 32 + ((i / DB) & 1) * 16, d = i % DB;
      lo = lds_read_tr(sv + key0 * DV, voff[d]);
      hi = lds_read_tr(sv + (key0 + 8) * DV, voff[d]);
    };
    u32x4_t kr[AH];
    u32x2_t vl[AH], vh[AH];
    if (grp == 0) prefetch_k(n);  // (group 1 read them before the barrier)
#pragma unroll
    for (int j = 0; j < AH; ++j) {
      kr[j] = kpre[j];
      readv(j, vl[j], vh[j]);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int kt = i >> 1, nb = i & 1;
      s[nb] = E::mfma32(as_vec8<E>(kr[i % AH]), qf[kt], (kFromBase && kt == 0) ? nbase : s[nb]);
      if (i + AH < NP) kr[i % AH] = readk(i + AH);
      const int pnbks = i / DB, d = i % DB;
      st.acc[d] = E::mfma32(as_vec8<E>(u32x4_t{vl[i % AH][0], vl[i % AH][1], vh[i % AH][0], vh[i % AH][1]}),
                            as_vec8<E>(pk[pnbks >> 1][pnbks & 1]), st.acc[d]);
      if (i + AH < NP) readv(i + AH, vl[i % AH], vh[i % AH]);
      if constexpr (kSpread) {  // own load l after pair 2 + l * NP / NI
        if (i >= 2 && (i - 2) % (NP / NI) == 0) issue_own(n, (i - 2) / (NP / NI));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto init_scores = [&]() {
    if constexpr (!kFromBase) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][r] = DROP ? 0.f : -st.base;
    }
  };
  // P = exp2(S - base) straight away; the row maximum is only computed (and the
  // base moved) when some P exceeds 2^threshold, or on a valid row's first tile.
  // (EXACT_SUM: the row sum is of the unrounded P, the softmax's own normaliser;
  // the launch takes it with dropout and at softmax scales up to 1.5x the
  // default, for Q/K head dims up to 128 -- at 192 the fp32 values kept for it
  // would spill)
  auto exp_pack = [&](float& lt) { lt = exp_pack_tile<E, (DQK > 128 ? 1 : 4), EXACT_SUM>(pk, s); };
  // Attention dropout of a tile's packed P, after its row sum (the normaliser
  // is the undropped softmax's): the lane's keys kb0 + 32 nb + 8 run + 4 half
  // + 0..3 sit in pk[nb][run / 2] words 2 (run % 2) (keys +0, +1) and
  // 2 (run % 2) + 1 (keys +2, +3), and take bytes 0..3 of their block's word.
  auto drop_tile = [&](int kb0) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      uint32_t u[4];
      drop_words_st(u, P.drop.seed_lo, P.drop.seed_hi, seq, head, qpos - col, kb0 + 32 * nb, lane);
#pragma unroll
      for (int run = 0; run < 4; ++run) {
        const int ks = run >> 1, j0 = 2 * (run & 1);
        pk[nb][ks][j0] &= drop_keep_pair(u[run], 0, P.drop.t);
        pk[nb][ks][j0 + 1] &= drop_keep_pair(u[run], 2, P.drop.t);
      }
    }
  };
  auto softmax = [&](const TileCursor& c) {
    if constexpr (DROP) {  // unscaled scores (chains from zero): S * scale * log2(e) - base
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][r] = fmaf(s[nb][r], P.scale_log2, -st.base);
    }
    if (c.partial) tile_mask(s, c.t * kBN, half, lo1, hi1, lo2, hi2);
    float lt;
    exp_pack(lt);
    // this lane's 32 values sum beyond 2^threshold iff one P may be too large for
    // the 16-bit P operand; a valid row with nothing accumulated has no base yet
    const bool slow = valid & ((lt > kRescaleLimit) | (st.l == 0.f));
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
      // both half-waves of a query column take the same decision: combined max and sum
      const float mx = tile_max(s);
      const bool empty = wave_half_sum(st.l) == 0.f;
      const bool grow = (mx > 0.f) | (empty & (mx > -INFINITY));
      const float shift = grow ? mx : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      st.base += shift;
      st.l *= alpha;
      if constexpr (!DROP) {  // (unused when !kFromBase; with dropout the chains start from zero)
#pragma unroll
        for (int r = 0; r < 16; ++r) nbase[r] = -st.base;
      }
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[d][r] *= alpha;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][r] -= shift;
      exp_pack(lt);
    }
    st.l += lt;
    if constexpr (DROP) drop_tile(c.t * kBN);
  };

  // Phases: group 0 runs X(n) in phase 2n+2 and Y(n+1) in phase 2n+3, group 1
  // one phase later.
  TileCursor cY = span_start(sSpan, 0);  // tile whose Y step comes next
  __syncthreads();                       // K(0) is in LDS
  if (grp == 1) __syncthreads();         // group 1 runs one phase behind

  // X(-1) = S(0); Y(0)
  if constexpr (kSpread) {
#pragma unroll
    for (int l = 0; l < NI; ++l) issue_own(-1, l);
  } else if (grp == 0) {
    issue_batch(-1);
  }
  init_scores();
  scores(0);
  if (kSpread && grp == 1) wait_vmem_le((NS - 2) * NI);  // V(0)
  __syncthreads();
  softmax(cY);
  cY = next_tile(cY, sSpan, nspan);
  init_scores();
  if constexpr (kSpread) {
    if (grp == 0) wait_vmem_le((NS - 2) * NI);  // K(1)
    read_own(0);
    if (grp == 1 && n_tiles > 1) prefetch_k(0);
  } else if (grp == 0) {
    wait_batch(-1);
    prepare_batch(0);
  }
  __syncthreads();
  // X(n) = PV(n) + S(n+1); Y(n+1)
  for (int n = 0; n + 1 < n_tiles; ++n) {
    if (!kSpread && grp == 0) {
      if constexpr (kSplitIssue) issue_k_part(n);
      else issue_batch(n);
    }
    if constexpr (DQK == DV) {
      // the MFMA step goes first on its SIMD: the partner wave's vector step is
      // shorter and fits into the MFMAs' shadow, while an MFMA issue that waits
      // behind vector instructions stretches the whole phase
      __builtin_amdgcn_s_setprio(1);
      x_step_interleaved(n);
      __builtin_amdgcn_s_setprio(0);
      if (grp == 1) wait_vmem_le((NS - 2) * NI);  // V(n+1): V(n+2) and V(n+3) may still be in flight
    } else {
    pv(n);
    scores(n + 1);
    {
      // operand reads run kReadAhead MFMAs ahead of their MFMA (the compiler
      // would otherwise issue each read just before its use and stall on it)
      constexpr int PVM = 4 * DB, SM = 2 * KSTEPS, AHEAD = DQK > 128 ? 3 : kReadAhead;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
      for (int i = 0; i < PVM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        const int next = i + AHEAD;
        if (next < PVM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (next - PVM < SM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (PVM + i + AHEAD < PVM + SM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    }
    __syncthreads();
    softmax(cY);
    cY = next_tile(cY, sSpan, nspan);
    init_scores();
    if constexpr (kSpread) {
      // K(n+2): the batches of steps n-1 and n may still be in flight (one
      // fewer load in step -1's, which fetched no indices)
      if (grp == 0) {
        // the indices of tile n+8 (here, where the vector step has slack, not
        // after the MFMA step, whose end sets the phase), then K(n+2)
        if (w4 == 0) {  // one wave fetches the indices for all
          fetch_idx_step();
          if (n == 0) wait_vmem_le(2 * NI + 1);
          else wait_vmem_le(2 * NI + 2);
        } else {
          wait_vmem_le(2 * NI);
        }
      }
      read_own(n + 1);
      if (grp == 1 && n + 2 < n_tiles) prefetch_k(n + 1);
    } else if (grp == 0) {
      if constexpr (kSplitIssue) issue_v_part(n);
      wait_batch(n);
      prepare_batch(n + 1);
    }
    __syncthreads();
  }
  // X(N-1) = PV(N-1)
  pv(n_tiles - 1);
  __syncthreads();
  if (grp == 0) __syncthreads();  // matches group 1's extra barrier
  wait_vmem_all();                // nothing may stay in flight past the kernel's end

  // ---- epilogue: normalise (and scale the kept probabilities), write O and LSE ----
  const float l_tot = wave_half_sum(st.l);
  const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * (DROP ? P.drop.scale : 1.f);
  if (P.slot != nullptr && split_slot >= 0) {  // one piece of a split K/V range: fp32 partials
    if (valid) {
      const int64_t srow =
          ((int64_t)(split_slot * P.n_head_groups + hg) * hpt + (w4 % hpt)) * P.tile_q + (a - q0);
      float* orow = P.ws_o + srow * DV;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dd = d * 32 + 8 * i + 4 * half;
          *(f32x4_t*)(orow + dd) = f32x4_t{st.acc[d][4 * i] * inv, st.acc[d][4 * i + 1] * inv,
                                           st.acc[d][4 * i + 2] * inv, st.acc[d][4 * i + 3] * inv};
        }
      }
      if (half == 0)
        P.ws_lse[srow] = l_tot > 0.f ? (st.base + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
    }
    return;
  }
  if (valid) {
    uint16_t* orow = (uint16_t*)P.o + ((int64_t)row * P.hq + head) * DV;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dd = d * 32 + 8 * i + 4 * half;
        u32x2_t w = {pack2<E>(st.acc[d][4 * i] * inv, st.acc[d][4 * i + 1] * inv),
                     pack2<E>(st.acc[d][4 * i + 2] * inv, st.acc[d][4 * i + 3] * inv)};
        *(u32x2_t*)(orow + dd) = w;
      }
    }
    if (half == 0) {
      const float lse = l_tot > 0.f ? (st.base + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
      P.lse[(int64_t)head * P.t_loc + row] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// Streamed (persistent) forward: one work-group per CU walks a fixed list of
// items (Q tile x head group) as one stream of K/V tiles, so that the next
// item's prefix indices and K/V tiles are fetched while the current item's last
// tiles run, instead of every work-group starting cold (tile record, segment,
// indices, Q and the first K tile one after another: several microseconds per
// item on short walks).
//
// Work-group w of head group hg walks the items the plan dealt to w (the same
// deal for every head group: each item, longest first, to the least loaded
// work-group), so that every work-group stays on one head group, i.e. on the
// XCD whose L2 holds that K/V head.  The items' records and spans are copied
// into LDS at the start.
//
// At an item boundary (tile L the last of item k, tile L+1 the first of item
// k+1) the steps differ from the single-item kernel only here:
//   Y(L):   before the softmax of tile L each wave loads item k+1's Q row
//           (into its Q registers: item k's last scores ran in X(L-1)) and
//           visible intervals, waits for them and pre-scales Q; after the
//           softmax the next scores start from 0 (item k+1 has no exponent
//           base yet).  The wait follows the loads at once: a load pending
//           where two paths join would make the compiler wait for all loads
//           (those of the tile stream included) before every later use of Q.
//   X(L):   unchanged: PV(L) of item k, S(L+1) of item k+1.
//   Y(L+1): item k's epilogue (normalise, write O and LSE or its partial),
//           then the softmax state is reset and item k+1's softmax runs.
// ---------------------------------------------------------------------------
constexpr int kStreamMaxItems = kFwdStreamMaxItems;  // items per work-group (the plan's deal keeps to it)
constexpr int kItemInts = 12;
enum { IT_Q0 = 0, IT_ROWS, IT_KVLEN, IT_QROW0, IT_KVOFF, IT_NSPAN, IT_SLOT, IT_FIRST, IT_NTILES };

// Cursor over the stream of K/V tiles of a work-group's items; it carries its
// item's span count, prefix offset and length (read from LDS only when it
// enters a span, so that advancing by a tile and fetching the tile's indices
// stay on scalar registers).
struct StreamCursor {
  int item, sp, t, t_end, partial, nspan, kv_off, kv_len;
};

__device__ __forceinline__ StreamCursor stream_span(const int32_t (*items)[kItemInts], const int32_t* spans,
                                                    int item, int sp) {
  const int4 r = *(const int4*)(spans + (item * kMaxSpans + sp) * 4);
  return StreamCursor{item, sp, __builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                      __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(items[item][IT_NSPAN]),
                      __builtin_amdgcn_readfirstlane(items[item][IT_KVOFF]),
                      __builtin_amdgcn_readfirstlane(items[item][IT_KVLEN])};
}

// First tile of the first item at or after `item` that has tiles (item == n_items: past the end).
__device__ __forceinline__ StreamCursor stream_item_start(const int32_t (*items)[kItemInts],
                                                          const int32_t* spans, int item, int n_items) {
  while (item < n_items && __builtin_amdgcn_readfirstlane(items[item][IT_NSPAN]) == 0) ++item;
  if (item >= n_items) return StreamCursor{n_items, 0, 0, 0, 0, 0, 0, 1};
  return stream_span(items, spans, item, 0);
}

__device__ __forceinline__ StreamCursor stream_next(StreamCursor c, const int32_t (*items)[kItemInts],
                                                    const int32_t* spans, int n_items) {
  ++c.t;
  if (c.t < c.t_end) return c;
  if (c.sp + 1 < c.nspan) return stream_span(items, spans, c.item, c.sp + 1);
  return stream_item_start(items, spans, c.item + 1, n_items);
}

template <typename E, int DQK, int DV>
__global__ __launch_bounds__(kThreads, 1) void fwd_stream_kernel(FwdParams P) {
  using TL = TileLoader<DQK, DV, kThreads / 2>;
  constexpr int KSTEPS = DQK / 16;
  constexpr int DB = DV / 32;
  constexpr int NI = TL::NIDX;
  constexpr int NS = kStages<DQK>;
  constexpr int NIR = 2 * NS;
  constexpr uint32_t KBUF = kBN * DQK * 2, VBUF = kBN * DV * 2;
  constexpr bool kSpread = DQK == DV;  // operand streams, as in fwd_mfma_kernel
  __shared__ __attribute__((aligned(16))) uint16_t sK[NS][kBN * DQK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NS][kBN * DV];
  __shared__ __attribute__((aligned(16))) int32_t sIdx[NIR][kBN];
  __shared__ __attribute__((aligned(16))) int32_t sItem[kStreamMaxItems][kItemInts];
  __shared__ __attribute__((aligned(16))) int32_t sSpans[kStreamMaxItems * kMaxSpans * 4];
  __shared__ int32_t sTotal;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, w4 = wave & 3;
  const int col = lane & 31, half = lane >> 5;
  const int ltid = w4 * 64 + lane;

  const int hg = blockIdx.x % P.n_head_groups;
  const int wg = blockIdx.x / P.n_head_groups;
  const int hpt = P.heads_per_tile;
  const int head = hg * hpt + (w4 % hpt);
  const int kvh = head / P.group;
  const int rowblk = w4 / hpt + grp * (4 / hpt);
  const int item0 = P.t.deal_start[wg];
  const int n_items = min(P.t.deal_start[wg + 1] - item0, kStreamMaxItems);

  const char* kg = (const char*)P.k + (int64_t)kvh * DQK * 2;
  const char* vg = (const char*)P.v + (int64_t)kvh * DV * 2;
  const uint32_t kstride = (uint32_t)P.hkv * DQK * 2, vstride = (uint32_t)P.hkv * DV * 2;

  // ---- the work-group's items into LDS ----
  if (tid < n_items) {
    const int ti = P.t.deal_items[item0 + tid];
    const int32_t* tr = P.t.fwd_tiles + ti * 5;
    const int32_t* sg = P.t.segs + tr[0] * 8;
    int32_t* it = sItem[tid];
    it[IT_Q0] = tr[1];
    it[IT_ROWS] = tr[2];
    it[IT_KVLEN] = sg[3];
    it[IT_QROW0] = sg[4];
    it[IT_KVOFF] = sg[5];
    it[IT_NSPAN] = tr[4];
    it[IT_SLOT] = P.slot != nullptr ? P.slot[ti] : -1;
    it[9] = tr[3];  // first span in the schedule
  }
  __syncthreads();
  for (int x = tid; x < n_items * kMaxSpans; x += kThreads) {
    const int i = x / kMaxSpans, sp = x % kMaxSpans;
    if (sp < sItem[i][IT_NSPAN])
      *(int4*)(sSpans + x * 4) = *(const int4*)(P.t.fwd_spans + (sItem[i][9] + sp) * 4);
  }
  __syncthreads();
  if (tid == 0) {
    int first = 0;
    for (int i = 0; i < n_items; ++i) {
      int nt = 0;
      for (int sp = 0; sp < sItem[i][IT_NSPAN]; ++sp)
        nt += sSpans[(i * kMaxSpans + sp) * 4 + 1] - sSpans[(i * kMaxSpans + sp) * 4];
      sItem[i][IT_FIRST] = first;
      sItem[i][IT_NTILES] = nt;
      first += nt;
    }
    sTotal = first;
  }
  __syncthreads();
  const int n_tiles = __builtin_amdgcn_readfirstlane(sTotal);  // tiles of the whole stream

  // Items without any visible key (unreachable for the supported masks): O = 0, LSE = -inf.
  for (int i = 0; i < n_items; ++i) {
    if (__builtin_amdgcn_readfirstlane(sItem[i][IT_NSPAN]) != 0) continue;
    const int q0 = sItem[i][IT_Q0], a = q0 + rowblk * 32 + col, slot = sItem[i][IT_SLOT];
    if (a < q0 + sItem[i][IT_ROWS]) {
      const int row = sItem[i][IT_QROW0] + a;
      if (slot >= 0) {
        const int64_t srow = ((int64_t)(slot * P.n_head_groups + hg) * hpt + (w4 % hpt)) * P.tile_q + (a - q0);
        for (int d = half; d < DV; d += 2) P.ws_o[srow * DV + d] = 0.f;
        if (half == 0) P.ws_lse[srow] = -INFINITY;
      } else {
        uint16_t* orow = (uint16_t*)P.o + ((int64_t)row * P.hq + head) * DV;
        for (int d = half; d < DV; d += 2) orow[d] = 0;
        if (half == 0) P.lse[(int64_t)head * P.t_loc + row] = -INFINITY;
      }
    }
  }
  if (n_tiles == 0) return;

  // ---- tile streaming (group 0), over the whole stream ----
  StreamCursor cI = stream_item_start(sItem, sSpans, 0, n_items);
  int next_idx = 0;
  int bcount[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) bcount[i] = 0;
  auto fetch_idx = [&]() {
    const int kb0 = cI.t * kBN;
    dma4(P.t.kv_index + cI.kv_off + min(kb0 + lane, cI.kv_len - 1), lds_addr(sIdx[next_idx % NIR]));
    ++next_idx;
    cI = stream_next(cI, sItem, sSpans, n_items);
  };
  int idxK[NI], idxV[NI];
  auto prepare_batch = [&](int n) {
    const int mk = n + NS, mv = n + NS - 1;
    if (mk >= 0 && mk < n_tiles) TL::read_index(idxK, sIdx[mk % NIR], ltid);
    if (mv >= 0 && mv < n_tiles) TL::read_index(idxV, sIdx[mv % NIR], ltid);
  };
  constexpr bool kSplitIssue = NS >= 4;
  auto issue_k_part = [&](int n) {
    int cnt = 0;
    const int mk = n + NS, mi = n + 2 * NS;
    if (mk >= 0 && mk < n_tiles) {
      TL::issue_k(sK[mk % NS], kg, idxK, kstride, ltid, w4 * 64);
      cnt += TL::KN;
    }
    if (mi >= 2 * NS && mi < n_tiles) {
      fetch_idx();
      cnt += 1;
    }
    bcount[(n + NS) % NS] = cnt;
  };
  auto issue_v_part = [&](int n) {
    const int mv = n + NS - 1;
    if (mv >= 0 && mv < n_tiles) {
      TL::issue_v(sV[mv % NS], vg, idxV, vstride, ltid, w4 * 64);
      bcount[(n + NS) % NS] += TL::VN;
    }
  };
  auto issue_batch = [&](int n) {
    issue_k_part(n);
    issue_v_part(n);
  };
  auto wait_batch = [&](int n) {
    int allowed = 0;
#pragma unroll
    for (int b = 0; b < NS - 2; ++b) allowed += bcount[(n - b + NS) % NS];
    wait_vmem_le(allowed);
  };
  // Operand streams (kSpread): as in fwd_mfma_kernel, over the stream's tiles.
  int own_idx[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) own_idx[i] = 0;
  const char* own_g = grp == 0 ? kg : vg;
  const uint32_t own_stride = grp == 0 ? kstride : vstride;
  const uint32_t own_ring = grp == 0 ? lds_addr(sK) : lds_addr(sV);
  auto own_tile = [&](int n) { return grp == 0 ? n + NS : n + NS - 1; };
  auto read_own = [&](int n) {
    const int m = own_tile(n);
    if (m >= 0 && m < n_tiles) TL::read_index(own_idx, sIdx[m % NIR], ltid);
  };
  auto issue_own = [&](int n, int l) {
    const int m = own_tile(n);
    const uint32_t chunk = grp == 0 ? TL::kchunk(l, ltid) : TL::vchunk(l, ltid);
    dma16(own_g + ((uint64_t)(uint32_t)own_idx[l] * own_stride + chunk),
          own_ring + (uint32_t)(m % NS) * KBUF + (uint32_t)(w4 * 64 + l * TL::kThreads) * 16);
  };
  static_assert(!kSpread || (TL::kShared && KBUF == VBUF), "operand streams need equal K and V tiles");
  static_assert(!kSpread || NS == 4, "the operand streams' wait counts assume a 4-deep ring");
  auto fetch_idx_step = [&]() {  // past the stream's last tile: a harmless re-fetch of entry 0
    if (next_idx < n_tiles) fetch_idx();
    else dma4(P.t.kv_index, lds_addr(sIdx[next_idx++ % NIR]));
  };

  // ---- per-item row state of this lane ----
  // cur: the item whose softmax / PV is running; nxt: the next item (its Q and
  // intervals are loaded at the end of the current item's last vector step).
  int cur = stream_item_start(sItem, sSpans, 0, n_items).item;
  int nxt = stream_item_start(sItem, sSpans, cur + 1, n_items).item;
  auto item_q0 = [&](int i) { return __builtin_amdgcn_readfirstlane(sItem[i][IT_Q0]); };
  auto lane_a = [&](int i) { return item_q0(i) + rowblk * 32 + col; };
  auto lane_valid = [&](int i) { return lane_a(i) < item_q0(i) + sItem[i][IT_ROWS]; };
  auto lane_row = [&](int i) { return sItem[i][IT_QROW0] + lane_a(i); };
  const float qscale = P.scale_log2;
  // Item i's visible intervals (into iv) and its Q row (raw, into qf; scale_q
  // pre-scales it by scale*log2(e) in place, which is where the compiler waits
  // for both loads: inside the vector step that issued them)
  int lo1, hi1, lo2, hi2;
  int4 niv;
  typename E::vec8 qf[KSTEPS];
  auto load_rows = [&](int i, int4& iv) {  // lanes past the item's rows load nothing
    const bool v = lane_valid(i);
    const int64_t row = lane_row(i);
    u32x4_t x[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) x[t] = u32x4_t{0u, 0u, 0u, 0u};
    iv = int4{0, 0, 0, 0};
    if (v) {
      iv = *(const int4*)(P.t.row_iv + row * 4);
      const uint16_t* qrow = (const uint16_t*)P.q + (row * P.hq + head) * DQK + 8 * half;
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) x[t] = *(const u32x4_t*)(qrow + 16 * t);
    }
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) qf[t] = as_vec8<E>(x[t]);
  };
  auto scale_q = [&]() {
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      const u32x4_t x = __builtin_bit_cast(u32x4_t, qf[t]);
      u32x4_t y;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        y[w] = pack2<E>(E::to_float((uint16_t)(x[w] & 0xFFFFu)) * qscale,
                        E::to_float((uint16_t)(x[w] >> 16)) * qscale);
      qf[t] = as_vec8<E>(y);
    }
  };

  // group 0: indices of the stream's first 2NS tiles, together with item 0's Q
  if (grp == 0)
    for (int m = 0; m < 2 * NS && m < n_tiles; ++m) fetch_idx();
  load_rows(cur, niv);
  wait_vmem_all();
  scale_q();
  lo1 = niv.x; hi1 = niv.y; lo2 = niv.z; hi2 = niv.w;
  if constexpr (kSpread) {
    __syncthreads();  // the first tiles' indices are in LDS for both groups
    for (int n = grp == 0 ? -NS : -NS + 1; n <= -2; ++n) {
      read_own(n);
#pragma unroll
      for (int l = 0; l < NI; ++l) issue_own(n, l);
    }
    if (grp == 0) wait_vmem_le((NS - 2) * NI);  // K(0)
    read_own(-1);
  } else if (grp == 0) {
    for (int n = -NS; n <= -2; ++n) {
      prepare_batch(n);
      issue_batch(n);
    }
    wait_batch(-2);
    prepare_batch(-1);
  }

  uint32_t koff[kKoff<DQK>], voff[DB];
  k_offsets<DQK>(koff, col, half);
  v_offsets<DV>(voff, lane);

  SoftmaxState<DB> st;
  st.base = 0.f;
  st.l = 0.f;
#pragma unroll
  for (int d = 0; d < DB; ++d) st.acc[d] = zero16();
  f32x16_t s[2];
  u32x4_t pk[2][2];

  auto pv = [&](int n) {
    const uint16_t* sv = (const uint16_t*)((const char*)sV + (n % NS) * VBUF);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const typename E::vec8 bfrag = as_vec8<E>(pk[nb][ks]);
        const int key0 = nb * 32 + ks * 16;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const u32x2_t lo = lds_read_tr(sv + key0 * DV, voff[d]);
          const u32x2_t hi = lds_read_tr(sv + (key0 + 8) * DV, voff[d]);
          st.acc[d] = E::mfma32(as_vec8<E>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), bfrag, st.acc[d]);
        }
      }
  };
  constexpr bool kFromBase = DQK <= 128;
  f32x16_t nbase;
#pragma unroll
  for (int r = 0; r < 16; ++r) nbase[r] = 0.f;
  auto scores = [&](int n) {
    tile_scores<E, DQK, kFromBase>(s, qf, (const uint16_t*)((const char*)sK + (n % NS) * KBUF), koff, nbase);
  };
  auto read_k_op = [&](int n, int i) {
    constexpr int KO = kKoff<DQK>;
    const uint16_t* skk = (const uint16_t*)((const char*)sK + ((n + 1) % NS) * KBUF);
    const int kt = i >> 1, nb = i & 1;
    return lds_read128(skk + nb * 32 * DQK + (kt / KO) * 16 * KO, koff[kt % KO]);
  };
  u32x4_t kpre[kXReadAhead];  // (kSpread) first K operand reads, issued before the barrier
  auto prefetch_k = [&](int n) {
#pragma unroll
    for (int j = 0; j < kXReadAhead; ++j) kpre[j] = read_k_op(n, j);
  };
  auto x_step_interleaved = [&](int n) {
    constexpr int NP = 2 * KSTEPS;
    constexpr int AH = kXReadAhead;
    const uint16_t* sv = (const uint16_t*)((const char*)sV + (n % NS) * VBUF);
    auto readk = [&](int i) { return read_k_op(n, i); };
    auto readv = [&](int i, u32x2_t& lo, u32x2_t& hi) {
      const int key0 = (i / (2 * DB)) * 32 + ((i / DB) & 1) * 16, d = i % DB;
      lo = lds_read_tr(sv + key0 * DV, voff[d]);
      hi = lds_read_tr(sv + (key0 + 8) * DV, voff[d]);
    };
    u32x4_t kr[AH];
    u32x2_t vl[AH], vh[AH];
    if constexpr (kSpread) {
      if (grp == 0) prefetch_k(n);  // (group 1 read them before the barrier)
    }
#pragma unroll
    for (int j = 0; j < AH; ++j) {
      kr[j] = kSpread ? kpre[j] : readk(j);
      readv(j, vl[j], vh[j]);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int kt = i >> 1, nb = i & 1;
      s[nb] = E::mfma32(as_vec8<E>(kr[i % AH]), qf[kt], (kFromBase && kt == 0) ? nbase : s[nb]);
      if (i + AH < NP) kr[i % AH] = readk(i + AH);
      const int pnbks = i / DB, d = i % DB;
      st.acc[d] = E::mfma32(as_vec8<E>(u32x4_t{vl[i % AH][0], vl[i % AH][1], vh[i % AH][0], vh[i % AH][1]}),
                            as_vec8<E>(pk[pnbks >> 1][pnbks & 1]), st.acc[d]);
      if (i + AH < NP) readv(i + AH, vl[i % AH], vh[i % AH]);
      if constexpr (kSpread) {
        if (i >= 2 && (i - 2) % (NP / NI) == 0) issue_own(n, (i - 2) / (NP / NI));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto x_step_grouped = [&](int n) {
    pv(n);
    scores(n + 1);
    constexpr int PVM = 4 * DB, SM = 2 * KSTEPS, AHEAD = DQK > 128 ? 3 : kReadAhead;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
    for (int i = 0; i < PVM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int next = i + AHEAD;
      if (next < PVM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (next - PVM < SM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (PVM + i + AHEAD < PVM + SM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto init_scores = [&]() {
    if constexpr (!kFromBase) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][r] = -st.base;
    }
  };
  auto exp_pack = [&](float& lt) { lt = exp_pack_tile<E, (DQK > 128 ? 1 : 4)>(pk, s); };
  bool valid = lane_valid(cur);
  auto softmax = [&](const StreamCursor& c) {
    if (c.partial) tile_mask(s, c.t * kBN, half, lo1, hi1, lo2, hi2);
    float lt;
    exp_pack(lt);
    const bool slow = valid & ((lt > kRescaleLimit) | (st.l == 0.f));
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
      const float mx = tile_max(s);
      const bool empty = wave_half_sum(st.l) == 0.f;
      const bool grow = (mx > 0.f) | (empty & (mx > -INFINITY));
      const float shift = grow ? mx : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      st.base += shift;
      st.l *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) nbase[r] = -st.base;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[d][r] *= alpha;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][r] -= shift;
      exp_pack(lt);
    }
    st.l += lt;
  };
  // Boundary work runs once per item; its inputs pass through an empty asm
  // statement so that the compiler does not hoist it (its LDS reads with their
  // wait for every LDS operation, the division and the log) into every tile.
  auto opaque = [](int x) {
    asm volatile("" : "+s"(x));
    return x;
  };
  // normalise and write item i's rows (O and LSE, or its fp32 partial)
  auto epilogue = [&](int i) {
    float l_sum = st.l;
    asm volatile("" : "+v"(l_sum));
    const float l_tot = wave_half_sum(l_sum);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (!valid) return;
    const int q0 = item_q0(i), a = lane_a(i), slot = sItem[i][IT_SLOT];
    const float lse2 = l_tot > 0.f ? st.base + __log2f(l_tot) : -INFINITY;
    if (slot >= 0) {
      const int64_t srow = ((int64_t)(slot * P.n_head_groups + hg) * hpt + (w4 % hpt)) * P.tile_q + (a - q0);
      float* orow = P.ws_o + srow * DV;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int dd = d * 32 + 8 * i4 + 4 * half;
          *(f32x4_t*)(orow + dd) = f32x4_t{st.acc[d][4 * i4] * inv, st.acc[d][4 * i4 + 1] * inv,
                                           st.acc[d][4 * i4 + 2] * inv, st.acc[d][4 * i4 + 3] * inv};
        }
      if (half == 0) P.ws_lse[srow] = lse2 * 0.69314718055994530942f;
      return;
    }
    const int row = lane_row(i);
    uint16_t* orow = (uint16_t*)P.o + ((int64_t)row * P.hq + head) * DV;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dd = d * 32 + 8 * i4 + 4 * half;
        *(u32x2_t*)(orow + dd) = u32x2_t{pack2<E>(st.acc[d][4 * i4] * inv, st.acc[d][4 * i4 + 1] * inv),
                                         pack2<E>(st.acc[d][4 * i4 + 2] * inv, st.acc[d][4 * i4 + 3] * inv)};
      }
    if (half == 0) P.lse[(int64_t)head * P.t_loc + row] = lse2 * 0.69314718055994530942f;
  };

  // The last vector step of item cur (cur's Q is done: its last scores ran in
  // the MFMA step before): item nxt's Q and intervals are loaded and awaited
  // at once, then Q is pre-scaled; after the softmax the next scores (item
  // nxt's first) start from 0, as nxt has no base.  (The wait sits right after
  // the loads so that no load is pending where the paths join: the compiler
  // would otherwise wait for every load before each later use of Q.)
  auto next_item_rows = [&]() {
    load_rows(opaque(nxt), niv);
    wait_vmem_all();
    scale_q();
  };
  auto next_item_seed = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) nbase[r] = 0.f;
    if constexpr (!kFromBase) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[nb] = zero16();
    }
  };
  // The first vector step of item nxt: cur's epilogue, then the switch.  The
  // epilogue's global stores share the vector-memory counter with the tile
  // loads but may retire ahead of loads issued before them, so a counted wait
  // for a tile load is only sound with no store in flight: they are drained
  // here (with the loads in flight, once per item).
  auto start_next_item = [&]() {
    epilogue(opaque(cur));
    wait_vmem_all();
    cur = opaque(nxt);
    valid = lane_valid(cur);
    lo1 = niv.x; hi1 = niv.y; lo2 = niv.z; hi2 = niv.w;
    st.base = 0.f;
    st.l = 0.f;
#pragma unroll
    for (int d = 0; d < DB; ++d) st.acc[d] = zero16();
    nxt = stream_item_start(sItem, sSpans, cur + 1, n_items).item;
  };

  // stream positions of the item boundaries: the first tile of the item after cur
  auto first_after = [&](int i) {
    const StreamCursor c = stream_item_start(sItem, sSpans, opaque(i) + 1, n_items);
    return c.item < n_items ? __builtin_amdgcn_readfirstlane(sItem[c.item][IT_FIRST]) : n_tiles;
  };
  int boundary = first_after(cur);  // stream index of item nxt's first tile (n_tiles: none)

  StreamCursor cY = stream_item_start(sItem, sSpans, 0, n_items);
  __syncthreads();                // K(0) is in LDS
  if (grp == 1) __syncthreads();  // group 1 runs one phase behind

  // X(-1) = S(0); Y(0)
  if constexpr (kSpread) {
#pragma unroll
    for (int l = 0; l < NI; ++l) issue_own(-1, l);
  } else if (grp == 0) {
    issue_batch(-1);
  }
  init_scores();
  scores(0);
  if (kSpread && grp == 1) wait_vmem_le((NS - 2) * NI);  // V(0)
  __syncthreads();
  {
    const bool last = boundary == 1 && nxt < n_items;  // item 0 has one tile
    if (last) next_item_rows();
    softmax(cY);
    if (last) next_item_seed();
    else init_scores();
  }
  cY = stream_next(cY, sItem, sSpans, n_items);
  if constexpr (kSpread) {
    if (grp == 0) wait_vmem_le((NS - 2) * NI);  // K(1)
    read_own(0);
    if (grp == 1 && n_tiles > 1) prefetch_k(0);
  } else if (grp == 0) {
    wait_batch(-1);
    prepare_batch(0);
  }
  __syncthreads();
  for (int n = 0; n + 1 < n_tiles; ++n) {
    // X(n) = PV(n) + S(n+1) (S(n+1) is item nxt's first when n + 1 == boundary)
    if (!kSpread && grp == 0) {
      if constexpr (kSplitIssue) issue_k_part(n);
      else issue_batch(n);
    }
    if constexpr (DQK == DV) {
      __builtin_amdgcn_s_setprio(1);
      x_step_interleaved(n);
      __builtin_amdgcn_s_setprio(0);
      if (grp == 1) wait_vmem_le((NS - 2) * NI);  // V(n+1)
    } else {
      x_step_grouped(n);
    }
    __syncthreads();
    // Y(n+1)
    if (n + 1 == boundary) {
      start_next_item();
      boundary = first_after(cur);
    }
    const bool last = n + 2 == boundary && nxt < n_items;  // tile n+1 is cur's last
    if (last) next_item_rows();
    softmax(cY);
    if (last) next_item_seed();
    else init_scores();
    cY = stream_next(cY, sItem, sSpans, n_items);
    if constexpr (kSpread) {
      if (grp == 0) {  // the indices of tile n+8, then K(n+2)
        fetch_idx_step();
        if (n == 0) wait_vmem_le(2 * NI + 1);
        else wait_vmem_le(2 * NI + 2);
      }
      read_own(n + 1);
      if (grp == 1 && n + 2 < n_tiles) prefetch_k(n + 1);
    } else if (grp == 0) {
      if constexpr (kSplitIssue) issue_v_part(n);
      wait_batch(n);
      prepare_batch(n + 1);
    }
    __syncthreads();
  }
  // X(N-1) = PV(N-1)
  pv(n_tiles - 1);
  __syncthreads();
  if (grp == 0) __syncthreads();
  wait_vmem_all();
  epilogue(cur);
}

// Merge of the pieces of split K/V ranges: for every (query row, head) of a split
// Q tile, O = sum_p w_p O_p / sum_p w_p and LSE = m + ln(sum_p w_p) with
// w_p = exp(LSE_p - m), m = max_p LSE_p (the log-sum-exp combination of
// partial softmax results); any number of pieces, none included (O = 0,
// LSE = -inf: no visible key).  HBM-bound and small: DV/8 threads per (row,
// head), 8 columns each, so that a wave reads whole partial rows; a work-group
// takes kMergeThreads / (DV/8) (row, head) pairs of one Q tile and head group.
constexpr int kMergeThreads = 256;
template <int DV>
constexpr int kMergePairs = kMergeThreads / (DV / 8);

template <typename E, int DV>
__global__ __launch_bounds__(kMergeThreads) void fwd_merge_kernel(FwdParams P) {
  constexpr int TPR = DV / 8;
  constexpr int RPB = kMergePairs<DV>;
  const int hpt = P.heads_per_tile;
  const int nsub = (hpt * P.tile_q + RPB - 1) / RPB;
  const int sub = blockIdx.x % nsub;
  const int item = blockIdx.x / nsub / P.n_head_groups;
  const int hg = blockIdx.x / nsub % P.n_head_groups;
  const int x = sub * RPB + (int)threadIdx.x / TPR;  // (head, row) pair inside the tile
  const int d = 8 * ((int)threadIdx.x % TPR);
  if (x >= hpt * P.tile_q) return;
  const int32_t* cb = P.combine + item * 5;
  const int seg = cb[0], q0 = cb[1], rows = cb[2], slot0 = cb[3], npiece = cb[4];
  const int32_t* sg = P.t.segs + seg * 8;
  const int q_row0 = sg[4];
  const int hh = x / P.tile_q, r = x % P.tile_q;
  if (r >= rows) return;
  const int a = q0 + r;
  const int head = hg * hpt + hh;
  const int64_t row = q_row0 + a;
  auto srow = [&](int pc) {
    return ((int64_t)((slot0 + pc) * P.n_head_groups + hg) * hpt + hh) * P.tile_q + r;
  };
  float m = -INFINITY;
  for (int pc = 0; pc < npiece; ++pc) m = fmaxf(m, P.ws_lse[srow(pc)]);
  uint16_t* orow = (uint16_t*)P.o + (row * P.hq + head) * DV + d;
  float* lrow = P.lse + (int64_t)head * P.t_loc + row;
  if (m == -INFINITY) {  // no visible key in any piece
    *(u32x4_t*)orow = u32x4_t{0u, 0u, 0u, 0u};
    if (d == 0) *lrow = -INFINITY;
    return;
  }
  float wsum = 0.f;
  f32x4_t lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
  for (int pc = 0; pc < npiece; ++pc) {
    const float w = expf(P.ws_lse[srow(pc)] - m);
    const float* src = P.ws_o + srow(pc) * DV + d;
    wsum += w;
    lo += w * *(const f32x4_t*)src;
    hi += w * *(const f32x4_t*)(src + 4);
  }
  const float inv = 1.f / wsum;
  *(u32x4_t*)orow = u32x4_t{pack2<E>(lo[0] * inv, lo[1] * inv), pack2<E>(lo[2] * inv, lo[3] * inv),
                            pack2<E>(hi[0] * inv, hi[1] * inv), pack2<E>(hi[2] * inv, hi[3] * inv)};
  if (d == 0) *lrow = m + logf(wsum);
}

// fp32 correctness kernel: one thread per (query row, head), keys one at a time,
// plain online softmax in fp32 on the VALU.  Uses the same tile schedule.
template <int DQK, int DV>
__global__ __launch_bounds__(256) void fwd_fp32_kernel(FwdParams P) {
  const int tile = blockIdx.x / P.n_head_groups;
  const int hg = blockIdx.x % P.n_head_groups;
  const int32_t* tr = P.t.fwd_tiles + tile * 5;
  const int seg = tr[0], q0 = tr[1], rows = tr[2], span0 = tr[3], nspan = tr[4];
  const int32_t* sg = P.t.segs + seg * 8;
  const int kv_len = sg[3], q_row0 = sg[4], kv_off = sg[5];
  const int hpt = P.heads_per_tile;
  const int head = hg * hpt + (threadIdx.x % hpt);
  const int a = q0 + threadIdx.x / hpt;
  if ((int)threadIdx.x / hpt >= rows) return;
  const int kvh = head / P.group;
  const int row = q_row0 + a;
  const int seq = sg[0], qpos = sg[6] + a;  // for dropout
  const float* qrow = (const float*)P.q + ((int64_t)row * P.hq + head) * DQK;
  const float* kg = (const float*)P.k;
  const float* vg = (const float*)P.v;
  const int32_t* iv = P.t.row_iv + (int64_t)row * 4;
  const int lo1 = iv[0], hi1 = iv[1], lo2 = iv[2], hi2 = iv[3];
  float qv[DQK];
  for (int d = 0; d < DQK; ++d) qv[d] = qrow[d];
  float acc[DV];
  for (int d = 0; d < DV; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int sp = 0; sp < nspan; ++sp) {
    const int32_t* spr = P.t.fwd_spans + (span0 + sp) * 4;
    const int b_end = min(spr[1] * P.tile_kv, kv_len);
    for (int b = spr[0] * P.tile_kv; b < b_end; ++b) {
      if (!((b >= lo1 && b < hi1) || (b >= lo2 && b < hi2))) continue;
      const int64_t g = P.t.kv_index[kv_off + b];
      const float* krow = kg + (g * P.hkv + kvh) * DQK;
      const float* vrow = vg + (g * P.hkv + kvh) * DV;
      float sdot = 0.f;
      for (int d = 0; d < DQK; ++d) sdot = fmaf(qv[d], krow[d], sdot);
      const float x = sdot * P.scale_log2;
      const float m_new = fmaxf(m_run, x);
      const float alpha = exp2f(m_run - m_new);
      const float p = exp2f(x - m_new);
      l_run = l_run * alpha + p;
      const bool kept = P.drop.t == 0 ||
                        drop_keep(drop_word(P.drop.seed_lo, P.drop.seed_hi, seq, head, qpos, b & ~3), b & 3, P.drop.t);
      const float pk = kept ? p : 0.f;  // dropout: the row sum keeps every probability
      for (int d = 0; d < DV; ++d) acc[d] = acc[d] * alpha + pk * vrow[d];
      m_run = m_new;
    }
  }
  const float inv = (l_run > 0.f ? 1.f / l_run : 0.f) * (P.drop.t != 0 ? P.drop.scale : 1.f);
  float* orow = (float*)P.o + ((int64_t)row * P.hq + head) * DV;
  for (int d = 0; d < DV; ++d) orow[d] = acc[d] * inv;
  P.lse[(int64_t)head * P.t_loc + row] =
      l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
}

// Row normaliser of the forward without dropout: the sum of the unrounded P
// (the softmax's own, and the faster form) at softmax scales up to 1.5x the
// default 1/sqrt(Dqk); for sharper scales the sum of the P values as rounded
// for the PV MFMA, so that O's weights sum to one exactly: with the pre-scaled
// 16-bit Q and a dominant weight the backward's rowsum(dO * O) needs that.
template <int DQK>
bool exact_row_sum(const FwdParams& p) {
  return DQK <= 128 && p.scale_log2 <= 1.5f * 1.4426950408889634f / std::sqrt((float)DQK);
}

template <typename E, int DQK, int DV>
hipError_t launch_mfma(const FwdParams& p, hipStream_t s, LaunchHook* hook) {
  const unsigned grid = (unsigned)p.n_tiles * (unsigned)p.n_head_groups;
  if (grid == 0) return hipSuccess;
  if (hook) hook->before(K_FWD, s);
  if (p.stream_wgs > 0 && p.drop.t == 0)
    hipLaunchKernelGGL((fwd_stream_kernel<E, DQK, DV>), dim3((unsigned)p.stream_wgs * (unsigned)p.n_head_groups),
                       dim3(kThreads), 0, s, p);
  else if (p.drop.t != 0)
    hipLaunchKernelGGL((fwd_mfma_kernel<E, DQK, DV, true, DQK <= 128>), dim3(grid), dim3(kThreads), 0, s, p);
  else if (exact_row_sum<DQK>(p))
    hipLaunchKernelGGL((fwd_mfma_kernel<E, DQK, DV, false, DQK <= 128>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<E, DQK, DV, false, false>), dim3(grid), dim3(kThreads), 0, s, p);
  if (hook) hook->after(K_FWD, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_combine == 0) return e;
  if (hook) hook->before(K_FWD_MERGE, s);
  const unsigned nsub = ((unsigned)(p.heads_per_tile * p.tile_q) + kMergePairs<DV> - 1) / kMergePairs<DV>;
  hipLaunchKernelGGL((fwd_merge_kernel<E, DV>), dim3((unsigned)p.n_combine * (unsigned)p.n_head_groups * nsub),
                     dim3(kMergeThreads), 0, s, p);
  if (hook) hook->after(K_FWD_MERGE, s);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_fp32(const FwdParams& p, hipStream_t s, LaunchHook* hook) {
  const unsigned grid = (unsigned)p.n_tiles * (unsigned)p.n_head_groups;
  if (grid == 0) return hipSuccess;
  if (hook) hook->before(K_FWD, s);
  hipLaunchKernelGGL((fwd_fp32_kernel<DQK, DV>), dim3(grid), dim3(256), 0, s, p);
  if (hook) hook->after(K_FWD, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(int dtype, int d_qk, int d_v, const FwdParams& p, hipStream_t s,
                      LaunchHook* h) {
  if (dtype == 0) {
    if (d_qk == 64 && d_v == 64) return launch_mfma<Bf16, 64, 64>(p, s, h);
    if (d_qk == 128 && d_v == 128) return launch_mfma<Bf16, 128, 128>(p, s, h);
    if (d_qk == 192 && d_v == 128) return launch_mfma<Bf16, 192, 128>(p, s, h);
  } else if (dtype == 1) {
    if (d_qk == 64 && d_v == 64) return launch_mfma<Fp16, 64, 64>(p, s, h);
    if (d_qk == 128 && d_v == 128) return launch_mfma<Fp16, 128, 128>(p, s, h);
    if (d_qk == 192 && d_v == 128) return launch_mfma<Fp16, 192, 128>(p, s, h);
  } else if (dtype == 2) {
    if (d_qk == 64 && d_v == 64) return launch_fp32<64, 64>(p, s, h);
    if (d_qk == 128 && d_v == 128) return launch_fp32<128, 128>(p, s, h);
    if (d_qk == 192 && d_v == 128) return launch_fp32<192, 128>(p, s, h);
  }
  return hipErrorInvalidValue;
}

}  // namespace cva
