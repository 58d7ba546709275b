// Backward attention kernels for gfx950.
//
// Gradients of masked softmax attention (the standard softmax Jacobian), with
// the scores recomputed from Q, K and the forward's LSE instead of being
// stored (DCP paper, background: block-wise attention never materialises
// Q K^T):
//
//   P = exp(scale * Q K^T - LSE),  dP = dO V^T,  Delta = rowsum(dO * O),
//   dS = P * (dP - Delta),  dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K.
//
// dK/dV go to the rank-major gradient buffer through the causal-prefix index
// (MindSpeed RFC section 3.1: index_add_ of dK/dV into the rank-major buffer).
// The sum over the duplicated prefix rows (a key seen by both local chunks of
// a sub-sequence) happens inside one work-group, which owns the key and walks
// the query tiles of both chunks and all heads of its K/V group; every output
// row is written exactly once, so the result is deterministic (no atomics).
//
// Kernels, in launch order:
//   dq_kernel /       Q-stationary like the forward: S^T = K Q^T, dP^T = V dO^T,
//   dq_pair_kernel    (the second with paired waves, for Q/K head dim 192)
//                     dQ^T += K^T dS^T.  Its prologue also forms the backward
//                     preprocess of its rows, Delta = rowsum(dO * O) and
//                     LSE * log2(e), in fp32 for the dK/dV kernel, and its last
//                     work-groups give dK = dV = 0 to the rank-major rows no
//                     local query sees.
//   dkdv_pair_kernel  K/V-stationary: a work-group owns 128 keys of one K/V
//                     head and walks the 64-row Q tiles that see them; paired
//                     waves per 32 keys, see below.
//
// Attention dropout (MindSpeed RFC section 3.5.2.2) is a second instantiation
// of each kernel (DROP): dV takes P with the dropped pairs zeroed and the kept
// ones scaled by 256 / (256 - t), and dS = P (dP' - Delta) with dP' the same
// mask and scale applied to dP; the keep bytes come from Philox4x32-10, one
// call per 4 x 4 block of (query, key) positions shared by a quad of lanes.
// The paired kernels split the mask work between their two waves.
#include <mutex>
#include <type_traits>

#include "../host/plan.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace cva {

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// zero dK / dV on rank-major rows outside every local prefix (one work-group
// per range of at most 8 rows; run by the dQ kernel's last work-groups)
// ---------------------------------------------------------------------------
template <int DQK, int DV, int NT = kThreads>
__device__ __forceinline__ void zero_rows_block(const BwdParams& P, int range) {
  const int32_t r0 = P.t.zero_rows[2 * range], r1 = P.t.zero_rows[2 * range + 1];
  const u32x4_t z = {0u, 0u, 0u, 0u};
  {
    const int64_t n = (int64_t)(r1 - r0) * P.hkv * DQK / 8;
    u32x4_t* base = (u32x4_t*)((uint16_t*)P.dk + (int64_t)r0 * P.hkv * DQK);
    for (int64_t i = threadIdx.x; i < n; i += NT) base[i] = z;
  }
  {
    const int64_t n = (int64_t)(r1 - r0) * P.hkv * DV / 8;
    u32x4_t* base = (u32x4_t*)((uint16_t*)P.dv + (int64_t)r0 * P.hkv * DV);
    for (int64_t i = threadIdx.x; i < n; i += NT) base[i] = z;
  }
}

// ---------------------------------------------------------------------------
// LDS layout of streamed row tiles (Q, dO, K): rows padded to a power of two
// (128, 256 or 512 bytes) and 16-byte chunks XOR-swizzled by bwd_swz(row), so
// that both the row reads (ds_read_b128, 16 consecutive rows per pass) and the
// transposing reads (ds_read_b64_tr_b16, 4 rows x 32 bytes per 16 lanes) are
// bank-conflict free on the 64-bank LDS.
// ---------------------------------------------------------------------------
template <int D>
constexpr int kRowBytes = D * 2 <= 128 ? 128 : (D * 2 <= 256 ? 256 : 512);

template <int RB>
__device__ __forceinline__ int bwd_swz(int r) {
  if constexpr (RB >= 256)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (r >> 1) & 7;
}

template <int RB>
__device__ __forceinline__ uint32_t swz_off(int r, int colbytes) {
  return (uint32_t)(r * RB + (((colbytes >> 4) ^ bwd_swz<RB>(r)) << 4) + (colbytes & 15));
}

// Per-lane offsets of the two operand reads of a streamed tile with D columns.
//  rows:  A operand = 32 rows x 16 columns, lane (row 32*qs + l%32, half h) reads
//         columns 16*kt + 8h .. +7:  row_off[kt % KO] + (kt / KO) * 32*KO + qs*32*RB
//  trans: A operand = 32 columns x 16 rows (transposed), lane (s = l&15, g = l>>4)
//         reads 4 rows (row0 + s>>2 ...) of column 32*blk + 16*(g&1) + 4*(s&3) where
//         row0 = 32*qs + 16*st + 4*h + 8*hi:  tr_off[hi][blk] + (32*qs + 16*st)*RB
template <int D>
struct TileOffsets {
  static constexpr int RB = kRowBytes<D>;
  static constexpr int KO = RB >= 256 ? 8 : 4;
  static constexpr int NB = D / 32;
  uint32_t row_off[KO];
  uint32_t tr_off[2][NB];
  __device__ void init(int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int u = 0; u < KO; ++u) row_off[u] = swz_off<RB>(col, (2 * u + half) * 16);
    const int s = lane & 15, g = lane >> 4;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
        tr_off[hi][blk] = swz_off<RB>(4 * (g >> 1) + 8 * hi + (s >> 2), (blk * 32 + 16 * (g & 1) + 4 * (s & 3)) * 2);
  }
  __device__ u32x4_t row(const char* base, int qs, int kt) const {
    return *(const u32x4_t*)(base + qs * 32 * RB + (kt / KO) * 32 * KO + row_off[kt % KO]);
  }
  __device__ u32x2_t trans(const char* base, int rows0, int hi, int blk) const {
    return lds_read_tr16((const uint16_t*)(base + rows0 * RB + tr_off[hi][blk]));
  }
};

// DMA of a 64-row tile with D columns into LDS (kRowBytes layout) by NT threads;
// row_src(r) gives the global address of row r's first element.
template <int D, int NT = 256, typename RowSrc>
__device__ __forceinline__ void dma_rows(char* lds, RowSrc row_src, int tid, int wave) {
  constexpr int RB = kRowBytes<D>, CH = RB / 16, VC = D / 8;
  constexpr int N = 64 * CH / NT;
  const uint32_t base = lds_addr(lds) + (uint32_t)wave * 64 * 16;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int s = i * NT + tid;
    const int r = s / CH;
    int c = (s % CH) ^ bwd_swz<RB>(r);
    if (c >= VC) c = 0;  // row padding: any in-bounds source
    dma16(row_src(r) + c * 16, base + i * NT * 16);
  }
}

// Bits [lo, hi) of a 32-bit word, both ends clamped to [0, 32].
__device__ __forceinline__ uint32_t key_bits(int lo, int hi) {
  lo = max(lo, 0);
  hi = min(hi, 32);
  if (hi <= lo) return 0u;
  const uint32_t upto = hi >= 32 ? ~0u : (1u << hi) - 1u;
  return upto & ~((1u << lo) - 1u);
}

// Score x, or -inf where bit `bit` of the lane's visibility word vw is clear
// (a sign-extending bit extract and a bitwise select).
__device__ __forceinline__ float mask_score(float x, uint32_t vw, int bit) {
  const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)vw, bit, 1);
  return __uint_as_float((__float_as_uint(x) & keep) | (0xFF800000u & ~keep));
}

// ---------------------------------------------------------------------------
// dQ with paired waves (Q/K head dimension 192, where the single-wave form needs
// more than 256 registers and so runs one wave per SIMD).  The same work item
// as dq_kernel, run by 8 waves: waves w and w+4 (one SIMD) own the same 32
// query rows of one head.  Wave w (the S wave) holds Q^T, forms S^T = K Q^T and
// P = exp2(S * scale * log2 e - LSE * log2 e) (masked on partial tiles) of both
// 32-key blocks of a tile; wave w+4 (the dS wave) holds dO^T and forms
// dP^T = V dO^T of both.  After the mid-tile barrier each forms dS = P (dP -
// Delta) and dQ^T += K^T dS^T for one block (the dS wave block 0, with P handed
// over in fp32 through LDS; the S wave block 1, with dP handed over likewise),
// into partial sums added at the end.  The dS waves also form Delta and
// LSE * log2 e of the rows (the backward preprocess) and stream the K/V tiles
// through a 2-deep LDS ring, issuing tile n+1 at the start of tile n.  P is
// never rounded, so the arithmetic is that of dq_kernel.
// ---------------------------------------------------------------------------
template <typename E, int DQK, int DV, bool DROP>
__global__ __launch_bounds__(2 * kThreads, 1) void dq_pair_kernel(BwdParams P) {
  constexpr int NT = 2 * kThreads;
  const int n_dq_wg = P.n_dq_tiles * P.dq_head_groups;
  if ((int)blockIdx.x >= n_dq_wg) {  // the grid's last work-groups do the zero fill
    zero_rows_block<DQK, DV, NT>(P, (int)blockIdx.x - n_dq_wg);
    return;
  }
  constexpr int BN = kDqTileKv;
  constexpr int QS = DQK / 16, VS = DV / 16;
  constexpr int NS = 2;
  constexpr int NIR = 2 * NS;  // index ring slots
  using KO = TileOffsets<DQK>;
  using VO = TileOffsets<DV>;
  constexpr int CHK = KO::RB / 16, CHV = VO::RB / 16;  // 16-byte chunks per LDS row
  constexpr int NK = BN * CHK / kThreads, NV = BN * CHV / kThreads;  // per dS-wave thread
  constexpr bool kSharedRows = CHK == CHV;
  constexpr int NI = kSharedRows ? NK : NK + NV;
  static_assert(BN == 64, "the index fetch covers 64 keys per tile");
  __shared__ __attribute__((aligned(16))) char sK[NS][BN * KO::RB];
  __shared__ __attribute__((aligned(16))) char sV[NS][BN * VO::RB];
  __shared__ __attribute__((aligned(16))) int32_t sIdx[NIR][BN];
  __shared__ __attribute__((aligned(16))) int32_t sSpan[kDqMaxSpans * 4];
  __shared__ __attribute__((aligned(16))) f32x4_t sP[4][4][64];   // P of key block 0: pair, r/4, lane
  __shared__ __attribute__((aligned(16))) f32x4_t sDP[4][4][64];  // dP of key block 1: pair, r/4, lane
  __shared__ __attribute__((aligned(16))) float sDelta[4][64];    // Delta of the pair's rows, per lane

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const bool dswave = wave >= 4;
  const int pw = wave & 3;              // the pair (row block / head) of this wave
  const int ltid = tid & (kThreads - 1);  // thread index inside its role

  const int tile = blockIdx.x / P.dq_head_groups;
  const int hg = blockIdx.x % P.dq_head_groups;
  const int32_t* tr = P.t.dq_tiles + tile * 5;
  const int seg = tr[0], q0 = tr[1], rows = tr[2], span0 = tr[3], nspan = tr[4];
  const int32_t* sg = P.t.segs + seg * 8;
  const int kv_len = sg[3], q_row0 = sg[4], kv_off = sg[5];
  const int hpt = P.dq_heads_per_tile;
  const int head = hg * hpt + (pw % hpt);
  const int kvh = head / P.group;
  const int a = q0 + (pw / hpt) * 32 + col;
  const bool valid = a < q0 + rows;  // the tile's own rows (a tile may end inside its segment)
  const int row = q_row0 + a;
  [[maybe_unused]] const int seq = sg[0], qpos = sg[6] + a;  // sequence, in-sequence query position (dropout)

  const char* kg = (const char*)P.k + (int64_t)kvh * DQK * 2;
  const char* vg = (const char*)P.v + (int64_t)kvh * DV * 2;
  const uint32_t kstride = (uint32_t)P.hkv * DQK * 2, vstride = (uint32_t)P.hkv * DV * 2;
  const int32_t* __restrict__ kvi = P.t.kv_index + kv_off;

  if (tid < 4 * nspan) sSpan[tid] = P.t.dq_spans[span0 * 4 + tid];
  wait_vmem_all();
  __syncthreads();
  int n_tiles = 0;
  for (int sp = 0; sp < nspan; ++sp) {
    const int4 r = *(const int4*)(sSpan + 4 * sp);
    n_tiles += __builtin_amdgcn_readfirstlane(r.y) - __builtin_amdgcn_readfirstlane(r.x);
  }

  struct Cur {
    int sp, t, t_end, partial;
  };
  auto span_at = [&](int sp) {
    const int4 r = *(const int4*)(sSpan + 4 * sp);
    return Cur{sp, __builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
               __builtin_amdgcn_readfirstlane(r.z)};
  };
  auto advance = [&](Cur c) {
    if (++c.t >= c.t_end && c.sp + 1 < nspan) c = span_at(c.sp + 1);
    return c;
  };

  // ---- streaming by the dS waves.  batch(m): K and V of tile m into ring slot
  // m % NS and, by wave 4, the prefix-index entries of tile m + NIR - 1 (clamped
  // to a valid address when that tile does not exist: the slot is then never read).
  Cur cF = nspan > 0 ? span_at(0) : Cur{0, 0, 0, 0};  // next tile whose indices get fetched
  int next_f = 0;
  auto fetch_idx = [&]() {
    const int kb0 = next_f < n_tiles ? cF.t * BN : 0;
    dma4(kvi + min(kb0 + lane, kv_len - 1), lds_addr(sIdx[next_f % NIR]));
    if (next_f < n_tiles) cF = advance(cF);
    ++next_f;
  };
  auto issue = [&](int m) {
    const int32_t* si = sIdx[m % NIR];
    int idx[NI];
#pragma unroll
    for (int i = 0; i < NK; ++i) idx[i] = si[(i * kThreads + ltid) / CHK];
    if constexpr (!kSharedRows) {
#pragma unroll
      for (int i = 0; i < NV; ++i) idx[NK + i] = si[(i * kThreads + ltid) / CHV];
    }
    const uint32_t kl = lds_addr(sK[m % NS]) + (uint32_t)pw * 64 * 16;
    const uint32_t vl = lds_addr(sV[m % NS]) + (uint32_t)pw * 64 * 16;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int s = i * kThreads + ltid;
      int c = (s % CHK) ^ bwd_swz<KO::RB>(s / CHK);
      if (c >= DQK / 8) c = 0;  // row padding: any in-bounds source
      dma16(kg + ((uint64_t)(uint32_t)idx[i] * kstride + c * 16), kl + i * kThreads * 16);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int s = i * kThreads + ltid;
      int c = (s % CHV) ^ bwd_swz<VO::RB>(s / CHV);
      if (c >= DV / 8) c = 0;
      const int id = kSharedRows ? idx[i] : idx[NK + i];
      dma16(vg + ((uint64_t)(uint32_t)id * vstride + c * 16), vl + i * kThreads * 16);
    }
    if (wave == 4) fetch_idx();
  };

  KO ko;
  VO vo;
  ko.init(lane);
  vo.init(lane);
  const float sl2 = P.scale_log2;

  // The tile loop is instantiated once per role.
  auto run = [&](auto role_c) {
    constexpr bool DSW = decltype(role_c)::value;
    // registers: Q^T (S wave) or dO^T (dS wave); lane holds row[16s + 8*half .. +7]
    constexpr int FS = DSW ? VS : QS;
    typename E::vec8 fr[FS];
    {
      const uint16_t* src = DSW ? (const uint16_t*)P.dout + ((int64_t)row * P.hq + head) * DV + 8 * half
                                : (const uint16_t*)P.q + ((int64_t)row * P.hq + head) * DQK + 8 * half;
#pragma unroll
      for (int s = 0; s < FS; ++s) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (valid) x = *(const u32x4_t*)(src + 16 * s);
        fr[s] = as_vec8<E>(x);
      }
    }
    float lse2 = INFINITY, delta = 0.f;
    int lo1 = 0, hi1 = 0, lo2 = 0, hi2 = 0;
    if constexpr (DSW) {
      // the backward preprocess of this lane's (row, head): Delta = rowsum(dO * O)
      // (each half-wave holds half of the row; the halves are summed across
      // lanes l and l + 32) and LSE * log2(e), for the dK/dV kernel
      u32x4_t ov[VS];
      if (valid) {
        const uint16_t* orow = (const uint16_t*)P.o + ((int64_t)row * P.hq + head) * DV + 8 * half;
#pragma unroll
        for (int s = 0; s < VS; ++s) ov[s] = *(const u32x4_t*)(orow + 16 * s);
        lse2 = P.lse[(int64_t)head * P.t_loc + row] * kLog2e;
      }
      wait_vmem_all();
      float dsum = 0.f;
      if (valid) {
#pragma unroll
        for (int s = 0; s < VS; ++s) {
          const u32x4_t g = __builtin_bit_cast(u32x4_t, fr[s]);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            dsum = fmaf(E::to_float((uint16_t)(ov[s][w] & 0xFFFFu)), E::to_float((uint16_t)(g[w] & 0xFFFFu)), dsum);
            dsum = fmaf(E::to_float((uint16_t)(ov[s][w] >> 16)), E::to_float((uint16_t)(g[w] >> 16)), dsum);
          }
        }
      }
      const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(dsum), __float_as_uint(dsum), false, false);
      delta = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
      if (valid && half == 0) {
        P.delta[(int64_t)head * P.t_loc + row] = delta;
        P.lse2[(int64_t)head * P.t_loc + row] = lse2;
      }
      sDelta[pw][lane] = delta;  // for the S wave (read after the next barrier)
    } else {
      if (valid) {
        const int32_t* iv = P.t.row_iv + (int64_t)row * 4;
        lo1 = iv[0]; hi1 = iv[1]; lo2 = iv[2]; hi2 = iv[3];
        lse2 = P.lse[(int64_t)head * P.t_loc + row] * kLog2e;
      }
      wait_vmem_all();
    }
    // first batch: the indices of tiles 0 .. NIR-2, then tile 0
    if (n_tiles > 0) {
      if (wave == 4)
        for (int m = 0; m < NIR - 1; ++m) fetch_idx();
      if constexpr (DSW) wait_vmem_all();
      __syncthreads();
      if constexpr (DSW) {
        issue(0);
        wait_vmem_all();
      }
      __syncthreads();
    }
    // dQ^T partial sums: the dS wave over key block 0 of every tile, the S wave
    // over key block 1 (added together at the end)
    f32x16_t acc[DQK / 32];
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d) acc[d] = zero16();
    if constexpr (!DSW) delta = sDelta[pw][lane];
    // dS^T of one key block from P and dP (lane layout of the S^T accumulators),
    // packed for the dQ MFMA, then dQ^T[d][q] += sum_key K^T[d][key] dS^T[key][q]
    auto ds_dq = [&](const char* k_s, int nb, const f32x4_t (&pv)[4], const f32x4_t (&dv)[4]) {
      uint32_t pd[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pd[i >> 1][2 * (i & 1)] = pack2<E>(pv[i][0] * (dv[i][0] - delta), pv[i][1] * (dv[i][1] - delta));
        pd[i >> 1][2 * (i & 1) + 1] = pack2<E>(pv[i][2] * (dv[i][2] - delta), pv[i][3] * (dv[i][3] - delta));
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int rows0 = nb * 32 + st * 16;
        const typename E::vec8 bd = as_vec8<E>(u32x4_t{pd[st][0], pd[st][1], pd[st][2], pd[st][3]});
#pragma unroll
        for (int d = 0; d < DQK / 32; ++d) {
          const u32x2_t lo = ko.trans(k_s, rows0, 0, d);
          const u32x2_t hi = ko.trans(k_s, rows0, 1, d);
          acc[d] = E::mfma32(as_vec8<E>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), bd, acc[d]);
        }
      }
    };
    Cur cC = nspan > 0 ? span_at(0) : Cur{0, 0, 0, 0};  // tile being computed
    for (int n = 0; n < n_tiles; ++n) {
      const char* k_s = sK[n % NS];
      const char* v_s = sV[n % NS];
      const int kb0 = cC.t * BN;
      const bool partial = cC.partial != 0;
      if constexpr (!DSW) {
        // ---- S wave: S^T and P of both 32-key blocks (phase 1); dS and dQ^T of
        // key block 1 (phase 2) ----
        f32x4_t p1[4];  // P of key block 1, kept in registers
        // dropout: bit 4i + j of keep1 says whether key 32 + 8i + 4*half + j is kept
        // (block 0's mask is formed by the dS wave, which applies it)
        [[maybe_unused]] uint32_t keep1 = 0;
#pragma unroll
        for (int nb = 0; nb < BN / 32; ++nb) {
          f32x16_t sc = zero16();
#pragma unroll
          for (int st = 0; st < QS; ++st) sc = E::mfma32(as_vec8<E>(ko.row(k_s, nb, st)), fr[st], sc);
          // lane holds keys nb*32 + 8i + 4*half + j (r = 4i + j) for its query;
          // on a partial tile bit 8i + j of vw says whether that key is visible
          uint32_t vw = ~0u;
          if (partial) {
            const int kb = kb0 + nb * 32 + 4 * half;
            vw = key_bits(lo1 - kb, hi1 - kb) | key_bits(lo2 - kb, hi2 - kb);
          }
          [[maybe_unused]] uint32_t du[4];  // dropout: random words of keys nb*32 + 8i + 4*half + 0..3
          if (DROP && nb == 1)
            drop_words_st(du, P.drop.seed_lo, P.drop.seed_hi, seq, head, qpos - col, kb0 + nb * 32, lane);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4_t pv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 4 * i + j;
              float x = fmaf(sc[r], sl2, -lse2);
              if (partial) x = mask_score(x, vw, 8 * i + j);
              pv[j] = __builtin_amdgcn_exp2f(x);
            }
            if (DROP && nb == 1) {
#pragma unroll
              for (int j = 0; j < 4; ++j) keep1 |= (drop_keep(du[i], j, P.drop.t) ? 1u : 0u) << (4 * i + j);
            }
            if (nb == 0) sP[pw][i][lane] = pv;
            else p1[i] = pv;
          }
        }
        __syncthreads();  // P of block 0 and dP of block 1 are in LDS
        f32x4_t dv1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dv1[i] = sDP[pw][i][lane];
        if constexpr (DROP) {  // a dropped pair passes no gradient, a kept one is scaled
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) dv1[i][j] = ((keep1 >> (4 * i + j)) & 1u) ? dv1[i][j] * P.drop.scale : 0.f;
        }
        ds_dq(k_s, 1, p1, dv1);
      } else {
        // ---- dS wave: the next tile's loads and dP^T of both key blocks (phase 1);
        // dS and dQ^T of key block 0 (phase 2) ----
        if (n + NS - 1 < n_tiles) issue(n + NS - 1);  // into the slot tile n-1 used
        f32x16_t dp[BN / 32];
#pragma unroll
        for (int nb = 0; nb < BN / 32; ++nb) dp[nb] = zero16();
#pragma unroll
        for (int st = 0; st < VS; ++st)
#pragma unroll
          for (int nb = 0; nb < BN / 32; ++nb) dp[nb] = E::mfma32(as_vec8<E>(vo.row(v_s, nb, st)), fr[st], dp[nb]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sDP[pw][i][lane] = f32x4_t{dp[1][4 * i], dp[1][4 * i + 1], dp[1][4 * i + 2], dp[1][4 * i + 3]};
        // dropout: block 0's random words (this wave's rows are its partner's),
        // formed while the S wave still exponentiates
        [[maybe_unused]] uint32_t du0[4];
        if constexpr (DROP) drop_words_st(du0, P.drop.seed_lo, P.drop.seed_hi, seq, head, qpos - col, kb0, lane);
        __syncthreads();  // P of block 0 and dP of block 1 are in LDS
        f32x4_t p0[4], dv0[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p0[i] = sP[pw][i][lane];
          dv0[i] = f32x4_t{dp[0][4 * i], dp[0][4 * i + 1], dp[0][4 * i + 2], dp[0][4 * i + 3]};
        }
        if constexpr (DROP) {  // a dropped pair passes no gradient, a kept one is scaled
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) dv0[i][j] = drop_keep(du0[i], j, P.drop.t) ? dv0[i][j] * P.drop.scale : 0.f;
        }
        ds_dq(k_s, 0, p0, dv0);
        if (n + 1 < n_tiles) wait_vmem_all();  // tile n+1 has landed
      }
      cC = advance(cC);
      __syncthreads();
    }
    wait_vmem_all();
    // the S wave's partial dQ^T joins the dS wave's through LDS, two 32-column
    // blocks at a time (sDP and sP are free once the tiles are done)
#pragma unroll
    for (int d = 0; d < DQK / 32; d += 2) {
      if constexpr (!DSW) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sDP[pw][i][lane] = f32x4_t{acc[d][4 * i], acc[d][4 * i + 1], acc[d][4 * i + 2], acc[d][4 * i + 3]};
          sP[pw][i][lane] =
              f32x4_t{acc[d + 1][4 * i], acc[d + 1][4 * i + 1], acc[d + 1][4 * i + 2], acc[d + 1][4 * i + 3]};
        }
      }
      __syncthreads();
      if constexpr (DSW) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4_t x = sDP[pw][i][lane], y = sP[pw][i][lane];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[d][4 * i + j] += x[j];
            acc[d + 1][4 * i + j] += y[j];
          }
        }
      }
      __syncthreads();
    }
    if constexpr (DSW) {
      if (valid) {
        uint16_t* dqr = (uint16_t*)P.dq + ((int64_t)row * P.hq + head) * DQK;
        const float sc = P.scale;
#pragma unroll
        for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int dd = d * 32 + 8 * i + 4 * half;
            *(u32x2_t*)(dqr + dd) = u32x2_t{pack2<E>(acc[d][4 * i] * sc, acc[d][4 * i + 1] * sc),
                                             pack2<E>(acc[d][4 * i + 2] * sc, acc[d][4 * i + 3] * sc)};
          }
      }
    }
  };
  if (dswave) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// dK / dV, K/V-stationary, with paired waves.  A work-group owns 128 keys of one
// K/V head and walks, for every query head of the group, the 64-row Q tiles of
// both local chunks that see its keys (Q, dO, LSE, Delta and the row intervals
// of those tiles stream through an NS-deep LDS ring, DMA issued NS-1 tiles
// ahead).  8 waves: waves w and w+4 (one SIMD) own the same 32 keys, with that
// key's K (or V) row in registers.  Wave w (the P wave) computes S = Q K^T and
// P = exp2(S*scale*log2e - LSE*log2e), hands P to its partner through LDS and
// accumulates dV^T += dO^T P; wave w+4 (the dS wave) computes dP = dO V^T,
// dS = P (dP - Delta) and accumulates dK^T += Q^T dS.  Each tile runs in two
// phases separated by a barrier -- (S, P | dP) then (dV | dS, dK) -- so that on
// every SIMD one wave's vector work overlaps the other's MFMAs, and each wave
// keeps one operand set and one accumulator set in registers (up to 244 VGPRs
// at Q/K head dim 192, so two waves per SIMD).  Each rank-major key row is
// written once: no atomics, deterministic.
// ---------------------------------------------------------------------------
// Q/dO ring depth: 512-byte Q rows (Q/K head dim 192) leave LDS for 2 stages.
template <int DQK>
constexpr int kDkvPairStages = DQK > 128 ? 2 : 4;

template <typename E, int DQK, int DV, bool DROP>
__global__ __launch_bounds__(2 * kThreads, 1) void dkdv_pair_kernel(BwdParams P) {
  constexpr int BQ = 64;           // queries per Q tile
  constexpr int QS = DQK / 16;     // reduction steps over Dqk
  constexpr int VS = DV / 16;      // reduction steps over Dv
  constexpr int NS = kDkvPairStages<DQK>;
  using QO = TileOffsets<DQK>;
  using OO = TileOffsets<DV>;
  constexpr int QB = BQ * QO::RB, OB = BQ * OO::RB;
  constexpr int QN = 64 * (QO::RB / 16) / kThreads, ON = 64 * (OO::RB / 16) / kThreads;
  constexpr int NA = (DQK > DV ? DQK : DV) / 32;
  __shared__ __attribute__((aligned(16))) char sQ[NS][QB];
  __shared__ __attribute__((aligned(16))) char sO[NS][OB];
  __shared__ __attribute__((aligned(16))) float sL[NS][BQ];
  __shared__ __attribute__((aligned(16))) float sD[NS][BQ];
  __shared__ __attribute__((aligned(16))) int32_t sIv[NS][BQ * 4];
  __shared__ __attribute__((aligned(16))) uint32_t sMask[4][BQ];          // per P wave: visible keys of each query
  __shared__ __attribute__((aligned(16))) u32x4_t sP[4][BQ / 32][2][64];  // packed P, in the MFMA operand layout
  __shared__ __attribute__((aligned(16))) uint32_t sKeep[4][64];  // dropout: second query half's keep bits, per dS wave
  __shared__ __attribute__((aligned(16))) int32_t sSpan[kDkvMaxSpans * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const bool dswave = wave >= 4;  // dP, dS, dK (else S, P, dV)
  const int kgrp = wave & 3;      // the wave's 32 keys

  const int tile = blockIdx.x / P.hkv;
  const int kvh = blockIdx.x % P.hkv;
  const int32_t* tr = P.t.kv_tiles + tile * 5;
  const int seq = tr[0], k0 = tr[1], keys = tr[2], span0 = tr[3], nspan = tr[4];
  const int32_t* segA = P.t.segs + (2 * seq) * 8;
  const int32_t* segB = P.t.segs + (2 * seq + 1) * 8;
  const int qlenA = segA[2], row0A = segA[4], qlenB = segB[2], row0B = segB[4];
  const int32_t* kvi = P.t.kv_index + segB[5];
  const int kl = kgrp * 32 + col;
  const int kpos = k0 + kl;
  const bool kvalid = kl < keys;
  const int64_t grow = kvalid ? (int64_t)kvi[kpos] : 0;

  // B operands in registers: K^T for the P wave, V^T for the dS wave; lane holds
  // row[key][16s + 8*half .. +7]
  constexpr int FS = QS > VS ? QS : VS;
  typename E::vec8 frag[FS];
  {
    const uint16_t* src = dswave ? (const uint16_t*)P.v + (grow * P.hkv + kvh) * DV + 8 * half
                                 : (const uint16_t*)P.k + (grow * P.hkv + kvh) * DQK + 8 * half;
    const int nst = dswave ? VS : QS;
#pragma unroll
    for (int st = 0; st < FS; ++st) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (kvalid && st < nst) x = *(const u32x4_t*)(src + 16 * st);
      frag[st] = as_vec8<E>(x);
    }
  }
  if (tid < 4 * nspan) sSpan[tid] = P.t.kv_spans[span0 * 4 + tid];
  wait_vmem_all();
  __syncthreads();

  // Q tiles are walked from the last one back, the heads of the group innermost:
  // under the causal masks every work-group's range ends at the same place, so
  // the work-groups running together on one XCD stream the same tiles at about
  // the same time and share them in L2; taking the group's heads together keeps
  // the rows in flight contiguous (one head's 256-byte slice of every row at a
  // time left 36 % of the L2 lookups missing on a 131072-token sequence, the
  // group's contiguous slices 16 %).
  struct Cur {
    int hh, sp, qt, qt_lo, seg, partial;
  };
  auto span_at = [&](Cur c, int sp) {  // the span's last tile
    const int4 r = *(const int4*)(sSpan + 4 * sp);
    c.sp = sp;
    c.seg = __builtin_amdgcn_readfirstlane(r.x);
    c.qt_lo = __builtin_amdgcn_readfirstlane(r.y);
    c.qt = __builtin_amdgcn_readfirstlane(r.z) - 1;
    c.partial = __builtin_amdgcn_readfirstlane(r.w);
    return c;
  };
  auto advance = [&](Cur c) {
    if (++c.hh < P.group) return c;
    c.hh = 0;
    if (--c.qt < c.qt_lo) {
      int sp = c.sp - 1;
      if (sp < 0) sp = nspan - 1;  // past the walk's end (the cursor is not used again)
      c = span_at(c, sp);
    }
    return c;
  };
  int n_tiles = 0;
  for (int sp = 0; sp < nspan; ++sp) {
    Cur c = span_at(Cur{0, 0, 0, 0, 0, 0}, sp);
    n_tiles += c.qt + 1 - c.qt_lo;
  }
  n_tiles *= P.group;
  const int sp_last = nspan > 0 ? nspan - 1 : 0;

  // Tile loads are issued where each role has slack: the P waves load Q and the
  // LSE at the end of their dV step, the dS waves load dO, Delta and the row
  // intervals after their dP MFMAs.
  const char* qgb = (const char*)P.q;
  const char* ogb = (const char*)P.dout;
  const int per_batch = dswave ? ON + (kgrp < 2 ? 1 : 0) : QN + (kgrp == 0 ? 1 : 0);
  auto issue = [&](const Cur& c, int m) {
    const int slot = m % NS;
    const int head = kvh * P.group + c.hh;
    const bool isB = (c.seg & 1) != 0;
    const int q_len = isB ? qlenB : qlenA, q_row0 = isB ? row0B : row0A;
    const int a0 = c.qt * BQ;
    auto lrow = [&](int r) { return q_row0 + min(a0 + r, q_len - 1); };
    const int rtid = tid & (kThreads - 1);
    if (!dswave) {
      dma_rows<DQK, kThreads>(sQ[slot], [&](int r) { return qgb + ((int64_t)lrow(r) * P.hq + head) * (DQK * 2); },
                              rtid, kgrp);
      if (kgrp == 0) dma4(P.lse2 + (int64_t)head * P.t_loc + lrow(lane), lds_addr(sL[slot]));
    } else {
      dma_rows<DV, kThreads>(sO[slot], [&](int r) { return ogb + ((int64_t)lrow(r) * P.hq + head) * (DV * 2); },
                             rtid, kgrp);
      if (kgrp == 0)
        dma4(P.delta + (int64_t)head * P.t_loc + lrow(lane), lds_addr(sD[slot]));
      else if (kgrp == 1)
        dma16(P.t.row_iv + (int64_t)lrow(lane) * 4, lds_addr(sIv[slot]));
    }
  };
  auto wait_for = [&](int m) {
    const int later = min(m + NS - 1, n_tiles) - (m + 1);
    wait_vmem_le(later > 0 ? later * per_batch : 0);
  };

  QO qo;
  OO oo;
  qo.init(lane);
  oo.init(lane);

  const float sl2 = P.scale_log2;

  Cur cI0 = span_at(Cur{0, 0, 0, 0, 0, 0}, sp_last);
  for (int m = 0; m < NS - 1 && m < n_tiles; ++m) {
    issue(cI0, m);
    cI0 = advance(cI0);
  }
  wait_for(0);
  __syncthreads();

  // The tile loop is instantiated once per role, so that each role keeps its
  // accumulators in registers of its own across iterations.
  auto run = [&](auto role_c) {
  constexpr bool DSW = decltype(role_c)::value;
  f32x16_t acc[NA];  // dV^T (P wave) or dK^T (dS wave): lane holds d = 32*blk + 8i + 4*half + j
#pragma unroll
  for (int d = 0; d < NA; ++d) acc[d] = zero16();
  Cur cI = cI0;
  Cur cC = span_at(Cur{0, 0, 0, 0, 0, 0}, sp_last);
  for (int n = 0; n < n_tiles; ++n) {
    const int slot = n % NS;
    const char* q_s = sQ[slot];
    const char* o_s = sO[slot];
    const bool isB = (cC.seg & 1) != 0;
    const int q_rem = (isB ? qlenB : qlenA) - cC.qt * BQ;  // valid rows of this tile
    [[maybe_unused]] const int qpos_t = (isB ? segB[6] : segA[6]) + cC.qt * BQ;  // its first query (dropout)
    if constexpr (!DSW) {
      // ---- P wave: S, P (phase 1); dV (phase 2) ----
      uint32_t pk[BQ / 32][2][4];
      auto phase1 = [&](auto part_c) {
        constexpr bool PART = decltype(part_c)::value;
        if constexpr (PART) {
          // lane q: bit kk set when query q of the tile sees key k0 + 32*kgrp + kk
          const int4 iv = *(const int4*)(sIv[slot] + 4 * lane);
          const int kb = k0 + kgrp * 32;
          const uint32_t m = lane < q_rem ? key_bits(iv.x - kb, iv.y - kb) | key_bits(iv.z - kb, iv.w - kb) : 0u;
          sMask[kgrp][lane] = m;
          // read back by the same wave only: LDS operations of one wave run in order
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        // S of both query halves first, ahead of the partner's dP MFMAs, so that
        // the exponentials below overlap them
        // (the two query halves' chains alternate, so that consecutive MFMAs are independent)
        f32x16_t sc[BQ / 32];
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int qs = 0; qs < BQ / 32; ++qs) sc[qs] = zero16();
#pragma unroll
        for (int st = 0; st < QS; ++st)
#pragma unroll
          for (int qs = 0; qs < BQ / 32; ++qs) sc[qs] = E::mfma32(as_vec8<E>(qo.row(q_s, qs, st)), frag[st], sc[qs]);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int qs = 0; qs < BQ / 32; ++qs) {
          // lane holds query qs*32 + 8i + 4*half + j (r = 4i + j) for its key
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const int i0 = r >> 2;
            const f32x4_t lv = *(const f32x4_t*)(sL[slot] + qs * 32 + 8 * i0 + 4 * half);
            u32x2_t mq = {~0u, ~0u};
            if constexpr (PART) mq = *(const u32x2_t*)(sMask[kgrp] + qs * 32 + 8 * i0 + 4 * half + (r & 3));
            float pv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              float x = fmaf(sc[qs][r + u], sl2, -lv[(r + u) & 3]);
              if constexpr (PART) x = ((mq[u] >> col) & 1u) ? x : -INFINITY;
              pv[u] = __builtin_amdgcn_exp2f(x);
            }
            pk[qs][r >> 3][(r & 7) >> 1] = pack2<E>(pv[0], pv[1]);
          }
          // dropout: the P handed to the dS wave carries a set sign bit on every
          // dropped pair (P >= 0); this wave's dV takes P with the dropped pairs zeroed
          // (dropout: the first query half's mask is formed here; the second
          // half's by the dS wave, which has slack in this phase, see below)
          [[maybe_unused]] uint32_t keepw[2][4];
          if (DROP && qs == 0) {
            // byte j of qb[i0]: the random byte of this lane's key and query
            // qs*32 + 8 i0 + 4 half + j of the tile
            uint32_t qb[4];
            drop_bytes_s(qb, P.drop.seed_lo, P.drop.seed_hi, seq, kvh * P.group + cC.hh, k0 + kgrp * 32,
                         qpos_t + qs * 32, lane);
#pragma unroll
            for (int i0 = 0; i0 < 4; ++i0) {
              uint32_t kw = 0;  // bit j: query 8 i0 + 4 half + j kept
#pragma unroll
              for (int j = 0; j < 4; ++j) kw |= (drop_keep(qb[i0], j, P.drop.t) ? 1u : 0u) << j;
              // elements r = 4 i0 + 0..3 sit in pk[qs][i0 / 2] words 2 (i0 % 2) and 2 (i0 % 2) + 1
#pragma unroll
              for (int h = 0; h < 2; ++h)
                keepw[i0 >> 1][2 * (i0 & 1) + h] =
                    (((kw >> (2 * h)) & 1u) ? 0x0000FFFFu : 0u) | (((kw >> (2 * h + 1)) & 1u) ? 0xFFFF0000u : 0u);
            }
          }
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            if (DROP && qs == 0) {
              sP[kgrp][qs][st][lane] =
                  u32x4_t{pk[qs][st][0] | (~keepw[st][0] & 0x80008000u), pk[qs][st][1] | (~keepw[st][1] & 0x80008000u),
                          pk[qs][st][2] | (~keepw[st][2] & 0x80008000u), pk[qs][st][3] | (~keepw[st][3] & 0x80008000u)};
#pragma unroll
              for (int w = 0; w < 4; ++w) pk[qs][st][w] &= keepw[st][w];
            } else {
              sP[kgrp][qs][st][lane] = u32x4_t{pk[qs][st][0], pk[qs][st][1], pk[qs][st][2], pk[qs][st][3]};
            }
          }
        }
      };
      if (cC.partial) phase1(std::true_type{});
      else phase1(std::false_type{});
      __syncthreads();  // P is in LDS
      if constexpr (DROP) {  // the second query half's keep bits from the dS wave
        const uint32_t kb = sKeep[kgrp][lane];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int r = 8 * st + 2 * w;  // elements r, r + 1 of the half
            pk[1][st][w] &= (((kb >> r) & 1u) ? 0x0000FFFFu : 0u) | (((kb >> (r + 1)) & 1u) ? 0xFFFF0000u : 0u);
          }
      }
#pragma unroll
      for (int qs = 0; qs < BQ / 32; ++qs)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int rows0 = qs * 32 + st * 16;
          const typename E::vec8 bp = as_vec8<E>(u32x4_t{pk[qs][st][0], pk[qs][st][1], pk[qs][st][2], pk[qs][st][3]});
          u32x2_t ta[DV / 32][2];
#pragma unroll
          for (int d = 0; d < DV / 32; ++d) {
            ta[d][0] = oo.trans(o_s, rows0, 0, d);
            ta[d][1] = oo.trans(o_s, rows0, 1, d);
          }
#pragma unroll
          for (int d = 0; d < DV / 32; ++d)
            acc[d] = E::mfma32(as_vec8<E>(u32x4_t{ta[d][0][0], ta[d][0][1], ta[d][1][0], ta[d][1][1]}), bp, acc[d]);
        }
      if (n + NS - 1 < n_tiles) issue(cI, n + NS - 1);  // into the slot tile n-1 used
    } else {
      // ---- dS wave: dP (phase 1); dS, dK (phase 2) ----
      // the two query halves' chains alternate, so that consecutive MFMAs are independent
      f32x16_t dp[BQ / 32];
#pragma unroll
      for (int qs = 0; qs < BQ / 32; ++qs) dp[qs] = zero16();
#pragma unroll
      for (int st = 0; st < VS; ++st)
#pragma unroll
        for (int qs = 0; qs < BQ / 32; ++qs) dp[qs] = E::mfma32(as_vec8<E>(oo.row(o_s, qs, st)), frag[st], dp[qs]);
      if (n + NS - 1 < n_tiles) issue(cI, n + NS - 1);  // into the slot tile n-1 used
      // dropout: the keep bits of the second query half (bit 4 i0 + j: query
      // 32 + 8 i0 + 4 half + j of the tile), for this wave's dS and, through
      // LDS, its partner's dV
      [[maybe_unused]] uint32_t kbits1 = 0;
      if constexpr (DROP) {
        uint32_t qb[4];
        drop_bytes_s(qb, P.drop.seed_lo, P.drop.seed_hi, seq, kvh * P.group + cC.hh, k0 + kgrp * 32,
                     qpos_t + 32, lane);
#pragma unroll
        for (int i0 = 0; i0 < 4; ++i0)
#pragma unroll
          for (int j = 0; j < 4; ++j) kbits1 |= (drop_keep(qb[i0], j, P.drop.t) ? 1u : 0u) << (4 * i0 + j);
        sKeep[kgrp][lane] = kbits1;
      }
      __syncthreads();  // P is in LDS
#pragma unroll
      for (int qs = 0; qs < BQ / 32; ++qs) {
        uint32_t pd[2][4];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4_t pw = sP[kgrp][qs][st][lane];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int r = 8 * st + 2 * w;  // elements r, r+1: queries 8i + 4*half + j, r = 4i + j
            const f32x4_t dv4 = *(const f32x4_t*)(sD[slot] + qs * 32 + 8 * (r >> 2) + 4 * half);
            if (DROP && qs == 0) {  // a set sign bit marks a dropped pair: no gradient through dP
              const float p0 = E::to_float((uint16_t)(pw[w] & 0x7FFFu));
              const float p1 = E::to_float((uint16_t)((pw[w] >> 16) & 0x7FFFu));
              const float d0 = (pw[w] & 0x8000u) ? 0.f : dp[qs][r] * P.drop.scale;
              const float d1 = (pw[w] & 0x80000000u) ? 0.f : dp[qs][r + 1] * P.drop.scale;
              pd[st][w] = pack2<E>(p0 * (d0 - dv4[r & 3]), p1 * (d1 - dv4[(r + 1) & 3]));
            } else if (DROP) {  // second half: this wave's own keep bits
              const float p0 = E::to_float((uint16_t)(pw[w] & 0xFFFFu));
              const float p1 = E::to_float((uint16_t)(pw[w] >> 16));
              const float d0 = ((kbits1 >> r) & 1u) ? dp[qs][r] * P.drop.scale : 0.f;
              const float d1 = ((kbits1 >> (r + 1)) & 1u) ? dp[qs][r + 1] * P.drop.scale : 0.f;
              pd[st][w] = pack2<E>(p0 * (d0 - dv4[r & 3]), p1 * (d1 - dv4[(r + 1) & 3]));
            } else {
              const float p0 = E::to_float((uint16_t)(pw[w] & 0xFFFFu));
              const float p1 = E::to_float((uint16_t)(pw[w] >> 16));
              pd[st][w] = pack2<E>(p0 * (dp[qs][r] - dv4[r & 3]), p1 * (dp[qs][r + 1] - dv4[(r + 1) & 3]));
            }
          }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int rows0 = qs * 32 + st * 16;
          const typename E::vec8 bd = as_vec8<E>(u32x4_t{pd[st][0], pd[st][1], pd[st][2], pd[st][3]});
          u32x2_t ta[DQK / 32][2];
#pragma unroll
          for (int d = 0; d < DQK / 32; ++d) {
            ta[d][0] = qo.trans(q_s, rows0, 0, d);
            ta[d][1] = qo.trans(q_s, rows0, 1, d);
          }
#pragma unroll
          for (int d = 0; d < DQK / 32; ++d)
            acc[d] = E::mfma32(as_vec8<E>(u32x4_t{ta[d][0][0], ta[d][0][1], ta[d][1][0], ta[d][1][1]}), bd, acc[d]);
        }
      }
    }
    if (n + NS - 1 < n_tiles) cI = advance(cI);
    cC = advance(cC);
    if (n + 1 < n_tiles) wait_for(n + 1);
    __syncthreads();
  }
  wait_vmem_all();

  // ---- write this lane's key row of dV (P wave) or dK (dS wave) ----
  if (kvalid) {
    if constexpr (DSW) {
      uint16_t* dkr = (uint16_t*)P.dk + (grow * P.hkv + kvh) * DQK;
      const float sc = P.scale;
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dd = d * 32 + 8 * i + 4 * half;
          *(u32x2_t*)(dkr + dd) = u32x2_t{pack2<E>(acc[d][4 * i] * sc, acc[d][4 * i + 1] * sc),
                                           pack2<E>(acc[d][4 * i + 2] * sc, acc[d][4 * i + 3] * sc)};
        }
    } else {
      uint16_t* dvr = (uint16_t*)P.dv + (grow * P.hkv + kvh) * DV;
      const float sc = DROP ? P.drop.scale : 1.f;  // dropout: kept probabilities are scaled
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dd = d * 32 + 8 * i + 4 * half;
          *(u32x2_t*)(dvr + dd) = u32x2_t{pack2<E>(acc[d][4 * i] * sc, acc[d][4 * i + 1] * sc),
                                           pack2<E>(acc[d][4 * i + 2] * sc, acc[d][4 * i + 3] * sc)};
        }
    }
  }
  };
  if (dswave) run(std::true_type{});
  else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// dQ, Q-stationary (Q/K head dim up to 128; 192 runs dq_pair_kernel below).
// A work-group holds 32 query rows of 4/heads_per_tile row
// blocks x heads_per_tile heads of one K/V group (one wave each; Q and dO of the
// lane's query in registers) and walks the 64-key K/V tiles of its schedule.  K
// and V stream through an NS-deep LDS ring by direct-to-LDS loads issued NS-1
// tiles ahead; the prefix-index entries of each tile come through a ring of
// their own, fetched 2NS-1 tiles ahead so that the loads never wait on them.
// Per 32 keys:  S^T = K Q^T, dP^T = V dO^T (A = K / V rows from LDS),
// dS^T = P^T (dP^T - Delta),  dQ^T += K^T dS^T (A = transposing reads of K).
// ---------------------------------------------------------------------------
template <int DQK>
constexpr int kDqStages = 2;
template <int DQK>
constexpr int kDqBlocksPerCu = 2;

template <typename E, int DQK, int DV, bool DROP>
__global__ __launch_bounds__(kThreads, kDqBlocksPerCu<DQK>) void dq_kernel(BwdParams P) {
  const int n_dq_wg = P.n_dq_tiles * P.dq_head_groups;
  if ((int)blockIdx.x >= n_dq_wg) {  // the grid's last work-groups do the zero fill
    zero_rows_block<DQK, DV>(P, (int)blockIdx.x - n_dq_wg);
    return;
  }
  constexpr int BN = kDqTileKv;
  constexpr int QS = DQK / 16, VS = DV / 16;
  constexpr int NS = kDqStages<DQK>;
  constexpr int NIR = 2 * NS;  // index ring slots
  using KO = TileOffsets<DQK>;
  using VO = TileOffsets<DV>;
  constexpr int CHK = KO::RB / 16, CHV = VO::RB / 16;  // 16-byte chunks per LDS row
  constexpr int NK = BN * CHK / kThreads, NV = BN * CHV / kThreads;
  constexpr bool kSharedRows = CHK == CHV;
  constexpr int NI = kSharedRows ? NK : NK + NV;
  static_assert(BN == 64, "the index fetch covers 64 keys per tile");
  __shared__ __attribute__((aligned(16))) char sK[NS][BN * KO::RB];
  __shared__ __attribute__((aligned(16))) char sV[NS][BN * VO::RB];
  __shared__ __attribute__((aligned(16))) int32_t sIdx[NIR][BN];
  __shared__ __attribute__((aligned(16))) int32_t sSpan[kDqMaxSpans * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;

  const int tile = blockIdx.x / P.dq_head_groups;
  const int hg = blockIdx.x % P.dq_head_groups;
  const int32_t* tr = P.t.dq_tiles + tile * 5;
  const int seg = tr[0], q0 = tr[1], rows = tr[2], span0 = tr[3], nspan = tr[4];
  const int32_t* sg = P.t.segs + seg * 8;
  const int kv_len = sg[3], q_row0 = sg[4], kv_off = sg[5];
  const int hpt = P.dq_heads_per_tile;
  const int head = hg * hpt + (wave % hpt);
  const int kvh = head / P.group;
  const int a = q0 + (wave / hpt) * 32 + col;
  const bool valid = a < q0 + rows;  // the tile's own rows (a tile may end inside its segment)
  const int row = q_row0 + a;
  [[maybe_unused]] const int seq = sg[0], qpos = sg[6] + a;  // sequence, in-sequence query position (dropout)

  const char* kg = (const char*)P.k + (int64_t)kvh * DQK * 2;
  const char* vg = (const char*)P.v + (int64_t)kvh * DV * 2;
  const uint32_t kstride = (uint32_t)P.hkv * DQK * 2, vstride = (uint32_t)P.hkv * DV * 2;
  const int32_t* __restrict__ kvi = P.t.kv_index + kv_off;

  // Q^T and dO^T operands in registers: lane holds row[16s + 8*half .. +7]
  typename E::vec8 qf[QS], of[VS];
  {
    const uint16_t* qr = (const uint16_t*)P.q + ((int64_t)row * P.hq + head) * DQK + 8 * half;
    const uint16_t* orr = (const uint16_t*)P.dout + ((int64_t)row * P.hq + head) * DV + 8 * half;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (valid) x = *(const u32x4_t*)(qr + 16 * s);
      qf[s] = as_vec8<E>(x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (valid) x = *(const u32x4_t*)(orr + 16 * s);
      of[s] = as_vec8<E>(x);
    }
  }
  // The backward preprocess of this lane's (row, head): Delta = rowsum(dO * O)
  // (each half-wave holds half of the row; the halves are summed across lanes
  // l and l + 32) and LSE * log2(e).  Both go to the workspace for the dK/dV
  // kernel, which runs after this one.
  u32x4_t ov[VS];
  int lo1 = 0, hi1 = 0, lo2 = 0, hi2 = 0;
  float lse2 = INFINITY;
  if (valid) {
    const uint16_t* orow = (const uint16_t*)P.o + ((int64_t)row * P.hq + head) * DV + 8 * half;
#pragma unroll
    for (int s = 0; s < VS; ++s) ov[s] = *(const u32x4_t*)(orow + 16 * s);
    const int32_t* iv = P.t.row_iv + (int64_t)row * 4;
    lo1 = iv[0]; hi1 = iv[1]; lo2 = iv[2]; hi2 = iv[3];
    lse2 = P.lse[(int64_t)head * P.t_loc + row] * kLog2e;
  }
  if (tid < 4 * nspan) sSpan[tid] = P.t.dq_spans[span0 * 4 + tid];
  wait_vmem_all();
  float dsum = 0.f;
  if (valid) {
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      const u32x4_t g = __builtin_bit_cast(u32x4_t, of[s]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dsum = fmaf(E::to_float((uint16_t)(ov[s][w] & 0xFFFFu)), E::to_float((uint16_t)(g[w] & 0xFFFFu)), dsum);
        dsum = fmaf(E::to_float((uint16_t)(ov[s][w] >> 16)), E::to_float((uint16_t)(g[w] >> 16)), dsum);
      }
    }
  }
  const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(dsum), __float_as_uint(dsum), false, false);
  const float delta = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
  if (valid && half == 0) {
    P.delta[(int64_t)head * P.t_loc + row] = delta;
    P.lse2[(int64_t)head * P.t_loc + row] = lse2;
  }
  __syncthreads();
  int n_tiles = 0;
  for (int sp = 0; sp < nspan; ++sp) {
    const int4 r = *(const int4*)(sSpan + 4 * sp);
    n_tiles += __builtin_amdgcn_readfirstlane(r.y) - __builtin_amdgcn_readfirstlane(r.x);
  }

  // ---- cursor over the work item's K/V tiles ----
  struct Cur {
    int sp, t, t_end, partial;
  };
  auto span_at = [&](int sp) {
    const int4 r = *(const int4*)(sSpan + 4 * sp);
    return Cur{sp, __builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
               __builtin_amdgcn_readfirstlane(r.z)};
  };
  auto advance = [&](Cur c) {
    if (++c.t >= c.t_end && c.sp + 1 < nspan) c = span_at(c.sp + 1);
    return c;
  };

  // ---- streaming.  batch(m): K and V of tile m into ring slot m % NS (all waves)
  // and, by wave 0, the prefix-index entries of tile m + NIR - 1 (clamped to a
  // valid address when that tile does not exist: the slot is then never read).
  Cur cF = nspan > 0 ? span_at(0) : Cur{0, 0, 0, 0};  // next tile whose indices get fetched
  int next_f = 0;
  auto fetch_idx = [&]() {
    const int kb0 = next_f < n_tiles ? cF.t * BN : 0;
    dma4(kvi + min(kb0 + lane, kv_len - 1), lds_addr(sIdx[next_f % NIR]));
    if (next_f < n_tiles) cF = advance(cF);
    ++next_f;
  };
  const int per_batch = NK + NV + (wave == 0 ? 1 : 0);  // loads per wave and batch
  auto issue = [&](int m) {
    const int32_t* si = sIdx[m % NIR];
    int idx[NI];
#pragma unroll
    for (int i = 0; i < NK; ++i) idx[i] = si[(i * kThreads + tid) / CHK];
    if constexpr (!kSharedRows) {
#pragma unroll
      for (int i = 0; i < NV; ++i) idx[NK + i] = si[(i * kThreads + tid) / CHV];
    }
    const uint32_t kl = lds_addr(sK[m % NS]) + (uint32_t)wave * 64 * 16;
    const uint32_t vl = lds_addr(sV[m % NS]) + (uint32_t)wave * 64 * 16;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int s = i * kThreads + tid;
      int c = (s % CHK) ^ bwd_swz<KO::RB>(s / CHK);
      if (c >= DQK / 8) c = 0;  // row padding: any in-bounds source
      dma16(kg + ((uint64_t)(uint32_t)idx[i] * kstride + c * 16), kl + i * kThreads * 16);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int s = i * kThreads + tid;
      int c = (s % CHV) ^ bwd_swz<VO::RB>(s / CHV);
      if (c >= DV / 8) c = 0;
      const int id = kSharedRows ? idx[i] : idx[NK + i];
      dma16(vg + ((uint64_t)(uint32_t)id * vstride + c * 16), vl + i * kThreads * 16);
    }
    if (wave == 0) fetch_idx();
  };
  // wait until tile m's batch has landed; the batches issued after it (tiles
  // m+1 .. m+NS-2, those that exist) may stay in flight
  auto wait_for = [&](int m) {
    const int later = min(m + NS - 1, n_tiles) - (m + 1);
    wait_vmem_le(later > 0 ? later * per_batch : 0);
  };

  KO ko;
  VO vo;
  ko.init(lane);
  vo.init(lane);

  f32x16_t acc[DQK / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) acc[d] = zero16();
  const float sl2 = P.scale_log2;

  if (n_tiles > 0) {
    if (wave == 0)
      for (int m = 0; m < NIR - 1; ++m) fetch_idx();
    wait_vmem_all();
    __syncthreads();
    for (int m = 0; m < NS - 1 && m < n_tiles; ++m) {
      issue(m);
      __syncthreads();  // batch m+1 overwrites the index slot batch m has just read
    }
    wait_for(0);
    __syncthreads();
  }
  Cur cC = nspan > 0 ? span_at(0) : Cur{0, 0, 0, 0};  // tile being computed
  for (int n = 0; n < n_tiles; ++n) {
    if (n + NS - 1 < n_tiles) issue(n + NS - 1);  // into the slot tile n-1 used
    const char* k_s = sK[n % NS];
    const char* v_s = sV[n % NS];
    const int kb0 = cC.t * BN;
    const bool partial = cC.partial != 0;
#pragma unroll
    for (int nb = 0; nb < BN / 32; ++nb) {
      // the S and dP chains alternate, so that consecutive MFMAs are independent
      f32x16_t s = zero16(), dp = zero16();
#pragma unroll
      for (int st = 0; st < (QS > VS ? QS : VS); ++st) {
        if (st < QS) s = E::mfma32(as_vec8<E>(ko.row(k_s, nb, st)), qf[st], s);
        if (st < VS) dp = E::mfma32(as_vec8<E>(vo.row(v_s, nb, st)), of[st], dp);
      }
      // lane holds keys nb*32 + 8i + 4*half + j (r = 4i + j) for its query
      if constexpr (DROP) {
        // dropout: a dropped pair passes no gradient through dP, a kept one is
        // scaled; the random word u[i] of keys nb*32 + 8i + 4*half + 0..3 covers r = 4i..4i+3
        uint32_t u[4];
        drop_words_st(u, P.drop.seed_lo, P.drop.seed_hi, seq, head, qpos - col, kb0 + nb * 32, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dp[4 * i + j] = drop_keep(u[i], j, P.drop.t) ? dp[4 * i + j] * P.drop.scale : 0.f;
      }
      uint32_t pd[2][4];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float dsv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float x = fmaf(s[r + u], sl2, -lse2);
          if (partial) {
            const int b = kb0 + nb * 32 + 8 * ((r + u) >> 2) + 4 * half + ((r + u) & 3);
            const bool vis = ((b >= lo1) & (b < hi1)) | ((b >= lo2) & (b < hi2));
            x = vis ? x : -INFINITY;
          }
          const float p = __builtin_amdgcn_exp2f(x);
          dsv[u] = p * (dp[r + u] - delta);
        }
        pd[r >> 3][(r & 7) >> 1] = pack2<E>(dsv[0], dsv[1]);
      }
      // dQ^T[d][q] += sum_key K^T[d][key] dS^T[key][q]
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int rows0 = nb * 32 + st * 16;
        const typename E::vec8 bd = as_vec8<E>(u32x4_t{pd[st][0], pd[st][1], pd[st][2], pd[st][3]});
#pragma unroll
        for (int d = 0; d < DQK / 32; ++d) {
          const u32x2_t lo = ko.trans(k_s, rows0, 0, d);
          const u32x2_t hi = ko.trans(k_s, rows0, 1, d);
          acc[d] = E::mfma32(as_vec8<E>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), bd, acc[d]);
        }
      }
    }
    cC = advance(cC);
    if (n + 1 < n_tiles) wait_for(n + 1);
    __syncthreads();
  }
  wait_vmem_all();

  if (valid) {
    uint16_t* dqr = (uint16_t*)P.dq + ((int64_t)row * P.hq + head) * DQK;
    const float sc = P.scale;
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dd = d * 32 + 8 * i + 4 * half;
        *(u32x2_t*)(dqr + dd) = u32x2_t{pack2<E>(acc[d][4 * i] * sc, acc[d][4 * i + 1] * sc),
                                         pack2<E>(acc[d][4 * i + 2] * sc, acc[d][4 * i + 3] * sc)};
      }
  }
}

template <typename E, int DQK, int DV>
hipError_t launch_all(const BwdParams& p, hipStream_t s, LaunchHook* hook) {
  hipError_t e = hipSuccess;
  auto launch = [&](int id, auto kernel, unsigned grid, unsigned threads = kThreads) {
    if (e != hipSuccess || grid == 0) return;
    if (hook) hook->before(id, s);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, p);
    if (hook) hook->after(id, s);
    e = hipGetLastError();
  };
  // dQ first: it also forms Delta and LSE * log2(e), which dK/dV read, and its
  // last n_zero_ranges work-groups zero the dK/dV rows no local query sees
  const unsigned dq_grid = (unsigned)p.n_dq_tiles * (unsigned)p.dq_head_groups + (unsigned)p.n_zero_ranges;
  const unsigned kv_grid = (unsigned)p.n_kv_tiles * (unsigned)p.hkv;
  if (p.drop.t != 0) {  // attention dropout
    if constexpr (DQK > 128)
      launch(K_BWD_DQ, dq_pair_kernel<E, DQK, DV, true>, dq_grid, 2 * kThreads);
    else
      launch(K_BWD_DQ, dq_kernel<E, DQK, DV, true>, dq_grid);
    launch(K_BWD_DKDV, dkdv_pair_kernel<E, DQK, DV, true>, kv_grid, 2 * kThreads);
    return e;
  }
  if constexpr (DQK > 128)
    launch(K_BWD_DQ, dq_pair_kernel<E, DQK, DV, false>, dq_grid, 2 * kThreads);
  else
    launch(K_BWD_DQ, dq_kernel<E, DQK, DV, false>, dq_grid);
  launch(K_BWD_DKDV, dkdv_pair_kernel<E, DQK, DV, false>, kv_grid, 2 * kThreads);
  return e;
}

}  // namespace

// Device memory of the allocation-free backward (cva_bwd_noalloc): the per-row
// statistics Delta and LSE*log2(e) that the dQ kernel writes and the dK/dV
// kernel reads, held by the library for the life of the process on every GPU
// it runs on.  Host code never names this array in a kernel argument or copy:
// it uses the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[kBwdNoAllocScratchBytes / sizeof(float)];

hipError_t bwd_noalloc_scratch(hipStream_t stream, float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // first use on this device: look the array up with the device current
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (a == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = (float*)addr[dev];
  return hipSuccess;
}

hipError_t launch_bwd(int dtype, int d_qk, int d_v, const BwdParams& p, hipStream_t s,
                      LaunchHook* h) {
  if (dtype == 0) {
    if (d_qk == 64 && d_v == 64) return launch_all<Bf16, 64, 64>(p, s, h);
    if (d_qk == 128 && d_v == 128) return launch_all<Bf16, 128, 128>(p, s, h);
    if (d_qk == 192 && d_v == 128) return launch_all<Bf16, 192, 128>(p, s, h);
  } else if (dtype == 1) {
    if (d_qk == 64 && d_v == 64) return launch_all<Fp16, 64, 64>(p, s, h);
    if (d_qk == 128 && d_v == 128) return launch_all<Fp16, 128, 128>(p, s, h);
    if (d_qk == 192 && d_v == 128) return launch_all<Fp16, 192, 128>(p, s, h);
  }
  return hipErrorInvalidValue;
}

}  // namespace cva
