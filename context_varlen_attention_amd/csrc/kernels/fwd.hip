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
// MFMA formulation.  A work-group is 4 waves; each wave owns 32 query rows of
// one head.  The kernel computes the transposed scores S^T = K Q^T with
// v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q from registers), so every lane
// ends up holding 16 keys of ONE query column: the softmax statistics are
// lane-local, plus one exchange with the lane 32 apart.  The output is kept
// transposed too, O^T = V^T P^T, with P^T taken straight from the S^T
// accumulators (the MFMA's reduction slots are permuted to match the layout the
// accumulators already have) and V^T staged in LDS by a register transpose
// during the tile load.  K/V rows are gathered through the prefix index while
// they are loaded (the index_select of the RFC, never materialised).
#include "common.hpp"
#include "launch.hpp"

namespace cva {

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 64;  // keys per K/V tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units: stale row max may lag by up to 2^8

// Issue the direct-to-LDS loads of K tile rows kb0..kb0+63 (rows past the
// prefix re-read its last row; those keys are masked).  Slot s of the tile holds
// row s / CH, logical 16-byte chunk (s % CH) ^ (row & 7): the XOR swizzle keeps the
// MFMA operand reads conflict-free without padding.
template <int DQK>
__device__ inline void load_k_tile(uint16_t* sk, const uint16_t* __restrict__ kg, const int32_t* kvi,
                                   int kb0, int kv_len, int hkv, int kvh, int tid) {
  constexpr int CH = DQK / 8;
  constexpr int SLOTS = kBN * CH;
  const int wave_base = tid & ~63;
#pragma unroll
  for (int i = 0; i < SLOTS / kThreads; ++i) {
    const int s = i * kThreads + tid;
    const int r = s / CH;
    const int c = (s % CH) ^ (r & 7);
    const int b = min(kb0 + r, kv_len - 1);
    const int64_t g = kvi[b];
    const uint16_t* src = kg + (g * hkv + kvh) * DQK + c * 8;
    __builtin_amdgcn_global_load_lds(
        (const void*)src,
        (__attribute__((address_space(3))) void*)(sk + (size_t)(i * kThreads + wave_base) * 8), 16, 0, 0);
  }
}

// V tile: thread (group g of 16 keys, half h, 8-dim chunk c) loads the 8 key
// rows of its reduction slots; they are transposed in registers later.
template <int DV>
__device__ inline void load_v_regs(u32x4_t (&vr)[8], const uint16_t* __restrict__ vg, const int32_t* kvi,
                                   int kb0, int kv_len, int hkv, int kvh, int tid) {
  constexpr int CH = DV / 8;
  if (tid >= (kBN / 8) * CH) return;
  const int c = tid % CH, gh = tid / CH;  // gh = 2 * group + half
  const int g = gh >> 1, h = gh & 1;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int key = 16 * g + (m < 4 ? 4 * h + m : 8 + 4 * h + (m - 4));
    const int b = min(kb0 + key, kv_len - 1);
    const int64_t row = kvi[b];
    vr[m] = *(const u32x4_t*)(vg + (row * hkv + kvh) * DV + c * 8);
  }
}

template <int DV>
__device__ inline void store_vt(uint16_t* svt, const u32x4_t (&vr)[8], int tid) {
  constexpr int CH = DV / 8;
  constexpr int VT_LD = kBN + 8;
  if (tid >= (kBN / 8) * CH) return;
  const int c = tid % CH, gh = tid / CH;
  const int g = gh >> 1, h = gh & 1;
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const int w = dd >> 1;
    const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
    u32x4_t out;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = __builtin_amdgcn_perm(vr[2 * j + 1][w], vr[2 * j][w], sel);
    *(u32x4_t*)(svt + (8 * c + dd) * VT_LD + 16 * g + 8 * h) = out;
  }
}

template <typename E, int DQK, int DV>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_kernel(FwdParams P) {
  constexpr int KSTEPS = DQK / 16;  // 16-wide reduction steps of S^T
  constexpr int DB = DV / 32;       // 32-row blocks of O^T
  constexpr int KCH = DQK / 8;
  constexpr int VT_LD = kBN + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBN * DQK];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][DV * VT_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  const int tile = blockIdx.x / P.n_head_groups;
  const int hg = blockIdx.x % P.n_head_groups;
  const int32_t* tr = P.t.fwd_tiles + tile * 5;
  const int seg = tr[0], q0 = tr[1], span0 = tr[3], nspan = tr[4];
  const int32_t* sg = P.t.segs + seg * 8;
  const int q_len = sg[2], kv_len = sg[3], q_row0 = sg[4], kv_off = sg[5];
  const int hpt = P.heads_per_tile;
  const int head = hg * hpt + (wave % hpt);
  const int kvh = head / P.group;
  const int a = q0 + (wave / hpt) * 32 + col;  // segment-relative query index of this lane
  const bool valid = a < q_len;
  const int row = q_row0 + a;                   // local row

  const uint16_t* __restrict__ kg = (const uint16_t*)P.k;
  const uint16_t* __restrict__ vg = (const uint16_t*)P.v;
  const int32_t* __restrict__ kvi = P.t.kv_index + kv_off;
  const int32_t* __restrict__ spans = P.t.fwd_spans + span0 * 4;

  // Q fragments: lane holds Q[row][16t + 8*half .. +7] for every step t.
  typename E::vec8 qf[KSTEPS];
  {
    const uint16_t* qrow = (const uint16_t*)P.q + ((int64_t)row * P.hq + head) * DQK + 8 * half;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (valid) x = *(const u32x4_t*)(qrow + 16 * t);
      qf[t] = as_vec8<E>(x);
    }
  }
  int lo1 = 0, hi1 = 0, lo2 = 0, hi2 = 0;
  if (valid) {
    const int32_t* iv = P.t.row_iv + (int64_t)row * 4;
    lo1 = iv[0]; hi1 = iv[1]; lo2 = iv[2]; hi2 = iv[3];
  }

  float m_run = -INFINITY, m_base = 0.f, l_run = 0.f;
  f32x16_t acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = zero16();
  const float sl2 = P.scale_log2;

  if (nspan == 0) {  // no visible key for any row of the tile (unreachable for the supported masks)
    if (valid) {
      uint16_t* orow = (uint16_t*)P.o + ((int64_t)row * P.hq + head) * DV;
      for (int d = half; d < DV; d += 2) orow[d] = 0;
      if (half == 0) P.lse[(int64_t)head * P.t_loc + row] = -INFINITY;
    }
    return;
  }
  // V^T tile layout: in every 16-key group, the two half-waves' reduction slots
  // {4h..4h+3, 8+4h..8+4h+3} are stored as one contiguous 8-element run, so each
  // PV operand is a single 16-byte read.
  // walk the spans' tiles as one sequence, double-buffered
  int sp = 0, t = spans[0], t_end = spans[1];
  bool partial = spans[2] != 0;
  u32x4_t vr[8];
  load_k_tile<DQK>(sK[0], kg, kvi, t * kBN, kv_len, P.hkv, kvh, tid);
  load_v_regs<DV>(vr, vg, kvi, t * kBN, kv_len, P.hkv, kvh, tid);
  store_vt<DV>(sVt[0], vr, tid);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int buf = 0;; buf ^= 1) {
    // next tile of the sequence
    int nsp = sp, nt = t + 1, nt_end = t_end;
    bool npartial = partial;
    if (nt >= nt_end) {
      ++nsp;
      if (nsp < nspan) {
        nt = spans[nsp * 4];
        nt_end = spans[nsp * 4 + 1];
        npartial = spans[nsp * 4 + 2] != 0;
      }
    }
    const bool has_next = nsp < nspan;
    if (has_next) {
      load_k_tile<DQK>(sK[buf ^ 1], kg, kvi, nt * kBN, kv_len, P.hkv, kvh, tid);
      load_v_regs<DV>(vr, vg, kvi, nt * kBN, kv_len, P.hkv, kvh, tid);
    }
    const int kb0 = t * kBN;
    const uint16_t* sk = sK[buf];
    const uint16_t* svt = sVt[buf];

    // ---- S^T = K Q^T for the 64 keys of the tile (two 32-key blocks) ----
    f32x16_t s[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      s[nb] = zero16();
      const int r = nb * 32 + col;
      const uint16_t* krow = sk + r * DQK;
#pragma unroll
      for (int kt = 0; kt < KSTEPS; ++kt) {
        const int c = (2 * kt + half) ^ (r & 7);
        const u32x4_t x = *(const u32x4_t*)(krow + c * 8);
        s[nb] = E::mfma32(as_vec8<E>(x), qf[kt], s[nb]);
      }
    }
    // ---- mask (partial tiles only) and running max of the raw scores ----
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[nb][r];
        if (partial) {
          const int b = kb0 + nb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = (b >= lo1 && b < hi1) || (b >= lo2 && b < hi2);
          x = vis ? x : -INFINITY;
          s[nb][r] = x;
        }
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, swap_halves(mx)) * sl2;
    // lazy rescale: move the exponent base only when the max grew by more than 2^8
    if (__ballot(mx > m_run + kRescaleThreshold) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float nb_ = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_base - nb_);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
      m_run = m_new;
      m_base = nb_;
    }
    const float nbase = -m_base;
    uint32_t pk[2][2][4];  // [nb][16-key step][packed pairs]
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[nb][r], sl2, nbase));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[nb][r + 1], sl2, nbase));
        l_run += p0 + p1;
        pk[nb][r >> 3][(r & 7) >> 1] = pack2<E>(p0, p1);
      }
    }
    // ---- O^T += V^T P^T: 4 reduction steps of 16 keys, one 16-byte V^T read each ----
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4_t pv = {pk[nb][st][0], pk[nb][st][1], pk[nb][st][2], pk[nb][st][3]};
        const typename E::vec8 bfrag = as_vec8<E>(pv);
        const int kofs = nb * 32 + st * 16 + 8 * half;
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const u32x4_t af = *(const u32x4_t*)(svt + (d * 32 + col) * VT_LD + kofs);
          acc[d] = E::mfma32(as_vec8<E>(af), bfrag, acc[d]);
        }
      }
    }
    if (!has_next) break;
    store_vt<DV>(sVt[buf ^ 1], vr, tid);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    sp = nsp; t = nt; t_end = nt_end; partial = npartial;
  }

  // ---- epilogue: normalise, write O and LSE ----
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (valid) {
    uint16_t* orow = (uint16_t*)P.o + ((int64_t)row * P.hq + head) * DV;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dd = d * 32 + 8 * i + 4 * half;
        u32x2_t w = {pack2<E>(acc[d][4 * i] * inv, acc[d][4 * i + 1] * inv),
                     pack2<E>(acc[d][4 * i + 2] * inv, acc[d][4 * i + 3] * inv)};
        *(u32x2_t*)(orow + dd) = w;
      }
    }
    if (half == 0) {
      const float lse = l_tot > 0.f ? (m_base + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
      P.lse[(int64_t)head * P.t_loc + row] = lse;
    }
  }
}

// fp32 correctness kernel: one thread per (query row, head), keys one at a time,
// plain online softmax in fp32 on the VALU.  Uses the same tile schedule.
template <int DQK, int DV>
__global__ __launch_bounds__(128) void fwd_fp32_kernel(FwdParams P) {
  const int tile = blockIdx.x / P.n_head_groups;
  const int hg = blockIdx.x % P.n_head_groups;
  const int32_t* tr = P.t.fwd_tiles + tile * 5;
  const int seg = tr[0], q0 = tr[1], span0 = tr[3], nspan = tr[4];
  const int32_t* sg = P.t.segs + seg * 8;
  const int q_len = sg[2], kv_len = sg[3], q_row0 = sg[4], kv_off = sg[5];
  const int hpt = P.heads_per_tile;
  const int head = hg * hpt + (threadIdx.x % hpt);
  const int a = q0 + threadIdx.x / hpt;
  if (a >= q_len || a >= q0 + P.tile_q) return;
  const int kvh = head / P.group;
  const int row = q_row0 + a;
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
      for (int d = 0; d < DV; ++d) acc[d] = acc[d] * alpha + p * vrow[d];
      m_run = m_new;
    }
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* orow = (float*)P.o + ((int64_t)row * P.hq + head) * DV;
  for (int d = 0; d < DV; ++d) orow[d] = acc[d] * inv;
  P.lse[(int64_t)head * P.t_loc + row] =
      l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : -INFINITY;
}

template <typename E, int DQK, int DV>
hipError_t launch_mfma(const FwdParams& p, hipStream_t s, LaunchHook* hook) {
  const unsigned grid = (unsigned)p.n_tiles * (unsigned)p.n_head_groups;
  if (grid == 0) return hipSuccess;
  if (hook) hook->before(K_FWD, s);
  hipLaunchKernelGGL((fwd_mfma_kernel<E, DQK, DV>), dim3(grid), dim3(kThreads), 0, s, p);
  if (hook) hook->after(K_FWD, s);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_fp32(const FwdParams& p, hipStream_t s, LaunchHook* hook) {
  const unsigned grid = (unsigned)p.n_tiles * (unsigned)p.n_head_groups;
  if (grid == 0) return hipSuccess;
  if (hook) hook->before(K_FWD, s);
  hipLaunchKernelGGL((fwd_fp32_kernel<DQK, DV>), dim3(grid), dim3(128), 0, s, p);
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
