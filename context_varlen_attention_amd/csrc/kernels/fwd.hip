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
constexpr int kBN = 64;

template <typename E, int DQK, int DV>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_kernel(FwdParams P) {
  constexpr int KSTEPS = DQK / 16;  // 16-wide reduction steps of S^T
  constexpr int DB = DV / 32;       // 32-row blocks of O^T
  constexpr int K_LD = DQK + 8;     // LDS row stride of K (elements), 16-byte aligned rows
  constexpr int VT_LD = kBN + 8;    // LDS row stride of V^T (elements)
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBN * K_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[DV * VT_LD];

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

  const uint16_t* __restrict__ qg = (const uint16_t*)P.q;
  const uint16_t* __restrict__ kg = (const uint16_t*)P.k;
  const uint16_t* __restrict__ vg = (const uint16_t*)P.v;
  const int32_t* __restrict__ kvi = P.t.kv_index + kv_off;

  // Q fragments: lane holds Q[row][16t + 8*half .. +7] for every step t.
  typename E::vec8 qf[KSTEPS];
  {
    const uint16_t* qrow = qg + ((int64_t)row * P.hq + head) * DQK + 8 * half;
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

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = zero16();

  const float sl2 = P.scale_log2;

  for (int sp = 0; sp < nspan; ++sp) {
    const int32_t* spr = P.t.fwd_spans + (span0 + sp) * 4;
    const int t_begin = spr[0], t_end = spr[1];
    const bool partial = spr[2] != 0;
    for (int t = t_begin; t < t_end; ++t) {
      const int kb0 = t * kBN;
      __syncthreads();
      // ---- K tile: rows kb0..kb0+63 gathered through the prefix index ----
      {
        constexpr int CH = DQK / 8;  // 16-byte chunks per row
        for (int idx = tid; idx < kBN * CH; idx += kThreads) {
          const int r = idx / CH, c = idx % CH;
          const int b = kb0 + r;
          u32x4_t x = {0u, 0u, 0u, 0u};
          if (b < kv_len) {
            const int64_t g = kvi[b];
            x = *(const u32x4_t*)(kg + (g * P.hkv + kvh) * DQK + c * 8);
          }
          *(u32x4_t*)(sK + r * K_LD + c * 8) = x;
        }
      }
      // ---- V^T tile: 4 keys x 8 dims per thread, transposed in registers ----
      {
        constexpr int CH = DV / 8;
        for (int idx = tid; idx < (kBN / 4) * CH; idx += kThreads) {
          const int g4 = idx / CH, c = idx % CH;
          u32x4_t rows[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int b = kb0 + 4 * g4 + j;
            rows[j] = u32x4_t{0u, 0u, 0u, 0u};
            if (b < kv_len) {
              const int64_t g = kvi[b];
              rows[j] = *(const u32x4_t*)(vg + (g * P.hkv + kvh) * DV + c * 8);
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            const bool hi = e & 1;
            uint32_t x0 = hi ? (rows[0][w] >> 16) : (rows[0][w] & 0xFFFFu);
            uint32_t x1 = hi ? (rows[1][w] >> 16) : (rows[1][w] & 0xFFFFu);
            uint32_t x2 = hi ? (rows[2][w] >> 16) : (rows[2][w] & 0xFFFFu);
            uint32_t x3 = hi ? (rows[3][w] >> 16) : (rows[3][w] & 0xFFFFu);
            u32x2_t out = {x0 | (x1 << 16), x2 | (x3 << 16)};
            *(u32x2_t*)(sVt + (8 * c + e) * VT_LD + 4 * g4) = out;
          }
        }
      }
      __syncthreads();

      // ---- S^T = K Q^T for the 64 keys of the tile (two 32-key blocks) ----
      f32x16_t s[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        s[nb] = zero16();
        const uint16_t* krow = sK + (nb * 32 + col) * K_LD + 8 * half;
#pragma unroll
        for (int kt = 0; kt < KSTEPS; ++kt) {
          u32x4_t x = *(const u32x4_t*)(krow + 16 * kt);
          s[nb] = E::mfma32(as_vec8<E>(x), qf[kt], s[nb]);
        }
      }
      // ---- scale, mask, running max ----
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[nb][r] * sl2;
          if (partial) {
            const int b = kb0 + nb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool vis = (b >= lo1 && b < hi1) || (b >= lo2 && b < hi2);
            x = vis ? x : -INFINITY;
          }
          s[nb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float base = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - base);
      m_run = m_new;
      float rs = 0.f;
      uint32_t pk[2][2][4];  // [nb][16-key step][packed pairs]
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(s[nb][r] - base);
          const float p1 = __builtin_amdgcn_exp2f(s[nb][r + 1] - base);
          rs += p0 + p1;
          pk[nb][r >> 3][(r & 7) >> 1] = pack2<E>(p0, p1);
        }
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;

      // ---- O^T += V^T P^T: 4 reduction steps of 16 keys ----
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4_t pv = {pk[nb][st][0], pk[nb][st][1], pk[nb][st][2], pk[nb][st][3]};
          const typename E::vec8 bfrag = as_vec8<E>(pv);
          const int kbase = nb * 32 + st * 16 + 4 * half;
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const uint16_t* vrow = sVt + (d * 32 + col) * VT_LD + kbase;
            const u32x2_t lo = *(const u32x2_t*)(vrow);
            const u32x2_t hi = *(const u32x2_t*)(vrow + 8);
            const u32x4_t af = {lo[0], lo[1], hi[0], hi[1]};
            acc[d] = E::mfma32(as_vec8<E>(af), bfrag, acc[d]);
          }
        }
      }
    }
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
      const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
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
