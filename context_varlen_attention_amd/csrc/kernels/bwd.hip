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
//   bwd_pre_kernel    Delta[h, row] in fp32 (HBM-bound, tiny)
//   zero_rows_kernel  rank-major rows no local query sees get dK = dV = 0
//   dkdv_kernel       K/V-stationary: 4 waves x 32 keys; for every Q tile of
//                     64 rows: S and dP on MFMA (A = Q / dO rows from LDS,
//                     B = K / V from registers), then dV^T += dO^T P and
//                     dK^T += Q^T dS with the transposed operands read by
//                     ds_read_b64_tr_b16 and P / dS taken in place from the
//                     accumulators.
//   dq_kernel         Q-stationary like the forward: S^T = K Q^T, dP^T = V dO^T,
//                     dQ^T += K^T dS^T.
#include "common.hpp"
#include "launch.hpp"

namespace cva {

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O), one thread per (local row, head)
// ---------------------------------------------------------------------------
template <typename E, int DV>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdParams P) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t n = (int64_t)P.t_loc * P.hq;
  if (idx >= n) return;
  const int64_t row = idx / P.hq;
  const int head = (int)(idx % P.hq);
  const uint16_t* o = (const uint16_t*)P.o + (row * P.hq + head) * DV;
  const uint16_t* g = (const uint16_t*)P.dout + (row * P.hq + head) * DV;
  float acc = 0.f;
#pragma unroll 4
  for (int d = 0; d < DV; d += 8) {
    const u32x4_t a = *(const u32x4_t*)(o + d);
    const u32x4_t b = *(const u32x4_t*)(g + d);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(E::to_float((uint16_t)(a[w] & 0xFFFFu)), E::to_float((uint16_t)(b[w] & 0xFFFFu)), acc);
      acc = fmaf(E::to_float((uint16_t)(a[w] >> 16)), E::to_float((uint16_t)(b[w] >> 16)), acc);
    }
  }
  P.delta[(int64_t)head * P.t_loc + row] = acc;
}

// ---------------------------------------------------------------------------
// zero dK / dV on rank-major rows outside every local prefix
// ---------------------------------------------------------------------------
template <int DQK, int DV>
__global__ __launch_bounds__(kThreads) void zero_rows_kernel(BwdParams P) {
  const int32_t r0 = P.t.zero_rows[2 * blockIdx.x], r1 = P.t.zero_rows[2 * blockIdx.x + 1];
  const u32x4_t z = {0u, 0u, 0u, 0u};
  {
    const int64_t n = (int64_t)(r1 - r0) * P.hkv * DQK / 8;
    u32x4_t* base = (u32x4_t*)((uint16_t*)P.dk + (int64_t)r0 * P.hkv * DQK);
    for (int64_t i = threadIdx.x; i < n; i += kThreads) base[i] = z;
  }
  {
    const int64_t n = (int64_t)(r1 - r0) * P.hkv * DV / 8;
    u32x4_t* base = (u32x4_t*)((uint16_t*)P.dv + (int64_t)r0 * P.hkv * DV);
    for (int64_t i = threadIdx.x; i < n; i += kThreads) base[i] = z;
  }
}

// ---------------------------------------------------------------------------
// dK / dV, K/V-stationary
// ---------------------------------------------------------------------------
template <typename E, int DQK, int DV>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdParams P) {
  constexpr int BQ = 64;          // queries per Q tile
  constexpr int QS = DQK / 16;    // reduction steps over Dqk
  constexpr int VS = DV / 16;     // reduction steps over Dv
  constexpr int QLD = DQK + 8;    // LDS row strides (elements): 16-byte aligned rows
  constexpr int OLD = DV + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[BQ * QLD];
  __shared__ __attribute__((aligned(16))) uint16_t sO[BQ * OLD];
  __shared__ float sL[BQ];
  __shared__ float sD[BQ];
  __shared__ int32_t sIv[BQ * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  const int tile = blockIdx.x / P.hkv;
  const int kvh = blockIdx.x % P.hkv;
  const int32_t* tr = P.t.kv_tiles + tile * 5;
  const int seq = tr[0], k0 = tr[1], keys = tr[2], span0 = tr[3], nspan = tr[4];
  // the longer prefix of the sub-sequence (its second segment) indexes every key of the tile
  const int32_t* segB = P.t.segs + (2 * seq + 1) * 8;
  const int32_t* kvi = P.t.kv_index + segB[5];
  const int kl = wave * 32 + col;          // key of this lane within the tile
  const int kpos = k0 + kl;                // in-sequence key position
  const bool kvalid = kl < keys;
  const int64_t grow = kvalid ? (int64_t)kvi[kpos] : 0;

  const uint16_t* __restrict__ kg = (const uint16_t*)P.k;
  const uint16_t* __restrict__ vg = (const uint16_t*)P.v;
  const uint16_t* __restrict__ qg = (const uint16_t*)P.q;
  const uint16_t* __restrict__ og = (const uint16_t*)P.dout;

  // K^T and V^T operands in registers: lane holds K[key][16s + 8*half .. +7]
  typename E::vec8 kf[QS], vf[VS];
  {
    const uint16_t* kr = kg + (grow * P.hkv + kvh) * DQK + 8 * half;
    const uint16_t* vr = vg + (grow * P.hkv + kvh) * DV + 8 * half;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (kvalid) x = *(const u32x4_t*)(kr + 16 * s);
      kf[s] = as_vec8<E>(x);
    }
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (kvalid) x = *(const u32x4_t*)(vr + 16 * s);
      vf[s] = as_vec8<E>(x);
    }
  }

  f32x16_t dk[DQK / 32], dv[DV / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dk[d] = zero16();
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) dv[d] = zero16();

  const float sl2 = P.scale_log2;

  for (int hh = 0; hh < P.group; ++hh) {
    const int head = kvh * P.group + hh;
    for (int sp = 0; sp < nspan; ++sp) {
      const int32_t* spr = P.t.kv_spans + (span0 + sp) * 4;
      const int seg = spr[0], qt0 = spr[1], qt1 = spr[2];
      const bool partial = spr[3] != 0;
      const int32_t* sg = P.t.segs + seg * 8;
      const int q_len = sg[2], q_row0 = sg[4];
      for (int qt = qt0; qt < qt1; ++qt) {
        const int a0 = qt * BQ;
        __syncthreads();
        // ---- stage the Q tile, dO tile, LSE, Delta and row intervals ----
        {
          constexpr int CQ = DQK / 8;
          for (int idx = tid; idx < BQ * CQ; idx += kThreads) {
            const int r = idx / CQ, c = idx % CQ;
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (a0 + r < q_len)
              x = *(const u32x4_t*)(qg + ((int64_t)(q_row0 + a0 + r) * P.hq + head) * DQK + c * 8);
            *(u32x4_t*)(sQ + r * QLD + c * 8) = x;
          }
          constexpr int CO = DV / 8;
          for (int idx = tid; idx < BQ * CO; idx += kThreads) {
            const int r = idx / CO, c = idx % CO;
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (a0 + r < q_len)
              x = *(const u32x4_t*)(og + ((int64_t)(q_row0 + a0 + r) * P.hq + head) * DV + c * 8);
            *(u32x4_t*)(sO + r * OLD + c * 8) = x;
          }
          if (tid < BQ) {
            const int r = tid;
            const bool ok = a0 + r < q_len;
            const int64_t lr = (int64_t)head * P.t_loc + q_row0 + a0 + r;
            sL[r] = ok ? P.lse[lr] * kLog2e : INFINITY;
            sD[r] = ok ? P.delta[lr] : 0.f;
            const int32_t* iv = P.t.row_iv + (int64_t)(q_row0 + a0 + r) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) sIv[r * 4 + j] = ok ? iv[j] : 0;
          }
        }
        __syncthreads();

#pragma unroll
        for (int qs = 0; qs < BQ / 32; ++qs) {
          // S[q][key] = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
          f32x16_t s = zero16(), dp = zero16();
          {
            const uint16_t* qrow = sQ + (qs * 32 + col) * QLD + 8 * half;
#pragma unroll
            for (int st = 0; st < QS; ++st)
              s = E::mfma32(as_vec8<E>(*(const u32x4_t*)(qrow + 16 * st)), kf[st], s);
            const uint16_t* orow = sO + (qs * 32 + col) * OLD + 8 * half;
#pragma unroll
            for (int st = 0; st < VS; ++st)
              dp = E::mfma32(as_vec8<E>(*(const u32x4_t*)(orow + 16 * st)), vf[st], dp);
          }
          // lane holds query qs*32 + 8i + 4*half + j (r = 4i + j) for key kpos
          uint32_t pp[2][4], pd[2][4];
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            float pv[2], dsv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int q = qs * 32 + 8 * ((r + u) >> 2) + 4 * half + ((r + u) & 3);
              float x = s[r + u] * sl2 - sL[q];
              if (partial) {
                const int32_t* iv = sIv + q * 4;
                const bool vis = (kpos >= iv[0] && kpos < iv[1]) || (kpos >= iv[2] && kpos < iv[3]);
                x = vis ? x : -INFINITY;
              }
              const float p = __builtin_amdgcn_exp2f(x);
              pv[u] = p;
              dsv[u] = p * (dp[r + u] - sD[q]);
            }
            pp[r >> 3][(r & 7) >> 1] = pack2<E>(pv[0], pv[1]);
            pd[r >> 3][(r & 7) >> 1] = pack2<E>(dsv[0], dsv[1]);
          }
          // dV^T[d][key] += sum_q dO^T[d][q] P[q][key];  dK^T += Q^T dS
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int qb = qs * 32 + st * 16 + 4 * half;
            const typename E::vec8 bp = as_vec8<E>(u32x4_t{pp[st][0], pp[st][1], pp[st][2], pp[st][3]});
            const typename E::vec8 bd = as_vec8<E>(u32x4_t{pd[st][0], pd[st][1], pd[st][2], pd[st][3]});
#pragma unroll
            for (int d = 0; d < DV / 32; ++d) {
              const u32x2_t lo = tr_operand(sO, OLD, qb, d * 32, lane);
              const u32x2_t hi = tr_operand(sO, OLD, qb + 8, d * 32, lane);
              dv[d] = E::mfma32(as_vec8<E>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), bp, dv[d]);
            }
#pragma unroll
            for (int d = 0; d < DQK / 32; ++d) {
              const u32x2_t lo = tr_operand(sQ, QLD, qb, d * 32, lane);
              const u32x2_t hi = tr_operand(sQ, QLD, qb + 8, d * 32, lane);
              dk[d] = E::mfma32(as_vec8<E>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), bd, dk[d]);
            }
          }
        }
      }
    }
  }

  // ---- write this lane's key row: dK^T / dV^T lane holds d = 32*blk + 8i + 4*half + j ----
  if (kvalid) {
    uint16_t* dkr = (uint16_t*)P.dk + (grow * P.hkv + kvh) * DQK;
    uint16_t* dvr = (uint16_t*)P.dv + (grow * P.hkv + kvh) * DV;
    const float sc = P.scale;
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dd = d * 32 + 8 * i + 4 * half;
        *(u32x2_t*)(dkr + dd) = u32x2_t{pack2<E>(dk[d][4 * i] * sc, dk[d][4 * i + 1] * sc),
                                         pack2<E>(dk[d][4 * i + 2] * sc, dk[d][4 * i + 3] * sc)};
      }
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dd = d * 32 + 8 * i + 4 * half;
        *(u32x2_t*)(dvr + dd) = u32x2_t{pack2<E>(dv[d][4 * i], dv[d][4 * i + 1]),
                                         pack2<E>(dv[d][4 * i + 2], dv[d][4 * i + 3])};
      }
  }
}

// ---------------------------------------------------------------------------
// dQ, Q-stationary (same work-group shape and schedule form as the forward)
// ---------------------------------------------------------------------------
template <typename E, int DQK, int DV>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(BwdParams P) {
  constexpr int BN = 64;
  constexpr int QS = DQK / 16, VS = DV / 16;
  constexpr int KLD = DQK + 8, VLD = DV + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BN * VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  const int tile = blockIdx.x / P.dq_head_groups;
  const int hg = blockIdx.x % P.dq_head_groups;
  const int32_t* tr = P.t.dq_tiles + tile * 5;
  const int seg = tr[0], q0 = tr[1], span0 = tr[3], nspan = tr[4];
  const int32_t* sg = P.t.segs + seg * 8;
  const int q_len = sg[2], kv_len = sg[3], q_row0 = sg[4], kv_off = sg[5];
  const int hpt = P.dq_heads_per_tile;
  const int head = hg * hpt + (wave % hpt);
  const int kvh = head / P.group;
  const int a = q0 + (wave / hpt) * 32 + col;
  const bool valid = a < q_len;
  const int row = q_row0 + a;

  const uint16_t* __restrict__ kg = (const uint16_t*)P.k;
  const uint16_t* __restrict__ vg = (const uint16_t*)P.v;
  const int32_t* __restrict__ kvi = P.t.kv_index + kv_off;

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
  int lo1 = 0, hi1 = 0, lo2 = 0, hi2 = 0;
  float lse2 = INFINITY, delta = 0.f;
  if (valid) {
    const int32_t* iv = P.t.row_iv + (int64_t)row * 4;
    lo1 = iv[0]; hi1 = iv[1]; lo2 = iv[2]; hi2 = iv[3];
    lse2 = P.lse[(int64_t)head * P.t_loc + row] * kLog2e;
    delta = P.delta[(int64_t)head * P.t_loc + row];
  }

  f32x16_t acc[DQK / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) acc[d] = zero16();
  const float sl2 = P.scale_log2;

  for (int sp = 0; sp < nspan; ++sp) {
    const int32_t* spr = P.t.dq_spans + (span0 + sp) * 4;
    const int t_begin = spr[0], t_end = spr[1];
    const bool partial = spr[2] != 0;
    for (int t = t_begin; t < t_end; ++t) {
      const int kb0 = t * BN;
      __syncthreads();
      {
        constexpr int CK = DQK / 8;
        for (int idx = tid; idx < BN * CK; idx += kThreads) {
          const int r = idx / CK, c = idx % CK;
          const int b = kb0 + r;
          u32x4_t x = {0u, 0u, 0u, 0u};
          if (b < kv_len) x = *(const u32x4_t*)(kg + ((int64_t)kvi[b] * P.hkv + kvh) * DQK + c * 8);
          *(u32x4_t*)(sK + r * KLD + c * 8) = x;
        }
        constexpr int CV = DV / 8;
        for (int idx = tid; idx < BN * CV; idx += kThreads) {
          const int r = idx / CV, c = idx % CV;
          const int b = kb0 + r;
          u32x4_t x = {0u, 0u, 0u, 0u};
          if (b < kv_len) x = *(const u32x4_t*)(vg + ((int64_t)kvi[b] * P.hkv + kvh) * DV + c * 8);
          *(u32x4_t*)(sV + r * VLD + c * 8) = x;
        }
      }
      __syncthreads();
#pragma unroll
      for (int nb = 0; nb < BN / 32; ++nb) {
        f32x16_t s = zero16(), dp = zero16();
        const uint16_t* kr = sK + (nb * 32 + col) * KLD + 8 * half;
#pragma unroll
        for (int st = 0; st < QS; ++st)
          s = E::mfma32(as_vec8<E>(*(const u32x4_t*)(kr + 16 * st)), qf[st], s);
        const uint16_t* vr = sV + (nb * 32 + col) * VLD + 8 * half;
#pragma unroll
        for (int st = 0; st < VS; ++st)
          dp = E::mfma32(as_vec8<E>(*(const u32x4_t*)(vr + 16 * st)), of[st], dp);
        uint32_t pd[2][4];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            float x = s[r + u] * sl2 - lse2;
            if (partial) {
              const int b = kb0 + nb * 32 + 8 * ((r + u) >> 2) + 4 * half + ((r + u) & 3);
              const bool vis = (b >= lo1 && b < hi1) || (b >= lo2 && b < hi2);
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
          const int kb = nb * 32 + st * 16 + 4 * half;
          const typename E::vec8 bd = as_vec8<E>(u32x4_t{pd[st][0], pd[st][1], pd[st][2], pd[st][3]});
#pragma unroll
          for (int d = 0; d < DQK / 32; ++d) {
            const u32x2_t lo = tr_operand(sK, KLD, kb, d * 32, lane);
            const u32x2_t hi = tr_operand(sK, KLD, kb + 8, d * 32, lane);
            acc[d] = E::mfma32(as_vec8<E>(u32x4_t{lo[0], lo[1], hi[0], hi[1]}), bd, acc[d]);
          }
        }
      }
    }
  }

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
  auto launch = [&](int id, auto kernel, unsigned grid) {
    if (e != hipSuccess || grid == 0) return;
    if (hook) hook->before(id, s);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, s, p);
    if (hook) hook->after(id, s);
    e = hipGetLastError();
  };
  const int64_t n_pre = (int64_t)p.t_loc * p.hq;
  launch(K_BWD_PRE, bwd_pre_kernel<E, DV>, (unsigned)((n_pre + kThreads - 1) / kThreads));
  launch(K_BWD_ZERO, zero_rows_kernel<DQK, DV>, (unsigned)p.n_zero_ranges);
  launch(K_BWD_DKDV, dkdv_kernel<E, DQK, DV>, (unsigned)p.n_kv_tiles * (unsigned)p.hkv);
  launch(K_BWD_DQ, dq_kernel<E, DQK, DV>, (unsigned)p.n_dq_tiles * (unsigned)p.dq_head_groups);
  return e;
}

}  // namespace

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
