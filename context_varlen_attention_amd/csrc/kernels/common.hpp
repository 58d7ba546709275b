// Device helpers for the gfx950 attention kernels: MFMA wrappers, 16-bit
// element types, LDS fragments, cross-half-wave exchange.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cva {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 16-bit element type tag: bf16 or fp16.  Values travel as raw bits (uint16 /
// packed uint32) and are reinterpreted only at the MFMA and at conversions.
struct Bf16 {
  using vec8 = bf16x8_t;
  __device__ static inline f32x16_t mfma32(vec8 a, vec8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint16_t from_float(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static inline float to_float(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
  }
};

struct Fp16 {
  using vec8 = f16x8_t;
  __device__ static inline f32x16_t mfma32(vec8 a, vec8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint16_t from_float(float x) {
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static inline float to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
};

template <typename E>
__device__ inline typename E::vec8 as_vec8(u32x4_t x) {
  return __builtin_bit_cast(typename E::vec8, x);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two floats to one packed 16-bit pair (round to nearest even; one v_cvt_pk).
template <typename E>
__device__ inline uint32_t pack2(float lo, float hi);

template <>
__device__ inline uint32_t pack2<Bf16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <>
__device__ inline uint32_t pack2<Fp16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}

// Value held by lane (l ^ 32): the two half-waves of a 32x32 MFMA output hold
// different rows of the same column.
__device__ inline float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16).  Within every group of 16 lanes,
// output lane i receives element (i % 4) of the 8-byte words addressed by
// source lanes i/4, i/4+4, i/4+8, i/4+12.  tr_operand() below turns that into
// "4 consecutive rows of one column" for an MFMA operand.
__device__ inline u32x2_t lds_read_tr16(const uint16_t* p) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// For a row-major LDS tile X (row stride ld elements, ld % 4 == 0), return
// to lane l the values X[row0 + k][col0 + (l % 32)] for k = 0..3, packed as
// four 16-bit elements.  row0 may differ between the two half-waves.
__device__ inline u32x2_t tr_operand(const uint16_t* X, int ld, int row0, int col0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  return lds_read_tr16(X + (row0 + (s >> 2)) * ld + col0 + 16 * (g & 1) + 4 * (s & 3));
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at LDS byte address lds + 16*l (lds is wave-uniform).
// Issued through inline assembly so that the compiler does not make LDS reads
// of the other buffer wait for this load; completion is awaited explicitly
// (s_waitcnt vmcnt(0) + barrier) before the destination buffer is read.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// s_waitcnt vmcnt(0) through the builtin, so that the compiler's own wait
// bookkeeping knows every vector memory load has completed here (encoding:
// vmcnt 0, expcnt 7, lgkmcnt 15).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 4 bytes per lane from global memory into LDS (global_load_lds_dword): lane l's
// word lands at LDS byte address lds + 4*l.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 63].
__device__ __forceinline__ void wait_vmem_le(int n) {
  switch (n) {
#define CVA_WAIT_CASE(k) \
  case k:                \
    __builtin_amdgcn_s_waitcnt(0x0F70 | (k & 15) | ((k >> 4) << 14)); \
    break;
    CVA_WAIT_CASE(0) CVA_WAIT_CASE(1) CVA_WAIT_CASE(2) CVA_WAIT_CASE(3) CVA_WAIT_CASE(4)
    CVA_WAIT_CASE(5) CVA_WAIT_CASE(6) CVA_WAIT_CASE(7) CVA_WAIT_CASE(8) CVA_WAIT_CASE(9)
    CVA_WAIT_CASE(10) CVA_WAIT_CASE(11) CVA_WAIT_CASE(12) CVA_WAIT_CASE(13) CVA_WAIT_CASE(14)
    CVA_WAIT_CASE(15) CVA_WAIT_CASE(16) CVA_WAIT_CASE(17) CVA_WAIT_CASE(18) CVA_WAIT_CASE(19)
    CVA_WAIT_CASE(20) CVA_WAIT_CASE(21) CVA_WAIT_CASE(22) CVA_WAIT_CASE(23) CVA_WAIT_CASE(24)
    CVA_WAIT_CASE(25) CVA_WAIT_CASE(26) CVA_WAIT_CASE(27) CVA_WAIT_CASE(28) CVA_WAIT_CASE(29)
    CVA_WAIT_CASE(30) CVA_WAIT_CASE(31) CVA_WAIT_CASE(32) CVA_WAIT_CASE(33) CVA_WAIT_CASE(34)
    CVA_WAIT_CASE(35) CVA_WAIT_CASE(36) CVA_WAIT_CASE(37) CVA_WAIT_CASE(38) CVA_WAIT_CASE(39)
    CVA_WAIT_CASE(40)
#undef CVA_WAIT_CASE
    default:
      __builtin_amdgcn_s_waitcnt(0x0F70);
      break;
  }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ inline f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

}  // namespace cva

// ---------------------------------------------------------------------------
// Attention dropout (MindSpeed RFC section 3.5.2.2, attention_dropout in [0, 1)).
// The random bits come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011): per round, the 64-bit products
// of counter words 0 and 2 with 0xD2511F53 and 0xCD9E8D57 give the new words
// (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0), and the key moves on by the Weyl
// increments 0x9E3779B9 and 0xBB67AE85.  One call covers a 4 x 4 block of
// (query, key) pairs of one sequence and head: counter (k / 4, q / 4, head,
// sequence) at in-sequence positions, key = the 64-bit seed; the pair's random
// byte is byte k % 4 of output word q % 4, and the pair is kept iff that byte is
// at least the threshold t = round(256 p) (t = 0: nothing dropped).  Kept
// probabilities are scaled by 256 / (256 - t) where the output is normalised.
// ---------------------------------------------------------------------------
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t y0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t y2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = y0;
    c2 = y2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// The word of the 4 x 4 block holding query qpos and keys kpos4 .. kpos4 + 3
// (kpos4 a multiple of 4): byte i is the random byte of key kpos4 + i.
__device__ __forceinline__ uint32_t drop_word(uint32_t seed_lo, uint32_t seed_hi, int seq, int head, int qpos,
                                              int kpos4) {
  const Philox4 x = philox4x32_10((uint32_t)kpos4 >> 2, (uint32_t)qpos >> 2, (uint32_t)head, (uint32_t)seq,
                                  seed_lo, seed_hi);
  const int i = qpos & 3;
  return i == 0 ? x.w[0] : i == 1 ? x.w[1] : i == 2 ? x.w[2] : x.w[3];
}

// The four words of the block holding queries 4*(qpos >> 2) .. + 3 and keys
// kpos4 .. kpos4 + 3: word i belongs to query 4*(qpos >> 2) + i.
__device__ __forceinline__ Philox4 drop_block(uint32_t seed_lo, uint32_t seed_hi, int seq, int head, int qpos,
                                              int kpos4) {
  return philox4x32_10((uint32_t)kpos4 >> 2, (uint32_t)qpos >> 2, (uint32_t)head, (uint32_t)seq, seed_lo,
                       seed_hi);
}

// Keep mask of the two 16-bit halves of a packed pair whose random bytes are
// bytes b and b + 1 of u: 0xFFFF in each kept half.
__device__ __forceinline__ uint32_t drop_keep_pair(uint32_t u, int b, uint32_t t) {
  const uint32_t lo = (u >> (8 * b)) & 0xFFu, hi = (u >> (8 * b + 8)) & 0xFFu;
  return (lo >= t ? 0x0000FFFFu : 0u) | (hi >= t ? 0xFFFF0000u : 0u);
}

// Is the pair with random byte b of u kept?
__device__ __forceinline__ bool drop_keep(uint32_t u, int b, uint32_t t) {
  return ((u >> (8 * b)) & 0xFFu) >= t;
}

// 4 x 4 transpose of 32-bit values over the four lanes of each quad (lanes
// 4m .. 4m+3): lane d holds x[0..3]; afterwards x[i] of lane d is what x[d]
// was in lane i.  Two butterfly stages (partners lane ^ 2, then lane ^ 1, by
// DPP quad permutes); every lane of the wave must be active.
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int lane) {
  const bool b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
#pragma unroll
  for (int p = 0; p < 2; ++p) {  // pairs (0, 2), (1, 3): swap the half whose index bit 1 differs
    const uint32_t send = b1 ? x[p] : x[p + 2];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0x4E, 0xF, 0xF, false);
    x[p] = b1 ? recv : x[p];
    x[p + 2] = b1 ? x[p + 2] : recv;
  }
#pragma unroll
  for (int p = 0; p < 4; p += 2) {  // pairs (0, 1), (2, 3): swap the element whose index bit 0 differs
    const uint32_t send = b0 ? x[p] : x[p + 1];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);
    x[p] = b0 ? recv : x[p];
    x[p + 1] = b0 ? x[p + 1] : recv;
  }
}

// The word of the 4 x 4 generator blocks that belongs to queries q0 + j
// (j = 0..3, q0 % 4 == off for every lane) and keys kp4 .. kp4 + 3: the blocks
// of q0 and q0 + 4 cover them.
__device__ __forceinline__ void drop_query_words(uint32_t (&w)[4], uint32_t s0, uint32_t s1, int seq, int head,
                                                 int q0, int off, int kp4) {
  const Philox4 a = drop_block(s0, s1, seq, head, q0, kp4);
  if (off == 0) {  // (wave-uniform)
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = a.w[j];
    return;
  }
  const Philox4 b = drop_block(s0, s1, seq, head, q0 + 4, kp4);
  // query q0 + j is word off + j of the first block, or of the second past 3
  const uint32_t c[7] = {a.w[0], a.w[1], a.w[2], a.w[3], b.w[0], b.w[1], b.w[2]};
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = off == 1 ? c[j + 1] : off == 2 ? c[j + 2] : c[j + 3];
}

// Random words of a 32-key block in the S^T layout (lane = query qw + (lane &
// 31), keys kb + 8 r + 4 (lane >> 5) + 0..3 for r = 0..3, kb % 32 == 0): u[r] is
// the word whose bytes 0..3 belong to those four keys.  The four lanes of a quad
// (four consecutive queries) need the same blocks: lane d runs the generator
// for run r = d and the quad exchanges the words.  qw: the wave's first query
// (the same in every lane).
__device__ __forceinline__ void drop_words_st(uint32_t (&u)[4], uint32_t s0, uint32_t s1, int seq, int head,
                                              int qw, int kb, int lane) {
  const int d = lane & 3, half = lane >> 5;
  const int q0 = qw + (lane & 28);  // the quad's first query
  drop_query_words(u, s0, s1, seq, head, q0, qw & 3, kb + 8 * d + 4 * half);
  quad_transpose(u, lane);
}

// Random bytes of a 32-query block in the S layout (lane = key kw + (lane & 31)
// with kw % 4 == 0; queries qb + 8 r + 4 (lane >> 5) + j for r, j = 0..3): byte j
// of b[r] belongs to query qb + 8 r + 4 (lane >> 5) + j.  The four lanes of a
// quad (four consecutive keys) need the same blocks: lane d runs the generator
// for run r = d, regroups the bytes by key and the quad exchanges them.
__device__ __forceinline__ void drop_bytes_s(uint32_t (&b)[4], uint32_t s0, uint32_t s1, int seq, int head,
                                             int kw, int qb, int lane) {
  const int d = lane & 3, half = lane >> 5;
  uint32_t w[4];  // w[j]: the word of query qb + 8 d + 4 half + j (its byte e: key + e of the quad)
  drop_query_words(w, s0, s1, seq, head, qb + 8 * d + 4 * half, qb & 3, kw + (lane & 28));
#pragma unroll
  for (int e = 0; e < 4; ++e)  // b[e]: byte e of w[0..3], i.e. the quad's key e for the run's four queries
    b[e] = ((w[0] >> (8 * e)) & 0xFFu) | (((w[1] >> (8 * e)) & 0xFFu) << 8) | (((w[2] >> (8 * e)) & 0xFFu) << 16) |
           (((w[3] >> (8 * e)) & 0xFFu) << 24);
  quad_transpose(b, lane);
}
