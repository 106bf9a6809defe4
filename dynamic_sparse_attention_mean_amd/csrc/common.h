// Shared device helpers for the gfx950 kernels (wave64, bf16 MFMA).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 bit helpers.  bf16 is the upper half of an fp32 bit pattern.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two fp32 values to packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// fp64 -> bf16 bits with a single round-to-nearest-even step taken on the
// fp64 pattern (no double rounding through fp32).  bf16 keeps the top 7
// mantissa bits, fp64 has 52: round at bit 45.  Finite values whose result is
// a normal bf16; zero maps to zero.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint64_t lsb = (u >> 45) & 1ull;
  u += 0x0fffffffffffull + lsb;
  u &= ~0x1fffffffffffull;
  float f = (float)__longlong_as_double((long long)u);   // exact: 8 significant bits
  return __float_as_uint(f) >> 16;
}

// Order-preserving map of fp32 to uint32: larger float -> larger key.
// -inf maps to the smallest non-NaN key.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Wave helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Inclusive prefix sum over the wave (Hillis-Steele with shuffles).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o, 64);
    if (l >= o) v += t;
  }
  return v;
}
// Number of set ballot bits below this lane.
__device__ __forceinline__ uint32_t ballot_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---------------------------------------------------------------------------
// 16 bytes per lane straight from global memory into LDS; lane l of the wave
// lands at LDS byte address lds_addr + 16 l (lds_addr is wave-uniform).
// Issued from inline assembly on purpose: the compiler does not track these
// LDS writes, so it adds no wait of its own before LDS reads or writes that it
// cannot tell apart from the DMA's target (its own wait would drain the DMA
// just issued for a later stage of a ring).  The caller orders a DMA before
// the reads of its stage with an explicit vmcnt wait; the "memory" clobber
// keeps the compiler from moving LDS accesses across the issue.  The
// instruction has no register results.  M0 (the LDS base) is saved and
// restored around it, so the compiler's view of M0 never changes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(save) : "v"(g), "s"(lds_addr) : "memory");
}

}  // namespace dsa
