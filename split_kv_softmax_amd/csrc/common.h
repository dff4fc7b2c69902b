// Device helpers shared by the gfx950 kernels of libflare.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flare {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// cache-policy operand of the buffer intrinsics: bit 1 is the non-temporal hint
constexpr int kCachePolicyNT = 2;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats -> two bfloat16 (round to nearest even) packed lo|hi.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maxima of scores straight from the matrix cores: the IEEE maximum that
// propagates NaN needs no input canonicalisation, so 3-input forms stay one
// instruction each (scores of padding are replaced by -inf before any max).
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmax2(fmax2(a, b), c); }

// 32x32x16 bf16 matrix-core product, D = A*B + C.
// Operand layout (lane l, wave of 64): A row i = l%32, columns k = 8*(l/32)+0..7;
// B column j = l%32, rows k = 8*(l/32)+0..7; result column j = l%32 and
// register r holds row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row index of result register r in half h of a 32x32 product tile, and the
// permutation that makes the registers of one half cover 8 consecutive
// contraction indices of a follow-up product: loading operand row
// swap23(i) into A row i puts token 16*(r/8) + 8*h + r%8 into register r.
__host__ __device__ constexpr int swap23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}

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

// Global load of 16 bytes that bypasses nothing special; kept as one helper so
// the access width is explicit.
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// ---- LDS ring helpers shared by the streaming kernels
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

// Direct HBM -> LDS load: lane l's 16 bytes at g land at lds_wave_base + 16*l.
// Written as inline asm on purpose: the compiler then does not treat the LDS
// ring as written by outstanding vector-memory operations, so it neither
// drains them before every LDS read nor at every barrier; the kernel counts
// and waits for them itself (wait_vm) before a barrier publishes a stage.
// M0 (which carries the LDS destination) is saved and restored around it.
// The loads are marked non-temporal: every streamed row is read once.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"                       // one wait state between an SALU write of M0 and its use
      "global_load_lds_dwordx4 %2, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_wave_base), "v"(g)
      : "memory");
}

// The same with a wave-uniform 64-bit base (scalar registers) plus a 32-bit
// per-lane byte offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16_off(const void* base, uint32_t voff, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_wave_base), "v"(voff), "s"(base)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding vector-memory operation, including the ring's
// in-flight tiles).  LDS writes made with ds_* are completed first.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ---- K/V tile rings (encoder and backward)
// XOR swizzle of the 16-byte chunks of row r of a [64 x D] bf16 tile.  Both
// read patterns are free of bank conflicts with it:
//  * row reads (one 16-byte chunk per lane, 16 consecutive rows per group of
//    16 lanes): the swizzle is a bijection on each parity class of 16 rows
//    (128-byte rows) or on all 16 rows (256-byte rows);
//  * transposing reads (4 consecutive rows x 4 consecutive chunks per 32
//    lanes): the 4 rows land in disjoint aligned groups of 4 chunks.
// D = 64 also serves any other buffer with 128-byte rows.
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  return D == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
}

template <int OPS, int S>
__device__ __forceinline__ void wait_tiles(int later) {
  // wait until at most `later` tiles' worth of this wave's loads are pending
  static_assert(S <= 5, "wait table covers S <= 5");
  if constexpr (S >= 5) {
    if (later >= 3) { wait_vm<3 * OPS < 64 ? 3 * OPS : 63>(); return; }
  }
  if constexpr (S >= 4) {
    if (later >= 2) { wait_vm<2 * OPS < 64 ? 2 * OPS : 63>(); return; }
  }
  if constexpr (S >= 3) {
    if (later >= 1) { wait_vm<OPS < 64 ? OPS : 63>(); return; }
  }
  wait_vm<0>();
}

// Wait until at most n (wave-uniform, 0 <= n) of this wave's vector-memory
// operations are pending; n above NMAX waits as for NMAX.
template <int NMAX>
__device__ __forceinline__ void wait_vm_le(int n) {
  static_assert(NMAX >= 0 && NMAX < 64, "vmcnt range");
  if constexpr (NMAX == 0) {
    wait_vm<0>();
  } else {
    if (n >= NMAX) { wait_vm<NMAX>(); return; }
    wait_vm_le<NMAX - 1>(n);
  }
}

// Wait until at most k * UNIT of this wave's vector-memory operations are
// pending (k = 0 .. KMAX, uniform); the immediate must be a constant, hence
// the table.  Counts beyond the counter's range wait for 63, which is
// stronger: loads complete in issue order.
template <int UNIT, int KMAX>
__device__ __forceinline__ void wait_units(int k) {
  static_assert(KMAX <= 8, "table covers k <= 8");
#define FL_WU(K)                                                   \
  if constexpr (K <= KMAX) {                                       \
    if (k == K) { wait_vm<(UNIT * K < 64 ? UNIT * K : 63)>(); return; } \
  }
  FL_WU(1) FL_WU(2) FL_WU(3) FL_WU(4) FL_WU(5) FL_WU(6) FL_WU(7) FL_WU(8)
#undef FL_WU
  wait_vm<0>();
}

// Validity bits of the 64 tokens [t0, t0+64) of batch row `mw` (aligned words),
// read through the constant address space so they become scalar loads.
typedef __attribute__((address_space(4))) const uint64_t const_u64;
typedef __attribute__((address_space(4))) const int32_t const_i32;

// Block index of this workgroup through an optional launch order (scalar load).
__device__ __forceinline__ int ordered_block(const int32_t* order) {
  return order ? ((const_i32*)order)[blockIdx.x] : (int)blockIdx.x;
}
__device__ __forceinline__ uint64_t mask_tile_bits(const_u64* mw, int t0) {
  const int w = t0 >> 6, sh = t0 & 63;
  const uint64_t lo = mw[w];
  if (sh == 0) return lo;
  return (lo >> sh) | (mw[w + 1] << (64 - sh));
}

}  // namespace flare
