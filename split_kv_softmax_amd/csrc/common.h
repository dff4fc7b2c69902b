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
// D = 64 also serves any other buffer with 128-byte rows.  D = 16 (32-byte
// rows of two chunks): rows 8..15 of every 16 swap their chunks, so the 16
// row reads of a lane group cover the 64 banks once, and 4 consecutive rows
// (transposing reads) are 128 contiguous bytes.
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  if constexpr (D == 16) return (r >> 3) & 1;
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
  static_assert(KMAX <= 16, "table covers k <= 16");
#define FL_WU(K)                                                   \
  if constexpr (K <= KMAX) {                                       \
    if (k == K) { wait_vm<(UNIT * K < 64 ? UNIT * K : 63)>(); return; } \
  }
  FL_WU(1) FL_WU(2) FL_WU(3) FL_WU(4) FL_WU(5) FL_WU(6) FL_WU(7) FL_WU(8)
  FL_WU(9) FL_WU(10) FL_WU(11) FL_WU(12) FL_WU(13) FL_WU(14) FL_WU(15) FL_WU(16)
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

// ---- merge of (m, l, acc) states ("Ring vs. Tree Attention": the online-
// softmax merge; "FLARE++" appendix, eq. 23).  Natural-log units: a leaf
// (O_r, L_r) enters as (L_r, 1, O_r), an empty one as (-inf, 0, 0).  Merging a
// state with an empty one returns it bit for bit (factor exp(0) = 1 on its
// side, exactly 0 on the empty side).  Shared by the tree merge kernel and the
// fused encode + merge, so both give the same bits.
struct MState {
  float m, l;
  f32x4_t acc;
};

__device__ __forceinline__ MState mstate_empty() { return MState{kNegInf, 0.f, f32x4_t{0.f, 0.f, 0.f, 0.f}}; }

__device__ __forceinline__ MState mstate_leaf(float L, f32x4_t O) {
  const bool e = L == kNegInf;
  return MState{L, e ? 0.f : 1.f, e ? f32x4_t{0.f, 0.f, 0.f, 0.f} : O};
}

// The roundings of a merge are spelled out (one product, then a fused
// multiply-add) and the compiler may not contract anything else, so that every
// kernel that merges rounds alike whatever it can prove about the operands.
__device__ __forceinline__ MState mstate_merge(const MState& x, const MState& y) {
#pragma clang fp contract(off)
  MState r;
  r.m = fmaxf(x.m, y.m);
  if (r.m == kNegInf) return mstate_empty();
  const float fx = __expf(x.m - r.m);   // exactly 0 for an empty side
  const float fy = __expf(y.m - r.m);
  r.l = __builtin_fmaf(x.l, fx, y.l * fy);
#pragma unroll
  for (int j = 0; j < 4; ++j) r.acc[j] = __builtin_fmaf(x.acc[j], fx, y.acc[j] * fy);
  return r;
}

// Normalised output of a merged state: O = acc / l (0 when empty), L = m + ln l (-inf when empty).
__device__ __forceinline__ void mstate_finish(const MState& cur, f32x4_t& z, float& L) {
#pragma clang fp contract(off)
  const bool empty = !(cur.l > 0.f);
  const float inv = empty ? 0.f : 1.f / cur.l;
  z = cur.acc * inv;
  if (empty) z = f32x4_t{0.f, 0.f, 0.f, 0.f};
  L = empty ? kNegInf : cur.m + __logf(cur.l);
}

// Fold of states s0 .. s0+n-1 (n >= 0) of one row and one 4-column piece:
// state s has log-normaliser in_L[s*rows + row] and output columns
// in_O[s*sstride + off .. +4) (off = row*D + 4*piece).  Up to 16 states every
// load is issued at once (indices past the end re-read the last state),
// absent leaves are empty, and the rounds of the 16-leaf tree run on them
// (fold_static, on the narrowest power-of-two width that holds n); merging
// with an empty leaf returns the state unchanged, so this is the tree with
// pass-through survivors.  Beyond 16 the leaves are visited in order
// (16 loads at a time) keeping one partial state per tree level, a binary
// counter: after leaf i the levels whose bit is set in i are merged into it
// (left subtree first), and at the end the occupied levels are merged from the
// lowest upwards, which is the round schedule with its pass-through
// survivors.  i is the same for every thread, so the branches are uniform.
// (The level walk is written out in each fold: behind a helper the level
// array is no longer promoted to registers.)
constexpr int kFoldBatch = 16;
constexpr int kFoldLevels = 16;   // up to 65536 states

// The rounds of the W-leaf tree over states s0 .. s0+n-1, 1 <= n <= W (W a
// power of two), every load issued at once.  For n <= W/2 the upper half of
// the leaves is empty and each merge with it returns the state unchanged, so
// the narrowest W that holds n gives the result of any wider one.
template <int W>
__device__ __forceinline__ MState fold_static(const float* in_O, const float* in_L, int64_t s0, int n,
                                              int64_t rows, int64_t row, int64_t off, int64_t sstride) {
  MState t[W];
  float Lb[W];
  f32x4_t Ob[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const int64_t s = s0 + (k < n ? k : n - 1);
    Lb[k] = in_L[s * rows + row];
    Ob[k] = *reinterpret_cast<const f32x4_t*>(in_O + s * sstride + off);
  }
#pragma unroll
  for (int k = 0; k < W; ++k) t[k] = k < n ? mstate_leaf(Lb[k], Ob[k]) : mstate_empty();
#pragma unroll
  for (int w2 = 1; w2 < W; w2 *= 2)
#pragma unroll
    for (int i = 0; i < W; i += 2 * w2) t[i] = mstate_merge(t[i], t[i + w2]);
  return t[0];
}

__device__ __forceinline__ MState fold_states(const float* in_O, const float* in_L, int64_t s0, int n,
                                              int64_t rows, int64_t row, int64_t off, int64_t sstride) {
  if (n == 0) return mstate_empty();
  if (n == 1) return fold_static<1>(in_O, in_L, s0, n, rows, row, off, sstride);
  if (n == 2) return fold_static<2>(in_O, in_L, s0, n, rows, row, off, sstride);
  if (n <= 4) return fold_static<4>(in_O, in_L, s0, n, rows, row, off, sstride);
  if (n <= 8) return fold_static<8>(in_O, in_L, s0, n, rows, row, off, sstride);
  if (n <= kFoldBatch) return fold_static<kFoldBatch>(in_O, in_L, s0, n, rows, row, off, sstride);
  MState lv[kFoldLevels];
  for (int i0 = 0; i0 < n; i0 += kFoldBatch) {
    float Lb[kFoldBatch];
    f32x4_t Ob[kFoldBatch];
#pragma unroll
    for (int k = 0; k < kFoldBatch; ++k) {
      const int64_t s = s0 + (i0 + k < n ? i0 + k : n - 1);
      Lb[k] = in_L[s * rows + row];
      Ob[k] = *reinterpret_cast<const f32x4_t*>(in_O + s * sstride + off);
    }
#pragma unroll
    for (int k = 0; k < kFoldBatch; ++k) {
      const int i = i0 + k;
      if (i < n) {
        MState leaf = mstate_leaf(Lb[k], Ob[k]);
        bool carry = true;
#pragma unroll
        for (int lvl = 0; lvl < kFoldLevels; ++lvl) {
          if (carry) {
            if ((i >> lvl) & 1) {
              leaf = mstate_merge(lv[lvl], leaf);
            } else {
              lv[lvl] = leaf;
              carry = false;
            }
          }
        }
      }
    }
  }
  MState cur = mstate_empty();
  bool have = false;
#pragma unroll
  for (int lvl = 0; lvl < kFoldLevels; ++lvl) {
    if ((n >> lvl) & 1) {
      cur = have ? mstate_merge(lv[lvl], cur) : lv[lvl];
      have = true;
    }
  }
  return cur;
}

// The same fold with few registers, for n <= 256 states: the binary counter
// over the leaves, four loads at a time.  Up to 16 states it counts exactly 16
// leaves (the absent ones empty), which builds the complete 16-leaf tree of
// fold_states merge by merge (left subtree first in every merge); beyond 16 it
// counts the n leaves as fold_states does.  The results are therefore
// identical.
__device__ __forceinline__ MState fold_states_lean(const float* in_O, const float* in_L, int64_t s0, int n,
                                                   int64_t rows, int64_t row, int64_t off, int64_t sstride) {
  constexpr int kLv = 9;   // 256 leaves
  if (n == 0) return mstate_empty();
  MState lv[kLv];
  const int total = n <= kFoldBatch ? kFoldBatch : n;
  for (int i0 = 0; i0 < total; i0 += 4) {
    float Lb[4];
    f32x4_t Ob[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t s = s0 + (i0 + k < n ? i0 + k : n - 1);
      Lb[k] = in_L[s * rows + row];
      Ob[k] = *reinterpret_cast<const f32x4_t*>(in_O + s * sstride + off);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = i0 + k;
      if (i < total) {
        MState leaf = i < n ? mstate_leaf(Lb[k], Ob[k]) : mstate_empty();
        bool carry = true;
#pragma unroll
        for (int lvl = 0; lvl < kLv; ++lvl) {
          if (carry) {
            if ((i >> lvl) & 1) {
              leaf = mstate_merge(lv[lvl], leaf);
            } else {
              lv[lvl] = leaf;
              carry = false;
            }
          }
        }
      }
    }
  }
  MState cur = mstate_empty();
  bool have = false;
#pragma unroll
  for (int lvl = 0; lvl < kLv; ++lvl) {
    if ((total >> lvl) & 1) {
      cur = have ? mstate_merge(lv[lvl], cur) : lv[lvl];
      have = true;
    }
  }
  return cur;
}

// Store a folded state as output state oi: normalised columns (and their
// bfloat16 copy when out_bf16 is set), and the log-normaliser from the thread
// that holds the row's first piece.
__device__ __forceinline__ void store_state(const MState& cur, float* out_O, float* out_L, uint16_t* out_bf16,
                                            int64_t oi, int64_t rows, int64_t row, int64_t off, int64_t sstride,
                                            int D) {
  f32x4_t z;
  float Lz;
  mstate_finish(cur, z, Lz);
  *reinterpret_cast<f32x4_t*>(out_O + oi * sstride + off) = z;
  if (off % D == 0) out_L[oi * rows + row] = Lz;
  if (out_bf16) {
    const u32x2_t wv = {pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
    *reinterpret_cast<u32x2_t*>(out_bf16 + oi * sstride + off) = wv;
  }
}

}  // namespace flare
