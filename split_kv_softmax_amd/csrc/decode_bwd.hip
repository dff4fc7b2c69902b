// Decode backward ("FLARE++: Low-rank attention with dynamic attention
// routing", appendix on context parallelism, FLARE++ backward paragraph: each
// token's local decoder contributes to the gradient of the replicated latent
// keys, and the latent values' gradient is the sum of the decoders'
// contributions).  For Y[n] = softmax_m(s Xq[n].Klat[m]) Z and an output
// gradient dY:
//   A = softmax over the M latents,  dA = dY Z^T,  delta[n] = sum_m A dA,
//   dT = A (dA - delta),  dXq = s dT Klat,  dKlat = s dT^T Xq,  dZ = A^T dY.
// Two passes: the token side (softmax over the latents is lane-local) writes
// dXq and each token's log2-normaliser and delta; the latent side streams the
// tokens again and sums dZ and dKlat per token chunk, which a fixed-order
// reduction adds up.
#include "common.h"
#include "kernels.h"

namespace flare {

namespace {
template <typename T>
__device__ __forceinline__ float ld1(const T* p) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(*p); else return *p;
}
template <typename T>
__device__ __forceinline__ void st1(T* p, float v) {
  if constexpr (sizeof(T) == 2) *p = to_bf16(v); else *p = v;
}
}  // namespace

// ---------------------------------------------------------------------------
// General vector kernels (float32, or shapes without a matrix-core variant).
// ---------------------------------------------------------------------------
// Token side: one wave per token, lanes over head dims; three passes over the
// latents (normaliser, delta, dXq) recompute the dot products.
template <typename TIn>
__global__ __launch_bounds__(256) void dbwd_tok_generic_kernel(const DecBwdArgs a) {
  constexpr int MAXDL = 4;   // D <= 256
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)a.B * a.H * a.N;
  if (tok >= total) return;
  const int n = (int)(tok % a.N);
  const int64_t bh = tok / a.N;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int D = a.D, M = a.M;
  const bool valid = !a.token_mask || a.token_mask[(int64_t)b * a.N + n] != 0;
  const int64_t srow = bh * a.stats_stride + n;
  TIn* dx = static_cast<TIn*>(a.dXq) + tok * D;
  if (!valid) {
    for (int d = lane; d < D; d += 64) st1(dx + d, 0.f);
    if (lane == 0) {
      a.lse2[srow] = __builtin_huge_valf();   // weights exp2(t - inf) = 0 on the latent side
      a.delta[srow] = 0.f;
    }
    return;
  }
  const TIn* Kl = static_cast<const TIn*>(a.Klat) + (int64_t)b * a.klat_bstride + (int64_t)h * M * D;
  const float* Zb = a.Z + bh * (int64_t)M * D;
  float x[MAXDL], g[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    x[j] = d < D ? ld1(static_cast<const TIn*>(a.Xq) + tok * D + d) : 0.f;
    g[j] = d < D ? ld1(static_cast<const TIn*>(a.dY) + tok * D + d) : 0.f;
  }
  auto score = [&](int m) {   // log2 units
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      const int d = lane + 64 * j;
      if (d < D) t = __builtin_fmaf(x[j], ld1(Kl + (int64_t)m * D + d), t);
    }
    return wave_sum(t) * a.scale_log2;
  };
  auto dgrad = [&](int m) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      const int d = lane + 64 * j;
      if (d < D) t = __builtin_fmaf(g[j], Zb[(int64_t)m * D + d], t);
    }
    return wave_sum(t);
  };
  float mx = kNegInf, l = 0.f;
  for (int m = 0; m < M; ++m) {
    const float t = score(m);
    const float nm = fmaxf(mx, t);
    l = l * exp2f(mx - nm) + exp2f(t - nm);
    mx = nm;
  }
  const float lse2 = mx + log2f(l);
  float delta = 0.f;
  for (int m = 0; m < M; ++m) delta = __builtin_fmaf(exp2f(score(m) - lse2), dgrad(m), delta);
  float acc[MAXDL] = {0.f, 0.f, 0.f, 0.f};
  for (int m = 0; m < M; ++m) {
    const float dt = exp2f(score(m) - lse2) * (dgrad(m) - delta);
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      const int d = lane + 64 * j;
      if (d < D) acc[j] = __builtin_fmaf(dt, ld1(Kl + (int64_t)m * D + d), acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) st1(dx + d, a.scale * acc[j]);
  }
  if (lane == 0) {
    a.lse2[srow] = lse2;
    a.delta[srow] = delta;
  }
}

// Latent side: one wave per latent row, over every valid token.
template <typename TIn>
__global__ __launch_bounds__(256) void dbwd_lat_generic_kernel(const DecBwdArgs a) {
  constexpr int MAXDL = 4;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  if (row >= rows) return;
  const int m = (int)(row % a.M);
  const int64_t bh = row / a.M;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int D = a.D;
  const TIn* kr = static_cast<const TIn*>(a.Klat) + (int64_t)b * a.klat_bstride + ((int64_t)h * a.M + m) * D;
  const float* zr = a.Z + row * D;
  const TIn* Xg = static_cast<const TIn*>(a.Xq) + bh * (int64_t)a.N * D;
  const TIn* Gg = static_cast<const TIn*>(a.dY) + bh * (int64_t)a.N * D;
  const uint8_t* mk = a.token_mask ? a.token_mask + (int64_t)b * a.N : nullptr;
  float kd[MAXDL], zd[MAXDL], az[MAXDL], ak[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    kd[j] = d < D ? ld1(kr + d) : 0.f;
    zd[j] = d < D ? zr[d] : 0.f;
    az[j] = ak[j] = 0.f;
  }
  for (int n = 0; n < a.N; ++n) {
    if (mk && mk[n] == 0) continue;
    float xd[MAXDL], gd[MAXDL], t = 0.f, da = 0.f;
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      const int d = lane + 64 * j;
      xd[j] = d < D ? ld1(Xg + (int64_t)n * D + d) : 0.f;
      gd[j] = d < D ? ld1(Gg + (int64_t)n * D + d) : 0.f;
      t = __builtin_fmaf(xd[j], kd[j], t);
      da = __builtin_fmaf(gd[j], zd[j], da);
    }
    t = wave_sum(t) * a.scale_log2;
    da = wave_sum(da);
    const float w = exp2f(t - a.lse2[bh * a.stats_stride + n]);
    const float dt = w * (da - a.delta[bh * a.stats_stride + n]);
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      az[j] = __builtin_fmaf(w, gd[j], az[j]);
      ak[j] = __builtin_fmaf(dt, xd[j], ak[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) {
      a.dZ[row * D + d] = az[j];
      a.dKlat[row * D + d] = a.scale * ak[j];
      if (a.dZ_cast) st1(static_cast<TIn*>(a.dZ_cast) + row * D + d, az[j]);
    }
  }
}

hipError_t launch_decode_bwd_generic(const DecBwdArgs& a, bool bf16, hipStream_t s) {
  const int64_t toks = (int64_t)a.B * a.H * a.N;
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  if (toks > 0) {
    const unsigned g = (unsigned)((toks + 3) / 4);
    if (bf16) hipLaunchKernelGGL(dbwd_tok_generic_kernel<uint16_t>, dim3(g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dbwd_tok_generic_kernel<float>, dim3(g), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    const unsigned g = (unsigned)((rows + 3) / 4);
    if (bf16) hipLaunchKernelGGL(dbwd_lat_generic_kernel<uint16_t>, dim3(g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dbwd_lat_generic_kernel<float>, dim3(g), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Matrix-core token side.  Like the forward decode: a workgroup owns one
// (batch, head) and a run of tokens, each wave 32 tokens at a time from its own
// direct-load ring (token queries and output gradients), lane = token:
//   T^T = Klat Xq^T, dA^T = Z dY^T         (A = latent rows from LDS)
//   A = softmax over the M latents (lane-local), delta = sum_m A dA
//   dT = A (dA - delta)
//   dXq^T = Klat^T dT^T                      (A = Klat^T by transposing reads)
// dXq rows leave through the consumed ring slot as whole rows; each token's
// log2-normaliser and delta go to the workspace for the latent side.
// ---------------------------------------------------------------------------
// 16-byte chunk swizzle of token row r, free of bank conflicts both for 16-lane
// reads (256 bytes per cycle) and for 8-lane writes (128 bytes per cycle) of one
// chunk per lane and row (the forward decode's layout)
__device__ __forceinline__ int tok_swz(int D, int r) {
  return D == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : D == 16 ? (((r >> 2) ^ (r >> 3)) & 1) : (r & 15);
}

template <int NI, int ST, int S>
__device__ __forceinline__ void wait_blk(int later_blocks, int later_stores) {
  // vector-memory ops issued after block j's loads: later_blocks more blocks of
  // NI loads and later_stores blocks of ST stores
#define FL_W(B, T)                                              \
  if (later_blocks == B && later_stores == T) {                 \
    wait_vm<(NI * B + ST * T) < 64 ? (NI * B + ST * T) : 63>(); \
    return;                                                     \
  }
  static_assert(S <= 3, "wait table covers S <= 3");
  static_assert(NI * (S - 2 > 0 ? S - 2 : 0) + ST * (S - 1) < 64, "vmcnt range");
  FL_W(0, 0) FL_W(0, 1) FL_W(0, 2) FL_W(1, 0) FL_W(1, 1) FL_W(1, 2)
#undef FL_W
  wait_vm<0>();
}

__device__ __forceinline__ int swap_bits2(int x) { return ((x & 1) << 1) | (x >> 1); }

template <int D, int MB, int NWV, int S>
__global__ __launch_bounds__(64 * NWV) void dbwd_tok_mfma_kernel(const DecBwdArgs a) {
  constexpr int M = 32 * MB;
  constexpr int KS = D / 16;   // k-steps over the head dim
  // 32-row blocks of dXq^T; at head dim 16 one block whose rows 16..31 are
  // products of repeated head dims, never stored
  constexpr int DB = D >= 32 ? D / 32 : 1;
  constexpr int NG = D >= 32 ? 2 : 1;   // 8-dim register groups of a block that hold head dims
  constexpr int MS = M / 16;   // k-steps over the latents
  constexpr int BLK = 32;
  constexpr int ROWB = 2 * D;
  constexpr int BB = BLK * ROWB;             // bytes of one tensor's block
  constexpr int NI = BB / 1024;              // direct loads per tensor and block
  constexpr int ST = NI + 2;                 // stores per block: dXq rows, log2-normaliser, delta
  // latent rows unpadded, 16-byte chunk c of row m at c ^ kv_swz(m): conflict-free
  // for the row reads of the score products and the transposing reads of dXq
  // FOLD (head dim 16, where the score products are cheap): the scores use the
  // bf16 pair hi + lo of s log2(e) Klat (16 significant bits), so a weight is
  // one exp2 of the product; dXq still uses Klat itself
  constexpr bool FOLD = D == 16;
  __shared__ __attribute__((aligned(1024))) uint8_t Kl[M * ROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t Zr[M * ROWB];
  __shared__ __attribute__((aligned(1024))) uint8_t Khi[FOLD ? M * ROWB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t Klo[FOLD ? M * ROWB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NWV * S * 2 * BB];
  auto lat = [](int m, int c) { return m * ROWB + ((c ^ kv_swz<D>(m)) * 16); };   // byte of chunk c, row m

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int lg = lane >> 4, li = lane & 15;
  const int nblk = (a.N + a.tokens_per_block - 1) / a.tokens_per_block;
  int bid = blockIdx.x;
  const int tb = bid % nblk;
  bid /= nblk;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int n_lo = tb * a.tokens_per_block;
  const int n_hi = min(a.N, n_lo + a.tokens_per_block);

  {  // stage latent keys and values (bf16 rows)
    constexpr int T = 64 * NWV;
    const uint16_t* kg = static_cast<const uint16_t*>(a.Klat) + (int64_t)b * a.klat_bstride + (int64_t)h * M * D;
    const float* zg = a.Z + bh * (int64_t)M * D;
    for (int f = tid; f < M * D / 8; f += T) {
      const int m = f / (D / 8), c = f % (D / 8);
      const u32x4_t kv = ld16(kg + 8 * (int64_t)f);
      st16(Kl + lat(m, c), kv);
      if constexpr (FOLD) {
        u32x4_t hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f0 = bf16lo(kv[e]) * a.scale_log2, f1 = bf16hi(kv[e]) * a.scale_log2;
          hi[e] = pack_bf16x2(f0, f1);
          lo[e] = pack_bf16x2(f0 - bf16lo(hi[e]), f1 - bf16hi(hi[e]));
        }
        st16(Khi + lat(m, c), hi);
        st16(Klo + lat(m, c), lo);
      }
      const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(zg + 8 * (int64_t)f);
      const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(zg + 8 * (int64_t)f + 4);
      st16(Zr + lat(m, c), u32x4_t{pack_bf16x2(z0[0], z0[1]), pack_bf16x2(z0[2], z0[3]), pack_bf16x2(z1[0], z1[1]),
                                   pack_bf16x2(z1[2], z1[3])});
    }
  }
  __syncthreads();   // also completes the staging loads before the ring starts
  // token validity: 64-bit words of the mask (scalar loads), or every token
  const_u64* mw = a.mask_words ? (const_u64*)(a.mask_words + (int64_t)b * a.mask_words_stride) : nullptr;

  const uint16_t* Xg = static_cast<const uint16_t*>(a.Xq) + bh * (int64_t)a.N * D;
  const uint16_t* Gg = static_cast<const uint16_t*>(a.dY) + bh * (int64_t)a.N * D;
  uint16_t* dXg = static_cast<uint16_t*>(a.dXq) + bh * (int64_t)a.N * D;
  float* lseg = a.lse2 + bh * a.stats_stride;
  float* delg = a.delta + bh * a.stats_stride;
  const float c2 = a.scale_log2;
  uint8_t* myring = ring + wave * (S * 2 * BB);
  const uint32_t myring_lds = lds_addr(myring);

  const int span = n_hi - n_lo - BLK * wave;
  const int nb = span > 0 ? (span + BLK * NWV - 1) / (BLK * NWV) : 0;
  uint32_t voff[NI], voff0[NI];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int byte = ii * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    const int ch = pc ^ tok_swz(D, r);
    voff[ii] = r * ROWB + ch * 16;
    voff0[ii] = ch * 16;
  }
  auto issue = [&](int j, int stage) {
    const int n0 = n_lo + BLK * (wave + NWV * j);
    const uint32_t st = myring_lds + stage * 2 * BB;
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      const int r = (ii * 1024) / ROWB + lane / (ROWB / 16);
      const uint32_t vo = n0 + r < n_hi ? voff[ii] : voff0[ii];
      dma16_off(Xg + (int64_t)n0 * D, vo, st + ii * 1024);
      dma16_off(Gg + (int64_t)n0 * D, vo, st + BB + ii * 1024);
    }
  };
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < nb) issue(j, j);

  const int swx = tok_swz(D, l32);
  // latent-row read offsets: rows 32*mb + swap23(l32) share one swizzle, so the
  // row block mb is an immediate offset; likewise the transposing reads' rows
  // 16*ks + .. share one swizzle per (q, db)
  int koff[KS], toff[2][DB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = lat(swap23(l32), 2 * ks + hh);
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = 8 * (lg >> 1) + 4 * q + (li >> 2);
      // head dim 16: the lanes of operand rows 16..31 read dims 0..15 again
      const int col = 32 * db + (D >= 32 ? 16 * (lg & 1) : 0) + 4 * swap_bits2(li & 3);
      toff[q][db] = lat(row, col >> 3) + (col & 7) * 2;
    }
  for (int j0 = 0; j0 < nb; j0 += S)
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int j = j0 + st;
    if (j >= nb) break;
    const int lb = min(S - 2, nb - 1 - j);
    const int ls = min(j, S - 1);
    wait_blk<2 * NI, ST, S>(lb > 0 ? lb : 0, ls);
    if (j + S - 1 < nb) issue(j + S - 1, (st + S - 1) % S);
    const int n0 = n_lo + BLK * (wave + NWV * j);
    const int n = n0 + l32;
    const bool inb = n < n_hi;
    uint8_t* xs = myring + st * 2 * BB;
    const uint8_t* gs = xs + BB;
    bf16x8_t xop[KS], gop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = l32 * ROWB + (((2 * ks + hh) ^ swx) * 16);
      xop[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + off));
      gop[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(gs + off));
    }
    // scores and dA; register r of block mb holds latent 32*mb + 16*(r/8) + 8*hh + r%8
    f32x16_t t[MB], da[MB];
    auto scores = [&]() {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        t[mb] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (FOLD) {
            t[mb] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, ld16(Khi + 32 * mb * ROWB + koff[ks])), xop[ks], t[mb]);
            t[mb] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, ld16(Klo + 32 * mb * ROWB + koff[ks])), xop[ks], t[mb]);
          } else {
            t[mb] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, ld16(Kl + 32 * mb * ROWB + koff[ks])), xop[ks], t[mb]);
          }
        }
      }
    };
    scores();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      da[mb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        da[mb] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, ld16(Zr + 32 * mb * ROWB + koff[ks])), gop[ks], da[mb]);
    }
    // Unnormalised weights p = exp2(s log2(e) (T - ref)) against a zero
    // reference, and their sum l; a token whose sum leaves [2^-64, 2^64]
    // (overflow, underflow, NaN) sends the wave through the exact form with
    // ref = the token's maximum.  The sum adds the token's own fp32 weights
    // (lane-local), so sum_m A = 1 holds to rounding.
    float ref2 = 0.f;   // the reference in log2 units
    float lsum = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        t[mb][r] = fast_exp2(FOLD ? t[mb][r] : t[mb][r] * c2);
        lsum += t[mb][r];
      }
    lsum += __shfl_xor(lsum, 32, 64);
    if (__ballot(!(lsum >= 0x1p-64f && lsum <= 0x1p64f))) {
      // (a compiler barrier: the latent rows are read again here rather than
      // kept in registers from the first products)
      asm volatile("" ::: "memory");
      scores();
      float mx = t[0][0];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmax2(mx, t[mb][r]);
      mx = fmax2(mx, __shfl_xor(mx, 32, 64));
      ref2 = FOLD ? mx : mx * c2;
      lsum = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          t[mb][r] = fast_exp2(FOLD ? t[mb][r] - ref2 : __builtin_fmaf(t[mb][r], c2, -ref2));
          lsum += t[mb][r];
        }
      lsum += __shfl_xor(lsum, 32, 64);
    }
    // A = p / l; delta = sum_m A dA; dT = A (dA - delta) = (p (dA - delta)) / l, the
    // 1/l joining the scale s of dXq below
    const float inv = 1.f / lsum;
    float delta = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) delta = __builtin_fmaf(t[mb][r], da[mb][r], delta);
    delta += __shfl_xor(delta, 32, 64);
    delta *= inv;
    bf16x8_t dtk[MS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = t[mb][8 * g + e] * (da[mb][8 * g + e] - delta);
        dtk[2 * mb + g] = __builtin_bit_cast(
            bf16x8_t, u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                              pack_bf16x2(v[6], v[7])});
      }
    // dXq^T = Klat^T dT^T; Klat^T rows (head dims) permuted so that each register
    // group holds 8 consecutive head dims: lane i of a 16-lane group reads
    // column swap23(i) of the 4x16 block
    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < MS; ++ks) {
        u32x2_t part[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
          part[q] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                    (lds_bf16x4*)(Kl + 16 * ks * ROWB + toff[q][db])));
        acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]}),
                               dtk[ks], acc[db]);
      }
    }
    const bool keep = inb && (!mw || ((mw[n0 >> 6] >> ((n0 & 63) + l32)) & 1ull));
    const float sl = a.scale * inv;   // s / l
    // stage dXq rows (register group g of lane half hh: dims 32*db + 16*g + 8*hh ..) in the consumed Xq slot
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        u32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t v = pack_bf16x2(sl * acc[db][8 * g + 2 * e], sl * acc[db][8 * g + 2 * e + 1]);
          w[e] = keep ? v : 0u;
        }
        const int pc = (4 * db + 2 * g + hh) ^ swx;
        st16(xs + l32 * ROWB + pc * 16, w);
      }
    const int valid_rows = min(BLK, n_hi - n0);
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(dXg + (int64_t)n0 * D, 0, valid_rows * ROWB, 0x00020000);
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      const int byte = ii * 1024 + lane * 16;
      const int r = byte / ROWB, pc = (byte % ROWB) / 16;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xs + byte);
      __builtin_amdgcn_raw_buffer_store_b128(v, yr, r * ROWB + ((pc ^ tok_swz(D, r)) * 16), 0, kCachePolicyNT);
    }
    // per-token statistics, negated (the latent side starts its accumulators
    // from them); lanes of the upper half and rows past the run fall outside the range
    const float lse2 = keep ? -(ref2 + __log2f(lsum)) : kNegInf;
    const float dl = keep ? -delta : 0.f;
    const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(lseg + n0, 0, valid_rows * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(delg + n0, 0, valid_rows * 4, 0x00020000);
    const int soff = hh ? (1 << 20) : l32 * 4;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse2), lr, soff, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, dl), dr, soff, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core latent side.  Like the encoder backward's query-gradient kernel:
// one workgroup per (batch, head, token chunk), wave w owns latent rows
// [32w, 32w+32) (lane = latent), 64-token tiles of Xq, dY and the tokens'
// statistics arrive through a direct-load ring:
//   S^T = Xq Klat^T, dA^T = dY Z^T          (A = token rows, B = latents in registers)
//   A = exp2(s log2e S - lse2[n]),  dT = A (dA - delta[n])   (-lse2 and -delta
//   arrive from the token side and start the accumulators of S and dA)
//   dZ^T += dY^T A^T,  dKlat^T += Xq^T dT^T  (A = transposing reads of the tiles)
// The chunk's sums go to its workspace slot (dKlat without the scale s).
// ---------------------------------------------------------------------------
template <int D, int NW, int S>
__global__ __launch_bounds__(64 * NW) void dbwd_lat_mfma_kernel(const DecBwdArgs a) {
  constexpr int TILE = 64;
  constexpr int ROWB = 2 * D;
  constexpr int TB = TILE * ROWB;
  constexpr int STAGE = 2 * TB + 1024;       // Xq tile, dY tile, statistics (512 B used)
  constexpr int NI = TB / 1024;
  // 1 KB loads per wave and tensor; a tile of fewer loads than waves (head dim
  // 16) is loaded by its first NI waves
  constexpr int NJ = NI >= NW ? NI / NW : 1;
  constexpr int KS = D / 16;
  // 32-row blocks of the products' outputs; at head dim 16 one block whose
  // rows 16..31 are products of repeated head dims, never stored
  constexpr int DB = D >= 32 ? D / 32 : 1;
  constexpr int NQ = D >= 32 ? 4 : 2;        // 4-row groups of a block that hold head dims
  constexpr int OPS = 2 * NJ + 1;            // loads per loading wave and tile (the statistics share one)
  constexpr int SPW = 32 / NW;               // 16-byte statistics pieces per wave
  static_assert(NI % NW == 0 || NI < NW, "loads must split evenly over the waves");
  static_assert(OPS * (S - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int lg = lane >> 4, li = lane & 15;
  const int nch = a.tab.nchunks;
  int bid = blockIdx.x;
  const int c = bid % nch;
  bid /= nch;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const int M = a.M;
  const uint16_t* Xg = static_cast<const uint16_t*>(a.Xq) + bh * (int64_t)a.N * D;
  const uint16_t* Gg = static_cast<const uint16_t*>(a.dY) + bh * (int64_t)a.N * D;
  const float* lseg = a.lse2 + bh * a.stats_stride;
  const float* delg = a.delta + bh * a.stats_stride;
  const_u64* mw = a.mask_words ? (const_u64*)(a.mask_words + (int64_t)b * a.mask_words_stride) : nullptr;

  const int m = 32 * wave + l32;
  bf16x8_t kop[KS], zop[KS];
  {
    const uint16_t* krow = static_cast<const uint16_t*>(a.Klat) + (int64_t)b * a.klat_bstride +
                           ((int64_t)h * M + m) * D + 8 * hh;
    const float* zrow = a.Z + (bh * M + m) * (int64_t)D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kop[ks] = __builtin_bit_cast(bf16x8_t, ld16(krow + 16 * ks));
      const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(zrow + 16 * ks);
      const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(zrow + 16 * ks + 4);
      zop[ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{pack_bf16x2(z0[0], z0[1]), pack_bf16x2(z0[2], z0[3]),
                                                     pack_bf16x2(z1[0], z1[1]), pack_bf16x2(z1[2], z1[3])});
    }
  }
  wait_vm<0>();   // only the ring's loads are in flight from here on
  const float c2 = a.scale_log2;
  // FOLD (head dim 16): the latent keys enter the score product as the bf16
  // pair hi + lo of s log2(e) Klat, so A = exp2 of the product
  constexpr bool FOLD = D == 16;
  bf16x8_t klo[KS];
  if constexpr (FOLD) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t w = __builtin_bit_cast(u32x4_t, kop[ks]);
      u32x4_t hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = bf16lo(w[e]) * c2, f1 = bf16hi(w[e]) * c2;
        hi[e] = pack_bf16x2(f0, f1);
        lo[e] = pack_bf16x2(f0 - bf16lo(hi[e]), f1 - bf16hi(hi[e]));
      }
      kop[ks] = __builtin_bit_cast(bf16x8_t, hi);
      klo[ks] = __builtin_bit_cast(bf16x8_t, lo);
    }
  }

  const int ntiles = (t_end - t_begin + TILE - 1) / TILE;
  auto tile_bits = [&](int u) -> uint64_t {
    if (u >= ntiles) return 0ull;
    const int t0 = t_begin + u * TILE;
    const int nn = t_end - t0;
    uint64_t bits = nn >= 64 ? ~0ull : ((1ull << nn) - 1ull);
    if (mw) bits &= mask_tile_bits(mw, t0);
    return bits;
  };
  const bool loads = NI >= NW || wave < NI;   // (wave-uniform)
  auto issue = [&](int u) {
    const int t0 = t_begin + u * TILE;
    const int nrows = t_end - t0;
    const uint32_t kst = lds_addr(smem) + (u % S) * STAGE;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (!loads) break;
      const int ii = wave + NW * j;
      const int byte = ii * 1024 + lane * 16;
      const int r = byte / ROWB, pc = (byte % ROWB) / 16;
      const int ch = pc ^ kv_swz<D>(r);
      const int rr = r < nrows ? r : 0;
      const int64_t off = (int64_t)(t0 + rr) * D + 8 * ch;
      dma16(Xg + off, kst + ii * 1024);
      dma16(Gg + off, kst + TB + ii * 1024);
    }
    // statistics of the tile's 64 tokens: pieces 0..15 the log2-normalisers, 16..31 the deltas
    // (the arrays are padded to whole tiles, so the reads stay in bounds)
    if (lane < SPW) {
      const int p = wave * SPW + lane;
      const float* src = p < 16 ? lseg + t0 + 4 * p : delg + t0 + 4 * (p - 16);
      dma16(src, kst + 2 * TB + wave * SPW * 16);
    }
  };

  f32x16_t accz[DB], acck[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    accz[i] = f32x16_t{};
    acck[i] = f32x16_t{};
  }
  uint64_t ring[S];
#pragma unroll
  for (int k = 0; k < S; ++k) ring[k] = 0ull;
#pragma unroll
  for (int k = 0; k < S - 1; ++k) {
    ring[k] = tile_bits(k);
    if (ring[k]) issue(k);
  }
  const int swk = kv_swz<D>(swap23(l32));
  for (int t = 0; t < ntiles; ++t) {
    int later = 0;
#pragma unroll
    for (int k = 1; k < S - 1; ++k) later += ring[k] != 0ull;
    // a wave that loads no tile rows issues the statistics piece alone
    if (loads)
      wait_tiles<OPS, S>(later);
    else
      wait_tiles<1, S>(later);
    barrier_lds();
    ring[S - 1] = tile_bits(t + S - 1);
    if (ring[S - 1]) issue(t + S - 1);
    const uint64_t bits = ring[0];
    if (bits) {
      uint8_t* xst = smem + (t % S) * STAGE;
      uint8_t* gst = xst + TB;
      const float* stt = reinterpret_cast<const float*>(xst + 2 * TB);
      if (bits != ~0ull) {
        // invalid rows of both tiles become zero: they meet A = dT = 0
        for (int f = tid; f < TILE * (ROWB / 16); f += 64 * NW) {
          const int r = f / (ROWB / 16), pc = f % (ROWB / 16);
          if (!((bits >> r) & 1ull)) {
            st16(xst + r * ROWB + pc * 16, u32x4_t{0, 0, 0, 0});
            st16(gst + r * ROWB + pc * 16, u32x4_t{0, 0, 0, 0});
          }
        }
        barrier_lds();
      }
      const uint64_t lb = bits >> (8 * hh);
      const bool full = bits == ~0ull;
      bf16x8_t pa[4], pd[4];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        // register r of lane half hh holds token 32*b2 + 16*(r/8) + 8*hh + r%8: the
        // tokens' -lse2 and -delta in the same order start the accumulators
        f32x16_t nl, nd;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int t0 = 32 * b2 + 16 * g + 8 * hh;
          const f32x4_t l0 = *reinterpret_cast<const f32x4_t*>(stt + t0);
          const f32x4_t l1 = *reinterpret_cast<const f32x4_t*>(stt + t0 + 4);
          const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(stt + 64 + t0);
          const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(stt + 64 + t0 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            nl[8 * g + e] = l0[e];
            nl[8 * g + 4 + e] = l1[e];
            nd[8 * g + e] = d0[e];
            nd[8 * g + 4 + e] = d1[e];
          }
        }
        f32x16_t sc = FOLD ? nl : f32x16_t{}, da = nd;
        const uint8_t* xrow = xst + (32 * b2 + swap23(l32)) * ROWB;
        const uint8_t* grow = gst + (32 * b2 + swap23(l32)) * ROWB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = (2 * ks + hh) ^ swk;
          const bf16x8_t xo = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xrow + ch * 16));
          sc = mfma32x32x16(xo, kop[ks], sc);
          if constexpr (FOLD) sc = mfma32x32x16(xo, klo[ks], sc);
          da = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(grow + ch * 16)),
                            zop[ks], da);
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float pv[8], dv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * g + e;
            pv[e] = fast_exp2(FOLD ? sc[r] : __builtin_fmaf(sc[r], c2, nl[r]));
            dv[e] = pv[e] * da[r];
          }
          if (!full) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              if (!((lb >> (32 * b2 + 16 * g + e)) & 1ull)) {
                pv[e] = 0.f;
                dv[e] = 0.f;
              }
            }
          }
          pa[2 * b2 + g] = __builtin_bit_cast(
              bf16x8_t, u32x4_t{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                                pack_bf16x2(pv[6], pv[7])});
          pd[2 * b2 + g] = __builtin_bit_cast(
              bf16x8_t, u32x4_t{pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3]), pack_bf16x2(dv[4], dv[5]),
                                pack_bf16x2(dv[6], dv[7])});
        }
      }
      // dZ^T += dY^T A^T and dKlat^T += Xq^T dT^T through transposing reads of the tiles
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // head dim 16: the lanes of operand rows 16..31 read dims 0..15 again
        const int d0 = 32 * db + (D >= 32 ? 16 * (lg & 1) : 0) + 4 * (li & 3);
        const int chl = d0 >> 3, half = (d0 & 7) * 2;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x2_t pg[2], px[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int nn = 16 * ks + 8 * (lg >> 1) + 4 * q + (li >> 2);
            const int off = nn * ROWB + ((chl ^ kv_swz<D>(nn)) * 16) + half;
            pg[q] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(gst + off)));
            px[q] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(xst + off)));
          }
          accz[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, u32x4_t{pg[0][0], pg[0][1], pg[1][0], pg[1][1]}),
                                  pa[ks], accz[db]);
          acck[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, u32x4_t{px[0][0], px[0][1], px[1][0], px[1][1]}),
                                  pd[ks], acck[db]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < S - 1; ++k) ring[k] = ring[k + 1];
  }
  // chunk sums -> workspace slot (row m, dims d): [slot][bh][2][M][D]
  float* W = a.ws_part + (((int64_t)a.tab.slot[c] * a.B * a.H + bh) * 2) * (int64_t)M * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int64_t off = (int64_t)m * D + 32 * db + 8 * q + 4 * hh;
      *reinterpret_cast<f32x4_t*>(W + off) = f32x4_t{accz[db][4 * q], accz[db][4 * q + 1], accz[db][4 * q + 2],
                                                     accz[db][4 * q + 3]};
      *reinterpret_cast<f32x4_t*>(W + (int64_t)M * D + off) =
          f32x4_t{acck[db][4 * q], acck[db][4 * q + 1], acck[db][4 * q + 2], acck[db][4 * q + 3]};
    }
}

// dZ = sum of the chunk slots, dKlat = s * sum (fixed order); dZ optionally also in bf16
__global__ __launch_bounds__(256) void dbwd_reduce_kernel(const float* __restrict__ ws, int nslots, int64_t bhs,
                                                          int64_t md4, float scale, float* __restrict__ dZ,
                                                          float* __restrict__ dK, uint16_t* __restrict__ dZb) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over bhs * md4
  if (i >= bhs * md4) return;
  const int64_t bh = i / md4, e = i % md4;
  f32x4_t sz = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < nslots; ++k) {
    const f32x4_t* base = reinterpret_cast<const f32x4_t*>(ws) + ((int64_t)k * bhs + bh) * 2 * md4;
    sz += base[e];
    sk += base[md4 + e];
  }
  reinterpret_cast<f32x4_t*>(dZ)[i] = sz;
  reinterpret_cast<f32x4_t*>(dK)[i] = sk * scale;
  if (dZb) reinterpret_cast<u32x2_t*>(dZb)[i] = u32x2_t{pack_bf16x2(sz[0], sz[1]), pack_bf16x2(sz[2], sz[3])};
}

bool decode_bwd_mfma_supported(int M, int D) {
  return (D == 16 || D == 64 || D == 128) && (M == 32 || M == 64 || M == 128);
}

// token-side waves per workgroup: at D=64 eight waves with 2-stage rings fill the
// LDS (128 KB of rings, up to 32 KB of latents), two waves per SIMD; D=16 the same
// with quarter-size rings
int decode_bwd_waves(int D) { return D == 128 ? 2 : 8; }

template <int D, int MB>
static hipError_t launch_dbwd_t(const DecBwdArgs& a, hipStream_t s) {
  constexpr int NWV = D == 128 ? 2 : 8;
  constexpr int S = 2;
  const int64_t nblk = (a.N + a.tokens_per_block - 1) / a.tokens_per_block;
  hipLaunchKernelGGL((dbwd_tok_mfma_kernel<D, MB, NWV, S>), dim3((unsigned)(nblk * a.H * a.B)), dim3(64 * NWV), 0,
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NW = MB;
  hipLaunchKernelGGL((dbwd_lat_mfma_kernel<D, NW, 3>), dim3((unsigned)((int64_t)a.tab.nchunks * a.H * a.B)),
                     dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_bwd_mfma(const DecBwdArgs& a, hipStream_t s) {
  if (a.tokens_per_block > 8192 || a.tokens_per_block % (32 * decode_bwd_waves(a.D)) != 0)
    return hipErrorInvalidValue;
  if (a.D == 64) {
    switch (a.M) {
      case 32: return launch_dbwd_t<64, 1>(a, s);
      case 64: return launch_dbwd_t<64, 2>(a, s);
      case 128: return launch_dbwd_t<64, 4>(a, s);
    }
  } else if (a.D == 16) {
    switch (a.M) {
      case 32: return launch_dbwd_t<16, 1>(a, s);
      case 64: return launch_dbwd_t<16, 2>(a, s);
      case 128: return launch_dbwd_t<16, 4>(a, s);
    }
  } else if (a.D == 128) {
    switch (a.M) {
      case 32: return launch_dbwd_t<128, 1>(a, s);
      case 64: return launch_dbwd_t<128, 2>(a, s);
      case 128: return launch_dbwd_t<128, 4>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_bwd_reduce(const DecBwdArgs& a, bool bf16, hipStream_t s) {
  const int64_t bhs = (int64_t)a.B * a.H;
  const int64_t md4 = (int64_t)a.M * a.D / 4;
  if (bhs * md4 == 0) return hipSuccess;
  hipLaunchKernelGGL(dbwd_reduce_kernel, dim3((unsigned)((bhs * md4 + 255) / 256)), dim3(256), 0, s, a.ws_part,
                     a.tab.nchunks, bhs, md4, a.scale, a.dZ, a.dKlat,
                     static_cast<uint16_t*>(bf16 ? a.dZ_cast : nullptr));
  return hipGetLastError();
}

}  // namespace flare
