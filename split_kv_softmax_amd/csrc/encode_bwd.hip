// Encoder backward with the global statistics ("FLARE++: Low-rank attention
// with dynamic attention routing", appendix on context parallelism, backward
// paragraph): the probabilities of every partition are normalised by the
// global log-normaliser L of the forward pass, P = exp(s q.k - L); the row
// term c = rowsum(dZ * Z) carries the redistribution of mass between
// partitions; dS = P (dZ.v - c); dV = P^T dZ, dK = s dS^T Q, and the query
// gradient s dS K is summed over all partitions.
#include "common.h"
#include "kernels.h"

namespace flare {

// c[row] = sum_d dZ[row, d] * Z[row, d]  (one wave per row)
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const TIn* __restrict__ dZ, const float* __restrict__ Z,
                                                         int64_t rows, int D, float* __restrict__ c) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  for (int d = lane; d < D; d += 64) {
    float g;
    if constexpr (sizeof(TIn) == 2) g = bf16_to_f32(dZ[row * D + d]); else g = dZ[row * D + d];
    acc = __builtin_fmaf(g, Z[row * D + d], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) c[row] = acc;
}

template <typename TIn>
__device__ __forceinline__ float ldg_(const TIn* p) {
  if constexpr (sizeof(TIn) == 2) return bf16_to_f32(*p); else return *p;
}
template <typename TIn>
__device__ __forceinline__ void stg_(TIn* p, float v) {
  if constexpr (sizeof(TIn) == 2) *p = to_bf16(v); else *p = v;
}
// v as stored in TIn, widened back (the identity for float)
template <typename TIn>
__device__ __forceinline__ float rnd_(float v) {
  if constexpr (sizeof(TIn) == 2) return bf16_to_f32(to_bf16(v)); else return v;
}

// ---------------------------------------------------------------------------
// General vector kernels (float32 inputs, or shapes without a matrix-core
// variant).  Float32 arithmetic throughout.
// ---------------------------------------------------------------------------
// dK, dV of one token per wave: lanes take head dims; the score and dP of each
// latent row are wave reductions.
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_kv_generic_kernel(const BwdArgs a) {
  constexpr int MAXDL = 4;   // D <= 256
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)a.B * a.H * a.N;
  if (tok >= total) return;
  const int n = (int)(tok % a.N);
  const int64_t bh = tok / a.N;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int D = a.D, M = a.M;
  TIn* dk = static_cast<TIn*>(a.dK) + tok * D;
  TIn* dv = static_cast<TIn*>(a.dV) + tok * D;
  const bool valid = !a.mask || a.mask[(int64_t)b * a.N + n] != 0;
  float kk[MAXDL], vv[MAXDL], ak[MAXDL], av[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    kk[j] = (valid && d < D) ? ldg_(static_cast<const TIn*>(a.K) + tok * D + d) : 0.f;
    vv[j] = (valid && d < D) ? ldg_(static_cast<const TIn*>(a.V) + tok * D + d) : 0.f;
    ak[j] = av[j] = 0.f;
  }
  if (valid) {
    const TIn* Q = static_cast<const TIn*>(a.Q) + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    const TIn* dZ = static_cast<const TIn*>(a.dZ) + bh * (int64_t)M * D;
    const float* Lr = a.L + bh * M;
    const float* cr = a.c + bh * M;
    for (int m = 0; m < M; ++m) {
      const float Lm = Lr[m];
      if (Lm == kNegInf) continue;   // row without any valid key: no gradient
      float qd[MAXDL], gd[MAXDL], sq = 0.f, sp = 0.f;
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) {
        const int d = lane + 64 * j;
        qd[j] = d < D ? ldg_(Q + (int64_t)m * D + d) : 0.f;
        gd[j] = d < D ? ldg_(dZ + (int64_t)m * D + d) : 0.f;
        sq = __builtin_fmaf(qd[j], kk[j], sq);
        sp = __builtin_fmaf(gd[j], vv[j], sp);
      }
      sq = wave_sum(sq);
      sp = wave_sum(sp);
      const float p = __expf(a.scale * sq - Lm);
      const float ds = p * (sp - cr[m]);
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) {
        av[j] = __builtin_fmaf(p, gd[j], av[j]);
        ak[j] = __builtin_fmaf(ds, qd[j], ak[j]);
      }
    }
  }
  // an accumulating call adds exactly the gradient a writing call stores: the
  // product is rounded to float (never contracted into the add) and then to the
  // output type before the add
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) {
#pragma clang fp contract(off)
      const float gk = a.scale * ak[j];
      stg_(dv + d, a.accumulate_dv ? rnd_<TIn>(av[j]) + ldg_(dv + d) : av[j]);
      stg_(dk + d, a.accumulate_dk ? rnd_<TIn>(gk) + ldg_(dk + d) : gk);
    }
  }
}

// dQ of one latent row per wave, summed over every valid token.
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_q_generic_kernel(const BwdArgs a) {
  constexpr int MAXDL = 4;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  if (row >= rows) return;
  const int m = (int)(row % a.M);
  const int64_t bh = row / a.M;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int D = a.D;
  const TIn* Qr = static_cast<const TIn*>(a.Q) + (int64_t)b * a.q_bstride + ((int64_t)h * a.M + m) * D;
  const TIn* gr = static_cast<const TIn*>(a.dZ) + row * D;
  const TIn* Kg = static_cast<const TIn*>(a.K) + bh * (int64_t)a.N * D;
  const TIn* Vg = static_cast<const TIn*>(a.V) + bh * (int64_t)a.N * D;
  const uint8_t* mk = a.mask ? a.mask + (int64_t)b * a.N : nullptr;
  const float Lm = a.L[row], cm = a.c[row];
  float qd[MAXDL], gd[MAXDL], acc[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    qd[j] = d < D ? ldg_(Qr + d) : 0.f;
    gd[j] = d < D ? ldg_(gr + d) : 0.f;
    acc[j] = 0.f;
  }
  if (Lm != kNegInf) {
    for (int n = 0; n < a.N; ++n) {
      if (mk && mk[n] == 0) continue;
      float kd[MAXDL], sq = 0.f, sp = 0.f;
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) {
        const int d = lane + 64 * j;
        kd[j] = d < D ? ldg_(Kg + (int64_t)n * D + d) : 0.f;
        const float vd = d < D ? ldg_(Vg + (int64_t)n * D + d) : 0.f;
        sq = __builtin_fmaf(qd[j], kd[j], sq);
        sp = __builtin_fmaf(gd[j], vd, sp);
      }
      sq = wave_sum(sq);
      sp = wave_sum(sp);
      const float ds = __expf(a.scale * sq - Lm) * (sp - cm);
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) acc[j] = __builtin_fmaf(ds, kd[j], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) {
#pragma clang fp contract(off)
      const float g = a.scale * acc[j];   // rounded before an accumulating add, as when written
      const float r = a.accumulate_dq ? g + a.dQ[row * D + d] : g;
      a.dQ[row * D + d] = r;
      if (a.dQ_cast) stg_(static_cast<TIn*>(a.dQ_cast) + row * D + d, r);
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core query gradient.  Same shape as the encoder: one workgroup per
// (batch, head, token chunk), wave w owns latent rows [32w, 32w+32), K and V
// tiles arrive through a direct-load LDS ring.  Per 64-token tile:
//   S^T  = K Q^T,  dP^T = V dZ^T                 (A = K / V rows, B = Q / dZ)
//   dS^T = P (dP - c) with P = exp(s S - L)       (L, c per lane: lane = row)
//   dQ^T += K^T dS^T                               (A = K^T by transposing reads)
// The chunk's unscaled sum goes to its workspace slot; bwd_dq_reduce adds the
// chunks in order and applies s.
// ---------------------------------------------------------------------------
template <int D, int NW, int S>
__global__ __launch_bounds__(64 * NW) void bwd_dq_mfma_kernel(const BwdArgs a) {
  constexpr int TILE = 64;
  constexpr int ROWB = 2 * D;
  constexpr int TB = TILE * ROWB;
  constexpr int STAGE = 2 * TB;
  constexpr int NI = TB / 1024;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int OPS = 2 * NI / NW;
  static_assert(NI % NW == 0, "loads must split evenly over the waves");
  static_assert(OPS * (S - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int nch = a.tab.nchunks;
  int bid = ordered_block(a.order);
  const int c = bid % nch;
  bid /= nch;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + bh * (int64_t)a.N * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + bh * (int64_t)a.N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + (int64_t)b * a.q_bstride + (int64_t)h * a.M * D;
  const uint16_t* Gg = static_cast<const uint16_t*>(a.dZ) + bh * (int64_t)a.M * D;
  const_u64* mw = a.mask_words ? (const_u64*)(a.mask_words + (int64_t)b * a.mask_words_stride) : nullptr;

  const int m = 32 * wave + l32;
  bf16x8_t qop[KS], gop[KS];
  {
    const uint16_t* qrow = Qg + (int64_t)m * D + 8 * hh;
    const uint16_t* grow = Gg + (int64_t)m * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qop[ks] = __builtin_bit_cast(bf16x8_t, ld16(qrow + 16 * ks));
      gop[ks] = __builtin_bit_cast(bf16x8_t, ld16(grow + 16 * ks));
    }
  }
  const float Lm = a.L[bh * a.M + m];
  const float cm = a.c[bh * a.M + m];
  wait_vm<0>();   // only the ring's loads are in flight from here on
  const float c2 = a.scale_log2;
  // P = exp2(s*log2e*S - L*log2e); a row with L = -inf gets P = 0
  const float nl2 = (Lm == kNegInf) ? __builtin_huge_valf() : Lm * kLog2e;

  const int ntiles = (t_end - t_begin + TILE - 1) / TILE;
  auto tile_bits = [&](int u) -> uint64_t {
    if (u >= ntiles) return 0ull;
    const int t0 = t_begin + u * TILE;
    const int n = t_end - t0;
    uint64_t bits = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
    if (mw) bits &= mask_tile_bits(mw, t0);
    return bits;
  };
  auto issue = [&](int u) {
    const int t0 = t_begin + u * TILE;
    const int nrows = t_end - t0;
    const uint32_t kst = lds_addr(smem) + (u % S) * STAGE;
#pragma unroll
    for (int j = 0; j < NI / NW; ++j) {
      const int ii = wave + NW * j;
      const int byte = ii * 1024 + lane * 16;
      const int r = byte / ROWB, pc = (byte % ROWB) / 16;
      const int ch = pc ^ kv_swz<D>(r);
      const int rr = r < nrows ? r : 0;
      const int64_t off = (int64_t)(t0 + rr) * D + 8 * ch;
      dma16(Kg + off, kst + ii * 1024);
      dma16(Vg + off, kst + TB + ii * 1024);
    }
  };

  f32x16_t acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16_t{};
  uint64_t ring[S];
#pragma unroll
  for (int k = 0; k < S; ++k) ring[k] = 0ull;
#pragma unroll
  for (int k = 0; k < S - 1; ++k) {
    ring[k] = tile_bits(k);
    if (ring[k]) issue(k);
  }
  const int swk = kv_swz<D>(swap23(l32));   // rows 32*b2 + swap23(l32)
  for (int t = 0; t < ntiles; ++t) {
    int later = 0;
#pragma unroll
    for (int k = 1; k < S - 1; ++k) later += ring[k] != 0ull;
    wait_tiles<OPS, S>(later);
    barrier_lds();
    ring[S - 1] = tile_bits(t + S - 1);
    if (ring[S - 1]) issue(t + S - 1);
    const uint64_t bits = ring[0];
    if (bits) {
      uint8_t* kst = smem + (t % S) * STAGE;
      uint8_t* vst = kst + TB;
      if (bits != ~0ull) {
        // invalid rows of both K and V become zero: they meet P = 0 and dS = 0
        for (int f = tid; f < TILE * (ROWB / 16); f += 64 * NW) {
          const int r = f / (ROWB / 16), pc = f % (ROWB / 16);
          if (!((bits >> r) & 1ull)) {
            st16(kst + r * ROWB + pc * 16, u32x4_t{0, 0, 0, 0});
            st16(vst + r * ROWB + pc * 16, u32x4_t{0, 0, 0, 0});
          }
        }
        barrier_lds();
      }
      f32x16_t sc[2], dp[2];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        sc[b2] = f32x16_t{};
        dp[b2] = f32x16_t{};
        const uint8_t* krow = kst + (32 * b2 + swap23(l32)) * ROWB;
        const uint8_t* vrow = vst + (32 * b2 + swap23(l32)) * ROWB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = (2 * ks + hh) ^ swk;
          sc[b2] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(krow + ch * 16)),
                                qop[ks], sc[b2]);
          dp[b2] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(vrow + ch * 16)),
                                gop[ks], dp[b2]);
        }
      }
      // register r of lane half hh in block b2 holds token 32*b2 + 16*(r/8) + 8*hh + r%8
      const uint64_t lb = bits >> (8 * hh);
      const bool full = bits == ~0ull;   // uniform: no per-element masking for whole tiles
      bf16x8_t pk[4];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 8 * g + j;
            const float p = fast_exp2(__builtin_fmaf(sc[b2][r], c2, -nl2));
            ds[j] = p * (dp[b2][r] - cm);
          }
          if (!full) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int tk = 32 * b2 + 16 * g + j;
              if (!((lb >> tk) & 1ull)) ds[j] = 0.f;
            }
          }
          u32x4_t w;
          w[0] = pack_bf16x2(ds[0], ds[1]);
          w[1] = pack_bf16x2(ds[2], ds[3]);
          w[2] = pack_bf16x2(ds[4], ds[5]);
          w[3] = pack_bf16x2(ds[6], ds[7]);
          pk[2 * b2 + g] = __builtin_bit_cast(bf16x8_t, w);
        }
      // dQ^T += K^T dS^T through transposing reads of the K tile
      const int lg = lane >> 4, li = lane & 15;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d0 = 32 * db + 16 * (lg & 1) + 4 * (li & 3);
        const int chl = d0 >> 3, half = (d0 & 7) * 2;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          u32x2_t part[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int n = 16 * ks + 8 * (lg >> 1) + 4 * q + (li >> 2);
            const uint8_t* src = kst + n * ROWB + ((chl ^ kv_swz<D>(n)) * 16) + half;
            part[q] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)src));
          }
          const u32x4_t av = {part[0][0], part[0][1], part[1][0], part[1][1]};
          acc[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), pk[ks], acc[db]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < S - 1; ++k) ring[k] = ring[k + 1];
  }
  // unscaled chunk sum -> workspace slot c (row m, dims d)
  float* W = a.ws_dq + (((int64_t)a.tab.slot[c] * a.B + b) * a.H + h) * (int64_t)a.M * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4_t v = {acc[db][4 * q], acc[db][4 * q + 1], acc[db][4 * q + 2], acc[db][4 * q + 3]};
      *reinterpret_cast<f32x4_t*>(W + (int64_t)m * D + 32 * db + 8 * q + 4 * hh) = v;
    }
}

// ---------------------------------------------------------------------------
// Matrix-core key/value gradients (FLARE++ appendix, backward pass): one
// workgroup per (b, h, token chunk); 64-token tiles through a direct-load ring.
// Phase A (one wave per 32 latent rows, lane = latent row):
//   S^T = K Q^T, dP^T = V dZ^T, P = exp(s S - L), s dS = P (s dP - s c)
//   P and s dS go to LDS as bf16 [m][token] (128-byte rows, pd_swz); with DQ the wave also adds
//   K^T (s dS)^T into its query-gradient partial (so those partials already carry s).
// Phase B (each wave one gradient tensor and a slice of output blocks,
// lane = token):
//   dV^T = dZ^T P,  dK^T = Q^T (s dS)      (contraction over the M latents)
// with dZ^T / Q^T slices held in registers for the whole chunk.  The tile's
// gradients are staged in the tile's own K/V slot and leave as whole
// coalesced rows.  Padded tokens get P = dS = 0, hence zero rows; tiles with
// no valid token are not loaded and only write zeros.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swap_bits2(int x) { return ((x & 1) << 1) | (x >> 1); }

// 16-byte chunk swizzle of the P / dS rows (128 bytes: 64 tokens of one latent).
// Phase A writes one chunk per lane and row, lanes on consecutive rows, and a
// 16-byte LDS write serves 8 lanes (128 bytes) per cycle, so the swizzle must be
// a bijection on r mod 8.  Phase B reads them transposed, 8 bytes per lane and
// 32 lanes (256 bytes) per cycle over four consecutive rows 4k..4k+3 and four
// chunks, where bit 1 of the row on bit 2 of the chunk keeps rows r and r+2
// (same bank half) apart.  The token-row swizzle of head dim 64 has the second
// property but repeats on row pairs; flipping both low chunk bits on odd rows
// gives the first as well.
__device__ __forceinline__ int pd_swz(int r) { return kv_swz<64>(r) ^ ((r & 1) * 3); }

template <int D, int M, int NW, int S, bool DQ, int ACC>
__global__ __launch_bounds__(64 * NW) void bwd_kv_mfma_kernel(const BwdArgs a) {
  constexpr int TILE = 64;
  constexpr int ROWB = 2 * D;          // bytes of one K/V/gradient row
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int TB = TILE * ROWB;
  constexpr int STAGE = 2 * TB;
  constexpr int NI = TB / 1024;
  constexpr int KS = D / 16;           // contraction steps over the head dim
  constexpr int KM = M / 16;           // contraction steps over the latents
  // 32-row head-dim blocks; at head dim 16 one block whose rows 16..31 are
  // products of repeated head dims, never stored
  constexpr int DB = D >= 32 ? D / 32 : 1;
  constexpr int NG = D >= 32 ? 2 : 1;  // 8-dim register groups of a block that hold head dims
  constexpr int MW = M / 32;           // waves with latent rows in phase A
  // loads per wave and tile; a 2 KB tile (head dim 16) is one 1 KB piece of K
  // or of V per wave, waves 0..NI-1 taking K and NI..2NI-1 taking V
  constexpr bool SPLIT = NI < NW;
  static_assert(!SPLIT || NW == 2 * NI, "one load per wave");
  constexpr int OPS = SPLIT ? 1 : 2 * NI / NW;
  constexpr int PDS = M * TILE * 2;    // one bf16 [M][64] buffer
  constexpr int RING = S * STAGE;
  constexpr int LDS_MAIN = RING + 2 * PDS;
  constexpr int LDS_STAT = 2 * M * D * 2;
  constexpr int LDS = LDS_MAIN > LDS_STAT ? LDS_MAIN : LDS_STAT;
  constexpr int WPT = NW / 2;          // phase-B waves per gradient tensor
  constexpr int NDW = DB >= WPT ? DB / WPT : 1;
  constexpr int NNB = DB >= WPT ? 2 : 2 * DB / WPT;
  constexpr int CPT = 2 * TILE * CPR / (64 * NW);   // copy-out chunks per thread
  // CPT even: each thread owns CPT/2 chunks of dK and as many of dV; CPT = 1
  // (head dim 16): threads 0..TILE*CPR-1 own one chunk of dK, the others one of dV
  static_assert((CPT % 2 == 0 || CPT == 1) && CPT * 64 * NW == 2 * TILE * CPR, "copy-out split");
  static_assert((S - 2) * OPS + (S - 1) * CPT < 64, "vmcnt range");
  static_assert(NI % NW == 0 || SPLIT, "loads must split evenly over the waves");
  static_assert(MW <= NW && NW % 2 == 0 && WPT <= 2 * DB, "wave layout");
  static_assert(OPS * (S - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  uint8_t* pbuf = smem + RING;
  uint8_t* dsbuf = pbuf + PDS;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int lg = lane >> 4, li = lane & 15;
  const int nch = a.tab.nchunks;
  int bid = ordered_block(a.order);
  const int c = bid % nch;
  bid /= nch;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + bh * (int64_t)a.N * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + bh * (int64_t)a.N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
  const uint16_t* Gg = static_cast<const uint16_t*>(a.dZ) + bh * (int64_t)M * D;
  uint16_t* dKg = static_cast<uint16_t*>(a.dK) + bh * (int64_t)a.N * D;
  uint16_t* dVg = static_cast<uint16_t*>(a.dV) + bh * (int64_t)a.N * D;
  const_u64* mw = a.mask_words ? (const_u64*)(a.mask_words + (int64_t)b * a.mask_words_stride) : nullptr;

  // ---- stationary operands: Q and dZ through LDS ([m][d], row-major) ----
  for (int f = tid; f < M * CPR; f += 64 * NW) {
    const int r = f / CPR, ch = f % CPR;
    const u32x4_t q = ld16(Qg + (int64_t)r * D + 8 * ch);
    const u32x4_t g = ld16(Gg + (int64_t)r * D + 8 * ch);
    st16(smem + r * ROWB + ch * 16, q);
    st16(smem + M * ROWB + r * ROWB + ch * 16, g);
  }
  __syncthreads();
  const bool pa = wave < MW;           // wave has latent rows in phase A
  const int m = 32 * (pa ? wave : 0) + l32;
  bf16x8_t qop[KS], gop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qop[ks] = __builtin_bit_cast(bf16x8_t, ld16(smem + m * ROWB + (16 * ks + 8 * hh) * 2));
    gop[ks] = __builtin_bit_cast(bf16x8_t, ld16(smem + M * ROWB + m * ROWB + (16 * ks + 8 * hh) * 2));
  }
  // phase-B role: tensor t (0 = dV from dZ^T, 1 = dK from Q^T), d-blocks, n-blocks
  const int tsel = wave / WPT, wi = wave % WPT;
  const int db0 = DB >= WPT ? wi * NDW : wi % DB;
  const int nb0 = DB >= WPT ? 0 : (wi / DB) * NNB;
  // A operand rows permuted so that each register group holds 8 consecutive d:
  // lane i of a 16-lane group reads column swap23(i) of the 4x16 block
  bf16x8_t ast[NDW][KM];
  {
    const uint8_t* src = smem + (tsel == 0 ? M * ROWB : 0);
#pragma unroll
    for (int j = 0; j < NDW; ++j)
#pragma unroll
      for (int ks = 0; ks < KM; ++ks) {
        u32x2_t part[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int row = 16 * ks + 8 * (lg >> 1) + 4 * q + (li >> 2);
          // head dim 16: the lanes of operand rows 16..31 read dims 0..15 again
          const int col = 32 * (db0 + j) + (D >= 32 ? 16 * (lg & 1) : 0) + 4 * swap_bits2(li & 3);
          part[q] = __builtin_bit_cast(
              u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(src + row * ROWB + col * 2)));
        }
        ast[j][ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]});
      }
  }
  const float Lm = a.L[bh * M + m];
  // FOLD (head dim 16, where the score products are cheap): Q enters the score
  // product as the bf16 pair hi + lo of s log2(e) Q with the accumulator
  // starting at -L log2(e), so P = exp2 of the product; dP's accumulator starts
  // at -c, so dS = P dP is one product per weight, unscaled (s is applied to
  // the key-gradient rows at staging and to the query gradient by the reduce)
  constexpr bool FOLD = D == 16;
  const float cms = FOLD ? a.c[bh * M + m] : a.scale * a.c[bh * M + m];
  wait_vm<0>();
  barrier_lds();   // the stationary copy is dead from here on: the ring reuses it
  const float c2 = a.scale_log2;
  const float sc1 = a.scale;
  const float nl2 = (Lm == kNegInf) ? __builtin_huge_valf() : Lm * kLog2e;
  bf16x8_t qlo[KS];
  f32x16_t sinit = f32x16_t{}, dpinit = f32x16_t{};
  if constexpr (FOLD) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t w = __builtin_bit_cast(u32x4_t, qop[ks]);
      u32x4_t hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = bf16lo(w[e]) * c2, f1 = bf16hi(w[e]) * c2;
        hi[e] = pack_bf16x2(f0, f1);
        lo[e] = pack_bf16x2(f0 - bf16lo(hi[e]), f1 - bf16hi(hi[e]));
      }
      qop[ks] = __builtin_bit_cast(bf16x8_t, hi);
      qlo[ks] = __builtin_bit_cast(bf16x8_t, lo);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sinit[r] = -nl2;   // -inf for a row without any valid key: P = 0
      dpinit[r] = -cms;
    }
  }

  const int ntiles = (t_end - t_begin + TILE - 1) / TILE;
  auto tile_bits = [&](int u) -> uint64_t {
    if (u >= ntiles) return 0ull;
    const int t0 = t_begin + u * TILE;
    const int n = t_end - t0;
    uint64_t bits = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
    if (mw) bits &= mask_tile_bits(mw, t0);
    return bits;
  };
  auto issue = [&](int u) {
    const int t0 = t_begin + u * TILE;
    const int nrows = t_end - t0;
    const uint32_t kst = lds_addr(smem) + (u % S) * STAGE;
    if constexpr (SPLIT) {
      const int ii = wave % NI;
      const bool isv = wave >= NI;   // (wave-uniform)
      const int byte = ii * 1024 + lane * 16;
      const int r = byte / ROWB, pc = (byte % ROWB) / 16;
      const int ch = pc ^ kv_swz<D>(r);
      const int rr = r < nrows ? r : 0;
      const int64_t off = (int64_t)(t0 + rr) * D + 8 * ch;
      dma16((isv ? Vg : Kg) + off, kst + (isv ? TB : 0) + ii * 1024);
      return;
    }
#pragma unroll
    for (int j = 0; j < NI / NW; ++j) {
      const int ii = wave + NW * j;
      const int byte = ii * 1024 + lane * 16;
      const int r = byte / ROWB, pc = (byte % ROWB) / 16;
      const int ch = pc ^ kv_swz<D>(r);
      const int rr = r < nrows ? r : 0;
      const int64_t off = (int64_t)(t0 + rr) * D + 8 * ch;
      dma16(Kg + off, kst + ii * 1024);
      dma16(Vg + off, kst + TB + ii * 1024);
    }
  };
  // staged gradient rows: 16-byte chunk ch of row n sits at ch ^ out_swz(n); each
  // lane writes one chunk of its own row (8 lanes, consecutive rows, per write
  // cycle), and the copy-out reads whole rows, so any swizzle that differs over 8
  // consecutive rows within a 128-byte bank window is conflict-free both ways
  // DIRECT (head dim 16): a gradient row is 32 bytes, so the 16-byte piece each
  // lane holds after phase B (token 32*nb + l32, chunk hh) already makes one
  // store of the wave a contiguous 1 KB of whole rows; the pieces leave straight
  // from registers, one store per lane and tile like the staged copy-out (the
  // ring's wait counts rely on that), with no staging and no barrier before it.
  // Not for the accumulating forms: their old rows, read by the lane itself,
  // would be consumed right after phase B, and the compiler's (in-order) wait
  // for them then also covers the ring loads issued at the top of the tile
  // (measured 2% slower; the staged copy-out consumes them a barrier later).
  constexpr bool DIRECT = D == 16 && ACC == 0;
  static_assert(!DIRECT || (CPT == 1 && NDW == 1 && NNB == 1 && NG == 1), "one piece per lane and tile");
  auto out_swz = [](int n) { return D == 64 ? (n & 7) : D == 16 ? (((n >> 2) ^ (n >> 3)) & 1) : (n & 15); };

  f32x16_t dq[DQ ? DB : 1];
#pragma unroll
  for (int i = 0; i < (DQ ? DB : 1); ++i) dq[i] = f32x16_t{};
  uint64_t ring[S];
#pragma unroll
  for (int k = 0; k < S; ++k) ring[k] = 0ull;
#pragma unroll
  for (int k = 0; k < S - 1; ++k) {
    ring[k] = tile_bits(k);
    if (ring[k]) issue(k);
  }
  // copy-out chunks of this thread: chunk i is 16-byte column ch0 of row r0 + RSTEP*(i % (CPT/2)) of
  // dK (first half) or dV; RSTEP keeps the staging swizzle of r0
  constexpr int RSTEP = 64 * NW / CPR;
  static_assert(CPT == 1 || RSTEP % 16 == 0, "copy-out rows share one swizzle");
  const int fo = CPT == 1 ? tid % (TILE * CPR) : tid;   // chunk within its tensor
  const bool ov = CPT == 1 && tid >= TILE * CPR;        // CPT = 1: this thread's chunk is of dV
  const int r0 = fo / CPR, ch0 = fo % CPR;
  const int lds0 = r0 * ROWB + (ch0 ^ out_swz(r0)) * 16;
  const int off0 = r0 * D + 8 * ch0;
  const int swk = kv_swz<D>(swap23(l32));   // rows 32*b2 + swap23(l32)
  for (int t = 0; t < ntiles; ++t) {
    // Tile t's loads are complete once at most the later tiles' loads and the
    // stores of the (up to S-1) tiles since its issue are pending: every tile
    // issues exactly CPT stores per wave (buffer stores, whose range check drops
    // rows outside the chunk), and any loads of the accumulating variant only
    // make the count conservative.
    int later = 0;
#pragma unroll
    for (int k = 1; k < S - 1; ++k) later += ring[k] != 0ull;
    wait_vm_le<(S - 2) * OPS + (S - 1) * CPT>(later * OPS + (t < S - 1 ? t : S - 1) * CPT);
    barrier_lds();
    ring[S - 1] = tile_bits(t + S - 1);
    if (ring[S - 1]) issue(t + S - 1);
    const uint64_t bits = ring[0];
    const int t0 = t_begin + t * TILE;
    const int nrows = t_end - t0 < TILE ? t_end - t0 : TILE;
    const bool whole = nrows == TILE;
    const int64_t tb = (int64_t)t0 * D;
    // the tile's gradient rows (bytes past the chunk are dropped); an empty tile
    // leaves an accumulated gradient as it is (a zero-length range drops every store)
    const __amdgpu_buffer_rsrc_t kout =
        __builtin_amdgcn_make_buffer_rsrc(dKg + tb, 0, ((ACC & 1) && !bits) ? 0 : nrows * ROWB, 0x00020000);
    const __amdgpu_buffer_rsrc_t vout =
        __builtin_amdgcn_make_buffer_rsrc(dVg + tb, 0, ((ACC & 2) && !bits) ? 0 : nrows * ROWB, 0x00020000);
    if (!bits) {
      // no valid token: zero gradient rows, nothing loaded
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const bool isv = CPT == 1 ? ov : i >= CPT / 2;
        const int k = CPT == 1 ? 0 : i % (CPT / 2 > 0 ? CPT / 2 : 1);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0, 0, 0, 0}, isv ? vout : kout, 2 * (off0 + RSTEP * D * k), 0,
                                               kCachePolicyNT);
      }
    } else {
      uint8_t* kst = smem + (t % S) * STAGE;
      uint8_t* vst = kst + TB;
      if (DQ && bits != ~0ull) {
        // invalid K rows become zero: they meet dS = 0 in the query gradient
        for (int f = tid; f < TILE * CPR; f += 64 * NW) {
          const int r = f / CPR, pc = f % CPR;
          if (!((bits >> r) & 1ull)) st16(kst + r * ROWB + pc * 16, u32x4_t{0, 0, 0, 0});
        }
        barrier_lds();
      }
      // ---- phase A ----
      if (pa) {
        const uint64_t lb = bits >> (8 * hh);
        const bool full = bits == ~0ull;   // uniform: no per-element masking for whole tiles
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          f32x16_t sc = sinit, dp = dpinit;
          const uint8_t* krow = kst + (32 * b2 + swap23(l32)) * ROWB;
          const uint8_t* vrow = vst + (32 * b2 + swap23(l32)) * ROWB;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int ch = (2 * ks + hh) ^ swk;
            const bf16x8_t kop = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(krow + ch * 16));
            sc = mfma32x32x16(kop, qop[ks], sc);
            if constexpr (FOLD) sc = mfma32x32x16(kop, qlo[ks], sc);
            dp = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(vrow + ch * 16)),
                              gop[ks], dp);
          }
          // register r of lane half hh holds token 32*b2 + 16*(r/8) + 8*hh + r%8
          bf16x8_t pk[2];
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            float pv[8], ds[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int r = 8 * g + j;
              if constexpr (FOLD) {
                pv[j] = fast_exp2(sc[r]);
                ds[j] = pv[j] * dp[r];                           // dS, unscaled
              } else {
                pv[j] = fast_exp2(__builtin_fmaf(sc[r], c2, -nl2));
                ds[j] = pv[j] * __builtin_fmaf(dp[r], sc1, -cms);   // s dS: dK and dQ take it unscaled
              }
            }
            if (!full) {
              // padding and rows past the chunk: exact zeros (their K/V rows may hold anything)
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int tk = 32 * b2 + 16 * g + j;
                if (!((lb >> tk) & 1ull)) {
                  pv[j] = 0.f;
                  ds[j] = 0.f;
                }
              }
            }
            const u32x4_t wp = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                                pack_bf16x2(pv[6], pv[7])};
            const u32x4_t wd = {pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                                pack_bf16x2(ds[6], ds[7])};
            const int pc = (4 * b2 + 2 * g + hh) ^ pd_swz(m);
            st16(pbuf + m * (TILE * 2) + pc * 16, wp);
            st16(dsbuf + m * (TILE * 2) + pc * 16, wd);
            pk[g] = __builtin_bit_cast(bf16x8_t, wd);
          }
          if constexpr (DQ) {
            // dQ^T += K^T dS^T over this block's 32 tokens
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int d0 = 32 * db + (D >= 32 ? 16 * (lg & 1) : 0) + 4 * (li & 3);
              const int chl = d0 >> 3, half = (d0 & 7) * 2;
#pragma unroll
              for (int g = 0; g < 2; ++g) {
                u32x2_t part[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                  const int n = 32 * b2 + 16 * g + 8 * (lg >> 1) + 4 * q + (li >> 2);
                  const uint8_t* src = kst + n * ROWB + ((chl ^ kv_swz<D>(n)) * 16) + half;
                  part[q] = __builtin_bit_cast(u32x2_t,
                                               __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)src));
                }
                const u32x4_t av = {part[0][0], part[0][1], part[1][0], part[1][1]};
                dq[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), pk[g], dq[db]);
              }
            }
          }
        }
      }
      barrier_lds();
      // ACC bit 0: dK += this gradient, bit 1: dV += (another product already
      // wrote its share); the old rows are read here so the loads overlap phase
      // B.  Separate instantiations, so that the kernel without them has no
      // register-tracked load in its loop (before reusing such registers the
      // compiler waits for every outstanding load, the ring's included).
      constexpr int HALF = CPT == 1 ? 1 : CPT / 2;   // chunks per tensor of a thread (CPT = 1: of one tensor)
      constexpr int NPK = (ACC & 1) ? HALF : 0, NPV = (ACC & 2) ? HALF : 0;
      u32x4_t prev[NPK + NPV > 0 ? NPK + NPV : 1];
#pragma unroll
      for (int k = 0; k < NPK; ++k) {   // rows past the chunk read row 0 (in range, unused)
        if (CPT == 1 && ov) break;
        const int rk = r0 + RSTEP * k;
        prev[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(dKg + tb + (whole || rk < nrows ? rk : 0) * D + 8 * ch0));
      }
#pragma unroll
      for (int k = 0; k < NPV; ++k) {
        if (CPT == 1 && !ov) break;
        const int rk = r0 + RSTEP * k;
        prev[NPK + k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(dVg + tb + (whole || rk < nrows ? rk : 0) * D + 8 * ch0));
      }
      // ---- phase B: this wave's output blocks, staged into the tile's K/V slot ----
      {
        const uint8_t* bsrc = tsel == 0 ? pbuf : dsbuf;
        uint8_t* stg = tsel == 0 ? vst : kst;
        // B operand (P or s dS over 16 latents x 32 tokens) of output block nb, step ks
        auto bload = [&](int nb, int ks) {
          u32x2_t part[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int row = 16 * ks + 8 * (lg >> 1) + 4 * q + (li >> 2);
            const int col = 32 * nb + 16 * (lg & 1) + 4 * (li & 3);
            const int pc = (col >> 3) ^ pd_swz(row);
            part[q] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                      (lds_bf16x4*)(bsrc + row * (TILE * 2) + pc * 16 + (col & 7) * 2)));
          }
          return __builtin_bit_cast(bf16x8_t, u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]});
        };
        // register r of lane half hh: d = 32*db + 16*(r/8) + 8*hh + r%8, token 32*nb + l32
        // FOLD: the key-gradient rows take s here (dS is unscaled)
        const float os = (FOLD && tsel == 1) ? sc1 : 1.f;
        auto stage_out = [&](int nb, const f32x16_t* acc) {
          const int n = 32 * nb + l32;
#pragma unroll
          for (int j = 0; j < NDW; ++j)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              const f32x16_t& v = acc[j];
              const u32x4_t w = {pack_bf16x2(v[8 * g + 0] * os, v[8 * g + 1] * os),
                                 pack_bf16x2(v[8 * g + 2] * os, v[8 * g + 3] * os),
                                 pack_bf16x2(v[8 * g + 4] * os, v[8 * g + 5] * os),
                                 pack_bf16x2(v[8 * g + 6] * os, v[8 * g + 7] * os)};
              const int ch = 4 * (db0 + j) + 2 * g + hh;
              if constexpr (DIRECT) {
                __builtin_amdgcn_raw_buffer_store_b128(w, tsel == 1 ? kout : vout, n * ROWB + ch * 16, 0,
                                                       kCachePolicyNT);
              } else {
                st16(stg + n * ROWB + (ch ^ out_swz(n)) * 16, w);
              }
            }
        };
        // all B operands of the wave in registers at once (M <= 128: 64 VGPRs at most)
        constexpr bool PRE = M <= 128 && NNB * KM * 4 <= 64;
        if constexpr (PRE) {
          // every read issued first, then NNB x NDW independent accumulation chains interleaved
          bf16x8_t bop[NNB][KM];
#pragma unroll
          for (int ks = 0; ks < KM; ++ks)
#pragma unroll
            for (int nbi = 0; nbi < NNB; ++nbi) bop[nbi][ks] = bload(nb0 + nbi, ks);
          f32x16_t acc[NNB][NDW];
#pragma unroll
          for (int nbi = 0; nbi < NNB; ++nbi)
#pragma unroll
            for (int j = 0; j < NDW; ++j) acc[nbi][j] = f32x16_t{};
#pragma unroll
          for (int ks = 0; ks < KM; ++ks)
#pragma unroll
            for (int nbi = 0; nbi < NNB; ++nbi)
#pragma unroll
              for (int j = 0; j < NDW; ++j) acc[nbi][j] = mfma32x32x16(ast[j][ks], bop[nbi][ks], acc[nbi][j]);
#pragma unroll
          for (int nbi = 0; nbi < NNB; ++nbi) stage_out(nb0 + nbi, acc[nbi]);
        } else {
#pragma unroll
          for (int nbi = 0; nbi < NNB; ++nbi) {
            f32x16_t acc[NDW];
#pragma unroll
            for (int j = 0; j < NDW; ++j) acc[j] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KM; ++ks) {
              const bf16x8_t bop = bload(nb0 + nbi, ks);
#pragma unroll
              for (int j = 0; j < NDW; ++j) acc[j] = mfma32x32x16(ast[j][ks], bop, acc[j]);
            }
            stage_out(nb0 + nbi, acc);
          }
        }
      }
      // ---- whole rows out: dK from the K slot, dV from the V slot; each thread
      // owns CPT fixed 16-byte chunks (the first half in dK) ----
      if constexpr (!DIRECT) {
        barrier_lds();
        // consume the old rows on every path here, so that the compiler's wait for
        // them sits in this block and no load is left pending into the next tile
#pragma unroll
        for (int k = 0; k < NPK + NPV; ++k) asm volatile("" ::"v"(prev[k]));
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          // read and add on every row (the staging holds all 64), store only rows in the chunk
          const bool isv = CPT == 1 ? ov : i >= CPT / 2;
          const int k = CPT == 1 ? 0 : i % (CPT / 2 > 0 ? CPT / 2 : 1);
          u32x4_t v = ld16((isv ? vst : kst) + lds0 + RSTEP * ROWB * k);
          if (((ACC & 1) && !isv) || ((ACC & 2) && isv)) {
            const u32x4_t& pv = prev[isv ? NPK + k : k];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = pack_bf16x2(bf16lo(v[e]) + bf16lo(pv[e]), bf16hi(v[e]) + bf16hi(pv[e]));
          }
          __builtin_amdgcn_raw_buffer_store_b128(v, isv ? vout : kout, 2 * (off0 + RSTEP * D * k), 0, kCachePolicyNT);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < S - 1; ++k) ring[k] = ring[k + 1];
  }
  if constexpr (DQ) {
    if (pa) {
      float* W = a.ws_dq + (((int64_t)a.tab.slot[c] * a.B + b) * a.H + h) * (int64_t)M * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 2 * NG; ++q) {
          f32x4_t v = {dq[db][4 * q], dq[db][4 * q + 1], dq[db][4 * q + 2], dq[db][4 * q + 3]};
          *reinterpret_cast<f32x4_t*>(W + (int64_t)m * D + 32 * db + 8 * q + 4 * hh) = v;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Key/value gradients at 256 latent rows and head dim 128, with wave roles
// (FLARE++ appendix, backward pass: P with the global L, the row term c, the
// local dK_r and dV_r).  In the kernel above every wave holds both the score-
// side operands (the Q and dZ rows of its 32 latents) and the gradient-side
// ones (a 32-dim slice of Q^T or dZ^T over all latents); at this shape that
// fills 256 registers, two waves per SIMD, which then run phases A and B in
// lock-step.  Here 16 waves split the roles and work on consecutive tiles:
//   waves 0..7 (A, lane = latent row 32w + l32), round u, tile u:
//     S^T = K Q^T, dP^T = V dZ^T, P = exp(s S - L), s dS = P (s dP - s c),
//     P and s dS as bf16 [latent][token] into buffer u % 2
//   waves 8..15 (B: tensor t = (w-8)/4, 0 = dV, 1 = dK; head-dim block (w-8)%4;
//   lane = token), round u:
//     rows 8*block .. 8*block+7 of tensor t of tile u-2, staged last round,
//     leave as whole rows; then dV^T = dZ^T P or dK^T = Q^T (s dS) of tile u-1
//     from buffer (u-1) % 2, staged in tile u-1's own K/V slot.
// Each role runs at most 128 registers, so four waves share a SIMD and the
// products of one role overlap the other's exponentials and LDS waits.
// 32-token tiles through a 5-slot direct-load ring (tile u+2 is loaded in
// round u); one barrier per round.  The tiles after a chunk's last valid
// token only write zero rows (or, accumulating, leave the rows as they are):
// up to two such tiles per round alongside the rounds (the rounds leave HBM
// bandwidth to spare), the rest after them.
// ---------------------------------------------------------------------------
// 16-byte chunk swizzle of the P / dS rows here (64 bytes: 32 tokens of one
// latent): phase A's 16-byte writes (8 lanes per cycle, rows r..r+7, one chunk)
// and phase B's transposing reads (4 rows x 4 chunks per 32 lanes) both cover
// all 16 bank groups once.
__device__ __forceinline__ int pd32_swz(int r) { return (r >> 2) & 1; }

template <int ACC, int S>
__global__ __launch_bounds__(1024) void bwd_kv_ws_kernel(const BwdArgs a) {
  constexpr int D = 128, M = 256, TILE = 32, NW = 16;
  constexpr int ROWB = 2 * D;              // bytes of one K/V/gradient row
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int TB = TILE * ROWB;          // a K (or V) tile: 8 KB
  constexpr int STAGE = 2 * TB;
  // ring of S slots: tile u (A reads it), u-1 (B stages into it), u-2 (B copies it
  // out) and the L = S-3 tiles in flight (tile u+L is loaded in round u)
  constexpr int L = S - 3;
  static_assert(L >= 1 && L <= 3, "ring depth");
  constexpr int RING = S * STAGE;
  constexpr int PDROW = 2 * TILE;          // one latent's bf16 weights of a tile
  constexpr int PD = M * PDROW;            // P (or dS) of a tile: 16 KB
  constexpr int LDS_MAIN = RING + 4 * PD;  // + two buffers of P and dS
  constexpr int LDS_STAT = 2 * M * D * 2;  // Q and dZ rows while the operands load: 128 KB
  constexpr int LDS = LDS_MAIN > LDS_STAT ? LDS_MAIN : LDS_STAT;
  constexpr int KS = D / 16;               // contraction steps over the head dim
  constexpr int KM = M / 16;               // contraction steps over the latents
  static_assert(NW * 1024 == 2 * TB, "one 1 KB load per wave and tile");
  static_assert(LDS_MAIN <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  uint8_t* pdb = smem + RING;              // buffer j: P at pdb + 2*j*PD, s dS at + PD

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int lg = lane >> 4, li = lane & 15;
  const int nch = a.tab.nchunks;
  int bid = ordered_block(a.order);
  const int c = bid % nch;
  bid /= nch;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + bh * (int64_t)a.N * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + bh * (int64_t)a.N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
  const uint16_t* Gg = static_cast<const uint16_t*>(a.dZ) + bh * (int64_t)M * D;
  uint16_t* dKg = static_cast<uint16_t*>(a.dK) + bh * (int64_t)a.N * D;
  uint16_t* dVg = static_cast<uint16_t*>(a.dV) + bh * (int64_t)a.N * D;
  const_u64* mw = a.mask_words ? (const_u64*)(a.mask_words + (int64_t)b * a.mask_words_stride) : nullptr;

  // ---- stationary operands: Q and dZ rows through LDS ([m][d], row-major) ----
  for (int f = tid; f < M * CPR; f += 64 * NW) {
    const int r = f / CPR, ch = f % CPR;
    const u32x4_t q = ld16(Qg + (int64_t)r * D + 8 * ch);
    const u32x4_t g = ld16(Gg + (int64_t)r * D + 8 * ch);
    st16(smem + r * ROWB + ch * 16, q);
    st16(smem + M * ROWB + r * ROWB + ch * 16, g);
  }
  __syncthreads();

  const int ntiles = (t_end - t_begin + TILE - 1) / TILE;
  // tiles up to the chunk's last valid token; the rest only get zero rows
  int nv = ntiles;
  if (mw) {
    const int w0 = t_begin >> 6, nwd = t_end > t_begin ? ((t_end - 1) >> 6) - w0 + 1 : 0;
    int last = -1;
    for (int k = lane; k < nwd; k += 64) {
      const int wi = w0 + k;
      uint64_t x = a.mask_words[(int64_t)b * a.mask_words_stride + wi];
      const int a0 = t_begin - 64 * wi, a1 = t_end - 64 * wi;   // keep bits [a0, a1)
      if (a0 > 0) x &= ~0ull << a0;
      if (a1 < 64) x &= (1ull << a1) - 1ull;
      if (x) last = 64 * wi + 63 - __clzll(x);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    last = __builtin_amdgcn_readfirstlane(last);
    nv = last < t_begin ? 0 : (last - t_begin) / TILE + 1;
  }
  // validity bits of tile t (0 for tiles outside [0, nv))
  auto tile_bits = [&](int t) -> uint32_t {
    if (t < 0 || t >= nv) return 0u;
    const int t0 = t_begin + t * TILE;
    const int n = t_end - t0;
    uint32_t bits = n >= TILE ? 0xffffffffu : ((1u << n) - 1u);
    if (mw) bits &= (uint32_t)mask_tile_bits(mw, t0);
    return bits;
  };
  // this wave's 1 KB piece of tile t: waves 0..7 the K tile, 8..15 the V tile
  auto issue = [&](int t) {
    const int t0 = t_begin + t * TILE;
    const int nrows = t_end - t0;
    const uint32_t dst = lds_addr(smem) + (t % S) * STAGE + wave * 1024;   // (V pieces follow the K tile)
    const int ii = wave & 7;
    const int byte = ii * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    const int ch = pc ^ kv_swz<D>(r);
    const int rr = r < nrows ? r : 0;
    dma16((wave < 8 ? Kg : Vg) + (int64_t)(t0 + rr) * D + 8 * ch, dst);
  };
  const int nrounds = nv > 0 ? nv + 2 : 0;
  // zero rows of the tiles after the last valid token, stored by the B waves (one
  // 16-byte chunk of dK and one of dV per thread and tile; none for a tensor that
  // accumulates): tiles nv+2r and nv+2r+1 in round r, the rest after the rounds
  constexpr int ZPR = 2;
  constexpr int NZT = ((ACC & 1) ? 0 : 1) + ((ACC & 2) ? 0 : 1);   // zero-row tensors
  const int zoff = ((tid >> 4) & 31) * ROWB + (tid & 15) * 16;
  auto zero_tile = [&](int t) {
    const int t0 = t_begin + t * TILE;
    const int len = min(TILE, t_end - t0) * ROWB;
    if constexpr (!(ACC & 1))
      __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0, 0, 0, 0},
                                             __builtin_amdgcn_make_buffer_rsrc(dKg + (int64_t)t0 * D, 0, len, 0x00020000),
                                             zoff, 0, kCachePolicyNT);
    if constexpr (!(ACC & 2))
      __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0, 0, 0, 0},
                                             __builtin_amdgcn_make_buffer_rsrc(dVg + (int64_t)t0 * D, 0, len, 0x00020000),
                                             zoff, 0, kCachePolicyNT);
  };
  // zero tiles of round r, and the stores they take per B thread
  auto ztiles = [&](int r) -> int {
    if (r < 0 || r >= nrounds) return 0;
    const int left = ntiles - (nv + ZPR * r);
    return left <= 0 ? 0 : (left < ZPR ? left : ZPR);
  };

  if (wave < 8) {
    // ================= role A: scores, weights and s dS of latent rows 32w .. 32w+31
    const int m = 32 * wave + l32;
    bf16x8_t qop[KS], gop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qop[ks] = __builtin_bit_cast(bf16x8_t, ld16(smem + m * ROWB + (16 * ks + 8 * hh) * 2));
      gop[ks] = __builtin_bit_cast(bf16x8_t, ld16(smem + M * ROWB + m * ROWB + (16 * ks + 8 * hh) * 2));
    }
    const float Lm = a.L[bh * M + m];
    const float cms = a.scale * a.c[bh * M + m];
    const float c2 = a.scale_log2, sc1 = a.scale;
    const float nl2 = (Lm == kNegInf) ? __builtin_huge_valf() : Lm * kLog2e;
    const int swk = kv_swz<D>(swap23(l32));   // K/V row swap23(l32) of the tile
    const int pm = m * PDROW;
    const int psw = pd32_swz(m);
    wait_vm<0>();
    barrier_lds();   // every wave has its operands: the ring may reuse the staging rows
    uint32_t rb[L + 3];  // rb[k]: bits of tile u-2+k
    rb[0] = rb[1] = 0u;
#pragma unroll
    for (int k = 0; k <= L; ++k) rb[2 + k] = tile_bits(k);
#pragma unroll
    for (int k = 0; k < L; ++k)
      if (rb[2 + k]) issue(k);
    for (int u = 0; u < nrounds; ++u) {
      // tile u's piece landed: later are the pieces of tiles u+1 .. u+L-1
      int later = 0;
#pragma unroll
      for (int k = 1; k < L; ++k) later += rb[2 + k] ? 1 : 0;
      wait_vm_le<L - 1>(later);
      barrier_lds();
      if (rb[2 + L]) issue(u + L);
      const uint32_t bits = rb[2];
      if (bits) {
        const uint8_t* kst = smem + (u % S) * STAGE;
        const uint8_t* krow = kst + swap23(l32) * ROWB;
        const uint8_t* vrow = krow + TB;
        f32x16_t sc = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = (2 * ks + hh) ^ swk;
          sc = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(krow + ch * 16)),
                            qop[ks], sc);
          dp = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(vrow + ch * 16)),
                            gop[ks], dp);
        }
        // register r of lane half hh holds token 16*(r/8) + 8*hh + r%8
        const uint32_t lb = bits >> (8 * hh);
        const bool full = bits == 0xffffffffu;
        uint8_t* pbuf = pdb + 2 * (u & 1) * PD;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float pv[8], ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 8 * g + j;
            pv[j] = fast_exp2(__builtin_fmaf(sc[r], c2, -nl2));
            ds[j] = pv[j] * __builtin_fmaf(dp[r], sc1, -cms);   // s dS
          }
          if (!full) {
            // padding and rows past the chunk: exact zeros (their K/V rows may hold anything)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              if (!((lb >> (16 * g + j)) & 1u)) {
                pv[j] = 0.f;
                ds[j] = 0.f;
              }
            }
          }
          const u32x4_t wp = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                              pack_bf16x2(pv[6], pv[7])};
          const u32x4_t wd = {pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                              pack_bf16x2(ds[6], ds[7])};
          const int pc = ((2 * g + hh) ^ psw) * 16;
          st16(pbuf + pm + pc, wp);
          st16(pbuf + PD + pm + pc, wd);
        }
      }
#pragma unroll
      for (int k = 0; k < L + 2; ++k) rb[k] = rb[k + 1];
      rb[L + 2] = tile_bits(u + L + 1);
    }
  } else {
    // ================= role B: gradient tensor tsel (0 = dV, 1 = dK), head dims 32*db .. 32*db+31
    const int wb = wave - 8;
    const int tsel = wb >> 2, db = wb & 3;
    // A operand rows permuted so that each register group holds 8 consecutive d:
    // lane i of a 16-lane group reads column swap_bits2(i%4) of the 4x16 block
    bf16x8_t ast[KM];
    {
      const uint8_t* src = smem + (tsel == 0 ? M * ROWB : 0);
#pragma unroll
      for (int ks = 0; ks < KM; ++ks) {
        u32x2_t part[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int row = 16 * ks + 8 * (lg >> 1) + 4 * q + (li >> 2);
          const int col = 32 * db + 16 * (lg & 1) + 4 * swap_bits2(li & 3);
          part[q] = __builtin_bit_cast(
              u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(src + row * ROWB + col * 2)));
        }
        ast[ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]});
      }
    }
    wait_vm<0>();
    barrier_lds();
    uint16_t* const outg = tsel == 1 ? dKg : dVg;
    constexpr int ACCT0 = ACC & 2, ACCT1 = ACC & 1;   // accumulate into dV / dK
    const bool acc_t = tsel == 1 ? ACCT1 != 0 : ACCT0 != 0;
    // copy-out rows of this wave: 8*db + 4*i + lane/16, 16-byte chunk lane%16
    const int crow = 8 * db + (lane >> 4), cch = lane & 15;
    uint32_t rb[L + 3];
    rb[0] = rb[1] = 0u;
#pragma unroll
    for (int k = 0; k <= L; ++k) rb[2 + k] = tile_bits(k);
#pragma unroll
    for (int k = 0; k < L; ++k)
      if (rb[2 + k]) issue(k);
    for (int u = 0; u < nrounds; ++u) {
      // this wave's piece of tile u (loaded in round u-L) landed: later are the
      // pieces of tiles u+1 .. u+L-1 and the zero-row and copy-out stores of rounds
      // u-L .. u-1 (two copy-out stores per round with a tile to copy)
      int later = 0;
#pragma unroll
      for (int k = 1; k < L; ++k) later += rb[2 + k] ? 1 : 0;
#pragma unroll
      for (int r = u - L; r < u; ++r) later += NZT * ztiles(r) + (r >= 2 && r - 2 < nv ? 2 : 0);
      wait_vm_le<(L - 1) + L * (2 * ZPR + 2)>(later);
      barrier_lds();
      // old rows of tile u-2 (accumulating forms), read before this round's load is issued
      constexpr int NPREV = ACC ? 2 : 1;
      u32x4_t prev[NPREV];
      const int tc = u - 2;   // tile copied out this round
      const bool copy = tc >= 0 && tc < nv;
      const int tc0 = t_begin + tc * TILE;
      const int ncr = copy ? min(TILE, t_end - tc0) : 0;
      if constexpr (ACC != 0) {
        if (copy && acc_t && rb[0]) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int r = crow + 4 * i;
            prev[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4_t*>(outg + (int64_t)(tc0 + (r < ncr ? r : 0)) * D + 8 * cch));
          }
        }
      }
      if (rb[2 + L]) issue(u + L);
      {
        const int k = ztiles(u);
        for (int i = 0; i < k; ++i) zero_tile(nv + ZPR * u + i);
      }
      if (copy) {
        // an empty tile leaves an accumulated gradient as it is (a zero-length range drops every store)
        const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
            outg + (int64_t)tc0 * D, 0, (acc_t && !rb[0]) ? 0 : ncr * ROWB, 0x00020000);
        const uint8_t* stg = smem + (tc % S) * STAGE + (tsel == 1 ? 0 : TB);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = crow + 4 * i;
          u32x4_t v = ld16(stg + r * ROWB + ((cch ^ (r & 15)) * 16));
          if constexpr (ACC != 0) {
            if (acc_t && rb[0]) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                v[e] = pack_bf16x2(bf16lo(v[e]) + bf16lo(prev[i][e]), bf16hi(v[e]) + bf16hi(prev[i][e]));
            }
          }
          __builtin_amdgcn_raw_buffer_store_b128(v, out, r * ROWB + cch * 16, 0, kCachePolicyNT);
        }
      }
      // gradient rows of tile u-1 into its own K (dK) or V (dV) slot
      const int tg = u - 1;
      if (tg >= 0 && tg < nv) {
        uint8_t* stg = smem + (tg % S) * STAGE + (tsel == 1 ? 0 : TB);
        const int n = l32;
        if (rb[1]) {
          const uint8_t* bsrc = pdb + 2 * (tg & 1) * PD + (tsel == 1 ? PD : 0);
          f32x16_t acc = f32x16_t{};
#pragma unroll
          for (int ks = 0; ks < KM; ++ks) {
            u32x2_t part[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int row = 16 * ks + 8 * (lg >> 1) + 4 * q + (li >> 2);
              const int col = 16 * (lg & 1) + 4 * (li & 3);
              const int pc = (col >> 3) ^ pd32_swz(row);
              part[q] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                        (lds_bf16x4*)(bsrc + row * PDROW + pc * 16 + (col & 7) * 2)));
            }
            const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, u32x4_t{part[0][0], part[0][1], part[1][0], part[1][1]});
            acc = mfma32x32x16(ast[ks], bop, acc);
          }
          // register r of lane half hh: d = 32*db + 16*(r/8) + 8*hh + r%8, token l32
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const u32x4_t w = {pack_bf16x2(acc[8 * g + 0], acc[8 * g + 1]), pack_bf16x2(acc[8 * g + 2], acc[8 * g + 3]),
                               pack_bf16x2(acc[8 * g + 4], acc[8 * g + 5]), pack_bf16x2(acc[8 * g + 6], acc[8 * g + 7])};
            const int ch = 4 * db + 2 * g + hh;
            st16(stg + n * ROWB + (ch ^ (n & 15)) * 16, w);
          }
        } else {
          // no valid token: zero gradient rows
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int ch = 4 * db + 2 * g + hh;
            st16(stg + n * ROWB + (ch ^ (n & 15)) * 16, u32x4_t{0, 0, 0, 0});
          }
        }
      }
#pragma unroll
      for (int k = 0; k < L + 2; ++k) rb[k] = rb[k + 1];
      rb[L + 2] = tile_bits(u + L + 1);
    }
  }
  // ---- zero tiles the rounds left (B waves)
  if (wave >= 8)
    for (int t = nv + ZPR * nrounds; t < ntiles; ++t) zero_tile(t);
}

// dQ = s * sum over chunk slots (fixed order) [+ dQ], one thread per 4
// elements; optionally also written rounded to bf16.
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(const float* __restrict__ ws, int nslots, int64_t n4,
                                                           float scale, float* __restrict__ dQ, int accumulate,
                                                           uint16_t* __restrict__ dQ_bf16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < nslots; ++k) s += reinterpret_cast<const f32x4_t*>(ws)[(int64_t)k * n4 + i];
  f32x4_t r = s * scale;
  if (accumulate) r += reinterpret_cast<const f32x4_t*>(dQ)[i];
  reinterpret_cast<f32x4_t*>(dQ)[i] = r;
  if (dQ_bf16) {
    const u32x2_t w = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    reinterpret_cast<u32x2_t*>(dQ_bf16)[i] = w;
  }
}

bool bwd_mfma_supported(int M, int D) {
  if (D == 16) return M == 32 || M == 64 || M == 128;
  return (D == 64 || D == 128) && (M == 32 || M == 64 || M == 128 || M == 256);
}

template <int D, int NW, int S>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * a.H * a.B;
  hipLaunchKernelGGL((bwd_dq_mfma_kernel<D, NW, S>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// Only the shape whose key/value kernel cannot also hold the query-gradient
// accumulators (bwd_kv_fuses_dq) runs this kernel.
hipError_t launch_bwd_dq_mfma(const BwdArgs& a, hipStream_t s) {
  if (a.D == 128 && a.M == 256) return launch_dq_t<128, 8, 3>(a, s);
  return hipErrorInvalidValue;
}

template <int D, int M, int NW, int S, bool DQ>
static hipError_t launch_kv_t(const BwdArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * a.H * a.B;
  switch ((a.accumulate_dk ? 1 : 0) | (a.accumulate_dv ? 2 : 0)) {
    case 0: hipLaunchKernelGGL((bwd_kv_mfma_kernel<D, M, NW, S, DQ, 0>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a); break;
    case 1: hipLaunchKernelGGL((bwd_kv_mfma_kernel<D, M, NW, S, DQ, 1>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a); break;
    case 2: hipLaunchKernelGGL((bwd_kv_mfma_kernel<D, M, NW, S, DQ, 2>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_kv_mfma_kernel<D, M, NW, S, DQ, 3>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a); break;
  }
  return hipGetLastError();
}

// 256 latent rows at head dim 128: the wave-role kernel (query gradient separate)
constexpr int kWsSlots = 4;
static hipError_t launch_kv_ws(const BwdArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * a.H * a.B;
  switch ((a.accumulate_dk ? 1 : 0) | (a.accumulate_dv ? 2 : 0)) {
    case 0: hipLaunchKernelGGL((bwd_kv_ws_kernel<0, kWsSlots>), dim3((unsigned)grid), dim3(1024), 0, s, a); break;
    case 1: hipLaunchKernelGGL((bwd_kv_ws_kernel<1, kWsSlots>), dim3((unsigned)grid), dim3(1024), 0, s, a); break;
    case 2: hipLaunchKernelGGL((bwd_kv_ws_kernel<2, kWsSlots>), dim3((unsigned)grid), dim3(1024), 0, s, a); break;
    default: hipLaunchKernelGGL((bwd_kv_ws_kernel<3, kWsSlots>), dim3((unsigned)grid), dim3(1024), 0, s, a); break;
  }
  return hipGetLastError();
}

bool bwd_kv_fuses_dq(int M, int D) { return !(M == 256 && D == 128); }

// whether the fused kernel's query-gradient partials already carry the scale s
// (head dim 16 forms dS unscaled)
bool bwd_kv_partials_scaled(int M, int D) { return bwd_kv_fuses_dq(M, D) && D != 16; }

// D=64 with M<=128: 4 waves of <=248 VGPRs and <=80 KB of LDS, so two per CU;
// the other shapes need more than half the LDS or all 256 VGPRs per lane
int bwd_kv_blocks_per_cu(int M, int D) { return (D == 64 || D == 16) && M <= 128 ? 2 : 1; }

// Every shape fuses the query gradient into the key/value kernel except
// M=256, D=128, which would not fit the registers (bwd_kv_fuses_dq).
hipError_t launch_bwd_kv_mfma(const BwdArgs& a, hipStream_t s) {
  if (a.D == 16) {
    switch (a.M) {
      case 32: return launch_kv_t<16, 32, 4, 3, true>(a, s);
      case 64: return launch_kv_t<16, 64, 4, 3, true>(a, s);
      case 128: return launch_kv_t<16, 128, 4, 3, true>(a, s);
    }
  } else if (a.D == 64) {
    switch (a.M) {
      case 32: return launch_kv_t<64, 32, 4, 3, true>(a, s);
      case 64: return launch_kv_t<64, 64, 4, 3, true>(a, s);
      case 128: return launch_kv_t<64, 128, 4, 3, true>(a, s);
      case 256: return launch_kv_t<64, 256, 8, 3, true>(a, s);
    }
  } else if (a.D == 128) {
    switch (a.M) {
      case 32: return launch_kv_t<128, 32, 4, 3, true>(a, s);
      case 64: return launch_kv_t<128, 64, 4, 3, true>(a, s);
      case 128: return launch_kv_t<128, 128, 4, 3, true>(a, s);
      case 256: return launch_kv_ws(a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_reduce(const float* ws, int nslots, int64_t elems, float scale, float* dQ, bool accumulate,
                                void* dQ_cast, hipStream_t s) {
  const int64_t n4 = elems / 4;
  if (n4 == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dq_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, ws, nslots, n4,
                     scale, dQ, (int)accumulate, static_cast<uint16_t*>(dQ_cast));
  return hipGetLastError();
}

hipError_t launch_bwd_rowdot(const void* dZ, bool bf16, const float* Z, int64_t rows, int D, float* c,
                             hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(bwd_rowdot_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<const uint16_t*>(dZ), Z, rows, D, c);
  else
    hipLaunchKernelGGL(bwd_rowdot_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(dZ), Z,
                       rows, D, c);
  return hipGetLastError();
}

hipError_t launch_bwd_kv_generic(const BwdArgs& a, bool bf16, hipStream_t s) {
  const int64_t toks = (int64_t)a.B * a.H * a.N;
  if (toks == 0) return hipSuccess;
  const unsigned g = (unsigned)((toks + 3) / 4);
  if (bf16) hipLaunchKernelGGL(bwd_kv_generic_kernel<uint16_t>, dim3(g), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(bwd_kv_generic_kernel<float>, dim3(g), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_generic(const BwdArgs& a, bool bf16, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  hipError_t e = launch_bwd_kv_generic(a, bf16, s);
  if (e != hipSuccess) return e;
  if (rows > 0) {
    const unsigned g = (unsigned)((rows + 3) / 4);
    if (bf16) hipLaunchKernelGGL(bwd_q_generic_kernel<uint16_t>, dim3(g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(bwd_q_generic_kernel<float>, dim3(g), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace flare
