// Local decode ("FLARE++: Low-rank attention with dynamic attention routing",
// appendix on context parallelism, FLARE and FLARE++ forward paragraphs):
// every token attends over the M replicated latents, Y[n] = softmax_m(s Xq[n].Klat[m]) Z,
// with no cross-partition work.  The softmax over m is exact (all M scores of a
// token are formed before any exponential).
#include <type_traits>
#include "common.h"
#include "kernels.h"

namespace flare {

// ---------------------------------------------------------------------------
// bf16 matrix-core decode.  A workgroup of NWV waves owns one (batch, head) and
// a run of tokens; each wave handles 32 tokens at a time:
//   T^T[m][n] = Klat Xq^T         (A = latent rows from LDS, B = token rows)
//   softmax over m                 (a token's M scores sit in one lane pair)
//   Y^T[d][n] = Z^T P^T            (A = Z^T in bf16 from LDS, B = P)
// so the normalisation by the row sum is lane-local.  Klat, Z and the token
// mask are staged in LDS once per workgroup.  Token rows travel HBM -> LDS by
// direct loads into a per-wave ring of S blocks: waves never wait for each
// other, and S-1 blocks of a wave are in flight while it computes one.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int row_swz(int D, int r) {
  // 16-byte chunk swizzle of token row r.  A 16-byte LDS read serves 16 lanes
  // (256 bytes over the 64 banks) per cycle, a 16-byte write only 8 lanes (128
  // bytes), and a lane here reads or writes one chunk of its own row, so the
  // chunk index must differ over any 8 consecutive rows that share their bank
  // window on a write and over any 16 on a read.  128-byte rows (D=64): chunk
  // c ^ (r mod 8) ^ bit 3 of r; 32-byte rows (D=16): the two chunks swap where
  // bits 2 and 3 of r differ; 256-byte rows (D=128): c ^ (r mod 16).
  return D == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : D == 16 ? (((r >> 2) ^ (r >> 3)) & 1) : (r & 15);
}

template <int NI, int ST, int S>
__device__ __forceinline__ void wait_block(int later_blocks, int later_stores) {
  // vector-memory ops issued after block j's loads: later_blocks more blocks of
  // NI loads and later_stores blocks of ST stores
  static_assert(NI * (S - 2 > 0 ? S - 2 : 0) + ST * (S - 1) < 64, "vmcnt range");
  if constexpr (S > 3) {
    // deeper rings (1 KB blocks): the general threshold wait
    wait_vm_le<NI * (S - 2) + ST * (S - 1)>(NI * later_blocks + ST * later_stores);
    return;
  }
#define FL_W(B, T)                                  \
  if (later_blocks == B && later_stores == T) {     \
    wait_vm<(NI * B + ST * T) < 64 ? (NI * B + ST * T) : 63>(); \
    return;                                         \
  }
  FL_W(0, 0) FL_W(0, 1) FL_W(0, 2) FL_W(1, 0) FL_W(1, 1) FL_W(1, 2)
#undef FL_W
  wait_vm<0>();
}

template <int D, int MB, int NWV, int S>
__global__ __launch_bounds__(64 * NWV) void decode_mfma_kernel(const DecodeArgs a) {
  constexpr int M = 32 * MB;
  constexpr int KS = D / 16;   // k-steps of the score product
  // 32-row blocks of Y^T; at head dim 16 one block whose rows 16..31 are
  // products of repeated head dims, never stored
  constexpr int DB = D >= 32 ? D / 32 : 1;
  constexpr int NG = D >= 32 ? 2 : 1;   // 8-dim register groups of a block that hold head dims
  constexpr int MS = M / 16;   // k-steps of the value product
  constexpr int KLD = D + 8;
  constexpr int ZLD = M + 8;
  constexpr int BLK = 32;                    // tokens per wave block
  constexpr int ROWB = 2 * D;
  constexpr int BB = BLK * ROWB;             // bytes per block
  constexpr int NI = BB / 1024;              // direct loads per block
  constexpr int ST = NI;                     // 1 KB row stores per block (as many as its loads)
  static_assert(D != 16 || DB * NG == ST, "head dim 16: Y leaves as one store per lane and block");
  constexpr int MAXT = 8192;                 // tokens per workgroup (host keeps tokens_per_block <= MAXT)
  // FOLD (head dim 16, where the score products are cheap): the latent keys
  // are staged as the bf16 pair hi + lo of s log2(e) Klat (16 significant
  // bits), so a weight against the zero reference is one exp2 of the product
  constexpr bool FOLD = D == 16;
  __shared__ __attribute__((aligned(16))) uint16_t Kl[M * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Klo[FOLD ? M * KLD : 8];
  // ONES (head dim 16): the value product's A operand has 32 rows, 16 of them
  // head dims; rows 16..31 hold ones, so that result rows 16..31 are the
  // tokens' row sums and no separate row-sum products run
  constexpr bool ONES = D == 16;
  constexpr int ZROWS = ONES ? 32 : D;
  __shared__ __attribute__((aligned(16))) uint16_t Zt[ZROWS * ZLD];
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NWV * S * BB];
  __shared__ uint8_t tmask[MAXT];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int nblk = (a.N + a.tokens_per_block - 1) / a.tokens_per_block;
  int bid = blockIdx.x;
  const int tb = bid % nblk;
  bid /= nblk;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int n_lo = tb * a.tokens_per_block;
  const int n_hi = min(a.N, n_lo + a.tokens_per_block);

  {  // stage latent keys (row-major), Z (transposed, rounded to bf16) and the token mask;
     // every load of a thread is issued before its first LDS store
    constexpr int T = 64 * NWV;
    constexpr int KI = (M * D / 8 + T - 1) / T;   // 16-byte pieces of Klat per thread
    constexpr int ZI = (M * D / 4 + T - 1) / T;   // float4 pieces of Z per thread
    const uint16_t* kg = static_cast<const uint16_t*>(a.Klat) + (int64_t)b * a.klat_bstride + (int64_t)h * M * D;
    const float* zg = a.Z + bh * (int64_t)M * D;
    u32x4_t kv[KI];
    f32x4_t zv[ZI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int f = tid + T * i;
      if (f < M * D / 8) kv[i] = ld16(kg + 8 * (int64_t)f);
    }
#pragma unroll
    for (int i = 0; i < ZI; ++i) {
      const int f = tid + T * i;
      if (f < M * D / 4) zv[i] = *reinterpret_cast<const f32x4_t*>(zg + 4 * (int64_t)f);
    }
    const uint8_t* tm = a.token_mask ? a.token_mask + (int64_t)b * a.N : nullptr;
    for (int i = tid; i < n_hi - n_lo; i += T) tmask[i] = tm ? tm[n_lo + i] : (uint8_t)1;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int f = tid + T * i;
      if (f < M * D / 8) {
        const int off = (f / (D / 8)) * KLD + 8 * (f % (D / 8));
        if constexpr (FOLD) {
          u32x4_t hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float f0 = bf16lo(kv[i][e]) * a.scale_log2, f1 = bf16hi(kv[i][e]) * a.scale_log2;
            hi[e] = pack_bf16x2(f0, f1);
            lo[e] = pack_bf16x2(f0 - bf16lo(hi[e]), f1 - bf16hi(hi[e]));
          }
          st16(&Kl[off], hi);
          st16(&Klo[off], lo);
        } else {
          st16(&Kl[off], kv[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < ZI; ++i) {
      const int f = tid + T * i;
      if (f < M * D / 4) {
        const int m = (4 * f) / D, d = (4 * f) % D;
#pragma unroll
        for (int e = 0; e < 4; ++e) Zt[(d + e) * ZLD + m] = to_bf16(zv[i][e]);
      }
    }
    if constexpr (ONES) {
      for (int i = tid; i < 16 * M; i += T) Zt[(16 + i / M) * ZLD + i % M] = 0x3f80;   // bf16 1.0
    }
  }
  __syncthreads();   // also completes the staging loads before the ring starts

  const uint16_t* Xg = static_cast<const uint16_t*>(a.Xq) + bh * (int64_t)a.N * D;
  uint16_t* Yg = static_cast<uint16_t*>(a.Y) + bh * (int64_t)a.N * D;
  const float c2 = a.scale_log2;
  uint8_t* myring = ring + wave * (S * BB);
  const uint32_t myring_lds = lds_addr(myring);

  // blocks of this wave: tokens n_lo + 32*(wave + NWV*j)
  const int span = n_hi - n_lo - BLK * wave;
  const int nb = span > 0 ? (span + BLK * NWV - 1) / (BLK * NWV) : 0;
  // this lane's 16-byte piece of each load: byte offset within a full block,
  // and within row 0 (rows past the run re-read row 0; results not stored)
  // (the row-0 offset is the low bits of the row's offset: ch * 16 < ROWB)
  uint32_t voff[NI];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int byte = ii * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    const int ch = pc ^ row_swz(D, r);
    voff[ii] = r * ROWB + ch * 16;
  }
  // (full: the block is known to lie inside the run)
  auto issue = [&](int j, int stage, bool full = false) {
    const int n0 = n_lo + BLK * (wave + NWV * j);
    const uint32_t st = myring_lds + stage * BB;
    const uint16_t* xb = Xg + (int64_t)n0 * D;
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      const int r = (ii * 1024) / ROWB + lane / (ROWB / 16);
      dma16_off(xb, (full || n0 + r < n_hi) ? voff[ii] : (voff[ii] & (ROWB - 1)), st + ii * 1024);
    }
  };
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < nb) issue(j, j);

  const int swx = row_swz(D, l32);
  // Latent operands in registers for the whole run (head dims 64 and 16 up to
  // 128 latents): the latent keys' score-product rows and Z^T's value-product
  // rows of this lane, read from LDS once instead of once per token block
  // (128 VGPRs at head dim 64; the exact form below keeps its row sums on the
  // vector ALUs so that the two waves of a SIMD still fit 256 registers).
  constexpr bool REGOP = (D == 64 || D == 16) && MB <= 4;
  u32x4_t kreg[REGOP ? MB * KS : 1], klreg[REGOP && FOLD ? MB * KS : 1], zreg[REGOP ? DB * MS : 1];
  if constexpr (REGOP) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ro = (32 * mb + swap23(l32)) * KLD + 8 * hh + 16 * ks;
        kreg[mb * KS + ks] = *reinterpret_cast<const u32x4_t*>(&Kl[ro]);
        if constexpr (FOLD) klreg[mb * KS + ks] = *reinterpret_cast<const u32x4_t*>(&Klo[ro]);
      }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ks = 0; ks < MS; ++ks) {
        const uint16_t* zrow = &Zt[(32 * db + swap23(l32)) * ZLD + 8 * hh];
        zreg[db * MS + ks] = *reinterpret_cast<const u32x4_t*>(zrow + 16 * ks);
      }
  }
  // Row sums on a 16x16x32 product: fed the weight operand of the 32x32x16
  // product as its B, lane l contributes token l%32, latents 8*(l/32)+0..7 of
  // the k-step as column l%16, contraction block l/16.  Selector rows 0 and 8
  // pick blocks 0 and 2 (tokens 0..15), rows 4 and 12 blocks 1 and 3 (tokens
  // 16..31), so register 0 of lane l (result row 4*(l/16), column l%16) sums
  // token l%32 in both lane halves.
  bf16x8_t sel;
  {
    const int si = lane & 15, kb = lane >> 4;
    const bool on = ((si == 0 || si == 8) && (kb & 1) == 0) || ((si == 4 || si == 12) && (kb & 1) == 1);
    const uint32_t w = on ? 0x3f803f80u : 0u;
    sel = __builtin_bit_cast(bf16x8_t, u32x4_t{w, w, w, w});
  }
  const bool has_mask = a.token_mask != nullptr;
  // Block j of this wave in ring stage st.  STEADY: j >= S-1 and block j+S-1
  // lies inside the run, so block j is full, its load is followed by S-2 full
  // loads and S-1 stores, and the block S-1 ahead is issued without a row check.
  auto block = [&](const int j, const int st, auto steady_t) {
    constexpr bool STEADY = decltype(steady_t)::value;
    if constexpr (STEADY) {
      wait_vm<NI * (S - 2) + ST * (S - 1)>();
      issue(j + S - 1, (st + S - 1) % S, true);
    } else {
      const int lb = min(S - 2, nb - 1 - j);          // blocks loaded after block j
      const int ls = min(j, S - 1);                   // blocks stored after block j was loaded
      wait_block<NI, ST, S>(lb > 0 ? lb : 0, ls);
      if (j + S - 1 < nb) issue(j + S - 1, (st + S - 1) % S);
    }
    const int n0 = n_lo + BLK * (wave + NWV * j);
    const int n = n0 + l32;
    const bool inb = STEADY || n < n_hi;
    const uint8_t* xs = myring + st * BB + l32 * ROWB;
    bf16x8_t xop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      xop[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xs + (((2 * ks + hh) ^ swx) * 16)));
    // Weights against a zero reference, streamed over the latent blocks: the
    // scores of block mb, their weights exp2(s log2(e) T), the row sums and the
    // value products that use them, so the products of one block overlap the
    // exponentials of the next.  A token whose row sum leaves [2^-64, 2^64]
    // (overflow, underflow, NaN) sends the wave through the exact form below,
    // which subtracts the token's maximum first.  Either way the weights are
    // the same softmax up to the bf16 rounding of p.
    auto scores_of = [&](int mb) -> f32x16_t {
      f32x16_t t = f32x16_t{};
      const int ro = (32 * mb + swap23(l32)) * KLD + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t khi, klo;
        if constexpr (REGOP) {
          khi = kreg[mb * KS + ks];
          klo = klreg[FOLD ? mb * KS + ks : 0];
        } else {
          khi = *reinterpret_cast<const u32x4_t*>(&Kl[ro + 16 * ks]);
          if constexpr (FOLD) klo = *reinterpret_cast<const u32x4_t*>(&Klo[ro + 16 * ks]);
        }
        t = mfma32x32x16(__builtin_bit_cast(bf16x8_t, khi), xop[ks], t);
        if constexpr (FOLD) t = mfma32x32x16(__builtin_bit_cast(bf16x8_t, klo), xop[ks], t);
      }
      return t;
    };
    // weights exp2(s log2(e) T + nm); FOLD: the scores are already s log2(e) T
    auto weigh = [&](const f32x16_t& t, float nm, bf16x8_t* pk2, bool shifted) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float p[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float x = t[8 * g + jj];
          p[jj] = fast_exp2(FOLD ? (shifted ? x + nm : x) : __builtin_fmaf(x, c2, nm));
        }
        const u32x4_t w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                           pack_bf16x2(p[6], p[7])};
        pk2[g] = __builtin_bit_cast(bf16x8_t, w);
      }
    };
    f32x16_t y[DB];
    f32x4_t ls4;
    auto accumulate = [&](int ks, const bf16x8_t& pk) {
      if constexpr (!ONES) ls4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pk, ls4, 0, 0, 0);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // Z^T rows permuted so that register group g of lane half hh holds the 8
        // consecutive head dims 32*db + 16*g + 8*hh .. +7
        u32x4_t zop;
        if constexpr (REGOP) {
          zop = zreg[db * MS + ks];
        } else {
          const uint16_t* zrow = &Zt[(32 * db + swap23(l32)) * ZLD + 8 * hh];
          zop = *reinterpret_cast<const u32x4_t*>(zrow + 16 * ks);
        }
        y[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, zop), pk, y[db]);
      }
    };
    auto clear = [&]() {
      ls4 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < DB; ++db) y[db] = f32x16_t{};
    };
    clear();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      bf16x8_t pk2[2];
      weigh(scores_of(mb), 0.f, pk2, false);
      accumulate(2 * mb, pk2[0]);
      accumulate(2 * mb + 1, pk2[1]);
      // 256 latents: keep the scheduler from forming every block's scores
      // ahead of the first weights (their registers would spill)
      if constexpr (MB >= 8) __builtin_amdgcn_sched_barrier(0);
    }
    // (ONES: result register 8 holds row 16 + 4 hh, a ones row)
    float lsum = ONES ? y[0][8] : ls4[0];
    if (__ballot(!(lsum >= 0x1p-64f && lsum <= 0x1p64f))) {
      // exact form: the token's maximum over its M scores first.  Its row sums
      // are added up on the vector ALUs from the lane's own rounded weights
      // (the selector form multiplies the neighbouring token's weights by 0,
      // and 0 x NaN from a padded row would leak across); lanes l and l+32
      // hold the two latent halves of token l%32.  The scores are formed twice
      // (for the maximum, then for the weights), so no block's scores are held
      // across the other blocks' products.
      float mx = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const f32x16_t t = scores_of(mb);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmax2(mx, t[r]);
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmax2(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float nmc = FOLD ? -mx : -mx * c2;
      clear();
      float half_sum = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        bf16x8_t pk2[2];
        weigh(scores_of(mb), nmc, pk2, true);
        accumulate(2 * mb, pk2[0]);
        accumulate(2 * mb + 1, pk2[1]);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const u32x4_t w = __builtin_bit_cast(u32x4_t, pk2[g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) half_sum += bf16lo(w[e]) + bf16hi(w[e]);
        }
      }
      {
        const auto sw =
            __builtin_amdgcn_permlane32_swap(__float_as_uint(half_sum), __float_as_uint(half_sum), false, false);
        lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
    }
    // Y block out.  Each lane holds 16-byte pieces of its own token's row.  At
    // head dim 16 a row is 32 bytes, so one 16-byte store per lane already
    // writes the block's 32 rows as one contiguous 1 KB and the pieces leave
    // straight from registers.  Longer rows go through the block's own
    // (consumed) ring stage first and leave as whole rows with 16-byte stores
    // (16-byte pieces spread over 128- or 256-byte rows measured 5-6% slower
    // on the step, and far slower with the non-temporal hint).  Buffer stores
    // drop the rows past the run, so every block issues the same ST stores (the
    // ring's wait counts rely on that).  Masked tokens are written as zeros;
    // only a wave that holds one selects.
    const bool keep = !has_mask || !inb || tmask[inb ? n - n_lo : 0] != 0;
    const float inv = __builtin_amdgcn_rcpf(lsum);
    const int valid_rows = STEADY ? BLK : min(BLK, n_hi - n0);
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(Yg + (int64_t)n0 * D, 0, valid_rows * ROWB, 0x00020000);
    uint8_t* stg = myring + st * BB;
    auto out_y = [&](auto masked) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          u32x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t v = pack_bf16x2(y[db][8 * g + 2 * e] * inv, y[db][8 * g + 2 * e + 1] * inv);
            w[e] = (decltype(masked)::value && !keep) ? 0u : v;
          }
          if constexpr (D == 16) {
            // (non-temporal: the output rows are not read again by this path)
            __builtin_amdgcn_raw_buffer_store_b128(w, yr, l32 * ROWB + hh * 16, 0, kCachePolicyNT);
          } else {
            const int pc = (4 * db + 2 * g + hh) ^ swx;
            st16(stg + l32 * ROWB + pc * 16, w);
          }
        }
    };
    if (__ballot(!keep))
      out_y(std::true_type{});
    else
      out_y(std::false_type{});
    if constexpr (D != 16) {
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) {
        const int byte = ii * 1024 + lane * 16;
        const int r = byte / ROWB, pc = (byte % ROWB) / 16;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + byte);
        __builtin_amdgcn_raw_buffer_store_b128(v, yr, r * ROWB + ((pc ^ row_swz(D, r)) * 16), 0, kCachePolicyNT);
      }
    }
  };
  // S blocks per trip, so that each block's ring stage is a compile-time
  // constant: the first trip (the ring fills), steady trips, then the rest
  const int nbf = span >= BLK ? (span - BLK) / (BLK * NWV) + 1 : 0;   // full blocks of this wave
#pragma unroll
  for (int st = 0; st < S; ++st)
    if (st < nb) block(st, st, std::false_type{});
  int j0 = S;
  for (; j0 + 2 * S - 1 <= nbf; j0 += S) {
#pragma unroll
    for (int st = 0; st < S; ++st) block(j0 + st, st, std::true_type{});
  }
  for (; j0 < nb; j0 += S) {
#pragma unroll
    for (int st = 0; st < S; ++st)
      if (j0 + st < nb) block(j0 + st, st, std::false_type{});
  }
}

bool decode_mfma_supported(int M, int D) {
  // register budget: the M scores and D outputs of 32 tokens per wave
  if (D == 64 || D == 16) return M == 32 || M == 64 || M == 128 || M == 256;
  if (D == 128) return M == 32 || M == 64 || M == 128;
  return false;
}

// waves per workgroup of the matrix-core decode (tokens_per_block is a multiple of 32 * this)
int decode_waves(int D) { return D == 128 ? 4 : 8; }

template <int D, int MB>
static hipError_t launch_dec_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int NWV = D == 128 ? 4 : 8;
  // LDS: ring + staged latents within 160 KB; 1 KB blocks at head dim 16 take a deeper ring
  constexpr int S = D == 16 ? 6 : (D == 64 && MB <= 4) ? 3 : 2;
  const int64_t nblk = (a.N + a.tokens_per_block - 1) / a.tokens_per_block;
  const int64_t grid = nblk * a.H * a.B;
  hipLaunchKernelGGL((decode_mfma_kernel<D, MB, NWV, S>), dim3((unsigned)grid), dim3(64 * NWV), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  if (a.tokens_per_block > 8192 || a.tokens_per_block % (32 * decode_waves(a.D)) != 0) return hipErrorInvalidValue;
  if (a.D == 64) {
    switch (a.M) {
      case 32: return launch_dec_t<64, 1>(a, s);
      case 64: return launch_dec_t<64, 2>(a, s);
      case 128: return launch_dec_t<64, 4>(a, s);
      case 256: return launch_dec_t<64, 8>(a, s);
    }
  } else if (a.D == 16) {
    switch (a.M) {
      case 32: return launch_dec_t<16, 1>(a, s);
      case 64: return launch_dec_t<16, 2>(a, s);
      case 128: return launch_dec_t<16, 4>(a, s);
      case 256: return launch_dec_t<16, 8>(a, s);
    }
  } else if (a.D == 128) {
    switch (a.M) {
      case 32: return launch_dec_t<128, 1>(a, s);
      case 64: return launch_dec_t<128, 2>(a, s);
      case 128: return launch_dec_t<128, 4>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// General vector decode (float32, or bf16 shapes without a matrix-core
// variant): one wave per token; lanes take latent rows for the scores and
// head dimensions for the output.  Float32 arithmetic throughout.
// ---------------------------------------------------------------------------
template <typename TIn>
__device__ __forceinline__ float ldx(const TIn* p);
template <>
__device__ __forceinline__ float ldx<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldx<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <typename TOut>
__device__ __forceinline__ void stx(TOut* p, float v);
template <>
__device__ __forceinline__ void stx<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void stx<uint16_t>(uint16_t* p, float v) { *p = to_bf16(v); }

template <typename TIn>
__global__ __launch_bounds__(256) void decode_generic_kernel(const DecodeArgs a) {
  constexpr int MAXL = 4;   // M <= 256 and D <= 256
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + wave;   // flattened (b, h, n)
  const int64_t total = (int64_t)a.B * a.H * a.N;
  if (tok >= total) return;
  const int n = (int)(tok % a.N);
  const int64_t bh = tok / a.N;
  const int h = (int)(bh % a.H);
  const int b = (int)(bh / a.H);
  const int D = a.D, M = a.M;
  const TIn* xr = static_cast<const TIn*>(a.Xq) + tok * D;
  const TIn* kl = static_cast<const TIn*>(a.Klat) + (int64_t)b * a.klat_bstride + (int64_t)h * M * D;
  const float* zg = a.Z + bh * (int64_t)M * D;
  TIn* yr = static_cast<TIn*>(a.Y) + tok * D;
  if (a.token_mask && a.token_mask[(int64_t)b * a.N + n] == 0) {
    for (int d = lane; d < D; d += 64) stx(yr + d, 0.f);
    return;
  }
  float sc[MAXL];
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    const int m = lane + 64 * j;
    sc[j] = kNegInf;
    if (m < M) {
      float d = 0.f;
      for (int i = 0; i < D; ++i) d = __builtin_fmaf(ldx(xr + i), ldx(kl + (int64_t)m * D + i), d);
      sc[j] = d;
      mx = fmaxf(mx, d);
    }
  }
  mx = wave_max(mx);
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    sc[j] = (lane + 64 * j < M) ? fast_exp2((sc[j] - mx) * a.scale_log2) : 0.f;
    ls += sc[j];
  }
  ls = wave_sum(ls);
  float acc[MAXL];
#pragma unroll
  for (int j = 0; j < MAXL; ++j) acc[j] = 0.f;
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    for (int i = 0; i < 64; ++i) {
      const int m = 64 * j + i;
      if (m >= M) break;
      const float pm = __shfl(sc[j], i, 64);
#pragma unroll
      for (int jj = 0; jj < MAXL; ++jj) {
        const int d = lane + 64 * jj;
        if (d < D) acc[jj] = __builtin_fmaf(pm, zg[(int64_t)m * D + d], acc[jj]);
      }
    }
  }
  const float inv = 1.f / ls;
#pragma unroll
  for (int jj = 0; jj < MAXL; ++jj) {
    const int d = lane + 64 * jj;
    if (d < D) stx(yr + d, acc[jj] * inv);
  }
}

hipError_t launch_decode_generic(const DecodeArgs& a, bool bf16, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.H * a.N;
  const int64_t grid = (total + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_generic_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace flare
