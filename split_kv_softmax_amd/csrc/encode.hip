// Encoder kernels: per-partition (O_r, L_r) states of softmax attention of M
// latent rows over the tokens of one chunk ("FLARE++: Low-rank attention with
// dynamic attention routing", appendix on context parallelism: the local-shard
// encoder between eq. 18 and eq. 23, which streams the shard's keys and values
// through an online softmax and returns both the normalised output and the
// log-normaliser; an attention row with no valid key returns (0, -inf)).
//
// The online softmax keeps, per row, the running maximum m of the raw dot
// products, the running sum l of exp(s (q.k - m)) and the unnormalised output
// acc; a new block of scores with maximum m' rescales l and acc by
// exp(s (m - m')) (the online-softmax merge of "Ring vs. Tree Attention").
// Exponentials are taken as exp2 of scores pre-multiplied by s log2(e); the
// returned log-normaliser is natural: L = s m + ln l.
#include <stdlib.h>

#include <type_traits>
#include "common.h"
#include "kernels.h"

namespace flare {

// Combine the G token groups' states of one chunk in LDS (the rings are idle
// by then) and store the chunk's normalised state: group g's lanes write their
// reference maximum, row sum and unnormalised accumulators; group 0 merges them
// in group order, normalises and writes O and L (to the output partition or to
// a workspace slot of a split partition).
template <int D, int NW, int G>
__device__ __forceinline__ void finish_chunk(uint8_t* smem, const EncodeArgs& a, int grp, int wave, int lane,
                                             f32x16_t (&o)[D >= 32 ? D / 32 : 1], float m_run, float l_tot, int b,
                                             int h, int c) {
  constexpr int DB = D >= 32 ? D / 32 : 1;
  constexpr int NQ = D >= 32 ? 4 : 2;   // 4-row groups of a block that hold head dims
  const int l32 = lane & 31, hh = lane >> 5;
  const float c2 = a.scale_log2;
  if constexpr (G > 1) {
    // ---- combine the G groups' states in LDS (the rings are idle now):
    // group g's lane writes its reference max, row sum and unnormalised
    // accumulators; group 0 merges them in group order.
    barrier_lds();
    float* cb = reinterpret_cast<float*>(smem);
    float* cm = cb + G * NW * 32 * 64;
    float* cl = cm + G * NW * 64;
    const int slot = grp * NW + wave;
    if (grp > 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) cb[(slot * 32 + 16 * db + r) * 64 + lane] = o[db][r];
      cm[slot * 64 + lane] = m_run;
      cl[slot * 64 + lane] = l_tot;
    }
    barrier_lds();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < G; ++g) {
      const int sg = g * NW + wave;
      const float mg = cm[sg * 64 + lane];
      const float lg2 = cl[sg * 64 + lane];
      const float mn = fmaxf(m_run, mg);
      if (mn == kNegInf) continue;                       // both empty
      const float fa = fast_exp2((m_run - mn) * c2);     // 0 for an empty side
      const float fb = fast_exp2((mg - mn) * c2);
      l_tot = l_tot * fa + lg2 * fb;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * fa + cb[(sg * 32 + 16 * db + r) * 64 + lane] * fb;
      m_run = mn;
    }
  }

  // ---- normalise and store this chunk's state
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const int slot = a.tab.slot[c];
  float* Ob;
  float* Lb;
  if (slot < 0) {
    const int r = -slot - 1;
    Ob = a.O_part + (((int64_t)r * a.B + b) * a.H + h) * (int64_t)a.M * D;
    Lb = a.L_part + (((int64_t)r * a.B + b) * a.H + h) * (int64_t)a.M;
  } else {
    Ob = a.ws_O + (((int64_t)slot * a.B + b) * a.H + h) * (int64_t)a.M * D;
    Lb = a.ws_L + (((int64_t)slot * a.B + b) * a.H + h) * (int64_t)a.M;
  }
  const int m = 32 * wave + l32;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      f32x4_t v = {o[db][4 * q] * inv, o[db][4 * q + 1] * inv, o[db][4 * q + 2] * inv, o[db][4 * q + 3] * inv};
      *reinterpret_cast<f32x4_t*>(Ob + (int64_t)m * D + 32 * db + 8 * q + 4 * hh) = v;
    }
  if (hh == 0) Lb[m] = empty ? kNegInf : (m_run * a.scale + __logf(l_tot));
}

// Fused merge (see FuseTable).  Publication: every wave waits until its own
// stores have reached the L2 of its XCD, the workgroup meets at a barrier, and
// one thread issues the device-scope release (a write-back of that L2, so the
// stores reach memory that every XCD reads) before it counts; the workgroup
// whose count completes a total issues the device-scope acquire (dropping
// stale cached lines) before it reads what the others stored.  One release
// per count and acquires only in the completing workgroups: a full fence in
// every thread would write back and invalidate the L2 under the workgroups
// still streaming.  Returns whether this workgroup completed the count.
// sflag: one int of LDS that no thread reads or writes any more.
__device__ __forceinline__ bool publish_and_count(uint32_t* cnt, uint32_t target, int* sflag) {
  wait_vm<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const bool last = atomicAdd(cnt, 1u) + 1u == target;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *sflag = last ? 1 : 0;
  }
  __syncthreads();
  const bool last = *sflag != 0;
  __syncthreads();   // every thread has read the flag before it can be reused
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// Merge tail of the workgroup that stored the state of chunk c of (b, h).  A
// chunk of a partition split over several chunks counts on that partition's
// counter; the workgroup that completes it folds the partition's chunk states
// into O_part / L_part (on its own CU, so the partitions of a slice fold in
// parallel) and then counts on the slice's counter, as a chunk that is a whole
// partition does at once.  The workgroup that completes the slice writes the
// empty state of the partitions without a token and merges the R partition
// states into Z / L.  Every fold takes the merge kernels' merges in their
// order, so the results equal those of the separate fold and merge launches
// bit for bit: fold_states itself up to 16 states (all loads of a piece in
// flight at once), fold_states_lean beyond (the same merges with fewer
// registers; at most 256 chunks and 256 partitions).
__device__ __forceinline__ void merge_tail(const EncodeArgs& a, int b, int h, int c, int* sflag) {
  if (a.fz.cnt == nullptr) return;
  const int64_t bh = (int64_t)b * a.H + h;
  const int D = a.D, D4 = D >> 2;
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  const int64_t sstride = rows * D;
  const int64_t p0 = bh * a.M * D4, p1 = p0 + (int64_t)a.M * D4;   // (row, 4-column piece) of (b, h)
  const int slot = a.tab.slot[c];
  if (slot >= 0) {
    // the partition r holding chunk c: the last r with pchunk[r] <= c
    int r = 0;
    for (int lo = 0, hi = a.R - 1; lo <= hi;) {
      const int mid = (lo + hi) >> 1;
      if (a.fz.pchunk[mid] <= c) { r = mid; lo = mid + 1; } else { hi = mid - 1; }
    }
    const int c0 = a.fz.pchunk[r], n = a.fz.pchunk[r + 1] - c0;
    uint32_t* pcnt = a.fz.cnt + (int64_t)a.B * a.H + bh * a.R + r;
    if (!publish_and_count(pcnt, (uint32_t)n, sflag)) return;
    const int s0 = a.tab.slot[c0];
    for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
      const int64_t row = p / D4, off = 4 * p;
      const MState st = n <= kFoldBatch ? fold_states(a.ws_O, a.ws_L, s0, n, rows, row, off, sstride)
                                        : fold_states_lean(a.ws_O, a.ws_L, s0, n, rows, row, off, sstride);
      store_state(st, a.O_part, a.L_part, nullptr, r, rows, row, off, sstride, D);
    }
    if (threadIdx.x == 0) *pcnt = 0;
  }
  if (!publish_and_count(a.fz.cnt + bh, (uint32_t)a.fz.target, sflag)) return;
  // partitions without a token: the empty state (0, -inf)
  for (int r = 0; r < a.R; ++r) {
    if (a.fz.pchunk[r + 1] != a.fz.pchunk[r]) continue;
    for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
      const int64_t row = p / D4, off = 4 * p;
      store_state(mstate_empty(), a.O_part, a.L_part, nullptr, r, rows, row, off, sstride, D);
    }
  }
  // ... read back below by other threads of this workgroup (same CU):
  // complete the stores, then meet
  wait_vm<0>();
  __syncthreads();
  // the R partition states -> Z, L
  for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int64_t row = p / D4, off = 4 * p;
    const MState st = a.R <= kFoldBatch ? fold_states(a.O_part, a.L_part, 0, a.R, rows, row, off, sstride)
                                        : fold_states_lean(a.O_part, a.L_part, 0, a.R, rows, row, off, sstride);
    store_state(st, a.fz.Z, a.fz.L, a.fz.Zb, 0, rows, row, off, sstride, D);
  }
  if (threadIdx.x == 0) a.fz.cnt[bh] = 0;
}

// ---------------------------------------------------------------------------
// bf16 matrix-core encoder.  One workgroup = one (batch, head, chunk) and all
// M = 32*NW latent rows, so each K/V byte is read from HBM exactly once.
// Wave w owns rows [32w, 32w+32).  Per 64-token tile:
//   S^T[n][m] = K_tile Q_w^T      (A = K rows from LDS, B = Q from registers)
//   online softmax over n          (the 32 scores of a row live in one lane
//                                   pair, so the row max needs one exchange)
//   O^T[d][m] += V_tile^T P^T      (A = V^T via transposing LDS reads, B = P)
// The result column of both products is the latent row, so the per-row
// rescale and normalisation are lane-local.
//
// K and V tiles travel HBM -> LDS by direct (VGPR-free) loads into a ring of S
// stages, so S-1 tiles are in flight while one is consumed; one barrier per
// tile.  Rows are stored unpadded with their 16-byte chunks XOR-swizzled by
// row so that the operand reads of a wave spread over the LDS banks.
// ---------------------------------------------------------------------------
template <int D, int NW, int S, int G>
__global__ __launch_bounds__(64 * NW * G) void encode_mfma_kernel(const EncodeArgs a) {
  constexpr int TILE = 64;
  constexpr int ROWB = 2 * D;              // bytes per row
  constexpr int TB = TILE * ROWB;          // bytes of a K (or V) tile
  constexpr int STAGE = 2 * TB;
  constexpr int NI = TB / 1024;            // 1 KB direct loads per tile and tensor
  constexpr int KS = D / 16;               // k-steps of the score product
  // 32-row blocks of O^T; at head dim 16 one block whose rows 16..31 are
  // products of repeated head dims, never stored
  constexpr int DB = D >= 32 ? D / 32 : 1;
  // a tile of fewer 1 KB loads than waves (head dim 16) is loaded by its first
  // NI waves; the others' waits pass at once
  constexpr int NJ = NI >= NW ? NI / NW : 1;
  constexpr int OPS = 2 * NJ;              // loads a loading wave issues per tile
  static_assert(D == 16 || D == 64 || D == 128, "head dim 16, 64 or 128");
  static_assert(NI >= 1 && (NI % NW == 0 || NI < NW), "loads must split evenly over the waves");
  static_assert(OPS * (S - 2) < 64, "vmcnt range");
  // G token groups of NW waves each: group g takes tiles g, g+G, g+2G, ...
  // of the chunk into its own LDS ring; their states are combined at the end.
  static_assert(G == 1 || (G * NW * 32 * 64 + 2 * G * NW * 64) * 4 <= G * S * STAGE,
                "the combine buffer reuses the rings");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[G * S * STAGE];

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv / NW, wave = wv % NW;                 // token group, row wave
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
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + (int64_t)b * a.q_bstride +
                       (int64_t)h * a.M * D;
  const_u64* mw = a.mask_words ? (const_u64*)(a.mask_words + (int64_t)b * a.mask_words_stride) : nullptr;

  // Q rows of this wave as the B operand: column j = latent row 32w + j.
  bf16x8_t qop[KS];
  {
    const uint16_t* qrow = Qg + (int64_t)(32 * wave + l32) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = __builtin_bit_cast(bf16x8_t, ld16(qrow + 16 * ks));
  }
  // Complete the Q loads now: afterwards the only vector-memory operations
  // in flight are the ring's, whose count the loop's waits rely on.
  wait_vm<0>();

  const int ntiles = (t_end - t_begin + TILE - 1) / TILE;
  const int nrounds = (ntiles + G - 1) / G;
  // validity bits of local tile u of group g (tile g + G*u of the chunk)
  auto tile_bits = [&](int g, int u) -> uint64_t {
    const int tt = g + G * u;
    if (tt >= ntiles) return 0ull;
    const int t0 = t_begin + tt * TILE;
    const int n = t_end - t0;
    uint64_t bits = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
    if (mw) bits &= mask_tile_bits(mw, t0);
    return bits;
  };
  uint8_t* myring = smem + grp * (S * STAGE);
  const uint32_t ring_lds = lds_addr(myring);
  // this lane's 16-byte piece of each of its loads: byte offset within a full
  // tile, and within row 0 (rows past the chunk re-read row 0: in bounds,
  // never used as valid)
  uint32_t voff[NJ], voff0[NJ];
  int vrow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int ii = wave + NW * j;
    const int byte = ii * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    const int ch = pc ^ kv_swz<D>(r);
    vrow[j] = r;
    voff[j] = r * ROWB + ch * 16;
    voff0[j] = ch * 16;
  }
  // K rows of local tile u go to K slot u % S, V rows to V slot u % S (the
  // second half of the stage).  Rows past the chunk re-read row 0.
  auto issue_half = [&](int u, int slot, bool is_v) {
    if (NI < NW && wave >= NI) return;   // (wave-uniform)
    const int t0 = t_begin + (grp + G * u) * TILE;
    const int nrows = t_end - t0;
    const uint16_t* base = (is_v ? Vg : Kg) + (int64_t)t0 * D;
    const uint32_t dst = ring_lds + slot * STAGE + (is_v ? TB : 0);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ii = wave + NW * j;
      dma16_off(base, vrow[j] < nrows ? voff[j] : voff0[j], dst + ii * 1024);
    }
  };

  f32x16_t o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16_t{};
  float m_run = kNegInf;   // reference maximum (raw dot products) of row 32w + l32
  // running row sum of the weights, on the matrix cores: ones x P^T puts the
  // row's sum of the bf16-rounded weights in every register of both lane halves
  f32x16_t lacc = f32x16_t{};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  const float c2 = a.scale_log2;

  // Round u needs K(u) and V(u) ("batch u"); scores, weights and values of a
  // tile in the same round.  vb[k] = validity bits of local tile u + k
  // (k = 0..S-1); nb[k] = number of this wave's loads in batch u + k (0 or 2 NJ).
  uint64_t vb[S];
#pragma unroll
  for (int k = 0; k < S; ++k) vb[k] = tile_bits(grp, k);
  int nb[S];
#pragma unroll
  for (int k = 0; k < S - 1; ++k) {
    nb[k] = 0;
    if (vb[k]) { issue_half(k, k % S, false); issue_half(k, k % S, true); nb[k] += 2 * NJ; }
  }
  nb[S - 1] = 0;
  // the scores of tile 0
  const int swk = kv_swz<D>(swap23(l32));             // rows 32*b2 + swap23(l32)
  // K operands are read in groups of KG k-steps for both 32-token blocks before
  // the products that use them, so the LDS latency is paid once per group
  constexpr int KG = D == 64 ? 4 : (D == 128 ? 2 : 1);
  auto scores = [&](const uint8_t* kst, f32x16_t* sc) {
    sc[0] = f32x16_t{};
    sc[1] = f32x16_t{};
    const uint8_t* krow0 = kst + swap23(l32) * ROWB;
#pragma unroll
    for (int k0 = 0; k0 < KS; k0 += KG) {
      u32x4_t kop[2][KG];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int k = 0; k < KG; ++k)
          kop[b2][k] = *reinterpret_cast<const u32x4_t*>(krow0 + 32 * b2 * ROWB + (((2 * (k0 + k) + hh) ^ swk) * 16));
#pragma unroll
      for (int k = 0; k < KG; ++k)
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
          sc[b2] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, kop[b2][k]), qop[k0 + k], sc[b2]);
      // scheduling: all reads of the group, then its products
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KG, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KG, 0);
    }
  };
  const int lg = lane >> 4, li = lane & 15;
  // S rounds per trip so that each round's ring slots are compile-time constants
  for (int u0 = 0; u0 < nrounds; u0 += S) {
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const int u = u0 + st;
      if (u < nrounds) {
        // batch u = {K(u), V(u)} complete for this wave; batches u+1 .. u+S-2 may be in flight
        int pend = 0;
#pragma unroll
        for (int k = 1; k < S - 1; ++k) pend += nb[k];
        wait_units<NJ, 2 * (S - 2)>(pend / NJ);
        barrier_lds();
        // every wave is past round u-1: stage (u-1) % S is free for batch u+S-1
        vb[S - 1] = tile_bits(grp, u + S - 1);
        nb[S - 1] = 0;
        if (vb[S - 1]) {
          issue_half(u + S - 1, (st + S - 1) % S, false);
          issue_half(u + S - 1, (st + S - 1) % S, true);
          nb[S - 1] += 2 * NJ;
        }
        const uint64_t bits = vb[0];
        bool partial = false;     // is any group's tile of this round partially valid?
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint64_t bg = g == grp ? bits : tile_bits(g, u);
          partial |= (bg != 0ull && bg != ~0ull);
        }
        uint8_t* vst = myring + st * STAGE + TB;
        if (partial) {
          // padding and rows past the chunk: zero their V rows so P = 0 never meets NaN
          if (bits != ~0ull && bits != 0ull) {
            for (int f = tid - grp * 64 * NW; f < TILE * (ROWB / 16); f += 64 * NW) {
              const int r = f / (ROWB / 16), pc = f % (ROWB / 16);
              if (!((bits >> r) & 1ull)) st16(vst + r * ROWB + pc * 16, u32x4_t{0, 0, 0, 0});
            }
          }
          barrier_lds();
        }
        f32x16_t sc[2];
        if (bits) {
          scores(myring + st * STAGE, sc);
          // register r of lane half hh in block b2 holds token 32*b2 + 16*(r/8) + 8*hh + r%8
          if (bits != ~0ull) {
            const uint64_t lb = bits >> (8 * hh);
#pragma unroll
            for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int tk = 32 * b2 + 16 * (r >> 3) + (r & 7);
                if (!((lb >> tk) & 1ull)) sc[b2][r] = kNegInf;
              }
          }
          // tile maximum: four independent chains of 3-input maxima, then one exchange
          float mc[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const f32x16_t& v = sc[k >> 1];
            const int r0 = 8 * (k & 1);
            float x = fmax3(v[r0], v[r0 + 1], v[r0 + 2]);
            x = fmax3(x, v[r0 + 3], v[r0 + 4]);
            x = fmax3(x, v[r0 + 5], v[r0 + 6]);
            mc[k] = fmax2(x, v[r0 + 7]);
          }
          float mx = fmax3(mc[0], mc[1], fmax2(mc[2], mc[3]));
          mx = fmax2(mx, __shfl_xor(mx, 32, 64));
          // Lazy reference: the subtracted maximum only moves when this tile's
          // maximum exceeds it by more than 2^kLazy in the exponent; the constant
          // cancels in O and L, and every weight stays below 2^kLazy.
          constexpr float kLazy = 8.f;
          const bool grow = m_run == kNegInf ? (mx != kNegInf) : ((mx - m_run) * c2 > kLazy);
          if (__ballot(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? fast_exp2((m_run - m_new) * c2) : 1.f;   // 0 when m_run = -inf
            lacc *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i) o[i] *= alpha;
            m_run = m_new;
          }
          const float nmc = -((m_run == kNegInf) ? 0.f : m_run) * c2;
          // weights, rounded to bf16 for the value product
          bf16x8_t pk[4];
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              float p[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) p[j] = fast_exp2(__builtin_fmaf(sc[b2][8 * g + j], c2, nmc));
              const u32x4_t w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                 pack_bf16x2(p[6], p[7])};
              pk[2 * b2 + g] = __builtin_bit_cast(bf16x8_t, w);
            }
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) lacc = mfma32x32x16(ones, pk[ks], lacc);
          // ---- O^T += V^T P^T ; k-step ks covers tokens 16ks .. 16ks+15.
          // Transposing reads: in each 16-lane group lane i points at token row
          // (i/4) of a 4-token block and 4 head dims starting at 4*(i%4); it gets
          // back the 4 tokens of head dim i of the group.
          // (the transposing reads of VK k-steps are issued before their products)
          constexpr int VK = D == 64 ? 2 : 1;
#pragma unroll
          for (int k0 = 0; k0 < 4; k0 += VK) {
            u32x2_t part[VK][DB][2];
#pragma unroll
            for (int kk = 0; kk < VK; ++kk)
#pragma unroll
              for (int db = 0; db < DB; ++db) {
                // head dim 16: the lanes of operand rows 16..31 read dims 0..15 again
                const int d0 = 32 * db + (D >= 32 ? 16 * (lg & 1) : 0) + 4 * (li & 3);
                const int chl = d0 >> 3, half = (d0 & 7) * 2;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                  const int n = 16 * (k0 + kk) + 8 * (lg >> 1) + 4 * q + (li >> 2);
                  const uint8_t* src = vst + n * ROWB + ((chl ^ kv_swz<D>(n)) * 16) + half;
                  part[kk][db][q] =
                      __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)src));
                }
              }
#pragma unroll
            for (int kk = 0; kk < VK; ++kk)
#pragma unroll
              for (int db = 0; db < DB; ++db) {
                const u32x4_t av = {part[kk][db][0][0], part[kk][db][0][1], part[kk][db][1][0], part[kk][db][1][1]};
                o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), pk[k0 + kk], o[db]);
              }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * VK * DB, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, VK * DB, 0);
          }
        }
#pragma unroll
        for (int k = 0; k < S - 1; ++k) vb[k] = vb[k + 1];
#pragma unroll
        for (int k = 0; k < S - 1; ++k) nb[k] = nb[k + 1];
      }
    }
  }

  const float l_tot = lacc[0];
  finish_chunk<D, NW, G>(smem, a, grp, wave, lane, o, m_run, l_tot, b, h, c);
  merge_tail(a, b, h, c, reinterpret_cast<int*>(smem));
}

// ---------------------------------------------------------------------------
// bf16 matrix-core encoder for inputs without a padding mask, pipelined by two
// tiles.  Same data flow as encode_mfma_kernel (one workgroup = one (batch,
// head, chunk) and all M rows; G token groups of NW waves, each with its own
// ring), but each wave's round u holds independent pieces of work:
//   * the weighted values of tile u          (matrix cores; weights from round u-1),
//   * the online softmax of tile u+1         (vector ALUs; scores from round u-1),
//     and the row sums of its weights        (matrix cores),
//   * the scores of tile u+2                 (matrix cores).
// Instruction-group barriers interleave the products of a round with its
// vector instructions, so the matrix cores work while the same wave issues
// its exponentials (a wave that issues a run of products back to back stalls
// on each one instead).
//
// The K ring runs two tiles ahead of the V ring: "batch" u carries K(u+2) and
// V(u) into K slot (u+2)%S and V slot u%S, and round u issues batch u+S-1 once
// the round's barrier shows every wave past round u-1 (the last reader of both
// slots).  Rows past the chunk re-read row 0 of the tile (finite values whose
// weights are exactly 0), so a partial tile only masks its scores.
//
// Padding masks (one token group): the chunk is cut at its last valid token;
// if every token before it is valid the chunk runs as unmasked, otherwise each
// round masks the scores of its tile's invalid tokens and zeroes their V rows
// in LDS (a padded row may hold NaN, which a weight of 0 must not meet).
// ---------------------------------------------------------------------------
template <int D, int NW, int S, int G, int TILE>
__global__ __launch_bounds__(64 * NW * G) void encode_ilv_kernel(const EncodeArgs a) {
  constexpr int NB = TILE / 32;            // 32-token blocks of the score product
  constexpr int NK = TILE / 16;            // 16-token k-steps of the value product
  static_assert(TILE == 32 || TILE == 64, "tile of 32 or 64 tokens");
  static_assert(D == 16 || D == 64 || D == 128, "head dim 16, 64 or 128");
  constexpr int ROWB = 2 * D;              // bytes per row
  constexpr int TB = TILE * ROWB;          // bytes of a K (or V) tile
  constexpr int RING = 2 * S * TB;         // S K slots, then S V slots
  constexpr int NI = TB / 1024;            // 1 KB direct loads per tile and tensor
  // ... issued by each wave; a tile of fewer loads than waves (head dim 16)
  // is loaded by its first NI waves, and the others' waits pass at once
  constexpr int NJ = NI >= NW ? NI / NW : 1;
  constexpr int KS = D / 16;               // k-steps of the score product
  // 32-row blocks of O^T; at head dim 16 one block whose rows 16..31 are
  // products of repeated head dims, never stored
  constexpr int DB = D >= 32 ? D / 32 : 1;
  static_assert(NI >= 1 && (NI % NW == 0 || NI < NW), "loads must split evenly over the waves");
  static_assert(S >= 4 && 2 * NJ * (S - 1) < 64, "ring depth / vmcnt range");
  static_assert(S * TB <= 65536, "slot offsets within a K or V ring are immediate LDS offsets");
  constexpr int COMBINE = G == 1 ? 0 : (G * NW * 32 * 64 + 2 * G * NW * 64) * 4;   // finish_chunk's buffer
  constexpr int SMEM = G * RING > COMBINE ? G * RING : COMBINE;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv / NW, wave = wv % NW;
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int lg = lane >> 4, li = lane & 15;
  const int nch = a.tab.nchunks;
  int bid = ordered_block(a.order);
  const int c = bid % nch;
  bid /= nch;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int t_begin = a.tab.bnd[c];
  int t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + bh * (int64_t)a.N * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + bh * (int64_t)a.N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + (int64_t)b * a.q_bstride +
                       (int64_t)h * a.M * D;

  // Padding mask (one token group only: its per-tile barriers must be uniform
  // over the workgroup).  The chunk ends at its last valid token; a chunk whose
  // valid tokens then form its whole range (a valid prefix) runs as unmasked.
  const_u64* mw = (G == 1 && a.mask_words) ? (const_u64*)(a.mask_words + (int64_t)b * a.mask_words_stride) : nullptr;
  if (mw) {
    int* red = reinterpret_cast<int*>(smem);   // (the ring is not in use yet)
    if (tid == 0) {
      red[0] = t_begin - 1;
      red[1] = 0;
    }
    __syncthreads();
    int last = t_begin - 1, cnt = 0;
    for (int w = (t_begin >> 6) + tid; w <= ((t_end - 1) >> 6); w += 64 * NW * G) {
      uint64_t x = reinterpret_cast<const uint64_t*>(a.mask_words + (int64_t)b * a.mask_words_stride)[w];
      const int lo = 64 * w;
      if (lo < t_begin) x &= ~0ull << (t_begin - lo);
      if (t_end - lo < 64) x &= (1ull << (t_end - lo)) - 1ull;
      if (x) {
        last = lo + 63 - __builtin_clzll(x);
        cnt += __builtin_popcountll(x);
      }
    }
    if (cnt) {
      atomicMax(&red[0], last);
      atomicAdd(&red[1], cnt);
    }
    __syncthreads();
    const int lastv = red[0], nvalid = red[1];
    __syncthreads();   // every thread has read the result before the ring reuses it
    t_end = lastv + 1;
    if (nvalid == t_end - t_begin) mw = nullptr;
  }

  // FOLD (head dim 16, where the score products are cheap): s log2(e) and the
  // row's reference are folded into the score products, so a weight is one
  // exp2 of the product's result.  Q enters as the bf16 pair hi + lo of
  // s log2(e) Q (16 significant bits: the scores carry a relative error below
  // 2^-16), and the accumulator starts at -R, R the row's reference in
  // log2 units.
  constexpr bool FOLD = D == 16;
  const float c2 = a.scale_log2;
  bf16x8_t qop[KS], qlo[KS];
  {
    const uint16_t* qrow = Qg + (int64_t)(32 * wave + l32) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = __builtin_bit_cast(bf16x8_t, ld16(qrow + 16 * ks));
  }
  wait_vm<0>();   // afterwards only the ring's loads are in flight
  if constexpr (FOLD) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t w = __builtin_bit_cast(u32x4_t, qop[ks]);
      u32x4_t hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = bf16lo(w[e]) * c2, f1 = bf16hi(w[e]) * c2;
        const uint32_t h2 = pack_bf16x2(f0, f1);
        hi[e] = h2;
        lo[e] = pack_bf16x2(f0 - bf16lo(h2), f1 - bf16hi(h2));
      }
      qop[ks] = __builtin_bit_cast(bf16x8_t, hi);
      qlo[ks] = __builtin_bit_cast(bf16x8_t, lo);
    }
  }

  // Local tiles 0 .. ntg-1 of this group are chunk tiles grp, grp+G, ...; only
  // the chunk's last tile can be partial.
  const int ntiles = (t_end - t_begin + TILE - 1) / TILE;
  const int nrounds = (ntiles + G - 1) / G;   // the same for every wave: one barrier per round
  const int ntg = ntiles > grp ? (ntiles - grp + G - 1) / G : 0;
  const int tail = t_end - t_begin - (ntiles - 1) * TILE;   // tokens of the chunk's last tile
  const bool owns_last = ntiles > 0 && (ntiles - 1) % G == grp;
  auto nval = [&](int u) -> int {
    if (u >= ntg) return 0;
    return (u == ntg - 1 && owns_last) ? tail : TILE;
  };
  // validity bits of local tile u (masked chunks): tokens in the chunk and valid
  constexpr uint64_t FULLB = TILE == 64 ? ~0ull : ((1ull << TILE) - 1ull);
  auto tbits = [&](int u) -> uint64_t {
    const int n = nval(u);
    if (n == 0) return 0ull;
    const uint64_t in = n >= 64 ? ~0ull : ((1ull << n) - 1ull);
    return in & mask_tile_bits(mw, t_begin + (grp + G * u) * TILE);
  };

  uint8_t* ring = smem + grp * RING;
  const uint32_t ring_lds = lds_addr(ring);
  uint32_t voff[NJ], voff0[NJ];
  int vrow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int byte = (wave + NW * j) * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    const int ch = pc ^ kv_swz<D>(r);
    vrow[j] = r;
    voff[j] = r * ROWB + ch * 16;
    voff0[j] = ch * 16;
  }
  // K (is_v false) or V rows of local tile u into ring slot `slot` (full:
  // the tile is known to hold TILE rows)
  auto issue = [&](int u, int slot, bool is_v, bool full = false) {
    if (NI < NW && wave >= NI) return;   // (wave-uniform)
    const int t0 = t_begin + (grp + G * u) * TILE;
    const int nrows = t_end - t0;
    const uint16_t* base = (is_v ? Vg : Kg) + (int64_t)t0 * D;
    const uint32_t dst = ring_lds + (is_v ? S + slot : slot) * TB;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      dma16_off(base, (full || vrow[j] < nrows) ? voff[j] : voff0[j], dst + (wave + NW * j) * 1024);
  };

  // Per-lane LDS addresses in slot 0; slots and k-steps are immediate offsets
  // (the swizzle depends on the row modulo 16 only).
  //  * score product, A operand: K row swap23(l32) (+32 per block), 16-byte chunk (2k+hh) ^ swizzle
  //  * value product, A operand by transposing reads: in each 16-lane group lane i
  //    points at token row (i/4) of a 4-token block and 4 head dims from 4*(i%4)
  uint32_t kaddr[KS], vaddr[DB][2];
  {
    const int swk = kv_swz<D>(swap23(l32));
#pragma unroll
    for (int k = 0; k < KS; ++k) kaddr[k] = ring_lds + swap23(l32) * ROWB + (((2 * k + hh) ^ swk) * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int n0 = 8 * (lg >> 1) + 4 * q + (li >> 2);
        // head dim 16: the lanes of operand rows 16..31 read dims 0..15 again
        const int d0 = 32 * db + (D >= 32 ? 16 * (lg & 1) : 0) + 4 * (li & 3);
        vaddr[db][q] = ring_lds + S * TB + n0 * ROWB + (((d0 >> 3) ^ kv_swz<D>(n0)) * 16) + (d0 & 7) * 2;
      }
  }
  typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4;

  // Row sums on a 16x16x32 product: fed the weight operand of the 32x32x16
  // product as its B, lane l contributes row l%32, tokens 8*(l/32)+0..7 as
  // column l%16, contraction block l/16.  Selector rows 0 and 8 pick blocks 0
  // and 2 (rows 0..15), rows 4 and 12 blocks 1 and 3 (rows 16..31), so that
  // register 0 of lane l (result row 4*(l/16), column l%16) is the sum of
  // row l%32: both lane halves hold their row's sum, like the softmax state.
  // The other result registers stay 0.
  bf16x8_t sel;
  {
    const int si = lane & 15, kb = lane >> 4;
    const bool on = ((si == 0 || si == 8) && (kb & 1) == 0) || ((si == 4 || si == 12) && (kb & 1) == 1);
    const uint32_t w = on ? 0x3f803f80u : 0u;
    sel = __builtin_bit_cast(bf16x8_t, u32x4_t{w, w, w, w});
  }

  // scores of the tile in K slot `slot`: register r of lane half hh in block b2
  // holds token 32*b2 + 16*(r/8) + 8*hh + r%8 of latent row l32
  // FOLD: -R of row l32 in every accumulator register (R = 0 until a rebase)
  f32x16_t cinit = f32x16_t{};
  auto scores = [&](int slot, f32x16_t* sc) {
    u32x4_t kop[KS][NB];
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int b2 = 0; b2 < NB; ++b2) kop[k][b2] = *(lds_u32x4*)(uintptr_t)(kaddr[k] + slot * TB + 32 * b2 * ROWB);
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2) sc[b2] = FOLD ? cinit : f32x16_t{};
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int b2 = 0; b2 < NB; ++b2) {
        sc[b2] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, kop[k][b2]), qop[k], sc[b2]);
        if constexpr (FOLD) sc[b2] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, kop[k][b2]), qlo[k], sc[b2]);
      }
  };
  f32x16_t o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16_t{};
  float lsum = 0.f;          // running row sum of the weights (row l32, both lane halves)
  // weighted values of the tile in V slot `slot` with weights pk
  auto values = [&](int slot, const bf16x8_t* pk) {
    u32x2_t part[NK][DB][2];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          part[ks][db][q] = __builtin_bit_cast(
              u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                           (lds_bf16x4*)(uintptr_t)(vaddr[db][q] + slot * TB + 16 * ks * ROWB)));
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4_t av = {part[ks][db][0][0], part[ks][db][0][1], part[ks][db][1][0], part[ks][db][1][1]};
        o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, av), pk[ks], o[db]);
      }
  };
  // scores of tokens at or past n of the tile become -inf (n = 0: a tile
  // past the group's end, whose slots hold stale or never-written rows)
  auto mask_tail = [&](f32x16_t* sc, int n) {
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tk = 32 * b2 + 16 * (r >> 3) + 8 * hh + (r & 7);
        if (tk >= n) sc[b2][r] = kNegInf;
      }
  };
  // scores of the tile's invalid tokens become -inf
  auto mask_bits = [&](f32x16_t* sc, uint64_t bits) {
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tk = 32 * b2 + 16 * (r >> 3) + 8 * hh + (r & 7);
        if (!((bits >> tk) & 1ull)) sc[b2][r] = kNegInf;
      }
  };
  // Weights of a (masked) score tile against the reference maximum m_run:
  // p = exp2(s log2(e) (score - m_run)) rounded to bf16, and the tile's row
  // sums of the rounded weights (matrix cores).  The reference is not checked
  // against the tile here: a tile whose row sum exceeds 2^12 (or is inf/NaN:
  // no reference yet, or a score far above it) is redone by `rebase`, so every
  // accepted weight is at most 2^12.
  float m_run = kNegInf;     // reference maximum of row l32 (raw dot products)
  float nmc = __builtin_huge_valf();   // -m_run s log2(e); +inf while m_run = -inf (forces a rebase)
  auto weights = [&](const f32x16_t* sc, bf16x8_t* pk, float nm, bool own_rows_only = false) -> float {
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = sc[b2][8 * g + j];
          p[j] = fast_exp2(FOLD ? (own_rows_only ? x + nm : x) : __builtin_fmaf(x, c2, nm));
        }
        const u32x4_t w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                           pack_bf16x2(p[6], p[7])};
        pk[2 * b2 + g] = __builtin_bit_cast(bf16x8_t, w);
      }
    if (own_rows_only) {
      // ones x P^T on the 32x32x16 product adds only the row's own weights
      // (the selector form multiplies the neighbouring row's weights by 0,
      // and 0 x NaN would leak across rows)
      const bf16x8_t ones =
          __builtin_bit_cast(bf16x8_t, u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
      f32x16_t la = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) la = mfma32x32x16(ones, pk[ks], la);
      return la[0];
    }
    f32x4_t ts = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pk[0], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < NK; ++ks) ts = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pk[ks], ts, 0, 0, 0);
    return ts[0];
  };
  constexpr float kSumMax = 4096.f;
  // FOLD keeps R at 0 from the start, so a row whose scores sit far below 0
  // sums to almost nothing: a row sum (with this tile) below 2^-64 also
  // sends it through the rebase.
  constexpr float kSumMin = 0x1p-64f;
  float rref = 0.f;          // FOLD: the reference R of row l32 (log2 units)
  auto bad_sum = [&](float ts) -> bool {
    if constexpr (FOLD) return !(ts <= kSumMax) || (lsum + ts < kSumMin);
    return !(ts <= kSumMax);
  };
  // Rare path: rows whose tile sum failed the check move their reference to
  // the tile's maximum (the online-softmax rescale of the value accumulators
  // and the row sum by exp2(s log2(e) (m_old - m_new)), 0 from an empty
  // state), then the tile's weights and sums are recomputed, the sums with
  // each row's own weights only.  FOLD: the scores are relative to R, so the
  // shift delta (the tile maximum, or log2 of the mass so far if that is
  // larger) moves R, the accumulator start and the scores already formed for
  // the next tile (sc_next); delta may be negative only while it stays at or
  // above the mass so far.
  auto rebase = [&](f32x16_t* sc, bf16x8_t* pk, float& ts, f32x16_t* sc_next) {
    float mc[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
      const f32x16_t& v = sc[k >> 1];
      const int r0 = 8 * (k & 1);
      float x = fmax3(v[r0], v[r0 + 1], v[r0 + 2]);
      x = fmax3(x, v[r0 + 3], v[r0 + 4]);
      x = fmax3(x, v[r0 + 5], v[r0 + 6]);
      mc[k] = fmax2(x, v[r0 + 7]);
    }
    float mx = fmax3(mc[0], mc[1], fmax2(mc[2], mc[3]));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmax2(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    if constexpr (FOLD) {
      const bool bad = bad_sum(ts);
      const float d = lsum > 0.f ? fmax2(mx, __log2f(lsum)) : mx;
      const float delta = (bad && d != kNegInf) ? d : 0.f;
      const float alpha = delta == 0.f ? 1.f : (lsum > 0.f ? fast_exp2(-delta) : 0.f);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) o[i] *= alpha;
      rref += delta;
#pragma unroll
      for (int r = 0; r < 16; ++r) cinit[r] -= delta;
#pragma unroll
      for (int b2 = 0; b2 < NB; ++b2)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc_next[b2][r] -= delta;
      ts = weights(sc, pk, -delta, true);
      return;
    }
    const bool bad = !(ts <= kSumMax);
    const float m_new = (bad && mx != kNegInf) ? fmax2(mx, m_run) : m_run;
    const float alpha = (m_new == m_run) ? 1.f : fast_exp2((m_run - m_new) * c2);   // 0 when m_run = -inf
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] *= alpha;
    m_run = m_new;
    nmc = m_run == kNegInf ? __builtin_huge_valf() : -m_run * c2;
    ts = weights(sc, pk, m_run == kNegInf ? 0.f : nmc, true);
  };


  // ---- V slots start as zeros: a round past the group's end multiplies
  // weights that are exactly 0 with whatever its slot holds, which must not
  // be NaN.  (Completed before the barrier that precedes the first load.)
  for (int i = tid - grp * 64 * NW; i < S * TB / 16; i += 64 * NW)
    st16(ring + S * TB + 16 * i, u32x4_t{0, 0, 0, 0});
  barrier_lds();

  // ---- prologue: K(0), K(1), then batches 0 .. S-3 (batch S-2 would reuse K(0)'s slot).
  // Batch t holds (t+2 < ntg) + (t < ntg) loads of NJ each.
  auto clampS2 = [](int x) { return x < 0 ? 0 : (x > S - 2 ? S - 2 : x); };
  if (ntg > 0) issue(0, 0, false);
  if (ntg > 1) issue(1, 1, false);
#pragma unroll
  for (int k = 0; k < S - 2; ++k) {
    if (k + 2 < ntg) issue(k + 2, (k + 2) % S, false);
    if (k < ntg) issue(k, k % S, true);
  }
  wait_units<NJ, 2 * (S - 2)>(clampS2(ntg - 2) + clampS2(ntg));   // K(0), K(1) landed
  barrier_lds();
  // scores and weights of tile t live in buffer t % 2: round u reads the
  // weights of tile u and the scores of tile u+1 and writes the weights of
  // tile u+1 and the scores of tile u+2
  f32x16_t scb[2][NB];
  bf16x8_t pkb[2][NK];
  float ts_pend;   // row sums of the weights made last round, checked at the start of the next
  {
    scores(0, scb[0]);
    scores(1, scb[1]);
    if (mw) {
      const uint64_t b0 = tbits(0);
      if (b0 != FULLB) mask_bits(scb[0], b0);
    } else if (nval(0) < TILE) {
      mask_tail(scb[0], nval(0));
    }
    ts_pend = weights(scb[0], pkb[0], nmc);
  }
  barrier_lds();             // every wave is done with K slots 0 and 1
  if (S < ntg) issue(S, 0, false);
  if (S - 2 < ntg) issue(S - 2, S - 2, true);

  // ---- rounds, 2S per trip so that ring slots and buffer parities are
  // compile-time constants.  Round u (slot st = u % S, parity sr % 2):
  auto round = [&](const int u, const int sr, auto steady_t) {
    // STEADY: u + S + 2 < ntg, so both of the round's loads are issued, every
    // tile they and the round touch is full, and S-2 full batches are in
    // flight behind batch u
    constexpr bool STEADY = decltype(steady_t)::value;
    const int st = sr % S;
    // batch u = {K(u+2), V(u)} complete for this wave; batches u+1 .. u+S-2 may be in flight
    if constexpr (STEADY)
      wait_vm<2 * (S - 2) * NJ>();
    else
      wait_units<NJ, 2 * (S - 2)>(clampS2(ntg - u - 3) + clampS2(ntg - u - 1));
    barrier_lds();
    // every wave is past round u-1: K slot (u+1)%S and V slot (u-1)%S are free
    if (STEADY || u + S + 1 < ntg) issue(u + S + 1, (st + 1) % S, false, STEADY);
    if (STEADY || u + S - 1 < ntg) issue(u + S - 1, (st + S - 1) % S, true, STEADY);
    const int e = sr % 2, f = 1 - e;     // tile u: buffer e; tile u+1: buffer f; tile u+2: buffer e
    if (!STEADY && mw) {
      // invalid rows of V(u) become zero (a padded row may hold NaN, and its
      // weight 0 must not meet it); uniform over the workgroup (one group)
      const uint64_t bu = tbits(u);
      if (bu != FULLB) {
        uint8_t* vs = ring + (S + st) * TB;
        for (int i = tid; i < TILE * (ROWB / 16); i += 64 * NW) {
          const int r = i / (ROWB / 16);
          if (!((bu >> r) & 1ull)) st16(vs + 16 * i, u32x4_t{0, 0, 0, 0});
        }
        barrier_lds();
      }
    }
    if (__ballot(bad_sum(ts_pend))) rebase(scb[e], pkb[e], ts_pend, scb[f]);
    lsum += ts_pend;
    if constexpr (!STEADY) {
      if (mw) {
        const uint64_t b1 = tbits(u + 1);
        if (b1 != FULLB) mask_bits(scb[f], b1);
      } else {
        const int n1 = nval(u + 1);
        if (n1 < TILE) mask_tail(scb[f], n1);
      }
    }
    // one straight-line block: the value products of tile u, the weights
    // of tile u+1 and their row sums, the score products of tile u+2
    scores((st + 2) % S, scb[e]);
    values(st, pkb[e]);
    ts_pend = weights(scb[f], pkb[f], nmc);
    // order: all operand reads (V, then K), a few exponentials while they
    // arrive, then each product with exponentials and conversions between
    // (vector groups take vector and transcendental instructions)
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NK * DB + NB * KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);
#pragma unroll
    for (int i = 0; i < NK * DB + (FOLD ? 2 : 1) * NB * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
    }
  };
  // steady trips first (no tile tail, fixed waits, unconditional loads), then
  // the remaining rounds with every check
  const int nsteady = mw ? 0 : ntg - S - 2;   // (masked chunks: every round checks its tiles)
  int u0 = 0;
  for (; u0 + 2 * S <= nsteady; u0 += 2 * S) {
#pragma unroll
    for (int sr = 0; sr < 2 * S; ++sr) round(u0 + sr, sr, std::true_type{});
  }
  for (; u0 < nrounds; u0 += 2 * S) {
#pragma unroll
    for (int sr = 0; sr < 2 * S; ++sr)
      if (u0 + sr < nrounds) round(u0 + sr, sr, std::false_type{});
  }

  // (the sums left pending belong to the tile after the group's last, which
  // holds no token)
  if constexpr (FOLD) m_run = lsum > 0.f ? rref / c2 : kNegInf;   // the reference in raw units
  finish_chunk<D, NW, G>(smem, a, grp, wave, lane, o, m_run, lsum, b, h, c);
  merge_tail(a, b, h, c, reinterpret_cast<int*>(smem));
}

bool encode_mfma_supported(int M, int D) {
  return (D == 16 || D == 64 || D == 128) && (M == 32 || M == 64 || M == 128 || M == 256);
}

template <int D, int NW, int S, int G>
static hipError_t launch_mfma_t(const EncodeArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * a.H * a.B;
  hipLaunchKernelGGL((encode_mfma_kernel<D, NW, S, G>), dim3((unsigned)grid), dim3(64 * NW * G), 0, s, a);
  return hipGetLastError();
}

// Matrix-core encoder variants, fixed at build time.  Head dim 64: one
// workgroup of 3-stage rings (16 KB stages) per 32*NW latent rows; at 128
// latent rows (padding masks: the pipelined encoder takes the unmasked case)
// three 4-wave token groups (12 waves, three 48 KB rings) fill a CU as one
// workgroup, so a partition needs no split and no fold.  Head dim 128: 32 KB
// stages, four of them from 128 latent rows on.  Head dim 16: 2 KB tiles,
// 4-stage rings.
int encode_mfma_per_cu(int M, int D, bool masked) {
  // workgroups of the chosen variant that fit on one CU (LDS and registers)
  if (encode_ilv_used(M, D, masked)) return 1;
  if (D == 64) return M == 128 ? 1 : 3;
  if (D == 16) return M >= 256 ? 2 : (M == 128 ? 4 : 8);   // 16 KB rings, up to 16 waves of <=128 VGPRs
  return M >= 128 ? 1 : 2;
}

// The two-tile pipelined encoder serves bf16 inputs without a padding mask at
// head dims 64 and 16: 128 latent rows as two 4-wave groups with 64-token
// tiles, 64 rows as four 2-wave groups (32-token tiles at head dim 64) --
// 8 waves and four-stage rings either way, one workgroup per CU.  At head dim
// 128 it serves 256 latent rows, masked or not, as one group of 8 waves with
// 32-token tiles and a six-stage ring.
bool encode_ilv_used(int M, int D, bool masked) {
  return ((D == 64 || D == 16) && (M == 128 || M == 64) && !masked) || (D == 128 && M == 256);
}

static bool encode_ilv_selected(const EncodeArgs& a) { return encode_ilv_used(a.M, a.D, a.mask_words != nullptr); }

hipError_t launch_encode_mfma(const EncodeArgs& a, hipStream_t s) {
  if (encode_ilv_selected(a)) {
    const int64_t grid = (int64_t)a.tab.nchunks * a.H * a.B;
    if (a.D == 16) {
      // 2 KB tiles; the loop is instruction-bound, and a 4-stage ring measured
      // faster than 6 or 8 stages (fewer wait cases per round)
      if (a.M == 128)
        hipLaunchKernelGGL((encode_ilv_kernel<16, 4, 4, 2, 64>), dim3((unsigned)grid), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((encode_ilv_kernel<16, 2, 4, 4, 64>), dim3((unsigned)grid), dim3(512), 0, s, a);
    } else if (a.D == 128) {
      // 256 latent rows: one group of eight waves, 32-token tiles, padding masks
      // handled per tile
      hipLaunchKernelGGL((encode_ilv_kernel<128, 8, 6, 1, 32>), dim3((unsigned)grid), dim3(512), 0, s, a);
    } else if (a.M == 128) {
      hipLaunchKernelGGL((encode_ilv_kernel<64, 4, 4, 2, 64>), dim3((unsigned)grid), dim3(512), 0, s, a);
    } else {
      hipLaunchKernelGGL((encode_ilv_kernel<64, 2, 4, 4, 32>), dim3((unsigned)grid), dim3(512), 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.D == 64) {
    switch (a.M) {
      case 32: return launch_mfma_t<64, 1, 3, 1>(a, s);
      case 64: return launch_mfma_t<64, 2, 3, 1>(a, s);
      case 128: return launch_mfma_t<64, 4, 3, 3>(a, s);
      case 256: return launch_mfma_t<64, 8, 3, 1>(a, s);
    }
  } else if (a.D == 16) {
    // padding masks at head dim 16 (the pipelined encoder takes the rest)
    switch (a.M) {
      case 32: return launch_mfma_t<16, 1, 4, 1>(a, s);
      case 64: return launch_mfma_t<16, 2, 4, 1>(a, s);
      case 128: return launch_mfma_t<16, 4, 4, 1>(a, s);
      case 256: return launch_mfma_t<16, 8, 4, 1>(a, s);
    }
  } else if (a.D == 128) {
    // (256 latent rows take the pipelined encoder)
    switch (a.M) {
      case 32: return launch_mfma_t<128, 1, 3, 1>(a, s);
      case 64: return launch_mfma_t<128, 2, 3, 1>(a, s);
      case 128: return launch_mfma_t<128, 4, 4, 1>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Padding mask -> one 64-bit validity word per 64 tokens (bit i of word w of
// batch b is mask[b][64w + i] != 0; tokens past N read as invalid), so that the
// matrix-core encoder tests a whole tile with two scalar loads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mask_words_kernel(const uint8_t* __restrict__ mask, int B, int N,
                                                          uint64_t* __restrict__ words, int64_t stride) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)B * stride) return;
  const int b = (int)(idx / stride);
  const int w = (int)(idx % stride);
  const uint8_t* mr = mask + (int64_t)b * N;
  uint64_t bits = 0;
  for (int i = 0; i < 64; ++i) {
    const int t = 64 * w + i;
    if (t < N && mr[t] != 0) bits |= 1ull << i;
  }
  words[idx] = bits;
}

// One workgroup: valid-token count of every (batch, chunk) pair from the mask
// words, rank by counting (heavier first, ties by index), then the order table.
// The counts are spread over all threads: consecutive threads take
// consecutive words of one pair (coalesced loads, LDS atomics), so no thread
// walks a whole chunk.
__global__ __launch_bounds__(1024) void heavy_first_kernel(const uint64_t* __restrict__ words, int64_t stride,
                                                           const ChunkTable tab, int B, int H,
                                                           int32_t* __restrict__ order) {
  __shared__ int key[kMaxOrderItems];
  __shared__ int maxw_s;
  const int nch = tab.nchunks, n = B * nch;
  if (threadIdx.x == 0) {
    int mw = 0;
    for (int c = 0; c < nch; ++c) {
      const int lo = tab.bnd[c], hi = tab.bnd[c + 1];
      if (hi > lo) mw = max(mw, ((hi - 1) >> 6) - (lo >> 6) + 1);
    }
    maxw_s = mw;
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) key[i] = 0;
  __syncthreads();
  const int W = maxw_s;
  const int64_t total = (int64_t)n * W;
  for (int64_t idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int i = (int)(idx / W), kk = (int)(idx % W);
    const int b = i / nch, c = i % nch;
    const int lo = tab.bnd[c], hi = tab.bnd[c + 1];
    const int k = (lo >> 6) + kk;
    if (lo >= hi || k > ((hi - 1) >> 6)) continue;
    uint64_t x = words[(int64_t)b * stride + k];
    const int a0 = lo - 64 * k, a1 = hi - 64 * k;   // keep bits [a0, a1) of this word
    if (a0 > 0) x &= ~0ull << a0;
    if (a1 < 64) x &= (1ull << a1) - 1ull;
    const int cnt = __popcll(x);
    if (cnt) atomicAdd(&key[i], cnt);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int ki = key[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) rank += (key[j] > ki) || (key[j] == ki && j < i);
    const int b = i / nch, c = i % nch;
    for (int h = 0; h < H; ++h) order[rank * H + h] = (b * H + h) * nch + c;
  }
}

hipError_t launch_heavy_first(const uint64_t* mask_words, int64_t mw_stride, const ChunkTable& tab, int B, int H,
                              int32_t* order, hipStream_t s) {
  if (B * tab.nchunks > kMaxOrderItems || B * tab.nchunks == 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(heavy_first_kernel, dim3(1), dim3(1024), 0, s, mask_words, mw_stride, tab, B, H, order);
  return hipGetLastError();
}

hipError_t launch_mask_words(const uint8_t* mask, int B, int N, uint64_t* words, int64_t stride, hipStream_t s) {
  const int64_t n = (int64_t)B * stride;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mask_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, mask, B, N, words, stride);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Single latent row (M = 1), bf16: split-KV decoding attention of one query
// against a chunk of keys.  This is a streaming dot-product/axpy over the
// chunk (HBM-bound, one flop pair per byte), done on the vector ALUs: a group
// of D/8 lanes owns one key at a time (16 contiguous bytes per lane, so a wave
// reads whole rows), reduces the dot product across its lanes, and keeps its
// own online-softmax state; the 256/(D/8) group states are merged in LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void encode_q1_kernel(const EncodeArgs a) {
  constexpr int LPK = D / 8;          // lanes per key
  constexpr int G = 256 / LPK;        // key groups per workgroup
  constexpr int U = 4;                // keys per group per iteration
  __shared__ float sm_m[G], sm_l[G];
  __shared__ float sm_acc[G][D];

  const int tid = threadIdx.x;
  const int g = tid / LPK, lig = tid % LPK;
  const int nch = a.tab.nchunks;
  int bid = blockIdx.x;
  const int c = bid % nch;
  bid /= nch;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + bh * (int64_t)a.N * D + 8 * lig;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + bh * (int64_t)a.N * D + 8 * lig;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + (int64_t)b * a.q_bstride + (int64_t)h * D + 8 * lig;
  const uint8_t* mk = a.mask ? a.mask + (int64_t)b * a.N : nullptr;
  const float c2 = a.scale_log2;

  float q[8];
  {
    const u32x4_t w = ld16(Qg);
#pragma unroll
    for (int j = 0; j < 4; ++j) { q[2 * j] = bf16lo(w[j]); q[2 * j + 1] = bf16hi(w[j]); }
  }
  float m_run = kNegInf, l_run = 0.f, acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  for (int base = t_begin; base < t_end; base += G * U) {
    u32x4_t kw[U], vw[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + g + G * u;
      ok[u] = t < t_end;
      if (ok[u] && mk) ok[u] = mk[t] != 0;
      if (ok[u]) {
        kw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Kg + (int64_t)t * D));
        vw[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Vg + (int64_t)t * D));
      } else {
        kw[u] = u32x4_t{0, 0, 0, 0};
        vw[u] = u32x4_t{0, 0, 0, 0};
      }
    }
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d = __builtin_fmaf(q[2 * j], bf16lo(kw[u][j]), d);
        d = __builtin_fmaf(q[2 * j + 1], bf16hi(kw[u][j]), d);
      }
#pragma unroll
      for (int o = LPK / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
      sc[u] = ok[u] ? d : kNegInf;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float nmc = -m_use * c2;
    const float alpha = fast_exp2(m_run * c2 + nmc);
    float p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) p[u] = fast_exp2(__builtin_fmaf(sc[u], c2, nmc));
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float e = acc[2 * j] * alpha, f = acc[2 * j + 1] * alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        e = __builtin_fmaf(p[u], bf16lo(vw[u][j]), e);
        f = __builtin_fmaf(p[u], bf16hi(vw[u][j]), f);
      }
      acc[2 * j] = e;
      acc[2 * j + 1] = f;
    }
    m_run = m_new;
  }
  if (lig == 0) { sm_m[g] = m_run; sm_l[g] = l_run; }
#pragma unroll
  for (int j = 0; j < 8; ++j) sm_acc[g][8 * lig + j] = acc[j];
  __syncthreads();

  const int slot = a.tab.slot[c];
  float* Ob;
  float* Lb;
  if (slot < 0) {
    const int r = -slot - 1;
    Ob = a.O_part + (((int64_t)r * a.B + b) * a.H + h) * (int64_t)D;
    Lb = a.L_part + (((int64_t)r * a.B + b) * a.H + h);
  } else {
    Ob = a.ws_O + (((int64_t)slot * a.B + b) * a.H + h) * (int64_t)D;
    Lb = a.ws_L + (((int64_t)slot * a.B + b) * a.H + h);
  }
  float M = kNegInf;
  for (int i = 0; i < G; ++i) M = fmaxf(M, sm_m[i]);
  const float Mu = (M == kNegInf) ? 0.f : M;
  float l = 0.f;
  for (int i = 0; i < G; ++i) l += sm_l[i] * fast_exp2((sm_m[i] - Mu) * c2);
  const bool empty = !(l > 0.f);
  if (tid < D) {
    float o = 0.f;
    for (int i = 0; i < G; ++i) o += sm_acc[i][tid] * fast_exp2((sm_m[i] - Mu) * c2);
    Ob[tid] = empty ? 0.f : o / l;
  }
  if (tid == 0) *Lb = empty ? kNegInf : (M * a.scale + __logf(l));
}

bool encode_q1_supported(int M, int D) { return M == 1 && (D == 32 || D == 64 || D == 128); }

hipError_t launch_encode_q1(const EncodeArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * a.H * a.B;
  switch (a.D) {
    case 32: hipLaunchKernelGGL(encode_q1_kernel<32>, dim3((unsigned)grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(encode_q1_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(encode_q1_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// General vector encoder (float32 inputs, or bf16 shapes without a matrix-core
// variant).  One wave per (batch, head, chunk, latent row); a token tile gives
// one score per lane, then lanes switch to head dimensions to accumulate the
// weighted values.  All arithmetic is float32.
// ---------------------------------------------------------------------------
template <typename TIn>
__device__ __forceinline__ float ldv(const TIn* p);
template <>
__device__ __forceinline__ float ldv<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldv<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// The workgroup's four waves take latent rows 4g .. 4g+3 of (b, h) over chunk
// c.  Token tiles of TT rows (64 up to head dim 64, then 64*64/D) are staged
// in LDS as float32 with rows padded to D+1 words (a lane reading its own row
// hits its own bank), once for all four rows.  Per tile: one score per lane
// (lane = token), the tile's maximum and weights, then lanes switch to head
// dimensions to accumulate the weighted values in token order.
constexpr int kGenTileWords = 2 * 64 * 65;   // K and V tiles: 2 * TT * (D+1) <= 8320 for D <= 256
template <typename TIn>
__global__ __launch_bounds__(256) void encode_generic_kernel(const EncodeArgs a) {
  constexpr int MAXDL = 4;  // D <= 256
  __shared__ float sm[kGenTileWords + 4 * 256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = a.tab.nchunks;
  const int mgroups = (a.M + 3) / 4;
  int bid = blockIdx.x;
  const int c = bid % nch;
  bid /= nch;
  const int mg = bid % mgroups;
  bid /= mgroups;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int m = 4 * mg + wave;
  const bool active = m < a.M;   // (wave-uniform) a row past M only helps stage the tiles
  const int D = a.D;
  const int DP = D + 1;
  const int TT = D <= 64 ? 64 : (D <= 128 ? 32 : 16);
  float* kt = sm;
  float* vt = sm + TT * DP;
  float* qs = sm + kGenTileWords + wave * 256;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const TIn* Kg = static_cast<const TIn*>(a.K) + bh * (int64_t)a.N * D;
  const TIn* Vg = static_cast<const TIn*>(a.V) + bh * (int64_t)a.N * D;
  const uint8_t* mk = a.mask ? a.mask + (int64_t)b * a.N : nullptr;
  const float c2 = a.scale_log2;
  if (active) {
    const TIn* Qr = static_cast<const TIn*>(a.Q) + (int64_t)b * a.q_bstride + ((int64_t)h * a.M + m) * D;
    for (int d = lane; d < D; d += 64) qs[d] = ldv(Qr + d);
  }

  float m_run = kNegInf, l_run = 0.f, acc[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) acc[j] = 0.f;

  for (int t0 = t_begin; t0 < t_end; t0 += TT) {
    const int n = t_end - t0 < TT ? t_end - t0 : TT;
    __syncthreads();   // every wave is done with the previous tile
    // padded tokens get zero value rows (their weights are 0 and a padded row
    // may hold NaN), so the value loop below needs no per-token branch
    for (int f = threadIdx.x; f < n * D; f += 256) {
      const int r = f / D, d = f - r * D;
      kt[r * DP + d] = ldv(Kg + (int64_t)t0 * D + f);
      vt[r * DP + d] = (!mk || mk[t0 + r] != 0) ? ldv(Vg + (int64_t)t0 * D + f) : 0.f;
    }
    __syncthreads();
    if (!active) continue;
    bool ok = lane < n;
    if (ok && mk) ok = mk[t0 + lane] != 0;
    float sdot = kNegInf;
    if (ok) {
      const float* kr = kt + lane * DP;
      float d = 0.f;
      for (int i = 0; i < D; i += 4) {   // D % 4 == 0
        const float k0 = kr[i], k1 = kr[i + 1], k2 = kr[i + 2], k3 = kr[i + 3];
        d = __builtin_fmaf(qs[i], k0, d);
        d = __builtin_fmaf(qs[i + 1], k1, d);
        d = __builtin_fmaf(qs[i + 2], k2, d);
        d = __builtin_fmaf(qs[i + 3], k3, d);
      }
      sdot = d;
    }
    const float mx = wave_max(sdot);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float nmc = -m_use * c2;
    const float alpha = fast_exp2(m_run * c2 + nmc);
    const float p = ok ? fast_exp2(__builtin_fmaf(sdot, c2, nmc)) : 0.f;
    l_run = l_run * alpha + wave_sum(p);
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) acc[j] *= alpha;
    // tokens in order, four per step so that their reads are issued together
    int i = 0;
    for (; i + 4 <= n; i += 4) {
      float pi[4], vv[4][MAXDL];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pi[k] = __shfl(p, i + k, 64);
#pragma unroll
        for (int j = 0; j < MAXDL; ++j) vv[k][j] = lane + 64 * j < D ? vt[(i + k) * DP + lane + 64 * j] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = 0; j < MAXDL; ++j) acc[j] = __builtin_fmaf(pi[k], vv[k][j], acc[j]);
    }
    for (; i < n; ++i) {
      const float pi = __shfl(p, i, 64);
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) {
        const int d = lane + 64 * j;
        if (d < D) acc[j] = __builtin_fmaf(pi, vt[i * DP + d], acc[j]);
      }
    }
    m_run = m_new;
  }
  if (!active) return;
  const int slot = a.tab.slot[c];
  float* Ob;
  float* Lb;
  if (slot < 0) {
    const int r = -slot - 1;
    Ob = a.O_part + ((((int64_t)r * a.B + b) * a.H + h) * a.M + m) * (int64_t)D;
    Lb = a.L_part + (((int64_t)r * a.B + b) * a.H + h) * a.M + m;
  } else {
    Ob = a.ws_O + ((((int64_t)slot * a.B + b) * a.H + h) * a.M + m) * (int64_t)D;
    Lb = a.ws_L + (((int64_t)slot * a.B + b) * a.H + h) * a.M + m;
  }
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) Ob[d] = acc[j] * inv;
  }
  if (lane == 0) *Lb = empty ? kNegInf : (m_run * a.scale + __logf(l_run));
}

hipError_t launch_encode_generic(const EncodeArgs& a, bool bf16, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * ((a.M + 3) / 4) * a.H * a.B;
  if (bf16)
    hipLaunchKernelGGL(encode_generic_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(encode_generic_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace flare
