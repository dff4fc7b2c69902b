/*
 * flare.h -- C ABI of the MI355X (gfx950) split-KV softmax library (libflare.so).
 *
 * The library computes exact softmax attention of M latent query rows over N
 * token keys/values that are split into R disjoint partitions, returns each
 * partition's normalised output and log-normaliser, merges those states with
 * the associative log-sum-exp rule, decodes every token against the latents,
 * and differentiates the encoder with the global statistics.  Sources:
 *
 *  [FLARE++] "FLARE++: Low-rank attention with dynamic attention routing",
 *            appendix on context parallelism (eq. 18, the local-shard states,
 *            eq. 23, the max-stabilised merge, the FLARE and FLARE++ forward
 *            paragraphs, the backward paragraph).
 *  [RING]    "Ring vs. Tree Attention" (the online-softmax merge, the balanced
 *            tree schedule, the failure mode of overlapping subsets).
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE pointers to dense row-major arrays owned by the
 *    caller; the library never allocates, frees or keeps them.  Offsets are a
 *    HOST array.
 *  - Layouts: Q is [H,M,D] replicated over the batch (q_batch_stride = 0) or
 *    [B,H,M,D] (q_batch_stride = H*M*D elements); K, V, Xq, Y, dK, dV are
 *    [B,H,N,D]; Z, dZ, dQ, O_part[r] are [B,H,M,D]; L, L_part[r] are [B,H,M];
 *    O_part is [R,B,H,M,D] and L_part is [R,B,H,M].
 *  - dtype selects the element type of Q, K, V, Xq, Klat, dZ, Y, dK, dV
 *    (FLARE_F32 = float, FLARE_BF16 = bfloat16).  O_part, L_part, Z, L and dQ
 *    are always float.  Arithmetic: products of bfloat16 operands accumulate
 *    in float (bf16 matrix cores), softmax statistics are float, and the
 *    softmax weights are rounded to bfloat16 before they multiply V.
 *  - scale is the score multiplier s (the pages use s = D^-1/2); scores are
 *    s * q.k.  Log-normalisers are natural logarithms of sums of exp(score).
 *  - mask (nullable) is [B,N] uint8, nonzero = valid key.  Masked keys never
 *    influence any output, whatever values (even NaN/Inf) they hold [FLARE++:
 *    padding is excluded by local masks].
 *  - stream is a hipStream_t (NULL = the null stream).  Every call is
 *    asynchronous on that stream and never synchronises the device.
 *  - Every argument is validated before anything is launched: a non-OK status
 *    means nothing was written.  flare_last_error() then describes the problem
 *    (thread-local).  FLARE_EHIP reports a failed launch.
 *  - The library holds no state between calls: the statistics saved by one
 *    encoder invocation are the caller's to keep [FLARE++ backward paragraph].
 *  - Supported shapes: D % 4 == 0 and 4 <= D <= 256, M >= 1; matrix-core paths
 *    for bfloat16 with D in {64,128} and M a multiple of 32 up to 256 (and D = 16:
 *    the encoder at M in {32,64,128,256}, the decode at M up to 256, both
 *    backwards at M in {32,64,128}), a vector path for M = 1, and a general vector
 *    path for everything else.
 */
#ifndef FLARE_H
#define FLARE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flare_status {
  FLARE_OK = 0,
  FLARE_EINVAL = -1,        /* bad argument: null pointer, negative size, bad offsets */
  FLARE_EUNSUPPORTED = -2,  /* valid but unsupported shape/dtype combination */
  FLARE_EHIP = -3,          /* a HIP launch failed */
  FLARE_EWORKSPACE = -4     /* workspace missing or smaller than the size query says */
} flare_status;

typedef enum flare_dtype { FLARE_F32 = 0, FLARE_BF16 = 1 } flare_dtype;

/* hipStream_t, passed as an opaque pointer so this header needs no HIP headers. */
typedef void* flare_stream_t;

/* Bytes of device workspace flare_encode needs for these arguments (0 if none);
 * masked != 0 when flare_encode will be given a padding mask.  Returns 0 as
 * well when the arguments are invalid; flare_encode reports those. */
size_t flare_encode_workspace_size(flare_dtype dtype, int B, int H, int N, int M, int D,
                                   int R, const int64_t* offsets, int masked);

/*
 * flare_encode -- the local-shard encoder of [FLARE++] (the equations between
 * eq. 18 and eq. 23), for all R partitions of every (batch, head) at once.
 *
 * Partition r holds tokens [offsets[r], offsets[r+1]); offsets has R+1 int64
 * entries with 0 = offsets[0] <= offsets[1] <= ... <= offsets[R] = N (empty
 * partitions allowed; overlapping or unsorted offsets are rejected with
 * FLARE_EINVAL since double counting would go unnoticed [RING, failure mode]).
 * For every (r, b, h, m) with S[n] = scale * Q[b,h,m,:].K[b,h,n,:] over the
 * valid tokens n of partition r:
 *     L_part[r,b,h,m]   = log sum_n exp(S[n])
 *     O_part[r,b,h,m,:] = sum_n exp(S[n] - L_part) V[b,h,n,:]
 * and a row with no valid token in the partition gets L = -inf, O = 0 (never
 * NaN).  workspace (device, nullable when the size query returns 0) must hold
 * flare_encode_workspace_size() bytes; it holds partial states between two
 * internal kernels and carries nothing between calls.
 */
flare_status flare_encode(flare_dtype dtype, int B, int H, int N, int M, int D,
                          const void* Q, int64_t q_batch_stride, const void* K, const void* V,
                          int R, const int64_t* offsets, const uint8_t* mask, float scale,
                          float* O_part, float* L_part,
                          void* workspace, size_t workspace_bytes, flare_stream_t stream);

/*
 * flare_encode_noalloc -- flare_encode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, outputs, validation and results (the
 * same kernels, bit for bit) as flare_encode without the workspace arguments:
 * the workspace comes from a fixed array in device memory that the library
 * holds on every device it runs on until the process ends.
 *  - The call allocates and frees nothing and issues no memset.
 *  - Arguments whose workspace (flare_encode_workspace_size) exceeds
 *    FLARE_NOALLOC_SCRATCH_BYTES are rejected with FLARE_EWORKSPACE before
 *    anything is launched.
 *  - All calls on one device share that device's array; it carries nothing
 *    from one call to the next that a call reads.  Two calls whose work may
 *    overlap in time on one device (other streams, graphs replayed alongside)
 *    race on it and must not be made.
 *  - The first call on a device looks up the array's address (thread-safe).
 */
#define FLARE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
flare_status flare_encode_noalloc(flare_dtype dtype, int B, int H, int N, int M, int D,
                                  const void* Q, int64_t q_batch_stride, const void* K, const void* V,
                                  int R, const int64_t* offsets, const uint8_t* mask, float scale,
                                  float* O_part, float* L_part, flare_stream_t stream);

/*
 * lse_merge -- the exact cross-partition merge of [FLARE++] (eqs. 21-23 and
 * the max-stabilised merge paragraph), evaluated as the balanced binary tree
 * of [RING]: leaves are (m, l, acc) = (L_r, 1, O_r) (or (-inf, 0, 0) for an
 * empty state); round k merges state i with state i + 2^k for i = 0 mod
 * 2^(k+1), a state without a partner passing through; each merge takes
 * m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m), acc likewise.  Outputs
 * Z = acc / l and L = m + log l per row; a row empty in every partition gets
 * Z = 0, L = -inf.
 *
 * O_part: [R, rows, D] float, L_part: [R, rows] float (rows = B*H*M).
 * Z: [rows, D] float, L: [rows] float.  Z_bf16 (nullable): [rows, D]
 * bfloat16 copy of Z, rounded to nearest even (used as the next encoder's
 * queries in FLARE++).  R >= 1.
 */
flare_status lse_merge(int R, int64_t rows, int D, const float* O_part, const float* L_part,
                       float* Z, float* L, void* Z_bf16, flare_stream_t stream);

/*
 * flare_encode_merge -- flare_encode followed by lse_merge of its R states,
 * in one call ([FLARE++]: the encoder, then the exact merge of eqs. 21-23;
 * [RING]: the tree schedule).  Outputs O_part, L_part, Z, L and Z_bf16 are
 * exactly those of flare_encode then lse_merge(R, B*H*M, D, O_part, L_part,
 * Z, L, Z_bf16) (same arithmetic in the same order, so bit for bit); the
 * arguments they share mean the same and are validated the same way, and the
 * workspace is flare_encode_workspace_size() bytes.
 *
 * On the matrix-core path (see flare_encode's supported shapes), when one
 * encoder launch covers every token chunk (up to 256 chunks) and R <= 256, the
 * merge runs inside that launch: the last workgroup to finish a partition that
 * was cut into chunks folds that partition, and the last one to finish a
 * (batch, head) slice merges its partitions, so the call makes a single launch
 * (plus the mask preparation of masked inputs).  Otherwise it makes the
 * launches of the two calls.
 *
 * counters: device array of B*H*(R+1) uint32, 4-byte aligned, owned by the caller.
 * It must hold zeros when the call runs, and every call puts it back to zero
 * by the time its work on the stream has finished (allocate it zeroed once and
 * keep it).  Two calls whose work may overlap in time on one device (other
 * streams, or a graph replayed alongside) need separate counter arrays; a
 * counter array left nonzero by a failed launch must be zeroed again before
 * the next call.  The call issues no memset and no allocation, so it may be
 * captured in a HIP graph.
 */
flare_status flare_encode_merge(flare_dtype dtype, int B, int H, int N, int M, int D,
                                const void* Q, int64_t q_batch_stride, const void* K, const void* V,
                                int R, const int64_t* offsets, const uint8_t* mask, float scale,
                                float* O_part, float* L_part, float* Z, float* L, void* Z_bf16,
                                uint32_t* counters, void* workspace, size_t workspace_bytes,
                                flare_stream_t stream);

/*
 * flare_decode -- the local decode of [FLARE++] (FLARE and FLARE++ forward
 * paragraphs): every token attends over the M replicated latents,
 *     Y[b,h,n,:] = sum_m softmax_m(scale * Xq[b,h,n,:].Klat[b,h,m,:]) Z[b,h,m,:]
 * Xq: [B,H,N,D] token-side queries (FLARE uses the token's key row K),
 * Klat: latent keys (FLARE: the latent queries Q; FLARE++: the dynamic
 * queries Q(X)), [H,M,D] with klat_batch_stride = 0 or [B,H,M,D] with
 * klat_batch_stride = H*M*D; Z: [B,H,M,D] float (the merged encoder output);
 * token_mask (nullable) [B,N] uint8, zero marks padding whose Y row is set
 * to 0.  Y: [B,H,N,D] in dtype.  No cross-partition work is involved.
 */
flare_status flare_decode(flare_dtype dtype, int B, int H, int N, int M, int D,
                          const void* Xq, const void* Klat, int64_t klat_batch_stride,
                          const float* Z, const uint8_t* token_mask, float scale, void* Y,
                          flare_stream_t stream);

/* Bytes of device workspace flare_encode_bwd needs (never 0 for valid
 * arguments: it always holds the per-row term c); masked != 0 when a padding
 * mask will be passed. */
size_t flare_encode_bwd_workspace_size(flare_dtype dtype, int B, int H, int N, int M, int D,
                                       int R, const int64_t* offsets, int masked);

/*
 * flare_encode_bwd -- the encoder backward of [FLARE++] (backward paragraph):
 * gradients of sum(dZ * Z) with the GLOBAL forward statistics Z and L (as
 * returned by lse_merge for this encoder invocation), for every partition:
 *     P[m,n]  = exp(S[m,n] - L[m])          (S as in flare_encode; 0 if masked)
 *     c[m]    = sum_d dZ[m,d] Z[m,d]        (between-partition row term)
 *     dS[m,n] = P[m,n] (dZ[m,:].V[n,:] - c[m])
 *     dV[n,:] = sum_m P[m,n] dZ[m,:]        dK[n,:] = scale sum_m dS[m,n] Q[m,:]
 *     dQ[m,:] = scale sum_n dS[m,n] K[n,:]  summed over all partitions
 * dQ: [B,H,M,D] float, one slice per batch even when Q is replicated (the sum
 * over the batch is the caller's).  dK, dV: [B,H,N,D] in dtype; rows of masked
 * tokens are written as 0 (kept as they were when accumulating).  Rows with L = -inf
 * get zero gradients.
 * dQ_cast (nullable): dQ also written in dtype (the dZ of the encoder that produced Q, in
 * the FLARE++ chain).  flags: FLARE_BWD_ACCUMULATE_* below, or 0.
 * Offsets are validated as in flare_encode; workspace must hold
 * flare_encode_bwd_workspace_size() bytes, 16-byte aligned.  For bf16 with
 * D in {64,128} and M in {32,64,128,256}, or D = 16 and M in {32,64,128}, the
 * matrix-core path runs; it needs
 * Q, K, V, dZ, dQ, dK, dV 16-byte aligned (else FLARE_EINVAL) and sums dQ over
 * token chunks in a fixed order, so results are bitwise reproducible.
 * For bf16 with M = 256 and D = 128 the query gradient runs on a second
 * non-blocking stream of the same device, which the library creates on first
 * use and keeps until the process ends, forked from and joined back to
 * `stream` with events: every result is ordered on `stream` as if all of the
 * work ran there, and a graph captured on `stream` takes in both branches
 * (make one eager call first, so that the stream is not created during the
 * capture).  Calls on different streams of one device share that second
 * stream, which orders their query-gradient kernels one after the other.
 */
flare_status flare_encode_bwd(flare_dtype dtype, int B, int H, int N, int M, int D,
                              const void* Q, int64_t q_batch_stride, const void* K, const void* V,
                              int R, const int64_t* offsets, const uint8_t* mask, float scale,
                              const float* Z, const float* L, const void* dZ,
                              float* dQ, void* dK, void* dV, void* dQ_cast, int flags,
                              void* workspace, size_t workspace_bytes, flare_stream_t stream);

/* flags of flare_encode_bwd (bitwise or).  The FLARE++ backward paragraph adds the
 * decoder's contributions to the encoder's: with these the encoder backward adds into
 * gradients that a preceding flare_decode_bwd (or flare_encode_bwd) wrote.  With the
 * projections of the query-synthesis encoder tied to K and V (the shared-projection
 * variant of [FLARE++], paragraph on the cost of the extra projections), that encoder's
 * key and value gradients add into those of the physical-value encoder.  Accumulating
 * calls leave the rows of masked tokens as they were. */
#define FLARE_BWD_ACCUMULATE_DQ 1   /* dQ += (instead of dQ =) */
#define FLARE_BWD_ACCUMULATE_DK 2   /* dK += (instead of dK =) */
#define FLARE_BWD_ACCUMULATE_DV 4   /* dV += (instead of dV =) */

/* Bytes of device workspace flare_decode_bwd needs (masked != 0 when a token mask
 * will be passed). */
size_t flare_decode_bwd_workspace_size(flare_dtype dtype, int B, int H, int N, int M, int D,
                                       int masked);

/*
 * flare_decode_bwd -- gradients of sum(dY * Y) for Y = flare_decode(Xq, Klat, Z) ([FLARE++],
 * FLARE++ backward paragraph: each token's local decoder contributes to the gradients of
 * the replicated latents, summed over the tokens):
 *     A[n,m]   = softmax_m(scale Xq[n].Klat[m])      dA[n,m] = dY[n].Z[m]
 *     delta[n] = sum_m A[n,m] dA[n,m]                dT = A (dA - delta)
 *     dXq[n,:] = scale sum_m dT[n,m] Klat[m,:]       dKlat[m,:] = scale sum_n dT[n,m] Xq[n,:]
 *     dZ[m,:]  = sum_n A[n,m] dY[n,:]
 * Xq, dY, dXq: [B,H,N,D] in dtype.  Klat: [H,M,D] (klat_batch_stride 0) or [B,H,M,D].
 * Z: [B,H,M,D] float.  dKlat, dZ: [B,H,M,D] float, one slice per batch even when Klat is
 * replicated.  dZ_cast (nullable): dZ also written in dtype (the dZ a following
 * flare_encode_bwd takes).  token_mask (nullable, [B,N] uint8): tokens with 0 take no part
 * (their Y is 0): dXq rows written as 0, no contribution to dKlat or dZ.
 * All pointers are device pointers owned by the caller; workspace must hold
 * flare_decode_bwd_workspace_size() bytes, 16-byte aligned.  Shapes as flare_decode
 * (M <= 256).  For bf16 with D in {16,64,128} and M in {32,64,128} the matrix-core path runs;
 * it needs every tensor 16-byte aligned (else FLARE_EINVAL) and sums the latent gradients
 * over token chunks in a fixed order (bitwise reproducible).
 */
flare_status flare_decode_bwd(flare_dtype dtype, int B, int H, int N, int M, int D,
                              const void* Xq, const void* Klat, int64_t klat_batch_stride,
                              const float* Z, const uint8_t* token_mask, float scale,
                              const void* dY, void* dXq, float* dKlat, float* dZ, void* dZ_cast,
                              void* workspace, size_t workspace_bytes, flare_stream_t stream);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* flare_last_error(void);

/* Library version string. */
const char* flare_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLARE_H */
