/*
 * h3attn.h -- C ABI of the MI355X (gfx950) causal grouped-query attention
 * forward.
 *
 * The operation.  The h3.c issue "Qwen text encoder: sequence exceeds Metal
 * threadgroup memory with reference video + ref images (>=150 frames)" traces
 * a failure of the text encoder's bf16 causal GQA ("Error" section) to a kernel
 * that kept a whole causal score row of the sequence in threadgroup memory, and
 * proposes tiling the score computation so that on-chip memory holds one tile
 * at a time ("Suggested fix directions").  This library computes that
 * operation with an on-chip footprint that does not depend on the sequence
 * length: for every query token i and query head h,
 *
 *     g        = h / (Hq / Hkv)                   query heads g*G..g*G+G-1 share KV head g
 *     x_j      = softmax_scale * <Q[i,h,:], K[j,g,:]>,   j = 0..i   (diagonal included)
 *     O[i,h,:] = sum_j softmax_j(x) * V[j,g,:]
 *     LSE[h,i] = log(sum_j exp(x_j))              natural log of the scaled scores
 *
 * Arithmetic: bf16 products with fp32 accumulation; the softmax weights are
 * rounded to bf16 before they multiply V; O is rounded to bf16 (nearest even).
 *
 * Conventions shared by every entry point:
 *   - Tensors are DEVICE pointers (memory the caller allocated on the current
 *     HIP device), dense and row-major in the shapes given; the caller owns
 *     them.  The library allocates no device memory (the fixed scratch array
 *     of h3attn_gqa_causal_splitkv_fwd_noalloc is part of its code object) and
 *     keeps no per-call state.
 *   - The call enqueues work on `hip_stream` (NULL: the null stream) and
 *     returns without waiting; the caller synchronises.  (The packed call's
 *     opt-in offsets check, H3ATTN_CHECK_CU_SEQLENS=1, waits for its own small
 *     copy of the offsets.)
 *   - Arguments are checked on the host before any device work.  On any
 *     nonzero status no kernel was enqueued and no output byte was written.
 *   - There is no limit on the sequence length other than 32-bit indexing:
 *     tokens * Hq * D < 2^31.  There is no capacity error.
 *   - Calls into the library from several host threads are safe.
 */
#ifndef H3ATTN_H
#define H3ATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define H3ATTN_API __attribute__((visibility("default")))
#else
#define H3ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
  H3ATTN_OK = 0,
  H3ATTN_ERR_NULL = 1,        /* a required pointer is NULL (tensors of a nonempty call, offsets) */
  H3ATTN_ERR_SHAPE = 2,       /* negative size, Hq not a multiple of Hkv, offsets inconsistent,
                                 or tokens * Hq * D >= 2^31 */
  H3ATTN_ERR_UNSUPPORTED = 3, /* head dim not 64 or 128, group size Hq/Hkv not 1, 2, 4 or 8,
                                 or unknown flag bits */
  H3ATTN_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  H3ATTN_ERR_SCALE = 5,       /* softmax_scale not finite or not > 0 */
  H3ATTN_ERR_LAUNCH = 6,      /* the HIP kernel launch failed (hipGetLastError) */
  H3ATTN_ERR_DEVICE = 7,      /* no usable gfx950 device is current */
  H3ATTN_ERR_WORKSPACE = 8    /* split-KV workspace NULL, not 256-byte aligned, or too small */
} h3attn_status;

/* Largest num_splits the split-KV entry point accepts. */
#define H3ATTN_MAX_SPLITS 64

/*
 * Fixed-length causal GQA forward over one sequence of S tokens.
 *
 *   q    [S, Hq,  D] bf16   (input)
 *   k    [S, Hkv, D] bf16   (input)
 *   v    [S, Hkv, D] bf16   (input)
 *   o    [S, Hq,  D] bf16   (output)
 *   lse  [Hq, S]     fp32   (output; may be NULL when the caller does not need it)
 *
 * S >= 0 (S == 0 is a no-op returning H3ATTN_OK; the tensor pointers may then
 * be NULL); Hq % Hkv == 0 with
 * Hq / Hkv in {1, 2, 4, 8}; D in {64, 128}; softmax_scale finite and > 0
 * (usually 1/sqrt(D)).  q, k, v, o and lse must not overlap.
 * hip_stream is a hipStream_t (NULL: the null stream).
 */
H3ATTN_API int h3attn_gqa_causal_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                          int S, int Hq, int Hkv, int D, float softmax_scale, void* hip_stream);

/* Flags of h3attn_gqa_fwd. */
#define H3ATTN_NONCAUSAL 1    /* every query attends to all S keys (no causal mask) */
#define H3ATTN_O_HEAD_MAJOR 2 /* o is [Hq, S, D] instead of [S, Hq, D] */

/*
 * GQA forward over one sequence with options.  With flags == 0 it is exactly
 * h3attn_gqa_causal_fwd.  H3ATTN_NONCAUSAL drops the causal mask: the
 * bidirectional attention of the video DiT that runs after the encoder (the
 * h3.c project README's SDPA; the vpipe issue "0.1.29: MiniMax-H3 bf16 refused on
 * a 64 GB Mac ...", whose logs show 19316- and 34121-row forwards) -- x_j over all
 * j = 0 .. S-1, LSE over all S keys.
 * H3ATTN_O_HEAD_MAJOR writes o head-major, [Hq, S, D] (the README's profiling
 * notes leave the SDPA output in [head, row, dimension] order); lse is [Hq, S]
 * either way.
 * Arguments, checks and errors as h3attn_gqa_causal_fwd; unknown flag bits return
 * H3ATTN_ERR_UNSUPPORTED.
 */
H3ATTN_API int h3attn_gqa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int S, int Hq, int Hkv, int D, float softmax_scale, int flags,
                              void* hip_stream);

/*
 * Packed variable-length causal GQA forward: num_seqs independent sequences
 * concatenated along the token axis.  Positions are local to each sequence and
 * no query attends to another sequence's keys.  The issue's table of runs
 * (section "Systematic single-variable experiments") lists the failing encoder
 * lengths 8184, 8199, 8510 and 10231 tokens; one call with those four sequences
 * packed (35124 tokens) serves them all.
 *
 *   q    [T, Hq,  D] bf16   k, v [T, Hkv, D] bf16   o [T, Hq, D] bf16
 *   lse  [Hq, T] fp32, indexed by packed token (may be NULL)
 *   cu_seqlens  DEVICE int32[num_seqs + 1]: cu[0] = 0, non-decreasing,
 *               cu[num_seqs] = T = total_tokens.  Sequence s holds packed
 *               tokens cu[s] .. cu[s+1]-1; empty sequences are allowed.
 *   max_seqlen  an upper bound on cu[s+1] - cu[s] over all s.
 *
 * The offsets live on the device and are not read on the host.  The kernel
 * clamps each sequence to [0, T] and to max_seqlen, so invalid offsets give
 * unspecified (but in-bounds) results, never an out-of-bounds access; in
 * particular the rows of a sequence longer than max_seqlen past its first
 * max_seqlen tokens are not written.  total_tokens == 0 is a no-op (tensor
 * pointers may then be NULL); so is max_seqlen == 0.
 *
 * Debug check: with the environment variable H3ATTN_CHECK_CU_SEQLENS set to 1
 * when the call is made, the call first copies cu_seqlens to the host (on
 * hip_stream, waiting for the copy to finish) and validates it with
 * h3attn_check_cu_seqlens; an offset table that fails the check returns
 * H3ATTN_ERR_SHAPE and launches nothing, a failed copy H3ATTN_ERR_LAUNCH.
 */
H3ATTN_API int h3attn_gqa_causal_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                 int max_seqlen, int Hq, int Hkv, int D, float softmax_scale,
                                 void* hip_stream);

/*
 * Host-side validation of a packed batch's offsets (no GPU work): cu_seqlens_host
 * is a HOST int32[num_seqs + 1].  Returns H3ATTN_OK when cu[0] = 0, the offsets
 * do not decrease, cu[num_seqs] = total_tokens and every length cu[s+1] - cu[s]
 * is at most max_seqlen; H3ATTN_ERR_NULL for a NULL table with num_seqs > 0;
 * H3ATTN_ERR_SHAPE otherwise (also for negative counts).  This is the check the
 * varlen forward runs under H3ATTN_CHECK_CU_SEQLENS=1.
 */
H3ATTN_API int h3attn_check_cu_seqlens(const int32_t* cu_seqlens_host, int num_seqs,
                                       int total_tokens, int max_seqlen);

/*
 * Split-KV (multi-dispatch) causal GQA forward over one sequence: the first fix
 * direction of the issue ("Suggested fix directions": the score computation split
 * across several dispatches with intermediate results in global memory).
 *
 * The query tokens are cut into blocks (32 tokens for G = 8; 256/G in general), and the
 * causal KV range of each block, ceil(min(block end, S) / 64) tiles of 64 keys, into
 * num_splits contiguous ranges of near-equal length: split c of a block with n tiles
 * covers tiles [floor(n*c/num_splits), floor(n*(c+1)/num_splits)).  A first kernel
 * writes, for every (split, token, head), the attention over that split's keys --
 * O_c normalised over those keys (fp32) and LSE_c (fp32, -inf when the row saw none)
 * -- into the workspace; a second kernel, on the same stream, combines them:
 *     LSE = log(sum_c exp(LSE_c)),   O = sum_c exp(LSE_c - LSE) * O_c   (rounded to bf16).
 * The result is the same function as h3attn_gqa_causal_fwd; only rounding differs.
 *
 *   q, k, v, o, lse, S, Hq, Hkv, D, softmax_scale, hip_stream: as h3attn_gqa_causal_fwd.
 *   num_splits       1 .. H3ATTN_MAX_SPLITS (else H3ATTN_ERR_SHAPE).
 *   workspace        DEVICE memory the caller allocated, 256-byte aligned, at least
 *                    h3attn_gqa_causal_splitkv_workspace_bytes(S, Hq, D, num_splits)
 *                    bytes (else H3ATTN_ERR_WORKSPACE); contents need no
 *                    initialisation and are left undefined.  The library allocates
 *                    nothing.  Two calls in flight must not share a workspace.
 *   workspace_bytes  its size.
 * S == 0 is a no-op (pointers may then be NULL).
 */
H3ATTN_API int h3attn_gqa_causal_splitkv_fwd(const void* q, const void* k, const void* v,
                                             void* o, float* lse, int S, int Hq, int Hkv,
                                             int D, float softmax_scale, int num_splits,
                                             void* workspace, size_t workspace_bytes,
                                             void* hip_stream);

/* Size of the fixed device scratch array h3attn_gqa_causal_splitkv_fwd_noalloc uses
 * (64 MiB, one copy per GPU the library runs on, held until the process ends). */
#define H3ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): h3attn_gqa_causal_splitkv_fwd with
 * the workspace taken from a fixed array inside the library instead of from the
 * caller.  Same arguments, checks and results as h3attn_gqa_causal_splitkv_fwd,
 * without workspace / workspace_bytes.
 *
 * The call allocates nothing (no hipMalloc, no allocating library routine).  Its
 * first call on a device looks up that device's copy of the array once.  A call whose
 * workspace need, h3attn_gqa_causal_splitkv_workspace_bytes(S, Hq, D, num_splits),
 * exceeds H3ATTN_NOALLOC_SCRATCH_BYTES returns H3ATTN_ERR_WORKSPACE and launches
 * nothing; H3ATTN_ERR_DEVICE if the array cannot be looked up.  Every call on one GPU
 * uses the same array: calls that overlap on one GPU (different streams, or different
 * host threads) race on it and give undefined results; calls in order on one stream
 * are safe.  The array keeps whatever the last call left; no call relies on its
 * contents.
 */
H3ATTN_API int h3attn_gqa_causal_splitkv_fwd_noalloc(const void* q, const void* k,
                                                     const void* v, void* o, float* lse,
                                                     int S, int Hq, int Hkv, int D,
                                                     float softmax_scale, int num_splits,
                                                     void* hip_stream);

/* Workspace bytes h3attn_gqa_causal_splitkv_fwd needs: partial O, fp32
 * [num_splits, S, Hq, D], then partial LSE, fp32 [num_splits, Hq, S], at the next
 * 256-byte boundary.  0 for invalid arguments. */
H3ATTN_API size_t h3attn_gqa_causal_splitkv_workspace_bytes(int S, int Hq, int D,
                                                            int num_splits);

/* Flag of h3attn_qk_norm_rope. */
#define H3ATTN_PROLOGUE_ROPE 1  /* apply the rotary position embedding */

/*
 * Q/K prologue: the step before attention that the h3.c project README runs as a
 * fused QK-normalization / RoPE kernel ("Checkpoint layout and media pipeline").  The
 * pages give no formulas; this computes the Qwen-family convention on every
 * (token, head) row x[0..D) of q [S, Hq, D] and k [S, Hkv, D] (bf16):
 *   RMS norm (when the tensor's weight pointer is non-NULL):
 *       y_d = x_d / sqrt(mean_d(x_d^2) + eps) * w_d,   w: D bf16 values
 *   rotary embedding (flags & H3ATTN_PROLOGUE_ROPE), rotate-half pairs (i, i+D/2):
 *       a_i = p * rope_theta^(-2i/D),  p = positions[token] (int32 [S] on the device)
 *             or the token index when positions == NULL
 *       z_i = y_i cos a_i - y_{i+D/2} sin a_i,   z_{i+D/2} = y_{i+D/2} cos a_i + y_i sin a_i
 * in fp32 (angles, cos and sin in fp64) with one bf16 rounding per output element.
 * q_out / k_out have q's / k's shapes and may equal q / k (in place).  D in {64, 128}.
 * Hq may be 0 (K only, as before h3attn_gqa_causal_qnorm_rope_fwd); q and q_out may then
 * be NULL.
 * Pointers: tensors and weights 16-byte aligned, positions 4-byte aligned,
 * all DEVICE memory.  eps must be finite and >= 0 when a weight is given (a row of
 * zeros with eps = 0 gives NaN, as the definition does); rope_theta finite and > 0 when
 * RoPE is on (else H3ATTN_ERR_SCALE).  S == 0 is a no-op.  HBM-bound: it reads and
 * writes every Q and K element once.
 */
H3ATTN_API int h3attn_qk_norm_rope(const void* q, const void* k, void* q_out, void* k_out, int S,
                                   int Hq, int Hkv, int D, const void* q_norm_weight,
                                   const void* k_norm_weight, float eps, float rope_theta,
                                   const int32_t* positions, int flags, void* hip_stream);

/*
 * Fixed-length causal GQA forward whose Q goes through the Q half of the prologue above
 * (the README's fused QK-normalization / RoPE step) inside the attention kernel, as it is
 * loaded: Q is read from HBM once and no normalised copy is written.  K must already be
 * normalised and rotated, e.g. by h3attn_qk_norm_rope with Hq = 0.
 *
 *   q [S, Hq, D], k and v [S, Hkv, D] bf16 -> o [S, Hq, D] bf16, lse [Hq, S] fp32 (or NULL)
 *   q_norm_weight  [D] bf16 or NULL (no norm); eps as in h3attn_qk_norm_rope
 *   flags          H3ATTN_PROLOGUE_ROPE: rotary embedding with rope_theta and positions
 *                  (int32 [S] or NULL: the token index), as in h3attn_qk_norm_rope
 *
 * The result is the causal forward of h3attn_gqa_causal_fwd applied to the bf16 output
 * q_out that h3attn_qk_norm_rope would produce, up to rounding: the angles are reduced
 * modulo 2 pi in fp64 and their cos / sin taken in fp32, and the row's sum of squares is
 * added in another order.  Checks and errors as h3attn_gqa_causal_fwd and
 * h3attn_qk_norm_rope; D = 128 with Hq == Hkv is not offered (H3ATTN_ERR_UNSUPPORTED).
 */
H3ATTN_API int h3attn_gqa_causal_qnorm_rope_fwd(const void* q, const void* k, const void* v,
                                                void* o, float* lse, int S, int Hq, int Hkv,
                                                int D, float softmax_scale,
                                                const void* q_norm_weight, float eps,
                                                float rope_theta, const int32_t* positions,
                                                int flags, void* hip_stream);

/*
 * Reference-video token pooling, the second fix direction of the issue ("Suggested fix
 * directions": pool or down-sample the video tokens before the text encoder so the
 * sequence gets shorter).  x [T, C] bf16 (token embeddings) -> out [T_out, C] bf16:
 * inside the span [begin, end) every `factor` consecutive tokens are replaced by their
 * mean (fp32 sum, one bf16 rounding; a shorter last group averages what it has); the
 * tokens before and after the span are copied.  T_out = T - L + ceil(L / factor),
 * L = end - begin (h3attn_pool_tokens_out_len).  0 <= begin <= end <= T, factor >= 1
 * (else H3ATTN_ERR_SHAPE); C a multiple of 8 (else H3ATTN_ERR_UNSUPPORTED); x, out
 * DEVICE memory, 16-byte aligned, not overlapping.  T_out == 0 is a no-op.
 */
H3ATTN_API int h3attn_pool_tokens(const void* x, void* out, int T, int C, int begin, int end,
                                  int factor, void* hip_stream);

/* Output length of h3attn_pool_tokens, or -1 for invalid arguments. */
H3ATTN_API int h3attn_pool_tokens_out_len(int T, int begin, int end, int factor);

/*
 * Calibration loops (not a step of the attention): the sustained rate of the two
 * resources the attention kernel's inner loop is built from, measured on the running GPU
 * at the clock it holds, so that the kernel's throughput can be set against what the chip
 * reaches as well as against its published peak.
 *   kind H3ATTN_CALIB_MFMA: each wave issues iters * 8 v_mfma_f32_32x32x16_bf16 (32768
 *     flop each) on fixed pseudo-random bf16 operands (eight A and eight B fragments, so
 *     consecutive MFMAs differ in both) into four accumulators;
 *   kind H3ATTN_CALIB_MFMA_ZERO: the same MFMA loop on all-zero operands (a datapath that
 *     does not toggle draws less power; the clock difference to H3ATTN_CALIB_MFMA shows
 *     how much the power limit sets the rate on real data);
 *   kind H3ATTN_CALIB_EXP: each wave issues iters * 16 v_exp_f32 on sixteen independent
 *     fp32 values;
 *   kind H3ATTN_CALIB_MFMA_PAIRED: the H3ATTN_CALIB_MFMA loop in workgroups that reserve
 *     64 KB of LDS instead of 96 KB, so that a compute unit holds two: with n_workgroups
 *     twice the number of compute units every SIMD runs two MFMA waves.
 * n_workgroups workgroups of 256 threads (four waves); except for
 * H3ATTN_CALIB_MFMA_PAIRED each reserves 96 KB of LDS, so no compute unit holds two of
 * them: with n_workgroups equal to the number of compute units every SIMD runs one wave,
 * the attention kernel's occupancy.
 *   stamps  DEVICE uint64 [n_workgroups * 4][4]: per wave, the shader-clock counter
 *           (s_memtime) before and after its loop, then the constant-rate counter
 *           (s_memrealtime) before and after;
 *   sink    DEVICE float [n_workgroups * 256]: one value per thread that keeps the loop's
 *           results live (no meaning otherwise);
 *   wall_clock_khz  HOST int or NULL: receives the rate of the constant-rate counter.
 * 1 <= n_workgroups <= 65535 and 1 <= iters <= 2^24 (else H3ATTN_ERR_SHAPE); another kind
 * is H3ATTN_ERR_UNSUPPORTED; stamps and sink non-NULL (H3ATTN_ERR_NULL), 8- and 4-byte
 * aligned (H3ATTN_ERR_ALIGN).  Enqueued on hip_stream like the other calls.
 */
#define H3ATTN_CALIB_MFMA 0
#define H3ATTN_CALIB_EXP 1
#define H3ATTN_CALIB_MFMA_ZERO 2
#define H3ATTN_CALIB_MFMA_PAIRED 3
H3ATTN_API int h3attn_calib_loop(int kind, int n_workgroups, int iters, uint64_t* stamps,
                                 float* sink, int* wall_clock_khz, void* hip_stream);

/* Static, NUL-terminated description of a status code (never NULL). */
H3ATTN_API const char* h3attn_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
H3ATTN_API int h3attn_version(void);

/* Size in bytes of the LDS (on-chip shared memory) one workgroup of the kernel
 * instance for head dim D and group size G uses, or -1 if the pair is
 * unsupported.  It does not depend on the sequence length. */
H3ATTN_API int h3attn_lds_bytes(int D, int G);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H */
