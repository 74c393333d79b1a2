/*
 * path_attn.h -- C ABI of libpath_attn: the causal PaTH attention forward pass
 * (optionally with the PaTH-FoX forget gate) on one AMD Instinct MI355X
 * (gfx950) GPU.
 *
 * The operation (PaTH discussion slides for arXiv:2505.16381v2, frame "PaTH
 * inserts a learned transformation along every path", paper Sec. 2.2; frame
 * "FoX adds a separate mechanism for forgetting"; the authors' response page,
 * "Implementation detail", for the scale and the -inf causal mask): for each
 * (batch b, head h) and query position i,
 *
 *     H_t   = I - beta_t w_t w_t^T
 *     c_ij  = k_j^T H_{j+1} H_{j+2} ... H_i q_i            (j <= i; c_ii = k_i.q_i)
 *     s_ij  = c_ij / sqrt(d) + sum_{s=j+1..i} log f_s      (gate term only with logf)
 *     o_i   = sum_{j<=i} softmax_j(s_ij) v_j
 *     lse_i = ln sum_{j<=i} exp(s_ij)
 *
 * The gate term is added outside the 1/sqrt(d) scale (the gate product sits
 * outside the exponential on the FoX frame).  w_t and beta_t are used exactly
 * as given: the library does not renormalise w_t nor clip beta_t.  The factors
 * H_0 and f_0 never enter a logit.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, caller-owned DEVICE pointers:
 *       q, k, v, w, out : [B, H, T, d]  elements of `dtype`
 *       beta, logf, lse : [B, H, T]     float32
 *   - dtype: PATH_ATTN_F32 (float32 storage, float32 arithmetic throughout)
 *            or PATH_ATTN_BF16 (bfloat16 storage; products on bf16 matrix
 *            cores with float32 accumulation; chunk preparation in float32).
 *   - Supported shapes: d in {64, 128}; T >= 1; B, H >= 1; B*H*Tp*d < 2^31
 *     with Tp = T rounded up to a multiple of 64 (the chunk length).  A T that
 *     is not a multiple of 64 is run at Tp with padded tokens whose factor is
 *     the identity (beta = 0, w = 0) and whose q, k, v and gate are zero; they
 *     come after every real token, so no real logit changes (they enter no
 *     path H_{j+1}...H_i with i < T, and the causal mask hides them).  The
 *     inputs are then copied into zero-padded staging inside the workspace and
 *     the first T rows of out and lse copied back, which costs extra traffic;
 *     a multiple of 64 needs no staging.  The authors' reference listing needs
 *     L % BT == 0; padding with identity factors is this library's reading.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: they enqueue kernels and return; results are valid once
 *     the caller has synchronised the stream.  The library keeps no pointer
 *     after a call returns and allocates no memory: all scratch space is the
 *     caller's `workspace` (path_attn_fwd_noalloc alone uses a fixed array of
 *     the library instead).  Concurrent calls on different streams must use
 *     different workspaces.
 *   - Pointers must be 16-byte aligned, the workspace 256-byte aligned.
 *   - Errors: argument checks run before any HIP call; on failure nothing is
 *     launched and a status below is returned.  Numerical contents are not
 *     checked (NaN/Inf propagate).
 */
#ifndef PATH_ATTN_H
#define PATH_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define PATH_ATTN_OK 0
#define PATH_ATTN_EINVAL 1      /* null pointer, size <= 0, bad dtype, misaligned
                                   pointer, or workspace too small */
#define PATH_ATTN_EUNSUPPORTED 2 /* d not in {64, 128}, the problem exceeds
                                   32-bit element indexing, or a prefill
                                   length / chunk unpack that is not a
                                   multiple of 64 */
#define PATH_ATTN_EHIP 3        /* a HIP launch reported an error */

/* Storage dtypes of q, k, v, w and out. */
#define PATH_ATTN_F32 0
#define PATH_ATTN_BF16 1

/* Flags of path_attn_stream_ex. */
#define PATH_ATTN_NO_SKIP 1u    /* compute every key block, even those the exact
                                   forget-gate skip would leave out */
#define PATH_ATTN_PRECISE 2u    /* bf16: cross-chunk logits from the running
                                   query tile as a bf16 hi + lo pair (for sharp
                                   attention; one more product per logit
                                   block); no effect for float32 */

/*
 * Workspace size in bytes that path_attn_fwd / path_attn_chunk_prep need for
 * this problem, or 0 if the arguments are invalid or unsupported.  The size
 * is linear in B*H*T: per 64-token chunk it holds the boundary-adjusted
 * queries (float32), the transformed keys, the values and the chunk transform
 * in the matrix-core operand order, the diagonal-block logits (float32) and
 * two float32 bounds used with the forget gate; per token, the forget-gate
 * prefix (float32) and, for bf16, the rounding remainders of the transformed
 * keys (written only for PATH_ATTN_PRECISE).  When T is not a multiple of
 * 64, it also holds the zero-padded staging copies of q, k, v, w, beta,
 * logf, out and lse.
 */
size_t path_attn_workspace_bytes(int B, int H, int T, int d, int dtype);

/*
 * Forward pass.  logf may be NULL (plain PaTH); otherwise it holds log f_t
 * (values <= 0 for gates in (0, 1]).  out receives o in `dtype`, rounded to
 * nearest even; lse receives the natural-log normaliser in float32.
 *
 * Launches, in order on `stream`: the forget-gate prefix sum (only with
 * logf), the chunk preparation (the UT form of each 64-token chunk: PaTH
 * slides, frames "A triangular representation makes paths computable" and
 * "Backup: fix orientation before implementing UT products", paper Secs.
 * 3.1-3.3), and the right-to-left streaming scan over key chunks with an
 * online softmax (frame "A right-to-left scan accumulates cross-block paths",
 * paper Sec. 3.3).
 *
 * Returns PATH_ATTN_OK or an error status (see above).
 */
int path_attn_fwd(const void *q, const void *k, const void *v, const void *w,
                  const float *beta, const float *logf, void *out, float *lse,
                  int B, int H, int T, int d, int dtype, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * path_attn_fwd with a softmax scale and flags.  scale > 0 multiplies the
 * path logits c_ij in place of 1/sqrt(d) (the authors' listing passes
 * `scale` as an argument); scale = 0 selects 1/sqrt(d).  A negative,
 * infinite or NaN scale is EINVAL (the scan takes each block's maximum on the
 * raw scores, which needs scale > 0).  flags: 0, or PATH_ATTN_NO_SKIP and/or
 * PATH_ATTN_PRECISE.  PATH_ATTN_PRECISE (bf16) feeds the S product of every
 * cross-chunk block the running query tile as a bf16 hi + lo pair instead of
 * its bf16 rounding, and the transformed keys ->K likewise (hi from the
 * operand block, lo from remainders the chunk preparation then also
 * writes): the two roundings otherwise set a relative error of about 2^-9 on
 * those logits, which matters for sharp attention (large logits).  It runs
 * the 32-query scan kernel with three products per S tile, slower than the
 * default.
 * path_attn_fwd(...) == path_attn_fwd_ex(..., 0.0f, 0, ...).
 */
int path_attn_fwd_ex(const void *q, const void *k, const void *v, const void *w,
                     const float *beta, const float *logf, void *out, float *lse,
                     int B, int H, int T, int d, int dtype, float scale,
                     unsigned flags, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Partial PaTH (the authors' response page, remark on applying PaTH to a
 * subset of the head dimensions for speed): the factors act on the leading
 * d_path coordinates only, and the other d - d_path coordinates carry a plain
 * dot product,
 *     H_t = I - beta_t w~_t w~_t^T,  w~_t = (w_t[0 .. d_path), 0, ..., 0),
 * i.e. the definition at the top of this header with w_t's trailing
 * coordinates taken as zero (they are not read).  The chunk transforms are
 * then d_path x d_path, so the chunk preparation's products with W and the
 * scan's transition product shrink.  d_path = d is path_attn_fwd_ex;
 * d_path = d / 2 is the other supported value (PATH_ATTN_EUNSUPPORTED for
 * any other d_path in (0, d]; EINVAL outside it).  A workspace of
 * path_attn_workspace_bytes(B, H, T, d, dtype) bytes suffices.  Other
 * arguments, results and errors as for path_attn_fwd_ex.
 */
int path_attn_fwd_partial(const void *q, const void *k, const void *v, const void *w,
                          const float *beta, const float *logf, void *out, float *lse,
                          int B, int H, int T, int d, int d_path, int dtype, float scale,
                          unsigned flags, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * path_attn_fwd_ex without a caller workspace.  The workspace is a fixed
 * array of PATH_ATTN_NOALLOC_MAX_BYTES in the library's device memory: each
 * GPU the library's code is loaded on (its first use there, by any entry
 * point) holds one copy until the process ends; the call allocates nothing.
 * A problem whose workspace (path_attn_workspace_bytes) exceeds that size is
 * EINVAL: 64 MiB holds about 80,000 token-heads (B*H*T) at d = 64 and about
 * 38,000 at d = 128 in bf16.  The GPU is the stream's (the current device for
 * a NULL stream); the array's address there is looked up once per device on
 * the first call (EHIP if that lookup fails).  Every call on one GPU uses the
 * same array: calls that overlap on one GPU (concurrent streams or host
 * threads) race and give wrong results, so the caller must order them.
 * Other arguments, results and errors as for path_attn_fwd_ex.
 */
#define PATH_ATTN_NOALLOC_MAX_BYTES (64u << 20)
int path_attn_fwd_noalloc(const void *q, const void *k, const void *v, const void *w,
                          const float *beta, const float *logf, void *out, float *lse,
                          int B, int H, int T, int d, int dtype, float scale,
                          unsigned flags, void *stream);

/*
 * The two phases of path_attn_fwd, for callers that time or schedule them
 * separately.  path_attn_prepare enqueues the forget-gate prefix (with logf)
 * and the chunk preparation into `workspace`; path_attn_stream enqueues the
 * streaming scan that reads that workspace and writes out and lse.  The
 * stream phase must see a workspace prepared by path_attn_prepare with the
 * same B, H, T, d, dtype (and use_gate = 1 exactly when logf was non-NULL),
 * ordered before it on the stream; path_attn_fwd is exactly
 * path_attn_prepare followed by path_attn_stream.
 */
int path_attn_prepare(const void *q, const void *k, const void *v,
                      const void *w, const float *beta, const float *logf,
                      int B, int H, int T, int d, int dtype, void *workspace,
                      size_t workspace_bytes, void *stream);
int path_attn_stream(const void *workspace, size_t workspace_bytes,
                     int use_gate, void *out, float *lse, int B, int H, int T,
                     int d, int dtype, void *stream);

/*
 * path_attn_stream with options.  With the forget gate (use_gate = 1) the
 * scan leaves out the S, softmax and P.V work of a key block when a bound on
 * every logit of the block (the query tile's norm times the chunk's largest
 * key norm, times the scale, plus the chunk's largest gate term) lies more
 * than 160 (log2 units) below every running max of the wave: each weight of
 * such a block is then below 2^-160, exactly zero in float32, so the outputs
 * are the same bits as without the skip (up to the sign of an output element
 * that is exactly zero).  The gate makes far blocks vanish (FoX slides,
 * "FoX adds a separate mechanism for forgetting"); the skip itself is this
 * library's, not the pages'.  The chunk transitions are always applied.
 *
 * flags:   0 or PATH_ATTN_NO_SKIP (compute every block); PATH_ATTN_PRECISE
 *          is EINVAL here (it needs ->K's rounding remainders, which only
 *          the one-shot calls write: path_attn_fwd_ex, _partial, _varlen,
 *          _noalloc).
 * skipped: NULL, or a device counter (8-byte aligned) to which the scan adds
 *          the number of steps it skipped, one per wave and key block (a
 *          wave covers 32 queries, 64 for bf16 d = 64); the caller zeroes it.
 * scale:   as for path_attn_fwd_ex (0 selects 1/sqrt(d)).
 * Other arguments and errors as path_attn_stream; unknown flag bits give
 * PATH_ATTN_EINVAL.  path_attn_stream(...) == path_attn_stream_ex(..., 0.0f,
 * 0, NULL, ...), and path_attn_fwd uses the skip.
 */
int path_attn_stream_ex(const void *workspace, size_t workspace_bytes,
                        int use_gate, float scale, unsigned flags,
                        unsigned long long *skipped, void *out, float *lse,
                        int B, int H, int T, int d, int dtype, void *stream);

/*
 * Chunk preparation only, with its results unpacked into plain float32
 * arrays so that each quantity can be checked on its own.  For chunk c of
 * 64 tokens (rows w_t^T stacked in W, D = diag(beta), U = (I +
 * strictLower(D W W^T))^{-1} D):
 *     qa  [B,H,T,d]       <-Q = Q - lower(Q W^T) U W   (row i: H_first...H_i q_i)
 *     kb  [B,H,T,d]       ->K = K - (U strictLower(W K^T))^T W
 *                               (row j: H_last...H_{j+1} k_j)
 *     m   [B,H,T/64,d,d]  M = W^T U W   (so that H_first...H_last = I - M^T)
 *     al  [B,H,T/64,64,64] lower(Q K^T) - lower(Q W^T) U strictLower(W K^T)
 *                          (raw diagonal-block logits; entries above the
 *                           diagonal are unspecified)
 *     lam [B,H,T]         sum_{s=1..t} log f_s (only if logf and lam non-NULL;
 *                          f_0 never enters a logit and is left out)
 * kb and m are reported at the precision the streaming kernel consumes them
 * (bf16-rounded for PATH_ATTN_BF16).  Any of qa/kb/m/al/lam may be NULL.
 * Uses the same workspace as path_attn_fwd.  T must be a multiple of 64
 * (PATH_ATTN_EUNSUPPORTED otherwise).
 */
int path_attn_chunk_prep(const void *q, const void *k, const void *v,
                         const void *w, const float *beta, const float *logf,
                         float *qa, float *kb, float *m, float *al, float *lam,
                         int B, int H, int T, int d, int dtype, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * ------------------------------------------------------------------------
 * Decoding with in-place key refinement (PaTH slides, frame "Decoding
 * updates historical keys in place", paper Sec. 3.4, Eq. (1); the authors'
 * response page, "Inference Latency", on fusing the refinement into
 * flash-decoding).  When token t arrives, every cached key is reflected by
 * H_t:  k_j <- k_j - beta_t w_t (w_t . k_j) for j < t; then k_j . q_t equals
 * the path logit k_j^T H_{j+1} ... H_t q_t and the readout is ordinary
 * softmax attention over the refined keys and the new key k_t.  A prompt's
 * keys must first be aligned to its last position L-1:
 *     kcache[j] = H_{L-1} ... H_{j+1} k_j    (j < L; kcache[L-1] = k_{L-1}).
 *
 * Caches (caller-owned device memory, capacity T_cap positions per head):
 *     kcache [B, H, T_cap, d]  kc_dtype (PATH_ATTN_F32 or PATH_ATTN_BF16)
 *     vcache [B, H, T_cap, d]  dtype
 *     gcache [B, H, T_cap]     float64 Lambda_j = sum_{1<=s<=j} log f_s
 *                              (only with the forget gate; NULL otherwise)
 * Positions >= the current length are never read.  With kc_dtype =
 * PATH_ATTN_BF16 every refinement rounds the stored key to bf16 again, so the
 * error grows with the number of decode steps; PATH_ATTN_F32 keeps the
 * refined keys in float32.  The logits use the keys as stored.
 * ------------------------------------------------------------------------
 */

/* Workspace bytes of path_attn_prefill_cache, 0 for invalid arguments. */
size_t path_attn_prefill_workspace_bytes(int B, int H, int L, int d);

/*
 * Fill positions 0..L-1 of the caches from a prompt of length L (a multiple
 * of 64, 0 <= L <= T_cap): aligned keys (float32 arithmetic: per 64-token
 * chunk the UT form of the forward pass, then the products of the later
 * chunks' transforms applied right to left), values copied, and with logf
 * the gate prefix Lambda_j (float64).  k, v, w: [B, H, L, d] of dtype; beta,
 * logf: [B, H, L] float32 (logf may be NULL; gcache is then unused).
 * Tokens of a prompt beyond a multiple of 64 are fed with
 * path_attn_decode_step, which also returns their outputs.
 * Errors: EINVAL for null/misaligned pointers (16 bytes; workspace 256),
 * bad dtypes, L < 0, L > T_cap or a small workspace; EUNSUPPORTED for d not
 * in {64, 128}, L % 64 != 0 or B*H*T_cap*d >= 2^31; EHIP on a launch error.
 */
int path_attn_prefill_cache(const void *k, const void *v, const void *w,
                            const float *beta, const float *logf,
                            void *kcache, void *vcache, double *gcache, int B,
                            int H, int L, int T_cap, int d, int dtype,
                            int kc_dtype, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Workspace bytes of path_attn_decode_step (the partial softmax states of
 * the key splits of every head), 0 for invalid arguments.  The workspace needs
 * no initialisation and serves all steps of any cache of at most B*H heads
 * and T_cap positions.  Steps that share a workspace must not run
 * concurrently. */
size_t path_attn_decode_workspace_bytes(int B, int H, int T_cap, int d);

/*
 * One decode step at position t (0 <= t < T_cap) for all B*H heads.  The
 * caches must hold positions 0..t-1 aligned to t-1 (after a prefill of
 * length t, or after the step at t-1).  The step reflects cached keys
 * 0..t-1 by H_t in place, appends k_t, v_t (and Lambda_t = Lambda_{t-1} +
 * log f_t, Lambda_0 = 0) at position t, and writes
 *     out[b,h,:] = sum_{j<=t} softmax_j(s_tj) v_j        (dtype, RNE)
 *     lse[b,h]   = ln sum_{j<=t} exp(s_tj)                (float32)
 * with s_tj = scale * (k_j . q_t) + Lambda_t - Lambda_j (gate term only
 * with logf; scale as for path_attn_fwd_ex, 0 selects 1/sqrt(d)).  q, k, v, w, out: [B, H, d] of dtype; beta, logf, lse: [B, H]
 * float32.  Keys are split over blocks (512 per block, one block when t = 0),
 * each writing a partial softmax state into the workspace; a second kernel,
 * one block per head, merges them (ordered after the first by the stream).
 * Alignment: q, k, v, w, out and
 * the caches 16 bytes; beta, logf and lse 4 bytes (one value per head).
 * Errors as for path_attn_prefill_cache; t outside [0, T_cap) is EINVAL.
 */
int path_attn_decode_step(const void *q, const void *k, const void *v,
                          const void *w, const float *beta, const float *logf,
                          void *kcache, void *vcache, double *gcache, int t,
                          void *out, float *lse, int B, int H, int T_cap, int d,
                          int dtype, int kc_dtype, float scale, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * ------------------------------------------------------------------------
 * Backward pass.  The pages time forward plus backward (the authors'
 * response page, "Efficiency Evaluation" table) without giving the backward
 * algorithm; this library computes the exact gradients of the forward's
 * definition, blockwise over the same 64-token chunks (per-chunk UT
 * quantities of frames "A triangular representation makes paths computable"
 * and "Backup: fix orientation before implementing UT products", keys of
 * earlier chunks aligned chunk by chunk as in frame "Decoding updates
 * historical keys in place", a downward sweep over query chunks, then the
 * per-chunk adjoint of the UT formulas).  Precision: the per-chunk algebra
 * (the triangular solve, the UT quantities and their adjoint) is float32;
 * the quadratic products (logits, P.V, dP, dV, dQ, dK and the chunk
 * transitions of the key levels and of the key gradients) take operands of
 * the input dtype with float32 accumulation, so bf16 operands for
 * PATH_ATTN_BF16, as the forward's; running values are float32.
 * ------------------------------------------------------------------------
 */

/* Workspace bytes of path_attn_bwd, 0 for invalid or unsupported arguments:
 * the smallest workspace it accepts.  The quadratic part of the backward
 * walks the keys aligned to every later chunk (key levels, about
 * B*H*d*T^2/128 values in all); past 33 chunks of 64 tokens it runs in
 * windows of 16 query chunks, holding one window of levels, float32
 * checkpoints of the walk at the window boundaries and one window of dM
 * partials at a time, so the workspace grows as about T^1.5 next to linear
 * per-chunk terms: 3.91 GiB at B=2, H=16, T=16384, d=64 in bf16, 6.01 GiB at
 * B=4, H=8, T=8192, d=128 in bf16, 9.91 GiB at B=2, H=16, T=32768, d=64. */
size_t path_attn_bwd_workspace_bytes(int B, int H, int T, int d, int dtype);

/* Workspace bytes of path_attn_bwd with windows of `window` query chunks
 * (window <= 0: the whole sweep as one window, which stores every key level
 * and keeps the per-chunk matrices of the adjoint instead of computing them
 * again: 18.19 GiB at B=2, H=16, T=16384, d=64 in bf16).  Longer windows mean
 * fewer passes and restarts of the walk, so a faster backward (12.8 ms
 * instead of 15.0 ms at that shape on one MI355X).  path_attn_bwd runs one
 * window when
 * its workspace allows, else the longest of 128, 64, 32 and 16 query chunks
 * whose layout fits the workspace_bytes it is given.  0 for invalid
 * arguments. */
size_t path_attn_bwd_workspace_bytes_window(int B, int H, int T, int d, int dtype, int window);

/*
 * Gradients of  L = sum <dout, out> + sum <dlse, lse>  with respect to q, k,
 * v, w, beta and (with the gate) log f, for the forward of path_attn_fwd_ex
 * with the same inputs and scale.  out and lse must be that forward's
 * outputs (the softmax weights are rebuilt as exp(s - lse)).
 *   q, k, v, w, out, dout : [B, H, T, d] of dtype     (inputs)
 *   beta, logf, lse       : [B, H, T] float32         (inputs; logf may be NULL)
 *   dlse                  : [B, H, T] float32 or NULL (NULL = zero)
 *   dq, dk, dv, dw        : [B, H, T, d] of dtype     (outputs, overwritten)
 *   dbeta, dlogf          : [B, H, T] float32         (outputs; dlogf only with
 *                                                      logf, where it is required;
 *                                                      dlogf[.., 0] = 0 as f_0
 *                                                      enters no logit)
 * scale: as for path_attn_fwd_ex (0 selects 1/sqrt(d)).  With dtype
 * PATH_ATTN_BF16 the gradients are accumulated in float32 and rounded once
 * (RNE): the quadratic products take bf16 operands (the forward's), the
 * per-chunk algebra keeps float32 values and multiplies them as bf16 hi/lo
 * pairs (about 16 significant bits).
 * Any T >= 1: a T that is not a multiple of 64 is run at the next multiple
 * with padded tokens as in the forward (identity factors, zero q, k, v, dout,
 * dlse and gate, lse = 0), which contribute nothing to any gradient; the
 * inputs are then staged in the workspace and the first T rows of the
 * gradients copied back.  Every pointer 16-byte aligned, the workspace
 * 256-byte aligned; workspace_bytes at least path_attn_bwd_workspace_bytes
 * (a larger workspace selects longer windows of the sweep, see
 * path_attn_bwd_workspace_bytes_window; the gradients agree to float32
 * rounding either way).  Every sum is taken in a fixed order (no atomics):
 * two calls with the same inputs and workspace size give the same bits.
 * Errors: EINVAL for null or misaligned pointers, a bad dtype or scale,
 * logf without dlogf, or a small workspace; EUNSUPPORTED for d not in
 * {64, 128} or B*H*Tp*d >= 2^31; EHIP on a launch error.
 */
int path_attn_bwd(const void *q, const void *k, const void *v, const void *w,
                  const float *beta, const float *logf, const void *out,
                  const float *lse, const void *dout, const float *dlse,
                  void *dq, void *dk, void *dv, void *dw, float *dbeta,
                  float *dlogf, int B, int H, int T, int d, int dtype,
                  float scale, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * path_attn_bwd with flags: 0 or PATH_ATTN_NO_SKIP.  With the gate, the bf16
 * d = 128 backward leaves out every block of 32 keys and a query chunk whose
 * weights exp(s - lse) are exactly zero in float32, judged by the bound
 *     scale * max|Qa| * max|Khat| * 1.01 + max(Lambda_q - lse_q) - min Lambda_j + 1 < -112
 * over the block (the same reasoning as the forward's skip): its products
 * add only zeros, so the gradients are the same bits as with every block
 * computed (up to the sign of a zero).  PATH_ATTN_NO_SKIP computes every
 * block.  path_attn_bwd(...) == path_attn_bwd_ex(..., scale, 0, ...).
 */
int path_attn_bwd_ex(const void *q, const void *k, const void *v, const void *w,
                     const float *beta, const float *logf, const void *out,
                     const float *lse, const void *dout, const float *dlse,
                     void *dq, void *dk, void *dv, void *dw, float *dbeta,
                     float *dlogf, int B, int H, int T, int d, int dtype,
                     float scale, unsigned flags, void *workspace,
                     size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Strided and packed (variable-length) batches.
 *
 * The same operation as path_attn_fwd_ex / path_attn_bwd (definition at the
 * top of this header), with every tensor given as a view instead of a dense
 * [B, H, T, ...] array; the pages' own listing takes dense [B, H, L, D]
 * arrays of one length, so views and packing are this library's extension.
 *
 * A view row (b, h, t) of a tensor (d elements for q, k, v, w, out, dout and
 * the vector gradients; one float32 for beta, logf, lse, dlse, dbeta, dlogf)
 * starts at element
 *
 *     (off_b + t) * s_t + b * s_b + h * s_h        of that tensor's pointer,
 *
 * with off_b = cu_seqlens[b] for packed batches (cu_seqlens non-NULL) and 0
 * otherwise; the d elements of a row are contiguous.  Sequence b has
 * len_b = cu_seqlens[b+1] - cu_seqlens[b] tokens (T without cu_seqlens), and
 * its tokens t < len_b are attended causally among themselves only: each
 * sequence is its own path, with its own first factor and gate prefix, as
 * if it were run alone.
 *
 *   strides    : HOST array of 3 long long per tensor, (s_b, s_h, s_t) in
 *                elements of that tensor, in the tensor order stated below.
 *                A packed token-major tensor [total, H, d] has (0, d, H*d);
 *                a dense one [B, H, T, d] has (H*T*d, T*d, d); the strides of
 *                an absent optional tensor (logf, dlse, dlogf when NULL) are
 *                not read.
 *   cu_seqlens : DEVICE int32 array of B + 1 sequence starts in tokens,
 *                non-decreasing, with every len_b <= T; or NULL.  A length
 *                above T is cut to T and a negative one read as 0 (the
 *                library reads cu_seqlens only on the device, so it cannot
 *                report them).
 *   T          : the longest sequence (the padded per-sequence length is T
 *                rounded up to 64; workspace and work scale with B*H*T).
 *
 * The caller guarantees that every existing row lies inside its allocation
 * and that output rows do not overlap one another or any input.  Output
 * rows of tokens t >= len_b are not written.  Pointers need 4-byte alignment
 * and every stride times the element size must be a multiple of 4 bytes (an
 * even stride for bf16); rows are moved 16 bytes at a time where base and
 * strides allow.  bf16 views without cu_seqlens, with T a multiple of 64 and
 * every q, k, v, w and out row on a 16-byte boundary (base and strides) with
 * a token stride below 2^31 elements, are read and written in place.  Other
 * calls gather the inputs into zero-padded staging in the workspace (an extra
 * read and write of each input and output) and scatter the results back.
 * Errors as for the dense entry points, plus EINVAL
 * for a NULL strides, a negative stride or one of 2^40 elements or more, or a
 * misaligned base or stride.
 * ------------------------------------------------------------------------
 */

/* Workspace bytes of path_attn_fwd_varlen (0 for invalid arguments). */
size_t path_attn_varlen_workspace_bytes(int B, int H, int T, int d, int dtype);

/* Forward pass on views.  strides: 8 x 3 values for q, k, v, w, out, beta,
 * logf, lse (in this order).  scale and flags as for path_attn_fwd_ex. */
int path_attn_fwd_varlen(const void *q, const void *k, const void *v, const void *w,
                         const float *beta, const float *logf, void *out, float *lse,
                         const long long *strides, const int *cu_seqlens, int B,
                         int H, int T, int d, int dtype, float scale, unsigned flags,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of path_attn_bwd_varlen (0 for invalid arguments). */
size_t path_attn_bwd_varlen_workspace_bytes(int B, int H, int T, int d, int dtype);

/* Backward pass on views.  strides: 16 x 3 values for q, k, v, w, out,
 * dout, dq, dk, dv, dw, beta, logf, lse, dlse, dbeta, dlogf (in this order).
 * out and lse are path_attn_fwd_varlen's outputs for the same inputs, views
 * and cu_seqlens.  Other arguments as for path_attn_bwd. */
int path_attn_bwd_varlen(const void *q, const void *k, const void *v, const void *w,
                         const float *beta, const float *logf, const void *out,
                         const float *lse, const void *dout, const float *dlse,
                         void *dq, void *dk, void *dv, void *dw, float *dbeta,
                         float *dlogf, const long long *strides, const int *cu_seqlens,
                         int B, int H, int T, int d, int dtype, float scale,
                         void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * The w / beta producer: the transitions' inputs from the hidden states.
 *
 * From the slides' frame "PaTH inserts a learned transformation along every
 * path" (beta_t = 2 sigmoid(u^T x_t + b), ||w_t||_2 = 1, w_t produced by a
 * low-rank projection, a width-3 convolution and an L2 normalisation) and the
 * discussion page's "Model Architecture Details" (the normalisation per head,
 * the projection low-rank), for H heads of size d:
 *     z_t       = Wu (Wd x_t)
 *     z'_t[c]   = cw[c][0] z_{t-2}[c] + cw[c][1] z_{t-1}[c] + cw[c][2] z_t[c]
 *                 (causal, z_t = 0 for t < 0)
 *     w_t[h]    = z'_t[h d .. h d + d) / || . ||_2   (0 if the vector is zero)
 *     beta_t[h] = 2 sigmoid(u[h] . x_t + ub[h])
 * (no biases in the projections, no activation after the convolution).
 *   x  : [B, T, Dm] bf16, row-major (hidden states; input)
 *   wd : [R, Dm] bf16 (low-rank down projection, output-major; input)
 *   wu : [H*d, R] bf16 (up projection; input)
 *   cw : [H*d, 3] float32 (convolution taps, oldest first; input)
 *   u  : [H, Dm] bf16, ub : [H] float32 (beta's projection and bias; inputs)
 *   w  : [B, H, T, d] bf16 (output, overwritten: path_attn_fwd's w layout)
 *   beta : [B, H, T] float32 (output, overwritten)
 * dtype must be PATH_ATTN_BF16.  Any T >= 1.  x, wd, wu, cw, u and w 16-byte
 * aligned, ub and beta 4-byte aligned.  Runs on the caller's stream; needs
 * no workspace.
 * Errors: EINVAL for null or misaligned pointers, sizes <= 0 or a bad dtype;
 * EUNSUPPORTED for PATH_ATTN_F32, d not in {64, 128}, Dm not a multiple of
 * 64, R not a multiple of 16 or above 128, or sizes beyond the library's
 * indexing; EHIP on a launch error.
 */
int path_attn_wbeta(const void *x, const void *wd, const void *wu, const float *cw,
                    const void *u, const float *ub, void *w, float *beta, int B, int T,
                    int Dm, int R, int H, int d, int dtype, void *stream);

/* Static, human-readable description of a status code. */
const char *path_attn_strerror(int status);

/* Library version string. */
const char *path_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PATH_ATTN_H */
