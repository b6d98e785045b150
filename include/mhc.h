/* mhc.h -- C ABI of the MI355X (gfx950) mHC hot path.
 *
 * Manifold-Constrained Hyper-Connections widen the residual into n = 4
 * parallel streams mixed by a per-token n x n matrix that is projected onto
 * the Birkhoff polytope of doubly stochastic matrices (entries >= 0, every row
 * and column summing to 1).  This library provides, for n = 4:
 *
 *   mhc_birkhoff_fwd    the projection of a batch of logit matrices
 *   mhc_birkhoff_bwd    its gradient by implicit differentiation
 *   mhc_birkhoff_fwd_n, mhc_birkhoff_bwd_n
 *                       the same projection and gradient for n x n matrices,
 *                       1 <= n <= 8
 *   mhc_birkhoff_bwd_recompute
 *                       the same gradient from the logits alone (the forward
 *                       solve is redone in registers; P is not stored)
 *   mhc_birkhoff_fwd_bwd
 *                       projection and gradient in one pass, for when dL/dP
 *                       is already known when the projection is computed
 *   mhc_birkhoff_pipeline_step
 *                       the projection of one batch and the gradient of
 *                       another in one launch (overlapped micro-batches)
 *   mhc_stream_mix      out[t,i,:] = sum_j H[t,i,j] x[t,j,:], optionally with
 *                       the projection of H's logits fused in
 *   mhc_stream_mix_bwd  gradients of the stream mix
 *   mhc_layer_fwd/bwd   one full mHC residual-layer step (RMSNorm, dynamic
 *                       map, sigmoid read/write maps, projected residual map,
 *                       read-mix and write-back)
 *
 * Sources (cited by page title and section):
 *  - Deep Signal, "DeepSeek mHC: Manifold-Constrained Hyper-Connections"
 *    article, sections on the Birkhoff polytope constraint and on the
 *    Sinkhorn-Knopp projection;
 *  - forpes.ru mHC explainer, sections "Hyper-Connections" and "mHC: bring
 *    back the guarantee" (stream widening, read/write maps, sigmoid on the
 *    pre/post maps);
 *  - neo-ai mHC paper summary, section on memory-bandwidth optimisation
 *    (fused RMSNorm + matmul + activation, mixed precision);
 *  - gist.science summary of "Accelerating Birkhoff projection for mHC",
 *    sections 2 (entropic-OT equivalence), 2.1 (Newton on the reduced dual,
 *    max-shift), 2.2 (implicit differentiation, Hessian reuse).
 *
 * Conventions for every call
 *  - All tensor pointers are DEVICE pointers (HBM) owned by the caller.  The
 *    library allocates nothing and keeps no state between calls; it is safe
 *    to call from several host threads.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work and returns; results are ready when the
 *    stream reaches that point.
 *  - Layouts are dense row-major (C order), no strides.  fp32 tensors must be
 *    16-byte aligned; bf16 tensors 16-byte aligned with C a multiple of 8.
 *  - Argument errors are detected on the host before anything is enqueued and
 *    return MHC_ERR_INVALID_ARGUMENT (or MHC_ERR_UNSUPPORTED for n != 4); a
 *    failed launch returns MHC_ERR_LAUNCH.  mhc_last_error() gives a message
 *    for the calling thread's last failure.
 *  - A batch size of 0 returns MHC_OK without enqueueing anything.
 *  - Outputs may alias inputs only where a call says so, and then exactly
 *    (same pointer); partial overlap is undefined and not detected.
 *  - Inputs must be finite.  Non-convergence of the forward solver is
 *    reported per matrix through the optional `iters` array, never as a
 *    status code.
 */
#ifndef MHC_H
#define MHC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version history: 1 first release; 2 adds mhc_birkhoff_fwd_bwd and makes
 * -1 (the solver's own choice) the default of mhc_proj_opts.warm_sweeps; 3
 * makes -1 the default of mhc_proj_opts.max_iters as well (30 Newton
 * iterations, 1000 Sinkhorn sweeps) and bounds every call's batch by
 * MHC_MAX_BATCH / MHC_MAX_TOKENS; 4 adds mhc_birkhoff_pipeline_step and
 * mhc_layer_bwd_noalloc. */
#define MHC_ABI_VERSION 4

/* Largest batch one call accepts: B matrices for the projection calls, T
 * tokens for the stream-mix and layer calls.  Larger values return
 * MHC_ERR_INVALID_ARGUMENT before anything is enqueued.  They are the sizes
 * whose launches stay below the 2^32 work-items one grid dimension can hold
 * (the 4x4 backward runs four lanes per matrix, the token kernels sixteen
 * per token); split larger batches into several calls.  At these limits one
 * [B,4,4] fp32 tensor is 64 GiB and one [T,4,8] bf16 stream tensor 16 GiB. */
#define MHC_MAX_BATCH ((int64_t)1073741760)  /* 2^30 - 64 */
#define MHC_MAX_TOKENS ((int64_t)268435440)  /* 2^28 - 16 */

typedef enum {
    MHC_OK = 0,
    MHC_ERR_INVALID_ARGUMENT = 1,
    MHC_ERR_UNSUPPORTED = 2,
    MHC_ERR_LAUNCH = 3
} mhc_status;

typedef enum {
    MHC_SOLVER_NEWTON = 0,   /* Newton on the three column potentials */
    MHC_SOLVER_SINKHORN = 1  /* alternating row / column normalisation */
} mhc_solver;

/* Forward-solver options.  mhc_proj_opts_default() fills the defaults. */
typedef struct {
    int32_t solver;      /* mhc_solver; default MHC_SOLVER_NEWTON */
    int32_t max_iters;   /* Newton iterations or Sinkhorn sweeps, 1 .. 10000,
                            or -1 (the default) for the solver's own limit:
                            30 Newton iterations, 1000 Sinkhorn sweeps */
    float tol;           /* stop once max_j |column sum_j - 1| <= tol (rows are
                            normalised last, so they sum to 1 up to rounding);
                            default 1e-6.  Sinkhorn with tol == 0 runs exactly
                            max_iters sweeps (fixed-count mode). */
    int32_t warm_sweeps; /* log-domain Sinkhorn sweeps between the starting
                            point and the first Newton step; 0 .. 64, or -1
                            (the default) for the solver's own choice: none
                            for n = 4, whose start (from the assignment
                            problem) leaves nothing for a sweep to gain, and
                            one for the general-n solver */
} mhc_proj_opts;

/* Iteration codes written to the optional `iters` output. */
#define MHC_ITERS_SATURATED 254u   /* 254 or more iterations */
#define MHC_ITERS_NOT_CONVERGED 255u

/* Fill *opts with the defaults (never fails for a non-NULL pointer). */
mhc_status mhc_proj_opts_default(mhc_proj_opts* opts);

/* mhc_birkhoff_fwd -- project B logit matrices onto the doubly stochastic
 * matrices.
 *
 * For each b, P[b] is the unique doubly stochastic matrix of the form
 * diag(u) exp(logits[b]) diag(v): the limit of Sinkhorn-Knopp normalisation
 * (Deep Signal article, Sinkhorn-Knopp section) and the entropic optimal
 * transport plan (gist.science summary, section 2).  The Newton solver works
 * on the three column potentials left after the row potentials are
 * eliminated by a row softmax and one potential is fixed (summary, section
 * 2.1), with each row max-shifted before the exponential.
 *
 *   logits  [B,4,4] fp32, device, 16-byte aligned (64 bytes per matrix)
 *   P       [B,4,4] fp32, device, 16-byte aligned; may alias logits exactly
 *   B       number of matrices, 0 <= B <= MHC_MAX_BATCH
 *   opts    solver options, NULL = defaults; host pointer, read during the call
 *   iters   NULL or device [B] uint8: Newton iterations (or Sinkhorn sweeps)
 *           used, 254 = 254 or more, 255 = stopped with the column residual
 *           above tol (fp32 noise floor, max_iters, or line-search failure);
 *           P is then the best row-stochastic iterate reached
 *   stream  hipStream_t
 */
mhc_status mhc_birkhoff_fwd(const float* logits, float* P, int64_t B,
                            const mhc_proj_opts* opts, uint8_t* iters, void* stream);

/* mhc_birkhoff_bwd -- gradient of a loss L through the projection.
 *
 * Given P = projection(A) and G = dL/dP, returns dL/dA by implicit
 * differentiation of the scaling conditions (gist.science summary, section
 * 2.2): dA = P o (G - alpha 1^T - 1 beta^T) with (I - P^T P) beta = b - P^T a,
 * beta_3 = 0, alpha = a - P beta, a = (P o G) 1, b = (P o G)^T 1.  The system
 * matrix is the last Newton Hessian, rebuilt from P; nothing else from the
 * forward pass is needed.
 *
 *   P            [B,4,4] fp32, device, as returned by mhc_birkhoff_fwd
 *   grad_P       [B,4,4] fp32, device
 *   grad_logits  [B,4,4] fp32, device; may alias grad_P exactly
 *   0 <= B <= MHC_MAX_BATCH, stream as above.
 */
mhc_status mhc_birkhoff_bwd(const float* P, const float* grad_P, float* grad_logits,
                            int64_t B, void* stream);

/* mhc_birkhoff_bwd_recompute -- dL/dA from the logits and dL/dP, without P.
 *
 * The recompute strategy of the mHC paper (neo-ai summary, section on
 * recomputation: intermediate results are recomputed in the backward pass
 * instead of stored) applied to the projection: each matrix is projected
 * again with the same solver and options as mhc_birkhoff_fwd, and the
 * implicit-differentiation gradient of mhc_birkhoff_bwd (gist.science
 * summary, section 2.2) is formed from that P while it is still in
 * registers.  Reads 128 bytes and writes 64 per matrix; the forward pass then
 * needs to keep only the logits.  Results equal mhc_birkhoff_bwd applied to
 * mhc_birkhoff_fwd's P up to fp32 rounding (the gradient is computed from P
 * in the matrix-per-lane arithmetic rather than the row-per-lane one).
 *
 *   logits       [B,4,4] fp32, device, 16-byte aligned
 *   grad_P       [B,4,4] fp32, device, 16-byte aligned
 *   grad_logits  [B,4,4] fp32, device, 16-byte aligned; may alias logits or
 *                grad_P exactly (each matrix is read whole before it is
 *                written), must not overlap them partially
 *   opts         solver options as for mhc_birkhoff_fwd (NULL = defaults)
 *   0 <= B <= MHC_MAX_BATCH, stream as above.  Errors as for mhc_birkhoff_fwd.
 */
mhc_status mhc_birkhoff_bwd_recompute(const float* logits, const float* grad_P,
                                      float* grad_logits, int64_t B,
                                      const mhc_proj_opts* opts, void* stream);

/* mhc_birkhoff_fwd_bwd -- P and dL/dA in one pass, when dL/dP is at hand.
 *
 * The last Newton Hessian is the matrix the implicit-differentiation
 * backward needs (gist.science summary, section 2.2), so when the gradient
 * dL/dP is already known at the time of the projection (a loss linear in P,
 * a fixed upstream gradient, a benchmark) both results come from one solve
 * kept in registers: P as mhc_birkhoff_fwd computes it and the gradient as
 * mhc_birkhoff_bwd_recompute computes it.  Reads 128 bytes and writes 128 per
 * matrix in one launch, against 128 + 192 in two for mhc_birkhoff_fwd then
 * mhc_birkhoff_bwd.  In training, where dL/dP depends on P, use those two.
 *
 *   logits       [B,4,4] fp32, device, 16-byte aligned
 *   grad_P       [B,4,4] fp32, device, 16-byte aligned
 *   P            [B,4,4] fp32, device, 16-byte aligned, written; may alias
 *                logits exactly, must not overlap grad_P or grad_logits
 *   grad_logits  [B,4,4] fp32, device, 16-byte aligned, written; may alias
 *                grad_P exactly, must not overlap logits or P
 *   opts, iters  as for mhc_birkhoff_fwd (iters must not overlap any of the
 *                four arrays)
 *   0 <= B <= MHC_MAX_BATCH, stream as above.  Errors as for mhc_birkhoff_fwd.
 */
mhc_status mhc_birkhoff_fwd_bwd(const float* logits, const float* grad_P, float* P,
                                float* grad_logits, int64_t B, const mhc_proj_opts* opts,
                                uint8_t* iters, void* stream);

/* mhc_birkhoff_pipeline_step -- the forward of one batch and the backward of
 * another, independent one, in a single launch.
 *
 * For schedules that overlap forward and backward work of different
 * micro-batches, or recompute one layer's projection during another layer's
 * backward instead of keeping it (neo-ai mHC paper summary, systems section:
 * recomputation of the mHC intermediates and the extended DualPipe
 * schedule).  P is bit for bit mhc_birkhoff_fwd's on (logits, B).  The
 * gradient is formed one matrix per lane, the arithmetic of
 * mhc_birkhoff_bwd_recompute and mhc_birkhoff_fwd_bwd: bit for bit what those
 * give when P_bwd is the forward's P of their logits, and equal to
 * mhc_birkhoff_bwd's on (P_bwd, grad_P) up to fp32 rounding (the same
 * implicit-differentiation formula, gist.science summary section 2.2,
 * evaluated in another order).  The forward solve is bound by its own
 * latency and leaves HBM mostly idle, the backward is bound by HBM, so the
 * pair takes about as long as the forward alone where two launches in
 * sequence take the sum.
 *
 *   logits, P, B, opts, iters
 *                as for mhc_birkhoff_fwd (the forward batch)
 *   P_bwd, grad_P, grad_logits, B_bwd
 *                as P, grad_P, grad_logits, B of mhc_birkhoff_bwd (the
 *                backward batch)
 *   The forward's outputs (P, iters) must not overlap any backward array and
 *   grad_logits must not overlap logits, P or iters; the two batches' inputs
 *   may share memory.  Either batch may be empty (B = 0 or B_bwd = 0: only the
 *   other half runs; its pointers are then not used).  Errors as for
 *   mhc_birkhoff_fwd and mhc_birkhoff_bwd; nothing is enqueued on error.
 */
mhc_status mhc_birkhoff_pipeline_step(const float* logits, float* P, int64_t B,
                                      const mhc_proj_opts* opts, uint8_t* iters,
                                      const float* P_bwd, const float* grad_P,
                                      float* grad_logits, int64_t B_bwd, void* stream);

/* mhc_birkhoff_fwd_n / mhc_birkhoff_bwd_n -- the projection and its gradient
 * for a batch of n x n matrices, 1 <= n <= 8.
 *
 * The method of mhc_birkhoff_fwd/bwd for any n (gist.science summary,
 * section 2.1: one potential per column, one of them fixed by the shift
 * invariance, leaving n - 1 Newton variables; section 2.2 for the gradient);
 * the pages build n = 4, which these calls pass to mhc_birkhoff_fwd/bwd
 * (with those calls' 16-byte alignment rule).  n = 1 gives P = [1] and a zero
 * gradient (neo-ai summary, properties of doubly stochastic matrices).
 *
 *   logits, P, grad_P, grad_logits
 *           [B,n,n] fp32 row-major, device, 4-byte aligned (16 for n = 4);
 *           aliasing as for the n = 4 calls (P may be logits, grad_logits
 *           may be grad_P; no partial overlap)
 *   n       1..8, else MHC_ERR_UNSUPPORTED
 *   opts, iters, stream, errors as for mhc_birkhoff_fwd.
 */
mhc_status mhc_birkhoff_fwd_n(const float* logits, float* P, int64_t B, int32_t n,
                              const mhc_proj_opts* opts, uint8_t* iters, void* stream);
mhc_status mhc_birkhoff_bwd_n(const float* P, const float* grad_P, float* grad_logits,
                              int64_t B, int32_t n, void* stream);

/* mhc_stream_mix -- apply per-token mixing matrices to the n residual streams:
 *   out[t,i,c] = sum_j H[t,i,j] x[t,j,c]
 * (forpes.ru explainer, "Hyper-Connections": the streams are mixed by an
 * n x n matrix at every layer).  bf16 in and out, fp32 accumulation, the
 * result rounded to nearest-even.
 *
 *   x            [T,n,C] bf16, device
 *   H_or_logits  [T,n,n] fp32, device: the mixing matrices H when proj is
 *                NULL, otherwise logits that are projected in the same kernel
 *                (as mhc_birkhoff_fwd with *proj) before the mix
 *   H_out        NULL or [T,n,n] fp32, device: receives the projected H (only
 *                used when proj != NULL)
 *   out          [T,n,C] bf16, device; must not overlap x
 *   0 <= T <= MHC_MAX_TOKENS, n == 4 (else MHC_ERR_UNSUPPORTED), C >= 8,
 *   C % 8 == 0
 *   proj         NULL or host pointer to solver options (see above)
 */
mhc_status mhc_stream_mix(const void* x, const float* H_or_logits, float* H_out, void* out,
                          int64_t T, int32_t n, int64_t C, const mhc_proj_opts* proj,
                          void* stream);

/* mhc_stream_mix_bwd -- gradients of the stream mix for upstream grad_out:
 *   grad_x[t,j,c] = sum_i H[t,i,j] grad_out[t,i,c]     (bf16, fp32 accumulation)
 *   grad_H[t,i,j] = sum_c grad_out[t,i,c] x[t,j,c]     (fp32)
 * The mix is linear in x and in H (forpes.ru explainer, "Hyper-Connections":
 * the n streams are mixed by an n x n matrix), so these are its two partial
 * derivatives by the chain rule: the transposed mix of grad_out, and the
 * per-token outer product of grad_out and x summed over the width C.  In mHC
 * grad_H then flows into the projection's backward (mhc_birkhoff_bwd).
 *
 *   x, grad_out  [T,n,C] bf16, device;  H [T,n,n] fp32, device
 *   grad_x       [T,n,C] bf16, device, must not overlap the inputs
 *   grad_H       [T,n,n] fp32, device, must not overlap any other tensor
 *   0 <= T <= MHC_MAX_TOKENS, n == 4, C % 8 == 0 as above.
 */
mhc_status mhc_stream_mix_bwd(const void* x, const float* H, const void* grad_out,
                              void* grad_x, float* grad_H, int64_t T, int32_t n, int64_t C,
                              void* stream);

/* One mHC residual-layer step for n = 4 streams of width C, per token t:
 *   r = sqrt(mean over the 4C values of x_t^2 + eps)          (RMSNorm, no gain)
 *   logits = (x_t W^T) / r                                     [24] per token
 *   H_pre = sigmoid(logits[0:4]), H_post = sigmoid(logits[4:8])
 *   H_res = Birkhoff projection of logits[8:24] (row-major 4x4)
 *   u = sum_j H_pre[j] x_t[j]                                  (read-mix)
 *   x_out[i] = H_post[i] f_t + sum_j H_res[i][j] x_t[j]        (write-back)
 * forpes.ru explainer, "Hyper-Connections" (streams projected to the model
 * width before the layer function F and expanded after) and "mHC" (sigmoid on
 * the pre/post maps, projected residual map); kimiseek V4-Flash article (the
 * maps are generated per token from the input); neo-ai summary (fused RMSNorm
 * + matmul + activation, mixed precision).  Layouts are row-major; bf16 for
 * the activations and W, fp32 for the small per-token tensors. */
typedef struct {
    int64_t T;        /* tokens, 0 .. MHC_MAX_TOKENS */
    int32_t n;        /* streams, must be 4 */
    int64_t C;        /* stream width, a positive multiple of 64 */
    float eps;        /* RMSNorm epsilon, > 0 (1e-6 in the reference workload) */
    const mhc_proj_opts* proj;  /* H_res solver options, NULL = defaults */
    /* inputs (device, bf16) */
    const void* x;    /* [T, 4, C] */
    const void* W;    /* [24, 4C]: rows pre 0:4 | post 4:8 | res 8:24 */
    const void* f;    /* [T, C]   layer-function output (write-back input) */
    /* forward outputs; rms, logits, H_pre, H_post and H_res are also inputs
       of the backward (device) */
    void* u;          /* [T, C] bf16 */
    void* x_out;      /* [T, 4, C] bf16 */
    float* rms;       /* [T] */
    float* logits;    /* [T, 24], already divided by rms */
    float* H_pre;     /* [T, 4] */
    float* H_post;    /* [T, 4] */
    float* H_res;     /* [T, 4, 4] */
    /* backward inputs (device, bf16) */
    const void* grad_x_out;  /* [T, 4, C] */
    const void* grad_u;      /* [T, C] */
    /* backward outputs (device) */
    void* grad_x;        /* [T, 4, C] bf16 */
    void* grad_f;        /* [T, C] bf16 */
    float* grad_W;       /* [24, 4C] fp32 */
    float* grad_logits;  /* [T, 24] fp32 */
    void* workspace;     /* backward scratch, >= mhc_layer_workspace_bytes() bytes,
                            256-byte aligned; contents need no initialisation */
    int64_t workspace_bytes;
} mhc_layer_args;

/* Bytes of device workspace mhc_layer_bwd needs for (T, n, C); -1 if the
 * shape is invalid. */
int64_t mhc_layer_workspace_bytes(int64_t T, int32_t n, int64_t C);

/* Forward of the layer step: fills u, x_out, rms, logits, H_pre, H_post,
 * H_res.  No output may overlap another tensor.  Two kernels on `stream`. */
mhc_status mhc_layer_fwd(const mhc_layer_args* a, void* stream);

/* Backward of the layer step for upstream grad_x_out and grad_u, using x, W,
 * f and the forward's rms, logits, H_pre, H_post, H_res: fills grad_x,
 * grad_f, grad_W (overwritten, not accumulated) and grad_logits.  The
 * projection's part is the implicit-differentiation backward of
 * mhc_birkhoff_bwd.  Five kernels on `stream`; the workspace must not be in
 * use by another call that overlaps on the device. */
mhc_status mhc_layer_bwd(const mhc_layer_args* a, void* stream);

/* mhc_layer_bwd_noalloc -- mhc_layer_bwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  It computes exactly what mhc_layer_bwd computes,
 * with the same kernels, but its workspace is a device array inside the
 * library (MHC_LAYER_NOALLOC_SCRATCH_BYTES, one per GPU, held from the
 * library's first use on that GPU until the process ends) instead of
 * a->workspace, which is ignored together with a->workspace_bytes.  The call
 * itself allocates nothing.
 *
 *  - Shapes whose workspace (mhc_layer_workspace_bytes) exceeds the array are
 *    refused with MHC_ERR_INVALID_ARGUMENT; at C = 7168 that admits up to
 *    about 200000 tokens per call.
 *  - The work runs on the current device; a non-NULL stream must belong to
 *    it (else MHC_ERR_INVALID_ARGUMENT).
 *  - Every call on one GPU shares that GPU's array: calls that overlap in
 *    time on one GPU (concurrent streams, several host threads) race and give
 *    undefined results.  Calls ordered on one stream are safe.  Nothing in the
 *    array needs to start at zero; each call overwrites what it reads.
 * Other arguments, outputs and errors as for mhc_layer_bwd. */
#define MHC_LAYER_NOALLOC_SCRATCH_BYTES ((int64_t)67108864) /* 64 MiB */
mhc_status mhc_layer_bwd_noalloc(const mhc_layer_args* a, void* stream);

const char* mhc_status_string(mhc_status s);
/* Message for the calling thread's last non-OK status ("" if none). */
const char* mhc_last_error(void);
int32_t mhc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H */
