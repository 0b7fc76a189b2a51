/*
 * lam.h -- C ABI of the MI355X (gfx950) recurrent-memory linear-attention
 * forward scan.
 *
 * The operation.  Per (batch, head) chain the scan keeps a fixed-size memory
 * W in R^{dv x dk} and, token by token, predicts the value from the current
 * key, writes only the residual, and reads with the query
 * ("Mechanisms, trade-offs and cross-layer routing of linear-attention
 * architectures", sections "Understanding the core idea" and "Technical
 * details": the unified recurrent-memory notation, memory W in
 * R^{dv x dphi}, read y = W phi(q), delta-rule residual r = v - vbar):
 *
 *   DeltaNet            r = v - W k;              W = W + beta r k^T
 *   Gated DeltaNet      r = v - (alpha W) k;      W = alpha W + beta r k^T
 *   Kimi Delta          r = v - W diag(a) k;      W = W diag(a) + beta r k^T
 *                       (a in R^dk: decay per key-feature channel)
 *   Gated DeltaNet-2    e = b*k, z = w*v;  r = z - (alpha W) e;
 *                       W = alpha W + beta r k^T  (erase b in R^dk, write w in R^dv)
 *   and every variant reads after its write:  y_t = W_t q_t.
 *
 * VLA ("Technical summary: Variational Linear Attention (VLA)", sections 2.2
 * and 2.3) keeps an inverse penalty A = M^{-1} (d x d) beside its state S
 * (d x d).  Per token: khat, qhat = unit-normalised ELU+1 features of k, q;
 * z = A p, A = A - z z^T / (1 + p^T z) (Sherman-Morrison for M + p p^T);
 * alphahat = A khat / |A khat|; S = S + (v - S khat) alphahat^T; y = S qhat.
 *
 * Conventions shared by both entry points.
 *   Layouts (row-major, contiguous): per-token streams [B,T,H,n] (n = dk for
 *   q, k, erase_b and Kimi Delta's alpha; n = dv for v, write_w, out; n = d
 *   for VLA's q, k, v, p, out); per-token scalars (beta, scalar alpha)
 *   [B,T,H]; states [B,H,dv,dk] (VLA: A and S [B,H,d,d]).
 *   dtype: every per-token stream and `out` share one storage dtype
 *   (LAM_F32 or LAM_BF16); states are always fp32, and so are every
 *   accumulation and every element-wise step.  The chunked delta-rule
 *   schedule on LAM_BF16 storage feeds bf16 operands to the matrix cores
 *   (products accumulated in fp32); all other schedules compute in fp32.
 *   alpha is the decay itself, in [0, 1]; beta, erase_b, write_w are used as
 *   given (gate squashing happens upstream).  Delta-rule q and k are used as
 *   given (normalise upstream); VLA takes raw q and k.
 *   Pointers: device memory owned by the caller; the library keeps none of
 *   them after returning.
 *   Workspace: the chunked schedules write state-independent per-chunk
 *   blocks to a device workspace between their kernels, which the caller
 *   provides: lam_forward_workspace_size / lam_vla_workspace_size give its
 *   size for a call's arguments (0 when the schedule the call runs needs
 *   none; then `workspace` may be NULL).  It must be device memory of at
 *   least that many bytes, 256-byte aligned, on the device `stream` belongs
 *   to, and not overlap any argument; too small or misaligned returns
 *   LAM_ERR_INVALID_ARG before any HIP call.  The call reads and writes it
 *   only through the work it enqueues on `stream`, so the caller may reuse
 *   it for any later work ordered after the call on that stream.  Sizes at
 *   dk = 128: 6,144 B per (b, h, 64-token chunk) for DeltaNet, Gated
 *   DeltaNet and Gated DeltaNet-2 (25.2 MB at B8 T4096 H8), and 14,848 B per
 *   (b, h, 16-token sub-chunk, counted in whole pairs) for Kimi Delta
 *   (487 MB at B2 T32768 H8); the fp32 chunked form (fp32 storage, and
 *   bf16 at dk 32 / 96): 26,640 B per (b, h, 16-token chunk) at dk = 128,
 *   8,208 B at dk = 32; plus the 256-byte status block.
 *   Status block: the first 256 bytes of a workspace.  Word 0 (uint32)
 *   receives LAM_DEVICE_* bits from the call's kernels: the call's first
 *   kernel sets it to 0, and a later kernel ORs in LAM_DEVICE_WAIT_TIMEOUT if
 *   one of its bounded in-kernel waits between waves ran out (the outputs of
 *   that call are then not trustworthy).  Read it after the call completes.
 *   The library allocates no device or host memory, creates no stream or
 *   event, never synchronises, and keeps no state between calls: everything
 *   a call touches is in its arguments.
 *   A NULL initial state means zero memory (VLA: A = I, S = 0); a NULL
 *   final-state pointer means the final state is not written.  A final-state
 *   buffer may be the same buffer as its initial state; `out` must not
 *   overlap any input (checked).
 *   Errors: all argument checks happen before any HIP call and return
 *   LAM_ERR_INVALID_ARG (NULL required pointer, negative size, size overflow,
 *   bad enum, overlapping out) or LAM_ERR_UNSUPPORTED (head size outside
 *   {32, 64, 96, 128}, or an algorithm not built for this variant and dtype).
 *   Work is enqueued on `stream` (NULL = default stream) and the call returns
 *   at once; a failed launch returns LAM_ERR_HIP, and faults during execution
 *   surface at the caller's next synchronisation.  No exception crosses the
 *   ABI and the library prints nothing.  Calls are re-entrant: calls that do
 *   not share a workspace may run concurrently from any threads and streams;
 *   calls that share one must be ordered on one stream.  Results are bitwise
 *   reproducible run to run.
 *   Limits (LAM_ERR_INVALID_ARG beyond them): B * H <= 2^24, T <= 2^30 - 1,
 *   H * max(dk, dv) <= 2^24 (token-row offsets within a chunk stay in 32
 *   bits), and at most 2^31 - 1 chunk tasks per call.
 *   Non-finite inputs are not checked: NaN and Inf propagate through the
 *   recurrence into later outputs and the final state of their chain.
 */
#ifndef LAM_H
#define LAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LAM_DELTANET = 0,         /* alpha = 1                                      */
    LAM_GATED_DELTANET = 1,   /* alpha [B,T,H]                                  */
    LAM_KIMI_DELTA = 2,       /* alpha [B,T,H,dk]                               */
    LAM_GATED_DELTANET2 = 3   /* alpha [B,T,H], erase_b [B,T,H,dk], write_w [B,T,H,dv] */
} lam_variant;

typedef enum { LAM_F32 = 0, LAM_BF16 = 1 } lam_dtype;

/* Bits of word 0 of a workspace's status block. */
#define LAM_DEVICE_WAIT_TIMEOUT 0x1u

typedef enum {
    LAM_OK = 0,
    LAM_ERR_INVALID_ARG = 1,
    LAM_ERR_UNSUPPORTED = 2,
    LAM_ERR_HIP = 3,
    LAM_ERR_SCRATCH_LIMIT = 4   /* lam_forward_noalloc: the call needs more than its scratch */
} lam_status;

/* Evaluation schedule.  Both compute the same scan; they differ only in
 * rounding order.  AUTO picks the fastest built one for the shape. */
typedef enum {
    LAM_ALGO_AUTO = 0,
    LAM_ALGO_RECURRENT = 1,   /* token by token, memory in registers           */
    LAM_ALGO_CHUNKED = 2      /* chunkwise-parallel, matrix-core contractions   */
} lam_algo;

/*
 * Delta-rule family forward scan over a [B,T] block (see the rules above).
 *   variant      lam_variant
 *   dtype        lam_dtype of q, k, v, alpha, beta, erase_b, write_w, out
 *   B, T, H      batch, tokens, heads (>= 0; any of them 0 is a no-op except
 *                that T = 0 still copies the initial state to state_out)
 *   dk, dv       key and value head sizes, each in {32, 64, 96, 128}
 *   q, k         [B,T,H,dk]                         required
 *   v            [B,T,H,dv]                         required
 *   alpha        [B,T,H] or, for Kimi Delta, [B,T,H,dk]; ignored by DeltaNet
 *   erase_b      [B,T,H,dk], Gated DeltaNet-2 only (ignored otherwise)
 *   write_w      [B,T,H,dv], Gated DeltaNet-2 only (ignored otherwise)
 *   beta         [B,T,H]                            required
 *   state_in     [B,H,dv,dk] fp32 or NULL (zero memory)
 *   out          [B,T,H,dv]                         required, written
 *   state_out    [B,H,dv,dk] fp32 or NULL; may equal state_in
 *   workspace    device scratch of workspace_bytes (see Workspace above);
 *                NULL allowed when the size query returns 0
 *   algo         lam_algo
 *   stream       HIP stream the work is enqueued on
 */
lam_status lam_forward(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                       int64_t dv, const void *q, const void *k, const void *v,
                       const void *alpha, const void *erase_b, const void *write_w,
                       const void *beta, const float *state_in, void *out, float *state_out,
                       void *workspace, size_t workspace_bytes, int algo, hipStream_t stream);

/*
 * Bytes of workspace lam_forward needs for these arguments (0: none),
 * written to *bytes.  Returns the status lam_forward would return for a
 * shape, dtype, variant or algorithm it rejects (pointers are not examined).
 */
lam_status lam_forward_workspace_size(int variant, int dtype, int64_t B, int64_t T, int64_t H,
                                      int64_t dk, int64_t dv, int algo, size_t *bytes);

/*
 * Cross-layer routing signal ("Mechanisms, trade-offs and cross-layer routing
 * of linear-attention architectures", sections "Methodology" and "Technical
 * details"): CLER and CLER-H route each token's delta-rule residual r (the
 * rules above: r = z - W~ e, taken against the decayed memory), CLVR routes
 * the write value (v; z = w*v for Gated DeltaNet-2).
 */
typedef enum { LAM_SIDE_NONE = 0, LAM_SIDE_RESIDUAL = 1, LAM_SIDE_VALUE = 2 } lam_side;

/*
 * lam_forward that also writes the routing signal of every token:
 *   side         lam_side (LAM_SIDE_NONE: exactly lam_forward)
 *   side_out     [B,T,H,dv] in dtype, required unless LAM_SIDE_NONE; may not
 *                overlap any other argument or the workspace
 * Same workspace (lam_forward_workspace_size), schedules and errors as
 * lam_forward.  On the bf16 chunked schedules the residual is rounded to bf16
 * where the scan rounds it for its own products (the value emitted is the one
 * the memory update uses); the fp32 chunked form and the token-recurrent
 * schedule compute it in fp32.
 */
lam_status lam_forward_side(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                            int64_t dv, const void *q, const void *k, const void *v,
                            const void *alpha, const void *erase_b, const void *write_w,
                            const void *beta, const float *state_in, void *out, float *state_out,
                            int side, void *side_out, void *workspace, size_t workspace_bytes,
                            int algo, hipStream_t stream);

/*
 * Routing epilogue: h <- h + s P^T, i.e. every token's signal s_t (all heads,
 * N = H * dv values) mapped to the model width by P and added to the residual
 * stream h_t (same passages: the zero-initialised projection P and
 * epsilon = P s added to h).  The projection is a contraction on the matrix
 * cores with fp32 accumulation; the add is fused into its epilogue (h is read
 * once and written once).
 *   dtype        lam_dtype of s, P and h (bf16 operands feed bf16 matrix
 *                cores; f32 operands fp32 ones)
 *   M            tokens (B * T), >= 0
 *   D            model width, a multiple of 16
 *   N            signal width, a multiple of 32
 *   s            [M, N], P [D, N], h [M, D] (row-major), each 16-byte
 *                aligned; h may not overlap s or P
 * Errors as lam_forward; results are bitwise reproducible.
 */
lam_status lam_route(int dtype, int64_t M, int64_t D, int64_t N, const void *s, const void *P, void *h,
                     hipStream_t stream);

/*
 * Log-linear (Fenwick-tree) readout of the delta-rule family ("Technical
 * summary: adaptive memory decay for log-linear attention", "Problem
 * definition": a Fenwick-tree hierarchy of O(log T) memory levels, each
 * step's output the lambda^(l)_t-weighted sum of the levels' reads;
 * "Complexity preservation": O(log T) decoding memory).  Levels, for the
 * query at absolute position t: token t is level 0, an earlier token s is
 * level msb(t xor s) + 1.  Every level takes the variant's transition each
 * step (decay, then the delta rule's erase along e with that level's own
 * prediction), level 0 alone receives the write beta z k^T, and at position
 * t >= 1 levels 0 .. ctz(t) merge into level ctz(t) + 1; the levels sum to
 * the plain scan's memory (lambda = 1 reproduces lam_forward).  Output
 * y_t = sum_l lambda_t[l] S_l q_t.  Computed token by token in fp32.
 *   variant .. beta   as lam_forward (one storage dtype)
 *   nL           levels, 1 .. 24, at least lam_loglinear_levels(t0 + T - 1)
 *                (LAM_ERR_INVALID_ARG if fewer)
 *   t0           absolute position of token 0 (>= 0; t0 + T < 2^23)
 *   lam          [B,T,H,nL] fp32 level weights (lam_loglinear_lambda makes
 *                them), required when T > 0
 *   state_in     [B,H,nL,dv,dk] fp32 level memories after position t0 - 1,
 *                or NULL (all empty)
 *   out          [B,T,H,dv] in dtype, required when T > 0
 *   state_out    [B,H,nL,dv,dk] fp32 or NULL; may equal state_in
 * A decode step is a call with T = 1 at t0 = the token's position, the
 * levels updated in place.  No workspace; errors as lam_forward.
 */
lam_status lam_loglinear_forward(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                                 int64_t dv, int64_t nL, int64_t t0, const void *q, const void *k,
                                 const void *v, const void *alpha, const void *erase_b,
                                 const void *write_w, const void *beta, const float *lam,
                                 const float *state_in, void *out, float *state_out,
                                 hipStream_t stream);

/* Levels the readout needs through absolute position last_position:
 * floor(log2(last_position)) + 2, or 1 for last_position < 1. */
int64_t lam_loglinear_levels(int64_t last_position);

/*
 * Adaptive level weights (same page, "Methodology", LambdaMLPSoftplus): two
 * linear layers and a softplus per row, lambda = softplus((d W1) W2 + b), for
 * every (token, head) row; the page initialises W2 = 0 and b = 0.54, so that
 * every weight starts at softplus(0.54), about 1.
 *   dtype        lam_dtype of d
 *   M            rows (B * T * H), >= 0
 *   nL           levels (1 .. 24); nh hidden width (1 .. 64; the page uses
 *                twice the level count)
 *   d            [M, nL] in dtype; W1 [nL, nh], W2 [nh, nL], b [nL] fp32
 *   lam          [M, nL] fp32, written (may not overlap the inputs)
 * softplus(x) is evaluated as max(x, 0) + log1p(exp(-|x|)).
 */
lam_status lam_loglinear_lambda(int dtype, int64_t M, int64_t nL, int64_t nh, const void *d,
                                const float *W1, const float *W2, const float *b, float *lam,
                                hipStream_t stream);

/*
 * VLA forward scan over a [B,T] block (dk = dv = d, d in {32, 64, 96, 128}).
 *   q, k, v, p   [B,T,H,d] raw queries, keys, values and penalty directions
 *   A_in, S_in   [B,H,d,d] fp32 or NULL (A = I, S = 0)
 *   out          [B,T,H,d] written
 *   A_out, S_out [B,H,d,d] fp32 or NULL; each may equal its input buffer
 *   workspace    as for lam_forward, sized by lam_vla_workspace_size
 */
lam_status lam_vla_forward(int dtype, int64_t B, int64_t T, int64_t H, int64_t d,
                           const void *q, const void *k, const void *v, const void *p,
                           const float *A_in, const float *S_in, void *out, float *A_out,
                           float *S_out, void *workspace, size_t workspace_bytes, int algo,
                           hipStream_t stream);

/*
 * VLA forward scan with the output read as a ratio of two recurrences
 * ("Technical summary: Variational Linear Attention (VLA)", section 2.3: the
 * output is a ratio of recurrences as in standard linear attention, where
 * numerator and denominator accumulate alike, the denominator over a value
 * of 1).  The denominator is a d-vector n per (b, h) that follows the write
 * rule with the value 1:
 *   n <- n + (1 - n . khat) alphahat,   y = (S qhat) / (n . qhat),
 * with S, A, khat, qhat and alphahat exactly as lam_vla_forward.  y is not
 * guarded against n . qhat near zero (a zero n_in makes the first token's
 * denominator alphahat . qhat).  Token-recurrent kernel; no workspace.
 *   q, k, v, p, A_in, S_in, out, A_out, S_out   as lam_vla_forward
 *   n_in         [B,H,d] fp32 or NULL (zero)
 *   n_out        [B,H,d] fp32 or NULL (not written); may equal n_in
 * An output may be its own input's buffer (A_out = A_in, S_out = S_in,
 * n_out = n_in) and must not otherwise overlap an input, another output or
 * `out`.  Errors as lam_vla_forward.
 */
lam_status lam_vla_forward_ratio(int dtype, int64_t B, int64_t T, int64_t H, int64_t d,
                                 const void *q, const void *k, const void *v, const void *p,
                                 const float *A_in, const float *S_in, const float *n_in, void *out,
                                 float *A_out, float *S_out, float *n_out, hipStream_t stream);

/* Bytes of workspace lam_vla_forward needs (0: none); as above. */
lam_status lam_vla_workspace_size(int dtype, int64_t B, int64_t T, int64_t H, int64_t d,
                                  int algo, size_t *bytes);

/*
 * Backward pass of lam_forward's delta-rule scan: the gradients of
 * L = sum <dout, out> + <dstate_out, state_out> with respect to q, k, v,
 * alpha, erase_b, write_w, beta and state_in.  It is the reverse-mode
 * adjoint of the per-token rule above ("Mechanisms, trade-offs and
 * cross-layer routing of linear-attention architectures", "Technical
 * details"; the pages train these layers, section "Main results"),
 * computed in fp32 from the same inputs as the forward (it recomputes the
 * forward; no forward outputs are needed).
 *   forward inputs  as lam_forward (q, k, v, alpha, erase_b, write_w, beta,
 *                   state_in), in dtype
 *   dout            [B,T,H,dv] in dtype, required
 *   dstate_out      [B,H,dv,dk] fp32 or NULL (zero)
 *   gradients, fp32, written: dq, dk [B,T,H,dk]; dv [B,T,H,dv]; dbeta
 *                   [B,T,H] (all required); dalpha like alpha (required
 *                   unless DeltaNet); derase_b [B,T,H,dk] and dwrite_w
 *                   [B,T,H,dv] (required for Gated DeltaNet-2); dstate_in
 *                   [B,H,dv,dk] or NULL.  No gradient buffer may overlap
 *                   another argument.
 *   algo            lam_algo.  LAM_ALGO_CHUNKED (DeltaNet, Gated DeltaNet,
 *                   Gated DeltaNet-2; what LAM_ALGO_AUTO picks for them when
 *                   T > 0): the adjoint in 16-token chunks on fp32 matrix
 *                   cores -- the chunk records, the forward again keeping
 *                   each chunk's start state and residuals, the state
 *                   cotangent scanned in reverse, then every chunk's
 *                   gradients in parallel; bitwise reproducible.
 *                   LAM_ALGO_RECURRENT (and Kimi Delta): token-recurrent,
 *                   forward checkpoints every 16 tokens; dq, dk, dbeta,
 *                   dalpha and derase_b sum over the memory's dv rows with
 *                   atomics across workgroups, so those five are not
 *                   bitwise reproducible run to run (dv, dwrite_w and
 *                   dstate_in are).  LAM_ALGO_CHUNKED for Kimi Delta
 *                   returns LAM_ERR_UNSUPPORTED.
 *   workspace       lam_backward_workspace_size bytes for the same algo.
 *                   Chunked: per (b, h, 16-token chunk) the two records
 *                   (52 KB at dk = 128), per (b, h, pair of chunks) a state
 *                   and a state cotangent (2 * dv * dk * 4 B), plus U and dX
 *                   (2 * B*T*H*dv * 4 B): 2.2 GB at B8 T4096 H8 d128.
 *                   Recurrent: the forward state every 16 tokens,
 *                   B*H*ceil(T/16)*dv*dk*4 B.  Both plus the status block.
 * T = 0 writes dstate_in = dstate_out (zero if NULL).
 */
lam_status lam_backward(int variant, int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                        int64_t dv, const void *q, const void *k, const void *v,
                        const void *alpha, const void *erase_b, const void *write_w,
                        const void *beta, const float *state_in, const void *dout,
                        const float *dstate_out, float *dq, float *dk_, float *dv_, float *dalpha,
                        float *derase_b, float *dwrite_w, float *dbeta, float *dstate_in, int algo,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace lam_backward needs with this algo (> 0 for any
 * non-empty call). */
lam_status lam_backward_workspace_size(int variant, int dtype, int64_t B, int64_t T, int64_t H,
                                       int64_t dk, int64_t dv, int algo, size_t *bytes);

/*
 * One-token decode step for N concurrent streams: the rule above applied to
 * one token per (stream, head), the memory updated in place ("Mechanisms,
 * trade-offs and cross-layer routing of linear-attention architectures",
 * "Technical details"; the fixed-size state that lets a stream decode with no
 * cache of past tokens is section 5 of the VLA summary).  Equivalent to
 * lam_forward with B = N, T = 1 and state_in = state_out = state.
 *   q, k         [N,H,dk]     v, out  [N,H,dv]     beta, scalar alpha [N,H]
 *   alpha        Kimi Delta: [N,H,dk]; erase_b [N,H,dk], write_w [N,H,dv]
 *                (Gated DeltaNet-2)
 *   state        [N,H,dv,dk] fp32, required, read and overwritten
 * Needs no workspace.  The step reads and writes the whole state once, so it
 * is bound by HBM; dk in {32, 64, 128} runs a dedicated kernel, dk = 96 the
 * token-recurrent one.  Errors as lam_forward (state NULL or overlapping
 * out: LAM_ERR_INVALID_ARG).
 */
lam_status lam_step(int variant, int dtype, int64_t N, int64_t H, int64_t dk, int64_t dv,
                    const void *q, const void *k, const void *v, const void *alpha,
                    const void *erase_b, const void *write_w, const void *beta, float *state,
                    void *out, hipStream_t stream);

/*
 * One-token VLA step for N concurrent streams ("Technical summary:
 * Variational Linear Attention (VLA)", sections 2.2-2.3 and 5): q, k, v, p
 * [N,H,d], A and S [N,H,d,d] fp32 updated in place (both required), out
 * [N,H,d].  Equivalent to lam_vla_forward with T = 1 and in-place states, on
 * the token-recurrent kernel.
 */
lam_status lam_vla_step(int dtype, int64_t N, int64_t H, int64_t d, const void *q, const void *k,
                        const void *v, const void *p, float *A, float *S, void *out,
                        hipStream_t stream);

/*
 * lam_vla_step with the ratio read: one token for N concurrent streams, A,
 * S [N,H,d,d] and the denominator n [N,H,d] fp32 updated in place (all
 * required).  Equivalent to lam_vla_forward_ratio with T = 1 and in-place
 * states.
 */
lam_status lam_vla_step_ratio(int dtype, int64_t N, int64_t H, int64_t d, const void *q, const void *k,
                              const void *v, const void *p, float *A, float *S, float *n, void *out,
                              hipStream_t stream);

/*
 * lam_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  The
 * same arguments, kernels and results as lam_forward, with the workspace
 * replaced by a fixed device array inside the library of
 * LAM_NOALLOC_SCRATCH_BYTES (32 MiB: the bf16 chunked schedule of Gated
 * DeltaNet at B8 T4096 H8 d128 needs 24.1 MB; the fp32 chunk records need
 * 26,640 B per (b, h, 16 tokens) at dk = 128), held on each GPU the library
 * runs on until the process ends.  With LAM_ALGO_AUTO, a call whose chunked
 * workspace exceeds the array runs the recurrent schedule (no workspace)
 * instead; with LAM_ALGO_CHUNKED such a call returns LAM_ERR_SCRATCH_LIMIT
 * before any HIP call.  Nothing is allocated or freed; the first call on a
 * device looks up that device's array address (the stream must belong to the
 * current device).  Every call on one GPU shares that GPU's array: calls that
 * may overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller.
 */
#define LAM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
lam_status lam_forward_noalloc(int variant, int dtype, int64_t B, int64_t T, int64_t H,
                               int64_t dk, int64_t dv, const void *q, const void *k,
                               const void *v, const void *alpha, const void *erase_b,
                               const void *write_w, const void *beta, const float *state_in,
                               void *out, float *state_out, int algo, hipStream_t stream);

/*
 * The schedule LAM_ALGO_AUTO runs for these arguments: LAM_ALGO_RECURRENT or
 * LAM_ALGO_CHUNKED (the chunked one computes its contractions with bf16
 * operands and fp32 accumulation when dtype is LAM_BF16 and dk is 64 or 128,
 * in fp32 on 16-token chunks otherwise; Kimi Delta's chunked schedule takes
 * bf16 at dk 64 / 128 only).  Returns -1 for arguments lam_forward would
 * reject.
 */
int lam_select_algo(int variant, int dtype, int64_t T, int64_t dk, int64_t dv);

/* Static, NUL-terminated description of a status code (any int; values that
 * are not a lam_status give "unknown status"). */
const char *lam_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int lam_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LAM_H */
