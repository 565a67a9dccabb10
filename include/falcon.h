/*
 * falcon.h -- C ABI of the MI355X (gfx950) implementation of Falcon
 * fast-weight attention: the chunk-parallel forward pass and the single-token
 * recurrent step, and the backward pass of the chunked form.
 *
 * Sources, cited by page title and section:
 *   [P1] zhouql-dev.github.io, "把状态更新写成一条学习规则：Falcon 家族重新对齐
 *        fast-weight 记忆": sections 本质 (prefix alignment), Falcon家族 (the
 *        family and the NLMS step), 三种等价形式 (recurrent / masked-parallel /
 *        chunked forms, positive-decay renormalisation), Figures 3 and 4.
 *   [P2] 59188saintaubert.com, "给记忆装一个“及时纠错”的开关：Falcon让循环模型
 *        学会边写边改": sections 一个被忽略的时间差, 把记忆更新变成一次梯度下降,
 *        六个变体, 正衰减钳制, 三种视角.
 *
 * What both entry points compute, per sequence (b, h) and step t = 1..T:
 *   x_t   = phi(k_{t-1})                  prefix-aligned key ([P1] 本质); x_1 = x_prev
 *   lam_t = max(exp(g_t), eps_gamma)      positive-decay clamp ([P2] 正衰减钳制)
 *   eta_t = beta_t / (eps_eta + |x_t|^2)  NLMS step ([P1] Falcon家族; [P2] 梯度下降)
 *   F1 : S_t = lam_t S_{t-1} + eta_t (v_t - S_{t-1} x_t) x_t^T
 *   F2 : as F1 with eta_t a vector over value channels (rows of S)
 *   F3 : S_t = lam_t S_{t-1} + (eta_t / Bw) sum_{j=t-Bw+1..t} (v_j - S_{t-1} x_j) x_j^T
 *   F1A/F2A/F3A: the same with the additive write (v_j instead of the residual)
 *   o_t   = S_t phi(q_t)                  read after write
 *   phi(a) = a / sqrt(|a|^2 + eps_phi)
 * The step definitions are [P1] Falcon家族 and [P2] 六个变体; the chunked
 * evaluation is [P1] 三种等价形式 form C / Figure 4-C (per-chunk Gram and WY
 * factors with a triangular solve) and [P2] 三种视角.
 *
 * Conventions shared by every entry point
 *   Layout   all arrays are dense, C order, no strides:
 *              q, k   [B, T, H, dk]   dtype (fp32 or bf16)
 *              v, o   [B, T, H, dv]   dtype
 *              beta   [B, T, H]  fp32, or [B, T, H, dv] for F2/F2A
 *              log_lambda (g) [B, T, H] fp32; any value <= 0 incl. -inf.
 *                     g > 0 (a decay above 1) is outside the contract and is
 *                     not checked: the chunked kernels factor every decay
 *                     exp(L_a - L_b), a >= b, as a number <= 1
 *              S      [B, H, dv, dk]  fp32, row i = value channel i
 *              x_prev [B, H, dk]      fp32
 *              win_x  [B, H, Bw-1, dk], win_v [B, H, Bw-1, dv] fp32, oldest first
 *            The single-step entry point drops the T axis.
 *   Memory   every pointer except `shape` and the state struct itself is a
 *            device pointer (hipMalloc / torch CUDA tensor).  The caller owns
 *            all memory; the library never allocates, frees, synchronises or
 *            keeps a pointer after the call returns.  Device pointers must be
 *            16-byte aligned.
 *   Streams  work is enqueued on `stream` (a hipStream_t, NULL = the null
 *            stream) and the call returns without waiting.  Buffers must stay
 *            alive until the stream reaches the work.
 *   Errors   the return value is a falcon_status_t.  Argument validation is
 *            done on the host before any HIP call, so an invalid call never
 *            touches the device.  A failed kernel launch returns
 *            FALCON_ERR_HIP; a fault inside a kernel shows up at the caller's
 *            next synchronisation.  NaN/Inf in the inputs are not checked;
 *            lam > 1 is outside the contract.
 *   Threads  no global mutable state: calls may be made from several threads.
 */
#ifndef FALCON_H
#define FALCON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FALCON_ABI_VERSION 4

typedef enum {
  FALCON_1 = 1,   /* scalar NLMS step, residual write            */
  FALCON_1A = 2,  /* scalar step, additive (inner-product) write  */
  FALCON_2 = 3,   /* per-value-channel step, residual write       */
  FALCON_2A = 4,  /* per-value-channel step, additive write       */
  FALCON_3 = 5,   /* window of Bw pairs, averaged residuals       */
  FALCON_3A = 6   /* window of Bw pairs, averaged additive write  */
} falcon_variant_t;

typedef enum { FALCON_F32 = 0, FALCON_BF16 = 1 } falcon_dtype_t;  /* of q, k, v, o */

/* Which key the pair written at step t carries ([P1] 本质; [P2] 一个被忽略的时间差):
 * the prefix pair (phi(k_{t-1}), v_t), the method's alignment, or the same-step
 * pair (phi(k_t), v_t) the pages contrast it with.  Same-step calls do not read
 * the carried x_prev (they still write x_prev = phi(k_T)); window pairs are
 * (phi(k_j), v_j).  Same-step runs on the chunk-parallel kernels (with or without
 * a workspace where they are built) and on the decode step; other shapes return
 * FALCON_ERR_UNSUPPORTED. */
typedef enum { FALCON_ALIGN_PREFIX = 0, FALCON_ALIGN_SAME = 1 } falcon_align_t;

typedef enum {
  FALCON_OK = 0,
  FALCON_ERR_INVALID_ARG = 1,  /* null pointer, bad enum, non-positive size, ... */
  FALCON_ERR_UNSUPPORTED = 2,  /* valid but not built: head dim, chunk, window, dtype */
  FALCON_ERR_WORKSPACE = 3,    /* workspace smaller than falcon_chunk_fwd_workspace() */
  FALCON_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} falcon_status_t;

typedef struct {
  int32_t variant;   /* falcon_variant_t */
  int32_t dtype;     /* falcon_dtype_t   */
  int32_t batch;     /* B >= 1 */
  int32_t seqlen;    /* T >= 1 (ignored by falcon_recurrent_step) */
  int32_t heads;     /* H >= 1 */
  int32_t dk;        /* key/query head dim: 32, 64 or 128 (fp32 inputs: 32 or 64).
                        The kernels are built for square states only: dk must
                        equal dv, else FALCON_ERR_UNSUPPORTED (every kernel tiles
                        both axes of S with the same 16-wide blocks and one
                        compile-time head dim).  fp32 at 128 is not built: its
                        tiles and staged rows do not fit a compute unit's LDS. */
  int32_t dv;        /* value head dim: equal to dk (see above) */
  int32_t chunk;     /* chunk length C: 16, 32 or 64; T need not be a multiple */
  int32_t window;    /* Bw for F3/F3A; must be 1 for the other variants.  The
                        decode step takes 1..8.  The chunked forms take 1, 2, 4
                        or 8 (Bw must divide 64: a system of 64 virtual rows
                        holds 64/Bw whole steps, and a step's Bw rows must not
                        straddle a 16-row MFMA block).  Larger windows (e.g. 16)
                        return FALCON_ERR_UNSUPPORTED: they are not built. */
  float eps_gamma;   /* decay floor, in (0, 1]; the pages' workloads use 1e-3 */
  float eps_phi;     /* feature-map epsilon, >= 0 (1e-6) */
  float eps_eta;     /* NLMS epsilon, > 0 (1e-6); 0 is FALCON_ERR_INVALID_ARG,
                        since a fresh sequence's first key is zero and its step
                        would divide by |x|^2 = 0 */
  int32_t align;     /* falcon_align_t */
} falcon_shape_t;

typedef struct {
  float *S;       /* [B, H, dv, dk]; required                                 */
  float *x_prev;  /* [B, H, dk] = phi(k) of the last consumed token; required  */
  float *win_x;   /* [B, H, Bw-1, dk], F3/F3A with Bw > 1 only, else ignored  */
  float *win_v;   /* [B, H, Bw-1, dv]                                         */
} falcon_state_t;

/* ABI version of the loaded library (FALCON_ABI_VERSION). */
int falcon_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *falcon_status_string(int status);

/* Bytes of device workspace that enable the chunk-parallel path of
 * falcon_chunk_fwd for this shape; 0 when that path does not apply (the
 * forward then runs a fused kernel that needs no workspace).  The workspace
 * holds, per system of rows (a chunk of C steps; for F3/F3A with Bw > 1,
 * C/Bw steps of Bw pairs each), the key-side factors (Gram / score blocks,
 * diagonal-block inverses, per-row factors) that a prep kernel over all
 * systems writes and the state scan reads, plus a copy of each sequence's
 * incoming x_prev and window; its contents are scratch and need no
 * initialisation.  The path covers F1/F1A/F2/F2A (chunk 16, 32, 64) and
 * F3/F3A with Bw = 2, 4, 8 at chunk 64; d = 32, 64 (fp32, bf16), 128 (bf16).
 * F3A with Bw = 2, 4, 8 at d = 64, chunk 64 (fp32 and bf16 inputs) uses a workspace for its
 * banded-weight form (the window-averaged additive write of [P1] Falcon家族
 * as decayed score weights): each chunk's state increment, then the state
 * entering it, 16 KiB per chunk and sequence, plus the carried-state copy; the
 * returned size covers both.
 * Returns 0 for an invalid shape as well; validation is the forward call's job. */
size_t falcon_chunk_fwd_workspace(const falcon_shape_t *shape);

/* Chunked forward pass over T tokens ([P1] 三种等价形式 form C, Figure 4-C;
 * [P2] 三种视角).
 *   init         NULL: fresh sequences (S = 0, x_prev = 0, zero window).
 *                Otherwise S and x_prev (and the window for F3/F3A, Bw > 1)
 *                are read.  May alias final_state (in-place continuation).
 *   final_state  NULL: not written.  Otherwise receives S_T, x_prev =
 *                phi(k_T) and the last Bw-1 pairs.
 *   o            [B, T, H, dv] in dtype; must not alias any input.
 *   chunk_states NULL, or [B, H, ceil(T/C), dv, dk] fp32: S at the end of
 *                every chunk (the last one equals S_T).
 *   workspace    caller-owned device scratch, 16-byte aligned, or NULL.  NULL
 *                (or a shape whose workspace size is 0) selects the fused
 *                path; otherwise workspace_bytes must be at least
 *                falcon_chunk_fwd_workspace(shape) (else FALCON_ERR_WORKSPACE)
 *                and the chunk-parallel path runs.  Both paths compute the
 *                same function; calls that share one workspace on different
 *                streams race.
 * Results are deterministic: the same inputs give bit-identical outputs. */
int falcon_chunk_fwd(const falcon_shape_t *shape,
                     const void *q, const void *k, const void *v,
                     const float *beta, const float *log_lambda,
                     const falcon_state_t *init, falcon_state_t *final_state,
                     void *o, float *chunk_states,
                     void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The same computation as
 * falcon_chunk_fwd on its chunk-parallel path (prep kernel + state scan), with
 * the scratch that path needs taken from a fixed device array inside the library
 * (FALCON_STATIC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends) instead of a caller's workspace.  The caller still
 * passes every input and output; the call allocates and frees nothing.
 *   Sizes  the shape must have that path (falcon_chunk_fwd_workspace(shape) > 0,
 *          else FALCON_ERR_UNSUPPORTED) and need at most
 *          FALCON_STATIC_SCRATCH_BYTES of it (else FALCON_ERR_WORKSPACE); e.g.
 *          the 130M-layer shape (B 8, H 12, T 2048, d 64, chunk 64) needs 41 MB.
 *   Races  every call on one GPU uses that GPU's one array: calls that overlap
 *          on a GPU (other streams, other threads) race and give wrong results.
 *          The scratch needs no initialisation; each call overwrites it.
 * Other arguments, aliasing and errors as falcon_chunk_fwd. */
#define FALCON_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int falcon_chunk_fwd_static(const falcon_shape_t *shape,
                            const void *q, const void *k, const void *v,
                            const float *beta, const float *log_lambda,
                            const falcon_state_t *init, falcon_state_t *final_state,
                            void *o, float *chunk_states, void *stream);

/* Bytes of device workspace that enable the chunk-parallel path of
 * falcon_chunk_fwd_varlen for this packed shape (shape->batch = N sequences,
 * shape->seqlen = their total token count); 0 when that path does not apply
 * (as for falcon_chunk_fwd_workspace).  Per head it holds one image slot per
 * system the N sequences can have, at most total/S + N + 1 for systems of S
 * steps (sequence n's images start at slot cu_seqlens[n] / S + n, so the layout
 * follows from cu_seqlens on the device), plus each sequence's carried-state
 * copy; no initialisation needed. */
size_t falcon_chunk_fwd_varlen_workspace(const falcon_shape_t *shape);

/* Chunked forward pass over a packed batch of sequences of different lengths
 * (the same computation as falcon_chunk_fwd, one sequence per entry):
 *   shape->batch  = N, the number of sequences; shape->seqlen = the total
 *                   number of tokens, cu_seqlens[N].
 *   cu_seqlens    device int32 [N + 1]: sequence n holds tokens
 *                   cu_seqlens[n] .. cu_seqlens[n+1] - 1 (non-decreasing,
 *                   cu_seqlens[0] = 0; read on the device, not checked).
 *   q, k [total, H, dk], v, o [total, H, dv] in dtype; beta [total, H] (F2/F2A:
 *   [total, H, dv]) and log_lambda [total, H] fp32; the state arrays are per
 *   sequence ([N, H, ...]) as in falcon_chunk_fwd.
 *   workspace     NULL: the one-pass kernel, where it is built for the shape
 *                 (bf16 at d <= 64, fp32 at small chunks); a shape it does not
 *                 build returns FALCON_ERR_WORKSPACE when the chunk-parallel path
 *                 exists for it (pass a workspace) and FALCON_ERR_UNSUPPORTED
 *                 otherwise.  Non-NULL: at least
 *                 falcon_chunk_fwd_varlen_workspace(shape) bytes (else
 *                 FALCON_ERR_WORKSPACE), 16-byte aligned, and the chunk-parallel
 *                 path runs (this covers d = 128 in bf16).
 * Sequence n starts from init (its own S, x_prev and window) and ends in
 * final_state.  A sequence of length 0 is skipped: its final state is not
 * written.  No per-chunk states.  Same aliasing and stream rules as
 * falcon_chunk_fwd; calls sharing a workspace race. */
int falcon_chunk_fwd_varlen(const falcon_shape_t *shape, const int32_t *cu_seqlens,
                            const void *q, const void *k, const void *v,
                            const float *beta, const float *log_lambda,
                            const falcon_state_t *init, falcon_state_t *final_state,
                            void *o, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace falcon_chunk_fwd_segmented needs for this shape
 * and segment count; 0 when the segmented form is not built for them: nseg
 * must divide T, segments must hold at least Bw steps, the shape must have the
 * two-kernel chunk-parallel path (see falcon_chunk_fwd_workspace), and F2 is
 * excluded (its step differs per row of S, so a segment's map is not one
 * matrix).  The workspace holds that path's scratch for B*nseg sequences of
 * T/nseg steps plus six per-segment state arrays; it needs no initialisation. */
size_t falcon_chunk_fwd_segmented_workspace(const falcon_shape_t *shape, int32_t nseg);

/* The chunked forward pass with every sequence cut into nseg segments that run
 * in parallel: the same function as falcon_chunk_fwd (up to rounding), for
 * batches too small to fill the GPU.  A segment maps its incoming state S_0 to
 * S_0 M + N ([P1] 三种等价形式: the chunk maps are affine and compose; [P2]
 * 三种视角), so the call builds the key-side images of all B*nseg segments
 * once, then runs (1) the scan from S_0 = 0 (giving N) and (2) from S_0 = I
 * (giving M + N), both keeping end states only, (3) the composition
 * S_start[p] = S_start[p-1] M_{p-1} + N_{p-1} along each sequence, and (4) the
 * scan from S_start, which writes o and the final state.  The carried key
 * and window entering a segment come from the inputs.  The arrays are the same
 * as falcon_chunk_fwd's ([B, T, H, d] is read as [B*nseg, T/nseg, H, d]); no
 * per-chunk states.  init may alias final_state.  Errors: nseg < 1 or not
 * dividing T -> FALCON_ERR_INVALID_ARG; NULL or misaligned workspace ->
 * FALCON_ERR_INVALID_ARG; a shape or nseg the form is not built for ->
 * FALCON_ERR_UNSUPPORTED; a short workspace -> FALCON_ERR_WORKSPACE. */
int falcon_chunk_fwd_segmented(const falcon_shape_t *shape, int32_t nseg,
                               const void *q, const void *k, const void *v,
                               const float *beta, const float *log_lambda,
                               const falcon_state_t *init, falcon_state_t *final_state,
                               void *o, void *workspace, size_t workspace_bytes, void *stream);

/* One token of the recurrent form ([P1] 三种等价形式 form A; [P2] 三种视角):
 * reads q, k [B, H, dk], v [B, H, dv], beta [B, H] (F2/F2A: [B, H, dv]) and
 * log_lambda [B, H]; updates `state` in place (S, x_prev and, for F3/F3A with
 * Bw > 1, the window) and writes o [B, H, dv] in dtype.  shape->seqlen and
 * shape->chunk are ignored. */
int falcon_recurrent_step(const falcon_shape_t *shape,
                          const void *q, const void *k, const void *v,
                          const float *beta, const float *log_lambda,
                          falcon_state_t *state, void *o, void *stream);

/* Bytes of device workspace falcon_chunk_bwd needs for this shape; 0 when the
 * backward pass is not built for it (or the shape is invalid).  Built for every
 * shape the chunked forward pass builds with d_k = d_v: chunk 16, 32 or 64 (the
 * chunk of the forward call that wrote the per-chunk states), fp32 or bf16
 * inputs, either pairing, by one of two paths:
 *  - chunk-parallel (F1, F1A, F2, F2A, and F3 / F3A with one pair; d = 64): the
 *    kernels work in 64-step chunks and read the states at 64-step boundaries.
 *    The workspace holds, per chunk, the chunk's transition of the reverse
 *    recurrence (d x d), the state gradient the chunk's outputs inject and the
 *    state gradient at the chunk's end (3 x 16 KiB + 4 bytes); for F2, whose
 *    solves are per value channel, the keys, the decayed Gram matrix, the
 *    injected gradient, the end gradient and the per-channel steps (5 x 16 KiB)
 *    plus 516 bytes of per-row factors.
 *  - recurrent form (F3 / F3A windows of 2, 4 or 8 pairs; d = 32, or 128 with
 *    bf16 inputs; every variant): the states at every forward chunk are the
 *    checkpoints.  The workspace holds, per 16 value rows of every sequence,
 *    the row sums of each token (2 d + 2 floats) and of each carried window
 *    pair (d floats): d/16 x (B T H (2 d + 2) + B H (Bw - 1) d) x 4 bytes.
 * It needs no initialisation. */
size_t falcon_chunk_bwd_workspace(const falcon_shape_t *shape);

/* Backward pass of the chunked form ([P1] 三种等价形式 form C / Figure 4-C: the
 * form a training framework runs): the gradients of the scalar
 *     <d_o, o> + <d_final_S, S_T>
 * for the forward pass falcon_chunk_fwd(shape, q, k, v, beta, log_lambda, init)
 * with respect to q, k, v, beta, log_lambda and the initial state.  The
 * outgoing x_prev takes no gradient.  The decay clamp passes no gradient where
 * exp(g) <= eps_gamma (there the decay does not depend on g).
 * Windows ([P1] Falcon家族, [P2] 六个变体): every pair of a step's window takes
 * its share of the gradient, the carried window's pairs included.
 *   init         as given to the forward pass (NULL = fresh sequences); S,
 *                x_prev and, for F3/F3A with Bw > 1, the window are read.
 *   chunk_states [B, H, ceil(T/C), d, d] fp32: the per-chunk states the
 *                forward pass wrote for these inputs at shape->chunk = C.
 *   d_o          [B, T, H, d] in dtype.
 *   d_final_S    [B, H, d, d] fp32, or NULL for a zero gradient on S_T.
 *   dq, dk, dv   [B, T, H, d] fp32, written whole (under the prefix pairing
 *                dk of the last token is 0).
 *   dbeta, dg    [B, T, H] fp32 (F2/F2A: dbeta [B, T, H, dv], like their beta).
 *   d_init       NULL, or S [B, H, d, d] and x_prev [B, H, d] fp32 (and, for
 *                F3/F3A with Bw > 1, win_x and win_v [B, H, Bw-1, d]) that
 *                receive the gradients w.r.t. the initial state (x_prev: 0
 *                under the same-step pairing, which does not read it; the
 *                window's keys are features, so win_x takes their gradient
 *                as they are).
 *   workspace    at least falcon_chunk_bwd_workspace(shape) bytes, else
 *                FALCON_ERR_WORKSPACE; calls sharing a workspace race.
 * Outputs must not alias inputs.  Other shapes return FALCON_ERR_UNSUPPORTED.
 * Results are deterministic. */
int falcon_chunk_bwd(const falcon_shape_t *shape,
                     const void *q, const void *k, const void *v,
                     const float *beta, const float *log_lambda,
                     const falcon_state_t *init, const float *chunk_states,
                     const void *d_o, const float *d_final_S,
                     float *dq, float *dk, float *dv, float *dbeta, float *dg,
                     falcon_state_t *d_init,
                     void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FALCON_H */
