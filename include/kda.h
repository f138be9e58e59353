/*
 * kda.h -- C ABI of libkda, the gfx950 (MI355X) forward pass of Kimi Delta
 * Attention (KDA) in chunk-parallel form, its recurrent decode step and its
 * gradient.
 *
 * The operation.  KDA is a delta-rule linear attention with a fixed-size state
 * matrix per (sequence, head), a forget gate, and a per-channel decay that
 * refines Gated DeltaNet ("What is Kimi Delta Attention (KDA)", Moonshot AI
 * Open-Sources FlashKDA, kongchang.com/en; "¿Qué es la atención Kimi Delta y
 * por qué es importante?", 7minutos.es).  For every token t of a sequence,
 * with S a K x V fp32 state:
 *
 *   k_t <- k_t / sqrt(|k_t|^2 + 1e-6),  q_t likewise           (in-kernel L2 norm)
 *   b_t  = sigmoid(beta_t)                                       (in-kernel sigmoid)
 *   a_t[d] = max(lower_bound, -exp(A_log[h]) * softplus(g_t[d] + dt_bias[h,d]))
 *   S_t = (I - b_t k_t k_t^T) Diag(exp(a_t)) S_{t-1} + b_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 *
 * The in-kernel norm, sigmoid and gate flags are those of the backend call on
 * "作为 FLA 后端的用法" (zuobiaodaohang.com FlashKDA page); the argument list,
 * dtypes and the K = V = 128 restriction are those of the forward call on
 * "Debajo del capó: CUTLASS en Hopper" (7minutos.es).  The gate formula is not
 * printed on the pages: the one above is the plain reading of the parameter
 * names, clamped to [lower_bound, 0].
 *
 * Every pointer argument is a DEVICE pointer on the current HIP device unless
 * stated otherwise.  All tensors are row-major and contiguous, as the pages
 * require ("性能与注意事项", zuobiaodaohang.com).  The library keeps no
 * reference to any pointer after a call returns and has no global mutable
 * state: calls on different streams may run concurrently if their buffers
 * (including workspaces) are disjoint.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the optional recurrent states. */
typedef enum { KDA_BF16 = 1, KDA_FP32 = 2 } kda_dtype_t;

/* Status codes.  Everything except KDA_ERR_HIP is detected on the host before
 * any work is enqueued; no output is touched in that case. */
typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL (q,k,v,g,beta,out may be NULL when T == 0) */
    KDA_ERR_SHAPE = 2,       /* B, H < 1, T < 0, num_seqs inconsistent, varlen with B != 1 */
    KDA_ERR_UNSUPPORTED = 3, /* K != 128 or V != 128                               */
    KDA_ERR_PARAM = 4,       /* lower_bound not finite or outside [-5, 0]; scale not finite */
    KDA_ERR_DTYPE = 5,       /* a state dtype other than KDA_BF16 / KDA_FP32      */
    KDA_ERR_ALIGN = 6,       /* a tensor pointer not 16-byte aligned (workspace: 256) */
    KDA_ERR_WORKSPACE = 7,   /* workspace_bytes smaller than kda_fwd_workspace_size() */
    KDA_ERR_HIP = 8,         /* a HIP launch error                                 */
    KDA_ERR_SCRATCH = 9      /* kda_fwd_noalloc: the call needs more workspace than its static scratch */
} kda_status_t;

/* Shapes and the caller-owned workspace of one call.
 *   q, k, g : [B, T, H, K] bf16      v, out : [B, T, H, V] bf16     beta : [B, T, H] bf16
 *   Without cu_seqlens, num_seqs must equal B and batch row n is one sequence.
 *   With cu_seqlens, B must be 1, T is the total packed token count and
 *   num_seqs = N is the number of packed sequences (cu_seqlens has N + 1 entries).
 *   workspace: device memory of at least kda_fwd_workspace_size(desc) bytes,
 *   256-byte aligned, owned by the caller, not read before it is written.  If
 *   workspace is NULL the library takes and releases one with
 *   hipMallocAsync / hipFreeAsync on the call's stream. */
typedef struct {
    int64_t B, T, H, K, V;
    int64_t num_seqs;
    int32_t initial_state_dtype;  /* kda_dtype_t; ignored when initial_state is NULL */
    int32_t final_state_dtype;    /* kda_dtype_t; ignored when final_state is NULL   */
    void *workspace;
    size_t workspace_bytes;
    /* Optional instrumentation: NULL, or an array of 4 hipEvent_t created by
     * the caller.  kda_fwd records event 0 before its first kernel, 1 after
     * the chunk-table kernel (packed batches only; otherwise right after 0),
     * 2 after the intra-chunk kernel and 3 after the state-chain kernel, all
     * on `stream`, so per-kernel device time can be measured (with split
     * chains, event 3 follows the last of the three chain-side launches). */
    hipEvent_t *phase_events;
    /* Split state chains (batches without cu_seqlens only).  The chunks of a
     * sequence form a serial chain; every chunk maps the state entering it
     * affinely, so a long chain can be cut into segments whose maps are
     * computed in parallel and then composed in order (see kda_fwd).
     *   0  : automatic -- split when the chains alone leave most of the GPU
     *        idle: segments = max(min(32 / (B * H), chunks / 32),
     *        min(64 / (B * H), chunks / 64)) when that is >= 3, otherwise no
     *        split (sized for the 256 CUs of an MI355X at 8 workgroups per
     *        segment and head: one round of workgroups with segments of at
     *        least 32 chunks, or two rounds with segments of at least 64; a
     *        split runs every chunk twice, so 2 segments would gain nothing);
     *   1  : never split;
     *   >= 2 : split every sequence into that many segments (at most one per
     *        64-token chunk; fewer when the chunks do not divide evenly).
     * Negative values are KDA_ERR_PARAM; a value >= 2 with cu_seqlens is
     * KDA_ERR_UNSUPPORTED.  The result is the same function of the inputs
     * either way, up to rounding. */
    int64_t chain_segments;
    /* Largest piece of a kernel grid one launch may cover (a testing aid):
     * 0 for the library's rule (see "Launch size" at kda_fwd); n > 0 caps each
     * launch at n chain groups of 8 (sequence, head) pairs, n 64-token chunk
     * rows or n decode (sequence, head) pairs, so that small inputs take the
     * several-launch path of very large ones.  Results are identical either
     * way.  Negative values are KDA_ERR_PARAM. */
    int64_t launch_piece;
    /* 0: the two-kernel forward (intra-chunk kernel, then the state chain);
     * 1: the pipelined forward where it applies -- batches without cu_seqlens,
     * H a multiple of 8, no split chains -- otherwise the two-kernel one.  The
     * pipelined forward runs the intra-chunk work and the state chains in one
     * grid and passes the intermediates through L2; on MI355X it measures
     * slower than the two-kernel forward on every workload tried, so it is
     * not the default.  Other values are KDA_ERR_PARAM.  The two give the same
     * bits. */
    int64_t pipeline;
    /* kda_bwd only (every other call ignores it): NULL, or the workspace of an
     * earlier kda_fwd call on the same inputs, shapes and cu_seqlens, still
     * holding what that call wrote (nothing may have reused it since).  kda_bwd
     * then reads the forward's intra-chunk intermediates from it instead of
     * recomputing them -- its intra-chunk pass is skipped, the gradients are
     * the same bits -- so a training step that keeps the forward's workspace
     * (about 72.5 KiB per 64-token chunk and head) until the backward saves
     * that pass.  It must be 256-byte aligned (else KDA_ERR_ALIGN); it is only
     * read.  The results are undefined if it does not hold that call's
     * intermediates.  kda_fwd_noalloc's scratch cannot serve: later calls
     * reuse it. */
    const void *forward_workspace;
    /* kda_fwd: 0, or 1 to also store in the workspace the fp32 state entering
     * every 64-token chunk (64 KiB per chunk and head more, which
     * kda_fwd_workspace_size counts), for a later kda_bwd on the same inputs
     * to read instead of recomputing.  The outputs are the same bits; the
     * pipelined forward does not apply.  kda_fwd_noalloc: must be 0.
     * kda_bwd: 1 when desc->forward_workspace holds such states too (a kda_fwd
     * call with save_states = 1 and the same chain_segments); kda_bwd then
     * runs none of the forward's kernels.  Ignored without forward_workspace.
     * Other values are KDA_ERR_PARAM. */
    int64_t save_states;
} kda_desc_t;

/* Bytes of workspace kda_fwd needs for these shapes (0 if the shapes are
 * invalid).  Pure host arithmetic; needs no device.  Grows linearly with the
 * number of 64-token chunks times H (about 72.5 KiB per chunk and head), plus
 * 192 KiB per (segment, head) when chains are split. */
size_t kda_fwd_workspace_size(const kda_desc_t *desc);

/* Number of segments kda_fwd splits each sequence's state chain into for
 * these shapes when called without cu_seqlens (1 = not split; calls with
 * cu_seqlens never split), or -1 if the descriptor is invalid.  Pure host
 * arithmetic. */
int64_t kda_fwd_chain_segments(const kda_desc_t *desc);

/* 1 if kda_fwd runs these shapes and desc->pipeline (without cu_seqlens) on
 * the pipelined forward, 0 if on the two-kernel one, -1 if the descriptor is
 * invalid.  Pure host arithmetic. */
int kda_fwd_pipelined(const kda_desc_t *desc);

/* Enqueue the KDA forward pass on `stream` and return without synchronising.
 *
 *   q, k, g, v, beta : inputs as in kda_desc_t; g is the gate before activation,
 *                      beta holds logits (the sigmoid is applied in-kernel).
 *   scale            : fp32 factor applied to every output.
 *   A_log            : fp32 [H], per-head log decay rate.
 *   dt_bias          : fp32 [H, K], per-channel gate bias.
 *   lower_bound      : fp32 in [-5, 0]; the per-channel log-decay is clamped to
 *                      [lower_bound, 0] (values below -5 are refused: the chunked
 *                      decay factorisation relies on them).
 *   initial_state    : [N, H, K, V] of initial_state_dtype, or NULL for zeros.
 *   final_state      : [N, H, K, V] of final_state_dtype, or NULL to skip it.
 *                      It may alias initial_state when both dtypes match.
 *   cu_seqlens       : device int64 [N + 1] cumulative lengths, or NULL.  Its
 *                      contents must satisfy cu[0] = 0, cu[n] <= cu[n+1],
 *                      cu[N] = T.  They are trusted (no host sync) unless the
 *                      environment has KDA_VALIDATE=1: then kda_fwd copies them
 *                      to the host, synchronising `stream`, and returns
 *                      KDA_ERR_SHAPE for contents that break these rules,
 *                      before anything is allocated or launched (a debugging
 *                      aid; such a call cannot be captured in a graph).
 *                      Empty sequences are allowed: their final state is their
 *                      initial state.
 *   out              : bf16 [B, T, H, V], caller-allocated, must not alias inputs.
 *   desc             : shapes, state dtypes and workspace (host pointer).
 *   stream           : HIP stream (0 = the null stream).
 * Returns KDA_OK when the work was enqueued; device faults surface at the
 * caller's next synchronisation.
 *
 * Launch size.  A kernel launch covers at most 2^30 work-items.  Bigger
 * batches (from about half a million (sequence, head) pairs) are enqueued as
 * several launches of the same kernel, with identical results
 * (desc->launch_piece forces that path for small inputs).
 *
 * Value range.  The matrix-core operands of the state path are fp16 (11-bit
 * significand, largest finite value 65504), with fp32 accumulation.  Every
 * factor built from q, k and the gate is bounded by 1 in magnitude (unit-norm
 * q and k, decays <= 1), so the limit falls on the terms that scale with v and
 * the state.  Writing s_j for column j of the state (a K-vector), the delta
 * rule only replaces the component of s_j along the written key, so
 *   |S[i, j]| <= |s_j|_2 <= sqrt(|s_j(0)|_2^2 + sum_t v_t[j]^2)
 * over the tokens t seen so far, and each pseudo-value
 *   |u_t[j]| <= |v_t[j]| + |s_j|_2.
 * The result is exact up to rounding while these stay below 65504: for
 * example |v| <= 160 and |initial_state| <= 100 for sequences of up to 131072
 * tokens (sqrt(128 * 100^2 + 131072 * 160^2) + 160 < 59000), or |v| <= 1500
 * and |initial_state| <= 1000 up to 1024 tokens (< 51000).  These are worst-case bounds
 * (keys chosen against the state); unit-scale activations stay orders of
 * magnitude below them.  Larger magnitudes overflow fp16 silently and give
 * inf or NaN outputs; no error is returned.  At the small end, values below
 * 2^-14 (6.1e-5) lose significand bits in fp16 subnormals: v and the state
 * should not be scaled below about 2^-12 of unit scale.
 *
 * With split chains (desc->chain_segments) the state chain of every sequence
 * runs in three launches instead of one: the map of every segment, an fp32
 * scan over the segments (the entering states and the final state), and the
 * chain with outputs from each segment's entering state. */
kda_status_t kda_fwd(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float scale, const float *A_log,
                     const float *dt_bias, float lower_bound,
                     const void *initial_state, void *final_state,
                     const int64_t *cu_seqlens, void *out,
                     const kda_desc_t *desc, hipStream_t stream);

/* kda_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation, arguments and errors as kda_fwd, except that the workspace
 * is the library's own static scratch -- a device array of
 * kda_fwd_noalloc_max_workspace() bytes (128 MiB) in the library's code
 * object, which every GPU the library runs on holds until the process ends --
 * and desc->workspace / workspace_bytes are ignored.  The call allocates
 * nothing (no hipMalloc, hipMallocAsync or host allocation; KDA_VALIDATE is
 * not honoured, since reading cu_seqlens back needs a host buffer).  A call
 * whose kda_fwd_workspace_size() exceeds the scratch returns KDA_ERR_SCRATCH
 * before anything is enqueued: 128 MiB covers about 1800 (64-token chunk,
 * head) pairs, e.g. 2048 tokens at 32 heads, or 4096 tokens at 16 heads.
 * The scratch holds no state between calls (every byte is written before it
 * is read), but all calls on one GPU share it: calls that can overlap on one
 * GPU (different streams, or different host threads) race and must be
 * serialised by the caller. */
kda_status_t kda_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, float scale, const float *A_log,
                             const float *dt_bias, float lower_bound,
                             const void *initial_state, void *final_state,
                             const int64_t *cu_seqlens, void *out,
                             const kda_desc_t *desc, hipStream_t stream);

/* Bytes of the static scratch kda_fwd_noalloc runs in (128 MiB). */
size_t kda_fwd_noalloc_max_workspace(void);

/* One recurrent step per sequence -- the token-by-token form used during
 * generation ("¿Qué es la atención Kimi Delta y por qué es importante?",
 * 7minutos.es).  For every sequence n and head h, with S the K x V state read
 * from initial_state (zeros when NULL) and the same in-kernel norms, sigmoid
 * and gate as kda_fwd:
 *
 *   S' = (I - b k k^T) Diag(exp(a)) S + b k v^T,   out = scale * S'^T q
 *
 *   desc             : B = N sequences, T = 1, num_seqs = N, K = V = 128;
 *                      workspace and phase_events are ignored.
 *   q, k, g, v       : [N, 1, H, 128] bf16 (one token per sequence); beta [N, 1, H] bf16.
 *   initial_state    : [N, H, K, V] of initial_state_dtype, or NULL for zeros.
 *   final_state      : [N, H, K, V] of final_state_dtype, or NULL to skip it;
 *                      it may alias initial_state (in-place update) when both
 *                      dtypes match.
 *   out              : [N, 1, H, 128] bf16.
 * Feeding kda_fwd's final_state in as initial_state continues a prefilled
 * sequence.  Errors as for kda_fwd (KDA_ERR_SHAPE when T != 1).  One kernel,
 * no workspace, no allocation; enqueued on `stream`.  The step itself runs in
 * fp32, but a state carried from kda_fwd is subject to kda_fwd's value range
 * ("Value range" above). */
kda_status_t kda_decode(const void *q, const void *k, const void *v, const void *g,
                        const void *beta, float scale, const float *A_log,
                        const float *dt_bias, float lower_bound,
                        const void *initial_state, void *final_state, void *out,
                        const kda_desc_t *desc, hipStream_t stream);

/* Bytes of workspace kda_bwd needs for these shapes (0 if the shapes are
 * invalid).  Pure host arithmetic.  About 355 KiB per 64-token chunk and head
 * (the forward's 72.5 KiB of intermediates, the fp32 state entering every
 * chunk and its gradient, 64 KiB each, 97 KiB of fp32 per-chunk quantities
 * and 62.5 KiB of fp16 operands for the reverse chain), plus kda_fwd's 192 KiB
 * per (segment, head) when chains are split (the reverse chains reuse it).
 * The recomputed forward produces the states only, not the output. */
size_t kda_bwd_workspace_size(const kda_desc_t *desc);

/* Enqueue the gradient of kda_fwd on `stream` and return without
 * synchronising.  The pages' kernels have no backward pass ("性能与注意事项",
 * zuobiaodaohang.com FlashKDA page: forward only); this is the vector-Jacobian
 * product of the operation stated at the top of this header: for the loss
 * gradients d_out (of out) and d_final_state (of final_state) it returns the
 * gradient of
 *     L = <d_out, out> + <d_final_state, final_state>
 * with respect to every input.  The forward is recomputed inside the call
 * (nothing from an earlier kda_fwd is needed), or, with
 * desc->forward_workspace set, only its state chain is: the intra-chunk
 * intermediates come from that kda_fwd call's workspace; with
 * desc->save_states = 1 as well, the states entering every chunk do too and
 * none of the forward is recomputed.
 *
 *   q ... lower_bound, initial_state, cu_seqlens : as for kda_fwd (the same
 *                      shapes, dtypes and rules; desc->initial_state_dtype
 *                      describes initial_state).
 *   d_out            : bf16 [B, T, H, V] (may be NULL when T == 0).
 *   d_final_state    : [N, H, K, V] of desc->final_state_dtype, or NULL for zeros.
 *   dq, dk, dg       : fp32 [B, T, H, K] outputs (gradients of q, k and of g,
 *                      the gate before activation).
 *   dv               : fp32 [B, T, H, V];  dbeta : fp32 [B, T, H] (of the logits).
 *   d_initial_state  : fp32 [N, H, K, V], or NULL to skip it.
 *   dA_log           : fp32 [H];  ddt_bias : fp32 [H, K] -- summed over every
 *                      sequence and token (each is shared by all of them).
 * All outputs are overwritten, never accumulated into.  Where the gate is
 * clamped (-exp(A_log) softplus(g + dt_bias) <= lower_bound) no gradient
 * reaches g, dt_bias or A_log; at the kink itself the clamped side is taken.
 * desc->chain_segments splits chains as for kda_fwd (the same rule and the
 * same errors; kda_fwd_chain_segments() gives the count): the recomputed
 * forward chain runs as kda_fwd's split chains (also storing the state
 * entering every chunk), and the reverse chain, whose step is affine in the
 * state's gradient with the transpose of the forward step's linear part, runs
 * in three launches too: every segment's reverse chain from a zero gradient,
 * an fp32 scan from the last segment to the first with the forward's segment
 * maps transposed (the gradient leaving every segment, and d_initial_state),
 * and every segment's reverse chain from the gradient leaving it.  The result
 * is the same function of the inputs either way, up to rounding;
 * desc->pipeline is ignored;
 * desc->phase_events, when set, is an array of 6 events recorded before the
 * first kernel (0), after the forward's intra-chunk kernel (1; right after 0
 * when desc->forward_workspace is set) and state
 * chain (2; right after 1 when the states are read as well), after the gradient's preparation kernel (3), its reverse state
 * chain (4) and its per-chunk kernel with the parameter sum (5);
 * launch_piece and the workspace rules are as for kda_fwd, with
 * kda_bwd_workspace_size() in place of kda_fwd_workspace_size().  The
 * forward's value range applies, and d_out must stay within fp16's range
 * (|d_out| < 65504): the reverse state chain takes it as an fp16 operand.  Gradients are computed from the
 * forward's fp16 intermediates and states on the matrix cores: fp32 products, or bf16 hi + lo splits of the
 * fp32 operands (good to about 2^-16 relative) where the sums do not cancel. */
kda_status_t kda_bwd(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, float scale, const float *A_log,
                     const float *dt_bias, float lower_bound,
                     const void *initial_state, const int64_t *cu_seqlens,
                     const void *d_out, const void *d_final_state,
                     float *dq, float *dk, float *dv, float *dg, float *dbeta,
                     float *d_initial_state, float *dA_log, float *ddt_bias,
                     const kda_desc_t *desc, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *kda_status_string(kda_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
