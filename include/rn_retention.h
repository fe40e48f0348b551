/*
 * rn_retention.h — C ABI of the multi-scale retention forward pass on MI355X (gfx950).
 *
 * Retention (RetNet, "Retentive Network") maps q, k, v to
 *     O_t = alpha * sum_{s<=t} gamma^(t-s) * Re[(q_t e^{i p_t theta})(k_s e^{i p_s theta})^dagger] v_s
 * (hwhale.com RetNet notes: closed form of O_n after diagonalising A; definition of
 * Q = (XW_Q) ⊙ Θ, K = (XW_K) ⊙ conj(Θ), D_nm = gamma^(n-m) for n >= m).
 * Three algebraically equal forms are exported — parallel, chunkwise and one
 * recurrent (decode) step — plus the per-head GroupNorm with the swish gate.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout (row-major, contiguous, the argument comments of the ParallelRetention /
 * RecurrentRetention / ChunkwiseRetention listings on the hwhale.com notes):
 *     q, k        [B, H, N, d_k]
 *     v, gate,out [B, H, N, d_v]
 *     state       [B, H, d_k, d_v]   always float32
 * Rotation: coordinates (2j, 2j+1) form one complex number (sdkjxy.cn walkthrough,
 * "Retention 機制": elements taken two by two as real and imaginary parts); pair j at
 * absolute position p is multiplied by e^{+i p theta_j}; k is conjugated in the
 * score. Positions are p_t = pos0 + t with 0-based t. The angle p*theta_j is formed
 * and reduced modulo 2*pi in float64 on the device before the float32 sine/cosine.
 * alpha (qk_scale) multiplies the score; it never enters the recurrent state, so
 * states are interchangeable between the chunkwise and recurrent entry points.
 *
 * Ownership: every tensor argument is a DEVICE pointer owned by the caller; the
 * library never allocates device memory on these paths (the chunkwise entry point
 * takes a caller-owned workspace). gamma and theta (in rn_desc) are HOST arrays
 * read during the call. gn_weight / gn_bias / gamma_pair are DEVICE arrays or NULL.
 * Asynchrony: each call enqueues kernels on `stream` (a hipStream_t; NULL = the
 * null stream) and returns without synchronising; device faults surface at the
 * caller's next synchronisation.
 * Errors: arguments are validated on the host before any HIP call, so an invalid
 * call launches nothing and touches no device memory. Return codes only (no
 * printing, no abort); rn_last_error() gives a thread-local message.
 * NaN/Inf in inputs propagate; they are never masked.
 * Overlapping calls that share a workspace or a state buffer race.
 */
#ifndef RN_RETENTION_H
#define RN_RETENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rn_status;
#define RN_OK               0
#define RN_ERR_INVALID_ARG (-1) /* null pointer, size < 1, odd d_k, chunk < 1, bad flags, eps < 0 ... */
#define RN_ERR_UNSUPPORTED (-2) /* valid but outside what is built: d_k > 256, d_v > 512, N > 2^30, H > 128 ... */
#define RN_ERR_HIP         (-3) /* HIP runtime / launch error; text via rn_last_error() */
#define RN_ERR_WORKSPACE   (-4) /* workspace NULL or smaller than rn_chunkwise_workspace_bytes() */
#define RN_ERR_EXCHANGE    (-5) /* reported by rn_chunkwise_check: a wait between the workgroups of
                                   the sequential chunkwise kernel hit its time limit (1 s); the
                                   call's out and state_out hold NaN where they were written */
#define RN_ERR_NONFINITE   (-6) /* reported by rn_chunkwise_check: a matrix-core chunkwise
                                   schedule produced a non-finite output or final state: a
                                   non-finite input, or a value beyond its half-precision operand
                                   range (see rn_retention_chunkwise) */

typedef int32_t rn_dtype;
#define RN_F32  0   /* IEEE float32 */
#define RN_BF16 1   /* bfloat16 (upper half of a float32) */

/* flags */
#define RN_NORM_D_ROW (1u << 0) /* parallel only: D_nm / sqrt(sum_{i<=n} D_ni)  (hwhale notes, 2nd rescaling) */
#define RN_NORM_R_ROW (1u << 1) /* parallel only: R_nm / max(|sum_{i<=n} R_ni|, 1) (hwhale notes, 3rd rescaling) */
#define RN_EPI_GN     (1u << 2) /* per-(token, head) GroupNorm over d_v (hwhale notes, multi-head paragraph) */
#define RN_EPI_GATE   (1u << 3) /* out = GN(.) * swish(gate); requires RN_EPI_GN (m0nads notes, swish gate) */
#define RN_FORCE_GENERIC (1u << 8) /* take the kernels that read their operands through
                                      pointers with 64-bit offsets (no per-head size bound):
                                      plain float32 arithmetic for the forward forms; for the
                                      backward, float32 staging with half-operand MFMA
                                      products when the inputs are bf16. For testing and for
                                      shapes past the other kernels' bounds. */
#define RN_CHUNK_PARALLEL (1u << 9) /* chunkwise: the two-kernel chunk-parallel pair (state
                                       snapshots per 256 tokens, then all chunks' outputs in
                                       parallel) instead of the single sequential kernel; same
                                       result, another workspace size. Without any schedule flag
                                       it runs only for gamma_pair at d_k 256, d_v 512 (where the
                                       sequential kernel does not apply because gamma^32 < 2^-6,
                                       the segmented schedule runs) */
#define RN_CHUNK_SEGMENTED (1u << 10) /* chunkwise, bf16 with d_k 256, d_v 512 and one decay per
                                       head: the segmented schedule (segment-local states per
                                       2048 tokens, a scan over segments, then all chunks'
                                       outputs in parallel); same result, another workspace size,
                                       no limit on gamma. Elsewhere the flag is ignored. At most
                                       one of RN_CHUNK_PARALLEL and RN_CHUNK_SEGMENTED may be set. */
#define RN_TEST_FORCE_TIMEOUT (1u << 12) /* testing only: every cross-workgroup wait of the
                                       sequential chunkwise kernel gives up at once, as if its time
                                       limit had passed, so that the error path (NaN outputs,
                                       RN_ERR_EXCHANGE from rn_chunkwise_check) can be exercised
                                       while every kernel still ends normally; other paths ignore it */

typedef struct rn_desc {
    int32_t B;             /* batch, >= 1 */
    int32_t H;             /* heads, 1..128 */
    int32_t N;             /* tokens; must be 1 for rn_retention_recurrent_step */
    int32_t d_k;           /* query/key head dim: even, 2..256 */
    int32_t d_v;           /* value head dim: 1..512 */
    rn_dtype in_dtype;     /* dtype of q, k, v, gate */
    rn_dtype out_dtype;    /* dtype of out; accumulation is always float32 */
    uint32_t flags;        /* RN_* flags above */
    int64_t pos0;          /* absolute position of token 0 (the step's position for decode), >= 0 */
    float qk_scale;        /* alpha; finite */
    float gn_eps;          /* GroupNorm epsilon, >= 0 (used with RN_EPI_GN) */
    const float* gamma;    /* HOST [H]: per-head decay, 0 < gamma <= 1 (hwhale notes: one gamma per head) */
    const float* theta;    /* HOST [d_k/2]: one angle per coordinate pair, finite */
    const float* gn_weight;/* DEVICE [H*d_v] GroupNorm scale, or NULL (= 1) */
    const float* gn_bias;  /* DEVICE [H*d_v] GroupNorm shift, or NULL (= 0) */
    const float* gamma_pair;
    /* DEVICE [H * d_k/2] float32, 4-byte aligned, or NULL. When set, each head keeps
     * one decay per coordinate pair instead of one number: gamma_pair[h*d_k/2 + j]
     * decays pair j (state rows 2j and 2j+1) of head h, and `gamma` is not read (it may
     * be NULL). This is the form the pages state before simplifying the decay to a
     * scalar (hwhale notes: A diagonalised as Λ(γe^{iθ})Λ^{-1}; m0nads notes,
     * "Retention": γ and θ as two vectors), under which the score becomes
     *     s_ts = alpha * Re sum_j gamma_j^(t-s) zq_{t,j} conj(zk_{s,j}).
     * Values must lie in (0, 1]; they are read by the kernels, so the host cannot check
     * them (other values give unspecified numbers, never an access outside the
     * buffers). Accepted by the parallel form (not with RN_NORM_D_ROW, whose rescaling
     * is defined by the scalar decay), the chunkwise forms and the decode steps; the
     * chunkwise backward returns RN_ERR_UNSUPPORTED. */
} rn_desc;

/*
 * Bytes of device workspace rn_retention_parallel needs for `desc` (0 for an invalid
 * descriptor or when the call needs none). The MFMA path stores the rotated k and the
 * blocked, transposed v in half precision there: 2*B*H*ceil(N/64)*64*(d_k + d_v) bytes,
 * linear in N (q is rotated where it is read).
 */
size_t rn_parallel_workspace_bytes(const rn_desc* desc);

/*
 * Parallel form: O = ((alpha * Qh Kh^T) ⊙ D) V with the optional row rescalings,
 * then the optional GroupNorm / gate epilogue.
 * (hwhale notes: parallel-form equation, the ParallelRetention listing and the list
 * of three rescalings; rescalings are applied in the listed order as per-row
 * scalars: c_t = 1/sqrt(sum_{m<=t} gamma^m) for RN_NORM_D_ROW, then division by
 * max(|signed row sum of R|, 1) for RN_NORM_R_ROW.)
 * q, k: [B,H,N,d_k]; v: [B,H,N,d_v]; gate: [B,H,N,d_v] (required iff RN_EPI_GATE,
 * else ignored); out: [B,H,N,d_v] in out_dtype. No state: the parallel form starts
 * from S = 0. workspace: device buffer of at least rn_parallel_workspace_bytes(desc)
 * bytes, 256-byte aligned (may be NULL when that size is 0); contents ignored.
 * Precision and range. bf16 inputs with d_k = 256, d_v = 512 and N * 2048 < 2^31
 * (N below 1,048,576) take matrix-core products on IEEE-half operands with float32
 * accumulation: alpha*Qh, Kh, v and the decayed scores alpha*gamma^(t-s) Qh_t.Kh_s
 * must stay below 65504 in magnitude (no decay factor is folded into the operands
 * here); other inputs run float32 kernels.
 */
rn_status rn_retention_parallel(const rn_desc* desc, const void* q, const void* k,
                                const void* v, const void* gate, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace rn_retention_chunkwise needs for `desc` (independent of
 * N). Returns 0 for an invalid descriptor.
 */
size_t rn_chunkwise_workspace_bytes(const rn_desc* desc, int32_t chunk);

/*
 * Chunkwise recurrent form (hwhale notes: chunkwise equation with
 * xi_j = gamma^(j+1), and the ChunkwiseRetention listing; m0nads notes,
 * "Chunkwise representation"). For chunk i of length L (the last may be shorter):
 *   O_[i]   = alpha * ((Qh Kh^T ⊙ D) V + (Qh S_i) ⊙ xi),  xi_j = gamma^(j+1)
 *   S_{i+1} = gamma^L S_i + sum_j gamma^(L-1-j) Kh_j^T V_j
 * then the optional GroupNorm / gate epilogue per token. The result does not
 * depend on `chunk` beyond rounding (every chunk length gives the same O and
 * S_final); the kernels carry the state at a granularity of their own.
 * state_in:  [B,H,d_k,d_v] float32 initial state S_0, or NULL for zeros.
 * state_out: [B,H,d_k,d_v] float32 final state, or NULL to discard; may equal
 *            state_in (updated in place).
 * workspace: device buffer of at least rn_chunkwise_workspace_bytes(desc, chunk)
 *            bytes, 256-byte aligned; contents on entry are ignored.
 * RN_NORM_D_ROW / RN_NORM_R_ROW are rejected (parallel form only).
 * Precision and range. float32 inputs run float32 kernels. bf16 inputs with d_k = 256 and
 * d_v in {256, 512} (the sequential kernel, the default) or d_v = 512 (the segmented and
 * chunk-parallel schedules) take matrix-core products whose operands are rounded to IEEE
 * half with float32 accumulation: the rotated q and k, v, the decayed scores and the copy
 * of the state used by the cross term must stay below 65504 in magnitude. In the
 * sequential kernel the rotated rows also carry decay factors up to gamma^-32 (at most 64,
 * since that kernel takes gamma^32 >= 2^-6), so |alpha q|, |k| < 1000 and |state| < 2^15
 * keep every operand in range; RetNet-scaled data sits many orders of magnitude below.
 * Outside that range the result is not finite; rn_chunkwise_check then reports
 * RN_ERR_NONFINITE (all three matrix-core schedules keep the status word).
 */
rn_status rn_retention_chunkwise(const rn_desc* desc, int32_t chunk, const void* q,
                                 const void* k, const void* v, const void* gate,
                                 const float* state_in, float* state_out, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * rn_retention_chunkwise without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a 32 MiB buffer the library keeps in device memory, one per
 * GPU, from the first call on that GPU until the process ends. The call allocates nothing.
 * Arguments, routing and results are those of rn_retention_chunkwise (chunkwise equation
 * of the hwhale notes, as above); a call whose rn_chunkwise_workspace_bytes exceeds 32 MiB
 * is rejected with RN_ERR_UNSUPPORTED before any launch (the default sequential kernel
 * with d_v = 512 needs at most 17 MiB, for any number of heads).
 * Every call on one GPU shares its buffer: calls that overlap on one GPU (on different
 * streams, or from several threads without ordering) race and their results are
 * undefined; calls ordered on one stream are safe. The buffer keeps the last call's
 * contents; the kernels clear what must start at zero themselves.
 */
rn_status rn_retention_chunkwise_noalloc(const rn_desc* desc, int32_t chunk, const void* q,
                                         const void* k, const void* v, const void* gate,
                                         const float* state_in, float* state_out, void* out,
                                         void* stream);

/*
 * Chunkwise form over a padded batch of sequences that start at positions of their own
 * and hold numbers of tokens of their own: the prompt (prefill) half of serving, whose
 * state_out the decode steps below continue from. (eepw translation, "inference cost"
 * section with Fig. 6: decoding runs on the recurrent representation, so its cost per
 * token does not grow with the length already processed; hwhale notes, chunkwise and
 * recurrent equations: the state after a prefix is all the recurrence needs.)
 * Sequence b takes rows [0, lengths[b]) of its [N, .] slices of q, k, v, gate and
 * out; token t of it sits at absolute position pos[b] + t. Everything else is as in
 * rn_retention_chunkwise, with N replaced by lengths[b] per sequence:
 *   out rows t >= lengths[b] are not written;
 *   state_out[b] is the state after lengths[b] tokens (state_in[b], or zeros, when
 *   lengths[b] == 0).
 * pos:     DEVICE int64 [B], 8-byte aligned, or NULL for desc->pos0 everywhere. The
 *          values are not checked (they move no memory access); angles are formed
 *          and reduced in float64 as for pos0, so |p| <= 2^40 keeps them accurate.
 * lengths: DEVICE int32 [B], 4-byte aligned, or NULL for N everywhere. Each value is
 *          clamped to [0, N] on the device, so no value can reach outside the padded
 *          buffers.
 * The same workspace size as rn_retention_chunkwise applies
 * (rn_chunkwise_workspace_bytes).
 */
rn_status rn_retention_chunkwise_varlen(const rn_desc* desc, int32_t chunk,
                                        const int64_t* pos, const int32_t* lengths,
                                        const void* q, const void* k, const void* v,
                                        const void* gate, const float* state_in,
                                        float* state_out, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * One recurrent (decode) step at absolute position desc->pos0 (desc->N must be 1):
 *   S <- gamma S + Kh^T v   (in place),   o = alpha Qh S,   optional GN / gate.
 * (hwhale notes: recurrent equations and the RecurrentRetention listing, which
 * includes the current token and sums over d_k.)
 * q, k: [B,H,1,d_k]; v, gate, out: [B,H,1,d_v]; state: [B,H,d_k,d_v] float32 in/out.
 */
rn_status rn_retention_recurrent_step(const rn_desc* desc, const void* q, const void* k,
                                      const void* v, const void* gate, float* state,
                                      void* out, void* stream);

/*
 * One recurrent (decode) step with a position per sequence: the token of sequence b
 * sits at pos[b] (batched decode of sequences of different lengths, e.g. continuing
 * from rn_retention_chunkwise_varlen with pos[b] = its pos[b] + lengths[b]).
 * Otherwise identical to rn_retention_recurrent_step; desc->pos0 is not used.
 * (eepw translation, "inference cost" section: batched decode on the recurrent
 * representation; hwhale notes, recurrent equations.)
 * pos: DEVICE int64 [B], 8-byte aligned, required; the values are not checked (they
 *      move no memory access); |p| <= 2^40 keeps the float64-reduced angles accurate.
 *      Keeping the positions on the device lets a decode loop advance them without
 *      host work.
 */
rn_status rn_retention_recurrent_step_at(const rn_desc* desc, const int64_t* pos,
                                         const void* q, const void* k, const void* v,
                                         const void* gate, float* state, void* out,
                                         void* stream);

/*
 * Bytes of device workspace rn_retention_chunkwise_backward needs for `desc`: the state
 * at every 256-token chunk start and the gradient reaching it (float32, d_k x d_v each,
 * per head), and the gradient of the pre-GroupNorm output (float32 [B,H,N,d_v]).
 * Returns 0 for an invalid descriptor.
 */
size_t rn_chunkwise_backward_workspace_bytes(const rn_desc* desc, int32_t chunk);

/*
 * Gradients of the chunkwise call (same descriptor, inputs and chunk as the forward call)
 * given the gradient of a loss with respect to its output and, optionally, its final
 * state: the chunkwise recurrence differentiated, the GroupNorm and gate included
 * (hwhale notes: chunkwise and recurrent equations, ChunkwiseRetention listing; GroupNorm
 * per head and swish gate of the multi-scale layer). Recomputes the forward pass
 * internally; nothing from the forward call is needed.
 * dout:       [B,H,N,d_v] in out_dtype; dstate_out: [B,H,d_k,d_v] float32 or NULL (zero).
 * dq, dk:     [B,H,N,d_k], dv: [B,H,N,d_v], in in_dtype (written).
 * dgate:      [B,H,N,d_v] in in_dtype, required iff RN_EPI_GATE (written).
 * dstate_in:  [B,H,d_k,d_v] float32 or NULL (not computed); gradient for state_in.
 * dgn_weight, dgn_bias: DEVICE float32 [H*d_v] or NULL, written when RN_EPI_GN (sums over
 *             the batch and the rows); ignored otherwise.
 * workspace:  at least rn_chunkwise_backward_workspace_bytes(desc, chunk), 256-byte aligned.
 * Arithmetic: float32 inputs take float32 products throughout.
 * bf16 inputs take matrix-core products (16x16x32 f16 MFMA, float32 accumulation): with
 * d_k and d_v multiples of 8, v, dv, dout, gate and dgate 16-byte aligned and q and k
 * 4-byte aligned, every operand is
 * rounded to IEEE half (so, as for the forward, operands must stay below 65504 in
 * magnitude); other bf16 shapes stage float32 operands and take the same products. Every
 * shape and dtype the forward accepts is accepted.
 */
rn_status rn_retention_chunkwise_backward(const rn_desc* desc, int32_t chunk, const void* q,
                                          const void* k, const void* v, const void* gate,
                                          const float* state_in, const void* dout,
                                          const float* dstate_out, void* dq, void* dk, void* dv,
                                          void* dgate, float* dstate_in, float* dgn_weight,
                                          float* dgn_bias, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * Gated multi-scale retention layer (m0nads notes and hwhale notes, "Gated Multi-Scale
 * Retention"; sdkjxy walkthrough, the MSR block):
 *     Q = X W_Q,  K = X W_K,  V = X W_V,  G = X W_G
 *     Y_h = GroupNorm_h(Retention_h(Q_h, K_h, V_h))      (chunkwise form, this desc)
 *     out = (swish(G) ⊙ Concat_h Y_h) W_O
 * where head h owns columns [h d_k, (h+1) d_k) of Q and K and [h d_v, (h+1) d_v) of V
 * and G. The pages state W_G and W_O as d x d; here they are d_model x (H d_v) and
 * (H d_v) x d_model, which is d x d when H d_v = d_model.
 * Arguments (DEVICE, row-major, caller-owned):
 *     x    [B, N, d_model] bf16            w_q, w_k [d_model, H*d_k] bf16
 *     w_v, w_g [d_model, H*d_v] bf16       w_o  [H*d_v, d_model] bf16
 *     out  [B, N, d_model] in desc->out_dtype (bf16 or float32)
 *     state_in / state_out [B, H, d_k, d_v] float32 or NULL, as for rn_retention_chunkwise.
 * desc: B, H, N, d_k, d_v, decays (gamma or gamma_pair), theta, pos0, qk_scale, GroupNorm
 * parameters and flags as for rn_retention_chunkwise; in_dtype must be RN_BF16 (else
 * RN_ERR_UNSUPPORTED); RN_EPI_GN applies the per-head GroupNorm, RN_EPI_GATE the gate
 * (w_g is then required; without the flag w_g is not read). d_v must be a multiple of 8.
 * The four projections and W_O run as rocBLAS GEMMs with bf16 operands and float32
 * accumulation; Q, K, V, G and the heads' outputs are held in bf16 in the workspace
 * (rn_msr_layer_workspace_bytes, linear in B*N), then the retention kernels run as in
 * rn_retention_chunkwise. The first call on a host thread and device creates a rocBLAS
 * handle, which keeps its own device memory for the life of the process.
 * Errors: as for rn_retention_chunkwise; a rocBLAS failure returns RN_ERR_HIP.
 */
size_t rn_msr_layer_workspace_bytes(const rn_desc* desc, int32_t d_model, int32_t chunk);
rn_status rn_msr_layer_forward(const rn_desc* desc, int32_t d_model, int32_t chunk,
                               const void* x, const void* w_q, const void* w_k,
                               const void* w_v, const void* w_g, const void* w_o,
                               const float* state_in, float* state_out, void* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Standalone per-head GroupNorm (+ swish gate):
 *   y = (x - mean) / sqrt(var + eps) * w + b over the d_v channels of each (b,h,t),
 *   out = y * g * sigmoid(g) if gate != NULL, else y.
 * (hwhale notes, multi-head paragraph: GroupNorm per head; m0nads notes, "Gated
 * Multi-Scale Retention": swish gate.) x, gate, out: [B,H,N,d_v]; x and gate in
 * in_dtype, out in out_dtype; w, b: DEVICE [H*d_v] or NULL. out may equal x when
 * both dtypes match.
 */
rn_status rn_groupnorm_gate(int32_t B, int32_t H, int32_t N, int32_t d_v,
                            rn_dtype in_dtype, rn_dtype out_dtype, const void* x,
                            const void* gate, const float* w, const float* b, float eps,
                            void* out, void* stream);

/*
 * Status of a completed rn_retention_chunkwise / rn_retention_chunkwise_varlen call (same
 * desc and chunk), read from its workspace: RN_OK; RN_ERR_EXCHANGE if a wait between the
 * workgroups of the sequential kernel hit its time limit (its outputs are then NaN);
 * RN_ERR_NONFINITE if the call's matrix-core schedule (sequential, segmented or
 * chunk-parallel) produced a non-finite output or final state. The float32 kernels
 * record nothing and give RN_OK.
 * workspace: the call's device workspace, in which case `stream` (the call's stream) is
 * synchronised and the status word copied to the host; or a host copy of at least its
 * first 256 bytes, read directly. Must be called before the workspace is reused.
 * (Host calls that cannot block until the GPU finishes should keep using the outputs'
 * own checks instead.)
 */
rn_status rn_chunkwise_check(const rn_desc* desc, int32_t chunk, const void* workspace,
                             size_t workspace_bytes, void* stream);

/* Static name of a status code. */
const char* rn_status_str(rn_status s);
/* Message describing the last failure on the calling thread ("" if none). */
const char* rn_last_error(void);
/* Library version, e.g. "0.1.0". */
const char* rn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RN_RETENTION_H */
