/*
 * gdn.h -- C ABI of the Gated DeltaNet token-mixer hot path on AMD Instinct
 * MI355X (gfx950).
 *
 * The mixer computes, per sequence b, value head h and token t:
 *
 *   u     = silu(sum_{j<4} w[c,j] x[t+j-3,c])  on the q, k and v channels
 *           ("Qwen3.8-27B" model spec, compute-graph node gdn.conv; "How
 *           Qwen3.5 works" §9.3);
 *   k^    = u_k / sqrt(sum u_k^2 + eps_l2),  q^ = u_q / sqrt(sum u_q^2 + eps_l2)
 *           / sqrt(Dk)  ("How Qwen3.5 works" §9.4; model spec node gdn.core),
 *           value head h reading key head h / (Hv/Hk);
 *   S_t   = e^{g_t} S_{t-1} + k^ d^T,  d = beta_t (v_t - e^{g_t} S_{t-1}^T k^),
 *   o_t   = S_t^T q^   ("How Qwen3.5 works" §9.6: decay, predict, correct,
 *           read; the model spec's gdn.core writes the same rule transposed);
 *   y_t   = w * o_t / sqrt(mean(o_t^2) + eps_norm) * silu(z_t)
 *           (model spec node gdn.norm; "How Qwen3.5 works" §9.9).
 *
 * State layout.  The recurrent state is fp32 [B][Hv][Dk][Dv], K-major: element
 * [b][h][i][j] is key dimension i, value dimension j (the orientation
 * S in R^{dk x dv} of "How Qwen3.5 works" §9.1).  The conv state is bf16
 * [B][3][Cc], Cc = 2*Hk*Dk + Hv*Dv: the raw (pre-conv) inputs of the last
 * three tokens, oldest first, channels ordered q heads, k heads, v heads
 * ("How Qwen3.5 works" §13.1/§13.3: the decode step shifts this window).
 *
 * Conventions for every call.
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous; bf16
 *    tensors are passed as uint16_t bit patterns.  The caller owns every
 *    buffer.  The library allocates no device memory, keeps no per-call state
 *    between calls, and never synchronises (gdn_prefill_check, which waits on
 *    the stream it is given, is the one exception, and says so).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it; results are visible once the caller syncs it.
 *  - Every argument is checked on the host before any HIP call; a failed
 *    check returns a negative status and enqueues nothing.  No exception
 *    crosses the ABI and the library never prints.
 *  - Pointers to bf16 tensors and to the state must be 16-byte aligned; g and
 *    beta 4-byte aligned.
 *  - Supported: Dk = Dv = 128, Hv a multiple of Hk, conv_width 0 or 4.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define GDN_OK 0
#define GDN_EINVAL (-1)      /* null or misaligned pointer, bad size, aliasing */
#define GDN_EUNSUPPORTED (-2) /* a head width other than 128, a conv width other than 0/4 */
#define GDN_EHIP (-3)        /* a HIP call or kernel launch failed */
#define GDN_EWORKSPACE (-4)  /* workspace too small */
#define GDN_ETIMEOUT (-5)    /* gdn_prefill_check: a bounded wait between workgroups timed out; outputs are wrong */
#define GDN_ESKIPPED (-6)    /* gdn_prefill_check: a packed sequence with invalid bounds was skipped */

/* flags */
#define GDN_NO_NORM 1u /* return the raw read-out o instead of the gated RMSNorm (z, norm_w unused) */
#define GDN_PACKED 2u  /* packed sequences: B sequences of different lengths, T tokens in all (gdn_prefill_packed) */

typedef struct gdn_shape {
    int32_t B;          /* sequences, >= 1 */
    int32_t T;          /* tokens per sequence, >= 1 (gdn_decode_step ignores it; gdn_decode_multi: 1..8) */
    int32_t Hk;         /* key / query heads, >= 1 */
    int32_t Hv;         /* value heads, a multiple of Hk */
    int32_t Dk;         /* key head width: must be 128 */
    int32_t Dv;         /* value head width: must be 128 */
    int32_t conv_width; /* 0: q, k, v enter the rule as given (no conv, no SiLU); 4: width-4 causal conv + SiLU */
    uint32_t flags;     /* GDN_NO_NORM, GDN_PACKED (prefill only), both or 0 */
    float eps_l2;       /* eps inside the q/k L2-norm root (1e-6 on the pages) */
    float eps_norm;     /* eps of the gated RMSNorm (1e-6 on the pages) */
    int32_t prefill_segments; /* prefill of an even batch: 0 lets the library choose, 1 runs the plain
                                 sequential pass, n >= 2 splits every sequence into n segments (the
                                 two-level scan; capped at the chunk count); must be 0 or 1 with
                                 GDN_PACKED; ignored by the decode calls */
} gdn_shape;

/*
 * Zero the recurrent state [B][Hv][Dk][Dv] fp32 and, when conv_state is not
 * NULL, the conv state [B][3][Cc] bf16: the state before the first token
 * ("How Qwen3.5 works" §9.8 starts from S_0 = 0; §9.10's reference loop
 * allocates zeros when no state is given).
 */
int gdn_state_init(const gdn_shape *shape, float *state, uint16_t *conv_state, void *stream);

/*
 * Bytes of device workspace gdn_prefill (gdn_prefill_packed, when the shape
 * carries GDN_PACKED) needs for `shape` (written to *bytes).
 * The workspace starts with a 256-byte header whose first 32-bit word is the
 * error word (see gdn_prefill_check), then the exchange area the workgroups of
 * one head trade through (the per-row sums of squares the gated RMSNorm needs
 * from every value slice, and work-queue tickets), then the state-independent
 * chunk operands that the first kernel of a call computes for the sequential
 * pass ("How Qwen3.5 works" §9.11): the normalised q/k rows in both the row and
 * the transposed fragment order (fp16, 3*B*T*Hk*Dk values), and per (chunk,
 * value head) the packed lower-triangular T diag(beta) and (Q K^T) o R blocks
 * and the decay vectors.  Returns GDN_EINVAL for a shape gdn_prefill would
 * reject.
 */
int gdn_prefill_workspace_size(const gdn_shape *shape, size_t *bytes);

/*
 * Prefill: run T tokens of every sequence through the mixer, chunked into
 * blocks of 64 tokens ("How Qwen3.5 works" §9.11: the unit lower-triangular
 * chunk form of the same recurrence; a partial last chunk is allowed).
 *
 * With few (sequence, value head) pairs and long sequences the library splits
 * each sequence into segments that run at the same time: a segment's effect on
 * the state is affine in its start state (the chunk form's update is linear in
 * S), so each segment is run from zero together with its transition map, the
 * maps are chained, and what each start state adds to the outputs is applied
 * last.  The workspace is then larger (gdn_prefill_workspace_size accounts for
 * it).  shape->prefill_segments overrides the choice: 1 never splits, n >= 2
 * asks for n segments.
 *
 *  q, k           [B][T][Hk][128] bf16
 *  v, z           [B][T][Hv][128] bf16 (z may be NULL iff GDN_NO_NORM)
 *  g, beta        [B][T][Hv] fp32: log-decay (alpha = e^g) and write strength
 *  conv_w         [Cc][4] bf16, tap 3 multiplies the current token (NULL iff conv_width == 0)
 *  norm_w         [128] bf16, the gated-norm weight, applied as w (NULL iff GDN_NO_NORM)
 *  state_in       [B][Hv][128][128] fp32, or NULL for zeros
 *  conv_state_in  [B][3][Cc] bf16, or NULL for zeros (must be NULL when conv_width == 0)
 *  o              [B][T][Hv][128] bf16 output (round to nearest even)
 *  state_out      [B][Hv][128][128] fp32 output; may be the same buffer as state_in
 *  conv_state_out [B][3][Cc] bf16, the raw inputs of the last three tokens, or
 *                 NULL; must not overlap conv_state_in
 *  workspace      device memory of at least gdn_prefill_workspace_size() bytes,
 *                 16-byte aligned, with no required contents: every call clears
 *                 the header and the exchange area before anything reads them
 *                 and overwrites the operand blocks.  Calls that may run at the
 *                 same time must not share a workspace.  After the call its error
 *                 word (the first 32-bit word) holds this call's error bits: bit 0
 *                 says a bounded wait between workgroups timed out (the affected
 *                 output rows are then NaN and the call's results are wrong),
 *                 bit 1 that gdn_prefill_packed skipped a sequence with invalid
 *                 bounds.
 *
 * `o` must not overlap any input.  Returns GDN_OK once the work is enqueued.
 */
int gdn_prefill(const gdn_shape *shape, const uint16_t *q, const uint16_t *k,
                const uint16_t *v, const float *g, const float *beta, const uint16_t *z,
                const uint16_t *conv_w, const uint16_t *norm_w, const float *state_in,
                const uint16_t *conv_state_in, uint16_t *o, float *state_out,
                uint16_t *conv_state_out, void *workspace, size_t workspace_bytes,
                void *stream);

/*
 * Wait for `stream` and read the error word that the last prefill call on
 * `workspace` left (the calls above never wait; this one synchronises the
 * stream, so call it when the results are needed anyway).  Returns GDN_OK when
 * the word is zero, GDN_ETIMEOUT when a bounded wait between workgroups timed
 * out (the outputs are wrong: the rows it affected are NaN), GDN_ESKIPPED when
 * only a packed sequence with invalid bounds was skipped, GDN_EINVAL for a null
 * workspace or one smaller than 256 bytes, GDN_EHIP if the wait or the copy
 * failed.  "How Qwen3.5 works" §9.10's reference loop rejects bad input rather
 * than returning quietly wrong results; this is how a caller learns of the
 * failures that only the device can see.
 */
int gdn_prefill_check(const void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine): its workspace is a file-scope device array
 * of the library, GDN_STATIC_SCRATCH_BYTES (128 MiB) on every GPU the library
 * runs on, held until the process ends.  Its address on a device is looked up
 * once, on the first call with that device current, after the host checks.
 *
 * Arguments, layouts, results and errors are those of gdn_prefill (even
 * batches only).  Where the library would choose the two-level scan
 * (prefill_segments = 0) and its workspace does not fit
 * GDN_STATIC_SCRATCH_BYTES, the call runs the plain sequential pass instead
 * (the same results to rounding).  A shape whose workspace still exceeds
 * GDN_STATIC_SCRATCH_BYTES is rejected with GDN_EWORKSPACE before any HIP
 * call (the 0.8B-shaped layer, 16/16 heads, fits up to T = 8192 tokens).
 * Every call on one GPU uses the same array, which keeps the last call's
 * contents; each call clears what must start at zero.  Calls that overlap in
 * time on one GPU (several streams, several host threads) race on the array
 * and give wrong results: serialise them.  Its error word cannot be read with
 * gdn_prefill_check (the caller holds no workspace pointer); a timed-out wait
 * shows as NaN rows, as for gdn_prefill.
 */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
int gdn_prefill_no_workspace(const gdn_shape *shape, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, const float *g, const float *beta, const uint16_t *z,
                             const uint16_t *conv_w, const uint16_t *norm_w, const float *state_in,
                             const uint16_t *conv_state_in, uint16_t *o, float *state_out,
                             uint16_t *conv_state_out, void *stream);

/*
 * One decode step: one new token per sequence, updating the recurrent state
 * and the conv window in place ("How Qwen3.5 works" §13.3: each linear layer
 * shifts its conv state and takes one recurrent step; the state is
 * overwritten, nothing grows).
 *
 *  q, k        [B][Hk][128] bf16;  v, z [B][Hv][128] bf16 (z NULL iff GDN_NO_NORM)
 *  g, beta     [B][Hv] fp32
 *  conv_w      [Cc][4] bf16 (NULL iff conv_width == 0);  norm_w [128] bf16
 *  state       [B][Hv][128][128] fp32, read and overwritten in place
 *  conv_state  [B][3][Cc] bf16, read and shifted in place (NULL iff conv_width == 0)
 *  o           [B][Hv][128] bf16 output
 *
 * shape->T is ignored.  `o` must not overlap any input.
 */
int gdn_decode_step(const gdn_shape *shape, const uint16_t *q, const uint16_t *k,
                    const uint16_t *v, const float *g, const float *beta, const uint16_t *z,
                    const uint16_t *conv_w, const uint16_t *norm_w, float *state,
                    uint16_t *conv_state, uint16_t *o, void *stream);

/*
 * The same two calls taking the raw gate inputs in place of g and beta ("How
 * Qwen3.5 works" §9.5: beta_t = sigmoid(b_t) and g_t = -exp(A_log)
 * softplus(a_t + dt_bias), per value head, computed in fp32 inside the kernels):
 *
 *  a, b      gate logits, fp32, laid out as g and beta ([B][T][Hv] for prefill,
 *            [B][Hv] for decode); 4-byte aligned
 *  A_log     [Hv] fp32 per value head (alpha_t = exp(g_t) multiplies the state)
 *  dt_bias   [Hv] fp32 per value head
 *
 * Every other argument, check and status is that of gdn_prefill or
 * gdn_decode_step; the four gate arrays count as inputs for the aliasing checks.
 */
int gdn_prefill_gate_logits(const gdn_shape *shape, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const float *a, const float *b, const float *A_log,
                            const float *dt_bias, const uint16_t *z, const uint16_t *conv_w,
                            const uint16_t *norm_w, const float *state_in,
                            const uint16_t *conv_state_in, uint16_t *o, float *state_out,
                            uint16_t *conv_state_out, void *workspace, size_t workspace_bytes,
                            void *stream);
int gdn_decode_step_gate_logits(const gdn_shape *shape, const uint16_t *q, const uint16_t *k,
                                const uint16_t *v, const float *a, const float *b,
                                const float *A_log, const float *dt_bias, const uint16_t *z,
                                const uint16_t *conv_w, const uint16_t *norm_w, float *state,
                                uint16_t *conv_state, uint16_t *o, void *stream);

/*
 * T decode steps in one call: T new tokens per sequence (1 <= T <= 8), for
 * checking draft tokens in one pass ("Qwen3.5-4B architecture", multi-token
 * prediction: a draft head proposes tokens and one forward pass verifies
 * them).  The tokens run through the recurrence one after the other exactly
 * as T calls of gdn_decode_step would; the state is read once and stays on
 * chip between the tokens.  A recurrent state cannot be rewound, so rolling
 * back to an accepted prefix needs snapshots ("How Qwen3.5 works" §13.5):
 * when state_snaps / conv_snaps are given, the state and the conv window
 * after each token t < T-1 are written there; after the last token they go
 * to state / conv_state in place.  Accepting tokens 0..j (j < T-1) then means
 * continuing from snapshot j.
 *
 *  shape->T    tokens per sequence, 1..8
 *  q, k        [B][T][Hk][128] bf16;  v, z, o  [B][T][Hv][128] bf16
 *  g, beta     [B][T][Hv] fp32 (gdn_decode_multi_gate_logits: the logits a, b,
 *              with A_log and dt_bias [Hv] as in gdn_prefill_gate_logits)
 *  state       [B][Hv][128][128] fp32, read, then overwritten with the state
 *              after the last token
 *  conv_state  [B][3][Cc] bf16, read, then overwritten with the window after
 *              the last token (NULL iff conv_width == 0)
 *  state_snaps [T-1][B][Hv][128][128] fp32 or NULL: snapshot t (one state
 *              tensor of the same layout as state) after token t
 *  conv_snaps  [T-1][B][3][Cc] bf16 or NULL (must be NULL when conv_width == 0)
 *
 * With T = 1 the snapshots are not used and the call is gdn_decode_step.  The
 * snapshots are outputs: they must not overlap any other argument.  Returns
 * GDN_EINVAL for T outside 1..8 and GDN_EUNSUPPORTED when T and Hv/Hk need
 * more on-chip memory than one workgroup has; otherwise as gdn_decode_step.
 */
int gdn_decode_multi(const gdn_shape *shape, const uint16_t *q, const uint16_t *k,
                     const uint16_t *v, const float *g, const float *beta, const uint16_t *z,
                     const uint16_t *conv_w, const uint16_t *norm_w, float *state,
                     uint16_t *conv_state, uint16_t *o, float *state_snaps, uint16_t *conv_snaps,
                     void *stream);
int gdn_decode_multi_gate_logits(const gdn_shape *shape, const uint16_t *q, const uint16_t *k,
                                 const uint16_t *v, const float *a, const float *b,
                                 const float *A_log, const float *dt_bias, const uint16_t *z,
                                 const uint16_t *conv_w, const uint16_t *norm_w, float *state,
                                 uint16_t *conv_state, uint16_t *o, float *state_snaps,
                                 uint16_t *conv_snaps, void *stream);

/*
 * Prefill over packed sequences of different lengths, one call for the whole
 * batch.  The shape carries GDN_PACKED; B is the number of sequences and T the
 * number of tokens of all of them together.  Sequence b owns the token rows
 * cu_seqlens[b] .. cu_seqlens[b+1] - 1 of the token-major tensors; its
 * recurrent state and conv window start from its own state_in / conv_state_in
 * entries at its first token and end in its own state_out / conv_state_out
 * entries, exactly as if it had been run alone through gdn_prefill with
 * B = 1, T = its length ("How Qwen3.5 works" §12.2: when several samples are
 * packed into one sequence, the conv and recurrent states must stop at every
 * sample boundary, and a packed run must agree with the samples run one by
 * one).  Chunks of 64 tokens start at each sequence's first token.
 *
 *  cu_seqlens     [B + 1] int32, DEVICE memory, 4-byte aligned: cu_seqlens[0] = 0,
 *                 cu_seqlens[B] = T, every sequence at least one token long
 *                 (cu_seqlens[b] < cu_seqlens[b+1]).  Read by the kernels, so the
 *                 call does not synchronise; a sequence whose bounds break this
 *                 rule is skipped (nothing of it is read or written, its outputs
 *                 keep their contents) and every other sequence is still computed.
 *                 Offsets that decrease anywhere (cu_seqlens[b] > cu_seqlens[b+1]
 *                 for some b) cannot be placed at all: then every sequence is
 *                 skipped.  Either case sets the error bit gdn_prefill_check reports
 *                 as GDN_ESKIPPED.
 *  q, k           [T][Hk][128] bf16 (token-major over the packed batch)
 *  v, z, o        [T][Hv][128] bf16
 *  g, beta        [T][Hv] fp32
 *  state_in/out   [B][Hv][128][128] fp32;  conv_state_in/out [B][3][Cc] bf16
 *
 * gdn_prefill_workspace_size() with the same shape (GDN_PACKED set) gives the
 * workspace, which follows the rules of gdn_prefill.  Every other argument,
 * check and status is that of gdn_prefill (or, for the _gate_logits variant,
 * of gdn_prefill_gate_logits); cu_seqlens counts as an input for the aliasing
 * checks.  gdn_prefill rejects a shape with GDN_PACKED, these two one without.
 */
int gdn_prefill_packed(const gdn_shape *shape, const int32_t *cu_seqlens, const uint16_t *q,
                       const uint16_t *k, const uint16_t *v, const float *g, const float *beta,
                       const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w,
                       const float *state_in, const uint16_t *conv_state_in, uint16_t *o,
                       float *state_out, uint16_t *conv_state_out, void *workspace,
                       size_t workspace_bytes, void *stream);
int gdn_prefill_packed_gate_logits(const gdn_shape *shape, const int32_t *cu_seqlens,
                                   const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                   const float *a, const float *b, const float *A_log,
                                   const float *dt_bias, const uint16_t *z, const uint16_t *conv_w,
                                   const uint16_t *norm_w, const float *state_in,
                                   const uint16_t *conv_state_in, uint16_t *o, float *state_out,
                                   uint16_t *conv_state_out, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* A static, NUL-terminated description of a status code. */
const char *gdn_status_string(int status);

/*
 * After a call on this thread returned GDN_EHIP: which HIP call or check
 * failed and HIP's own message for it.  The string is owned by the library,
 * stays valid until the thread's next failing call, and is empty before the
 * first failure.
 */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
