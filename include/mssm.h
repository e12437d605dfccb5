/*
 * mssm.h -- C ABI of the MI355X (gfx950) selective-scan library (libmssm.so).
 *
 * Two forward operations, described below, and around them:
 *  - token-by-token (decode) counterparts that advance a stored state in
 *    place: mssm_selective_state_update, mssm_ssd_state_update;
 *  - the gradients of the first (mssm_selective_scan_bwd), and its training
 *    forward that stores the state checkpoints those gradients can start
 *    from (mssm_selective_scan_fwd_ckpt);
 *  - the first with its short causal convolution fused in front
 *    (mssm_selective_scan_conv_fwd; decode: mssm_selective_state_update_conv);
 *  - the second under the Mamba-3 exponential-trapezoidal input rule
 *    (mssm_ssd_trapezoidal_fwd; decode: mssm_ssd_trapezoidal_state_update),
 *    with a complex-valued state as well (mssm_mamba3_siso_update), and with
 *    several inputs and outputs per channel, Mamba-3 MIMO
 *    (mssm_ssd_mimo_fwd; decode: mssm_ssd_mimo_state_update).
 *
 *  1. mssm_selective_scan_fwd -- the Mamba-1 selective scan.  Defined by the
 *     linear state recurrence h_t = A h_{t-1} + B x_t with readout y_t = C h_t
 *     ("Mamba-2 y state-space models", 4.1), made selective -- B, C and the
 *     step delta depend on the token ("03 - Modelos de espacio de estados",
 *     "El mecanismo selectivo de Mamba"; "P20 - Mamba", 5) -- and discretised
 *     by zero-order hold with a diagonal A, so that exp(delta * A) is taken
 *     elementwise ("03 - ...", "Discretizacion").  Per (batch b, channel c,
 *     state n) and time t:
 *         h[n]     = exp(delta[b,t,c] * A[c,n]) * h[n] + delta[b,t,c] * B[b,t,n] * x[b,t,c]
 *         y[b,t,c] = sum_n C[b,t,n] * h[n] + D[c] * x[b,t,c]
 *         out      = y * silu(z[b,t,c]),   silu(v) = v / (1 + exp(-v))
 *     with h = h0[b,c,:] (or 0) before t = 0.  The input term delta*B*x is
 *     the Euler step for B (the pages' own ZOH formula for Bbar was lost);
 *     D and z are optional.
 *
 *  2. mssm_ssd_fwd -- the Mamba-2 multi-head form, whose transition is a
 *     scalar times the identity ("Mamba-3" blog, introduction) on a state
 *     organised in heads of size headdim ("Mamba-2 y state-space models",
 *     4.2 and 4.3 notes).  Per (b, head h, p < headdim, n) with group
 *     g = h / (nheads / ngroups):
 *         S[p,n]     = exp(delta[b,t,h] * A[h]) * S[p,n] + delta[b,t,h] * B[b,t,g,n] * x[b,t,h,p]
 *         y[b,t,h,p] = sum_n C[b,t,g,n] * S[p,n] + D[h] * x[b,t,h,p],   out = y * silu(z)
 *     Computed chunk by chunk with matrix-core contractions (the
 *     attention-like "SSD" form of "Mamba-2 y state-space models", 4.2);
 *     the result does not depend on the chunk length except by rounding.
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is a DEVICE pointer owned by the caller, on the
 *    device of `stream` (the device current at the call for the null
 *    stream): the kernels run there, and memory of another GPU faults.
 *    The library never allocates, frees or keeps a pointer after returning,
 *    and never synchronises: work is enqueued on `stream` (a hipStream_t
 *    passed as void*; NULL = the null stream) and the call returns at once.
 *    A call enqueues kernel launches only (no memset, no copy), and every
 *    workspace element is written by a kernel before one reads it, so a
 *    call may be captured into a HIP graph on a capturing stream and
 *    replayed; each replay reads the buffers as they are at that time.
 *  - Tensors are dense, row-major and contiguous (last index fastest).
 *    x, delta, B, C, z and out share io_dtype; A, D, h0 and final_state are
 *    always fp32.  fp32 results are rounded to bf16 to nearest-even.
 *  - Accumulation and state are fp32 whatever io_dtype is.
 *  - `out` and `final_state` must not alias any input or each other.
 *  - Errors: a negative mssm_status.  All argument checks run on the host
 *    before anything is enqueued; on error nothing is enqueued and outputs
 *    are untouched.  MSSM_ERR_HIP means a launch failed; the HIP error text
 *    of the calling thread's last failure is returned by
 *    mssm_last_error_detail().
 *  - Thread-safe: no mutable global state (apart from that per-thread error
 *    text, and the per-device scratch address that
 *    mssm_selective_scan_fwd_noalloc looks up once).  Calls on different
 *    streams may overlap (mssm_selective_scan_fwd_noalloc excepted: see there).
 */
#ifndef MSSM_H
#define MSSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSSM_ABI_VERSION 1

typedef enum {
    MSSM_OK = 0,
    MSSM_ERR_INVALID_ARG = -1,   /* null required pointer, size <= 0, size overflow, aliasing */
    MSSM_ERR_UNSUPPORTED = -2,   /* dtype, dstate/headdim outside the supported set, nheads % ngroups != 0, bad chunk */
    MSSM_ERR_MISALIGNED = -3,    /* a pointer not aligned to its element size */
    MSSM_ERR_WORKSPACE = -4,     /* workspace missing or smaller than the size query asks */
    MSSM_ERR_HIP = -5            /* a HIP launch failed (see mssm_last_error_detail) */
} mssm_status;

typedef enum { MSSM_F32 = 0, MSSM_BF16 = 1 } mssm_dtype;

/* Mamba-1 selective scan problem.
 *   x, delta, z, out : [batch, seqlen, dim]      (io_dtype)
 *   B, C             : [batch, seqlen, dstate]   (io_dtype; shared by all channels)
 *   A                : [dim, dstate] fp32 (the values of A, normally negative)
 *   D                : [dim] fp32, nullable
 *   h0, final_state  : [batch, dim, dstate] fp32, nullable
 * split_seq   : number of sequence chunks scanned in parallel with an exact
 *               inter-chunk state carry (0 = library's choice, else 1..4096).
 * split_state : lanes that share one channel's dstate states (0 = library's
 *               choice, else 1, 2, 4, 8 or 16).
 * dstate must be 1..256. */
typedef struct {
    int64_t batch, seqlen, dim, dstate;
    int32_t io_dtype;   /* mssm_dtype */
    int32_t split_seq;
    int32_t split_state;
    uint32_t flags;     /* reserved, must be 0 */
} mssm_scan_desc;

/* Mamba-2 scalar-A multi-head problem.
 *   x, z, out        : [batch, seqlen, nheads, headdim]   (io_dtype)
 *   delta            : [batch, seqlen, nheads]             (io_dtype)
 *   B, C             : [batch, seqlen, ngroups, dstate]    (io_dtype)
 *   A, D             : [nheads] fp32 (D nullable)
 *   h0, final_state  : [batch, nheads, headdim, dstate] fp32, nullable
 * chunk: time-chunk length of the matrix form: 0 (library's choice), 64, 128
 * or 256; a chunk longer than 64 steps is evaluated as consecutive 64-step
 * blocks with the state carried between them (the same algebra, so only
 * rounding differs).  The matrix-core block kernel takes io_dtype MSSM_BF16
 * (the matrix cores take bf16 operands), headdim a multiple of 8 (it works in
 * 64-wide slices, the last one cut at headdim), dstate a
 * multiple of 16 up to 128 (and, for the MIMO calls below, a rank of 1, 2,
 * 4, 8 or 16), or with one input per channel a multiple of 16 up to 256;
 * there the state never leaves the chip between blocks, and x,
 * z, out, B, C, h0 and final_state must be 16-byte aligned.  Above 128 states
 * the kernel runs twice, on states 0-127 and on the rest, each writing its
 * share of the output's state sum in fp32 to the workspace, and a third
 * kernel adds the shares, D x and the gate (workspace: 8 * batch * seqlen *
 * nheads * headdim bytes, see mssm_ssd_workspace_size).  Any other problem with io_dtype
 * MSSM_F32 or MSSM_BF16 and dstate up to 256 runs token by token through the
 * recurrent update kernel (state from h0, written to final_state; the chunk
 * is then unused), with element-aligned pointers.  The state update's
 * entry points (below) take the same descriptor. */
typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int32_t io_dtype;
    uint32_t flags;     /* reserved, must be 0 */
} mssm_ssd_desc;

/* Selective scan forward.  workspace: device memory of at least
 * mssm_selective_scan_workspace_size(desc) bytes (may be NULL when that size
 * is 0), 256-byte aligned, reusable once the stream has passed this call. */
int mssm_selective_scan_fwd(const mssm_scan_desc* desc,
                            const void* x, const void* delta, const float* A,
                            const void* B, const void* C, const float* D, const void* z,
                            const float* h0, void* out, float* final_state,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mssm_selective_scan_fwd needs for this problem (0 when
 * the sequence is not split).  Returns 0 for an invalid descriptor too. */
size_t mssm_selective_scan_workspace_size(const mssm_scan_desc* desc);

/* mssm_selective_scan_fwd for callers that cannot allocate device memory at
 * the call (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): no workspace argument.  A split sequence keeps its
 * chunk aggregates in a fixed scratch array of 32 MiB that the library holds
 * on each GPU it runs on, from the first such call there until the process
 * ends; this call itself allocates nothing.  With split_seq = 0 the library's
 * plan is used, with fewer chunks where its workspace
 * (mssm_selective_scan_workspace_size) would exceed 32 MiB; a forced
 * split_seq whose workspace exceeds 32 MiB returns MSSM_ERR_WORKSPACE.  Every
 * call on one GPU shares that GPU's scratch: calls ordered on one stream are
 * safe (kernels write each scratch element before reading it, so nothing
 * needs clearing between calls), calls that overlap on one GPU race.
 * Results equal mssm_selective_scan_fwd's for the same plan, bit for bit.
 * All other arguments and rules as mssm_selective_scan_fwd. */
int mssm_selective_scan_fwd_noalloc(const mssm_scan_desc* desc,
                                    const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    const float* h0, void* out, float* final_state, void* stream);

/* Mamba-2 scalar-A multi-head forward.  Same ownership, stream and error rules
 * as mssm_selective_scan_fwd. */
int mssm_ssd_fwd(const mssm_ssd_desc* desc,
                 const void* x, const void* delta, const float* A,
                 const void* B, const void* C, const float* D, const void* z,
                 const float* h0, void* out, float* final_state,
                 void* workspace, size_t workspace_bytes, void* stream);

size_t mssm_ssd_workspace_size(const mssm_ssd_desc* desc);

/* Mamba-3 SISO recurrence in the Mamba-2 multi-head form: the step's input
 * integral is taken by the exponential-trapezoidal rule ("Mamba-3" blog,
 * "El modelo Mamba-3" item 1: a more general recurrence from that
 * discretisation; "Arquitectura": it acts as an implicit convolution on the
 * state input, which replaces the short convolution).  The pages give no
 * formula; this is the weighted trapezoidal rule on the exact one-step
 * integral of the zero-order-hold system, weight lam on the step's own input
 * and 1 - lam on the previous one (carried through the step's decay):
 *     a        = exp(delta[b,t,h] * A[h])
 *     S[p,n]   = a * S[p,n] + (1 - lam[b,t,h]) * delta[b,t,h] * a * B[b,t-1,g,n] * x[b,t-1,h,p]
 *                           + lam[b,t,h] * delta[b,t,h] * B[b,t,g,n] * x[b,t,h,p]
 *     y, out   as in mssm_ssd_fwd.
 * lam = 1 is exactly mssm_ssd_fwd; lam = 1/2 the trapezoidal rule.
 *   lam : [batch, seqlen, nheads] (io_dtype), required when seqlen > 0; any
 *         value is accepted (the rule interpolates for 0 <= lam <= 1).
 * Before step 0 there is no input (the previous-input term of step 0 is 0)
 * and h0 is the state entering step 0; final_state is the state after the
 * last step.  To continue a sequence in a later call, pass final_state as
 * h0 after adding (1 - lam) * delta * B * x of the boundary (the next call's
 * first lam and delta with this call's last B and x) -- that term belongs to
 * the next call's first step.  Descriptor, layouts, workspace, ownership,
 * stream and error rules as mssm_ssd_fwd. */
int mssm_ssd_trapezoidal_fwd(const mssm_ssd_desc* desc,
                             const void* x, const void* delta, const void* lam, const float* A,
                             const void* B, const void* C, const float* D, const void* z,
                             const float* h0, void* out, float* final_state,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Mamba-3 MIMO ("Mamba-3" blog, "El modelo Mamba-3" item 3: multi-input
 * multi-output SSMs model several SSMs in parallel, against the single-input
 * single-output ones, for more work per update at about the same decode
 * latency; "Arquitectura": the MIMO projections widen B and C; "Tareas de
 * recuperacion": the state does not grow).  The pages give no formula; the
 * plain reading: each channel p of head h takes `rank` inputs and gives
 * `rank` outputs, and all of them share the head's one state and transition.
 * With U_t[p,n] = sum_r B[b,t,g,r,n] * x[b,t,h,r,p]:
 *     a        = exp(delta[b,t,h] * A[h])
 *     S[p,n]   = a * S[p,n] + (1 - lam) * delta * a * U_{t-1}[p,n] + lam * delta * U_t[p,n]
 *     y[b,t,h,r,p] = sum_n C[b,t,g,r,n] * S[p,n] + D[h] * x[b,t,h,r,p],   out = y * silu(z)
 * lam NULL is lam = 1 (the Mamba-2 rule, delta * U_t); rank 1 is
 * mssm_ssd_trapezoidal_fwd (mssm_ssd_fwd without lam).  Layouts:
 *   x, z, out : [batch, seqlen, nheads, rank, headdim]   (io_dtype; z nullable)
 *   B, C      : [batch, seqlen, ngroups, rank, dstate]   (io_dtype)
 *   delta, lam: [batch, seqlen, nheads] (io_dtype; lam nullable)
 *   A, D, h0, final_state: as mssm_ssd_fwd.
 * rank: 1..64 (MSSM_ERR_UNSUPPORTED above, MSSM_ERR_INVALID_ARG below 1).
 * The matrix-core block kernel takes rank 1, 2, 4, 8 or 16 (besides the
 * mssm_ssd_desc conditions): its 64-row blocks then hold 64 / rank steps, and
 * the rows of a step share that step's decay.  Any other rank or shape runs
 * token by token through the recurrent update kernel.  Before step 0 there is
 * no input (U_{-1} = 0); to continue a sequence, pass final_state as h0 after
 * adding (1 - lam) * delta * U of the boundary, or step on with
 * mssm_ssd_mimo_state_update.  Other rules as mssm_ssd_fwd. */
int mssm_ssd_mimo_fwd(const mssm_ssd_desc* desc, int32_t rank,
                      const void* x, const void* delta, const void* lam, const float* A,
                      const void* B, const void* C, const float* D, const void* z,
                      const float* h0, void* out, float* final_state,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Token-by-token state update (decode), Mamba-1 form.  At inference the layer
 * keeps only its fixed-size state and advances it one token at a time, at a
 * cost that does not grow with the tokens already seen ("03 - Modelos de
 * espacio de estados", "Coste de inferencia"; "P20 - Mamba", 5).  Applies the
 * recurrence and readout of mssm_selective_scan_fwd to desc->seqlen new
 * tokens (normally 1), starting from `state` and writing the advanced state
 * back into `state` (in place):
 *   state         : [batch, dim, dstate] fp32, read and overwritten
 *   x, delta, z, out : [batch, seqlen, dim]  (io_dtype; z nullable)
 *   B, C          : [batch, seqlen, dstate]  (io_dtype)
 *   A             : [dim, dstate] fp32;  D : [dim] fp32, nullable
 * split_seq and split_state are ignored.  The result equals
 * mssm_selective_scan_fwd with h0 = state and final_state written to state,
 * up to rounding.  `out` and `state` must not alias any input or each other.
 * Same ownership, stream and error rules as mssm_selective_scan_fwd; no
 * workspace. */
int mssm_selective_state_update(const mssm_scan_desc* desc, float* state,
                                const void* x, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                void* out, void* stream);

/* Token-by-token state update with the short causal convolution in front (the
 * decode counterpart of mssm_selective_scan_conv_fwd): besides the SSM state,
 * the layer keeps the last conv_width - 1 inputs of the convolution, and each
 * new token is convolved with them, passed through SiLU, and fed to the
 * update of mssm_selective_state_update.
 *   conv_state : [batch, conv_width - 1, dim] (io_dtype), oldest first (the
 *                layout of conv_init), read and advanced in place (nullable
 *                when conv_width is 1)
 *   xin        : [batch, seqlen, dim] the convolution's input for the new tokens
 *   conv_w, conv_b : as in mssm_selective_scan_conv_fwd; conv_width 1..4
 * Equals mssm_selective_scan_conv_fwd with conv_init = conv_state and
 * h0 = state, up to rounding; conv_state then holds the last conv_width - 1
 * inputs exactly.  Any dstate (1..256); no alignment beyond the elements'. */
int mssm_selective_state_update_conv(const mssm_scan_desc* desc, int32_t conv_width,
                                     float* state, void* conv_state, const void* xin,
                                     const float* conv_w, const float* conv_b, const void* delta,
                                     const float* A, const void* B, const void* C, const float* D,
                                     const void* z, void* out, void* stream);

/* Token-by-token state update, multi-head (scalar A per head) form:
 *   state         : [batch, nheads, headdim, dstate] fp32, read and overwritten
 *   x, z, out     : [batch, seqlen, nheads, headdim]  (io_dtype; z nullable)
 *   delta         : [batch, seqlen, nheads]           (io_dtype)
 *   B, C          : [batch, seqlen, ngroups, dstate]  (io_dtype)
 *   A, D          : [nheads] fp32 (D nullable)
 * io_dtype may be MSSM_F32 or MSSM_BF16; dstate 1..256; any headdim; chunk is
 * ignored.  Equals mssm_ssd_fwd with h0 = state, final_state written to
 * state, up to rounding. */
int mssm_ssd_state_update(const mssm_ssd_desc* desc, float* state,
                          const void* x, const void* delta, const float* A,
                          const void* B, const void* C, const float* D, const void* z,
                          void* out, void* stream);

/* Token-by-token state update under the Mamba-3 SISO rule (see
 * mssm_ssd_trapezoidal_fwd; "Mamba-3" blog, "El modelo Mamba-3" item 1, and
 * the decode latency it is designed for, "Kernels por todas partes").  Each
 * step needs the previous token's x and B besides the state:
 *   x_prev : [batch, nheads, headdim] (io_dtype), nullable
 *   B_prev : [batch, ngroups, dstate] (io_dtype), nullable
 * the token before the first of the seqlen new ones (NULL: there is none, as
 * at the start of a sequence; both or either may be NULL and then count as
 * zero).  Within the call each token's left-end term uses the token before
 * it.  They are read only: to step again, pass this call's last x and B.
 *   lam    : [batch, seqlen, nheads] (io_dtype), required.
 * Equals mssm_ssd_trapezoidal_fwd with h0 = state + (1 - lam_0) * delta_0 *
 * x_prev (x) B_prev and final_state written to state, up to rounding.  Other
 * arguments, shapes and rules as mssm_ssd_state_update. */
int mssm_ssd_trapezoidal_state_update(const mssm_ssd_desc* desc, float* state,
                                      const void* x_prev, const void* B_prev,
                                      const void* x, const void* delta, const void* lam,
                                      const float* A, const void* B, const void* C,
                                      const float* D, const void* z, void* out, void* stream);

/* The Mamba-3 SISO recurrence with a complex-valued state ("Mamba-3" blog,
 * "El modelo Mamba-3" item 2: state tracking by a complex-valued SSM;
 * "Arquitectura": its transitions act as rotations, RoPE; "Kernels por todas
 * partes": data-dependent).  The pages give no formula; the plain reading:
 * state pairs (2k, 2k+1) are complex numbers and head h's transition is
 * A[h] + i*omega[h,k] per pair, so zero-order hold gives a decay times a
 * rotation by delta*omega (data-dependent through delta):
 *     (u, v)  = S[p,2k], S[p,2k+1] + (1 - lam) * delta * x_prev[p] * B_prev[g,2k], [g,2k+1]
 *     S[p,2k]   = a * (c*u - s*v) + lam * delta * B[b,t,g,2k]   * x[b,t,h,p]
 *     S[p,2k+1] = a * (s*u + c*v) + lam * delta * B[b,t,g,2k+1] * x[b,t,h,p]
 * with a = exp(delta*A[h]), c, s = cos, sin(delta*omega[h,k]); readout
 * y = sum_n C[n] S[p,n] (the real part of conj(C_k) S_k) as before.
 *   omega : [nheads, dstate/2] fp32, required; dstate must be even
 *           (MSSM_ERR_UNSUPPORTED otherwise).
 * The state is kept in its own (unrotated) frame, so it can be stored and
 * resumed like any other.  omega = 0 is mssm_ssd_trapezoidal_state_update
 * bit for bit.  Any number of tokens: with seqlen = L this is also the
 * sequence form of the complex state (recurrent, no matrix cores; h0 =
 * state, final_state written to state).  Other arguments and rules as
 * mssm_ssd_trapezoidal_state_update. */
int mssm_mamba3_siso_update(const mssm_ssd_desc* desc, float* state,
                            const void* x_prev, const void* B_prev,
                            const void* x, const void* delta, const void* lam,
                            const float* A, const float* omega,
                            const void* B, const void* C, const float* D, const void* z,
                            void* out, void* stream);

/* The MIMO decode step (see mssm_ssd_mimo_fwd): desc->seqlen new tokens
 * (normally 1) from `state`, written back in place.  The state is read and
 * written once per call whatever the rank: the rank multiplies the work per
 * byte of state, not the bytes ("Mamba-3" blog, "Resultados experimentales":
 * MIMO does not raise decode latency).
 *   x_prev : [batch, nheads, rank, headdim], B_prev : [batch, ngroups, rank, dstate]
 *            (io_dtype, nullable: no previous token; read only, and ignored
 *            when lam is NULL)
 *   x, z, out, B, C, delta, lam: as mssm_ssd_mimo_fwd with seqlen tokens.
 * Equals mssm_ssd_mimo_fwd with h0 = state + (1 - lam_0) * delta_0 * U_prev
 * and final_state written to state, up to rounding.  Any headdim, dstate up
 * to 256, fp32 or bf16; other rules as mssm_ssd_state_update. */
int mssm_ssd_mimo_state_update(const mssm_ssd_desc* desc, int32_t rank, float* state,
                               const void* x_prev, const void* B_prev,
                               const void* x, const void* delta, const void* lam,
                               const float* A, const void* B, const void* C,
                               const float* D, const void* z, void* out, void* stream);

/* Selective scan with the short causal convolution + SiLU that precedes it in
 * the Mamba-1/2 block fused in front ("Mamba-3" blog, "Arquitectura": the
 * block's short causal convolution on the state input, which Mamba-3 drops).
 * The scan's x is computed on chip from its input xin and never stored:
 *   x[b,t,c] = silu(conv_b[c] + sum_{k < W} conv_w[c,k] * xin[b, t-(W-1)+k, c])
 * with W = conv_width (1..4) and xin at a step s < 0 taken from
 * conv_init[b, W-1+s, c] (or 0 when conv_init is NULL).  Everything else is
 * mssm_selective_scan_fwd with that x.
 *   xin              : [batch, seqlen, dim]        (io_dtype)
 *   conv_w           : [dim, conv_width] fp32 (tap k multiplies the input k - (W-1) steps away)
 *   conv_b           : [dim] fp32, nullable
 *   conv_init        : [batch, conv_width - 1, dim] (io_dtype), nullable: the
 *                      inputs before t = 0, oldest first (xin's layout)
 * The fused block kernel takes dstate 16, dim * sizeof(io) a multiple of 16,
 * every io pointer (xin, delta, B, C, z, out, conv_init) 16-byte aligned and
 * split_state 0 or 16.  Any other problem (dstate up to 256, element-aligned
 * pointers) runs token by token through the recurrent update kernel, which
 * reads conv_init and leaves it unchanged.  workspace: at least
 * mssm_selective_scan_conv_workspace_size(desc) bytes (0 off the fused path).  Same ownership,
 * stream and error rules as mssm_selective_scan_fwd. */
int mssm_selective_scan_conv_fwd(const mssm_scan_desc* desc, int32_t conv_width,
                                 const void* xin, const float* conv_w, const float* conv_b,
                                 const void* conv_init, const void* delta, const float* A,
                                 const void* B, const void* C, const float* D, const void* z,
                                 const float* h0, void* out, float* final_state,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mssm_selective_scan_conv_fwd needs (0 when the sequence
 * is not split, or for an invalid or unsupported descriptor). */
size_t mssm_selective_scan_conv_workspace_size(const mssm_scan_desc* desc);

/* Training-mode forward: mssm_selective_scan_fwd (same results) that also
 * stores the state entering every 16-step tile, for mssm_selective_scan_bwd to
 * start from.  Training runs the forward before the gradients anyway; storing
 * 4 bytes per lane every 16 steps spares the gradient pass a second walk over
 * the sequence.
 *   checkpoints : [batch][ceil(seqlen/16)][16*ceil(dim/16)][16] fp32, at least
 *                 mssm_selective_scan_checkpoint_size(desc) bytes; entry
 *                 [b][k][c][n] is h[n] of channel c before step 16k (channels
 *                 past dim are not written).
 * Supported: dstate 16, dim * sizeof(io) a multiple of 16, 16-byte aligned io
 * pointers, split_state 0 or 16; workspace as given by
 * mssm_selective_scan_fwd_ckpt_workspace_size.  Same rules otherwise. */
int mssm_selective_scan_fwd_ckpt(const mssm_scan_desc* desc,
                                 const void* x, const void* delta, const float* A,
                                 const void* B, const void* C, const float* D, const void* z,
                                 const float* h0, void* out, float* final_state, float* checkpoints,
                                 void* workspace, size_t workspace_bytes, void* stream);

size_t mssm_selective_scan_fwd_ckpt_workspace_size(const mssm_scan_desc* desc);

/* Bytes of the checkpoint array (0 for an invalid descriptor or dstate != 16). */
size_t mssm_selective_scan_checkpoint_size(const mssm_scan_desc* desc);

/* Gradients of mssm_selective_scan_fwd (reverse mode through the same
 * recurrence; training a selective SSM needs them, "P20 - Mamba", 5).  For
 * the loss sum(out * dout) + sum(final_state * dfinal) it writes
 *   dx, ddelta, dz : [batch, seqlen, dim]     (io_dtype)
 *   dB, dC         : [batch, seqlen, dstate]  fp32 (summed over channels)
 *   dA             : [dim, dstate] fp32,  dD : [dim] fp32 (summed over batch and time)
 *   dh0            : [batch, dim, dstate] fp32 (nullable: not written)
 * from the forward inputs (same layouts as mssm_selective_scan_fwd; h0 nullable
 * = zero) and the upstream gradients
 *   dout           : [batch, seqlen, dim]     (io_dtype)
 *   dfinal         : [batch, dim, dstate] fp32, nullable (= zero).
 * dz is required when z is given and dD when D is given (each is ignored, and
 * may be NULL, otherwise).  With y = sum_n C h + D x and out = y silu(z):
 *   dy = dout silu(z); lam_t = C_t dy_t + exp(delta_{t+1} A) lam_{t+1}
 *   (lam after the last step = dfinal); dC_t = sum_c dy_t h_t;
 *   dB_t = sum_c lam_t delta_t x_t; dz = dout y silu'(z); dh0 = exp(delta_0 A) lam_0.
 * Without checkpoints (below) the states are recomputed from h0: nothing is
 * kept from the forward call.
 * dstate up to 256 (the states are taken in slices of 16); split_seq and
 * split_state are ignored.  The result is deterministic: every sum is taken
 * in a fixed order.  workspace: at least
 * mssm_selective_scan_bwd_workspace_size(desc) bytes, 256-byte aligned.  With
 * S = ceil(dstate / 16) that is about 4 * batch * ceil(seqlen / 16) * 16 *
 * ceil(dim / 16) * 16 S bytes of state checkpoints, plus 8 * batch * seqlen *
 * ceil(dim / 16) * 16 S bytes of per-block dB/dC partial sums, plus, when
 * S > 1, 12 * S * batch * seqlen * dim bytes of the slices' partial sums
 * (added by a finishing kernel).
 * checkpoints: nullable; the array mssm_selective_scan_fwd_ckpt wrote for
 * these inputs (dstate 16 only).  Given it, the kernel starts every tile from
 * the stored state instead of walking the sequence forward once more (the
 * first workspace segment then goes unused).
 * Outputs and workspace must not alias any input or each other.  Same
 * ownership, stream and error rules as mssm_selective_scan_fwd. */
int mssm_selective_scan_bwd(const mssm_scan_desc* desc,
                            const void* x, const void* delta, const float* A,
                            const void* B, const void* C, const float* D, const void* z,
                            const float* h0, const void* dout, const float* dfinal,
                            void* dx, void* ddelta, float* dA, float* dB, float* dC, float* dD,
                            void* dz, float* dh0, const float* checkpoints,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace mssm_selective_scan_bwd needs (0 for an invalid or
 * unsupported descriptor). */
size_t mssm_selective_scan_bwd_workspace_size(const mssm_scan_desc* desc);

/* The plan the library would use for a selective-scan descriptor:
 * writes the sequence-chunk count and lanes-per-channel; returns a status. */
int mssm_selective_scan_plan(const mssm_scan_desc* desc, int32_t* split_seq, int32_t* split_state);

/* Which kernel a multi-head descriptor runs on (mssm_ssd_fwd and
 * mssm_ssd_trapezoidal_fwd): MSSM_SSD_ROUTE_BLOCK, the matrix-core block
 * kernel, or MSSM_SSD_ROUTE_RECURRENT, the token-by-token update kernel (see
 * mssm_ssd_desc).  Writes *route; returns a status (the descriptor's). */
#define MSSM_SSD_ROUTE_BLOCK 0
#define MSSM_SSD_ROUTE_RECURRENT 1
int mssm_ssd_plan(const mssm_ssd_desc* desc, int32_t* route);
/* The same for mssm_ssd_mimo_fwd with this rank. */
int mssm_ssd_mimo_plan(const mssm_ssd_desc* desc, int32_t rank, int32_t* route);

/* Static text for a status code (never NULL). */
const char* mssm_status_string(int status);

/* Text of the calling thread's last MSSM_ERR_HIP failure ("" if none). */
const char* mssm_last_error_detail(void);

int mssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSSM_H */
