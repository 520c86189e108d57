/*
 * ss_scan.h -- C ABI of the MI355X (gfx950) selective-scan library (libssscan.so).
 *
 * The operation is the S6 selective-scan forward.  For batch b, channel d and time t:
 *
 *   dt_t  = softplus(delta[b, hd, t] + delta_bias[hd])   if SS_DELTA_SOFTPLUS, else delta + bias
 *   h_t   = exp(dt_t * A) (.) h_{t-1} + dt_t * B[b, g, :, t] * u[b, d, t]        h_{-1} = 0
 *   y_t   = C[b, g, :, t] . h_t + D * u[b, d, t]
 *   y_t  *= silu(z[b, d, t]) = z / (1 + exp(-z))          if SS_Z_GATE_SILU
 *
 * hd = d / (channels / heads) is the head of channel d (hd = d when delta is per channel) and
 * g = d / (channels / groups) the B/C group.  The state h has N entries per channel; with a
 * per-channel A [channels, N] the decay is diagonal (Mamba-1), with A [heads] it is one scalar
 * per head shared by all N states (Mamba-2 style scalar decay).
 *
 * Where this is defined (pages of the method's description):
 *  - the recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t, y_t = C_t h_t, and the input-dependent
 *    B_t, C_t and Delta_t = softplus(Linear(x_t)): omica.com.cn Mamba explainer (news 823493),
 *    sections 3 and 5; the bqwf.cn state-space survey (news 437117), sections 2.1 and 2.2;
 *  - Abar = exp(Delta A), Bbar = Delta B (exponential-Euler; explainer section 6.3) and the one-step
 *    pseudocode h_t = exp(-Delta) h_{t-1} + Delta B x_t in the "Mamba -- selective state space
 *    model" study notes (estelledc.github.io), case 1;
 *  - the D feed-through: explainer section 3 (output equation);
 *  - scalar decay A_t = alpha_t I with heads: survey section 3.2; explainer section 6.2;
 *  - the gate after the selective SSM: juejin.cn post on Mamba's history, section 2 (the pages
 *    give no formula; silu(z) = z * sigmoid(z) is the reading taken);
 *  - one SISO system per channel (channels independent): explainer section 6.3.
 *
 * Conventions shared by every entry point:
 *  - All tensor data pointers are DEVICE pointers owned by the caller.  The library only
 *    borrows them until the enqueued work completes; it never frees or retains them.
 *  - Strides are in elements.  The innermost (time / last) stride of every time-major tensor
 *    must be 1; outer strides are free (non-negative).
 *  - Every argument is validated on the host before anything is enqueued.  On any error the
 *    call returns a negative SS_ERR_* code, enqueues nothing and leaves y untouched.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL = the default
 *    stream).  Kernel execution errors surface at stream synchronisation or via ss_check().
 *  - Calls on different streams may run concurrently; the library keeps no per-call global state.
 *  - Results are deterministic: the same inputs give bitwise the same y on every run (the
 *    backward's sums over channels and batch are the exception; see ss_scan_bwd).
 */
#ifndef SS_SCAN_H
#define SS_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_VERSION 100 /* 1.0.0 */

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

/* A strided view of caller-owned device memory. */
typedef struct {
  void* data;        /* device pointer (may be NULL only for an optional, absent tensor) */
  int32_t dtype;     /* ss_dtype */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];  /* sizes, outermost first */
  int64_t stride[4]; /* in elements */
} ss_tensor;

/* flags */
#define SS_DELTA_SOFTPLUS (1u << 0) /* dt = softplus(delta + delta_bias) */
#define SS_Z_GATE_SILU (1u << 1)    /* y *= silu(z); requires z */
/* a request for bitwise run-to-run reproducibility.  Every forward path (ss_scan_fwd,
 * ss_scan_fwd_state, ss_scan_step) is deterministic by construction -- each output is one fixed
 * chain of f32 operations, with no atomics and no order that depends on scheduling -- so there
 * the flag changes nothing.  ss_scan_bwd sums over channels and batch with atomic adds and
 * rejects it with SS_ERR_UNSUPPORTED. */
#define SS_DETERMINISTIC (1u << 2)
/* zero-order hold: the input enters as (exp(dt A) - 1) / A * B * u (dt * B * u at A = 0) instead
 * of the exponential-Euler dt * B * u -- the ZOH discretisation Bbar = (dt A)^-1 (exp(dt A) - I)
 * dt B of the omica.com.cn explainer, sections 3 and 5.  Forward and decoding step only. */
#define SS_ZOH (1u << 3)
/* exponential-trapezoidal rule: h_t = exp(dt_t A) h_{t-1} + (e_t + exp(dt_t A) e_{t-1}) / 2 with
 * e_t = Bbar_t u_t (the explainer's Mamba-3 recurrence, section 6.3).  The state passed in and
 * out (h_init, h_final, the decoding state) is h_t + e_t / 2 of the step before / the last step,
 * which carries the rule across call boundaries.  Forward and decoding step only. */
#define SS_TRAPEZOID (1u << 4)

/* return codes */
#define SS_OK 0
#define SS_ERR_NULL (-1)        /* a required tensor or data pointer is NULL */
#define SS_ERR_DTYPE (-2)       /* unsupported dtype or dtype mix */
#define SS_ERR_SHAPE (-3)       /* inconsistent shapes */
#define SS_ERR_STRIDE (-4)      /* innermost stride != 1, or a negative stride */
#define SS_ERR_FLAGS (-5)       /* unknown flag bits, or SS_Z_GATE_SILU without z */
#define SS_ERR_UNSUPPORTED (-6) /* valid but unsupported size (N > 128, > 2^31 steps per row, conv width > 8) */
#define SS_ERR_ALIAS (-7)       /* an output (y, a final state) overlaps an input or another output */
#define SS_ERR_HIP (-8)         /* a HIP runtime call failed (launch, workspace allocation) */
/* reported by ss_check only: inside a kernel, a wave's bounded wait for another wave of its
 * block ran out of polls (never expected; the environment variable SS_SPIN_LIMIT lowers the
 * bound for tests).  The wave went on instead of hanging, so the results of the calls since the
 * previous ss_check are wrong. */
#define SS_ERR_DEADLOCK (-9)
/* ss_scan_fwd_noalloc only: the call needs more scratch than that entry point's static buffer
 * (SS_NOALLOC_SCRATCH_BYTES) holds.  Nothing was enqueued and y is untouched. */
#define SS_ERR_SCRATCH (-10)

/*
 * ss_scan_fwd -- selective-scan forward, y = S6(u, delta, A, B, C, D, z, delta_bias).
 *
 *   u          [batch, channels, L]          f32 | bf16
 *   delta      [batch, heads, L]             same dtype as u; heads divides channels
 *   A          [channels, N] f32  (diagonal decay per channel), or
 *              [heads] f32        (one scalar decay per head, shared by its N states)
 *   B, C       [batch, groups, N, L]         same dtype as u; groups divides channels
 *   D          [channels] or [heads] f32     optional (NULL or data == NULL): no feed-through
 *   z          [batch, channels, L]          same dtype as u; optional, required by SS_Z_GATE_SILU
 *                                            (a z of no elements may have data == NULL)
 *   delta_bias [heads] f32                   optional: no bias
 *   flags      SS_DELTA_SOFTPLUS | SS_Z_GATE_SILU | SS_DETERMINISTIC | SS_ZOH | SS_TRAPEZOID
 *   y          [batch, channels, L]          f32 | bf16, written; must not overlap any input
 *   stream     hipStream_t (as void*), NULL for the default stream
 *
 * N must be 1..128.  L = 0 or batch * channels = 0 is a successful no-op.  The state starts at
 * zero for every (b, d).  Internally the computation is in f32 (bf16 inputs are widened exactly);
 * y in bf16 is rounded to nearest even once.  Scalar-decay calls use a stream-ordered device
 * workspace (per-chunk operands of B and C, and the states handed between sequence segments;
 * O(batch * groups * L * N) bytes), allocated and freed on `stream` from a memory pool that the
 * library keeps on each device and never shrinks, so repeated calls reuse it without a device
 * allocation (SS_ERR_HIP, with nothing enqueued, if the allocation fails; the environment
 * variable SS_FAULT=alloc forces that failure for tests).  Diagonal-decay calls use no
 * workspace, except one batch row with at most two channels per compute unit, bf16 inputs in
 * 16-byte aligned rows, L a multiple of 2048 and at least 6144, and N from 5 to 32 without
 * zero-order hold or the trapezoidal rule: the sequence is then cut into segments run in
 * parallel, and the states handed between them (O(channels * N) floats per segment) come from
 * the same pool.
 *
 * Returns SS_OK or a negative SS_ERR_* code.
 */
int ss_scan_fwd(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                const ss_tensor* C, const ss_tensor* D, const ss_tensor* z,
                const ss_tensor* delta_bias, uint32_t flags, ss_tensor* y, void* stream);

/*
 * ss_scan_fwd_state -- ss_scan_fwd that starts from a given state and returns the final one, so
 * that a long sequence can be scanned in consecutive pieces (chunked prefill, streaming): the
 * recurrent reading of the method keeps a state of fixed size per channel and carries it from
 * token to token ("Mamba -- selective state space model" study notes, core points and case 3;
 * bqwf.cn state-space survey, section 1, the recurrent mode).  Scanning [0, T) and then [T, L)
 * from the carried state gives the same y as one scan over [0, L), up to rounding.
 *
 *   arguments as ss_scan_fwd, and
 *   h_init     [batch, channels, N] f32      optional (NULL or data == NULL): the state starts
 *                                            at zero, as in ss_scan_fwd
 *   h_final    [batch, channels, N] f32      optional: not written.  Written with the state
 *                                            after step L - 1 (h_init itself when L = 0).
 *                                            Must not overlap h_init, any input or y
 *                                            (SS_ERR_ALIAS); use two buffers in turn to carry a
 *                                            state from call to call.
 *
 * The state index n is innermost (stride 1); the other strides are free.  Ownership, errors and
 * asynchrony are those of ss_scan_fwd.
 */
int ss_scan_fwd_state(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                      const ss_tensor* C, const ss_tensor* D, const ss_tensor* z,
                      const ss_tensor* delta_bias, uint32_t flags, const ss_tensor* h_init,
                      ss_tensor* h_final, ss_tensor* y, void* stream);

/*
 * ss_scan_fwd_noalloc -- ss_scan_fwd_state for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results, validation and asynchrony as ss_scan_fwd_state; it calls no hipMalloc, hipFree or
 * allocating library routine.
 *
 * The scratch that scalar-decay calls need (the per-chunk operands of B and C and the states
 * handed between sequence segments, which ss_scan_fwd_state takes from its memory pool) comes
 * instead from one static device array of SS_NOALLOC_SCRATCH_BYTES (64 MiB), which each GPU
 * the library runs on holds until the process ends.  A call whose scratch would exceed it
 * returns SS_ERR_SCRATCH (nothing enqueued, y untouched); diagonal-decay calls use scratch only
 * for the states handed between sequence segments (a few MB at most).  Every call on one GPU shares that GPU's array and leaves its contents
 * behind (every byte a call reads, it wrote first): calls that overlap on one GPU -- on two
 * streams, or from two host threads -- race and give wrong results; order them on one stream.
 */
#define SS_NOALLOC_SCRATCH_BYTES (64ull << 20)
int ss_scan_fwd_noalloc(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                        const ss_tensor* C, const ss_tensor* D, const ss_tensor* z,
                        const ss_tensor* delta_bias, uint32_t flags, const ss_tensor* h_init,
                        ss_tensor* h_final, ss_tensor* y, void* stream);

/*
 * ss_scan_step -- one decoding step: the recurrence advanced by a single token from a persistent
 * state, h <- exp(dt A) h + dt B u, y = C h + D u (times silu(z)), the inference mode in which
 * each new token updates a state of fixed size (study notes, core points and cases 1 and 3).
 * Equal, up to rounding, to ss_scan_fwd_state over L = 1 with h_init = h_final = h.
 *
 *   u          [batch, channels]             f32 | bf16
 *   delta      [batch, heads]                same dtype as u
 *   A          [channels, N] or [heads] f32  as in ss_scan_fwd
 *   B, C       [batch, groups, N]            same dtype as u
 *   D          [channels] or [heads] f32     optional
 *   z          [batch, channels]             same dtype as u; optional, required by SS_Z_GATE_SILU
 *   delta_bias [heads] f32                   optional
 *   flags      SS_DELTA_SOFTPLUS | SS_Z_GATE_SILU | SS_DETERMINISTIC | SS_ZOH | SS_TRAPEZOID
 *   h          [batch, channels, N] f32      read and updated in place (state index innermost)
 *   y          [batch, channels]             f32 | bf16, written
 *
 * h and y must not overlap each other or any input (SS_ERR_ALIAS).  batch * channels = 0 is a
 * successful no-op.  No workspace.  Errors, ownership and asynchrony as in ss_scan_fwd.
 */
int ss_scan_step(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                 const ss_tensor* C, const ss_tensor* D, const ss_tensor* z,
                 const ss_tensor* delta_bias, uint32_t flags, ss_tensor* h, ss_tensor* y, void* stream);

/*
 * ss_scan_bwd -- backward of ss_scan_fwd: the gradients of sum(dy * y) with respect to every
 * input, for training.  The pages train the scan by recomputing its states rather than storing
 * them (bqwf.cn state-space survey, section 2.2); so does this call: it stores only the state at
 * the start of every window of 512 steps (a stream-ordered workspace of batch * channels *
 * ceil(L / 512) * N floats, from the pool described at ss_scan_fwd) and recomputes the rest.
 * Scalar-decay calls whose heads and B/C groups are whole 64-channel slabs take the chunked
 * matrix form instead, whose workspace holds the state at the start of every 32-step chunk
 * (batch * channels * ceil(L / 32) * N' floats, N' = N rounded up to 32, 64 or 128) and C B^T
 * per chunk.  With a gate, either form first recomputes the output before the gate into the
 * workspace (batch * channels * L floats more); the per-channel kernel takes dz and dy s(z) from
 * it where it reads dy, the matrix form in a pass of its own.  Without a gate, a diagonal-decay
 * call with few rows (at most 4 per CU) and at least three 1024-step windows also runs that
 * forward, for the checkpoints it stores as it goes (its output, batch * channels * L floats of
 * workspace, is unused), since it is several times faster there than a checkpoint pass that
 * walks each row on one wave.  Chain rule, with s(z) =
 * z sigmoid(z) and
 * dy0 = dy s(z):  g_t = C_t dy0_t + exp(dt_{t+1} A) g_{t+1} (the gradient of h_t),
 * dC_t = dy0_t h_t,  dB_t = g_t dt_t u_t,  du_t = dy0_t D + sum_n g_t dt_t B_t,
 * ddt_t = sum_n g_t (h_{t-1} exp(dt_t A) A + B_t u_t),  dA = sum_t g_t h_{t-1} exp(dt_t A) dt_t,
 * ddelta_t = ddt_t sigmoid(delta_t + bias) with softplus (ddt_t without),  dbias = sum ddelta,
 * dD = sum dy0_t u_t,  dz_t = dy_t y0_t s'(z_t)  (y0: the output before the gate).
 *
 *   u, delta, A, B, C, D, z, delta_bias, flags    as in ss_scan_fwd (diagonal A [channels, N] or
 *              scalar A [heads], delta per channel or per head), without SS_ZOH, SS_TRAPEZOID or
 *              SS_DETERMINISTIC (SS_ERR_UNSUPPORTED: the summed gradients use atomic adds), and
 *              channels / groups a multiple of 4 (SS_ERR_UNSUPPORTED)
 *   dy         [batch, channels, L]          f32 | bf16: the gradient of the loss at y
 *   du         [batch, channels, L] f32      written
 *   ddelta     [batch, heads, L] f32         written (the gradient of the raw delta; summed over
 *                                            the head's channels)
 *   dA         f32, the shape of A           written (scalar decay: summed over the head's channels
 *                                            and states)
 *   dB, dC     [batch, groups, N, L] f32     written (summed over each group's channels)
 *   dD         f32, the shape of D           written; required exactly when D is given
 *   dz         [batch, channels, L] f32      written; required exactly with SS_Z_GATE_SILU
 *   ddelta_bias [heads] f32                  optional: written when given
 *
 * Every gradient is f32 with innermost stride 1 and must not overlap an input or another
 * gradient (SS_ERR_ALIAS).  The state starts at zero.  Sums over channels and over the batch
 * (dA, dB, dC, dD, dbias, and ddelta when a head has several channels) are accumulated with
 * atomic adds, so their last bits may differ from run to run; everything else is deterministic.
 * Errors, ownership and asynchrony as in ss_scan_fwd.
 */
int ss_scan_bwd(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                const ss_tensor* C, const ss_tensor* D, const ss_tensor* z, const ss_tensor* delta_bias,
                uint32_t flags, const ss_tensor* dy, ss_tensor* du, ss_tensor* ddelta, ss_tensor* dA,
                ss_tensor* dB, ss_tensor* dC, ss_tensor* dD, ss_tensor* dz, ss_tensor* ddelta_bias,
                void* stream);

/* flags of ss_conv1d */
#define SS_CONV_SILU (1u << 0) /* out = out * sigmoid(out) */

/*
 * ss_conv1d -- causal depthwise convolution along time: the short convolution that each Mamba
 * block applies to the scan's input before the selective SSM, adding local context (bqwf.cn
 * state-space survey, section 3.1; the omica.com.cn explainer, section 6.3, places it before the
 * SSM in Mamba-1 and -2, which the trapezoidal rule of SS_TRAPEZOID makes unnecessary); in
 * decoding the block keeps the last inputs as a state next to the SSM's (the "Mamba -- selective
 * state space model" study notes, pitfalls).  For batch b,
 * channel d and time t, with the inputs before t = 0 taken from state_in (zero without it):
 *
 *   out[b, d, t] = bias[d] + sum_{j=0}^{W-1} weight[d, j] * x[b, d, t - (W-1) + j]
 *   out[b, d, t] *= sigmoid(out[b, d, t])                             if SS_CONV_SILU
 *
 * (weight[d, W-1] multiplies the newest input).  The pages give no width, padding or activation:
 * a causal window of W taps per channel, the inputs before the sequence taken as zero, and silu
 * as an option are the reading taken.
 *
 *   x          [batch, channels, L]          f32 | bf16
 *   weight     [channels, W] f32             W = 1..8 (larger: SS_ERR_UNSUPPORTED; so is
 *                                            batch * channels * ceil(L / 8) >= 2^32 - 256)
 *   bias       [channels] f32                optional (NULL or data == NULL)
 *   state_in   [batch, channels, W-1] f32    optional: x at t = -(W-1) .. -1, oldest first
 *   state_out  [batch, channels, W-1] f32    optional: written with the last W - 1 inputs of
 *                                            state_in followed by x (so the next call continues
 *                                            the sequence; with L < W - 1 part of it comes from
 *                                            state_in).  Must not overlap any other tensor,
 *                                            state_in included (SS_ERR_ALIAS): use two buffers
 *                                            in turn.
 *   flags      SS_CONV_SILU
 *   out        [batch, channels, L]          f32 | bf16, written; must not overlap an input
 *
 * The arithmetic is f32 (bf16 inputs widened exactly; out in bf16 rounded once), the taps summed
 * from the newest input back, so a sequence convolved in pieces with the state carried gives
 * bitwise the out of one call.  L = 0 (state_out = state_in) and batch * channels = 0 are
 * valid.  No workspace.  Errors, ownership and asynchrony as in ss_scan_fwd.
 */
int ss_conv1d(const ss_tensor* x, const ss_tensor* weight, const ss_tensor* bias, const ss_tensor* state_in,
              ss_tensor* state_out, uint32_t flags, ss_tensor* out, void* stream);

/* Synchronises `stream` and returns SS_OK, SS_ERR_HIP if any enqueued work failed, or
 * SS_ERR_DEADLOCK if a kernel's bounded wait ran out since the previous check (on the current
 * device; the record is cleared). */
int ss_check(void* stream);

/* Static, NUL-terminated description of a return code (never NULL). */
const char* ss_strerror(int code);

/* SS_VERSION of the built library. */
int ss_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_SCAN_H */
