/*
 * ssd.h -- C ABI of the MI355X (gfx950) SSD / 2Mamba sequence-mixer library
 * (libssd.so).
 *
 * The library computes the masked linear-attention mixer of Mamba-2,
 * Mamba-2S and 2Mamba ("2Mamba2Furious: Linear in Complexity, Competitive in
 * Accuracy", Mongaras & Larson):
 *
 *     y_i = sum_{j<=i} w_ij V_dt,j / sum_{j<=i} w_ij,
 *     w_ij = (q_i . k_j)^order * exp(A^CS_i - A^CS_j),
 *
 * with A^CS the inclusive cumulative sum of A*dt (Algorithm 3, the Mamba-2
 * forward pass), the decay and causal masks of Algorithms 4 and 5, the
 * squared scores of 2Mamba at order 2 (Algorithm 5) and the row-sum
 * normaliser of Algorithm 1.  The recurrent decode step is the order-p
 * state update of Algorithm 6 (2Mamba inference).  The backward pass (for
 * training; not printed on the pages) is the chain rule through the same
 * definitions.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them.  Arrays are dense, row-major,
 *    with the batch index outermost: [B,H,N,d_h] for q/k/v/y (the pages'
 *    R^{H,N,d_h} per sequence), [B,H,N] for per-token scalars, [H] for
 *    per-head parameters.  Every pointer must be 16-byte aligned.
 *  - order p is 1 (Mamba-2 / Mamba-2S) or 2 (2Mamba); the state width is
 *    D = d_h^p and the order-2 feature of x is vec(x x^T) flattened row-major
 *    (index a*d_h + b).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising.  SSD_OK means "validated and
 *    enqueued"; a device fault surfaces at the caller's next synchronisation.
 *  - Every argument check runs before any HIP call, so a rejected call has no
 *    side effects.  On failure a nonzero ssd_status is returned and
 *    ssd_last_error() describes it (thread-local).  No C++ exception crosses
 *    the ABI.
 *  - Outputs must not overlap inputs (SSD_ERR_ALIAS), except the decode
 *    state, which is updated in place by design.
 *  - Sizes B, H, N (decode: S, H) may be 0: an empty input is valid and the
 *    call does no work (ssd_forward with N = 0 still sets the final states
 *    to the initial ones, or to zero).  A pointer to an array of zero bytes
 *    may be NULL.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 6

typedef enum {
  SSD_OK = 0,
  SSD_ERR_NULL = 1,        /* a required pointer is NULL */
  SSD_ERR_SHAPE = 2,       /* a size is < 1, or sizes overflow */
  SSD_ERR_UNSUPPORTED = 3, /* a parameter combination this build does not implement */
  SSD_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  SSD_ERR_ALIAS = 5,       /* an output overlaps an input or another output */
  SSD_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
  SSD_ERR_HIP = 7          /* the HIP runtime reported an error (see ssd_last_error) */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Layout of the decode states.  SSD_STATE_FULL: D = d_h^p rows, the layout of
 * ssd_forward's states.  SSD_STATE_PACKED (order 2 only): the order-2 feature
 * k (x) k is symmetric in its two indices (Algorithm 6), so state rows (a, b)
 * and (b, a) are equal; the packed layout keeps the rows a <= b only,
 * D' = d_h (d_h + 1) / 2 of them, row-major over the upper triangle (row
 * a d_h - a (a - 1) / 2 + b - a).  Not on the pages: the same state in about
 * half the bytes, which is what a decode step streams. */
typedef enum { SSD_STATE_FULL = 0, SSD_STATE_PACKED = 1 } ssd_state_layout;

/* ABI version of the loaded library (SSD_ABI_VERSION). */
int ssd_abi_version(void);

/* Static, human-readable name of a status code. */
const char* ssd_status_str(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* ssd_last_error(void);

/*
 * ssd_prep -- discretisation and chunk-local log-decay cumsum
 * (Algorithm 3: A = -exp(A_log), dt = softplus(dt_P + dt_bias),
 *  A^CS = cumsum(A * dt); initialisation of dt_bias and A_log per Algorithm 2).
 *
 *   dt_proj [B,H,N] f32   per-token dt logits dt_P
 *   dt_bias [H]     f32
 *   A_log   [H]     f32
 *   chunk           cumsum segment length: 64 or 128
 *   dt      [B,H,N] f32   out: softplus(dt_P + dt_bias)
 *   a_cs    [B,H,N] f32   out: inclusive cumsum of A*dt restarted at every
 *                         multiple of `chunk` (chunk-local A^CS)
 *   a_chunk [B,H,ceil(N/chunk)] f32  out: total of A*dt over each chunk
 *
 * The global A^CS of Algorithm 3 is a_cs plus the sum of the earlier chunk
 * totals; it is never formed, so that decays are always exponentials of
 * non-positive sums of at most `chunk` terms.
 */
ssd_status ssd_prep(const float* dt_proj, const float* dt_bias, const float* A_log,
                    int64_t B, int64_t H, int64_t N, int64_t chunk,
                    float* dt, float* a_cs, float* a_chunk, hipStream_t stream);

/*
 * ssd_prep_amask -- the A-mask of Mamba-2S and 2Mamba (Algorithms 4 and 5):
 * a per-token A = -softplus(A_P) and A^CS = cumsum(A), with no dt in the
 * decay; Algorithm 4's dt = softplus(dt_P) (no bias) for the value operand
 * V*dt, or no dt at all (Algorithm 5 multiplies the scores by plain V: pass
 * dt_proj = dt = NULL here and dt = NULL to ssd_forward).
 *
 *   A_proj  [B,H,N] f32   per-token projection A_P = h W_A
 *   dt_proj [B,H,N] f32   per-token dt logits, or NULL
 *   chunk           cumsum segment length: 64 or 128
 *   dt      [B,H,N] f32   out: softplus(dt_P); must be NULL iff dt_proj is NULL
 *   a_cs    [B,H,N] f32   out: inclusive cumsum of A restarted at every
 *                         multiple of `chunk`
 *   a_chunk [B,H,ceil(N/chunk)] f32  out: total of A over each chunk
 *
 * All pointers are device pointers owned by the caller; errors as ssd_prep
 * (SSD_ERR_NULL also when exactly one of dt_proj, dt is NULL).  a_cs and
 * a_chunk feed ssd_forward exactly as ssd_prep's do.
 */
ssd_status ssd_prep_amask(const float* A_proj, const float* dt_proj, int64_t B, int64_t H,
                          int64_t N, int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                          hipStream_t stream);

/* Workspace bytes ssd_forward needs for these sizes (0 if none; the same
 * validation as ssd_forward applies, and an invalid combination returns 0). */
size_t ssd_forward_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d_h,
                                  int order, int64_t chunk, int dtype);

/*
 * ssd_forward -- chunked parallel form of the masked mixer
 * (Algorithm 1 normaliser and product; Algorithms 4/5 masks; order-2 squared
 *  scores of Algorithm 5; the inter-chunk state is the Algorithm 6 state).
 *
 *   q, k, v [B,H,N,d_h]  dtype (SSD_F32: float, SSD_BF16: bfloat16 bits)
 *   dt      [B,H,N] f32  from ssd_prep; the value operand is V*dt.  NULL means
 *                        v already is the value operand (as Algorithm 5
 *                        prints it, plain V).
 *   a_cs    [B,H,N] f32  chunk-local cumsum from ssd_prep with the same
 *                        `chunk` (every decay is derived from it alone)
 *   initial_state [B,H,D,d_h] f32, initial_norm [B,H,D] f32: in, optional
 *                        (both or neither; NULL = zero): the numerator and
 *                        normaliser states before token 0 (Algorithm 6 H_up,
 *                        H_down; the layout of final_state / final_norm,
 *                        e.g. a previous segment's), decayed from the segment
 *                        start by the cumsum of this segment's a_cs.  At
 *                        order 2 they must be symmetric in (a, b) as
 *                        Algorithm 6's states are (rows (a, b) and (b, a)
 *                        equal; those of ssd_forward, ssd_decode_step and
 *                        ssd_state_unpack are): the forward may read either
 *                        row of such a pair.  Must not overlap any output.
 *   d_h                  32 or 64 (order 1); 64 (order 2)
 *   order                1 or 2 (order 2 requires SSD_BF16)
 *   chunk                64 or 128 (the a_cs segmentation)
 *   y       [B,H,N,d_h] f32  out: normalised output
 *   den     [B,H,N] f32  out, optional (NULL): the row-sum normaliser
 *   final_state [B,H,D,d_h] f32, final_norm [B,H,D] f32: out, optional
 *                        (both or neither): the numerator and normaliser
 *                        states after token N-1 (Algorithm 6 H_up, H_down),
 *                        the hand-off to ssd_decode_step.
 *   workspace            device scratch of >= ssd_forward_workspace_size bytes
 *
 * Internally the sequence is processed in blocks of 64 tokens; the result
 * does not depend on `chunk` beyond floating-point rounding.  The division
 * by the normaliser is exact (no epsilon): rows whose normaliser is 0 give
 * inf/nan, as the definition does.
 */
ssd_status ssd_forward(const void* q, const void* k, const void* v, const float* dt,
                       const float* a_cs, const float* initial_state, const float* initial_norm,
                       int64_t B, int64_t H, int64_t N, int64_t d_h, int order, int64_t chunk,
                       int dtype, float* y, float* den, float* final_state, float* final_norm,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_forward_noalloc -- ssd_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and kernels, with no workspace
 * argument.  Its scratch is a device array inside the library, of
 * SSD_NOALLOC_SCRATCH_BYTES per GPU, held from the library's first use on
 * that GPU until the process ends; the call itself allocates nothing.
 *
 *   arguments      exactly those of ssd_forward without workspace and
 *                  workspace_bytes
 *   sizes          those whose ssd_forward_workspace_size exceeds
 *                  SSD_NOALLOC_SCRATCH_BYTES are rejected with
 *                  SSD_ERR_WORKSPACE (use ssd_forward with a workspace)
 *   concurrency    every call on one GPU uses that GPU's one scratch array:
 *                  calls that overlap in time on one GPU (other streams,
 *                  other threads) race and give wrong results; calls queued
 *                  on one stream are ordered and safe.  No call needs the
 *                  scratch cleared (every byte read is written first in the
 *                  same call).
 * Errors as ssd_forward.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ssd_status ssd_forward_noalloc(const void* q, const void* k, const void* v, const float* dt,
                               const float* a_cs, const float* initial_state,
                               const float* initial_norm, int64_t B, int64_t H, int64_t N,
                               int64_t d_h, int order, int64_t chunk, int dtype, float* y,
                               float* den, float* final_state, float* final_norm,
                               hipStream_t stream);

/*
 * ssd_set_timing_events -- optional per-kernel timing of the next ssd_forward
 * call on the calling thread (used by the benchmark; not part of the math).
 *
 *   events  caller-owned hipEvent_t array of length n (created by the caller)
 *   n       must be >= 5
 *
 * The next ssd_forward on this thread records events[0] on its stream before
 * its first kernel and events[i] after its i-th kernel (i = 1..count); the
 * kernel count is returned by that call's ssd_timing_count().  The
 * registration is consumed by that call.  Passing events = NULL clears it.
 * Order 1 runs 3 kernels (block states, state pass, output); order 2 runs 4
 * (normaliser block states, normaliser pass, numerator state scan, output).
 */
ssd_status ssd_set_timing_events(hipEvent_t* events, int n);

/* Number of kernels the last ssd_forward on this thread timed (0 if none). */
int ssd_timing_count(void);

/*
 * ssd_decode_step -- one recurrent token step (Algorithm 6), in place, with
 * the Mamba-2 discretisation of Algorithm 3.
 *
 *   q, k, v    [S,H,d_h] dtype      this step's token for S sequences
 *   dt_proj    [S,H] f32; dt_bias, A_log [H] f32
 *   layout     ssd_state_layout (SSD_STATE_PACKED requires order 2)
 *   state      [S,H,D,d_h] f32 in/out  numerator state H_up
 *   norm_state [S,H,D] f32 in/out      normaliser state H_down
 *   y          [S,H,d_h] f32 out
 *
 * D = d_h^p (full layout) or d_h (d_h + 1) / 2 (packed).
 * dt = softplus(dt_P + dt_bias); alpha = exp(-exp(A_log) dt);
 * state <- alpha state + phi(k) (v dt)^T; norm_state <- alpha norm_state + phi(k);
 * y = phi(q)^T state / phi(q)^T norm_state, using the updated states (packed:
 * the off-diagonal rows count twice).  d_h is 32 or 64; order 1 or 2.
 */
ssd_status ssd_decode_step(const void* q, const void* k, const void* v,
                           const float* dt_proj, const float* dt_bias, const float* A_log,
                           int64_t S, int64_t H, int64_t d_h, int order, int dtype, int layout,
                           float* state, float* norm_state, float* y, hipStream_t stream);

/*
 * ssd_decode_step_amask -- the decode step as Algorithm 6 prints it: the
 * step's decay factor is a_t = exp(-softplus(h_t W_A)), per sequence and
 * head, with no dt in it (the A-mask of Algorithms 4 and 5, whose prefill is
 * ssd_prep_amask + ssd_forward).
 *
 *   A_proj     [S,H] f32   the projection A_P = h W_A
 *   dt_proj    [S,H] f32 or NULL: the value operand is v softplus(dt_P)
 *              (Algorithm 4's dt, no bias), or plain v when NULL (Algorithms
 *              5 and 6)
 *   everything else as ssd_decode_step.
 */
ssd_status ssd_decode_step_amask(const void* q, const void* k, const void* v,
                                 const float* A_proj, const float* dt_proj, int64_t S,
                                 int64_t H, int64_t d_h, int order, int dtype, int layout,
                                 float* state, float* norm_state, float* y, hipStream_t stream);

/*
 * ssd_decode_step_conv -- the decode step with Algorithm 6's short
 * convolution in front of it: q^c_t, k^c_t, v^c_t = conv_1d(q_t, k_t, v_t,
 * q_{t-1}, k_{t-1}, v_{t-1}, window_size = 2).  The pages name conv_1d
 * without spelling it out; it is taken as the depthwise causal convolution
 * of the q, k, v channels (the d_conv = 3 d_ssm channels of Algorithm 2) that
 * Algorithms 3-5 apply over a whole sequence, one step of it:
 *     x^c = conv_w[.., 0] x_{t-1} + conv_w[.., 1] x_t (+ conv_b), per channel,
 * then SiLU if conv_act = 1 (Algorithm 3 applies sigma after its conv;
 * Algorithm 6 none: conv_act = 0).  The convolved q^c, k^c, v^c (fp32, not
 * rounded to the input type) then take the step of ssd_decode_step_amask
 * (A_proj given: a_t = exp(-softplus(A_P)), value v^c or v^c softplus(dt_P))
 * or of ssd_decode_step (A_proj NULL: dt_proj, dt_bias and A_log required).
 *
 *   q, k, v    [S,H,d_h] dtype   this step's raw projections h_t W_QKV
 *   conv_w     [3,H,d_h,2] f32   per channel (q, k, v planes): the weight of
 *                                the previous token, then of this token
 *   conv_b     [3,H,d_h] f32 or NULL (no bias)
 *   conv_act   0 (none) or 1 (SiLU)
 *   conv_state [S,3,H,d_h] dtype, in/out: the previous step's raw q, k, v
 *              (zeros before a sequence's first token); replaced by this
 *              step's raw q, k, v.  Must not overlap any other argument.
 *   A_proj, dt_proj, dt_bias, A_log: the decay, as described above (with
 *              A_proj, dt_bias and A_log must be NULL)
 *   everything else as ssd_decode_step (state, norm_state in place; y out).
 *
 * Errors as ssd_decode_step; SSD_ERR_NULL when conv_w or conv_state is NULL,
 * SSD_ERR_UNSUPPORTED for another conv_act or for dt_bias / A_log given with
 * A_proj, SSD_ERR_ALIAS when conv_state overlaps another argument.
 */
ssd_status ssd_decode_step_conv(const void* q, const void* k, const void* v, const float* conv_w,
                                const float* conv_b, int conv_act, void* conv_state,
                                const float* A_proj, const float* dt_proj, const float* dt_bias,
                                const float* A_log, int64_t S, int64_t H, int64_t d_h, int order,
                                int dtype, int layout, float* state, float* norm_state, float* y,
                                hipStream_t stream);

/*
 * ssd_state_pack / ssd_state_unpack -- convert order-2 states between the
 * full layout (ssd_forward's final_state / final_norm and initial_state /
 * initial_norm) and the packed one (SSD_STATE_PACKED), for BH (sequence,
 * head) pairs.
 *
 *   full:   state [BH, d_h^2, d_h] f32, norm [BH, d_h^2] f32
 *   packed: state [BH, d_h (d_h + 1) / 2, d_h] f32, norm [BH, d_h (d_h + 1) / 2] f32
 *
 * Packing stores, for every a <= b, the mean of the full rows (a, b) and
 * (b, a): the symmetric part of the state, which is all that phi(q)^T H
 * reads, and exactly the rows themselves when they are equal.  Unpacking
 * writes packed row (min(a,b), max(a,b)) to both full rows.  d_h is 32 or
 * 64; source and destination must not overlap.  Errors as the other calls.
 */
ssd_status ssd_state_pack(const float* state, const float* norm_state, int64_t BH, int64_t d_h,
                          float* state_p, float* norm_p, hipStream_t stream);
ssd_status ssd_state_unpack(const float* state_p, const float* norm_p, int64_t BH, int64_t d_h,
                            float* state, float* norm_state, hipStream_t stream);

/*
 * ssd_backward -- gradients of ssd_forward's y, for training.
 * The pages train these models but print no backward pass: this is the chain
 * rule through the same definitions (Algorithm 1's masked product and row-sum
 * normaliser, Algorithm 4's decay mask, Algorithm 5's squared scores at order
 * 2), on the same 64-token blocks: the states entering each block are
 * recomputed, the gradient of the state leaving each block is scanned in
 * reverse, and each block then forms its gradients from its own tokens and
 * those two states (at order 2 the d_h^2-row states go through HBM, one
 * 1 MiB slot per block and head each).  Sums, scans and pair quantities are
 * fp32; the matrix products run on the bf16 matrix cores with each fp32
 * operand split into a high and a low bf16 part (three products per pair of
 * operands), so every product term carries up to about 3 * 2^-16 of its
 * magnitude instead of fp32's 2^-24, for fp32 and bf16 inputs alike.
 *
 *   q, k, v, dt, a_cs, B..dtype   exactly as given to ssd_forward (dt may be NULL)
 *   y, den    [B,H,N,d_h], [B,H,N] f32   ssd_forward's outputs (den is required)
 *   dy        [B,H,N,d_h] f32            gradient of the loss with respect to y
 *   dq, dk, dv [B,H,N,d_h] f32   out: gradients with respect to q, k, v
 *   ddt       [B,H,N] f32        out: gradient with respect to dt through the
 *                                value operand v dt (sum_c dL/d(v dt)_c v_c);
 *                                NULL iff dt is NULL
 *   da        [B,H,N] f32        out: gradient with respect to the per-token
 *                                log-decay a (A dt, or the A-mask's
 *                                -softplus(A_P)) whose chunk-local cumsum is a_cs
 *   workspace  >= ssd_backward_workspace_size bytes (order 1: ~17 KB per
 *              64-token block and head; order 2: ~2.1 MB per block and head,
 *              the states and state gradients of every block)
 *
 * Orders and sizes as ssd_forward (order 1: d_h 32 or 64, fp32 or bf16;
 * order 2: d_h 64, bf16); no initial state.  Feed (da, ddt) to
 * ssd_prep_backward or ssd_prep_amask_backward for the parameter gradients.
 */
size_t ssd_backward_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d_h, int order,
                                   int64_t chunk, int dtype);
ssd_status ssd_backward(const void* q, const void* k, const void* v, const float* dt,
                        const float* a_cs, const float* y, const float* den, const float* dy,
                        int64_t B, int64_t H, int64_t N, int64_t d_h, int order, int64_t chunk,
                        int dtype, float* dq, float* dk, float* dv, float* ddt, float* da,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_prep_backward -- chain rule through Algorithm 3's discretisation
 * (a = A dt, A = -exp(A_log), dt = softplus(dt_P + dt_bias)):
 *   d_dt_proj = (ddt + da A) sigmoid(dt_P + dt_bias)      [B,H,N]
 *   d_dt_bias[h] = sum over b, n of d_dt_proj              [H]
 *   d_A_log[h] = A_h sum over b, n of da dt                [H]
 * ddt may be NULL (no value-operand use of dt).  The per-head sums are
 * taken in a fixed order (deterministic).
 */
ssd_status ssd_prep_backward(const float* dt_proj, const float* dt_bias, const float* A_log,
                             const float* da, const float* ddt, int64_t B, int64_t H, int64_t N,
                             float* d_dt_proj, float* d_dt_bias, float* d_A_log, hipStream_t stream);

/*
 * ssd_prep_amask_backward -- chain rule through the A-mask of Algorithms 4
 * and 5 (a = -softplus(A_P); dt = softplus(dt_P)):
 *   d_A_proj = -da sigmoid(A_P);  d_dt_proj = ddt sigmoid(dt_P)
 * dt_proj, ddt and d_dt_proj are all given or all NULL.
 */
ssd_status ssd_prep_amask_backward(const float* A_proj, const float* dt_proj, const float* da,
                                   const float* ddt, int64_t B, int64_t H, int64_t N,
                                   float* d_A_proj, float* d_dt_proj, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
