/*
 * mss.h -- C ABI of libmss, the MI355X (gfx950) Mamba selective-scan library.
 *
 * Six operations.  The scan forward and backward can also run in reverse
 * time (mss_scan_args.reverse), the second direction of a bidirectional
 * layer (SpeechLens kernel-optimization notes, the bidirectional variant in
 * its rejected-fusion list):
 *
 *  1. mss_selective_scan_fwd: the selective-scan forward over whole sequences.
 *     For every channel (b, d) and time step t, with n over the dstate
 *     diagonal state entries:
 *        delta_t = softplus(delta_raw[b,d,t] + dt_bias[d])   (or without softplus)
 *        A[n]    = -exp(A_log[d,n])
 *        h_t[n]  = exp(delta_t * A[n]) * h_{t-1}[n] + delta_t * B[b,n,t] * u[b,d,t]
 *        y_t     = sum_n C[b,n,t] * h_t[n] + D[d] * u[b,d,t]
 *        out[b,d,t] = y_t * z[b,d,t] * sigmoid(z[b,d,t])      (if z is given)
 *     with h_{-1} = initial_state (or 0), and optionally exporting the state
 *     after the last step.
 *     Sources: the recurrence and its diagonal discretisation
 *     ("mamba-metal: Apple Silicon で Mamba を動かす", section
 *     "Selective scan の本質"; createcentury's reading of the official CUDA
 *     kernel, sections "なぜ「scan」か" and "1チャンク内の処理フロー");
 *     softplus and -exp(A_log) fused into the scan, tensor roles and the
 *     fixed 16-entry state (SpeechLens kernel-optimization notes, selective-scan
 *     contract table); the final-state hand-off ("mamba-metal", section
 *     "残り課題").
 *
 *  2. mss_selective_state_update: one decode step, O(1) per token: the loop
 *     body above applied once to a caller-held state, updated in place
 *     ("mamba-metal", section "O(L) インクリメンタルデコード", per-step
 *     equation, closed by the z gate).
 *
 *  3. mss_causal_conv1d_fwd: the causal depthwise conv1d, with an optional
 *     SiLU, that produces the scan's input u in a Mamba block
 *     ("mamba-metal", section "カーネルから推論まで": in_proj -> conv1d ->
 *     SiLU -> ... -> SSM).  Per channel (b, d) and step t, with `width` taps
 *     (4 in the pages' models):
 *        pre[b,d,t] = bias[d] + sum_k weight[d,k] * x~[b,d,t-(width-1)+k]
 *        out[b,d,t] = silu(pre) (or pre without the activation)
 *     where x~ is x extended to the left by the carried window
 *     initial_state[b,d,0..width-2] (oldest first), or by zeros when it is
 *     NULL: three zero samples on the causal left edge for width 4
 *     (SpeechLens kernel-optimization notes, causal depthwise convolution
 *     section and its contract table).  The window after the last step (the
 *     last width-1 samples of x~) can be exported for decoding.
 *
 *  4. mss_causal_conv1d_update: one decode step of that conv: the carried
 *     window followed by the new sample is filtered, and the window slides
 *     by one in place ("mamba-metal", section "O(L) インクリメンタルデコード":
 *     the conv1d sliding window is carried between calls).
 *
 *  5. mss_selective_scan_bwd: the backward of operation 1 for training, which
 *     the pages list as not yet written ("mamba-metal", section "残り課題").
 *     Given dout = dLoss/dout (and optionally dfinal_state = dLoss/d final
 *     state) it returns dLoss/d(u, delta_raw, A_log, B, C, D, z, dt_bias,
 *     initial_state), the chain rule through the forward taken in reverse
 *     time:  with G_t[n] the adjoint of h_t[n], g[n] the part that reaches
 *     h_t[n] from later steps (dfinal_state at the end), dy_t = dout_t silu(z_t):
 *        G_t[n] = g[n] + dy_t C_t[n];   g[n] <- G_t[n] exp(delta_t A[n]);
 *        dC_t[n] = sum_d dy_t h_t[n];   dB_t[n] = sum_d G_t[n] delta_t u_t;
 *        du_t = dy_t D + delta_t sum_n G_t[n] B_t[n];
 *        ddelta_t = u_t sum_n G_t[n] B_t[n] + sum_n G_t[n] h_{t-1}[n] exp(delta_t A[n]) A[n];
 *        ddelta_raw_t = ddelta_t sigmoid(delta_raw_t + dt_bias) (softplus on);
 *        dz_t = dout_t y_t silu'(z_t);  dD = sum dy u;  ddt_bias = sum ddelta_raw;
 *        dA_log[d,n] = A[n] sum_(b,t) G_t[n] h_{t-1}[n] exp(delta_t A[n]) delta_t;
 *        dinitial_state = g after the first step.
 *
 *  6. mss_selective_scan_fwd_complex: operation 1 with a complex diagonal A,
 *     the variant the official CUDA kernel carries with its own complex exp2
 *     (createcentury's reading of the kernel, section "主要な最適化テクニック"):
 *        A[n]   = -exp(A_log[d,n]) + i A_imag[d,n]
 *        h_t[n] = exp(delta_t * A[n]) * h_{t-1}[n] + delta_t * B[b,n,t] * u[b,d,t]
 *        y_t    = Re(sum_n C[b,n,t] * h_t[n]) + D[d] * u[b,d,t]
 *     with complex B, C and states, real u, delta_raw, z and out, and delta,
 *     the skip term and the gate as in operation 1.  The pages do not spell
 *     out the parameters; this is the plainest reading (the decay from the
 *     real part as in the real case, the rotation from the imaginary part,
 *     the real part of the output).  fp32 activations only.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains caller memory and keeps no per-call
 *    state; it caches nothing but compiled kernels and the device address of
 *    the scratch array of mss_selective_scan_fwd_noalloc.
 *  - Tensors are described by element strides in LOGICAL index order:
 *    u / delta_raw / z / out as (b, d, t), B / C as (b, n, t), A_log as (d, n).
 *    For the scan forward, u, delta_raw, z and out must share a unit-stride
 *    axis, t or d (for example [B,D,L] or channel-last [B,L,D] buffers), and
 *    B and C must share one, t or n, unless both have time stride 0
 *    (time-invariant B and C, any state stride: the forward then holds them
 *    in registers); the conv1d and the backward accept any non-negative
 *    strides.  Other strides are free (views into larger buffers are fine).
 *    A dimension of size 1 may have any stride.  D, dt_bias and the states
 *    are contiguous.
 *  - io_dtype selects the element type of u, delta_raw, z, B, C and out
 *    (fp32 or bf16).  A_log, D, dt_bias and every state are always fp32;
 *    arithmetic is fp32 throughout and bf16 outputs are rounded to nearest even.
 *  - Execution is asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *    the null stream).  Functions return once the work is enqueued.  Nothing
 *    synchronises the device.
 *  - Errors are reported by return value, never by exceptions or aborts.  All
 *    argument checks run before any HIP call: on an error nothing is launched
 *    and no memory is touched.  MSS_ERR_HIP reports a failure that the HIP
 *    runtime returned while enqueuing.
 *  - out and final_state must not overlap any input (the scan reads its inputs
 *    after it has started writing); the state of a state update is the only
 *    in/out buffer.
 *  - Thread-safe: concurrent calls on different streams are independent,
 *    except calls of mss_selective_scan_fwd_noalloc on one GPU (they share
 *    its scratch array).
 */
#ifndef MSS_H
#define MSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSS_ABI_VERSION 5

/* Chunk states: the state entering every MSS_STATE_CHUNK-step chunk of
 * logical time, fp32, laid out [ceil(L / MSS_STATE_CHUNK)][b][d][MSS_MAX_DSTATE]
 * contiguous (entries n >= dstate hold 0).  The forward can record them
 * (mss_scan_args.chunk_states) for the backward to read
 * (mss_scan_bwd_args.chunk_states), which then skips its own forward pass
 * over the sequence: the saved-activation scheme of a training step. */
#define MSS_STATE_CHUNK 16
#define MSS_MAX_DSTATE 16
#define MSS_MAX_CONV_WIDTH 4

/* Device scratch that mss_selective_scan_fwd_noalloc holds per GPU (16 MiB):
 * enough for the time-segment carries of any shape (at most 6.3 MB, for
 * fewer than 16384 (batch, channel) pairs) together with its ragged-tail
 * state hand-off, and for the hand-off alone of up to 262144 pairs (64 bytes
 * each). */
#define MSS_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef enum mss_status {
    MSS_OK = 0,
    MSS_ERR_NULL_POINTER = 1,       /* a required pointer is NULL                      */
    MSS_ERR_BAD_SHAPE = 2,          /* batch, dim, seqlen < 1, sizes overflow, or a    */
                                    /* conv width outside [1, MSS_MAX_CONV_WIDTH]      */
    MSS_ERR_BAD_STRIDE = 3,         /* negative, overlapping or no unit-stride axis    */
    MSS_ERR_UNSUPPORTED_DTYPE = 4,  /* io_dtype is not MSS_F32 or MSS_BF16             */
    MSS_ERR_UNSUPPORTED_DSTATE = 5, /* dstate outside [1, MSS_MAX_DSTATE]              */
    MSS_ERR_MISALIGNED = 6,         /* a pointer is not aligned to its element size    */
    MSS_ERR_WORKSPACE_TOO_SMALL = 7,/* workspace_bytes below the required size         */
    MSS_ERR_ALIASING = 8,           /* an output overlaps an input                     */
    MSS_ERR_BAD_STRUCT = 9,         /* args is NULL or struct_size does not match      */
    MSS_ERR_HIP = 10,               /* the HIP runtime reported an error               */
    MSS_ERR_SCRATCH_LIMIT = 11      /* mss_selective_scan_fwd_noalloc: the shape needs */
                                    /* more than MSS_NOALLOC_SCRATCH_BYTES of scratch  */
} mss_status;

typedef enum mss_dtype {
    MSS_F32 = 0,
    MSS_BF16 = 1
} mss_dtype;

/* Activation applied after the conv1d. */
typedef enum mss_activation {
    MSS_ACT_NONE = 0,
    MSS_ACT_SILU = 1             /* silu(v) = v * sigmoid(v)                             */
} mss_activation;

/* Arguments of mss_selective_scan_fwd.  Set struct_size = sizeof(mss_scan_args). */
typedef struct mss_scan_args {
    uint32_t struct_size;
    int32_t io_dtype;            /* mss_dtype of u, delta_raw, z, B, C, out              */
    int64_t batch;               /* B >= 1                                               */
    int64_t dim;                 /* D >= 1 (d_inner channels)                            */
    int64_t seqlen;              /* 1 <= L <= 2^30                                       */
    int64_t dstate;              /* N, 1..MSS_MAX_DSTATE                                 */

    const void *u;               /* [b,d,t] input activation                            */
    int64_t u_stride[3];
    const void *delta_raw;       /* [b,d,t] time step before bias and softplus           */
    int64_t delta_stride[3];
    const float *A_log;          /* [d,n] fp32, A = -exp(A_log)                          */
    int64_t A_log_stride[2];
    const void *B;               /* [b,n,t] input coefficients                           */
    int64_t B_stride[3];
    const void *C;               /* [b,n,t] output coefficients                          */
    int64_t C_stride[3];
    const float *D;              /* [d] fp32 skip, contiguous; NULL means 0              */
    const void *z;               /* [b,d,t] gate; NULL means no gate                     */
    int64_t z_stride[3];
    const float *dt_bias;        /* [d] fp32, contiguous; NULL means 0                   */
    const float *initial_state;  /* [b,d,n] fp32 contiguous h_{-1}; NULL means 0         */

    void *out;                   /* [b,d,t] result, io_dtype                             */
    int64_t out_stride[3];
    float *final_state;          /* [b,d,n] fp32 contiguous h_{L-1}; NULL: not written   */
    float *chunk_states;         /* see MSS_STATE_CHUNK, 8-byte aligned; NULL: not       */
                                 /* written                                              */

    int32_t delta_softplus;      /* nonzero: delta = softplus(delta_raw + dt_bias)       */
    int32_t reverse;             /* 0: forward in time.  1: reverse time, logical step   */
                                 /* tau reads and writes storage step seqlen-1-tau (the  */
                                 /* backward half of a bidirectional layer, no copies);  */
                                 /* final_state is then the state after storage step 0   */

    void *workspace;             /* device scratch, 256-byte aligned, of at least        */
    size_t workspace_bytes;      /* mss_selective_scan_workspace_size bytes (may be 0)   */
} mss_scan_args;

/* Arguments of mss_selective_state_update.  Set struct_size = sizeof(mss_step_args). */
typedef struct mss_step_args {
    uint32_t struct_size;
    int32_t io_dtype;            /* mss_dtype of u, delta_raw, z, B, C, out              */
    int64_t batch;
    int64_t dim;
    int64_t dstate;              /* 1..MSS_MAX_DSTATE                                    */

    float *state;                /* [b,d,n] fp32 contiguous, read and updated in place   */
    const void *u;               /* [b,d]                                                */
    int64_t u_stride[2];
    const void *delta_raw;       /* [b,d]                                                */
    int64_t delta_stride[2];
    const float *A_log;          /* [d,n] fp32                                           */
    int64_t A_log_stride[2];
    const void *B;               /* [b,n]                                                */
    int64_t B_stride[2];
    const void *C;               /* [b,n]                                                */
    int64_t C_stride[2];
    const float *D;              /* [d] fp32 contiguous; NULL means 0                    */
    const void *z;               /* [b,d]; NULL means no gate                            */
    int64_t z_stride[2];
    const float *dt_bias;        /* [d] fp32 contiguous; NULL means 0                    */
    void *out;                   /* [b,d] result, io_dtype                               */
    int64_t out_stride[2];
    int32_t delta_softplus;
    int32_t reserved0;           /* must be 0                                            */
} mss_step_args;

/* Arguments of mss_causal_conv1d_fwd.  Set struct_size = sizeof(mss_conv_args). */
typedef struct mss_conv_args {
    uint32_t struct_size;
    int32_t io_dtype;            /* mss_dtype of x, out and both windows                 */
    int64_t batch;               /* B >= 1                                               */
    int64_t dim;                 /* D >= 1 channels                                      */
    int64_t seqlen;              /* 1 <= L <= 2^30                                       */
    int64_t width;               /* taps, 1..MSS_MAX_CONV_WIDTH                          */

    const void *x;               /* [b,d,t] input                                        */
    int64_t x_stride[3];
    const float *weight;         /* [d,k] fp32 taps, oldest sample first (a framework    */
    int64_t weight_stride[2];    /* Conv1d weight [D,1,W] or [D,W,1] viewed as [D,W])    */
    const float *bias;           /* [d] fp32 contiguous; NULL means 0                    */
    const void *initial_state;   /* [b,d,width-1] io_dtype contiguous: the window before */
                                 /* t = 0, oldest first; NULL means zeros                */
    void *out;                   /* [b,d,t] result, io_dtype                             */
    int64_t out_stride[3];
    void *final_state;           /* [b,d,width-1] io_dtype contiguous: the window after  */
                                 /* the last step; NULL: not written                     */
    int32_t activation;          /* mss_activation                                       */
    int32_t reserved0;           /* must be 0                                            */
} mss_conv_args;

/* Arguments of mss_causal_conv1d_update.  Set struct_size = sizeof(mss_conv_step_args). */
typedef struct mss_conv_step_args {
    uint32_t struct_size;
    int32_t io_dtype;            /* mss_dtype of state, x and out                        */
    int64_t batch;
    int64_t dim;
    int64_t width;               /* 1..MSS_MAX_CONV_WIDTH                                */

    void *state;                 /* [b,d,width-1] io_dtype contiguous window, oldest     */
                                 /* first, read and slid in place (NULL iff width == 1)  */
    const void *x;               /* [b,d] new sample                                     */
    int64_t x_stride[2];
    const float *weight;         /* [d,k] fp32                                           */
    int64_t weight_stride[2];
    const float *bias;           /* [d] fp32 contiguous; NULL means 0                    */
    void *out;                   /* [b,d] result, io_dtype                               */
    int64_t out_stride[2];
    int32_t activation;          /* mss_activation                                       */
    int32_t reserved0;           /* must be 0                                            */
} mss_conv_step_args;

/* Arguments of mss_selective_scan_bwd.  Set struct_size = sizeof(mss_scan_bwd_args).
 * The forward's inputs have the meaning, layout rules and nullability of
 * mss_scan_args, except that any non-negative strides are accepted. */
typedef struct mss_scan_bwd_args {
    uint32_t struct_size;
    int32_t io_dtype;            /* mss_dtype of u, delta_raw, z, B, C, dout and of the  */
                                 /* gradients du, ddelta_raw, dz, dB, dC                 */
    int64_t batch;
    int64_t dim;
    int64_t seqlen;
    int64_t dstate;              /* 1..MSS_MAX_DSTATE                                    */

    const void *u;               /* [b,d,t]                                              */
    int64_t u_stride[3];
    const void *delta_raw;       /* [b,d,t]                                              */
    int64_t delta_stride[3];
    const float *A_log;          /* [d,n] fp32                                           */
    int64_t A_log_stride[2];
    const void *B;               /* [b,n,t]                                              */
    int64_t B_stride[3];
    const void *C;               /* [b,n,t]                                              */
    int64_t C_stride[3];
    const float *D;              /* [d] fp32 contiguous; NULL means 0                    */
    const void *z;               /* [b,d,t]; NULL means no gate                          */
    int64_t z_stride[3];
    const float *dt_bias;        /* [d] fp32 contiguous; NULL means 0                    */
    const float *initial_state;  /* [b,d,n] fp32 contiguous; NULL means 0                */
    int32_t delta_softplus;
    int32_t reverse;             /* 0 or 1, as in mss_scan_args: the backward of the     */
                                 /* reverse-time forward                                 */

    const void *dout;            /* [b,d,t] dLoss/dout                                   */
    int64_t dout_stride[3];
    const float *dfinal_state;   /* [b,d,n] fp32 contiguous; NULL means 0                */
    const float *chunk_states;   /* chunk states recorded by the forward on the same     */
                                 /* inputs and flags (see MSS_STATE_CHUNK), 8-byte       */
                                 /* aligned; NULL: the backward recomputes them          */

    void *du;                    /* [b,d,t] required                                     */
    int64_t du_stride[3];
    void *ddelta_raw;            /* [b,d,t] required                                     */
    int64_t ddelta_stride[3];
    float *dA_log;               /* [d,n] fp32 contiguous, required                      */
    void *dB;                    /* [b,n,t] required                                     */
    int64_t dB_stride[3];
    void *dC;                    /* [b,n,t] required                                     */
    int64_t dC_stride[3];
    float *dD;                   /* [d] fp32; NULL: not written                          */
    void *dz;                    /* [b,d,t]; NULL: not written (must be NULL without z)  */
    int64_t dz_stride[3];
    float *ddt_bias;             /* [d] fp32; NULL: not written                          */
    float *dinitial_state;       /* [b,d,n] fp32 contiguous; NULL: not written           */

    void *workspace;             /* device scratch, 256-byte aligned, of at least        */
    size_t workspace_bytes;      /* mss_selective_scan_bwd_workspace_size bytes          */
} mss_scan_bwd_args;

/* ABI version of the loaded library (MSS_ABI_VERSION of its build). */
int mss_abi_version(void);

/* Static text for a status code (never NULL). */
const char *mss_status_string(mss_status status);

/* Bytes of device workspace mss_selective_scan_fwd needs for these arguments.
 * It is 0 unless the shape is split into time segments (few channels, long
 * sequence), in which case it holds the per-segment state carries.  Depends
 * only on the shapes, so it can be called before any pointer is set.  Returns 0
 * and sets *status (if non-NULL) to an error code when the shapes are
 * invalid. */
size_t mss_selective_scan_workspace_size(const mss_scan_args *args, mss_status *status);

/* Selective-scan forward (see the top of this file).  `stream` is a
 * hipStream_t.  The workspace, when needed, is overwritten; it carries no
 * state between calls, and calls that share one workspace on different
 * streams race. */
mss_status mss_selective_scan_fwd(const mss_scan_args *args, void *stream);

/* Selective-scan forward that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code recorded under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * arguments, checks, kernels and results as mss_selective_scan_fwd, except:
 *  - args->workspace must be NULL and args->workspace_bytes 0
 *    (MSS_ERR_BAD_STRUCT otherwise);
 *  - what the workspace would hold (the time-segment carries and the
 *    ragged-tail state hand-off) lives in a device array of the library,
 *    MSS_NOALLOC_SCRATCH_BYTES on every GPU it runs on, held from the first
 *    call on that GPU until the process ends.  A shape whose
 *    mss_selective_scan_workspace_size exceeds it returns
 *    MSS_ERR_SCRATCH_LIMIT, like every argument error before any HIP call;
 *  - every call on one GPU uses that GPU's one array: calls that overlap in
 *    time on one GPU (on different streams, or from several host threads)
 *    race and give wrong results.  Order them on one stream.  Nothing in the
 *    array has to start at zero: a call reads only what it wrote before;
 *  - the first call on a GPU looks up the array's device address (a HIP
 *    runtime query, no allocation), so record that call outside a graph
 *    capture, or call once before capturing.
 * No hipMalloc, hipFree or allocating library routine is ever called. */
mss_status mss_selective_scan_fwd_noalloc(const mss_scan_args *args, void *stream);

/* One-token state update (see the top of this file). */
mss_status mss_selective_state_update(const mss_step_args *args, void *stream);

/* Arguments of mss_selective_scan_fwd_complex.  Set struct_size =
 * sizeof(mss_scan_complex_args).  Complex values are (re, im) fp32 pairs
 * (8 bytes, 8-byte aligned, the layout of C99 float _Complex); their strides
 * count complex elements. */
typedef struct mss_scan_complex_args {
    uint32_t struct_size;
    int32_t reserved0;           /* must be 0                                            */
    int64_t batch;               /* B >= 1                                               */
    int64_t dim;                 /* D >= 1                                               */
    int64_t seqlen;              /* 1 <= L <= 2^30                                       */
    int64_t dstate;              /* N, 1..MSS_MAX_DSTATE                                 */

    const float *u;              /* [b,d,t] fp32                                         */
    int64_t u_stride[3];
    const float *delta_raw;      /* [b,d,t] fp32                                         */
    int64_t delta_stride[3];
    const float *A_log;          /* [d,n] fp32, Re(A) = -exp(A_log)                      */
    int64_t A_log_stride[2];
    const float *A_imag;         /* [d,n] fp32, Im(A)                                    */
    int64_t A_imag_stride[2];
    const void *B;               /* [b,n,t] complex                                      */
    int64_t B_stride[3];
    const void *C;               /* [b,n,t] complex                                      */
    int64_t C_stride[3];
    const float *D;              /* [d] fp32 contiguous; NULL means 0                    */
    const float *z;              /* [b,d,t] fp32; NULL means no gate                     */
    int64_t z_stride[3];
    const float *dt_bias;        /* [d] fp32 contiguous; NULL means 0                    */
    const void *initial_state;   /* [b,d,n] complex contiguous; NULL means 0             */

    float *out;                  /* [b,d,t] fp32 result                                  */
    int64_t out_stride[3];
    void *final_state;           /* [b,d,n] complex contiguous; NULL: not written        */

    int32_t delta_softplus;      /* nonzero: delta = softplus(delta_raw + dt_bias)       */
    int32_t reserved1;           /* must be 0                                            */

    void *workspace;             /* device scratch, 256-byte aligned, of at least        */
    size_t workspace_bytes;      /* mss_selective_scan_fwd_complex_workspace_size bytes  */
                                 /* (may be 0)                                           */
} mss_scan_complex_args;

/* Bytes of device workspace mss_selective_scan_fwd_complex needs.  It is 0
 * unless the shape has few channels (fewer than 512 tiles of 16) and is cut
 * into time segments, whose complex state carries it holds.  Depends only on
 * the shapes.  Returns 0 and sets *status (if non-NULL) on invalid shapes. */
size_t mss_selective_scan_fwd_complex_workspace_size(const mss_scan_complex_args *args,
                                                     mss_status *status);

/* Selective-scan forward with complex A (operation 6 at the top of this
 * file).  The same checks and errors as mss_selective_scan_fwd, and the same
 * workspace rules.  out and final_state must not overlap any input or each
 * other. */
mss_status mss_selective_scan_fwd_complex(const mss_scan_complex_args *args, void *stream);

/* Bytes of device workspace mss_selective_scan_bwd needs: the states entering
 * every 16-step chunk (batch * dim * seqlen * 4 bytes, rounded up) and the
 * per-32-channel partial sums of dB and dC (batch * ceil(dim/32) * 32 *
 * seqlen * 4 bytes).  Depends only on the shapes.  Returns 0 and sets
 * *status on invalid shapes. */
size_t mss_selective_scan_bwd_workspace_size(const mss_scan_bwd_args *args, mss_status *status);

/* Selective-scan backward (see the top of this file).  Every gradient output
 * is overwritten (not accumulated into).  Outputs must not overlap any input,
 * each other or the workspace.  Deterministic: sums run in a fixed order. */
mss_status mss_selective_scan_bwd(const mss_scan_bwd_args *args, void *stream);

/* Causal depthwise conv1d with optional SiLU (see the top of this file).
 * Any non-negative strides are accepted.  When x and out share a unit-stride
 * axis, t or d ([B,D,L] or channel-last [B,L,D] buffers), and 4-element
 * vectors along it are aligned (base pointers aligned to 4 elements, the other
 * strides multiples of 4, and for the d axis dim a multiple of 4), the kernel
 * moves whole vectors; otherwise it reads element by element.  The result is
 * the same either way.  out and final_state must not overlap any input.  No
 * workspace. */
mss_status mss_causal_conv1d_fwd(const mss_conv_args *args, void *stream);

/* One decode step of the conv1d (see the top of this file).  The window
 * `state` is the only in/out buffer; out must not overlap it or any input. */
mss_status mss_causal_conv1d_update(const mss_conv_step_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSS_H */
