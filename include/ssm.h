/*
 * ssm.h -- C ABI of libssm.so: the Mamba-1 selective scan on MI355X (gfx950): the
 * forward pass, with a carried state, the single-token decode step, and the
 * backward pass.
 *
 * What it computes, per batch b, channel d, time t (t = 0 .. L-1), with a state
 * h[b,d,:] of dstate values that starts at zero:
 *
 *   dt      = softplus(delta[b,d,t] + dt_bias[d])
 *   h[n]    = exp(dt * A[d,n]) * h[n] + dt * B[b,n,t] * u[b,d,t]      (n = 0 .. dstate-1)
 *   y[b,d,t] = (sum_n C[b,n,t] * h[n] + D[d] * u[b,d,t]) * SiLU(z[b,d,t])
 *
 * Sources (page titles as printed on the pages):
 *   - the selective parameterisation (B, C and the step size are functions of the
 *     token, the step size passes through softplus, A stays fixed and diagonal):
 *     yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答" Q4 and Q5;
 *     gongshangzheng.github.io "Mamba" §2.1;
 *   - the recurrence h_t = exp(dt A) h_{t-1} + input term, y_t = C_t h_t:
 *     qubittool.com "Mamba 与状态空间模型：机制、演进与工程选型", section
 *     "Mamba 增加了内容相关的选择机制"; the input term dt*B*u is the first-order
 *     rule that cnblogs.com "Mamba3 技术浅析" §3.1 attributes to Mamba-1;
 *   - read-out after the update and a zero initial state: the scalar model in
 *     section "一个可运行的标量模型" of the qubittool.com page;
 *   - the skip D*u: the continuous output equation, yo3nglau.github.io Q1;
 *   - the SiLU gate: gongshangzheng.github.io "Mamba" §3.1;
 *   - scalar-times-identity decay (nheads > 0): yo3nglau.github.io Q9.
 *
 * Layouts (row-major, last index contiguous, no padding):
 *   u, delta, z, y : (batch, dim, seqlen)   in io_dtype
 *   B, C           : (batch, dstate, seqlen) in io_dtype; one B_t and C_t per token,
 *                                            shared by every channel
 *   A              : float32 (dim, dstate) when nheads == 0;
 *                    float32 (nheads,) when nheads > 0 -- channel d then uses
 *                    A[d / (dim / nheads)] for every n (heads are contiguous
 *                    channel blocks)
 *   D, dt_bias     : float32 (dim,)
 * The state and all arithmetic are float32; y is rounded to io_dtype
 * (round-to-nearest-even for bf16).
 *
 * Memory and ownership: every array pointer is a DEVICE pointer owned by the
 * caller; the library allocates nothing, keeps no global state and never frees
 * caller memory.  u, delta, A, B, C and y are required; D, z and dt_bias may be
 * NULL, meaning no skip, no gate and a zero bias.  y must not overlap any input.
 *
 * Errors: every status except SSM_ERR_HIP is returned synchronously before
 * anything is enqueued, so a refused call has no effect on the device.
 * SSM_ERR_HIP reports a failure of this call's own kernel launches only (each
 * launch's return value is checked).  A HIP error that the caller's earlier HIP
 * calls left pending is neither reported as this call's nor read nor cleared: the
 * caller still gets it from hipGetLastError.  Work is
 * enqueued on `stream` (a hipStream_t; NULL is the default stream) and runs
 * asynchronously; results are visible after the stream is synchronised.  Values
 * are not inspected: NaN or Inf inputs propagate into y as IEEE arithmetic does.
 * Calls that run concurrently must use distinct workspaces.
 */
#ifndef SSM_SELECTIVE_SCAN_H
#define SSM_SELECTIVE_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported from libssm.so even when the library is built with hidden visibility. */
#define SSM_API __attribute__((visibility("default")))

typedef enum ssm_status {
    SSM_OK = 0,
    SSM_ERR_NULL = -1,      /* dims or a required array pointer is NULL */
    SSM_ERR_EMPTY = -2,     /* batch, seqlen, dim or dstate is < 1 */
    SSM_ERR_DIMS = -3,      /* sizes inconsistent or out of range (see ssm_dims) */
    SSM_ERR_DTYPE = -4,     /* io_dtype is not an ssm_dtype value */
    SSM_ERR_ALIGN = -5,     /* an array is not aligned to its element size */
    SSM_ERR_WORKSPACE = -6, /* workspace missing, too small or not 256-byte aligned */
    SSM_ERR_HIP = -7,       /* the HIP runtime reported an error when enqueuing */
    SSM_ERR_ALIAS = -8,     /* an output or the workspace overlaps an input or another output */
    SSM_ERR_DEVICE = -9,    /* ssm_selective_scan_fwd_noalloc: the stream is not the current device's */
    SSM_ERR_SCRATCH = -10   /* ssm_selective_scan_fwd_noalloc: the call needs more scratch than it holds */
} ssm_status;

typedef enum ssm_dtype {
    SSM_F32 = 0,  /* IEEE float32 */
    SSM_BF16 = 1  /* bfloat16 */
} ssm_dtype;

/* Largest dstate a call accepts. */
#define SSM_MAX_DSTATE 256
/* Largest forced chunk count (ssm_dims.nchunks). */
#define SSM_MAX_CHUNKS 1024

typedef struct ssm_dims {
    int64_t batch;    /* B >= 1 */
    int64_t seqlen;   /* L >= 1 */
    int64_t dim;      /* D >= 1, channels */
    int64_t dstate;   /* N, 1 .. SSM_MAX_DSTATE */
    int64_t nheads;   /* 0: A is (dim, dstate); > 0: A is (nheads,), dim % nheads == 0 */
    int32_t io_dtype; /* ssm_dtype of u, delta, z, B, C and y */
    int32_t nchunks;  /* 0: the library decides how many pieces each sequence is cut
                         into along L; k in 1 .. SSM_MAX_CHUNKS forces k pieces (k is
                         clamped to seqlen).  The result is the same up to float
                         rounding whatever the choice. */
    int32_t states_per_lane; /* 0: library choice; 1, 2, 4, 8 or 16 forces how many
                                state entries one GPU lane carries (tuning and tests;
                                same result up to rounding). */
    int32_t reserved;        /* must be 0 */
    void* workspace;         /* device memory for the carries between pieces of one
                                sequence; may be NULL when the required size is 0; it
                                may overlap no input and no output (SSM_ERR_ALIAS) */
    size_t workspace_bytes;  /* size of workspace in bytes */
} ssm_dims;

/* Bytes of workspace the call described by dims needs (0 when it needs none).
 * Returns 0 for a dims pointer that ssm_selective_scan_fwd would refuse. */
SSM_API size_t ssm_selective_scan_workspace_bytes(const ssm_dims* dims);

/* Enqueue the selective-scan forward pass.  Returns an ssm_status value. */
SSM_API int ssm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                   const float* D, const void* z, const float* dt_bias, void* y,
                                   const ssm_dims* dims, void* stream);

/* The same pass with a carried state.  h0 (nullable: zeros) is the float32 state
 * (batch, dim, dstate) before the first step; h_last (nullable: not returned)
 * receives the state after the last step, in the same layout.  h_last may be h0
 * itself (the state is then updated in place) but must not overlap any other array.
 * Carrying the fixed-size state from one call to the next is the recurrent decoding
 * of yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答" Q8 and Q11. */
SSM_API int ssm_selective_scan_fwd_state(const void* u, const void* delta, const float* A, const void* B,
                                         const void* C, const float* D, const void* z, const float* dt_bias,
                                         const float* h0, void* y, float* h_last, const ssm_dims* dims,
                                         void* stream);

/* One decoding step (dims->seqlen must be 1): for every batch row b and channel d,
 *   h[b,d,n] <- exp(dt*A[d,n]) * h[b,d,n] + dt * B[b,n] * u[b,d],  dt = softplus(delta[b,d] + dt_bias[d])
 *   y[b,d]    = (sum_n C[b,n] * h[b,d,n] + D[d] * u[b,d]) * SiLU(z[b,d])
 * u, delta, z, y: (batch, dim) in io_dtype; B, C: (batch, dstate) in io_dtype;
 * h: float32 (batch, dim, dstate), read and updated in place (required).  The O(1)
 * per-token update of yo3nglau.github.io Q8/Q11.  Needs no workspace.  Same error
 * rules as ssm_selective_scan_fwd; seqlen != 1 gives SSM_ERR_DIMS. */
SSM_API int ssm_selective_scan_step(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                    const float* D, const void* z, const float* dt_bias, float* h, void* y,
                                    const ssm_dims* dims, void* stream);

/* The fused front end: a causal depthwise convolution of the scan's input, the "local
 * convolution" a real Mamba layer places before the scan (qubittool.com
 * "Mamba 与状态空间模型：机制、演进与工程选型", the remark after the runnable scalar
 * model), optionally followed by SiLU.  With x the convolution's input, per batch row b,
 * channel d and step t:
 *     u[b,d,t] = act(bias[d] + sum_{k=0}^{width-1} weight[d,k] * x[b,d,t-width+1+k])
 * where x before the first step is the carried history (conv_state, the width-1 inputs
 * before the sequence, oldest first) or 0.  The conv state is part of the per-layer
 * state recurrent decoding keeps (the same page, on inference memory).
 *   weight: float32 (dim, width), required;  bias: float32 (dim,), nullable;
 *   width: 1 .. 4;  silu: 1 = SiLU after the convolution, 0 = none. */
typedef struct ssm_conv {
    const float* weight;
    const float* bias;
    int32_t width;
    int32_t silu;
} ssm_conv;

/* ssm_selective_scan_fwd_state on u = act(conv(x)): x (batch, dim, seqlen) in io_dtype
 * takes the place of u; conv_state (batch, dim, width-1) in io_dtype is the history
 * before x (nullable: zeros).  u is formed inside the scan's staging in float32 and is
 * not rounded before the scan; u_out (nullable, (batch, dim, seqlen) in io_dtype)
 * receives it rounded to io_dtype.  The state after this call's last input, for a
 * following call, is the last width-1 columns of x (with the history when seqlen <
 * width-1).  Same workspace, layouts and rules as the plain forward; u_out may overlap
 * no other array.  conv NULL gives SSM_ERR_NULL, a width outside 1..4 or silu not 0/1
 * SSM_ERR_DIMS. */
SSM_API int ssm_selective_scan_fwd_conv(const void* x, const ssm_conv* conv, const void* conv_state, const void* delta,
                                        const float* A, const void* B, const void* C, const float* D, const void* z,
                                        const float* dt_bias, const float* h0, void* u_out, void* y, float* h_last,
                                        const ssm_dims* dims, void* stream);

/* One decoding step of the fused front end and the scan: x (batch, dim) in io_dtype is
 * the new input; conv_state (batch, dim, width-1) in io_dtype holds the previous
 * width-1 inputs, oldest first, and is shifted in place (required when width > 1);
 * u = act(conv) feeds the step exactly as u does in ssm_selective_scan_step (h updated
 * in place, y written); u_out (nullable) receives u rounded to io_dtype.  Equal, step
 * by step, to ssm_selective_scan_fwd_conv over the same inputs. */
SSM_API int ssm_selective_scan_step_conv(const void* x, const ssm_conv* conv, void* conv_state, const void* delta,
                                         const float* A, const void* B, const void* C, const float* D, const void* z,
                                         const float* dt_bias, float* h, void* u_out, void* y, const ssm_dims* dims,
                                         void* stream);

/* Largest dstate the backward pass accepts. */
#define SSM_MAX_DSTATE_BWD 128

/* Where ssm_selective_scan_bwd writes the gradients.  All device pointers, owned by
 * the caller:
 *   du, ddelta : (batch, dim, seqlen) in io_dtype (rounded to nearest even for bf16)
 *                -- required; ddelta is the gradient at the raw delta input, i.e.
 *                through the softplus
 *   dA         : float32, the shape of A -- required
 *   dB, dC     : float32 (batch, dstate, seqlen) -- required
 *   dD         : float32 (dim,) -- nullable (not computed); the gradient at D, or at
 *                D = 0 when the forward had no skip
 *   dz         : (batch, dim, seqlen) in io_dtype -- nullable; written only when z is
 *                given
 *   ddt_bias   : float32 (dim,) -- nullable; the gradient at dt_bias (or at 0)
 *   dh0        : float32 (batch, dim, dstate) -- nullable; the gradient at h0 (or at
 *                the zero starting state) */
typedef struct ssm_grads {
    void* du;
    void* ddelta;
    float* dA;
    float* dB;
    float* dC;
    float* dD;
    void* dz;
    float* ddt_bias;
    float* dh0;
} ssm_grads;

/* Bytes of workspace ssm_selective_scan_bwd needs for dims (never 0 for a valid
 * dims; 0 for a dims pointer the backward would refuse).  The workspace holds the
 * states recomputed every 16 steps (every 8 steps when dstate > 64): 4 bytes per
 * state entry and interval of every channel, rounded up to whole 64-channel blocks
 * and to the padded entry count; per-block partial sums of dB and dC (8*dstate bytes
 * per token and 64-channel block); and the carries between pieces. */
SSM_API size_t ssm_selective_scan_bwd_workspace_bytes(const ssm_dims* dims);

/* Enqueue the backward pass: the gradients, with respect to every input of
 * ssm_selective_scan_fwd_state, of the scalar
 *     sum_{b,d,t} dy[b,d,t] * y[b,d,t]  +  sum_{b,d,n} dh_last[b,d,n] * h_L[b,d,n]
 * where y and h_L are what the forward computes from the same inputs (dy: the
 * gradient arriving at y, in io_dtype (batch, dim, seqlen), required; dh_last: the
 * gradient arriving at the final state, float32 (batch, dim, dstate), nullable = 0).
 * Training differentiates the scan; as the pages describe for Mamba's kernels, the
 * states are recomputed from the inputs rather than kept from the forward
 * (yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答" Q7; qubittool.com
 * "Mamba 与状态空间模型：机制、演进与工程选型", section "并行训练不会消除递推关系").
 * The inputs are those of the forward call, with the same layouts and nullability;
 * dims is the forward's dims with a workspace of at least
 * ssm_selective_scan_bwd_workspace_bytes(dims) bytes (256-byte aligned).
 * dstate must be <= SSM_MAX_DSTATE_BWD; dims->states_per_lane may force 1, 2, 4, 8
 * or 16 entries per lane as long as that needs at most 8 waves (else SSM_ERR_DIMS).
 * No output may overlap an input, another output or the workspace (SSM_ERR_ALIAS).
 * Every sum (over state entries, channels, batch rows and time) is formed in a fixed
 * order, so repeated calls give bitwise identical gradients.  The workspace holds
 * no state between calls.  Other rules as ssm_selective_scan_fwd. */
SSM_API int ssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                   const float* D, const void* z, const float* dt_bias, const float* h0,
                                   const void* dy, const float* dh_last, const ssm_grads* grads,
                                   const ssm_dims* dims, void* stream);

/* ------------------------------------------------------------------------------
 * Training with saved state checkpoints.  The backward needs the forward's states;
 * like Mamba's kernels it recomputes them instead of storing every step
 * (yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答" Q7).  It recomputes each
 * 16-step interval from the state at the interval's start, and ordinarily first
 * re-walks the sequence to find those states.  A forward that is run anyway (a
 * training step) can keep them instead, and the backward then skips that walk.
 *
 * Checkpoint buffer: float32 [batch][ceil(dim/64)][ceil(seqlen/16)][16][64]; element
 * (b, c, k, n, l) is the state h[b, 64c+l, n] before step 16k (k = 0: h0 or zeros).
 * Elements with n >= dstate or 64c+l >= dim are written by the forward and ignored by
 * the backward.  Supported: 9 <= dstate <= 16 with dims->states_per_lane = 0. */

/* Bytes of the checkpoint buffer for dims; 0 when dims is invalid or not supported. */
SSM_API size_t ssm_selective_scan_ckpt_bytes(const ssm_dims* dims);

/* ssm_selective_scan_fwd_state that also writes the checkpoints to ckpt (required,
 * 4-byte aligned, ssm_selective_scan_ckpt_bytes(dims) bytes, overlapping no input, no
 * other output and no workspace: SSM_ERR_ALIAS).  y and h_last are bitwise those of
 * ssm_selective_scan_fwd_state.  Unsupported dims give SSM_ERR_DIMS. */
SSM_API int ssm_selective_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                                        const void* C, const float* D, const void* z, const float* dt_bias,
                                        const float* h0, void* y, float* h_last, float* ckpt,
                                        const ssm_dims* dims, void* stream);

/* ssm_selective_scan_bwd with the checkpoints that ssm_selective_scan_fwd_ckpt wrote
 * for the same inputs (ckpt: required, 4-byte aligned, read only; no output may
 * overlap it).  Same workspace and results up to float rounding; unsupported dims
 * give SSM_ERR_DIMS. */
SSM_API int ssm_selective_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                                        const void* C, const float* D, const void* z, const float* dt_bias,
                                        const float* h0, const void* dy, const float* dh_last, const float* ckpt,
                                        const ssm_grads* grads, const ssm_dims* dims, void* stream);

/* ------------------------------------------------------------------------------
 * The forward pass for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as ssm_selective_scan_fwd_state, except that the carries between the pieces
 * of a sequence live in a scratch array inside the library instead of a caller
 * workspace (dims->workspace and dims->workspace_bytes are ignored).  The call
 * itself allocates nothing and calls no allocating routine.
 *
 * The scratch is a fixed SSM_NOALLOC_SCRATCH_BYTES per device, held from the moment
 * the library is loaded on that device until the process ends.  A call whose pieces
 * need more (ssm_selective_scan_workspace_bytes(dims) > SSM_NOALLOC_SCRATCH_BYTES)
 * is refused with SSM_ERR_SCRATCH before anything is enqueued.  Nothing in the
 * scratch needs to start at zero: every call writes each carry before it reads it.
 * Every call on a device shares that device's scratch, so calls that may overlap in
 * time on one device (on different streams, or from different threads) race and
 * must be serialised by the caller.  The stream must belong to the current device
 * (else SSM_ERR_DEVICE); the scratch's device address is looked up once per device
 * on its first call that needs pieces (device ordinals 0 .. 63; a call that needs the
 * scratch on a higher ordinal returns SSM_ERR_HIP).  y and h_last are bitwise those of
 * ssm_selective_scan_fwd_state with a workspace.  Other rules as
 * ssm_selective_scan_fwd_state. */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
SSM_API size_t ssm_selective_scan_noalloc_scratch_bytes(void);
SSM_API int ssm_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                                           const void* C, const float* D, const void* z, const float* dt_bias,
                                           const float* h0, void* y, float* h_last, const ssm_dims* dims,
                                           void* stream);

/* Static English text for a status value. */
SSM_API const char* ssm_status_string(int status);

/* How a call would be run: pieces per sequence, states per lane, lanes' waves per
 * workgroup, time tile and workgroup count of the lane walk, and which form runs the
 * full pass: form 0 is the lane walk; form 1 (a scalar decay with bf16 rows of 64 or
 * 128 states and the library's choice of states per lane) is the chunked form, whose
 * state reads and updates are matrix-core products over 16-step chunks, used when the
 * call's rows also allow 16-byte loads (else the walk runs with the same pieces);
 * lds_bytes is that of the form's full pass.  Returns an ssm_status value; fills
 * *plan only on SSM_OK.  Pure host function, never touches the device. */
typedef struct ssm_plan {
    int32_t nchunks;
    int32_t states_per_lane;
    int32_t waves_per_group;
    int32_t time_tile;
    int64_t chunk_len;
    int64_t workgroups;
    size_t workspace_bytes;
    size_t lds_bytes;
    int32_t form;
    int32_t reserved;
} ssm_plan;
SSM_API int ssm_selective_scan_plan(const ssm_dims* dims, ssm_plan* plan);

/* The same for ssm_selective_scan_bwd (workspace_bytes as
 * ssm_selective_scan_bwd_workspace_bytes; time_tile is the recompute interval). */
SSM_API int ssm_selective_scan_bwd_plan(const ssm_dims* dims, ssm_plan* plan);

/* ------------------------------------------------------------------------------
 * Scalar decay with one step size per head: the chunked state-space-duality form.
 *
 * When the state matrix of a head is a scalar times the identity (A = a_h * I,
 * yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答" Q9) and the head's
 * channels share one step size per token, the scan is a masked linear attention and
 * can be computed chunk by chunk with matrix products (the same page, Q10: the
 * duality of SSMs and attention, and the chunked algorithm that processes token
 * blocks on chip).  ssm_ssd_fwd computes, for head h owning channels
 * d = h*headdim .. h*headdim+headdim-1:
 *
 *   dt       = softplus(delta[b,h,t] + dt_bias[h])
 *   h[d,n]   = exp(dt * A[h]) * h[d,n] + dt * B[b,n,t] * u[b,d,t]
 *   y[b,d,t] = (sum_n C[b,n,t] * h[d,n] + D[d] * u[b,d,t]) * SiLU(z[b,d,t])
 *
 * i.e. ssm_selective_scan_fwd_state in scalar-decay mode with delta and dt_bias
 * repeated over each head's channels; the result is the same up to float rounding.
 * The products run on the matrix cores with fp32 accumulation; operands that are not
 * bf16 inputs are split into two bf16 parts, so the arithmetic error stays near fp32
 * scan level rather than bf16 level.
 *
 * Layouts (row-major, no padding; dim = nheads * headdim):
 *   u, z, y : (batch, dim, seqlen) bf16
 *   delta   : (batch, nheads, seqlen) bf16 -- the raw step input, one per head
 *   B, C    : (batch, dstate, seqlen) bf16, shared by every head
 *   A       : float32 (nheads,)
 *   dt_bias : float32 (nheads,), nullable (0)
 *   D       : float32 (dim,), nullable (no skip);  z nullable (no gate)
 *   h0      : float32 (batch, dim, dstate), nullable (zeros) -- the state before the
 *             first step;  h_last: same layout, nullable -- the state after the last
 *             step.  h_last may not overlap h0 or any array.
 * Supported: io_dtype SSM_BF16, headdim 64, dstate 64 or 128 (else SSM_ERR_DTYPE /
 * SSM_ERR_DIMS); seqlen * max(64, dstate) * 2 < 2^31.  Each sequence is cut into
 * nsegments pieces of whole 64-step chunks (0: library choice); C^T B of each chunk
 * and the pieces' end states travel through the workspace (required, 256-byte
 * aligned, ssm_ssd_fwd_workspace_bytes(dims) bytes).
 * Ownership, asynchrony and the other error rules are those of ssm_selective_scan_fwd
 * (y may not overlap an input, and the workspace no input or output: SSM_ERR_ALIAS).
 */
typedef struct ssm_ssd_dims {
    int64_t batch;           /* >= 1 */
    int64_t seqlen;          /* >= 1 */
    int64_t nheads;          /* >= 1 */
    int64_t headdim;         /* channels per head; 64 */
    int64_t dstate;          /* N: 64 or 128 */
    int32_t io_dtype;        /* SSM_BF16 */
    int32_t nsegments;       /* 0: library choice; k in 1 .. SSM_MAX_CHUNKS forces k pieces
                                (clamped to the number of 64-step chunks) */
    int32_t reserved;        /* must be 0 */
    int32_t reserved2;       /* ignored (padding) */
    void* workspace;         /* device memory for C^T B per chunk and the pieces' end
                                states, 256-byte aligned */
    size_t workspace_bytes;
} ssm_ssd_dims;

/* Bytes of workspace ssm_ssd_fwd needs (never 0 for a valid dims; 0 for a dims that
 * ssm_ssd_fwd would refuse): 10240 bytes per batch row and 64-step chunk for C^T B of
 * the chunk (shared by all heads), then 4 * batch * dim * dstate bytes and one float per
 * head for each state piece -- (nsegments - 1) * state_pieces of them, ssm_ssd_fwd_plan
 * -- each part rounded up to 256 bytes. */
SSM_API size_t ssm_ssd_fwd_workspace_bytes(const ssm_ssd_dims* dims);

/* How ssm_ssd_fwd would run dims: pieces (segments) per sequence, 64-step chunks per
 * segment (the last may have fewer), the number of state pieces each segment before
 * the last is cut into for the end-state pass (whole chunks; 1 when nsegments is 1), the
 * chunk length and count, and the workspace size.  Returns an ssm_status value; fills
 * *plan only on SSM_OK.  Pure host function. */
typedef struct ssm_ssd_plan {
    int32_t nsegments;
    int32_t chunks_per_segment;
    int32_t chunk_len;
    int32_t state_pieces;
    int64_t nchunks;
    size_t workspace_bytes;
} ssm_ssd_plan;
SSM_API int ssm_ssd_fwd_plan(const ssm_ssd_dims* dims, ssm_ssd_plan* plan);

/* Enqueue the scalar-decay per-head-step forward pass.  Returns an ssm_status value. */
SSM_API int ssm_ssd_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                        const float* D, const void* z, const float* dt_bias, const float* h0, void* y,
                        float* h_last, const ssm_ssd_dims* dims, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SELECTIVE_SCAN_H */
