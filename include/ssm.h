/*
 * ssm.h -- C ABI of libssm.so: the Mamba-1 selective-scan forward pass on MI355X (gfx950).
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
 * anything is enqueued, so a refused call has no effect on the device.  Work is
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
    SSM_ERR_ALIAS = -8      /* y overlaps one of the inputs */
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
                                sequence; may be NULL when the required size is 0 */
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

/* Static English text for a status value. */
SSM_API const char* ssm_status_string(int status);

/* How a call would be run: pieces per sequence, states per lane, lanes' waves per
 * workgroup, time tile and workgroup count.  Returns an ssm_status value; fills
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
} ssm_plan;
SSM_API int ssm_selective_scan_plan(const ssm_dims* dims, ssm_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SELECTIVE_SCAN_H */
