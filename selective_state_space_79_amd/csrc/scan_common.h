// scan_common.h -- device helpers shared by the forward (scan_fwd.hip) and backward
// (scan_bwd.hip) kernels of libssm: element I/O of fp32 and bf16 rows, and the fp32
// elementwise functions of the scan (softplus in log2 units, SiLU, sigmoid).
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <tuple>

#include "ssm.h"

// ------------------------------------------------------------------ kernel launches
// Every kernel is launched through launch_kernel(), which calls hipLaunchKernel and
// keeps the first failure of the calling thread's current entry point in
// ssm_detail::launch_error.  An entry point resets it before its first launch and
// reports it after its last, so SSM_ERR_HIP is exactly this call's launch failures;
// the thread's pending HIP error (hipGetLastError), which the caller's earlier HIP
// calls may have left, is never read, reported or cleared by the library.
namespace ssm_detail {
inline thread_local hipError_t launch_error = hipSuccess;
}  // namespace ssm_detail

template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                          Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> held(static_cast<KArgs>(args)...);
    const hipError_t e = std::apply(
        [&](auto&... a) {
            void* ptrs[] = {static_cast<void*>(&a)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream);
        },
        held);
    if (e != hipSuccess && ssm_detail::launch_error == hipSuccess) ssm_detail::launch_error = e;
}

namespace {

constexpr int kLanes = 64;               // wave64: one lane per channel
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ element I/O
// bf16 values travel as uint16_t; f32 as float.  A "vector" is 16 bytes of one row.
template <typename IO> struct IOT;
template <> struct IOT<float> {
    static constexpr int VW = 4;
    __device__ static inline float to_f32(float v) { return v; }
    __device__ static inline float from_f32(float v) { return v; }
};
template <> struct IOT<uint16_t> {
    static constexpr int VW = 8;
    __device__ static inline float to_f32(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
    __device__ static inline uint16_t from_f32(float v) {
        __bf16 b = static_cast<__bf16>(v);   // v_cvt_pk_bf16_f32: round to nearest even
        uint16_t r;
        __builtin_memcpy(&r, &b, 2);
        return r;
    }
};

template <typename IO> struct Vec {
    IO e[IOT<IO>::VW];
};

// Load one 16-byte vector of a row: vector instruction when aligned, else per element.
template <typename IO, bool VEC>
__device__ inline Vec<IO> load_vec(const IO* __restrict__ row, int64_t t, int64_t tend, bool ok) {
    constexpr int VW = IOT<IO>::VW;
    Vec<IO> v;
    if constexpr (VEC) {
        if (ok && t < tend) {
            uint4 raw = *reinterpret_cast<const uint4*>(row + t);
            __builtin_memcpy(&v, &raw, 16);
        } else {
            uint4 raw = make_uint4(0, 0, 0, 0);
            __builtin_memcpy(&v, &raw, 16);
        }
    } else {
#pragma unroll
        for (int e = 0; e < VW; ++e) v.e[e] = (ok && t + e < tend) ? row[t + e] : IO(0);
    }
    return v;
}

template <typename IO, bool VEC>
__device__ inline void store_vec(IO* __restrict__ row, int64_t t, int64_t tend, bool ok, const Vec<IO>& v) {
    constexpr int VW = IOT<IO>::VW;
    if constexpr (VEC) {
        if (ok && t < tend) {
            uint4 raw;
            __builtin_memcpy(&raw, &v, 16);
            *reinterpret_cast<uint4*>(row + t) = raw;
        }
    } else {
#pragma unroll
        for (int e = 0; e < VW; ++e)
            if (ok && t + e < tend) row[t + e] = v.e[e];
    }
}

// ------------------------------------------------------------------ elementwise math (fp32)
// Step sizes are carried in log2 units, dt2 = softplus(v) / ln 2, so that the decay
// exp(dt * A) is one exp2(dt2 * A) and no ln 2 scaling is needed per state entry
// (ln 2 is folded into B once per token instead).
//
// dt2 = max(v, 0) * log2(e) + log2(1 + e),  e = 2^(-|v| log2 e) in (0, 1].
// w = fl(1 + e) carries the rounding error c = (w - 1) - e, which is exact in fp32
// (both subtractions are exact by Sterbenz' lemma), so log2(1 + e) = log2(w - c)
// = log2(w) - c / (w ln 2) + O(c^2).  Using c / ln 2 instead of c / (w ln 2) changes
// the result by at most |c| (1 - 1/w) / ln 2 <= 2^-25 / ln 2 absolute, and by at most
// 2^-24 relative when e is small (w close to 1), i.e. below fp32 rounding.
__device__ inline float softplus_log2(float v) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
    const float w = 1.0f + e;
    const float c = (w - 1.0f) - e;
    const float l = fmaf(c, -kLog2e, __builtin_amdgcn_logf(w));
    return fmaf(fmaxf(v, 0.0f), kLog2e, l);
}

// SiLU(v) = v / (1 + exp(-v)); exp(-v) = inf for very negative v gives -0, the limit.
__device__ inline float silu_f32(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// sigmoid(v) = 1 / (1 + exp(-v)), the derivative of softplus; 0 and 1 in the limits.
__device__ inline float sigmoid_f32(float v) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// d SiLU / dv = sigmoid(v) (1 + v (1 - sigmoid(v))).
__device__ inline float silu_grad_f32(float v) {
    const float sg = sigmoid_f32(v);
    return sg * fmaf(v, 1.0f - sg, 1.0f);
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Piece count for a launch of `groups` x n equal workgroups of which `slots` run at
// once: such a launch takes ceil(groups*n/slots) rounds of L/n steps, so the cost is
// proportional to ceil(groups*n/slots)/n.  Returns the cheapest n in [want, 2*want]
// (at most `cap`, at least `want`), the smallest on ties; want <= 1 is returned as is.
inline int64_t round_friendly_pieces(int64_t groups, int64_t want, int64_t cap, int64_t slots) {
    if (want <= 1 || groups <= 0 || slots <= 0) return want;
    int64_t best = want, best_rounds = cdiv(groups * want, slots);
    const int64_t hi = (2 * want < cap) ? 2 * want : cap;
    for (int64_t n = want + 1; n <= hi; ++n) {
        const int64_t rounds = cdiv(groups * n, slots);
        if (rounds * best < best_rounds * n) {   // rounds/n < best_rounds/best
            best = n;
            best_rounds = rounds;
        }
    }
    return best;
}

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

inline bool misaligned(const void* q, size_t a) { return q && (reinterpret_cast<uintptr_t>(q) % a) != 0; }

// Checks shared by every entry point that takes an ssm_dims.
inline int validate_dims(const ssm_dims* d) {
    if (!d) return SSM_ERR_NULL;
    if (d->batch < 1 || d->seqlen < 1 || d->dim < 1 || d->dstate < 1) return SSM_ERR_EMPTY;
    if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (d->dstate > SSM_MAX_DSTATE) return SSM_ERR_DIMS;
    if (d->nheads < 0 || (d->nheads > 0 && d->dim % d->nheads != 0)) return SSM_ERR_DIMS;
    if (d->nchunks < 0 || d->nchunks > SSM_MAX_CHUNKS) return SSM_ERR_DIMS;
    const int s = d->states_per_lane;
    if (!(s == 0 || s == 1 || s == 2 || s == 4 || s == 8 || s == 16)) return SSM_ERR_DIMS;
    if (d->reserved != 0) return SSM_ERR_DIMS;
    // every element index must fit comfortably in int64 and the grid in int32
    const int64_t lim = int64_t(1) << 40;
    if (d->batch > lim / d->dim || d->batch * d->dim > lim / d->seqlen) return SSM_ERR_DIMS;
    if (d->batch * d->dstate > lim / d->seqlen) return SSM_ERR_DIMS;
    if (d->batch > 65535 * 16) return SSM_ERR_DIMS;
    return SSM_OK;
}

}  // namespace

// Piece end states on the matrix cores (scalar decay, bf16 rows that allow 16-byte
// loads, nstate in {32, 64, 128}); defined in scan_fwd.hip, used by the forward's and
// the backward's piece carries.
//   forward (reverse = 0), pieces piece_base..:  H[d,n] = state after the piece from a
//     zero start, S[d] = the piece's sum of dt2 (step sizes in log2 units);
//   reverse (reverse = 1): H[d,n] = the gradient reaching the piece's first state from
//     the piece alone, sum_t 2^(a_h * sum_{s<=t} dt2_s) * ds_t * C[n,t] with
//     ds = dy * SiLU(z) (dy without z), and S[d] as above.
// H and S in the carry layouts [groups][nchunks][nstate][64] and [groups][nchunks][64].
namespace ssm_detail {
struct PieceStatesArgs {
    const void* x;        // forward: u; reverse: dy
    const void* delta;
    const void* z;        // reverse: gate input, nullable
    const void* BC;       // forward: B; reverse: C
    const float* A;       // (nheads,)
    const float* bias;    // nullable
    int64_t L, dim, nstate, head_dim, chunk_len;
    int32_t nchunks, nblk_d, batch, piece_base;
    float* H;
    float* S;
};
// Launches one workgroup per (batch row, 64-channel block, piece) for npieces pieces
// from piece_base; returns false (launching nothing) when nstate is not supported.
bool launch_piece_states(const PieceStatesArgs& a, bool reverse, int64_t npieces, hipStream_t s);
}  // namespace ssm_detail

// The full pass in chunked form for a scalar decay per head with a step size per channel
// (scan_chunked.hip): bf16 rows that allow 16-byte loads, 64 or 128 states.  One
// workgroup per (batch row, 64-channel block, piece); every piece starts from Hin
// ([groups][nchunks][nstate][64], the piece carries) when nchunks > 1, else from h0 or
// zero; the last piece writes h_last when given.
namespace ssm_detail {
struct ChunkedArgs {
    const void* u;
    const void* delta;
    const void* z;        // nullable
    const void* B;
    const void* C;
    const float* A;       // (nheads,)
    const float* D;       // nullable
    const float* bias;    // nullable
    void* y;
    const float* h0;      // nullable
    float* h_last;        // nullable
    const float* Hin;     // piece starting states when nchunks > 1
    int64_t L, dim, nstate, head_dim, chunk_len;
    int32_t nchunks, nblk_d, batch;
};
bool chunked_supported(int64_t nstate);
size_t chunked_lds_bytes(int64_t nstate);
// Launches the full pass; returns false (launching nothing) when nstate is not supported.
bool launch_chunked(const ChunkedArgs& a, hipStream_t s);
}  // namespace ssm_detail
