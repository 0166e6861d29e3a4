// scan_fwd.hip -- selective-scan forward kernels for gfx950 (MI355X) and the C ABI
// declared in include/ssm.h.
//
// The operation (see include/ssm.h for the full statement and its sources):
//   dt = softplus(delta + dt_bias);  h = exp(dt*A) * h + dt*B*u;  y = (C.h + D*u) * SiLU(z)
// The pages this follows: yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答"
// (Q1, Q4-Q7, Q9), gongshangzheng.github.io "Mamba" (§2.1, §3.1, "Hardware-aware
// Parallel Scan"), qubittool.com "Mamba 与状态空间模型：机制、演进与工程选型"
// (sections "Mamba 增加了内容相关的选择机制", "一个可运行的标量模型",
// "并行训练不会消除递推关系") and cnblogs.com "Mamba3 技术浅析" (§3.1).
//
// Work decomposition (MI355X-first; the pages' A100 kernel is prior art only):
//   * One workgroup owns 64 channels of one batch row over one piece ("chunk") of
//     the sequence.  Lane l of every wave is channel c0 + l, so the wave-uniform
//     B_t / C_t values reach all lanes as LDS broadcasts and the per-channel state
//     never leaves VGPRs.
//   * The dstate state entries of a channel are split over the G waves of the
//     workgroup, SPL entries per lane; each wave walks the time tile sequentially
//     (one exp + 4 VALU ops per state update) and leaves a partial read-out in
//     LDS that the whole workgroup sums in a fixed order (deterministic).
//   * Per time tile of T steps: coalesced 16-byte loads of u, delta, z (B, D, L
//     rows) and B, C (B, N, L rows) are issued one tile ahead into registers; the
//     workgroup turns them into (dt, dt*u) pairs and fp32 B/C in LDS (softplus is
//     paid once per element, not once per wave); the waves walk; the workgroup
//     applies skip, gate and bf16 rounding and stores y with 16-byte stores.
//   * Parallelism along L (the inter-chunk carry): when the channel blocks alone
//     cannot fill the 1024 SIMDs, each sequence is cut into nchunks pieces.  Pass 1
//     computes each piece's end state from a zero start and its step-size sum;
//     a small carry kernel composes the affine maps h -> exp(A*sum dt)*h + H of the
//     pieces in order (merging interval results, qubittool.com section
//     "并行训练不会消除递推关系"); pass 2 re-walks every piece from its true
//     starting state.  The (batch, L, dim, dstate) state is never written to HBM
//     (yo3nglau.github.io Q7).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include "ssm.h"

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
// softplus(v) = max(v, 0) + log1p(exp(-|v|)).  log1p(e) for e in (0, 1] is taken as
// log(w) * e / (w - 1) with w = 1 + e, which cancels the rounding of w (Goldberg's
// log1p identity); w == 1 means e is below half an ulp of 1 and log1p(e) = e.
__device__ inline float softplus_f32(float v) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
    const float w = 1.0f + e;
    const float wm1 = w - 1.0f;
    const float lw = __builtin_amdgcn_logf(w) * kLn2;
    const float lp = (wm1 == 0.0f) ? e : lw * (e * __builtin_amdgcn_rcpf(wm1));
    return fmaxf(v, 0.0f) + lp;
}

// SiLU(v) = v / (1 + exp(-v)); exp(-v) = inf for very negative v gives -0, the limit.
__device__ inline float silu_f32(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// ------------------------------------------------------------------ kernel parameters
struct Params {
    const void* u;
    const void* delta;
    const void* z;        // nullable
    const void* Bm;
    const void* Cm;
    const float* A;
    const float* Dskip;   // nullable
    const float* bias;    // nullable
    void* y;
    int64_t L, dim, N;
    int64_t head_dim;     // channels per head in scalar-decay mode, 0 in diagonal mode
    int64_t chunk_len;    // multiple of the time tile
    int32_t nchunks;
    int32_t nblk_d;       // channel blocks per batch row
    int32_t batch;
    int32_t np;           // padded state count = waves * SPL
    float* ws_H;          // [blocks][nchunks][np][64] piece end states from zero (pass 1)
    float* ws_S;          // [blocks][nchunks][64]     sum of dt over each piece (pass 1)
    float* ws_Hin;        // [blocks][nchunks][np][64] true starting state of each piece
};

enum Mode { kFull = 0, kAggregate = 1 };

// LDS layout (floats): dx[T][64] float2 | sB[T][np] | sC[T][np] | sY[G][T][64]
inline size_t lds_floats(int T, int G, int np, bool full) {
    return size_t(T) * kLanes * 2 + 2 * size_t(T) * np + (full ? size_t(G) * T * kLanes : 0);
}

// One launch processes, for every (batch, channel block, piece), the piece's time
// tiles in order.  MODE kFull reads out and stores y (starting from ws_Hin when the
// piece is not the first); MODE kAggregate only records the piece's end state from
// zero and its dt sum.
//
// Threads: NT = 64 * max(G, 4).  Waves 0 .. G-1 walk (SPL state entries per lane);
// all waves stage and finish tiles.  With T <= 32 this bounds the vectors each
// thread stages per tile to KMAX (1 for bf16, 2 for f32), checked on the host.
template <typename IO, int SPL, bool SCALAR, int MODE, bool VEC, int NTMAX>
__global__ void __launch_bounds__(NTMAX) scan_fwd_kernel(Params p, int T, int G) {
    constexpr int VW = IOT<IO>::VW;
    constexpr int KMAX = (VW == 4) ? 2 : 1;
    constexpr bool kFullMode = (MODE == kFull);

    extern __shared__ float smem[];
    const int NT = blockDim.x;
    const int tid = threadIdx.x;
    const int w = tid / kLanes;
    const int lane = tid % kLanes;
    const int np = p.np;
    const int TV = T / VW;                         // vectors per row per tile
    const bool walker = w < G;

    float2* sDX = reinterpret_cast<float2*>(smem);
    float* sB = smem + size_t(T) * kLanes * 2;
    float* sC = sB + size_t(T) * np;
    float* sY = sC + size_t(T) * np;

    // blockIdx.x -> (piece, batch, channel block), channel block fastest
    const int64_t bid = blockIdx.x;
    const int cblk = int(bid % p.nblk_d);
    const int b = int((bid / p.nblk_d) % p.batch);
    const int piece = int(bid / (int64_t(p.nblk_d) * p.batch));
    const int64_t blk = int64_t(b) * p.nblk_d + cblk;
    const int64_t c0 = int64_t(cblk) * kLanes;
    const int64_t tbeg = int64_t(piece) * p.chunk_len;
    const int64_t tend = (tbeg + p.chunk_len < p.L) ? tbeg + p.chunk_len : p.L;

    const IO* __restrict__ gu = static_cast<const IO*>(p.u);
    const IO* __restrict__ gdl = static_cast<const IO*>(p.delta);
    const IO* __restrict__ gz = static_cast<const IO*>(p.z);
    const IO* __restrict__ gB = static_cast<const IO*>(p.Bm);
    const IO* __restrict__ gC = static_cast<const IO*>(p.Cm);
    IO* __restrict__ gy = static_cast<IO*>(p.y);

    // ---- per-lane constants: this lane's channel and its SPL decay rates (log2 units)
    const int64_t dch = c0 + lane;
    const bool lane_ok = dch < p.dim;
    float A2[SPL];
    float a2_scalar = 0.0f;
    if constexpr (SCALAR) {
        a2_scalar = lane_ok ? p.A[dch / p.head_dim] * kLog2e : 0.0f;
#pragma unroll
        for (int j = 0; j < SPL; ++j) A2[j] = a2_scalar;
    } else {
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const int64_t n = int64_t(w) * SPL + j;
            A2[j] = (walker && lane_ok && n < p.N) ? p.A[dch * p.N + n] * kLog2e : 0.0f;
        }
    }

    // ---- starting state of this piece
    float h[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) h[j] = 0.0f;
    if (kFullMode && piece > 0 && walker) {
        const float* hin = p.ws_Hin + ((blk * p.nchunks + piece) * np + int64_t(w) * SPL) * kLanes + lane;
#pragma unroll
        for (int j = 0; j < SPL; ++j) h[j] = hin[int64_t(j) * kLanes];
    }
    float dtsum = 0.0f, dtcomp = 0.0f;   // compensated (Kahan) sum of dt over the piece

    // ---- tile vectors this thread stages: v = tid + k*NT
    const int nvx = kLanes * TV;                   // u/delta/z vectors per tile
    const int nvb = np * TV;                       // B/C vectors per tile
    Vec<IO> nu[KMAX], ndl[KMAX], nz[KMAX], cu[KMAX], cz[KMAX], nB[KMAX], nC[KMAX];

    auto issue_loads = [&](int64_t t0) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int v = tid + k * NT;
            if (v < nvx) {
                const int ch = v / TV, tv = v % TV;
                const int64_t d = c0 + ch;
                const bool ok = d < p.dim;
                const int64_t row = (int64_t(b) * p.dim + (ok ? d : 0)) * p.L;
                const int64_t t = t0 + tv * VW;
                nu[k] = load_vec<IO, VEC>(gu + row, t, tend, ok);
                ndl[k] = load_vec<IO, VEC>(gdl + row, t, tend, ok);
                if (kFullMode && gz) nz[k] = load_vec<IO, VEC>(gz + row, t, tend, ok);
            }
            if (v < nvb) {
                const int n = v / TV, tv = v % TV;
                const bool ok = n < p.N;
                const int64_t row = (int64_t(b) * p.N + (ok ? n : 0)) * p.L;
                const int64_t t = t0 + tv * VW;
                nB[k] = load_vec<IO, VEC>(gB + row, t, tend, ok);
                if (kFullMode) nC[k] = load_vec<IO, VEC>(gC + row, t, tend, ok);
            }
        }
    };

    issue_loads(tbeg);
    for (int64_t t0 = tbeg; t0 < tend; t0 += T) {
        const int tlen = int((tend - t0) < T ? (tend - t0) : T);

        // ---- stage: (dt, dt*u) or (exp(dt*a_h), dt*u) per element; fp32 B and C
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int v = tid + k * NT;
            if (v < nvx) {
                const int ch = v / TV, tv = v % TV;
                const int64_t d = c0 + ch;
                const bool ok = d < p.dim;
                const float bs = (ok && p.bias) ? p.bias[d] : 0.0f;
                float a2h = 0.0f;
                if constexpr (SCALAR) a2h = ok ? p.A[d / p.head_dim] * kLog2e : 0.0f;
#pragma unroll
                for (int e = 0; e < VW; ++e) {
                    const float uu = IOT<IO>::to_f32(nu[k].e[e]);
                    const float dt = ok ? softplus_f32(IOT<IO>::to_f32(ndl[k].e[e]) + bs) : 0.0f;
                    float first = dt;
                    if constexpr (SCALAR && kFullMode) first = __builtin_amdgcn_exp2f(dt * a2h);
                    sDX[(tv * VW + e) * kLanes + ch] = make_float2(first, dt * uu);
                }
                if constexpr (kFullMode) {
                    cu[k] = nu[k];
                    if (gz) cz[k] = nz[k];
                }
            }
            if (v < nvb) {
                const int n = v / TV, tv = v % TV;
#pragma unroll
                for (int e = 0; e < VW; ++e) {
                    sB[(tv * VW + e) * np + n] = IOT<IO>::to_f32(nB[k].e[e]);
                    if constexpr (kFullMode) sC[(tv * VW + e) * np + n] = IOT<IO>::to_f32(nC[k].e[e]);
                }
            }
        }
        // prefetch the next tile while this one is walked
        if (t0 + T < tend) issue_loads(t0 + T);
        __syncthreads();

        // ---- walk: SPL state entries per lane, sequential in t
        if (walker) {
            const float* sBw = sB + w * SPL;
            const float* sCw = sC + w * SPL;
            for (int t = 0; t < tlen; ++t) {
                const float2 dx = sDX[t * kLanes + lane];
                float a_shared = 0.0f;
                if constexpr (SCALAR) {
                    if constexpr (kFullMode) a_shared = dx.x;
                    else a_shared = __builtin_amdgcn_exp2f(dx.x * a2_scalar);
                }
                if constexpr (!kFullMode) {
                    const float yk = dx.x - dtcomp;
                    const float tk = dtsum + yk;
                    dtcomp = (tk - dtsum) - yk;
                    dtsum = tk;
                }
                float yp = 0.0f;
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const float bb = sBw[t * np + j];
                    const float a = SCALAR ? a_shared : __builtin_amdgcn_exp2f(dx.x * A2[j]);
                    h[j] = fmaf(a, h[j], dx.y * bb);
                    if constexpr (kFullMode) yp = fmaf(sCw[t * np + j], h[j], yp);
                }
                if constexpr (kFullMode) sY[(size_t(w) * T + t) * kLanes + lane] = yp;
            }
        }
        __syncthreads();

        // ---- epilogue: sum the G partial read-outs in wave order, skip, gate, store
        if constexpr (kFullMode) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                const int v = tid + k * NT;
                if (v < nvx) {
                    const int ch = v / TV, tv = v % TV;
                    const int64_t d = c0 + ch;
                    const bool ok = d < p.dim;
                    const float dsk = (ok && p.Dskip) ? p.Dskip[d] : 0.0f;
                    Vec<IO> out;
#pragma unroll
                    for (int e = 0; e < VW; ++e) {
                        const int tl = tv * VW + e;
                        float acc = 0.0f;
                        for (int ww = 0; ww < G; ++ww) acc += sY[(size_t(ww) * T + tl) * kLanes + ch];
                        float o = fmaf(dsk, IOT<IO>::to_f32(cu[k].e[e]), acc);
                        if (gz) o *= silu_f32(IOT<IO>::to_f32(cz[k].e[e]));
                        out.e[e] = IOT<IO>::from_f32(o);
                    }
                    const int64_t row = (int64_t(b) * p.dim + (ok ? d : 0)) * p.L;
                    store_vec<IO, VEC>(gy + row, t0 + tv * VW, tend, ok, out);
                }
            }
        }
    }

    if constexpr (!kFullMode) {
        if (walker) {
            float* hout = p.ws_H + ((blk * p.nchunks + piece) * np + int64_t(w) * SPL) * kLanes + lane;
#pragma unroll
            for (int j = 0; j < SPL; ++j) hout[int64_t(j) * kLanes] = h[j];
            if (w == 0) p.ws_S[(blk * p.nchunks + piece) * kLanes + lane] = dtsum;
        }
    }
}

// Compose the pieces' affine maps in sequence order: one thread per (block, state, lane).
//   Hin[0] = 0;  Hin[c+1] = exp(A * S[c]) * Hin[c] + H[c]
__global__ void __launch_bounds__(256) scan_carry_kernel(Params p, int64_t total) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int lane = int(i % kLanes);
    const int64_t n = (i / kLanes) % p.np;
    const int64_t blk = i / (int64_t(kLanes) * p.np);
    const int64_t cblk = blk % p.nblk_d;
    const int64_t d = cblk * kLanes + lane;
    float a2 = 0.0f;
    if (d < p.dim && n < p.N) a2 = (p.head_dim ? p.A[d / p.head_dim] : p.A[d * p.N + n]) * kLog2e;
    float hcur = 0.0f;
    for (int c = 0; c < p.nchunks; ++c) {
        const int64_t hidx = ((blk * p.nchunks + c) * p.np + n) * kLanes + lane;
        p.ws_Hin[hidx] = hcur;
        if (c + 1 < p.nchunks) {
            const float s = p.ws_S[(blk * p.nchunks + c) * kLanes + lane];
            hcur = fmaf(__builtin_amdgcn_exp2f(a2 * s), hcur, p.ws_H[hidx]);
        }
    }
}

// ------------------------------------------------------------------ host side: planning

struct Plan {
    int nchunks;
    int spl;
    int G;
    int T;
    int64_t chunk_len;
    int64_t nblk_d;
    int64_t blocks;     // workgroups per pass
    size_t ws_bytes;
    size_t lds_bytes;
    bool scalar;
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int validate_dims(const ssm_dims* d) {
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

int make_plan(const ssm_dims* d, Plan* pl) {
    int st = validate_dims(d);
    if (st != SSM_OK) return st;
    const int64_t N = d->dstate;
    pl->scalar = d->nheads > 0;
    int spl = d->states_per_lane;
    if (spl == 0) {
        // aim for 4 waves per workgroup (scalar decay: 8), at most 16 states per lane
        const int64_t target_waves = pl->scalar ? 8 : 4;
        spl = 1;
        while (spl < 16 && cdiv(N, spl) > target_waves) spl *= 2;
    }
    if (cdiv(N, spl) > 16) return SSM_ERR_DIMS;       // more than 1024 threads
    pl->spl = spl;
    pl->G = int(cdiv(N, spl));
    // time tile: 32 steps; 16 when the partial read-outs of 16 waves or a wide
    // B/C tile would not fit the 160 KB of LDS
    pl->T = (pl->G > 8 || pl->G * spl > 128) ? 16 : 32;
    pl->nblk_d = cdiv(d->dim, kLanes);
    const int64_t groups = d->batch * pl->nblk_d;
    const int64_t tiles = cdiv(d->seqlen, pl->T);
    int64_t nch = d->nchunks;
    if (nch == 0) {
        // one wave per SIMD (256 CUs x 4 SIMDs) is the floor below which the sequence is
        // cut into pieces; pieces cost a second pass over all but the first, so cut
        // only when the machine would otherwise be at most half busy.
        const int64_t waves = groups * pl->G;
        nch = 1;
        if (waves * 2 <= 1024) {
            nch = cdiv(2048, waves);
            const int64_t max_pieces = tiles / 8 > 1 ? tiles / 8 : 1;   // keep >= 8 tiles per piece
            if (nch > max_pieces) nch = max_pieces;
            if (nch > SSM_MAX_CHUNKS) nch = SSM_MAX_CHUNKS;
        }
    }
    if (nch > tiles) nch = tiles;
    if (nch < 1) nch = 1;
    pl->chunk_len = cdiv(tiles, nch) * pl->T;
    pl->nchunks = int(cdiv(d->seqlen, pl->chunk_len));   // drop empty trailing pieces
    pl->blocks = groups * pl->nchunks;
    if (pl->blocks > 0x7fffffffLL) return SSM_ERR_DIMS;
    const int np = pl->G * pl->spl;
    pl->ws_bytes = 0;
    if (pl->nchunks > 1) {
        const size_t per = size_t(groups) * pl->nchunks * kLanes * sizeof(float);
        size_t bytes = per * np * 2 + per;   // H, Hin, S
        pl->ws_bytes = (bytes + 255) & ~size_t(255);
    }
    pl->lds_bytes = lds_floats(pl->T, pl->G, np, true) * sizeof(float);
    return SSM_OK;
}

// ------------------------------------------------------------------ host side: launching
template <typename IO, int SPL, bool SCALAR, bool VEC, int NTMAX>
hipError_t launch_all(const Params& p, const Plan& pl, hipStream_t stream) {
    const dim3 block(unsigned((pl.G > 4 ? pl.G : 4) * kLanes));
    if (block.x > unsigned(NTMAX)) return hipErrorInvalidConfiguration;
    const size_t lds_full = lds_floats(pl.T, pl.G, p.np, true) * sizeof(float);
    const size_t lds_agg = lds_floats(pl.T, pl.G, p.np, false) * sizeof(float);
    if (pl.nchunks > 1) {
        const int64_t groups = int64_t(p.batch) * p.nblk_d;
        // pass 1 on every piece but the last
        const dim3 grid1(unsigned(groups * (pl.nchunks - 1)));
        hipLaunchKernelGGL((scan_fwd_kernel<IO, SPL, SCALAR, kAggregate, VEC, NTMAX>), grid1, block, lds_agg, stream, p, pl.T, pl.G);
        const int64_t total = groups * p.np * kLanes;
        hipLaunchKernelGGL(scan_carry_kernel, dim3(unsigned(cdiv(total, 256))), dim3(256), 0, stream, p, total);
    }
    hipLaunchKernelGGL((scan_fwd_kernel<IO, SPL, SCALAR, kFull, VEC, NTMAX>), dim3(unsigned(pl.blocks)), block, lds_full,
                       stream, p, pl.T, pl.G);
    return hipGetLastError();
}

// Workgroups of up to 4 waves get the 256-thread launch bound (up to 512 VGPRs per
// lane); larger ones the 1024-thread bound (128 VGPRs).  Row layouts that cannot use
// 16-byte vectors only get the latter.
template <typename IO, bool SCALAR, bool VEC, int NTMAX>
hipError_t dispatch_spl(const Params& p, const Plan& pl, hipStream_t s) {
    switch (pl.spl) {
        case 1: return launch_all<IO, 1, SCALAR, VEC, NTMAX>(p, pl, s);
        case 2: return launch_all<IO, 2, SCALAR, VEC, NTMAX>(p, pl, s);
        case 4: return launch_all<IO, 4, SCALAR, VEC, NTMAX>(p, pl, s);
        case 8: return launch_all<IO, 8, SCALAR, VEC, NTMAX>(p, pl, s);
        default: return launch_all<IO, 16, SCALAR, VEC, NTMAX>(p, pl, s);
    }
}

template <typename IO, bool SCALAR>
hipError_t dispatch_nt(const Params& p, const Plan& pl, bool vec, hipStream_t s) {
    if (!vec) return dispatch_spl<IO, SCALAR, false, 1024>(p, pl, s);
    if (pl.G <= 4) return dispatch_spl<IO, SCALAR, true, 256>(p, pl, s);
    return dispatch_spl<IO, SCALAR, true, 1024>(p, pl, s);
}

template <typename IO>
hipError_t dispatch(const Params& p, const Plan& pl, bool vec, hipStream_t s) {
    return pl.scalar ? dispatch_nt<IO, true>(p, pl, vec, s) : dispatch_nt<IO, false>(p, pl, vec, s);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

// ------------------------------------------------------------------ C ABI
extern "C" {

const char* ssm_status_string(int status) {
    switch (status) {
        case SSM_OK: return "ok";
        case SSM_ERR_NULL: return "a required pointer is NULL";
        case SSM_ERR_EMPTY: return "batch, seqlen, dim and dstate must all be >= 1";
        case SSM_ERR_DIMS: return "sizes are inconsistent or out of range";
        case SSM_ERR_DTYPE: return "unknown io_dtype";
        case SSM_ERR_ALIGN: return "an array is not aligned to its element size";
        case SSM_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case SSM_ERR_HIP: return "the HIP runtime reported an error";
        case SSM_ERR_ALIAS: return "y overlaps an input array";
        default: return "unknown status";
    }
}

int ssm_selective_scan_plan(const ssm_dims* dims, ssm_plan* plan) {
    if (!plan) return SSM_ERR_NULL;
    Plan pl;
    const int st = make_plan(dims, &pl);
    if (st != SSM_OK) return st;
    plan->nchunks = pl.nchunks;
    plan->states_per_lane = pl.spl;
    plan->waves_per_group = pl.G;
    plan->time_tile = pl.T;
    plan->chunk_len = pl.chunk_len;
    plan->workgroups = pl.blocks;
    plan->workspace_bytes = pl.ws_bytes;
    plan->lds_bytes = pl.lds_bytes;
    return SSM_OK;
}

size_t ssm_selective_scan_workspace_bytes(const ssm_dims* dims) {
    Plan pl;
    if (make_plan(dims, &pl) != SSM_OK) return 0;
    return pl.ws_bytes;
}

int ssm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* dt_bias, void* y, const ssm_dims* dims,
                           void* stream) {
    if (!dims) return SSM_ERR_NULL;
    Plan pl;
    int st = make_plan(dims, &pl);
    if (st != SSM_OK) return st;
    if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;

    const size_t esz = dims->io_dtype == SSM_BF16 ? 2 : 4;
    auto misaligned = [](const void* q, size_t a) { return q && (reinterpret_cast<uintptr_t>(q) % a) != 0; };
    if (misaligned(u, esz) || misaligned(delta, esz) || misaligned(z, esz) || misaligned(B, esz) ||
        misaligned(C, esz) || misaligned(y, esz) || misaligned(A, 4) || misaligned(D, 4) || misaligned(dt_bias, 4))
        return SSM_ERR_ALIGN;

    const size_t nel = size_t(dims->batch) * dims->dim * dims->seqlen * esz;
    const size_t nbc = size_t(dims->batch) * dims->dstate * dims->seqlen * esz;
    const size_t na = (dims->nheads > 0 ? size_t(dims->nheads) : size_t(dims->dim) * dims->dstate) * 4;
    const size_t nd = size_t(dims->dim) * 4;
    if (overlaps(y, nel, u, nel) || overlaps(y, nel, delta, nel) || overlaps(y, nel, z, nel) ||
        overlaps(y, nel, B, nbc) || overlaps(y, nel, C, nbc) || overlaps(y, nel, A, na) ||
        overlaps(y, nel, D, nd) || overlaps(y, nel, dt_bias, nd))
        return SSM_ERR_ALIAS;

    if (pl.ws_bytes > 0) {
        if (!dims->workspace || dims->workspace_bytes < pl.ws_bytes ||
            (reinterpret_cast<uintptr_t>(dims->workspace) % 256) != 0)
            return SSM_ERR_WORKSPACE;
        if (overlaps(dims->workspace, pl.ws_bytes, y, nel)) return SSM_ERR_ALIAS;
    }

    // vector (16-byte) loads need 16-byte aligned rows: aligned base pointers and a
    // row length that is a whole number of vectors
    const size_t vw = 16 / esz;
    auto a16 = [](const void* q) { return !q || (reinterpret_cast<uintptr_t>(q) % 16) == 0; };
    const bool vec = (dims->seqlen % int64_t(vw)) == 0 && a16(u) && a16(delta) && a16(z) && a16(B) && a16(C) && a16(y);

    Params p;
    p.u = u;
    p.delta = delta;
    p.z = z;
    p.Bm = B;
    p.Cm = C;
    p.A = A;
    p.Dskip = D;
    p.bias = dt_bias;
    p.y = y;
    p.L = dims->seqlen;
    p.dim = dims->dim;
    p.N = dims->dstate;
    p.head_dim = dims->nheads > 0 ? dims->dim / dims->nheads : 0;
    p.chunk_len = pl.chunk_len;
    p.nchunks = pl.nchunks;
    p.nblk_d = int32_t(pl.nblk_d);
    p.batch = int32_t(dims->batch);
    p.np = pl.G * pl.spl;
    p.ws_H = p.ws_S = p.ws_Hin = nullptr;
    if (pl.ws_bytes > 0) {
        const size_t per = size_t(dims->batch) * pl.nblk_d * pl.nchunks * kLanes;
        float* base = static_cast<float*>(dims->workspace);
        p.ws_H = base;
        p.ws_Hin = base + per * p.np;
        p.ws_S = base + 2 * per * p.np;
    }

    // per-thread staging capacity of the kernel: KMAX vectors (1 for bf16, 2 for f32)
    const int64_t nthreads = int64_t(pl.G > 4 ? pl.G : 4) * kLanes;
    const int64_t kmax = esz == 2 ? 1 : 2;
    const int64_t tv = pl.T / int64_t(vw);
    if (int64_t(kLanes) * tv > kmax * nthreads || int64_t(p.np) * tv > kmax * nthreads) return SSM_ERR_DIMS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = dims->io_dtype == SSM_BF16 ? dispatch<uint16_t>(p, pl, vec, s) : dispatch<float>(p, pl, vec, s);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
