// scan_bwd.hip -- backward pass of the selective scan for gfx950 (MI355X) and the C
// ABI entry points ssm_selective_scan_bwd* declared in include/ssm.h.
//
// Gradients of  sum dy*y + sum dh_last*h_L  for the forward of scan_fwd.hip.  With
// dt2 = softplus(delta + dt_bias) / ln 2 (log2 units, as in the forward), x = dt2*u,
// a = exp2(dt2*A), B' = B*ln 2 and the per-step total gradient g[n] at h_t[n],
// walking t backwards with the carried e[n] = a_{t+1}[n] g_{t+1}[n]:
//   ds = dy * SiLU(z)                   dz = dy * SiLU'(z) * (C.h_t + D*u)
//   g[n] = ds*C[n] + e[n]               e[n] <- a[n] * g[n]
//   dC_t[n] += ds * h_t[n]              dB_t[n] += ln2 * g[n] * x        (summed over channels)
//   dA[n]   += ln2 * dt2 * g[n] * a[n] h_{t-1}[n]                         (summed over b, t)
//   ddt = sum_n A[n] g[n] a[n] h_{t-1}[n] + u * sum_n g[n] B'[n] / ln2
//   du  = D*ds + dt2 * sum_n g[n] B'[n]          ddelta = ddt * sigmoid(delta + dt_bias)
// Training needs these; as the pages say of Mamba's kernels, the states the backward
// needs are recomputed from the inputs instead of being kept from the forward
// (yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答" Q7; qubittool.com
// "Mamba 与状态空间模型：机制、演进与工程选型", section "并行训练不会消除递推关系").
//
// Work decomposition (one workgroup per batch row, 64 channels and piece of the
// sequence; lane = channel, the dstate entries split over the G waves, SPL per lane,
// as in the forward):
//   1. checkpoint pass: walk the piece forward and write the state at the start of
//      every 16-step tile (4*dstate bytes per 16 steps of a channel);
//   2. gradient pass: walk the tiles backwards.  Per tile the lanes reload the tile's
//      start state, recompute its 16 states forward (kept in VGPRs; with more than 4
//      entries per lane in sub-blocks, re-walked from saved sub-block starts), then
//      step backwards through them.  The per-step sums over state entries (the
//      read-out, sum A g a h, sum g B') are left per wave in LDS and summed over the
//      waves in a fixed order;
//      the sums over channels (dB, dC) are reduced across the 64 lanes through a
//      per-wave LDS transpose, 16 values at a time, in a fixed order;
//   3. reduce kernels add the per-workgroup partials of dB, dC, dA, dD and ddt_bias
//      in a fixed order.
// With 9..16 state entries per channel the checkpoint and gradient passes run with
// separate roles instead: four walking waves (4 entries per lane) beside four helper
// waves that stage and finish, over double-buffered tiles (scan_bwd_ckpt_ws_kernel,
// scan_bwd_grad_ws_kernel).
// Long sequences are cut into pieces exactly as in the forward: the pieces' start
// states come from a forward aggregate pass and carry, their incoming gradients from
// a reverse aggregate pass (e from zero at the piece end, and the dt2 sum) and a
// reverse carry: e_in(c-1) = exp2(A * S_c) * e_in(c) + G_c.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "ssm.h"

#include "scan_common.h"

namespace {

// time tile = recompute interval: 16 steps, 8 when a workgroup carries more than 64
// state entries per channel (the per-wave partial slabs must fit the LDS)
inline constexpr int bwd_tile(int np) { return np <= 64 ? 16 : 8; }
constexpr int kRound = 8;    // values per cross-lane reduction round

struct BwdParams {
    const void* u;
    const void* delta;
    const void* z;         // nullable
    const void* Bm;
    const void* Cm;
    const float* A;
    const float* Dskip;    // nullable
    const float* bias;     // nullable
    const float* h0;       // nullable
    const void* dy;
    const float* dh_last;  // nullable
    void* du;
    void* ddelta;
    void* dz;              // nullable
    float* dh0;            // nullable
    int64_t L, dim, N, head_dim, chunk_len, ntiles_seq;
    int32_t nchunks, nblk_d, batch, np;
    int32_t piece_base;    // first piece index of the launch
    int32_t mfma_agg;      // piece aggregates on the matrix cores (scalar decay, bf16
                           // rows that allow 16-byte loads, 32/64/128 states)
    float* ck;             // [groups][ntiles_seq][np][64]   tile start states
    float* pBC;            // [nblk_d][batch][2][N][L]       per-block dB (unscaled), dC
    float* pA;             // [nchunks][batch][dim][np]      per-piece dA / ln 2
    float* pD;             // [nchunks][batch][dim]
    float* pbias;          // [nchunks][batch][dim]
    float* fH;             // [groups][nchunks][np][64]      piece end states from zero
    float* fS;             // [groups][nchunks][64]          sum of dt2 over each piece
    float* fHin;           // [groups][nchunks][np][64]      true start state of each piece
    float* rG;             // [groups][nchunks][np][64]      e at piece start from zero at its end
    float* rS;             // [groups][nchunks][64]
    float* rEin;           // [groups][nchunks][np][64]      true incoming e at each piece end
};

enum BwdMode { kCkpt = 0, kFwdAgg = 1, kRevAgg = 2, kGrad = 3 };

template <int SPL, int G> struct BShape {
    static constexpr int T = bwd_tile(G * SPL);
    static constexpr int NP = G * SPL;
    static constexpr int NT = G * kLanes;
    static constexpr int TS = (64 / SPL < T) ? 64 / SPL : T;   // states a lane keeps per sub-block
    static constexpr int NSB = T / TS;
    static constexpr int JR = SPL < 4 ? SPL : 4;              // entries per reduction round
    static constexpr int RS = 4 / JR;                         // steps per reduction round
    static constexpr int NJR = SPL / JR;                      // rounds per step (SPL > 4)
};

// LDS floats of one workgroup:
//   sW  [T][64] float4     (dt2, dt2*u, ds, scalar decay)         all modes
//   sF  [T][64] float4     (u, sigmoid(r), dy*SiLU'(z), D*u)      gradient pass
//   sBC [T][NP] float2     (B*ln2, C)                             all modes
//   sP  [3][G][T][64]      per-wave partial read-out, sum A g a h, sum g B' of each
//                          step and channel, summed over the waves in a fixed order
//   sdBC [2][NP][T]        per-block dB, dC of the tile            gradient pass
//   sRed [G][8][64]        per-wave transpose for lane sums        gradient pass
inline size_t bwd_lds_floats(int G, int SPL, int mode) {
    const size_t NP = size_t(G) * SPL, T = bwd_tile(G * SPL);
    size_t f = T * kLanes * 4 + T * NP * 2;
    if (mode == kGrad) f += T * kLanes * 4 + 3 * size_t(G) * T * kLanes + 2 * NP * T + size_t(G) * kRound * kLanes;
    return f;
}

// EPT consecutive elements of one row: one load or store of EPT*sizeof(IO) bytes when
// the row is aligned for it (vec), else element by element.  Elements at or beyond
// tend (or of a row that does not exist, ok == false) read as 0 and are not written.
template <int BYTES> struct RawOf;
template <> struct RawOf<2> { using T = uint16_t; };
template <> struct RawOf<4> { using T = uint32_t; };
template <> struct RawOf<8> { using T = uint2; };
template <> struct RawOf<16> { using T = uint4; };
struct Raw32 {
    uint4 lo, hi;
};
template <> struct RawOf<32> { using T = Raw32; };

// Output elements of one thread's segment.
template <typename IO, int EPT> struct Seg {
    IO e[EPT];
};

// Prefetched input elements of one thread's segment, kept as loaded (one raw word
// when VEC) until the consumer unpacks them: unpacking right after the load would
// make the compiler wait for it there.
template <typename IO, int EPT, bool VEC> struct InSeg {
    using R = typename RawOf<EPT * int(sizeof(IO))>::T;
    R raw;
    IO e[VEC ? 1 : EPT];
    __device__ inline float get(int k) const {
        if constexpr (VEC) {
            IO t[EPT];
            __builtin_memcpy(t, &raw, sizeof(R));
            return IOT<IO>::to_f32(t[k]);
        } else {
            return IOT<IO>::to_f32(e[k]);
        }
    }
};

// Prefetch loads never branch and never inspect what they load: an element outside
// the row's valid range is read from the row's start (always valid memory) and the
// consumer masks it (stage tests the same range).  A load inside a branch, or a select
// on its value right after it, makes the compiler wait for the load on the spot,
// which would serialise the prefetch.
template <typename IO, int EPT, bool VEC>
__device__ inline InSeg<IO, EPT, VEC> load_seg(const IO* __restrict__ row, int64_t t, int64_t tend, bool ok) {
    using R = typename RawOf<EPT * int(sizeof(IO))>::T;
    InSeg<IO, EPT, VEC> v;
    if constexpr (VEC) {
        v.raw = *reinterpret_cast<const R*>(row + ((ok && t < tend) ? t : 0));
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) v.e[e] = row[(ok && t + e < tend) ? t + e : 0];
    }
    return v;
}

template <typename IO, int EPT, bool VEC>
__device__ inline void store_seg(IO* __restrict__ row, int64_t t, int64_t tend, bool ok, const Seg<IO, EPT>& v) {
    using R = typename RawOf<EPT * int(sizeof(IO))>::T;
    if constexpr (VEC) {
        if (ok && t < tend) {
            R raw;
            __builtin_memcpy(&raw, &v, sizeof(R));
            *reinterpret_cast<R*>(row + t) = raw;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            if (ok && t + e < tend) row[t + e] = v.e[e];
    }
}

// A lane permutation inside each 16-lane row (quad swaps, half-row mirror, rotation),
// so no lane reads outside its row; written as an update with zero fill so that the
// compiler folds it into the add that consumes it (v_add_f32_dpp).
template <int CTRL>
__device__ inline float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <typename IO, int SPL, int G, bool SCALAR, int MODE, bool VEC>
__global__ void __launch_bounds__(G * kLanes) scan_bwd_kernel(BwdParams p) {
    using S = BShape<SPL, G>;
    constexpr int T = S::T, NP = S::NP, NT = S::NT, TS = S::TS, NSB = S::NSB;
    constexpr int JR = S::JR, RS = S::RS, NJR = S::NJR;
    constexpr int EPT = T / G;                    // elements per thread and tile: wave w takes
                                                  // steps w*EPT .. w*EPT+EPT-1 of all 64 channels
    constexpr int NBCV = 2 * NP * T;              // B and C values per tile
    constexpr int KB = (NBCV + NT - 1) / NT;      // of them per thread
    constexpr bool kG = MODE == kGrad;
    constexpr bool kRev = MODE == kRevAgg || MODE == kGrad;
    constexpr bool kUseB = MODE != kRevAgg;
    constexpr bool kUseC = MODE == kRevAgg || MODE == kGrad;
    constexpr bool kUseU = MODE != kRevAgg;
    static_assert(T % G == 0 && EPT * G == T, "a tile's steps must split evenly over the waves");
    static_assert(TS % RS == 0 && RS * 2 * JR == kRound, "reduction rounds must tile the sub-block");

    extern __shared__ float smem[];
    float4* sW = reinterpret_cast<float4*>(smem);
    float* const after_w = smem + T * kLanes * 4;
    float4* sF = reinterpret_cast<float4*>(after_w);
    float* const sBC = after_w + (kG ? T * kLanes * 4 : 0);
    float* const sP = sBC + T * NP * 2;                 // [3][G][T][64]
    constexpr int kSlab = G * T * kLanes;
    float* const sdBC = sP + 3 * kSlab;
    float* const sRed = sdBC + 2 * NP * T;

    const int tid = threadIdx.x;
    const int w = tid / kLanes;
    const int lane = tid % kLanes;
    const int64_t bid = blockIdx.x;
    const int cblk = int(bid % p.nblk_d);
    const int b = int((bid / p.nblk_d) % p.batch);
    const int piece = int(bid / (int64_t(p.nblk_d) * p.batch)) + p.piece_base;
    const int64_t blk = int64_t(b) * p.nblk_d + cblk;
    const int64_t c0 = int64_t(cblk) * kLanes;
    const int64_t tbeg = int64_t(piece) * p.chunk_len;
    const int64_t tend = (tbeg + p.chunk_len < p.L) ? tbeg + p.chunk_len : p.L;
    const int ntiles = int((tend - tbeg + T - 1) / T);
    const int64_t tile0 = tbeg / T;
    const bool has_z = kRev && p.z != nullptr;

    const IO* __restrict__ gu = static_cast<const IO*>(p.u);
    const IO* __restrict__ gdl = static_cast<const IO*>(p.delta);
    const IO* __restrict__ gz = static_cast<const IO*>(p.z);
    const IO* __restrict__ gdy = static_cast<const IO*>(p.dy);
    const IO* __restrict__ gB = static_cast<const IO*>(p.Bm);
    const IO* __restrict__ gC = static_cast<const IO*>(p.Cm);

    // ---- walk constants: this lane's channel and its SPL decay rates
    const int64_t dch = c0 + lane;
    const bool lane_ok = dch < p.dim;
    float Ar[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const int64_t n = int64_t(w) * SPL + j;
        if constexpr (SCALAR) Ar[j] = lane_ok ? p.A[dch / p.head_dim] : 0.0f;
        else Ar[j] = (lane_ok && n < p.N) ? p.A[dch * p.N + n] : 0.0f;
    }
    const int64_t state_base = ((blk * p.nchunks + piece) * NP + int64_t(w) * SPL) * kLanes + lane;

    // ---- element constants: thread tid takes steps e_seg*EPT .. +EPT-1 of channel e_ch.
    //      Lane = channel keeps every LDS access of staging and finishing free of bank
    //      conflicts; each global access then moves EPT elements of 64 different rows.
    const int e_ch = lane;
    const int e_seg = w;
    const int64_t e_d = c0 + e_ch;
    const bool e_ok = e_d < p.dim;
    const float e_bias = (e_ok && p.bias) ? p.bias[e_d] : 0.0f;
    const float e_skip = (e_ok && p.Dskip) ? p.Dskip[e_d] : 0.0f;
    const float e_ah = (SCALAR && e_ok) ? p.A[e_d / p.head_dim] : 0.0f;
    const int64_t e_row = (int64_t(b) * p.dim + (e_ok ? e_d : 0)) * p.L;

    // ---- B/C constants: value v = tid + k*NT -> (B or C, entry n, step t of the tile)
    const IO* bc_ptr[KB];
    int bc_slot[KB], bc_t[KB];
    bool bc_on[KB], bc_ok[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int v = tid + k * NT;
        bc_on[k] = v < NBCV;
        const int isC = v / (NP * T);
        const int n = (v / T) % NP;
        bc_t[k] = v % T;
        bc_ok[k] = bc_on[k] && n < p.N && (isC ? kUseC : kUseB);
        bc_ptr[k] = (isC ? gC : gB) + (int64_t(b) * p.N + (bc_ok[k] ? n : 0)) * p.L + bc_t[k];
        bc_slot[k] = (bc_t[k] * NP + n) * 2 + isC;
    }

    // ---- prefetch registers (one tile ahead): checkpoint entries first, so that the
    //      wait for a tile's staging data also covers them
    InSeg<IO, EPT, VEC> nu, ndl, nz, ndy;
    IO nbc[KB];
    float ckn[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) ckn[j] = 0.0f;
    auto issue_loads = [&](int kt) {
        const int64_t t0 = tbeg + int64_t(kt) * T;
        if constexpr (kG) {
            const float* ck = p.ck + ((blk * p.ntiles_seq + tile0 + kt) * NP + int64_t(w) * SPL) * kLanes + lane;
#pragma unroll
            for (int j = 0; j < SPL; ++j) ckn[j] = ck[int64_t(j) * kLanes];
        }
        const int64_t t = t0 + e_seg * EPT;
        if constexpr (kUseU) nu = load_seg<IO, EPT, VEC>(gu + e_row, t, tend, e_ok);
        ndl = load_seg<IO, EPT, VEC>(gdl + e_row, t, tend, e_ok);
        if constexpr (kRev) {
            ndy = load_seg<IO, EPT, VEC>(gdy + e_row, t, tend, e_ok);
            nz = load_seg<IO, EPT, VEC>((has_z ? gz : gdy) + e_row, t, tend, e_ok && has_z);
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) nbc[k] = *((bc_ok[k] && t0 + bc_t[k] < tend) ? bc_ptr[k] + t0 : gB);
    };

    // ---- registers -> LDS for the tile starting at t0.  Steps beyond the piece's end
    //      are identity steps (dt2 = 0, x = 0, ds = 0, decay 1).
    auto stage = [&](int64_t t0) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int tl = e_seg * EPT + e;
            const bool in = e_ok && t0 + tl < tend;   // else the prefetched value is not this element's
            const float uu = (kUseU && in) ? nu.get(e) : 0.0f;
            const float r = in ? ndl.get(e) + e_bias : 0.0f;
            const float dt2 = in ? softplus_log2(r) : 0.0f;
            const float decay = SCALAR ? __builtin_amdgcn_exp2f(dt2 * e_ah) : 0.0f;
            float ds = 0.0f, dyv = 0.0f, zz = 0.0f;
            if constexpr (kRev) {
                dyv = in ? ndy.get(e) : 0.0f;
                zz = (has_z && in) ? nz.get(e) : 0.0f;
                ds = has_z ? dyv * silu_f32(zz) : dyv;
            }
            const int idx = tl * kLanes + e_ch;
            sW[idx] = make_float4(dt2, dt2 * uu, ds, decay);
            if constexpr (kG) {
                const float dzf = has_z ? dyv * silu_grad_f32(zz) : 0.0f;
                sF[idx] = make_float4(uu, sigmoid_f32(r), dzf, e_skip * uu);
            }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const bool in = bc_ok[k] && t0 + bc_t[k] < tend;
            if (bc_on[k]) sBC[bc_slot[k]] = in ? IOT<IO>::to_f32(nbc[k]) * ((bc_slot[k] & 1) ? 1.0f : kLn2) : 0.0f;
        }
    };

    // ---- per-lane LDS reads of one step
    const float4* swl = sW + lane;
    const float* sbw = sBC + w * SPL * 2;
    auto read_bc = [&](int t, float (&Bv)[SPL], float (&Cv)[SPL]) {
        const float* q = sbw + t * NP * 2;
        if constexpr (SPL == 1) {
            const float2 v = *reinterpret_cast<const float2*>(q);
            Bv[0] = v.x;
            Cv[0] = v.y;
        } else {
#pragma unroll
            for (int i = 0; i < SPL / 2; ++i) {
                const float4 v = reinterpret_cast<const float4*>(q)[i];
                Bv[2 * i] = v.x;
                Cv[2 * i] = v.y;
                Bv[2 * i + 1] = v.z;
                Cv[2 * i + 1] = v.w;
            }
        }
    };

    float h[SPL], e[SPL], dAacc[SPL], hst[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) h[j] = e[j] = dAacc[j] = hst[j] = 0.0f;
    float dtsum = 0.0f, dtcomp = 0.0f;   // compensated (Kahan) sum of dt2 (aggregate passes)
    auto kahan = [&](float v) {
        const float yk = v - dtcomp;
        const float tk = dtsum + yk;
        dtcomp = (tk - dtsum) - yk;
        dtsum = tk;
    };

    // ---- starting values
    if constexpr (MODE == kCkpt) {
        if (p.nchunks > 1) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) h[j] = p.fHin[state_base + int64_t(j) * kLanes];
        } else if (p.h0 && lane_ok) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const int64_t n = int64_t(w) * SPL + j;
                if (n < p.N) h[j] = p.h0[(int64_t(b) * p.dim + dch) * p.N + n];
            }
        }
    }
    if constexpr (kG) {
        if (p.nchunks > 1) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) e[j] = p.rEin[state_base + int64_t(j) * kLanes];
        } else if (p.dh_last && lane_ok) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const int64_t n = int64_t(w) * SPL + j;
                if (n < p.N) e[j] = p.dh_last[(int64_t(b) * p.dim + dch) * p.N + n];
            }
        }
    }

    // ---- one forward step from LDS (all modes but the reverse aggregate)
    auto fwd_step = [&](int t, float (&hh)[SPL], float (&Bv)[SPL], float (&Cv)[SPL], float4& W) {
        W = swl[t * kLanes];
        read_bc(t, Bv, Cv);
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const float a = SCALAR ? W.w : __builtin_amdgcn_exp2f(W.x * Ar[j]);
            hh[j] = fmaf(a, hh[j], W.y * Bv[j]);
        }
    };

    // ---- reduce 8 per-lane values over the wave's 64 lanes (channels) in a fixed
    //      order and write the sums to sdBC: value v = (s*2 + isC)*JR + jj belongs to
    //      step t_base + s and state entry w*SPL + j0 + jj.  The values go to LDS as
    //      [v][lane]; lane 8o+q then sums lanes 8q..8q+7 of value o, and the 8 lanes of
    //      an output combine their partials with DPP (quad swaps, then the half-row
    //      mirror), so every lane of the group holds the same total.  A wave's LDS
    //      operations complete in issue order, so the reads see this batch's writes and
    //      the next batch's writes cannot overtake these reads.
    float* red = sRed + w * kRound * kLanes;
    auto flush = [&](const float (&pv)[kRound], int t_base, int j0) {
#pragma unroll
        for (int v = 0; v < kRound; ++v) red[v * kLanes + lane] = pv[v];
        const int o = lane >> 3, q = lane & 7;
        const float4* rr = reinterpret_cast<const float4*>(red + o * kLanes + q * 8);
        const float4 a0 = rr[0], a1 = rr[1];
        float sum = ((a0.x + a0.y) + (a0.z + a0.w)) + ((a1.x + a1.y) + (a1.z + a1.w));
        sum += dpp_move<0xB1>(sum);    // quad_perm [1,0,3,2]: lanes 0<->1, 2<->3
        sum += dpp_move<0x4E>(sum);    // quad_perm [2,3,0,1]: lanes 0<->2, 1<->3
        sum += dpp_move<0x141>(sum);   // row_half_mirror: lane i <-> 7-i of each 8
        if (q == 0) {
            const int s = o / (2 * JR), isC = (o / JR) % 2, jj = o % JR;
            sdBC[(isC * NP + w * SPL + j0 + jj) * T + t_base + s] = sum;
        }
    };

    // ---- the same 8-value channel sum in registers (lane-swap butterfly, see the
    //      role-split gradient pass): dB of entries j0..j0+3 of this wave, then dC
    const bool lo8 = (lane & 8) == 0;
    const int red_v = ((lane >> 3) & 1) * 4 + ((lane >> 4) & 1) * 2 + (lane >> 5);
    auto reduce8 = [&](const float (&pv)[kRound], int t, int j0) {
        auto swap_add = [](float x, float y, auto swap) {
            const auto r = swap(__float_as_uint(x), __float_as_uint(y));
            return __uint_as_float(r[0]) + __uint_as_float(r[1]);
        };
        auto p32 = [](unsigned x, unsigned y) { return __builtin_amdgcn_permlane32_swap(x, y, false, false); };
        auto p16 = [](unsigned x, unsigned y) { return __builtin_amdgcn_permlane16_swap(x, y, false, false); };
        const float r0 = swap_add(pv[0], pv[1], p32), r1 = swap_add(pv[2], pv[3], p32);
        const float r2 = swap_add(pv[4], pv[5], p32), r3 = swap_add(pv[6], pv[7], p32);
        const float s0 = swap_add(r0, r1, p16), s1 = swap_add(r2, r3, p16);
        float sum = (lo8 ? s0 : s1) + dpp_move<0x128>(lo8 ? s1 : s0);   // row_ror:8
        sum += dpp_move<0xB1>(sum);
        sum += dpp_move<0x4E>(sum);
        sum += dpp_move<0x141>(sum);
        if ((lane & 7) == 0) sdBC[((red_v / 4) * NP + w * SPL + j0 + (red_v % 4)) * T + t] = sum;
    };

    // ---- the gradient walk of one tile (all waves); hst holds the tile's start state.
    //      Both walks read the LDS operands of the next step before the arithmetic of
    //      the current one, so that the LDS latency overlaps the work.
    struct StepOps {
        float4 W;
        float Bv[SPL], Cv[SPL];
    };
    auto read_step = [&](int t, StepOps& o) {
        o.W = swl[t * kLanes];
        read_bc(t, o.Bv, o.Cv);
    };
    auto get_bc = [&](const StepOps& o, int j, float& Bj, float& Cj) {
        Bj = o.Bv[j];
        Cj = o.Cv[j];
    };
    auto grad_tile = [&]() {
        float hsb[NSB > 1 ? NSB - 1 : 1][SPL];
        if constexpr (NSB > 1) {
            float hh[SPL];
#pragma unroll
            for (int j = 0; j < SPL; ++j) hh[j] = hst[j];
            StepOps cur, nxt;
            read_step(0, cur);
#pragma unroll
            for (int t = 0; t < (NSB - 1) * TS; ++t) {
                if (t + 1 < (NSB - 1) * TS) read_step(t + 1, nxt);
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    float Bj, Cj;
                    get_bc(cur, j, Bj, Cj);
                    const float a = SCALAR ? cur.W.w : __builtin_amdgcn_exp2f(cur.W.x * Ar[j]);
                    hh[j] = fmaf(a, hh[j], cur.W.y * Bj);
                }
                if ((t + 1) % TS == 0) {
#pragma unroll
                    for (int j = 0; j < SPL; ++j) hsb[t / TS][j] = hh[j];
                }
                cur = nxt;
            }
        }
#pragma unroll
        for (int sb = NSB - 1; sb >= 0; --sb) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            float hb[SPL], H[TS][SPL];
#pragma unroll
            for (int j = 0; j < SPL; ++j) hb[j] = (sb == 0) ? hst[j] : hsb[sb > 0 ? sb - 1 : 0][j];
            {
                float hh[SPL];
#pragma unroll
                for (int j = 0; j < SPL; ++j) hh[j] = hb[j];
                StepOps cur, nxt;
                read_step(sb * TS, cur);
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
                    const int t = sb * TS + ts;
                    if (ts + 1 < TS) read_step(t + 1, nxt);
                    float yp = 0.0f;
#pragma unroll
                    for (int j = 0; j < SPL; ++j) {
                        float Bj, Cj;
                        get_bc(cur, j, Bj, Cj);
                        const float a = SCALAR ? cur.W.w : __builtin_amdgcn_exp2f(cur.W.x * Ar[j]);
                        hh[j] = fmaf(a, hh[j], cur.W.y * Bj);
                        H[ts][j] = hh[j];
                        yp = fmaf(Cj, hh[j], yp);
                    }
                    sP[(w * T + t) * kLanes + lane] = yp;
                    cur = nxt;
                }
            }
            // re-read the step operands from LDS below rather than keeping the forward
            // recompute's copies of a whole sub-block live in VGPRs
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            float pv[kRound];
            StepOps cur, nxt;
            read_step(sb * TS + TS - 1, cur);
#pragma unroll
            for (int ts = TS - 1; ts >= 0; --ts) {
                const int t = sb * TS + ts;
                if (ts > 0) read_step(t - 1, nxt);
                float s1 = 0.0f, s2 = 0.0f;
                const int s = ts % RS;
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    float Bj, Cj;
                    get_bc(cur, j, Bj, Cj);
                    const float a = SCALAR ? cur.W.w : __builtin_amdgcn_exp2f(cur.W.x * Ar[j]);
                    const float hp = ts > 0 ? H[ts > 0 ? ts - 1 : 0][j] : hb[j];
                    const float g = fmaf(cur.W.z, Cj, e[j]);
                    const float t1 = g * (a * hp);
                    dAacc[j] = fmaf(cur.W.x, t1, dAacc[j]);
                    s1 = fmaf(Ar[j], t1, s1);
                    s2 = fmaf(g, Bj, s2);
                    e[j] = a * g;
                    const int jj = j % JR;
                    pv[(s * 2) * JR + jj] = g * cur.W.y;              // dB (unscaled)
                    pv[(s * 2 + 1) * JR + jj] = cur.W.z * H[ts][j];   // dC
                    if constexpr (NJR > 1) {
                        if (jj == JR - 1) flush(pv, t, j - jj);
                    }
                }
                sP[kSlab + (w * T + t) * kLanes + lane] = s1;
                sP[2 * kSlab + (w * T + t) * kLanes + lane] = s2;
                if constexpr (NJR == 1) {
                    if (s == 0) flush(pv, t, 0);
                }
                cur = nxt;
            }
        }
    };

    // ---- the gradient walk with 8 or more entries per lane: the entries in groups of
    //      4, each group recomputing the tile's states from the checkpoint and walking
    //      back through them, so only one group's states are live in VGPRs (a whole
    //      tile of 8 or 16 entries did not fit and spilled).  The group loop is not
    //      unrolled (unrolled, the compiler interleaved the groups and spilled more);
    //      the group always works on entries 0..3 of the per-entry arrays, which are
    //      rotated by 4 after each group and so return to their order after the last.
    //      The per-step sums over entries (read-out, sum A g a h, sum g B') are
    //      accumulated over the groups in the wave's LDS slab rows.  Each
    //      phase addresses the LDS step operands through its own opaque zero offset:
    //      with equal addresses the compiler kept the recompute's B and C values for
    //      the reverse walk instead of reading them again, and spilled them.
    auto grad_tile_grouped = [&]() {
        constexpr int GS = 4, NG = SPL / GS;
        static_assert(SPL < 8 || (SPL % GS == 0 && JR == GS && RS == 1), "one reduction round per step and group");
        // per-step sums of this wave: the first group writes its slab rows, later
        // groups add to them
        float* const yrow = sP + (w * T) * kLanes + lane;
        auto rotate = [](float (&v)[SPL]) {
            float first[GS];
#pragma unroll
            for (int k = 0; k < GS; ++k) first[k] = v[k];
#pragma unroll
            for (int k = 0; k + GS < SPL; ++k) v[k] = v[k + GS];
#pragma unroll
            for (int k = 0; k < GS; ++k) v[SPL - GS + k] = first[k];
        };
        // the step's operands for the group: (dt2, x, ds, decay) and (B, C) of its 4
        // entries, read one step ahead
        struct GOps {
            float4 W, bc0, bc1;
        };
        auto gread = [&](int off, int t, int j0, GOps& o) {
            o.W = swl[off + t * kLanes];
            const float4* q = reinterpret_cast<const float4*>(sbw + off + t * NP * 2 + 2 * j0);
            o.bc0 = q[0];
            o.bc1 = q[1];
        };
        auto bj = [](const GOps& o, int jj) { return jj == 0 ? o.bc0.x : jj == 1 ? o.bc0.z : jj == 2 ? o.bc1.x : o.bc1.z; };
        auto cj = [](const GOps& o, int jj) { return jj == 0 ? o.bc0.y : jj == 1 ? o.bc0.w : jj == 2 ? o.bc1.y : o.bc1.w; };
#pragma unroll 1
        for (int gi = 0; gi < NG; ++gi) {
            const int j0 = gi * GS;       // the group's first entry
            const bool first = gi == 0;
            float H[T][GS];
            {
                int off = 0;
                asm volatile("" : "+v"(off));
                float hh[GS];
#pragma unroll
                for (int jj = 0; jj < GS; ++jj) hh[jj] = hst[jj];
                GOps cur, nxt;
                gread(off, 0, j0, cur);
                // the earlier groups' partial sum of a step is read a step ahead,
                // together with the step's operands (the rows of later steps are not
                // written before they are read)
                float ypc = yrow[0], ypn = 0.0f;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    if (t + 1 < T) {
                        gread(off, t + 1, j0, nxt);
                        ypn = yrow[(t + 1) * kLanes];
                    }
                    float yp = first ? 0.0f : ypc;
#pragma unroll
                    for (int jj = 0; jj < GS; ++jj) {
                        const float a = SCALAR ? cur.W.w : __builtin_amdgcn_exp2f(cur.W.x * Ar[jj]);
                        hh[jj] = fmaf(a, hh[jj], cur.W.y * bj(cur, jj));
                        H[t][jj] = hh[jj];
                        yp = fmaf(cj(cur, jj), hh[jj], yp);
                    }
                    yrow[t * kLanes] = yp;
                    cur = nxt;
                    ypc = ypn;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            int off = 0;
            asm volatile("" : "+v"(off));
            float pv[kRound];
            GOps cur, nxt;
            gread(off, T - 1, j0, cur);
            float s1c = yrow[kSlab + (T - 1) * kLanes], s2c = yrow[2 * kSlab + (T - 1) * kLanes];
            float s1n = 0.0f, s2n = 0.0f;
#pragma unroll
            for (int t = T - 1; t >= 0; --t) {
                if (t > 0) {
                    gread(off, t - 1, j0, nxt);
                    s1n = yrow[kSlab + (t - 1) * kLanes];
                    s2n = yrow[2 * kSlab + (t - 1) * kLanes];
                }
                float s1 = first ? 0.0f : s1c;
                float s2 = first ? 0.0f : s2c;
                float t1s = 0.0f;   // scalar decay: sum over the group of g * a * h_prev
#pragma unroll
                for (int jj = 0; jj < GS; ++jj) {
                    const float Bj = bj(cur, jj), Cj = cj(cur, jj);
                    const float a = SCALAR ? cur.W.w : __builtin_amdgcn_exp2f(cur.W.x * Ar[jj]);
                    const float hp = t > 0 ? H[t > 0 ? t - 1 : 0][jj] : hst[jj];
                    const float g = fmaf(cur.W.z, Cj, e[jj]);
                    if constexpr (SCALAR) {
                        t1s = fmaf(g, a * hp, t1s);
                    } else {
                        const float t1 = g * (a * hp);
                        dAacc[jj] = fmaf(cur.W.x, t1, dAacc[jj]);
                        s1 = fmaf(Ar[jj], t1, s1);
                    }
                    s2 = fmaf(g, Bj, s2);
                    e[jj] = a * g;
                    pv[jj] = g * cur.W.y;              // dB (unscaled)
                    pv[GS + jj] = cur.W.z * H[t][jj];  // dC
                }
                if constexpr (SCALAR) {
                    // the head's rate is every entry's: its dA goes to the group's first
                    // entry (a padding entry only when the whole group is padding, whose
                    // terms are zero); the head sum adds all entries
                    dAacc[0] = fmaf(cur.W.x, t1s, dAacc[0]);
                    s1 = fmaf(Ar[0], t1s, s1);
                }
                yrow[kSlab + t * kLanes] = s1;
                yrow[2 * kSlab + t * kLanes] = s2;
                reduce8(pv, t, j0);
                cur = nxt;
                s1c = s1n;
                s2c = s2n;
                __builtin_amdgcn_sched_barrier(0);
            }
            rotate(e);
            rotate(dAacc);
            rotate(hst);
            if constexpr (!SCALAR) rotate(Ar);
        }
    };

    // ---- finish the tile starting at t0 (all threads): per-element outputs, the
    //      per-thread dD / ddt_bias sums, and the tile's dB / dC partials
    IO* __restrict__ gdu = static_cast<IO*>(p.du);
    IO* __restrict__ gdd = static_cast<IO*>(p.ddelta);
    IO* __restrict__ gdz = static_cast<IO*>(p.dz);
    const bool write_dz = p.dz != nullptr && p.z != nullptr;
    float accD = 0.0f, accBias = 0.0f;
    auto finish = [&](int64_t t0) {
        Seg<IO, EPT> odu, odd, odz;
#pragma unroll
        for (int e2 = 0; e2 < EPT; ++e2) {
            const int tl = e_seg * EPT + e2;
            const int idx = tl * kLanes + e_ch;
            const bool in = e_ok && t0 + tl < tend;
            const float4 Wv = sW[idx];
            const float4 Fv = sF[idx];
            float yp = sP[idx], s1 = sP[kSlab + idx], s2 = sP[2 * kSlab + idx];
#pragma unroll
            for (int ww = 1; ww < G; ++ww) {
                const int o = ww * T * kLanes + idx;
                yp += sP[o];
                s1 += sP[kSlab + o];
                s2 += sP[2 * kSlab + o];
            }
            const float ddt = fmaf(Fv.x * kLog2e, s2, s1);
            const float dd = ddt * Fv.y;
            const float dui = fmaf(e_skip, Wv.z, Wv.x * s2);
            const float dzi = Fv.z * (yp + Fv.w);
            if (in) {
                accD = fmaf(Wv.z, Fv.x, accD);
                accBias += dd;
            }
            odu.e[e2] = IOT<IO>::from_f32(dui);
            odd.e[e2] = IOT<IO>::from_f32(dd);
            odz.e[e2] = IOT<IO>::from_f32(dzi);
        }
        const int64_t t = t0 + e_seg * EPT;
        store_seg<IO, EPT, VEC>(gdu + e_row, t, tend, e_ok, odu);
        store_seg<IO, EPT, VEC>(gdd + e_row, t, tend, e_ok, odd);
        if (write_dz) store_seg<IO, EPT, VEC>(gdz + e_row, t, tend, e_ok, odz);
        for (int i = tid; i < 2 * int(p.N) * T; i += NT) {
            const int isC = i / (int(p.N) * T);
            const int rem = i % (int(p.N) * T);
            const int n = rem / T, tt = rem % T;
            if (t0 + tt < tend)
                p.pBC[(((int64_t(cblk) * p.batch + b) * 2 + isC) * p.N + n) * p.L + t0 + tt] = sdBC[(isC * NP + n) * T + tt];
        }
    };

    // ---- forward walk of one tile (checkpoint pass, forward aggregate)
    auto fwd_tile = [&](int kt) {
        if constexpr (MODE == kCkpt) {
            float* ck = p.ck + ((blk * p.ntiles_seq + tile0 + kt) * NP + int64_t(w) * SPL) * kLanes + lane;
#pragma unroll
            for (int j = 0; j < SPL; ++j) ck[int64_t(j) * kLanes] = h[j];
        }
        float Bv[SPL], Cv[SPL];
        float4 W;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            fwd_step(t, h, Bv, Cv, W);
            if constexpr (MODE == kFwdAgg) kahan(W.x);
        }
    };

    // ---- reverse walk of one tile without gradients (reverse aggregate)
    auto rev_tile = [&]() {
#pragma unroll
        for (int t = T - 1; t >= 0; --t) {
            const float4 W = swl[t * kLanes];
            float Bv[SPL], Cv[SPL];
            read_bc(t, Bv, Cv);
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const float a = SCALAR ? W.w : __builtin_amdgcn_exp2f(W.x * Ar[j]);
                e[j] = a * fmaf(W.z, Cv[j], e[j]);
            }
            kahan(W.x);
        }
    };

    // ---- tile loop: stage (from the prefetch), prefetch the next tile, walk, finish
    const int first = kRev ? ntiles - 1 : 0;
    issue_loads(first);
    for (int i = 0; i < ntiles; ++i) {
        const int kt = kRev ? ntiles - 1 - i : i;
        const int64_t t0 = tbeg + int64_t(kt) * T;
        stage(t0);
        if constexpr (kG) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) hst[j] = ckn[j];
        }
        if (i + 1 < ntiles) issue_loads(kRev ? kt - 1 : kt + 1);
        __syncthreads();
        if constexpr (kG) {
            if constexpr (SPL >= 8) grad_tile_grouped();   // 8 or 16 entries per lane
            else grad_tile();
        }
        else if constexpr (MODE == kRevAgg) rev_tile();
        else fwd_tile(kt);
        __syncthreads();
        if constexpr (kG) {
            finish(t0);
            __syncthreads();
        }
    }

    // ---- results of the pass
    if constexpr (MODE == kFwdAgg || MODE == kRevAgg) {
        float* dst = (MODE == kFwdAgg ? p.fH : p.rG) + state_base;
#pragma unroll
        for (int j = 0; j < SPL; ++j) dst[int64_t(j) * kLanes] = MODE == kFwdAgg ? h[j] : e[j];
        if (w == 0) (MODE == kFwdAgg ? p.fS : p.rS)[(blk * p.nchunks + piece) * kLanes + lane] = dtsum;
    }
    if constexpr (kG) {
        if (lane_ok) {
            float* pa = p.pA + ((int64_t(piece) * p.batch + b) * p.dim + dch) * NP + int64_t(w) * SPL;
#pragma unroll
            for (int j = 0; j < SPL; ++j) pa[j] = dAacc[j];
            if (piece == 0 && p.dh0) {
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const int64_t n = int64_t(w) * SPL + j;
                    if (n < p.N) p.dh0[(int64_t(b) * p.dim + dch) * p.N + n] = e[j];
                }
            }
        }
        // per-channel sums of the G threads of a channel, in segment order
        float* fin = smem;   // [2][G][64], the segment index is the wave index
        fin[e_seg * kLanes + e_ch] = accD;
        fin[(G + e_seg) * kLanes + e_ch] = accBias;
        __syncthreads();
        if (tid < kLanes && c0 + tid < p.dim) {
            float sd = 0.0f, sb = 0.0f;
#pragma unroll
            for (int sg = 0; sg < G; ++sg) {
                sd += fin[sg * kLanes + tid];
                sb += fin[(G + sg) * kLanes + tid];
            }
            const int64_t o = (int64_t(piece) * p.batch + b) * p.dim + c0 + tid;
            p.pD[o] = sd;
            p.pbias[o] = sb;
        }
    }
}

// ---------------------------------------------------------------- gradient pass with
// separate roles.  G walking waves (wave w holds entries SPL*w..SPL*w+SPL-1 of all 64
// channels) walk tile k while four helper waves finish tile k-1 and stage tile k+1, so
// the staging and finishing work fills the issue slots the walk leaves on each SIMD
// instead of running between barriers.  Tiles are double-buffered in LDS and there is
// one barrier per tile.  A helper thread stages and finishes the same elements (T/4
// consecutive steps of one channel), so finishing tile k-1 and then staging tile k+1
// into the same buffer needs no barrier between them; the per-element values finishing
// needs besides the walk's sums (u, sigmoid of the step input, the gate's derivative)
// stay in the helper's registers, one set per buffer.
//   SPL = 4, G = 4, T = 16 (9..16 state entries): the walk keeps the tile's recomputed
//     states and decays in VGPRs, so the reverse step evaluates no second exponential;
//   SPL = 16, G = 8, T = 8 (65..128 entries, scalar decay): the entries are walked in
//     groups of 4 as in the generic kernel's grouped walk, the per-step sums over
//     entries accumulated in the wave's slab rows.
template <int SPL_, int G_, int T_> struct WsShape {
    static constexpr int SPL = SPL_, G = G_, H = 4, T = T_, NP = G * SPL, EPT = T / H, NTH = H * kLanes;
    static constexpr int kW = T * kLanes * 4;        // (dt2, dt2*u, ds, scalar decay) per step and channel
    static constexpr int kBC = T * NP * 2;           // (B*ln2, C) per step and entry
    static constexpr int kSlab = G * T * kLanes;     // per-wave sums over the wave's entries, per step and channel
    static constexpr int kDBC = 2 * NP * T;          // the tile's dB (unscaled), dC summed over the 64 channels
    static constexpr int kBuf = kW + kBC + 3 * kSlab + kDBC;
    static constexpr int kThreads = (G + H) * kLanes;
    static constexpr size_t kLdsBytes = size_t(2 * kBuf) * sizeof(float);
    static constexpr int KB = (2 * NP * T + NTH - 1) / NTH;   // B/C values per helper thread and tile
};
namespace wsg {   // 9..16 entries
constexpr int SPL = 4, G = 4, T = 16, NP = G * SPL, EPT = T / 4;
using Shape = WsShape<SPL, G, T>;
}  // namespace wsg
namespace wsw {   // 65..128 entries, scalar decay
using Shape = WsShape<16, 8, 8>;
}  // namespace wsw

template <typename IO, bool SCALAR, bool VEC, int SPL_, int G_, int T_>
__global__ void __launch_bounds__((WsShape<SPL_, G_, T_>::kThreads)) scan_bwd_grad_ws_kernel(BwdParams p) {
    using S = WsShape<SPL_, G_, T_>;
    constexpr int SPL = S::SPL, G = S::G, H = S::H, T = S::T, NP = S::NP, EPT = S::EPT, NTH = S::NTH;
    constexpr int kW = S::kW, kBC = S::kBC, kSlab = S::kSlab, kBuf = S::kBuf, KB = S::KB;
    constexpr bool kGrouped = SPL > 4;            // entries walked in groups of 4
    static_assert(SPL == 4 || (SPL % 4 == 0 && SCALAR), "wide lanes are built for scalar decay only");
    static_assert(KB * NTH == 2 * NP * T, "the tile's B and C values must split evenly over the helpers");
    extern __shared__ float smem[];
    const int tid = threadIdx.x;
    const int wv = tid / kLanes;
    const int lane = tid % kLanes;
    const bool walker = wv < G;                   // wave-uniform
    const int64_t bid = blockIdx.x;
    const int cblk = int(bid % p.nblk_d);
    const int b = int((bid / p.nblk_d) % p.batch);
    const int piece = int(bid / (int64_t(p.nblk_d) * p.batch)) + p.piece_base;
    const int64_t blk = int64_t(b) * p.nblk_d + cblk;
    const int64_t c0 = int64_t(cblk) * kLanes;
    const int64_t tbeg = int64_t(piece) * p.chunk_len;
    const int64_t tend = (tbeg + p.chunk_len < p.L) ? tbeg + p.chunk_len : p.L;
    const int ntiles = int((tend - tbeg + T - 1) / T);
    const int64_t tile0 = tbeg / T;
    auto kt_of = [&](int i) { return ntiles - 1 - i; };   // tiles in reverse order
    auto buf = [&](int par) { return smem + par * kBuf; };

    // ================================================================ walkers
    // lane = channel c0 + lane, entries n = 4*wv + j
    const int64_t dch = c0 + lane;
    const bool lane_ok = dch < p.dim;
    float Ar[SPL], e[SPL], dAacc[SPL], hst[SPL], ckn[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
        const int64_t n = int64_t(wv) * SPL + j;
        Ar[j] = 0.0f;
        if (walker && lane_ok) {
            if constexpr (SCALAR) Ar[j] = p.A[dch / p.head_dim];
            else if (n < p.N) Ar[j] = p.A[dch * p.N + n];
        }
        e[j] = dAacc[j] = hst[j] = ckn[j] = 0.0f;
    }
    if (walker) {
        if (p.nchunks > 1) {
            const int64_t sb = ((blk * p.nchunks + piece) * NP + int64_t(wv) * SPL) * kLanes + lane;
#pragma unroll
            for (int j = 0; j < SPL; ++j) e[j] = p.rEin[sb + int64_t(j) * kLanes];
        } else if (p.dh_last && lane_ok) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const int64_t n = int64_t(wv) * SPL + j;
                if (n < p.N) e[j] = p.dh_last[(int64_t(b) * p.dim + dch) * p.N + n];
            }
        }
    }
    bool ck_ok[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) ck_ok[j] = lane_ok && int64_t(wv) * SPL + j < p.N;
    auto load_ck = [&](int kt) {
        const float* ck = p.ck + ((blk * p.ntiles_seq + tile0 + kt) * NP + int64_t(wv) * SPL) * kLanes + lane;
#pragma unroll
        for (int j = 0; j < SPL; ++j) ckn[j] = ck[int64_t(j) * kLanes];
    };

    struct StepOps {
        float4 W;
        float Bv[SPL], Cv[SPL];
    };
    auto read_step = [&](const float* bf, int t, StepOps& o) {
        o.W = reinterpret_cast<const float4*>(bf)[t * kLanes + lane];
        const float4* q = reinterpret_cast<const float4*>(bf + kW + t * NP * 2 + wv * SPL * 2);
        const float4 v0 = q[0], v1 = q[1];
        o.Bv[0] = v0.x; o.Cv[0] = v0.y; o.Bv[1] = v0.z; o.Cv[1] = v0.w;
        o.Bv[2] = v1.x; o.Cv[2] = v1.y; o.Bv[3] = v1.z; o.Cv[3] = v1.w;
    };

    // sum 8 per-lane values over the wave's 64 lanes (channels) in registers, in a
    // fixed order.  Value v < 4 is dB of entry 4*wv+v, v >= 4 dC of entry 4*wv+v-4.
    //   1. v_permlane32_swap on value pairs (2k, 2k+1), then add: register k holds
    //      value 2k in lanes 0-31 and 2k+1 in lanes 32-63, each lane m the sum of
    //      lanes m and m^32;
    //   2. v_permlane16_swap on register pairs, then add: two registers whose 16-lane
    //      rows hold values (0, 2, 1, 3) and (4, 6, 5, 7), each lane the sum of 4;
    //   3. within each row, lanes 0-7 keep the first register plus its other half-row
    //      and lanes 8-15 the second (a row rotation by 8): each lane the sum of 8;
    //   4. DPP quad swaps and the half-row mirror sum the 8 lanes of each group.
    // Group g = lane / 8 then holds value (g % 2) * 4 + ((g / 2) % 2) * 2 + g / 4.
    const bool lo8 = (lane & 8) == 0;
    const int red_v = ((lane >> 3) & 1) * 4 + ((lane >> 4) & 1) * 2 + (lane >> 5);
    auto swap_add = [](float x, float y, auto swap) {
        const auto r = swap(__float_as_uint(x), __float_as_uint(y));
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    };
    auto p32 = [](unsigned x, unsigned y) { return __builtin_amdgcn_permlane32_swap(x, y, false, false); };
    auto p16 = [](unsigned x, unsigned y) { return __builtin_amdgcn_permlane16_swap(x, y, false, false); };
    auto reduce8 = [&](const float (&pv)[kRound], float* sdBC, int t, int j0) {
        const float r0 = swap_add(pv[0], pv[1], p32), r1 = swap_add(pv[2], pv[3], p32);
        const float r2 = swap_add(pv[4], pv[5], p32), r3 = swap_add(pv[6], pv[7], p32);
        const float s0 = swap_add(r0, r1, p16), s1 = swap_add(r2, r3, p16);
        float sum = (lo8 ? s0 : s1) + dpp_move<0x128>(lo8 ? s1 : s0);   // row_ror:8
        sum += dpp_move<0xB1>(sum);    // quad_perm [1,0,3,2]
        sum += dpp_move<0x4E>(sum);    // quad_perm [2,3,0,1]
        sum += dpp_move<0x141>(sum);   // row_half_mirror
        if ((lane & 7) == 0) sdBC[((red_v / 4) * NP + wv * SPL + j0 + (red_v % 4)) * T + t] = sum;
    };

    auto walk = [&](float* bf) {
        float* sP = bf + kW + kBC;
        float* sdBC = sP + 3 * kSlab;
        float Hs[T][SPL], Aa[T][SPL];
        {
            float hh[SPL];
#pragma unroll
            for (int j = 0; j < SPL; ++j) hh[j] = hst[j];
            StepOps cur, nxt;
            read_step(bf, 0, cur);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                if (t + 1 < T) read_step(bf, t + 1, nxt);
                float yp = 0.0f;
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const float a = SCALAR ? cur.W.w : __builtin_amdgcn_exp2f(cur.W.x * Ar[j]);
                    hh[j] = fmaf(a, hh[j], cur.W.y * cur.Bv[j]);
                    Hs[t][j] = hh[j];
                    Aa[t][j] = a;
                    yp = fmaf(cur.Cv[j], hh[j], yp);
                }
                sP[(wv * T + t) * kLanes + lane] = yp;
                cur = nxt;
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        StepOps cur, nxt;
        read_step(bf, T - 1, cur);
#pragma unroll
        for (int t = T - 1; t >= 0; --t) {
            if (t > 0) read_step(bf, t - 1, nxt);
            float s1 = 0.0f, s2 = 0.0f, pv[kRound];
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const float a = Aa[t][j];
                const float hp = t > 0 ? Hs[t > 0 ? t - 1 : 0][j] : hst[j];
                const float g = fmaf(cur.W.z, cur.Cv[j], e[j]);
                const float t1 = g * (a * hp);
                dAacc[j] = fmaf(cur.W.x, t1, dAacc[j]);
                s1 = fmaf(Ar[j], t1, s1);
                s2 = fmaf(g, cur.Bv[j], s2);
                e[j] = a * g;
                pv[j] = g * cur.W.y;                 // dB (unscaled)
                pv[SPL + j] = cur.W.z * Hs[t][j];    // dC
            }
            sP[kSlab + (wv * T + t) * kLanes + lane] = s1;
            sP[2 * kSlab + (wv * T + t) * kLanes + lane] = s2;
            reduce8(pv, sdBC, t, 0);
            cur = nxt;
        }
    };

    // entries in groups of 4 (wide lanes, scalar decay): each group recomputes the
    // tile's states from the checkpoint and walks back through them; the group always
    // works on entries 0..3 of the per-entry arrays, which rotate by 4 after each group
    // (the group loop is not unrolled); the per-step sums accumulate in the wave's slab
    // rows; the decay is every entry's, so one running sum of g * a * h_prev per step
    // gives both the dA term (kept in entry 0 of each group) and the sum of A g a h.
    struct GOps {
        float4 W, bc0, bc1;
    };
    auto gread = [&](const float* bf, int off, int t, int j0, GOps& o) {
        o.W = reinterpret_cast<const float4*>(bf)[off + t * kLanes + lane];
        const float4* q = reinterpret_cast<const float4*>(bf + off + kW + t * NP * 2 + (wv * SPL + j0) * 2);
        o.bc0 = q[0];
        o.bc1 = q[1];
    };
    auto gb = [](const GOps& o, int jj) { return jj == 0 ? o.bc0.x : jj == 1 ? o.bc0.z : jj == 2 ? o.bc1.x : o.bc1.z; };
    auto gc = [](const GOps& o, int jj) { return jj == 0 ? o.bc0.y : jj == 1 ? o.bc0.w : jj == 2 ? o.bc1.y : o.bc1.w; };
    auto rotate = [](float (&v)[SPL]) {
        float first[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) first[k] = v[k];
#pragma unroll
        for (int k = 0; k + 4 < SPL; ++k) v[k] = v[k + 4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[SPL - 4 + k] = first[k];
    };
    auto walk_grouped = [&](float* bf) {
        float* const yrow = bf + kW + kBC + (wv * T) * kLanes + lane;
        float* sdBC = bf + kW + kBC + 3 * kSlab;
#pragma unroll 1
        for (int gi = 0; gi < SPL / 4; ++gi) {
            const int j0 = gi * 4;
            const bool first = gi == 0;
            float Hg[T][4];
            {
                int off = 0;
                asm volatile("" : "+v"(off));
                float hh[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) hh[jj] = hst[jj];
                GOps cur, nxt;
                gread(bf, off, 0, j0, cur);
                // the earlier groups' partial sum of a step is read a step ahead,
                // together with the step's operands (the rows of later steps are not
                // written before they are read)
                float ypc = yrow[0], ypn = 0.0f;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    if (t + 1 < T) {
                        gread(bf, off, t + 1, j0, nxt);
                        ypn = yrow[(t + 1) * kLanes];
                    }
                    float yp = first ? 0.0f : ypc;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        hh[jj] = fmaf(cur.W.w, hh[jj], cur.W.y * gb(cur, jj));
                        Hg[t][jj] = hh[jj];
                        yp = fmaf(gc(cur, jj), hh[jj], yp);
                    }
                    yrow[t * kLanes] = yp;
                    cur = nxt;
                    ypc = ypn;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            int off = 0;
            asm volatile("" : "+v"(off));
            float pv[kRound];
            GOps cur, nxt;
            gread(bf, off, T - 1, j0, cur);
            float s1c = yrow[kSlab + (T - 1) * kLanes], s2c = yrow[2 * kSlab + (T - 1) * kLanes];
            float s1n = 0.0f, s2n = 0.0f;
#pragma unroll
            for (int t = T - 1; t >= 0; --t) {
                if (t > 0) {
                    gread(bf, off, t - 1, j0, nxt);
                    s1n = yrow[kSlab + (t - 1) * kLanes];
                    s2n = yrow[2 * kSlab + (t - 1) * kLanes];
                }
                float s1 = first ? 0.0f : s1c;
                float s2 = first ? 0.0f : s2c;
                float t1s = 0.0f;
                const float a = cur.W.w;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float hp = t > 0 ? Hg[t > 0 ? t - 1 : 0][jj] : hst[jj];
                    const float g = fmaf(cur.W.z, gc(cur, jj), e[jj]);
                    t1s = fmaf(g, a * hp, t1s);
                    s2 = fmaf(g, gb(cur, jj), s2);
                    e[jj] = a * g;
                    pv[jj] = g * cur.W.y;              // dB (unscaled)
                    pv[4 + jj] = cur.W.z * Hg[t][jj];  // dC
                }
                dAacc[0] = fmaf(cur.W.x, t1s, dAacc[0]);
                s1 = fmaf(Ar[0], t1s, s1);
                yrow[kSlab + t * kLanes] = s1;
                yrow[2 * kSlab + t * kLanes] = s2;
                reduce8(pv, sdBC, t, j0);
                cur = nxt;
                s1c = s1n;
                s2c = s2n;
                __builtin_amdgcn_sched_barrier(0);
            }
            rotate(e);
            rotate(dAacc);
            rotate(hst);
        }
    };

    // ================================================================ helpers
    // helper hw = wv - G, thread ht: channel c0 + lane, steps 4*hw .. 4*hw+3 of a tile
    const int ht = tid - G * kLanes;              // negative on walkers (unused there)
    const int e_seg = walker ? 0 : wv - G;
    const int64_t e_d = c0 + lane;
    const bool e_ok = !walker && e_d < p.dim;
    const float e_bias = (e_ok && p.bias) ? p.bias[e_d] : 0.0f;
    const float e_skip = (e_ok && p.Dskip) ? p.Dskip[e_d] : 0.0f;
    const float e_ah = (SCALAR && e_ok) ? p.A[e_d / p.head_dim] : 0.0f;
    const int64_t e_row = (int64_t(b) * p.dim + (e_ok ? e_d : 0)) * p.L;
    const bool has_z = p.z != nullptr;
    const IO* __restrict__ gu = static_cast<const IO*>(p.u);
    const IO* __restrict__ gdl = static_cast<const IO*>(p.delta);
    const IO* __restrict__ gz = static_cast<const IO*>(p.z);
    const IO* __restrict__ gdy = static_cast<const IO*>(p.dy);
    const IO* __restrict__ gB = static_cast<const IO*>(p.Bm);
    const IO* __restrict__ gC = static_cast<const IO*>(p.Cm);

    // B/C value v = ht + k*NTH -> (B or C, entry n, step t of the tile)
    const IO* bc_ptr[KB];
    int bc_slot[KB], bc_t[KB];
    bool bc_ok[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int v = (walker ? 0 : ht) + k * NTH;
        const int isC = v / (NP * T);
        const int n = (v / T) % NP;
        bc_t[k] = v % T;
        bc_ok[k] = !walker && n < p.N;
        bc_ptr[k] = (isC ? gC : gB) + (int64_t(b) * p.N + (bc_ok[k] ? n : 0)) * p.L + bc_t[k];
        bc_slot[k] = (bc_t[k] * NP + n) * 2 + isC;
    }

    InSeg<IO, EPT, VEC> nu, ndl, nz, ndy;
    IO nbc[KB];
    auto issue_loads = [&](int kt) {
        const int64_t t0 = tbeg + int64_t(kt) * T;
        const int64_t t = t0 + e_seg * EPT;
        nu = load_seg<IO, EPT, VEC>(gu + e_row, t, tend, e_ok);
        ndl = load_seg<IO, EPT, VEC>(gdl + e_row, t, tend, e_ok);
        ndy = load_seg<IO, EPT, VEC>(gdy + e_row, t, tend, e_ok);
        nz = load_seg<IO, EPT, VEC>((has_z ? gz : gdy) + e_row, t, tend, e_ok && has_z);
#pragma unroll
        for (int k = 0; k < KB; ++k) nbc[k] = *((bc_ok[k] && t0 + bc_t[k] < tend) ? bc_ptr[k] + t0 : gB);
    };

    // finishing inputs kept from staging: u, sigmoid(delta + bias), dy * SiLU'(z);
    // set P belongs to the tiles staged into buffer P
    float Fu[2][EPT], Fsg[2][EPT], Fdz[2][EPT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int k = 0; k < EPT; ++k) Fu[s][k] = Fsg[s][k] = Fdz[s][k] = 0.0f;

    // registers -> LDS buffer P for tile kt; steps beyond the piece's end are identity
    // steps (dt2 = 0, x = 0, ds = 0, decay 1)
    auto stage = [&](int kt, auto par) {
        constexpr int P = decltype(par)::value;
        float* bf = buf(P);
        const int64_t t0 = tbeg + int64_t(kt) * T;
        float4* sW = reinterpret_cast<float4*>(bf);
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int tl = e_seg * EPT + k;
            const bool in = e_ok && t0 + tl < tend;
            const float uu = in ? nu.get(k) : 0.0f;
            const float r = in ? ndl.get(k) + e_bias : 0.0f;
            const float dt2 = in ? softplus_log2(r) : 0.0f;
            const float decay = SCALAR ? __builtin_amdgcn_exp2f(dt2 * e_ah) : 0.0f;
            const float dyv = in ? ndy.get(k) : 0.0f;
            const float zz = (has_z && in) ? nz.get(k) : 0.0f;
            const float ds = has_z ? dyv * silu_f32(zz) : dyv;
            sW[tl * kLanes + lane] = make_float4(dt2, dt2 * uu, ds, decay);
            Fu[P][k] = uu;
            Fsg[P][k] = sigmoid_f32(r);
            Fdz[P][k] = has_z ? dyv * silu_grad_f32(zz) : 0.0f;
        }
        float* sBC = bf + kW;
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const bool in = bc_ok[k] && t0 + bc_t[k] < tend;
            sBC[bc_slot[k]] = in ? IOT<IO>::to_f32(nbc[k]) * ((bc_slot[k] & 1) ? 1.0f : kLn2) : 0.0f;
        }
    };

    IO* __restrict__ gdu = static_cast<IO*>(p.du);
    IO* __restrict__ gdd = static_cast<IO*>(p.ddelta);
    IO* __restrict__ gdz = static_cast<IO*>(p.dz);
    const bool write_dz = p.dz != nullptr && has_z;
    float accD = 0.0f, accBias = 0.0f;
    auto finish = [&](int kt, auto par) {
        constexpr int P = decltype(par)::value;
        const float* bf = buf(P);
        const int64_t t0 = tbeg + int64_t(kt) * T;
        const float4* sW = reinterpret_cast<const float4*>(bf);
        const float* sP = bf + kW + kBC;
        const float* sdBC = sP + 3 * kSlab;
        Seg<IO, EPT> odu, odd, odz;
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int tl = e_seg * EPT + k;
            const int idx = tl * kLanes + lane;
            const bool in = e_ok && t0 + tl < tend;
            const float4 Wv = sW[idx];
            float yp = sP[idx], s1 = sP[kSlab + idx], s2 = sP[2 * kSlab + idx];
#pragma unroll
            for (int w = 1; w < G; ++w) {
                const int o = w * T * kLanes + idx;
                yp += sP[o];
                s1 += sP[kSlab + o];
                s2 += sP[2 * kSlab + o];
            }
            const float uu = Fu[P][k];
            const float ddt = fmaf(uu * kLog2e, s2, s1);
            const float dd = ddt * Fsg[P][k];
            const float dui = fmaf(e_skip, Wv.z, Wv.x * s2);
            const float dzi = Fdz[P][k] * fmaf(e_skip, uu, yp);
            if (in) {
                accD = fmaf(Wv.z, uu, accD);
                accBias += dd;
            }
            odu.e[k] = IOT<IO>::from_f32(dui);
            odd.e[k] = IOT<IO>::from_f32(dd);
            odz.e[k] = IOT<IO>::from_f32(dzi);
        }
        const int64_t t = t0 + e_seg * EPT;
        store_seg<IO, EPT, VEC>(gdu + e_row, t, tend, e_ok, odu);
        store_seg<IO, EPT, VEC>(gdd + e_row, t, tend, e_ok, odd);
        if (write_dz) store_seg<IO, EPT, VEC>(gdz + e_row, t, tend, e_ok, odz);
        for (int i = ht; i < 2 * int(p.N) * T; i += NTH) {
            const int isC = i / (int(p.N) * T);
            const int rem = i % (int(p.N) * T);
            const int n = rem / T, tt = rem % T;
            if (t0 + tt < tend)
                p.pBC[(((int64_t(cblk) * p.batch + b) * 2 + isC) * p.N + n) * p.L + t0 + tt] = sdBC[(isC * NP + n) * T + tt];
        }
    };

    // ================================================================ pipeline
    // period i: walkers walk tile i (buffer i % 2); helpers finish tile i-1 and stage
    // tile i+1 (both buffer (i+1) % 2), then prefetch tile i+2.  The two roles run
    // separate loops with the same number of barriers, so neither keeps the other's
    // registers live.
    if (walker) {
        load_ck(kt_of(0));
        __syncthreads();
        for (int i = 0; i <= ntiles; ++i) {
            if (i < ntiles) {
                // checkpoint entries of absent channels and padding entries are not
                // used (they may hold anything when the checkpoints come from the caller)
#pragma unroll
                for (int j = 0; j < SPL; ++j) hst[j] = ck_ok[j] ? ckn[j] : 0.0f;
                if (i + 1 < ntiles) load_ck(kt_of(i + 1));
                if constexpr (kGrouped) walk_grouped(buf(i & 1));
                else walk(buf(i & 1));
            }
            __syncthreads();
        }
    } else {
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        issue_loads(kt_of(0));
        stage(kt_of(0), P0{});
        if (ntiles > 1) issue_loads(kt_of(1));
        __syncthreads();
        auto period = [&](int i, auto par) {
            using Q = std::integral_constant<int, 1 - decltype(par)::value>;
            if (i >= 1) finish(kt_of(i - 1), Q{});
            if (i + 1 < ntiles) {
                stage(kt_of(i + 1), Q{});
                if (i + 2 < ntiles) issue_loads(kt_of(i + 2));
            }
            __syncthreads();
        };
        for (int i = 0; i <= ntiles; i += 2) {
            period(i, P0{});
            if (i + 1 <= ntiles) period(i + 1, P1{});
        }
    }

    // ================================================================ results
    if (walker && lane_ok) {
        float* pa = p.pA + ((int64_t(piece) * p.batch + b) * p.dim + dch) * NP + int64_t(wv) * SPL;
#pragma unroll
        for (int j = 0; j < SPL; ++j) pa[j] = dAacc[j];
        if (piece == 0 && p.dh0) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const int64_t n = int64_t(wv) * SPL + j;
                if (n < p.N) p.dh0[(int64_t(b) * p.dim + dch) * p.N + n] = e[j];
            }
        }
    }
    // per-channel sums of the helper threads of a channel, in step-segment order
    float* fin = smem;   // [2][H][64]
    if (!walker) {
        fin[e_seg * kLanes + lane] = accD;
        fin[(H + e_seg) * kLanes + lane] = accBias;
    }
    __syncthreads();
    if (tid < kLanes && c0 + tid < p.dim) {
        float sd = 0.0f, sb = 0.0f;
#pragma unroll
        for (int sg = 0; sg < H; ++sg) {
            sd += fin[sg * kLanes + tid];
            sb += fin[(H + sg) * kLanes + tid];
        }
        const int64_t o = (int64_t(piece) * p.batch + b) * p.dim + c0 + tid;
        p.pD[o] = sd;
        p.pbias[o] = sb;
    }
}

// ---------------------------------------------------------------- checkpoint pass with
// separate roles (16 state entries per channel): four walking waves (4 entries per
// lane) walk 32-step tiles forward and write the state at the start of every 16-step
// tile of the gradient pass, while four helper waves stage the next tile's step sizes,
// weighted inputs and B.  Tiles are double-buffered in LDS, one barrier per tile.
// Shapes: SPL = 4, G = 4 (9..16 entries, checkpoints every 16 steps) and SPL = 16,
// G = 8 (65..128 entries with scalar decay, every 8 steps); 32-step tiles.
template <int SPL_, int G_, int TC_> struct WscShape {
    static constexpr int SPL = SPL_, G = G_, H = 4, T = 32, TC = TC_, NP = G * SPL, EPT = T / H, NTH = H * kLanes;
    static constexpr int kRowB = NP + 4;       // B row stride (floats): 16-byte aligned, few bank conflicts
    static constexpr int kX = T * kLanes * 2;  // (dt2 or the scalar decay, dt2*u) per step and channel
    static constexpr int kB = T * kRowB;       // B*ln2 per step and entry
    static constexpr int kBuf = kX + kB;
    static constexpr int kThreads = (G + H) * kLanes;
    static constexpr size_t kLdsBytes = size_t(2 * kBuf) * sizeof(float);
    static constexpr int KB = (T * NP + NTH - 1) / NTH;
};
namespace wsc {
using Shape = WscShape<4, 4, 16>;
constexpr int EPT = Shape::EPT, NP = Shape::NP;
}  // namespace wsc
namespace wscw {
using Shape = WscShape<16, 8, 8>;
}  // namespace wscw

template <typename IO, bool SCALAR, bool VEC, int SPL_, int G_, int TC_>
__global__ void __launch_bounds__((WscShape<SPL_, G_, TC_>::kThreads)) scan_bwd_ckpt_ws_kernel(BwdParams p) {
    using S = WscShape<SPL_, G_, TC_>;
    constexpr int SPL = S::SPL, G = S::G, T = S::T, TC = S::TC, NP = S::NP, EPT = S::EPT, NTH = S::NTH;
    constexpr int kRowB = S::kRowB, kX = S::kX, kBuf = S::kBuf, KB = S::KB;
    constexpr int NQ = SPL / 4;   // float4 B reads per step
    static_assert(SPL % 4 == 0, "B is read 4 entries at a time");
    static_assert(KB * NTH == T * NP, "the tile's B values must split evenly over the helpers");
    static_assert(T % TC == 0, "checkpoint tiles must nest in walk tiles");
    extern __shared__ float smem[];
    const int tid = threadIdx.x;
    const int wv = tid / kLanes;
    const int lane = tid % kLanes;
    const bool walker = wv < G;
    const int64_t bid = blockIdx.x;
    const int cblk = int(bid % p.nblk_d);
    const int b = int((bid / p.nblk_d) % p.batch);
    const int piece = int(bid / (int64_t(p.nblk_d) * p.batch)) + p.piece_base;
    const int64_t blk = int64_t(b) * p.nblk_d + cblk;
    const int64_t c0 = int64_t(cblk) * kLanes;
    const int64_t tbeg = int64_t(piece) * p.chunk_len;
    const int64_t tend = (tbeg + p.chunk_len < p.L) ? tbeg + p.chunk_len : p.L;
    const int ntiles = int((tend - tbeg + T - 1) / T);
    auto buf = [&](int par) { return smem + par * kBuf; };

    if (walker) {
        const int64_t dch = c0 + lane;
        const bool lane_ok = dch < p.dim;
        float Ar[SPL], h[SPL];
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const int64_t n = int64_t(wv) * SPL + j;
            Ar[j] = 0.0f;
            h[j] = 0.0f;
            if (lane_ok) {
                if constexpr (SCALAR) Ar[j] = p.A[dch / p.head_dim];
                else if (n < p.N) Ar[j] = p.A[dch * p.N + n];
            }
        }
        if (p.nchunks > 1) {
            const int64_t sb = ((blk * p.nchunks + piece) * NP + int64_t(wv) * SPL) * kLanes + lane;
#pragma unroll
            for (int j = 0; j < SPL; ++j) h[j] = p.fHin[sb + int64_t(j) * kLanes];
        } else if (p.h0 && lane_ok) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const int64_t n = int64_t(wv) * SPL + j;
                if (n < p.N) h[j] = p.h0[(int64_t(b) * p.dim + dch) * p.N + n];
            }
        }
        __syncthreads();
        for (int i = 0; i < ntiles; ++i) {
            const float* bf = buf(i & 1);
            const float2* sx = reinterpret_cast<const float2*>(bf) + lane;
            const float4* sb4 = reinterpret_cast<const float4*>(bf + kX + wv * SPL);
            const int64_t t0 = tbeg + int64_t(i) * T;
            float2 xc = sx[0], xn;
            float4 bc[NQ], bn[NQ];
#pragma unroll
            for (int k = 0; k < NQ; ++k) bc[k] = sb4[k];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                if (t % TC == 0 && t0 + t < tend) {
                    float* ck = p.ck + ((blk * p.ntiles_seq + (t0 + t) / TC) * NP + int64_t(wv) * SPL) * kLanes + lane;
#pragma unroll
                    for (int j = 0; j < SPL; ++j) ck[int64_t(j) * kLanes] = h[j];
                }
                if (t + 1 < T) {
                    xn = sx[(t + 1) * kLanes];
#pragma unroll
                    for (int k = 0; k < NQ; ++k) bn[k] = sb4[(t + 1) * (kRowB / 4) + k];
                }
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const float4 q = bc[j / 4];
                    const float bj = (j % 4 == 0) ? q.x : (j % 4 == 1) ? q.y : (j % 4 == 2) ? q.z : q.w;
                    const float a = SCALAR ? xc.x : __builtin_amdgcn_exp2f(xc.x * Ar[j]);
                    h[j] = fmaf(a, h[j], xc.y * bj);
                }
                xc = xn;
#pragma unroll
                for (int k = 0; k < NQ; ++k) bc[k] = bn[k];
            }
            __syncthreads();
        }
    } else {
        const int e_seg = wv - G;
        const int ht = tid - G * kLanes;
        const int64_t e_d = c0 + lane;
        const bool e_ok = e_d < p.dim;
        const float e_bias = (e_ok && p.bias) ? p.bias[e_d] : 0.0f;
        const float e_ah = (SCALAR && e_ok) ? p.A[e_d / p.head_dim] : 0.0f;
        const int64_t e_row = (int64_t(b) * p.dim + (e_ok ? e_d : 0)) * p.L;
        const IO* __restrict__ gu = static_cast<const IO*>(p.u);
        const IO* __restrict__ gdl = static_cast<const IO*>(p.delta);
        const IO* __restrict__ gB = static_cast<const IO*>(p.Bm);
        // B value v = ht + k*NTH -> (entry n, step t of the tile)
        const IO* bp[KB];
        int bslot[KB], bt[KB];
        bool bok[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int v = ht + k * NTH;
            const int n = v / T;
            bt[k] = v % T;
            bok[k] = n < p.N;
            bp[k] = gB + (int64_t(b) * p.N + (bok[k] ? n : 0)) * p.L + bt[k];
            bslot[k] = bt[k] * kRowB + n;
        }
        InSeg<IO, EPT, VEC> nu, ndl;
        IO nb[KB];
        auto issue_loads = [&](int kt) {
            const int64_t t0 = tbeg + int64_t(kt) * T;
            const int64_t t = t0 + e_seg * EPT;
            nu = load_seg<IO, EPT, VEC>(gu + e_row, t, tend, e_ok);
            ndl = load_seg<IO, EPT, VEC>(gdl + e_row, t, tend, e_ok);
#pragma unroll
            for (int k = 0; k < KB; ++k) nb[k] = *((bok[k] && t0 + bt[k] < tend) ? bp[k] + t0 : gB);
        };
        // steps beyond the piece's end are identity steps (decay 1, input 0)
        auto stage = [&](int kt) {
            float* bf = buf(kt & 1);
            const int64_t t0 = tbeg + int64_t(kt) * T;
            float2* sx = reinterpret_cast<float2*>(bf);
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const int tl = e_seg * EPT + k;
                const bool in = e_ok && t0 + tl < tend;
                const float uu = in ? nu.get(k) : 0.0f;
                const float r = in ? ndl.get(k) + e_bias : 0.0f;
                const float dt2 = in ? softplus_log2(r) : 0.0f;
                const float first = SCALAR ? __builtin_amdgcn_exp2f(dt2 * e_ah) : dt2;
                sx[tl * kLanes + lane] = make_float2(first, dt2 * uu);
            }
            float* sB = bf + kX;
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const bool in = bok[k] && t0 + bt[k] < tend;
                sB[bslot[k]] = in ? IOT<IO>::to_f32(nb[k]) * kLn2 : 0.0f;
            }
        };
        issue_loads(0);
        stage(0);
        if (ntiles > 1) issue_loads(1);
        __syncthreads();
        for (int i = 0; i < ntiles; ++i) {
            if (i + 1 < ntiles) {
                stage(i + 1);
                if (i + 2 < ntiles) issue_loads(i + 2);
            }
            __syncthreads();
        }
    }
}

// Piece carries, one thread per (group, state entry, lane), in sequence order:
//   forward:  Hin[0] = h0 (or 0),     Hin[c+1] = exp2(A*S[c]) Hin[c] + H[c]
//   reverse:  Ein[P-1] = dh_last (or 0), Ein[c-1] = exp2(A*S[c]) Ein[c] + G[c]
__global__ void __launch_bounds__(256) bwd_carry_kernel(BwdParams p, int64_t total, int reverse) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int lane = int(i % kLanes);
    const int64_t n = (i / kLanes) % p.np;
    const int64_t blk = i / (int64_t(kLanes) * p.np);
    const int64_t d = (blk % p.nblk_d) * kLanes + lane;
    const int64_t b = blk / p.nblk_d;
    const bool ok = d < p.dim && n < p.N;
    const float a = ok ? (p.head_dim ? p.A[d / p.head_dim] : p.A[d * p.N + n]) : 0.0f;
    const int P = p.nchunks;
    auto at = [&](int c) { return ((blk * P + c) * p.np + n) * kLanes + lane; };
    float cur = 0.0f;
    if (!reverse) {
        if (ok && p.h0) cur = p.h0[(b * p.dim + d) * p.N + n];
        for (int c = 0; c < P; ++c) {
            p.fHin[at(c)] = cur;
            if (c + 1 < P) cur = fmaf(__builtin_amdgcn_exp2f(a * p.fS[(blk * P + c) * kLanes + lane]), cur, p.fH[at(c)]);
        }
    } else {
        if (ok && p.dh_last) cur = p.dh_last[(b * p.dim + d) * p.N + n];
        for (int c = P - 1; c >= 0; --c) {
            p.rEin[at(c)] = cur;
            if (c > 0) cur = fmaf(__builtin_amdgcn_exp2f(a * p.rS[(blk * P + c) * kLanes + lane]), cur, p.rG[at(c)]);
        }
    }
}

// dB[b,n,t] = ln2 * sum over channel blocks, dC likewise unscaled; one thread per output.
__global__ void __launch_bounds__(256) bwd_reduce_bc_kernel(BwdParams p, float* dB, float* dC, int64_t total) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t t = i % p.L;
    int64_t r = i / p.L;
    const int64_t n = r % p.N;
    r /= p.N;
    const int isC = int(r % 2);
    const int64_t b = r / 2;
    const int64_t stride = int64_t(p.batch) * 2 * p.N * p.L;
    const float* src = p.pBC + ((b * 2 + isC) * p.N + n) * p.L + t;
    float sum = 0.0f;
    for (int cb = 0; cb < p.nblk_d; ++cb) sum += src[cb * stride];
    (isC ? dC : dB)[(b * p.N + n) * p.L + t] = isC ? sum : sum * kLn2;
}

// Diagonal A: dA[d,n] = ln2 * sum over pieces and batch rows.  Also dD and ddt_bias
// (threads with d < dim, n == 0).
__global__ void __launch_bounds__(256) bwd_reduce_param_kernel(BwdParams p, float* dA, float* dD, float* dbias,
                                                               int64_t total) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t d = i / p.N, n = i % p.N;
    const int64_t rows = int64_t(p.nchunks) * p.batch;
    if (dA) {
        float s = 0.0f;
        for (int64_t r = 0; r < rows; ++r) s += p.pA[(r * p.dim + d) * p.np + n];
        dA[d * p.N + n] = s * kLn2;
    }
    if (n == 0) {
        float sd = 0.0f, sb = 0.0f;
        for (int64_t r = 0; r < rows; ++r) {
            sd += p.pD[r * p.dim + d];
            sb += p.pbias[r * p.dim + d];
        }
        if (dD) dD[d] = sd;
        if (dbias) dbias[d] = sb;
    }
}

// Scalar decay: dA[h] = ln2 * sum over pieces, batch rows, the head's channels and
// the state entries; one workgroup per head, fixed-order tree.
__global__ void __launch_bounds__(256) bwd_reduce_heads_kernel(BwdParams p, float* dA) {
    __shared__ float part[256];
    const int64_t hd = blockIdx.x;
    const int64_t per_row = p.head_dim * p.N;
    const int64_t total = int64_t(p.nchunks) * p.batch * per_row;
    float s = 0.0f;
    for (int64_t k = threadIdx.x; k < total; k += 256) {
        const int64_t r = k / per_row, q = k % per_row;
        const int64_t d = hd * p.head_dim + q / p.N, n = q % p.N;
        s += p.pA[(r * p.dim + d) * p.np + n];
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (int(threadIdx.x) < off) part[threadIdx.x] += part[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) dA[hd] = part[0] * kLn2;
}

// ------------------------------------------------------------------ host side
struct BwdPlan {
    int spl, G, nch, T;
    bool ws;       // gradient pass with separate walking and helper waves (9..16 entries)
    bool ws_wide;  // the same for 65..128 entries with scalar decay
    int64_t chunk_len, nblk_d, groups, ntiles_seq;
    size_t off_ck, off_bc, off_a, off_d, off_bias, off_fh, off_fs, off_fhin, off_rg, off_rs, off_rein, ws_bytes;
    size_t lds_grad, lds_fwd;
};

inline size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int make_bwd_plan(const ssm_dims* d, BwdPlan* pl) {
    int st = validate_dims(d);
    if (st != SSM_OK) return st;
    const int64_t N = d->dstate;
    if (N > SSM_MAX_DSTATE_BWD) return SSM_ERR_DIMS;
    int spl = d->states_per_lane;
    if (spl == 0) {
        // The gradient walk keeps a tile's recomputed states in VGPRs (16 steps x SPL
        // per lane) next to the staging and finishing registers, so few entries per
        // lane keep the kernel at two waves per SIMD without spills: up to 8 waves
        // of 2 entries for N <= 16, then more entries per lane at 8 waves.
        if (N <= 4) spl = 1;
        else if (N <= 16) spl = 2;
        else if (N <= 32) spl = 4;
        else if (N <= 64) spl = 8;
        else spl = 16;
    }
    const int64_t g = cdiv(N, spl);
    if (g > 8) return SSM_ERR_DIMS;
    pl->spl = spl;
    pl->G = g <= 4 ? 4 : 8;
    if ((pl->G == 4 && spl > 4) || (pl->G == 8 && spl < 2)) return SSM_ERR_DIMS;   // no such kernel
    const int np = pl->G * spl;
    pl->nblk_d = cdiv(d->dim, kLanes);
    pl->groups = d->batch * pl->nblk_d;
    const int T = bwd_tile(np);
    pl->T = T;
    pl->ntiles_seq = cdiv(d->seqlen, T);
    int64_t nch = d->nchunks;
    const bool ws = spl == 2 && pl->G == 8;   // role-split checkpoint and gradient passes
    if (nch == 0) {
        // Pieces cost a forward and a reverse aggregate walk each, keeping >= 8 tiles
        // per piece.  Role-split passes (one workgroup per CU): cut only when fewer
        // than half the CUs would get a workgroup, then aim for ~1024 workgroups
        // (measured: 1.3B-layer shapes at 192 groups 0.68 ms uncut against 0.89 ms in
        // 2 pieces; the long sequence at 32 groups 7.6 ms in 32 pieces, 9.1 ms in 8).
        // Otherwise below two waves per SIMD the sequence is cut.
        const int64_t waves = pl->groups * pl->G;
        if (ws)
            nch = pl->groups < 128 ? cdiv(1024, pl->groups) : 1;
        else
            nch = waves < 2048 ? cdiv(2048, waves) : 1;
        const int64_t max_pieces = pl->ntiles_seq / 8 > 1 ? pl->ntiles_seq / 8 : 1;
        // then the piece count, up to twice that, that leaves no part-filled last round
        // of gradient-pass workgroups
        const bool wide = spl == 16 && pl->G == 8 && d->nheads > 0;
        const size_t lds = ws ? wsg::Shape::kLdsBytes
                              : wide ? wsw::Shape::kLdsBytes : bwd_lds_floats(pl->G, spl, kGrad) * sizeof(float);
        const int64_t per_cu = int64_t(163840 / lds);
        const int64_t cap = max_pieces < SSM_MAX_CHUNKS ? max_pieces : SSM_MAX_CHUNKS;
        nch = round_friendly_pieces(pl->groups, nch, cap, 256 * (per_cu > 1 ? per_cu : 1));
        if (nch > max_pieces) nch = max_pieces;
        if (nch > SSM_MAX_CHUNKS) nch = SSM_MAX_CHUNKS;
    }
    if (nch > pl->ntiles_seq) nch = pl->ntiles_seq;
    if (nch < 1) nch = 1;
    pl->chunk_len = cdiv(pl->ntiles_seq, nch) * T;
    pl->nch = int(cdiv(d->seqlen, pl->chunk_len));
    if (pl->groups * pl->nch > 0x7fffffffLL) return SSM_ERR_DIMS;
    const size_t f = sizeof(float);
    size_t off = 0;
    pl->off_ck = off;
    off += round256(size_t(pl->groups) * pl->ntiles_seq * np * kLanes * f);
    pl->off_bc = off;
    off += round256(size_t(pl->nblk_d) * d->batch * 2 * N * d->seqlen * f);
    pl->off_a = off;
    off += round256(size_t(pl->nch) * d->batch * d->dim * np * f);
    pl->off_d = off;
    off += round256(size_t(pl->nch) * d->batch * d->dim * f);
    pl->off_bias = off;
    off += round256(size_t(pl->nch) * d->batch * d->dim * f);
    const size_t st_bytes = round256(size_t(pl->groups) * pl->nch * np * kLanes * f);
    const size_t s_bytes = round256(size_t(pl->groups) * pl->nch * kLanes * f);
    pl->off_fh = pl->off_fs = pl->off_fhin = pl->off_rg = pl->off_rs = pl->off_rein = 0;
    if (pl->nch > 1) {
        pl->off_fh = off;
        off += st_bytes;
        pl->off_fs = off;
        off += s_bytes;
        pl->off_fhin = off;
        off += st_bytes;
        pl->off_rg = off;
        off += st_bytes;
        pl->off_rs = off;
        off += s_bytes;
        pl->off_rein = off;
        off += st_bytes;
    }
    pl->ws_bytes = off;
    static_assert(wsg::T == bwd_tile(wsg::NP), "both gradient kernels read the same checkpoints");
    pl->ws = ws;
    pl->ws_wide = spl == 16 && pl->G == 8 && d->nheads > 0;
    static_assert(wsw::Shape::T == bwd_tile(wsw::Shape::NP), "both gradient kernels read the same checkpoints");
    pl->lds_grad = pl->ws ? wsg::Shape::kLdsBytes
                          : pl->ws_wide ? wsw::Shape::kLdsBytes : bwd_lds_floats(pl->G, spl, kGrad) * f;
    pl->lds_fwd = bwd_lds_floats(pl->G, spl, kCkpt) * f;
    return SSM_OK;
}

// ext_ck: the checkpoints at p.ck come from the caller (the forward kept them), so the
// forward aggregate, the forward carry and the checkpoint pass are skipped.
template <typename IO, int SPL, int G, bool SCALAR, bool VEC>
hipError_t bwd_launch(BwdParams p, const BwdPlan& pl, bool vec_g, bool vec_c, bool ext_ck, float* dA, float* dB,
                      float* dC, float* dD, float* dbias, hipStream_t s) {
    const dim3 block(unsigned(G * kLanes));
    const int64_t groups = pl.groups;
    if (pl.nch > 1) {
        const dim3 grid1(unsigned(groups * (pl.nch - 1)));
        bool mfma_fwd = false, mfma_rev = false;
        if (p.mfma_agg) {
            ssm_detail::PieceStatesArgs a;
            a.delta = p.delta;
            a.A = p.A;
            a.bias = p.bias;
            a.L = p.L;
            a.dim = p.dim;
            a.nstate = p.N;
            a.head_dim = p.head_dim;
            a.chunk_len = p.chunk_len;
            a.nchunks = p.nchunks;
            a.nblk_d = p.nblk_d;
            a.batch = p.batch;
            if (!ext_ck) {
                a.x = p.u;
                a.z = nullptr;
                a.BC = p.Bm;
                a.piece_base = 0;
                a.H = p.fH;
                a.S = p.fS;
                mfma_fwd = ssm_detail::launch_piece_states(a, false, pl.nch - 1, s);
            }
            a.x = p.dy;
            a.z = p.z;
            a.BC = p.Cm;
            a.piece_base = 1;
            a.H = p.rG;
            a.S = p.rS;
            mfma_rev = ssm_detail::launch_piece_states(a, true, pl.nch - 1, s);
        }
        p.piece_base = 0;
        if (!ext_ck && !mfma_fwd)
            launch_kernel((scan_bwd_kernel<IO, SPL, G, SCALAR, kFwdAgg, VEC>), grid1, block, pl.lds_fwd, s, p);
        p.piece_base = 1;
        if (!mfma_rev)
            launch_kernel((scan_bwd_kernel<IO, SPL, G, SCALAR, kRevAgg, VEC>), grid1, block, pl.lds_fwd, s, p);
        p.piece_base = 0;
        const int64_t total = groups * p.np * kLanes;
        const dim3 gridc(unsigned(cdiv(total, 256)));
        if (!ext_ck) launch_kernel(bwd_carry_kernel, gridc, dim3(256), 0, s, p, total, 0);
        launch_kernel(bwd_carry_kernel, gridc, dim3(256), 0, s, p, total, 1);
    }
    p.piece_base = 0;
    const dim3 grid(unsigned(groups * pl.nch));
    if (ext_ck) {
        // nothing to recompute
    } else if constexpr (SPL == wsc::NP / G && G == 8) {
        const dim3 blk_c(static_cast<unsigned>(wsc::Shape::kThreads), 1, 1);
        if (vec_c)
            launch_kernel((scan_bwd_ckpt_ws_kernel<IO, SCALAR, true, 4, 4, 16>), grid, blk_c, wsc::Shape::kLdsBytes, s, p);
        else
            launch_kernel((scan_bwd_ckpt_ws_kernel<IO, SCALAR, false, 4, 4, 16>), grid, blk_c, wsc::Shape::kLdsBytes, s, p);
    } else if constexpr (SPL == 16 && G == 8 && SCALAR) {
        const dim3 blk_c(static_cast<unsigned>(wscw::Shape::kThreads), 1, 1);
        if (vec_c)
            launch_kernel((scan_bwd_ckpt_ws_kernel<IO, SCALAR, true, 16, 8, 8>), grid, blk_c, wscw::Shape::kLdsBytes, s, p);
        else
            launch_kernel((scan_bwd_ckpt_ws_kernel<IO, SCALAR, false, 16, 8, 8>), grid, blk_c, wscw::Shape::kLdsBytes, s, p);
    } else {
        launch_kernel((scan_bwd_kernel<IO, SPL, G, SCALAR, kCkpt, VEC>), grid, block, pl.lds_fwd, s, p);
    }
    if constexpr (SPL == wsg::NP / G && G == 8) {
        const dim3 blk_ws(static_cast<unsigned>(wsg::Shape::kThreads), 1, 1);
        if (vec_g)
            launch_kernel((scan_bwd_grad_ws_kernel<IO, SCALAR, true, 4, 4, 16>), grid, blk_ws, pl.lds_grad, s, p);
        else
            launch_kernel((scan_bwd_grad_ws_kernel<IO, SCALAR, false, 4, 4, 16>), grid, blk_ws, pl.lds_grad, s, p);
    } else if constexpr (SPL == 16 && G == 8 && SCALAR) {
        const dim3 blk_ws(static_cast<unsigned>(wsw::Shape::kThreads), 1, 1);
        if (vec_g)
            launch_kernel((scan_bwd_grad_ws_kernel<IO, SCALAR, true, 16, 8, 8>), grid, blk_ws, pl.lds_grad, s, p);
        else
            launch_kernel((scan_bwd_grad_ws_kernel<IO, SCALAR, false, 16, 8, 8>), grid, blk_ws, pl.lds_grad, s, p);
    } else {
        launch_kernel((scan_bwd_kernel<IO, SPL, G, SCALAR, kGrad, VEC>), grid, block, pl.lds_grad, s, p);
    }
    const int64_t nbc = int64_t(p.batch) * 2 * p.N * p.L;
    launch_kernel(bwd_reduce_bc_kernel, dim3(unsigned(cdiv(nbc, 256))), dim3(256), 0, s, p, dB, dC, nbc);
    const int64_t npar = p.dim * p.N;
    launch_kernel(bwd_reduce_param_kernel, dim3(unsigned(cdiv(npar, 256))), dim3(256), 0, s, p,
                       SCALAR ? nullptr : dA, dD, dbias, npar);
    if (SCALAR) {
        const int64_t nheads = p.dim / p.head_dim;
        launch_kernel(bwd_reduce_heads_kernel, dim3(unsigned(nheads)), dim3(256), 0, s, p, dA);
    }
    return ssm_detail::launch_error;
}

// The (entries per lane, waves) pairs the planner produces: 1..4 entries with 4 waves
// (dstate <= 16, or forced), and 2..16 entries with 8 waves.
template <typename IO, bool SCALAR, bool VEC>
hipError_t bwd_dispatch_vec(const BwdParams& p, const BwdPlan& pl, bool vec_g, bool vec_c, bool ext_ck, float* dA,
                            float* dB, float* dC, float* dD, float* dbias, hipStream_t s) {
#define SSM_BWD_CASE(S_, G_)                                                                               \
    if (pl.spl == S_ && pl.G == G_)                                                                        \
        return bwd_launch<IO, S_, G_, SCALAR, VEC>(p, pl, vec_g, vec_c, ext_ck, dA, dB, dC, dD, dbias, s);
    SSM_BWD_CASE(1, 4)
    SSM_BWD_CASE(2, 4)
    SSM_BWD_CASE(4, 4)
    SSM_BWD_CASE(2, 8)
    SSM_BWD_CASE(4, 8)
    SSM_BWD_CASE(8, 8)
    SSM_BWD_CASE(16, 8)
#undef SSM_BWD_CASE
    return hipErrorInvalidConfiguration;
}

template <typename IO, bool SCALAR>
hipError_t bwd_dispatch(const BwdParams& p, const BwdPlan& pl, bool vec, bool vec_g, bool vec_c, bool ext_ck,
                        float* dA, float* dB, float* dC, float* dD, float* dbias, hipStream_t s) {
    return vec ? bwd_dispatch_vec<IO, SCALAR, true>(p, pl, vec_g, vec_c, ext_ck, dA, dB, dC, dD, dbias, s)
               : bwd_dispatch_vec<IO, SCALAR, false>(p, pl, vec_g, vec_c, ext_ck, dA, dB, dC, dD, dbias, s);
}

}  // namespace

// ------------------------------------------------------------------ C ABI
extern "C" {

size_t ssm_selective_scan_bwd_workspace_bytes(const ssm_dims* dims) {
    BwdPlan pl;
    if (make_bwd_plan(dims, &pl) != SSM_OK) return 0;
    return pl.ws_bytes;
}

int ssm_selective_scan_bwd_plan(const ssm_dims* dims, ssm_plan* plan) {
    if (!plan) return SSM_ERR_NULL;
    BwdPlan pl;
    const int st = make_bwd_plan(dims, &pl);
    if (st != SSM_OK) return st;
    plan->nchunks = pl.nch;
    plan->states_per_lane = pl.spl;
    plan->waves_per_group = pl.G;
    plan->time_tile = pl.T;
    plan->chunk_len = pl.chunk_len;
    plan->workgroups = pl.groups * pl.nch;
    plan->workspace_bytes = pl.ws_bytes;
    plan->lds_bytes = pl.lds_grad;
    plan->form = 0;
    plan->reserved = 0;
    return SSM_OK;
}

}  // extern "C"

namespace {

int bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
             const void* z, const float* dt_bias, const float* h0, const void* dy, const float* dh_last,
             const ssm_grads* grads, const ssm_dims* dims, void* stream, bool with_ckpt, const float* ckpt) {
    if (!dims || !grads) return SSM_ERR_NULL;
    BwdPlan pl;
    int st = make_bwd_plan(dims, &pl);
    if (st != SSM_OK) return st;
    if (with_ckpt && (ssm_selective_scan_ckpt_bytes(dims) == 0 || !pl.ws)) return SSM_ERR_DIMS;
    if (!u || !delta || !A || !B || !C || !dy || !grads->du || !grads->ddelta || !grads->dA || !grads->dB ||
        !grads->dC || (with_ckpt && !ckpt))
        return SSM_ERR_NULL;
    void* dz = z ? grads->dz : nullptr;
    const size_t esz = dims->io_dtype == SSM_BF16 ? 2 : 4;
    if (misaligned(u, esz) || misaligned(delta, esz) || misaligned(z, esz) || misaligned(B, esz) ||
        misaligned(C, esz) || misaligned(dy, esz) || misaligned(grads->du, esz) || misaligned(grads->ddelta, esz) ||
        misaligned(dz, esz) || misaligned(A, 4) || misaligned(D, 4) || misaligned(dt_bias, 4) ||
        misaligned(h0, 4) || misaligned(dh_last, 4) || misaligned(grads->dA, 4) || misaligned(grads->dB, 4) ||
        misaligned(grads->dC, 4) || misaligned(grads->dD, 4) || misaligned(grads->ddt_bias, 4) ||
        misaligned(grads->dh0, 4) || misaligned(ckpt, 4))
        return SSM_ERR_ALIGN;

    const size_t nel = size_t(dims->batch) * dims->dim * dims->seqlen * esz;
    const size_t nbc = size_t(dims->batch) * dims->dstate * dims->seqlen * esz;
    const size_t nbc4 = size_t(dims->batch) * dims->dstate * dims->seqlen * 4;
    const size_t na = (dims->nheads > 0 ? size_t(dims->nheads) : size_t(dims->dim) * dims->dstate) * 4;
    const size_t nd = size_t(dims->dim) * 4;
    const size_t nh = size_t(dims->batch) * dims->dim * dims->dstate * 4;
    const size_t nck = with_ckpt ? ssm_selective_scan_ckpt_bytes(dims) : 0;
    const void* ins[] = {u, delta, z, B, C, A, D, dt_bias, h0, dy, dh_last, with_ckpt ? ckpt : nullptr};
    const size_t in_sz[] = {nel, nel, nel, nbc, nbc, na, nd, nd, nh, nel, nh, nck};
    const void* outs[] = {grads->du, grads->ddelta, dz, grads->dA, grads->dB, grads->dC, grads->dD,
                          grads->ddt_bias, grads->dh0, dims->workspace};
    const size_t out_sz[] = {nel, nel, nel, na, nbc4, nbc4, nd, nd, nh, pl.ws_bytes};
    constexpr int kIn = 12, kOut = 10;
    for (int i = 0; i < kOut; ++i) {
        for (int k = 0; k < kIn; ++k)
            if (overlaps(outs[i], out_sz[i], ins[k], in_sz[k])) return SSM_ERR_ALIAS;
        for (int k = i + 1; k < kOut; ++k)
            if (overlaps(outs[i], out_sz[i], outs[k], out_sz[k])) return SSM_ERR_ALIAS;
    }
    if (!dims->workspace || dims->workspace_bytes < pl.ws_bytes ||
        (reinterpret_cast<uintptr_t>(dims->workspace) % 256) != 0)
        return SSM_ERR_WORKSPACE;

    // each thread moves ept consecutive elements of a row at once when the rows allow
    // it: T/G in the aggregate passes (and the checkpoint and gradient passes without
    // helper waves); 4 in the gradient pass and 8 in the checkpoint pass with helpers
    auto rows_allow = [&](int64_t ept) {
        const size_t seg = size_t(ept) * esz;
        auto aligned = [seg](const void* q) { return !q || (reinterpret_cast<uintptr_t>(q) % seg) == 0; };
        return (dims->seqlen % ept) == 0 && aligned(u) && aligned(delta) && aligned(z) && aligned(dy) &&
               aligned(grads->du) && aligned(grads->ddelta) && aligned(dz);
    };
    const bool vec = rows_allow(pl.T / pl.G);
    const bool vec_g = pl.ws ? rows_allow(wsg::EPT) : pl.ws_wide ? rows_allow(wsw::Shape::EPT) : vec;
    const bool vec_c = pl.ws ? rows_allow(wsc::EPT) : pl.ws_wide ? rows_allow(wscw::Shape::EPT) : vec;

    BwdParams p;
    p.u = u;
    p.delta = delta;
    p.z = z;
    p.Bm = B;
    p.Cm = C;
    p.A = A;
    p.Dskip = D;
    p.bias = dt_bias;
    p.h0 = h0;
    p.dy = dy;
    p.dh_last = dh_last;
    p.du = grads->du;
    p.ddelta = grads->ddelta;
    p.dz = dz;
    p.dh0 = grads->dh0;
    p.L = dims->seqlen;
    p.dim = dims->dim;
    p.N = dims->dstate;
    p.head_dim = dims->nheads > 0 ? dims->dim / dims->nheads : 0;
    p.chunk_len = pl.chunk_len;
    p.ntiles_seq = pl.ntiles_seq;
    p.nchunks = pl.nch;
    p.nblk_d = int32_t(pl.nblk_d);
    p.batch = int32_t(dims->batch);
    p.np = pl.G * pl.spl;
    p.piece_base = 0;
    {
        auto a16 = [](const void* q) { return !q || (reinterpret_cast<uintptr_t>(q) % 16) == 0; };
        const int64_t N = dims->dstate;
        p.mfma_agg = dims->nheads > 0 && dims->io_dtype == SSM_BF16 && p.np == N &&
                     (N == 32 || N == 64 || N == 128) && dims->seqlen % 8 == 0 && a16(u) && a16(delta) &&
                     a16(z) && a16(dy) && a16(B) && a16(C);
    }
    char* ws = static_cast<char*>(dims->workspace);
    auto at = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
    p.ck = with_ckpt ? const_cast<float*>(ckpt) : at(pl.off_ck);   // read only when given
    p.pBC = at(pl.off_bc);
    p.pA = at(pl.off_a);
    p.pD = at(pl.off_d);
    p.pbias = at(pl.off_bias);
    p.fH = p.fS = p.fHin = p.rG = p.rS = p.rEin = nullptr;
    if (pl.nch > 1) {
        p.fH = at(pl.off_fh);
        p.fS = at(pl.off_fs);
        p.fHin = at(pl.off_fhin);
        p.rG = at(pl.off_rg);
        p.rS = at(pl.off_rs);
        p.rEin = at(pl.off_rein);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    ssm_detail::launch_error = hipSuccess;   // this call's launch failures only (the caller's pending HIP error is left alone)
    const bool scalar = dims->nheads > 0;
    hipError_t e;
    if (dims->io_dtype == SSM_BF16)
        e = scalar ? bwd_dispatch<uint16_t, true>(p, pl, vec, vec_g, vec_c, with_ckpt, grads->dA, grads->dB, grads->dC, grads->dD, grads->ddt_bias, s)
                   : bwd_dispatch<uint16_t, false>(p, pl, vec, vec_g, vec_c, with_ckpt, grads->dA, grads->dB, grads->dC, grads->dD, grads->ddt_bias, s);
    else
        e = scalar ? bwd_dispatch<float, true>(p, pl, vec, vec_g, vec_c, with_ckpt, grads->dA, grads->dB, grads->dC, grads->dD, grads->ddt_bias, s)
                   : bwd_dispatch<float, false>(p, pl, vec, vec_g, vec_c, with_ckpt, grads->dA, grads->dB, grads->dC, grads->dD, grads->ddt_bias, s);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* dt_bias, const float* h0, const void* dy,
                           const float* dh_last, const ssm_grads* grads, const ssm_dims* dims, void* stream) {
    return bwd_impl(u, delta, A, B, C, D, z, dt_bias, h0, dy, dh_last, grads, dims, stream, false, nullptr);
}

int ssm_selective_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                const float* D, const void* z, const float* dt_bias, const float* h0, const void* dy,
                                const float* dh_last, const float* ckpt, const ssm_grads* grads, const ssm_dims* dims,
                                void* stream) {
    return bwd_impl(u, delta, A, B, C, D, z, dt_bias, h0, dy, dh_last, grads, dims, stream, true, ckpt);
}

}  // extern "C"
