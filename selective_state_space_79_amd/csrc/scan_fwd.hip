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

#include <mutex>
#include <type_traits>

#include "ssm.h"

#include "scan_common.h"

namespace {

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
    const float* h0;      // nullable: (batch, dim, N) state before the first step
    float* h_last;        // nullable: (batch, dim, N) state after the last step
    float* ws_H;          // [groups][nchunks][np][64] piece end states from zero (pass 1)
    float* ws_S;          // [groups][nchunks][64]     sum of dt2 over each piece (pass 1)
    float* ws_Hin;        // [groups][nchunks][np][64] true starting state of each piece
    // fused front end (conv_w != nullptr): the rows at `u` hold the convolution's input
    // x and the scan's input is u = act(conv_b + sum_k conv_w[d,k] x[t-K+1+k])
    const float* conv_w;     // (dim, conv_k)
    const float* conv_b;     // nullable
    const void* conv_state;  // nullable: (batch, dim, conv_k-1) inputs before the sequence
    void* u_out;             // nullable: u, rounded to the I/O type (full mode)
    int32_t conv_k;          // 1 .. kMaxConv
    int32_t conv_silu;       // 1: SiLU after the convolution
    // state checkpoints (kernels instantiated with checkpoints only, 16 padded state
    // entries): [groups][ntiles_ck][16][64], the state before every 16th step
    float* ckpt;
    int64_t ntiles_ck;       // ceil(L / 16)
};

constexpr int kCkptSteps = 16;   // steps between state checkpoints

enum Mode { kFull = 0, kAggregate = 1 };
constexpr int kMaxConv = 4;   // widest fused convolution: its history fits one 4-element halo

// LDS layout of one tile buffer (floats):
//   sDX [T][kRow] float2  per (step, channel): (dt2, dt2*u), or (exp(dt*a_h), dt2*u) in
//                         scalar-decay full mode; rows padded to kRow so that the
//                         staging writes, whose lanes span several steps of a few
//                         channels, fall in distinct banks
//   sBC [G][T][2*SPL]     per (wave, step): B*ln2 of the wave's SPL state entries, then C
// then, in full mode, the partial read-outs, in one of two layouts:
//   * four walkers of at most 4 entries (two waves per SIMD: yswizzled):
//     sY [T][G][64]       per (step, wave, channel).  Channel c of step t sits in column
//                         c ^ ysw(t), a permutation of the 64 columns per step, so that
//                         the walkers' row writes and the finishing lanes' reads (several
//                         steps of a few channels) each touch 64 distinct banks, and every
//                         row is 256 bytes, so a finishing thread's reads take immediate
//                         offsets from one address.  The skip terms D*u and gates SiLU(z)
//                         stay in the staging thread's registers until it finishes the
//                         same elements.
//   * otherwise, rows padded to kRowY for distinct banks:
//     sY  [G][T][kRowY]   per (wave, step, channel): partial read-out
//     sSk [T][kRowY]      per (step, channel): skip term D*u
//     sGt [T][kRowY]      per (step, channel): gate SiLU(z), or 1 without z
constexpr int kRow = kLanes + 1;
constexpr int kRowY = kLanes + 2;
__host__ __device__ constexpr bool yswizzled(int G, int spl) { return G == 4 && spl <= 4; }
inline size_t lds_floats(int T, int G, int np, bool full) {
    const size_t out = yswizzled(G, np / G) ? size_t(G) * T * kLanes : size_t(G + 2) * T * kRowY;
    return size_t(T) * kRow * 2 + 2 * size_t(T) * np + (full ? out : 0);
}

// Column swizzle of the swizzled sY: steps t of one 16-byte vector (VW steps) share a
// value, and the TV vectors of a tile take distinct multiples of 64 / TV.
template <int T, int VW>
__host__ __device__ constexpr int ysw(int t) {
    return ((t / VW) % (T / VW)) * (kLanes / (T / VW));
}

template <int SPL> struct BCVec { float v[2 * SPL]; };

template <int SPL>
__device__ inline BCVec<SPL> read_bc(const float* __restrict__ q) {
    BCVec<SPL> r;
    if constexpr (SPL == 1) {
        const float2 t = *reinterpret_cast<const float2*>(q);
        r.v[0] = t.x;
        r.v[1] = t.y;
    } else {
#pragma unroll
        for (int i = 0; i < SPL / 2; ++i) {
            const float4 t = reinterpret_cast<const float4*>(q)[i];
            r.v[4 * i + 0] = t.x;
            r.v[4 * i + 1] = t.y;
            r.v[4 * i + 2] = t.z;
            r.v[4 * i + 3] = t.w;
        }
    }
    return r;
}

// Raw buffer windows.  A workgroup addresses each array through a window: a
// workgroup-uniform base, the first byte of the rows it reads (the block's 64 channel
// rows, or the batch row's dstate rows of B or C), and their size in bytes, below 2^31
// (the host takes this path only then), both in scalar registers.  A tile's accesses
// take the window advanced to the tile's first step and a 32-bit lane offset fixed for
// the whole piece; an access at or past the window's end -- every lane offset kOob --
// reads zeros or is dropped.  Word 3 of the descriptor selects 32-bit data, untyped.
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((ext_vector_type(4))) unsigned int bvec4;
constexpr uint32_t kOob = 0x80000000u;
struct Window {
    const char* base;
    uint32_t bytes;
    // the window from `off` bytes on (off < bytes)
    __device__ Rsrc at(uint32_t off) const {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + off), 0, int(bytes - off), 0x00020000);
    }
};

// Kernel shape, by the number G of waves that walk (4, 8 or 16):
//   G <= 8: 4 more "helper" waves stage tile k+1 and finish tile k-1 while the G
//           walkers walk tile k (double-buffered LDS, one barrier per tile), so every
//           SIMD runs a walker and a helper side by side;
//   G == 16: all waves stage, walk and finish in turn (single buffer, 2 barriers).
template <int G, int SPL> struct Shape {
    static constexpr bool kSpec = G <= 8;
    static constexpr int NW = kSpec ? G + 4 : G;          // waves per workgroup
    static constexpr int NS = (kSpec ? 4 : G) * kLanes;    // staging threads
    static constexpr int T = (G == 4 && SPL <= 8) ? 32 : 16;   // time tile (LDS budget)
    static constexpr int NBUF = kSpec ? 2 : 1;
};

inline int tile_len(int G, int spl) { return (G == 4 && spl <= 8) ? 32 : 16; }

inline size_t lds_floats_g(int G, int spl, bool full) {
    return (G <= 8 ? 2 : 1) * lds_floats(tile_len(G, spl), G, G * spl, full);
}

// One launch processes, for every (batch, channel block, piece), the piece's time
// tiles in order.  MODE kFull reads out and stores y (starting from ws_Hin when the
// piece is not the first); MODE kAggregate only records the piece's end state from
// zero and its dt2 sum.  With CK (full mode, 16 padded entries) the walkers also
// write their state before every 16th step to p.ckpt, the checkpoints the backward's
// gradient pass starts its tiles from.
//
// The G walking waves each carry SPL state entries of every channel; entries
// n >= N are padding with A = 0 and B = C = 0, which stay zero.  Staged steps beyond
// the piece's end are identity steps (dt2 = 0, x = 0), so the walk always runs
// whole tiles.
template <typename IO, int SPL, bool SCALAR, int MODE, bool VEC, int G, bool CK = false, bool CONV = false>
__global__ void __launch_bounds__((Shape<G, SPL>::NW * kLanes)) scan_fwd_kernel(Params p) {
    using S = Shape<G, SPL>;
    constexpr int NP_ = G * SPL;
    constexpr bool kSpec = S::kSpec;
    constexpr int NS = S::NS;
    constexpr int T = S::T;
    constexpr int VW = IOT<IO>::VW;
    constexpr int TV = T / VW;                     // vectors per row per tile
    constexpr int NVX = kLanes * TV;               // u/delta/z vectors per tile
    constexpr int KX = (NVX + NS - 1) / NS;        // of them per staging thread
    constexpr bool kFullMode = (MODE == kFull);
    constexpr int BCW = 2 * SPL;                   // floats per (wave, step) in sBC
    constexpr int NBC = G * T * BCW;               // sBC values per tile
    // B/C staging, two ways.  Small tiles: single values, the first half of the staging
    // threads taking B's and the second half C's (wave-uniform, so each load's buffer
    // window stays in scalar registers).  Large tiles (more than 8 values per thread):
    // 16-byte row vectors of B and C, each thread writing its vector's values down one
    // sBC column.
    constexpr int KBC = (NBC + NS - 1) / NS;       // values per staging thread
    constexpr bool kVecBC = KBC > 8;
    constexpr int NBV = 2 * NP_ * TV;              // B and C row vectors per tile
    constexpr int KBV = kVecBC ? (NBV + NS - 1) / NS : 0;   // of them per staging thread
    constexpr int NBH = NBC / 2;                   // sBC values of one matrix per tile
    constexpr int KBE = kVecBC ? 0 : (VEC ? (NBH + NS / 2 - 1) / (NS / 2) : KBC);
    constexpr int QB = SPL <= 4 ? 4 : (SPL == 8 ? 2 : 1);   // steps whose LDS operands are read together
    constexpr int NP = NP_;                        // padded state count
    constexpr float kLn2f = kLn2;
    // Two LDS layouts of the read-out (see lds_floats).  With four walkers of at most
    // 4 entries and four helpers (two waves per SIMD, the N <= 16 shapes) the partial
    // read-outs sit in swizzled 64-float rows and the skip terms and gates stay in the
    // helper's registers; otherwise padded rows and LDS for all three.
    constexpr bool kSGReg = yswizzled(G, SPL);
    constexpr int BUF = T * kRow * 2 + NBC + (kFullMode ? (kSGReg ? G * T * kLanes : (G + 2) * T * kRowY) : 0);   // floats per buffer
    constexpr int kEsz = int(sizeof(IO));
    static_assert(T % 8 == 0, "time tile must hold whole vectors and step groups");
    static_assert(!CK || (MODE == kFull && NP_ == 16 && T % kCkptSteps == 0 && kCkptSteps % QB == 0),
                  "checkpoints: full mode, 16 padded entries, whole checkpoint intervals per tile");
    static_assert(!kVecBC || (NP * TV) % kLanes == 0, "B/C row vectors: whole waves per matrix");
    static_assert(NS % (2 * kLanes) == 0, "B/C single values: whole waves per matrix");

    extern __shared__ float smem[];
    const int tid = threadIdx.x;
    const int w = tid / kLanes;
    const int lane = tid % kLanes;
    const bool walker = w < G;
    const bool stager = kSpec ? !walker : true;
    const int stid = kSpec ? tid - G * kLanes : tid;     // index among the staging threads

    // blockIdx.x -> (piece, batch, channel block), channel block fastest
    const int64_t bid = blockIdx.x;
    const int cblk = int(bid % p.nblk_d);
    const int b = int((bid / p.nblk_d) % p.batch);
    const int piece = int(bid / (int64_t(p.nblk_d) * p.batch));
    const int64_t blk = int64_t(b) * p.nblk_d + cblk;
    const int64_t c0 = int64_t(cblk) * kLanes;
    const int64_t tbeg = int64_t(piece) * p.chunk_len;
    const int64_t tend = (tbeg + p.chunk_len < p.L) ? tbeg + p.chunk_len : p.L;
    const int ntiles = int((tend - tbeg + T - 1) / T);
    const bool has_z = kFullMode && p.z != nullptr;

    const IO* __restrict__ gu = static_cast<const IO*>(p.u);
    const IO* __restrict__ gdl = static_cast<const IO*>(p.delta);
    const IO* __restrict__ gz = static_cast<const IO*>(p.z);
    const IO* __restrict__ gB = static_cast<const IO*>(p.Bm);
    const IO* __restrict__ gC = static_cast<const IO*>(p.Cm);
    IO* __restrict__ gy = static_cast<IO*>(p.y);

    // ---- buffer windows (rows of 16-byte vectors): the block's channel rows of u, delta,
    //      z and y, and the batch row's N rows of B and C
    const int64_t xoff = (int64_t(b) * p.dim + c0) * p.L * kEsz;
    const int64_t xrows = p.dim - c0 < kLanes ? p.dim - c0 : kLanes;
    const uint32_t xbytes = VEC ? uint32_t(xrows * p.L * kEsz) : 0u;
    const int64_t bcoff = int64_t(b) * p.N * p.L * kEsz;
    const uint32_t bcbytes = VEC ? uint32_t(p.N * p.L * kEsz) : 0u;
    const Window win_u{reinterpret_cast<const char*>(p.u) + xoff, xbytes};
    const Window win_dl{reinterpret_cast<const char*>(p.delta) + xoff, xbytes};
    const Window win_z{reinterpret_cast<const char*>(has_z ? p.z : p.u) + xoff, xbytes};
    const Window win_y{reinterpret_cast<const char*>(p.y) + xoff, xbytes};
    const Window win_B{reinterpret_cast<const char*>(p.Bm) + bcoff, bcbytes};
    const Window win_C{reinterpret_cast<const char*>(kFullMode ? p.Cm : p.Bm) + bcoff, bcbytes};

    // ---- walk constants: this lane's channel and its SPL decay rates
    const int64_t dch = c0 + lane;
    const bool lane_ok = walker && dch < p.dim;
    float Ar[SPL];
    float a_scalar = 0.0f;
    if constexpr (SCALAR) {
        a_scalar = lane_ok ? p.A[dch / p.head_dim] : 0.0f;
#pragma unroll
        for (int j = 0; j < SPL; ++j) Ar[j] = a_scalar;
    } else {
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const int64_t n = int64_t(w) * SPL + j;
            Ar[j] = (lane_ok && n < p.N) ? p.A[dch * p.N + n] : 0.0f;
        }
    }

    // ---- staging/epilogue constants: the channels of this thread's vectors
    int sv_ch[KX], sv_tv[KX];
    bool sv_on[KX], sv_ok[KX];
    float sv_bias[KX], sv_skip[KX], sv_ah[KX];
    int64_t sv_row[KX];
    uint32_t sv_voff[KX];   // byte offset of the vector in the block's window (kOob: none)
#pragma unroll
    for (int k = 0; k < KX; ++k) {
        const int v = stid + k * NS;
        sv_on[k] = stager && v < NVX;
        sv_ch[k] = (v / TV) % kLanes;
        sv_tv[k] = v % TV;
        const int64_t d = c0 + sv_ch[k];
        sv_ok[k] = sv_on[k] && d < p.dim;
        sv_bias[k] = (sv_ok[k] && p.bias) ? p.bias[d] : 0.0f;
        sv_skip[k] = (sv_ok[k] && p.Dskip) ? p.Dskip[d] : 0.0f;
        sv_ah[k] = 0.0f;
        if constexpr (SCALAR) sv_ah[k] = sv_ok[k] ? p.A[d / p.head_dim] : 0.0f;
        sv_row[k] = (int64_t(b) * p.dim + (sv_ok[k] ? d : 0)) * p.L;
        sv_voff[k] = sv_ok[k] ? uint32_t((int64_t(sv_ch[k]) * p.L + sv_tv[k] * VW) * kEsz) : kOob;
    }
    // ---- fused convolution: tap j of a vector's halo-extended window multiplies
    //      x[t - 3 + j] (taps before the first weight are 0)
    // the fused front end is a template flag (launched exactly when p.conv_w is set), so
    // that the plain scan carries none of its registers or address arithmetic
    constexpr bool conv = CONV;
    static_assert(!(CK && CONV), "checkpoints are kept by the plain scan only");
    float sv_cw[KX][kMaxConv], sv_cb[KX];
#pragma unroll
    for (int k = 0; k < KX; ++k) {
        const int64_t d = c0 + sv_ch[k];
#pragma unroll
        for (int j = 0; j < kMaxConv; ++j) {
            const int kk = j - (kMaxConv - p.conv_k);
            sv_cw[k][j] = (conv && sv_ok[k] && kk >= 0) ? p.conv_w[d * p.conv_k + kk] : 0.0f;
        }
        sv_cb[k] = (conv && sv_ok[k] && p.conv_b) ? p.conv_b[d] : 0.0f;
    }

    // ---- B/C staging constants: row vectors v = stid + k*NS, B rows first, then C
    const IO* bc_row[KBV > 0 ? KBV : 1];
    int bc_dst[KBV > 0 ? KBV : 1], bc_tv[KBV > 0 ? KBV : 1];
    bool bc_on[KBV > 0 ? KBV : 1], bc_ok[KBV > 0 ? KBV : 1], bc_isC[KBV > 0 ? KBV : 1];
    uint32_t bc_voff[KBV > 0 ? KBV : 1];
#pragma unroll
    for (int k = 0; k < KBV; ++k) {
        const int v = stid + k * NS;
        bc_on[k] = stager && v >= 0 && v < NBV;
        const int isC = v / (NP * TV);
        const int rem = v % (NP * TV);
        const int n = rem / TV;
        bc_tv[k] = rem % TV;
        bc_isC[k] = isC != 0;
        bc_ok[k] = bc_on[k] && n < p.N && (kFullMode || !isC);
        bc_row[k] = (isC ? gC : gB) + (int64_t(b) * p.N + (bc_ok[k] ? n : 0)) * p.L;
        bc_dst[k] = (n / SPL) * T * BCW + (n % SPL) + (isC ? SPL : 0);
        bc_voff[k] = bc_ok[k] ? uint32_t((int64_t(n) * p.L + bc_tv[k] * VW) * kEsz) : kOob;
    }

    // single B/C values.  With buffer loads (VEC) staging threads stid < NS/2 take B's and
    // the others C's (value i of a matrix is entry n = (i / (T*SPL)) * SPL + i % SPL at
    // step (i / SPL) % T), so that each wave reads one matrix through one window; with
    // element loads, value idx = stid + k*NS of the tile's sBC, B or C by its slot.
    const IO* bce_ptr[KBE > 0 ? KBE : 1];
    int bce_t[KBE > 0 ? KBE : 1];
    bool bce_on[KBE > 0 ? KBE : 1];
    uint32_t bce_voff[KBE > 0 ? KBE : 1];
    int bce_dst[VEC && KBE > 0 ? KBE : 1];
    const bool bce_isC = VEC && stid >= NS / 2;
    const int bce_i0 = bce_isC ? stid - NS / 2 : stid;
#pragma unroll
    for (int k = 0; k < KBE; ++k) {
        if constexpr (VEC) {
            const int i = bce_i0 + k * (NS / 2);
            const int wn = i / (T * SPL), j = i % SPL, t = (i / SPL) % T;
            const int64_t n = int64_t(wn) * SPL + j;
            bce_on[k] = stager && i < NBH && n < p.N && (kFullMode || !bce_isC);
            bce_t[k] = t;
            bce_dst[k] = (wn * T + t) * BCW + j + (bce_isC ? SPL : 0);
            bce_voff[k] = bce_on[k] ? uint32_t((n * p.L + t) * kEsz) : kOob;
        } else {
            const int idx = stid + k * NS;
            const int wn = idx / (T * BCW), rem = idx % (T * BCW);
            const int t = rem / BCW, slot = rem % BCW;
            const int64_t n = int64_t(wn) * SPL + (slot % SPL);
            const bool isC = slot >= SPL;
            bce_on[k] = stager && idx >= 0 && idx < NBC && n < p.N && (kFullMode || !isC);
            bce_t[k] = t;
            bce_ptr[k] = (isC ? gC : gB) + (int64_t(b) * p.N + (bce_on[k] ? n : 0)) * p.L + t;
        }
    }

    // ---- starting state of this piece
    float h[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) h[j] = 0.0f;
    if (kFullMode && walker) {
        if (p.nchunks > 1) {
            // every piece, the first included, starts from the carried state, so h0 is
            // read only by the carry kernel and may be the same array as h_last
            const float* hin = p.ws_Hin + ((blk * p.nchunks + piece) * NP + int64_t(w) * SPL) * kLanes + lane;
#pragma unroll
            for (int j = 0; j < SPL; ++j) h[j] = hin[int64_t(j) * kLanes];
        } else if (p.h0 && lane_ok) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const int64_t n = int64_t(w) * SPL + j;
                if (n < p.N) h[j] = p.h0[(int64_t(b) * p.dim + dch) * p.N + n];
            }
        }
    }
    // Settle these loads now: left pending, they make the compiler wait for every
    // outstanding load (the next tile's prefetch included) inside the walk.
    __builtin_amdgcn_s_waitcnt(0);
    float dtsum = 0.0f, dtcomp = 0.0f;   // compensated (Kahan) sum of dt2 over the piece

    Vec<IO> nu[KX], ndl[KX], nz[KX], nbc[KBV > 0 ? KBV : 1];
    IO nbce[KBE > 0 ? KBE : 1];
    IO nhalo[KX][kMaxConv];   // fused convolution: x[t-4 .. t-1] before each vector
    // the skip term D*u and the gate SiLU(z) of the elements a thread stages, kept until
    // it finishes them: slot (tile index & 1) with helper waves, slot 0 without
    float skr[kSGReg && kSpec ? 2 : 1][KX][VW], gtr[kSGReg && kSpec ? 2 : 1][KX][VW];

    // ---- global -> registers for the tile starting at t0 (staging threads).  With
    //      16-byte rows (VEC) every load goes through a buffer window advanced to the
    //      tile (scalar arithmetic only) at a fixed lane offset: no address arithmetic
    //      and no bounds checks in the vector unit; reads past the array return zeros,
    //      and values past the piece's end are masked where they are staged.
    auto issue_loads = [&](int64_t t0) __attribute__((always_inline)) {
        if constexpr (VEC) {
            const uint32_t toff = uint32_t(t0) * kEsz;
            const Rsrc ru = win_u.at(toff), rd = win_dl.at(toff), rz = win_z.at(toff);
#pragma unroll
            for (int k = 0; k < KX; ++k) {
                if (NVX % NS == 0 || sv_on[k]) {
                    nu[k] = __builtin_bit_cast(Vec<IO>, __builtin_amdgcn_raw_buffer_load_b128(ru, sv_voff[k], 0, 0));
                    ndl[k] = __builtin_bit_cast(Vec<IO>, __builtin_amdgcn_raw_buffer_load_b128(rd, sv_voff[k], 0, 0));
                    if (has_z)
                        nz[k] = __builtin_bit_cast(Vec<IO>, __builtin_amdgcn_raw_buffer_load_b128(rz, sv_voff[k], 0, 0));
                }
            }
            if constexpr (KBV > 0) {
                const Rsrc rb = win_B.at(toff), rc = win_C.at(toff);
#pragma unroll
                for (int k = 0; k < KBV; ++k) {
                    // B or C is the same for a whole wave (whole waves per matrix)
                    const bool isC = __builtin_amdgcn_readfirstlane(int(bc_isC[k])) != 0;
                    nbc[k] = __builtin_bit_cast(
                        Vec<IO>, __builtin_amdgcn_raw_buffer_load_b128(isC ? rc : rb, bc_voff[k], 0, 0));
                }
            }
            if constexpr (KBE > 0) {
                // B or C is the same for a whole wave: read the choice from the first lane so
                // that the window stays in scalar registers
                const bool isC = __builtin_amdgcn_readfirstlane(int(bce_isC)) != 0;
                const Rsrc rbc = isC ? win_C.at(toff) : win_B.at(toff);
#pragma unroll
                for (int k = 0; k < KBE; ++k) {
                    if constexpr (sizeof(IO) == 2)
                        nbce[k] = __builtin_bit_cast(IO, __builtin_amdgcn_raw_buffer_load_b16(rbc, bce_voff[k], 0, 0));
                    else
                        nbce[k] = __builtin_bit_cast(IO, __builtin_amdgcn_raw_buffer_load_b32(rbc, bce_voff[k], 0, 0));
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < KX; ++k) {
                if (sv_on[k]) {
                    const int64_t t = t0 + sv_tv[k] * VW;
                    nu[k] = load_vec<IO, VEC>(gu + sv_row[k], t, tend, sv_ok[k]);
                    ndl[k] = load_vec<IO, VEC>(gdl + sv_row[k], t, tend, sv_ok[k]);
                    if (has_z) nz[k] = load_vec<IO, VEC>(gz + sv_row[k], t, tend, sv_ok[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < KBV; ++k)
                if (bc_on[k]) nbc[k] = load_vec<IO, VEC>(bc_row[k], t0 + bc_tv[k] * VW, tend, bc_ok[k]);
#pragma unroll
            for (int k = 0; k < KBE; ++k)
                nbce[k] = (bce_on[k] && t0 + bce_t[k] < tend) ? bce_ptr[k][t0] : IO(0);
        }
        if constexpr (conv) {
#pragma unroll
            for (int k = 0; k < KX; ++k) {
                if (sv_on[k]) {
                    // the 4 inputs before the vector (t is a multiple of the vector width,
                    // so t >= 4 unless t == 0, whose history stage takes from conv_state)
                    const int64_t t = t0 + sv_tv[k] * VW;
                    const IO* src = gu + sv_row[k] + (t >= kMaxConv ? t - kMaxConv : 0);
                    if constexpr (VEC) {
                        using R = typename std::conditional<sizeof(IO) == 2, uint2, uint4>::type;
                        const R raw = *reinterpret_cast<const R*>(src);
                        __builtin_memcpy(nhalo[k], &raw, sizeof(R));
                    } else {
#pragma unroll
                        for (int j = 0; j < kMaxConv; ++j) nhalo[k][j] = src[j];
                    }
                }
            }
        }
    };

    // ---- registers -> LDS buffer `buf` for the tile starting at t0 (staging threads):
    //      per element (dt2, dt2*u) or (exp(dt*a_h), dt2*u); B*ln2 and C; the skip term
    //      and gate into register slot SL
    auto stage = [&](float* buf, int64_t t0, auto slot) __attribute__((always_inline)) {
        constexpr int SL = decltype(slot)::value;
        float2* sDX = reinterpret_cast<float2*>(buf);
        float* sBC = buf + T * kRow * 2;
        const bool full_tile = t0 + T <= tend;
        float uval[KX][VW];   // the scan's input u of each vector element
#pragma unroll
        for (int k = 0; k < KX; ++k) {
#pragma unroll
            for (int e = 0; e < VW; ++e) uval[k][e] = IOT<IO>::to_f32(nu[k].e[e]);
            if (conv && sv_on[k]) {
                const int64_t t = t0 + sv_tv[k] * VW;
                float xx[kMaxConv + VW];
#pragma unroll
                for (int j = 0; j < kMaxConv; ++j) xx[j] = (t >= kMaxConv) ? IOT<IO>::to_f32(nhalo[k][j]) : 0.0f;
                if (t == 0 && p.conv_state && sv_ok[k] && p.conv_k > 1) {
                    // history before the sequence: the last conv_k-1 inputs, oldest first
                    const int64_t d = c0 + sv_ch[k];
                    const IO* st = static_cast<const IO*>(p.conv_state) + (int64_t(b) * p.dim + d) * (p.conv_k - 1);
#pragma unroll
                    for (int j = 0; j < kMaxConv; ++j) {
                        const int q = j - (kMaxConv - (p.conv_k - 1));
                        if (q >= 0) xx[j] = IOT<IO>::to_f32(st[q]);
                    }
                }
#pragma unroll
                for (int e = 0; e < VW; ++e) xx[kMaxConv + e] = uval[k][e];
#pragma unroll
                for (int e = 0; e < VW; ++e) {
                    float acc = sv_cb[k];
#pragma unroll
                    for (int j = 0; j < kMaxConv; ++j) acc = fmaf(sv_cw[k][j], xx[e + 1 + j], acc);
                    uval[k][e] = p.conv_silu ? silu_f32(acc) : acc;
                }
                if (kFullMode && p.u_out) {
                    Vec<IO> ov;
#pragma unroll
                    for (int e = 0; e < VW; ++e) ov.e[e] = IOT<IO>::from_f32(uval[k][e]);
                    store_vec<IO, VEC>(static_cast<IO*>(p.u_out) + sv_row[k], t, tend, sv_ok[k], ov);
                }
            }
        }
        // element e of vector k: `in` = inside the piece and the channels; outside, the
        // step is an identity step (dt2 = 0, x = 0) whatever the loaded values were
        auto elem = [&](int k, int e, bool in) __attribute__((always_inline)) {
            // (element loads already read zeros outside; buffer loads read what is there)
            const float uu = (!VEC || in) ? uval[k][e] : 0.0f;
            const float dt2 = in ? softplus_log2(IOT<IO>::to_f32(ndl[k].e[e]) + sv_bias[k]) : 0.0f;
            float first = dt2;
            if constexpr (SCALAR && kFullMode) first = __builtin_amdgcn_exp2f(dt2 * sv_ah[k]);
            const int tl = sv_tv[k] * VW + e;
            sDX[tl * kRow + sv_ch[k]] = make_float2(first, dt2 * uu);
            if constexpr (kFullMode) {
                const float sk = sv_skip[k] * uu;
                const float gt = has_z ? silu_f32(IOT<IO>::to_f32(nz[k].e[e])) : 1.0f;
                if constexpr (kSGReg) {
                    skr[SL][k][e] = sk;
                    gtr[SL][k][e] = gt;
                } else {
                    float* sSk = buf + T * kRow * 2 + NBC + G * T * kRowY;
                    sSk[tl * kRowY + sv_ch[k]] = sk;
                    sSk[(T + tl) * kRowY + sv_ch[k]] = gt;
                }
            }
        };
#pragma unroll
        for (int k = 0; k < KX; ++k) {
            if (NVX % NS == 0 || sv_on[k]) {
                if (full_tile && sv_ok[k]) {
#pragma unroll
                    for (int e = 0; e < VW; ++e) elem(k, e, true);
                } else {
                    const int64_t lim = tend - (t0 + sv_tv[k] * VW);
#pragma unroll
                    for (int e = 0; e < VW; ++e) elem(k, e, sv_ok[k] && e < lim);
                }
            }
        }
        // steps of this tile inside the piece (a workgroup-uniform count)
        const int tin = full_tile ? T : int(tend - t0);
#pragma unroll
        for (int k = 0; k < KBV; ++k) {
            if (bc_on[k]) {
                const float sc = bc_isC[k] ? 1.0f : kLn2f;
                float* dst = sBC + bc_dst[k] + bc_tv[k] * VW * BCW;
                if (!VEC || full_tile) {
#pragma unroll
                    for (int e = 0; e < VW; ++e) dst[e * BCW] = IOT<IO>::to_f32(nbc[k].e[e]) * sc;
                } else {
                    const int lim = tin - bc_tv[k] * VW;
#pragma unroll
                    for (int e = 0; e < VW; ++e) dst[e * BCW] = e < lim ? IOT<IO>::to_f32(nbc[k].e[e]) * sc : 0.0f;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < KBE; ++k) {
            if constexpr (VEC) {
                if (stager && (NBH % (NS / 2) == 0 || bce_i0 + k * (NS / 2) < NBH)) {
                    const float v = IOT<IO>::to_f32(nbce[k]) * (bce_isC ? 1.0f : kLn2f);
                    if (full_tile)
                        sBC[bce_dst[k]] = v;
                    else
                        sBC[bce_dst[k]] = bce_t[k] < tin ? v : 0.0f;
                }
            } else {
                const int idx = stid + k * NS;
                if (stager && (NBC % NS == 0 || idx < NBC))
                    sBC[idx] = IOT<IO>::to_f32(nbce[k]) * ((idx % BCW) < SPL ? kLn2f : 1.0f);
            }
        }
    };

    // ---- walk one tile from LDS buffer `buf` (walking waves): SPL state entries per
    //      lane, sequential in t; the LDS operands of QB steps are read up front
    // this lane's sY column for each vector of steps of a tile (see ysw)
    int ycol[kSGReg ? TV : 1];
#pragma unroll
    for (int j = 0; j < (kSGReg ? TV : 1); ++j) ycol[j] = lane ^ ysw<T, VW>(j * VW);
    auto walk = [&](float* buf, int64_t t0) __attribute__((always_inline)) {
        const float2* dxp = reinterpret_cast<const float2*>(buf) + lane;
        const float* bcp = buf + T * kRow * 2 + w * T * BCW;
        float* yo = buf + T * kRow * 2 + NBC + (kSGReg ? w * kLanes : w * T * kRowY + lane);
#pragma unroll
        for (int t = 0; t < T; t += QB) {
            if constexpr (CK) {
                if (t % kCkptSteps == 0 && t0 + t < tend) {
                    float* ck = p.ckpt + ((blk * p.ntiles_ck + (t0 + t) / kCkptSteps) * NP + int64_t(w) * SPL) * kLanes + lane;
#pragma unroll
                    for (int j = 0; j < SPL; ++j) ck[int64_t(j) * kLanes] = h[j];
                }
            }
            float2 dx[QB];
            BCVec<SPL> bc[QB];
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                dx[q] = dxp[(t + q) * kRow];
                bc[q] = read_bc<SPL>(bcp + (t + q) * BCW);
            }
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                float a_shared = 0.0f;
                if constexpr (SCALAR) {
                    if constexpr (kFullMode) a_shared = dx[q].x;
                    else a_shared = __builtin_amdgcn_exp2f(dx[q].x * a_scalar);
                }
                if constexpr (!kFullMode) {
                    const float yk = dx[q].x - dtcomp;
                    const float tk = dtsum + yk;
                    dtcomp = (tk - dtsum) - yk;
                    dtsum = tk;
                }
                float yp = 0.0f;
#pragma unroll
                for (int j = 0; j < SPL; ++j) {
                    const float a = SCALAR ? a_shared : __builtin_amdgcn_exp2f(dx[q].x * Ar[j]);
                    h[j] = fmaf(a, h[j], dx[q].y * bc[q].v[j]);
                    if constexpr (kFullMode) yp = fmaf(bc[q].v[SPL + j], h[j], yp);
                }
                if constexpr (kFullMode) {
                    if constexpr (kSGReg)
                        yo[(t + q) * G * kLanes + ycol[(t + q) / VW]] = yp;
                    else
                        yo[(t + q) * kRowY] = yp;
                }
            }
        }
    };

    // ---- finish the tile starting at t0 from LDS buffer `buf` (staging threads): sum
    //      the G partial read-outs in wave order, skip and gate from register slot SL,
    //      round, store.
    // With bf16 rows and 32-step tiles a tile covers half of each row's 128-byte
    // cache line; the even tile's output is held and stored together with the odd
    // tile's, so both halves of a line reach the L2 back to back and are written to
    // HBM as one full line.
    constexpr bool kPairStores = VEC && (T * int(sizeof(IO)) == 64);
    Vec<IO> held[KX];
    // vector k of this thread's row in the tile starting at tile_t0 (a workgroup-uniform
    // step, so that the window stays in scalar registers)
    auto store = [&](int k, int64_t tile_t0, const Vec<IO>& v, bool full_tile) __attribute__((always_inline)) {
        if constexpr (VEC) {
            if (full_tile) {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(bvec4, v), win_y.at(uint32_t(tile_t0) * kEsz),
                                                       sv_voff[k], 0, 0);
                return;
            }
        }
        store_vec<IO, VEC>(gy + sv_row[k], tile_t0 + sv_tv[k] * VW, tend, sv_ok[k], v);
    };
    auto finish = [&](const float* buf, int64_t t0, int kt, auto slot) __attribute__((always_inline)) {
        constexpr int SL = decltype(slot)::value;
        if constexpr (kFullMode) {
            const float* sY = buf + T * kRow * 2 + NBC;
            const bool full_tile = t0 + T <= tend;
#pragma unroll
            for (int k = 0; k < KX; ++k) {
                if (NVX % NS == 0 || sv_on[k]) {
                    // steps tv*VW .. +VW-1 of channel ch, summed over the walkers in order
                    float acc[VW];
                    if constexpr (kSGReg) {
                        // column ch ^ ysw, rows (t, w)
                        const float* src = sY + sv_tv[k] * VW * G * kLanes + (sv_ch[k] ^ ysw<T, VW>(sv_tv[k] * VW));
#pragma unroll
                        for (int e = 0; e < VW; ++e) acc[e] = src[e * G * kLanes];
#pragma unroll
                        for (int ww = 1; ww < G; ++ww)
#pragma unroll
                            for (int e = 0; e < VW; ++e) acc[e] += src[(e * G + ww) * kLanes];
                    } else {
                        const int off = (sv_tv[k] * VW) * kRowY + sv_ch[k];
#pragma unroll
                        for (int e = 0; e < VW; ++e) acc[e] = sY[off + e * kRowY];
#pragma unroll
                        for (int ww = 1; ww < G; ++ww)
#pragma unroll
                            for (int e = 0; e < VW; ++e) acc[e] += sY[off + (ww * T + e) * kRowY];
                    }
                    Vec<IO> out;
#pragma unroll
                    for (int e = 0; e < VW; ++e) {
                        float sk, gt;
                        if constexpr (kSGReg) {
                            sk = skr[SL][k][e];
                            gt = gtr[SL][k][e];
                        } else {
                            const float* sSk = sY + G * T * kRowY;
                            const int off = (sv_tv[k] * VW + e) * kRowY + sv_ch[k];
                            sk = sSk[off];
                            gt = sSk[T * kRowY + off];
                        }
                        out.e[e] = IOT<IO>::from_f32((acc[e] + sk) * gt);
                    }
                    if constexpr (kPairStores) {
                        if ((kt & 1) == 0 && kt + 1 < ntiles) {
                            held[k] = out;            // stored with the next tile's vector
                            continue;
                        }
                        if (kt & 1) store(k, t0 - T, held[k], true);
                    }
                    store(k, t0, out, full_tile);
                }
            }
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if constexpr (kSpec) {
        // walkers walk tile kt from buffer kt&1 while the helpers finish tile kt-1
        // (buffer (kt-1)&1) and then stage tile kt+1 into that same buffer; tile k's
        // skip terms and gates are in register slot k&1, so the loop takes two tiles
        // per turn and every slot index is a compile-time constant
        if (stager) {
            issue_loads(tbeg);
            stage(smem, tbeg, I0{});
            if (ntiles > 1) issue_loads(tbeg + T);
        }
        __syncthreads();
        auto period = [&](int kt, auto par) __attribute__((always_inline)) {
            constexpr int P = decltype(par)::value;
            using Other = std::integral_constant<int, 1 - P>;
            float* cur = smem + P * BUF;
            float* oth = smem + (1 - P) * BUF;
            const int64_t t0 = tbeg + int64_t(kt) * T;
            if (walker) {
                walk(cur, t0);
            } else {
                if (kt >= 1) finish(oth, t0 - T, kt - 1, Other{});
                if (kt + 1 < ntiles) {
                    stage(oth, t0 + T, Other{});
                    if (kt + 2 < ntiles) issue_loads(t0 + 2 * T);
                }
            }
            __syncthreads();
        };
        if constexpr (kSGReg) {
            for (int kt = 0; kt < ntiles; kt += 2) {
                period(kt, I0{});
                if (kt + 1 < ntiles) period(kt + 1, I1{});
            }
            if (stager) {
                const int kl = ntiles - 1;
                const int64_t tl = tbeg + int64_t(kl) * T;
                if (kl & 1)
                    finish(smem + BUF, tl, kl, I1{});
                else
                    finish(smem, tl, kl, I0{});
            }
        } else {
            // skip terms and gates in LDS: one tile per turn (a two-tile body would hold
            // both tiles' walk in registers at three waves per SIMD)
            for (int kt = 0; kt < ntiles; ++kt) {
                float* cur = smem + (kt & 1) * BUF;
                float* oth = smem + ((kt + 1) & 1) * BUF;
                const int64_t t0 = tbeg + int64_t(kt) * T;
                if (walker) {
                    walk(cur, t0);
                } else {
                    if (kt >= 1) finish(oth, t0 - T, kt - 1, I0{});
                    if (kt + 1 < ntiles) {
                        stage(oth, t0 + T, I0{});
                        if (kt + 2 < ntiles) issue_loads(t0 + 2 * T);
                    }
                }
                __syncthreads();
            }
            if (stager) finish(smem + ((ntiles - 1) & 1) * BUF, tbeg + int64_t(ntiles - 1) * T, ntiles - 1, I0{});
        }
    } else {
        issue_loads(tbeg);
        for (int kt = 0; kt < ntiles; ++kt) {
            const int64_t t0 = tbeg + int64_t(kt) * T;
            stage(smem, t0, I0{});
            if (kt + 1 < ntiles) issue_loads(t0 + T);   // prefetch the next tile
            __syncthreads();
            walk(smem, t0);
            __syncthreads();
            finish(smem, t0, kt, I0{});
        }
    }

    if constexpr (kFullMode) {
        if (walker && lane_ok && p.h_last && piece == p.nchunks - 1) {
#pragma unroll
            for (int j = 0; j < SPL; ++j) {
                const int64_t n = int64_t(w) * SPL + j;
                if (n < p.N) p.h_last[(int64_t(b) * p.dim + dch) * p.N + n] = h[j];
            }
        }
    }
    if constexpr (!kFullMode) {
        if (walker) {
            float* hout = p.ws_H + ((blk * p.nchunks + piece) * NP + int64_t(w) * SPL) * kLanes + lane;
#pragma unroll
            for (int j = 0; j < SPL; ++j) hout[int64_t(j) * kLanes] = h[j];
            if (w == 0) p.ws_S[(blk * p.nchunks + piece) * kLanes + lane] = dtsum;
        }
    }
}

// ------------------------------------------------------------------ pass 1 on the matrix cores
// (Forward mode; the reverse mode, for the backward, is described with
// launch_piece_states in scan_common.h: the same contraction with ds against C,
// the chunks taken from the piece's end and prefix sums in place of suffix sums.)
// With one decay rate a_h per head, the end state of a piece from zero is
//   H[d,n] = ln2 * sum_t x[d,t] * 2^(a_h * sum_{s>t} dt2[d,s]) * B[n,t],   x = dt2 * u
// (dt2 = dt / ln 2: step sizes in log2 units, as in the walk, which folds the ln 2
// into B),
// i.e. for each 64-channel block the product of a (channels x steps) weight matrix and
// the (steps x states) matrix B: a dense contraction over the steps.  Chunk by chunk of
// 64 steps, H <- 2^(a_h * S_chunk) H + W_chunk B_chunk on v_mfma_f32_16x16x32_bf16,
// with the fp32 weights split into two bf16 parts (B is a bf16 input, exact).  Same
// outputs as scan_fwd_kernel<kAggregate>: ws_H and ws_S (the piece's sum of dt2).
//
// Wave w owns channels 16w..16w+15.  As the A operand, lane l supplies channel
// 16w + l%16 at steps 8(l/16)..+7 (k-step 0) and 32 + 8(l/16)..+7 (k-step 1) of the
// chunk; it computes those 16 weights itself.  The suffix sums over the chunk come
// from the 8 group totals of its channel, exchanged through LDS among the 4 lanes of
// the channel (all in the same wave).  The result rows are channels 4(l/16)..+3 of
// column n = 16j + l%16, so the chunk's decay scales each accumulator row.
namespace agg {
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
constexpr int kQ = 64;             // steps per chunk
constexpr int kRowB = kQ + 8;      // B row stride in LDS (bf16): 144 bytes, so the 16 rows
                                   // a 16-lane group reads start in distinct bank quads
constexpr int kThreads = 256;

__device__ inline uint32_t pack2(float x0, float x1) {
    const f32x2 x = {x0, x1};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
// x = hi + lo (hi = bf16(x), lo = bf16(x - hi)) for 8 floats, packed two per word
__device__ inline void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t hw = pack2(x[2 * j], x[2 * j + 1]);
        h[j] = hw;
        l[j] = pack2(x[2 * j] - __uint_as_float(hw << 16), x[2 * j + 1] - __uint_as_float(hw & 0xFFFF0000u));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}
}  // namespace agg

template <int N, bool REV>
__global__ void __launch_bounds__(agg::kThreads) scan_piece_states_kernel(ssm_detail::PieceStatesArgs p) {
    using namespace agg;
    constexpr int NT = N / 16;                    // 16-state column tiles
    constexpr int KBV = N * (kQ / 8) / kThreads;  // 16-byte B vectors per thread and chunk
    static_assert(N % 16 == 0 && KBV * kThreads == N * (kQ / 8), "B vectors must split evenly");
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][N * kRowB];
    __shared__ __attribute__((aligned(16))) float sTot[kLanes * 8];
    __shared__ __attribute__((aligned(16))) float sDec[kLanes];

    const int tid = threadIdx.x;
    const int wv = tid / kLanes, lane = tid % kLanes, g = lane / 16;
    const int64_t bid = blockIdx.x;
    const int cblk = int(bid % p.nblk_d);
    const int b = int((bid / p.nblk_d) % p.batch);
    const int piece = int(bid / (int64_t(p.nblk_d) * p.batch)) + p.piece_base;
    const int64_t blk = int64_t(b) * p.nblk_d + cblk;
    const int64_t c0 = int64_t(cblk) * kLanes;
    const int64_t tbeg = int64_t(piece) * p.chunk_len;
    const int64_t tend = (tbeg + p.chunk_len < p.L) ? tbeg + p.chunk_len : p.L;
    const int nq = int((tend - tbeg + kQ - 1) / kQ);

    // A side: channel chl of the block, steps 8g..8g+7 and 32+8g..32+8g+7 of each chunk
    const int chl = 16 * wv + (lane % 16);
    const int64_t d = c0 + chl;
    const bool dok = d < p.dim;
    const float a_h = dok ? p.A[d / p.head_dim] : 0.0f;
    const float bias = (dok && p.bias) ? p.bias[d] : 0.0f;
    const int64_t row = (int64_t(b) * p.dim + (dok ? d : 0)) * p.L;
    const uint16_t* __restrict__ urow = static_cast<const uint16_t*>(p.x) + row;   // u, or dy
    const uint16_t* __restrict__ drow = static_cast<const uint16_t*>(p.delta) + row;
    const bool has_z = REV && p.z != nullptr;
    const uint16_t* __restrict__ zrow = static_cast<const uint16_t*>(has_z ? p.z : p.x) + row;
    // B (or C) side: vector v = tid + k*256 is row n = v/8, steps 8(v%8)..+7 of the chunk
    const uint16_t* __restrict__ gB = static_cast<const uint16_t*>(p.BC) + int64_t(b) * N * p.L;

    // loads never branch: an 8-step group wholly outside the piece reads the row start
    // and is masked where it is used (pieces hold whole 8-step groups)
    // chunk i of the loop: chunks in step order, or from the piece's end (reverse)
    auto chunk_of = [&](int i) { return REV ? nq - 1 - i : i; };
    auto a_off = [&](int i, int grp) {
        const int64_t t = tbeg + int64_t(chunk_of(i)) * kQ + grp * 32 + 8 * g;
        return t < tend ? t : int64_t(0);
    };
    // (the prefetched 16-byte vectors are native vector types: with HIP's uint4, a
    //  struct, the compiler kept them in scratch memory)
    const int bcol = 8 * (tid % 8);      // every vector of a thread has the same steps

    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float ssum = 0.0f, scomp = 0.0f;   // compensated sum of dt2 over the piece

    u32x4 d0 = *reinterpret_cast<const u32x4*>(drow + a_off(0, 0));
    u32x4 u0 = *reinterpret_cast<const u32x4*>(urow + a_off(0, 0));
    u32x4 d1 = *reinterpret_cast<const u32x4*>(drow + a_off(0, 1));
    u32x4 u1 = *reinterpret_cast<const u32x4*>(urow + a_off(0, 1));
    u32x4 z0 = {0u, 0u, 0u, 0u}, z1 = z0, z0n = z0, z1n = z0;
    if constexpr (REV) {
        z0 = *reinterpret_cast<const u32x4*>(zrow + a_off(0, 0));
        z1 = *reinterpret_cast<const u32x4*>(zrow + a_off(0, 1));
    }
    u32x4 d0n, u0n, d1n, u1n, bv[KBV];
    {
        const int64_t t = tbeg + int64_t(chunk_of(0)) * kQ + bcol;
#pragma unroll
        for (int k = 0; k < KBV; ++k)
            bv[k] = *reinterpret_cast<const u32x4*>(gB + int64_t((tid + k * kThreads) / 8) * p.L + (t < tend ? t : 0));
#pragma unroll
        for (int k = 0; k < KBV; ++k)
            *reinterpret_cast<u32x4*>(&sB[0][((tid + k * kThreads) / 8) * kRowB + bcol]) = bv[k];
    }
    __syncthreads();
    for (int q = 0; q < nq; ++q) {
        if (q + 1 < nq) {
            d0n = *reinterpret_cast<const u32x4*>(drow + a_off(q + 1, 0));
            u0n = *reinterpret_cast<const u32x4*>(urow + a_off(q + 1, 0));
            d1n = *reinterpret_cast<const u32x4*>(drow + a_off(q + 1, 1));
            u1n = *reinterpret_cast<const u32x4*>(urow + a_off(q + 1, 1));
            if constexpr (REV) {
                z0n = *reinterpret_cast<const u32x4*>(zrow + a_off(q + 1, 0));
                z1n = *reinterpret_cast<const u32x4*>(zrow + a_off(q + 1, 1));
            }
            const int64_t t = tbeg + int64_t(chunk_of(q + 1)) * kQ + bcol;
#pragma unroll
            for (int k = 0; k < KBV; ++k)
                bv[k] = *reinterpret_cast<const u32x4*>(gB + int64_t((tid + k * kThreads) / 8) * p.L + (t < tend ? t : 0));
        }
        // dt2 and the weighted value (forward: x = dt2*u; reverse: ds = dy*SiLU(z)) of
        // the lane's two 8-step groups; steps outside the piece are identity steps
        // (dt2 = 0, value 0)
        float dt[2][8], x[2][8], tot[2];
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            const int64_t t = tbeg + int64_t(chunk_of(q)) * kQ + grp * 32 + 8 * g;
            const bool in = dok && t < tend;
            uint16_t dr[8], uu[8], zz[8];
            const u32x4 dv = grp == 0 ? d0 : d1, uv = grp == 0 ? u0 : u1, zv = grp == 0 ? z0 : z1;
            __builtin_memcpy(dr, &dv, 16);
            __builtin_memcpy(uu, &uv, 16);
            __builtin_memcpy(zz, &zv, 16);
            tot[grp] = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float r = IOT<uint16_t>::to_f32(dr[j]) + bias;
                dt[grp][j] = in ? softplus_log2(r) : 0.0f;
                const float v = in ? IOT<uint16_t>::to_f32(uu[j]) : 0.0f;
                if constexpr (REV)
                    x[grp][j] = has_z ? v * silu_f32(IOT<uint16_t>::to_f32(zz[j])) : v;
                else
                    x[grp][j] = dt[grp][j] * v;
                tot[grp] += dt[grp][j];
            }
        }
        // the channel's 8 group totals in step order: groups 0..3 are the first groups
        // of lanes g = 0..3, groups 4..7 their second
        sTot[chl * 8 + g] = tot[0];
        sTot[chl * 8 + 4 + g] = tot[1];
        __builtin_amdgcn_wave_barrier();   // the wave's LDS writes complete before its reads
        const f32x4 t03 = *reinterpret_cast<const f32x4*>(&sTot[chl * 8]);
        const f32x4 t47 = *reinterpret_cast<const f32x4*>(&sTot[chl * 8 + 4]);
        const float G[8] = {t03[0], t03[1], t03[2], t03[3], t47[0], t47[1], t47[2], t47[3]};
        // forward: after[k] = sum of the groups after group k; reverse: before[k] =
        // sum of the groups before group k
        float after[8], before[8];
        after[7] = 0.0f;
        before[0] = 0.0f;
#pragma unroll
        for (int k = 6; k >= 0; --k) after[k] = after[k + 1] + G[k + 1];
#pragma unroll
        for (int k = 1; k < 8; ++k) before[k] = before[k - 1] + G[k - 1];
        const float schunk = after[0] + G[0];
        // weights: forward w_t = x_t * 2^(a_h * sum of dt2 after step t within the
        // chunk); reverse w_t = ds_t * 2^(a_h * sum of dt2 up to and including step t)
        bf16x8 ahi[2], alo[2];
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
            // the group's base without indexing by the lane's group (that would put
            // the arrays in scratch memory)
            const int k0 = grp * 4;
            const float (&base)[8] = REV ? before : after;
            float part = g == 0 ? base[k0] : g == 1 ? base[k0 + 1] : g == 2 ? base[k0 + 2] : base[k0 + 3];
            float w[8];
            if constexpr (REV) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    part += dt[grp][j];
                    w[j] = x[grp][j] * __builtin_amdgcn_exp2f(a_h * part);
                }
            } else {
#pragma unroll
                for (int j = 7; j >= 0; --j) {
                    w[j] = x[grp][j] * __builtin_amdgcn_exp2f(a_h * part);
                    part += dt[grp][j];
                }
            }
            split8(w, ahi[grp], alo[grp]);
        }
        // the chunk's decay of the rows this lane accumulates (channels 4g..4g+3)
        if (g == 0) sDec[chl] = __builtin_amdgcn_exp2f(a_h * schunk);
        __builtin_amdgcn_wave_barrier();
        const f32x4 dec = *reinterpret_cast<const f32x4*>(&sDec[16 * wv + 4 * g]);
        {
            const float yk = schunk - scomp;
            const float tk = ssum + yk;
            scomp = (tk - ssum) - yk;
            ssum = tk;
        }
        const uint16_t* bb = sB[q & 1] + (lane % 16) * kRowB + 8 * g;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc[j] *= dec;
            const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(bb + 16 * j * kRowB);
            const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(bb + 16 * j * kRowB + 32);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[0], b0, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[0], b0, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[1], b1, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[1], b1, acc[j], 0, 0, 0);
        }
        if (q + 1 < nq) {
            uint16_t* sb = sB[(q + 1) & 1];
#pragma unroll
            for (int k = 0; k < KBV; ++k)
                *reinterpret_cast<u32x4*>(&sb[((tid + k * kThreads) / 8) * kRowB + bcol]) = bv[k];
            d0 = d0n;
            u0 = u0n;
            d1 = d1n;
            u1 = u1n;
            z0 = z0n;
            z1 = z1n;
        }
        __syncthreads();
    }

    // H rows 16w+4g..+3 of column n = 16j + l%16, in the [n][64 channels] layout
    // (the forward's B carries the ln 2 of the log2 step sizes; the reverse's C none)
    float* hout = p.H + (blk * p.nchunks + piece) * int64_t(N) * kLanes;
    const float scale = REV ? 1.0f : kLn2;
#pragma unroll
    for (int j = 0; j < NT; ++j)
        *reinterpret_cast<f32x4*>(hout + int64_t(16 * j + lane % 16) * kLanes + 16 * wv + 4 * g) = acc[j] * scale;
    if (g == 0) p.S[(blk * p.nchunks + piece) * kLanes + chl] = ssum;
}

// Compose the pieces' affine maps in sequence order: one thread per (group, state, lane).
//   Hin[0] = h0 (or 0);  Hin[c+1] = exp2(A * S2[c]) * Hin[c] + H[c]     (S2 = sum of dt2)
__global__ void __launch_bounds__(256) scan_carry_kernel(Params p, int64_t total) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int lane = int(i % kLanes);
    const int64_t n = (i / kLanes) % p.np;
    const int64_t blk = i / (int64_t(kLanes) * p.np);
    const int64_t cblk = blk % p.nblk_d;
    const int64_t d = cblk * kLanes + lane;
    const int64_t b = blk / p.nblk_d;
    float a = 0.0f, hcur = 0.0f;
    if (d < p.dim && n < p.N) {
        a = p.head_dim ? p.A[d / p.head_dim] : p.A[d * p.N + n];
        if (p.h0) hcur = p.h0[(b * p.dim + d) * p.N + n];
    }
    for (int c = 0; c < p.nchunks; ++c) {
        const int64_t hidx = ((blk * p.nchunks + c) * p.np + n) * kLanes + lane;
        p.ws_Hin[hidx] = hcur;
        if (c + 1 < p.nchunks) {
            const float s = p.ws_S[(blk * p.nchunks + c) * kLanes + lane];
            hcur = fmaf(__builtin_amdgcn_exp2f(a * s), hcur, p.ws_H[hidx]);
        }
    }
}

// ------------------------------------------------------------------ decode step
// One token for every (batch, channel): h <- exp(dt*A) h + dt*B*u in place and
// y = (C.h + D*u) * SiLU(z).  The state round trip (8 bytes per entry) dominates:
// the kernel is bound by HBM.
//
// Vector form (N a multiple of 4, aligned rows): R lanes share one (batch, channel)
// row, each lane taking every R-th group of 4 entries, so that one load instruction
// covers 16*R contiguous bytes of every row it touches; the R partial read-outs are
// summed with lane shuffles.  Every lane computes the row's step size itself.  A
// lane may serve several rows (ROWS), issuing their loads together.
// Scalar form: one lane per row, entry by entry.
struct StepParams {
    const void* u;
    const void* delta;
    const void* z;        // nullable
    const void* Bm;       // (batch, N)
    const void* Cm;       // (batch, N)
    const float* A;
    const float* Dskip;   // nullable
    const float* bias;    // nullable
    float* h;             // (batch, dim, N), updated in place
    void* y;
    int64_t batch, dim, N, head_dim;
    // fused front end (conv_w != nullptr): `u` holds the new input x, conv_state the
    // previous conv_k-1 inputs (oldest first, updated in place), u = act(conv)
    const float* conv_w;  // (dim, conv_k)
    const float* conv_b;  // nullable
    void* conv_state;     // (batch, dim, conv_k-1), may be nullptr when conv_k == 1
    void* u_out;          // nullable
    int32_t conv_k;
    int32_t conv_silu;
};

// The scan input of row i (batch*dim + d) for this token: the stored u, or the fused
// convolution of the row's history and its new input.  When `update` is set the history
// is shifted in place: lane q of the row's R lanes writes entries q, q + R, ... (so the
// R lanes of consecutive rows store consecutive entries together) and lane 0 writes u
// to u_out.  All lanes of a row run in the same wave, so every lane reads the history
// before it is written.
template <typename IO>
__device__ inline float step_input(const StepParams& p, int64_t i, int64_t d, bool update, int q = 0, int R = 1) {
    const float x = IOT<IO>::to_f32(static_cast<const IO*>(p.u)[i]);
    if (!p.conv_w) return x;
    const int K = p.conv_k;
    const float* w = p.conv_w + d * K;
    IO* st = static_cast<IO*>(p.conv_state) + i * (K - 1);
    float acc = p.conv_b ? p.conv_b[d] : 0.0f;
    float hist[kMaxConv];
#pragma unroll
    for (int j = 0; j < kMaxConv - 1; ++j) hist[j] = (j < K - 1) ? IOT<IO>::to_f32(st[j]) : 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxConv - 1; ++j)
        if (j < K - 1) acc = fmaf(w[j], hist[j], acc);
    acc = fmaf(w[K - 1], x, acc);
    const float u = p.conv_silu ? silu_f32(acc) : acc;
    if (update) {
        // the shifted history: entry j takes entry j + 1, the last entry the new input
        const IO xin = static_cast<const IO*>(p.u)[i];
#pragma unroll
        for (int j = 0; j < kMaxConv - 1; ++j) {
            if (j < K - 1 && j % R == q) {
                IO v = xin;
#pragma unroll
                for (int k = 0; k + 1 < kMaxConv - 1; ++k)
                    if (j == k && k + 1 < K - 1) v = IOT<IO>::from_f32(hist[k + 1]);
                st[j] = v;
            }
        }
        if (p.u_out && q == 0) static_cast<IO*>(p.u_out)[i] = IOT<IO>::from_f32(u);
    }
    return u;
}

// 4 consecutive values of an I/O row as fp32 (16-byte or 8-byte aligned)
__device__ inline float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline float4 load4(const uint16_t* p) {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
}

template <typename IO, bool SCALAR>
__device__ inline void step_row_prologue(const StepParams& p, int64_t i, int64_t d, float& uu, float& dt2) {
    uu = step_input<IO>(p, i, d, true);
    const float dr = IOT<IO>::to_f32(static_cast<const IO*>(p.delta)[i]) + (p.bias ? p.bias[d] : 0.0f);
    dt2 = softplus_log2(dr);
}

template <typename IO>
__device__ inline void step_row_epilogue(const StepParams& p, int64_t i, int64_t d, float uu, float acc) {
    float o = acc + (p.Dskip ? p.Dskip[d] : 0.0f) * uu;
    if (p.z) o *= silu_f32(IOT<IO>::to_f32(static_cast<const IO*>(p.z)[i]));
    static_cast<IO*>(p.y)[i] = IOT<IO>::from_f32(o);
}

template <typename IO, bool SCALAR, int R, int ROWS>
__global__ void __launch_bounds__(256) scan_step_rows_kernel(StepParams p) {
    // lane group s takes rows s, s + S, ..., s + (ROWS-1) S (S lane groups in the grid),
    // so that each load instruction of a wave still covers consecutive rows; all
    // loads of the first 4-entry group of every row are issued before any arithmetic
    const int64_t rows = p.batch * p.dim;
    const int64_t S = int64_t(gridDim.x) * (256 / R);
    const int64_t s0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) / R;
    const int q = threadIdx.x % R;
    const int64_t n0 = 4 * q;   // < N, since 4 R <= N
    int64_t ri[ROWS];
    bool live[ROWS];
    float4 hv[ROWS], bv[ROWS], cv[ROWS], ar[ROWS];
    float uu[ROWS], dr[ROWS], zz[ROWS];
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
        const int64_t r = s0 + k * S;
        live[k] = r < rows;
        ri[k] = live[k] ? r : rows - 1;   // idle lanes read the last row, write nothing
        const int64_t b = ri[k] / p.dim, d = ri[k] % p.dim;
        hv[k] = *reinterpret_cast<const float4*>(p.h + ri[k] * p.N + n0);
        bv[k] = load4(static_cast<const IO*>(p.Bm) + b * p.N + n0);
        cv[k] = load4(static_cast<const IO*>(p.Cm) + b * p.N + n0);
        if constexpr (!SCALAR) ar[k] = *reinterpret_cast<const float4*>(p.A + d * p.N + n0);
        uu[k] = step_input<IO>(p, ri[k], ri[k] % p.dim, live[k], q, R);
        dr[k] = IOT<IO>::to_f32(static_cast<const IO*>(p.delta)[ri[k]]) + (p.bias ? p.bias[d] : 0.0f);
        zz[k] = p.z ? IOT<IO>::to_f32(static_cast<const IO*>(p.z)[ri[k]]) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
        const int64_t i = ri[k], b = i / p.dim, d = i % p.dim;
        const float dt2 = softplus_log2(dr[k]);
        const float x = dt2 * uu[k];
        const float a_s = SCALAR ? __builtin_amdgcn_exp2f(dt2 * p.A[d / p.head_dim]) : 0.0f;
        const IO* gB = static_cast<const IO*>(p.Bm) + b * p.N;
        const IO* gC = static_cast<const IO*>(p.Cm) + b * p.N;
        const float* Arow = p.A + d * p.N;
        float* hrow = p.h + i * p.N;
        float acc = 0.0f;
        auto group = [&](float4 h4, float4 b4, float4 c4, float4 a4, int64_t n) {
            float4 av = make_float4(a_s, a_s, a_s, a_s);
            if constexpr (!SCALAR)
                av = make_float4(__builtin_amdgcn_exp2f(dt2 * a4.x), __builtin_amdgcn_exp2f(dt2 * a4.y),
                                 __builtin_amdgcn_exp2f(dt2 * a4.z), __builtin_amdgcn_exp2f(dt2 * a4.w));
            h4.x = fmaf(av.x, h4.x, x * (b4.x * kLn2));
            h4.y = fmaf(av.y, h4.y, x * (b4.y * kLn2));
            h4.z = fmaf(av.z, h4.z, x * (b4.z * kLn2));
            h4.w = fmaf(av.w, h4.w, x * (b4.w * kLn2));
            acc = fmaf(c4.x, h4.x, acc);
            acc = fmaf(c4.y, h4.y, acc);
            acc = fmaf(c4.z, h4.z, acc);
            acc = fmaf(c4.w, h4.w, acc);
            if (live[k]) *reinterpret_cast<float4*>(hrow + n) = h4;
        };
        group(hv[k], bv[k], cv[k], ar[k], n0);
        for (int64_t n = n0 + 4 * R; n < p.N; n += 4 * R) {
            const float4 a4 = SCALAR ? make_float4(0.f, 0.f, 0.f, 0.f) : *reinterpret_cast<const float4*>(Arow + n);
            group(*reinterpret_cast<const float4*>(hrow + n), load4(gB + n), load4(gC + n), a4, n);
        }
#pragma unroll
        for (int off = R / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, R);
        if (live[k] && q == 0) {
            float o = acc + (p.Dskip ? p.Dskip[d] : 0.0f) * uu[k];
            if (p.z) o *= silu_f32(zz[k]);
            static_cast<IO*>(p.y)[i] = IOT<IO>::from_f32(o);
        }
    }
}

template <typename IO, bool SCALAR>
__global__ void __launch_bounds__(256) scan_step_kernel(StepParams p) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= p.batch * p.dim) return;
    const int64_t b = i / p.dim, d = i % p.dim;
    float uu, dt2;
    step_row_prologue<IO, SCALAR>(p, i, d, uu, dt2);
    const float x = dt2 * uu;
    const float a_s = SCALAR ? __builtin_amdgcn_exp2f(dt2 * p.A[d / p.head_dim]) : 0.0f;
    const IO* gB = static_cast<const IO*>(p.Bm) + b * p.N;
    const IO* gC = static_cast<const IO*>(p.Cm) + b * p.N;
    const float* Arow = p.A + d * p.N;
    float* hrow = p.h + i * p.N;
    float acc = 0.0f;
    for (int64_t n = 0; n < p.N; ++n) {
        const float a = SCALAR ? a_s : __builtin_amdgcn_exp2f(dt2 * Arow[n]);
        const float hn = fmaf(a, hrow[n], x * (IOT<IO>::to_f32(gB[n]) * kLn2));
        acc = fmaf(IOT<IO>::to_f32(gC[n]), hn, acc);
        hrow[n] = hn;
    }
    step_row_epilogue<IO>(p, i, d, uu, acc);
}

// lanes per row of the vector form: the largest power of two <= min(N/4, 16)
inline int step_lanes(int64_t N) {
    int r = 1;
    while (r < 16 && 4 * (2 * r) <= N) r *= 2;
    return r;
}

template <typename IO, bool SCALAR>
hipError_t launch_step(const StepParams& p, bool vec4, hipStream_t s) {
    const int64_t rows = p.batch * p.dim;
    const dim3 block(256);
    if (!vec4) {
        launch_kernel((scan_step_kernel<IO, SCALAR>), dim3(unsigned(cdiv(rows, 256))), block, 0, s, p);
        return ssm_detail::launch_error;
    }
    const int R = step_lanes(p.N);
    constexpr int ROWS = 1;   // measured: 4 rows per lane (a quarter of the waves) was slower
    const dim3 grid(unsigned(cdiv(rows * R, 256 * ROWS)));
    switch (R) {
        case 1: launch_kernel((scan_step_rows_kernel<IO, SCALAR, 1, ROWS>), grid, block, 0, s, p); break;
        case 2: launch_kernel((scan_step_rows_kernel<IO, SCALAR, 2, ROWS>), grid, block, 0, s, p); break;
        case 4: launch_kernel((scan_step_rows_kernel<IO, SCALAR, 4, ROWS>), grid, block, 0, s, p); break;
        case 8: launch_kernel((scan_step_rows_kernel<IO, SCALAR, 8, ROWS>), grid, block, 0, s, p); break;
        default: launch_kernel((scan_step_rows_kernel<IO, SCALAR, 16, ROWS>), grid, block, 0, s, p); break;
    }
    return ssm_detail::launch_error;
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
    int form;           // 0: lane walk; 1: chunked form on the matrix cores (scan_chunked.hip)
};


int make_plan(const ssm_dims* d, Plan* pl) {
    int st = validate_dims(d);
    if (st != SSM_OK) return st;
    const int64_t N = d->dstate;
    pl->scalar = d->nheads > 0;
    int spl = d->states_per_lane;
    if (spl == 0) {
        // aim for 4 waves per workgroup (scalar decay: 8), at most 16 states per lane
        const int64_t target_waves = pl->scalar ? 8 : 4;
        // (with fewer state entries than waves, lanes carry one entry each)
        spl = 1;
        while (spl < 16 && cdiv(N, spl) > target_waves) spl *= 2;
    }
    if (cdiv(N, spl) > 16) return SSM_ERR_DIMS;       // more than 1024 threads
    pl->spl = spl;
    // waves per workgroup, rounded up to 4, 8 or 16 (state entries beyond N are padding)
    const int64_t g = cdiv(N, spl);
    pl->G = g <= 4 ? 4 : (g <= 8 ? 8 : 16);
    // time tile: 32 steps for 4 walking waves of up to 8 entries per lane, else 16,
    // so that the (double-buffered) LDS tiles fit the 160 KB of a CU
    pl->T = tile_len(pl->G, spl);
    pl->nblk_d = cdiv(d->dim, kLanes);
    const int64_t groups = d->batch * pl->nblk_d;
    const int64_t tiles = cdiv(d->seqlen, pl->T);
    // A scalar decay with bf16 rows of 64 or 128 states and the library's choice of
    // states per lane runs its full pass in the chunked form (when, at the call, the rows
    // also allow 16-byte loads; else the walk runs with the same pieces).
    const int64_t rows_bytes = (N > kLanes ? N : kLanes) * d->seqlen * 2;
    pl->form = (pl->scalar && d->io_dtype == SSM_BF16 && ssm_detail::chunked_supported(N) &&
                d->states_per_lane == 0 && d->seqlen % 8 == 0 && pl->T == 16 && rows_bytes < (int64_t(1) << 31))
                   ? 1 : 0;
    int64_t nch = d->nchunks;
    if (nch == 0 && pl->form == 1) {
        // The chunked pass holds 3 workgroups per CU (160 VGPRs: three waves per SIMD);
        // its pieces' carries come from the matrix-core aggregate, so aim for one full
        // round of 3 x 256 workgroups, at least 8 tiles per piece.
        const int64_t slots = 3 * 256;
        const int64_t max_pieces = tiles / 8 > 1 ? tiles / 8 : 1;
        nch = cdiv(slots, groups);
        const int64_t cap = max_pieces < SSM_MAX_CHUNKS ? max_pieces : SSM_MAX_CHUNKS;
        nch = round_friendly_pieces(groups, nch, cap, slots);
        if (nch > cap) nch = cap;
        if (nch < 1) nch = 1;
    } else if (nch == 0) {
        // One wave per SIMD (256 CUs x 4 SIMDs) is the floor below which the sequence is
        // cut into pieces; pieces cost a second pass over all but the last, so cut
        // only when the machine would otherwise be at most half busy.
        // Also cut when the workgroups (one CU each: their LDS tiles take most of a
        // CU's 160 KB) would leave at least half of the 256 CUs idle.
        const int64_t waves = groups * pl->G;
        const int64_t cus = 256;
        nch = 1;
        if (waves * 2 <= 1024) nch = cdiv(2048, waves);
        if (groups * 2 <= cus && cdiv(cus, groups) > nch) nch = cdiv(cus, groups);
        // With a scalar decay and bf16 rows of 32, 64 or 128 states the first pass runs on
        // the matrix cores (scan_piece_states_kernel) and pieces are cheap: aim for two
        // workgroups per CU (the per-channel scalar-decay workload, 128 groups: 1.00 ms in
        // 4 pieces against 1.05 ms in 2).
        const bool cheap_pieces = pl->scalar && d->io_dtype == SSM_BF16 && pl->G * spl == N &&
                                  (N == 32 || N == 64 || N == 128) && d->seqlen % 8 == 0;
        if (cheap_pieces && groups < 2 * cus && cdiv(2 * cus, groups) > nch) nch = cdiv(2 * cus, groups);
        const int64_t max_pieces = tiles / 8 > 1 ? tiles / 8 : 1;   // keep >= 8 tiles per piece
        // then the piece count, up to twice that, that leaves no part-filled last round
        // of workgroups (long sequence, 32 groups of 64 channels: 12 pieces 2.60 ms, 16
        // pieces 1.97 ms, 20 pieces 2.33 ms)
        const int64_t per_cu = int64_t(163840 / lds_floats_g(pl->G, spl, true) / sizeof(float));
        const int64_t cap = max_pieces < SSM_MAX_CHUNKS ? max_pieces : SSM_MAX_CHUNKS;
        nch = round_friendly_pieces(groups, nch, cap, cus * (per_cu > 1 ? per_cu : 1));
        if (nch > max_pieces) nch = max_pieces;
        if (nch > SSM_MAX_CHUNKS) nch = SSM_MAX_CHUNKS;
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
    pl->lds_bytes = pl->form == 1 ? ssm_detail::chunked_lds_bytes(N) : lds_floats_g(pl->G, spl, true) * sizeof(float);
    return SSM_OK;
}

// ------------------------------------------------------------------ host side: launching
template <typename IO, int SPL, bool SCALAR, bool VEC, int G, bool CK = false, bool CONV = false>
hipError_t launch_all(const Params& p, const Plan& pl, hipStream_t stream) {
    using S = Shape<G, SPL>;
    if (pl.G != G || pl.T != S::T || p.np != G * SPL) return hipErrorInvalidConfiguration;
    const dim3 block(unsigned(S::NW * kLanes));
    const size_t lds_full = lds_floats_g(G, SPL, true) * sizeof(float);
    const size_t lds_agg = lds_floats_g(G, SPL, false) * sizeof(float);
    if (pl.nchunks > 1) {
        const int64_t groups = int64_t(p.batch) * p.nblk_d;
        // pass 1 on every piece but the last: on the matrix cores when the decay is a
        // scalar per head and the rows allow 16-byte loads, else by walking.  The matrix
        // form reads the scan input from `u` directly, so it is not used with the fused
        // convolution front end (whose `u` rows hold the convolution's input).
        const dim3 grid1(unsigned(groups * (pl.nchunks - 1)));
        bool done = false;
        if constexpr (SCALAR && VEC && !CONV && std::is_same<IO, uint16_t>::value) {
            if (p.np == p.N) {
                ssm_detail::PieceStatesArgs a;
                a.x = p.u;
                a.delta = p.delta;
                a.z = nullptr;
                a.BC = p.Bm;
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
                a.piece_base = 0;
                a.H = p.ws_H;
                a.S = p.ws_S;
                done = ssm_detail::launch_piece_states(a, false, pl.nchunks - 1, stream);
            }
        }
        if (!done)
            launch_kernel((scan_fwd_kernel<IO, SPL, SCALAR, kAggregate, VEC, G, false, CONV>), grid1, block, lds_agg,
                               stream, p);
        const int64_t total = groups * p.np * kLanes;
        launch_kernel(scan_carry_kernel, dim3(unsigned(cdiv(total, 256))), dim3(256), 0, stream, p, total);
    }
    if constexpr (SCALAR && VEC && !CONV && !CK && std::is_same<IO, uint16_t>::value) {
        if (pl.form == 1) {
            ssm_detail::ChunkedArgs a;
            a.u = p.u;
            a.delta = p.delta;
            a.z = p.z;
            a.B = p.Bm;
            a.C = p.Cm;
            a.A = p.A;
            a.D = p.Dskip;
            a.bias = p.bias;
            a.y = p.y;
            a.h0 = p.h0;
            a.h_last = p.h_last;
            a.Hin = p.ws_Hin;
            a.L = p.L;
            a.dim = p.dim;
            a.nstate = p.N;
            a.head_dim = p.head_dim;
            a.chunk_len = p.chunk_len;
            a.nchunks = p.nchunks;
            a.nblk_d = p.nblk_d;
            a.batch = p.batch;
            if (ssm_detail::launch_chunked(a, stream)) return ssm_detail::launch_error;
        }
    }
    launch_kernel((scan_fwd_kernel<IO, SPL, SCALAR, kFull, VEC, G, CK, CONV>), dim3(unsigned(pl.blocks)), block,
                       lds_full, stream, p);
    return ssm_detail::launch_error;
}

// One instantiation per (states per lane, waves per workgroup) pair the planner can
// produce: waves are 4, 8 or 16 and states per lane 1..16.
template <typename IO, bool SCALAR, bool VEC, int G, bool CONV>
hipError_t dispatch_spl_c(const Params& p, const Plan& pl, hipStream_t s) {
    switch (pl.spl) {
        case 1: return launch_all<IO, 1, SCALAR, VEC, G, false, CONV>(p, pl, s);
        case 2: return launch_all<IO, 2, SCALAR, VEC, G, false, CONV>(p, pl, s);
        case 4: return launch_all<IO, 4, SCALAR, VEC, G, false, CONV>(p, pl, s);
        case 8: return launch_all<IO, 8, SCALAR, VEC, G, false, CONV>(p, pl, s);
        default: return launch_all<IO, 16, SCALAR, VEC, G, false, CONV>(p, pl, s);
    }
}

template <typename IO, bool SCALAR, bool VEC, int G>
hipError_t dispatch_spl(const Params& p, const Plan& pl, hipStream_t s) {
    return p.conv_w ? dispatch_spl_c<IO, SCALAR, VEC, G, true>(p, pl, s)
                    : dispatch_spl_c<IO, SCALAR, VEC, G, false>(p, pl, s);
}

template <typename IO, bool SCALAR, bool VEC>
hipError_t dispatch_g(const Params& p, const Plan& pl, hipStream_t s) {
    if (pl.G == 4) return dispatch_spl<IO, SCALAR, VEC, 4>(p, pl, s);
    if (pl.G == 8) return dispatch_spl<IO, SCALAR, VEC, 8>(p, pl, s);
    return dispatch_spl<IO, SCALAR, VEC, 16>(p, pl, s);
}

template <typename IO, bool SCALAR>
hipError_t dispatch_nt(const Params& p, const Plan& pl, bool vec, hipStream_t s) {
    return vec ? dispatch_g<IO, SCALAR, true>(p, pl, s) : dispatch_g<IO, SCALAR, false>(p, pl, s);
}

template <typename IO>
hipError_t dispatch(const Params& p, const Plan& pl, bool vec, hipStream_t s) {
    return pl.scalar ? dispatch_nt<IO, true>(p, pl, vec, s) : dispatch_nt<IO, false>(p, pl, vec, s);
}

// Plans with a checkpointing kernel: the automatic plans for 9..16 state entries
// (diagonal decay: 4 walking waves of 4 entries; scalar decay: 8 of 2).
inline bool ckpt_plan(const Plan& pl) {
    return pl.G * pl.spl == 16 && ((!pl.scalar && pl.spl == 4 && pl.G == 4) || (pl.scalar && pl.spl == 2 && pl.G == 8));
}

template <typename IO, bool VEC>
hipError_t dispatch_ckpt_vec(const Params& p, const Plan& pl, hipStream_t s) {
    if (!pl.scalar && pl.spl == 4 && pl.G == 4) return launch_all<IO, 4, false, VEC, 4, true>(p, pl, s);
    if (pl.scalar && pl.spl == 2 && pl.G == 8) return launch_all<IO, 2, true, VEC, 8, true>(p, pl, s);
    return hipErrorInvalidConfiguration;
}

template <typename IO>
hipError_t dispatch_ckpt(const Params& p, const Plan& pl, bool vec, hipStream_t s) {
    return vec ? dispatch_ckpt_vec<IO, true>(p, pl, s) : dispatch_ckpt_vec<IO, false>(p, pl, s);
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
        case SSM_ERR_ALIAS: return "an output or the workspace overlaps an input or another output";
        case SSM_ERR_DEVICE: return "the stream belongs to a device other than the current one";
        case SSM_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point holds";
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
    plan->form = pl.form;
    plan->reserved = 0;
    return SSM_OK;
}

size_t ssm_selective_scan_workspace_bytes(const ssm_dims* dims) {
    Plan pl;
    if (make_plan(dims, &pl) != SSM_OK) return 0;
    return pl.ws_bytes;
}

}  // extern "C"

namespace {

// The forward entry points share this: the plain scan (conv == nullptr) or the scan of
// u = act(conv(x)) with x at `u` (conv != nullptr).
int fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
             const void* z, const float* dt_bias, const float* h0, void* y, float* h_last, const ssm_dims* dims,
             void* stream, const ssm_conv* conv, const void* conv_state, void* u_out, bool with_ckpt = false,
             float* ckpt = nullptr) {
    if (!dims) return SSM_ERR_NULL;
    Plan pl;
    int st = make_plan(dims, &pl);
    if (st != SSM_OK) return st;
    if (with_ckpt && (ssm_selective_scan_ckpt_bytes(dims) == 0 || !ckpt_plan(pl))) return SSM_ERR_DIMS;
    if (!u || !delta || !A || !B || !C || !y || (with_ckpt && !ckpt)) return SSM_ERR_NULL;

    const size_t esz = dims->io_dtype == SSM_BF16 ? 2 : 4;
    if (misaligned(u, esz) || misaligned(delta, esz) || misaligned(z, esz) || misaligned(B, esz) ||
        misaligned(C, esz) || misaligned(y, esz) || misaligned(A, 4) || misaligned(D, 4) || misaligned(dt_bias, 4) ||
        misaligned(h0, 4) || misaligned(h_last, 4) || misaligned(ckpt, 4))
        return SSM_ERR_ALIGN;

    const size_t nel = size_t(dims->batch) * dims->dim * dims->seqlen * esz;
    const size_t nbc = size_t(dims->batch) * dims->dstate * dims->seqlen * esz;
    const size_t na = (dims->nheads > 0 ? size_t(dims->nheads) : size_t(dims->dim) * dims->dstate) * 4;
    const size_t nd = size_t(dims->dim) * 4;
    const size_t nh = size_t(dims->batch) * dims->dim * dims->dstate * 4;
    if (overlaps(y, nel, u, nel) || overlaps(y, nel, delta, nel) || overlaps(y, nel, z, nel) ||
        overlaps(y, nel, B, nbc) || overlaps(y, nel, C, nbc) || overlaps(y, nel, A, na) ||
        overlaps(y, nel, D, nd) || overlaps(y, nel, dt_bias, nd) || overlaps(y, nel, h0, nh) ||
        overlaps(y, nel, h_last, nh))
        return SSM_ERR_ALIAS;
    // h_last may be h0 itself (an in-place state update) but no other input
    if (h_last && ((h0 != h_last && overlaps(h_last, nh, h0, nh)) || overlaps(h_last, nh, u, nel) ||
                   overlaps(h_last, nh, delta, nel) || overlaps(h_last, nh, z, nel) || overlaps(h_last, nh, B, nbc) ||
                   overlaps(h_last, nh, C, nbc) || overlaps(h_last, nh, A, na) || overlaps(h_last, nh, D, nd) ||
                   overlaps(h_last, nh, dt_bias, nd)))
        return SSM_ERR_ALIAS;

    if (conv) {
        if (!conv->weight) return SSM_ERR_NULL;
        if (conv->width < 1 || conv->width > kMaxConv || (conv->silu != 0 && conv->silu != 1)) return SSM_ERR_DIMS;
        const size_t nw = size_t(dims->dim) * conv->width * 4;
        const size_t ns = size_t(dims->batch) * dims->dim * (conv->width - 1) * esz;
        if (misaligned(conv->weight, 4) || misaligned(conv->bias, 4) || misaligned(conv_state, esz) ||
            misaligned(u_out, esz))
            return SSM_ERR_ALIGN;
        // u_out is an output like y: it may overlap no input and no other output
        const void* ins[] = {u, delta, z, B, C, A, D, dt_bias, h0, conv->weight, conv->bias, conv_state};
        const size_t sizes[] = {nel, nel, nel, nbc, nbc, na, nd, nd, nh, nw, nd, ns};
        for (int k = 0; k < 12; ++k)
            if (overlaps(u_out, nel, ins[k], sizes[k]) || overlaps(y, nel, ins[k], sizes[k]) ||
                (h_last && k >= 9 && overlaps(h_last, nh, ins[k], sizes[k])))
                return SSM_ERR_ALIAS;
        if (overlaps(u_out, nel, y, nel) || overlaps(u_out, nel, h_last, nh)) return SSM_ERR_ALIAS;
    } else if (conv_state || u_out) {
        return SSM_ERR_DIMS;
    }

    if (pl.ws_bytes > 0) {
        if (!dims->workspace || dims->workspace_bytes < pl.ws_bytes ||
            (reinterpret_cast<uintptr_t>(dims->workspace) % 256) != 0)
            return SSM_ERR_WORKSPACE;
        // the carry passes write the workspace before the full pass reads the inputs, so
        // it may overlap no input and no output
        const size_t nw = conv ? size_t(dims->dim) * conv->width * 4 : 0;
        const size_t ns = conv ? size_t(dims->batch) * dims->dim * (conv->width - 1) * esz : 0;
        const void* all[] = {u,  delta, z,      B,     C,     A,  D, dt_bias, h0, y, h_last, u_out,
                             conv ? conv->weight : nullptr, conv ? conv->bias : nullptr, conv_state};
        const size_t all_sz[] = {nel, nel, nel, nbc, nbc, na, nd, nd, nh, nel, nh, nel, nw, nd, ns};
        for (int k = 0; k < 15; ++k)
            if (overlaps(dims->workspace, pl.ws_bytes, all[k], all_sz[k])) return SSM_ERR_ALIAS;
    }

    if (with_ckpt) {
        // the checkpoints are an output: they may overlap no input, no other output
        // and no workspace
        const size_t nck = ssm_selective_scan_ckpt_bytes(dims);
        const void* all[] = {u, delta, z, B, C, A, D, dt_bias, h0, y, h_last};
        const size_t all_sz[] = {nel, nel, nel, nbc, nbc, na, nd, nd, nh, nel, nh};
        for (int k = 0; k < 11; ++k)
            if (overlaps(ckpt, nck, all[k], all_sz[k])) return SSM_ERR_ALIAS;
        if (pl.ws_bytes > 0 && overlaps(ckpt, nck, dims->workspace, pl.ws_bytes)) return SSM_ERR_ALIAS;
    }

    // vector (16-byte) loads need 16-byte aligned rows: aligned base pointers and a
    // row length that is a whole number of vectors
    const size_t vw = 16 / esz;
    auto a16 = [](const void* q) { return !q || (reinterpret_cast<uintptr_t>(q) % 16) == 0; };
    // (the kernels' buffer windows also need a block's 64 rows and a batch row's dstate
    // rows to span less than 2^31 bytes)
    const int64_t rows_bytes = (dims->dstate > kLanes ? dims->dstate : kLanes) * dims->seqlen * int64_t(esz);
    const bool vec = (dims->seqlen % int64_t(vw)) == 0 && a16(u) && a16(delta) && a16(z) && a16(B) && a16(C) &&
                     a16(y) && rows_bytes < (int64_t(1) << 31);

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
    p.h0 = h0;
    p.h_last = h_last;
    p.conv_w = conv ? conv->weight : nullptr;
    p.conv_b = conv ? conv->bias : nullptr;
    p.conv_state = conv ? conv_state : nullptr;
    p.u_out = conv ? u_out : nullptr;
    p.conv_k = conv ? conv->width : 0;
    p.conv_silu = conv ? conv->silu : 0;
    p.ckpt = with_ckpt ? ckpt : nullptr;
    p.ntiles_ck = cdiv(dims->seqlen, kCkptSteps);
    p.ws_H = p.ws_S = p.ws_Hin = nullptr;
    if (pl.ws_bytes > 0) {
        const size_t per = size_t(dims->batch) * pl.nblk_d * pl.nchunks * kLanes;
        float* base = static_cast<float*>(dims->workspace);
        p.ws_H = base;
        p.ws_Hin = base + per * p.np;
        p.ws_S = base + 2 * per * p.np;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    ssm_detail::launch_error = hipSuccess;   // this call's launch failures only (the caller's pending HIP error is left alone)
    hipError_t e;
    if (with_ckpt)
        e = dims->io_dtype == SSM_BF16 ? dispatch_ckpt<uint16_t>(p, pl, vec, s) : dispatch_ckpt<float>(p, pl, vec, s);
    else
        e = dims->io_dtype == SSM_BF16 ? dispatch<uint16_t>(p, pl, vec, s) : dispatch<float>(p, pl, vec, s);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_selective_scan_fwd_state(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                 const float* D, const void* z, const float* dt_bias, const float* h0, void* y,
                                 float* h_last, const ssm_dims* dims, void* stream) {
    return fwd_impl(u, delta, A, B, C, D, z, dt_bias, h0, y, h_last, dims, stream, nullptr, nullptr, nullptr);
}

int ssm_selective_scan_fwd_conv(const void* x, const ssm_conv* conv, const void* conv_state, const void* delta,
                                const float* A, const void* B, const void* C, const float* D, const void* z,
                                const float* dt_bias, const float* h0, void* u_out, void* y, float* h_last,
                                const ssm_dims* dims, void* stream) {
    if (!conv) return SSM_ERR_NULL;
    return fwd_impl(x, delta, A, B, C, D, z, dt_bias, h0, y, h_last, dims, stream, conv, conv_state, u_out);
}

int ssm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* dt_bias, void* y, const ssm_dims* dims,
                           void* stream) {
    return ssm_selective_scan_fwd_state(u, delta, A, B, C, D, z, dt_bias, nullptr, y, nullptr, dims, stream);
}

size_t ssm_selective_scan_ckpt_bytes(const ssm_dims* dims) {
    if (validate_dims(dims) != SSM_OK) return 0;
    if (dims->dstate < 9 || dims->dstate > 16 || dims->states_per_lane != 0) return 0;
    return size_t(dims->batch) * size_t(cdiv(dims->dim, kLanes)) * size_t(cdiv(dims->seqlen, kCkptSteps)) * 16 *
           kLanes * sizeof(float);
}

int ssm_selective_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                const float* D, const void* z, const float* dt_bias, const float* h0, void* y,
                                float* h_last, float* ckpt, const ssm_dims* dims, void* stream) {
    return fwd_impl(u, delta, A, B, C, D, z, dt_bias, h0, y, h_last, dims, stream, nullptr, nullptr, nullptr, true,
                    ckpt);
}

}  // extern "C"

// ------------------------------------------------------------------ the entry point that allocates nothing
// For callers that cannot allocate device memory (code under graph capture, tight
// serving loops): the carries between the pieces of a sequence live in this
// file-scope array instead of a caller workspace.  Each device holds its own copy,
// from the moment the library's code object is loaded until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of `scratch` on the current device, which must be the device of
// `stream` (a NULL stream is the current device's).
int scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSM_ERR_HIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SSM_ERR_HIP;
        if (int(sdev) != dev) return SSM_ERR_DEVICE;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return SSM_ERR_HIP;
    *out = g_scratch_ptr[dev];
    return SSM_OK;
}

}  // namespace

extern "C" {

size_t ssm_selective_scan_noalloc_scratch_bytes(void) { return SSM_NOALLOC_SCRATCH_BYTES; }

int ssm_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                   const float* D, const void* z, const float* dt_bias, const float* h0, void* y,
                                   float* h_last, const ssm_dims* dims, void* stream) {
    if (!dims) return SSM_ERR_NULL;
    Plan pl;
    const int st = make_plan(dims, &pl);
    if (st != SSM_OK) return st;
    if (pl.ws_bytes > SSM_NOALLOC_SCRATCH_BYTES) return SSM_ERR_SCRATCH;
    ssm_dims d = *dims;   // the caller's workspace fields are ignored
    d.workspace = nullptr;
    d.workspace_bytes = 0;
    if (pl.ws_bytes > 0) {
        void* ptr = nullptr;
        const int sst = scratch_address(static_cast<hipStream_t>(stream), &ptr);
        if (sst != SSM_OK) return sst;
        d.workspace = ptr;
        d.workspace_bytes = SSM_NOALLOC_SCRATCH_BYTES;
    }
    return fwd_impl(u, delta, A, B, C, D, z, dt_bias, h0, y, h_last, &d, stream, nullptr, nullptr, nullptr);
}

}  // extern "C"

namespace {

int step_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
              const void* z, const float* dt_bias, float* h, void* y, const ssm_dims* dims, void* stream,
              const ssm_conv* conv, void* conv_state, void* u_out) {
    const int st = validate_dims(dims);
    if (st != SSM_OK) return st;
    if (dims->seqlen != 1) return SSM_ERR_DIMS;
    if (!u || !delta || !A || !B || !C || !h || !y) return SSM_ERR_NULL;
    const size_t esz = dims->io_dtype == SSM_BF16 ? 2 : 4;
    if (misaligned(u, esz) || misaligned(delta, esz) || misaligned(z, esz) || misaligned(B, esz) ||
        misaligned(C, esz) || misaligned(y, esz) || misaligned(A, 4) || misaligned(D, 4) || misaligned(dt_bias, 4) ||
        misaligned(h, 4))
        return SSM_ERR_ALIGN;
    const size_t nel = size_t(dims->batch) * dims->dim * esz;
    const size_t nbc = size_t(dims->batch) * dims->dstate * esz;
    const size_t na = (dims->nheads > 0 ? size_t(dims->nheads) : size_t(dims->dim) * dims->dstate) * 4;
    const size_t nd = size_t(dims->dim) * 4;
    const size_t nh = size_t(dims->batch) * dims->dim * dims->dstate * 4;
    const void* ins[] = {u, delta, z, B, C, A, D, dt_bias};
    const size_t sizes[] = {nel, nel, nel, nbc, nbc, na, nd, nd};
    for (int k = 0; k < 8; ++k)
        if (overlaps(y, nel, ins[k], sizes[k]) || overlaps(h, nh, ins[k], sizes[k])) return SSM_ERR_ALIAS;
    if (overlaps(y, nel, h, nh)) return SSM_ERR_ALIAS;
    if (conv) {
        if (!conv->weight) return SSM_ERR_NULL;
        if (conv->width < 1 || conv->width > kMaxConv || (conv->silu != 0 && conv->silu != 1)) return SSM_ERR_DIMS;
        if (conv->width > 1 && !conv_state) return SSM_ERR_NULL;
        if (misaligned(conv->weight, 4) || misaligned(conv->bias, 4) || misaligned(conv_state, esz) ||
            misaligned(u_out, esz))
            return SSM_ERR_ALIGN;
        const size_t nw = size_t(dims->dim) * conv->width * 4;
        const size_t ns = size_t(dims->batch) * dims->dim * (conv->width - 1) * esz;
        // conv_state is read and written (in place); u_out is written: neither may
        // overlap any other array
        const void* all[] = {u, delta, z, B, C, A, D, dt_bias, conv->weight, conv->bias, h, y};
        const size_t all_sz[] = {nel, nel, nel, nbc, nbc, na, nd, nd, nw, nd, nh, nel};
        for (int k = 0; k < 12; ++k)
            if (overlaps(conv_state, ns, all[k], all_sz[k]) || overlaps(u_out, nel, all[k], all_sz[k]))
                return SSM_ERR_ALIAS;
        if ((overlaps(conv_state, ns, u_out, nel)) ||
            overlaps(h, nh, conv->weight, nw) || overlaps(h, nh, conv->bias, nd) ||
            overlaps(y, nel, conv->weight, nw) || overlaps(y, nel, conv->bias, nd))
            return SSM_ERR_ALIAS;
    } else if (conv_state || u_out) {
        return SSM_ERR_DIMS;
    }

    StepParams p;
    p.u = u;
    p.delta = delta;
    p.z = z;
    p.Bm = B;
    p.Cm = C;
    p.A = A;
    p.Dskip = D;
    p.bias = dt_bias;
    p.h = h;
    p.y = y;
    p.batch = dims->batch;
    p.dim = dims->dim;
    p.N = dims->dstate;
    p.head_dim = dims->nheads > 0 ? dims->dim / dims->nheads : 0;
    p.conv_w = conv ? conv->weight : nullptr;
    p.conv_b = conv ? conv->bias : nullptr;
    p.conv_state = conv ? conv_state : nullptr;
    p.u_out = conv ? u_out : nullptr;
    p.conv_k = conv ? conv->width : 0;
    p.conv_silu = conv ? conv->silu : 0;
    // the vector form reads 4 entries at once: rows of h and A 16-byte aligned, of B and C 4*esz
    const bool vec4 = dims->dstate % 4 == 0 && !misaligned(h, 16) && !misaligned(B, 4 * esz) &&
                      !misaligned(C, 4 * esz) && (dims->nheads > 0 || !misaligned(A, 16));
    if (cdiv(dims->batch * dims->dim * 16, 256) > 0x7fffffff) return SSM_ERR_DIMS;
    const bool scalar = dims->nheads > 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    ssm_detail::launch_error = hipSuccess;   // this call's launch failures only (the caller's pending HIP error is left alone)
    hipError_t e;
    if (dims->io_dtype == SSM_BF16)
        e = scalar ? launch_step<uint16_t, true>(p, vec4, s) : launch_step<uint16_t, false>(p, vec4, s);
    else
        e = scalar ? launch_step<float, true>(p, vec4, s) : launch_step<float, false>(p, vec4, s);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_selective_scan_step(const void* u, const void* delta, const float* A, const void* B, const void* C,
                            const float* D, const void* z, const float* dt_bias, float* h, void* y,
                            const ssm_dims* dims, void* stream) {
    return step_impl(u, delta, A, B, C, D, z, dt_bias, h, y, dims, stream, nullptr, nullptr, nullptr);
}

int ssm_selective_scan_step_conv(const void* x, const ssm_conv* conv, void* conv_state, const void* delta,
                                 const float* A, const void* B, const void* C, const float* D, const void* z,
                                 const float* dt_bias, float* h, void* u_out, void* y, const ssm_dims* dims,
                                 void* stream) {
    if (!conv) return SSM_ERR_NULL;
    return step_impl(x, delta, A, B, C, D, z, dt_bias, h, y, dims, stream, conv, conv_state, u_out);
}

}  // extern "C"

namespace ssm_detail {

bool launch_piece_states(const PieceStatesArgs& a, bool reverse, int64_t npieces, hipStream_t s) {
    const dim3 grid(unsigned(int64_t(a.batch) * a.nblk_d * npieces)), block(agg::kThreads);
#define SSM_PIECE_CASE(N_)                                                                              \
    case N_:                                                                                            \
        if (reverse)                                                                                    \
            launch_kernel((scan_piece_states_kernel<N_, true>), grid, block, 0, s, a);             \
        else                                                                                            \
            launch_kernel((scan_piece_states_kernel<N_, false>), grid, block, 0, s, a);            \
        return true;
    switch (a.nstate) {
        SSM_PIECE_CASE(32)
        SSM_PIECE_CASE(64)
        SSM_PIECE_CASE(128)
        default: return false;
    }
#undef SSM_PIECE_CASE
}

}  // namespace ssm_detail
