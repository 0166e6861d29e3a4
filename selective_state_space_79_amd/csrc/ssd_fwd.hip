// ssd_fwd.hip -- the scalar-decay selective scan with one step size per head, computed
// in its chunked state-space-duality form with every contraction on the gfx950 matrix
// cores (v_mfma_f32_16x16x32_bf16).
//
// What it computes is the recurrence of ssm.h for a head h whose channels share the
// decay A = a_h * I and the step size dt[b,h,t] = softplus(delta[b,h,t] + dt_bias[h])
// (the entry point ssm_ssd_fwd).  When the state matrix is a scalar times the
// identity, the scan equals a masked linear attention, and a chunked algorithm can
// process blocks of tokens on chip (yo3nglau.github.io "Mamba 与状态空间模型：面试问题与
// 推荐回答" Q10).  For a chunk of kQ steps entered with the per-head state Hin
// (N x P, one column per channel) and cum_t = sum_{k<=t} dt_k a_h inside the chunk:
//
//   y[t,p] = sum_{s<=t} G[t,s] exp(cum_t - cum_s) dt_s u[s,p]  +  exp(cum_t) sum_n C[n,t] Hin[n,p]
//   Hout   = exp(cum_last) Hin + sum_s exp(cum_last - cum_s) dt_s B[:,s] u[s,:]
//
// with G[t,s] = sum_n C[n,t] B[n,s]; then y = (y + D u) SiLU(z) as in the recurrence.
// The four products (G, the masked-decay product, the read of Hin, the chunk's state
// contribution) are MFMA tiles.  G's operands are the bf16 inputs themselves; the
// other products multiply a bf16 input by an fp32 value (the decayed mask, the
// weighted inputs, the state), which is split into a high and a low bf16 part and
// multiplied twice, so the operand carries ~2^-16 relative error instead of bf16's
// 2^-9 (plain bf16 operands exceed a 2e-2 output error on the N = 128 workload).
// Products accumulate in fp32.
//
// Work split: ssd_gram_kernel forms C^T B of every chunk once for all heads.  A sequence
// is cut into segments of whole chunks, and each segment before the last into pieces.
// ssd_state_kernel (ssd_state_dma_kernel with 16-byte rows) computes each such piece's
// end state from a zero start (and its total decay); ssd_out_kernel composes the states of the pieces before its segment
// with h0, then walks its chunks in order, producing y and carrying the state in
// registers.  In
// both, wave w of a workgroup owns the head's channels 16w .. 16w+15: their state
// columns (all N rows), the chunk's state contribution to them, and their outputs.
// The masked decay matrix of a chunk is shared by all channels: its 10 lower-
// triangular 16x16 tiles are computed once, spread over the waves, and exchanged
// through LDS.  The next chunk's inputs are loaded into registers while the current
// one is computed.
#include "scan_common.h"

#include <algorithm>
#include <type_traits>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kQ = 64;                  // steps per chunk
constexpr int kP = 64;                  // channels per head
constexpr int kWaves = 4;               // wave w owns channels 16w .. 16w+15
constexpr int kThreads = kWaves * kLanes;
constexpr int kRow = kQ + 8;            // LDS row (bf16): 144 bytes, 36 dwords
static_assert(kQ == kLanes, "one step per lane in the step-size prefix");

// fp32 step arrays of a chunk (offsets in floats): cum (log2 units), dt, the state
// weights exp(cum_last - cum_s) dt_s, the read-out decays exp(cum_t), and cum_last.
// The kernels keep two such sets, chunk c using set c % 2, so that one wave can fill the
// next chunk's set while the others still read the current one.
constexpr int kFCum = 0, kFDt = kQ, kFW = 2 * kQ, kFE = 3 * kQ, kFTot = 4 * kQ;
constexpr int kFSet = 4 * kQ + 4;       // floats per set (16-byte multiple)

// LDS, in bf16 units: B[n][s], C[n][t], u[p][s], z[p][t] (the gate input; a wave's
// outputs y[p][t] replace its rows of it once read), and the masked decay matrix
// M[t][s] as high and low bf16 parts; then the two sets of step arrays.
// With 16-byte rows (DMA) B and C arrive straight from global memory and sit in 128-byte
// rows with swizzled pieces instead (swz_off for B, swz_c_off for C).
template <int N, bool DMA = false> struct OutLds {
    static constexpr int Bn = 0;
    static constexpr int Cn = Bn + N * (DMA ? 64 : kRow);
    static constexpr int U = Cn + N * (DMA ? 64 : kRow);
    static constexpr int Z = U + kP * kRow;
    static constexpr int Mhi = Z + kP * kRow;
    static constexpr int Mlo = Mhi + kQ * kRow;
    static constexpr int F = Mlo + kQ * kRow;
    static constexpr size_t bytes = size_t(F) * 2 + 2 * kFSet * sizeof(float);
};
template <int N> struct StateLds {
    static constexpr int Bn = 0;
    static constexpr int U = Bn + N * kRow;
    static constexpr int F = U + kP * kRow;
    static constexpr size_t bytes = size_t(F) * 2 + 2 * kFSet * sizeof(float);
};
// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at lds + 16 l
// (lds wave-uniform), counted like any other vector-memory load.  (A plain device
// function: the builtin inside a kernel template left that template without a host
// stub.)
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// The end-state pass with 16-byte rows (VEC): B and u go straight from global memory to
// LDS, double-buffered: two buffers of B [N][64] and u [64][64] in 128-byte rows with
// swizzled pieces (swz_off), then the two step-array sets.
template <int N> struct StateDmaLds {
    static constexpr int Bn = 0;
    static constexpr int U = N * 64;
    static constexpr int Buf = (N + kP) * 64;    // bf16 per buffer
    static constexpr int F = 2 * Buf;
    static constexpr size_t bytes = size_t(F) * 2 + 2 * kFSet * sizeof(float);
};

struct SsdParams {
    const uint16_t* u;
    const uint16_t* delta;
    const float* A;
    const uint16_t* B;
    const uint16_t* C;
    const float* D;
    const uint16_t* z;       // NULL: no gate
    const float* dt_bias;
    const float* h0;
    uint16_t* y;
    float* h_last;
    float* gram;             // (batch, nchunks, 10 tiles, 64 lanes, 4) fp32: C^T B per chunk
    float* seg_state;        // ((nseg-1) * pps, batch*nheads) blocks of P*N fp32, in lane order
    float* seg_decay;        // ((nseg-1) * pps, batch*nheads) fp32, log2 units
    int64_t L, nheads, bh_total;
    int nseg, cps, nchunks;
    int pps, cpp;            // state pieces per segment before the last, chunks per piece
};

// Workgroup barrier for LDS traffic only.  __syncthreads() also orders global memory,
// which makes every wave wait for all of its outstanding global loads -- including the
// next chunk's prefetch, issued just before -- at every barrier.  No wave of these
// kernels reads global memory another wave wrote, so waiting for the wave's own LDS
// operations (lgkmcnt) before s_barrier is enough; the memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ state row order
// A 32-wide block kb of the contraction over the state index feeds MFMA slot j of
// lane group g from row
//     nrow(kb, g, half, j) = 32 kb + 16 half + 8 (g % 2) + g / 2 + 2 j,
// half = 0 for slots 0..3 and 1 for slots 4..7.  Any fixed order is correct as long
// as both operands use it.  This one keeps the LDS reads free of bank conflicts with
// 64 four-byte banks and a 36-dword row stride, where row r starts at bank
// 4 * (9 r mod 16): a transposed read (two lane groups, rows 2 apart in each, 8 rows
// apart between the groups) and a 16-lane row read in the state product (rows of all
// 16 residues mod 16) both touch every bank once.  The state tile nb of a wave holds,
// at row m = 4 g + r of its MFMA result, state index nrow(nb / 2, g, nb % 2, r): the
// same order, so the tiles 2kb and 2kb+1 of a lane are exactly the B operand slots of
// block kb when the state is read out.
__device__ constexpr int nrow(int kb, int g, int half, int j) {
    return 32 * kb + 16 * half + 8 * (g & 1) + (g >> 1) + 2 * j;
}

// Row of piece k (16 bytes, 8 steps) of a chunk's [row][step] array: lanes 8s .. 8s+7 of
// each 16 take the 8 pieces of one row, and the two halves of the 16 take rows 8
// apart, whose starts are 32 banks apart.
__device__ constexpr int piece_row(int k) { return 16 * (k >> 7) + ((k >> 4) & 7) + 8 * ((k >> 3) & 1); }

__device__ inline float bf_half(uint32_t word, int hi) {
    return __uint_as_float(hi ? (word & 0xFFFF0000u) : (word << 16));
}

__device__ inline f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 lds16(const uint16_t* q) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q));
}

// Transposed operand read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// 4a + c receives, as element j, element c of the four bf16 that lane 4j + a of the
// group addresses.  With lane 16g + 4j + a addressing row nrow(kb, g, half, j) at
// column col0 + 4a of a [row][col] array, lane 16g + i therefore gets the four rows'
// entries at column col0 + i: an operand whose column is the lane and whose
// contraction index is the row.
// Element offset of (row r, column c) in a [row][64] bf16 array of 128-byte rows whose
// 16-byte pieces sit at position piece ^ (2 ((r >> 1) mod 4)): for the transposed reads
// below, the four rows 2 apart that one lane group reads then take pieces in distinct
// pairs of positions, so the group's 8-byte reads cover distinct banks.
__device__ constexpr int swz_c_off(int r, int c) {
    return r * 64 + (((c >> 3) ^ (2 * ((r >> 1) & 3))) << 3) + (c & 7);
}

template <bool SWZ = false>
__device__ inline bf16x8 lds_tr(const uint16_t* base, int kb, int col0, int lane) {
    const int g = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
    auto at = [](int r, int c) { return SWZ ? swz_c_off(r, c) : r * kRow + c; };
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + at(nrow(kb, g, 0, j), col0 + 4 * a)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + at(nrow(kb, g, 1, j), col0 + 4 * a)));
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Two floats to packed bf16 (round to nearest even): one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16(float x0, float x1) {
    const f32x2 x = {x0, x1};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// x = hi + lo for K (even) floats with hi = bf16(x) and lo = bf16(x - hi) (x - hi is
// exact in fp32), packed two per word: per pair one conversion for hi, the two hi
// values back to fp32 by a shift and a mask, two subtractions, one conversion for lo.
template <int K>
__device__ inline void split(const float (&x)[K], uint32_t (&hi)[K / 2], uint32_t (&lo)[K / 2]) {
#pragma unroll
    for (int j = 0; j < K / 2; ++j) {
        const uint32_t h = pack_bf16(x[2 * j], x[2 * j + 1]);
        hi[j] = h;
        lo[j] = pack_bf16(x[2 * j] - __uint_as_float(h << 16), x[2 * j + 1] - __uint_as_float(h & 0xFFFF0000u));
    }
}

__device__ inline bf16x8 as_bf16x8(const uint32_t (&w)[4]) {
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------------ global I/O
// 8 bf16 of a row starting at step t (zeros past L).  VEC: 16-byte loads, which the
// host allows only when L % 8 == 0 and the arrays are 16-byte aligned, so a vector is
// either wholly inside the row or wholly past its end.
template <bool VEC>
__device__ inline u32x4 ld8(const uint16_t* __restrict__ row, int64_t t, int64_t L) {
    if constexpr (VEC) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (t < L) v = *reinterpret_cast<const u32x4*>(row + t);
        return v;
    } else {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = (t + 2 * j < L) ? row[t + 2 * j] : 0u;
            const uint32_t b = (t + 2 * j + 1 < L) ? row[t + 2 * j + 1] : 0u;
            w[j] = a | (b << 16);
        }
        return u32x4{w[0], w[1], w[2], w[3]};
    }
}

template <bool VEC>
__device__ inline u32x2 ld4(const uint16_t* __restrict__ row, int64_t t, int64_t L) {
    if constexpr (VEC) {
        u32x2 v = {0u, 0u};
        if (t < L) v = *reinterpret_cast<const u32x2*>(row + t);
        return v;
    } else {
        uint32_t w[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t a = (t + 2 * j < L) ? row[t + 2 * j] : 0u;
            const uint32_t b = (t + 2 * j + 1 < L) ? row[t + 2 * j + 1] : 0u;
            w[j] = a | (b << 16);
        }
        return u32x2{w[0], w[1]};
    }
}

template <bool VEC>
__device__ inline void st4(uint16_t* __restrict__ row, int64_t t, int64_t L, u32x2 v) {
    if constexpr (VEC) {
        if (t < L) *reinterpret_cast<u32x2*>(row + t) = v;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (t + j < L) row[t + j] = uint16_t(j & 1 ? v[j >> 1] >> 16 : v[j >> 1] & 0xFFFFu);
    }
}

// Raw buffer descriptors: a workgroup-uniform base and byte size in scalar
// registers, a 32-bit per-lane byte offset and a uniform scalar offset (the chunk's
// first step) per access; a read past the size returns zeros.  Word 3 selects 32-bit
// data format, untyped.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ inline Rsrc make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// A chunk's inputs in registers: 16-byte pieces of the rows of B (and C) and u (8
// pieces per row), thread tid taking pieces tid, tid + 256, ...; and the raw step
// input of step t0 + lane.  Consecutive lanes take consecutive pieces of one row, so
// loads and LDS stores are contiguous.  A thread's pieces all start at step
// t0 + 8 (tid % 8): with VEC they are either all inside their rows or all past the
// end, and `ok` records which, so that the pieces past the end (the next row's data,
// or zeros past the block) are stored to LDS as zeros a chunk later, with no compare
// between a load and its use.
template <int N, bool WITH_C>
struct Chunk {
    static constexpr int kBC = (WITH_C ? 2 : 1) * N * (kQ / 8) / kThreads;
    static constexpr int kU = kP * (kQ / 8) / kThreads;
    u32x4 bc[kBC];
    u32x4 u[kU];
    bool ok;
    uint32_t draw;
};

// Per-thread addressing of the chunk loads, fixed for the whole sequence.
template <int N, bool WITH_C>
struct ChunkSrc {
    using Ch = Chunk<N, WITH_C>;
    Rsrc rb, rc, ru, rd;
    uint32_t off_bc[Ch::kBC];   // byte offsets of the pieces at step 0
    uint32_t off_u[Ch::kU];
};

template <int N, bool WITH_C>
__device__ inline void init_src(ChunkSrc<N, WITH_C>& a, const SsdParams& p, int64_t b, int64_t bh, int tid) {
    using Ch = Chunk<N, WITH_C>;
    const uint32_t L32 = uint32_t(p.L);
    a.rb = make_rsrc(p.B + b * N * p.L, 2 * N * p.L);
    a.rc = make_rsrc(p.C + b * N * p.L, 2 * N * p.L);
    a.ru = make_rsrc(p.u + bh * kP * p.L, 2 * kP * p.L);
    a.rd = make_rsrc(p.delta + bh * p.L, 2 * p.L);
#pragma unroll
    for (int q = 0; q < Ch::kBC; ++q) {
        const int k = (tid + q * kThreads) % (N * (kQ / 8));
        a.off_bc[q] = 2u * (uint32_t(piece_row(k)) * L32 + uint32_t(k & 7) * 8u);
    }
#pragma unroll
    for (int q = 0; q < Ch::kU; ++q) {
        const int i = tid + q * kThreads;
        a.off_u[q] = 2u * (uint32_t(piece_row(i)) * L32 + uint32_t(i & 7) * 8u);
    }
}

// PART 0 loads everything; the passes spread their loads over the chunk's phases
// instead (1: the first half of the B/C pieces -- B's -- 2: the second half -- C's, or
// B's when there is no C -- 3: u and the step input).
template <int N, bool WITH_C, bool VEC, int PART = 0>
__device__ inline void load_chunk(Chunk<N, WITH_C>& c, const ChunkSrc<N, WITH_C>& a, const SsdParams& p, int64_t b,
                                  int64_t bh, int64_t t0, int tid) {
    using Ch = Chunk<N, WITH_C>;
    constexpr int q0 = PART == 2 ? Ch::kBC / 2 : 0;
    constexpr int q1 = PART == 0 ? Ch::kBC : PART == 1 ? Ch::kBC / 2 : PART == 2 ? Ch::kBC : 0;
    constexpr bool with_u = PART == 0 || PART == 3;
    if constexpr (VEC) {
        const int so = int(2 * t0);
#pragma unroll
        for (int q = q0; q < q1; ++q) {
            // pieces tid + 256 q: all B's without C, else the first kBC/2 values of q are
            // B's and the rest C's (a compile-time choice, so the descriptor stays in
            // scalar registers)
            const bool isC = WITH_C && q >= Ch::kBC / 2;
            c.bc[q] = __builtin_amdgcn_raw_buffer_load_b128(isC ? a.rc : a.rb, a.off_bc[q], so, 0);
        }
        if constexpr (with_u) {
#pragma unroll
            for (int q = 0; q < Ch::kU; ++q) c.u[q] = __builtin_amdgcn_raw_buffer_load_b128(a.ru, a.off_u[q], so, 0);
            c.ok = t0 + (tid & 7) * 8 < p.L;
            c.draw = __builtin_amdgcn_raw_buffer_load_b16(a.rd, 2u * uint32_t(tid & 63), so, 0);
        }
    } else {
#pragma unroll
        for (int q = q0; q < q1; ++q) {
            const int i = tid + q * kThreads;
            const int arr = i / (N * (kQ / 8)), k = i % (N * (kQ / 8));
            c.bc[q] = ld8<false>((arr ? p.C : p.B) + (b * N + piece_row(k)) * p.L, t0 + (k & 7) * 8, p.L);
        }
        if constexpr (with_u) {
#pragma unroll
            for (int q = 0; q < Ch::kU; ++q) {
                const int i = tid + q * kThreads;
                c.u[q] = ld8<false>(p.u + (bh * kP + piece_row(i)) * p.L, t0 + (i & 7) * 8, p.L);
            }
            c.ok = true;
            const int64_t t = t0 + (tid & 63);
            c.draw = t < p.L ? p.delta[bh * p.L + t] : 0;
        }
    }
}

template <int N, bool WITH_C>
__device__ inline void store_chunk(const Chunk<N, WITH_C>& c, uint16_t* lds, int bn, int cn, int un, int tid,
                                   bool full) {
    using Ch = Chunk<N, WITH_C>;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // `full` (the whole chunk inside the sequence) is uniform: no per-piece select then
    const bool ok = full || c.ok;
#pragma unroll
    for (int q = 0; q < Ch::kBC; ++q) {
        const int i = tid + q * kThreads;
        const int arr = i / (N * (kQ / 8)), k = i % (N * (kQ / 8));
        u32x4* dst = reinterpret_cast<u32x4*>(lds + (arr ? cn : bn) + piece_row(k) * kRow + (k & 7) * 8);
        if (full) *dst = c.bc[q];
        else *dst = ok ? c.bc[q] : zero;
    }
#pragma unroll
    for (int q = 0; q < Ch::kU; ++q) {
        const int i = tid + q * kThreads;
        u32x4* dst = reinterpret_cast<u32x4*>(lds + un + piece_row(i) * kRow + (i & 7) * 8);
        if (full) *dst = c.u[q];
        else *dst = ok ? c.u[q] : zero;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by 1, 2, 4
// and 8 inside each row of 16 lanes (a lane shifted in from outside its row reads 0),
// then lane 15 is added to row 1 (and lane 47 to row 3), and lane 31 to rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_in(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}

__device__ inline float wave_prefix_sum(float v) {
    v += dpp_in<0x111, 0xF>(v);   // row_shr:1
    v += dpp_in<0x112, 0xF>(v);   // row_shr:2
    v += dpp_in<0x114, 0xF>(v);   // row_shr:4
    v += dpp_in<0x118, 0xF>(v);   // row_shr:8
    v += dpp_in<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_in<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// One wave, one step per lane: step sizes (in log2 units, dl2 = dt / ln 2, so that the
// decay exp(dt a) is exp2(dl2 a)), their decay prefix inside the chunk, and the
// per-step weights.  Steps past L get dt = 0: they leave the state unchanged and add
// nothing, so the last chunk needs no other masking.
__device__ inline void stage_steps(uint32_t draw, bool valid, float a, float bias, float* sf, int lane) {
    const float dl2 = valid ? softplus_log2(__uint_as_float(draw << 16) + bias) : 0.0f;
    const float cum = wave_prefix_sum(dl2 * a);
    const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), kLanes - 1));
    const float dt = dl2 * kLn2;
    sf[kFCum + lane] = cum;
    sf[kFDt + lane] = dt;
    sf[kFW + lane] = __builtin_amdgcn_exp2f(tot - cum) * dt;
    sf[kFE + lane] = __builtin_amdgcn_exp2f(cum);
    if (lane == 0) sf[kFTot] = tot;
}

// ------------------------------------------------------------------ the state
// H[nb] (nb < N/16) is the wave's state tile nb: result row m = 4 lg + r holds state
// index nrow(nb / 2, lg, nb % 2, r), column lr holds channel 16 w + lr.
//
// The chunk's contribution: H <- exp2(cum_last) H + B[n][s] X[s][p], X[s][p] = w_s u[s][p],
// contracted over the chunk's 64 steps in two 32-step blocks.
// Element offset of (row r, column c) in a [row][64] bf16 array of exactly 128-byte rows
// whose 16-byte pieces are stored at position (piece ^ ((r >> 1) & 7)) of their row:
// rows written whole by direct global-to-LDS loads, 16 bytes per lane (no padding is
// possible there), and read 16 bytes per lane by 16 lanes at 16 rows whose residues mod
// 16 are all distinct (the state update's operand reads) -- the XOR puts those 16 reads
// on distinct bank quads, as the padded 144-byte rows do for the other layout.
__device__ constexpr int swz_off(int r, int c) { return r * 64 + (((c >> 3) ^ ((r >> 1) & 7)) << 3) + (c & 7); }

template <int N, bool SWZB = false, bool SWZU = false>
__device__ inline void chunk_state(f32x4 (&H)[N / 16], const uint16_t* sBn, const uint16_t* sU, const float* sf,
                                   int w, int lr, int lg) {
    auto atb = [](int r, int c) { return SWZB ? swz_off(r, c) : r * kRow + c; };
    auto atu = [](int r, int c) { return SWZU ? swz_off(r, c) : r * kRow + c; };
    const float dec = __builtin_amdgcn_exp2f(sf[kFTot]);
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) H[nb] *= dec;
#pragma unroll
    for (int kb = 0; kb < kQ / 32; ++kb) {
        const int s0 = 32 * kb + 8 * lg;
        const u32x4 uv = *reinterpret_cast<const u32x4*>(sU + atu(16 * w + lr, s0));
        float xv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = sf[kFW + s0 + j] * bf_half(uv[j >> 1], j & 1);
        uint32_t xh[4], xl[4];
        split<8>(xv, xh, xl);
        const bf16x8 xo_h = as_bf16x8(xh), xo_l = as_bf16x8(xl);
#pragma unroll
        for (int nb = 0; nb < N / 16; ++nb) {
            const bf16x8 bo = lds16(sBn + atb(nrow(nb >> 1, lr >> 2, nb & 1, lr & 3), s0));
            H[nb] = mfma(bo, xo_h, H[nb]);
            H[nb] = mfma(bo, xo_l, H[nb]);
        }
    }
}

// Block k of the workspace's segment states holds tile nb of wave w at
// ((k * NB + nb) * 4 + w) * 64 + lane, four floats each (the register layout).
template <int N>
__device__ inline int64_t seg_index(int64_t k, int nb, int w, int lane) {
    return (((k * (N / 16) + nb) * kWaves + w) * kLanes + lane) * 4;
}

// ------------------------------------------------------------------ pass 0: C^T B per chunk
// The 10 lower-triangular 16x16 tiles (t block tb, s block sb <= tb) of a chunk's
// matrices, numbered row by row; wave w of a workgroup handles tiles w, w + 4, w + 8.
__device__ inline int tile_t(int ti) { return (ti >= 1) + (ti >= 3) + (ti >= 6); }
__device__ inline int tile_s(int ti) { const int tb = tile_t(ti); return ti - tb * (tb + 1) / 2; }
constexpr int kTiles = 10;

// Tile k (0..2) of wave w in the output pass: w, w + 4, then w + 6 for waves 2 and 3
// (tiles 8 and 9).  Waves 0 and 1 instead write the two tiles above the diagonal that
// the 32-step contraction blocks include (t block 0 x s block 1, t block 2 x s block 3:
// all zeros, as every s > t there), so that all waves take the same branch-free path.
// out_tile names the C^T B tile the wave reads (for waves 0 and 1 at k = 2 it is read
// unused); out_tb / out_sb the tile of M it writes.
__device__ inline int out_tile(int w, int k) { return k < 2 ? w + 4 * k : w + 6; }
__device__ inline int out_tb(int w, int k) { return k < 2 || w >= 2 ? tile_t(out_tile(w, k)) : 2 * w; }
__device__ inline int out_sb(int w, int k) { return k < 2 || w >= 2 ? tile_s(out_tile(w, k)) : 2 * w + 1; }

// G[t][s] = sum_n C[n][t] B[n][s] does not depend on the head, so it is formed once per
// (batch row, chunk) and stored as GT tiles in the register layout the output pass uses:
// tile ti of chunk c of batch row b at ((b * nchunks + c) * 10 + ti) * 64 + lane, four
// floats per lane (result row 4 lg + r is step s, column lr step t).
template <int N, bool VEC>
__global__ void __launch_bounds__(kThreads) ssd_gram_kernel(SsdParams p) {
    constexpr int NK = N / 32;
    constexpr int kPieces = N * (kQ / 8);
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int c = int(blockIdx.x % unsigned(p.nchunks));
    const int64_t b = blockIdx.x / unsigned(p.nchunks);
    const int64_t t0 = int64_t(c) * kQ;
    for (int i = tid; i < 2 * kPieces; i += kThreads) {
        const int arr = i / kPieces, k = i % kPieces;
        const uint16_t* row = (arr ? p.C : p.B) + (b * N + piece_row(k)) * p.L;
        *reinterpret_cast<u32x4*>(lds + arr * N * kRow + piece_row(k) * kRow + (k & 7) * 8) =
            ld8<VEC>(row, t0 + (k & 7) * 8, p.L);
    }
    lds_barrier();
    float* out = p.gram + (b * p.nchunks + c) * (kTiles * 256);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int ti = w + 4 * k;
        if (ti < kTiles) {
            const int tb = tile_t(ti), sb = tile_s(ti);
            f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < NK; ++kb)
                g = mfma(lds_tr(lds, kb, 16 * sb, l), lds_tr(lds + N * kRow, kb, 16 * tb, l), g);
            *reinterpret_cast<f32x4*>(out + (ti * 64 + l) * 4) = g;
        }
    }
}

// ------------------------------------------------------------------ pass 1: segment end states
template <int N, bool VEC>
__global__ void __launch_bounds__(kThreads) ssd_state_kernel(SsdParams p) {
    using Lay = StateLds<N>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    float* const sf0 = reinterpret_cast<float*>(lds + Lay::F);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    // piece pc of a segment before the last: chunks j * cpp .. of segment seg
    const int npc = (p.nseg - 1) * p.pps;
    const int pc = int(blockIdx.x % unsigned(npc));
    const int64_t bh = blockIdx.x / unsigned(npc);
    const int seg = pc / p.pps, j = pc % p.pps;
    const int64_t b = bh / p.nheads, h = bh % p.nheads;
    const float a = p.A[h];
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;

    f32x4 H[N / 16];
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) H[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float dsum = 0.0f;
    const int c0 = seg * p.cps + j * p.cpp, c1 = min(c0 + p.cpp, (seg + 1) * p.cps);
    // Every chunk of a segment before the last lies wholly inside the sequence (the last
    // segment holds the last chunk), so no chunk here needs masking, and the chunk after
    // a piece (at most the following segment's first) is always in bounds.
    // Loads are issued in one order throughout -- u and the step input (from HBM)
    // first, then B -- and each after the last use of the registers it refills.
    Chunk<N, false> nx;
    ChunkSrc<N, false> src;
    init_src<N, false>(src, p, b, bh, tid);
    load_chunk<N, false, VEC, 3>(nx, src, p, b, bh, int64_t(c0) * kQ, tid);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads in the loop's order
    load_chunk<N, false, VEC, 1>(nx, src, p, b, bh, int64_t(c0) * kQ, tid);
    load_chunk<N, false, VEC, 2>(nx, src, p, b, bh, int64_t(c0) * kQ, tid);
    // Wave 0 stages each chunk's step arrays a chunk ahead, at the end of the one before
    // (whose step input it has by then), so no wave waits for them between barriers.
    if (w == 0) stage_steps(nx.draw, true, a, bias, sf0 + (c0 & 1) * kFSet, l);
    for (int c = c0; c < c1; ++c) {
        const int64_t t0 = int64_t(c) * kQ;
        const float* sf = sf0 + (c & 1) * kFSet;
        lds_barrier();
        store_chunk<N, false>(nx, lds, Lay::Bn, 0, Lay::U, tid, true);
        load_chunk<N, false, VEC, 3>(nx, src, p, b, bh, t0 + kQ, tid);
        lds_barrier();
        load_chunk<N, false, VEC, 1>(nx, src, p, b, bh, t0 + kQ, tid);
        load_chunk<N, false, VEC, 2>(nx, src, p, b, bh, t0 + kQ, tid);
        dsum += sf[kFTot];
        chunk_state<N>(H, lds + Lay::Bn, lds + Lay::U, sf, w, lr, lg);
        if (w == 0) stage_steps(nx.draw, true, a, bias, sf0 + ((c + 1) & 1) * kFSet, l);
    }
    const int64_t k = int64_t(pc) * p.bh_total + bh;
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb)
        *reinterpret_cast<f32x4*>(p.seg_state + seg_index<N>(k, nb, w, l)) = H[nb];
    if (tid == 0) p.seg_decay[k] = dsum;
}

// The same pass with 16-byte rows: B and u of chunk c + 1 go straight from global memory
// into the other LDS buffer (buffer_load ... lds, 16 bytes per lane, each wave 8 whole
// rows per load) while chunk c is computed, so a chunk needs one barrier and no
// register staging.  A load's lane l lands at byte 16 l of the wave's 1 KB block (a
// 16-byte slot per lane); the lane loads the row's piece that belongs in that slot.
template <int N>
__global__ void __launch_bounds__(kThreads) ssd_state_dma_kernel(SsdParams p) {
    using Lay = StateDmaLds<N>;
    constexpr int QB = N / 32;                     // 1 KB blocks of B per wave (N rows / 8 / 4 waves)
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    float* const sf0 = reinterpret_cast<float*>(lds + Lay::F);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int npc = (p.nseg - 1) * p.pps;
    const int pc = int(blockIdx.x % unsigned(npc));
    const int64_t bh = blockIdx.x / unsigned(npc);
    const int seg = pc / p.pps, j = pc % p.pps;
    const int64_t b = bh / p.nheads, h = bh % p.nheads;
    const float a = p.A[h];
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;

    f32x4 H[N / 16];
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) H[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float dsum = 0.0f;
    const int c0 = seg * p.cps + j * p.cpp, c1 = min(c0 + p.cpp, (seg + 1) * p.cps);
    // (every chunk of a segment before the last lies wholly inside the sequence)
    const uint32_t L32 = uint32_t(p.L);
    const Rsrc rb = make_rsrc(p.B + b * N * p.L, 2 * N * p.L);
    const Rsrc ru = make_rsrc(p.u + bh * kP * p.L, 2 * kP * p.L);
    const Rsrc rd = make_rsrc(p.delta + bh * p.L, 2 * p.L);
    // B block q of wave w: rows 8 (QB w + q) .. + 7; u block q: rows 8 (2 w + q) .. + 7
    uint32_t voff_b[QB], voff_u[2];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int r = 8 * (QB * w + q) + (l >> 3);
        voff_b[q] = 2u * (uint32_t(r) * L32 + 8u * uint32_t((l & 7) ^ ((r >> 1) & 7)));
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = 8 * (2 * w + q) + (l >> 3);
        voff_u[q] = 2u * (uint32_t(r) * L32 + 8u * uint32_t((l & 7) ^ ((r >> 1) & 7)));
    }
    auto issue = [&](int cc, int buf) {
        const uint32_t so = uint32_t(2 * int64_t(cc) * kQ);
        uint16_t* base = lds + buf * Lay::Buf;
#pragma unroll
        for (int q = 0; q < QB; ++q) load_lds16(rb, base + Lay::Bn + (QB * w + q) * 512, voff_b[q], so);
#pragma unroll
        for (int q = 0; q < 2; ++q) load_lds16(ru, base + Lay::U + (2 * w + q) * 512, voff_u[q], so);
    };
    auto load_draw = [&](int cc) {
        return __builtin_amdgcn_raw_buffer_load_b16(rd, 2u * uint32_t(l), int(2 * int64_t(cc) * kQ), 0);
    };
    uint32_t draw = load_draw(c0);
    issue(c0, 0);
    if (w == 0) stage_steps(draw, true, a, bias, sf0, l);
    for (int c = c0; c < c1; ++c) {
        const int par = (c - c0) & 1;
        const float* sf = sf0 + par * kFSet;
        // this wave's direct loads of the chunk have landed; after the barrier every
        // wave's have, and every wave is done with the other buffer and step-array set
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        // the step input goes first: waiting for it below does not wait for the loads
        if (c + 1 < c1) {
            draw = load_draw(c + 1);
            issue(c + 1, par ^ 1);
        }
        dsum += sf[kFTot];
        chunk_state<N, true, true>(H, lds + par * Lay::Buf + Lay::Bn, lds + par * Lay::Buf + Lay::U, sf, w, lr, lg);
        if (w == 0 && c + 1 < c1) stage_steps(draw, true, a, bias, sf0 + (par ^ 1) * kFSet, l);
    }
    const int64_t k = int64_t(pc) * p.bh_total + bh;
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb)
        *reinterpret_cast<f32x4*>(p.seg_state + seg_index<N>(k, nb, w, l)) = H[nb];
    if (tid == 0) p.seg_decay[k] = dsum;
}

// ------------------------------------------------------------------ pass 2: outputs

template <int N, bool VEC, bool GATE>
__global__ void __launch_bounds__(kThreads) ssd_out_kernel(SsdParams p) {
    constexpr bool DMA = VEC;     // B and C straight from global memory into LDS
    using Lay = OutLds<N, DMA>;
    constexpr int NK = N / 32;    // 32-wide blocks of the state index
    constexpr int NB = N / 16;    // state tiles per wave
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    float* const sf0 = reinterpret_cast<float*>(lds + Lay::F);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int seg = int(blockIdx.x % unsigned(p.nseg));
    const int64_t bh = blockIdx.x / unsigned(p.nseg);
    const int64_t b = bh / p.nheads, h = bh % p.nheads;
    const float a = p.A[h];
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const int pc = 16 * w + lr;                          // the lane's channel within the head
    const float Dp = p.D ? p.D[h * kP + pc] : 0.0f;
    const uint16_t* zb = p.z + bh * kP * p.L;            // the head's rows
    uint16_t* yb = p.y + bh * kP * p.L;
    const Rsrc rz = make_rsrc(GATE ? zb : p.u, 2 * kP * p.L);
    const Rsrc ry = make_rsrc(yb, 2 * kP * p.L);
    const uint32_t prow = uint32_t(pc) * uint32_t(p.L);
    // y leaves in 16-byte pieces of the wave's rows, 8 lanes per 128-byte run of a row:
    // lane l takes row 16 w + l / 8 (and the row 8 below it), steps 8 (l % 8) .. + 7
    const int yrow = 16 * w + (l >> 3);
    const uint32_t y_off = 2u * (uint32_t(yrow) * uint32_t(p.L) + 8u * uint32_t(l & 7));
    const uint32_t y_8rows = 16u * uint32_t(p.L);

    const int c0 = seg * p.cps, c1 = min(c0 + p.cps, p.nchunks);
    Chunk<N, true> nx;
    ChunkSrc<N, true> src;
    init_src<N, true>(src, p, b, bh, tid);
    // this wave's tiles of C^T B: tiles w and w + 4, and tile w + 6 for waves 2 and 3
    // (wave 0 also stages the step arrays); waves 0 and 1 read their third tile unused
    const Rsrc rg = make_rsrc(p.gram + b * p.nchunks * (kTiles * 256), int64_t(p.nchunks) * kTiles * 1024);
    u32x4 gn[3];
    auto load_g = [&](int c) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
            gn[k] = __builtin_amdgcn_raw_buffer_load_b128(rg, uint32_t((out_tile(w, k) * 64 + l) * 16),
                                                          c * kTiles * 1024, 0);
    };
    // The chunk's gate inputs: 16-byte pieces of the head's z rows, taken and staged in
    // LDS like u's (full 128-byte runs of a row per 8 lanes, where reading each lane's
    // own outputs' steps directly would touch 16 rows in 32-byte pieces per access).
    constexpr int kZ = Chunk<N, true>::kU;
    u32x4 zc[kZ];
    auto load_z = [&](int64_t t0) {
        if constexpr (GATE) {
#pragma unroll
            for (int q = 0; q < kZ; ++q) {
                if constexpr (VEC) {
                    zc[q] = __builtin_amdgcn_raw_buffer_load_b128(rz, src.off_u[q], int(2 * t0), 0);
                } else {
                    const int i = tid + q * kThreads;
                    zc[q] = ld8<false>(zb + int64_t(piece_row(i)) * p.L, t0 + (i & 7) * 8, p.L);
                }
            }
        }
    };
    // (nx.ok, from the same chunk's u loads, marks the pieces past L: stored as zeros)
    auto store_z = [&](bool full_chunk) {
        if constexpr (GATE) {
            const bool ok = full_chunk || nx.ok;
#pragma unroll
            for (int q = 0; q < kZ; ++q) {
                const int i = tid + q * kThreads;
                u32x4* dst = reinterpret_cast<u32x4*>(lds + Lay::Z + piece_row(i) * kRow + (i & 7) * 8);
                *dst = ok ? zc[q] : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // With 16-byte rows, B and C of chunk cc go straight into LDS: load q of wave w covers
    // rows 8 (QB w + q) .. + 7 of B (and of C), lane l row + l / 8 and the 16-byte slot
    // l % 8 of it, which holds the row's piece (l % 8) ^ swizzle.  In the sequence's
    // ragged last chunk a piece past L (16-byte rows: a piece lies wholly inside L or
    // past it) would read the next row's first steps; its offset is moved past the
    // descriptor's range instead, where the load writes zeros.
    constexpr int QB = N / 32;
    uint32_t voff_b[DMA ? QB : 1], voff_c[DMA ? QB : 1];
    if constexpr (DMA) {
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            const int r = 8 * (QB * w + q) + (l >> 3);
            voff_b[q] = 2u * (uint32_t(r) * uint32_t(p.L) + 8u * uint32_t((l & 7) ^ ((r >> 1) & 7)));
            voff_c[q] = 2u * (uint32_t(r) * uint32_t(p.L) + 8u * uint32_t((l & 7) ^ (2 * ((r >> 1) & 3))));
        }
    }
    auto issue_bc = [&](int cc) {
        if constexpr (DMA) {
            const uint32_t so = uint32_t(2 * int64_t(cc) * kQ);
            const int64_t rem = p.L - int64_t(cc) * kQ;   // the chunk's steps inside L
            uint32_t vb[QB], vc[QB];
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                vb[q] = voff_b[q];
                vc[q] = voff_c[q];
            }
            if (rem < kQ) {
                // the chunk's offset is below 2^31, so its sum with 2^31 neither wraps nor
                // lands inside the range (at most 2^31 - 1 bytes)
                constexpr uint32_t kPast = 0x80000000u;
#pragma unroll
                for (int q = 0; q < QB; ++q) {
                    const int r = 8 * (QB * w + q) + (l >> 3);
                    if (8 * ((l & 7) ^ ((r >> 1) & 7)) >= rem) vb[q] = kPast;
                    if (8 * ((l & 7) ^ (2 * ((r >> 1) & 3))) >= rem) vc[q] = kPast;
                }
            }
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                load_lds16(src.rb, lds + Lay::Bn + (QB * w + q) * 512, vb[q], so);
                load_lds16(src.rc, lds + Lay::Cn + (QB * w + q) * 512, vc[q], so);
            }
        }
    };
    // B and C of chunk cc, from the registers into LDS (pieces past L as zeros).  They
    // go in once the chunk before has read its own B and C (its third barrier), a chunk
    // ahead of their use, so that the top of a chunk stores only u and z.
    auto store_bc = [&](int cc) {
        using Ch = Chunk<N, true>;
        const int64_t tc = int64_t(cc) * kQ;
        const bool ok = tc + kQ <= p.L || tc + 8 * (tid & 7) < p.L;
#pragma unroll
        for (int q = 0; q < Ch::kBC; ++q) {
            const int i = tid + q * kThreads;
            const int arr = i / (N * (kQ / 8)), k = i % (N * (kQ / 8));
            u32x4* dst = reinterpret_cast<u32x4*>(lds + (arr ? Lay::Cn : Lay::Bn) + piece_row(k) * kRow + (k & 7) * 8);
            *dst = ok ? nx.bc[q] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_u = [&](bool full_chunk) {
        using Ch = Chunk<N, true>;
        const bool ok = full_chunk || nx.ok;
#pragma unroll
        for (int q = 0; q < Ch::kU; ++q) {
            const int i = tid + q * kThreads;
            u32x4* dst = reinterpret_cast<u32x4*>(lds + Lay::U + piece_row(i) * kRow + (i & 7) * 8);
            *dst = ok ? nx.u[q] : u32x4{0u, 0u, 0u, 0u};
        }
    };
    // The first chunk's inputs, in the order the chunk loop issues them (u, z and the
    // step input -- read from HBM, so first --, then the C^T B tiles; B and C, stored
    // here, then the next chunk's): loads complete in order, and with the same order
    // before the loop as inside it the compiler can wait for exactly the loads each use
    // needs.
    load_chunk<N, true, VEC, 3>(nx, src, p, b, bh, int64_t(c0) * kQ, tid);
    load_z(int64_t(c0) * kQ);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads in the loop's order
    load_g(c0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DMA) {
        issue_bc(c0);
    } else {
        load_chunk<N, true, VEC, 1>(nx, src, p, b, bh, int64_t(c0) * kQ, tid);
        __builtin_amdgcn_sched_barrier(0);
        load_chunk<N, true, VEC, 2>(nx, src, p, b, bh, int64_t(c0) * kQ, tid);
        store_bc(c0);
        load_chunk<N, true, VEC, 1>(nx, src, p, b, bh, int64_t(c0 + 1) * kQ, tid);
        load_chunk<N, true, VEC, 2>(nx, src, p, b, bh, int64_t(c0 + 1) * kQ, tid);
    }
    // The state entering the segment: h0 carried through the state pieces before it, read
    // while the first chunk's loads are in flight, three pieces' reads at a time (the
    // fold is serial, the reads are not).
    f32x4 H[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        H[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (p.h0) {
            const float* hr = p.h0 + (bh * kP + pc) * N + nrow(nb >> 1, lg, nb & 1, 0);
            H[nb] = f32x4{hr[0], hr[2], hr[4], hr[6]};
        }
    }
    const int npieces = seg * p.pps;
    for (int j0 = 0; j0 < npieces; j0 += 3) {
        f32x4 st[3][NB];
        float dg[3];
#pragma unroll
        for (int g = 0; g < 3; ++g) {
            const int64_t k = int64_t(min(j0 + g, npieces - 1)) * p.bh_total + bh;   // past the end: read unused
            dg[g] = p.seg_decay[k];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                st[g][nb] = *reinterpret_cast<const f32x4*>(p.seg_state + seg_index<N>(k, nb, w, l));
        }
#pragma unroll
        for (int g = 0; g < 3; ++g) {
            const bool in = j0 + g < npieces;
            const float dec = in ? __builtin_amdgcn_exp2f(dg[g]) : 1.0f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) H[nb] = dec * H[nb] + (in ? st[g][nb] : f32x4{0.0f, 0.0f, 0.0f, 0.0f});
        }
    }
    // Wave 0 stages each chunk's step arrays a chunk ahead, at the end of the one before
    // (whose step input it has by then), so no wave waits for them between barriers.
    if (w == 0) stage_steps(nx.draw, int64_t(c0) * kQ + l < p.L, a, bias, sf0 + (c0 & 1) * kFSet, l);
    // One chunk.  FULL: the chunk lies wholly inside the sequence, so every global
    // access takes one straight path (with a per-element tail path the compiler would
    // drain all outstanding loads and stores at the top of every chunk); the sequence's
    // ragged last chunk, if any, runs the checked copy after the loop.
    auto chunk = [&](const int c, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int64_t t0 = int64_t(c) * kQ;
        const float* sf = sf0 + (c & 1) * kFSet;
        // this wave's B and C loads for the chunk have landed (see issue_bc)
        if constexpr (DMA) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        lds_barrier();
        store_u(FULL);
        store_z(FULL);
        load_chunk<N, true, VEC, 3>(nx, src, p, b, bh, t0 + kQ, tid);
        load_z(t0 + kQ);
        // The next chunks' inputs are loaded over this chunk's phases, each after the
        // last use of the registers it replaces, so no copies (and no early waits) are
        // needed between iterations: u, z, the step input and C^T B of the next chunk,
        // B and C of the one after (B and C are a chunk ahead in LDS).  Past the
        // segment's last chunk they are the next segment's or past the end: read but
        // unused (buffer reads past a block return zeros; flat reads past L are not made).
        lds_barrier();

        // masked decay tiles: M[t][s] = GT[s][t] exp2(cum_t - cum_s) dt_s for s <= t,
        // GT[s][t] = sum_n B[n][s] C[n][t]; result row 4 lg + r is step s, column lr step t
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            {
                const int tb = out_tb(w, k), sb = out_sb(w, k);
                const f32x4 g = __builtin_bit_cast(f32x4, gn[k]);
                const int t = 16 * tb + lr;
                // the lane's four steps s = 16 sb + 4 lg + r are adjacent: one read each
                const float cum_t = sf[kFCum + t];
                const f32x4 cum_s = *reinterpret_cast<const f32x4*>(sf + kFCum + 16 * sb + 4 * lg);
                const f32x4 dt_s = *reinterpret_cast<const f32x4*>(sf + kFDt + 16 * sb + 4 * lg);
                float m[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * sb + 4 * lg + r;
                    const float e = __builtin_amdgcn_exp2f(cum_t - cum_s[r]) * dt_s[r];
                    m[r] = s <= t ? g[r] * e : 0.0f;   // a select: inf or NaN above the diagonal is dropped
                }
                uint32_t mh[2], ml[2];
                split<4>(m, mh, ml);
                const int off = t * kRow + 16 * sb + 4 * lg;
                *reinterpret_cast<u32x2*>(lds + Lay::Mhi + off) = u32x2{mh[0], mh[1]};
                *reinterpret_cast<u32x2*>(lds + Lay::Mlo + off) = u32x2{ml[0], ml[1]};
            }
        }

        load_g(c + 1);

        // read-out of the chunk's starting state: yo[tb][t][p] = sum_n C[n][t] H[n][p]
        f32x4 yo[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) yo[tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < NK; ++kb) {
            float hv[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hv[r] = H[2 * kb][r];
                hv[4 + r] = H[2 * kb + 1][r];
            }
            uint32_t hh[4], hl[4];
            split<8>(hv, hh, hl);
            const bf16x8 ho_h = as_bf16x8(hh), ho_l = as_bf16x8(hl);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const bf16x8 co = lds_tr<DMA>(lds + Lay::Cn, kb, 16 * tb, l);
                yo[tb] = mfma(co, ho_h, yo[tb]);
                yo[tb] = mfma(co, ho_l, yo[tb]);
            }
        }

        chunk_state<N, DMA, false>(H, lds + Lay::Bn, lds + Lay::U, sf, w, lr, lg);
        lds_barrier();   // M complete; this chunk's B and C read
        if constexpr (DMA) {
            issue_bc(c + 1);
            // the only vector-memory operations after these loads in a chunk are its two
            // 16-byte y stores per lane: the top of the next chunk waits for the loads
            // with vmcnt(2) (vector memory completes in issue order)
            __builtin_amdgcn_sched_barrier(0);
        } else {
            store_bc(c + 1);
            load_chunk<N, true, VEC, 1>(nx, src, p, b, bh, t0 + 2 * kQ, tid);
            load_chunk<N, true, VEC, 2>(nx, src, p, b, bh, t0 + 2 * kQ, tid);
        }

        // within the chunk: yd[tb][t][p] = sum_{s} M[t][s] u[s][p] over the 32-step
        // blocks that reach the diagonal of t block tb
        f32x4 yd[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            yd[tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb <= tb / 2; ++kb) {
                const int s0 = 32 * kb + 8 * lg;
                const bf16x8 uo = lds16(lds + Lay::U + pc * kRow + s0);
                const int moff = (16 * tb + lr) * kRow + s0;
                yd[tb] = mfma(lds16(lds + Lay::Mhi + moff), uo, yd[tb]);
                yd[tb] = mfma(lds16(lds + Lay::Mlo + moff), uo, yd[tb]);
            }
        }

        // y = (yd + exp(cum_t) yo + D u) SiLU(z); the lane owns steps 16 tb + 4 lg + r
        constexpr bool full = VEC && FULL;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int tq = 16 * tb + 4 * lg;
            const f32x4 e4 = *reinterpret_cast<const f32x4*>(sf + kFE + tq);
            const u32x2 uu = *reinterpret_cast<const u32x2*>(lds + Lay::U + pc * kRow + tq);
            u32x2 zz = {0u, 0u};
            if constexpr (GATE) zz = *reinterpret_cast<const u32x2*>(lds + Lay::Z + pc * kRow + tq);
            uint32_t o[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float v[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * q + e;
                    float x = fmaf(e4[r], yo[tb][r], yd[tb][r]);
                    x = fmaf(Dp, bf_half(uu[q], e), x);
                    if constexpr (GATE) x *= silu_f32(bf_half(zz[q], e));
                    v[e] = x;
                }
                o[q] = pack_bf16(v[0], v[1]);
            }
            if constexpr (full)   // in place of the gate inputs just read (this lane's own)
                *reinterpret_cast<u32x2*>(lds + Lay::Z + pc * kRow + tq) = u32x2{o[0], o[1]};
            else
                st4<false>(yb + prow, t0 + tq, p.L, u32x2{o[0], o[1]});
        }
        if constexpr (full) {
            // the wave's 16 rows of y, written by its own lanes just above (a wave's LDS
            // accesses take effect in order), leave in whole 128-byte runs
            const u32x4 y0 = *reinterpret_cast<const u32x4*>(lds + Lay::Z + yrow * kRow + 8 * (l & 7));
            const u32x4 y1 = *reinterpret_cast<const u32x4*>(lds + Lay::Z + (yrow + 8) * kRow + 8 * (l & 7));
            __builtin_amdgcn_raw_buffer_store_b128(y0, ry, y_off, int(2 * t0), 0);
            __builtin_amdgcn_raw_buffer_store_b128(y1, ry, y_off + y_8rows, int(2 * t0), 0);
        }
        if (w == 0) stage_steps(nx.draw, t0 + kQ + l < p.L, a, bias, sf0 + ((c + 1) & 1) * kFSet, l);
    };
    // the first chunk's B and C (the loop's own wait counts only the chunks' loads)
    if constexpr (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int c_full = std::min<int64_t>(c1, p.L / kQ);   // chunks wholly inside L
    int c = c0;
    for (; c < c_full; ++c) chunk(c, std::true_type{});
    for (; c < c1; ++c) chunk(c, std::false_type{});

    if (p.h_last && seg == p.nseg - 1) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float* hr = p.h_last + (bh * kP + pc) * N + nrow(nb >> 1, lg, nb & 1, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) hr[2 * r] = H[nb][r];
        }
    }
}

// ------------------------------------------------------------------ host side
struct SsdPlan {
    int nseg, cps, nchunks, pps, cpp;
    int64_t bh_total;
    size_t ws_bytes, state_floats, gram_bytes;
};

inline size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int ssd_plan(const ssm_ssd_dims* d, SsdPlan* pl) {
    if (!d) return SSM_ERR_NULL;
    if (d->batch < 1 || d->seqlen < 1 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1) return SSM_ERR_EMPTY;
    if (d->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
    if (d->headdim != kP || (d->dstate != 64 && d->dstate != 128)) return SSM_ERR_DIMS;
    if (d->nsegments < 0 || d->nsegments > SSM_MAX_CHUNKS || d->reserved != 0) return SSM_ERR_DIMS;
    const int64_t lim = int64_t(1) << 40;
    if (d->batch > lim / d->nheads) return SSM_ERR_DIMS;
    const int64_t bh = d->batch * d->nheads;
    if (bh > lim / (kP * d->seqlen) || bh > lim / (d->dstate * kP)) return SSM_ERR_DIMS;
    if (d->batch > lim / (d->dstate * d->seqlen)) return SSM_ERR_DIMS;
    // kernels address a head's (64, L) block of u, z and y and a batch row's (N, L)
    // block of B and C through buffer descriptors of at most 2^31 - 1 bytes
    if (d->seqlen > (int64_t(1) << 31) / (2 * kP) || d->seqlen > (int64_t(1) << 31) / (2 * d->dstate))
        return SSM_ERR_DIMS;
    const int64_t nchunks = cdiv(d->seqlen, kQ);
    if (nchunks > (int64_t(1) << 30) || d->batch * nchunks > int64_t(INT32_MAX)) return SSM_ERR_DIMS;
    // default: whole rounds of the 512 output workgroups that run at once (two per CU at
    // N = 128).  The most segments that fit in one round; two rounds instead when one
    // round would stay under 80% full and two rounds take more than twice the segments.
    // Measured at N = 128: 24 head rows, 21 segments 126 us against 22 segments (a
    // second round of 24 workgroups) 156 us; 40 rows, 12 segments 170 us against 13
    // segments 211 us; 192 rows, 5 segments 327 us against 2 and 3 segments 390 and
    // 417 us.
    int64_t nseg = d->nsegments;
    if (nseg == 0) {
        constexpr int64_t kSlots = 512;
        nseg = std::max<int64_t>(kSlots / bh, 1);
        const int64_t two_rounds = std::max<int64_t>(2 * kSlots / bh, 1);
        if (5 * bh * nseg < 4 * kSlots && two_rounds > 2 * nseg) nseg = two_rounds;
    }
    nseg = std::min<int64_t>(std::max<int64_t>(nseg, 1), nchunks);
    const int64_t cps = cdiv(nchunks, nseg);
    nseg = cdiv(nchunks, cps);
    // The end states of the segments before the last are computed in pieces of cpp
    // chunks, pps per segment, enough for about three of the state pass's workgroups per
    // CU (its time is that of the most loaded CU: at N = 128, 384 segment-long
    // workgroups take 51 us, 896 half as long 44 us).
    int64_t pps = 1;
    if (nseg > 1) pps = std::max<int64_t>(1, std::min<int64_t>({cdiv(768, (nseg - 1) * bh), 4, cps}));
    const int64_t cpp = cdiv(cps, pps);
    pps = cdiv(cps, cpp);
    if (nseg * bh > int64_t(INT32_MAX) || (nseg - 1) * pps * bh > int64_t(INT32_MAX)) return SSM_ERR_DIMS;
    pl->nseg = int(nseg);
    pl->cps = int(cps);
    pl->pps = int(pps);
    pl->cpp = int(cpp);
    pl->nchunks = int(nchunks);
    pl->bh_total = bh;
    pl->state_floats = size_t(nseg - 1) * size_t(pps) * size_t(bh) * size_t(kP) * size_t(d->dstate);  // P*N per head
    pl->gram_bytes = round256(size_t(d->batch) * size_t(nchunks) * kTiles * 1024);
    pl->ws_bytes = pl->gram_bytes +
                   (nseg > 1 ? round256(pl->state_floats * 4) + round256(size_t(nseg - 1) * size_t(pps) * size_t(bh) * 4)
                             : 0);
    return SSM_OK;
}

template <int N, bool VEC>
int ssd_launch(const SsdParams& p, const SsdPlan& pl, hipStream_t s) {
    launch_kernel((ssd_gram_kernel<N, VEC>), dim3(unsigned(pl.bh_total / p.nheads * pl.nchunks)), dim3(kThreads),
                       size_t(2 * N * kRow * 2), s, p);
    if (pl.nseg > 1) {
        const dim3 sgrid(unsigned((pl.nseg - 1) * pl.pps * pl.bh_total));
        if constexpr (VEC)
            launch_kernel((ssd_state_dma_kernel<N>), sgrid, dim3(kThreads), StateDmaLds<N>::bytes, s, p);
        else
            launch_kernel((ssd_state_kernel<N, VEC>), sgrid, dim3(kThreads), StateLds<N>::bytes, s, p);
    }
    const dim3 grid(unsigned(pl.nseg * pl.bh_total));
    if (p.z)
        launch_kernel((ssd_out_kernel<N, VEC, true>), grid, dim3(kThreads), OutLds<N>::bytes, s, p);
    else
        launch_kernel((ssd_out_kernel<N, VEC, false>), grid, dim3(kThreads), OutLds<N>::bytes, s, p);
    return ssm_detail::launch_error == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" SSM_API int ssm_ssd_fwd_plan(const ssm_ssd_dims* dims, ssm_ssd_plan* plan) {
    SsdPlan pl;
    const int st = ssd_plan(dims, &pl);
    if (st != SSM_OK) return st;
    if (!plan) return SSM_ERR_NULL;
    plan->nsegments = pl.nseg;
    plan->chunks_per_segment = pl.cps;
    plan->chunk_len = kQ;
    plan->state_pieces = pl.pps;
    plan->nchunks = pl.nchunks;
    plan->workspace_bytes = pl.ws_bytes;
    return SSM_OK;
}

extern "C" SSM_API size_t ssm_ssd_fwd_workspace_bytes(const ssm_ssd_dims* dims) {
    SsdPlan pl;
    return ssd_plan(dims, &pl) == SSM_OK ? pl.ws_bytes : 0;
}

extern "C" SSM_API int ssm_ssd_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                   const float* D, const void* z, const float* dt_bias, const float* h0, void* y,
                                   float* h_last, const ssm_ssd_dims* dims, void* stream) {
    SsdPlan pl;
    const int st = ssd_plan(dims, &pl);
    if (st != SSM_OK) return st;
    if (!u || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
    for (const void* q : {u, delta, B, C, z, static_cast<const void*>(y)})
        if (misaligned(q, 2)) return SSM_ERR_ALIGN;
    for (const void* q : {static_cast<const void*>(A), static_cast<const void*>(D),
                          static_cast<const void*>(dt_bias)})
        if (misaligned(q, 4)) return SSM_ERR_ALIGN;
    if (misaligned(h0, 4) || misaligned(h_last, 4)) return SSM_ERR_ALIGN;

    const int64_t N = dims->dstate, L = dims->seqlen, H = dims->nheads, dim = H * kP;
    const size_t io = size_t(dims->batch * dim * L) * 2, dl = size_t(dims->batch * H * L) * 2;
    const size_t bc = size_t(dims->batch * N * L) * 2, stb = size_t(dims->batch * dim * N) * 4;
    const size_t hb = size_t(H) * 4, db = size_t(dim) * 4;
    const struct {
        const void* q;
        size_t n;
    } ins[] = {{u, io}, {delta, dl}, {B, bc}, {C, bc}, {z, io}, {A, hb}, {D, db}, {dt_bias, hb}, {h0, stb}};
    for (const auto& in : ins) {
        if (overlaps(y, io, in.q, in.n)) return SSM_ERR_ALIAS;
        if (overlaps(h_last, stb, in.q, in.n)) return SSM_ERR_ALIAS;
    }
    if (overlaps(h_last, stb, y, io)) return SSM_ERR_ALIAS;

    SsdParams p{};
    if (!dims->workspace || dims->workspace_bytes < pl.ws_bytes || misaligned(dims->workspace, 256))
        return SSM_ERR_WORKSPACE;
    // the workspace is written: it may overlap no input or output
    for (const auto& in : ins)
        if (overlaps(dims->workspace, pl.ws_bytes, in.q, in.n)) return SSM_ERR_ALIAS;
    if (overlaps(dims->workspace, pl.ws_bytes, y, io) || overlaps(dims->workspace, pl.ws_bytes, h_last, stb))
        return SSM_ERR_ALIAS;
    {
        char* ws = static_cast<char*>(dims->workspace);
        p.gram = reinterpret_cast<float*>(ws);
        p.seg_state = reinterpret_cast<float*>(ws + pl.gram_bytes);
        p.seg_decay = reinterpret_cast<float*>(ws + pl.gram_bytes + round256(pl.state_floats * 4));
    }
    p.u = static_cast<const uint16_t*>(u);
    p.delta = static_cast<const uint16_t*>(delta);
    p.A = A;
    p.B = static_cast<const uint16_t*>(B);
    p.C = static_cast<const uint16_t*>(C);
    p.D = D;
    p.z = static_cast<const uint16_t*>(z);
    p.dt_bias = dt_bias;
    p.h0 = h0;
    p.y = static_cast<uint16_t*>(y);
    p.h_last = h_last;
    p.L = L;
    p.nheads = H;
    p.bh_total = pl.bh_total;
    p.nseg = pl.nseg;
    p.cps = pl.cps;
    p.pps = pl.pps;
    p.cpp = pl.cpp;
    p.nchunks = pl.nchunks;

    bool vec = L % 8 == 0;
    for (const void* q : {u, B, C, z, static_cast<const void*>(y)}) vec = vec && !misaligned(q, 16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    ssm_detail::launch_error = hipSuccess;   // this call's launch failures only (the caller's pending HIP error is left alone)
    if (N == 128) return vec ? ssd_launch<128, true>(p, pl, s) : ssd_launch<128, false>(p, pl, s);
    return vec ? ssd_launch<64, true>(p, pl, s) : ssd_launch<64, false>(p, pl, s);
}
