// scan_chunked.hip -- the full pass of the selective scan for a scalar decay per head
// (A = a_h I) with a step size per channel, in a chunked form whose contractions over
// the state run on the gfx950 matrix cores.
//
// With a scalar decay the state update of channel d is h_t = al_t h_{t-1} + x_t B_t,
// al_t = exp(dt_t a_h), x_t = dt_t u_t: every state entry of a channel decays by the same
// factor.  For a chunk of kQ steps entered with state H (N x channels) and, per channel,
// E(t,s) = prod_{s<k<=t} al_k (the decay from step s to step t inside the chunk):
//
//   y_t   = sum_{s<=t} (C_t . B_s) E(t,s) x_s  +  E(t,-1) sum_n C[n,t] H[n]
//   H'    = E(Q-1,-1) H + sum_s B_s E(Q-1,s) x_s
//
// the chunked form of the recurrence (the state-space duality of
// yo3nglau.github.io "Mamba 与状态空间模型：面试问题与推荐回答" Q10, and the semiseparable
// sum of cnblogs.com "Mamba3 技术浅析" §2.2.2).  The state read C^T H, the state update
// B (E x) and the chunk's Gram matrix G = C^T B are dense products on
// v_mfma_f32_16x16x32_bf16.  The decays E(t,s) differ per channel, so the masked
// in-chunk part sum_{s<=t} G[t,s] E(t,s) x_s has no decay matrix shared by the
// channels.  Since E(t,s) = E(Q-1,s) / E(Q-1,t), it is the masked G times the state
// update's weighted inputs E(Q-1,s) x_s (one more product), each output then divided
// by E(Q-1,t) -- when the chunk's decay stays above 2^-80, so that the division is
// safe; a wave where it does not evaluates the part per channel in Horner form,
//   acc <- acc * al_s + G[t,s] x_s   for s = 0..t,
// two operations per (t, s) pair (8.5 pairs per output with kQ = 16, against the
// N = 128 state updates per output of the lane walk).
//
// Precision: G multiplies bf16 inputs exactly (fp32 accumulation).  The state and the
// weighted inputs E x are fp32 quantities, split into a high and a low bf16 part
// (x = hi + lo, hi = bf16(x), lo = bf16(x - hi)) and multiplied twice, so each carries
// about 2^-16 relative error.  The Horner part runs in fp32.
//
// Work split: one workgroup per (batch row, 64-channel block, piece of the sequence),
// four waves.  Wave w owns channels 16w .. 16w+15: their state columns (all N rows, in
// the MFMA result layout), and lane l the channel 16w + l % 16 at steps 4(l/16)..+3 of
// each chunk, for everything elementwise.  B and C of a chunk are staged once in LDS
// for the four waves (double-buffered, one barrier per chunk).  delta, u and z come in
// groups of 4 chunks -- each row's whole 128-byte line of 64 steps at once, straight
// into a per-wave LDS area -- so that a line is fetched once instead of once per chunk;
// everything else is exchanged within a wave.  The pieces' starting states come from
// the piece carries (scan_piece_states_kernel and scan_carry_kernel in scan_fwd.hip).
#include "scan_common.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __amdgpu_buffer_rsrc_t Rsrc;

namespace chk {
constexpr int kQ = 16;                      // steps per chunk
constexpr int kWaves = 4;                   // wave w owns channels 16w .. 16w+15
constexpr int kThreads = kWaves * kLanes;
constexpr int kRs = 20;                     // row stride (floats) of the per-wave arrays:
                                            // 16-lane row accesses of 16 bytes cover all banks
constexpr uint32_t kPast = 0x80000000u;     // a buffer offset past every window

// Per-wave LDS (floats): the 4 group sums of dt2 of each channel and the chunk's Gram
// matrix G[t][s] (times ln2).
constexpr int kTot = 0;                     // [16 ch][4]
constexpr int kG = kTot + 64;               // [16 t][kRs]
constexpr int kWaveFloats = kG + 16 * kRs;

// Per-wave staging of the wave's 16 channel rows of delta, u and z for a group of 4
// chunks (64 steps: one whole 128-byte line per row), loaded straight into LDS.
constexpr int kGroup = 4 * kQ;              // steps per group
constexpr int kStage = 16 * kGroup;         // bf16 per array and wave
enum { kSD = 0, kSU = 1, kSZ = 2 };

template <int N> constexpr size_t lds_bytes() {
    return size_t(2) * 2 * N * kQ * sizeof(uint16_t) + size_t(kWaves) * kWaveFloats * sizeof(float) +
           size_t(kWaves) * 3 * kStage * sizeof(uint16_t);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at lds + 16 l
// (lds wave-uniform), counted like any other vector-memory load.  (A plain device
// function: the builtin inside a kernel template leaves the template without a host
// stub.)
__device__ inline void load_lds16(Rsrc r, void* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Staged row r (0..15) keeps its 16-byte piece p (steps 8p..8p+7 of the group) in slot
// p ^ ((r >> 1) & 7) of its 128-byte row: the 8-byte reads of a chunk (rows 0..15, one
// piece each, two lane groups per pass) then touch each bank once.
__device__ constexpr int stage_slot(int r, int p) { return p ^ ((r >> 1) & 7); }

__device__ inline Rsrc make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// B and C of a chunk in LDS: [N rows][16 steps] bf16, 32-byte rows of four 8-byte pieces
// (4 steps each); piece k of row n sits at position k ^ (2 ((n >> 3) & 1)).  With this
// placement the 16-lane row reads of the state update (rows n .. n+15, one piece each,
// two lane groups per pass) and the transposed reads (four whole rows per lane group)
// touch distinct banks.
__device__ constexpr int bc_off(int n, int k) { return n * kQ + 4 * (k ^ (2 * ((n >> 3) & 1))); }

// Transposed operand read (ds_read_b64_tr_b16): within each group of 16 lanes, lane
// 4a + e receives, as element j, element e of the four bf16 that lane 4j + a of the
// group addresses.  Lane 16g + 4j + a addresses row 32 kb + 16 half + 4g + j at piece a,
// so lane 16g + i gets column (step) i of those four rows: an operand whose column is
// the lane and whose contraction slots 0..7 are the rows
//     32 kb + 16 (slot / 4) + 4g + slot % 4.
__device__ inline bf16x8 tr_read(const uint16_t* mat, int kb, int lane) {
    const int g = lane >> 4, j = (lane >> 2) & 3, aa = lane & 3;
    const int r0 = 32 * kb + 4 * g + j;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(mat + bc_off(r0, aa)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(mat + bc_off(r0 + 16, aa)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ inline uint32_t pack_bf16(float x0, float x1) {
    const f32x2 x = {x0, x1};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// x = hi + lo (hi = bf16(x), lo = bf16(x - hi), x - hi exact in fp32) for two floats,
// packed into one word each.
__device__ inline void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(x0, x1);
    lo = pack_bf16(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u));
}

__device__ inline f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Workgroup barrier for LDS traffic only: the wave's own LDS operations complete, then
// s_barrier; outstanding global loads (the next chunk's prefetch) are not waited for.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace chk

template <int N>
__global__ void __launch_bounds__(chk::kThreads) scan_chunked_kernel(ssm_detail::ChunkedArgs p) {
    using namespace chk;
    constexpr int NT = N / 16;                 // state tiles of 16 rows
    constexpr int NKB = N / 32;                // 32-deep blocks of the contraction over the state
    constexpr int MAT = N * kQ;                // bf16 per matrix and buffer
    constexpr int VPT = N / 64;                // 16-byte B/C pieces per thread and chunk
    static_assert(N == 64 || N == 128, "64 or 128 states");
    __shared__ __attribute__((aligned(16))) uint16_t sBC[2][2 * MAT];
    __shared__ __attribute__((aligned(16))) float sWave[kWaves * kWaveFloats];
    __shared__ __attribute__((aligned(16))) uint16_t sStage[kWaves][3][kStage];

    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, c = lane & 15;
    float* const sw = sWave + wv * kWaveFloats;

    const int64_t bid = blockIdx.x;
    const int cblk = int(bid % p.nblk_d);
    const int b = int((bid / p.nblk_d) % p.batch);
    const int piece = int(bid / (int64_t(p.nblk_d) * p.batch));
    const int64_t blk = int64_t(b) * p.nblk_d + cblk;
    const int64_t c0 = int64_t(cblk) * kLanes;
    const int64_t tbeg = int64_t(piece) * p.chunk_len;
    const int64_t tend = (tbeg + p.chunk_len < p.L) ? tbeg + p.chunk_len : p.L;
    const int nq = int((tend - tbeg + kQ - 1) / kQ);

    const int chl = 16 * wv + c;              // the lane's channel within the block
    const int64_t d = c0 + chl;
    const bool dok = d < p.dim;
    const float a = dok ? p.A[d / p.head_dim] : 0.0f;
    const float bias = (dok && p.bias) ? p.bias[d] : 0.0f;
    const float Dd = (dok && p.D) ? p.D[d] : 0.0f;
    const bool has_z = p.z != nullptr;

    // Buffer windows: the block's channel rows of u, delta, z and y, and batch row b's
    // state rows of B and C.  Reads past a window return zeros and stores past it are
    // dropped; channels past dim get an offset past every window.
    const int64_t rowbytes = p.L * 2;
    const int64_t nrows = (p.dim - c0 < kLanes) ? p.dim - c0 : kLanes;
    const int64_t roff = (int64_t(b) * p.dim + c0) * p.L;
    const Rsrc ru = make_rsrc(static_cast<const uint16_t*>(p.u) + roff, nrows * rowbytes);
    const Rsrc rd = make_rsrc(static_cast<const uint16_t*>(p.delta) + roff, nrows * rowbytes);
    const Rsrc rz = make_rsrc(static_cast<const uint16_t*>(has_z ? p.z : p.u) + roff, nrows * rowbytes);
    const Rsrc ry = make_rsrc(static_cast<uint16_t*>(p.y) + roff, nrows * rowbytes);
    const int64_t bcoff = int64_t(b) * N * p.L;
    const Rsrc rB = make_rsrc(static_cast<const uint16_t*>(p.B) + bcoff, N * rowbytes);
    const Rsrc rC = make_rsrc(static_cast<const uint16_t*>(p.C) + bcoff, N * rowbytes);
    const uint32_t lane_off = uint32_t(chl) * uint32_t(rowbytes) + 8u * uint32_t(g);

    // B/C staging, one 16-byte piece (8 steps of a row) per thread and matrix: for
    // N = 128 every thread loads row tid / 2 of B and of C; for N = 64 waves 0-1 load B
    // and waves 2-3 C (the descriptor is chosen per wave, never per lane)
    const int bc_n = (N == 128 ? tid : (tid & 127)) >> 1, bc_h = tid & 1;
    const uint32_t bc_goff = uint32_t(bc_n) * uint32_t(rowbytes) + 16u * uint32_t(bc_h);
    const int bc_loff = bc_n * kQ + 8 * (bc_h ^ ((bc_n >> 3) & 1));
    auto load_bc = [&](u32x4 (&v)[VPT], int64_t t0) {
        const uint32_t off = (t0 + 8 * bc_h < p.L) ? bc_goff + uint32_t(2 * t0) : kPast;
        if constexpr (N == 128) {
            v[0] = __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0);
            v[1] = __builtin_amdgcn_raw_buffer_load_b128(rC, off, 0, 0);
        } else {
            v[0] = __builtin_amdgcn_raw_buffer_load_b128(wv < 2 ? rB : rC, off, 0, 0);
        }
    };
    auto store_bc = [&](const u32x4 (&v)[VPT], int buf) {
        if constexpr (N == 128) {
            *reinterpret_cast<u32x4*>(&sBC[buf][bc_loff]) = v[0];
            *reinterpret_cast<u32x4*>(&sBC[buf][MAT + bc_loff]) = v[1];
        } else {
            *reinterpret_cast<u32x4*>(&sBC[buf][(wv < 2 ? 0 : MAT) + bc_loff]) = v[0];
        }
    };
    auto elem_off = [&](int64_t t0) {
        return (dok && t0 + 4 * g < tend) ? lane_off + uint32_t(2 * t0) : kPast;
    };
    // Group loads: instruction h of an array puts rows 8h..8h+7 of the wave; lane l
    // loads piece (l & 7) ^ ((r >> 1) & 7) of row r = 8h + (l >> 3), so that it lands in
    // the slot stage_slot() gives.  Rows past dim and steps past L read zeros.
    uint32_t st_off[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + (lane >> 3);
        st_off[h] = uint32_t(16 * wv + r) * uint32_t(rowbytes) + 16u * uint32_t(stage_slot(r, lane & 7));
    }
    auto stage = [&](int arr, const Rsrc& rs, int64_t tg) {
#pragma unroll
        for (int h = 0; h < 2; ++h) load_lds16(rs, &sStage[wv][arr][512 * h], st_off[h] + uint32_t(2 * tg));
    };
    // this lane's 4 steps (16k + 4g ..) of chunk k of the group in array arr
    auto staged = [&](int arr, int k) {
        const int slot = stage_slot(c, 2 * k + (g >> 1));
        return *reinterpret_cast<const u32x2*>(&sStage[wv][arr][c * kGroup + 8 * slot + 4 * (g & 1)]);
    };

    // ---- starting state: rows n = 16 jt + 4g + r of column chl
    f32x4 H[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) H[jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (p.nchunks > 1) {
        const float* hin = p.Hin + (blk * p.nchunks + piece) * int64_t(N) * kLanes + chl;
#pragma unroll
        for (int jt = 0; jt < NT; ++jt)
#pragma unroll
            for (int r = 0; r < 4; ++r) H[jt][r] = hin[int64_t(16 * jt + 4 * g + r) * kLanes];
    } else if (p.h0 && dok) {
        const float* h0 = p.h0 + (int64_t(b) * p.dim + d) * N;
#pragma unroll
        for (int jt = 0; jt < NT; ++jt)
#pragma unroll
            for (int r = 0; r < 4; ++r) H[jt][r] = h0[16 * jt + 4 * g + r];
    }

    float sc = 1.0f;   // the true state is sc * H (sc per channel)

    // ---- chunk 0's inputs
    u32x4 bcv[VPT];
    stage(kSD, rd, tbeg);
    stage(kSU, ru, tbeg);
    if (has_z) stage(kSZ, rz, tbeg);
    load_bc(bcv, tbeg);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_bc(bcv, 0);
    lds_barrier();

    // Loads: B and C one chunk ahead (registers, then LDS); delta, u and z one group of
    // 4 chunks ahead, straight into the wave's staging area, each issued right after the
    // group's last read of it (delta and u after the last chunk's elementwise part, z
    // after its outputs) and waited for at their first read in the next group:
    // vector memory completes in issue order, and after the delta and u loads at most
    // the outputs' store, the 2 z loads and this chunk's VPT B/C loads are issued; after
    // the z loads only the VPT B/C loads.  The loads after a piece's last chunk read
    // zeros or the next piece's data, unused.
    uint32_t eoff = elem_off(tbeg);
    for (int q = 0; q < nq; ++q) {
        const int64_t t0 = tbeg + int64_t(q) * kQ;
        const uint16_t* sb = sBC[q & 1];
        const int k = q & 3;
        const bool group_end = (k == 3) && (q + 1 < nq);   // the next group's loads go out in this chunk
        const uint32_t eoffn = elem_off(t0 + kQ);
        load_bc(bcv, t0 + kQ);
        if (k == 0 && q > 0) {
            // after this group's delta and u loads: the previous chunk's store (counted or
            // not), its 2 z loads when there is a gate, and the VPT B/C loads just issued
            if (has_z)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 + VPT) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VPT) : "memory");
        }
        const u32x2 dr = staged(kSD, k);
        const u32x2 uu = staged(kSU, k);

        // ---- elementwise: steps 4g..4g+3 of channel chl (steps past the piece are
        // identity steps: dt2 = 0, x = 0)
        const bool valid = dok && t0 + 4 * g < tend;
        const float draw[4] = {bf_lo(dr[0]), bf_hi(dr[0]), bf_lo(dr[1]), bf_hi(dr[1])};
        const float uv[4] = {bf_lo(uu[0]), bf_hi(uu[0]), bf_lo(uu[1]), bf_hi(uu[1])};
        float dt2[4], xs[4], al[4], pre[4], skip[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dt2[i] = valid ? softplus_log2(draw[i] + bias) : 0.0f;
            xs[i] = valid ? dt2[i] * uv[i] : 0.0f;        // x / ln2
            al[i] = __builtin_amdgcn_exp2f(a * dt2[i]);
            pre[i] = (i == 0) ? dt2[0] : pre[i - 1] + dt2[i];
            skip[i] = Dd * uv[i];
        }
        sw[kTot + 4 * c + g] = pre[3];
        __builtin_amdgcn_wave_barrier();
        const f32x4 tot = *reinterpret_cast<const f32x4*>(&sw[kTot + 4 * c]);
        const float excl = g == 0 ? 0.0f : g == 1 ? tot[0] : g == 2 ? tot[0] + tot[1] : tot[0] + tot[1] + tot[2];
        const float cumq = (tot[0] + tot[1]) + (tot[2] + tot[3]);
        // The state is held scaled: the true state is sc * H, so a chunk's decay changes
        // sc (one multiply) instead of every entry of H.  The read-out decays
        // sc * E(t,-1) = sc 2^(a cum_t) are a running product of the steps' decays from
        // one exponential.
        constexpr float kLog2Ln2 = -0.5287663729448977f;   // log2(ln 2)
        float ev[4], wx[4];
        ev[0] = sc * __builtin_amdgcn_exp2f(a * (excl + pre[0]));
#pragma unroll
        for (int i = 1; i < 4; ++i) ev[i] = ev[i - 1] * al[i];
        const float dec = __builtin_amdgcn_exp2f(a * cumq);
        float scn = sc * dec;
        // The in-chunk part as a matrix product (fast) needs the chunk's decay to stay
        // above 2^-80 in every lane of the wave; otherwise the wave sums it per channel in
        // Horner form.
        const bool fast = __builtin_amdgcn_ballot_w64(dec < 0x1p-80f) == 0;
        // the next group's delta and u, once this group's last reads of them are done
        // (the Horner form reads them again further down)
        auto stage_du = [&]() {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            stage(kSD, rd, t0 + kQ);
            stage(kSU, ru, t0 + kQ);
        };
        if (group_end && fast) stage_du();

        // ---- matrix cores: G = C^T B, the state read C^T H, the state update
        bf16x8 ct[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) ct[kb] = tr_read(sb + MAT, kb, lane);
        f32x4 gm = {0.0f, 0.0f, 0.0f, 0.0f}, rd4 = gm;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) gm = mfma(ct[kb], tr_read(sb, kb, lane), gm);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            uint32_t hi[4], lo[4];
            split2(H[2 * kb][0], H[2 * kb][1], hi[0], lo[0]);
            split2(H[2 * kb][2], H[2 * kb][3], hi[1], lo[1]);
            split2(H[2 * kb + 1][0], H[2 * kb + 1][1], hi[2], lo[2]);
            split2(H[2 * kb + 1][2], H[2 * kb + 1][3], hi[3], lo[3]);
            rd4 = mfma(ct[kb], __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]}), rd4);
            rd4 = mfma(ct[kb], __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]}), rd4);
        }
        bf16x8 xop;
        float rwv[4];
        {
            // the state update of the scaled state: when some lane's new scale would fall
            // below 2^-60 the wave first folds the scales into H (scale 1), so that 1 / scale
            // stays finite; the weights ln2 2^(a (cumq - cum_s)) (x_s / ln2) / scale are a
            // running product of the steps' decays from one exponential
            if (__builtin_amdgcn_ballot_w64(scn < 0x1p-60f) != 0) {
#pragma unroll
                for (int jt = 0; jt < NT; ++jt) H[jt] *= scn;
                scn = 1.0f;
            }
            float rw = __builtin_amdgcn_exp2f(fmaf(a, cumq - (excl + pre[3]), kLog2Ln2)) * __builtin_amdgcn_rcpf(scn);
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                rwv[i] = rw;
                wx[i] = rw * xs[i];
                if (i > 0) rw *= al[i];
            }
            sc = scn;
            uint32_t whi[2], wlo[2];
            split2(wx[0], wx[1], whi[0], wlo[0]);
            split2(wx[2], wx[3], whi[1], wlo[1]);
            xop = __builtin_bit_cast(bf16x8, u32x4{whi[0], whi[1], wlo[0], wlo[1]});
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) {
                const int n = 16 * jt + c;
                const u32x2 bw = *reinterpret_cast<const u32x2*>(sb + bc_off(n, g));
                H[jt] = mfma(__builtin_bit_cast(bf16x8, u32x4{bw[0], bw[1], bw[0], bw[1]}), xop, H[jt]);
            }
        }
        // G (times ln2) into the wave's [t][s] array: rows 4g..4g+3 of column c
#pragma unroll
        for (int r = 0; r < 4; ++r) sw[kG + (4 * g + r) * kRs + c] = gm[r] * kLn2;
        __builtin_amdgcn_wave_barrier();

        // ---- in-chunk part sum_{s<=t} G[t,s] E(t,s) x_s
        f32x4 intra;
        if (fast) {
            // E(t,s) = E(15,s) / E(15,t): the state update's weighted inputs
            // wx_s = E(15,s) x_s / sc (its B operand, already split) times the masked G,
            // one matrix product, then each output divided by its own E(15,t) / sc factor
            // (1 / rw_t, ln2 included: the array holds G times ln2).  Lane l supplies
            // row t = l % 16 of G at the slots of steps 4(l/16)..+3, both parts.
            const f32x4 gv = *reinterpret_cast<const f32x4*>(&sw[kG + c * kRs + 4 * g]);
            float gmk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) gmk[e] = (4 * g + e <= c) ? gv[e] : 0.0f;
            uint32_t ghi[2], glo[2];
            split2(gmk[0], gmk[1], ghi[0], glo[0]);
            split2(gmk[2], gmk[3], ghi[1], glo[1]);
            f32x4 ia = mfma(__builtin_bit_cast(bf16x8, u32x4{ghi[0], ghi[1], ghi[0], ghi[1]}), xop,
                            f32x4{0.0f, 0.0f, 0.0f, 0.0f});
            ia = mfma(__builtin_bit_cast(bf16x8, u32x4{glo[0], glo[1], glo[0], glo[1]}), xop, ia);
#pragma unroll
            for (int i = 0; i < 4; ++i) intra[i] = ia[i] * __builtin_amdgcn_rcpf(rwv[i]);
        } else {
            // ---- in-chunk part per channel in Horner form, acc <- acc * al_s + G[t][s] x_s
            // over s = 0..t for the lane's outputs t = 4g + i: every lane recomputes its
            // channel's step sizes, decays and values from the staged rows, 4 steps at a
            // time (this wave only, when a chunk's decay falls below 2^-80)
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
            for (int m = 0; m < 4; ++m) {
                const int slot = stage_slot(c, 2 * k + (m >> 1));
                const u32x2 bd = *reinterpret_cast<const u32x2*>(&sStage[wv][kSD][c * kGroup + 8 * slot + 4 * (m & 1)]);
                const u32x2 bu = *reinterpret_cast<const u32x2*>(&sStage[wv][kSU][c * kGroup + 8 * slot + 4 * (m & 1)]);
                const bool vm = dok && t0 + 4 * m < tend;
                const float bdr[4] = {bf_lo(bd[0]), bf_hi(bd[0]), bf_lo(bd[1]), bf_hi(bd[1])};
                const float buv[4] = {bf_lo(bu[0]), bf_hi(bu[0]), bf_lo(bu[1]), bf_hi(bu[1])};
                float alm[4], xsm[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float dt = vm ? softplus_log2(bdr[e] + bias) : 0.0f;
                    xsm[e] = vm ? dt * buv[e] : 0.0f;
                    alm[e] = __builtin_amdgcn_exp2f(a * dt);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 gv = *reinterpret_cast<const f32x4*>(&sw[kG + (4 * g + i) * kRs + 4 * m]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float nv = fmaf(acc[i], alm[e], gv[e] * xsm[e]);
                        acc[i] = (4 * m + e <= 4 * g + i) ? nv : acc[i];
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) intra[i] = acc[i];
            if (group_end) stage_du();
        }

        // ---- outputs of steps 4g..4g+3: (in-chunk + decayed read + D u) * SiLU(z)
        float yv[4];
        if (k == 0 && q > 0 && has_z) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VPT) : "memory");
        const u32x2 zz = has_z ? staged(kSZ, k) : u32x2{0u, 0u};
        const float zv[4] = {bf_lo(zz[0]), bf_hi(zz[0]), bf_lo(zz[1]), bf_hi(zz[1])};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pre_gate = fmaf(ev[i], rd4[i], intra[i]) + skip[i];
            yv[i] = has_z ? pre_gate * silu_f32(zv[i]) : pre_gate;
        }
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16(yv[0], yv[1]), pack_bf16(yv[2], yv[3])}, ry, eoff, 0, 0);
        if (group_end && has_z) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this group's z reads are done
            stage(kSZ, rz, t0 + kQ);
        }
        eoff = eoffn;

        store_bc(bcv, (q + 1) & 1);
        lds_barrier();
    }

    if (p.h_last && dok && piece == p.nchunks - 1) {
        float* hl = p.h_last + (int64_t(b) * p.dim + d) * N;
#pragma unroll
        for (int jt = 0; jt < NT; ++jt)
#pragma unroll
            for (int r = 0; r < 4; ++r) hl[16 * jt + 4 * g + r] = sc * H[jt][r];
    }
}

}  // namespace

namespace ssm_detail {

bool chunked_supported(int64_t nstate) { return nstate == 64 || nstate == 128; }

size_t chunked_lds_bytes(int64_t nstate) {
    return nstate == 128 ? chk::lds_bytes<128>() : chk::lds_bytes<64>();
}

bool launch_chunked(const ChunkedArgs& a, hipStream_t s) {
    const dim3 grid(unsigned(int64_t(a.batch) * a.nblk_d * a.nchunks)), block(chk::kThreads);
    if (a.nstate == 128)
        launch_kernel(scan_chunked_kernel<128>, grid, block, 0, s, a);
    else if (a.nstate == 64)
        launch_kernel(scan_chunked_kernel<64>, grid, block, 0, s, a);
    else
        return false;
    return true;
}

}  // namespace ssm_detail
