// lib_host_checks.cpp -- libssm's host code (argument checks, planners, workspace
// layouts, kernel dispatch) run on the CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer, with hip_stub.cpp in place of the HIP runtime: nothing
// reaches a device, and every launch is checked and recorded by the stub.
// Test infrastructure only.  Exits 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ssm.h"

extern "C" {
size_t stub_launch_count(void);
const char* stub_launch_name(size_t i);
unsigned stub_launch_grid(size_t i);
unsigned stub_launch_block(size_t i);
size_t stub_launch_lds(size_t i);
void stub_launch_reset(void);
void stub_fail_next_launch(int n);
}

static int g_checks = 0, g_failed = 0;
#define CHECK(cond, ...)                                                        \
    do {                                                                        \
        ++g_checks;                                                             \
        if (!(cond)) {                                                          \
            ++g_failed;                                                         \
            fprintf(stderr, "FAILED %s:%d: %s: ", __FILE__, __LINE__, #cond); \
            fprintf(stderr, __VA_ARGS__);                                       \
            fprintf(stderr, "\n");                                              \
        }                                                                       \
    } while (0)

// Fake device addresses, 1 TiB apart (never dereferenced: the kernels do not run).
static void* dev(int slot) { return reinterpret_cast<void*>((uintptr_t(slot) + 1) << 40); }

static ssm_dims dims(int64_t b, int64_t L, int64_t d, int64_t n, int64_t heads, int io, int nch = 0, int spl = 0) {
    ssm_dims x;
    memset(&x, 0, sizeof(x));
    x.batch = b;
    x.seqlen = L;
    x.dim = d;
    x.dstate = n;
    x.nheads = heads;
    x.io_dtype = io;
    x.nchunks = nch;
    x.states_per_lane = spl;
    return x;
}

static int fwd(ssm_dims* d) {
    return ssm_selective_scan_fwd(dev(0), dev(1), (const float*)dev(2), dev(3), dev(4), (const float*)dev(5),
                                  dev(6), (const float*)dev(7), dev(8), d, nullptr);
}

// the forward's plans over a sweep of shapes, and a call for each through the stub
static void forward_sweep() {
    const int64_t Bs[] = {1, 3, 8};
    const int64_t Ls[] = {1, 7, 64, 1000, 4096, 131072};
    const int64_t Ds[] = {1, 63, 64, 65, 1536, 4096};
    const int64_t Ns[] = {1, 3, 4, 16, 17, 64, 128, 256};
    int calls = 0;
    for (int64_t B : Bs)
        for (int64_t L : Ls)
            for (int64_t D : Ds)
                for (int64_t N : Ns)
                    for (int io = 0; io < 2; ++io)
                        for (int scalar = 0; scalar < 2; ++scalar) {
                            const int64_t heads = scalar ? (D % 64 == 0 ? D / 64 : 1) : 0;
                            ssm_dims d = dims(B, L, D, N, heads, io);
                            ssm_plan pl;
                            const int st = ssm_selective_scan_plan(&d, &pl);
                            CHECK(st == SSM_OK, "plan B%ld L%ld D%ld N%ld: %d", (long)B, (long)L, (long)D, (long)N, st);
                            if (st != SSM_OK) continue;
                            CHECK(pl.nchunks >= 1 && pl.chunk_len * pl.nchunks >= L && pl.chunk_len * (pl.nchunks - 1) < L,
                                  "pieces %d x %ld for L %ld", pl.nchunks, (long)pl.chunk_len, (long)L);
                            CHECK(pl.chunk_len % pl.time_tile == 0, "chunk %ld tile %d", (long)pl.chunk_len, pl.time_tile);
                            CHECK(pl.waves_per_group * pl.states_per_lane >= N, "waves %d spl %d N %ld",
                                  pl.waves_per_group, pl.states_per_lane, (long)N);
                            CHECK(pl.lds_bytes <= 160 * 1024, "lds %zu", pl.lds_bytes);
                            CHECK(pl.workgroups == B * ((D + 63) / 64) * pl.nchunks, "workgroups %ld", (long)pl.workgroups);
                            CHECK((pl.workspace_bytes == 0) == (pl.nchunks == 1), "workspace %zu pieces %d",
                                  pl.workspace_bytes, pl.nchunks);
                            CHECK(ssm_selective_scan_workspace_bytes(&d) == pl.workspace_bytes, "ws query");
                            if (pl.workspace_bytes) {
                                d.workspace = dev(9);
                                d.workspace_bytes = pl.workspace_bytes;
                            }
                            stub_launch_reset();
                            const int fs = fwd(&d);
                            CHECK(fs == SSM_OK, "fwd B%ld L%ld D%ld N%ld io%d: %d", (long)B, (long)L, (long)D, (long)N, io, fs);
                            const size_t n = stub_launch_count();
                            CHECK(n == (pl.nchunks > 1 ? 3u : 1u), "launches %zu for %d pieces", n, pl.nchunks);
                            if (n >= 1) {
                                CHECK(stub_launch_grid(n - 1) == unsigned(pl.workgroups), "grid %u", stub_launch_grid(n - 1));
                                // the chunked form's full pass (form 1; the sweep's pointers allow
                                // 16-byte loads) holds its LDS statically, the lane walk asks for it
                                const bool chunked = pl.form == 1;
                                CHECK(stub_launch_lds(n - 1) == (chunked ? 0 : pl.lds_bytes), "lds %zu vs %zu",
                                      stub_launch_lds(n - 1), pl.lds_bytes);
                                CHECK(strstr(stub_launch_name(n - 1), chunked ? "scan_chunked_kernel" : "scan_fwd_kernel") !=
                                          nullptr,
                                      "%s", stub_launch_name(n - 1));
                            }
                            ++calls;
                            // the no-allocation entry point: same launches, no workspace
                            stub_launch_reset();
                            ssm_dims d2 = d;
                            d2.workspace = nullptr;
                            d2.workspace_bytes = 0;
                            const int ns = ssm_selective_scan_fwd_noalloc(dev(0), dev(1), (const float*)dev(2), dev(3),
                                                                          dev(4), nullptr, nullptr, nullptr, nullptr,
                                                                          dev(8), nullptr, &d2, nullptr);
                            if (pl.workspace_bytes > SSM_NOALLOC_SCRATCH_BYTES)
                                CHECK(ns == SSM_ERR_SCRATCH, "noalloc beyond the scratch: %d", ns);
                            else
                                CHECK(ns == SSM_OK && stub_launch_count() == n, "noalloc: %d, %zu launches", ns,
                                      stub_launch_count());
                        }
    CHECK(calls > 1000, "calls %d", calls);
}

static void forward_refusals() {
    ssm_dims d = dims(2, 4096, 128, 16, 0, SSM_BF16, 4);
    CHECK(fwd(nullptr) == SSM_ERR_NULL, "null dims");
    CHECK(fwd(&d) == SSM_ERR_WORKSPACE, "no workspace");
    const size_t need = ssm_selective_scan_workspace_bytes(&d);
    d.workspace = dev(9);
    d.workspace_bytes = need - 1;
    CHECK(fwd(&d) == SSM_ERR_WORKSPACE, "short workspace");
    d.workspace_bytes = need;
    d.workspace = dev(0);   // over u
    CHECK(fwd(&d) == SSM_ERR_ALIAS, "workspace over u");
    d.workspace = (char*)dev(9) + 16;
    CHECK(fwd(&d) == SSM_ERR_WORKSPACE, "unaligned workspace");
    ssm_dims e = dims(1, 64, 4, 4, 0, SSM_F32);
    e.dstate = SSM_MAX_DSTATE + 1;
    CHECK(fwd(&e) == SSM_ERR_DIMS, "dstate");
    e = dims(int64_t(1) << 30, int64_t(1) << 20, 1 << 10, 4, 0, SSM_F32);
    CHECK(fwd(&e) == SSM_ERR_DIMS, "huge sizes");
    e = dims(1, 64, 4, 4, 0, 9);
    CHECK(fwd(&e) == SSM_ERR_DTYPE, "dtype");
    // a launch failure is this call's SSM_ERR_HIP
    e = dims(1, 64, 4, 4, 0, SSM_F32);
    stub_fail_next_launch(1);
    CHECK(fwd(&e) == SSM_ERR_HIP, "failed launch");
    stub_fail_next_launch(0);
    CHECK(fwd(&e) == SSM_OK, "next call after a failed launch");
    for (int s = -10; s <= 0; ++s) CHECK(strcmp(ssm_status_string(s), "unknown status") != 0, "status %d", s);
}

static void backward_sweep() {
    const int64_t Ls[] = {1, 16, 1000, 8192};
    const int64_t Ds[] = {1, 64, 100, 2048};
    const int64_t Ns[] = {1, 4, 16, 32, 64, 128};
    for (int64_t L : Ls)
        for (int64_t D : Ds)
            for (int64_t N : Ns)
                for (int io = 0; io < 2; ++io)
                    for (int scalar = 0; scalar < 2; ++scalar) {
                        const int64_t heads = scalar ? (D % 64 == 0 ? D / 64 : 1) : 0;
                        ssm_dims d = dims(2, L, D, N, heads, io);
                        ssm_plan pl;
                        const int st = ssm_selective_scan_bwd_plan(&d, &pl);
                        CHECK(st == SSM_OK, "bwd plan L%ld D%ld N%ld: %d", (long)L, (long)D, (long)N, st);
                        if (st != SSM_OK) continue;
                        CHECK(pl.workspace_bytes > 0 && pl.lds_bytes <= 160 * 1024, "bwd ws %zu lds %zu",
                              pl.workspace_bytes, pl.lds_bytes);
                        d.workspace = dev(20);
                        d.workspace_bytes = pl.workspace_bytes;
                        ssm_grads g;
                        memset(&g, 0, sizeof(g));
                        g.du = dev(10);
                        g.ddelta = dev(11);
                        g.dA = (float*)dev(12);
                        g.dB = (float*)dev(13);
                        g.dC = (float*)dev(14);
                        g.dD = (float*)dev(15);
                        g.dz = dev(16);
                        g.ddt_bias = (float*)dev(17);
                        g.dh0 = (float*)dev(18);
                        stub_launch_reset();
                        const int bs = ssm_selective_scan_bwd(dev(0), dev(1), (const float*)dev(2), dev(3), dev(4),
                                                              (const float*)dev(5), dev(6), (const float*)dev(7),
                                                              nullptr, dev(8), nullptr, &g, &d, nullptr);
                        CHECK(bs == SSM_OK && stub_launch_count() >= 3, "bwd L%ld D%ld N%ld: %d, %zu launches", (long)L,
                              (long)D, (long)N, bs, stub_launch_count());
                        const size_t nck = ssm_selective_scan_ckpt_bytes(&d);
                        if (nck) {
                            const int cs = ssm_selective_scan_fwd_ckpt(
                                dev(0), dev(1), (const float*)dev(2), dev(3), dev(4), nullptr, nullptr, nullptr, nullptr,
                                dev(8), nullptr, (float*)dev(19), &d, nullptr);
                            CHECK(cs == SSM_OK || cs == SSM_ERR_DIMS, "fwd ckpt %d", cs);
                        }
                    }
}

static void step_conv_ssd() {
    ssm_dims d = dims(64, 1, 4096, 16, 0, SSM_BF16);
    stub_launch_reset();
    CHECK(ssm_selective_scan_step(dev(0), dev(1), (const float*)dev(2), dev(3), dev(4), nullptr, nullptr, nullptr,
                                  (float*)dev(5), dev(6), &d, nullptr) == SSM_OK && stub_launch_count() == 1,
          "step");
    ssm_conv c = {(const float*)dev(30), nullptr, 4, 1};
    ssm_dims dc = dims(2, 1000, 130, 16, 0, SSM_BF16);
    dc.workspace = dev(9);
    dc.workspace_bytes = ssm_selective_scan_workspace_bytes(&dc);
    const int cs = ssm_selective_scan_fwd_conv(dev(0), &c, nullptr, dev(1), (const float*)dev(2), dev(3), dev(4),
                                               nullptr, nullptr, nullptr, nullptr, nullptr, dev(8), nullptr, &dc, nullptr);
    CHECK(cs == SSM_OK, "conv: %d", cs);
    c.width = 5;
    CHECK(ssm_selective_scan_fwd_conv(dev(0), &c, nullptr, dev(1), (const float*)dev(2), dev(3), dev(4), nullptr,
                                      nullptr, nullptr, nullptr, nullptr, dev(8), nullptr, &dc, nullptr) == SSM_ERR_DIMS,
          "conv width");
    const int64_t Ls[] = {1, 63, 64, 300, 8192, 16384};
    const int64_t Hs[] = {1, 3, 64};
    const int64_t Ns[] = {64, 128};
    for (int64_t L : Ls)
        for (int64_t H : Hs)
            for (int64_t N : Ns)
                for (int seg = 0; seg < 3; ++seg) {
                    ssm_ssd_dims s;
                    memset(&s, 0, sizeof(s));
                    s.batch = 2;
                    s.seqlen = L;
                    s.nheads = H;
                    s.headdim = 64;
                    s.dstate = N;
                    s.io_dtype = SSM_BF16;
                    s.nsegments = seg * 3;
                    ssm_ssd_plan sp;
                    CHECK(ssm_ssd_fwd_plan(&s, &sp) == SSM_OK, "ssd plan");
                    s.workspace = dev(40);
                    s.workspace_bytes = sp.workspace_bytes;
                    stub_launch_reset();
                    const int st = ssm_ssd_fwd(dev(0), dev(1), (const float*)dev(2), dev(3), dev(4), nullptr, nullptr,
                                               nullptr, nullptr, dev(8), nullptr, &s, nullptr);
                    CHECK(st == SSM_OK && stub_launch_count() >= 2, "ssd L%ld H%ld N%ld: %d", (long)L, (long)H,
                          (long)N, st);
                }
}

int main() {
    forward_sweep();
    forward_refusals();
    backward_sweep();
    step_conv_ssd();
    printf("%d checks, %d failed\n", g_checks, g_failed);
    return g_failed ? 1 : 0;
}
