// hip_stub.cpp -- a stand-in for the HIP runtime, for checking libssm's host code on a
// machine without a GPU under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The library's sources are compiled for the host only (no device code), so every
// kernel is a host stub that nobody runs.  This file supplies what those objects
// import from the HIP runtime: the code-object registration calls (which record each
// kernel stub's name), the launch call (which checks and records the launch instead of
// running it), and the device queries of the entry point that allocates nothing.
// Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <string>
#include <vector>

namespace {
std::map<const void*, std::string>& names() {
    static std::map<const void*, std::string> m;
    return m;
}
struct Launch {
    std::string name;
    dim3 grid, block;
    size_t lds;
};
std::vector<Launch>& launches() {
    static std::vector<Launch> v;
    return v;
}
int g_fail_launch = 0;   // > 0: the n-th next launch fails
alignas(256) char g_scratch_dummy[256];   // stands for the library's device scratch array
}  // namespace

// the code objects' fat binaries: the host-only objects reference one symbol each
#define SSM_STUB_FATBIN(name) extern "C" const unsigned char name[16] = {0};
#include "fatbin_symbols.inc"

extern "C" {

void** __hipRegisterFatBinary(const void* data) {
    static void* handle = nullptr;
    (void)data;
    return &handle;
}
void __hipUnregisterFatBinary(void** modules) { (void)modules; }
void __hipRegisterFunction(void** modules, const void* hostFunction, char* deviceFunction, const char* deviceName,
                           unsigned int threadLimit, uint3* tid, uint3* bid, dim3* blockDim, dim3* gridDim,
                           int* wSize) {
    (void)modules; (void)deviceFunction; (void)threadLimit; (void)tid; (void)bid; (void)blockDim; (void)gridDim;
    (void)wSize;
    names()[hostFunction] = deviceName ? deviceName : "?";
}
void __hipRegisterVar(void** modules, void* var, char* hostVar, char* deviceVar, int ext, size_t size, int constant,
                      int global) {
    (void)modules; (void)var; (void)hostVar; (void)deviceVar; (void)ext; (void)size; (void)constant; (void)global;
}
hipError_t __hipPopCallConfiguration(dim3* gridDim, dim3* blockDim, size_t* sharedMem, hipStream_t* stream) {
    (void)gridDim; (void)blockDim; (void)sharedMem; (void)stream;
    fprintf(stderr, "stub: a kernel was launched through <<<>>> instead of hipLaunchKernel\n");
    abort();
}

hipError_t hipLaunchKernel(const void* function_address, dim3 numBlocks, dim3 dimBlocks, void** args,
                           size_t sharedMemBytes, hipStream_t stream) {
    (void)stream;
    auto it = names().find(function_address);
    if (it == names().end()) {
        fprintf(stderr, "stub: launch of an unregistered kernel\n");
        abort();
    }
    const uint64_t threads = uint64_t(dimBlocks.x) * dimBlocks.y * dimBlocks.z;
    if (numBlocks.x < 1 || numBlocks.y < 1 || numBlocks.z < 1 || threads < 1 || threads > 1024 || threads % 64 ||
        sharedMemBytes > 160 * 1024 || !args || !args[0]) {
        fprintf(stderr, "stub: bad launch of %s: grid %u,%u,%u block %u,%u,%u lds %zu\n", it->second.c_str(),
                numBlocks.x, numBlocks.y, numBlocks.z, dimBlocks.x, dimBlocks.y, dimBlocks.z, sharedMemBytes);
        abort();
    }
    launches().push_back({it->second, numBlocks, dimBlocks, sharedMemBytes});
    if (g_fail_launch > 0 && --g_fail_launch == 0) return hipErrorLaunchFailure;
    return hipSuccess;
}

hipError_t hipGetDevice(int* deviceId) {
    *deviceId = 0;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t stream, hipDevice_t* device) {
    (void)stream;
    *device = 0;
    return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** devPtr, const void* symbol) {
    (void)symbol;
    *devPtr = g_scratch_dummy;
    return hipSuccess;
}

// ---- for the checks
size_t stub_launch_count(void) { return launches().size(); }
const char* stub_launch_name(size_t i) { return launches()[i].name.c_str(); }
unsigned stub_launch_grid(size_t i) { return launches()[i].grid.x; }
unsigned stub_launch_block(size_t i) { return launches()[i].block.x; }
size_t stub_launch_lds(size_t i) { return launches()[i].lds; }
void stub_launch_reset(void) { launches().clear(); }
void stub_fail_next_launch(int n) { g_fail_launch = n; }

}  // extern "C"
