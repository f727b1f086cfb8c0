// Exact attention that allocates nothing, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// It is the dense baseline of sparsepr_dense_attn, the same attention kernel launched over
// one group that holds every key, without a context: its only scratch, the work-unit
// metadata, lives in a file-scope device array of fixed size. Each device that runs it holds
// its own copy of the array until the process ends, at the address hipGetSymbolAddress gives
// on that device; every call on a device rewrites the whole of it, so calls that overlap on
// one device (concurrent streams or threads) race.
#include "../../include/sparsepr.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "kernels.h"

namespace spr {

namespace {

constexpr int kNoAllocMaxUnits = 8192;             // kDenseRows-row units: n <= 2,097,152
constexpr size_t kMetaBytes = 256;                 // offsets, block list, unit count
constexpr size_t kScratchBytes = kMetaBytes + sizeof(int2) * kNoAllocMaxUnits;   // 65,792 bytes

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};                 // the array's device address, per device

// meta[0..1] query offsets {0, n}, meta[2..3] key offsets {0, n}, meta[4] the one routed
// block (group 0), meta[5] the unit count, meta[6] the built unit count (k_units writes it)
__global__ void k_dense_meta(int32_t* meta, int n, int units) {
    if (threadIdx.x == 0) {
        meta[0] = 0;
        meta[1] = n;
        meta[2] = 0;
        meta[3] = n;
        meta[4] = 0;
        meta[5] = units;
        meta[6] = 0;
        meta[7] = 0;
    }
}

int32_t fail(int32_t status, const std::string& what) {
    set_call_error(what.c_str());
    return status;
}

// The array's address on the current device, looked up once per device.
int32_t scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SPARSEPR_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SPARSEPR_ERR_INVALID_ARG, "device index beyond " + std::to_string(kMaxDevices));
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(SPARSEPR_ERR_HIP, std::string("hipGetSymbolAddress (scratch): ") + hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SPARSEPR_OK;
}

}  // namespace
}  // namespace spr

using namespace spr;

int32_t sparsepr_dense_attn_noalloc(int32_t heads, int32_t n, int32_t d, const void* q, const void* k,
                                    const void* v, void* o, void* stream) {
    set_call_error("");
    if (heads < 1 || n < 1 || (d != 64 && d != 128))
        return fail(SPARSEPR_ERR_SHAPE, "heads >= 1, n >= 1 and d in {64, 128} required");
    if ((int64_t)heads * n > 0x7fffffffLL)
        return fail(SPARSEPR_ERR_SHAPE, "heads * n beyond 2^31 - 1");
    const int64_t units = ((int64_t)n + kDenseRows - 1) / kDenseRows;
    if (units > kNoAllocMaxUnits)
        return fail(SPARSEPR_ERR_SHAPE, "n = " + std::to_string(n) + " needs " + std::to_string(units) +
                                            " work units; the static scratch holds " +
                                            std::to_string(kNoAllocMaxUnits) + " (n <= " +
                                            std::to_string((int64_t)kNoAllocMaxUnits * kDenseRows) + ")");
    auto aligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (!q || !k || !v || !o || !aligned(q) || !aligned(k) || !aligned(v) || !aligned(o))
        return fail(SPARSEPR_ERR_INVALID_ARG, "null or misaligned q, k, v or o");
    void* base = nullptr;
    if (const int32_t rc = scratch_ptr(&base)) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t* meta = static_cast<int32_t*>(base);
    int2* unit_list = reinterpret_cast<int2*>(static_cast<char*>(base) + kMetaBytes);
    hipLaunchKernelGGL(k_dense_meta, dim3(1), dim3(64), 0, st, meta, n, (int)units);
    launch_units(meta, 1, 1, kDenseRows, (int)units, unit_list, meta + 6, st);
    launch_vbsa(static_cast<const bf16_t*>(q), nullptr, static_cast<const bf16_t*>(k), v, nullptr, heads, n, d,
                meta, 0, meta + 2, 0, meta + 4, 0, 1, unit_list, 0, meta + 6, 0, (int)units, kDenseRows, o,
                1, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SPARSEPR_ERR_HIP, std::string("launch (dense attention): ") + hipGetErrorString(e));
    return SPARSEPR_OK;
}
