// noalloc.hip -- mm_execute_noalloc: mm_execute with the split partial sums
// in a fixed device array of the library instead of the plan's workspace,
// for callers that cannot allocate device memory.
//
// The array lives for the whole process on every device the library runs
// on.  Its device address differs per device and is not the host name of the
// symbol: it is looked up once per device, with that device current, and
// only that address is ever handed to kernels.  Every call on one device
// shares the array, so calls that overlap on a device (concurrent streams or
// threads) race; a call overwrites every partial sum it later reads, so
// nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "plan.h"

namespace mm {

// Largest workspace a plan may need to run here: 16 MiB (for example 256
// partitions of a 64 x 64 FP32 output take 4 MiB).
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::mutex g_scratch_mutex;
static void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call for that device).
static mm_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(MM_ERR_HIP, "device %d beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(MM_ERR_HIP, "hipGetSymbolAddress of the scratch array on device %d: %s", dev,
                        hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MM_OK;
}

}  // namespace mm

using namespace mm;

extern "C" mm_status mm_execute_noalloc(mm_plan_t p, const void *A, const void *B, void *Y, void *stream) {
    clear_error();
    if (!p) return fail(MM_ERR_NULL_ARG, "plan is NULL");
    if (p->is_gemm) return fail(MM_ERR_BAD_OPTION, "a Gemm plan runs through mm_gemm_execute");
    if (p->is_int) return fail(MM_ERR_BAD_OPTION, "a MatMulInteger plan runs through mm_int_execute");
    if (p->workspace_bytes > (int64_t)kScratchBytes)
        return fail(MM_ERR_TOO_LARGE,
                    "the plan needs %lld workspace bytes; mm_execute_noalloc has %zu (use mm_execute, or a plan "
                    "with fewer K partitions)",
                    (long long)p->workspace_bytes, kScratchBytes);
    void *ws = nullptr;
    if (p->workspace_bytes > 0 && p->algo != MM_ALGO_EMPTY && p->algo != MM_ALGO_ZERO_FILL) {
        mm_status st = scratch_address(&ws);
        if (st != MM_OK) return st;
    }
    return execute_plan(p, A, B, nullptr, Y, stream, ws);
}
