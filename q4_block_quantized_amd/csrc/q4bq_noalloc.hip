// Fixed device scratch for the entry point that allocates nothing
// (mul_mat_q4_0_q8_0_noalloc): a file-scope device array of
// Q4BQ_NOALLOC_SCRATCH_BYTES, one copy per GPU the library runs on, held until
// the process ends.  The host never uses the array's name as an address: its
// device address is looked up once per device, with that device current, and
// that pointer is what the launches receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "q4bq.h"
#include "q4bq_internal.h"

static __device__ __align__(256) uint8_t scratch[Q4BQ_NOALLOC_SCRATCH_BYTES];

namespace q4bq {

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

void* noalloc_scratch(int device, hipError_t* err) {
    if (device < 0 || device >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_once[device], [device] {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_err[device] = e == hipSuccess && p == nullptr ? hipErrorInvalidSymbol : e;
        g_ptr[device] = e == hipSuccess ? p : nullptr;
    });
    *err = g_err[device];
    return g_err[device] == hipSuccess ? g_ptr[device] : nullptr;
}

}  // namespace q4bq
