// Mask prediction for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the same
// computation as sa_predict_mask_gather, with its workspace in a fixed
// device array of this library instead of a caller buffer.
//
// The array lives in the code object, one copy per GPU the library is loaded
// on, for the life of the process.  Its address on a device is looked up once,
// with that device current, on the first call there; host code only ever
// passes that address on (the array's name in host code is a stand-in, not a
// device address).  Every call on one GPU uses the same array, so calls that
// overlap on one GPU (on different streams, without ordering between them)
// race; calls ordered on one stream do not.  Nothing in the array has to start
// at zero: every section the prediction reads is written by the same call
// before it is read.
#include <mutex>

#include "sa_internal.h"

namespace sa {
namespace {

static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

// Address of this device's copy of the array (looked up once per device).
int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SA_ERR_HIP;
    if (dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SA_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return SA_OK;
}

}  // namespace
}  // namespace sa

using namespace sa;

extern "C" int sa_predict_mask_gather_noalloc(const uint16_t* q, const uint16_t* k, const int32_t* perm_dev,
                                              const sa_mask_params* p, int32_t* row_ptr, int32_t* col_idx,
                                              int64_t col_cap, uint8_t* mask_out, float* sim_q, float* sim_k,
                                              int32_t* dev_status, void* stream) {
    if (!perm_dev) return SA_ERR_INVALID_ARGUMENT;
    PredictShape s;
    const int st = predict_shape(p, &s);
    if (st != SA_OK) return st;
    if (s.bytes > size_t(SA_NOALLOC_SCRATCH_BYTES)) return SA_ERR_CAPACITY;
    void* ws = nullptr;
    const int got = scratch_of_current_device(&ws);
    if (got != SA_OK) return got;
    return predict_mask_impl(q, k, perm_dev, nullptr, p, ws, size_t(SA_NOALLOC_SCRATCH_BYTES), row_ptr, col_idx,
                             col_cap, mask_out, sim_q, sim_k, dev_status, stream);
}
