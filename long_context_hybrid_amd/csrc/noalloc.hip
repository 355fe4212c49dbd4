// lightning_prefill_noalloc: the prefill for callers that cannot allocate device memory.
//
// The prefill's only scratch memory is its workspace of segment-boundary states (written by the
// state-only pass and the scan, read by the main pass, all within one call).  Here it is a
// file-scope device array instead of a caller-owned buffer.  Each device the library runs on
// holds its own copy of the array from the time the code object is loaded until the process
// ends; its address on a device is taken once, with that device current, through
// hipGetSymbolAddress and cached.  Host code never uses the array's name as an address (on the
// host the name is only a stand-in): kernels receive the queried pointer, like the workspace.
//
// Nothing in the array needs to start at zero (every state slot is written before it is read in
// the same call), so the calls clear nothing.  All calls on one device share the array and it
// keeps the last call's contents: calls that overlap on one device (two streams, two threads)
// race and must be ordered by the caller.
#include <mutex>

#include "lt_internal.h"

namespace {

constexpr size_t kScratchBytes = LT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once queried

// The scratch array's device address on the current device.
lt_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return LT_ERR_HIP;
    }
    if (dev >= kMaxDevices) return LT_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return LT_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LT_OK;
}

}  // namespace

extern "C" {

lt_status lightning_prefill_noalloc(const void* q, const void* k, const void* v, const void* gate,
                                    const float* q_norm_w, const float* k_norm_w,
                                    const float* o_norm_w, int norm_w_head_stride,
                                    const double* lambda, double rope_base, double rms_eps,
                                    int64_t pos0, const float* state_in, float* state_out,
                                    void* y, float* o_raw, int B, int T, int H, int d, lt_dtype dtype,
                                    int chunk, int segments, void* stream) {
    if (H <= 0 || d <= 0 || (long long)H * d > 0x7fffffffLL) return LT_ERR_INVALID_ARG;
    // every argument check of the prefill first, so bad arguments launch and query nothing
    lt_status st = lt::prefill_strided(q, k, v, gate, H * d, q_norm_w, k_norm_w, o_norm_w,
                                       norm_w_head_stride, lambda, rope_base, rms_eps, pos0,
                                       state_in, state_out, y, o_raw, B, T, H, d, dtype, chunk,
                                       segments, nullptr, 0, nullptr, stream,
                                       /*validate_only=*/true);
    if (st != LT_OK) return st;
    int c = 0;
    if ((st = lightning_prefill_plan(B, T, H, d, dtype, chunk, segments, &c, nullptr, nullptr)) !=
        LT_OK)
        return st;
    const size_t need = lightning_prefill_workspace_size(B, T, H, d, dtype, chunk, segments);
    if (need > kScratchBytes) return LT_ERR_UNSUPPORTED;  // use lightning_prefill instead
    void* ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws)) != LT_OK) return st;
    return lt::prefill_strided(q, k, v, gate, H * d, q_norm_w, k_norm_w, o_norm_w,
                               norm_w_head_stride, lambda, rope_base, rms_eps, pos0, state_in,
                               state_out, y, o_raw, B, T, H, d, dtype, chunk, segments, ws,
                               need > 0 ? kScratchBytes : 0, nullptr, stream, false);
}

}  // extern "C"
