// moe_forward_noalloc: the whole layer with its scratch memory in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array lives once per GPU for the life of the process.  Its device
// address is taken with hipGetSymbolAddress on the first call made on each
// device (with that device current) and kept per device; host code only ever
// passes that address on, never the array's own name, which in host code is
// a stand-in rather than a device address.  Nothing here allocates: the
// layer's kernels run as in moe_forward, on the address of the array, all
// on the caller's stream (the shared expert too: no side stream is made).
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "moe.h"

namespace moe {
// Sets the calling thread's moe_last_error() text and returns `code`.
int report_error(int code, const char* msg);
// moe_forward, with the shared expert on the caller's stream when
// overlap_shared is false (no side stream or event is created).
int forward(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
            const uint16_t* w_gate_up, const uint16_t* w_down, const void* packed_weights,
            const uint16_t* ws_gate_up, const uint16_t* ws_down, float* out,
            int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out, void* workspace,
            size_t ws_bytes, void* stream, bool overlap_shared);
}  // namespace moe

namespace {

static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up once.
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return moe::report_error(MOE_ERR_HIP, (std::string("hipGetDevice: ") +
                                               hipGetErrorString(e)).c_str());
    if (dev < 0 || dev >= kMaxDevices)
        return moe::report_error(MOE_ERR_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return moe::report_error(MOE_ERR_HIP, (std::string("hipGetSymbolAddress(scratch): ") +
                                                   hipGetErrorString(e)).c_str());
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const moe_shape* shape, const uint16_t* x,
                                   const float* w_router, const float* bias,
                                   const uint16_t* w_gate_up, const uint16_t* w_down,
                                   const void* packed_weights, const uint16_t* ws_gate_up,
                                   const uint16_t* ws_down, float* out, int32_t* topk_ids_out,
                                   float* topk_w_out, int32_t* counts_out, void* stream) {
    const size_t need = moe_workspace_bytes(shape);
    if (need == 0) {
        // Invalid shape: moe_forward reports it (with its text) before any work.
        return moe_forward(shape, x, w_router, bias, w_gate_up, w_down, packed_weights,
                           ws_gate_up, ws_down, out, topk_ids_out, topk_w_out, counts_out,
                           nullptr, 0, stream);
    }
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return moe::report_error(
            MOE_ERR_WORKSPACE,
            ("moe_forward_noalloc: this shape needs " + std::to_string(need) +
             " bytes of scratch, above the fixed MOE_NOALLOC_SCRATCH_BYTES = " +
             std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES) + "; use moe_forward")
                .c_str());
    void* ws = nullptr;
    if (int rc = scratch_address(&ws)) return rc;
    return moe::forward(shape, x, w_router, bias, w_gate_up, w_down, packed_weights, ws_gate_up,
                        ws_down, out, topk_ids_out, topk_w_out, counts_out, ws,
                        MOE_NOALLOC_SCRATCH_BYTES, stream, false);
}
