// prefill_static.hip -- kda_prefill_varlen_static: the chunked prefill with
// its workspace in a static device buffer, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The kernels are the prefill's own; only the workspace differs.

#include <hip/hip_runtime.h>

#include <atomic>

#include "kda.h"
#include "kda_launch.h"

namespace {

// The workspace of every kda_prefill_varlen_static call on a device.  Each
// device that runs the library holds its own copy from the moment the code is
// loaded onto it until the process ends.  In host code `scratch` names a host
// stand-in, never the device memory: kernels receive the address that
// hipGetSymbolAddress returns for the current device (scratch_on_device).
static __device__ __align__(256) char scratch[KDA_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (a lookup racing with another thread's stores the same address).
hipError_t scratch_on_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" kda_status kda_prefill_varlen_static(const kda_config* cfg, int32_t num_seqs, int64_t total_tokens,
                                                const int32_t* cu_seqlens, const int64_t* start_pos, const void* q,
                                                const void* k, const void* v, const void* z, const float* g,
                                                const float* beta, const float* conv_w, const float* norm_w,
                                                void* state_pool, void* conv_pool, int32_t num_slots,
                                                const int32_t* init_slot, const int32_t* final_slot,
                                                int32_t ckpt_interval, void* ckpt_state, void* ckpt_conv,
                                                int32_t num_ckpt_slots, const int32_t* ckpt_base, int32_t flags,
                                                void* out, void* stream) {
    // the size check first: a call the buffer cannot hold launches nothing
    const size_t need = kda_prefill_workspace_bytes(cfg, num_seqs, total_tokens, ckpt_interval, flags);
    if (need == 0) {
        // invalid configuration, sizes or flags: kda_prefill_varlen reports
        // them (and launches nothing)
        return kda_prefill_varlen(cfg, num_seqs, total_tokens, cu_seqlens, start_pos, q, k, v, z, g, beta, conv_w,
                                  norm_w, state_pool, conv_pool, num_slots, init_slot, final_slot, ckpt_interval,
                                  ckpt_state, ckpt_conv, num_ckpt_slots, ckpt_base, flags, out, nullptr, 0, stream);
    }
    if (need > static_cast<size_t>(KDA_STATIC_WORKSPACE_BYTES))
        return static_cast<kda_status>(kda::set_error(
            KDA_ERR_WORKSPACE, "this call needs %zu bytes of workspace; the static workspace holds %lld",
            need, static_cast<long long>(KDA_STATIC_WORKSPACE_BYTES)));
    void* ws = nullptr;
    const hipError_t e = scratch_on_device(&ws);
    if (e != hipSuccess)
        return static_cast<kda_status>(
            kda::set_error(KDA_ERR_HIP, "static workspace address: %s", hipGetErrorString(e)));
    return kda_prefill_varlen(cfg, num_seqs, total_tokens, cu_seqlens, start_pos, q, k, v, z, g, beta, conv_w,
                              norm_w, state_pool, conv_pool, num_slots, init_slot, final_slot, ckpt_interval,
                              ckpt_state, ckpt_conv, num_ckpt_slots, ckpt_base, flags, out, ws,
                              static_cast<size_t>(KDA_STATIC_WORKSPACE_BYTES), stream);
}
