// noalloc.hip -- hda_decode_step_noalloc: hda_decode_step with its
// workspace in a static device array of the library instead of a caller
// buffer, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array (`scratch`, kScratchBytes) exists once per GPU the library runs
// on and is held until the process ends.  Host code never passes the
// array's name to a kernel or a copy: the name is a host-side stand-in, not
// a device address.  The first call on a device, with that device current,
// takes the array's device address (hipGetSymbolAddress) and keeps it for
// that device, and zero-fills the array on the caller's stream (the step's
// arrival counters must start at zero; every step leaves them zero).  All
// calls on one GPU share its array: calls that overlap on one GPU (other
// streams, other host threads) race.
#include "hda.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "hda_kernels.h"

namespace hda {
hda_status report_error(hda_status st, const char *msg);
}

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_fill_kernel(uint4 *p, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

std::mutex g_scratch_mu;
void *g_scratch[hda::kMaxDevices];  // device address of `scratch` per device, once set up

// This device's scratch address; set up on the first call on the device.
hda_status device_scratch(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= hda::kMaxDevices) {
        (void)hipGetLastError();
        return hda::report_error(HDA_ERR_HIP, "no current HIP device for the static scratch");
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return hda::report_error(HDA_ERR_HIP, "hipGetSymbolAddress of the static scratch failed");
        }
        hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint4 *>(ptr),
                           kScratchBytes / sizeof(uint4));
        if ((e = hipGetLastError()) != hipSuccess)
            return hda::report_error(HDA_ERR_HIP, "zero fill of the static scratch failed to launch");
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return HDA_OK;
}

}  // namespace

extern "C" hda_status hda_decode_step_noalloc(const void *q, const void *k_new, const void *v_new,
                                              const int32_t *pos, hda_layer_type layer,
                                              const hda_cache_desc *cache, const float *sinks,
                                              const float *gate, float scale, void *out, float *lse,
                                              void *stream) {
    const size_t need = hda_decode_step_workspace_bytes(cache, layer);
    if (need == 0)  // a description hda_decode_step refuses, or nothing to do: it says which
        return hda_decode_step(q, k_new, v_new, pos, layer, cache, sinks, gate, scale, out, lse,
                               nullptr, 0, stream);
    if (need > kScratchBytes) {
        char msg[160];
        snprintf(msg, sizeof(msg), "the step needs %zu bytes of workspace; the static scratch holds %zu",
                 need, kScratchBytes);
        return hda::report_error(HDA_ERR_WORKSPACE, msg);
    }
    void *ws = nullptr;
    const hda_status st = device_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != HDA_OK) return st;
    return hda_decode_step(q, k_new, v_new, pos, layer, cache, sinks, gate, scale, out, lse, ws,
                           kScratchBytes, stream);
}
