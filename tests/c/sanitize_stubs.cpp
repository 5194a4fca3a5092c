// Host-only stand-ins for the kernel launchers of the C ABI, so that the
// argument validation in api.cpp can be built and run under AddressSanitizer
// and UndefinedBehaviorSanitizer on a machine without a GPU.  Each stand-in
// records the call and reports success; no device code exists in this
// build.
#include <hip/hip_runtime.h>

#include "../../block_sparse_gemm_amd/csrc/kernels.hpp"

int g_launches = 0;             // read by the driver
bsg::TopoJob g_route_topo = {};  // the last routing launch's topology job
bsg::PermJob g_route_perm = {};  // and its permutation job

bsg::GemmParams g_dsd = {};      // the last DSD launch's parameters

extern "C" const char* hipGetErrorString(hipError_t) { return "host-only build"; }
// the compute-unit lookup behind bsg_dsd's split and its size query: one
// device with 256 compute units
extern "C" hipError_t hipGetDevice(int* dev) {
    *dev = 0;
    return hipSuccess;
}
extern "C" hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* dev) {
    *dev = 0;
    return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
    *value = 256;
    return hipSuccess;
}

namespace bsg {

static int32_t g_scratch[16];

hipError_t route_scratch(hipStream_t, int32_t** out) {
    *out = g_scratch;
    return hipSuccess;
}

hipError_t launch_route(const float*, int64_t, int, int, int, int, int32_t*, float*, int32_t*,
                        int32_t*, int32_t*, int32_t*, const TopoJob& topo, const PermJob& perm,
                        hipStream_t) {
    ++g_launches;
    g_route_topo = topo;
    g_route_perm = perm;
    return hipSuccess;
}

hipError_t launch_route_backward(const float*, int64_t, int, int, int, const int32_t*,
                                 const int32_t*, const void*, int, int, const void*, int, int64_t,
                                 float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_permute_pad(const void*, int, int64_t, int, int, const int32_t*, const float*,
                              const int32_t*, const int32_t*, int, int, int64_t, int32_t*, void*,
                              hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_permute_gate_backward(const void*, int, int64_t, int, int, const int32_t*,
                                        const float*, const int32_t*, const int32_t*, int, int,
                                        int64_t, int32_t*, void*, const float*, int,
                                        const int32_t*, const void*, int, int64_t, float*,
                                        hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_build_topology(const int32_t*, int, int, int, int64_t, int64_t, int32_t*,
                                 int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*,
                                 int32_t*, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_sdd(const GemmParams&, int64_t, int, int, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_dsd(const GemmParams& p, int64_t, int, int, int, hipStream_t) {
    ++g_launches;
    g_dsd = p;
    return hipSuccess;
}

hipError_t launch_dstd(const GemmParams&, int, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_unpermute_combine(const void*, int, int64_t, const int32_t*, const float*,
                                    int64_t, int, int, void*, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_stream_copy(const void*, void*, int64_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

}  // namespace bsg
