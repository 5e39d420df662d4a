// HBM streaming probes: a read-only and a copy kernel with the access pattern
// of one 32 KiB checkpoint tile per 256-thread workgroup (8 x 16-byte loads
// per thread, whole rows per wave instruction); and the stochastic fp16
// rounding of the FP16 checkpoint's flush, applied to a given array.
#include <hip/hip_runtime.h>

#include "../../include/replayssm.h"
#include "../../include/replayssm_probe.h"
#include "common.h"

namespace rssm {
namespace {

constexpr int kBlock = 32768;
constexpr int kThreads = 256;
constexpr int kVec = kBlock / 16 / kThreads;  // 8

__global__ __launch_bounds__(kThreads) void probe_read_kernel(const v4u* src, float* sink) {
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const v4u* p = src + (size_t)wg * (kBlock / 16);
    v4u r[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) r[i] = __builtin_nontemporal_load(p + i * kThreads + threadIdx.x);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kVec; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    // a store the compiler cannot prove dead keeps the loads; it never happens
    // for data whose words do not xor to this pattern
    if (acc == 0x9E3779B9u) sink[wg] = 1.0f;
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(v4u* dst, const v4u* src) {
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const size_t off = (size_t)wg * (kBlock / 16);
    v4u r[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) r[i] = __builtin_nontemporal_load(src + off + i * kThreads + threadIdx.x);
#pragma unroll
    for (int i = 0; i < kVec; ++i) __builtin_nontemporal_store(r[i], dst + off + i * kThreads + threadIdx.x);
}

// fp32 -> fp16 with stochastic rounding, one vector of 4 values per thread,
// with the counters the flush of an FP16 checkpoint uses (vector vec0 + i).
__global__ __launch_bounds__(256) void probe_sr_kernel(const v4f* src, uint2* dst, size_t nvec, uint64_t vec0,
                                                       uint64_t seed) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < nvec) dst[i] = f32x4_to_f16x4_sr(src[i], vec0 + i, seed);
}

int check(size_t bytes) {
    if (bytes % kBlock != 0 || bytes / kBlock > 0x7FFFFFFF) return RSSM_ERR_SHAPE;
    return RSSM_OK;
}

}  // namespace
}  // namespace rssm

extern "C" {

size_t rssm_probe_sink_elems(size_t bytes) { return bytes / rssm::kBlock; }

int rssm_probe_read(const void* src, size_t bytes, float* sink, void* stream) {
    if (!src || !sink) return RSSM_ERR_NULL;
    if (rssm::check(bytes)) return RSSM_ERR_SHAPE;
    if (bytes == 0) return RSSM_OK;
    hipLaunchKernelGGL(rssm::probe_read_kernel, dim3(bytes / rssm::kBlock), dim3(rssm::kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const rssm::v4u*>(src), sink);
    return hipGetLastError() == hipSuccess ? RSSM_OK : RSSM_ERR_HIP;
}

int rssm_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!src || !dst) return RSSM_ERR_NULL;
    if (rssm::check(bytes)) return RSSM_ERR_SHAPE;
    if (bytes == 0) return RSSM_OK;
    hipLaunchKernelGGL(rssm::probe_copy_kernel, dim3(bytes / rssm::kBlock), dim3(rssm::kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<rssm::v4u*>(dst),
                       static_cast<const rssm::v4u*>(src));
    return hipGetLastError() == hipSuccess ? RSSM_OK : RSSM_ERR_HIP;
}

int rssm_probe_sr_f16(const float* src, uint16_t* dst, size_t n, uint64_t vec0, uint64_t seed, void* stream) {
    if (!src || !dst) return RSSM_ERR_NULL;
    if (n % 4 != 0 || n / 4 / 256 >= 0x7FFFFFFF || (uintptr_t)src % 16 || (uintptr_t)dst % 8) return RSSM_ERR_SHAPE;
    if (n == 0) return RSSM_OK;
    const size_t nvec = n / 4;
    hipLaunchKernelGGL(rssm::probe_sr_kernel, dim3((nvec + 255) / 256), dim3(256), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<const rssm::v4f*>(src),
                       reinterpret_cast<uint2*>(dst), nvec, vec0, seed);
    return hipGetLastError() == hipSuccess ? RSSM_OK : RSSM_ERR_HIP;
}

}  // extern "C"
