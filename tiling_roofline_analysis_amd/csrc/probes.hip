// probes.hip -- measured roofs for the roofline model.
//
// Page "Roofline & Tiling notes"
// (legato-user-group.github.io/tensor2silicon-lab/week04/researchers/jaehyeong)
// bounds a kernel by min(peak flops, bandwidth x arithmetic intensity) and
// uses a vector add as the example of a kernel with almost no reuse (section
// 1, Vector Add example).  These probes measure the two roofs on the device
// itself instead of taking them from a datasheet:
//   * copy  -- a streaming non-temporal float4 copy (no reuse at all): HBM
//              bandwidth when the buffers exceed the caches;
//   * mfma  -- back-to-back independent v_mfma_f32_32x32x2_f32 from
//              registers: the FP32 matrix-core roof;
//   * fma   -- independent v_fma_f32 chains from registers: the FP32 VALU
//              roof of code compiled without packed-FP32 instructions;
//   * launch -- an empty kernel: what a launch costs when it does no work,
//              the floor under the time of any one-launch GEMM.
// Each compute probe writes one value per lane to a sink so nothing is
// optimised away; results are meaningless numbers.
#include <algorithm>

#include "gemm_internal.h"
#include "tra_gemm.h"

namespace tra {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Grid-stride float4 copy with non-temporal loads and stores (streamed data
// is not kept in the caches).  Among copies timed on MI355X (1 GiB, plain or
// non-temporal, 1-4 float4 per lane per step, 1024-16384 workgroups) this
// form with 1024 workgroups moved the most bytes per second.
__global__ __launch_bounds__(kProbeThreads)
void probe_copy_f32(int64_t n4, const f32x4 *__restrict__ src, f32x4 *__restrict__ dst) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x; i < n4;
         i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

__global__ __launch_bounds__(1)
void probe_copy_tail(int64_t from, int64_t n, const float *__restrict__ src,
                     float *__restrict__ dst) {
    for (int64_t i = from; i < n; ++i) dst[i] = src[i];
}

// Four independent accumulators per wave keep the matrix pipe busy.
__global__ __launch_bounds__(kProbeThreads)
void probe_mfma_f32(int64_t iters, float *__restrict__ sink) {
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    const float a = 1e-3f * static_cast<float>(threadIdx.x);
    const float b = 1.0f + 1e-6f * static_cast<float>(blockIdx.x);
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
}

// Eight independent FMA chains per lane.
__global__ __launch_bounds__(kProbeThreads)
void probe_fma_f32(int64_t iters, float *__restrict__ sink) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 1e-3f * static_cast<float>(threadIdx.x + j);
    const float m = 0.999f, c = 1e-7f * static_cast<float>(blockIdx.x + 1);
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = fmaf(x[j], m, c);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += x[j];
    sink[static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
}

// No work: the time of back-to-back launches of this kernel is the launch
// floor (command processing, the cache operations between dependent
// launches, dispatch and completion).  `never` is nonzero at run time, so
// the store is never made; it keeps the kernel from being an empty body.
__global__ __launch_bounds__(kProbeThreads)
void probe_launch(int never, float *__restrict__ sink) {
    if (never == 0 && threadIdx.x == 0) sink[blockIdx.x] = 0.0f;
}

constexpr int64_t kCopyBlocks = 1024;

tra_status finish(hipError_t err) {
    if (err != hipSuccess) {
        record_hip_error(err);
        return TRA_ERR_HIP;
    }
    return TRA_OK;
}

}  // namespace
}  // namespace tra

extern "C" {

double tra_probe_work(int probe, int64_t amount) {
    if (amount < 0) return -1.0;
    const double a = static_cast<double>(amount);
    switch (probe) {
        case TRA_PROBE_COPY: return 8.0 * a;   // bytes: n floats read + n written
        case TRA_PROBE_MFMA:                   // flops
            return static_cast<double>(TRA_PROBE_BLOCKS) * 4 * a * 4 * (2.0 * 32 * 32 * 2);
        case TRA_PROBE_FMA:
            return static_cast<double>(TRA_PROBE_SINK_FLOATS) * a * 8 * 2.0;
        default: return -1.0;
    }
}

tra_status tra_probe_copy_f32(int64_t n, const float *src, float *dst, void *stream) {
    if (n < 0) return TRA_ERR_INVALID_ARG;
    if (n == 0) return TRA_OK;
    if (src == nullptr || dst == nullptr) return TRA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
        return TRA_ERR_INVALID_ARG;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t bytes = static_cast<uintptr_t>(n) * sizeof(float);
    if (s0 < d0 + bytes && d0 < s0 + bytes) return TRA_ERR_INVALID_ARG;   // overlap
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n4 = n / 4;
    if (n4 > 0) {
        const int64_t blocks = std::min<int64_t>(tra::kCopyBlocks, tra::ceil_div(n4, tra::kProbeThreads));
        hipLaunchKernelGGL(tra::probe_copy_f32, dim3(static_cast<uint32_t>(blocks)),
                           dim3(tra::kProbeThreads), 0, s, n4,
                           reinterpret_cast<const tra::f32x4 *>(src), reinterpret_cast<tra::f32x4 *>(dst));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return tra::finish(e);
    }
    if (n4 * 4 < n) {
        hipLaunchKernelGGL(tra::probe_copy_tail, dim3(1), dim3(1), 0, s, n4 * 4, n, src, dst);
        return tra::finish(hipGetLastError());
    }
    return TRA_OK;
}

tra_status tra_probe_launch(int64_t workgroups, void *stream) {
    if (workgroups < 1 || workgroups * tra::kProbeThreads > tra::kMaxGridLanes)
        return TRA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(tra::probe_launch, dim3(static_cast<uint32_t>(workgroups)),
                       dim3(tra::kProbeThreads), 0, static_cast<hipStream_t>(stream), 1,
                       static_cast<float *>(nullptr));
    return tra::finish(hipGetLastError());
}

tra_status tra_probe_mfma_f32(int64_t iters, float *sink, void *stream) {
    if (iters < 0 || sink == nullptr) return TRA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(tra::probe_mfma_f32, dim3(TRA_PROBE_BLOCKS), dim3(tra::kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    return tra::finish(hipGetLastError());
}

tra_status tra_probe_fma_f32(int64_t iters, float *sink, void *stream) {
    if (iters < 0 || sink == nullptr) return TRA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(tra::probe_fma_f32, dim3(TRA_PROBE_BLOCKS), dim3(tra::kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    return tra::finish(hipGetLastError());
}

}  // extern "C"
