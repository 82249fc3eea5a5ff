// Measured bf16 MFMA throughput of this GPU (a reference for the attention kernel's utilisation).
//
// Every wavefront issues `iters` rounds of eight independent v_mfma_f32_32x32x16_bf16 chains on
// register operands: no memory traffic, no LDS, no dependences closer than eight instructions,
// so the matrix pipe of each SIMD is the only limit.  FLOPs per launch =
// wgs * 4 wavefronts * iters * 8 * (2 * 32 * 32 * 16).  Built into its own library (libsift_probe.so):
// it is a measuring tool, not part of the prefill path.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr int kChains = 8;

__global__ __launch_bounds__(kProbeThreads) void mfma_peak_kernel(int iters, float seed, float *__restrict__ sink) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(seed * static_cast<float>((threadIdx.x + i) & 7));
        b[i] = static_cast<__bf16>(seed * static_cast<float>((threadIdx.x ^ i) & 7));
    }
    f32x16 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += c[j][i];
    sink[static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = s;
}

}  // namespace

// Launch `wgs` workgroups of 256 threads on `stream`; d_sink must hold wgs * 256 floats.
// Returns the launch's hipError_t (0 = success); rejects non-positive sizes with
// hipErrorInvalidValue before any launch.
extern "C" int sift_probe_mfma_bf16(int wgs, int iters, float *d_sink, hipStream_t stream) {
    if (wgs <= 0 || iters <= 0 || d_sink == nullptr) return static_cast<int>(hipErrorInvalidValue);
    mfma_peak_kernel<<<wgs, kProbeThreads, 0, stream>>>(iters, 1.0e-3f, d_sink);
    return static_cast<int>(hipGetLastError());
}

// FLOPs of one launch with these sizes.
extern "C" double sift_probe_mfma_bf16_flops(int wgs, int iters) {
    return static_cast<double>(wgs) * (kProbeThreads / 64) * iters * kChains * (2.0 * 32 * 32 * 16);
}
