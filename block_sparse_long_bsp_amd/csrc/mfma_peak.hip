// mfma_peak.hip -- measured matrix-core rate of the part the attention kernel
// runs on (gfx950), for the benchmark's roofline report next to the datasheet
// peak.
//
// Each wave issues a long unrolled chain of MFMAs on kAcc independent
// accumulators, whose operands stay in registers, so nothing but the matrix
// core's issue rate bounds it. One store per lane at the end keeps the work
// live. The launch puts several waves on every SIMD of every compute unit.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kAcc = 4;     // independent accumulators per wave
constexpr int kUnroll = 8;  // MFMAs per accumulator per loop trip

__global__ void __launch_bounds__(256) peak_bf16(int iters, float seed, float *out) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(seed * (float)(lane + i));
        b[i] = (__bf16)(seed * (float)(lane - i));
    }
    f32x16 acc[kAcc];
#pragma unroll
    for (int x = 0; x < kAcc; ++x) acc[x] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int x = 0; x < kAcc; ++x) acc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[x], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < kAcc; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[x][i];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) peak_fp8(int iters, float seed, float *out) {
    const int lane = threadIdx.x & 63;
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (int)(0x38383838u + (uint32_t)((lane + i) & 7) * 0x01010101u);  // small e4m3 codes
        b[i] = (int)(0x38383838u + (uint32_t)((lane ^ i) & 7) * 0x01010101u);
    }
    (void)seed;
    f32x16 acc[kAcc];
#pragma unroll
    for (int x = 0; x < kAcc; ++x) acc[x] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int x = 0; x < kAcc; ++x)
                acc[x] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[x], 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < kAcc; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[x][i];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// FLOPs one call of bsp_probe_mfma performs: 2*M*N*K per MFMA per wave.
double bsp_probe_mfma_flops(int fp8, int blocks, int iters) {
    const double per = fp8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
    return per * kAcc * kUnroll * (double)iters * blocks * 4 /* waves per block */;
}

// Launches the probe on `stream` (asynchronous): `blocks` workgroups of four
// waves, each running iters * kUnroll * kAcc MFMAs. out: device float[blocks * 256].
// Returns 0, or the HIP error code of the launch.
int bsp_probe_mfma(int fp8, int blocks, int iters, float *out, void *stream) {
    if (blocks <= 0 || iters <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
    if (fp8)
        hipLaunchKernelGGL(peak_fp8, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, 1.0f, out);
    else
        hipLaunchKernelGGL(peak_bf16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, 1.0f / 64, out);
    return (int)hipGetLastError();
}

}  // extern "C"
