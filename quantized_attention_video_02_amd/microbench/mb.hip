// Microbenchmarks of the MI355X (gfx950) units the attention kernels are
// bound by: the dense matrix-core rate for INT8, FP8 and FP16 MFMAs, and the
// v_exp_f32 rate.  Register-only kernels: each wave runs eight independent
// accumulation chains (so the matrix core never waits on a result), and one
// float per thread is stored at the end so nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mb_mfma_i8(int iters, float* out) {
    const int t = threadIdx.x;
    v4i a = {t, t + 1, t + 2, t + 3}, b = {t ^ 5, t ^ 6, t ^ 7, t ^ 8};
    v16i c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = v16i{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[k], 0, 0, 0);
    int s = 0;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][15];
    out[blockIdx.x * blockDim.x + t] = (float)s;
}

__global__ __launch_bounds__(256) void mb_mfma_f8(int iters, float* out) {
    const int t = threadIdx.x;
    v8i a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = 0x38383838 ^ (t & 7);
        b[e] = 0x30303030 ^ (e & 3);
    }
    v16f c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = v16f{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int k = 0; k < kChains; ++k)
            c[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[k], 0, 0, 0, 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][15];
    out[blockIdx.x * blockDim.x + t] = s;
}

__global__ __launch_bounds__(256) void mb_mfma_f16(int iters, float* out) {
    const int t = threadIdx.x;
    v8h a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)(0.001f * (t + e));
        b[e] = (_Float16)(0.002f * (e + 1));
    }
    v16f c[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = v16f{};
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[k], 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][15];
    out[blockIdx.x * blockDim.x + t] = s;
}

// v_exp_f32 throughput: 16 independent chains x = exp2(x * -0.5) per thread
__global__ __launch_bounds__(256) void mb_exp(int iters, float* out) {
    const int t = threadIdx.x;
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = 0.001f * (t + k);
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int k = 0; k < 16; ++k) x[k] = __builtin_amdgcn_exp2f(x[k] * -0.5f);
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += x[k];
    out[blockIdx.x * blockDim.x + t] = s;
}

}  // namespace

extern "C" {

// Operations one launch performs: (blocks * 256 threads) / 64 waves x iters x
// chains x the instruction's ops (INT8 32x32x32: 65536, FP8 32x32x64: 131072,
// FP16 32x32x16: 32768; exp: one per lane and chain, 64 per wave instruction).
__attribute__((visibility("default"))) double mb_ops(int kind, int blocks, int iters) {
    const double waves = (double)blocks * 256 / 64;
    switch (kind) {
        case 0: return waves * iters * kChains * 65536.0;
        case 1: return waves * iters * kChains * 131072.0;
        case 2: return waves * iters * kChains * 32768.0;
        case 3: return waves * iters * 16 * 64.0;
        default: return 0.0;
    }
}

// Launch microbenchmark `kind` (0 INT8, 1 FP8, 2 FP16 MFMA, 3 v_exp_f32) with
// `blocks` workgroups of 256 threads; out: device float[blocks * 256].
// Returns 0, or -1 for a bad argument / launch failure.
__attribute__((visibility("default"))) int mb_run(int kind, int blocks, int iters, float* out,
                                                  void* stream) {
    if (!out || blocks < 1 || iters < 1 || kind < 0 || kind > 3) return -1;
    void (*fns[4])(int, float*) = {mb_mfma_i8, mb_mfma_f8, mb_mfma_f16, mb_exp};
    hipLaunchKernelGGL(fns[kind], dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
