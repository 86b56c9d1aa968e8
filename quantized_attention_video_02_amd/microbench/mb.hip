// Microbenchmarks of the MI355X (gfx950) units the attention kernels are
// bound by: the dense matrix-core rate for INT8, FP8 and FP16 MFMAs, and the
// v_exp_f32 rate; and premise checks of the hardware behaviour the
// attention kernels rely on (FP8 matrix-core accumulation, the fp32 -> e4m3
// and fp32 -> E2M1 converts).  The timing kernels are register-only: each wave runs eight independent
// accumulation chains (so the matrix core never waits on a result), and one
// float per thread is stored at the end so nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
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

// Premise checks (not timings).  One wave per problem: D = A B + C on the FP8
// matrix core with the attention kernels' call form (e4m3 operands, no block
// scales), shape 0 the 32x32x64 instruction, 1 the 16x16x128 one.  Operands
// are register images: A and B 8 dwords per lane, C and D 16 (shape 0) or 4
// (shape 1) floats per lane, lane-major, one image per problem.
__global__ __launch_bounds__(64) void mb_f8_mfma_k(int shape, const int* __restrict__ A,
                                                   const int* __restrict__ B,
                                                   const float* __restrict__ C,
                                                   float* __restrict__ D) {
    const int l = threadIdx.x, pb = blockIdx.x;
    v8i a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = A[(pb * 64 + l) * 8 + e];
        b[e] = B[(pb * 64 + l) * 8 + e];
    }
    if (shape == 0) {
        v16f c;
#pragma unroll
        for (int r = 0; r < 16; ++r) c[r] = C[(pb * 64 + l) * 16 + r];
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) D[(pb * 64 + l) * 16 + r] = c[r];
    } else {
        v4f c;
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = C[(pb * 64 + l) * 4 + r];
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) D[(pb * 64 + l) * 4 + r] = c[r];
    }
}

// The packed fp32 -> e4m3 convert in the attention kernels' call form (no
// clamp; two calls fill the low then the high half of a dword): thread i
// converts the fp32 bit patterns first + 4i .. first + 4i + 3.
__global__ __launch_bounds__(256) void mb_cvt_e4m3_k(uint32_t first, uint32_t nquad,
                                                     uint32_t* __restrict__ out) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= nquad) return;
    const uint32_t u = first + 4u * i;
    const float x0 = __uint_as_float(u), x1 = __uint_as_float(u + 1), x2 = __uint_as_float(u + 2),
                x3 = __uint_as_float(u + 3);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
    out[i] = (uint32_t)w;
}

// Eight consecutive fp32 bit patterns first + 8 i + [0, 8) per thread, each
// pair (2 j, 2 j + 1) through v_cvt_scalef32_pk_fp4_f32 with the given scale
// into byte j of one output dword.
__global__ __launch_bounds__(256) void mb_cvt_fp4_k(uint32_t first, uint32_t noct, float scale,
                                                    uint32_t* __restrict__ out) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= noct) return;
    const uint32_t u = first + 8u * i;
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(u), __uint_as_float(u + 1), scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(u + 2), __uint_as_float(u + 3), scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(u + 4), __uint_as_float(u + 5), scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __uint_as_float(u + 6), __uint_as_float(u + 7), scale, 3);
    out[i] = w;
}

}  // namespace

extern "C" {

// D = A B + C for nprob independent problems on the FP8 matrix core (see
// mb_f8_mfma_k for the operand images; all device pointers).  Returns 0, or
// -1 for a bad argument / launch failure.
__attribute__((visibility("default"))) int mb_f8_mfma(int shape, int nprob, const int* A,
                                                      const int* B, const float* C, float* D,
                                                      void* stream) {
    if (!A || !B || !C || !D || (shape != 0 && shape != 1) || nprob < 1 || nprob > 65535)
        return -1;
    hipLaunchKernelGGL(mb_f8_mfma_k, dim3(nprob), dim3(64), 0, (hipStream_t)stream, shape, A, B,
                       C, D);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// out[j] = e4m3 code of the fp32 bit pattern first + j, j < count (device
// uint8 buffer of count bytes, 4-byte aligned).  count: a multiple of 4 with
// first + count <= 2^32.  Returns 0 or -1.
__attribute__((visibility("default"))) int mb_cvt_e4m3(uint32_t first, uint64_t count, void* out,
                                                       void* stream) {
    if (!out || ((uintptr_t)out & 3u) || count == 0 || (count & 3u) ||
        (uint64_t)first + count > (1ull << 32))
        return -1;
    const uint32_t nquad = (uint32_t)(count / 4);
    hipLaunchKernelGGL(mb_cvt_e4m3_k, dim3((nquad + 255u) / 256u), dim3(256), 0,
                       (hipStream_t)stream, first, nquad, (uint32_t*)out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// out[j] = the byte v_cvt_scalef32_pk_fp4_f32 makes of the fp32 bit patterns
// first + 2 j and first + 2 j + 1 with the given scale, j < count / 2 (device
// uint8 buffer of count / 2 bytes, 4-byte aligned).  count: a multiple of 8
// with first + count <= 2^32.  Returns 0 or -1.
__attribute__((visibility("default"))) int mb_cvt_fp4(uint32_t first, uint64_t count, float scale,
                                                      void* out, void* stream) {
    if (!out || ((uintptr_t)out & 3u) || count == 0 || (count & 7u) ||
        (uint64_t)first + count > (1ull << 32))
        return -1;
    const uint32_t noct = (uint32_t)(count / 8);
    hipLaunchKernelGGL(mb_cvt_fp4_k, dim3((noct + 255u) / 256u), dim3(256), 0, (hipStream_t)stream,
                       first, noct, scale, (uint32_t*)out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

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
