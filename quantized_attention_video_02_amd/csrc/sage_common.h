// Internal definitions shared by the libsage HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef unsigned short u16;

constexpr int kBlk = 128;          // rows per Q / K quantization block
constexpr int kBc = 128;           // keys per online-softmax tile (== kBlk)
constexpr int kBr = 256;           // queries per dense attention workgroup (8 waves x 32)
constexpr int kAttnThreads = 512;  // 8 wave64s
// Q-smoothing correction kernel: keys per thread, query blocks per register
// group (q_mean is padded to a multiple of this many blocks), blocks per
// workgroup slice.
constexpr int kBiasKeys = 4, kBiasBlocks = 16, kBiasSlice = 128;
constexpr int kMaxSparseTiles = 2048;  // key tiles a sparse launch may list (N <= 262144)
constexpr int kStatsChunk = 512;   // tokens per statistics workgroup
constexpr int kQuantThreads = 256;
constexpr float kPScale = 448.0f;
// fp32 nearest to log2(448) = 8.807354922057604...
constexpr float kLog2PScale = 0x1.19d5dap+3f;

// Offset (in elements) of row n of head (b, h) in a [B,H,N,d] or [B,N,H,d] tensor.
__device__ __host__ inline int64_t row_offset(int layout, int b, int h, int n, int H, int N,
                                              int d) {
    return layout == 0 ? ((int64_t)(b * H + h) * N + n) * d : ((int64_t)b * N + n) * H * d +
                                                                  (int64_t)h * d;
}

__device__ inline float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ inline uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Wave-wide max of a non-negative float (all 64 lanes hold a value).
__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Arguments of the fused attention kernel (one struct, passed by value).
struct AttnArgs {
    const int8_t* q8;
    const float* q_scale;
    const int8_t* k8;
    const float* k_scale;
    const void* vq;
    const float* v_scale;
    void* out;
    int32_t* s_out;  // debug dump (dump instantiations only)
    int H, N, N_pad, nblk, nqt, total, layout, out_fp32;
    int qtok;  // 1: q_scale per query row [bh][N_pad]; 0: per block of kBlk rows [bh][nblk]
    const uint8_t* tmask;  // NULL (dense) or [B*H][nblk][nblk]: query block x key tile, nonzero = visit
    const float* bias;     // NULL, or the Q-smoothing correction [B*H][nblk][N_pad] (exp2 units)
    float lambda;    // fp32(sm_scale * log2 e)
    int dbh, drow0, dnrows;
    float* lse = nullptr;  // NULL, or [B*H][N]: each row's log-sum-exp in the exp2 domain
};

// The 8-bit backward: the operands prepared once per call (workspace) and
// the two sweeps' arguments.
struct BwdPrep {
    const u16* o;   // forward output, bf16, layout
    const u16* dO;  // upstream gradient, bf16, layout
    const u16* v;   // V, bf16, layout
};
// Per-tile record of the dK/dV sweep, one per (bh, query block), copied into
// LDS with the tile: lse and D of the block's rows, its Q scale and dO scale.
constexpr int kRecFloats = 512;  // 2 KB: [0, 128) lse, [128, 256) -D, 256 q_scale, 257 s_do
struct BwdArgs {
    const int8_t* q8;
    const float* q_scale;  // per block of kBlk queries [bh][nblk]
    const int8_t* k8;
    const float* k_scale;
    const float* lse;      // [bh][N]
    float* Dq;             // [bh][N_pad]: dO_i . O_i
    float* s_do;           // [bh][nblk]: FP8 scale of dO per block
    _Float16* do16;        // [bh][N_pad][d]
    _Float16* v16;         // [bh][N_pad][d]
    uint8_t* do8;          // [bh][nblk][d][128], rows in the FP8 reduction order
    int8_t* qT8;           // [bh][nblk][d][128], rows in the INT8 reduction order
    int8_t* kT8;
    float* rec;            // [bh][nblk][kRecFloats]
    float* dq;             // outputs, fp32, layout
    float* dk;
    float* dv;
    int H, N, N_pad, nblk, total, layout;
    float lambda, sm_scale;
};

hipError_t launch_quant_qk(const u16* q, const u16* k, int B, int H, int N, int d, int layout,
                           int qtok,
                           int8_t* q8, float* qs, int8_t* k8, float* ks, float* kmean,
                           float* qmean, uint64_t* ws, hipStream_t s);
hipError_t launch_q_bias(const float* qmean, const u16* k, const float* kmean, int B, int H, int N,
                         int d, int layout, float lambda, float* bias, hipStream_t s);
// MX element format fmt: 6 = E2M3 (MXFP6), 4 = E2M1 (MXFP4)
hipError_t launch_quant_qk_mx(const u16* q, const u16* k, int B, int H, int N, int d, int layout,
                              int fmt, uint8_t* q6, uint8_t* k6, float* kmean, uint64_t* ws,
                              hipStream_t s);
hipError_t launch_quant_v_mx(const u16* v, int B, int H, int N, int d, int layout, int fmt,
                             uint8_t* v6, hipStream_t s);
hipError_t launch_attn_mx(const AttnArgs& args, int B, int d, int causal, int fmt, hipStream_t s);
hipError_t launch_quant_v(const u16* v, int B, int H, int N, int d, int layout, int pv16,
                          void* vq, float* vscale, float* ws, hipStream_t s);
hipError_t launch_quant_qkv(const u16* q, const u16* k, const u16* v, int B, int H, int N, int d,
                            int layout, int pv16, int8_t* q8, float* qs, int8_t* k8, float* ks,
                            float* kmean, void* vq, float* vscale, uint64_t* kws, float* vws,
                            hipStream_t s);
// Bytes of the fixed scratch behind sage_quant_qkv_noalloc, and its device
// address for the stream's (current) device.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(hipStream_t s, void** out);
hipError_t launch_attn(const AttnArgs& args, int B, int d, int pv16, int causal, int dump,
                       hipStream_t s);
hipError_t launch_attn_bwd(const BwdPrep& pp, const BwdArgs& args, int B, int d, int causal,
                           hipStream_t s);

}  // namespace sage
