// Smoothing and quantization pass of libsage (gfx950): HBM-bound kernels.
//
//   k_stats / v_stats : per (b, h, chunk of 512 tokens) partial column
//                       statistics (exact fixed-point K sums; V absmax),
//   k_mean / v_scale  : per (b, h, channel) combination of the partials,
//   quant_qk          : per (b, h, block of 128 rows) INT8 codes + scale
//                       (optionally Q smoothed by the block's token mean),
//   q_bias            : the Q-smoothing correction q_mean . k' per (block, key),
//   quant_v           : per (b, h, tile of 128 keys) FP8 e4m3 (or FP16) codes,
//                       transposed to [channel][key] with the key order the
//                       attention kernel's P V operand expects.
//
// Method: wxsanhe.com TurboDiffusion post, section 三.1 (Q K to INT8, P V to
// FP8/FP16, outlier smoothing); reportify.cn SageAttention3 summary, bullet
// 8比特训练 (per-block INT8).  Every read is a 16-byte vector load of a row
// chunk; consecutive lanes read consecutive chunks of a row, so each wave
// reads whole rows.  The partial-sum layout makes every reduction order-free
// (wrapping int64 adds, max), so results are bitwise deterministic.
#include <mutex>

#include "sage_common.h"

namespace sage {

// trunc(x * 2^30) of the bf16 value with bit pattern u, saturated at +-2^62,
// NaN -> 0 (the fixed-point grid of the K mean).
__device__ inline uint64_t fix30_bf16(uint32_t u) {
    const uint32_t e = (u >> 7) & 0xffu, man = u & 0x7fu;
    const bool neg = (u >> 15) & 1u;
    uint64_t mag;
    if (e == 0xffu) {
        if (man) return 0;
        mag = 1ull << 62;
    } else {
        const uint32_t M = e ? (128u + man) : man;  // value = M * 2^(E - 134)
        const int sh = (e ? (int)e : 1) - 104;      // x * 2^30 = M * 2^sh
        if (sh > 54) mag = 1ull << 62;
        else if (sh >= 0) mag = (uint64_t)M << sh;
        else mag = (-sh >= 32) ? 0ull : (uint64_t)(M >> (-sh));
    }
    return neg ? (0ull - mag) : mag;
}

// Workgroup body of the K statistics: chunk blockIdx.x of head blockIdx.y;
// red is the workgroup's LDS reduction buffer.
template <int D>
__device__ inline void k_stats_body(const u16* __restrict__ k, int H, int N, int layout,
                                    int nchunk, uint64_t* __restrict__ part,
                                    uint64_t (*red)[D]) {
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    constexpr int RPI = kQuantThreads / CPR;    // rows per pass
    const int chunk = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, cg = t % CPR, tr = t / CPR;
    const int n0 = chunk * kStatsChunk, n1 = min(N, n0 + kStatsChunk);
    uint64_t acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0;
    // Fast path: while every value of a load has |x| < 2^18, each term
    // trunc(x 2^30) is an integer below 2^48 and the fp64 chain
    // bf16 -> fp32 -> fp64, * 2^30, trunc, + is exact; a thread adds at most
    // 512 / RPI <= 32 such terms per channel, below 2^53, so its fp64 sum is the
    // exact integer.  Loads holding larger values, infinities or NaNs take
    // the integer path (saturation, NaN -> 0), the same function of the data.
    double accd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) accd[e] = 0.0;
    static_assert(kStatsChunk / RPI <= 32, "fp64 partial sums must stay below 2^53");
#pragma unroll 4
    for (int n = n0 + tr; n < n1; n += RPI) {
        const uint4 w = *(const uint4*)(k + row_offset(layout, b, h, n, H, N, D) + cg * 8);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        bool big = false;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            big |= ((ws[e] & 0x7fffu) >= 0x4880u) | (((ws[e] >> 16) & 0x7fffu) >= 0x4880u);
        if (!big) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                accd[2 * e] += __builtin_trunc((double)__uint_as_float(ws[e] << 16) * 1073741824.0);
                accd[2 * e + 1] += __builtin_trunc((double)__uint_as_float(ws[e] & 0xffff0000u) *
                                                   1073741824.0);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += fix30_bf16(ws[e] & 0xffffu);
                acc[2 * e + 1] += fix30_bf16(ws[e] >> 16);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tr][cg * 8 + e] = acc[e] + (uint64_t)(int64_t)accd[e];
    __syncthreads();
    if (t < D) {
        uint64_t s = 0;
#pragma unroll 8
        for (int r = 0; r < RPI; ++r) s += red[r][t];
        part[((int64_t)bh * nchunk + chunk) * D + t] = s;
    }
}

template <int D>
__global__ __launch_bounds__(kQuantThreads) void k_stats_kernel(const u16* __restrict__ k, int H,
                                                                int N, int layout, int nchunk,
                                                                uint64_t* __restrict__ part) {
    __shared__ uint64_t red[kQuantThreads / (D / 8)][D];
    k_stats_body<D>(k, H, N, layout, nchunk, part, red);
}

// Combination kernels: workgroup (b*h, group of 32 channels), 256 threads =
// 32 channels x 8 chunk lanes; lane j adds chunks j, j + 8, ... (coalesced
// across the 32 channels), then the 8 lane results are combined in LDS.
constexpr int kCombCh = 32, kCombLanes = kQuantThreads / kCombCh;

__device__ inline void k_mean_body(const uint64_t* __restrict__ part, int nchunk, int D, int N,
                                   float* __restrict__ mean, uint64_t (*red)[kCombCh]) {
    const int bh = blockIdx.x, c = blockIdx.y * kCombCh + threadIdx.x % kCombCh;
    const int j = threadIdx.x / kCombCh;
    uint64_t s = 0;
    for (int ch = j; ch < nchunk; ch += kCombLanes) s += part[((int64_t)bh * nchunk + ch) * D + c];
    red[j][threadIdx.x % kCombCh] = s;
    __syncthreads();
    if (j == 0) {
#pragma unroll
        for (int r = 1; r < kCombLanes; ++r) s += red[r][threadIdx.x];
        mean[bh * D + c] = (float)((double)(int64_t)s / ((double)N * 1073741824.0));
    }
}

__global__ __launch_bounds__(kQuantThreads) void k_mean_kernel(const uint64_t* __restrict__ part,
                                                               int nchunk, int D, int N,
                                                               float* __restrict__ mean) {
    __shared__ uint64_t red[kCombLanes][kCombCh];
    k_mean_body(part, nchunk, D, N, mean, red);
}

template <int D>
__device__ inline void v_stats_body(const u16* __restrict__ v, int H, int N, int layout,
                                    int nchunk, float* __restrict__ part, float (*red)[D]) {
    constexpr int CPR = D / 8;
    constexpr int RPI = kQuantThreads / CPR;
    const int chunk = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, cg = t % CPR, tr = t / CPR;
    const int n0 = chunk * kStatsChunk, n1 = min(N, n0 + kStatsChunk);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll 4
    for (int n = n0 + tr; n < n1; n += RPI) {
        const uint4 w = *(const uint4*)(v + row_offset(layout, b, h, n, H, N, D) + cg * 8);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = fmaxf(acc[2 * e], bf16_bits_to_f32(ws[e] & 0x7fffu));
            acc[2 * e + 1] = fmaxf(acc[2 * e + 1], bf16_bits_to_f32((ws[e] >> 16) & 0x7fffu));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tr][cg * 8 + e] = acc[e];
    __syncthreads();
    if (t < D) {
        float s = 0.0f;
        for (int r = 0; r < RPI; ++r) s = fmaxf(s, red[r][t]);
        part[((int64_t)bh * nchunk + chunk) * D + t] = s;
    }
}

template <int D>
__global__ __launch_bounds__(kQuantThreads) void v_stats_kernel(const u16* __restrict__ v, int H,
                                                                int N, int layout, int nchunk,
                                                                float* __restrict__ part) {
    __shared__ float red[kQuantThreads / (D / 8)][D];
    v_stats_body<D>(v, H, N, layout, nchunk, part, red);
}

// v_scale = fp32(a / 448); inv = fp32(448 / a) (0 for a == 0), both via fp64.
__device__ inline void v_scale_body(const float* __restrict__ part, int nchunk, int D,
                                    float* __restrict__ v_scale, float* __restrict__ v_inv,
                                    float (*red)[kCombCh]) {
    const int bh = blockIdx.x, c = blockIdx.y * kCombCh + threadIdx.x % kCombCh;
    const int j = threadIdx.x / kCombCh;
    float a = 0.0f;
    for (int ch = j; ch < nchunk; ch += kCombLanes)
        a = fmaxf(a, part[((int64_t)bh * nchunk + ch) * D + c]);
    red[j][threadIdx.x % kCombCh] = a;
    __syncthreads();
    if (j == 0) {
#pragma unroll
        for (int r = 1; r < kCombLanes; ++r) a = fmaxf(a, red[r][threadIdx.x]);
        const int i = bh * D + c;
        v_scale[i] = (float)((double)a / 448.0);
        v_inv[i] = a > 0.0f ? (float)(448.0 / (double)a) : 0.0f;
    }
}

__global__ __launch_bounds__(kQuantThreads) void v_scale_kernel(const float* __restrict__ part,
                                                                int nchunk, int D,
                                                                float* __restrict__ v_scale,
                                                                float* __restrict__ v_inv) {
    __shared__ float red[kCombLanes][kCombCh];
    v_scale_body(part, nchunk, D, v_scale, v_inv, red);
}

// The K and V statistics of one quantization pass in one launch: grid
// (nchunk, B*H, 2), blockIdx.z 0 the K sums, 1 the V absmax.  The two share
// one LDS buffer (a workgroup runs only one of them).
template <int D>
__global__ __launch_bounds__(kQuantThreads) void kv_stats_kernel(
    const u16* __restrict__ k, const u16* __restrict__ v, int H, int N, int layout, int nchunk,
    uint64_t* __restrict__ kpart, float* __restrict__ vpart) {
    constexpr int RPI = kQuantThreads / (D / 8);
    __shared__ uint64_t red[RPI][D];
    if (blockIdx.z == 0)
        k_stats_body<D>(k, H, N, layout, nchunk, kpart, red);
    else
        v_stats_body<D>(v, H, N, layout, nchunk, vpart, reinterpret_cast<float(*)[D]>(&red[0][0]));
}

// k_mean (blockIdx.z 0) and v_scale (1) in one launch: grid (B*H, D/32, 2).
__global__ __launch_bounds__(kQuantThreads) void kv_combine_kernel(
    const uint64_t* __restrict__ kpart, const float* __restrict__ vpart, int nchunk, int D, int N,
    float* __restrict__ kmean, float* __restrict__ v_scale, float* __restrict__ v_inv) {
    __shared__ uint64_t red[kCombLanes][kCombCh];
    if (blockIdx.z == 0)
        k_mean_body(kpart, nchunk, D, N, kmean, red);
    else
        v_scale_body(vpart, nchunk, D, v_scale, v_inv,
                     reinterpret_cast<float(*)[kCombCh]>(&red[0][0]));
}

// trunc(x * 2^30) saturated at +-2^62, NaN -> 0 (the grid of the K mean), for
// an fp32 x: the fp64 product is exact (a power-of-two scaling).
__device__ inline uint64_t fix30_f32(float x) {
    if (x != x) return 0;
    const double t = (double)x * 1073741824.0;
    if (t >= 4611686018427387904.0) return 1ull << 62;
    if (t <= -4611686018427387904.0) return 0ull - (1ull << 62);
    return (uint64_t)(int64_t)t;
}

// One block of 128 rows of Q (blockIdx.z == 0) or of smoothed K (z == 1).
// qmean != NULL: Q is smoothed first by the block's channel means, taken on
// the K mean's exact 2^-30 grid over the block's valid rows; the means go to
// qmean [bh][D][nbp] (channel-major, blocks padded to nbp = 16 ceil(nblk/16)
// with zeros).
template <int D, bool QSM>
__global__ __launch_bounds__(kQuantThreads) void quant_qk_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, int H, int N, int N_pad, int nblk,
    int layout, int qtok, const float* __restrict__ kmean, int8_t* __restrict__ q8,
    float* __restrict__ q_scale, int8_t* __restrict__ k8, float* __restrict__ k_scale,
    float* __restrict__ qmean) {
    constexpr int CPR = D / 8;
    constexpr int RPI = kQuantThreads / CPR;
    constexpr int IT = kBlk / RPI;
    __shared__ float wmax[kQuantThreads / 64];
    __shared__ uint64_t red[QSM ? RPI : 1][D];
    __shared__ float bmean[QSM ? D : 1];
    const int blk = blockIdx.x, bh = blockIdx.y, isk = blockIdx.z;
    const int b = bh / H, h = bh % H;
    const int t = threadIdx.x, cg = t % CPR, tr = t / CPR;
    const int nbp = (nblk + kBiasBlocks - 1) / kBiasBlocks * kBiasBlocks;
    const u16* src = isk ? k : q;
    float mu[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = isk ? kmean[bh * D + cg * 8 + e] : 0.0f;
    float x[IT][8];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int row = blk * kBlk + tr + it * RPI;
        if (row < N) {
            const uint4 w = *(const uint4*)(src + row_offset(layout, b, h, row, H, N, D) + cg * 8);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[it][2 * e] = bf16_bits_to_f32(ws[e] & 0xffffu) - mu[2 * e];
                x[it][2 * e + 1] = bf16_bits_to_f32(ws[e] >> 16) - mu[2 * e + 1];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[it][e] = 0.0f;
        }
    }
    if (QSM && !isk) {
        // block means: exact wrapping int64 sums of trunc(x 2^30) per channel
        // (padded rows hold 0 and add 0), combined over the RPI row lanes
        uint64_t acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0;
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += fix30_f32(x[it][e]);
#pragma unroll
        for (int e = 0; e < 8; ++e) red[tr][cg * 8 + e] = acc[e];
        __syncthreads();
        if (t < D) {
            uint64_t sum = 0;
#pragma unroll 8
            for (int r = 0; r < RPI; ++r) sum += red[r][t];
            const int nrows = min(kBlk, N - blk * kBlk);
            const float m = (float)((double)(int64_t)sum / ((double)nrows * 1073741824.0));
            bmean[t] = m;
            float* col = qmean + ((int64_t)bh * D + t) * nbp;
            col[blk] = m;
            if (blk == nblk - 1)
                for (int r = nblk; r < nbp; ++r) col[r] = 0.0f;
        }
        __syncthreads();
        float qm[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qm[e] = bmean[cg * 8 + e];
#pragma unroll
        for (int it = 0; it < IT; ++it)
            if (blk * kBlk + tr + it * RPI < N)
#pragma unroll
                for (int e = 0; e < 8; ++e) x[it][e] -= qm[e];
    }
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[it][e]));
    if (!isk && qtok) {
        // one scale per query row: the row's CPR lanes are consecutive lanes of
        // one wave, so its absmax is a butterfly over them.  Padded rows get
        // codes 0 and scale 0.
        int8_t* dst = q8;
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int row = blk * kBlk + tr + it * RPI;
            float ra = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ra = fmaxf(ra, fabsf(x[it][e]));
#pragma unroll
            for (int off = 1; off < CPR; off <<= 1) ra = fmaxf(ra, __shfl_xor(ra, off, 64));
            const float rinv = ra > 0.0f ? (float)(127.0 / (double)ra) : 0.0f;
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = __builtin_rintf(x[it][e] * rinv);
                v = fminf(fmaxf(v, -127.0f), 127.0f);
                packed[e >> 2] |= ((uint32_t)(int)v & 0xffu) << (8 * (e & 3));
            }
            *(uint2*)(dst + ((int64_t)bh * N_pad + row) * D + cg * 8) = make_uint2(packed[0], packed[1]);
            if (cg == 0) q_scale[(int64_t)bh * N_pad + row] = (float)((double)ra / 127.0);
        }
        return;
    }
    amax = wave_max(amax);
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    float a = wmax[0];
#pragma unroll
    for (int i = 1; i < kQuantThreads / 64; ++i) a = fmaxf(a, wmax[i]);
    const float inv = a > 0.0f ? (float)(127.0 / (double)a) : 0.0f;
    int8_t* dst = isk ? k8 : q8;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int row = blk * kBlk + tr + it * RPI;
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = __builtin_rintf(x[it][e] * inv);
            v = fminf(fmaxf(v, -127.0f), 127.0f);
            packed[e >> 2] |= ((uint32_t)(int)v & 0xffu) << (8 * (e & 3));
        }
        *(uint2*)(dst + ((int64_t)bh * N_pad + row) * D + cg * 8) = make_uint2(packed[0], packed[1]);
    }
    if (t == 0) (isk ? k_scale : q_scale)[bh * nblk + blk] = (float)((double)a / 127.0);
}

// Q-smoothing correction: bias[bh][r][j] = fp32(acc * lambda) with acc the
// fp32 fma chain over c = 0 .. D-1 (ascending) of qmean[r][c] * k'[j][c],
// k' = fp32(K - kmean).  A thread owns kBiasKeys consecutive keys and
// kBiasBlocks query blocks at a time (64 accumulators), so each mean feeds 4
// fused multiply-adds.  The means of the current 16 blocks (qmean is
// channel-major: [c][16 blocks] is one contiguous 64-byte run per channel)
// are staged in LDS and read as broadcasts, 4 blocks per 16-byte read.  K is
// re-read per group of blocks in chunks of 32 channels (from L2: a workgroup
// covers 1024 keys = 256 KB at d = 128).  Keys j in [N, N_pad) get 0.
template <int D>
__global__ __launch_bounds__(kQuantThreads) void q_bias_kernel(
    const float* __restrict__ qmean, const u16* __restrict__ k, const float* __restrict__ kmean,
    int H, int N, int N_pad, int nblk, int layout, float lambda, float* __restrict__ bias) {
    constexpr int CH = 32;  // channels per chunk
    __shared__ __attribute__((aligned(16))) float qs[D][kBiasBlocks];
    const int j0 = (blockIdx.x * kQuantThreads + threadIdx.x) * kBiasKeys;
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int nbp = (nblk + kBiasBlocks - 1) / kBiasBlocks * kBiasBlocks;
    const int s0 = blockIdx.z * kBiasSlice, s1 = min(nbp, s0 + kBiasSlice);
    const float* km = kmean + bh * D;
    for (int r0 = s0; r0 < s1; r0 += kBiasBlocks) {
        __syncthreads();  // the previous group's reads of qs are done
        for (int i = threadIdx.x; i < D * kBiasBlocks / 4; i += kQuantThreads) {
            const int c = i / (kBiasBlocks / 4), q4 = i % (kBiasBlocks / 4);
            *(float4*)&qs[c][4 * q4] = *(const float4*)(qmean + ((int64_t)bh * D + c) * nbp + r0 + 4 * q4);
        }
        __syncthreads();
        float acc[kBiasBlocks][kBiasKeys];
#pragma unroll
        for (int g = 0; g < kBiasBlocks; ++g)
#pragma unroll
            for (int e = 0; e < kBiasKeys; ++e) acc[g][e] = 0.0f;
        for (int cc = 0; cc < D; cc += CH) {
            float kp[kBiasKeys][CH];
#pragma unroll
            for (int e = 0; e < kBiasKeys; ++e) {
                const int j = j0 + e;
                if (j < N) {
                    const u16* row = k + row_offset(layout, b, h, j, H, N, D) + cc;
#pragma unroll
                    for (int c8 = 0; c8 < CH / 8; ++c8) {
                        const uint4 w = *(const uint4*)(row + 8 * c8);
                        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            kp[e][8 * c8 + 2 * u] = bf16_bits_to_f32(ws[u] & 0xffffu) - km[cc + 8 * c8 + 2 * u];
                            kp[e][8 * c8 + 2 * u + 1] =
                                bf16_bits_to_f32(ws[u] >> 16) - km[cc + 8 * c8 + 2 * u + 1];
                        }
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < CH; ++c) kp[e][c] = 0.0f;
                }
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                float qv[kBiasBlocks];
#pragma unroll
                for (int q4 = 0; q4 < kBiasBlocks / 4; ++q4) {
                    const float4 f = *(const float4*)&qs[cc + c][4 * q4];
                    qv[4 * q4] = f.x;
                    qv[4 * q4 + 1] = f.y;
                    qv[4 * q4 + 2] = f.z;
                    qv[4 * q4 + 3] = f.w;
                }
#pragma unroll
                for (int g = 0; g < kBiasBlocks; ++g)
#pragma unroll
                    for (int e = 0; e < kBiasKeys; ++e)
                        acc[g][e] = __builtin_fmaf(qv[g], kp[e][c], acc[g][e]);
            }
        }
        if (j0 < N_pad)
#pragma unroll
            for (int g = 0; g < kBiasBlocks; ++g)
                if (r0 + g < nblk)
                    *(float4*)(bias + ((int64_t)bh * nblk + r0 + g) * N_pad + j0) =
                        make_float4(acc[g][0] * lambda, acc[g][1] * lambda, acc[g][2] * lambda,
                                    acc[g][3] * lambda);
    }
}

// Position of key r (0..127) of a tile inside the tile's [channel][128] rows.
__device__ __host__ inline int vperm_pos(int r) {
    const int kb = r >> 5, bb = (r >> 3) & 3, g = (r >> 2) & 1, qq = r & 3;
    return 64 * g + 16 * kb + 4 * bb + qq;
}
// First key of the run of 4 keys stored at positions 4w .. 4w+3.
__device__ inline int vperm_key0(int w) {
    const int g = w >> 4, kb = (w >> 2) & 3, bb = w & 3;
    return 32 * kb + 8 * bb + 4 * g;
}

// V -> e4m3 codes of one tile of 128 keys, written as [D][128] (permuted keys).
template <int D>
__global__ __launch_bounds__(kQuantThreads) void quant_v_fp8_kernel(
    const u16* __restrict__ v, int H, int N, int nblk, int layout, const float* __restrict__ v_inv,
    uint8_t* __restrict__ vq) {
    constexpr int CPR = D / 8;
    constexpr int RPI = kQuantThreads / CPR;
    constexpr int IT = kBc / RPI;
    constexpr int LSTR = D + 4;  // bytes per key row in LDS (4-byte pad: conflict-free columns)
    __shared__ __attribute__((aligned(16))) uint8_t tile[kBc * LSTR];
    const int blk = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, cg = t % CPR, tr = t / CPR;
    float inv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) inv[e] = v_inv[bh * D + cg * 8 + e];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int key = tr + it * RPI, row = blk * kBc + key;
        uint32_t w0 = 0u, w1 = 0u;
        if (row < N) {
            const uint4 w = *(const uint4*)(v + row_offset(layout, b, h, row, H, N, D) + cg * 8);
            float x[8];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16_bits_to_f32(ws[e] & 0xffffu) * inv[2 * e];
                x[2 * e + 1] = bf16_bits_to_f32(ws[e] >> 16) * inv[2 * e + 1];
            }
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], w0, false);
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w0, true);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], w1, false);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], w1, true);
        }
        *(uint32_t*)&tile[key * LSTR + cg * 8] = w0;
        *(uint32_t*)&tile[key * LSTR + cg * 8 + 4] = w1;
    }
    __syncthreads();
    uint8_t* dst = vq + ((int64_t)bh * nblk + blk) * D * kBc;
    const int w = t & 31, key0 = vperm_key0(w);
    for (int c4 = t >> 5; c4 < D / 4; c4 += kQuantThreads / 32) {
        uint32_t r[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) r[kk] = *(const uint32_t*)&tile[(key0 + kk) * LSTR + 4 * c4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t o = ((r[0] >> (8 * j)) & 0xffu) | (((r[1] >> (8 * j)) & 0xffu) << 8) |
                               (((r[2] >> (8 * j)) & 0xffu) << 16) |
                               (((r[3] >> (8 * j)) & 0xffu) << 24);
            *(uint32_t*)(dst + (4 * c4 + j) * kBc + 4 * w) = o;
        }
    }
}

// V -> binary16 codes (saturating), same tiled/permuted layout; v_scale = 1.
template <int D>
__global__ __launch_bounds__(kQuantThreads) void quant_v_fp16_kernel(
    const u16* __restrict__ v, int H, int N, int nblk, int layout, u16* __restrict__ vq,
    float* __restrict__ v_scale) {
    constexpr int CPR = D / 8;
    constexpr int RPI = kQuantThreads / CPR;
    constexpr int IT = kBc / RPI;
    constexpr int LSTR = D + 2;  // u16 elements per key row in LDS (4-byte pad)
    __shared__ __attribute__((aligned(16))) u16 tile[kBc * LSTR];
    const int blk = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, cg = t % CPR, tr = t / CPR;
    if (blk == 0 && t < D) v_scale[bh * D + t] = 1.0f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int key = tr + it * RPI, row = blk * kBc + key;
        uint32_t o[4] = {0u, 0u, 0u, 0u};
        if (row < N) {
            const uint4 w = *(const uint4*)(v + row_offset(layout, b, h, row, H, N, D) + cg * 8);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = fminf(fmaxf(bf16_bits_to_f32(ws[e] & 0xffffu), -65504.0f), 65504.0f);
                const float x1 = fminf(fmaxf(bf16_bits_to_f32(ws[e] >> 16), -65504.0f), 65504.0f);
                const u16 h0 = __builtin_bit_cast(u16, (_Float16)x0);
                const u16 h1 = __builtin_bit_cast(u16, (_Float16)x1);
                o[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) *(uint32_t*)&tile[key * LSTR + cg * 8 + 2 * e] = o[e];
    }
    __syncthreads();
    u16* dst = vq + ((int64_t)bh * nblk + blk) * D * kBc;
    const int w = t & 31, key0 = vperm_key0(w);
    for (int c2 = t >> 5; c2 < D / 2; c2 += kQuantThreads / 32) {
        uint32_t r[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) r[kk] = *(const uint32_t*)&tile[(key0 + kk) * LSTR + 2 * c2];
        const uint2 lo = make_uint2((r[0] & 0xffffu) | (r[1] << 16), (r[2] & 0xffffu) | (r[3] << 16));
        const uint2 hi = make_uint2((r[0] >> 16) | (r[1] & 0xffff0000u),
                                    (r[2] >> 16) | (r[3] & 0xffff0000u));
        *(uint2*)(dst + (2 * c2) * kBc + 4 * w) = lo;
        *(uint2*)(dst + (2 * c2 + 1) * kBc + 4 * w) = hi;
    }
}

// ------------------------------------------------------- MXFP6 quantization
// MX blocks of 32 elements in E2M3 (FP6) with one E8M0 scale (OCP
// Microscaling): e = floor(log2(amax)) - 2 (2 = the largest E2M3 exponent);
// a block with amax below 2^-100 (zero included) is all zero codes with
// scale byte 0.  Each block is stored as 32 bytes: the 24 bytes of 32 packed
// E2M3 codes as v_cvt_scalef32_2xpk16_fp6_f32 lays them out (element 2i from
// the first 16 values, 2i + 1 from the second 16), the E8M0 byte at offset
// 24 (the scale operand of the matrix instruction, read with the codes), 7
// zero bytes.

// Codes and scale byte of one block of 32 fp32 values (x[0..15] first,
// x[16..31] second); returns the 8 dwords of the stored block.
__device__ inline v8i mx6_block(const float* x) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    v8i out = v8i{};
    if (!(amax >= 0x1p-100f)) return out;  // zeros, scale byte 0
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 2;
    const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
    v16f a, b;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        a[i] = x[i];
        b[i] = x[16 + i];
    }
    v6i r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, scale);
    // the conversion is multi-pass: keep its sources (scale included) live
    // past it so that the register allocator cannot give the result
    // registers that overlap them.  The result passes through the empty asm,
    // which orders the asm after the conversion.
    asm volatile("" : "+v"(r) : "v"(a), "v"(b), "v"(scale));
#pragma unroll
    for (int i = 0; i < 6; ++i) out[i] = r[i];
    out[6] = e + 127;
    return out;
}

// The same block in E2M1 (FP4), stored as 32 bytes too: byte i (i < 16)
// holds value i of the block in its low nibble and value 16 + i in its high
// nibble (the order the FP6 packing gives the elements, so P and V pair up
// the same way in both formats), the E8M0 byte at offset 24, every other byte
// zero.  v_cvt_scalef32_pk_fp4_f32 converts two values x / scale to E2M1,
// rounded to nearest even and saturated at 6, into one byte of a dword.
__device__ inline v8i mx4_block(const float* x) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    v8i out = v8i{};
    if (!(amax >= 0x1p-100f)) return out;  // zeros, scale byte 0
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 2;
    const float scale = __uint_as_float((uint32_t)(e + 127) << 23);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t d = 0u;
        d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[4 * w], x[16 + 4 * w], scale, 0);
        d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[4 * w + 1], x[17 + 4 * w], scale, 1);
        d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[4 * w + 2], x[18 + 4 * w], scale, 2);
        d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, x[4 * w + 3], x[19 + 4 * w], scale, 3);
        out[w] = (int)d;
    }
    out[6] = e + 127;
    return out;
}

// One MX block of element format FMT (6: E2M3, 4: E2M1).
template <int FMT>
__device__ inline v8i mx_block(const float* x) {
    if constexpr (FMT == 4) return mx4_block(x);
    else return mx6_block(x);
}

// Q (blockIdx.z == 0) or smoothed K (z == 1) to MX (FMT) per row and 32
// channels: one thread per (row, block), rows >= N zero.  Output rows of D
// bytes, [bh][N_pad][D].
template <int D, int FMT>
__global__ __launch_bounds__(kQuantThreads) void quant_qk_mx_kernel(
    const u16* __restrict__ q, const u16* __restrict__ k, int H, int N, int N_pad, int layout,
    const float* __restrict__ kmean, uint8_t* __restrict__ q6, uint8_t* __restrict__ k6) {
    constexpr int NB = D / 32;
    const int idx = blockIdx.x * kQuantThreads + threadIdx.x;
    const int row = idx / NB, blk = idx % NB;
    const int bh = blockIdx.y, b = bh / H, h = bh % H, isk = blockIdx.z;
    if (row >= N_pad) return;
    v8i out = v8i{};
    if (row < N) {
        const u16* src = (isk ? k : q) + row_offset(layout, b, h, row, H, N, D) + 32 * blk;
        float x[32];
#pragma unroll
        for (int c8 = 0; c8 < 4; ++c8) {
            const uint4 w = *(const uint4*)(src + 8 * c8);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[8 * c8 + 2 * u] = bf16_bits_to_f32(ws[u] & 0xffffu);
                x[8 * c8 + 2 * u + 1] = bf16_bits_to_f32(ws[u] >> 16);
            }
        }
        if (isk) {
            const float* km = kmean + bh * D + 32 * blk;
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] -= km[i];
        }
        out = mx_block<FMT>(x);
    }
    uint8_t* dst = (isk ? k6 : q6) + ((int64_t)bh * N_pad + row) * D + 32 * blk;
    *(uint4*)dst = make_uint4(out[0], out[1], out[2], out[3]);
    *(uint4*)(dst + 16) = make_uint4(out[4], out[5], out[6], out[7]);
}

// V to MX (FMT) per channel and 32 keys, one tile of 128 keys per workgroup:
// the tile is staged in LDS channel-major (fp32), then one thread per
// (channel, block of 32 keys) packs its block.  Output [bh][nblk][D][128]
// bytes: channel row = the tile's 4 key blocks of 32 bytes; keys >= N are 0.
template <int D, int FMT>
__global__ __launch_bounds__(kQuantThreads) void quant_v_mx_kernel(
    const u16* __restrict__ v, int H, int N, int nblk, int layout, uint8_t* __restrict__ v6) {
    constexpr int CPR = D / 8;
    constexpr int RPI = kQuantThreads / CPR;
    constexpr int LSTR = kBc + 4;  // floats per channel row in LDS (pad: fewer bank conflicts)
    __shared__ float tile[D * LSTR];
    const int blk = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, cg = t % CPR, tr = t / CPR;
    for (int key = tr; key < kBc; key += RPI) {
        const int row = blk * kBc + key;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        if (row < N) {
            const uint4 w = *(const uint4*)(v + row_offset(layout, b, h, row, H, N, D) + cg * 8);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16_bits_to_f32(ws[e] & 0xffffu);
                x[2 * e + 1] = bf16_bits_to_f32(ws[e] >> 16);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[(cg * 8 + e) * LSTR + key] = x[e];
    }
    __syncthreads();
    uint8_t* dst = v6 + ((int64_t)bh * nblk + blk) * D * kBc;
    for (int i = t; i < D * 4; i += kQuantThreads) {
        const int c = i >> 2, kb = i & 3;
        float x[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) x[j] = tile[c * LSTR + 32 * kb + j];
        const v8i out = mx_block<FMT>(x);
        uint8_t* o = dst + c * kBc + 32 * kb;
        *(uint4*)o = make_uint4(out[0], out[1], out[2], out[3]);
        *(uint4*)(o + 16) = make_uint4(out[4], out[5], out[6], out[7]);
    }
}

// ------------------------------------------------------------------ launchers
static inline hipError_t launch(const void* fn, dim3 grid, dim3 block, void** args,
                                hipStream_t s) {
    return hipLaunchKernel(fn, grid, block, args, 0, s);
}

// INT8 codes and scales of Q and smoothed K, once k_mean is in place.
static hipError_t launch_qk_codes(const u16* q, const u16* k, int B, int H, int N, int d,
                                  int layout, int qtok, int8_t* q8, float* qs, int8_t* k8,
                                  float* ks, const float* kmean, float* qmean, hipStream_t s) {
    int nblk = (N + kBlk - 1) / kBlk, N_pad = nblk * kBlk;
    void* args[] = {(void*)&q,      (void*)&k,    (void*)&H,     (void*)&N,
                    (void*)&N_pad,  (void*)&nblk, (void*)&layout, (void*)&qtok,
                    (void*)&kmean,  (void*)&q8,   (void*)&qs,     (void*)&k8,
                    (void*)&ks,     (void*)&qmean};
    const void* fn = qmean ? (d == 128 ? (const void*)quant_qk_kernel<128, true>
                                       : (const void*)quant_qk_kernel<64, true>)
                           : (d == 128 ? (const void*)quant_qk_kernel<128, false>
                                       : (const void*)quant_qk_kernel<64, false>);
    return launch(fn, dim3(nblk, B * H, 2), dim3(kQuantThreads), args, s);
}

// FP8 (or FP16) codes of V, once v_inv is in place (FP8 only).
static hipError_t launch_v_codes(const u16* v, int B, int H, int N, int d, int layout, int pv16,
                                 const float* vinv, void* vq, float* vscale, hipStream_t s) {
    int nblk = (N + kBc - 1) / kBc;
    if (pv16) {
        void* args[] = {(void*)&v, (void*)&H, (void*)&N, (void*)&nblk, (void*)&layout, (void*)&vq,
                        (void*)&vscale};
        const void* fn = d == 128 ? (const void*)quant_v_fp16_kernel<128>
                                  : (const void*)quant_v_fp16_kernel<64>;
        return launch(fn, dim3(nblk, B * H), dim3(kQuantThreads), args, s);
    }
    void* args[] = {(void*)&v, (void*)&H, (void*)&N, (void*)&nblk, (void*)&layout, (void*)&vinv,
                    (void*)&vq};
    const void* fn = d == 128 ? (const void*)quant_v_fp8_kernel<128>
                              : (const void*)quant_v_fp8_kernel<64>;
    return launch(fn, dim3(nblk, B * H), dim3(kQuantThreads), args, s);
}

hipError_t launch_quant_qk(const u16* q, const u16* k, int B, int H, int N, int d, int layout,
                           int qtok, int8_t* q8, float* qs, int8_t* k8, float* ks, float* kmean,
                           float* qmean, uint64_t* ws, hipStream_t s) {
    const int nblk = (N + kBlk - 1) / kBlk, N_pad = nblk * kBlk;
    const int nchunk = (N + kStatsChunk - 1) / kStatsChunk;
    const int BH = B * H;
    hipError_t e;
    {
        void* args[] = {(void*)&k, (void*)&H, (void*)&N, (void*)&layout, (void*)&nchunk, (void*)&ws};
        const void* fn = d == 128 ? (const void*)k_stats_kernel<128> : (const void*)k_stats_kernel<64>;
        if ((e = launch(fn, dim3(nchunk, BH), dim3(kQuantThreads), args, s)) != hipSuccess) return e;
    }
    {
        void* args[] = {(void*)&ws, (void*)&nchunk, (void*)&d, (void*)&N, (void*)&kmean};
        if ((e = launch((const void*)k_mean_kernel, dim3(BH, d / kCombCh), dim3(kQuantThreads), args,
                        s)) != hipSuccess)
            return e;
    }
    return launch_qk_codes(q, k, B, H, N, d, layout, qtok, q8, qs, k8, ks, kmean, qmean, s);
}

hipError_t launch_q_bias(const float* qmean, const u16* k, const float* kmean, int B, int H, int N,
                         int d, int layout, float lambda, float* bias, hipStream_t s) {
    const int nblk = (N + kBlk - 1) / kBlk, N_pad = nblk * kBlk;
    void* args[] = {(void*)&qmean, (void*)&k,     (void*)&kmean,  (void*)&H,      (void*)&N,
                    (void*)&N_pad, (void*)&nblk, (void*)&layout, (void*)&lambda, (void*)&bias};
    const void* fn = d == 128 ? (const void*)q_bias_kernel<128> : (const void*)q_bias_kernel<64>;
    const int nbp = (nblk + kBiasBlocks - 1) / kBiasBlocks * kBiasBlocks;
    const dim3 grid((N_pad + kQuantThreads * kBiasKeys - 1) / (kQuantThreads * kBiasKeys), B * H,
                    (nbp + kBiasSlice - 1) / kBiasSlice);
    return launch(fn, grid, dim3(kQuantThreads), args, s);
}

hipError_t launch_quant_qk_mx(const u16* q, const u16* k, int B, int H, int N, int d, int layout,
                              int fmt, uint8_t* q6, uint8_t* k6, float* kmean, uint64_t* ws,
                              hipStream_t s) {
    const int nblk = (N + kBlk - 1) / kBlk, N_pad = nblk * kBlk;
    const int nchunk = (N + kStatsChunk - 1) / kStatsChunk;
    const int BH = B * H;
    hipError_t e;
    {
        void* args[] = {(void*)&k, (void*)&H, (void*)&N, (void*)&layout, (void*)&nchunk, (void*)&ws};
        const void* fn = d == 128 ? (const void*)k_stats_kernel<128> : (const void*)k_stats_kernel<64>;
        if ((e = launch(fn, dim3(nchunk, BH), dim3(kQuantThreads), args, s)) != hipSuccess) return e;
    }
    {
        void* args[] = {(void*)&ws, (void*)&nchunk, (void*)&d, (void*)&N, (void*)&kmean};
        if ((e = launch((const void*)k_mean_kernel, dim3(BH, d / kCombCh), dim3(kQuantThreads), args,
                        s)) != hipSuccess)
            return e;
    }
    void* args[] = {(void*)&q, (void*)&k, (void*)&H, (void*)&N, (void*)&N_pad, (void*)&layout,
                    (void*)&kmean, (void*)&q6, (void*)&k6};
    const void* fn = fmt == 4 ? (d == 128 ? (const void*)quant_qk_mx_kernel<128, 4>
                                          : (const void*)quant_qk_mx_kernel<64, 4>)
                              : (d == 128 ? (const void*)quant_qk_mx_kernel<128, 6>
                                          : (const void*)quant_qk_mx_kernel<64, 6>);
    const int items = N_pad * (d / 32);
    return launch(fn, dim3((items + kQuantThreads - 1) / kQuantThreads, BH, 2), dim3(kQuantThreads),
                  args, s);
}

hipError_t launch_quant_v_mx(const u16* v, int B, int H, int N, int d, int layout, int fmt,
                             uint8_t* v6, hipStream_t s) {
    const int nblk = (N + kBc - 1) / kBc;
    void* args[] = {(void*)&v, (void*)&H, (void*)&N, (void*)&nblk, (void*)&layout, (void*)&v6};
    const void* fn = fmt == 4 ? (d == 128 ? (const void*)quant_v_mx_kernel<128, 4>
                                          : (const void*)quant_v_mx_kernel<64, 4>)
                              : (d == 128 ? (const void*)quant_v_mx_kernel<128, 6>
                                          : (const void*)quant_v_mx_kernel<64, 6>);
    return launch(fn, dim3(nblk, B * H), dim3(kQuantThreads), args, s);
}

hipError_t launch_quant_v(const u16* v, int B, int H, int N, int d, int layout, int pv16,
                          void* vq, float* vscale, float* ws, hipStream_t s) {
    const int nblk = (N + kBc - 1) / kBc;
    const int nchunk = (N + kStatsChunk - 1) / kStatsChunk;
    const int BH = B * H;
    hipError_t e;
    if (pv16) return launch_v_codes(v, B, H, N, d, layout, 1, nullptr, vq, vscale, s);
    float* part = ws;
    float* vinv = ws + (size_t)BH * nchunk * d;
    {
        void* args[] = {(void*)&v, (void*)&H, (void*)&N, (void*)&layout, (void*)&nchunk, (void*)&part};
        const void* fn = d == 128 ? (const void*)v_stats_kernel<128> : (const void*)v_stats_kernel<64>;
        if ((e = launch(fn, dim3(nchunk, BH), dim3(kQuantThreads), args, s)) != hipSuccess) return e;
    }
    {
        void* args[] = {(void*)&part, (void*)&nchunk, (void*)&d, (void*)&vscale, (void*)&vinv};
        if ((e = launch((const void*)v_scale_kernel, dim3(BH, d / kCombCh), dim3(kQuantThreads), args,
                        s)) != hipSuccess)
            return e;
    }
    return launch_v_codes(v, B, H, N, d, layout, 0, vinv, vq, vscale, s);
}

// One quantization pass over Q, K and V: the K and V statistics in one launch
// and their combinations in one more (FP8 V; FP16 V needs no statistics),
// then the Q/K and V codes.  kws: B*H*nchunk*d uint64 K partials; vws:
// B*H*nchunk*d float V partials followed by B*H*d floats of v_inv (FP8 only).
hipError_t launch_quant_qkv(const u16* q, const u16* k, const u16* v, int B, int H, int N, int d,
                            int layout, int pv16, int8_t* q8, float* qs, int8_t* k8, float* ks,
                            float* kmean, void* vq, float* vscale, uint64_t* kws, float* vws,
                            hipStream_t s) {
    int nchunk = (N + kStatsChunk - 1) / kStatsChunk;
    const int BH = B * H;
    float* vinv = vws + (size_t)BH * nchunk * d;
    hipError_t e;
    {
        void* args[] = {(void*)&k,      (void*)&v,      (void*)&H,   (void*)&N,
                        (void*)&layout, (void*)&nchunk, (void*)&kws, (void*)&vws};
        const void* fn = d == 128 ? (const void*)kv_stats_kernel<128> : (const void*)kv_stats_kernel<64>;
        if ((e = launch(fn, dim3(nchunk, BH, pv16 ? 1 : 2), dim3(kQuantThreads), args, s)) !=
            hipSuccess)
            return e;
    }
    {
        void* args[] = {(void*)&kws, (void*)&vws,    (void*)&nchunk, (void*)&d,
                        (void*)&N,   (void*)&kmean, (void*)&vscale, (void*)&vinv};
        if ((e = launch((const void*)kv_combine_kernel, dim3(BH, d / kCombCh, pv16 ? 1 : 2),
                        dim3(kQuantThreads), args, s)) != hipSuccess)
            return e;
    }
    if ((e = launch_qk_codes(q, k, B, H, N, d, layout, 0, q8, qs, k8, ks, kmean, nullptr, s)) !=
        hipSuccess)
        return e;
    return launch_v_codes(v, B, H, N, d, layout, pv16, vinv, vq, vscale, s);
}

// Fixed device scratch of the allocation-free quantization pass
// (sage_quant_qkv_noalloc): the K and V partial statistics of one call, laid
// out as the workspace of sage_quant_qkv.  Each GPU holds its own copy for
// the life of the process; every call on a GPU reuses it, so calls that
// overlap on one GPU (other streams or threads) race.  Nothing in it needs
// clearing: each call writes every partial before reading it.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_at[kMaxDevices];  // device address of `scratch` per device, once looked up
}  // namespace

// The device address of `scratch` on the stream's device, which must be the
// current device (the symbol is looked up with that device current, once per
// device).  hipErrorInvalidDevice if the stream belongs to another device.
hipError_t noalloc_scratch(hipStream_t s, void** out) {
    int dev = -1, sdev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if ((e = hipStreamGetDevice(s, &sdev)) != hipSuccess) return e;
    if (sdev != dev || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_at[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_at[dev] = p;
    }
    *out = scratch_at[dev];
    return hipSuccess;
}

}  // namespace sage
