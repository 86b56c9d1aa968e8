// Fused low-bit attention forward of libsage for gfx950 (CDNA4).
//
// Method (wxsanhe.com TurboDiffusion post, section 三.1; reportify.cn
// SageAttention3 summary, bullet 8比特训练; hunxia.com glossary entry on
// FlashAttention): INT8 Q K^T into int32, dequantize by q_scale * k_scale,
// exp2 online softmax in FP32 over key tiles of 128, P to FP8 e4m3 with the
// static scale 448 (FP16 path: binary16), P V on FP8 (FP16) matrix cores into
// a fresh FP32 sum per key tile, added into the FP32 running output.
//
// Work decomposition: one workgroup = 8 wave64s = 256 queries of one (b, h);
// each wave owns 32 queries for the whole key sweep.  Per key tile:
//   S^T (128 keys x 32 queries) = K8 tile (LDS) . Q8^T (registers),
//     16 x v_mfma_i32_32x32x32_i8 (d = 128);
//   in the 32x32 accumulator layout each lane holds one query (lane & 31) and
//   64 of the tile's keys, so the row max / row sum stay in the lane plus one
//   exchange with lane ^ 32, and the P values a lane produces are exactly the
//   B operand of the P V product;
//   O^T (d x 32 queries) += V^T tile (LDS) . P^T (registers),
//     8 x v_mfma_f32_32x32x64_f8f6f4 (d = 128) -- O^T keeps queries on lanes,
//     so the per-query rescale alpha is a per-lane scalar.
// K and V tiles are staged global -> registers -> LDS, double-buffered: the
// loads of tile t+1 are in flight while tile t is computed; one barrier per
// tile.  LDS rows carry a 16-byte pad so the 16-byte operand reads of 8
// consecutive lanes (8 different rows) hit distinct banks.
// The grid is remapped so that consecutive workgroups of one head run on the
// same XCD (hardware dispatches workgroups round-robin over the 8 XCDs), so a
// head's K/V tiles are shared through that XCD's L2.
#include <limits.h>

#include "sage_common.h"

namespace sage {


__device__ inline int xcd_remap(int bid, int total) {
    constexpr int nx = 8;
    const int q = total / nx, r = total % nx, x = bid % nx, s = bid / nx;
    return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

template <int D, bool PV16>
struct AttnSmem {
    static constexpr int KSTR = D + 16;                      // bytes per key row
    static constexpr int VES = PV16 ? 2 : 1;
    static constexpr int VSTR = kBc * VES + 16;              // bytes per channel row
    static constexpr int KBYTES = kBc * KSTR;
    static constexpr int VBYTES = D * VSTR;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int TOTAL = 2 * STAGE;
    static constexpr int KCH = kBc * D / 16 / kAttnThreads;       // 16-B K chunks per thread
    static constexpr int VCH = D * kBc * VES / 16 / kAttnThreads; // 16-B V chunks per thread
    static constexpr int KCPR = D / 16;
    static constexpr int VCPR = kBc * VES / 16;
};

template <int D, bool PV16, bool CAUSAL, bool DUMP>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_fwd_kernel(AttnArgs a) {
    using SM = AttnSmem<D, PV16>;
    constexpr int KK = D / 32;  // 32-channel steps of the Q K^T product
    constexpr int CB = D / 32;  // 32-channel blocks of the output
    __shared__ __attribute__((aligned(16))) uint8_t smem[SM::TOTAL];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, a.total);
    const int bh = wg / a.nqt;
    int qt = wg - bh * a.nqt;
    if (CAUSAL) qt = a.nqt - 1 - qt;  // longest rows first
    const int H = a.H, N = a.N;
    const int b = bh / H, h = bh - b * H;
    const int qbase = qt * kBr + wave * 32;
    const bool active = qbase < N;
    const int qi = qbase + n;

    int ntiles = a.nblk;
    if (CAUSAL) ntiles = (min(N, qt * kBr + kBr) - 1) / kBc + 1;
    const int wave_tiles = CAUSAL ? (min(N, qbase + 32) - 1) / kBc + 1 : ntiles;
    const bool tail = (N % kBc) != 0;

    // Q8^T operand: lane (query n, half hh) holds channels [32 kk + 16 hh, +16).
    v4i qf[KK];
    float sigma = 0.0f;
    if (active) {
        const int8_t* qrow = a.q8 + ((int64_t)bh * a.N_pad + qi) * D + 16 * hh;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const v4i*)(qrow + 32 * kk);
        sigma = a.q_scale[bh * a.nblk + qbase / kBlk] * a.lambda;
    }

    const v4i* kg = (const v4i*)(a.k8 + (int64_t)bh * a.N_pad * D);
    const v4i* vg = (const v4i*)((const uint8_t*)a.vq + (int64_t)bh * a.nblk * D * kBc * SM::VES);
    v4i kst[SM::KCH], vst[SM::VCH];
    auto gload = [&](int t) {
        const v4i* kt = kg + (int64_t)t * (kBc * D / 16);
        const v4i* vt = vg + (int64_t)t * (D * kBc * SM::VES / 16);
#pragma unroll
        for (int i = 0; i < SM::KCH; ++i) kst[i] = kt[tid + kAttnThreads * i];
#pragma unroll
        for (int i = 0; i < SM::VCH; ++i) vst[i] = vt[tid + kAttnThreads * i];
    };
    auto swrite = [&](int buf) {
        uint8_t* kb = smem + buf * SM::STAGE;
        uint8_t* vb = kb + SM::KBYTES;
#pragma unroll
        for (int i = 0; i < SM::KCH; ++i) {
            const int ci = tid + kAttnThreads * i;
            *(v4i*)(kb + (ci / SM::KCPR) * SM::KSTR + (ci % SM::KCPR) * 16) = kst[i];
        }
#pragma unroll
        for (int i = 0; i < SM::VCH; ++i) {
            const int ci = tid + kAttnThreads * i;
            *(v4i*)(vb + (ci / SM::VCPR) * SM::VSTR + (ci % SM::VCPR) * 16) = vst[i];
        }
    };

    float m = -INFINITY, l = 0.0f;
    v16f O[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) O[cb][e] = 0.0f;

    gload(0);
    swrite(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) gload(t + 1);
        if (active && t < wave_tiles) {
            const uint8_t* kb = smem + (t & 1) * SM::STAGE;
            const uint8_t* vb = kb + SM::KBYTES;
            // ---- S^T = K8 . Q8^T (exact int32)
            v16i S[4];
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
#pragma unroll
                for (int e = 0; e < 16; ++e) S[k4][e] = 0;
                const uint8_t* krow = kb + (32 * k4 + n) * SM::KSTR + 16 * hh;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const v4i av = *(const v4i*)(krow + 32 * kk);
                    S[k4] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, qf[kk], S[k4], 0, 0, 0);
                }
            }
            const int key_t = t * kBc;
            if (DUMP && bh == a.dbh && qi >= a.drow0 && qi < a.drow0 + a.dnrows) {
                int32_t* srow = a.s_out + (int64_t)(qi - a.drow0) * N;
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key_t + 32 * k4 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (key < N && (!CAUSAL || key <= qi)) srow[key] = S[k4][r];
                    }
            }
            const bool needmask = (tail && t == a.nblk - 1) || (CAUSAL && key_t + kBc - 1 > qbase);
            if (needmask) {
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key_t + 32 * k4 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        if (key >= N || (CAUSAL && key > qi)) S[k4][r] = INT_MIN;
                    }
            }
            // ---- tile max on the integers (c > 0 keeps the order)
            int mx = INT_MIN;
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = max(mx, S[k4][r]);
            mx = max(mx, __shfl_xor(mx, 32, 64));
            const float c = sigma * a.k_scale[bh * a.nblk + t];
            const float mt = (mx == INT_MIN) ? -INFINITY : (float)mx * c;
            const float mn = fmaxf(m, mt);
            const float alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
            const float mu = mn - kLog2PScale;
            // ---- p = exp2(S c - (m' - log2 448)), row sum, P -> FP8 / FP16
            float ls = 0.0f;
            if constexpr (!PV16) {
                v8i P[2];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        float p[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int s = S[k4][4 * u + j];
                            p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s, c, -mu));
                            if (needmask && s == INT_MIN) p[j] = 0.0f;
                            ls += p[j];
                        }
                        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
                        P[k4 >> 1][(k4 & 1) * 4 + u] = w;
                    }
                // ---- level 1: T = V^T . P^T (fresh fp32); level 2: O = alpha O + T
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    v16f T;
#pragma unroll
                    for (int e = 0; e < 16; ++e) T[e] = 0.0f;
                    const uint8_t* vrow = vb + (32 * cb + n) * SM::VSTR + 64 * hh;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const v8i av = *(const v8i*)(vrow + 32 * hf);
                        T = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, P[hf], T, 0, 0, 0, 0,
                                                                            0, 0);
                    }
#pragma unroll
                    for (int e = 0; e < 16; ++e) O[cb][e] = __builtin_fmaf(alpha, O[cb][e], T[e]);
                }
            } else {
                v8h P[8];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int s = S[k4][r];
                        float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s, c, -mu));
                        if (needmask && s == INT_MIN) p = 0.0f;
                        ls += p;
                        P[2 * k4 + (r >> 3)][r & 7] = (_Float16)p;
                    }
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    v16f T;
#pragma unroll
                    for (int e = 0; e < 16; ++e) T[e] = 0.0f;
                    const uint8_t* vrow = vb + (32 * cb + n) * SM::VSTR + 2 * 64 * hh;
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const v8h av = *(const v8h*)(vrow + 16 * u);
                        T = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, P[u], T, 0, 0, 0);
                    }
#pragma unroll
                    for (int e = 0; e < 16; ++e) O[cb][e] = __builtin_fmaf(alpha, O[cb][e], T[e]);
                }
            }
            l = alpha * l + ls;
            m = mn;
        }
        if (t + 1 < ntiles) swrite((t + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: out = O * v_scale / l (l summed over both lane halves)
    const float lt = l + __shfl_xor(l, 32, 64);
    if (!active || qi >= N) return;
    const int64_t obase = row_offset(a.layout, b, h, qi, H, N, D);
    const float* vs = a.v_scale + bh * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int c0 = 32 * cb + 8 * r4 + 4 * hh;
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = (O[cb][4 * r4 + j] * vs[c0 + j]) / lt;
            if (a.out_fp32) {
                *(float4*)((float*)a.out + obase + c0) = make_float4(o[0], o[1], o[2], o[3]);
            } else {
                const uint32_t w0 = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
                const uint32_t w1 = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
                *(uint2*)((u16*)a.out + obase + c0) = make_uint2(w0, w1);
            }
        }
}

template <int D, bool PV16, bool CAUSAL, bool DUMP>
static const void* attn_fn() {
    return (const void*)attn_fwd_kernel<D, PV16, CAUSAL, DUMP>;
}

template <int D, bool PV16>
static const void* attn_fn_rt(bool causal, bool dump) {
    if (causal) return dump ? attn_fn<D, PV16, true, true>() : attn_fn<D, PV16, true, false>();
    return dump ? attn_fn<D, PV16, false, true>() : attn_fn<D, PV16, false, false>();
}

hipError_t launch_attn(const AttnArgs& args, int B, int d, int pv16, int causal, int dump,
                       hipStream_t s) {
    const void* fn;
    if (d == 128) fn = pv16 ? attn_fn_rt<128, true>(causal, dump) : attn_fn_rt<128, false>(causal, dump);
    else fn = pv16 ? attn_fn_rt<64, true>(causal, dump) : attn_fn_rt<64, false>(causal, dump);
    AttnArgs a = args;
    void* kargs[] = {(void*)&a};
    return hipLaunchKernel(fn, dim3(a.total), dim3(kAttnThreads), kargs, 0, s);
}

}  // namespace sage
