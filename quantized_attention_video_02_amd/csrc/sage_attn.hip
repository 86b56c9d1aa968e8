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

// Value of lane ^ 32 combined with this lane's (v_permlane32_swap: the two
// halves of the wave exchange registers; both results hold one value from
// each half, so max/sum of the pair is the same on both lanes).
__device__ inline int pair_max(int x) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return max((int)r[0], (int)r[1]);
}
__device__ inline float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key index held by lane half hh in register r of 32-key block k4 of a tile
// (the 32x32 MFMA accumulator layout: row 8*(r/4) + 4*hh + r%4).
__device__ inline int tile_key(int key_t, int k4, int r, int hh) {
    return key_t + 32 * k4 + 8 * (r >> 2) + 4 * hh + (r & 3);
}

// S^T (128 keys x 32 queries) = K8 tile (LDS, rows of KSTR bytes) . Q8^T.
template <int D, int KSTR>
__device__ inline void qk_tile(const uint8_t* kb, const v4i* qf, v16i* S, int n, int hh) {
    constexpr int KK = D / 32;
    const uint8_t* krow = kb + n * KSTR + 16 * hh;
    v4i a[2][KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) a[0][kk] = *(const v4i*)(krow + 32 * kk);
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
        if (k4 + 1 < 4) {
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                a[(k4 + 1) & 1][kk] = *(const v4i*)(krow + 32 * (k4 + 1) * KSTR + 32 * kk);
        }
        v16i acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[k4 & 1][0], qf[0], v16i{}, 0, 0, 0);
#pragma unroll
        for (int kk = 1; kk < KK; ++kk)
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[k4 & 1][kk], qf[kk], acc, 0, 0, 0);
        S[k4] = acc;
    }
}

__device__ inline void dump_tile(const v16i* S, int32_t* srow, int key_t, int N, bool causal,
                                 int qi, int hh) {
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = tile_key(key_t, k4, r, hh);
            if (key < N && (!causal || key <= qi)) srow[key] = S[k4][r];
        }
}

// Online-softmax step of one tile for this lane's query.  In: S (int32), the
// dequantization constant c, the running max m.  Out: P (the PV B operand),
// alpha, the partial row sum ls of this lane's 64 keys; m is updated.
// p = exp2(fma(S, c, -(m' - log2 448))).  MASK: keys >= N (and, causal,
// keys > qi) get p = 0 and do not enter the max.
template <bool MASK, typename PT>
__device__ inline void softmax_tile(v16i* S, PT* P, float c, float& m, float& alpha, float& ls,
                                    int key_t, int N, bool causal, int qi, int hh) {
    if (MASK) {
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = tile_key(key_t, k4, r, hh);
                if (key >= N || (causal && key > qi)) S[k4][r] = INT_MIN;
            }
    }
    int mk[4];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
        int x = max(S[k4][0], S[k4][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) x = max(x, max(S[k4][r], S[k4][r + 1]));
        mk[k4] = x;
    }
    const int mx = pair_max(max(max(mk[0], mk[1]), max(mk[2], mk[3])));
    const float mt = (MASK && mx == INT_MIN) ? -INFINITY : (float)mx * c;
    const float mn = fmaxf(m, mt);
    alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    const float mu = mn - kLog2PScale;
    float part[4];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
        float sum = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = S[k4][4 * u + j];
                p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s, c, -mu));
                if (MASK && s == INT_MIN) p[j] = 0.0f;
            }
            sum += (p[0] + p[1]) + (p[2] + p[3]);
            if constexpr (sizeof(PT) == 32 && __is_same(PT, v8i)) {
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __builtin_nondeterministic_value(0),
                                                        false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
                P[k4 >> 1][(k4 & 1) * 4 + u] = w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) P[2 * k4 + (u >> 1)][4 * (u & 1) + j] = (_Float16)p[j];
            }
        }
        part[k4] = sum;
    }
    ls = (part[0] + part[1]) + (part[2] + part[3]);
}

// Level 1: T = V^T tile (LDS) . P^T, a fresh fp32 accumulator per output
// block; level 2: O = alpha O + T.
template <int D, int VSTR>
__device__ inline void pv_tile_fp8(const uint8_t* vb, const v8i* P, v16f* O, float alpha, int n,
                                   int hh) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
        const uint8_t* vrow = vb + (32 * cb + n) * VSTR + 64 * hh;
        const v8i a0 = *(const v8i*)(vrow);
        const v8i a1 = *(const v8i*)(vrow + 32);
        v16f T = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, P[0], v16f{}, 0, 0, 0, 0, 0, 0);
        T = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, P[1], T, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) O[cb][e] = __builtin_fmaf(alpha, O[cb][e], T[e]);
    }
}

template <int D, int VSTR>
__device__ inline void pv_tile_fp16(const uint8_t* vb, const v8h* P, v16f* O, float alpha, int n,
                                    int hh) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
        const uint8_t* vrow = vb + (32 * cb + n) * VSTR + 2 * 64 * hh;
        v16f T = v16f{};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const v8h av = *(const v8h*)(vrow + 16 * u);
            T = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, P[u], T, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) O[cb][e] = __builtin_fmaf(alpha, O[cb][e], T[e]);
    }
}

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
            v16i S[4];
            qk_tile<D, SM::KSTR>(kb, qf, S, n, hh);
            const int key_t = t * kBc;
            if (DUMP && bh == a.dbh && qi >= a.drow0 && qi < a.drow0 + a.dnrows)
                dump_tile(S, a.s_out + (int64_t)(qi - a.drow0) * N, key_t, N, CAUSAL, qi, hh);
            const float c = sigma * a.k_scale[bh * a.nblk + t];
            const bool needmask = (tail && t == a.nblk - 1) || (CAUSAL && key_t + kBc - 1 > qbase);
            float alpha, ls;
            if constexpr (!PV16) {
                v8i P[2];
                if (needmask) softmax_tile<true>(S, P, c, m, alpha, ls, key_t, N, CAUSAL, qi, hh);
                else softmax_tile<false>(S, P, c, m, alpha, ls, key_t, N, CAUSAL, qi, hh);
                pv_tile_fp8<D, SM::VSTR>(vb, P, O, alpha, n, hh);
            } else {
                v8h P[8];
                if (needmask) softmax_tile<true>(S, P, c, m, alpha, ls, key_t, N, CAUSAL, qi, hh);
                else softmax_tile<false>(S, P, c, m, alpha, ls, key_t, N, CAUSAL, qi, hh);
                pv_tile_fp16<D, SM::VSTR>(vb, P, O, alpha, n, hh);
            }
            l = alpha * l + ls;
        }
        if (t + 1 < ntiles) swrite((t + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: out = O * v_scale / l (l summed over both lane halves)
    const float lt = pair_sum(l);
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
