// Fused low-bit attention forward of libsage for gfx950 (CDNA4).
//
// Method (wxsanhe.com TurboDiffusion post, section 三.1; reportify.cn
// SageAttention3 summary, bullet 8比特训练; hunxia.com glossary entry on
// FlashAttention): INT8 Q K^T into int32, dequantize by q_scale * k_scale,
// exp2 online softmax in FP32 over key tiles of 128, P to FP8 e4m3 with the
// static scale 448 (FP16 path: binary16), P V on FP8 (FP16) matrix cores with
// FP32 accumulation into the running output.  The pages accumulate each tile's
// P V in a fresh FP32 sum and add it to the output (two levels) because the
// FP8 tensor cores they target keep fewer accumulator bits; the gfx950 MFMA
// accumulates in full FP32, so the product is accumulated straight into the
// rescaled output (O = alpha O + P V, one rounding per MFMA step).
//
// Work decomposition: one workgroup = 8 wave64s = 256 queries of one (b, h)
// (4 waves = one 128-query block for the block-sparse sweep; 12 waves for the
// non-pipelined d = 64 sweep); each wave owns 32 queries for the whole key
// sweep.  Per key tile:
//   S^T (128 keys x 32 queries) = K8 tile (LDS) . Q8^T (registers),
//     16 x v_mfma_i32_32x32x32_i8 (d = 128);
//   in the 32x32 accumulator layout each lane holds one query (lane & 31) and
//   64 of the tile's keys, so the row max / row sum stay in the lane plus one
//   exchange with lane ^ 32 (v_permlane32_swap), and the P values a lane
//   produces are exactly the B operand of the P V product;
//   O^T (d x 32 queries) += V^T tile (LDS) . P^T (registers),
//     8 x v_mfma_f32_32x32x64_f8f6f4 (d = 128) -- O^T keeps queries on lanes,
//     so the per-query rescale alpha is a per-lane scalar.
// Schedule: a per-wave software pipeline with one workgroup barrier per tile.
// Iteration t runs A = P V of tile t-1 (MFMA) with the max / alpha / float(S)
// and exponent arguments of tile t (VALU), then B = the Q K^T of tile t+1
// (MFMA) with the exp2 / FP8 packing of tile t (VALU).  Each phase is written
// as chunks of one MFMA (its LDS operand read one chunk ahead) followed by a
// share of the phase's vector work, kept in that order by scheduling barriers,
// so the vector instructions issue in the MFMAs' shadow.  The row sum of the
// FP8 P is two more MFMAs (a 0/1 pattern times P).  The second wave of each
// SIMD passes each step's barrier between its A and B, so the two waves of a
// SIMD run opposite phases.  Per wave and tile: 26 MFMAs and about 300
// vector instructions (65 of them v_exp_f32); the vector issue of one wave and
// the arbitration of the two waves for the matrix core bound the kernel.
// K and V tiles go straight from global memory into LDS (global_load_lds_dwordx4
// issued from asm, no register staging), double-buffered: K(t+2) and V(t) are
// loaded during iteration t and awaited before its closing barrier.  LDS rows
// carry a 16-byte pad so that the operand reads of 16 consecutive lanes (16
// rows, same column) fall in 16 distinct 16-byte slots of the 64-bank LDS.
// The grid is remapped so that consecutive workgroups of one head run on the
// same XCD (hardware dispatches workgroups round-robin over the 8 XCDs), so a
// head's K/V tiles are shared through that XCD's L2.
#include <limits.h>

#include <type_traits>

#include "sage_common.h"
#include "sage_device.h"

// Build switches for timing the schedules against each other (every setting
// computes the same result): SAGE_FWD_SCHED=0 builds the FP8 sweep with the
// unchunked per-tile code the FP16 and Q-smoothing sweeps use;
// SAGE_PINGPONG=0 keeps both waves of a SIMD on the same step order.
#ifndef SAGE_FWD_SCHED
#define SAGE_FWD_SCHED 1
#endif
#ifndef SAGE_PINGPONG
#define SAGE_PINGPONG 1
#endif

namespace sage {

// LDS: two K tiles (128 key rows of D bytes) and two V tiles (D channel rows
// of 128 keys x 1 or 2 bytes).  Every row carries a 16-byte pad: the 16-byte
// operand reads of 16 consecutive lanes (16 consecutive rows, same column)
// then fall in 16 distinct 16-byte slots of the 64-bank LDS.
template <int D, bool PV16>
struct Lds {
    static constexpr int VES = PV16 ? 2 : 1;
    static constexpr int KROW = D;                 // bytes of a K row in HBM
    static constexpr int VROW = kBc * VES;         // bytes of a V row in HBM
    static constexpr int KSTR = KROW + 16;         // bytes of a K row in LDS
    static constexpr int VSTR = VROW + 16;
    static constexpr int KBYTES = kBc * KSTR;      // one K tile in LDS
    static constexpr int VBYTES = D * VSTR;
    static constexpr int VBASE = 2 * KBYTES;
    static constexpr int TOTAL = 2 * (KBYTES + VBYTES);
    static constexpr int KPIECES = KBYTES / 1024;  // 1 KB direct-load pieces per tile
    static constexpr int VPIECES = VBYTES / 1024;
    static constexpr int KHBM = kBc * KROW;        // one K tile in HBM
    static constexpr int VHBM = D * VROW;
    static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "tiles must be whole 1 KB pieces");
};

// Key index held by lane half hh in register r of 32-key block k4 of a tile
// (the 32x32 MFMA accumulator layout: row 8*(r/4) + 4*hh + r%4).
__device__ inline int tile_key(int key_t, int k4, int r, int hh) {
    return key_t + 32 * k4 + 8 * (r >> 2) + 4 * hh + (r & 3);
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

// x with its bits replaced by `fill` when lim - OFF < 0 (the key at offset OFF
// of the lane's tile run is masked): v_subrev, v_ashrrev (sign word), v_bfi.
// Written as one ALU asm block so the compiler keeps it a branch-free 3-op
// sequence instead of hoisting 64 compares into scalar masks.
template <int OFF>
__device__ inline uint32_t mask_key(uint32_t x, int lim, uint32_t fill) {
    uint32_t w;
    asm("v_subrev_u32 %1, %4, %2\n\t"
        "v_ashrrev_i32 %1, 31, %1\n\t"
        "v_bfi_b32 %0, %1, %3, %0"
        : "+v"(x), "=&v"(w)
        : "v"(lim), "s"(fill), "i"(OFF));
    return x;
}

template <int K4, int R>
struct MaskTile {
    static constexpr int OFF = 32 * K4 + 8 * (R >> 2) + (R & 3);
    __device__ static void apply_int(v16i* S, int lim) {
        S[K4][R] = (int)mask_key<OFF>((uint32_t)S[K4][R], lim, 0x80000000u);
        if constexpr (R + 1 < 16) MaskTile<K4, R + 1>::apply_int(S, lim);
        else if constexpr (K4 + 1 < 4) MaskTile<K4 + 1, 0>::apply_int(S, lim);
    }
    __device__ static void apply_float(v16f* F, int lim) {
        F[K4][R] = __uint_as_float(mask_key<OFF>(__float_as_uint(F[K4][R]), lim, 0xff800000u));
        if constexpr (R + 1 < 16) MaskTile<K4, R + 1>::apply_float(F, lim);
        else if constexpr (K4 + 1 < 4) MaskTile<K4 + 1, 0>::apply_float(F, lim);
    }
    // INT32 scores held as fp32 bit patterns: masked keys get INT_MIN
    __device__ static void apply_intbits(v16f* S, int lim) {
        S[K4][R] = __uint_as_float(mask_key<OFF>(__float_as_uint(S[K4][R]), lim, 0x80000000u));
        if constexpr (R + 1 < 16) MaskTile<K4, R + 1>::apply_intbits(S, lim);
        else if constexpr (K4 + 1 < 4) MaskTile<K4 + 1, 0>::apply_intbits(S, lim);
    }
};

// First half of the online-softmax step of one tile for this lane's query:
// masking, the tile max (on the integers: c > 0 and rounding is monotone, so
// max_j fp32(S_j c) = fp32(max_j S_j * c)), the new running max m and alpha,
// and F = float(S) with masked keys at -inf.  With needmask (wave-uniform),
// the keys past `lim` (key - key_t - 4 hh > lim: beyond N, or after the query
// when causal) are masked.
// With Q smoothing (brow = this lane's block row of the tile's correction in
// LDS): F = s = fma(float(S), c, bias) and the max is taken over s.
template <bool QSM>
__device__ inline void softmax_prep(v16i* S, v16f* F, float c, const uint8_t* brow, float& m,
                                    float& alpha, float& mu, bool needmask, int lim, int hh) {
    if constexpr (QSM) {
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // keys 32 k4 + 8 i + 4 hh + (0..3): registers 4 i .. 4 i + 3
                const float4 bb = *(const float4*)(brow + 4 * (32 * k4 + 8 * i + 4 * hh));
                F[k4][4 * i + 0] = __builtin_fmaf((float)S[k4][4 * i + 0], c, bb.x);
                F[k4][4 * i + 1] = __builtin_fmaf((float)S[k4][4 * i + 1], c, bb.y);
                F[k4][4 * i + 2] = __builtin_fmaf((float)S[k4][4 * i + 2], c, bb.z);
                F[k4][4 * i + 3] = __builtin_fmaf((float)S[k4][4 * i + 3], c, bb.w);
            }
        if (needmask) MaskTile<0, 0>::apply_float(F, lim);
        float mk[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            float x = fmaxf(F[k4][0], F[k4][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) x = fmaxf(fmaxf(x, F[k4][r]), F[k4][r + 1]);
            mk[k4] = x;
        }
        const float mt = pair_fmax(fmaxf(fmaxf(mk[0], mk[1]), fmaxf(mk[2], mk[3])));
        const float mn = fmaxf(m, mt);
        alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        mu = mn - kLog2PScale;
        return;
    }
    if (needmask) MaskTile<0, 0>::apply_int(S, lim);
    int mk[4];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
        int x = max(S[k4][0], S[k4][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) x = max(max(x, S[k4][r]), S[k4][r + 1]);
        mk[k4] = x;
    }
    const int mx = pair_max(max(max(mk[0], mk[1]), max(mk[2], mk[3])));
    const float mt = mx == INT_MIN ? -INFINITY : (float)mx * c;
    const float mn = fmaxf(m, mt);
    alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    mu = mn - kLog2PScale;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
        for (int r = 0; r < 16; ++r) F[k4][r] = (float)S[k4][r];
    if (needmask) MaskTile<0, 0>::apply_float(F, lim);
}

// Second half, one 32-key block k4: p = exp2(fma(F, c, -mu)) (= 448 * 2^(s - m')),
// P (FP8 e4m3 or FP16) into the P V operand, and the partial row sum of the
// quantized P (the values the P V product weights V with, decoded from the
// operand).  XS: also the partial sum of the unquantized p into xs (the
// log-sum-exp of the scores).
// c == 0 only when the whole tile's S is 0; any positive factor then gives
// the same argument, and a positive one keeps -inf * factor = -inf.
// With Q smoothing F already holds s: p = exp2(fp32(s - mu)).
template <bool QSM, bool XS, typename PT, bool SUM = true>
__device__ inline float softmax_block(const v16f& Fk, PT* P, int k4, float cf, float mu,
                                      float& xs) {
    float part[4], xpart[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            p[j] = __builtin_amdgcn_exp2f(QSM ? Fk[4 * u + j] - mu
                                              : __builtin_fmaf(Fk[4 * u + j], cf, -mu));
        if constexpr (XS) xpart[u] = (p[0] + p[1]) + (p[2] + p[3]);
        if constexpr (__is_same(PT, v8i)) {
            // the first half-word write keeps the other half of its old operand;
            // p[0]'s own register (dead after this) serves, so no zeroing move
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
            P[k4 >> 1][(k4 & 1) * 4 + u] = w;
            if constexpr (SUM) {
                const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
                const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
                part[u] = (lo.x + lo.y) + (hi.x + hi.y);
            } else {
                part[u] = 0.0f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) P[2 * k4 + (u >> 1)][4 * (u & 1) + j] = (_Float16)p[j];
            const v2h h01 = v2h{(_Float16)p[0], (_Float16)p[1]};
            const v2h h23 = v2h{(_Float16)p[2], (_Float16)p[3]};
            const v2h one = v2h{(_Float16)1.0f, (_Float16)1.0f};
            part[u] = __builtin_amdgcn_fdot2(h01, one, 0.0f, false) +
                      __builtin_amdgcn_fdot2(h23, one, 0.0f, false);
        }
    }
    if constexpr (XS) xs = (xpart[0] + xpart[1]) + (xpart[2] + xpart[3]);
    return (part[0] + part[1]) + (part[2] + part[3]);
}

// P V into the running output: O = alpha O + V^T P^T.  The MFMA accumulates in
// FP32 straight into O (the rescale by alpha is skipped when every lane's
// alpha is 1).  Lane (channel n, hh) reads V row 32 cb + n, key positions
// [64 hh + 32 hf, +32) (FP8) or [64 hh + 8 u, +8) (FP16).
template <int D>
__device__ inline void pv_tile(const uint8_t* vb, const v8i* P, v16f* O, float alpha, int n,
                               int hh) {
    using L = Lds<D, false>;
    const uint8_t* vrow = vb + n * L::VSTR + 64 * hh;
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[cb][e] *= alpha;
    }
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
        const v8i a0 = *(const v8i*)(vrow + 32 * cb * L::VSTR);
        const v8i a1 = *(const v8i*)(vrow + 32 * cb * L::VSTR + 32);
        O[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, P[0], O[cb], 0, 0, 0, 0, 0, 0);
        O[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, P[1], O[cb], 0, 0, 0, 0, 0, 0);
    }
}

template <int D>
__device__ inline void pv_tile(const uint8_t* vb, const v8h* P, v16f* O, float alpha, int n,
                               int hh) {
    using L = Lds<D, true>;
    const uint8_t* vrow = vb + n * L::VSTR + 128 * hh;
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[cb][e] *= alpha;
    }
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const v8h av = *(const v8h*)(vrow + 32 * cb * L::VSTR + 16 * u);
            O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, P[u], O[cb], 0, 0, 0);
        }
}

// O = alpha O when some lane's alpha differs from 1 (a wave-uniform branch).
template <int D>
__device__ inline void rescale_o(v16f* O, float alpha) {
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[cb][e] *= alpha;
    }
}

// The P V MFMAs of pv_tile alone (O already rescaled).
template <int D>
__device__ inline void pv_mfma(const uint8_t* vb, const v8i* P, v16f* O, int n, int hh) {
    using L = Lds<D, false>;
    const uint8_t* vrow = vb + n * L::VSTR + 64 * hh;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
        const v8i a0 = *(const v8i*)(vrow + 32 * cb * L::VSTR);
        const v8i a1 = *(const v8i*)(vrow + 32 * cb * L::VSTR + 32);
        O[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, P[0], O[cb], 0, 0, 0, 0, 0, 0);
        O[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, P[1], O[cb], 0, 0, 0, 0, 0, 0);
    }
}

template <int D>
__device__ inline void pv_mfma(const uint8_t* vb, const v8h* P, v16f* O, int n, int hh) {
    using L = Lds<D, true>;
    const uint8_t* vrow = vb + n * L::VSTR + 128 * hh;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const v8h av = *(const v8h*)(vrow + 32 * cb * L::VSTR + 16 * u);
            O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, P[u], O[cb], 0, 0, 0);
        }
}

// 32-key block k4 of S^T = K8 tile . Q8^T: lane (n, hh) reads key row 32 k4 + n,
// channels [32 kk + 16 hh, +16).
template <int D, int KSTR>
__device__ inline v16i qk_block(const uint8_t* kb, const v4i* qf, int k4, int n, int hh) {
    constexpr int KK = D / 32;
    const uint8_t* krow = kb + (32 * k4 + n) * KSTR + 16 * hh;
    v4i av[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) av[kk] = *(const v4i*)(krow + 32 * kk);
    v16i acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[0], qf[0], v16i{}, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < KK; ++kk) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[kk], qf[kk], acc, 0, 0, 0);
    return acc;
}

// Q8^T operand of this lane (query qi, half hh: channels [32 kk + 16 hh, +16))
// and the row's dequantization factor q_scale * lambda.  A wave whose 32
// queries are all padding runs the sweep on zero codes; its rows are never
// written.
template <int D>
__device__ inline float load_q(const AttnArgs& a, int bh, int qbase, int qi, int hh, bool active,
                               v4i* qf) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qf[kk] = v4i{};
    if (!active) return 0.0f;
    const int8_t* qrow = a.q8 + ((int64_t)bh * a.N_pad + qi) * D + 16 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qf[kk] = *(const v4i*)(qrow + 32 * kk);
    // per block: one scale for the wave's 32 queries; per token: one per lane
    const float qs = a.qtok ? a.q_scale[(int64_t)bh * a.N_pad + qi] : a.q_scale[bh * a.nblk + qbase / kBlk];
    return qs * a.lambda;
}

// Output row qi = O^T column * v_scale / lt, this lane's half of the channels
// (32 cb + 8 r4 + 4 hh + j).  ZERO_EMPTY: a row that saw no key (lt = 0) is 0.
template <int D, bool ZERO_EMPTY>
__device__ inline void store_row(const AttnArgs& a, const v16f* O, float lt, int b, int h, int bh,
                                 int qi, int hh) {
    const int64_t obase = row_offset(a.layout, b, h, qi, a.H, a.N, D);
    const float* vs = a.v_scale + bh * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int c0 = 32 * cb + 8 * r4 + 4 * hh;
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = (ZERO_EMPTY && !(lt > 0.0f)) ? 0.0f : (O[cb][4 * r4 + j] * vs[c0 + j]) / lt;
            if (a.out_fp32) {
                *(float4*)((float*)a.out + obase + c0) = make_float4(o[0], o[1], o[2], o[3]);
            } else {
                const uint32_t w0 = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
                const uint32_t w1 = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
                *(uint2*)((u16*)a.out + obase + c0) = make_uint2(w0, w1);
            }
        }
}

// The two halves of one key tile's step in the pipelined sweep, written as
// chunks that __builtin_amdgcn_sched_barrier keeps in program order: each
// chunk issues one MFMA (its LDS operand read one chunk ahead) and then a
// share of the tile's vector work, so the vector instructions issue while the
// MFMAs run instead of before or after all of them.
// An empty asm that takes x and gives it back: x is computed at this point of
// the program and not moved by the compiler's code motion (sinking towards its
// uses would pull a chunk's vector work out of the MFMA shadow it was placed
// in).
__device__ inline float pinned(float x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ inline int pinned(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

__device__ inline v16f mfma_pv(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ inline v16f mfma_pv(const v8h& a, const v8h& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Row sum of the FP8 P operand on the matrix core: one 16x16x128 MFMA per
// 64-key half of the tile, A = a 0/1 pattern in FP8 (e4m3, 1.0 = 0x38),
// B = the P V operand (32 keys of one query per lane).  Lane l of the
// B operand holds column l % 16 of key group l / 16 (query l % 32); the
// pattern row r takes key groups g with g % 2 == (r / 4) % 2, so output row
// r, column c sums both key halves of query c + 16 ((r / 4) % 2), which is
// what lane c + 16 (r / 4) holds in its 4 accumulator registers: each lane
// gets its own query's sum over all 128 keys (both lane halves).
__device__ inline v4f rowsum_p(const v8i& ones, const v8i* P, const v4f& acc, int half) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, P[half], acc, 0, 0, 0, 0, 0, 0);
}
__device__ inline v4f rowsum_p(const v8i&, const v8h*, const v4f& acc, int) { return acc; }
__device__ inline v8i rowsum_pattern(int lane) {
    const int on = (((lane >> 4) & 1) == (((lane & 15) >> 2) & 1)) ? 0x38383838 : 0;
    return v8i{on, on, on, on, on, on, on, on};
}

// Phase A: P V of the previous tile (O already rescaled by its alpha) with, in
// the MFMAs' shadow, this tile's integer row max and float(S) (one 32-key
// block per unit), then the running max m, alpha and mu, then the exponent
// arguments F = fma(float(S), c, -mu) (one block per unit).  Same arithmetic
// as pv_tile + softmax_prep + the argument of softmax_block.
template <int D, bool PV16, bool SPARSE, bool RS, typename PT>
__device__ inline void phase_a(const uint8_t* vb, const PT* P, v16f* O, const v16f* S, v16f* F,
                               float c, float& m, float& alpha, float& l, const v8i& ones, int n,
                               int hh) {
    using L = Lds<D, PV16>;
    constexpr int NPV = (PV16 ? 8 : 2) * (D / 32);
    // MFMA i: fp8 -> channel block i / 2, 32 key bytes at 32 (i % 2);
    //         fp16 -> channel block i / 8, 8 keys at 16 (i % 8) bytes
    const uint8_t* vrow = vb + n * L::VSTR + (PV16 ? 128 : 64) * hh;
    auto vop = [&](int i) -> PT {
        return PV16 ? *(const PT*)(vrow + 32 * (i / 8) * L::VSTR + 16 * (i % 8))
                    : *(const PT*)(vrow + 32 * (i / 2) * L::VSTR + 32 * (i % 2));
    };
    constexpr int PER = PV16 ? 8 : 2;
    int mk[4];
    float cf = 1.0f, mu = 0.0f;
    PT op[2];
    op[0] = vop(0);
    v4f rs = v4f{};
    const float alpha_prev = alpha;  // the previous tile's, which its P was formed with
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
        if (i + 1 < NPV) op[(i + 1) & 1] = vop(i + 1);
        O[i / PER] = mfma_pv(op[i & 1], P[i % PER], O[i / PER]);
        if constexpr (RS) {
            // the previous tile's row sum of P on the matrix core (see rowsum_p)
            if (i == 0) rs = rowsum_p(ones, P, rs, 0);
            if (i == 1) rs = rowsum_p(ones, P, rs, 1);
            if (i == NPV - 1) l = alpha_prev * l + rs[0];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (u * NPV / 8 != i) continue;
            if (u < 4) {
                const v16i Si = __builtin_bit_cast(v16i, S[u]);
                int x = max(Si[0], Si[1]);
#pragma unroll
                for (int r = 2; r < 16; r += 2) x = max(max(x, Si[r]), Si[r + 1]);
                mk[u] = pinned(x);
#pragma unroll
                for (int r = 0; r < 16; ++r) F[u][r] = pinned((float)Si[r]);
            } else {
                if (u == 4) {
                    const int mx = pair_max(max(max(mk[0], mk[1]), max(mk[2], mk[3])));
                    const float mt = mx == INT_MIN ? -INFINITY : (float)mx * c;
                    const float mn = fmaxf(m, mt);
                    alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
                    m = mn;
                    mu = mn - kLog2PScale;
                    // no key seen yet (m = -inf): any finite mu keeps p = exp2(-inf) = 0
                    if (SPARSE && m == -INFINITY) mu = 0.0f;
                    cf = c == 0.0f ? 1.0f : c;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    F[u - 4][r] = pinned(__builtin_fmaf(F[u - 4][r], cf, -mu));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// P (FP8 or FP16) of 4 consecutive values of block k4 (registers 4u .. 4u+3)
// into the P V operand, and their partial sum (p0 + p1) + (p2 + p3).
// The sum is formed first and pinned in place (an empty asm that takes it),
// so the compiler neither sinks the adds to the end of the sweep step nor
// keeps p0 alive past the pack (whose first write reuses p0's register for
// the dword's other half).
template <bool SUM>
__device__ inline float pack_group(const v16f& Fk, v8i* P, int k4, int u) {
    const float p0 = Fk[4 * u], p1 = Fk[4 * u + 1], p2 = Fk[4 * u + 2], p3 = Fk[4 * u + 3];
    float sum = 0.0f;
    if constexpr (SUM) {
        sum = (p0 + p1) + (p2 + p3);
        asm volatile("" : "+v"(sum));
    }
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __float_as_int(p0), false);
    w = pinned(__builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true));
    P[k4 >> 1][(k4 & 1) * 4 + u] = w;
    return sum;
}
template <bool SUM>
__device__ inline float pack_group(const v16f& Fk, v8h* P, int k4, int u) {
    float sum = (Fk[4 * u] + Fk[4 * u + 1]) + (Fk[4 * u + 2] + Fk[4 * u + 3]);
    asm volatile("" : "+v"(sum));
#pragma unroll
    for (int j = 0; j < 4; ++j) P[2 * k4 + (u >> 1)][4 * (u & 1) + j] = (_Float16)Fk[4 * u + j];
    return sum;
}

// Phase B: Q K^T of the next tile (16 INT8 MFMAs at d = 128) with, in their
// shadow, p = exp2(F) of this tile in groups of 4 values, each group packed
// into P and summed one chunk after its exponentials (so no exp2 result is
// read right after it is written).  part[k4] = the row sum of block k4, in
// softmax_block's association.
template <int D, int KSTR, bool SUM, typename PT>
__device__ inline void phase_b(const uint8_t* kb, const v4i* qf, v16f* S, v16f* F, PT* P,
                               float* part, int n, int hh) {
    constexpr int KK = D / 32, NQK = 4 * KK;
    // MFMA j: key block j / KK, channel chunk j % KK
    auto kop = [&](int j) -> v4i {
        return *(const v4i*)(kb + (32 * (j / KK) + n) * KSTR + 16 * hh + 32 * (j % KK));
    };
    float gs[16];
    v4i op[2];
    op[0] = kop(0);
#pragma unroll
    for (int j = 0; j <= NQK; ++j) {
        if (j < NQK) {
            if (j + 1 < NQK) op[(j + 1) & 1] = kop(j + 1);
            S[j / KK] = __builtin_bit_cast(
                v16f, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                          op[j & 1], qf[j % KK],
                          (j % KK) ? __builtin_bit_cast(v16i, S[j / KK]) : v16i{}, 0, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            const int cj = g * NQK / 16;  // chunk of this group's exponentials
            if (cj == j && j < NQK)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    F[g >> 2][4 * (g & 3) + q] = __builtin_amdgcn_exp2f(F[g >> 2][4 * (g & 3) + q]);
                    F[g >> 2][4 * (g & 3) + q] = pinned(F[g >> 2][4 * (g & 3) + q]);
                }
            if (cj + 1 == j) gs[g] = pack_group<SUM>(F[g >> 2], P, g >> 2, g & 3);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
        part[k4] = (gs[4 * k4] + gs[4 * k4 + 1]) + (gs[4 * k4 + 2] + gs[4 * k4 + 3]);
}

// MODE: kDense, kDump (also writes the int32 Q K^T of one head), kSparse
// (visits only the key tiles a tile mask selects), kLse (dense, and writes
// each row's log-sum-exp: the forward of 8-bit training).  QSM: Q smoothing,
// the scores carry the per-(query block, key) correction a.bias.
enum { kDense = 0, kDump = 1, kSparse = 2, kLse = 3 };

// Waves per workgroup: 8 (256 queries, one workgroup per CU), or 4 (128
// queries = one query block, two workgroups per CU) for the sparse sweep, so
// that a workgroup's tile list is its own block's and no wave computes tiles
// its block skips (FP16 P V at d = 128 keeps 8: its LDS fits one per CU).
template <int D, bool PV16, int MODE>
constexpr int attn_waves() {
    return (MODE == kSparse && !(PV16 && D == 128)) ? 4 : 8;
}

// LDS bytes of one slot of the correction tile: one 512-byte row (128 keys)
// per 128-query block of the workgroup, a whole 1 KB copy piece in any case.
constexpr int kBiasSlot = 1024;

template <int D, bool PV16, bool CAUSAL, int MODE, bool QSM>
__global__ __launch_bounds__((64 * attn_waves<D, PV16, MODE>()), (8 / attn_waves<D, PV16, MODE>()))
void attn_fwd_kernel(AttnArgs a) {
    constexpr bool DUMP = MODE == kDump, SPARSE = MODE == kSparse, LSE = MODE == kLse;
    static_assert(!(QSM && DUMP), "the dump runs without Q smoothing");
    constexpr int NW = attn_waves<D, PV16, MODE>(), NT = 64 * NW, BR = 32 * NW;
    using L = Lds<D, PV16>;
    using PT = typename std::conditional<PV16, v8h, v8i>::type;
    constexpr int NP = PV16 ? 8 : 2;
    constexpr int KK = D / 32;
    constexpr int CB = D / 32;
    constexpr int BBASE = L::TOTAL;  // correction tiles (Q smoothing), two slots
    // PP: the two waves of a SIMD run the halves of a sweep step in opposite
    // order (see the loop), which needs a third K slot, after the V slots
    constexpr bool PP = MODE != kSparse && !QSM && !PV16 && SAGE_FWD_SCHED && SAGE_PINGPONG;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::TOTAL + (QSM ? 2 * kBiasSlot : 0) +
                                                          (PP ? L::KBYTES : 0)];
    // sparse: the key tiles this workgroup visits, ascending; bits 14 / 15 say
    // whether the first / second 128-query block of the workgroup visits it
    __shared__ uint16_t vlist[SPARSE ? kMaxSparseTiles : 1];
    __shared__ int vcount;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, a.total);
    const int bh = wg / a.nqt;
    int qt = wg - bh * a.nqt;
    if (CAUSAL) qt = a.nqt - 1 - qt;  // longest rows first
    const int H = a.H, N = a.N;
    const int b = bh / H, h = bh - b * H;
    const int qbase = qt * BR + wave * 32;
    const bool active = qbase < N;
    const int qi = qbase + n;

    int ntiles = a.nblk;
    if (CAUSAL) ntiles = (min(N, qt * BR + BR) - 1) / kBc + 1;
    const bool tail = (N % kBc) != 0;

    v4i qf[KK];
    const float sigma = load_q<D>(a, bh, qbase, qi, hh, active, qf);

    const uint8_t* kg = (const uint8_t*)a.k8 + (int64_t)bh * a.N_pad * D;
    const uint8_t* vg = (const uint8_t*)a.vq + (int64_t)bh * a.nblk * L::VHBM;
    constexpr int KMAXP = (L::KPIECES + NW - 1) / NW, VMAXP = (L::VPIECES + NW - 1) / NW;
    int koff[KMAXP], voff[VMAXP];
#pragma unroll
    for (int j = 0; j < KMAXP; ++j) koff[j] = slot_src<L::KROW, L::KSTR>(64 * (wave + NW * j) + lane);
#pragma unroll
    for (int j = 0; j < VMAXP; ++j) voff[j] = slot_src<L::VROW, L::VSTR>(64 * (wave + NW * j) + lane);
    const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // step t of the sweep works on key tile T (every tile when dense: T = t);
    // the tile goes to LDS slot t & 1
    // K slot of step t: t & 1, or t % 3 with PP (slot 2 after the V slots)
    auto kslot = [&](int t) -> uint32_t {
        if constexpr (PP) {
            const int s3 = t % 3;
            return s3 == 2 ? (uint32_t)L::TOTAL : (uint32_t)(s3 * L::KBYTES);
        }
        return (uint32_t)((t & 1) * L::KBYTES);
    };
    auto load_k = [&](int t, int T) {
        tile_to_lds<L::KPIECES, KMAXP, NW>(kg + (int64_t)T * L::KHBM, lbase + kslot(t), wv, koff);
    };
    auto load_v = [&](int t, int T) {
        tile_to_lds<L::VPIECES, VMAXP, NW>(vg + (int64_t)T * L::VHBM,
                                           lbase + L::VBASE + (t & 1) * L::VBYTES, wv, voff);
    };
    // Q smoothing: the correction rows of the workgroup's query blocks for key
    // tile T, one 1 KB piece issued by the last wave: lanes 0-31 copy the
    // first block's 512 bytes, lanes 32-63 the second block's (the first
    // again when the workgroup has one block or its second is past the end)
    const uint8_t* bg = nullptr;
    uint32_t boff = 0;
    if (QSM) {
        const int r0 = qt * (NW / 4);
        const int r1 = (NW == 8 && r0 + 1 < a.nblk) ? r0 + 1 : r0;
        bg = (const uint8_t*)(a.bias + ((int64_t)bh * a.nblk + r0) * a.N_pad);
        boff = (uint32_t)((hh ? (r1 - r0) : 0) * a.N_pad * 4 + 16 * n);
    }
    auto load_bias = [&](int t, int T) {
        if (QSM && wv == NW - 1) dma_piece(bg + (int64_t)T * 512, boff, lbase + BBASE + (t & 1) * kBiasSlot);
    };
    if (SPARSE) {
        // wave 0 compacts the visited tiles: tile T is visited when one of the
        // workgroup's query blocks (one or two) has a nonzero mask byte for it
        if (wave == 0) {
            const int r0 = qt * (NW / 4), nbq = a.nblk;
            const uint8_t* m0 = a.tmask + ((int64_t)bh * nbq + r0) * a.nblk;
            const bool has1 = NW == 8 && r0 + 1 < nbq;
            int cnt = 0;
            for (int base = 0; base < ntiles; base += 64) {
                const int T = base + lane;
                int e = 0;
                if (T < ntiles) e = (m0[T] != 0) | ((has1 && m0[a.nblk + T] != 0) << 1);
                const uint64_t bal = __ballot(e != 0);
                const int pos = cnt + __popcll(bal & ((1ull << lane) - 1ull));
                if (e) vlist[pos] = (uint16_t)(T | (e << 14));
                cnt += __popcll(bal);
            }
            if (lane == 0) vcount = cnt;
        }
        __syncthreads();
        ntiles = vcount;
    }
    // sparse: list entries of steps t, t+1, t+2 in scalar registers; the entry
    // of step t+3 is read from LDS early in step t and shifted in at its end,
    // so no list read sits on the path to a copy's address
    const int vbit = 14 + (wave >= 4);
    auto entry = [&](int t) {
        return (SPARSE && t < ntiles) ? __builtin_amdgcn_readfirstlane((int)vlist[t]) : 0;
    };
    int e0 = entry(0), e1 = entry(1), e2 = entry(2);

    float m = -INFINITY, l = 0.0f;
    float alpha = 1.0f;  // alpha of the tile whose P is held (tile -1: P = 0, alpha = 1)
    // RS: the row sum l of the quantized P is taken on the matrix core (the
    // chunked schedule, FP8 P); otherwise each lane adds its half of the
    // decoded P values.  LSE also keeps lx, the row sum of the unquantized p,
    // for the log-sum-exp of the scores.
    constexpr bool RS = !QSM && !PV16 && SAGE_FWD_SCHED;
    float lx = 0.0f;
    const v8i ones = rowsum_pattern(lane);
    v16f O[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) O[cb] = v16f{};
    // NEW: the chunked schedule (phase_a / phase_b).  X holds S(t) (INT32
    // scores as fp32 bit patterns) at the start of step t; phase A turns it
    // into the exponent arguments F(t) in Y, phase B forms S(t+1) in X.
    constexpr bool NEW = !QSM && !PV16 && SAGE_FWD_SCHED;
    v16i S[4];  // the older path's INT32 scores
    v16f F[4];  // the older path's exponent arguments
    v16f X[4], Y[4];
    float part[4];  // row sums by 32-key block (when not taken on the matrix core)
    PT P[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) P[i] = PT{};
    const int kmax = CAUSAL ? min(N - 1, qi) : N - 1;  // last key this lane's query sees

    // Software pipeline, one barrier per tile.  Iteration t:
    //   loads in flight: K(t+2), V(t);  LDS holds K(t+1), V(t-1)
    //   A: P V of tile t-1 (MFMA)      || mask + max + float(S) of tile t (VALU)
    //   B: per 32-key block, Q K^T of tile t+1 (MFMA) || exp / sum / FP8 of tile t (VALU)
    // so each wave always has independent MFMA and VALU work for the SIMD to
    // overlap with the other wave's.  V buffer 1 is zero-filled for tile -1.
    // PP: the second wave of each SIMD (waves 4-7) reaches each step's
    // barrier between A and B.  Between two barriers the first waves then run
    // A and B of step t while the second waves run B of step t-1 and A of
    // step t, so the two waves of a SIMD work on opposite halves at once, one
    // on P V + max + exponent arguments, the other on Q K^T + exp2 + P, and
    // the matrix core and the vector ALU both have a wave's work at all times.
    // Same code and arithmetic per wave; a K tile is read half a step longer,
    // hence the third K slot.
    const bool second = PP && wv >= 4;
    {
        uint4* vz = (uint4*)(smem + L::VBASE + L::VBYTES);
        for (int i = tid; i < L::VBYTES / 16; i += NT) vz[i] = make_uint4(0, 0, 0, 0);
    }
    if (!SPARSE || ntiles > 0) load_k(0, SPARSE ? (e0 & 0x3fff) : 0);
    if (ntiles > 1) load_k(1, SPARSE ? (e1 & 0x3fff) : 1);
    if (!SPARSE || ntiles > 0) load_bias(0, SPARSE ? (e0 & 0x3fff) : 0);
    wait_vmem();
    __syncthreads();
    if constexpr (NEW) {
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
            X[k4] = __builtin_bit_cast(v16f, qk_block<D, L::KSTR>(smem, qf, k4, n, hh));
    } else {
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) S[k4] = qk_block<D, L::KSTR>(smem, qf, k4, n, hh);
    }
    __syncthreads();

    const float* ksrow = a.k_scale + bh * a.nblk;
    float ks = (!SPARSE || ntiles > 0) ? ksrow[SPARSE ? (e0 & 0x3fff) : 0] : 0.0f;
    for (int t = 0; t < ntiles; ++t) {
        // the dequantization constant of tile t, taken before this iteration's
        // copies are issued (its load was issued one iteration earlier, so the
        // wait the compiler places before this use does not cover the copies)
        float c = sigma * ks;
        asm volatile("" : "+v"(c));
        const int T = SPARSE ? (e0 & 0x3fff) : t;
        ks = ksrow[SPARSE ? (t + 1 < ntiles ? (e1 & 0x3fff) : T) : min(t + 1, a.nblk - 1)];
        const uint32_t e3raw = (SPARSE && t + 3 < ntiles) ? vlist[t + 3] : 0u;
        if (t + 2 < ntiles) load_k(t + 2, SPARSE ? (e2 & 0x3fff) : t + 2);
        load_v(t, T);
        if (t + 1 < ntiles) load_bias(t + 1, SPARSE ? (e1 & 0x3fff) : t + 1);
        const int key_t = T * kBc;
        // a tile this wave's query block does not visit is masked whole: with
        // p = 0 and alpha = 1 it changes nothing, as if never seen
        const bool visits = !SPARSE || ((e0 >> vbit) & 1);
        const bool needmask = (tail && T == a.nblk - 1) || (CAUSAL && key_t + kBc - 1 > qbase) ||
                              !visits;
        const int lim = visits ? kmax - key_t - 4 * hh : -1;
        const uint8_t* vbuf = smem + L::VBASE + ((t + 1) & 1) * L::VBYTES;
        const bool dumps = DUMP && bh == a.dbh && qi >= a.drow0 && qi < a.drow0 + a.dnrows;
        if constexpr (NEW) {
            // A: P V of tile t-1 || max, float(S) and exponent arguments of tile t
            if (dumps) {
                v16i Sd[4];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) Sd[k4] = __builtin_bit_cast(v16i, X[k4]);
                dump_tile(Sd, a.s_out + (int64_t)(qi - a.drow0) * N, key_t, N, CAUSAL, qi, hh);
            }
            rescale_o<D>(O, alpha);
            if (needmask) MaskTile<0, 0>::apply_intbits(X, lim);
            phase_a<D, PV16, SPARSE, RS>(vbuf, P, O, X, Y, c, m, alpha, l, ones, n, hh);
            if (needmask) MaskTile<0, 0>::apply_float(Y, lim);
            // PP: the second waves reach this step's barrier between A and B,
            // so their B of this tile runs after it, beside the first waves' A
            // of the next tile
            if (second) {
                wait_vmem();
                __syncthreads();
            }
            // B: Q K^T of tile t+1 || exp2, P (and row sums) of tile t
            phase_b<D, L::KSTR, LSE>(smem + kslot(t + 1), qf, X, Y, P, part, n, hh);
            if constexpr (LSE) lx = alpha * lx + ((part[0] + part[1]) + (part[2] + part[3]));
        } else {
            if (dumps) dump_tile(S, a.s_out + (int64_t)(qi - a.drow0) * N, key_t, N, CAUSAL, qi, hh);
            // A
            pv_tile<D>(vbuf, P, O, alpha, n, hh);
            float mu;
            softmax_prep<QSM>(S, F, c, smem + BBASE + (t & 1) * kBiasSlot + (wave >> 2) * 512, m,
                              alpha, mu, needmask, lim, hh);
            // no key seen yet (m = -inf): any finite mu keeps p = exp2(-inf) = 0
            if (SPARSE && m == -INFINITY) mu = 0.0f;
            const float cf = c == 0.0f ? 1.0f : c;
            // B (the Q K^T of "tile ntiles" reads a stale buffer; its result is unused)
            const uint8_t* kb = smem + kslot(t + 1);
            float xpart[4];
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                S[k4] = qk_block<D, L::KSTR>(kb, qf, k4, n, hh);
                part[k4] = softmax_block<QSM, LSE>(F[k4], P, k4, cf, mu, xpart[k4]);
            }
            l = alpha * l + ((part[0] + part[1]) + (part[2] + part[3]));
            if constexpr (LSE) lx = alpha * lx + ((xpart[0] + xpart[1]) + (xpart[2] + xpart[3]));
        }
        if (SPARSE) {
            e0 = e1;
            e1 = e2;
            e2 = __builtin_amdgcn_readfirstlane((int)e3raw);
        }
        if (!second) {
            wait_vmem();
            __syncthreads();
        }
    }
    pv_tile<D>(smem + L::VBASE + ((ntiles + 1) & 1) * L::VBYTES, P, O, alpha, n, hh);
    if constexpr (RS) {
        v4f rs = rowsum_p(ones, P, v4f{}, 0);
        rs = rowsum_p(ones, P, rs, 1);
        l = alpha * l + rs[0];
    }
    // the final P V completes while every lane is active (see attn_mx_kernel)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) consume(O[cb]);

    // ---- epilogue: out = O * v_scale / l (l summed over both lane halves)
    const float lt = RS ? l : pair_sum(l);
    if (!active || qi >= N) return;
    // the row's log-sum-exp in the exp2 domain: p = 448 * 2^(s - m) makes
    // 2^(s - lse) = p / lx the softmax probability with lse = (m - log2 448) + log2 lx,
    // lx the row sum of the unquantized p
    if constexpr (LSE) {
        const float lxt = pair_sum(lx);
        if (hh == 0) a.lse[(int64_t)bh * N + qi] = (m - kLog2PScale) + log2f(lxt);
    }
    store_row<D, SPARSE>(a, O, lt, b, h, bh, qi, hh);
}

// Non-pipelined sweep with 12 waves (384 queries) per workgroup, three per
// SIMD, for d = 64: at d = 64 a wave needs about 135 VGPRs without the
// software pipeline, so a third wave per SIMD fits and hides more latency than
// the pipeline does (+24 % per query measured against the 8-wave kernel on
// the d = 64 outlier workload).  Per tile: Q K^T, softmax, rescale and P V in
// program order; K(t+1) and V(t+1) load into the other slot meanwhile.  Same
// arithmetic per query as attn_fwd_kernel, so the outputs are identical.
template <int D, bool PV16, int NW>
__global__ __launch_bounds__((64 * NW), 3) void attn_np_kernel(AttnArgs a) {
    using L = Lds<D, PV16>;
    using PT = typename std::conditional<PV16, v8h, v8i>::type;
    constexpr int NP = PV16 ? 8 : 2;
    constexpr int BR = 32 * NW, KK = D / 32, CB = D / 32;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * (L::KBYTES + L::VBYTES)];
    constexpr int VB = 2 * L::KBYTES;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, a.total);
    const int bh = wg / a.nqt;
    const int qt = wg - bh * a.nqt;
    const int H = a.H, N = a.N;
    const int b = bh / H, h = bh - b * H;
    const int qbase = qt * BR + wave * 32;
    const bool active = qbase < N;
    const int qi = qbase + n;
    const int ntiles = a.nblk;
    const bool tail = (N % kBc) != 0;
    v4i qf[KK];
    const float sigma = load_q<D>(a, bh, qbase, qi, hh, active, qf);
    const uint8_t* kg = (const uint8_t*)a.k8 + (int64_t)bh * a.N_pad * D;
    const uint8_t* vg = (const uint8_t*)a.vq + (int64_t)bh * a.nblk * L::VHBM;
    constexpr int KMAXP = (L::KPIECES + NW - 1) / NW, VMAXP = (L::VPIECES + NW - 1) / NW;
    int koff[KMAXP], voff[VMAXP];
#pragma unroll
    for (int j = 0; j < KMAXP; ++j) koff[j] = slot_src<L::KROW, L::KSTR>(64 * (wave + NW * j) + lane);
#pragma unroll
    for (int j = 0; j < VMAXP; ++j) voff[j] = slot_src<L::VROW, L::VSTR>(64 * (wave + NW * j) + lane);
    const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto load_kv = [&](int t) {
        tile_to_lds<L::KPIECES, KMAXP, NW>(kg + (int64_t)t * L::KHBM, lbase + (t & 1) * L::KBYTES,
                                           wv, koff);
        tile_to_lds<L::VPIECES, VMAXP, NW>(vg + (int64_t)t * L::VHBM,
                                           lbase + VB + (t & 1) * L::VBYTES, wv, voff);
    };
    float m = -INFINITY, l = 0.0f;
    v16f O[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) O[cb] = v16f{};
    PT P[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) P[i] = PT{};
    // FP8 P: the row sum of the quantized P on the matrix core (two 16x16x128
    // MFMAs per tile, see rowsum_p); FP16 P: each lane adds its half
    constexpr bool RSN = !PV16;
    const v8i ones = rowsum_pattern(lane);
    const int kmax = N - 1;
    load_kv(0);
    wait_vmem();
    __syncthreads();
    typedef __attribute__((address_space(4))) const float cfloat;
    cfloat* ksrow = (cfloat*)(a.k_scale + bh * a.nblk);
    for (int t = 0; t < ntiles; ++t) {
        const float c = sigma * ksrow[t];
        if (t + 1 < ntiles) load_kv(t + 1);
        const int key_t = t * kBc;
        const uint8_t* kb = smem + (t & 1) * L::KBYTES;
        v16i S[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) S[k4] = qk_block<D, L::KSTR>(kb, qf, k4, n, hh);
        const bool needmask = tail && t == a.nblk - 1;
        v16f F[4];
        float mu, alpha;
        softmax_prep<false>(S, F, c, nullptr, m, alpha, mu, needmask, kmax - key_t - 4 * hh, hh);
        const float cf = c == 0.0f ? 1.0f : c;
        float part[4];
        float xs;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
            part[k4] = softmax_block<false, false, PT, !RSN>(F[k4], P, k4, cf, mu, xs);
        if constexpr (RSN) {
            v4f rs = rowsum_p(ones, P, v4f{}, 0);
            rs = rowsum_p(ones, P, rs, 1);
            l = alpha * l + rs[0];
        } else {
            l = alpha * l + ((part[0] + part[1]) + (part[2] + part[3]));
        }
        pv_tile<D>(smem + VB + (t & 1) * L::VBYTES, P, O, alpha, n, hh);
        wait_vmem();
        __syncthreads();
    }
    // the last P V completes while every lane is active (see attn_mx_kernel)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) consume(O[cb]);
    const float lt = RSN ? l : pair_sum(l);
    if (!active || qi >= N) return;
    store_row<D, false>(a, O, lt, b, h, bh, qi, hh);
}

// -------------------------------------------------------------- MX attention
// Q, K, P and V in MXFP6 (E2M3 elements) or MXFP4 (E2M1), one E8M0 scale per
// 32 along the reduction; each 32-element block stored as 32 bytes: 24 (FP6)
// or 16 (FP4) code bytes, the scale byte at offset 24.  Q K^T and P V on
// v_mfma_scale_f32_32x32x64_f8f6f4 (FP6 or FP4 operands, the same rate), the
// online softmax in FP32 between them.
// The matrix core applies the block scales, so S arrives as fp32 and the
// epilogue needs no V scale.
//
// Key order: LDS row 32 k4 + n of a K tile holds tile key mx_row_key(k4, n),
// so accumulator register r of lane half hh in block k4 is key
// 32 (k4 / 2) + 16 k4 + 32 hh + r.  A lane's 32 values of the 64-key chunk
// u = k4 / 2 are then the consecutive keys 64 u + 32 hh + [0, 32): one MX
// block of P per lane and chunk, packed from S[2u] (first 16) and S[2u+1]
// (second 16) in the order the V blocks are packed.
// x y rounded toward -infinity (x = -inf gives -inf): the product rounded
// to nearest, stepped down one ulp when it came out above the exact product.
__device__ inline float mul_round_down(float x, float y) {
    const float p = x * y;
    if (!(__builtin_fmaf(x, y, -p) < 0.0f)) return p;
    const uint32_t u = __float_as_uint(p);
    return p > 0.0f ? __uint_as_float(u - 1u) : p < 0.0f ? __uint_as_float(u + 1u) : -0x1p-149f;
}

__device__ inline int mx_row_key(int k4, int n) {
    return 32 * (k4 >> 1) + 16 * k4 + 32 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
}

template <int K4, int R>
struct MaskTileMx {
    static constexpr int OFF = 32 * (K4 >> 1) + 16 * K4 + R;
    __device__ static void apply(v16f* F, int lim) {
        F[K4][R] = __uint_as_float(mask_key<OFF>(__float_as_uint(F[K4][R]), lim, 0xff800000u));
        if constexpr (R + 1 < 16) MaskTileMx<K4, R + 1>::apply(F, lim);
        else if constexpr (K4 + 1 < 4) MaskTileMx<K4 + 1, 0>::apply(F, lim);
    }
};

// Operand format code of the scaled matrix instruction for element format
// FMT: 2 = E2M3 (FP6), 4 = E2M1 (FP4; only the first 4 dwords of an operand
// are read).
template <int FMT>
constexpr int mx_code() { return FMT == 4 ? 4 : 2; }

// 32-key block k4 of S^T = K6 tile . Q6^T (fp32, block scales applied): lane
// (n, hh) reads LDS row 32 k4 + n, MX block 2 kk + hh of each 64-channel chunk.
template <int D, int KSTR, int FMT>
__device__ inline v16f qk_mx(const uint8_t* kb, const v8i* qv, int k4, int n, int hh) {
    const uint8_t* krow = kb + (32 * k4 + n) * KSTR + 32 * hh;
    v16f acc = v16f{};
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
        const v8i av = *(const v8i*)(krow + 64 * kk);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qv[kk], acc, mx_code<FMT>(),
                                                              mx_code<FMT>(), 0, av[6], 0, qv[kk][6]);
    }
    return acc;
}

// P V into the running output: O = alpha O + V^T P^T.  Lane (channel n, hh)
// reads V row 32 cb + n, MX block 2 u + hh (keys 64 u + 32 hh + [0, 32)).
template <int D, int FMT>
__device__ inline void pv_mx(const uint8_t* vb, const v8i* P, const int* pe, v16f* O, float alpha,
                             int n, int hh) {
    using L = Lds<D, false>;
    const uint8_t* vrow = vb + n * L::VSTR + 32 * hh;
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[cb][e] *= alpha;
    }
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const v8i av = *(const v8i*)(vrow + 32 * cb * L::VSTR + 64 * u);
            O[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, P[u], O[cb], mx_code<FMT>(),
                                                                    mx_code<FMT>(), 0, av[6], 0, pe[u]);
        }
}

// One MX block of P: 32 probabilities (pa: keys +0..15, pb: +16..31) with
// the block exponent e (scale 2^e; a zero block comes with scale 2^127, so
// every code is 0).  E2M1: byte i of the operand holds keys i and 16 + i,
// the layout the V blocks are stored in.
template <int FMT>
__device__ inline v8i pack_p_mx(const v16f& pa, const v16f& pb, float scale) {
    if constexpr (FMT == 4) {
        v8i o = v8i{};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t d = 0u;
            d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, pa[4 * w], pb[4 * w], scale, 0);
            d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, pa[4 * w + 1], pb[4 * w + 1], scale, 1);
            d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, pa[4 * w + 2], pb[4 * w + 2], scale, 2);
            d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, pa[4 * w + 3], pb[4 * w + 3], scale, 3);
            o[w] = (int)d;
        }
        return o;
    }
    v6i r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(pa, pb, scale);
    // multi-pass conversion: its sources stay live past it, so the result
    // registers cannot overlap them.  The result passes through the same
    // empty asm, which orders it after the conversion (an asm without that
    // dependence may be scheduled before it and protect nothing).
    asm volatile("" : "+v"(r) : "v"(pa), "v"(pb), "v"(scale));
    v8i o = v8i{};
#pragma unroll
    for (int i = 0; i < 6; ++i) o[i] = r[i];
    return o;
}

template <int D, bool CAUSAL, int FMT>
__global__ __launch_bounds__(512, 1) void attn_mx_kernel(AttnArgs a) {
    constexpr int NW = 8, NT = 64 * NW, BR = 32 * NW;
    using L = Lds<D, false>;
    constexpr int CB = D / 32;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::TOTAL];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, a.total);
    const int bh = wg / a.nqt;
    int qt = wg - bh * a.nqt;
    if (CAUSAL) qt = a.nqt - 1 - qt;  // longest rows first
    const int H = a.H, N = a.N;
    const int b = bh / H, h = bh - b * H;
    const int qbase = qt * BR + wave * 32;
    const bool active = qbase < N;
    const int qi = qbase + n;
    int ntiles = a.nblk;
    if (CAUSAL) ntiles = (min(N, qt * BR + BR) - 1) / kBc + 1;
    const bool tail = (N % kBc) != 0;

    // Q6^T operand: lane (query qi, hh) holds MX block 2 kk + hh of each
    // 64-channel chunk (codes and the scale dword); zero for padding waves
    v8i qv[D / 64];
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) qv[kk] = v8i{};
    if (active) {
        const uint8_t* qrow = (const uint8_t*)a.q8 + ((int64_t)bh * a.N_pad + qi) * D + 32 * hh;
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) qv[kk] = *(const v8i*)(qrow + 64 * kk);
    }
    const float lam = a.lambda;

    const uint8_t* kg = (const uint8_t*)a.k8 + (int64_t)bh * a.N_pad * D;
    const uint8_t* vg = (const uint8_t*)a.vq + (int64_t)bh * a.nblk * L::VHBM;
    constexpr int KMAXP = (L::KPIECES + NW - 1) / NW, VMAXP = (L::VPIECES + NW - 1) / NW;
    // K: LDS row R = 32 k4 + n takes tile key mx_row_key(k4, n)
    int koff[KMAXP], voff[VMAXP];
#pragma unroll
    for (int j = 0; j < KMAXP; ++j) {
        constexpr int CPR = L::KSTR / 16;
        const int P = 64 * (wave + NW * j) + lane, R = P / CPR, c = P % CPR;
        const int key = mx_row_key(R >> 5, R & 31);
        koff[j] = key * L::KROW + (c < L::KROW / 16 ? 16 * c : 0);
    }
#pragma unroll
    for (int j = 0; j < VMAXP; ++j) voff[j] = slot_src<L::VROW, L::VSTR>(64 * (wave + NW * j) + lane);
    const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto load_k = [&](int t) {
        tile_to_lds<L::KPIECES, KMAXP, NW>(kg + (int64_t)t * L::KHBM, lbase + (t & 1) * L::KBYTES, wv,
                                           koff);
    };
    auto load_v = [&](int t) {
        tile_to_lds<L::VPIECES, VMAXP, NW>(vg + (int64_t)t * L::VHBM,
                                           lbase + L::VBASE + (t & 1) * L::VBYTES, wv, voff);
    };

    float m = -INFINITY, l = 0.0f;
    float alpha = 1.0f;  // alpha of the tile whose P is held (tile -1: P = 0, alpha = 1)
    v16f O[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) O[cb] = v16f{};
    v16f S[4];
    v8i P[2] = {v8i{}, v8i{}};
    int pe[2] = {0, 0};
    const int kmax = CAUSAL ? min(N - 1, qi) : N - 1;

    // Same software pipeline as the INT8 / FP8 kernel; V buffer 1 is
    // zero-filled for tile -1 (P = 0 must not meet stale bytes)
    {
        uint4* vz = (uint4*)(smem + L::VBASE + L::VBYTES);
        for (int i = tid; i < L::VBYTES / 16; i += NT) vz[i] = make_uint4(0, 0, 0, 0);
    }
    load_k(0);
    if (ntiles > 1) load_k(1);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) S[k4] = qk_mx<D, L::KSTR, FMT>(smem, qv, k4, n, hh);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        if (t + 2 < ntiles) load_k(t + 2);
        load_v(t);
        const int key_t = t * kBc;
        // A
        pv_mx<D, FMT>(smem + L::VBASE + ((t + 1) & 1) * L::VBYTES, P, pe, O, alpha, n, hh);
        const bool needmask = (tail && t == a.nblk - 1) || (CAUSAL && key_t + kBc - 1 > qbase);
        if (needmask) MaskTileMx<0, 0>::apply(S, kmax - key_t - 32 * hh);
        float mk[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            float x = fmaxf(S[k4][0], S[k4][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) x = fmaxf(fmaxf(x, S[k4][r]), S[k4][r + 1]);
            mk[k4] = x;
        }
        // row max over both lane halves (lambda > 0: max(S) lambda = max(S lambda)),
        // rounded down: the largest element's exponent argument is then >= 0
        // and its p at least 1, so its block's exponent cannot hang on how
        // exp2 rounds just below 1
        const float mt = mul_round_down(pair_fmax(fmaxf(fmaxf(mk[0], mk[1]), fmaxf(mk[2], mk[3]))), lam);
        const float mn = fmaxf(m, mt);
        alpha = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        const float mu = mn;
        // P block exponents: the block's largest p is the p of its largest S
        float sc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float pmax = __builtin_amdgcn_exp2f(__builtin_fmaf(fmaxf(mk[2 * u], mk[2 * u + 1]), lam, -mu));
            const bool zero = !(pmax >= 0x1p-100f);
            const int e = (int)((__float_as_uint(pmax) >> 23) & 0xffu) - 129;
            sc[u] = __uint_as_float(zero ? (254u << 23) : (uint32_t)(e + 127) << 23);
            pe[u] = zero ? 0 : e + 127;
        }
        // B: the exponentials of tile t, interleaved with Q K^T of tile t+1
        // into the same registers (the Q K^T of "tile ntiles" reads a stale
        // buffer; its result is unused)
        const uint8_t* kb = smem + ((t + 1) & 1) * L::KBYTES;
        float part[4];
        v16f pa;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            v16f p;
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[k4][r], lam, -mu));
            float s4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) s4[u] = (p[4 * u] + p[4 * u + 1]) + (p[4 * u + 2] + p[4 * u + 3]);
            part[k4] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
            S[k4] = qk_mx<D, L::KSTR, FMT>(kb, qv, k4, n, hh);
            if (k4 & 1) P[k4 >> 1] = pack_p_mx<FMT>(pa, p, sc[k4 >> 1]);
            else pa = p;
        }
        l = alpha * l + ((part[0] + part[1]) + (part[2] + part[3]));
        wait_vmem();
        __syncthreads();
    }
    pv_mx<D, FMT>(smem + L::VBASE + ((ntiles + 1) & 1) * L::VBYTES, P, pe, O, alpha, n, hh);
    // The matrix instructions read operands from all 64 lanes, but the
    // operand moves feeding them obey EXEC: the final P V must complete
    // before the exit below turns padding-query lanes off, so its results
    // are consumed here, where every lane is active.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) consume(O[cb]);

    const float lt = pair_sum(l);
    if (!active || qi >= N) return;
    const int64_t obase = row_offset(a.layout, b, h, qi, H, N, D);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int c0 = 32 * cb + 8 * r4 + 4 * hh;
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = O[cb][4 * r4 + j] / lt;
            if (a.out_fp32) {
                *(float4*)((float*)a.out + obase + c0) = make_float4(o[0], o[1], o[2], o[3]);
            } else {
                const uint32_t w0 = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
                const uint32_t w1 = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
                *(uint2*)((u16*)a.out + obase + c0) = make_uint2(w0, w1);
            }
        }
}

template <int FMT>
static const void* attn_mx_fn(int d, int causal) {
    if (d == 128)
        return causal ? (const void*)attn_mx_kernel<128, true, FMT> : (const void*)attn_mx_kernel<128, false, FMT>;
    return causal ? (const void*)attn_mx_kernel<64, true, FMT> : (const void*)attn_mx_kernel<64, false, FMT>;
}

hipError_t launch_attn_mx(const AttnArgs& args, int B, int d, int causal, int fmt, hipStream_t s) {
    AttnArgs a = args;
    a.nqt = (a.N + 255) / 256;
    a.total = B * a.H * a.nqt;
    const void* fn = fmt == 4 ? attn_mx_fn<4>(d, causal) : attn_mx_fn<6>(d, causal);
    void* kargs[] = {(void*)&a};
    return hipLaunchKernel(fn, dim3(a.total), dim3(512), kargs, 0, s);
}

template <int D, bool PV16, bool CAUSAL, int MODE, bool QSM>
static const void* attn_fn() {
    return (const void*)attn_fwd_kernel<D, PV16, CAUSAL, MODE, QSM>;
}

template <int D, bool PV16, int MODE, bool QSM>
static const void* attn_fn_rt(bool causal) {
    return causal ? attn_fn<D, PV16, true, MODE, QSM>() : attn_fn<D, PV16, false, MODE, QSM>();
}

template <int D, bool PV16>
static const void* attn_fn_rt(bool causal, int mode, bool qsm) {
    if (mode == kDump) return attn_fn_rt<D, PV16, kDump, false>(causal);
    if (mode == kLse) return attn_fn_rt<D, PV16, kLse, false>(causal);
    if (mode == kSparse)
        return qsm ? attn_fn_rt<D, PV16, kSparse, true>(causal) : attn_fn_rt<D, PV16, kSparse, false>(causal);
    return qsm ? attn_fn_rt<D, PV16, kDense, true>(causal) : attn_fn_rt<D, PV16, kDense, false>(causal);
}

// The 12-wave d = 64 sweep processes about 1.24x the queries per unit time of
// the 8-wave one in steady state (measured), but its workgroups are 1.5x
// larger: use it when its rounds of workgroups over the CUs do not lose that.
static bool np12_pays(int bh, int N) {
    static int ncu = 0;
    if (ncu == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            ncu = v;
        else
            ncu = 256;
    }
    const int64_t w8 = (int64_t)bh * ((N + 255) / 256), w12 = (int64_t)bh * ((N + 383) / 384);
    const int64_t r8 = (w8 + ncu - 1) / ncu, r12 = (w12 + ncu - 1) / ncu;
    return r12 * 150 < r8 * 124;   // r12 * 1.5 / 1.24 < r8
}

static int sparse_waves(int d, int pv16) {
    if (d == 128) return pv16 ? attn_waves<128, true, kSparse>() : attn_waves<128, false, kSparse>();
    return pv16 ? attn_waves<64, true, kSparse>() : attn_waves<64, false, kSparse>();
}

hipError_t launch_attn(const AttnArgs& args, int B, int d, int pv16, int causal, int dump,
                       hipStream_t s) {
    const int mode = dump ? kDump : (args.tmask ? kSparse : (args.lse ? kLse : kDense));
    const bool qsm = args.bias != nullptr && !dump;
    const void* fn;
    if (d == 128)
        fn = pv16 ? attn_fn_rt<128, true>(causal, mode, qsm) : attn_fn_rt<128, false>(causal, mode, qsm);
    else
        fn = pv16 ? attn_fn_rt<64, true>(causal, mode, qsm) : attn_fn_rt<64, false>(causal, mode, qsm);
    AttnArgs a = args;
    int nw = mode == kSparse ? sparse_waves(d, pv16) : 8;
    if (mode == kDense && !qsm && !causal && d == 64 && !a.lse && np12_pays(B * a.H, a.N)) {
        nw = 12;
        fn = pv16 ? (const void*)attn_np_kernel<64, true, 12> : (const void*)attn_np_kernel<64, false, 12>;
    }
    a.nqt = (a.N + 32 * nw - 1) / (32 * nw);
    a.total = B * a.H * a.nqt;
    void* kargs[] = {(void*)&a};
    return hipLaunchKernel(fn, dim3(a.total), dim3(64 * nw), kargs, 0, s);
}

}  // namespace sage

