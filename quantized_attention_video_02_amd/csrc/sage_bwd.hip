// 8-bit attention backward of libsage for gfx950 (CDNA4).
//
// Method (reportify.cn SageAttention tag page, SageAttention3 summary, bullet
// 8比特训练): per-block INT8 Q/K/V and per-token P with no quantization
// overhead; in the backward pass dO V^T stays FP16 and the other four products
// are quantized.  Per tile pair (query block of 128 x key block of 128), in the
// exp2 domain with the forward's log-sum-exp lse:
//   S  = q8 . k8 (INT8 MFMA, the forward's codes, K smoothed)
//   P  = exp2(fma(S, c, -lse_i)),  c = fp32(fp32(q_scale * lambda) * k_scale)
//   dP = f16(dO) . f16(V)^T (FP16 MFMA, FP32 accumulation)
//   dS = P (dP - D_i),  D_i = dO_i . O_i (dP's MFMA chain starts at -D_i)
//   dV += dO8^T . e4m3(448 P) * s_do / 448        (FP8 MFMA; dO8 per 128-row block)
//   dK += Q8^T . dS8 * s_ds * q_scale * sm_scale   (INT8 MFMA; dS8 per tile pair)
//   dQ += K8^T . dS8^T * s_ds * k_scale * sm_scale (INT8 MFMA)
// Three sweeps, each mirroring the forward's register layout: the dQ sweep
// keeps a wave's 32 queries (S^T, dP^T with queries on lanes; dS^T is directly
// the B operand of dQ^T = K^T dS^T) and sweeps key tiles; the dV and dK sweeps
// keep a wave's 32 keys (S, dP with keys on lanes; P and dS are directly the B
// operands of dV^T = dO8^T P~ and dK^T = Q8^T dS8) and sweep query tiles, one
// sum each.  The operands that meet an accumulator-shaped operand along the
// reduction are stored transposed with the matching order of the reduction
// index (the forward's V order for FP8, a 32-element order for INT8), written
// once by the preparation kernels.  A tile's dS absmax is reduced over the 4
// waves of its 128-row block through LDS.  Every sweep runs two waves per SIMD:
// the dQ and dK sweeps form S, dP and dS one 32-row block at a time and keep
// two row blocks per workgroup (8 waves), the dV sweep needs no dP or dS and
// runs two 4-wave workgroups per CU.
#include <limits.h>

#include "sage_common.h"
#include "sage_device.h"

namespace sage {

constexpr int kBwdThreads = 256;  // 4 waves: 128 rows per workgroup, 32 per wave
// LDS row strides, each with a 16-byte pad (16 consecutive rows then start in
// distinct 16-byte bank groups: the strides are odd multiples of 16 bytes):
// the transposed tiles have rows of 128 elements (queries or keys, 1 byte);
// the row tiles have rows of D channels (INT8 codes, 1 byte, or fp16).
constexpr int kKstr = 128 + 16;
template <int D>
struct BwdRow {
    static constexpr int I8 = D + 16;       // a row of D INT8 codes
    static constexpr int F16 = 2 * D + 16;  // a row of D fp16 values
};

// Order of a run of 128 elements along a reduction (element e = 32 kb + 8 b +
// 4 g + q, kb and b in 0..3, g in 0..1, q in 0..3):
//   pi32: e at 32 kb + 16 g + 4 b + q -- the 16 bytes a lane half g reads per
//         32-element block are the 16 accumulator registers of that block
//         (INT8 32x32x32 operands);
//   pi64: e at 64 g + 16 kb + 4 b + q -- the 32 bytes per 64-element step
//         (FP8 32x32x64 operands; the forward's V order).
__device__ inline int pi32_elem(int p) {
    return 32 * (p >> 5) + 8 * ((p >> 2) & 3) + 4 * ((p >> 4) & 1) + (p & 3);
}
__device__ inline int pi64_elem(int p) {
    return 32 * ((p >> 4) & 3) + 8 * ((p >> 2) & 3) + 4 * (p >> 6) + (p & 3);
}

__device__ inline float wave_fmax(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
    return x;
}

__device__ inline _Float16 f16_sat(float x) {
    return (_Float16)fminf(fmaxf(x, -65504.0f), 65504.0f);
}

// One block of 128 rows of a head: D_i = dO_i . O_i (fp32; the tile record
// keeps -D_i, the start of the key sweeps' dP chains), fp16 copies of dO
// and V (row-major, padded rows 0), and dO in FP8 e4m3 for the block's absmax
// scale s_do = fp32(a / 448) (codes of fp32(dO * fp32(448 / a))), written
// channel-major [D][128] with the rows in pi64 order.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(
    const u16* __restrict__ o, const u16* __restrict__ dO, const u16* __restrict__ v, int H, int N,
    int nblk, int layout, const float* __restrict__ lse, const float* __restrict__ q_scale,
    float* __restrict__ Dq, _Float16* __restrict__ do16, _Float16* __restrict__ v16,
    uint8_t* __restrict__ do8, float* __restrict__ s_do, float* __restrict__ rec) {
    constexpr int CPR = D / 8, RPI = kBwdThreads / CPR;
    constexpr int LSTR = kBlk + 4;  // floats per channel row of the fp32 dO tile
    __shared__ float tile[D * LSTR];
    __shared__ float red[kBwdThreads / 64];
    const int blk = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = threadIdx.x, cg = t % CPR, tr = t / CPR;
    const int64_t N_pad = (int64_t)nblk * kBlk;
    float amax = 0.0f;
    for (int r = tr; r < kBlk; r += RPI) {
        const int row = blk * kBlk + r;
        float xo[8], xd[8], xv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xo[e] = xd[e] = xv[e] = 0.0f;
        if (row < N) {
            const int64_t off = row_offset(layout, b, h, row, H, N, D) + cg * 8;
            const uint4 wo = *(const uint4*)(o + off), wd = *(const uint4*)(dO + off),
                        wv = *(const uint4*)(v + off);
            const uint32_t so[4] = {wo.x, wo.y, wo.z, wo.w}, sd[4] = {wd.x, wd.y, wd.z, wd.w},
                           sv[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xo[2 * e] = bf16_bits_to_f32(so[e] & 0xffffu);
                xo[2 * e + 1] = bf16_bits_to_f32(so[e] >> 16);
                xd[2 * e] = bf16_bits_to_f32(sd[e] & 0xffffu);
                xd[2 * e + 1] = bf16_bits_to_f32(sd[e] >> 16);
                xv[2 * e] = bf16_bits_to_f32(sv[e] & 0xffffu);
                xv[2 * e + 1] = bf16_bits_to_f32(sv[e] >> 16);
            }
        }
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) part = part + xd[e] * xo[e];
        // the row's CPR threads are consecutive lanes
#pragma unroll
        for (int s = CPR / 2; s >= 1; s >>= 1) part += __shfl_xor(part, s);
        float* rc = rec + ((int64_t)bh * nblk + blk) * kRecFloats;
        if (cg == 0) {
            Dq[bh * N_pad + row] = part;
            rc[kBlk + r] = -part;
            rc[r] = row < N ? lse[(int64_t)bh * N + row] : 0.0f;
        }
        v8h hd, hv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hd[e] = f16_sat(xd[e]);
            hv[e] = f16_sat(xv[e]);
            tile[(cg * 8 + e) * LSTR + r] = xd[e];
            amax = fmaxf(amax, fabsf(xd[e]));
        }
        *(v8h*)(do16 + (bh * N_pad + row) * D + cg * 8) = hd;
        *(v8h*)(v16 + (bh * N_pad + row) * D + cg * 8) = hv;
    }
    amax = wave_fmax(amax);
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    float a = red[0];
#pragma unroll
    for (int w = 1; w < kBwdThreads / 64; ++w) a = fmaxf(a, red[w]);
    const float inv = a > 0.0f ? (float)(448.0 / (double)a) : 0.0f;
    if (t == 0) {
        const float sd = (float)((double)a / 448.0);
        s_do[bh * nblk + blk] = sd;
        float* rc = rec + ((int64_t)bh * nblk + blk) * kRecFloats;
        rc[2 * kBlk] = q_scale[bh * nblk + blk];
        rc[2 * kBlk + 1] = sd;
    }
    uint8_t* dst = do8 + ((int64_t)bh * nblk + blk) * D * kBlk;
    for (int i = t; i < D * kBlk / 4; i += kBwdThreads) {
        const int c = i / (kBlk / 4), w = i % (kBlk / 4);
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = tile[c * LSTR + pi64_elem(4 * w + j)] * inv;
        int o4 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
        o4 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], o4, true);
        *(int*)(dst + c * kBlk + 4 * w) = o4;
    }
}

// INT8 codes [bh][N_pad][D] -> per block of 128 rows [D][128] with the rows in
// pi32 order (the Q and K codes as reduction-ordered operands).
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_t8_kernel(const int8_t* __restrict__ x8,
                                                            int nblk, int8_t* __restrict__ xt) {
    constexpr int LSTR = D + 4;
    __shared__ __attribute__((aligned(16))) uint8_t tile[kBlk * LSTR];
    const int blk = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const uint8_t* src = (const uint8_t*)x8 + ((int64_t)bh * nblk + blk) * kBlk * D;
    for (int i = t; i < kBlk * D / 4; i += kBwdThreads) {
        const int r = i / (D / 4), c4 = i % (D / 4);
        *(uint32_t*)&tile[r * LSTR + 4 * c4] = *(const uint32_t*)(src + (int64_t)r * D + 4 * c4);
    }
    __syncthreads();
    uint8_t* dst = (uint8_t*)xt + ((int64_t)bh * nblk + blk) * D * kBlk;
    for (int i = t; i < D * kBlk / 4; i += kBwdThreads) {
        const int c = i / (kBlk / 4), w = i % (kBlk / 4);
        uint32_t o4 = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) o4 |= (uint32_t)tile[pi32_elem(4 * w + j) * LSTR + c] << (8 * j);
        *(uint32_t*)(dst + c * kBlk + 4 * w) = o4;
    }
}

// Empty uses: the loads that produce x complete here (a kernel's one-time
// loads are waited for before its sweep, not inside it, where the wait
// would also cover the tile copies in flight).
__device__ inline void settle(const v4i& x) { asm volatile("" ::"v"(x)); }
__device__ inline void settle(const v8h& x) { asm volatile("" ::"v"(x)); }
__device__ inline void settle(float x) { asm volatile("" ::"v"(x)); }

// 16 accumulator registers of one 32-row block as INT8 codes (rne of
// y = fp32(x * inv), inv = fp32(127 / a) with a >= |x|, so the codes stay
// within +-127): the B operand of a 32x32x32 INT8 MFMA whose reduction runs
// over that block.  fp32(y + 1.5 * 2^23) is 1.5 * 2^23 + rne(y) exactly (for
// |y| < 2^22 the sum's ulp is 1), so the low byte of its bit pattern is the
// two's-complement code; v_perm_b32 gathers the low bytes of two sums.
__device__ inline v4i pack_i8(const float* x, float inv) {
    v4i r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t z[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) z[j] = __float_as_uint(x[4 * w + j] * inv + 12582912.0f);
        // bytes (z0.b0, z1.b0, 0, 0) and (0, 0, z2.b0, z3.b0)
        const uint32_t lo = __builtin_amdgcn_perm(z[1], z[0], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(z[3], z[2], 0x04000c0cu);
        r[w] = (int)(lo | hi);
    }
    return r;
}

// The tile's dS absmax over the 4 waves red[base .. base + 3] of one 128-row
// block (red: a float of LDS per wave of the workgroup) and its INT8 scale
// s = fp32(a / 127), inv = fp32(127 / a) (0 for a = 0).
__device__ inline void tile_scale(float amax, float* red, int wave, int lane, float& s, float& inv,
                                  int base = 0) {
    amax = wave_fmax(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    const float a = fmaxf(fmaxf(red[base], red[base + 1]), fmaxf(red[base + 2], red[base + 3]));
    s = (float)((double)a / 127.0);
    inv = a > 0.0f ? (float)(127.0 / (double)a) : 0.0f;
}

// Store of a 32x32 accumulator row set: the lane's row `row` of [.., D] fp32
// output, channels 32 cb + 8 r4 + 4 hh + j.
template <int D>
__device__ inline void store_f32_row(float* out, int64_t off, const v16f* X, int hh) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            *(float4*)(out + off + 32 * cb + 8 * r4 + 4 * hh) =
                make_float4(X[cb][4 * r4], X[cb][4 * r4 + 1], X[cb][4 * r4 + 2], X[cb][4 * r4 + 3]);
}

// ---------------------------------------------------------------- dQ sweep
// Workgroup = two query blocks of 128 (8 waves, two per SIMD), key tiles swept
// in ascending order, double-buffered in LDS: K codes [128 keys][BwdRow::I8],
// V fp16 [128 keys][BwdRow::F16], K codes transposed [D channels][kKstr].
// wave w keeps queries 128 (2 qg + w / 4) + 32 (w % 4) .. + 31, and both
// blocks share each key tile in LDS.  Per tile, S^T, dP^T, P^T and dS^T are
// formed one 32-key block at a time (one block's products live beside the
// tile's dS), the masked entries are zeroed after the blocks (a branch inside
// them would let the compiler hoist every block's products above it), and
// the transposed K operands of each channel block are read just before its
// dQ MFMAs; the dS scale is each query block's own (its 4 waves).  Causal:
// the sweep runs to the second block's diagonal tile; for the first block
// the tile after its own diagonal is masked whole.  (One wave keeps dQ, its
// Q codes and fp16 dO rows and one block's products in about 232 registers,
// so two waves share a SIMD.)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(BwdArgs a) {
    constexpr int NW = 8, KK = D / 32, CB = D / 32, HK = D / 16;
    constexpr int R8 = BwdRow<D>::I8, R16 = BwdRow<D>::F16;
    constexpr int K8B = kBc * R8, V16B = kBc * R16, KTB = D * kKstr;
    constexpr int SLOT = K8B + V16B + KTB;
    constexpr int KP = K8B / 1024, VP = V16B / 1024, TP = KTB / 1024;
    constexpr int KMAXP = (KP + NW - 1) / NW, VMAXP = (VP + NW - 1) / NW, TMAXP = (TP + NW - 1) / NW;
    static_assert(K8B % 1024 == 0 && V16B % 1024 == 0 && KTB % 1024 == 0, "1 KB copy pieces");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * SLOT];
    __shared__ float red[NW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, a.total);
    const int nqg = (a.nblk + 1) / 2;  // workgroups per head
    const int bh = wg / nqg;
    int qg = wg - bh * nqg;
    // causal: the pair sweeps 2 qg + 2 key tiles, so the longest sweeps are
    // dispatched first (the key sweeps are longest for the first key blocks
    // already)
    if (CAUSAL) qg = nqg - 1 - qg;
    const int H = a.H, N = a.N, b = bh / H, h = bh - b * H;
    const int qb = 2 * qg + (wave >> 2);  // this wave's query block
    const bool qbvalid = qb < a.nblk;     // (the second block of the last pair may not exist)
    const int qi = qb * kBlk + (wave & 3) * 32 + n;
    const bool valid = qi < N;
    const int64_t rowp = (int64_t)bh * a.N_pad + (qbvalid ? qi : 0);

    v4i qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qf[kk] = qbvalid ? *(const v4i*)(a.q8 + rowp * D + 32 * kk + 16 * hh) : v4i{};
    v8h dof[HK];
#pragma unroll
    for (int kk = 0; kk < HK; ++kk)
        dof[kk] = qbvalid ? *(const v8h*)(a.do16 + rowp * D + 16 * kk + 8 * hh) : v8h{};
    const float sigma = qbvalid ? a.q_scale[bh * a.nblk + qb] * a.lambda : 0.0f;
    const float lse = valid ? a.lse[(int64_t)bh * N + qi] : 0.0f;
    const float Di = qbvalid ? a.Dq[rowp] : 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) settle(qf[kk]);
#pragma unroll
    for (int kk = 0; kk < HK; ++kk) settle(dof[kk]);
    settle(sigma);
    settle(lse);
    settle(Di);

    int koff[KMAXP], voff[VMAXP], toff[TMAXP];
#pragma unroll
    for (int j = 0; j < KMAXP; ++j) koff[j] = slot_src<D, R8>(64 * (wave + NW * j) + lane);
#pragma unroll
    for (int j = 0; j < VMAXP; ++j) voff[j] = slot_src<2 * D, R16>(64 * (wave + NW * j) + lane);
#pragma unroll
    for (int j = 0; j < TMAXP; ++j) toff[j] = slot_src<kBc, kKstr>(64 * (wave + NW * j) + lane);
    const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint8_t* kg = (const uint8_t*)a.k8 + (int64_t)bh * a.N_pad * D;
    const uint8_t* vg = (const uint8_t*)a.v16 + (int64_t)bh * a.N_pad * D * 2;
    const uint8_t* tg = (const uint8_t*)a.kT8 + (int64_t)bh * a.nblk * D * kBc;
    auto load = [&](int t) {
        const uint32_t l = lbase + (t & 1) * SLOT;
        tile_to_lds<KP, KMAXP, NW>(kg + (int64_t)t * kBc * D, l, wv, koff);
        tile_to_lds<VP, VMAXP, NW>(vg + (int64_t)t * kBc * D * 2, l + K8B, wv, voff);
        tile_to_lds<TP, TMAXP, NW>(tg + (int64_t)t * D * kBc, l + K8B + V16B, wv, toff);
    };

    v16f dq[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dq[cb] = v16f{};
    // dP^T's accumulation starts at -D_i, so the chain yields dP - D directly
    v16f negD;
#pragma unroll
    for (int r = 0; r < 16; ++r) negD[r] = -Di;
    const int ntiles = CAUSAL ? min(2 * qg + 2, a.nblk) : a.nblk;
    const float* ksrow = a.k_scale + bh * a.nblk;
    float ks_next = ksrow[0];
    load(0);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        // tile t's K scale (loaded one tile earlier; taken before this tile's
        // copies are issued, so its wait does not cover them)
        float ks = ks_next;
        asm volatile("" : "+v"(ks));
        if (t + 1 < ntiles) {
            ks_next = ksrow[t + 1];
            load(t + 1);
        }
        const uint8_t* kbuf = smem + (t & 1) * SLOT;
        const uint8_t* vbuf = kbuf + K8B;
        const uint8_t* tbuf = vbuf + V16B;
        const float c = sigma * ks;
        const int key_t = t * kBc;
        float ds[4][16];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            // (the barrier keeps the next block's operand reads from being
            // hoisted above this block's work, which would hold them all)
            __builtin_amdgcn_sched_barrier(0);
            v4i ka[KK];
            const uint8_t* krow = kbuf + (32 * k4 + n) * R8 + 16 * hh;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) ka[kk] = *(const v4i*)(krow + 32 * kk);
            const uint8_t* vrow = vbuf + (32 * k4 + n) * R16 + 16 * hh;
            v16i Sk = v16i{};
            v16f dPk = negD;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                v8h va[HK / 2];
#pragma unroll
                for (int kk = 0; kk < HK / 2; ++kk)
                    va[kk] = *(const v8h*)(vrow + 32 * ((HK / 2) * half + kk));
#pragma unroll
                for (int kk = 0; kk < HK / 2; ++kk) {
                    const int ks8 = (KK / 2) * half + kk;  // S takes KK steps over both halves
                    if (kk < KK / 2)
                        Sk = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[ks8], qf[ks8], Sk, 0, 0, 0);
                    dPk = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[kk], dof[(HK / 2) * half + kk], dPk,
                                                                 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)Sk[r], c, -lse));
                ds[k4][r] = p * dPk[r];
            }
        }
        // P^T and dS^T of masked entries (key >= N, causal key > query) to 0;
        // padding queries give dS = 0 by themselves (their dO, D and codes are 0)
        const bool needmask = key_t + kBc > N || (CAUSAL && t >= qb);
        if (needmask) {
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key_t + 32 * k4 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const bool ok = key < N && (!CAUSAL || key <= qi);
                    ds[k4][r] = ok ? ds[k4][r] : 0.0f;
                }
        }
        float amax = 0.0f;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
            for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(ds[k4][r]));
        float s_ds, inv;
        tile_scale(amax, red, wave, lane, s_ds, inv, wave & ~3);
        v4i dsb[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) dsb[k4] = pack_i8(ds[k4], inv);
        // dQ^T (channels x queries) += K8^T dS8^T for this tile, scaled
        const float fq = (s_ds * ks) * a.sm_scale;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            v4i ta[4];
            const uint8_t* trow = tbuf + (32 * cb + n) * kKstr + 16 * hh;
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) ta[k4] = *(const v4i*)(trow + 32 * k4);
            v16i qacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(ta[0], dsb[0], v16i{}, 0, 0, 0);
#pragma unroll
            for (int k4 = 1; k4 < 4; ++k4)
                qacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(ta[k4], dsb[k4], qacc, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 16; ++e) dq[cb][e] = __builtin_fmaf((float)qacc[e], fq, dq[cb][e]);
        }
        wait_vmem();
        __syncthreads();
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) consume(dq[cb]);
    if (!valid) return;
    store_f32_row<D>(a.dq, row_offset(a.layout, b, h, qi, H, N, D), dq, hh);
}

// ------------------------------------------------------------- dK / dV sweep
// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order).
template <int N>
__device__ inline void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Copy pieces wave w issues for a tile of P pieces (piece J = w + 4 j).
constexpr int pieces_of(int P, int w, int nw = 4) { return P > w ? (P - w + nw - 1) / nw : 0; }

// wait_vm with this wave's own count (w uniform)
template <int N0, int N1, int N2, int N3>
__device__ inline void wait_vm_wave(int w) {
    if (w == 0) wait_vm<N0>();
    else if (w == 1) wait_vm<N1>();
    else if (w == 2) wait_vm<N2>();
    else wait_vm<N3>();
}

// The vector-memory loads wave w of NW issues for tiles of P1, P2 and P3
// pieces (piece J = w + NW j): wait until at most that many are in flight.
template <int NW, int P1, int P2, int P3>
__device__ inline void wait_own_pieces(int w) {
#define SAGE_WAIT_W(W)                                                                   \
    if (w == W) {                                                                        \
        wait_vm<pieces_of(P1, W, NW) + pieces_of(P2, W, NW) + pieces_of(P3, W, NW)>(); \
        return;                                                                          \
    }
    SAGE_WAIT_W(0)
    SAGE_WAIT_W(1)
    SAGE_WAIT_W(2)
    SAGE_WAIT_W(3)
    if constexpr (NW > 4) {
        SAGE_WAIT_W(4)
        SAGE_WAIT_W(5)
        SAGE_WAIT_W(6)
        SAGE_WAIT_W(7)
    }
#undef SAGE_WAIT_W
}

// The key sweeps, one per sum: kDV (the dV sum: S, P and dO8^T P~) and kDK
// (the dK sum: S, dP, dS and Q8^T dS8).  Workgroup = 4 waves x 32 keys = one
// key block (kDV, two workgroups per CU) or 8 waves = two key blocks sharing
// each query tile (kDK, one per CU); either way two waves per SIMD.  Query
// tiles swept in ascending order.  LDS: slot A, double-buffered: Q codes
// [128 queries][BwdRow::I8], dO fp16 [128][BwdRow::F16] (kDK) and the tile's
// record (lse, D, q_scale, s_do); slot B, single: dO FP8 transposed [D][kKstr]
// (kDV) or Q codes transposed [D][kKstr] (kDK).  A(t + 1) is copied while
// tile t computes; B(t + 1) after tile t's product, awaited only before tile
// t + 1's.  Every vector-memory load of the sweep is a tile copy, so the
// waits count them.  Two sweeps instead of one joint one (which kept dK, dV
// and the tile's S, dP and dS: 400-500 registers, one wave per SIMD and
// moves out of the accumulation registers) cost one more S product and one
// more exp2 per score and run 1.5x faster.
enum { kDV = 1, kDK = 2 };

template <int MODE>
constexpr int dkdv_waves() { return MODE == kDK ? 8 : 4; }

template <int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(64 * dkdv_waves<MODE>(), MODE == kDV ? 2 : 1) void bwd_dkdv_kernel(BwdArgs a) {
    constexpr bool WDV = MODE == kDV, WDK = MODE == kDK;  // which sum this sweep keeps
    constexpr int NW = dkdv_waves<MODE>(), KBW = NW / 4;   // waves, key blocks per workgroup
    constexpr int KK = D / 32, CB = D / 32, HK = D / 16;
    constexpr int R8 = BwdRow<D>::I8, R16 = BwdRow<D>::F16;
    constexpr int Q8B = kBlk * R8, DO16B = WDK ? kBlk * R16 : 0, RECB = kRecFloats * 4;
    constexpr int SLOTA = Q8B + DO16B + RECB;
    constexpr int DO8B = WDV ? D * kKstr : 0, QTB = WDK ? D * kKstr : 0;
    constexpr int QP = Q8B / 1024, HP = DO16B / 1024, LP = RECB / 1024, FP = DO8B / 1024, TP = QTB / 1024;
    constexpr int QMAXP = (QP + NW - 1) / NW, HMAXP = (HP + NW - 1) / NW, LMAXP = (LP + NW - 1) / NW,
                  FMAXP = (FP + NW - 1) / NW, TMAXP = (TP + NW - 1) / NW;
    static_assert(Q8B % 1024 == 0 && DO16B % 1024 == 0 && RECB % 1024 == 0 && DO8B % 1024 == 0,
                  "1 KB copy pieces");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * SLOTA + DO8B + QTB];
    __shared__ float red[NW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, a.total);
    const int nkg = (a.nblk + KBW - 1) / KBW;  // workgroups per head
    const int bh = wg / nkg, kg = wg - bh * nkg;
    const int H = a.H, N = a.N, b = bh / H, h = bh - b * H;
    const int kb = kg * KBW + (wave >> 2);  // this wave's key block
    const bool kbvalid = kb < a.nblk;       // (the second block of the last pair may not exist)
    const int kj = kb * kBc + (wave & 3) * 32 + n;
    const bool kvalid = kj < N;
    const int64_t rowk = (int64_t)bh * a.N_pad + (kbvalid ? kj : 0);

    v4i kf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        kf[kk] = kbvalid ? *(const v4i*)(a.k8 + rowk * D + 32 * kk + 16 * hh) : v4i{};
    v8h vf[WDK ? HK : 1];
    if constexpr (WDK) {
#pragma unroll
        for (int kk = 0; kk < HK; ++kk)
            vf[kk] = kbvalid ? *(const v8h*)(a.v16 + rowk * D + 16 * kk + 8 * hh) : v8h{};
    }
    const float ks = kbvalid ? a.k_scale[bh * a.nblk + kb] : 0.0f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) settle(kf[kk]);
    if constexpr (WDK) {
#pragma unroll
        for (int kk = 0; kk < HK; ++kk) settle(vf[kk]);
    }
    settle(ks);

    int qoff[QMAXP], hoff[HMAXP > 0 ? HMAXP : 1], loff[LMAXP], foff[FMAXP > 0 ? FMAXP : 1],
        toff[TMAXP > 0 ? TMAXP : 1];
#pragma unroll
    for (int j = 0; j < QMAXP; ++j) qoff[j] = slot_src<D, R8>(64 * (wave + NW * j) + lane);
#pragma unroll
    for (int j = 0; j < HMAXP; ++j) hoff[j] = slot_src<2 * D, R16>(64 * (wave + NW * j) + lane);
#pragma unroll
    for (int j = 0; j < LMAXP; ++j) loff[j] = 16 * (64 * (wave + NW * j) + lane);
#pragma unroll
    for (int j = 0; j < FMAXP; ++j) foff[j] = slot_src<kBlk, kKstr>(64 * (wave + NW * j) + lane);
#pragma unroll
    for (int j = 0; j < TMAXP; ++j) toff[j] = slot_src<kBlk, kKstr>(64 * (wave + NW * j) + lane);
    const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint8_t* qg = (const uint8_t*)a.q8 + (int64_t)bh * a.N_pad * D;
    const uint8_t* hg = (const uint8_t*)a.do16 + (int64_t)bh * a.N_pad * D * 2;
    const uint8_t* lg = (const uint8_t*)a.rec + (int64_t)bh * a.nblk * RECB;
    const uint8_t* fg = (const uint8_t*)a.do8 + (int64_t)bh * a.nblk * D * kBlk;
    const uint8_t* tg = (const uint8_t*)a.qT8 + (int64_t)bh * a.nblk * D * kBlk;
    const uint32_t lB = lbase + 2 * SLOTA;
    auto copy_a = [&](int qt) {
        const uint32_t l = lbase + (qt & 1) * SLOTA;
        tile_to_lds<QP, QMAXP, NW>(qg + (int64_t)qt * kBlk * D, l, wv, qoff);
        tile_to_lds<HP, HMAXP, NW>(hg + (int64_t)qt * kBlk * D * 2, l + Q8B, wv, hoff);
        tile_to_lds<LP, LMAXP, NW>(lg + (int64_t)qt * RECB, l + Q8B + DO16B, wv, loff);
    };
    auto copy_b = [&](int qt) {
        tile_to_lds<FP, FMAXP, NW>(fg + (int64_t)qt * D * kBlk, lB, wv, foff);
        tile_to_lds<TP, TMAXP, NW>(tg + (int64_t)qt * D * kBlk, lB + DO8B, wv, toff);
    };

    v16f dk[WDK ? CB : 1], dv[WDV ? CB : 1];
    if constexpr (WDK) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) dk[cb] = v16f{};
    }
    if constexpr (WDV) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) dv[cb] = v16f{};
    }
    const int t0 = CAUSAL ? kg * KBW : 0;  // the first key block's diagonal tile
    copy_a(t0);
    copy_b(t0);
    for (int qt = t0; qt < a.nblk; ++qt) {
        // A(qt) complete (only B(qt) may still be in flight), for every wave
        wait_own_pieces<NW, FP, TP, 0>(wv);
        __syncthreads();
        const bool more = qt + 1 < a.nblk;
        if (more) copy_a(qt + 1);
        const uint8_t* qbuf = smem + (qt & 1) * SLOTA;
        const uint8_t* hbuf = qbuf + Q8B;
        const float* recL = (const float*)(hbuf + DO16B);
        const uint8_t* fbuf = smem + 2 * SLOTA;
        const uint8_t* tbuf = fbuf + DO8B;
        const float qsc = recL[2 * kBlk], sdo = recL[2 * kBlk + 1];
        const float c = (qsc * a.lambda) * ks;
        // (causal: a tile before this wave's block, possible for the second
        // block of a pair, is masked whole)
        const bool needmask = kb * kBc + kBc > N || (CAUSAL && qt <= kb);
        float ds[WDK ? 4 : 1][16];
        v8i P8[2];
        float amax = 0.0f;
        if constexpr (MODE == kDK) {
            // dK alone: S, dP, P and dS one 32-query block at a time, so only
            // one block's scores and products are live beside the tile's dS
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                // (the barrier keeps the next block's operand reads from being
                // hoisted above this block's work, which would hold them all)
                __builtin_amdgcn_sched_barrier(0);
                v4i qa[KK];
                const uint8_t* qrow = qbuf + (32 * q4 + n) * R8 + 16 * hh;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) qa[kk] = *(const v4i*)(qrow + 32 * kk);
                const uint8_t* hrow = hbuf + (32 * q4 + n) * R16 + 16 * hh;
                v16i Sq = v16i{};
                // dP's accumulation starts at the record's -D of each query
                v16f dPq;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 D4 = *(const float4*)&recL[kBlk + 32 * q4 + 8 * i + 4 * hh];
                    dPq[4 * i] = D4.x;
                    dPq[4 * i + 1] = D4.y;
                    dPq[4 * i + 2] = D4.z;
                    dPq[4 * i + 3] = D4.w;
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    // dP's operands in two halves of the channels
                    v8h ha[HK / 2];
#pragma unroll
                    for (int kk = 0; kk < HK / 2; ++kk)
                        ha[kk] = *(const v8h*)(hrow + 32 * ((HK / 2) * half + kk));
#pragma unroll
                    for (int kk = 0; kk < HK / 2; ++kk) {
                        const int ks8 = (KK / 2) * half + kk;  // S takes KK steps over both halves
                        if (kk < KK / 2)
                            Sq = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[ks8], kf[ks8], Sq, 0, 0, 0);
                        dPq = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha[kk], vf[(HK / 2) * half + kk], dPq,
                                                                     0, 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 L4 = *(const float4*)&recL[32 * q4 + 8 * i + 4 * hh];
                    const float Lv[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 4 * i + j;
                        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf((float)Sq[r], c, -Lv[j]));
                        ds[q4][r] = pv * dPq[r];
                    }
                }
            }
            // masked entries to 0 after the blocks (a branch inside them would
            // let the compiler hoist every block's products above it and keep
            // them all live), then the tile's absmax
            if (needmask) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int q = qt * kBlk + 32 * q4 + 8 * (r >> 2) + 4 * hh + (r & 3);
                        const bool ok = kvalid && (!CAUSAL || kj <= q);
                        ds[q4][r] = ok ? ds[q4][r] : 0.0f;
                    }
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(ds[q4][r]));
        } else {
        // dV alone: S = Q K^T (queries x keys) of the four 32-query blocks,
        // then P, each group of 4 probabilities straight into the FP8 operand
        // at the static scale 448.  Padding queries add nothing to dV (their
        // dO codes are 0); padding keys and, causal, keys after the query are
        // masked on the tiles that hold any.
        v16i S[4];
        {
            v4i qa[4][KK];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint8_t* qrow = qbuf + (32 * q4 + n) * R8 + 16 * hh;
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) qa[q4][kk] = *(const v4i*)(qrow + 32 * kk);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) S[q4] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[q4][0], kf[0], v16i{}, 0, 0, 0);
#pragma unroll
            for (int kk = 1; kk < KK; ++kk)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    S[q4] = __builtin_amdgcn_mfma_i32_32x32x32_i8(qa[q4][kk], kf[kk], S[q4], 0, 0, 0);
        }
        // (p of every entry first, the mask of a tile that needs one applied
        // to the block's 16 values after them: one uniform branch per block
        // instead of a divergent one around each exp2)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            float pq[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 L4 = *(const float4*)&recL[32 * q4 + 8 * i + 4 * hh];
                const float Lv[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pq[4 * i + j] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)S[q4][4 * i + j], c, -Lv[j]));
            }
            if (needmask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q = qt * kBlk + 32 * q4 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const bool ok = kvalid && (!CAUSAL || kj <= q);
                    pq[r] = ok ? pq[r] : 0.0f;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(pq[4 * i] * 448.0f, pq[4 * i + 1] * 448.0f, 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(pq[4 * i + 2] * 448.0f, pq[4 * i + 3] * 448.0f, w, true);
                P8[q4 >> 1][(q4 & 1) * 4 + i] = w;
            }
        }
        }
        // B(qt) complete for this wave (A(qt + 1), issued after it, may still
        // be in flight); the next barrier (in tile_scale for dK) makes it so
        // for all waves
        if (more) {
            wait_own_pieces<NW, QP, HP, LP>(wv);
        } else {
            wait_vmem();
        }
        float s_ds = 0.0f, inv = 0.0f;
        if constexpr (WDK)
            tile_scale(amax, red, wave, lane, s_ds, inv, wave & ~3);
        else
            __syncthreads();
        if constexpr (WDV) {
            // dV^T (channels x keys) += dO8^T P~ over this tile, scaled by s_do / 448
            const float fv = (float)((double)sdo / 448.0);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const uint8_t* frow = fbuf + (32 * cb + n) * kKstr + 64 * hh;
                v16f T = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(*(const v8i*)frow, P8[0], v16f{}, 0, 0,
                                                                         0, 0, 0, 0);
                T = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(*(const v8i*)(frow + 32), P8[1], T, 0, 0, 0,
                                                                    0, 0, 0);
#pragma unroll
                for (int e = 0; e < 16; ++e) dv[cb][e] = __builtin_fmaf(T[e], fv, dv[cb][e]);
            }
        }
        if constexpr (WDK) {
            v4i dsb[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) dsb[q4] = pack_i8(ds[q4], inv);
            // dK^T (channels x keys) += Q8^T dS8 over this tile, scaled
            const float fk = (s_ds * qsc) * a.sm_scale;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const uint8_t* trow = tbuf + (32 * cb + n) * kKstr + 16 * hh;
                v16i acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(*(const v4i*)trow, dsb[0], v16i{}, 0, 0, 0);
#pragma unroll
                for (int q4 = 1; q4 < 4; ++q4)
                    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(*(const v4i*)(trow + 32 * q4), dsb[q4], acc, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 16; ++e) dk[cb][e] = __builtin_fmaf((float)acc[e], fk, dk[cb][e]);
            }
        }
        // every wave is done with slot B (and this tile's slot A) before
        // B(qt + 1) is copied
        __syncthreads();
        if (more) copy_b(qt + 1);
    }
    if constexpr (WDK) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) consume(dk[cb]);
    }
    if constexpr (WDV) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) consume(dv[cb]);
    }
    if (!kvalid) return;
    const int64_t off = row_offset(a.layout, b, h, kj, H, N, D);
    if constexpr (WDK) store_f32_row<D>(a.dk, off, dk, hh);
    if constexpr (WDV) store_f32_row<D>(a.dv, off, dv, hh);
}

template <int D>
static hipError_t launch_attn_bwd_d(const BwdPrep& pp, const BwdArgs& args, int B, int causal,
                                    hipStream_t s) {
    const int BH = B * args.H;
    hipError_t e;
    {
        void* kargs[] = {(void*)&pp.o, (void*)&pp.dO, (void*)&pp.v, (void*)&args.H, (void*)&args.N,
                         (void*)&args.nblk, (void*)&args.layout, (void*)&args.lse, (void*)&args.q_scale,
                         (void*)&args.Dq, (void*)&args.do16, (void*)&args.v16, (void*)&args.do8,
                         (void*)&args.s_do, (void*)&args.rec};
        if ((e = hipLaunchKernel((const void*)bwd_prep_kernel<D>, dim3(args.nblk, BH),
                                 dim3(kBwdThreads), kargs, 0, s)) != hipSuccess)
            return e;
    }
    {
        void* kargs[] = {(void*)&args.q8, (void*)&args.nblk, (void*)&args.qT8};
        if ((e = hipLaunchKernel((const void*)bwd_t8_kernel<D>, dim3(args.nblk, BH),
                                 dim3(kBwdThreads), kargs, 0, s)) != hipSuccess)
            return e;
    }
    {
        void* kargs[] = {(void*)&args.k8, (void*)&args.nblk, (void*)&args.kT8};
        if ((e = hipLaunchKernel((const void*)bwd_t8_kernel<D>, dim3(args.nblk, BH),
                                 dim3(kBwdThreads), kargs, 0, s)) != hipSuccess)
            return e;
    }
    // dQ sweep: one workgroup per pair of query blocks
    BwdArgs aq = args;
    aq.total = BH * ((args.nblk + 1) / 2);
    void* kq[] = {(void*)&aq};
    const void* fq = causal ? (const void*)bwd_dq_kernel<D, true> : (const void*)bwd_dq_kernel<D, false>;
    if ((e = hipLaunchKernel(fq, dim3(aq.total), dim3(512), kq, 0, s)) != hipSuccess) return e;
    // dV sweep: one workgroup per key block (or pair of them with 8 waves)
    BwdArgs av = args;
    constexpr int kbw_v = dkdv_waves<kDV>() / 4;
    av.total = BH * ((args.nblk + kbw_v - 1) / kbw_v);
    void* kv[] = {(void*)&av};
    const void* fv = causal ? (const void*)bwd_dkdv_kernel<D, true, kDV>
                            : (const void*)bwd_dkdv_kernel<D, false, kDV>;
    if ((e = hipLaunchKernel(fv, dim3(av.total), dim3(64 * dkdv_waves<kDV>()), kv, 0, s)) !=
        hipSuccess)
        return e;
    // dK sweep: one workgroup per pair of key blocks
    BwdArgs ak = args;
    ak.total = BH * ((args.nblk + 1) / 2);
    void* kk[] = {(void*)&ak};
    const void* fk = causal ? (const void*)bwd_dkdv_kernel<D, true, kDK>
                            : (const void*)bwd_dkdv_kernel<D, false, kDK>;
    return hipLaunchKernel(fk, dim3(ak.total), dim3(64 * dkdv_waves<kDK>()), kk, 0, s);
}

hipError_t launch_attn_bwd(const BwdPrep& pp, const BwdArgs& args, int B, int d, int causal,
                           hipStream_t s) {
    if (d == 128) return launch_attn_bwd_d<128>(pp, args, B, causal, s);
    if (d == 64) return launch_attn_bwd_d<64>(pp, args, B, causal, s);
    return hipErrorInvalidValue;
}

}  // namespace sage
