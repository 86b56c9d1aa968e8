/*
 * sage_oracle_bwd.c -- TEST INFRASTRUCTURE ONLY (part of the CPU oracle).
 *
 * The backward pass of the 8-bit trainable attention: reportify.cn
 * SageAttention tag page, SageAttention3 summary, bullet 8比特训练 -- per-block
 * INT8 Q/K/V, per-token quantization of P with no quantization overhead, and in
 * the backward pass dO V^T kept in FP16 while the other four products are
 * quantized.  Everything below the level of those three statements is a
 * reading (the plainest one the forward already fixes):
 *
 *   - the forward is the library's forward (INT8 Q K^T with K smoothed, FP8
 *     P V, exp2 online softmax); it also returns, per query,
 *     lse2 = mu + log2(l) with mu = fp32(m' - log2 448) and l its row sum, so
 *     that 2^(S c - lse2) is the softmax probability in the exp2 domain;
 *   - the five backward products, per tile pair (query block of 128 rows x
 *     key block of 128 keys), in fp32 unless quantized:
 *       S   = q8 . k8 (int32, exact): the forward's codes, K smoothed;
 *       P   = exp2(fma(S, c, -lse2_i)),  c = fp32(fp32(q_scale * lambda) * k_scale);
 *       dP  = fp32(sum_c f16(dO_ic) f16(V_jc))   -- the FP16 product (exact sum,
 *             rounded once);
 *       D_i = fp32(sum_c fp32(dO_ic) fp32(O_ic))  (exact sum, rounded once);
 *       dS  = fp32(P * fp32(dP - D_i));
 *       dV_j += fp32(T * f_v),  T = sum_i dec(P~_ij) dec(dO8_ic) (fp32, ascending i),
 *             P~ = e4m3(fp32(P * 448)) -- the forward's static per-token scale,
 *             dO8 = e4m3 of dO per block of 128 rows (absmax / 448 scale, as V in
 *             the forward), f_v = fp32(s_do / 448);
 *       dK_j += fp32(fp32(I) * f_k),  I = sum_i dS~_ij q8_ic (int32, exact),
 *             f_k = fp32(fp32(s_ds * q_scale) * sm_scale);
 *       dQ_i += fp32(fp32(I) * f_q),  I = sum_j dS~_ij k8_jc (int32, exact),
 *             f_q = fp32(fp32(s_ds * k_scale) * sm_scale);
 *     dS~ = INT8 of dS per tile pair (absmax / 127 scale s_ds, the forward's
 *     INT8 rule); the tile pairs are accumulated in ascending block order.
 *   - K smoothed in dQ: sum_j dS_ij = 0 exactly (D_i = sum_j P_ij dP_ij), so
 *     the smoothed K gives the same dQ in exact arithmetic and the forward's
 *     K codes serve; only the quantization of dS leaves a residue.
 *   - causal: keys j > i masked (P = 0, dS = 0); tile pairs wholly above the
 *     diagonal are never visited.
 * Pinned against FP64 autograd of softmax attention, the zero row sums of dS,
 * one-hot output gradients (dV = P^T dO picks rows of P), exact doubling
 * under dO -> 2 dO, and the causal corner cases (tests/test_oracle_bwd.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define OR_API __attribute__((visibility("default")))

float or_bf16_to_f32(uint16_t h);
float or_e4m3_to_f32(uint8_t c);
uint8_t or_f32_to_e4m3(float x);
float or_f16_to_f32(uint16_t h);
uint16_t or_f32_to_f16(float x);
float or_lambda(float sm_scale);

#define OR_BLK 128

static int32_t bwd_dot_i8(const int8_t* a, const int8_t* b, int d) {
    int32_t s = 0;
    for (int c = 0; c < d; ++c) s += (int32_t)a[c] * (int32_t)b[c];
    return s;
}

/* Per query: D_i = fp32(sum_c fp32(dO_ic) fp32(O_ic)) (fp64 sum), and dO to
 * FP8 per block of 128 rows: s_do = fp32(a / 448), codes e4m3(fp32(dO * inv))
 * with inv = fp32(448 / a) (a = the block's absmax; a = 0 gives codes 0). */
OR_API void or_bwd_prep(const uint16_t* o, const uint16_t* dO, int N, int d, float* Dq,
                        uint8_t* do8, float* s_do) {
    for (int i = 0; i < N; ++i) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
            acc += (double)or_bf16_to_f32(dO[(int64_t)i * d + c]) * (double)or_bf16_to_f32(o[(int64_t)i * d + c]);
        Dq[i] = (float)acc;
    }
    const int nblk = (N + OR_BLK - 1) / OR_BLK;
    for (int b = 0; b < nblk; ++b) {
        const int r0 = b * OR_BLK, r1 = r0 + OR_BLK < N ? r0 + OR_BLK : N;
        float a = 0.0f;
        for (int i = r0; i < r1; ++i)
            for (int c = 0; c < d; ++c) {
                float v = fabsf(or_bf16_to_f32(dO[(int64_t)i * d + c]));
                if (v > a) a = v;
            }
        const float inv = a > 0.0f ? (float)(448.0 / (double)a) : 0.0f;
        s_do[b] = (float)((double)a / 448.0);
        for (int i = r0; i < r1; ++i)
            for (int c = 0; c < d; ++c)
                do8[(int64_t)i * d + c] = or_f32_to_e4m3(or_bf16_to_f32(dO[(int64_t)i * d + c]) * inv);
    }
}

/* The tile pair (query block qb, key block kb): P and dS [nq][nk] (rows of
 * the query block, keys of the key block), masked entries 0.  Returns 0 when
 * the pair is wholly masked (causal, above the diagonal). */
static int bwd_tile(const int8_t* q8, const float* qs, const int8_t* k8, const float* ks,
                    const float* v16, const float* do16, const float* lse2, const float* Dq,
                    int N, int d, int causal, float lambda, int qb, int kb, float* P, float* dS,
                    int* nq_out, int* nk_out) {
    const int i0 = qb * OR_BLK, i1 = i0 + OR_BLK < N ? i0 + OR_BLK : N;
    const int j0 = kb * OR_BLK, j1 = j0 + OR_BLK < N ? j0 + OR_BLK : N;
    const int nq = i1 - i0, nk = j1 - j0;
    *nq_out = nq;
    *nk_out = nk;
    if (causal && j0 > i1 - 1) return 0;
    const float c = (qs[qb] * lambda) * ks[kb];
    for (int i = 0; i < nq; ++i) {
        const int gi = i0 + i;
        for (int j = 0; j < nk; ++j) {
            const int gj = j0 + j;
            float p = 0.0f, ds = 0.0f;
            if (!(causal && gj > gi)) {
                const int32_t S = bwd_dot_i8(q8 + (int64_t)gi * d, k8 + (int64_t)gj * d, d);
                p = exp2f(fmaf((float)S, c, -lse2[gi]));
                double acc = 0.0;
                for (int cc = 0; cc < d; ++cc)
                    acc += (double)do16[(int64_t)gi * d + cc] * (double)v16[(int64_t)gj * d + cc];
                const float dp = (float)acc;
                ds = p * (dp - Dq[gi]);
            }
            P[i * nk + j] = p;
            dS[i * nk + j] = ds;
        }
    }
    return 1;
}

/* INT8 of a tile (the forward's rule): scale = fp32(a / 127), codes
 * rne(fp32(x * fp32(127 / a))), a = absmax over the tile. */
static float bwd_quant_tile(const float* x, int n, int8_t* out) {
    float a = 0.0f;
    for (int i = 0; i < n; ++i) {
        const float v = fabsf(x[i]);
        if (v > a) a = v;
    }
    const float inv = a > 0.0f ? (float)(127.0 / (double)a) : 0.0f;
    for (int i = 0; i < n; ++i) {
        float q = rintf(x[i] * inv);
        if (q > 127.0f) q = 127.0f;
        if (q < -127.0f) q = -127.0f;
        out[i] = (int8_t)q;
    }
    return (float)((double)a / 127.0);
}

/* f16 rounding of bf16 values (the operands of the FP16 product dO V^T),
 * returned as floats. */
OR_API void or_bf16_to_f16f_n(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_f16_to_f32(or_f32_to_f16(or_bf16_to_f32(in[i])));
}

/* dQ of the rows of query block qb: dq [nq][d] fp32; v16 / do16 the f16
 * roundings of V and dO (or_bf16_to_f16f_n).
 * scratch: 2 * 128 * 128 floats + 128 * 128 bytes. */
OR_API void or_bwd_dq_block(const int8_t* q8, const float* qs, const int8_t* k8, const float* ks,
                            const float* v16, const float* do16, const float* lse2,
                            const float* Dq, int N, int d, int causal, float sm_scale, int qb,
                            float* dq, float* scratch) {
    const float lambda = or_lambda(sm_scale);
    float* P = scratch;
    float* dS = scratch + OR_BLK * OR_BLK;
    int8_t* dS8 = (int8_t*)(scratch + 2 * OR_BLK * OR_BLK);
    const int nblk = (N + OR_BLK - 1) / OR_BLK;
    const int nq0 = (qb * OR_BLK + OR_BLK < N ? OR_BLK : N - qb * OR_BLK);
    for (int i = 0; i < nq0 * d; ++i) dq[i] = 0.0f;
    for (int kb = 0; kb < nblk; ++kb) {
        int nq, nk;
        if (!bwd_tile(q8, qs, k8, ks, v16, do16, lse2, Dq, N, d, causal, lambda, qb, kb, P, dS, &nq, &nk))
            continue;
        const float s_ds = bwd_quant_tile(dS, nq * nk, dS8);
        const float f = (s_ds * ks[kb]) * sm_scale;
        for (int i = 0; i < nq; ++i)
            for (int cc = 0; cc < d; ++cc) {
                int32_t I = 0;
                for (int j = 0; j < nk; ++j)
                    I += (int32_t)dS8[i * nk + j] * (int32_t)k8[(int64_t)(kb * OR_BLK + j) * d + cc];
                dq[i * d + cc] = dq[i * d + cc] + (float)I * f;
            }
    }
}

/* dK and dV of the keys of key block kb: dk, dv [nk][d] fp32.
 * do8 / s_do from or_bwd_prep.  scratch as for or_bwd_dq_block plus 128 * d
 * floats. */
OR_API void or_bwd_dkdv_block(const int8_t* q8, const float* qs, const int8_t* k8, const float* ks,
                              const float* v16, const float* do16, const uint8_t* do8,
                              const float* s_do, const float* lse2, const float* Dq, int N, int d,
                              int causal, float sm_scale, int kb, float* dk, float* dv,
                              float* scratch) {
    const float lambda = or_lambda(sm_scale);
    float* P = scratch;
    float* dS = scratch + OR_BLK * OR_BLK;
    int8_t* dS8 = (int8_t*)(scratch + 2 * OR_BLK * OR_BLK);
    float* T = scratch + 2 * OR_BLK * OR_BLK + OR_BLK * OR_BLK / 4;
    const int nblk = (N + OR_BLK - 1) / OR_BLK;
    const int nk0 = (kb * OR_BLK + OR_BLK < N ? OR_BLK : N - kb * OR_BLK);
    for (int i = 0; i < nk0 * d; ++i) dk[i] = dv[i] = 0.0f;
    for (int qb = 0; qb < nblk; ++qb) {
        int nq, nk;
        if (!bwd_tile(q8, qs, k8, ks, v16, do16, lse2, Dq, N, d, causal, lambda, qb, kb, P, dS, &nq, &nk))
            continue;
        const float s_ds = bwd_quant_tile(dS, nq * nk, dS8);
        const float fk = (s_ds * qs[qb]) * sm_scale;
        const float fv = (float)((double)s_do[qb] / 448.0);
        for (int j = 0; j < nk; ++j) {
            for (int cc = 0; cc < d; ++cc) {
                int32_t I = 0;
                for (int i = 0; i < nq; ++i)
                    I += (int32_t)dS8[i * nk + j] * (int32_t)q8[(int64_t)(qb * OR_BLK + i) * d + cc];
                dk[j * d + cc] = dk[j * d + cc] + (float)I * fk;
            }
            for (int cc = 0; cc < d; ++cc) T[cc] = 0.0f;
            for (int i = 0; i < nq; ++i) {
                const float pq = or_e4m3_to_f32(or_f32_to_e4m3(P[i * nk + j] * 448.0f));
                const uint8_t* orow = do8 + (int64_t)(qb * OR_BLK + i) * d;
                for (int cc = 0; cc < d; ++cc) T[cc] += pq * or_e4m3_to_f32(orow[cc]);
            }
            for (int cc = 0; cc < d; ++cc) dv[j * d + cc] = dv[j * d + cc] + T[cc] * fv;
        }
    }
}

/* P and dS of the tile pair (qb, kb) [nq][nk] (for the tests); returns 0
 * when the pair is wholly masked. */
OR_API int or_bwd_tile_pd(const int8_t* q8, const float* qs, const int8_t* k8, const float* ks,
                          const float* v16, const float* do16, const float* lse2, const float* Dq,
                          int N, int d, int causal, float sm_scale, int qb, int kb, float* P,
                          float* dS) {
    int nq, nk;
    return bwd_tile(q8, qs, k8, ks, v16, do16, lse2, Dq, N, d, causal, or_lambda(sm_scale), qb, kb,
                    P, dS, &nq, &nk);
}

/* FP64 reference gradients of plain softmax attention (no quantization) for
 * one head from the bf16 inputs: out = softmax(q k^T sm) v, and for the
 * upstream gradient dO, dq/dk/dv [N][d] in fp64.  The textbook backward:
 * P = softmax rows, dP = dO v^T, dS = P (dP - rowsum(dO * out)), dq = sm dS k,
 * dk = sm dS^T q, dv = P^T dO.  scratch: 2 N doubles. */
OR_API void or_bwd_ref64(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dO, int N, int d, int causal, double sm_scale,
                         double* dq, double* dk, double* dv, double* scratch) {
    double* p = scratch;
    double* dp = scratch + N;
    for (int64_t i = 0; i < (int64_t)N * d; ++i) dq[i] = dk[i] = dv[i] = 0.0;
    double* out = (double*)malloc(sizeof(double) * d);
    for (int i = 0; i < N; ++i) {
        const int n = causal ? i + 1 : N;
        double mx = -INFINITY;
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int c = 0; c < d; ++c)
                s += (double)or_bf16_to_f32(q[(int64_t)i * d + c]) * (double)or_bf16_to_f32(k[(int64_t)j * d + c]);
            p[j] = s * sm_scale;
            if (p[j] > mx) mx = p[j];
        }
        double sum = 0.0;
        for (int j = 0; j < n; ++j) {
            p[j] = exp(p[j] - mx);
            sum += p[j];
        }
        for (int c = 0; c < d; ++c) out[c] = 0.0;
        for (int j = 0; j < n; ++j) {
            p[j] /= sum;
            for (int c = 0; c < d; ++c) out[c] += p[j] * (double)or_bf16_to_f32(v[(int64_t)j * d + c]);
        }
        double Di = 0.0;
        for (int c = 0; c < d; ++c) Di += (double)or_bf16_to_f32(dO[(int64_t)i * d + c]) * out[c];
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int c = 0; c < d; ++c)
                s += (double)or_bf16_to_f32(dO[(int64_t)i * d + c]) * (double)or_bf16_to_f32(v[(int64_t)j * d + c]);
            dp[j] = p[j] * (s - Di);
        }
        for (int j = 0; j < n; ++j)
            for (int c = 0; c < d; ++c) {
                dq[(int64_t)i * d + c] += sm_scale * dp[j] * (double)or_bf16_to_f32(k[(int64_t)j * d + c]);
                dk[(int64_t)j * d + c] += sm_scale * dp[j] * (double)or_bf16_to_f32(q[(int64_t)i * d + c]);
                dv[(int64_t)j * d + c] += p[j] * (double)or_bf16_to_f32(dO[(int64_t)i * d + c]);
            }
    }
    free(out);
}
