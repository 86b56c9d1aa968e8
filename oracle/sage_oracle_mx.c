/*
 * sage_oracle_mx.c -- TEST INFRASTRUCTURE ONLY (part of the CPU oracle).
 *
 * The microscaled variant of the attention: Q, K, P and V in an MX format
 * (OCP Microscaling: small floating-point elements, one power-of-two E8M0
 * scale per block of 32 along the reduction), Q K^T and P V on those
 * operands, the online softmax in FP32 between them.  Source: reportify.cn
 * SageAttention tag page, the SageAttention3 summary, bullet FP4量化创新 --
 * microscaling FP4 attention, with MXFP4 named next to NVFP4 and rated less
 * accurate (NVFP4's FP8 block scales are not a format the target's matrix
 * cores take; MX formats are).  Elements (fmt): 4 = E2M1 (MXFP4), 6 = E2M3
 * (MXFP6, the same matrix-core rate on the target, 3 mantissa bits).
 * Readings:
 *   - E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; E2M3 magnitudes m/8
 *     (m < 8) and 2^(e-1) (1 + m/8) for e = 1..3, up to 7.5.  Conversion
 *     rounds to nearest with ties to the even code and saturates at the
 *     largest magnitude; the sign is kept (a negative value that rounds to
 *     zero gives -0); NaN -> +0.
 *   - block scale (OCP MX rule): e = floor(log2(amax)) - 2 (2 = the largest
 *     element exponent of both formats), at most 127; elements
 *     elem(x / 2^e) (an exact division); the E8M0 byte is e + 127.  A block
 *     whose amax is below 2^-100 (zero included) is stored as zeros with
 *     byte 0 (2^-127): no value that small carries weight here, and the
 *     scale stays a normal fp32 power of two.  Values in (max, 8) 2^e
 *     saturate, as the rule implies.
 *   - blocks: Q and K per token and 32 consecutive channels (K smoothed
 *     first, k' = fp32(K - mean)); V per channel and 32 consecutive keys
 *     (aligned to 32); P per query and 32 consecutive keys of a key tile.
 *   - S_j = the exact value of sum_b 2^(eq_b + ek_b) sum_{c in b} q_c k_c,
 *     rounded once to fp32 (every partial product and sum is exact).
 *   - softmax in the exp2 domain as in the INT8 path with c = lambda and no
 *     static P scale (P's scale is per block):  m_t = max_j RD(S_j lambda)
 *     (the product rounded toward -infinity), m' = max(m, m_t),
 *     alpha = exp2(fp32(m - m')) (0 at start), mu = m',
 *     p_j = exp2(fma(S_j, lambda, -mu)), l = fp32(alpha l) + sum p_j
 *     (unquantized p, ascending j).  The subtracted maximum cancels in the
 *     exact result; rounding it down makes the largest element's exponent
 *     argument >= 0, so its p is at least 1 (at most one ulp above) and the
 *     scale of its P block is 2^-2 whichever way an exp2 rounds just
 *     below 1; rounded to nearest, that block's scale would depend on the
 *     last bit of exp2 (p = 1 - 2^-24 gives exponent -3 and saturates the
 *     element to 0.9375).
 *   - P: per block of 32 keys, amax = max p_j, codes elem(p_j / 2^e) as above.
 *   - P V in two levels as in the INT8 path: T = fp32 sum over the tile's
 *     keys (ascending) of dec(p~) dec(v~), O = fp32(fp32(alpha O) + T);
 *     out = fp32(O / l) (the V scales live in dec(v~)); a row with l = 0
 *     gives 0.
 * Pinned: the codecs by round trips, monotone code order, the formats'
 * extreme values, ties between every pair of neighbours and saturation; the
 * block rule's invariants (the absmax element's code, the half-step error
 * bound, the exponent against frexp); S against exact rational arithmetic;
 * a single tile against FP64 attention over the dequantized operands; a
 * tile-by-tile non-online recomputation; the FP64 attention cosine of the
 * whole path (MXFP6 close to the INT8 path, MXFP4 far below it).
 */
#include <math.h>
#include <stdint.h>

#define OR_API __attribute__((visibility("default")))

float or_bf16_to_f32(uint16_t h);
float or_lambda(float sm_scale);

/* Magnitude of code c (sign bit excluded) of element format fmt. */
static float or_mx_mag(int fmt, int c) {
    if (fmt == 4) {
        static const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
        return kE2M1[c & 7];
    }
    int e = (c >> 3) & 3, m = c & 7;
    return e == 0 ? m / 8.0f : ldexpf(1.0f + m / 8.0f, e - 1);
}
static int or_mx_signbit(int fmt) { return fmt == 4 ? 8 : 32; }

OR_API float or_mx_to_f32(int fmt, uint8_t c) {
    float v = or_mx_mag(fmt, c & (or_mx_signbit(fmt) - 1));
    return (c & or_mx_signbit(fmt)) ? -v : v;
}

/* Nearest magnitude, ties to the code with an even mantissa bit (even code
 * number), saturating at the largest magnitude. */
OR_API uint8_t or_f32_to_mx(int fmt, float x) {
    if (isnan(x)) return 0;
    const int ncode = or_mx_signbit(fmt);
    uint8_t sign = signbit(x) ? (uint8_t)ncode : 0;
    float a = fabsf(x);
    if (a >= or_mx_mag(fmt, ncode - 1)) return sign | (uint8_t)(ncode - 1);
    int best = 0;
    for (int c = 1; c < ncode; ++c) {
        float dc = fabsf(a - or_mx_mag(fmt, c)), db = fabsf(a - or_mx_mag(fmt, best));
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return sign | (uint8_t)best;
}

/* Shared exponent of a block with absolute maximum amax (the OCP MX rule;
 * -127 for a block below 2^-100, whose codes are then all 0). */
static int or_mx_exponent(float amax) {
    if (!(amax >= 0x1p-100f)) return -127;
    int k;
    frexpf(amax, &k);        /* amax = f 2^k, f in [0.5, 1): floor(log2 amax) = k - 1 */
    int e = (k - 1) - 2;
    if (e > 127) e = 127;
    return e;
}

/* One block of n <= 32 values (stride apart): codes and the E8M0 byte. */
static uint8_t or_mx_block(int fmt, const float* x, int n, int stride, uint8_t* codes,
                           int cstride) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(x[(int64_t)i * stride]);
        if (a > amax) amax = a;
    }
    int e = or_mx_exponent(amax);
    for (int i = 0; i < n; ++i)
        codes[(int64_t)i * cstride] =
            e == -127 ? 0 : or_f32_to_mx(fmt, (float)ldexp((double)x[(int64_t)i * stride], -e));
    return (uint8_t)(e + 127);
}

static float or_mx_dec(int fmt, uint8_t code, uint8_t ebyte) {
    return (float)ldexp((double)or_mx_to_f32(fmt, code), (int)ebyte - 127);
}

/* Q (mean == NULL) or K (k' = fp32(K - mean)) of one head: codes [N][d]
 * (one element code per byte), ebytes [N][d/32]. */
OR_API void or_mx_quant_rows(int fmt, const uint16_t* x, const float* mean, int N, int d,
                             uint8_t* codes, uint8_t* ebytes, float* tmp /* d */) {
    for (int j = 0; j < N; ++j) {
        for (int c = 0; c < d; ++c) {
            float v = or_bf16_to_f32(x[(int64_t)j * d + c]);
            tmp[c] = mean ? v - mean[c] : v;
        }
        for (int b = 0; b < d / 32; ++b)
            ebytes[(int64_t)j * (d / 32) + b] =
                or_mx_block(fmt, tmp + 32 * b, 32, 1, codes + (int64_t)j * d + 32 * b, 1);
    }
}

/* V of one head: per channel and 32 consecutive keys; codes [N][d],
 * ebytes [ceil(N/32)][d]. */
OR_API void or_mx_quant_v(int fmt, const uint16_t* v, int N, int d, uint8_t* codes,
                          uint8_t* ebytes, float* tmp /* 32 */) {
    int nb = (N + 31) / 32;
    for (int b = 0; b < nb; ++b) {
        int j0 = 32 * b, n = (N - j0 < 32) ? N - j0 : 32;
        for (int c = 0; c < d; ++c) {
            for (int i = 0; i < n; ++i) tmp[i] = or_bf16_to_f32(v[(int64_t)(j0 + i) * d + c]);
            ebytes[(int64_t)b * d + c] = or_mx_block(fmt, tmp, n, 1, codes + (int64_t)j0 * d + c, d);
        }
    }
}

/* Exact MX dot product of query row i and key row j, rounded once to fp32.
 * Both element formats hold multiples of 1/8: 8x is an integer of magnitude
 * <= 60, a block's sum of 32 products is below 2^17, and the sum of the
 * scaled block sums is exact in fp64 for any realistic exponent spread. */
OR_API float or_mx_dot(int fmt, const uint8_t* qc, const uint8_t* qe, const uint8_t* kc,
                       const uint8_t* ke, int d) {
    double acc = 0.0;
    for (int b = 0; b < d / 32; ++b) {
        int64_t s = 0;
        for (int c = 32 * b; c < 32 * b + 32; ++c)
            s += (int64_t)(8.0f * or_mx_to_f32(fmt, qc[c])) * (int64_t)(8.0f * or_mx_to_f32(fmt, kc[c]));
        acc += ldexp((double)s, (int)qe[b] - 127 + (int)ke[b] - 127 - 6);
    }
    return (float)acc;
}

/* Rows rows[0..nrows) of one head; out [nrows][d]; m_out / l_out optional.
 * scratch: 3*128 + 2*d floats. */
OR_API void or_mx_attn_rows(int fmt, const uint8_t* qc, const uint8_t* qe, const uint8_t* kc,
                            const uint8_t* ke, const uint8_t* vc, const uint8_t* ve, int N, int d,
                            const int32_t* rows, int nrows, int causal, float sm_scale, float* out,
                            float* m_out, float* l_out, float* scratch) {
    const float lambda = or_lambda(sm_scale);
    float* S = scratch;
    float* P = scratch + 128;
    float* Pq = scratch + 256;
    float* T = scratch + 384;
    float* O = T + d;
    const int nq = d / 32;
    for (int r = 0; r < nrows; ++r) {
        const int i = rows[r];
        float m = -INFINITY, l = 0.0f;
        for (int c = 0; c < d; ++c) O[c] = 0.0f;
        for (int j0 = 0; j0 < N; j0 += 128) {
            if (causal && j0 > i) break;
            int j1 = j0 + 128 < N ? j0 + 128 : N;
            if (causal && j1 > i + 1) j1 = i + 1;
            const int n = j1 - j0;
            float mt = -INFINITY;
            for (int j = 0; j < n; ++j) {
                S[j] = or_mx_dot(fmt, qc + (int64_t)i * d, qe + (int64_t)i * nq,
                                 kc + (int64_t)(j0 + j) * d, ke + (int64_t)(j0 + j) * nq, d);
                float s = S[j] * lambda;
                /* round down: the double product of two floats is exact */
                if ((double)s > (double)S[j] * (double)lambda) s = nextafterf(s, -INFINITY);
                if (s > mt) mt = s;
            }
            const float mn = m > mt ? m : mt;
            const float alpha = (m == -INFINITY) ? 0.0f : exp2f(m - mn);
            const float mu = mn;
            float psum = 0.0f;
            for (int j = 0; j < n; ++j) {
                P[j] = exp2f(fmaf(S[j], lambda, -mu));
                psum += P[j];
            }
            l = alpha * l + psum;
            /* P per block of 32 consecutive keys of the tile */
            for (int b0 = 0; b0 < n; b0 += 32) {
                const int nb = (n - b0 < 32) ? n - b0 : 32;
                uint8_t codes[32];
                uint8_t eb = or_mx_block(fmt, P + b0, nb, 1, codes, 1);
                for (int u = 0; u < nb; ++u) Pq[b0 + u] = or_mx_dec(fmt, codes[u], eb);
            }
            for (int c = 0; c < d; ++c) T[c] = 0.0f;
            for (int j = 0; j < n; ++j) {
                const int key = j0 + j;
                const uint8_t* vrow = vc + (int64_t)key * d;
                const uint8_t* verow = ve + (int64_t)(key / 32) * d;
                for (int c = 0; c < d; ++c) T[c] += Pq[j] * or_mx_dec(fmt, vrow[c], verow[c]);
            }
            for (int c = 0; c < d; ++c) O[c] = alpha * O[c] + T[c];
            m = mn;
        }
        for (int c = 0; c < d; ++c) out[(int64_t)r * d + c] = l > 0.0f ? O[c] / l : 0.0f;
        if (m_out) m_out[r] = m;
        if (l_out) l_out[r] = l;
    }
}

/* Array forms of the codec and of the block rule (for the tests). */
OR_API void or_f32_to_mx_n(int fmt, const float* in, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_f32_to_mx(fmt, in[i]);
}
OR_API void or_mx_to_f32_n(int fmt, const uint8_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_mx_to_f32(fmt, in[i]);
}
OR_API void or_mx_blocks_n(int fmt, const float* x, int64_t nblocks, uint8_t* codes,
                           uint8_t* ebytes) {
    for (int64_t b = 0; b < nblocks; ++b)
        ebytes[b] = or_mx_block(fmt, x + 32 * b, 32, 1, codes + 32 * b, 1);
}
