/*
 * sage_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU implementation of SageAttention-style
 * low-bit attention, O = softmax(Q K^T * sm_scale) V, computed the quantized
 * way: K smoothed by its per-head token mean (optionally Q by its per-block
 * token mean, with the mean's share of the scores restored in FP32), Q and K
 * quantized per block of
 * rows to INT8 for an exact integer Q K^T, an exp2 online softmax in FP32 over
 * key tiles, P taken to FP8 e4m3 (or FP16) with a static scale, V taken to
 * FP8 e4m3 with per-channel scales (or FP16), and P V accumulated in two
 * levels (a fresh FP32 sum per key tile, then an FP32 running accumulator).
 *
 * Sources (the pages this follows):
 *   - wxsanhe.com blog post on TurboDiffusion, section 三.1 (混合注意力):
 *     Q K goes to INT8, P V to FP8 or FP16, outlier smoothing and two-level
 *     accumulation recover the precision; usable as a quantized FlashAttention.
 *   - reportify.cn SageAttention tag page, SageAttention3 summary, bullet
 *     8比特训练: per-block INT8 quantization of Q/K/V and per-token
 *     quantization of P "with no quantization overhead".
 *   - txrjy.com repost of the QbitAI TurboDiffusion article, section
 *     四个步骤极限压缩时间: INT8 attention with outlier smoothing.
 *   - hunxia.com article, glossary entry on FlashAttention (tiled attention
 *     that optimises memory access): the online-softmax tile structure.
 * Every step finer than those pages state is a reading; each reading is
 * named where it is used below.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may call this library.  It shares no code, header, table or constant
 * generator with the GPU path.  Build: gcc -O2 -ffp-contract=off
 * -fno-fast-math (no FMA contraction: every fused multiply-add below is an
 * explicit fmaf call).
 *
 * Parity status of each function is stated in its comment.  All functions
 * here are pinned by tests against something other than themselves
 * (library casts, exact integer arithmetic, FP64 attention, closed forms).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OR_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Codecs.                                                                   */
/* ------------------------------------------------------------------------ */

/* bf16 -> fp32: the bf16 pattern is the top half of the fp32 pattern.
 * Pinned against torch's bfloat16 cast (all 65536 codes). */
OR_API float or_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest even.  NaN stays NaN.
 * Pinned against torch's bfloat16 cast. */
OR_API uint16_t or_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* OCP FP8 e4m3fn decode: sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * no infinities; 0x7f / 0xff are NaN; largest finite 448; subnormals are
 * m * 2^-9.  Pinned against torch.float8_e4m3fn for all 256 codes. */
OR_API float or_e4m3_to_f32(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
    float v;
    if (e == 0xf && m == 7) return NAN;
    if (e == 0) v = ldexpf((float)m, -9);
    else v = ldexpf((float)(8 + m), e - 10);
    return s ? -v : v;
}

/* fp32 -> OCP FP8 e4m3fn, round to nearest even, saturating: every finite
 * value of magnitude >= 448 maps to +-448 (values in [448, 464] are also what
 * plain round-to-nearest-even gives); NaN maps to 0x7f.
 * Reading: the pages name FP8 without a rounding rule; round-to-nearest-even
 * with saturation is the plainest.  Pinned against torch.float8_e4m3fn on a
 * dense sweep of [0, 464]. */
OR_API uint8_t or_f32_to_e4m3(float x) {
    if (isnan(x)) return 0x7f;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    float a = fabsf(x);
    if (a >= 448.0f) return sign | 0x7e;
    if (a < 0x1p-6f) {                         /* subnormal range: step 2^-9 */
        float q = rintf(a * 0x1p9f);           /* exact scaling, RNE */
        return sign | (uint8_t)q;              /* q == 8 is the smallest normal */
    }
    int k;
    frexpf(a, &k);                             /* a in [2^(k-1), 2^k) */
    int E = k - 1;
    float t = ldexpf(a, 3 - E);                /* in [8, 16), exact */
    int q = (int)rintf(t);
    if (q == 16) { q = 8; E += 1; }
    if (E + 7 > 15 || (E + 7 == 15 && q - 8 == 7)) return sign | 0x7e;
    return sign | (uint8_t)(((E + 7) << 3) | (q - 8));
}

/* IEEE binary16 decode.  Pinned against numpy float16. */
OR_API float or_f16_to_f32(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    float v;
    if (e == 0x1f) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexpf((float)m, -24);
    else v = ldexpf((float)(1024 + m), e - 25);
    return s ? -v : v;
}

/* fp32 -> IEEE binary16, round to nearest even, saturating at +-65504
 * (reading: finite inputs never become infinities).  NaN -> 0x7e00.
 * Pinned against numpy float16 inside the finite range. */
OR_API uint16_t or_f32_to_f16(float x) {
    if (isnan(x)) return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    float a = fabsf(x);
    if (a >= 65504.0f) return sign | 0x7bff;
    if (a < 0x1p-14f) {
        float q = rintf(a * 0x1p24f);
        return sign | (uint16_t)q;
    }
    int k;
    frexpf(a, &k);
    int E = k - 1;
    float t = ldexpf(a, 10 - E);               /* in [1024, 2048) */
    int q = (int)rintf(t);
    if (q == 2048) { q = 1024; E += 1; }
    if (E + 15 >= 31) return sign | 0x7bff;
    return sign | (uint16_t)(((E + 15) << 10) | (q - 1024));
}

/* ------------------------------------------------------------------------ */
/* Smoothing of K: the per-head token mean of each channel.                  */
/* ------------------------------------------------------------------------ */

/* One K value on the fixed-point grid 2^-30: trunc(x * 2^30), saturated at
 * +-2^62, NaN -> 0.
 * Reading: the pages name only "outlier smoothing"; the per-head token mean
 * is the plainest smoothing vector.  The sum is taken exactly on a 2^-30
 * grid (wrapping int64) so that it has one value whatever the summation
 * order; the mean then differs from the real mean by under 2^-30. */
OR_API int64_t or_fix30(float x) {
    if (isnan(x)) return 0;
    double t = (double)x * 1073741824.0;       /* exact: power-of-two scaling */
    if (t >= 4611686018427387904.0) return INT64_C(4611686018427387904);
    if (t <= -4611686018427387904.0) return -INT64_C(4611686018427387904);
    return (int64_t)t;                          /* C conversion truncates */
}

/* mu[c] = fp32( fp64(I_c) / (fp64(N) * 2^30) ), I_c = sum_j fix30(K[j][c])
 * taken modulo 2^64 (two's complement).  k is one head, [N][d] bf16.
 * Pinned: exact Python-integer evaluation on small inputs, numpy float64
 * mean to within one fp32 ulp + 2^-30, constant columns. */
OR_API void or_k_mean(const uint16_t* k, int N, int d, float* mean) {
    for (int c = 0; c < d; ++c) {
        uint64_t acc = 0;
        for (int j = 0; j < N; ++j)
            acc += (uint64_t)or_fix30(or_bf16_to_f32(k[(int64_t)j * d + c]));
        int64_t I = (int64_t)acc;
        mean[c] = (float)((double)I / ((double)N * 1073741824.0));
    }
}

/* ------------------------------------------------------------------------ */
/* Per-block INT8 quantization (reportify SageAttention3 summary, 8比特训练: */
/* per-block INT8 of Q and K; wxsanhe §三.1: Q K in INT8).                   */
/* ------------------------------------------------------------------------ */

/* x: rows x d fp32 values of one block.  a = max |x|;
 * scale = fp32(fp64(a) / 127); inv = a > 0 ? fp32(127 / fp64(a)) : 0;
 * code = clamp(rne(fp32(x * inv)), -127, 127).
 * Reading: symmetric range +-127 (-128 unused), absmax scale per block,
 * quotients formed in fp64 and rounded once to fp32 (= the correctly
 * rounded fp32 quotient), round to nearest even.
 * Pinned by hand-written codes on blocks whose scaled values sit exactly on
 * k + 1/2 (ties to even, both signs) and on a block where x * inv and
 * x / scale round to different codes; and by invariants: |code| <= 127, the
 * absmax element maps to +-127, |code * scale - x| <= scale / 2 (1 + 2^-20),
 * sign preserved, zero block. */
OR_API void or_quant_block(const float* x, int rows, int d, int8_t* out, float* scale) {
    float a = 0.0f;
    for (int i = 0; i < rows * d; ++i) {
        float v = fabsf(x[i]);
        if (v > a) a = v;
    }
    float inv = a > 0.0f ? (float)(127.0 / (double)a) : 0.0f;
    *scale = (float)((double)a / 127.0);
    for (int i = 0; i < rows * d; ++i) {
        float q = rintf(x[i] * inv);
        if (q > 127.0f) q = 127.0f;
        if (q < -127.0f) q = -127.0f;
        out[i] = (int8_t)q;
    }
}

/* Q of one head: q [N][d] bf16 -> q8 [N][d], qs [ceil(N/blk)].
 * Blocks are rows [r*blk, min(N, (r+1)*blk)). */
OR_API void or_quant_q(const uint16_t* q, int N, int d, int blk, int8_t* q8, float* qs,
                       float* tmp /* blk*d */) {
    int nb = (N + blk - 1) / blk;
    for (int r = 0; r < nb; ++r) {
        int r0 = r * blk, rows = (N - r0 < blk) ? N - r0 : blk;
        for (int i = 0; i < rows * d; ++i) tmp[i] = or_bf16_to_f32(q[(int64_t)r0 * d + i]);
        or_quant_block(tmp, rows, d, q8 + (int64_t)r0 * d, &qs[r]);
    }
}

/* Q of one head with smoothing: per block r of 128 rows, qmean[r][c] is the
 * block's token mean of channel c, taken exactly as the K mean (or_k_mean over
 * the block's rows); q' = fp32(Q - qmean[r]) (one rounding) is quantized to
 * INT8 per qblk rows (qblk = 128: one scale per block; qblk = 1: one per row).
 * The mean's share of each score comes back through or_q_smooth_bias.
 * Reading: the pages name "outlier smoothing" without saying which operand
 * it applies to; this is the same per-channel mean subtraction as for K, over
 * the query block that shares a scale, with its contribution q̄·k' restored in
 * FP32 so the scores still approximate Q K^T (subtracting a query's mean is
 * not softmax-invariant, unlike the key mean).  Pinned: block means against
 * FP64 numpy, reconstruction codes * scale + mean ~ Q, the FP64 attention
 * cosine on Q-offset inputs with and without it. */
OR_API void or_quant_q_smooth(const uint16_t* q, int N, int d, int qblk, int8_t* q8, float* qs,
                              float* qmean /* [nb][d] */, float* tmp /* 128*d */) {
    int nb = (N + 127) / 128;
    for (int r = 0; r < nb; ++r) {
        int r0 = r * 128, rows = (N - r0 < 128) ? N - r0 : 128;
        float* qm = qmean + (int64_t)r * d;
        or_k_mean(q + (int64_t)r0 * d, rows, d, qm);
        for (int i = 0; i < rows; ++i)
            for (int c = 0; c < d; ++c)
                tmp[i * d + c] = or_bf16_to_f32(q[(int64_t)(r0 + i) * d + c]) - qm[c];
        if (qblk == 1)
            for (int i = 0; i < rows; ++i)
                or_quant_block(tmp + (int64_t)i * d, 1, d, q8 + (int64_t)(r0 + i) * d, &qs[r0 + i]);
        else
            or_quant_block(tmp, rows, d, q8 + (int64_t)r0 * d, &qs[r]);
    }
}

/* K of one head: k' = fp32(K - mu) (one rounding), then per-block INT8 as
 * for Q.  smooth == 0 skips the mean (mu = 0): a switch for the tests that
 * show what smoothing buys; the method always smooths. */
OR_API void or_quant_k(const uint16_t* k, int N, int d, int blk, int smooth, int8_t* k8,
                       float* ks, float* mean, float* tmp /* blk*d */) {
    if (smooth) or_k_mean(k, N, d, mean);
    else for (int c = 0; c < d; ++c) mean[c] = 0.0f;
    int nb = (N + blk - 1) / blk;
    for (int r = 0; r < nb; ++r) {
        int r0 = r * blk, rows = (N - r0 < blk) ? N - r0 : blk;
        for (int i = 0; i < rows; ++i)
            for (int c = 0; c < d; ++c)
                tmp[i * d + c] = or_bf16_to_f32(k[(int64_t)(r0 + i) * d + c]) - mean[c];
        or_quant_block(tmp, rows, d, k8 + (int64_t)r0 * d, &ks[r]);
    }
}

/* V of one head, FP8 path: per channel a_c = max_j |V[j][c]|;
 * v_scale_c = fp32(a_c / 448); inv_c = a_c > 0 ? fp32(448 / a_c) : 0;
 * code = e4m3(fp32(V * inv_c)).   FP16 path: code = f16(V), v_scale = 1.
 * Reading: 448 (the largest e4m3fn value) maps the channel's absmax onto the
 * top of the FP8 range.  v8: uint8 codes (fp8) or uint16 codes (fp16), [N][d]
 * in natural order. */
OR_API void or_quant_v(const uint16_t* v, int N, int d, int pv_fp16, void* vq, float* vs) {
    if (pv_fp16) {
        uint16_t* o = (uint16_t*)vq;
        for (int64_t i = 0; i < (int64_t)N * d; ++i) o[i] = or_f32_to_f16(or_bf16_to_f32(v[i]));
        for (int c = 0; c < d; ++c) vs[c] = 1.0f;
        return;
    }
    uint8_t* o = (uint8_t*)vq;
    for (int c = 0; c < d; ++c) {
        float a = 0.0f;
        for (int j = 0; j < N; ++j) {
            float x = fabsf(or_bf16_to_f32(v[(int64_t)j * d + c]));
            if (x > a) a = x;
        }
        float inv = a > 0.0f ? (float)(448.0 / (double)a) : 0.0f;
        vs[c] = (float)((double)a / 448.0);
        for (int j = 0; j < N; ++j)
            o[(int64_t)j * d + c] = or_f32_to_e4m3(or_bf16_to_f32(v[(int64_t)j * d + c]) * inv);
    }
}

/* ------------------------------------------------------------------------ */
/* Attention over the quantized operands, one query row at a time.           */
/* ------------------------------------------------------------------------ */

/* Integer score of query row qi against key row kj: exact int32 dot product
 * of the INT8 codes (|S| <= 127^2 d < 2^24).  This is what the debug dump of
 * the GPU path must reproduce bit for bit.  Pinned against an int64 matmul. */
static int32_t or_dot_i8(const int8_t* a, const int8_t* b, int d) {
    int32_t s = 0;
    for (int c = 0; c < d; ++c) s += (int32_t)a[c] * (int32_t)b[c];
    return s;
}

OR_API void or_dump_s(const int8_t* q8, const int8_t* k8, int N, int d, int row0, int nrows,
                      int causal, int32_t* s_out /* [nrows][N] */) {
    for (int r = 0; r < nrows; ++r) {
        int i = row0 + r;
        for (int j = 0; j < N; ++j)
            s_out[(int64_t)r * N + j] =
                (causal && j > i) ? 0 : or_dot_i8(q8 + (int64_t)i * d, k8 + (int64_t)j * d, d);
    }
}

/* log2 of the static P scale 448, rounded once to fp32. */
static float or_log2_pscale(void) { return (float)log2(448.0); }

/* sm_scale * log2(e), rounded once to fp32 (the exp2-domain softmax scale). */
OR_API float or_lambda(float sm_scale) { return (float)((double)sm_scale * 1.4426950408889634); }

/* The Q-smoothing correction of one head: for query block r and key j,
 *   bias[r][j] = fp32(acc * lambda),  acc = fma chain over c = 0 .. d-1 of
 *   qmean[r][c] * k'[j][c] starting from 0 (fp32, ascending c),
 *   k'[j][c] = fp32(K[j][c] - kmean[c])  (the smoothed K the quantizer sees).
 * It is the block mean's part q̄·k' of every score of the block, in the exp2
 * units of the attention (lambda = sm_scale log2 e).  Pinned against FP64
 * numpy within the fp32 dot-product error bound; zero means give 0. */
OR_API void or_q_smooth_bias(const float* qmean, const uint16_t* k, const float* kmean, int N,
                             int d, float sm_scale, int r0, int r1,
                             float* bias /* [r1 - r0][N]: blocks r0 .. r1-1 */) {
    float lambda = or_lambda(sm_scale);
    for (int r = r0; r < r1; ++r)
        for (int j = 0; j < N; ++j) {
            float acc = 0.0f;
            for (int c = 0; c < d; ++c) {
                float kp = or_bf16_to_f32(k[(int64_t)j * d + c]) - kmean[c];
                acc = fmaf(qmean[(int64_t)r * d + c], kp, acc);
            }
            bias[(int64_t)(r - r0) * N + j] = acc * lambda;
        }
}

/* One query row i of one head.  Online softmax in the exp2 domain over key
 * tiles [t*bc, (t+1)*bc) in ascending t; with causal, keys j > i are masked
 * and tiles wholly above the diagonal are never visited.
 *
 * Per tile (all arithmetic fp32, each operation rounded once):
 *   c     = fp32(sigma * s_k[tile of keys])  with sigma = fp32(s_q * lambda)
 *   m_t   = max_j fp32(S_j * c)              over unmasked keys
 *   m'    = max(m, m_t)
 *   alpha = m == -inf ? 0 : exp2(fp32(m - m'))
 *   mu    = fp32(m' - log2 448)
 *   p_j   = exp2(fma(S_j, c, -mu))           (= 448 * 2^(S_j c - m') up to rounding)
 *   pq_j  = e4m3(p_j)   (FP16 path: f16(p_j))           -- static scale 448
 *   l     = fp32(fp32(alpha * l) + sum_j dec(pq_j))  (sum in ascending j)
 *   lx    = fp32(fp32(alpha * lx) + sum_j p_j)       (the unquantized sum: the
 *           log-sum-exp of the scores, mu + log2 lx, for the backward)
 *   T_c   = sum_j dec(pq_j) * dec(v_jc)      level 1: a fresh fp32 sum per tile
 *   O_c   = fp32(fp32(alpha * O_c) + T_c)    level 2: the running fp32 accumulator
 * Epilogue: out_c = fp32( fp32(O_c * v_scale_c) / l ).
 * With Q smoothing (bias = the row's block row of or_q_smooth_bias), the
 * score carries the block mean's share and the exponent is taken from it:
 *   s_j = fma(S_j, c, bias_j);  m_t = max_j s_j;  p_j = exp2(fp32(s_j - mu))
 * (m', alpha, mu, l and the rest unchanged).
 *
 * Readings: the static P scale is 448 (the e4m3fn maximum: the running max
 * makes every p <= 1, so 448 p fills the FP8 range with no per-token
 * statistics -- the "no quantization overhead" of the reportify summary);
 * the 448 is folded into the exp2 argument through mu; l sums the P values
 * the P V product uses (after their FP8 / FP16 rounding), so that the
 * weights applied to V sum to exactly one (a constant V comes out unchanged);
 * key tiles of bc = 128 keys in ascending order, no split;
 * the two accumulation levels are one key tile and the whole row.
 * qs is indexed by query block of qblk rows: qblk = 128 is the per-block
 * quantization (reportify SageAttention3 summary, bullet 8比特训练), qblk = 1
 * the per-token one, the finest reading of the "thread-level quantization" in
 * the txrjy.com repost of the QbitAI article, section 四个步骤极限压缩时间;
 * ks by key block of kblk keys, and bc == kblk.
 * Block-sparse tile skipping (the sparse half of sparse-linear attention,
 * wxsanhe §三.1 and the pages' point that sparsity stacks on low-bit
 * attention): with a tile mask, key tile t is visited only when
 * tmask[t] != 0 for the query's block of 128 rows; a skipped tile is never
 * seen, exactly as if all its keys were masked.  A row that visits no key has
 * l = 0 and gets the output 0 (reading: an empty softmax contributes nothing).
 * Pinned: FP64 attention (cosine), brute force of the single-tile case,
 * P rows summing to 1 through the final (m, l), a tile-by-tile non-online
 * recomputation, constant keys and peaked rows in closed form; with a tile
 * mask, against FP64 attention over the visited keys only. */
static void or_attn_row(const int8_t* q8, const float* qs, const int8_t* k8, const float* ks,
                        const void* vq, const float* vs, int N, int d, int i, int causal,
                        float lambda, int pv_fp16, int qblk, int kblk, int bc,
                        const uint8_t* tmask, const float* bias, float* out, float* m_out,
                        float* l_out, float* lx_out, int32_t* S, float* T, float* O, float* P) {
    const uint8_t* v8 = (const uint8_t*)vq;
    const uint16_t* v16 = (const uint16_t*)vq;
    const float L = or_log2_pscale();
    const float sigma = qs[i / qblk] * lambda;
    const int8_t* qi = q8 + (int64_t)i * d;
    float m = -INFINITY, l = 0.0f, lx = 0.0f;
    for (int c = 0; c < d; ++c) O[c] = 0.0f;
    int ntiles = (N + bc - 1) / bc;
    for (int t = 0; t < ntiles; ++t) {
        int j0 = t * bc;
        if (causal && j0 > i) break;
        if (tmask && !tmask[t]) continue;
        int j1 = j0 + bc < N ? j0 + bc : N;
        if (causal && j1 > i + 1) j1 = i + 1;
        int n = j1 - j0;
        float c = sigma * ks[j0 / kblk];
        float mt = -INFINITY;
        for (int j = 0; j < n; ++j) {
            S[j] = or_dot_i8(qi, k8 + (int64_t)(j0 + j) * d, d);
            float s = bias ? fmaf((float)S[j], c, bias[j0 + j]) : (float)S[j] * c;
            if (s > mt) mt = s;
        }
        float mn = m > mt ? m : mt;
        float alpha = (m == -INFINITY) ? 0.0f : exp2f(m - mn);
        float mu = mn - L;
        float psum = 0.0f, xsum = 0.0f;
        for (int j = 0; j < n; ++j) {
            float p = bias ? exp2f(fmaf((float)S[j], c, bias[j0 + j]) - mu)
                           : exp2f(fmaf((float)S[j], c, -mu));
            P[j] = pv_fp16 ? or_f16_to_f32(or_f32_to_f16(p)) : or_e4m3_to_f32(or_f32_to_e4m3(p));
            psum += P[j];
            xsum += p;
        }
        l = alpha * l + psum;
        lx = alpha * lx + xsum;
        for (int cc = 0; cc < d; ++cc) T[cc] = 0.0f;
        for (int j = 0; j < n; ++j) {
            int64_t row = (int64_t)(j0 + j) * d;
            for (int cc = 0; cc < d; ++cc) {
                float vv = pv_fp16 ? or_f16_to_f32(v16[row + cc]) : or_e4m3_to_f32(v8[row + cc]);
                T[cc] += P[j] * vv;
            }
        }
        for (int cc = 0; cc < d; ++cc) O[cc] = alpha * O[cc] + T[cc];
        m = mn;
    }
    for (int cc = 0; cc < d; ++cc) out[cc] = l > 0.0f ? (O[cc] * vs[cc]) / l : 0.0f;
    if (m_out) *m_out = m;
    if (l_out) *l_out = l;
    if (lx_out) *lx_out = lx;
}

/* Rows rows[0..nrows) of one head; out [nrows][d]; m_out/l_out optional.
 * tmask: NULL (dense) or the head's tile mask [ceil(N/128)][ntiles] (query
 * block of 128 rows x key tile), nonzero = visit.
 * bias: NULL, or the head's Q-smoothing correction [ceil(N/128)][N] from
 * or_q_smooth_bias (row i uses row i / 128).
 * scratch must hold 4*bc + 3*d floats. */
OR_API void or_attn_rows(const int8_t* q8, const float* qs, const int8_t* k8, const float* ks,
                         const void* vq, const float* vs, int N, int d, const int32_t* rows,
                         int nrows, int causal, float sm_scale, int pv_fp16, int qblk,
                         int kblk, int bc, const uint8_t* tmask, const float* bias,
                         float* out, float* m_out, float* l_out, float* lx_out,
                         float* scratch) {
    float lambda = or_lambda(sm_scale);
    int32_t* S = (int32_t*)scratch;
    float* P = scratch + bc;
    float* T = scratch + 2 * bc;
    float* O = T + d;
    for (int r = 0; r < nrows; ++r)
        or_attn_row(q8, qs, k8, ks, vq, vs, N, d, rows[r], causal, lambda, pv_fp16, qblk, kblk, bc,
                    tmask ? tmask + (int64_t)(rows[r] / 128) * ((N + bc - 1) / bc) : 0,
                    bias ? bias + (int64_t)(rows[r] / 128) * N : 0, out + (int64_t)r * d,
                    m_out ? m_out + r : 0, l_out ? l_out + r : 0, lx_out ? lx_out + r : 0, S, T,
                    O, P);
}

/* ------------------------------------------------------------------------ */
/* Exact attention in FP64 from the bf16 inputs (no quantization).           */
/* ------------------------------------------------------------------------ */

/* out[r][c] = sum_j softmax_j(q_i . k_j * sm_scale) v_jc in fp64, with the
 * causal mask j <= i.  The plain definition of attention that the quantized
 * method approximates.  scratch: N doubles. */
OR_API void or_ref64_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int N, int d,
                          const int32_t* rows, int nrows, int causal, double sm_scale,
                          double* out, double* scratch) {
    for (int r = 0; r < nrows; ++r) {
        int i = rows[r];
        int n = causal ? i + 1 : N;
        double mx = -INFINITY;
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int c = 0; c < d; ++c)
                s += (double)or_bf16_to_f32(q[(int64_t)i * d + c]) *
                     (double)or_bf16_to_f32(k[(int64_t)j * d + c]);
            s *= sm_scale;
            scratch[j] = s;
            if (s > mx) mx = s;
        }
        double den = 0.0;
        for (int j = 0; j < n; ++j) {
            scratch[j] = exp(scratch[j] - mx);
            den += scratch[j];
        }
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int j = 0; j < n; ++j) acc += scratch[j] * (double)or_bf16_to_f32(v[(int64_t)j * d + c]);
            out[(int64_t)r * d + c] = acc / den;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Array forms of the codecs (one call per array, for the tests).            */
/* ------------------------------------------------------------------------ */

OR_API void or_bf16_to_f32_n(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_to_f32(in[i]);
}
OR_API void or_f32_to_bf16_n(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_f32_to_bf16(in[i]);
}
OR_API void or_e4m3_to_f32_n(const uint8_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_e4m3_to_f32(in[i]);
}
OR_API void or_f32_to_e4m3_n(const float* in, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_f32_to_e4m3(in[i]);
}
OR_API void or_f16_to_f32_n(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_f16_to_f32(in[i]);
}
OR_API void or_f32_to_f16_n(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_f32_to_f16(in[i]);
}
OR_API void or_fix30_n(const float* in, int64_t n, int64_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_fix30(in[i]);
}
