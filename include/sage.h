/*
 * sage.h -- C ABI of libsage: SageAttention-style low-bit attention (the
 * forward and the 8-bit backward) on AMD Instinct MI355X (gfx950).
 *
 *   O = softmax(Q K^T * sm_scale) V, computed as
 *     1. smooth K by subtracting its per-head token mean,
 *     2. quantize Q and K per block of 128 rows to INT8 (absmax scales) and
 *        form Q K^T exactly in INT32 on INT8 matrix cores,
 *     3. dequantize by q_scale * k_scale and run an exp2 online softmax in
 *        FP32 over key tiles of 128,
 *     4. take P to FP8 e4m3 with the static scale 448 and V to FP8 e4m3 with
 *        per-channel scales (or both to FP16) and run P V on FP8 (FP16)
 *        matrix cores with FP32 accumulation into the running output.  The
 *        pages accumulate each tile in a fresh FP32 sum and add it to the
 *        output (two-level accumulation) because their FP8 tensor cores keep
 *        fewer accumulator bits; gfx950 matrix cores accumulate in full FP32,
 *        so libsage accumulates straight into the rescaled output.  The two
 *        forms agree up to FP32 rounding order.
 *
 * What the pages say about the method: the wxsanhe.com blog post on
 * TurboDiffusion, section 三.1 (混合注意力) -- Q K in INT8, P V in FP8 or
 * FP16, outlier smoothing and two-level accumulation, usable as a quantized
 * FlashAttention; the reportify.cn SageAttention tag page, SageAttention3
 * summary, bullet 8比特训练 -- per-block INT8 quantization and per-token
 * quantization of P with no overhead; the txrjy.com repost of the QbitAI
 * article, section 四个步骤极限压缩时间 -- INT8 attention with outlier
 * smoothing.  Finer details (block sizes, rounding, the fixed-point mean,
 * the exp2 argument order) are this library's readings, fixed below.
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer allocated by the caller
 *     (e.g. by PyTorch), except the outputs of sage_get_config and of the
 *     *_sizes calls (host memory).  libsage never allocates, frees, synchronises, or changes the
 *     current device.  All work is enqueued asynchronously on `stream`
 *     (a hipStream_t; NULL means the null stream) on the current device.
 *   - Device buffers must be 16-byte aligned.
 *   - Inputs Q, K, V and the output O are contiguous with d innermost, in the
 *     layout given by `layout`: SAGE_LAYOUT_HND = [B][H][N][d],
 *     SAGE_LAYOUT_NHD = [B][N][H][d].  Q, K, V are bf16.
 *   - Quantized buffers are always head-major and have library-defined
 *     layouts (below); their byte sizes come from sage_quant_sizes.
 *     N_pad = 128 * ceil(N / 128), nblk = ceil(N / 128).
 *   - Supported: d in {64, 128}; 1 <= N; B, H >= 1; B*H*N_pad*d < 2^40.
 *   - Every argument is validated on the host before anything is enqueued;
 *     a failed check returns its status code and enqueues nothing.  Launch
 *     failures return SAGE_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - The library holds no mutable global state; calls are thread-safe.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_ABI_VERSION 1

enum sage_status {
    SAGE_OK = 0,
    SAGE_ERR_NULL = -1,        /* a required pointer is NULL */
    SAGE_ERR_INVALID = -2,     /* bad size, enum, flag, sm_scale or dump window */
    SAGE_ERR_UNSUPPORTED = -3, /* d not in {64, 128} */
    SAGE_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned */
    SAGE_ERR_SIZE = -5,        /* the problem exceeds the supported size */
    SAGE_ERR_HIP = -6,         /* a HIP launch failed */
    SAGE_ERR_WORKSPACE = -7,   /* workspace smaller than the matching *_sizes call asks */
    SAGE_ERR_SCRATCH = -8      /* sage_quant_qkv_noalloc: more than its fixed scratch needed */
};

enum sage_layout { SAGE_LAYOUT_HND = 0, SAGE_LAYOUT_NHD = 1 };
enum sage_pv_dtype { SAGE_PV_FP8 = 0, SAGE_PV_FP16 = 1 };
enum sage_out_dtype { SAGE_OUT_BF16 = 0, SAGE_OUT_FP32 = 1 };
/* Granularity of the Q scales (the _ex entry points).  The pages give the
 * per-block INT8 quantization (reportify SageAttention3 summary, bullet
 * 8比特训练) and a finer "thread-level" one (the txrjy.com repost of the
 * QbitAI article, section 四个步骤极限压缩时间); SAGE_QGRAN_TOKEN is the finest
 * Q granularity: one scale per query row.  K stays per block of 128 rows. */
enum sage_q_gran { SAGE_QGRAN_BLOCK = 0, SAGE_QGRAN_TOKEN = 1 };
/* Element format of the microscaled path: E2M3 (MXFP6) or E2M1 (MXFP4). */
enum sage_mx_fmt { SAGE_MX_FP4 = 4, SAGE_MX_FP6 = 6 };

/* Compile-time constants of the method as built. */
typedef struct {
    int abi_version;     /* SAGE_ABI_VERSION */
    int blkq;            /* rows per Q quantization block (128) */
    int blkk;            /* rows per K quantization block (128) */
    int bc;              /* keys per online-softmax tile (128; equals blkk) */
    int br;              /* queries per attention workgroup (256) */
    int stats_chunk;     /* tokens per statistics workgroup (512) */
    float p_scale;       /* static FP8 scale of P (448, the e4m3fn maximum) */
    float log2_p_scale;  /* fp32(log2(448)), folded into the exp2 argument */
    int fp8_format;      /* 0 = OCP e4m3fn (max 448, no infinities) */
} sage_config;

/* Fill *out with the constants for head dimension d.
 * Returns SAGE_OK, SAGE_ERR_NULL, or SAGE_ERR_UNSUPPORTED. */
int sage_get_config(int d, sage_config* out);

/* Indices into the sizes array of sage_quant_sizes. */
enum sage_buffer {
    SAGE_BUF_Q8 = 0,   /* int8  [B][H][N_pad][d]; rows >= N are 0 */
    SAGE_BUF_QSCALE,   /* fp32  [B][H][nblk] */
    SAGE_BUF_K8,       /* int8  [B][H][N_pad][d]; rows >= N are 0 */
    SAGE_BUF_KSCALE,   /* fp32  [B][H][nblk] */
    SAGE_BUF_KMEAN,    /* fp32  [B][H][d] */
    SAGE_BUF_VQ,       /* fp8 e4m3 (1 B) or fp16 (2 B): [B][H][nblk][d][128], see below */
    SAGE_BUF_VSCALE,   /* fp32  [B][H][d] */
    SAGE_BUF_WS_QK,    /* workspace bytes for sage_quant_qk */
    SAGE_BUF_WS_V,     /* workspace bytes for sage_quant_v */
    SAGE_NBUF
};

/* Byte sizes of every buffer above for the given problem (sizes has
 * SAGE_NBUF entries, host memory).  Returns SAGE_OK, SAGE_ERR_NULL,
 * SAGE_ERR_INVALID, SAGE_ERR_UNSUPPORTED or SAGE_ERR_SIZE. */
int sage_quant_sizes(int B, int H, int N, int d, int pv_dtype, size_t* sizes);

/* As sage_quant_sizes, for Q scales of granularity q_gran (sage_q_gran):
 * with SAGE_QGRAN_TOKEN, SAGE_BUF_QSCALE is fp32 [B][H][N_pad] (rows >= N
 * get scale 0).  Returns the codes of sage_quant_sizes; SAGE_ERR_INVALID for
 * an unknown q_gran. */
int sage_quant_sizes_ex(int B, int H, int N, int d, int pv_dtype, int q_gran, size_t* sizes);

/*
 * Smooth K and quantize Q and K (per block of 128 rows, INT8).
 *
 * K smoothing (wxsanhe §三.1 "outlier smoothing"; txrjy 四个步骤 section): per
 * (b, h, c), I = sum over tokens j of trunc(K[j][c] * 2^30) in wrapping
 * 64-bit two's complement (each term saturated at +-2^62, NaN -> 0), then
 * k_mean = fp32(fp64(I) / (fp64(N) * 2^30)).  This is the token mean on an
 * exact 2^-30 grid, so it does not depend on summation order.
 * Then k' = fp32(K - k_mean).
 * Per block r of rows [128 r, min(N, 128 r + 128)) of Q (and of k'):
 *   a = max |x| over the block's valid rows and all d channels,
 *   scale = fp32(fp64(a) / 127), inv = a > 0 ? fp32(127 / fp64(a)) : 0,
 *   code = clamp(round_half_even(fp32(x * inv)), -127, 127).
 * (reportify SageAttention3 summary, 8比特训练: per-block INT8.)
 *
 * q, k: bf16 inputs [B,H,N,d] or [B,N,H,d] (layout).
 * Outputs (caller-allocated, sizes from sage_quant_sizes): q8, q_scale, k8,
 * k_scale, k_mean.  workspace: SAGE_BUF_WS_QK bytes of device scratch (no
 * initialisation needed; contents undefined on return).
 */
int sage_quant_qk(const void* q, const void* k, int B, int H, int N, int d, int layout,
                  int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, float* k_mean,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_quant_qk with the Q scale granularity q_gran (sage_q_gran).
 * SAGE_QGRAN_BLOCK is sage_quant_qk.  SAGE_QGRAN_TOKEN quantizes each query
 * row n < N on its own: a = max_c |Q[n][c]|, q_scale[b][h][n] = fp32(fp64(a)/127),
 * codes as above with inv = fp32(127/fp64(a)); rows N..N_pad-1 get codes 0 and
 * scale 0.  K smoothing and K quantization are unchanged.  q_scale must hold
 * the SAGE_BUF_QSCALE bytes sage_quant_sizes_ex gives for q_gran.
 */
int sage_quant_qk_ex(const void* q, const void* k, int B, int H, int N, int d, int layout,
                     int q_gran, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale,
                     float* k_mean, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Quantize V (wxsanhe §三.1: P V in FP8 or FP16).
 * pv_dtype = SAGE_PV_FP8: per (b, h, c), a = max_j |V[j][c]|;
 *   v_scale = fp32(fp64(a) / 448), inv = a > 0 ? fp32(448 / fp64(a)) : 0,
 *   code = e4m3fn(round_half_even(fp32(V * inv))) (saturating).
 * pv_dtype = SAGE_PV_FP16: code = binary16(round_half_even(V)) saturating at
 *   +-65504; v_scale = 1.
 * vq layout: [B][H][nblk][d][128]: for each tile of 128 keys, one row of 128
 * codes per channel, keys permuted within the tile: key
 *   r = 32*kb + 8*b + 4*g + q   (kb, b, q in 0..3, g in 0..1)
 * is stored at position 64*g + 16*kb + 4*b + q.  Keys >= N are 0.
 * (This order makes the P V operand of one lane a contiguous run.)
 * workspace: SAGE_BUF_WS_V bytes of device scratch (fp8 path only; may be
 * NULL with 0 bytes for fp16).
 */
int sage_quant_v(const void* v, int B, int H, int N, int d, int layout, int pv_dtype,
                 void* vq, float* v_scale, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * One quantization pass over Q, K and V: exactly sage_quant_qk followed by
 * sage_quant_v (the same codes, scales and k_mean, bit for bit), with the K
 * and V column statistics taken in one launch and combined in one more
 * (wxsanhe §三.1: Q K to INT8 with K smoothing, P V in FP8 or FP16).
 * Buffers and layouts as in those two calls (sizes from sage_quant_sizes with
 * pv_dtype).  workspace: sizes[SAGE_BUF_WS_QK] + sizes[SAGE_BUF_WS_V] bytes
 * of device scratch (no initialisation needed; contents undefined on return).
 * Errors as sage_quant_qk and sage_quant_v; SAGE_ERR_WORKSPACE if workspace
 * is smaller than that sum.
 */
int sage_quant_qkv(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                   int layout, int pv_dtype, int8_t* q8, float* q_scale, int8_t* k8,
                   float* k_scale, float* k_mean, void* vq, float* v_scale, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * sage_quant_qkv without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * results, buffers and errors as sage_quant_qkv; the K and V partial
 * statistics live in a fixed 32 MiB device array of the library instead
 * (one per GPU, held until the process ends).  The problem must need at most
 * that much: sizes[SAGE_BUF_WS_QK] + sizes[SAGE_BUF_WS_V] <= 32 MiB (FP8 V:
 * 12 B H d ceil(N / 512) + 4 B H d bytes, so B = 1, H = 40, d = 128 allows
 * N <= 279040), else SAGE_ERR_SCRATCH before any launch.
 * stream must belong to the current device (else SAGE_ERR_HIP); the
 * library looks the array up once per device on the first call there.
 * Every call on one GPU shares the array: calls that overlap on one GPU
 * (other streams or host threads) race and must be serialised by the caller.
 */
int sage_quant_qkv_noalloc(const void* q, const void* k, const void* v, int B, int H, int N,
                           int d, int layout, int pv_dtype, int8_t* q8, float* q_scale,
                           int8_t* k8, float* k_scale, float* k_mean, void* vq, float* v_scale,
                           void* stream);

/*
 * Fused attention over the quantized operands (hunxia glossary, FlashAttention:
 * tiled, online softmax; wxsanhe §三.1: FP8 P V with FP32 accumulation).
 * For each query i (with sigma = fp32(q_scale * lambda), lambda =
 * fp32(sm_scale * log2 e)), key tiles t = 0, 1, ... of 128 keys in ascending
 * order (causal: keys j > i masked, tiles wholly above the diagonal skipped):
 *   c = fp32(sigma * k_scale[t]);  S_j = exact int32 dot(q8_i, k8_j)
 *   m_t = max_j fp32(S_j c);  m' = max(m, m_t);  alpha = exp2(m - m') (0 at start)
 *   p_j = exp2(fma(S_j, c, -fp32(m' - log2 448)))     (about 448 * P_ij)
 *   l = alpha l + sum_j e4m3(p_j)         (the quantized P the product uses; fp16
 *                                         path: binary16(p_j)), so the weights
 *                                         applied to V sum to one
 *   O = alpha O + sum_j e4m3(p_j) * v_j   (fp16 path: binary16(p_j)), FP32 MFMA
 *                                         accumulation (the two-level form, a fresh
 *                                         FP32 sum per tile added to O, differs only
 *                                         in rounding order);  m = m'
 * and finally out_i = O * v_scale / l.  Sums over j run in the hardware's
 * order; results match the two-level ascending-order definition within FP32
 * rounding (measured max-abs difference about 1e-6 at |O| ~ 1).
 * causal: 0 or 1 (top-left aligned, j <= i).  sm_scale: finite, > 0.
 * out: [B,H,N,d] or [B,N,H,d] (layout), bf16 (out_dtype 0) or fp32 (1).
 */
int sage_attn_fwd(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                  const void* vq, const float* v_scale, int B, int H, int N, int d, int layout,
                  int causal, float sm_scale, int pv_dtype, void* out, int out_dtype,
                  void* stream);

/*
 * sage_attn_fwd that also returns each query row's log-sum-exp, the forward
 * half of 8-bit training (reportify.cn SageAttention3 summary, bullet
 * 8比特训练: the backward recomputes P from it):
 *   lse[b][h][i] = fp32(fp32(m_i - log2 448) + log2(lx_i))
 * with m_i the row's final running max and lx_i = alpha lx + sum_j p_j its row
 * sum of the unquantized p (the log-sum-exp of the scores), so that
 * 2^(S_ij c - lse_i) is the softmax probability P_ij in the exp2 domain (log2
 * on the GPU's own log2; differs from a correctly rounded one by about an
 * ulp).  lse: fp32 [B][H][N], 16-byte aligned, written for every row; the
 * rest as sage_attn_fwd (the same kernel; at d = 64 the pipelined one).
 */
int sage_attn_fwd_lse(const int8_t* q8, const float* q_scale, const int8_t* k8,
                      const float* k_scale, const void* vq, const float* v_scale, int B, int H,
                      int N, int d, int layout, int causal, float sm_scale, int pv_dtype,
                      void* out, int out_dtype, float* lse, void* stream);

/*
 * The backward pass of 8-bit trainable attention (reportify.cn SageAttention3
 * summary, bullet 8比特训练: per-block INT8 Q/K/V, per-token P with no
 * quantization overhead, dO V^T kept in FP16, the other four backward products
 * quantized).  Per tile pair of 128 queries x 128 keys, in the exp2 domain:
 *   S = q8 . k8 (the forward's INT8 codes, K smoothed -- the rows of dS sum to
 *       zero, so smoothing leaves dQ unchanged in exact arithmetic)
 *   P = exp2(fma(S, c, -lse_i)), c = fp32(fp32(q_scale * lambda) * k_scale)
 *   dP = f16(dO) . f16(V)^T (FP16 matrix cores, FP32 accumulation)
 *   D_i = dO_i . O_i;  dS = fp32(P * fp32(dP - D_i)) (the FP16 product's
 *       accumulation starts at -D_i, so dP - D_i leaves the matrix core)
 *   dV += (dO8^T . e4m3(448 P)) * fp32(s_do / 448): dO in FP8 e4m3 per block
 *         of 128 rows (absmax / 448 scale), P at the forward's static scale
 *   dS8 = INT8 of dS per tile pair (absmax / 127 scale s_ds)
 *   dK += (Q8^T . dS8) * fp32(fp32(s_ds * q_scale) * sm_scale)
 *   dQ += (K8^T . dS8^T) * fp32(fp32(s_ds * k_scale) * sm_scale)
 * (causal: keys j > i masked).  Inputs: q8 / q_scale / k8 / k_scale from
 * sage_quant_qk (per-block Q), v the bf16 V, o the forward's bf16 output,
 * dO the upstream gradient (bf16), all in `layout`; lse from
 * sage_attn_fwd_lse.  Outputs dq, dk, dv: fp32 in `layout`, overwritten.
 * workspace: sage_bwd_sizes bytes of device scratch, 256-byte aligned, owned by
 * the caller and free again when the call's stream work has finished.  With
 * nblk = ceil(N / 128) and N_pad = 128 nblk it holds, in this order and each
 * part rounded up to 256 bytes: D [B*H][N_pad] f32, s_do [B*H][nblk] f32, dO
 * and V in fp16 [B*H][N_pad][d] (two parts), dO in FP8 and the Q and K codes
 * transposed [B*H][nblk][d][128] bytes (three parts), and the per-tile
 * records of the dK/dV sweep [B*H][nblk][512] f32.  d in {64, 128}.
 */
int sage_bwd_sizes(int B, int H, int N, int d, size_t* workspace_bytes);
int sage_attn_bwd(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                  const void* v, const void* o, const void* dO, const float* lse, int B, int H,
                  int N, int d, int layout, int causal, float sm_scale, float* dq, float* dk,
                  float* dv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd over Q scales of granularity q_gran (sage_q_gran), as
 * produced by sage_quant_qk_ex: sigma above is fp32(q_scale[b][h][i] *
 * lambda) for SAGE_QGRAN_TOKEN (fp32(q_scale[b][h][i / 128] * lambda) for
 * SAGE_QGRAN_BLOCK, which is sage_attn_fwd).  Same kernel, same cost.
 */
int sage_attn_fwd_ex(const int8_t* q8, const float* q_scale, const int8_t* k8,
                     const float* k_scale, const void* vq, const float* v_scale, int B, int H,
                     int N, int d, int layout, int causal, float sm_scale, int pv_dtype,
                     int q_gran, void* out, int out_dtype, void* stream);

/*
 * Block-sparse attention: sage_attn_fwd_ex that visits, for each block of
 * 128 queries, only the key tiles its mask selects (the pages present sparse
 * attention as orthogonal to low-bit attention and stackable with it:
 * wxsanhe §三.1; the block-sparse half of sparse-linear attention).
 * tile_mask: device uint8 [B][H][nblk][nblk], row = query block (queries
 * [128 r, 128 r + 128)), column = key tile (keys [128 t, 128 t + 128));
 * nonzero = visit.  A skipped tile contributes nothing: the online softmax of
 * the block's rows runs over the visited tiles in ascending order, exactly as
 * if the skipped tiles' keys were masked; with causal, keys after the query
 * stay masked as well.  A row that visits no key gets the output 0.
 * A workgroup (one query block; two with FP16 P V at d = 128) loads and
 * computes only the tiles its block(s) visit.  Requires nblk <= 2048
 * (N <= 262144; else SAGE_ERR_SIZE); tile_mask 16-byte aligned.
 */
int sage_attn_fwd_sparse(const int8_t* q8, const float* q_scale, const int8_t* k8,
                         const float* k_scale, const void* vq, const float* v_scale, int B, int H,
                         int N, int d, int layout, int causal, float sm_scale, int pv_dtype,
                         int q_gran, const uint8_t* tile_mask, void* out, int out_dtype,
                         void* stream);

/*
 * Q smoothing (the pages' outlier smoothing -- wxsanhe §三.1, txrjy.com
 * QbitAI repost, section 四个步骤极限压缩时间 -- applied to Q as well as K).
 * Queries that share a per-channel offset waste the INT8 range of Q on it;
 * subtracting each 128-query block's channel means before quantizing keeps the
 * range for what varies.  Unlike the K mean, the Q mean changes the scores
 * (by q_mean . k_j per key), so that share is put back in FP32:
 *   1. sage_quant_qk_smooth: as sage_quant_qk_ex, except that Q is first
 *      smoothed: q_mean[b][h][c][r] = the mean of channel c over block r's
 *      valid rows, taken on the K mean's exact 2^-30 grid
 *      (fp32(fp64(I) / (fp64(rows) 2^30)), I the wrapping int64 sum of
 *      trunc(x 2^30)); the codes quantize fp32(Q - q_mean[.][r]) (block or
 *      token scales as q_gran says).  q_mean: fp32 [B][H][d][nbp],
 *      channel-major, nbp = 16 ceil(nblk / 16); entries r >= nblk are 0.
 *   2. sage_q_smooth_bias: bias[b][h][r][j] = fp32(acc * lambda), acc the fp32
 *      fused-multiply-add chain over c = 0 .. d-1 (ascending, from 0) of
 *      q_mean[c][r] * fp32(K[j][c] - k_mean[c]); lambda = fp32(sm_scale *
 *      log2 e).  bias: fp32 [B][H][nblk][N_pad]; keys j >= N get 0.  k is
 *      the same bf16 K (same layout) that sage_quant_qk_smooth read.
 *   3. sage_attn_fwd_smooth: as sage_attn_fwd_ex (tile_mask == NULL) or
 *      sage_attn_fwd_sparse (tile_mask != NULL), with the scores of query i
 *      (block r = i / 128) and key j taken as
 *        s_j = fma(S_j, c, bias[r][j]),  m_t = max_j s_j,
 *        p_j = exp2(fp32(s_j - mu))
 *      (m', alpha, mu, l, P and the epilogue unchanged).  sm_scale must be the
 *      one the bias was computed with.  About 20 % more vector work per score
 *      than the unsmoothed kernel.
 * sage_qsmooth_sizes gives the byte sizes of q_mean and bias (host pointers).
 * Errors: as the functions they extend; NULL q_mean / bias -> SAGE_ERR_NULL;
 * sage_q_smooth_bias: bias elements >= 2^40 -> SAGE_ERR_SIZE.
 */
int sage_qsmooth_sizes(int B, int H, int N, int d, size_t* q_mean_bytes, size_t* bias_bytes);
int sage_quant_qk_smooth(const void* q, const void* k, int B, int H, int N, int d, int layout,
                         int q_gran, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale,
                         float* k_mean, float* q_mean, void* workspace, size_t workspace_bytes,
                         void* stream);
int sage_q_smooth_bias(const float* q_mean, const void* k, const float* k_mean, int B, int H,
                       int N, int d, int layout, float sm_scale, float* bias, void* stream);
int sage_attn_fwd_smooth(const int8_t* q8, const float* q_scale, const int8_t* k8,
                         const float* k_scale, const void* vq, const float* v_scale, int B, int H,
                         int N, int d, int layout, int causal, float sm_scale, int pv_dtype,
                         int q_gran, const float* bias, const uint8_t* tile_mask, void* out,
                         int out_dtype, void* stream);

/*
 * Microscaled attention, MXFP6 or MXFP4 (reportify.cn SageAttention3
 * summary, bullet FP4量化创新: microscaling FP4 attention; MXFP4 rated less
 * accurate there).  The gfx950 matrix cores take MX operands with E8M0
 * block scales of 32 (OCP Microscaling), FP4 and FP6 at the same rate.  The
 * default entry points use FP6 E2M3 elements (3 mantissa bits); the _fmt
 * forms take fmt = SAGE_MX_FP6 or SAGE_MX_FP4 (E2M1, 1 mantissa bit: the
 * cosine against FP64 attention drops from ~0.998 to ~0.97 on Gaussian
 * inputs).  The pages' two-stage quantization of P answers the narrow range
 * of NVFP4's FP8 block scales; an E8M0 scale is any power of two, so P is
 * quantized in one stage here.
 * Every MX block of 32 elements is stored as 32 bytes.  E2M3: the 24 bytes
 * of the 32 packed codes (element 2i at bits [12i, 12i + 6) is value i of
 * the block, element 2i + 1 is value 16 + i: the packing of
 * v_cvt_scalef32_2xpk16_fp6_f32).  E2M1: 16 bytes, byte i holding value i
 * in its low nibble and value 16 + i in its high nibble (the packing of
 * v_cvt_scalef32_pk_fp4_f32 with those two values), then 8 zero bytes.
 * Both: the E8M0 scale byte at offset 24, then 7 zero bytes.  Block rule:
 * e = floor(log2(amax)) - 2, codes = element(x / 2^e) rounded to nearest
 * even and saturated at the largest magnitude (7.5 for E2M3, 6 for E2M1),
 * byte e + 127; a block with amax < 2^-100 is all zero with byte 0.
 *   sage_quant_qk_mx: K smoothed as in sage_quant_qk (k_mean, same
 *     workspace), then Q and K' per row and 32 channels:
 *     q6, k6 [B][H][N_pad][d] bytes (d / 32 blocks per row), rows >= N 0.
 *   sage_quant_v_mx: V per channel and 32 keys: v6 [B][H][nblk][d][128]
 *     bytes: for each tile of 128 keys, one 128-byte row per channel holding
 *     the tile's 4 key blocks in key order; keys >= N are 0.
 *   sage_attn_fwd_mx: S_j = Q6 . K6_j with the block scales (fp32 from the
 *     matrix core); m_t = max_j S_j lambda rounded toward -infinity,
 *     m' = max(m, m_t), alpha = exp2(m - m'), p_j = exp2(fma(S_j, lambda,
 *     -m')) (the largest is in [1, 1 + 2^-23), so its P block always takes
 *     scale 2^-2), l = alpha l + sum p_j; P per query and 32 consecutive
 *     keys of a tile to MXFP6 by the block rule; O = alpha O + P6 V6;
 *     out = O / l.  Layout, causal, sm_scale, out / out_dtype as for
 *     sage_attn_fwd; d = 64 or 128.
 * Errors as for the INT8 / FP8 entry points (status codes, nothing
 * launched on an invalid argument).
 * Buffer sizes: q6 and k6 as SAGE_BUF_Q8, v6 as SAGE_BUF_VQ with
 * SAGE_PV_FP8, workspace as SAGE_BUF_WS_QK (sage_quant_sizes).
 */
int sage_quant_qk_mx(const void* q, const void* k, int B, int H, int N, int d, int layout,
                     uint8_t* q6, uint8_t* k6, float* k_mean, void* workspace,
                     size_t workspace_bytes, void* stream);
int sage_quant_v_mx(const void* v, int B, int H, int N, int d, int layout, uint8_t* v6,
                    void* stream);
int sage_attn_fwd_mx(const uint8_t* q6, const uint8_t* k6, const uint8_t* v6, int B, int H, int N,
                     int d, int layout, int causal, float sm_scale, void* out, int out_dtype,
                     void* stream);
/* The same three calls for element format fmt (SAGE_MX_FP6 or SAGE_MX_FP4;
 * any other value: SAGE_ERR_INVALID, nothing launched).  The three calls of
 * one attention take the same fmt; buffers and sizes do not depend on it. */
int sage_quant_qk_mx_fmt(const void* q, const void* k, int B, int H, int N, int d, int layout,
                         int fmt, uint8_t* q6, uint8_t* k6, float* k_mean, void* workspace,
                         size_t workspace_bytes, void* stream);
int sage_quant_v_mx_fmt(const void* v, int B, int H, int N, int d, int layout, int fmt,
                        uint8_t* v6, void* stream);
int sage_attn_fwd_mx_fmt(const uint8_t* q6, const uint8_t* k6, const uint8_t* v6, int B, int H,
                         int N, int d, int layout, int fmt, int causal, float sm_scale, void* out,
                         int out_dtype, void* stream);

/*
 * sage_attn_fwd that also writes the raw int32 Q K^T accumulators of head
 * (b, h), queries [row0, row0 + nrows), all keys, to s_out [nrows][N]
 * (row-major).  With causal, only entries j <= i are written; the others are
 * left untouched.  Same kernel source and arguments as sage_attn_fwd; the
 * attention output is written as well.
 */
int sage_attn_fwd_debug(const int8_t* q8, const float* q_scale, const int8_t* k8,
                        const float* k_scale, const void* vq, const float* v_scale, int B, int H,
                        int N, int d, int layout, int causal, float sm_scale, int pv_dtype,
                        void* out, int out_dtype, int b, int h, int row0, int nrows,
                        int32_t* s_out, void* stream);

/* A static, human-readable name for a status code. */
const char* sage_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H */
