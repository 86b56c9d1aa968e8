// Host side of the libsage C ABI: argument validation (entirely before any
// launch), buffer-size arithmetic, and the kernel launches.  Declarations and
// the meaning of every argument are in include/sage.h.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "sage.h"
#include "sage_common.h"


namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID;
    if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
    const int64_t nblk = ((int64_t)N + sage::kBlk - 1) / sage::kBlk;
    const int64_t elems = (int64_t)B * H * nblk * sage::kBlk * d;
    if (elems >= kMaxElems) return SAGE_ERR_SIZE;
    // grid limits: attention grid is B*H*ceil(N/256) workgroups; stats grid y is B*H
    if ((int64_t)B * H > 65535 || (int64_t)B * H * ((N + sage::kBr - 1) / sage::kBr) >= (1ll << 31))
        return SAGE_ERR_SIZE;
    return SAGE_OK;
}

int check_layout(int layout) {
    return (layout == SAGE_LAYOUT_HND || layout == SAGE_LAYOUT_NHD) ? SAGE_OK : SAGE_ERR_INVALID;
}
int check_pv(int pv) { return (pv == SAGE_PV_FP8 || pv == SAGE_PV_FP16) ? SAGE_OK : SAGE_ERR_INVALID; }
int check_qgran(int g) {
    return (g == SAGE_QGRAN_BLOCK || g == SAGE_QGRAN_TOKEN) ? SAGE_OK : SAGE_ERR_INVALID;
}

struct Sizes {
    size_t v[SAGE_NBUF];
};

Sizes sizes_of(int B, int H, int N, int d, int pv, int q_gran = SAGE_QGRAN_BLOCK) {
    const size_t nblk = ((size_t)N + sage::kBlk - 1) / sage::kBlk;
    const size_t npad = nblk * sage::kBlk;
    const size_t bh = (size_t)B * H;
    const size_t nchunk = ((size_t)N + sage::kStatsChunk - 1) / sage::kStatsChunk;
    Sizes s;
    s.v[SAGE_BUF_Q8] = bh * npad * d;
    s.v[SAGE_BUF_QSCALE] = bh * (q_gran == SAGE_QGRAN_TOKEN ? npad : nblk) * sizeof(float);
    s.v[SAGE_BUF_K8] = bh * npad * d;
    s.v[SAGE_BUF_KSCALE] = bh * nblk * sizeof(float);
    s.v[SAGE_BUF_KMEAN] = bh * d * sizeof(float);
    s.v[SAGE_BUF_VQ] = bh * npad * d * (pv == SAGE_PV_FP16 ? 2 : 1);
    s.v[SAGE_BUF_VSCALE] = bh * d * sizeof(float);
    s.v[SAGE_BUF_WS_QK] = bh * nchunk * d * sizeof(uint64_t);
    s.v[SAGE_BUF_WS_V] = pv == SAGE_PV_FP16 ? 0 : (bh * nchunk * d + bh * d) * sizeof(float);
    return s;
}

#define SAGE_TRY(expr)                 \
    do {                               \
        const int _st = (expr);        \
        if (_st != SAGE_OK) return _st; \
    } while (0)

int attn_common(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                const void* vq, const float* v_scale, int B, int H, int N, int d, int layout,
                int causal, float sm_scale, int pv_dtype, int q_gran, const uint8_t* tmask,
                int sparse, const float* bias, int smooth, void* out, int out_dtype, int dump,
                int db, int dh, int row0, int nrows, int32_t* s_out, void* stream,
                float* lse = nullptr) {
    if (!q8 || !q_scale || !k8 || !k_scale || !vq || !v_scale || !out) return SAGE_ERR_NULL;
    if (smooth && !bias) return SAGE_ERR_NULL;
    if (sparse && !tmask) return SAGE_ERR_NULL;
    if (dump && !s_out) return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    SAGE_TRY(check_pv(pv_dtype));
    SAGE_TRY(check_qgran(q_gran));
    if (causal != 0 && causal != 1) return SAGE_ERR_INVALID;
    if (out_dtype != SAGE_OUT_BF16 && out_dtype != SAGE_OUT_FP32) return SAGE_ERR_INVALID;
    if (!(isfinite(sm_scale) && sm_scale > 0.0f)) return SAGE_ERR_INVALID;
    if (dump) {
        if (db < 0 || db >= B || dh < 0 || dh >= H || row0 < 0 || nrows < 1 ||
            (int64_t)row0 + nrows > N)
            return SAGE_ERR_INVALID;
        if ((int64_t)nrows * N >= kMaxElems) return SAGE_ERR_SIZE;
    }
    if (sparse && ((int64_t)N + sage::kBc - 1) / sage::kBc > sage::kMaxSparseTiles)
        return SAGE_ERR_SIZE;
    if (!aligned16(q8) || !aligned16(q_scale) || !aligned16(k8) || !aligned16(k_scale) ||
        !aligned16(vq) || !aligned16(v_scale) || !aligned16(out) || (dump && !aligned16(s_out)) ||
        (sparse && !aligned16(tmask)) || (smooth && !aligned16(bias)) || (lse && !aligned16(lse)))
        return SAGE_ERR_ALIGN;
    sage::AttnArgs a;
    a.q8 = q8;
    a.q_scale = q_scale;
    a.k8 = k8;
    a.k_scale = k_scale;
    a.vq = vq;
    a.v_scale = v_scale;
    a.out = out;
    a.s_out = s_out;
    a.H = H;
    a.N = N;
    a.nblk = (N + sage::kBlk - 1) / sage::kBlk;
    a.N_pad = a.nblk * sage::kBlk;
    // a.nqt / a.total (workgroups per head / in all) are set by the launcher,
    // which knows the workgroup size of the variant it picks
    a.layout = layout;
    a.out_fp32 = out_dtype == SAGE_OUT_FP32;
    a.qtok = q_gran == SAGE_QGRAN_TOKEN;
    a.tmask = sparse ? tmask : nullptr;
    a.bias = smooth ? bias : nullptr;
    a.lambda = (float)((double)sm_scale * 1.4426950408889634);
    a.dbh = dump ? db * H + dh : -1;
    a.drow0 = row0;
    a.dnrows = nrows;
    a.lse = lse;
    const hipError_t e = sage::launch_attn(a, B, d, pv_dtype == SAGE_PV_FP16, causal, dump,
                                           (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int sage_get_config(int d, sage_config* out) {
    if (!out) return SAGE_ERR_NULL;
    if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
    out->abi_version = SAGE_ABI_VERSION;
    out->blkq = sage::kBlk;
    out->blkk = sage::kBlk;
    out->bc = sage::kBc;
    out->br = sage::kBr;
    out->stats_chunk = sage::kStatsChunk;
    out->p_scale = sage::kPScale;
    out->log2_p_scale = sage::kLog2PScale;
    out->fp8_format = 0;
    return SAGE_OK;
}

__attribute__((visibility("default"))) int sage_quant_sizes_ex(int B, int H, int N, int d,
                                                               int pv_dtype, int q_gran,
                                                               size_t* sizes) {
    if (!sizes) return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_pv(pv_dtype));
    SAGE_TRY(check_qgran(q_gran));
    const Sizes s = sizes_of(B, H, N, d, pv_dtype, q_gran);
    for (int i = 0; i < SAGE_NBUF; ++i) sizes[i] = s.v[i];
    return SAGE_OK;
}

__attribute__((visibility("default"))) int sage_quant_sizes(int B, int H, int N, int d,
                                                            int pv_dtype, size_t* sizes) {
    return sage_quant_sizes_ex(B, H, N, d, pv_dtype, SAGE_QGRAN_BLOCK, sizes);
}

namespace {

int quant_qk_common(const void* q, const void* k, int B, int H, int N, int d, int layout,
                    int q_gran, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale,
                    float* k_mean, int smooth, float* q_mean, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (!q || !k || !q8 || !q_scale || !k8 || !k_scale || !k_mean || !workspace ||
        (smooth && !q_mean))
        return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    SAGE_TRY(check_qgran(q_gran));
    if (!aligned16(q) || !aligned16(k) || !aligned16(q8) || !aligned16(q_scale) ||
        !aligned16(k8) || !aligned16(k_scale) || !aligned16(k_mean) || !aligned16(workspace) ||
        (smooth && !aligned16(q_mean)))
        return SAGE_ERR_ALIGN;
    const Sizes s = sizes_of(B, H, N, d, SAGE_PV_FP8, q_gran);
    if (workspace_bytes < s.v[SAGE_BUF_WS_QK]) return SAGE_ERR_WORKSPACE;
    const hipError_t e = sage::launch_quant_qk((const sage::u16*)q, (const sage::u16*)k, B, H, N,
                                               d, layout, q_gran == SAGE_QGRAN_TOKEN, q8, q_scale,
                                               k8, k_scale, k_mean, smooth ? q_mean : nullptr,
                                               (uint64_t*)workspace, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

}  // namespace

__attribute__((visibility("default"))) int sage_quant_qk_ex(const void* q, const void* k, int B,
                                                            int H, int N, int d, int layout,
                                                            int q_gran, int8_t* q8,
                                                            float* q_scale, int8_t* k8,
                                                            float* k_scale, float* k_mean,
                                                            void* workspace,
                                                            size_t workspace_bytes,
                                                            void* stream) {
    return quant_qk_common(q, k, B, H, N, d, layout, q_gran, q8, q_scale, k8, k_scale, k_mean, 0,
                           nullptr, workspace, workspace_bytes, stream);
}

__attribute__((visibility("default"))) int sage_qsmooth_sizes(int B, int H, int N, int d,
                                                              size_t* q_mean_bytes,
                                                              size_t* bias_bytes) {
    if (!q_mean_bytes || !bias_bytes) return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    const size_t nblk = ((size_t)N + sage::kBlk - 1) / sage::kBlk;
    const size_t bh = (size_t)B * H;
    const size_t nbp = (nblk + sage::kBiasBlocks - 1) / sage::kBiasBlocks * sage::kBiasBlocks;
    *q_mean_bytes = bh * d * nbp * sizeof(float);
    *bias_bytes = bh * nblk * nblk * sage::kBlk * sizeof(float);
    return SAGE_OK;
}

__attribute__((visibility("default"))) int sage_quant_qk_smooth(
    const void* q, const void* k, int B, int H, int N, int d, int layout, int q_gran, int8_t* q8,
    float* q_scale, int8_t* k8, float* k_scale, float* k_mean, float* q_mean, void* workspace,
    size_t workspace_bytes, void* stream) {
    return quant_qk_common(q, k, B, H, N, d, layout, q_gran, q8, q_scale, k8, k_scale, k_mean, 1,
                           q_mean, workspace, workspace_bytes, stream);
}

__attribute__((visibility("default"))) int sage_q_smooth_bias(const float* q_mean, const void* k,
                                                              const float* k_mean, int B, int H,
                                                              int N, int d, int layout,
                                                              float sm_scale, float* bias,
                                                              void* stream) {
    if (!q_mean || !k || !k_mean || !bias) return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    if (!(isfinite(sm_scale) && sm_scale > 0.0f)) return SAGE_ERR_INVALID;
    const int64_t nblk = ((int64_t)N + sage::kBlk - 1) / sage::kBlk;
    if ((int64_t)B * H * nblk * nblk * sage::kBlk >= kMaxElems || nblk > 65535 * 32)
        return SAGE_ERR_SIZE;
    if (!aligned16(q_mean) || !aligned16(k) || !aligned16(k_mean) || !aligned16(bias))
        return SAGE_ERR_ALIGN;
    const float lambda = (float)((double)sm_scale * 1.4426950408889634);
    const hipError_t e = sage::launch_q_bias(q_mean, (const sage::u16*)k, k_mean, B, H, N, d,
                                             layout, lambda, bias, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

__attribute__((visibility("default"))) int sage_quant_qk(const void* q, const void* k, int B,
                                                         int H, int N, int d, int layout,
                                                         int8_t* q8, float* q_scale, int8_t* k8,
                                                         float* k_scale, float* k_mean,
                                                         void* workspace, size_t workspace_bytes,
                                                         void* stream) {
    return sage_quant_qk_ex(q, k, B, H, N, d, layout, SAGE_QGRAN_BLOCK, q8, q_scale, k8, k_scale,
                            k_mean, workspace, workspace_bytes, stream);
}

__attribute__((visibility("default"))) int sage_quant_v(const void* v, int B, int H, int N, int d,
                                                        int layout, int pv_dtype, void* vq,
                                                        float* v_scale, void* workspace,
                                                        size_t workspace_bytes, void* stream) {
    if (!v || !vq || !v_scale) return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    SAGE_TRY(check_pv(pv_dtype));
    const Sizes s = sizes_of(B, H, N, d, pv_dtype);
    if (pv_dtype == SAGE_PV_FP8 && !workspace) return SAGE_ERR_NULL;
    if (!aligned16(v) || !aligned16(vq) || !aligned16(v_scale) ||
        (workspace && !aligned16(workspace)))
        return SAGE_ERR_ALIGN;
    if (workspace_bytes < s.v[SAGE_BUF_WS_V]) return SAGE_ERR_WORKSPACE;
    const hipError_t e = sage::launch_quant_v((const sage::u16*)v, B, H, N, d, layout,
                                              pv_dtype == SAGE_PV_FP16, vq, v_scale,
                                              (float*)workspace, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

namespace {

// Validation and launch of one quantization pass; workspace == NULL with
// noalloc: the library's fixed scratch instead.
int quant_qkv_common(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                     int layout, int pv_dtype, int8_t* q8, float* q_scale, int8_t* k8,
                     float* k_scale, float* k_mean, void* vq, float* v_scale, void* workspace,
                     size_t workspace_bytes, int noalloc, void* stream) {
    if (!q || !k || !v || !q8 || !q_scale || !k8 || !k_scale || !k_mean || !vq || !v_scale ||
        (!noalloc && !workspace))
        return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    SAGE_TRY(check_pv(pv_dtype));
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(q_scale) ||
        !aligned16(k8) || !aligned16(k_scale) || !aligned16(k_mean) || !aligned16(vq) ||
        !aligned16(v_scale) || (!noalloc && !aligned16(workspace)))
        return SAGE_ERR_ALIGN;
    const Sizes s = sizes_of(B, H, N, d, pv_dtype);
    const size_t need = s.v[SAGE_BUF_WS_QK] + s.v[SAGE_BUF_WS_V];
    if (noalloc) {
        if (need > sage::kNoAllocScratchBytes) return SAGE_ERR_SCRATCH;
        if (sage::noalloc_scratch((hipStream_t)stream, &workspace) != hipSuccess)
            return SAGE_ERR_HIP;
    } else if (workspace_bytes < need) {
        return SAGE_ERR_WORKSPACE;
    }
    uint64_t* kws = (uint64_t*)workspace;
    float* vws = (float*)((char*)workspace + s.v[SAGE_BUF_WS_QK]);
    const hipError_t e = sage::launch_quant_qkv(
        (const sage::u16*)q, (const sage::u16*)k, (const sage::u16*)v, B, H, N, d, layout,
        pv_dtype == SAGE_PV_FP16, q8, q_scale, k8, k_scale, k_mean, vq, v_scale, kws, vws,
        (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

}  // namespace

__attribute__((visibility("default"))) int sage_quant_qkv(
    const void* q, const void* k, const void* v, int B, int H, int N, int d, int layout,
    int pv_dtype, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, float* k_mean, void* vq,
    float* v_scale, void* workspace, size_t workspace_bytes, void* stream) {
    return quant_qkv_common(q, k, v, B, H, N, d, layout, pv_dtype, q8, q_scale, k8, k_scale,
                            k_mean, vq, v_scale, workspace, workspace_bytes, 0, stream);
}

__attribute__((visibility("default"))) int sage_quant_qkv_noalloc(
    const void* q, const void* k, const void* v, int B, int H, int N, int d, int layout,
    int pv_dtype, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, float* k_mean, void* vq,
    float* v_scale, void* stream) {
    return quant_qkv_common(q, k, v, B, H, N, d, layout, pv_dtype, q8, q_scale, k8, k_scale,
                            k_mean, vq, v_scale, nullptr, 0, 1, stream);
}

__attribute__((visibility("default"))) int sage_attn_fwd(
    const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
    const void* vq, const float* v_scale, int B, int H, int N, int d, int layout, int causal,
    float sm_scale, int pv_dtype, void* out, int out_dtype, void* stream) {
    return attn_common(q8, q_scale, k8, k_scale, vq, v_scale, B, H, N, d, layout, causal, sm_scale,
                       pv_dtype, SAGE_QGRAN_BLOCK, nullptr, 0, nullptr, 0, out, out_dtype, 0, 0, 0,
                       0, 1, nullptr, stream);
}

__attribute__((visibility("default"))) int sage_attn_fwd_lse(
    const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
    const void* vq, const float* v_scale, int B, int H, int N, int d, int layout, int causal,
    float sm_scale, int pv_dtype, void* out, int out_dtype, float* lse, void* stream) {
    if (!lse) return SAGE_ERR_NULL;
    return attn_common(q8, q_scale, k8, k_scale, vq, v_scale, B, H, N, d, layout, causal, sm_scale,
                       pv_dtype, SAGE_QGRAN_BLOCK, nullptr, 0, nullptr, 0, out, out_dtype, 0, 0, 0,
                       0, 1, nullptr, stream, lse);
}

// Workspace of the 8-bit backward, carved in this order, each part 256-byte
// aligned: D [bh][N_pad] f32, s_do [bh][nblk] f32, dO and V in fp16
// [bh][N_pad][d], dO in FP8 and Q, K codes transposed [bh][nblk][d][128],
// the per-tile records of the dK/dV sweep [bh][nblk][512] f32.
static size_t bwd_parts(int B, int H, int N, int d, size_t* off) {
    const size_t bh = (size_t)B * H, nblk = ((size_t)N + sage::kBlk - 1) / sage::kBlk;
    const size_t np = nblk * sage::kBlk;
    const size_t sz[8] = {bh * np * 4, bh * nblk * 4, bh * np * d * 2, bh * np * d * 2,
                          bh * np * d, bh * np * d, bh * np * d, bh * nblk * sage::kRecFloats * 4};
    size_t o = 0;
    for (int i = 0; i < 8; ++i) {
        if (off) off[i] = o;
        o += (sz[i] + 255) / 256 * 256;
    }
    return o;
}

__attribute__((visibility("default"))) int sage_bwd_sizes(int B, int H, int N, int d,
                                                          size_t* workspace_bytes) {
    if (!workspace_bytes) return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    *workspace_bytes = bwd_parts(B, H, N, d, nullptr);
    return SAGE_OK;
}

__attribute__((visibility("default"))) int sage_attn_bwd(
    const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale, const void* v,
    const void* o, const void* dO, const float* lse, int B, int H, int N, int d, int layout,
    int causal, float sm_scale, float* dq, float* dk, float* dv, void* workspace,
    size_t workspace_bytes, void* stream) {
    if (!q8 || !q_scale || !k8 || !k_scale || !v || !o || !dO || !lse || !dq || !dk || !dv ||
        !workspace)
        return SAGE_ERR_NULL;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    if (causal != 0 && causal != 1) return SAGE_ERR_INVALID;
    if (!(isfinite(sm_scale) && sm_scale > 0.0f)) return SAGE_ERR_INVALID;
    if (!aligned16(q8) || !aligned16(q_scale) || !aligned16(k8) || !aligned16(k_scale) ||
        !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(lse) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || ((uintptr_t)workspace & 255u))
        return SAGE_ERR_ALIGN;
    size_t off[8];
    if (workspace_bytes < bwd_parts(B, H, N, d, off)) return SAGE_ERR_WORKSPACE;
    uint8_t* ws = (uint8_t*)workspace;
    sage::BwdPrep pp;
    pp.o = (const sage::u16*)o;
    pp.dO = (const sage::u16*)dO;
    pp.v = (const sage::u16*)v;
    sage::BwdArgs a;
    a.q8 = q8;
    a.q_scale = q_scale;
    a.k8 = k8;
    a.k_scale = k_scale;
    a.lse = lse;
    a.Dq = (float*)(ws + off[0]);
    a.s_do = (float*)(ws + off[1]);
    a.do16 = (_Float16*)(ws + off[2]);
    a.v16 = (_Float16*)(ws + off[3]);
    a.do8 = ws + off[4];
    a.qT8 = (int8_t*)(ws + off[5]);
    a.kT8 = (int8_t*)(ws + off[6]);
    a.rec = (float*)(ws + off[7]);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.H = H;
    a.N = N;
    a.nblk = (N + sage::kBlk - 1) / sage::kBlk;
    a.N_pad = a.nblk * sage::kBlk;
    a.total = 0;  // set by the launcher
    a.layout = layout;
    a.lambda = (float)((double)sm_scale * 1.4426950408889634);
    a.sm_scale = sm_scale;
    const hipError_t e = sage::launch_attn_bwd(pp, a, B, d, causal, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

__attribute__((visibility("default"))) int sage_attn_fwd_ex(
    const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
    const void* vq, const float* v_scale, int B, int H, int N, int d, int layout, int causal,
    float sm_scale, int pv_dtype, int q_gran, void* out, int out_dtype, void* stream) {
    return attn_common(q8, q_scale, k8, k_scale, vq, v_scale, B, H, N, d, layout, causal, sm_scale,
                       pv_dtype, q_gran, nullptr, 0, nullptr, 0, out, out_dtype, 0, 0, 0, 0, 1,
                       nullptr, stream);
}

__attribute__((visibility("default"))) int sage_attn_fwd_sparse(
    const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
    const void* vq, const float* v_scale, int B, int H, int N, int d, int layout, int causal,
    float sm_scale, int pv_dtype, int q_gran, const uint8_t* tile_mask, void* out,
    int out_dtype, void* stream) {
    return attn_common(q8, q_scale, k8, k_scale, vq, v_scale, B, H, N, d, layout, causal, sm_scale,
                       pv_dtype, q_gran, tile_mask, 1, nullptr, 0, out, out_dtype, 0, 0, 0, 0, 1,
                       nullptr, stream);
}

__attribute__((visibility("default"))) int sage_attn_fwd_smooth(
    const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
    const void* vq, const float* v_scale, int B, int H, int N, int d, int layout, int causal,
    float sm_scale, int pv_dtype, int q_gran, const float* bias, const uint8_t* tile_mask,
    void* out, int out_dtype, void* stream) {
    return attn_common(q8, q_scale, k8, k_scale, vq, v_scale, B, H, N, d, layout, causal, sm_scale,
                       pv_dtype, q_gran, tile_mask, tile_mask != nullptr, bias, 1, out, out_dtype,
                       0, 0, 0, 0, 1, nullptr, stream);
}

__attribute__((visibility("default"))) int sage_attn_fwd_debug(
    const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
    const void* vq, const float* v_scale, int B, int H, int N, int d, int layout, int causal,
    float sm_scale, int pv_dtype, void* out, int out_dtype, int b, int h, int row0, int nrows,
    int32_t* s_out, void* stream) {
    return attn_common(q8, q_scale, k8, k_scale, vq, v_scale, B, H, N, d, layout, causal, sm_scale,
                       pv_dtype, SAGE_QGRAN_BLOCK, nullptr, 0, nullptr, 0, out, out_dtype, 1, b,
                       h, row0, nrows, s_out, stream);
}

static bool mx_fmt_ok(int fmt) { return fmt == SAGE_MX_FP6 || fmt == SAGE_MX_FP4; }

__attribute__((visibility("default"))) int sage_quant_qk_mx_fmt(const void* q, const void* k, int B,
                                                                int H, int N, int d, int layout,
                                                                int fmt, uint8_t* q6, uint8_t* k6,
                                                                float* k_mean, void* workspace,
                                                                size_t workspace_bytes,
                                                                void* stream) {
    if (!q || !k || !q6 || !k6 || !k_mean || !workspace) return SAGE_ERR_NULL;
    if (!mx_fmt_ok(fmt)) return SAGE_ERR_INVALID;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    if (!aligned16(q) || !aligned16(k) || !aligned16(q6) || !aligned16(k6) || !aligned16(k_mean) ||
        !aligned16(workspace))
        return SAGE_ERR_ALIGN;
    const Sizes s = sizes_of(B, H, N, d, SAGE_PV_FP8);
    if (workspace_bytes < s.v[SAGE_BUF_WS_QK]) return SAGE_ERR_WORKSPACE;
    const hipError_t e = sage::launch_quant_qk_mx((const sage::u16*)q, (const sage::u16*)k, B, H, N,
                                                  d, layout, fmt, q6, k6, k_mean,
                                                  (uint64_t*)workspace, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

__attribute__((visibility("default"))) int sage_quant_qk_mx(const void* q, const void* k, int B,
                                                            int H, int N, int d, int layout,
                                                            uint8_t* q6, uint8_t* k6,
                                                            float* k_mean, void* workspace,
                                                            size_t workspace_bytes,
                                                            void* stream) {
    return sage_quant_qk_mx_fmt(q, k, B, H, N, d, layout, SAGE_MX_FP6, q6, k6, k_mean, workspace,
                                workspace_bytes, stream);
}

__attribute__((visibility("default"))) int sage_quant_v_mx_fmt(const void* v, int B, int H, int N,
                                                               int d, int layout, int fmt,
                                                               uint8_t* v6, void* stream) {
    if (!v || !v6) return SAGE_ERR_NULL;
    if (!mx_fmt_ok(fmt)) return SAGE_ERR_INVALID;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    if (!aligned16(v) || !aligned16(v6)) return SAGE_ERR_ALIGN;
    const hipError_t e = sage::launch_quant_v_mx((const sage::u16*)v, B, H, N, d, layout, fmt, v6,
                                                 (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

__attribute__((visibility("default"))) int sage_quant_v_mx(const void* v, int B, int H, int N, int d,
                                                           int layout, uint8_t* v6, void* stream) {
    return sage_quant_v_mx_fmt(v, B, H, N, d, layout, SAGE_MX_FP6, v6, stream);
}

__attribute__((visibility("default"))) int sage_attn_fwd_mx_fmt(const uint8_t* q6, const uint8_t* k6,
                                                                const uint8_t* v6, int B, int H,
                                                                int N, int d, int layout, int fmt,
                                                                int causal, float sm_scale,
                                                                void* out, int out_dtype,
                                                                void* stream) {
    if (!q6 || !k6 || !v6 || !out) return SAGE_ERR_NULL;
    if (!mx_fmt_ok(fmt)) return SAGE_ERR_INVALID;
    SAGE_TRY(check_dims(B, H, N, d));
    SAGE_TRY(check_layout(layout));
    if (causal != 0 && causal != 1) return SAGE_ERR_INVALID;
    if (out_dtype != SAGE_OUT_BF16 && out_dtype != SAGE_OUT_FP32) return SAGE_ERR_INVALID;
    if (!(isfinite(sm_scale) && sm_scale > 0.0f)) return SAGE_ERR_INVALID;
    if (!aligned16(q6) || !aligned16(k6) || !aligned16(v6) || !aligned16(out)) return SAGE_ERR_ALIGN;
    sage::AttnArgs a = {};
    a.q8 = (const int8_t*)q6;
    a.k8 = (const int8_t*)k6;
    a.vq = v6;
    a.out = out;
    a.H = H;
    a.N = N;
    a.nblk = (N + sage::kBlk - 1) / sage::kBlk;
    a.N_pad = a.nblk * sage::kBlk;
    a.layout = layout;
    a.out_fp32 = out_dtype == SAGE_OUT_FP32;
    a.lambda = (float)((double)sm_scale * 1.4426950408889634);
    const hipError_t e = sage::launch_attn_mx(a, B, d, causal, fmt, (hipStream_t)stream);
    return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

__attribute__((visibility("default"))) int sage_attn_fwd_mx(const uint8_t* q6, const uint8_t* k6,
                                                            const uint8_t* v6, int B, int H, int N,
                                                            int d, int layout, int causal,
                                                            float sm_scale, void* out,
                                                            int out_dtype, void* stream) {
    return sage_attn_fwd_mx_fmt(q6, k6, v6, B, H, N, d, layout, SAGE_MX_FP6, causal, sm_scale, out,
                                out_dtype, stream);
}

__attribute__((visibility("default"))) const char* sage_status_string(int status) {
    switch (status) {
        case SAGE_OK: return "SAGE_OK";
        case SAGE_ERR_NULL: return "SAGE_ERR_NULL: a required pointer is NULL";
        case SAGE_ERR_INVALID: return "SAGE_ERR_INVALID: invalid argument";
        case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED: head dimension must be 64 or 128";
        case SAGE_ERR_ALIGN: return "SAGE_ERR_ALIGN: device buffers must be 16-byte aligned";
        case SAGE_ERR_SIZE: return "SAGE_ERR_SIZE: problem exceeds the supported size";
        case SAGE_ERR_HIP: return "SAGE_ERR_HIP: a HIP launch failed";
        case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE: workspace too small";
        case SAGE_ERR_SCRATCH:
            return "SAGE_ERR_SCRATCH: the problem needs more than the library's fixed 32 MiB "
                   "scratch (use sage_quant_qkv with a workspace)";
        default: return "SAGE_ERR_UNKNOWN";
    }
}

}  // extern "C"
