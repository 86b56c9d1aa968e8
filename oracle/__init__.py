"""CPU oracle for SageAttention-style INT8-QK / FP8-PV attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It is a thin
ctypes wrapper (argument marshalling, per-head slicing) around
``sage_oracle.c``, a plain single-threaded C implementation of the quantized
method; the arithmetic and the readings of the pages are documented there.
It shares no code with the HIP path and imports nothing from it.

Arrays are numpy; bf16 tensors are passed as ``uint16`` code arrays in the
layout ``[B, H, N, d]`` (callers convert from other layouts first).
"""
from __future__ import annotations

import ctypes as ct
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "sage_oracle.c"), os.path.join(_HERE, "sage_oracle_mx.c"),
         os.path.join(_HERE, "sage_oracle_bwd.c")]
_LIB_PATH = os.path.join(_HERE, "libsage_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra"]

_lib = None

# Block / tile constants of the method (reading: 128, the only block size the
# pages give; the key tile of the online softmax equals the K block).
BLK = 128
BC = 128
P_SCALE = 448.0


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or _stale():
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _stale() -> bool:
    return not os.path.exists(_LIB_PATH) or any(
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(src) for src in _SRCS)


def lib():
    global _lib
    if _lib is None:
        if _stale():
            build(force=True)
        L = ct.CDLL(_LIB_PATH)
        P = ct.c_void_p
        i32, i64, f32, f64 = ct.c_int, ct.c_int64, ct.c_float, ct.c_double
        sigs = {
            "or_bf16_to_f32_n": [P, i64, P], "or_f32_to_bf16_n": [P, i64, P],
            "or_e4m3_to_f32_n": [P, i64, P], "or_f32_to_e4m3_n": [P, i64, P],
            "or_f16_to_f32_n": [P, i64, P], "or_f32_to_f16_n": [P, i64, P],
            "or_fix30_n": [P, i64, P],
            "or_k_mean": [P, i32, i32, P],
            "or_quant_block": [P, i32, i32, P, P],
            "or_quant_q": [P, i32, i32, i32, P, P, P],
            "or_quant_q_smooth": [P, i32, i32, i32, P, P, P, P],
            "or_q_smooth_bias": [P, P, P, i32, i32, f32, i32, i32, P],
            "or_quant_k": [P, i32, i32, i32, i32, P, P, P, P],
            "or_quant_v": [P, i32, i32, i32, P, P],
            "or_dump_s": [P, P, i32, i32, i32, i32, i32, P],
            "or_attn_rows": [P, P, P, P, P, P, i32, i32, P, i32, i32, f32, i32, i32, i32, i32, P, P,
                             P, P, P, P, P],
            "or_ref64_rows": [P, P, P, i32, i32, P, i32, i32, f64, P, P],
            "or_f32_to_mx_n": [i32, P, i64, P], "or_mx_to_f32_n": [i32, P, i64, P],
            "or_mx_blocks_n": [i32, P, i64, P, P],
            "or_mx_quant_rows": [i32, P, P, i32, i32, P, P, P],
            "or_mx_quant_v": [i32, P, i32, i32, P, P, P],
            "or_mx_attn_rows": [i32, P, P, P, P, P, P, i32, i32, P, i32, i32, f32, P, P, P, P],
            "or_bf16_to_f16f_n": [P, i64, P],
            "or_bwd_prep": [P, P, i32, i32, P, P, P],
            "or_bwd_dq_block": [P, P, P, P, P, P, P, P, i32, i32, i32, f32, i32, P, P],
            "or_bwd_dkdv_block": [P, P, P, P, P, P, P, P, P, P, i32, i32, i32, f32, i32, P, P, P],
            "or_bwd_ref64": [P, P, P, P, i32, i32, i32, f64, P, P, P, P],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = None
        L.or_lambda.argtypes = [f32]
        L.or_lambda.restype = f32
        L.or_mx_dot.argtypes = [i32, P, P, P, P, i32]
        L.or_mx_dot.restype = f32
        L.or_bwd_tile_pd.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, f32, i32, i32, P, P]
        L.or_bwd_tile_pd.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ct.c_void_p)


# --------------------------------------------------------------------------- codecs
def _codec(name, x, in_dtype, out_dtype):
    x = np.ascontiguousarray(x, dtype=in_dtype)
    out = np.empty(x.shape, dtype=out_dtype)
    getattr(lib(), name)(_p(x), x.size, _p(out))
    return out


def bf16_to_f32(x):
    return _codec("or_bf16_to_f32_n", x, np.uint16, np.float32)


def f32_to_bf16(x):
    return _codec("or_f32_to_bf16_n", x, np.float32, np.uint16)


def e4m3_to_f32(x):
    return _codec("or_e4m3_to_f32_n", x, np.uint8, np.float32)


def f32_to_e4m3(x):
    return _codec("or_f32_to_e4m3_n", x, np.float32, np.uint8)


def f16_to_f32(x):
    return _codec("or_f16_to_f32_n", x, np.uint16, np.float32)


def f32_to_f16(x):
    return _codec("or_f32_to_f16_n", x, np.float32, np.uint16)


def fix30(x):
    return _codec("or_fix30_n", x, np.float32, np.int64)


def lam(sm_scale: float) -> float:
    """sm_scale * log2(e) rounded once to fp32."""
    return float(lib().or_lambda(sm_scale))


# --------------------------------------------------------------------- quantization
def k_mean_head(k_head: np.ndarray) -> np.ndarray:
    k_head = np.ascontiguousarray(k_head, dtype=np.uint16)
    N, d = k_head.shape
    out = np.empty(d, np.float32)
    lib().or_k_mean(_p(k_head), N, d, _p(out))
    return out


def quant_block(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, d = x.shape
    out = np.empty((rows, d), np.int8)
    s = np.empty(1, np.float32)
    lib().or_quant_block(_p(x), rows, d, _p(out), _p(s))
    return out, float(s[0])


def quant_qk(q: np.ndarray, k: np.ndarray, blk: int = BLK, smooth: bool = True,
             q_gran: str = "block", q_smooth: bool = False):
    """q, k: uint16 bf16 codes [B, H, N, d].  Returns a dict with q8/k8 int8
    [B,H,N,d], q_scale fp32 [B,H,ceil(N/qblk)], k_scale fp32 [B,H,nblk],
    k_mean fp32 [B,H,d] and qblk.  q_gran "block": Q blocks of blk rows like
    K; "token": one scale per query row (qblk = 1).  q_smooth: Q is smoothed
    by its per-block token mean first (q_mean fp32 [B,H,nblk,d] is added to
    the dict; the scores need smooth_bias then)."""
    B, H, N, d = q.shape
    assert blk == BLK or not q_smooth
    qblk = {"block": blk, "token": 1}[q_gran]
    nb = (N + blk - 1) // blk
    nbq = (N + qblk - 1) // qblk
    q8 = np.empty((B, H, N, d), np.int8)
    k8 = np.empty((B, H, N, d), np.int8)
    qs = np.empty((B, H, nbq), np.float32)
    ks = np.empty((B, H, nb), np.float32)
    km = np.empty((B, H, d), np.float32)
    qm = np.empty((B, H, nb, d), np.float32)
    tmp = np.empty(blk * d, np.float32)
    L = lib()
    for b in range(B):
        for h in range(H):
            qh = np.ascontiguousarray(q[b, h], dtype=np.uint16)
            kh = np.ascontiguousarray(k[b, h], dtype=np.uint16)
            q8h = np.empty((N, d), np.int8)
            k8h = np.empty((N, d), np.int8)
            qsh = np.empty(nbq, np.float32)
            ksh = np.empty(nb, np.float32)
            kmh = np.empty(d, np.float32)
            if q_smooth:
                qmh = np.empty((nb, d), np.float32)
                L.or_quant_q_smooth(_p(qh), N, d, qblk, _p(q8h), _p(qsh), _p(qmh), _p(tmp))
                qm[b, h] = qmh
            else:
                L.or_quant_q(_p(qh), N, d, qblk, _p(q8h), _p(qsh), _p(tmp))
            L.or_quant_k(_p(kh), N, d, blk, int(smooth), _p(k8h), _p(ksh), _p(kmh), _p(tmp))
            q8[b, h], k8[b, h], qs[b, h], ks[b, h], km[b, h] = q8h, k8h, qsh, ksh, kmh
    out = dict(q8=q8, q_scale=qs, k8=k8, k_scale=ks, k_mean=km, qblk=qblk)
    if q_smooth:
        out["q_mean"] = qm
    return out


def smooth_bias(qz: dict, k: np.ndarray, sm_scale: float, blocks=None) -> np.ndarray:
    """The Q-smoothing correction of every head: fp32 [B, H, nblk, N] (block
    r, key j) from qz["q_mean"], qz["k_mean"] and the bf16 K codes.  With
    ``blocks`` (a list of block indices) only those rows are computed; the
    others are left NaN."""
    B, H, N, d = k.shape
    nb = (N + BLK - 1) // BLK
    blocks = range(nb) if blocks is None else sorted(set(int(r) for r in blocks))
    out = np.full((B, H, nb, N), np.nan, np.float32)
    L = lib()
    for b in range(B):
        for h in range(H):
            qmh = np.ascontiguousarray(qz["q_mean"][b, h], np.float32)
            kh = np.ascontiguousarray(k[b, h], np.uint16)
            kmh = np.ascontiguousarray(qz["k_mean"][b, h], np.float32)
            row = np.empty(N, np.float32)
            for r in blocks:
                L.or_q_smooth_bias(_p(qmh), _p(kh), _p(kmh), N, d, float(sm_scale), r, r + 1,
                                   _p(row))
                out[b, h, r] = row
    return out


def quant_v(v: np.ndarray, pv: str = "fp8"):
    """v: uint16 bf16 codes [B,H,N,d].  Returns v codes in natural [B,H,N,d]
    order (uint8 e4m3 for fp8, uint16 binary16 for fp16) and v_scale [B,H,d]."""
    B, H, N, d = v.shape
    fp16 = pv == "fp16"
    vq = np.empty((B, H, N, d), np.uint16 if fp16 else np.uint8)
    vs = np.empty((B, H, d), np.float32)
    L = lib()
    for b in range(B):
        for h in range(H):
            vh = np.ascontiguousarray(v[b, h], dtype=np.uint16)
            vqh = np.empty((N, d), vq.dtype)
            vsh = np.empty(d, np.float32)
            L.or_quant_v(_p(vh), N, d, int(fp16), _p(vqh), _p(vsh))
            vq[b, h], vs[b, h] = vqh, vsh
    return vq, vs


# ------------------------------------------------------------------------ attention
def dump_s(q8h: np.ndarray, k8h: np.ndarray, row0: int, nrows: int, causal: bool = False):
    """Integer Q K^T of one head, rows [row0, row0+nrows), all keys (int32 [nrows, N])."""
    q8h = np.ascontiguousarray(q8h, np.int8)
    k8h = np.ascontiguousarray(k8h, np.int8)
    N, d = k8h.shape
    out = np.empty((nrows, N), np.int32)
    lib().or_dump_s(_p(q8h), _p(k8h), N, d, row0, nrows, int(causal), _p(out))
    return out


def attn_rows_head(qz: dict, vq, vs, b: int, h: int, rows, causal: bool, sm_scale: float,
                   pv: str = "fp8", blk: int = BLK, bc: int = BC, return_ml: bool = False,
                   tile_mask=None, bias=None, return_lx: bool = False):
    """Quantized attention for query rows ``rows`` of head (b, h): fp32 [len(rows), d].
    tile_mask: None (dense) or uint8 [B, H, ceil(N/128), ceil(N/bc)], nonzero =
    the query block visits the key tile.  bias: None, or the Q-smoothing
    correction fp32 [B, H, ceil(N/128), N] of smooth_bias.  return_ml: also the
    final running max m and row sum l (of the quantized P) per row; return_lx:
    also lx, the row sum of the unquantized p (the log-sum-exp's)."""
    q8h = np.ascontiguousarray(qz["q8"][b, h])
    k8h = np.ascontiguousarray(qz["k8"][b, h])
    qsh = np.ascontiguousarray(qz["q_scale"][b, h])
    ksh = np.ascontiguousarray(qz["k_scale"][b, h])
    vqh = np.ascontiguousarray(vq[b, h])
    vsh = np.ascontiguousarray(vs[b, h])
    N, d = k8h.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    out = np.empty((len(rows), d), np.float32)
    m = np.empty(len(rows), np.float32)
    l = np.empty(len(rows), np.float32)
    lx = np.empty(len(rows), np.float32)
    scratch = np.empty(4 * bc + 3 * d, np.float32)
    qblk = int(qz.get("qblk", blk))
    tm = None
    if tile_mask is not None:
        tm = np.ascontiguousarray(tile_mask[b, h], np.uint8)
        assert tm.shape == ((N + 127) // 128, (N + bc - 1) // bc), tm.shape
    bs = None
    if bias is not None:
        bs = np.ascontiguousarray(bias[b, h], np.float32)
        assert bs.shape == ((N + 127) // 128, N), bs.shape
    lib().or_attn_rows(_p(q8h), _p(qsh), _p(k8h), _p(ksh), _p(vqh), _p(vsh), N, d, _p(rows),
                       len(rows), int(causal), float(sm_scale), int(pv == "fp16"), qblk, blk, bc,
                       None if tm is None else _p(tm), None if bs is None else _p(bs), _p(out),
                       _p(m), _p(l), _p(lx), _p(scratch))
    if return_lx:
        return out, m, l, lx
    if return_ml:
        return out, m, l
    return out


def ref64_rows_head(q, k, v, b: int, h: int, rows, causal: bool, sm_scale: float):
    """Exact softmax attention in FP64 from the bf16 inputs (uint16 codes)."""
    qh = np.ascontiguousarray(q[b, h], np.uint16)
    kh = np.ascontiguousarray(k[b, h], np.uint16)
    vh = np.ascontiguousarray(v[b, h], np.uint16)
    N, d = kh.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    out = np.empty((len(rows), d), np.float64)
    scratch = np.empty(N, np.float64)
    lib().or_ref64_rows(_p(qh), _p(kh), _p(vh), N, d, _p(rows), len(rows), int(causal),
                        float(sm_scale), _p(out), _p(scratch))
    return out


def attention(q, k, v, causal: bool, sm_scale: float, pv: str = "fp8", rows=None,
              q_gran: str = "block", tile_mask=None, q_smooth: bool = False):
    """Whole oracle pipeline: quantize, then attention for ``rows`` (default all)
    of every head.  Returns (out fp32 [B,H,len(rows),d], quantized dict, vq, vs);
    with q_smooth the dict also holds the correction under "bias"."""
    B, H, N, d = q.shape
    qz = quant_qk(q, k, q_gran=q_gran, q_smooth=q_smooth)
    if q_smooth:
        qz["bias"] = smooth_bias(qz, k, sm_scale)
    vq, vs = quant_v(v, pv)
    rows = np.arange(N, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    out = np.empty((B, H, len(rows), d), np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = attn_rows_head(qz, vq, vs, b, h, rows, causal, sm_scale, pv,
                                       tile_mask=tile_mask, bias=qz.get("bias"))
    return out, qz, vq, vs


# ---------------------------------------------------------- microscaled variant
MX_FMT = {"mxfp4": 4, "mxfp6": 6}


def f32_to_mx(x, fmt="mxfp6"):
    """fp32 -> MX element codes (one per byte): E2M1 for mxfp4, E2M3 for mxfp6."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().or_f32_to_mx_n(MX_FMT[fmt], _p(x), x.size, _p(out))
    return out


def mx_to_f32(c, fmt="mxfp6"):
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().or_mx_to_f32_n(MX_FMT[fmt], _p(c), c.size, _p(out))
    return out


def mx_blocks(x, fmt="mxfp6"):
    """MX quantization of consecutive blocks of 32 fp32 values: (codes uint8
    [..., 32] one element code per byte, E8M0 bytes [...])."""
    x = np.ascontiguousarray(x, np.float32).reshape(-1, 32)
    codes = np.empty(x.shape, np.uint8)
    eb = np.empty(x.shape[0], np.uint8)
    lib().or_mx_blocks_n(MX_FMT[fmt], _p(x), x.shape[0], _p(codes), _p(eb))
    return codes, eb


def mx_dequant(codes, ebytes, fmt="mxfp6"):
    """Values of element codes times 2^(e - 127); ebytes broadcast against codes."""
    return mx_to_f32(codes, fmt).astype(np.float64) * np.exp2(ebytes.astype(np.float64) - 127.0)


def mx_quant_qk(q: np.ndarray, k: np.ndarray, fmt="mxfp6"):
    """q, k: uint16 bf16 codes [B, H, N, d].  MX per token and 32 channels,
    K smoothed by its token mean first.  Returns q_c/k_c (one element code per
    byte, [B,H,N,d]), q_e/k_e (E8M0 bytes [B,H,N,d/32]) and k_mean."""
    B, H, N, d = q.shape
    f = MX_FMT[fmt]
    out = {key: np.empty((B, H, N, d), np.uint8) for key in ("q_c", "k_c")}
    out.update({key: np.empty((B, H, N, d // 32), np.uint8) for key in ("q_e", "k_e")})
    out["k_mean"] = np.empty((B, H, d), np.float32)
    out["fmt"] = fmt
    tmp = np.empty(d, np.float32)
    L = lib()
    for b in range(B):
        for h in range(H):
            qh = np.ascontiguousarray(q[b, h], np.uint16)
            kh = np.ascontiguousarray(k[b, h], np.uint16)
            km = np.empty(d, np.float32)
            L.or_k_mean(_p(kh), N, d, _p(km))
            for key, src, mean in (("q", qh, None), ("k", kh, km)):
                c = np.empty((N, d), np.uint8)
                e = np.empty((N, d // 32), np.uint8)
                L.or_mx_quant_rows(f, _p(src), None if mean is None else _p(mean), N, d, _p(c),
                                   _p(e), _p(tmp))
                out[key + "_c"][b, h], out[key + "_e"][b, h] = c, e
            out["k_mean"][b, h] = km
    return out


def mx_quant_v(v: np.ndarray, fmt="mxfp6"):
    """v: uint16 bf16 codes [B,H,N,d].  MX per channel and 32 keys:
    (v_c codes [B,H,N,d], v_e E8M0 bytes [B,H,ceil(N/32),d])."""
    B, H, N, d = v.shape
    nb = (N + 31) // 32
    vc = np.empty((B, H, N, d), np.uint8)
    ve = np.empty((B, H, nb, d), np.uint8)
    tmp = np.empty(32, np.float32)
    for b in range(B):
        for h in range(H):
            vh = np.ascontiguousarray(v[b, h], np.uint16)
            c = np.empty((N, d), np.uint8)
            e = np.empty((nb, d), np.uint8)
            lib().or_mx_quant_v(MX_FMT[fmt], _p(vh), N, d, _p(c), _p(e), _p(tmp))
            vc[b, h], ve[b, h] = c, e
    return vc, ve


def mx_attn_rows_head(mz: dict, v_c, v_e, b: int, h: int, rows, causal: bool, sm_scale: float,
                      return_ml: bool = False):
    """MX attention for query rows ``rows`` of head (b, h): fp32 [len(rows), d]."""
    hd = {key: np.ascontiguousarray(mz[key][b, h]) for key in ("q_c", "q_e", "k_c", "k_e")}
    vch, veh = np.ascontiguousarray(v_c[b, h]), np.ascontiguousarray(v_e[b, h])
    N, d = hd["k_c"].shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    out = np.empty((len(rows), d), np.float32)
    m = np.empty(len(rows), np.float32)
    l = np.empty(len(rows), np.float32)
    scratch = np.empty(3 * 128 + 2 * d, np.float32)
    lib().or_mx_attn_rows(MX_FMT[mz["fmt"]], _p(hd["q_c"]), _p(hd["q_e"]), _p(hd["k_c"]),
                          _p(hd["k_e"]), _p(vch), _p(veh), N, d, _p(rows), len(rows), int(causal),
                          float(sm_scale), _p(out), _p(m), _p(l), _p(scratch))
    if return_ml:
        return out, m, l
    return out


def mx_attention(q, k, v, causal: bool, sm_scale: float, rows=None, fmt="mxfp6"):
    """Whole MX pipeline for ``rows`` (default all) of every head: (out fp32
    [B,H,len(rows),d], quantized dict, v_c, v_e)."""
    B, H, N, d = q.shape
    mz = mx_quant_qk(q, k, fmt)
    vc, ve = mx_quant_v(v, fmt)
    rows = np.arange(N, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    out = np.empty((B, H, len(rows), d), np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = mx_attn_rows_head(mz, vc, ve, b, h, rows, causal, sm_scale)
    return out, mz, vc, ve


# ------------------------------------------------------------- 8-bit backward
def lse2_from_ml(m, l):
    """The forward's log-sum-exp in the exp2 domain: lse2 = fp32(mu + log2(l))
    with mu = fp32(m - log2 448) (log2 rounded once to fp32), l the row sum of
    the unquantized p."""
    mu = (np.asarray(m, np.float32) - np.float32(np.log2(P_SCALE))).astype(np.float32)
    return (mu + np.log2(np.asarray(l, np.float64)).astype(np.float32)).astype(np.float32)


def train_forward_head(qz: dict, vq, vs, b: int, h: int, rows, causal: bool, sm_scale: float):
    """The training forward for ``rows`` of head (b, h): the bf16 output (uint16
    codes, as a training step keeps it) and lse2 per row."""
    out, m, _, lx = attn_rows_head(qz, vq, vs, b, h, rows, causal, sm_scale, "fp8", return_lx=True)
    return f32_to_bf16(out), lse2_from_ml(m, lx)


def bwd_prep_head(o, dO):
    """Per head (uint16 bf16 [N, d] each): D [N] fp32, dO FP8 codes [N, d] and
    the per-block FP8 scales [ceil(N/128)]."""
    o = np.ascontiguousarray(o, np.uint16)
    dO = np.ascontiguousarray(dO, np.uint16)
    N, d = dO.shape
    Dq = np.empty(N, np.float32)
    do8 = np.empty((N, d), np.uint8)
    s_do = np.empty(-(-N // BLK), np.float32)
    lib().or_bwd_prep(_p(o), _p(dO), N, d, _p(Dq), _p(do8), _p(s_do))
    return Dq, do8, s_do


def _f16f(x):
    x = np.ascontiguousarray(x, np.uint16)
    out = np.empty(x.shape, np.float32)
    lib().or_bf16_to_f16f_n(_p(x), x.size, _p(out))
    return out


def bwd_head(qz: dict, v, o, dO, lse2, b: int, h: int, causal: bool, sm_scale: float,
             qblocks=None, kblocks=None):
    """The 8-bit backward of head (b, h) (sage_oracle_bwd.c): dq for the query
    blocks ``qblocks`` and dk, dv for the key blocks ``kblocks`` (default all),
    as dicts block -> fp32 [rows, d].  v, o, dO: uint16 bf16 [N, d] of the
    head; lse2 [N] from train_forward_head (only the rows the blocks need
    are read: dq of a query block needs its rows, dk/dv all rows)."""
    q8 = np.ascontiguousarray(qz["q8"][b, h])
    k8 = np.ascontiguousarray(qz["k8"][b, h])
    qs = np.ascontiguousarray(qz["q_scale"][b, h])
    ks = np.ascontiguousarray(qz["k_scale"][b, h])
    N, d = k8.shape
    nblk = -(-N // BLK)
    v16, do16 = _f16f(v), _f16f(dO)
    Dq, do8, s_do = bwd_prep_head(o, dO)
    lse2 = np.ascontiguousarray(lse2, np.float32)
    scratch = np.empty(2 * BLK * BLK + BLK * BLK // 4 + d, np.float32)
    L = lib()
    dq, dk, dv = {}, {}, {}
    for qb in (range(nblk) if qblocks is None else qblocks):
        rows = min(BLK, N - qb * BLK)
        out = np.empty((rows, d), np.float32)
        L.or_bwd_dq_block(_p(q8), _p(qs), _p(k8), _p(ks), _p(v16), _p(do16), _p(lse2), _p(Dq), N, d,
                          int(causal), float(sm_scale), int(qb), _p(out), _p(scratch))
        dq[qb] = out
    for kb in (range(nblk) if kblocks is None else kblocks):
        rows = min(BLK, N - kb * BLK)
        ok, ov = np.empty((rows, d), np.float32), np.empty((rows, d), np.float32)
        L.or_bwd_dkdv_block(_p(q8), _p(qs), _p(k8), _p(ks), _p(v16), _p(do16), _p(do8), _p(s_do),
                            _p(lse2), _p(Dq), N, d, int(causal), float(sm_scale), int(kb), _p(ok),
                            _p(ov), _p(scratch))
        dk[kb], dv[kb] = ok, ov
    return dq, dk, dv


def bwd_tile_head(qz: dict, v, o, dO, lse2, b: int, h: int, causal: bool, sm_scale: float,
                  qb: int, kb: int):
    """P and dS (fp32 [rows of qb, keys of kb]) of one tile pair of the backward,
    or None when the pair is wholly masked."""
    q8 = np.ascontiguousarray(qz["q8"][b, h])
    k8 = np.ascontiguousarray(qz["k8"][b, h])
    qs = np.ascontiguousarray(qz["q_scale"][b, h])
    ks = np.ascontiguousarray(qz["k_scale"][b, h])
    N, d = k8.shape
    v16, do16 = _f16f(v), _f16f(dO)
    Dq, _, _ = bwd_prep_head(o, dO)
    nq, nk = min(BLK, N - qb * BLK), min(BLK, N - kb * BLK)
    P = np.empty((nq, nk), np.float32)
    dS = np.empty((nq, nk), np.float32)
    ok = lib().or_bwd_tile_pd(_p(q8), _p(qs), _p(k8), _p(ks), _p(v16), _p(do16),
                              _p(np.ascontiguousarray(lse2, np.float32)), _p(Dq), N, d, int(causal),
                              float(sm_scale), int(qb), int(kb), _p(P), _p(dS))
    return (P, dS) if ok else None


def train_step_head(q, k, v, dO, b: int, h: int, causal: bool, sm_scale: float):
    """Whole training step of one small head through the oracle: quantization,
    forward (all rows), backward (all blocks).  Returns (o bf16 codes [N, d],
    lse2 [N], dq, dk, dv fp32 [N, d])."""
    qz = quant_qk(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1])
    vq, vs = quant_v(v[b:b + 1, h:h + 1], "fp8")
    N = q.shape[2]
    o, lse2 = train_forward_head(qz, vq, vs, 0, 0, np.arange(N), causal, sm_scale)
    dq, dk, dv = bwd_head(qz, v[b, h], o, dO[b, h], lse2, 0, 0, causal, sm_scale)
    cat = lambda dct: np.concatenate([dct[i] for i in sorted(dct)])
    return o, lse2, cat(dq), cat(dk), cat(dv)


def bwd_ref64_head(q, k, v, dO, b: int, h: int, causal: bool, sm_scale: float):
    """FP64 gradients of plain softmax attention (no quantization) for head
    (b, h): dq, dk, dv [N, d]."""
    qh, kh, vh, dh = (np.ascontiguousarray(x[b, h], np.uint16) for x in (q, k, v, dO))
    N, d = qh.shape
    dq, dk, dv = (np.empty((N, d), np.float64) for _ in range(3))
    scratch = np.empty(2 * N, np.float64)
    lib().or_bwd_ref64(_p(qh), _p(kh), _p(vh), _p(dh), N, d, int(causal), float(sm_scale), _p(dq),
                       _p(dk), _p(dv), _p(scratch))
    return dq, dk, dv
