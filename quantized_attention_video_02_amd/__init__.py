"""libsage: SageAttention-style INT8-QK / FP8-PV attention on MI355X (gfx950).

A thin ctypes binding over the C ABI declared in ``include/sage.h``: every step
of the computation runs in the library's HIP kernels; this module only
marshals arguments.  PyTorch is used for device memory and the current stream.

Two-line drop-in use::

    import quantized_attention_video_02_amd as sage
    out = sage.attn(q, k, v)            # q, k, v: bf16 [B, H, N, d] on the GPU

The library must be built first (``python -m quantized_attention_video_02_amd.build``);
there is no fallback: without libsage.so every call raises.
"""
from __future__ import annotations

import ctypes as ct
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsage.so")

SAGE_OK = 0
LAYOUTS = {"HND": 0, "NHD": 1}
PV = {"fp8": 0, "fp16": 1}
OUT = {torch.bfloat16: 0, torch.float32: 1}
QGRAN = {"block": 0, "token": 1}
(BUF_Q8, BUF_QSCALE, BUF_K8, BUF_KSCALE, BUF_KMEAN, BUF_VQ, BUF_VSCALE, BUF_WS_QK,
 BUF_WS_V, NBUF) = range(10)


class SageError(RuntimeError):
    pass


class SageConfig(ct.Structure):
    _fields_ = [("abi_version", ct.c_int), ("blkq", ct.c_int), ("blkk", ct.c_int),
                ("bc", ct.c_int), ("br", ct.c_int), ("stats_chunk", ct.c_int),
                ("p_scale", ct.c_float), ("log2_p_scale", ct.c_float), ("fp8_format", ct.c_int)]


EXPORTS = ["sage_get_config", "sage_quant_sizes", "sage_quant_sizes_ex", "sage_quant_qk",
           "sage_quant_qk_ex", "sage_quant_v", "sage_quant_qkv", "sage_quant_qkv_noalloc", "sage_attn_fwd", "sage_attn_fwd_lse", "sage_attn_fwd_ex",
           "sage_attn_fwd_sparse", "sage_attn_fwd_debug", "sage_qsmooth_sizes",
           "sage_quant_qk_smooth", "sage_q_smooth_bias", "sage_attn_fwd_smooth",
           "sage_quant_qk_mx", "sage_quant_v_mx", "sage_attn_fwd_mx", "sage_quant_qk_mx_fmt",
           "sage_quant_v_mx_fmt", "sage_attn_fwd_mx_fmt", "sage_bwd_sizes",
           "sage_attn_bwd", "sage_status_string"]

_lib = None


def lib():
    """Load libsage.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SageError(f"{LIB_PATH} is missing: build it with "
                        "`python -m quantized_attention_video_02_amd.build`")
    L = ct.CDLL(LIB_PATH)
    P, I, F, S = ct.c_void_p, ct.c_int, ct.c_float, ct.c_size_t
    L.sage_get_config.argtypes = [I, ct.POINTER(SageConfig)]
    L.sage_quant_sizes.argtypes = [I, I, I, I, I, ct.POINTER(S)]
    L.sage_quant_sizes_ex.argtypes = [I, I, I, I, I, I, ct.POINTER(S)]
    L.sage_quant_qk.argtypes = [P, P, I, I, I, I, I, P, P, P, P, P, P, S, P]
    L.sage_quant_qk_ex.argtypes = [P, P, I, I, I, I, I, I, P, P, P, P, P, P, S, P]
    L.sage_quant_v.argtypes = [P, I, I, I, I, I, I, P, P, P, S, P]
    L.sage_quant_qkv.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, S, P]
    L.sage_quant_qkv_noalloc.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P, P, P, P, P]
    L.sage_attn_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, I, P]
    L.sage_attn_fwd_lse.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, I, P, P]
    L.sage_attn_fwd_ex.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P, I, P]
    L.sage_attn_fwd_sparse.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P, P, I, P]
    L.sage_attn_fwd_debug.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, I, I, I, I, I,
                                      P, P]
    L.sage_qsmooth_sizes.argtypes = [I, I, I, I, ct.POINTER(S), ct.POINTER(S)]
    L.sage_quant_qk_smooth.argtypes = [P, P, I, I, I, I, I, I, P, P, P, P, P, P, P, S, P]
    L.sage_q_smooth_bias.argtypes = [P, P, P, I, I, I, I, I, F, P, P]
    L.sage_attn_fwd_smooth.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P, P, P, I, P]
    L.sage_quant_qk_mx.argtypes = [P, P, I, I, I, I, I, P, P, P, P, S, P]
    L.sage_quant_v_mx.argtypes = [P, I, I, I, I, I, P, P]
    L.sage_attn_fwd_mx.argtypes = [P, P, P, I, I, I, I, I, I, F, P, I, P]
    L.sage_quant_qk_mx_fmt.argtypes = [P, P, I, I, I, I, I, I, P, P, P, P, S, P]
    L.sage_quant_v_mx_fmt.argtypes = [P, I, I, I, I, I, I, P, P]
    L.sage_attn_fwd_mx_fmt.argtypes = [P, P, P, I, I, I, I, I, I, I, F, P, I, P]
    L.sage_bwd_sizes.argtypes = [I, I, I, I, ct.POINTER(ct.c_size_t)]
    L.sage_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, P, S, P]
    for name in EXPORTS[:-1]:
        getattr(L, name).restype = I
    L.sage_status_string.argtypes = [I]
    L.sage_status_string.restype = ct.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != SAGE_OK:
        raise SageError(lib().sage_status_string(status).decode())


def _ptr(t):
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream(device):
    return ct.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _one_gpu(*ts):
    """The one GPU every given tensor lives on.  The C ABI takes raw device
    pointers, so a host tensor (or one on another GPU) is refused here rather
    than handed to a kernel."""
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1 or next(iter(devs)).type != "cuda":
        raise ValueError("all tensors must be on one GPU, got " + ", ".join(sorted(map(str, devs))))
    return next(iter(devs))


def _check_out(out, shape, dev):
    if tuple(out.shape) != shape or out.dtype not in OUT or not out.is_contiguous() or \
            out.device != dev:
        raise ValueError(f"out must be contiguous {shape} (bfloat16 or float32) on {dev}")


def get_config(d: int = 128) -> dict:
    c = SageConfig()
    _check(lib().sage_get_config(d, ct.byref(c)))
    return {f: getattr(c, f) for f, _ in SageConfig._fields_}


def quant_sizes(B: int, H: int, N: int, d: int, pv: str = "fp8", q_gran: str = "block") -> list[int]:
    arr = (ct.c_size_t * NBUF)()
    if q_gran == "block":
        _check(lib().sage_quant_sizes(B, H, N, d, PV[pv], arr))
    else:
        _check(lib().sage_quant_sizes_ex(B, H, N, d, PV[pv], QGRAN[q_gran], arr))
    return list(arr)


def _dims(x: torch.Tensor, layout: str):
    if x.dim() != 4:
        raise ValueError("expected a 4-d tensor")
    if layout == "HND":
        B, H, N, d = x.shape
    elif layout == "NHD":
        B, N, H, d = x.shape
    else:
        raise ValueError(f"layout must be HND or NHD, not {layout!r}")
    return B, H, N, d


def _empty(nbytes: int, device, dtype=torch.uint8):
    itemsize = torch.empty((), dtype=dtype).element_size()
    return torch.empty(max(1, nbytes // itemsize), dtype=dtype, device=device)


def qsmooth_sizes(B: int, H: int, N: int, d: int) -> tuple[int, int]:
    """Bytes of q_mean and of the Q-smoothing correction (sage_qsmooth_sizes)."""
    a, b = ct.c_size_t(), ct.c_size_t()
    _check(lib().sage_qsmooth_sizes(B, H, N, d, ct.byref(a), ct.byref(b)))
    return a.value, b.value


def quant_qk(q: torch.Tensor, k: torch.Tensor, layout: str = "HND", q_gran: str = "block",
             q_smooth: bool = False, sm_scale: float | None = None) -> dict:
    """Smooth K and quantize Q, K to INT8 (sage_quant_qk; sage_quant_qk_ex with
    q_gran="token" for one Q scale per query row).  q_smooth: Q is smoothed by
    its per-block mean too (sage_quant_qk_smooth; q_mean is channel-major
    [B, H, d, nbp]) and the correction of the
    scores is computed for ``sm_scale`` (sage_q_smooth_bias; default
    1/sqrt(d)); attn_fwd then has to run with the same sm_scale."""
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise TypeError("q and k must be bfloat16")
    if q.shape != k.shape or not q.is_contiguous() or not k.is_contiguous():
        raise ValueError("q and k must be contiguous and of the same shape")
    if q_gran not in QGRAN:
        raise ValueError(f"q_gran must be one of {list(QGRAN)}, not {q_gran!r}")
    B, H, N, d = _dims(q, layout)
    dev = _one_gpu(q, k)
    sz = quant_sizes(B, H, N, d, q_gran=q_gran)
    nblk = -(-N // 128)
    r = dict(q8=torch.empty((B, H, nblk * 128, d), dtype=torch.int8, device=dev),
             q_scale=torch.empty((B, H, nblk * 128 if q_gran == "token" else nblk),
                                 dtype=torch.float32, device=dev),
             k8=torch.empty((B, H, nblk * 128, d), dtype=torch.int8, device=dev),
             k_scale=torch.empty((B, H, nblk), dtype=torch.float32, device=dev),
             k_mean=torch.empty((B, H, d), dtype=torch.float32, device=dev),
             workspace=_empty(sz[BUF_WS_QK], dev, torch.int64))
    bufs = (_ptr(r["q8"]), _ptr(r["q_scale"]), _ptr(r["k8"]), _ptr(r["k_scale"]),
            _ptr(r["k_mean"]), _ptr(r["workspace"]), sz[BUF_WS_QK], _stream(dev))
    if q_smooth:
        sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
        nbp = -(-nblk // 16) * 16
        r["q_mean"] = torch.empty((B, H, d, nbp), dtype=torch.float32, device=dev)
        r["bias"] = torch.empty((B, H, nblk, nblk * 128), dtype=torch.float32, device=dev)
        _check(lib().sage_quant_qk_smooth(_ptr(q), _ptr(k), B, H, N, d, LAYOUTS[layout],
                                          QGRAN[q_gran], *bufs[:5], _ptr(r["q_mean"]), *bufs[5:]))
        _check(lib().sage_q_smooth_bias(_ptr(r["q_mean"]), _ptr(k), _ptr(r["k_mean"]), B, H, N, d,
                                        LAYOUTS[layout], sm, _ptr(r["bias"]), _stream(dev)))
        r["bias_sm_scale"] = sm
    elif q_gran == "block":
        _check(lib().sage_quant_qk(_ptr(q), _ptr(k), B, H, N, d, LAYOUTS[layout], *bufs))
    else:
        _check(lib().sage_quant_qk_ex(_ptr(q), _ptr(k), B, H, N, d, LAYOUTS[layout], QGRAN[q_gran],
                                      *bufs))
    r.update(B=B, H=H, N=N, d=d, layout=layout, q_gran=q_gran)
    return r


def quant_v(v: torch.Tensor, pv: str = "fp8", layout: str = "HND"):
    """Quantize V (sage_quant_v): returns (vq, v_scale); vq is the library's
    tiled [B, H, nblk, d, 128] layout with permuted keys (see sage.h)."""
    if v.dtype != torch.bfloat16 or not v.is_contiguous():
        raise TypeError("v must be a contiguous bfloat16 tensor")
    B, H, N, d = _dims(v, layout)
    dev = _one_gpu(v)
    sz = quant_sizes(B, H, N, d, pv)
    nblk = -(-N // 128)
    vq = torch.empty((B, H, nblk, d, 128), dtype=torch.uint8 if pv == "fp8" else torch.float16,
                     device=dev)
    vs = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    ws = _empty(sz[BUF_WS_V], dev, torch.float32) if sz[BUF_WS_V] else None
    _check(lib().sage_quant_v(_ptr(v), B, H, N, d, LAYOUTS[layout], PV[pv], _ptr(vq), _ptr(vs),
                              _ptr(ws), sz[BUF_WS_V], _stream(dev)))
    return vq, vs


def quant_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pv: str = "fp8",
              layout: str = "HND", noalloc: bool = False) -> tuple[dict, torch.Tensor, torch.Tensor]:
    """One quantization pass over Q, K and V (sage_quant_qkv): returns
    (qz, vq, v_scale), the same results as quant_qk(q, k) and quant_v(v, pv),
    with the K and V statistics taken in one launch.  noalloc: through
    sage_quant_qkv_noalloc (the library's fixed scratch, no workspace)."""
    if any(t.dtype != torch.bfloat16 for t in (q, k, v)):
        raise TypeError("q, k and v must be bfloat16")
    if not (q.shape == k.shape == v.shape) or not all(t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k and v must be contiguous and of the same shape")
    B, H, N, d = _dims(q, layout)
    dev = _one_gpu(q, k, v)
    sz = quant_sizes(B, H, N, d, pv)
    nblk = -(-N // 128)
    r = dict(q8=torch.empty((B, H, nblk * 128, d), dtype=torch.int8, device=dev),
             q_scale=torch.empty((B, H, nblk), dtype=torch.float32, device=dev),
             k8=torch.empty((B, H, nblk * 128, d), dtype=torch.int8, device=dev),
             k_scale=torch.empty((B, H, nblk), dtype=torch.float32, device=dev),
             k_mean=torch.empty((B, H, d), dtype=torch.float32, device=dev))
    vq = torch.empty((B, H, nblk, d, 128), dtype=torch.uint8 if pv == "fp8" else torch.float16,
                     device=dev)
    vs = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), B, H, N, d, LAYOUTS[layout], PV[pv], _ptr(r["q8"]),
            _ptr(r["q_scale"]), _ptr(r["k8"]), _ptr(r["k_scale"]), _ptr(r["k_mean"]), _ptr(vq),
            _ptr(vs))
    if noalloc:
        with torch.cuda.device(dev):
            _check(lib().sage_quant_qkv_noalloc(*args, _stream(dev)))
    else:
        ws_bytes = sz[BUF_WS_QK] + sz[BUF_WS_V]
        r["workspace"] = _empty(ws_bytes, dev, torch.int64)
        _check(lib().sage_quant_qkv(*args, _ptr(r["workspace"]), ws_bytes, _stream(dev)))
    r.update(B=B, H=H, N=N, d=d, layout=layout, q_gran="block")
    return r, vq, vs


def attn_fwd(qz: dict, vq: torch.Tensor, vs: torch.Tensor, causal: bool = False,
             sm_scale: float | None = None, pv: str = "fp8", out_dtype=torch.bfloat16,
             out: torch.Tensor | None = None, debug: tuple | None = None,
             tile_mask: torch.Tensor | None = None):
    """Fused attention over quantized operands (sage_attn_fwd).  With
    ``debug=(b, h, row0, nrows)`` calls sage_attn_fwd_debug and also returns
    the int32 Q K^T accumulators [nrows, N].  With ``tile_mask`` (uint8 or
    bool [B, H, nblk, nblk] on the device: query block x key tile, nonzero =
    visit) calls sage_attn_fwd_sparse.  When ``qz`` comes from quant_qk with
    q_smooth, calls sage_attn_fwd_smooth (dense or with the tile mask)."""
    B, H, N, d, layout = qz["B"], qz["H"], qz["N"], qz["d"], qz["layout"]
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    shape = (B, H, N, d) if layout == "HND" else (B, N, H, d)
    dev = _one_gpu(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], vq, vs, out, qz.get("bias"))
    nblk = -(-N // 128)
    if pv not in PV:
        raise ValueError(f"pv must be one of {list(PV)}, not {pv!r}")
    if vq.dtype != (torch.uint8 if pv == "fp8" else torch.float16) or \
            tuple(vq.shape) != (B, H, nblk, d, 128) or not vq.is_contiguous():
        raise ValueError(f"vq must be quant_v's contiguous [{B}, {H}, {nblk}, {d}, 128] "
                         f"({'uint8' if pv == 'fp8' else 'float16'} for pv={pv})")
    if vs.dtype != torch.float32 or tuple(vs.shape) != (B, H, d) or not vs.is_contiguous():
        raise ValueError(f"vs must be contiguous float32 [{B}, {H}, {d}]")
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    else:
        _check_out(out, shape, dev)
    args = (_ptr(qz["q8"]), _ptr(qz["q_scale"]), _ptr(qz["k8"]), _ptr(qz["k_scale"]), _ptr(vq),
            _ptr(vs), B, H, N, d, LAYOUTS[layout], int(bool(causal)), sm, PV[pv], _ptr(out),
            OUT[out.dtype])
    q_gran = qz.get("q_gran", "block")
    tm = None
    if tile_mask is not None:
        if debug is not None:
            raise ValueError("the debug dump runs dense")
        if tuple(tile_mask.shape) != (B, H, nblk, nblk) or tile_mask.device != dev:
            raise ValueError(f"tile_mask must be [B, H, {nblk}, {nblk}] on {dev}")
        tm = tile_mask.to(torch.uint8).contiguous()
    if "bias" in qz:
        if debug is not None:
            raise ValueError("the debug dump runs without Q smoothing")
        if sm != qz["bias_sm_scale"]:
            raise ValueError(f"the Q-smoothing correction was computed for sm_scale "
                             f"{qz['bias_sm_scale']}, not {sm}")
        _check(lib().sage_attn_fwd_smooth(*args[:14], QGRAN[q_gran], _ptr(qz["bias"]), _ptr(tm),
                                          *args[14:], _stream(dev)))
        return out
    if tm is not None:
        _check(lib().sage_attn_fwd_sparse(*args[:14], QGRAN[q_gran], _ptr(tm), *args[14:],
                                          _stream(dev)))
        return out
    if debug is None:
        if q_gran == "block":
            _check(lib().sage_attn_fwd(*args, _stream(dev)))
        else:
            _check(lib().sage_attn_fwd_ex(*args[:14], QGRAN[q_gran], *args[14:], _stream(dev)))
        return out
    if q_gran != "block":
        raise ValueError("the debug dump runs with per-block Q scales (the int32 Q K^T it "
                         "writes does not depend on them)")
    b, h, row0, nrows = debug
    s = torch.zeros((nrows, N), dtype=torch.int32, device=dev)
    _check(lib().sage_attn_fwd_debug(*args, b, h, row0, nrows, _ptr(s), _stream(dev)))
    return out, s


def attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
         sm_scale: float | None = None, pv: str = "fp8", layout: str = "HND",
         out_dtype=torch.bfloat16, q_gran: str = "block",
         tile_mask: torch.Tensor | None = None, q_smooth: bool = False) -> torch.Tensor:
    """softmax(Q K^T sm_scale) V through the quantized path (quantize, then the
    fused kernel), all on q's device and current stream."""
    qz = quant_qk(q, k, layout, q_gran, q_smooth=q_smooth, sm_scale=sm_scale)
    vq, vs = quant_v(v, pv, layout)
    return attn_fwd(qz, vq, vs, causal=causal, sm_scale=sm_scale, pv=pv, out_dtype=out_dtype,
                    tile_mask=tile_mask)


def attn_fwd_lse(qz: dict, vq: torch.Tensor, vs: torch.Tensor, causal: bool = False,
                 sm_scale: float | None = None, pv: str = "fp8", out_dtype=torch.bfloat16):
    """The training forward (sage_attn_fwd_lse): the attention output and each
    row's log-sum-exp in the exp2 domain, fp32 [B, H, N]."""
    if qz.get("q_gran", "block") != "block" or "bias" in qz:
        raise ValueError("the training forward takes per-block Q without smoothing")
    B, H, N, d, layout = qz["B"], qz["H"], qz["N"], qz["d"], qz["layout"]
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    dev = _one_gpu(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], vq, vs)
    nblk = -(-N // 128)
    if pv not in PV:
        raise ValueError(f"pv must be one of {list(PV)}, not {pv!r}")
    if vq.dtype != (torch.uint8 if pv == "fp8" else torch.float16) or \
            tuple(vq.shape) != (B, H, nblk, d, 128) or not vq.is_contiguous():
        raise ValueError(f"vq must be quant_v's contiguous [{B}, {H}, {nblk}, {d}, 128] for pv={pv}")
    if vs.dtype != torch.float32 or tuple(vs.shape) != (B, H, d) or not vs.is_contiguous():
        raise ValueError(f"vs must be contiguous float32 [{B}, {H}, {d}]")
    out = torch.empty((B, H, N, d) if layout == "HND" else (B, N, H, d), dtype=out_dtype, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check(lib().sage_attn_fwd_lse(_ptr(qz["q8"]), _ptr(qz["q_scale"]), _ptr(qz["k8"]),
                                   _ptr(qz["k_scale"]), _ptr(vq), _ptr(vs), B, H, N, d,
                                   LAYOUTS[layout], int(bool(causal)), sm, PV[pv], _ptr(out),
                                   OUT[out.dtype], _ptr(lse), _stream(dev)))
    return out, lse


def bwd_sizes(B: int, H: int, N: int, d: int) -> int:
    """Workspace bytes of sage_attn_bwd."""
    n = ct.c_size_t(0)
    _check(lib().sage_bwd_sizes(B, H, N, d, ct.byref(n)))
    return n.value


def attn_bwd(qz: dict, v: torch.Tensor, o: torch.Tensor, do: torch.Tensor, lse: torch.Tensor,
             causal: bool = False, sm_scale: float | None = None):
    """The 8-bit backward (sage_attn_bwd): dq, dk, dv fp32 in qz's layout, from
    the forward's quantized Q/K (qz of quant_qk), V, its bf16 output o, the
    upstream gradient do (bf16) and lse from attn_fwd_lse."""
    B, H, N, d, layout = qz["B"], qz["H"], qz["N"], qz["d"], qz["layout"]
    if qz.get("q_gran", "block") != "block" or "bias" in qz:
        raise ValueError("the backward takes per-block Q without smoothing")
    shape = (B, H, N, d) if layout == "HND" else (B, N, H, d)
    for name, t in (("v", v), ("o", o), ("do", do)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous bfloat16 {shape}")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError(f"lse must be contiguous float32 [{B}, {H}, {N}]")
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    dev = _one_gpu(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], v, o, do, lse)
    dq, dk, dv = (torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    nbytes = bwd_sizes(B, H, N, d)
    ws = torch.empty(nbytes // 8 + 32, dtype=torch.int64, device=dev)
    _check(lib().sage_attn_bwd(_ptr(qz["q8"]), _ptr(qz["q_scale"]), _ptr(qz["k8"]),
                               _ptr(qz["k_scale"]), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), B, H, N,
                               d, LAYOUTS[layout], int(bool(causal)), sm, _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(ws), nbytes, _stream(dev)))
    return dq, dk, dv


# ------------------------------------------------------------- MX path
MX_FMT = {"mxfp6": 6, "mxfp4": 4}   # sage_mx_fmt: E2M3, E2M1


def _mx_fmt(fmt: str) -> int:
    if fmt not in MX_FMT:
        raise ValueError(f"fmt must be one of {sorted(MX_FMT)}")
    return MX_FMT[fmt]


def quant_qk_mx(q: torch.Tensor, k: torch.Tensor, layout: str = "HND", fmt: str = "mxfp6") -> dict:
    """Smooth K, then Q and K to MXFP6 or MXFP4 (sage_quant_qk_mx_fmt): q6, k6
    uint8 [B, H, N_pad, d] (32-byte MX blocks, see sage.h), k_mean."""
    f = _mx_fmt(fmt)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16:
        raise TypeError("q and k must be bfloat16")
    if q.shape != k.shape or not q.is_contiguous() or not k.is_contiguous():
        raise ValueError("q and k must be contiguous and of the same shape")
    B, H, N, d = _dims(q, layout)
    dev = _one_gpu(q, k)
    sz = quant_sizes(B, H, N, d)
    nblk = -(-N // 128)
    r = dict(q6=torch.empty((B, H, nblk * 128, d), dtype=torch.uint8, device=dev),
             k6=torch.empty((B, H, nblk * 128, d), dtype=torch.uint8, device=dev),
             k_mean=torch.empty((B, H, d), dtype=torch.float32, device=dev),
             workspace=_empty(sz[BUF_WS_QK], dev, torch.int64))
    _check(lib().sage_quant_qk_mx_fmt(_ptr(q), _ptr(k), B, H, N, d, LAYOUTS[layout], f,
                                      _ptr(r["q6"]), _ptr(r["k6"]), _ptr(r["k_mean"]),
                                      _ptr(r["workspace"]), sz[BUF_WS_QK], _stream(dev)))
    r.update(B=B, H=H, N=N, d=d, layout=layout, fmt=fmt)
    return r


def quant_v_mx(v: torch.Tensor, layout: str = "HND", fmt: str = "mxfp6") -> torch.Tensor:
    """V to MXFP6 or MXFP4 (sage_quant_v_mx_fmt): uint8 [B, H, nblk, d, 128]."""
    f = _mx_fmt(fmt)
    if v.dtype != torch.bfloat16 or not v.is_contiguous():
        raise TypeError("v must be a contiguous bfloat16 tensor")
    B, H, N, d = _dims(v, layout)
    dev = _one_gpu(v)
    nblk = -(-N // 128)
    v6 = torch.empty((B, H, nblk, d, 128), dtype=torch.uint8, device=dev)
    _check(lib().sage_quant_v_mx_fmt(_ptr(v), B, H, N, d, LAYOUTS[layout], f, _ptr(v6),
                                     _stream(dev)))
    return v6


def attn_fwd_mx(mz: dict, v6: torch.Tensor, causal: bool = False, sm_scale: float | None = None,
                out_dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """MX attention over quantized operands (sage_attn_fwd_mx_fmt), in the
    element format Q and K were quantized to (mz["fmt"]; v6 must have been
    quantized to the same one)."""
    B, H, N, d, layout = mz["B"], mz["H"], mz["N"], mz["d"], mz["layout"]
    f = _mx_fmt(mz.get("fmt", "mxfp6"))
    sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    shape = (B, H, N, d) if layout == "HND" else (B, N, H, d)
    dev = _one_gpu(mz["q6"], mz["k6"], v6, out)
    nblk = -(-N // 128)
    if v6.dtype != torch.uint8 or tuple(v6.shape) != (B, H, nblk, d, 128) or \
            not v6.is_contiguous():
        raise ValueError(f"v6 must be contiguous uint8 [{B}, {H}, {nblk}, {d}, 128] on {dev}")
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    else:
        _check_out(out, shape, dev)
    _check(lib().sage_attn_fwd_mx_fmt(_ptr(mz["q6"]), _ptr(mz["k6"]), _ptr(v6), B, H, N, d,
                                      LAYOUTS[layout], f, int(bool(causal)), sm, _ptr(out),
                                      OUT[out.dtype], _stream(dev)))
    return out


def attn_mx(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
            sm_scale: float | None = None, layout: str = "HND",
            out_dtype=torch.bfloat16, fmt: str = "mxfp6") -> torch.Tensor:
    """softmax(Q K^T sm_scale) V through the MX path (MXFP6 or MXFP4)."""
    mz = quant_qk_mx(q, k, layout, fmt)
    v6 = quant_v_mx(v, layout, fmt)
    return attn_fwd_mx(mz, v6, causal=causal, sm_scale=sm_scale, out_dtype=out_dtype)
