"""Buffer discipline and determinism of the whole library on the GPU.

* Every quantization entry point writes inside the buffers sage_quant_sizes
  gives (codes, scales, K mean, V codes) and inside its workspace: each buffer
  sits between two guard bands of a canary byte that must survive, called
  through the C ABI on ragged N, both head sizes, both P V types and both Q
  scale granularities; the MX quantization in both element formats, the
  training forward and the backward likewise.
* Every forward variant (MXFP4 included) returns the same bytes on a repeated call, with other
  launches of other shapes in between (no state carried between calls, no
  order-dependent reduction).
"""
import ctypes as ct

import numpy as np
import pytest
import torch

import quantized_attention_video_02_amd as sage
import synthetic_inputs as si

pytestmark = pytest.mark.gpu

G = 4096          # guard bytes on each side (a multiple of 16 keeps every buffer aligned)
CANARY = 0xA5


class Guarded:
    """A device buffer of nbytes between two guard bands of CANARY."""

    def __init__(self, nbytes):
        self.n = int(nbytes)
        self.t = torch.full((self.n + 2 * G,), CANARY, dtype=torch.uint8, device="cuda")

    @property
    def ptr(self):
        return ct.c_void_p(self.t.data_ptr() + G)

    def body(self):
        return self.t[G:G + self.n]

    def intact(self):
        return bool(torch.all(self.t[:G] == CANARY)) and bool(torch.all(self.t[G + self.n:] == CANARY))


def _sizes(B, H, N, d, pv, gran="block"):
    arr = (ct.c_size_t * 9)()
    assert sage.lib().sage_quant_sizes_ex(B, H, N, d, sage.PV[pv], sage.QGRAN[gran], arr) == 0
    return list(arr)


CASES = [("tiny", dict(N=333, H=2), "fp8", "block", "HND"),
         ("tiny", dict(N=333, H=2), "fp16", "token", "NHD"),
         ("outlier", dict(N=700, B=1, H=3), "fp8", "token", "HND"),   # d = 64
         ("outlier", dict(N=129, B=1, H=1), "fp16", "block", "NHD")]


@pytest.mark.parametrize("name,kw,pv,gran,layout", CASES)
def test_quantization_outputs_stay_inside_their_buffers(name, kw, pv, gran, layout):
    wl = si.make(name, **kw)
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    q, k, v = ((x if layout == "HND" else x.permute(0, 2, 1, 3)).contiguous().cuda()
               for x in (wl.q, wl.k, wl.v))
    L = sage.lib()
    lay, pvc = sage.LAYOUTS[layout], sage.PV[pv]
    st = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    sz = _sizes(B, H, N, d, pv, gran)
    print(f"  case {name} {kw} {pv} {gran} {layout}", flush=True)

    def bufs():
        return [Guarded(sz[i]) for i in range(7)]

    # sage_quant_qk_ex + sage_quant_v, each with an exact-size workspace
    a = bufs()
    wqk, wv = Guarded(sz[7]), Guarded(max(sz[8], 16))
    assert L.sage_quant_qk_ex(ct.c_void_p(q.data_ptr()), ct.c_void_p(k.data_ptr()), B, H, N, d,
                              lay, sage.QGRAN[gran], *(x.ptr for x in a[:5]), wqk.ptr, sz[7],
                              st) == 0
    assert L.sage_quant_v(ct.c_void_p(v.data_ptr()), B, H, N, d, lay, pvc, a[5].ptr, a[6].ptr,
                          wv.ptr, sz[8], st) == 0
    torch.cuda.synchronize()
    for i, x in enumerate(a + [wqk, wv]):
        assert x.intact(), ("quant_qk/quant_v buffer", i)
    if gran != "block":
        return
    # sage_quant_qkv with the summed workspace, then the allocation-free form
    b = bufs()
    wall = Guarded(sz[7] + sz[8])
    assert L.sage_quant_qkv(ct.c_void_p(q.data_ptr()), ct.c_void_p(k.data_ptr()),
                            ct.c_void_p(v.data_ptr()), B, H, N, d, lay, pvc,
                            *(x.ptr for x in b[:5]), b[5].ptr, b[6].ptr, wall.ptr,
                            sz[7] + sz[8], st) == 0
    c = bufs()
    assert L.sage_quant_qkv_noalloc(ct.c_void_p(q.data_ptr()), ct.c_void_p(k.data_ptr()),
                                    ct.c_void_p(v.data_ptr()), B, H, N, d, lay, pvc,
                                    *(x.ptr for x in c[:5]), c[5].ptr, c[6].ptr, st) == 0
    torch.cuda.synchronize()
    for i, x in enumerate(b + [wall] + c):
        assert x.intact(), ("quant_qkv buffer", i)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x.body(), y.body()) and torch.equal(x.body(), z.body())


MX_CASES = [("tiny", dict(N=333, H=2), "HND"), ("outlier", dict(N=129, B=1, H=1), "NHD")]


@pytest.mark.parametrize("fmt", [6, 4])
@pytest.mark.parametrize("name,kw,layout", MX_CASES)
def test_mx_quantization_outputs_stay_inside_their_buffers(name, kw, layout, fmt):
    wl = si.make(name, **kw)
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    q, k, v = ((x if layout == "HND" else x.permute(0, 2, 1, 3)).contiguous().cuda()
               for x in (wl.q, wl.k, wl.v))
    L = sage.lib()
    lay = sage.LAYOUTS[layout]
    st = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    sz = _sizes(B, H, N, d, "fp8")
    print(f"  case {name} {kw} {layout} fmt {fmt}", flush=True)
    # q6, k6 as the INT8 codes, k_mean, the Q/K workspace, v6 as the FP8 V codes
    q6, k6, km, ws, v6 = (Guarded(sz[i]) for i in (0, 2, 4, 7, 5))
    assert L.sage_quant_qk_mx_fmt(ct.c_void_p(q.data_ptr()), ct.c_void_p(k.data_ptr()), B, H, N,
                                  d, lay, fmt, q6.ptr, k6.ptr, km.ptr, ws.ptr, sz[7], st) == 0
    assert L.sage_quant_v_mx_fmt(ct.c_void_p(v.data_ptr()), B, H, N, d, lay, fmt, v6.ptr, st) == 0
    torch.cuda.synchronize()
    for i, x in enumerate((q6, k6, km, ws, v6)):
        assert x.intact(), ("mx buffer", i)


@pytest.mark.parametrize("name,kw,causal", [("tiny", dict(N=333, H=2), False),
                                             ("outlier", dict(N=300, B=1, H=2), True)])
def test_training_outputs_stay_inside_their_buffers(name, kw, causal):
    """sage_attn_fwd_lse (output and log-sum-exp) and sage_attn_bwd (dq, dk,
    dv and the workspace) write inside their buffers."""
    wl = si.make(name, **kw)
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    q, k, v = (x.contiguous().cuda() for x in (wl.q, wl.k, wl.v))
    do = si.output_grad(wl).contiguous().cuda()
    L = sage.lib()
    st = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    print(f"  case {name} {kw} causal={causal}", flush=True)
    qz = sage.quant_qk(q, k)
    vq, vs = sage.quant_v(v)
    p = lambda t: ct.c_void_p(t.data_ptr())
    o, lse = Guarded(B * H * N * d * 2), Guarded(B * H * N * 4)
    assert L.sage_attn_fwd_lse(p(qz["q8"]), p(qz["q_scale"]), p(qz["k8"]), p(qz["k_scale"]), p(vq),
                               p(vs), B, H, N, d, 0, int(causal), wl.sm_scale, 0, o.ptr, 0,
                               lse.ptr, st) == 0
    n = ct.c_size_t()
    assert L.sage_bwd_sizes(B, H, N, d, ct.byref(n)) == 0
    dq, dk, dv = (Guarded(B * H * N * d * 4) for _ in range(3))
    ws = Guarded(n.value)
    assert L.sage_attn_bwd(p(qz["q8"]), p(qz["q_scale"]), p(qz["k8"]), p(qz["k_scale"]), p(v),
                           o.ptr, p(do), lse.ptr, B, H, N, d, 0, int(causal), wl.sm_scale,
                           dq.ptr, dk.ptr, dv.ptr, ws.ptr, n.value, st) == 0
    torch.cuda.synchronize()
    for i, x in enumerate((o, lse, dq, dk, dv, ws)):
        assert x.intact(), ("training buffer", i)
    assert torch.isfinite(dq.body().view(torch.float32)).all()


def _forward_variants():
    """name -> callable returning the bytes of one forward of that variant."""
    wl = si.make("causal_prefill", B=1, H=2, N=900)
    wl64 = si.make("outlier", N=777, B=1, H=2)
    q, k, v = (x.cuda() for x in (wl.q, wl.k, wl.v))
    q6, k6, v6 = (x.cuda() for x in (wl64.q, wl64.k, wl64.v))
    nblk = -(-wl.N // 128)
    rng = np.random.default_rng(3)
    tm = torch.from_numpy((rng.random((1, 2, nblk, nblk)) < 0.6).astype(np.uint8)).cuda()

    def dense(causal, pv):
        qz, vq, vs = sage.quant_qkv(q, k, v, pv)
        return sage.attn_fwd(qz, vq, vs, causal=causal, sm_scale=wl.sm_scale, pv=pv)

    def d64(pv):
        qz, vq, vs = sage.quant_qkv(q6, k6, v6, pv)
        return sage.attn_fwd(qz, vq, vs, causal=False, sm_scale=wl64.sm_scale, pv=pv)

    def token():
        qz = sage.quant_qk(q, k, q_gran="token")
        vq, vs = sage.quant_v(v)
        return sage.attn_fwd(qz, vq, vs, causal=True, sm_scale=wl.sm_scale)

    def sparse():
        qz, vq, vs = sage.quant_qkv(q, k, v)
        return sage.attn_fwd(qz, vq, vs, causal=False, sm_scale=wl.sm_scale, tile_mask=tm)

    def lse():
        qz, vq, vs = sage.quant_qkv(q, k, v)
        o, l = sage.attn_fwd_lse(qz, vq, vs, causal=True, sm_scale=wl.sm_scale)
        return torch.cat([o.float().flatten(), l.flatten()])

    def mx(fmt="mxfp6"):
        return sage.attn_fwd_mx(sage.quant_qk_mx(q, k, fmt=fmt), sage.quant_v_mx(v, fmt=fmt),
                                causal=True, sm_scale=wl.sm_scale)

    return {"dense fp8": lambda: dense(False, "fp8"), "causal fp8": lambda: dense(True, "fp8"),
            "causal fp16": lambda: dense(True, "fp16"), "d64 fp8": lambda: d64("fp8"),
            "d64 fp16": lambda: d64("fp16"), "per-token causal": token, "sparse": sparse,
            "lse causal": lse, "mxfp6 causal": mx, "mxfp4 causal": lambda: mx("mxfp4")}


def test_every_forward_variant_is_deterministic():
    variants = _forward_variants()
    first = {}
    for rnd in range(2):
        # the second round runs the variants in reverse order, so each call
        # follows different work than it did the first time
        for name in (list(variants) if rnd == 0 else list(variants)[::-1]):
            print(f"  round {rnd} {name}", flush=True)
            out = variants[name]()
            torch.cuda.synchronize()
            raw = out.contiguous().view(torch.uint8).cpu()
            if rnd == 0:
                first[name] = raw
            else:
                assert torch.equal(raw, first[name]), name
