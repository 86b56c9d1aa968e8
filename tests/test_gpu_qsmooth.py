"""GPU parity of Q smoothing (sage_quant_qk_smooth, sage_q_smooth_bias,
sage_attn_fwd_smooth) against the CPU oracle, through the C ABI.

Bars as for the unsmoothed path: codes, scales, both means and the
correction compared bit for bit (the correction is one fixed fp32 fma chain
on both sides); the fp32 attention output within max-abs 2e-3 and cosine >=
0.9999 of the oracle, and the FP64 cosine checked.  Inputs carry a
per-channel query offset (the case smoothing is for).
"""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from sage_layouts import codes, to_hnd

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
COS_ORACLE = 0.9999
COS_FP64 = 0.999


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


@pytest.fixture(scope="module")
def sage():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_attention_video_02_amd as s

    s.lib()
    return s


def _to_layout(x, layout):
    return x.contiguous() if layout == "HND" else x.permute(0, 2, 1, 3).contiguous()


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _q_mean(qz):
    """The GPU's channel-major, block-padded q_mean as [B, H, nblk, d]; the
    padding must be 0."""
    m = qz["q_mean"].cpu().numpy()
    nblk = -(-qz["N"] // 128)
    assert not m[..., nblk:].any()
    return np.ascontiguousarray(np.swapaxes(m[..., :nblk], -1, -2))


def _check_quant(qz, oz, obias, N):
    g = lambda key: _q_mean(qz) if key == "q_mean" else qz[key].cpu().numpy()
    assert np.array_equal(g("q8")[:, :, :N], oz["q8"]) and not g("q8")[:, :, N:].any()
    assert np.array_equal(g("k8")[:, :, :N], oz["k8"])
    for key in ("q_scale", "k_scale", "k_mean", "q_mean"):
        got = g(key)
        if key == "q_scale" and got.shape != oz[key].shape:       # per token: padded rows
            got = got[:, :, :N]
        assert np.array_equal(_bits(got), _bits(oz[key])), key
    gb = g("bias")
    assert np.array_equal(_bits(gb[..., :N]), _bits(obias)), "bias"
    assert not gb[..., N:].any()                                  # padded keys: 0


QS_CASES = [
    ("tiny", dict(N=300, H=2), "fp8", "HND", "block", None),
    ("tiny", dict(N=1024, H=2), "fp16", "NHD", "block", None),
    ("tiny", dict(N=700, H=1), "fp8", "HND", "token", None),
    ("causal_prefill", dict(B=2, H=1, N=900), "fp8", "HND", "block", None),
    ("outlier", dict(B=1, H=2, N=1100), "fp8", "HND", "block", None),
    ("outlier", dict(B=1, H=1, N=600), "fp16", "NHD", "token", None),
    ("tiny", dict(N=1000, H=2), "fp8", "HND", "block", "random"),
    ("tiny", dict(N=1000, H=1), "fp16", "HND", "block", "random"),
    ("causal_prefill", dict(B=1, H=2, N=1000), "fp8", "NHD", "block", "band"),
]


def _mask(B, H, N, kind, seed=7):
    nb = -(-N // 128)
    rng = np.random.default_rng(seed)
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    if kind == "random":
        m = rng.random((B, H, nb, nb)) < 0.5
        m[:, :, 1] = False                       # a query block that visits nothing
    else:
        m = np.broadcast_to((np.abs(i - j) <= 1) | (j == 0), (B, H, nb, nb)).copy()
    return m.astype(np.uint8)


@pytest.mark.parametrize("name,kw,pv,layout,q_gran,mask_kind", QS_CASES)
def test_qsmooth_matches_oracle(sage, orc, name, kw, pv, layout, q_gran, mask_kind):
    print(f"[qsmooth parity] {name} {kw} pv={pv} {layout} {q_gran} mask={mask_kind}", flush=True)
    wl = si.make(name, q_sigma=6.0, **kw)
    qd, kd, vd = (_to_layout(t, layout).cuda() for t in (wl.q, wl.k, wl.v))
    qz = sage.quant_qk(qd, kd, layout, q_gran=q_gran, q_smooth=True, sm_scale=wl.sm_scale)
    vq, vs = sage.quant_v(vd, pv, layout)
    mask = None if mask_kind is None else _mask(wl.B, wl.H, wl.N, mask_kind)
    out = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                        out_dtype=torch.float32,
                        tile_mask=None if mask is None else torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    out = to_hnd(out, layout).cpu().numpy()
    q, k, v = codes(wl.q), codes(wl.k), codes(wl.v)
    oz = orc.quant_qk(q, k, q_gran=q_gran, q_smooth=True)
    obias = orc.smooth_bias(oz, k, wl.sm_scale)
    _check_quant(qz, oz, obias, wl.N)
    ovq, ovs = orc.quant_v(v, pv)
    rows = np.arange(wl.N)
    o_or = np.stack([np.stack([orc.attn_rows_head(oz, ovq, ovs, b, h, rows, wl.causal, wl.sm_scale,
                                                  pv, tile_mask=mask, bias=obias)
                               for h in range(wl.H)]) for b in range(wl.B)])
    assert np.isfinite(out).all()
    err, c = np.abs(out - o_or).max(), _cos(out, o_or)
    print(f"  max-abs {err:.3e} cos(oracle) {c:.7f}")
    assert err <= MAX_ABS and c >= COS_ORACLE, (err, c)
    if mask is not None:
        empty = o_or.reshape(wl.B, wl.H, wl.N, -1).any(axis=-1) == 0
        assert not out[empty].any()
        return
    ref = np.stack([np.stack([orc.ref64_rows_head(q, k, v, b, h, rows, wl.causal, wl.sm_scale)
                              for h in range(wl.H)]) for b in range(wl.B)])
    c_gpu, c_or = _cos(out, ref), _cos(o_or, ref)
    if name == "outlier":
        assert abs(c_gpu - c_or) < 2e-4, (c_gpu, c_or)
    else:
        assert c_gpu >= COS_FP64, c_gpu


def test_qsmooth_gains_over_plain_on_query_offsets(sage):
    """With query offsets the smoothed GPU path is closer to FP64 attention
    than the plain one (the oracle-level claim, here on the GPU outputs)."""
    import oracle as orc

    wl = si.make("tiny", H=2, q_sigma=6.0, seed=17)
    qd, kd, vd = (t.cuda() for t in (wl.q, wl.k, wl.v))
    vq, vs = sage.quant_v(vd, "fp16")
    plain = sage.attn_fwd(sage.quant_qk(qd, kd), vq, vs, sm_scale=wl.sm_scale, pv="fp16",
                          out_dtype=torch.float32)
    qz = sage.quant_qk(qd, kd, q_smooth=True, sm_scale=wl.sm_scale)
    smooth = sage.attn_fwd(qz, vq, vs, sm_scale=wl.sm_scale, pv="fp16", out_dtype=torch.float32)
    torch.cuda.synchronize()
    q, k, v = codes(wl.q), codes(wl.k), codes(wl.v)
    for h in range(2):
        ref = orc.ref64_rows_head(q, k, v, 0, h, np.arange(wl.N), False, wl.sm_scale)
        c0 = _cos(plain[0, h].cpu().numpy(), ref)
        c1 = _cos(smooth[0, h].cpu().numpy(), ref)
        assert c1 >= 0.99995 and (1 - c1) * 10 < 1 - c0, (h, c0, c1)
    with pytest.raises(ValueError, match="sm_scale"):
        sage.attn_fwd(qz, vq, vs, sm_scale=2 * wl.sm_scale, pv="fp16")


def test_qsmooth_full_size_sampled(sage, orc):
    """video_14b_720p with query offsets (sigma 3) at full size in the
    benchmark's launch configuration: quantization, means and the correction
    bit-exact on two heads, attention on sampled rows of them."""
    print("[qsmooth full-size parity] video_14b_720p fp8", flush=True)
    wl = si.make("video_14b_720p", device="cuda", q_sigma=3.0)
    qz = sage.quant_qk(wl.q, wl.k, q_smooth=True, sm_scale=wl.sm_scale)
    vq, vs = sage.quant_v(wl.v, "fp8")
    out = sage.attn_fwd(qz, vq, vs, sm_scale=wl.sm_scale, pv="fp8", out_dtype=torch.float32)
    torch.cuda.synchronize()
    N, nblk = wl.N, -(-wl.N // 128)
    rng = np.random.default_rng(3)
    o_all, or_all, r_all = [], [], []
    for b, h in [(0, 0), (0, wl.H - 1)]:
        q = codes(wl.q[b:b + 1, h:h + 1])
        k = codes(wl.k[b:b + 1, h:h + 1])
        v = codes(wl.v[b:b + 1, h:h + 1])
        oz = orc.quant_qk(q, k, q_smooth=True)
        blocks = sorted({0, 1, nblk - 1, int(rng.integers(2, nblk - 1))})
        obias = orc.smooth_bias(oz, k, wl.sm_scale, blocks=blocks)
        assert np.array_equal(qz["q8"][b, h, :N].cpu().numpy(), oz["q8"][0, 0])
        for key in ("q_scale", "k_scale", "k_mean"):
            assert np.array_equal(_bits(qz[key][b, h].cpu().numpy()), _bits(oz[key][0, 0])), key
        assert np.array_equal(_bits(_q_mean(qz)[b, h]), _bits(oz["q_mean"][0, 0]))
        assert np.array_equal(_bits(qz["bias"][b, h, blocks, :N].cpu().numpy()),
                              _bits(obias[0, 0, blocks]))
        ovq, ovs = orc.quant_v(v, "fp8")
        rows = np.array(sorted({r for blk in blocks
                                for r in list(range(blk * 128, min(N, blk * 128 + 12))) +
                                list(range(max(blk * 128, min(N, blk * 128 + 128) - 12),
                                           min(N, blk * 128 + 128)))}), np.int32)
        or_all.append(orc.attn_rows_head(oz, ovq, ovs, 0, 0, rows, False, wl.sm_scale, "fp8",
                                         bias=obias))
        o_all.append(out[b, h, torch.from_numpy(rows).long().cuda()].cpu().numpy())
        r_all.append(orc.ref64_rows_head(q, k, v, 0, 0, rows, False, wl.sm_scale))
    o_gpu, o_or, ref = (np.concatenate(x) for x in (o_all, or_all, r_all))
    err, c = np.abs(o_gpu - o_or).max(), _cos(o_gpu, o_or)
    print(f"  max-abs {err:.3e} cos(oracle) {c:.7f} cos64 {_cos(o_gpu, ref):.6f}")
    assert err <= MAX_ABS and c >= COS_ORACLE, (err, c)
    assert _cos(o_gpu, ref) >= COS_FP64
