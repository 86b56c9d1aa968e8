"""GPU parity of libsage against the CPU oracle (through the C ABI).

Bars: quantized codes, scales, the K mean and the int32 Q K^T accumulators are
compared bit for bit; the fp32 attention output within max-abs 2e-3 and
cosine >= 0.9999 of the oracle; and the cosine against FP64 attention is
checked (>= 0.999 where the method reaches it; on the outlier workload the
method itself stays below that bar, so there the GPU must match the oracle's
own FP64 cosine to 2e-4).
"""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from sage_layouts import codes, to_hnd, vq_natural

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


def run_gpu(sage, wl, pv, layout="HND", out_dtype=torch.float32):
    qd, kd, vd = (_to_layout(t, layout).cuda() for t in (wl.q, wl.k, wl.v))
    qz = sage.quant_qk(qd, kd, layout)
    vq, vs = sage.quant_v(vd, pv, layout)
    out = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    return qz, vq, vs, to_hnd(out, layout)


def gpu_quant_np(qz, vq, vs, N, pv):
    g = {k: qz[k].cpu().numpy() for k in ("q8", "q_scale", "k8", "k_scale", "k_mean")}
    vqn = vq.cpu()
    vqn = (vqn.view(torch.int16).numpy().view(np.uint16) if pv == "fp16" else vqn.numpy())
    g["vq"] = vq_natural(vqn, N)
    g["vq_pad"] = vqn
    g["v_scale"] = vs.cpu().numpy()
    return g


def assert_quant_bitexact(g, oz, ovq, ovs, N, heads=None):
    """GPU quantization equals the oracle's bit for bit (for the listed heads)."""
    sel = (lambda a: a) if heads is None else (lambda a: np.stack([a[b, h] for b, h in heads]))
    bits = lambda a: np.ascontiguousarray(a).view(np.uint32)
    assert np.array_equal(sel(g["q8"][:, :, :N]), sel(oz["q8"]) if heads is None else oz["q8"])
    assert np.array_equal(sel(g["k8"][:, :, :N]), sel(oz["k8"]) if heads is None else oz["k8"])
    assert not sel(g["q8"][:, :, N:]).any() and not sel(g["k8"][:, :, N:]).any()
    for key in ("q_scale", "k_scale", "k_mean"):
        ref = oz[key] if heads is None else oz[key]
        assert np.array_equal(bits(sel(g[key])), bits(ref)), key
    assert np.array_equal(sel(g["vq"]), ovq)
    assert np.array_equal(bits(sel(g["v_scale"])), bits(ovs))


def oracle_quant(orc, wl, pv, heads=None):
    q, k, v = codes(wl.q), codes(wl.k), codes(wl.v)
    if heads is not None:
        q, k, v = (np.stack([x[b, h] for b, h in heads])[None] for x in (q, k, v))
    oz = orc.quant_qk(q, k)
    ovq, ovs = orc.quant_v(v, pv)
    if heads is not None:
        oz = {key: (val[0] if isinstance(val, np.ndarray) else val) for key, val in oz.items()}
        ovq, ovs = ovq[0], ovs[0]
    return q, k, v, oz, ovq, ovs


# ------------------------------------------------------------------ quantization
QUANT_CASES = [
    ("tiny", dict(), "fp8", "HND"),
    ("tiny", dict(N=300, H=3), "fp8", "NHD"),
    ("tiny", dict(N=1, H=1), "fp8", "HND"),
    ("outlier", dict(N=1000, B=1, H=2), "fp16", "HND"),
    ("outlier", dict(N=1000, B=1, H=2), "fp8", "NHD"),
    ("causal_prefill", dict(B=2, H=2, N=777), "fp8", "HND"),
]


@pytest.mark.parametrize("name,kw,pv,layout", QUANT_CASES)
def test_quantization_bitexact(sage, orc, name, kw, pv, layout):
    wl = si.make(name, **kw)
    qz, vq, vs, _ = run_gpu(sage, wl, pv, layout)
    g = gpu_quant_np(qz, vq, vs, wl.N, pv)
    _, _, _, oz, ovq, ovs = oracle_quant(orc, wl, pv)
    assert_quant_bitexact(g, oz, ovq, ovs, wl.N)
    nblk = -(-wl.N // 128)
    pad = g["vq_pad"].reshape(wl.B, wl.H, nblk, wl.d, 128)
    tail = wl.N - (nblk - 1) * 128
    from sage_layouts import vperm_positions

    assert not pad[:, :, -1][..., vperm_positions()[tail:]].any()  # padded keys are 0


FUSED_CASES = QUANT_CASES + [("outlier", dict(N=700, B=1, H=3), "fp8", "HND"),  # d = 64
                             ("outlier", dict(N=700, B=1, H=3), "fp16", "NHD")]


@pytest.mark.parametrize("name,kw,pv,layout", FUSED_CASES)
def test_fused_quantization_pass_bitexact(sage, orc, name, kw, pv, layout):
    """sage_quant_qkv (K and V statistics in one launch) gives the oracle's
    codes, scales and K mean bit for bit, and the same bytes as
    sage_quant_qk + sage_quant_v, padding included."""
    wl = si.make(name, **kw)
    qd, kd, vd = (_to_layout(t, layout).cuda() for t in (wl.q, wl.k, wl.v))
    qz, vq, vs = sage.quant_qkv(qd, kd, vd, pv, layout)
    torch.cuda.synchronize()
    g = gpu_quant_np(qz, vq, vs, wl.N, pv)
    _, _, _, oz, ovq, ovs = oracle_quant(orc, wl, pv)
    assert_quant_bitexact(g, oz, ovq, ovs, wl.N)
    qz2 = sage.quant_qk(qd, kd, layout)
    vq2, vs2 = sage.quant_v(vd, pv, layout)
    torch.cuda.synchronize()
    for key in ("q8", "q_scale", "k8", "k_scale", "k_mean"):
        assert torch.equal(qz[key].view(torch.uint8), qz2[key].view(torch.uint8)), key
    assert torch.equal(vq.view(torch.uint8), vq2.view(torch.uint8))
    assert torch.equal(vs.view(torch.int32), vs2.view(torch.int32))


def test_int8_rounding_ties(sage, orc):
    """Q and K blocks whose scaled values sit exactly on k + 1/2: the codes are
    round-half-to-even of the value (absmax 127, so the inverse scale is 1),
    per block and per token, on the GPU and in the oracle alike."""
    ties = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 126.5, -126.5, 62.5, -63.5,
                     4.5, -5.5, 100.5, -101.5], np.float32)
    d, N = 128, 128
    x = np.resize(ties, (N, d)).astype(np.float32)
    x[:, 0] = 127.0  # every row's (and the block's) absmax
    # K: the second half is the negated first half, so each channel's mean is 0
    # exactly and the smoothed K equals K
    k = np.concatenate([x[: N // 2], -x[: N // 2]])
    want_q = np.rint(x).astype(np.int8)  # ties to even: 0.5 -> 0, 2.5 -> 2, -3.5 -> -4 ...
    want_k = np.rint(k).astype(np.int8)
    assert want_q[0, 1:5].tolist() == [2, 2, 4, 0]  # 1.5, 2.5, 3.5, -0.5
    tb = lambda a: torch.from_numpy(a).to(torch.bfloat16).reshape(1, 1, N, d).cuda()
    for gran in ("block", "token"):
        qz = sage.quant_qk(tb(x), tb(k), "HND", q_gran=gran)
        torch.cuda.synchronize()
        assert np.all(qz["q_scale"].cpu().numpy().ravel()[: (N if gran == "token" else 1)] == 1.0)
        assert np.array_equal(qz["q8"][0, 0, :N].cpu().numpy(), want_q), gran
        assert np.array_equal(qz["k8"][0, 0, :N].cpu().numpy(), want_k), gran
        assert not qz["k_mean"].cpu().numpy().any()
    oz = orc.quant_qk(codes(tb(x).cpu()), codes(tb(k).cpu()), q_gran="token")
    assert np.array_equal(oz["q8"][0, 0], want_q) and np.array_equal(oz["k8"][0, 0], want_k)


def test_fp8_encoder_ties_and_boundaries(sage, orc):
    """Every bf16 value in [-448, 448] through V quantization with inv = 1
    (each channel's absmax is 448): codes equal the oracle's RNE encoder."""
    vals = np.arange(0, 0x43E1, dtype=np.uint16)  # +0 .. 448 as bf16 codes
    allv = np.concatenate([vals, vals | 0x8000])
    d = 128
    N = 1 + -(-allv.size // d)
    grid = np.full(N * d, 0x43E0, np.uint16)  # 448 fills the first row and the remainder
    grid[d:d + allv.size] = allv
    v = torch.from_numpy(grid.view(np.int16).reshape(1, 1, N, d)).view(torch.bfloat16)
    vq, vs = sage.quant_v(v.cuda(), "fp8")
    torch.cuda.synchronize()
    assert np.all(vs.cpu().numpy() == 1.0)
    got = vq_natural(vq.cpu().numpy(), N).reshape(-1)
    ref = orc.f32_to_e4m3(orc.bf16_to_f32(grid))
    assert np.array_equal(got, ref)


# --------------------------------------------------------------- int32 dump
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_qk_accumulators_bitexact(sage, orc, causal, d):
    name = "tiny" if d == 128 else "outlier"
    wl = si.make(name, B=1, H=2, N=700)
    qd, kd, vd = wl.q.cuda(), wl.k.cuda(), wl.v.cuda()
    qz = sage.quant_qk(qd, kd)
    vq, vs = sage.quant_v(vd)
    for (b, h, row0, nrows) in [(0, 1, 0, 70), (0, 0, 250, 300), (0, 1, 640, 60)]:
        _, s = sage.attn_fwd(qz, vq, vs, causal=causal, sm_scale=wl.sm_scale,
                             out_dtype=torch.float32, debug=(b, h, row0, nrows))
        torch.cuda.synchronize()
        s = s.cpu().numpy()
        q8 = qz["q8"][b, h, :wl.N].cpu().numpy()
        k8 = qz["k8"][b, h, :wl.N].cpu().numpy()
        ref = orc.dump_s(q8, k8, row0, nrows, causal)
        assert np.array_equal(s, ref)
        assert np.array_equal(s.astype(np.int64),
                              np.where(ref != 0, q8[row0:row0 + nrows].astype(np.int64)
                                       @ k8.astype(np.int64).T, 0))


# ------------------------------------------------------------ attention output
ATTN_CASES = [
    ("tiny", dict(), "fp8", "HND"),
    ("tiny", dict(), "fp16", "HND"),
    ("tiny", dict(N=300, H=2), "fp8", "NHD"),
    ("tiny", dict(N=1, H=1), "fp8", "HND"),
    ("tiny", dict(N=17, H=1), "fp16", "HND"),
    ("tiny", dict(N=129, H=1), "fp8", "HND"),
    ("tiny", dict(N=515, B=2, H=1), "fp8", "HND"),
    ("causal_prefill", dict(B=1, H=2, N=1000), "fp8", "HND"),
    ("causal_prefill", dict(B=2, H=1, N=300), "fp16", "NHD"),
    ("causal_prefill", dict(B=1, H=1, N=1), "fp8", "HND"),
    ("outlier", dict(B=1, H=2, N=1100), "fp8", "HND"),
    ("outlier", dict(B=1, H=2, N=1100), "fp16", "HND"),
]


@pytest.mark.parametrize("name,kw,pv,layout", ATTN_CASES)
def test_attention_matches_oracle(sage, orc, name, kw, pv, layout):
    wl = si.make(name, **kw)
    qz, vq, vs, out = run_gpu(sage, wl, pv, layout)
    out = out.cpu().numpy()
    q, k, v, oz, ovq, ovs = oracle_quant(orc, wl, pv)
    g = gpu_quant_np(qz, vq, vs, wl.N, pv)
    assert_quant_bitexact(g, oz, ovq, ovs, wl.N)
    rows = np.arange(wl.N)
    o_or = np.stack([np.stack([orc.attn_rows_head(oz, ovq, ovs, b, h, rows, wl.causal, wl.sm_scale, pv)
                               for h in range(wl.H)]) for b in range(wl.B)])
    assert np.isfinite(out).all()
    err = np.abs(out - o_or).max()
    c = _cos(out, o_or)
    assert err <= MAX_ABS and c >= COS_ORACLE, (err, c)
    if wl.N >= 64:
        ref = np.stack([np.stack([orc.ref64_rows_head(q, k, v, b, h, rows, wl.causal, wl.sm_scale)
                                  for h in range(wl.H)]) for b in range(wl.B)])
        c_gpu, c_or = _cos(out, ref), _cos(o_or, ref)
        if name == "outlier":
            assert abs(c_gpu - c_or) < 2e-4, (c_gpu, c_or)
        else:
            assert c_gpu >= COS_FP64, c_gpu


def test_binding_refuses_operands_of_the_wrong_size(sage):
    """Operands that would make a kernel read or write outside them are
    refused before anything is launched."""
    wl = si.make("tiny", N=300, H=2, device="cuda")
    qz = sage.quant_qk(wl.q, wl.k)
    vq, vs = sage.quant_v(wl.v, "fp8")
    vq16, _ = sage.quant_v(wl.v, "fp16")
    with pytest.raises(ValueError, match="vq"):
        sage.attn_fwd(qz, vq[:, :, :-1].contiguous(), vs)
    with pytest.raises(ValueError, match="vq"):
        sage.attn_fwd(qz, vq16, vs, pv="fp8")
    with pytest.raises(ValueError, match="vs"):
        sage.attn_fwd(qz, vq, vs.double())
    with pytest.raises(ValueError, match="out"):
        sage.attn_fwd(qz, vq, vs, out=torch.empty((1, 2, 299, 128), dtype=torch.bfloat16,
                                                  device="cuda"))
    with pytest.raises(ValueError, match="one GPU"):
        sage.attn_fwd(qz, vq, vs.cpu())
    with pytest.raises(ValueError, match="vq"):
        sage.attn_fwd_lse(qz, vq16, vs)
    o, lse = sage.attn_fwd_lse(qz, vq, vs)
    with pytest.raises(ValueError, match="lse"):
        sage.attn_bwd(qz, wl.v, o, o, lse[:, :, :-1].contiguous())
    with pytest.raises(ValueError, match="one GPU"):
        sage.attn_bwd(qz, wl.v, o, o.cpu(), lse)
    torch.cuda.synchronize()


def test_bf16_output_is_rounded_fp32_output(sage, orc):
    wl = si.make("tiny", N=400, H=2)
    *_, o32 = run_gpu(sage, wl, "fp8", out_dtype=torch.float32)
    *_, o16 = run_gpu(sage, wl, "fp8", out_dtype=torch.bfloat16)
    ref = orc.f32_to_bf16(o32.cpu().numpy())
    assert np.array_equal(codes(o16), ref)


def test_deterministic_across_runs(sage):
    wl = si.make("causal_prefill", B=1, H=2, N=900)
    outs = []
    for pv in ("fp8", "fp8", "fp16", "fp8"):
        qz, vq, vs, out = run_gpu(sage, wl, pv)
        if pv == "fp8":
            outs.append((qz["q8"].cpu(), qz["k8"].cpu(), vq.cpu(), out.cpu()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_output_guard_bands_untouched(sage):
    """Every output lands inside its buffer: guard bands around it survive."""
    wl = si.make("tiny", N=333, H=2)
    qd, kd, vd = wl.q.cuda(), wl.k.cuda(), wl.v.cuda()
    G = 4096
    qz = sage.quant_qk(qd, kd)
    vq, vs = sage.quant_v(vd)
    n = wl.B * wl.H * wl.N * wl.d
    buf = torch.full((n + 2 * G,), -7.0, dtype=torch.float32, device="cuda")
    out = buf[G:G + n].view(wl.B, wl.H, wl.N, wl.d)
    sage.attn_fwd(qz, vq, vs, sm_scale=wl.sm_scale, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:G] == -7.0) and torch.all(buf[G + n:] == -7.0)
    assert torch.isfinite(out).all()


# ------------------------------------------------- full workload sizes, sampled
FULL = [
    ("video_1p3b_480p", "fp8"),
    ("video_14b_720p", "fp8"),
    ("video_14b_720p", "fp16"),
    ("causal_prefill", "fp8"),
    ("outlier", "fp8"),
    ("outlier", "fp16"),
]


def sample_rows(wl, b, h, rng):
    nblk = -(-wl.N // 128)
    blocks = sorted({0, 1, nblk - 1, int(rng.integers(2, nblk - 1))})
    rows = []
    for blk in blocks:
        r0, r1 = blk * 128, min(wl.N, blk * 128 + 128)
        rows += list(range(r0, min(r1, r0 + 16))) + list(range(max(r0, r1 - 16), r1))
    if wl.outlier_tokens is not None:
        rows += wl.outlier_tokens[b, h, :16].cpu().tolist()
    return np.array(sorted(set(rows)), np.int32)


@pytest.mark.parametrize("name,pv", FULL)
def test_full_size_sampled(sage, orc, name, pv):
    """The workload at full size in the benchmark's launch configuration;
    quantization bit-exact on sampled heads, attention on sampled rows."""
    print(f"[full-size parity] {name} pv={pv}", flush=True)
    wl = si.make(name, device="cuda")
    qz = sage.quant_qk(wl.q, wl.k)
    vq, vs = sage.quant_v(wl.v, pv)
    out = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = [(0, 0), (wl.B - 1, wl.H - 1)]
    rng = np.random.default_rng(1)
    q, k, v, oz, ovq, ovs = oracle_quant(orc, wl, pv, heads)
    nblk = -(-wl.N // 128)
    g = {key: np.stack([qz[key][b, h].cpu().numpy() for b, h in heads])
         for key in ("q8", "q_scale", "k8", "k_scale", "k_mean")}
    vqh = torch.stack([vq[b, h] for b, h in heads]).cpu()
    vqh = vqh.view(torch.int16).numpy().view(np.uint16) if pv == "fp16" else vqh.numpy()
    g["vq"] = vq_natural(vqh[None], wl.N)[0]
    g["v_scale"] = np.stack([vs[b, h].cpu().numpy() for b, h in heads])
    bits = lambda a: np.ascontiguousarray(a).view(np.uint32)
    assert np.array_equal(g["q8"][:, :wl.N], oz["q8"]) and np.array_equal(g["k8"][:, :wl.N], oz["k8"])
    for key in ("q_scale", "k_scale", "k_mean"):
        assert np.array_equal(bits(g[key]), bits(oz[key])), key
    assert np.array_equal(g["vq"], ovq) and np.array_equal(bits(g["v_scale"]), bits(ovs))
    o_all, r_all, or_all = [], [], []
    for i, (b, h) in enumerate(heads):
        rows = sample_rows(wl, b, h, rng)
        ozh = {key: (val[i][None, None] if isinstance(val, np.ndarray) else val)
               for key, val in oz.items()}
        o_or = orc.attn_rows_head(ozh, ovq[i][None, None], ovs[i][None, None], 0, 0, rows,
                                  wl.causal, wl.sm_scale, pv)
        o_gpu = out[b, h, torch.from_numpy(rows).long().cuda()].cpu().numpy()
        ref = orc.ref64_rows_head(q[0][i][None, None], k[0][i][None, None], v[0][i][None, None],
                                  0, 0, rows, wl.causal, wl.sm_scale)
        o_all.append(o_gpu), or_all.append(o_or), r_all.append(ref)
    o_gpu, o_or, ref = (np.concatenate(x) for x in (o_all, or_all, r_all))
    err, c = np.abs(o_gpu - o_or).max(), _cos(o_gpu, o_or)
    c_gpu, c_or = _cos(o_gpu, ref), _cos(o_or, ref)
    print(f"  max-abs {err:.3e} cos(oracle) {c:.7f} cos64 gpu {c_gpu:.6f} oracle {c_or:.6f}")
    assert err <= MAX_ABS and c >= COS_ORACLE, (err, c)
    if name == "outlier":
        assert abs(c_gpu - c_or) < 2e-4, (c_gpu, c_or)
    else:
        assert c_gpu >= COS_FP64, c_gpu


@pytest.mark.xfail(strict=True, reason=(
    "unmet bar, kept visible: the outlier workload (d = 64, x30 query tokens) reaches "
    "about 0.9968 against FP64 attention at full size, as the oracle does (the INT8 "
    "resolution of K times the large queries); test_full_size_sampled holds the GPU "
    "to the oracle's own FP64 cosine within 2e-4"))
@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_outlier_full_size_gpu_meets_fp64_bar(sage, orc, pv):
    """The FP64 bar (cosine >= 0.999 against plain attention) on the GPU output
    of the outlier workload at full size, on the first head's sampled rows (the
    outlier tokens included)."""
    print(f"[outlier FP64 bar] pv={pv}", flush=True)
    wl = si.make("outlier", device="cuda")
    qz = sage.quant_qk(wl.q, wl.k)
    vq, vs = sage.quant_v(wl.v, pv)
    out = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sample_rows(wl, 0, 0, np.random.default_rng(2))
    q, k, v = (codes(x[:1, :1]) for x in (wl.q, wl.k, wl.v))
    ref = orc.ref64_rows_head(q, k, v, 0, 0, rows, wl.causal, wl.sm_scale)
    o_gpu = out[0, 0, torch.from_numpy(rows).long().cuda()].cpu().numpy()
    c = _cos(o_gpu, ref)
    print(f"  cos64 gpu {c:.6f}")
    assert c >= COS_FP64, c


# ------------------------------------------------------- per-token Q scales
def run_gpu_token(sage, wl, pv, layout="HND"):
    qd, kd, vd = (_to_layout(t, layout).cuda() for t in (wl.q, wl.k, wl.v))
    qz = sage.quant_qk(qd, kd, layout, q_gran="token")
    vq, vs = sage.quant_v(vd, pv, layout)
    out = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    return qz, vq, vs, to_hnd(out, layout)


TOKEN_CASES = [
    ("tiny", dict(N=300, H=2), "fp8", "HND"),
    ("tiny", dict(N=1, H=1), "fp8", "NHD"),
    ("tiny", dict(N=129, H=1), "fp16", "HND"),
    ("causal_prefill", dict(B=2, H=1, N=700), "fp8", "NHD"),
    ("outlier", dict(B=1, H=2, N=1100), "fp8", "HND"),
    ("outlier", dict(B=1, H=2, N=1100), "fp16", "HND"),
]


@pytest.mark.parametrize("name,kw,pv,layout", TOKEN_CASES)
def test_per_token_q_matches_oracle(sage, orc, name, kw, pv, layout):
    """sage_quant_qk_ex / sage_attn_fwd_ex with one Q scale per query row:
    codes and scales bit-exact (padded rows: codes 0, scale 0; K as with
    per-block Q), the output within the parity bars of the oracle run with
    the same granularity."""
    wl = si.make(name, **kw)
    qz, vq, vs, out = run_gpu_token(sage, wl, pv, layout)
    out = out.cpu().numpy()
    q, k, v = codes(wl.q), codes(wl.k), codes(wl.v)
    oz = orc.quant_qk(q, k, q_gran="token")
    ovq, ovs = orc.quant_v(v, pv)
    N = wl.N
    q8, qs = qz["q8"].cpu().numpy(), qz["q_scale"].cpu().numpy()
    assert qs.shape == (wl.B, wl.H, -(-N // 128) * 128)
    assert np.array_equal(q8[:, :, :N], oz["q8"]) and not q8[:, :, N:].any()
    assert np.array_equal(qs[:, :, :N].view(np.uint32), oz["q_scale"].view(np.uint32))
    assert not qs[:, :, N:].any()
    assert np.array_equal(qz["k8"][:, :, :N].cpu().numpy(), oz["k8"])
    assert np.array_equal(qz["k_scale"].cpu().numpy().view(np.uint32), oz["k_scale"].view(np.uint32))
    rows = np.arange(N)
    o_or = np.stack([np.stack([orc.attn_rows_head(oz, ovq, ovs, b, h, rows, wl.causal, wl.sm_scale, pv)
                               for h in range(wl.H)]) for b in range(wl.B)])
    assert np.isfinite(out).all()
    err, c = np.abs(out - o_or).max(), _cos(out, o_or)
    assert err <= MAX_ABS and c >= COS_ORACLE, (err, c)
    if N >= 64:
        ref = np.stack([np.stack([orc.ref64_rows_head(q, k, v, b, h, rows, wl.causal, wl.sm_scale)
                                  for h in range(wl.H)]) for b in range(wl.B)])
        c_gpu, c_or = _cos(out, ref), _cos(o_or, ref)
        assert abs(c_gpu - c_or) < 2e-4, (c_gpu, c_or)


@pytest.mark.parametrize("name,pv", [("outlier", "fp8"), ("video_14b_720p", "fp8")])
def test_per_token_q_full_size_sampled(sage, orc, name, pv):
    """Per-token Q at full size in the benchmark's launch configuration, on
    sampled heads and rows (the outlier tokens included)."""
    print(f"[full-size per-token parity] {name} pv={pv}", flush=True)
    wl = si.make(name, device="cuda")
    qz = sage.quant_qk(wl.q, wl.k, q_gran="token")
    vq, vs = sage.quant_v(wl.v, pv)
    out = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = [(0, 0), (wl.B - 1, wl.H - 1)]
    rng = np.random.default_rng(2)
    qa, ka, va = codes(wl.q.cpu()), codes(wl.k.cpu()), codes(wl.v.cpu())
    o_all, or_all, r_all = [], [], []
    for b, h in heads:
        q, k, v = (x[b, h][None, None] for x in (qa, ka, va))
        oz = orc.quant_qk(q, k, q_gran="token")
        ovq, ovs = orc.quant_v(v, pv)
        assert np.array_equal(qz["q8"][b, h, :wl.N].cpu().numpy(), oz["q8"][0, 0])
        assert np.array_equal(qz["q_scale"][b, h, :wl.N].cpu().numpy().view(np.uint32),
                              oz["q_scale"][0, 0].view(np.uint32))
        rows = sample_rows(wl, b, h, rng)
        o_or = orc.attn_rows_head(oz, ovq, ovs, 0, 0, rows, wl.causal, wl.sm_scale, pv)
        o_gpu = out[b, h, torch.from_numpy(rows).long().cuda()].cpu().numpy()
        ref = orc.ref64_rows_head(q, k, v, 0, 0, rows, wl.causal, wl.sm_scale)
        o_all.append(o_gpu), or_all.append(o_or), r_all.append(ref)
    o_gpu, o_or, ref = (np.concatenate(x) for x in (o_all, or_all, r_all))
    err, c = np.abs(o_gpu - o_or).max(), _cos(o_gpu, o_or)
    c_gpu, c_or = _cos(o_gpu, ref), _cos(o_or, ref)
    print(f"  max-abs {err:.3e} cos(oracle) {c:.7f} cos64 gpu {c_gpu:.6f} oracle {c_or:.6f}")
    assert err <= MAX_ABS and c >= COS_ORACLE, (err, c)
    assert abs(c_gpu - c_or) < 2e-4, (c_gpu, c_or)
    if name != "outlier":
        assert c_gpu >= COS_FP64, c_gpu


# ------------------------------------------------------ block-sparse tile skipping
def make_tile_mask(B, H, N, kind, seed=0, keep=0.5):
    """uint8 [B, H, nblk, nblk] (query block x key tile, nonzero = visit)."""
    nb = -(-N // 128)
    rng = np.random.default_rng(seed)
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    if kind == "ones":
        m = np.ones((B, H, nb, nb), bool)
    elif kind == "random":
        m = rng.random((B, H, nb, nb)) < keep
    elif kind == "band":                       # a local window plus the first tile
        m = np.broadcast_to((np.abs(i - j) <= 1) | (j == 0), (B, H, nb, nb)).copy()
    elif kind == "split":                      # the two query blocks of a workgroup differ
        m = np.broadcast_to(((i % 2 == 0) & (j % 2 == 0)) | ((i % 2 == 1) & (j % 3 == 1)),
                            (B, H, nb, nb)).copy()
    elif kind == "empty_rows":                 # some query blocks visit nothing at all
        m = rng.random((B, H, nb, nb)) < keep
        m[:, :, 1] = False
        m[:, :, -1] = False
    else:
        raise ValueError(kind)
    return m.astype(np.uint8)


SPARSE_CASES = [
    ("tiny", dict(N=1000, H=2), "fp8", "HND", "random", "block"),
    ("tiny", dict(N=1000, H=2), "fp8", "HND", "ones", "block"),
    ("tiny", dict(N=700, H=1), "fp16", "NHD", "random", "block"),
    ("tiny", dict(N=1000, H=2), "fp8", "HND", "empty_rows", "block"),
    ("tiny", dict(N=900, H=2), "fp8", "HND", "split", "token"),
    ("causal_prefill", dict(B=2, H=1, N=900), "fp8", "HND", "random", "block"),
    ("causal_prefill", dict(B=1, H=2, N=1000), "fp8", "NHD", "band", "block"),
    ("outlier", dict(B=1, H=2, N=1100), "fp8", "HND", "band", "block"),
]


@pytest.mark.parametrize("name,kw,pv,layout,kind,q_gran", SPARSE_CASES)
def test_sparse_matches_oracle(sage, orc, name, kw, pv, layout, kind, q_gran):
    """sage_attn_fwd_sparse against the oracle run with the same tile mask;
    an all-ones mask reproduces the dense kernel bit for bit; query blocks
    that visit nothing get exact zeros."""
    wl = si.make(name, **kw)
    mask = make_tile_mask(wl.B, wl.H, wl.N, kind, seed=7)
    qd, kd, vd = (_to_layout(t, layout).cuda() for t in (wl.q, wl.k, wl.v))
    qz = sage.quant_qk(qd, kd, layout, q_gran=q_gran)
    vq, vs = sage.quant_v(vd, pv, layout)
    out = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                        out_dtype=torch.float32, tile_mask=torch.from_numpy(mask).cuda())
    dense = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    out, dense = to_hnd(out, layout).cpu().numpy(), to_hnd(dense, layout).cpu().numpy()
    q, k, v = codes(wl.q), codes(wl.k), codes(wl.v)
    oz = orc.quant_qk(q, k, q_gran=q_gran)
    ovq, ovs = orc.quant_v(v, pv)
    rows = np.arange(wl.N)
    o_or = np.stack([np.stack([orc.attn_rows_head(oz, ovq, ovs, b, h, rows, wl.causal, wl.sm_scale,
                                                  pv, tile_mask=mask)
                               for h in range(wl.H)]) for b in range(wl.B)])
    assert np.isfinite(out).all()
    err, c = np.abs(out - o_or).max(), _cos(out, o_or)
    assert err <= MAX_ABS and c >= COS_ORACLE, (err, c)
    if kind == "ones":
        assert np.array_equal(out, dense)
    empty = o_or.reshape(wl.B, wl.H, wl.N, -1).any(axis=-1) == 0
    assert not out[empty].any()
    if kind == "empty_rows":
        assert empty.any()


def test_sparse_full_size_sampled(sage, orc):
    """video_14b_720p with a band-plus-random tile mask (about 1/4 of the
    tiles), in the benchmark's launch configuration, on sampled heads/rows."""
    print("[full-size sparse parity] video_14b_720p pv=fp8", flush=True)
    wl = si.make("video_14b_720p", device="cuda")
    mask = make_tile_mask(wl.B, wl.H, wl.N, "random", seed=3, keep=0.2)
    mask |= make_tile_mask(wl.B, wl.H, wl.N, "band")
    qz = sage.quant_qk(wl.q, wl.k)
    vq, vs = sage.quant_v(wl.v, "fp8")
    out = sage.attn_fwd(qz, vq, vs, sm_scale=wl.sm_scale, out_dtype=torch.float32,
                        tile_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    heads = [(0, 0), (0, wl.H - 1)]
    rng = np.random.default_rng(4)
    qa, ka, va = codes(wl.q.cpu()), codes(wl.k.cpu()), codes(wl.v.cpu())
    o_all, or_all = [], []
    for b, h in heads:
        q, k, v = (x[b, h][None, None] for x in (qa, ka, va))
        oz = orc.quant_qk(q, k)
        ovq, ovs = orc.quant_v(v, "fp8")
        rows = sample_rows(wl, b, h, rng)
        o_or = orc.attn_rows_head(oz, ovq, ovs, 0, 0, rows, False, wl.sm_scale, "fp8",
                                  tile_mask=mask[b:b + 1, h:h + 1])
        o_all.append(out[b, h, torch.from_numpy(rows).long().cuda()].cpu().numpy())
        or_all.append(o_or)
    o_gpu, o_or = np.concatenate(o_all), np.concatenate(or_all)
    err, c = np.abs(o_gpu - o_or).max(), _cos(o_gpu, o_or)
    print(f"  max-abs {err:.3e} cos(oracle) {c:.7f} kept {mask.mean():.3f} of the tiles")
    assert err <= MAX_ABS and c >= COS_ORACLE, (err, c)


def test_k_mean_exact_with_large_and_special_values(sage, orc):
    """The K statistics take an fp64 fast path while every value of a load is
    below 2^18 and the saturating integer path otherwise: mix both (large
    finite values, +-inf, NaN) into some rows; the K mean stays bit-exact."""
    wl = si.make("tiny", N=1500, H=2, seed=23)
    k = codes(wl.k).copy()
    rng = np.random.default_rng(5)
    specials = np.array([0x4880, 0xC880, 0x4F00, 0xCF00, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC1,
                         0x4A00, 0x0001, 0x8001], np.uint16)
    rows = rng.choice(wl.N, 40, replace=False)
    for i, r in enumerate(rows):
        k[0, i % 2, r, rng.integers(0, 128, 3)] = specials[i % len(specials)]
    kt = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).cuda()
    qz = sage.quant_qk(wl.q.cuda(), kt)
    fz, _, _ = sage.quant_qkv(wl.q.cuda(), kt, wl.v.cuda())
    torch.cuda.synchronize()
    ref = np.stack([orc.k_mean_head(k[0, h]) for h in range(2)])[None]
    for z in (qz, fz):
        got = z["k_mean"].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_d64_many_heads_matches_oracle(sage, orc, pv):
    """d = 64 with many heads: the launcher runs the 12-wave (384-query)
    non-pipelined sweep here (its rounds over the CUs beat the 8-wave ones);
    sampled heads against the oracle, every row, ragged N."""
    print(f"[d=64 many heads] pv={pv}", flush=True)
    wl = si.make("outlier", B=1, H=256, N=1000, seed=31)
    qz, vq, vs, out = run_gpu(sage, wl, pv)
    out = out.cpu().numpy()
    heads = [(0, 0), (0, 97), (0, 255)]
    q, k, v, oz, ovq, ovs = oracle_quant(orc, wl, pv, heads)
    rows = np.arange(wl.N)
    for i, (b, h) in enumerate(heads):
        ozh = {key: (val[i][None, None] if isinstance(val, np.ndarray) else val)
               for key, val in oz.items()}
        o_or = orc.attn_rows_head(ozh, ovq[i][None, None], ovs[i][None, None], 0, 0, rows, False,
                                  wl.sm_scale, pv)
        err, c = np.abs(out[b, h] - o_or).max(), _cos(out[b, h], o_or)
        assert err <= MAX_ABS and c >= COS_ORACLE, (h, err, c)


# --------------------------------------------------------- degenerate inputs
def _bf16_tensor(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_degenerate_inputs(sage, orc, pv):
    """Constant keys (smoothed K is exactly 0, so k_scale = 0 and the
    dequantization constant c = 0), an all-zero Q, an all-zero V and a zero V
    channel, each against the oracle and against its closed form."""
    rng = np.random.default_rng(41)
    N, d = 700, 128
    q = rng.standard_normal((1, 4, N, d)).astype(np.float32)
    k = rng.standard_normal((1, 4, N, d)).astype(np.float32)
    v = rng.standard_normal((1, 4, N, d)).astype(np.float32)
    k[0, 0] = rng.standard_normal(d)[None, :]      # head 0: every key the same
    q[0, 1] = 0.0                                  # head 1: Q all zero
    v[0, 2] = 0.0                                  # head 2: V all zero
    v[0, 3, :, 5] = 0.0                            # head 3: one zero V channel
    qt, kt, vt = (_bf16_tensor(x).cuda() for x in (q, k, v))
    qz = sage.quant_qk(qt, kt)
    vq, vs = sage.quant_v(vt, pv)
    sm = 1.0 / math.sqrt(d)
    out = sage.attn_fwd(qz, vq, vs, sm_scale=sm, pv=pv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    qc, kc, vc = (codes(_bf16_tensor(x)) for x in (q, k, v))
    oz = orc.quant_qk(qc, kc)
    ovq, ovs = orc.quant_v(vc, pv)
    assert np.array_equal(qz["k8"][:, :, :N].cpu().numpy(), oz["k8"])
    assert not oz["k8"][0, 0].any() and oz["k_scale"][0, 0].max() == 0.0
    rows = np.arange(N)
    for h in range(4):
        o_or = orc.attn_rows_head(oz, ovq, ovs, 0, h, rows, False, sm, pv)
        err = np.abs(out[0, h] - o_or).max()
        assert err <= MAX_ABS, (h, err)
    dec = orc.f16_to_f32 if pv == "fp16" else orc.e4m3_to_f32
    vdq = dec(ovq[0]).reshape(4, N, d).astype(np.float64) * ovs[0][:, None, :]
    # constant keys and zero Q: every score is equal, so O = the mean of the dequantized V
    for h in (0, 1):
        assert np.allclose(out[0, h], vdq[h].mean(axis=0)[None, :], rtol=1e-5, atol=1e-6), h
    assert not out[0, 2].any()
    assert not out[0, 3, :, 5].any()


def test_maximum_sequence_length(sage, orc):
    """N = 2^20 keys (8192 key tiles; offsets beyond 2^31 bytes per tensor
    pair): quantization of sampled heads bit-exact, sampled rows (first,
    last, middle, ragged) against the oracle."""
    print("[max size] B=1 H=2 N=2^20 d=128", flush=True)
    N = 1 << 20
    wl = si.make("tiny", N=N, H=2, seed=43, device="cuda")
    qz = sage.quant_qk(wl.q, wl.k)
    vq, vs = sage.quant_v(wl.v, "fp8")
    out = sage.attn_fwd(qz, vq, vs, sm_scale=wl.sm_scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 300_001, N // 2, N - 129, N - 2, N - 1], np.int32)
    for h in range(2):
        q, k, v = (codes(t[0:1, h:h + 1].cpu()) for t in (wl.q, wl.k, wl.v))
        oz = orc.quant_qk(q, k)
        ovq, ovs = orc.quant_v(v, "fp8")
        assert np.array_equal(qz["k8"][0, h, :N].cpu().numpy(), oz["k8"][0, 0])
        assert np.array_equal(qz["k_mean"][0, h].cpu().numpy().view(np.uint32),
                              oz["k_mean"][0, 0].view(np.uint32))
        o_or = orc.attn_rows_head(oz, ovq, ovs, 0, 0, rows, False, wl.sm_scale, "fp8")
        o_gpu = out[0, h, torch.from_numpy(rows).long().cuda()].cpu().numpy()
        err, c = np.abs(o_gpu - o_or).max(), _cos(o_gpu, o_or)
        print(f"  head {h}: max-abs {err:.3e} cos {c:.7f}", flush=True)
        assert err <= MAX_ABS and c >= COS_ORACLE, (h, err, c)
