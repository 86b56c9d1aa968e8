"""Pins of the oracle's Q smoothing (outlier smoothing applied to Q as well).

Per block of 128 queries the channel means are taken exactly like the K
mean, Q minus its block mean is quantized, and the mean's share of each score
returns as an FP32 correction.  Pinned by FP64 numpy block means, the
reconstruction codes * scale + mean ~ Q, the correction against an FP64 dot
product within the fp32 error bound, exact zeros for zero-mean blocks, the
single-tile one-shot softmax, a tile-by-tile non-online recomputation with the
correction, and the FP64 attention cosine with and without smoothing on
inputs whose queries carry a per-channel offset.
"""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si

L8 = np.float32(math.log2(448.0))
LOG2E = 1.4426950408889634


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _codes(N, H=1, seed=3, q_sigma=4.0):
    wl = si.make("tiny", N=N, H=H, seed=seed, q_sigma=q_sigma)
    return wl, *(si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))


def test_block_means_match_fp64(orc):
    wl, q, k, v = _codes(300)                       # blocks of 128, 128, 44 rows
    z = orc.quant_qk(q, k, q_smooth=True)
    qf = orc.bf16_to_f32(q).reshape(q.shape)[0, 0].astype(np.float64)
    assert z["q_mean"].shape == (1, 1, 3, 128)
    for r, (r0, r1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        ref = qf[r0:r1].mean(axis=0)
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(z["q_mean"][0, 0, r].astype(np.float64) - ref) <= ulp + 2.0**-30), r
    # a column that is constant inside a block has that constant as its mean
    col = np.array([1.5, -0.375, 96.0, 0.0] * 32, np.float32)
    qc = _bf16(np.tile(col, (200, 1))).reshape(1, 1, 200, 128)
    zc = orc.quant_qk(qc, qc, q_smooth=True)
    assert np.array_equal(zc["q_mean"][0, 0, 0], col) and np.array_equal(zc["q_mean"][0, 0, 1], col)
    assert not zc["q8"].any() and not zc["q_scale"].any()     # Q minus its mean is 0


@pytest.mark.parametrize("q_gran", ["block", "token"])
def test_codes_are_the_plain_quantization_of_q_minus_its_mean(orc, q_gran):
    wl, q, k, v = _codes(300, seed=5)
    z = orc.quant_qk(q, k, q_gran=q_gran, q_smooth=True)
    qf = orc.bf16_to_f32(q).reshape(q.shape)[0, 0]
    rowmean = np.repeat(z["q_mean"][0, 0], 128, axis=0)[:300]
    shifted = (qf - rowmean).astype(np.float32)           # one fp32 rounding, in numpy
    if q_gran == "block":
        for r, (r0, r1) in enumerate([(0, 128), (128, 256), (256, 300)]):
            codes, s = orc.quant_block(shifted[r0:r1])
            assert np.array_equal(z["q8"][0, 0, r0:r1], codes) and z["q_scale"][0, 0, r] == np.float32(s)
        scale = np.repeat(z["q_scale"][0, 0], 128)[:300, None]
    else:
        for i in (0, 1, 127, 128, 299):
            codes, s = orc.quant_block(shifted[i:i + 1])
            assert np.array_equal(z["q8"][0, 0, i], codes[0]) and z["q_scale"][0, 0, i] == np.float32(s)
        scale = z["q_scale"][0, 0][:, None]
    # reconstruction: codes * scale + mean is Q within half a step (plus the mean's rounding)
    rec = z["q8"][0, 0].astype(np.float64) * scale + rowmean
    slack = np.spacing(np.abs(qf).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(rec - qf) <= scale * (0.5 + 1e-5) + slack)
    # the offset is gone from the quantized part: the block absmax shrinks
    assert z["q_scale"].max() < orc.quant_qk(q, k, q_gran=q_gran)["q_scale"].max() / 2


def test_bias_matches_fp64_dot_product(orc):
    wl, q, k, v = _codes(300, H=2, seed=7)
    z = orc.quant_qk(q, k, q_smooth=True)
    bias = orc.smooth_bias(z, k, wl.sm_scale)
    assert bias.shape == (1, 2, 3, 300) and bias.dtype == np.float32
    lam = np.float64(orc.lam(wl.sm_scale))
    kf = orc.bf16_to_f32(k).reshape(k.shape)
    d = k.shape[-1]
    gamma = d * 2.0**-24 / (1 - d * 2.0**-24)               # fp32 dot-product error bound
    for h in range(2):
        kp = (kf[0, h] - z["k_mean"][0, h]).astype(np.float32).astype(np.float64)
        qm = z["q_mean"][0, h].astype(np.float64)
        ref = lam * (qm @ kp.T)
        bound = lam * gamma * (np.abs(qm) @ np.abs(kp).T) + np.spacing(np.abs(ref).astype(np.float32))
        assert np.all(np.abs(bias[0, h].astype(np.float64) - ref) <= bound), h
    # sign and scale: doubling sm_scale doubles lambda, and the bias with it
    b2 = orc.smooth_bias(z, k, 2 * wl.sm_scale)
    assert np.allclose(b2, 2 * bias, rtol=1e-6, atol=0)


def test_zero_mean_blocks_change_nothing(orc):
    """Blocks whose rows come in +-x pairs have mean 0: codes, scales and the
    correction are those of the unsmoothed quantization, bias 0."""
    rng = np.random.default_rng(9)
    half = rng.standard_normal((64, 128)).astype(np.float32)
    qb = np.concatenate([half, -half])
    q = _bf16(np.concatenate([qb, qb[::-1]])).reshape(1, 1, 256, 128)
    k = _bf16(rng.standard_normal((256, 128)) + 2).reshape(1, 1, 256, 128)
    zs = orc.quant_qk(q, k, q_smooth=True)
    zp = orc.quant_qk(q, k)
    assert not zs["q_mean"].any()
    assert np.array_equal(zs["q8"], zp["q8"]) and np.array_equal(zs["q_scale"], zp["q_scale"])
    assert not orc.smooth_bias(zs, k, 0.1).any()


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
@pytest.mark.parametrize("N", [1, 40, 128])
def test_single_tile_brute_force_with_bias(orc, pv, N):
    """One key tile: the online softmax is the one-shot softmax of the scores
    dq . dk^T sm_scale + bias / log2(e) (the correction in natural units)."""
    wl, q, k, v = _codes(N, seed=11 + N, q_sigma=5.0)
    z = orc.quant_qk(q, k, q_smooth=True)
    bias = orc.smooth_bias(z, k, wl.sm_scale)
    vq, vs = orc.quant_v(v, pv)
    out = orc.attn_rows_head(z, vq, vs, 0, 0, np.arange(N), False, wl.sm_scale, pv, bias=bias)
    dq = z["q8"][0, 0].astype(np.float64) * np.float64(z["q_scale"][0, 0, 0])
    dk = z["k8"][0, 0].astype(np.float64) * np.float64(z["k_scale"][0, 0, 0])
    dec = orc.f16_to_f32(vq) if pv == "fp16" else orc.e4m3_to_f32(vq)
    dv = dec.reshape(vq.shape)[0, 0].astype(np.float64) * vs[0, 0]
    s = dq @ dk.T * wl.sm_scale + bias[0, 0, 0][None, :].astype(np.float64) / LOG2E
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ dv
    rel = 2.0**-11 if pv == "fp16" else 2.0**-4
    assert np.abs(out - ref).max() <= rel * 1.05 * np.abs(dv).max() + 1e-5


def _non_online_bias(orc, z, bias, vq, vs, i, causal, sm_scale, pv):
    """Row i tile by tile with the correction, tiles combined at the end with
    weights 2^(M_t - M_final) (no running rescale)."""
    q8 = z["q8"][0, 0].astype(np.int64)
    k8 = z["k8"][0, 0].astype(np.int64)
    N = k8.shape[0]
    lam = np.float32(orc.lam(sm_scale))
    sigma = np.float32(z["q_scale"][0, 0, i // z["qblk"]] * lam)
    dec = orc.f16_to_f32 if pv == "fp16" else orc.e4m3_to_f32
    enc = orc.f32_to_f16 if pv == "fp16" else orc.f32_to_e4m3
    vdec = dec(vq[0, 0]).reshape(vq.shape[2:]).astype(np.float64)
    brow = bias[0, 0, i // 128]
    n_keys = i + 1 if causal else N
    S = q8[i] @ k8[:n_keys].T
    Ms, Ls, Ts = [], [], []
    M = np.float32(-np.inf)
    for t0 in range(0, n_keys, 128):
        St = S[t0:t0 + 128]
        c = np.float32(sigma * z["k_scale"][0, 0, t0 // 128])
        # fma(S, c, bias): the exact value rounded once
        s = (St.astype(np.float64) * np.float64(c) + brow[t0:t0 + len(St)].astype(np.float64)).astype(np.float32)
        M = max(M, s.max())
        mu = np.float32(M - L8)
        p = np.exp2((s - mu).astype(np.float32).astype(np.float64)).astype(np.float32)
        Ms.append(M)
        pq = dec(enc(p)).astype(np.float64)
        Ls.append(pq.sum())  # the row sum adds the quantized P the P V product uses
        Ts.append(pq @ vdec[t0:t0 + len(St)])
    w = np.exp2(np.array(Ms, np.float64) - np.float64(M))
    num = sum(wt * Tt for wt, Tt in zip(w, Ts))
    return num * vs[0, 0] / (w @ np.array(Ls)), M, w @ np.array(Ls)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("q_gran", ["block", "token"])
def test_online_bookkeeping_with_bias_matches_non_online(orc, pv, causal, q_gran):
    wl, q, k, v = _codes(700, seed=13)                    # 6 tiles, the last ragged
    z = orc.quant_qk(q, k, q_gran=q_gran, q_smooth=True)
    bias = orc.smooth_bias(z, k, wl.sm_scale)
    vq, vs = orc.quant_v(v, pv)
    rows = np.array([0, 5, 127, 128, 300, 511, 640, 699])
    out, m, l = orc.attn_rows_head(z, vq, vs, 0, 0, rows, causal, wl.sm_scale, pv,
                                   return_ml=True, bias=bias)
    for r, i in enumerate(rows):
        ref, M, Lf = _non_online_bias(orc, z, bias, vq, vs, i, causal, wl.sm_scale, pv)
        assert m[r] == M
        assert abs(l[r] / Lf - 1) < 2e-6
        assert np.abs(out[r] - ref).max() <= 2e-6 * np.abs(ref).max() + 1e-7


@pytest.mark.parametrize("pv,floor,gain", [("fp8", 0.9996, 1.25), ("fp16", 0.99995, 10.0)])
def test_smoothing_q_restores_accuracy_under_query_offsets(orc, pv, floor, gain):
    """Queries with a per-channel offset (sigma 6): without Q smoothing the
    offset eats the INT8 range of Q; with it the FP64 cosine is back near the
    offset-free level (the FP8 P then dominates what error is left)."""
    wl, q, k, v = _codes(1024, H=2, seed=17, q_sigma=6.0)
    plain, *_ = orc.attention(q, k, v, False, wl.sm_scale, pv)
    smooth, *_ = orc.attention(q, k, v, False, wl.sm_scale, pv, q_smooth=True)
    rows = np.arange(wl.N)
    for h in range(2):
        ref = orc.ref64_rows_head(q, k, v, 0, h, rows, False, wl.sm_scale)
        c0, c1 = _cos(plain[0, h], ref), _cos(smooth[0, h], ref)
        assert c1 >= floor and (1 - c1) * gain < 1 - c0, (h, c0, c1)


def test_smoothing_q_is_harmless_without_offsets(orc):
    wl = si.make("tiny")
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    smooth, *_ = orc.attention(q, k, v, False, wl.sm_scale, "fp8", q_smooth=True)
    for h in range(wl.H):
        ref = orc.ref64_rows_head(q, k, v, 0, h, np.arange(wl.N), False, wl.sm_scale)
        assert _cos(smooth[0, h], ref) >= 0.999
