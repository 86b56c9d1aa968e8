"""Pins of the oracle's quantized attention.

Nothing on the pages is numeric for this path, so the oracle is pinned by
FP64 softmax attention (its cosine), brute force on single-tile inputs, a
tile-by-tile non-online recomputation of the online bookkeeping, rows of P
summing to 1, the exact invariance of softmax to a per-channel key offset, and
closed-form special cases (constant keys, a peaked row, the first causal row).
"""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si

L8 = np.float32(math.log2(448.0))


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _quantize(orc, q, k, v, pv):
    z = orc.quant_qk(q, k)
    vq, vs = orc.quant_v(v, pv)
    return z, vq, vs


def _deq_v(orc, vq, vs, pv):
    dec = orc.f16_to_f32(vq) if pv == "fp16" else orc.e4m3_to_f32(vq)
    return dec.reshape(vq.shape).astype(np.float64) * vs[:, :, None, :]


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_tiny_workload_vs_fp64(orc, pv):
    wl = si.make("tiny")
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    out, *_ = orc.attention(q, k, v, False, wl.sm_scale, pv)
    rows = np.arange(wl.N)
    for h in range(wl.H):
        ref = orc.ref64_rows_head(q, k, v, 0, h, rows, False, wl.sm_scale)
        c = _cos(out[0, h], ref)
        assert c >= (0.999 if pv == "fp8" else 0.9998), (h, c)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64])
@pytest.mark.parametrize("q_gran", ["block", "token"])
def test_single_tile_brute_force(orc, pv, causal, N, q_gran):
    """N <= 64: one key tile, so the online softmax is the one-shot softmax.
    Compare with FP64 one-shot attention over the dequantized operands; the
    only gap left is P's rounding (fp16: 2^-11 relative, fp8: 2^-4)."""
    wl = si.make("tiny", N=N, H=1, seed=77 + N)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    z = orc.quant_qk(q, k, q_gran=q_gran)
    vq, vs = orc.quant_v(v, pv)
    rows = np.arange(N)
    out = orc.attn_rows_head(z, vq, vs, 0, 0, rows, causal, wl.sm_scale, pv)
    qsc = z["q_scale"][0, 0] if q_gran == "token" else np.full(N, z["q_scale"][0, 0, 0])
    dq = z["q8"][0, 0].astype(np.float64) * qsc[:, None].astype(np.float64)
    dk = z["k8"][0, 0].astype(np.float64) * z["k_scale"][0, 0, 0]
    dv = _deq_v(orc, vq, vs, pv)[0, 0]
    s = dq @ dk.T * wl.sm_scale
    if causal:
        s = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ dv
    rel = 2.0**-11 if pv == "fp16" else 2.0**-4
    assert np.abs(out - ref).max() <= rel * 1.05 * np.abs(dv).max() + 1e-6


def _non_online(orc, z, vq, vs, b, h, i, causal, sm_scale, pv):
    """Row i recomputed tile by tile without the online recurrence: every tile
    is evaluated against its running max, then the tiles are combined at once
    with weights 2^(M_t - M_final)."""
    q8 = z["q8"][b, h].astype(np.int64)
    k8 = z["k8"][b, h].astype(np.int64)
    N = k8.shape[0]
    lam = np.float32(orc.lam(sm_scale))
    sigma = np.float32(z["q_scale"][b, h, i // z["qblk"]] * lam)
    dec = orc.f16_to_f32 if pv == "fp16" else orc.e4m3_to_f32
    enc = orc.f32_to_f16 if pv == "fp16" else orc.f32_to_e4m3
    vdec = dec(vq[b, h]).reshape(vq.shape[2:]).astype(np.float64)
    n_keys = i + 1 if causal else N
    S = q8[i] @ k8[:n_keys].T
    Ms, Ls, Ts = [], [], []
    M = np.float32(-np.inf)
    for t0 in range(0, n_keys, 128):
        St = S[t0:t0 + 128]
        c = np.float32(sigma * z["k_scale"][b, h, t0 // 128])
        s = St.astype(np.float32) * c
        M = max(M, s.max())
        mu = np.float32(M - L8)
        arg = (St.astype(np.float64) * np.float64(c) - np.float64(mu)).astype(np.float32)
        p = np.exp2(arg.astype(np.float64)).astype(np.float32)
        pq = dec(enc(p)).astype(np.float64)
        Ms.append(M)
        Ls.append(pq.sum())  # the row sum adds the quantized P the P V product uses
        Ts.append(pq @ vdec[t0:t0 + len(St)])
    w = np.exp2(np.array(Ms, np.float64) - np.float64(M))
    num = sum(wt * Tt for wt, Tt in zip(w, Ts))
    return num * vs[b, h] / (w @ np.array(Ls)), M, w @ np.array(Ls)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("q_gran", ["block", "token"])
def test_online_bookkeeping_matches_non_online(orc, pv, causal, q_gran):
    wl = si.make("tiny", N=700, H=1, seed=91)  # 6 tiles, the last ragged (60 keys)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    z = orc.quant_qk(q, k, q_gran=q_gran)
    vq, vs = orc.quant_v(v, pv)
    rows = np.array([0, 5, 127, 128, 300, 511, 640, 699])
    out, m, l = orc.attn_rows_head(z, vq, vs, 0, 0, rows, causal, wl.sm_scale, pv, return_ml=True)
    for r, i in enumerate(rows):
        ref, M, Lf = _non_online(orc, z, vq, vs, 0, 0, i, causal, wl.sm_scale, pv)
        assert m[r] == M
        assert abs(l[r] / Lf - 1) < 2e-6
        assert np.abs(out[r] - ref).max() <= 2e-6 * np.abs(ref).max() + 1e-7


def test_p_rows_sum_to_one(orc):
    """With the final m and the unquantized row sum lx,
    sum_j 448 * 2^(s_j - m) / lx == 1 for every row (the log-sum-exp of the
    scores); with the row sum l of the quantized P the same holds up to the
    FP8 rounding of P (each value within 2^-4 of its p; the errors mostly
    cancel over a row)."""
    wl = si.make("causal_prefill", N=900, B=1, H=1, seed=5)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    z, vq, vs = _quantize(orc, q, k, v, "fp8")
    lam = orc.lam(wl.sm_scale)
    rows = np.array([0, 1, 63, 64, 129, 450, 899])
    for causal in (False, True):
        _, m, l, lx = orc.attn_rows_head(z, vq, vs, 0, 0, rows, causal, wl.sm_scale, "fp8",
                                         return_lx=True)
        S = z["q8"][0, 0].astype(np.int64) @ z["k8"][0, 0].astype(np.int64).T
        for r, i in enumerate(rows):
            n = i + 1 if causal else wl.N
            c = np.array([np.float32(np.float32(z["q_scale"][0, 0, i // 128] * np.float32(lam))
                                     * z["k_scale"][0, 0, j // 128]) for j in range(n)], np.float64)
            tot = (448.0 * np.exp2(S[i, :n] * c - np.float64(m[r]))).sum()
            assert abs(tot / lx[r] - 1) < 1e-5, (causal, i, tot / lx[r])
            assert abs(tot / l[r] - 1) < 2.0**-4, (causal, i, tot / l[r])


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_pass_through(orc, pv, causal):
    """Softmax weights sum to one, so a V whose rows are all equal comes out
    unchanged whatever Q and K are.  Each channel's value is its own absmax,
    so it is exactly +-448 in FP8 (exact in FP16): the quantized method keeps
    this exactly, up to fp32 rounding, only when the row sum l adds the same
    quantized P values the P V product weights V with (with l summed from the
    unquantized p the output is off by the FP8 rounding of P, ~1e-3 here)."""
    wl = si.make("tiny", N=700, H=1, seed=17)  # 6 tiles, the last ragged
    q, k = (si.bf16_codes(t) for t in (wl.q, wl.k))
    rng = np.random.default_rng(17)
    row = (rng.standard_normal(wl.d) * 2).astype(np.float32)
    v = np.broadcast_to(_bf16(row), (1, 1, wl.N, wl.d)).copy()
    vrow = orc.bf16_to_f32(v[0, 0, 0]).astype(np.float64)
    rows = np.array([0, 1, 2, 5, 127, 128, 300, 511, 640, 699])
    out, *_ = orc.attention(q, k, v, causal, wl.sm_scale, pv, rows=rows)
    # v_scale * 448 reproduces each channel value to about one fp32 rounding
    err = np.abs(out[0, 0] - vrow[None, :]).max() / np.abs(vrow).max()
    assert err <= 4e-7, err


def test_fp64_reference_offset_invariance(orc):
    """softmax is exactly invariant to adding a per-channel offset to every key."""
    rng = np.random.default_rng(11)
    N, d = 200, 64
    base = np.round(rng.uniform(-2, 2, (1, 1, N, d)) * 16) / 16
    off = rng.integers(-3, 4, (1, 1, 1, d)).astype(np.float64)
    q = _bf16(rng.standard_normal((1, 1, N, d))).reshape(1, 1, N, d)
    v = _bf16(rng.standard_normal((1, 1, N, d))).reshape(1, 1, N, d)
    k1 = _bf16(base).reshape(1, 1, N, d)
    k2 = _bf16(base + off).reshape(1, 1, N, d)
    rows = np.arange(N)
    for causal in (False, True):
        r1 = orc.ref64_rows_head(q, k1, v, 0, 0, rows, causal, 0.125)
        r2 = orc.ref64_rows_head(q, k2, v, 0, 0, rows, causal, 0.125)
        assert np.abs(r1 - r2).max() <= 1e-12
    o1, *_ = orc.attention(q, k1, v, False, 0.125)
    o2, *_ = orc.attention(q, k2, v, False, 0.125)
    assert _cos(o1, o2) > 0.9999


def test_fp64_reference_textbook(orc):
    """The FP64 reference equals torch's float64 softmax attention."""
    wl = si.make("tiny", N=150, H=1, seed=3)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    rows = np.arange(150)
    for causal in (False, True):
        mine = orc.ref64_rows_head(q, k, v, 0, 0, rows, causal, wl.sm_scale)
        Q, K, V = (t[0, 0].double() for t in (wl.q, wl.k, wl.v))
        mask = torch.ones(150, 150, dtype=torch.bool).tril() if causal else None
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[None], K[None], V[None], attn_mask=mask, scale=wl.sm_scale)[0].numpy()
        assert np.abs(mine - ref).max() < 1e-12


def test_smoothing_keeps_error_flat_under_key_offsets(orc):
    """With smoothing the error against FP64 stays flat as the per-channel key
    offset grows; with the mean left in (smooth=False) it does not."""
    rng = np.random.default_rng(12)
    B, H, N, d = 1, 2, 512, 64
    q = rng.standard_normal((B, H, N, d))
    kb = rng.standard_normal((B, H, N, d))
    v = _bf16(rng.standard_normal((B, H, N, d))).reshape(B, H, N, d)
    qc = _bf16(q).reshape(B, H, N, d)
    rows = np.arange(N)
    res = {}
    for sigma in (0.0, 3.0, 20.0):
        k = _bf16(kb + rng.standard_normal((B, H, 1, d)) * sigma).reshape(B, H, N, d)
        ref = np.stack([orc.ref64_rows_head(qc, k, v, 0, h, rows, False, 0.125) for h in range(H)])
        for smooth in (True, False):
            z = orc.quant_qk(qc, k, smooth=smooth)
            vq, vs = orc.quant_v(v)
            out = np.stack([orc.attn_rows_head(z, vq, vs, 0, h, rows, False, 0.125) for h in range(H)])
            res[(sigma, smooth)] = _cos(out, ref)
    for sigma in (0.0, 3.0, 20.0):
        assert res[(sigma, True)] >= 0.999, res
    assert res[(20.0, False)] < 0.995, res
    assert res[(20.0, False)] < res[(20.0, True)] - 0.005, res
    assert res[(20.0, False)] < res[(3.0, False)] < res[(0.0, False)] + 1e-5, res


def test_constant_keys_give_mean_of_v(orc):
    """All keys equal: smoothed K is exactly 0, every p is the same, and the
    output is the mean of the dequantized V column."""
    rng = np.random.default_rng(13)
    N, d = 300, 128
    row = rng.standard_normal(d)
    k = _bf16(np.tile(row, (N, 1))).reshape(1, 1, N, d)
    q = _bf16(rng.standard_normal((N, d)) * 5).reshape(1, 1, N, d)
    v = _bf16(rng.standard_normal((N, d))).reshape(1, 1, N, d)
    for pv in ("fp8", "fp16"):
        out, z, vq, vs = orc.attention(q, k, v, False, 0.088, pv, rows=[0, 150, 299])
        assert not z["k8"].any() and z["k_scale"].max() == 0.0
        dv = _deq_v(orc, vq, vs, pv)[0, 0]
        ref = dv.mean(axis=0)
        for r in range(3):
            assert np.allclose(out[0, 0, r], ref, rtol=1e-5, atol=1e-7)


def test_peaked_row_selects_one_value_row(orc):
    """A logit gap above log2(448) + 10 (log2 units) rounds every other P to 0
    in FP8, so the output is the dequantized V row of the peak key, up to the
    fp32 rounding of m - log2(448) (relative 2^-24 |m| ln 2)."""
    rng = np.random.default_rng(14)
    N, d = 400, 128
    kf = rng.standard_normal((N, d))
    qf = rng.standard_normal((N, d))
    qf[10] = 3 * kf[333]
    qf[200] = 3 * kf[17]
    q, k = _bf16(qf).reshape(1, 1, N, d), _bf16(kf).reshape(1, 1, N, d)
    v = _bf16(rng.standard_normal((N, d))).reshape(1, 1, N, d)
    out, z, vq, vs = orc.attention(q, k, v, False, 1 / math.sqrt(d), "fp8", rows=[10, 200])
    dv = _deq_v(orc, vq, vs, "fp8")[0, 0]
    s = z["q8"][0, 0].astype(np.int64) @ z["k8"][0, 0].astype(np.int64).T
    for r, (i, j) in enumerate([(10, 333), (200, 17)]):
        sig = np.float32(z["q_scale"][0, 0, i // 128] * np.float32(orc.lam(1 / math.sqrt(d))))
        c = (sig * np.repeat(z["k_scale"][0, 0], 128)[:N]).astype(np.float32)
        logits = s[i] * c.astype(np.float64)
        gap = logits[j] - np.delete(logits, j).max()
        assert gap > math.log2(448) + 10
        rtol = 2 * 2.0**-24 * abs(logits[j]) * math.log(2) + 1e-6
        assert np.allclose(out[0, 0, r], dv[j], rtol=rtol, atol=1e-7)


def test_first_causal_row_is_first_value_row(orc):
    wl = si.make("causal_prefill", N=256, B=1, H=1, seed=21)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    for pv in ("fp8", "fp16"):
        out, z, vq, vs = orc.attention(q, k, v, True, wl.sm_scale, pv, rows=[0])
        dv = _deq_v(orc, vq, vs, pv)[0, 0]
        assert np.allclose(out[0, 0, 0], dv[0], rtol=1e-6, atol=1e-7)


def test_outlier_recipe_accuracy_is_reported(orc):
    """The outlier workload at reduced N: the quantized method still tracks
    FP64 attention (the full-size figure is measured by the benchmark)."""
    wl = si.make("outlier", B=1, H=2, N=1500, seed=4)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    out, *_ = orc.attention(q, k, v, False, wl.sm_scale, "fp8")
    rows = np.arange(wl.N)
    ref = np.stack([orc.ref64_rows_head(q, k, v, 0, h, rows, False, wl.sm_scale) for h in range(2)])
    assert _cos(out[0], ref) > 0.995


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_per_token_q_is_closer_to_fp64_on_outlier_tokens(orc, pv):
    """Finer Q scales are the remedy the pages' "thread-level" quantization
    points at: on the outlier recipe (query tokens scaled x30 share a block
    with normal ones) per-token Q scales bring the output closer to FP64
    attention than per-block ones."""
    wl = si.make("outlier", B=1, H=2, N=1500, seed=4)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    rows = np.arange(wl.N)
    ref = np.stack([orc.ref64_rows_head(q, k, v, 0, h, rows, False, wl.sm_scale) for h in range(2)])
    cb = _cos(orc.attention(q, k, v, False, wl.sm_scale, pv)[0][0], ref)
    ct = _cos(orc.attention(q, k, v, False, wl.sm_scale, pv, q_gran="token")[0][0], ref)
    assert ct > cb + 1e-3, (cb, ct)


@pytest.mark.xfail(strict=True, reason=(
    "unmet bar, kept visible: on the outlier recipe at full length the quantized "
    "method itself stays near cosine 0.996-0.998 against FP64 attention (INT8 K "
    "resolution times the x30 query tokens); the GPU path matches this oracle's FP64 "
    "cosine to 2e-4 on the same rows"))
@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_outlier_full_length_meets_fp64_bar(orc, pv):
    """The FP64 bar (cosine >= 0.999 against plain attention) on the outlier
    workload at its full length N = 17550, one head, rows of the first and the
    last (ragged) query block and the head's outlier tokens."""
    wl = si.make("outlier", B=1, H=1)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    rows = sorted(set(range(0, 64)) | set(range(wl.N - 14, wl.N))
                  | set(wl.outlier_tokens[0, 0, :32].tolist()))
    rows = np.array(rows, np.int32)
    out, *_ = orc.attention(q, k, v, False, wl.sm_scale, pv, rows=rows)
    ref = orc.ref64_rows_head(q, k, v, 0, 0, rows, False, wl.sm_scale)
    c = _cos(out[0, 0], ref)
    print(f"outlier N={wl.N} pv={pv}: cosine vs FP64 {c:.6f} on {len(rows)} rows")
    assert c >= 0.999, c
