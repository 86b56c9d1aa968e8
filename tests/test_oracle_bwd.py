"""Pins of the oracle's 8-bit backward pass (sage_oracle_bwd.c).

Against things the oracle's own arithmetic does not produce: FP64 gradients of
plain softmax attention (or_bwd_ref64, itself pinned to torch float64
autograd here), the zero row sums of dS (D_i = sum_j P_ij dP_ij), probabilities
that sum to 1 through the forward's log-sum-exp, a one-hot output gradient
(dV = P^T dO returns a row of P in one column and exact zeros elsewhere),
exact doubling of every gradient when dO doubles (all scales are absmax
scales), and causal corner cases in closed form.
"""
import numpy as np
import pytest
import torch

import synthetic_inputs as si


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _inputs(name="tiny", **kw):
    wl = si.make(name, **kw)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    return wl, q, k, v, si.bf16_codes(si.output_grad(wl))


def test_ref64_matches_torch_autograd(orc):
    wl, q, k, v, dO = _inputs(N=96, H=1)
    for causal in (False, True):
        rq, rk, rv = orc.bwd_ref64_head(q, k, v, dO, 0, 0, causal, wl.sm_scale)
        t = [torch.from_numpy(orc.bf16_to_f32(x[0, 0]).astype(np.float64)).requires_grad_(i < 3)
             for i, x in enumerate((q, k, v, dO))]
        s = t[0] @ t[1].T * wl.sm_scale
        if causal:
            s = s.masked_fill(torch.triu(torch.ones_like(s, dtype=torch.bool), 1), float("-inf"))
        (torch.softmax(s, -1) @ t[2]).backward(t[3])
        for got, ref in ((rq, t[0].grad), (rk, t[1].grad), (rv, t[2].grad)):
            assert np.allclose(got, ref.numpy(), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("name,kw,causal", [("tiny", dict(N=300, H=1), False),
                                            ("tiny", dict(N=384, H=1), True),
                                            ("causal_prefill", dict(B=1, H=1, N=260), True)])
def test_gradients_against_fp64(orc, name, kw, causal):
    """The quantized gradients stay close to FP64 softmax-attention gradients
    (measured 0.998-0.999 in cosine on these inputs); a transposed operand, a
    dropped D term or a wrong scale lands far below."""
    wl, q, k, v, dO = _inputs(name, **kw)
    _, _, dq, dk, dv = orc.train_step_head(q, k, v, dO, 0, 0, causal, wl.sm_scale)
    rq, rk, rv = orc.bwd_ref64_head(q, k, v, dO, 0, 0, causal, wl.sm_scale)
    assert _cos(dq, rq) >= 0.997 and _cos(dk, rk) >= 0.997 and _cos(dv, rv) >= 0.998, \
        (_cos(dq, rq), _cos(dk, rk), _cos(dv, rv))
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.abs(got - ref).max() <= 0.08 * np.abs(ref).max()


def _forward(orc, q, k, v, causal, sm_scale):
    qz = orc.quant_qk(q, k)
    vq, vs = orc.quant_v(v, "fp8")
    N = q.shape[2]
    o, lse2 = orc.train_forward_head(qz, vq, vs, 0, 0, np.arange(N), causal, sm_scale)
    return qz, o, lse2


@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_and_ds_row_sums(orc, causal):
    """Over all key blocks, each row of P sums to 1 (the forward's lse2 is the
    log-sum-exp of the same scores).  With the output the backward's own P
    gives (O = bf16(P V)), each row of dS sums to 0: D_i = dO_i . O_i equals
    sum_j P_ij dP_ij, up to the bf16 rounding of O."""
    wl, q, k, v, dO = _inputs(N=300, H=1)
    N = 300
    qz, o, lse2 = _forward(orc, q, k, v, causal, wl.sm_scale)
    sizes = [min(128, N - 128 * b) for b in range(3)]

    def rows_of(o_codes, qb, which):
        parts = []
        for kb in range(3):
            t = orc.bwd_tile_head(qz, v[0, 0], o_codes, dO[0, 0], lse2, 0, 0, causal, wl.sm_scale, qb, kb)
            parts.append(t[which] if t else np.zeros((sizes[qb], sizes[kb]), np.float32))
        return np.concatenate(parts, axis=1).astype(np.float64)

    vf = orc.bf16_to_f32(v[0, 0]).astype(np.float64)
    o_cons = np.empty((N, 128), np.float64)
    for qb in range(3):
        P = rows_of(o, qb, 0)
        assert np.allclose(P.sum(1), 1.0, atol=2e-5), P.sum(1)
        if causal:
            rows = np.arange(128 * qb, 128 * qb + sizes[qb])
            assert not P[np.arange(N)[None, :] > rows[:, None]].any()
        o_cons[128 * qb:128 * qb + sizes[qb]] = P @ vf
    o_cons = orc.f32_to_bf16(o_cons.astype(np.float32))
    for qb in range(3):
        dS = rows_of(o_cons, qb, 1)
        assert np.all(np.abs(dS.sum(1)) <= 1e-2 * np.abs(dS).sum(1) + 1e-6), \
            np.max(np.abs(dS.sum(1)) / (np.abs(dS).sum(1) + 1e-12))


def test_one_hot_output_gradient(orc):
    """dO = 1 at (row i, channel c), 0 elsewhere: dV's column c is row i of P
    (to the FP8 rounding of P) and every other column of dV is exactly 0."""
    wl, q, k, v, _ = _inputs(N=200, H=1)
    i, c = 77, 5
    dO = np.zeros_like(q)
    dO[0, 0, i, c] = 0x3F80
    qz, o, lse2 = _forward(orc, q, k, v, False, wl.sm_scale)
    _, _, dv = orc.bwd_head(qz, v[0, 0], o, dO[0, 0], lse2, 0, 0, False, wl.sm_scale, qblocks=[])
    dv = np.concatenate([dv[b] for b in sorted(dv)])
    assert not np.delete(dv, c, axis=1).any()
    P = np.concatenate([orc.bwd_tile_head(qz, v[0, 0], o, dO[0, 0], lse2, 0, 0, False, wl.sm_scale,
                                          i // 128, kb)[0][i % 128] for kb in range(2)])
    assert np.allclose(dv[:, c], P, rtol=2.0**-4, atol=2.0**-10 / 448)
    # and P is the FP64 softmax row within the INT8 scores' resolution
    qf, kf = orc.bf16_to_f32(q[0, 0]).astype(np.float64), orc.bf16_to_f32(k[0, 0]).astype(np.float64)
    s = qf[i] @ kf.T * wl.sm_scale
    p64 = np.exp(s - s.max())
    p64 /= p64.sum()
    assert _cos(P, p64) >= 0.9999


@pytest.mark.parametrize("name,kw", [("tiny", dict(N=260, H=1)), ("outlier", dict(B=1, H=1, N=260))])
def test_doubling_dO_doubles_every_gradient_exactly(orc, name, kw):
    wl, q, k, v, dO = _inputs(name, **kw)
    g1 = orc.train_step_head(q, k, v, dO, 0, 0, False, wl.sm_scale)
    d2 = orc.f32_to_bf16(2.0 * orc.bf16_to_f32(dO))
    assert np.array_equal(orc.bf16_to_f32(d2), 2.0 * orc.bf16_to_f32(dO))
    g2 = orc.train_step_head(q, k, v, d2, 0, 0, False, wl.sm_scale)
    for a, b in zip(g1[2:], g2[2:]):
        assert np.array_equal(b, 2.0 * a)


def test_causal_corners(orc):
    """Causal: the first query sees only key 0, so its P is 1, its dS is
    dO_0 . (V_0 - O_0) (the forward's output error: O_0 is V_0 through FP8)
    and its dQ is that one score's gradient times key 0: exactly parallel to
    key 0's codes, with the sign of the FP64 closed form.  The last key is seen
    only by the last query, so dV_last = P_last,last dO_last."""
    wl, q, k, v, dO = _inputs(N=200, H=1)
    qz, o, lse2 = _forward(orc, q, k, v, True, wl.sm_scale)
    dq, dk, dv = orc.bwd_head(qz, v[0, 0], o, dO[0, 0], lse2, 0, 0, True, wl.sm_scale)
    dq0 = dq[0][0].astype(np.float64)
    k0 = qz["k8"][0, 0, 0].astype(np.float64)
    f16 = lambda x: orc.f16_to_f32(orc.f32_to_f16(orc.bf16_to_f32(x))).astype(np.float64)
    ds00 = f16(dO[0, 0, 0]) @ f16(v[0, 0, 0]) - orc.bf16_to_f32(dO[0, 0, 0]).astype(np.float64) @ \
        orc.bf16_to_f32(o[0]).astype(np.float64)
    assert abs(ds00) > 1e-3
    c = _cos(dq0, k0)
    assert abs(abs(c) - 1.0) <= 1e-6 and np.sign(c) == np.sign(ds00), (c, ds00)
    dv = np.concatenate([dv[b] for b in sorted(dv)])
    do_last = orc.bf16_to_f32(dO[0, 0, -1]).astype(np.float64)
    qf, kf = orc.bf16_to_f32(q[0, 0]).astype(np.float64), orc.bf16_to_f32(k[0, 0]).astype(np.float64)
    s = qf[-1] @ kf.T * wl.sm_scale
    p = np.exp(s - s.max())
    p_last = p[-1] / p.sum()
    assert _cos(dv[-1], p_last * do_last) >= 0.999
    rq, rk, rv = orc.bwd_ref64_head(q, k, v, dO, 0, 0, True, wl.sm_scale)
    assert np.allclose(rv[-1], p_last * do_last)
