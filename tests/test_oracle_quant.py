"""Pins of the oracle's smoothing and quantization steps.

The pages give no worked numbers for these steps, so they are pinned by exact
integer arithmetic (Python ints / fractions), library reductions (numpy), and
invariants that a dropped term, a wrong scale or a sign error would break.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthetic_inputs as si


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _exact_fix30(x: float) -> int:
    """trunc(x * 2^30) in exact rational arithmetic, saturated at 2^62."""
    if x != x:
        return 0
    if x in (float("inf"), float("-inf")):
        return (1 << 62) if x > 0 else -(1 << 62)
    t = Fraction(x) * (1 << 30)
    v = int(t)  # int() of a Fraction truncates toward zero
    return max(-(1 << 62), min(1 << 62, v))


def test_fix30_exact(orc):
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.standard_normal(2000) * 5, rng.standard_normal(500) * 1e-8, rng.standard_normal(200) * 1e12,
        [0.0, -0.0, 2.0**-30, -2.0**-30, 3 * 2.0**-31, -(3 * 2.0**-31), 2.0**32, -(2.0**33)]])
    codes = _bf16(vals)
    x = orc.bf16_to_f32(codes)
    mine = orc.fix30(x)
    ref = np.array([_exact_fix30(float(v)) for v in x], dtype=np.int64)
    assert np.array_equal(mine, ref)


def test_k_mean_exact_integer_definition(orc):
    """mu_c = fp32(fp64(I_c) / (N 2^30)) with I_c the exact wrapped sum."""
    rng = np.random.default_rng(4)
    N, d = 37, 8
    k = rng.standard_normal((N, d)) * 3 + rng.standard_normal(d) * 5
    k[5, 2] = 1e-12   # below the grid: truncated to 0
    k[7, 3] = -7e-10  # truncated toward zero
    codes = _bf16(k)
    x = orc.bf16_to_f32(codes).reshape(N, d)
    mine = orc.k_mean_head(codes.reshape(N, d))
    for c in range(d):
        s = sum(_exact_fix30(float(v)) for v in x[:, c])
        s = (s + (1 << 63)) % (1 << 64) - (1 << 63)
        ref = np.float32(float(s) / (N * 2.0**30))
        assert mine[c] == ref, c


def test_k_mean_close_to_numpy_mean(orc):
    rng = np.random.default_rng(5)
    N, d = 5000, 64
    k = rng.standard_normal((N, d)) + rng.standard_normal(d) * 3
    codes = _bf16(k).reshape(N, d)
    x = orc.bf16_to_f32(codes).reshape(N, d).astype(np.float64)
    mine = orc.k_mean_head(codes).astype(np.float64)
    ref = x.mean(axis=0)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(mine - ref) <= ulp + 2.0**-30)


def test_k_mean_constant_column(orc):
    N, d = 301, 4
    col = np.array([1.5, -0.375, 96.0, 0.0], np.float32)
    codes = _bf16(np.tile(col, (N, 1)))
    assert np.array_equal(orc.k_mean_head(codes), col)


def test_quant_block_invariants(orc):
    rng = np.random.default_rng(6)
    for trial in range(20):
        x = (rng.standard_normal((128, 64)) * rng.uniform(0.01, 100)).astype(np.float32)
        if trial == 3:
            x[:, :] = np.abs(x)  # one-signed
        q, s = orc.quant_block(x)
        a = np.abs(x).max()
        assert abs(s - a / 127.0) <= np.spacing(np.float32(a / 127.0))
        assert np.abs(q.astype(np.int32)).max() == 127
        i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert q[i] == (127 if x[i] > 0 else -127)
        assert np.all(np.abs(q.astype(np.float64) * s - x) <= s * (0.5 + 1e-5))
        nz = q != 0
        assert np.all(np.sign(q[nz]) == np.sign(x[nz]))
        order = np.argsort(x.ravel(), kind="stable")  # monotone
        assert np.all(np.diff(q.ravel()[order].astype(np.int32)) >= 0)
    q, s = orc.quant_block(np.zeros((5, 64), np.float32))
    assert s == 0.0 and not q.any()


def test_quant_block_rounding_rule_hand_codes(orc):
    """The INT8 rounding rule itself: code = rne(fp32(x * fp32(127 / a))).

    Expected codes are written out by hand, on blocks whose scaled values land
    exactly on k + 1/2 (for even and odd k, both signs), where round half to
    even, round half away from zero and truncation all differ; and on a block
    where x * fp32(127 / a) and x / fp32(a / 127) fall on opposite sides of a
    half step, so dividing by the scale instead of multiplying by the inverse
    gives another code."""
    # absmax 127: inv = fp32(127 / 127) = 1 exactly, the values are their own
    # scaled values
    x = np.array([[0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 126.5, -126.5, 62.5, -63.5, 127.0]],
                 np.float32)
    q, s = orc.quant_block(x)
    assert s == np.float32(1.0)
    assert q.tolist() == [[0, 2, 2, 4, 0, -2, -2, -4, 126, -126, 62, -64, 127]]
    # absmax 254: inv = 0.5 exactly; 5 -> 2.5 -> 2, 7 -> 3.5 -> 4, -9 -> -4.5 -> -4
    x = np.array([[5.0, 7.0, -9.0, 1.0, 254.0]], np.float32)
    q, s = orc.quant_block(x)
    assert s == np.float32(2.0)
    assert q.tolist() == [[2, 4, -4, 0, 127]]
    # absmax 63.5, one row (the per-token case): inv = 2 exactly
    x = np.array([[1.25, 0.75, -0.25, -1.75, 63.5]], np.float32)
    q, s = orc.quant_block(x)
    assert q.tolist() == [[2, 2, 0, -4, 127]]
    # absmax 5.9375: fp32(127 / 5.9375) is below 127 / 5.9375, so -2.96875 (exactly
    # half of the absmax, -63.5 in real arithmetic) scales to -63.499996 -> -63,
    # while -2.96875 / fp32(5.9375 / 127) gives -63.5 -> -64.
    x = np.array([[5.9375, -2.96875]], np.float32)
    inv = np.float32(127.0 / 5.9375)
    assert np.float32(x[0, 1] * inv) > np.float32(-63.5)
    assert np.float32(x[0, 1] / np.float32(5.9375 / 127.0)) == np.float32(-63.5)
    q, s = orc.quant_block(x)
    assert q.tolist() == [[127, -63]]
    # absmax 4.5: the other way round, the product lands on -63.5 exactly -> -64
    x = np.array([[4.5, -2.25]], np.float32)
    assert np.float32(x[0, 1] * np.float32(127.0 / 4.5)) == np.float32(-63.5)
    q, s = orc.quant_block(x)
    assert q.tolist() == [[127, -64]]


def test_quant_block_matches_numpy_rule(orc):
    """Every code of random blocks (Gaussian and bf16-grid values, one-row and
    many-row) equals numpy's rint(fp32(x) * fp32(127 / fp64(a))), clamped."""
    rng = np.random.default_rng(12)
    for trial in range(40):
        rows = 1 if trial % 2 else 128
        x = (rng.standard_normal((rows, 64)) * rng.uniform(0.01, 50)).astype(np.float32)
        if trial % 4 == 1:  # coarse grid: many exact half steps
            x = (np.round(x * 4) / 4).astype(np.float32)
        q, _ = orc.quant_block(x)
        a = np.float64(np.abs(x).max())
        inv = np.float32(127.0 / a)
        ref = np.clip(np.rint(x * inv), -127, 127).astype(np.int8)
        assert np.array_equal(q, ref), trial


def test_quant_qk_blocks_and_tail(orc):
    wl = si.make("tiny", N=300, H=1)  # blocks of 128, 128, 44 rows
    q, k = si.bf16_codes(wl.q), si.bf16_codes(wl.k)
    z = orc.quant_qk(q, k)
    qf = orc.bf16_to_f32(q).reshape(q.shape)
    kf = orc.bf16_to_f32(k).reshape(k.shape)
    mu = z["k_mean"][0, 0]
    assert np.array_equal(mu, orc.k_mean_head(k[0, 0]))
    ks = (kf[0, 0] - mu).astype(np.float32)
    for r, (r0, r1) in enumerate([(0, 128), (128, 256), (256, 300)]):
        aq = np.abs(qf[0, 0, r0:r1]).max()
        ak = np.abs(ks[r0:r1]).max()
        assert z["q_scale"][0, 0, r] == np.float32(np.float64(aq) / 127)
        assert z["k_scale"][0, 0, r] == np.float32(np.float64(ak) / 127)
    # smoothing removes the per-channel offset: smoothed K has ~zero channel mean
    assert np.abs(ks.mean(axis=0)).max() < 1e-4
    dq = z["k8"][0, 0].astype(np.float64) * np.repeat(z["k_scale"][0, 0], 128)[:300, None]
    assert np.abs(dq - ks).max() <= z["k_scale"].max() * 0.5001


def test_per_token_q_scales(orc):
    """Per-token Q ("thread-level" granularity): one scale per query row.  Every
    nonzero row reaches +-127, its scale is its own absmax / 127, codes stay
    within half a step, K is unchanged, and the row that holds a block's absmax
    gets exactly the codes the per-block quantization gives it."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 1, 300, 128)).astype(np.float32)
    x[0, 0, 7] *= 30.0        # an outlier token, like the outlier workload's
    x[0, 0, 200] = 0.0        # an all-zero row
    q = _bf16(x).reshape(x.shape)
    k = _bf16(rng.standard_normal(x.shape).astype(np.float32) + 2.0).reshape(x.shape)
    zt = orc.quant_qk(q, k, q_gran="token")
    zb = orc.quant_qk(q, k)
    assert zt["q_scale"].shape == (1, 1, 300) and zt["qblk"] == 1 and zb["qblk"] == 128
    assert np.array_equal(zt["k8"], zb["k8"]) and np.array_equal(zt["k_scale"], zb["k_scale"])
    qf = orc.bf16_to_f32(q).reshape(x.shape)[0, 0].astype(np.float64)
    a = np.abs(qf).max(axis=1)
    assert np.array_equal(zt["q_scale"][0, 0], (a / 127).astype(np.float32))
    c = zt["q8"][0, 0].astype(np.int64)
    top = np.abs(c).max(axis=1)
    assert np.all((top == 127) | (a == 0)) and not c[200].any()
    deq = c * zt["q_scale"][0, 0][:, None].astype(np.float64)
    assert np.all(np.abs(deq - qf) <= zt["q_scale"][0, 0][:, None] * 0.5001 + 1e-30)
    for r0 in (0, 128, 256):
        blk = qf[r0:r0 + 128]
        i = r0 + int(np.argmax(np.abs(blk).max(axis=1)))
        assert np.array_equal(zt["q8"][0, 0, i], zb["q8"][0, 0, i])
    # finer scales never lose resolution: per-token error <= per-block error, row by row
    eb = np.abs(zb["q8"][0, 0] * np.repeat(zb["q_scale"][0, 0], 128)[:300, None] - qf).max(axis=1)
    et = np.abs(deq - qf).max(axis=1)
    assert np.all(et <= eb * 1.0001 + 1e-12)


def test_quant_v_fp8_and_fp16(orc):
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((1, 2, 333, 64)) * rng.uniform(0.1, 10, (1, 2, 1, 64))).astype(np.float32)
    v[0, 1, :, 5] = 0.0  # an all-zero channel
    codes = _bf16(v).reshape(v.shape)
    vf = orc.bf16_to_f32(codes).reshape(v.shape)
    vq, vs = orc.quant_v(codes, "fp8")
    a = np.abs(vf).max(axis=2)
    assert np.array_equal(vs, (a.astype(np.float64) / 448).astype(np.float32))
    deq = orc.e4m3_to_f32(vq).reshape(v.shape) * vs[:, :, None, :]
    # e4m3 relative step is 2^-3: rounding error <= 2^-4 relative, or half the
    # subnormal step (2^-10 of the scale) near zero
    bound = np.maximum(np.abs(vf) * 2.0**-4, vs[:, :, None, :] * 2.0**-10) * 1.0001 + 1e-30
    assert np.all(np.abs(deq - vf) <= bound)
    # each channel's absmax element lands on the top code (+-448)
    top = np.abs(orc.e4m3_to_f32(vq)).reshape(v.shape).max(axis=2)
    assert np.all((top == 448.0) | (a == 0))
    assert not vq[0, 1, :, 5].any()
    vq16, vs16 = orc.quant_v(codes, "fp16")
    assert np.all(vs16 == 1.0)
    assert np.array_equal(orc.f16_to_f32(vq16).reshape(v.shape), vf)  # bf16 values are exact in fp16


def test_dump_s_matches_int64_matmul(orc):
    rng = np.random.default_rng(8)
    q8 = rng.integers(-127, 128, (70, 128), dtype=np.int8)
    k8 = rng.integers(-127, 128, (150, 128), dtype=np.int8)
    s = orc.dump_s(q8, k8, 10, 50)
    ref = q8[10:60].astype(np.int64) @ k8.astype(np.int64).T
    assert np.array_equal(s.astype(np.int64), ref)
    sc = orc.dump_s(q8, k8, 10, 50, causal=True)
    mask = np.arange(150)[None, :] <= np.arange(10, 60)[:, None]
    assert np.array_equal(sc[mask], s[mask]) and not sc[~mask].any()
    ext = np.full((1, 128), 127, np.int8), np.full((1, 128), -127, np.int8)
    assert orc.dump_s(ext[0], ext[1], 0, 1)[0, 0] == -127 * 127 * 128
