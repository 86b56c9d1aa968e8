"""Pins of the oracle's microscaled (MX) attention: MXFP6 (E2M3 elements) and
MXFP4 (E2M1) with E8M0 block scales of 32.

The codecs are pinned by invariants a wrong table or rounding rule breaks
(round trips, monotone code order, the formats' extreme values and steps,
ties between neighbours, saturation, sign symmetry); the block rule by its
bounds and the exponent from numpy's frexp; the MX dot product by exact
rational arithmetic; the attention by a single tile against FP64 attention
over the dequantized operands, a tile-by-tile non-online recomputation, the
largest probability of each row dequantizing to exactly 1 (the running
maximum rounded down), and its FP64 cosine.
"""
from fractions import Fraction

import numpy as np
import pytest

import synthetic_inputs as si

FMTS = {"mxfp4": (8, 6.0), "mxfp6": (32, 7.5)}     # positive codes, largest magnitude


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


@pytest.mark.parametrize("fmt", list(FMTS))
def test_codec_invariants(orc, fmt):
    n, top = FMTS[fmt]
    codes = np.arange(2 * n, dtype=np.uint8)
    vals = orc.mx_to_f32(codes, fmt).astype(np.float64)
    pos = vals[:n]
    assert pos[0] == 0.0 and pos[-1] == top and np.all(np.diff(pos) > 0)   # monotone, extremes
    assert np.array_equal(vals[n:], -pos)                                   # sign bit
    assert np.array_equal(orc.f32_to_mx(pos.astype(np.float32), fmt), codes[:n])   # round trip
    if fmt == "mxfp4":
        assert list(pos) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    else:
        # E2M3: 1/8 steps up to 2, then 1/4 up to 4, then 1/2 up to 7.5
        assert np.allclose(np.diff(pos[:16]), 0.125) and np.allclose(np.diff(pos[16:24]), 0.25)
        assert np.allclose(np.diff(pos[24:]), 0.5) and pos[16] == 2.0 and pos[24] == 4.0
    # ties between neighbours go to the even code; just off a tie, to the nearer
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    got = orc.f32_to_mx(mid, fmt).astype(int)
    lo = np.arange(n - 1)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    eps = np.float32(1e-3)
    assert np.array_equal(orc.f32_to_mx(mid - eps * mid, fmt).astype(int), lo)
    assert np.array_equal(orc.f32_to_mx(mid + eps * mid, fmt).astype(int), lo + 1)
    # saturation and signed zero
    assert np.all(orc.f32_to_mx(np.float32([top * 1.01, 1e30, np.inf]), fmt) == n - 1)
    assert np.all(orc.f32_to_mx(np.float32([-top * 1.01, -1e30]), fmt) == 2 * n - 1)
    assert orc.f32_to_mx(np.float32([-1e-6]), fmt)[0] == n                  # -0
    assert orc.f32_to_mx(np.float32([np.nan]), fmt)[0] == 0


@pytest.mark.parametrize("fmt", list(FMTS))
def test_block_rule(orc, fmt):
    n, top = FMTS[fmt]
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((400, 32)) * np.exp2(rng.integers(-20, 20, (400, 1)))).astype(np.float32)
    x[7] = 0.0
    x[8] = 1e-31                                   # below 2^-100: stored as zeros
    x[9, :] = 0.0
    x[9, 5] = -3.0                                 # a lone negative maximum
    codes, eb = orc.mx_blocks(x, fmt)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    big = amax >= 2.0**-100
    k = np.frexp(amax[big])[1]                     # amax = f 2^k, f in [0.5, 1)
    assert np.array_equal(eb[big].astype(int) - 127, k - 1 - 2)
    assert np.all(eb[~big] == 0) and not codes[~big].any()
    dec = orc.mx_dequant(codes, eb[:, None], fmt)
    scale = np.exp2(eb.astype(np.float64) - 127)[:, None]
    # the absmax element: its scaled value is in [4, 8): code >= 4 and saturation only above top
    i = np.argmax(np.abs(x), axis=1)
    am = np.abs(dec[np.arange(400), i]) / scale[:, 0]
    assert np.all(am[big] >= 4.0) and np.all(am[big] <= top)
    # error: half a step of the element's binade (steps 2^(e-3) / 2^(e-1) scaled), or saturation
    step = 0.125 if fmt == "mxfp6" else 0.5
    scaled = np.abs(x.astype(np.float64)) / scale
    binade_step = step * np.maximum(1.0, np.exp2(np.floor(np.log2(np.maximum(scaled, 1e-300)))))
    err = np.abs(dec - x) / scale
    sat = scaled > top
    assert np.all(err[big][~sat[big]] <= binade_step[big][~sat[big]] / 2 * (1 + 1e-9))
    assert np.all(np.sign(dec[big]) * np.sign(x[big]) >= 0)


@pytest.mark.parametrize("fmt", list(FMTS))
def test_mx_dot_is_exact(orc, fmt):
    n, _ = FMTS[fmt]
    rng = np.random.default_rng(5)
    for trial in range(30):
        d = 128 if trial % 2 else 64
        qc = rng.integers(0, 2 * n, d, dtype=np.uint8)
        kc = rng.integers(0, 2 * n, d, dtype=np.uint8)
        qe = rng.integers(100, 150, d // 32, dtype=np.uint8)
        ke = rng.integers(100, 150, d // 32, dtype=np.uint8)
        qv = orc.mx_to_f32(qc, fmt)
        kv = orc.mx_to_f32(kc, fmt)
        exact = sum(Fraction(float(qv[c])) * Fraction(float(kv[c])) *
                    Fraction(2) ** (int(qe[c // 32]) + int(ke[c // 32]) - 254) for c in range(d))
        got = orc.lib().or_mx_dot(orc.MX_FMT[fmt], orc._p(qc), orc._p(qe), orc._p(kc), orc._p(ke), d)
        assert got == np.float32(float(exact)), trial


def _deq_head(orc, mz, vc, ve, fmt, h=0):
    N, d = mz["q_c"].shape[2:]
    rep = lambda e: np.repeat(e, 32, axis=-1)
    dq = orc.mx_dequant(mz["q_c"][0, h], rep(mz["q_e"][0, h]), fmt)
    dk = orc.mx_dequant(mz["k_c"][0, h], rep(mz["k_e"][0, h]), fmt)
    dv = orc.mx_dequant(vc[0, h], np.repeat(ve[0, h], 32, axis=0)[:N], fmt)
    return dq, dk, dv


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("N", [1, 40, 128])
def test_single_tile_against_fp64_over_dequantized(orc, fmt, N):
    """One key tile: the online softmax is one-shot; against FP64 attention over
    the dequantized Q, K, V the gap left is P's block rounding (half a step of
    the element format: 2^-4 relative for E2M3, 2^-2 for E2M1)."""
    wl = si.make("tiny", N=N, H=1, seed=31 + N)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    out, mz, vc, ve = orc.mx_attention(q, k, v, False, wl.sm_scale, fmt=fmt)
    dq, dk, dv = _deq_head(orc, mz, vc, ve, fmt)
    s = dq @ dk.T * wl.sm_scale
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ dv
    rel = 2.0**-4 if fmt == "mxfp6" else 2.0**-2
    assert np.abs(out[0, 0] - ref).max() <= rel * 1.05 * np.abs(dv).max() + 1e-5


def _non_online(orc, mz, vc, ve, i, causal, sm_scale, fmt):
    """Row i tile by tile: each tile against its running max (S lambda rounded
    toward -infinity), P blocks of 32
    quantized by the oracle's block rule, tiles combined at the end with
    weights 2^(M_t - M)."""
    N, d = mz["q_c"].shape[2:]
    dq, dk, dv = _deq_head(orc, mz, vc, ve, fmt)
    lam = np.float32(orc.lam(sm_scale))
    n_keys = i + 1 if causal else N
    S = np.array([orc.lib().or_mx_dot(orc.MX_FMT[fmt], orc._p(np.ascontiguousarray(mz["q_c"][0, 0, i])),
                                      orc._p(np.ascontiguousarray(mz["q_e"][0, 0, i])),
                                      orc._p(np.ascontiguousarray(mz["k_c"][0, 0, j])),
                                      orc._p(np.ascontiguousarray(mz["k_e"][0, 0, j])), d)
                  for j in range(n_keys)], np.float32)
    Ms, Ls, Ts = [], [], []
    M = np.float32(-np.inf)
    for t0 in range(0, n_keys, 128):
        St = S[t0:t0 + 128]
        exact = St.astype(np.float64) * np.float64(lam)           # exact products
        rd = exact.astype(np.float32)
        rd = np.where(rd > exact, np.nextafter(rd, np.float32(-np.inf)), rd)  # toward -inf
        M = max(M, rd.max())
        arg = (St.astype(np.float64) * np.float64(lam) - np.float64(M)).astype(np.float32)
        p = np.exp2(arg.astype(np.float64)).astype(np.float32)
        pq = np.zeros(len(p))
        for b0 in range(0, len(p), 32):
            blk = np.zeros(32, np.float32)
            blk[:len(p[b0:b0 + 32])] = p[b0:b0 + 32]
            c, e = orc.mx_blocks(blk, fmt)
            pq[b0:b0 + 32] = orc.mx_dequant(c[0], e[0], fmt)[:len(p[b0:b0 + 32])]
        Ms.append(M)
        Ls.append(p.astype(np.float64).sum())
        Ts.append(pq @ dv[t0:t0 + len(St)])
    w = np.exp2(np.array(Ms, np.float64) - np.float64(M))
    return sum(wt * Tt for wt, Tt in zip(w, Ts)) / (w @ np.array(Ls)), M


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("causal", [False, True])
def test_online_bookkeeping_matches_non_online(orc, fmt, causal):
    wl = si.make("tiny", N=600, H=1, seed=91)                # 5 tiles, the last ragged
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    mz = orc.mx_quant_qk(q, k, fmt)
    vc, ve = orc.mx_quant_v(v, fmt)
    rows = np.array([0, 3, 127, 128, 300, 599])
    out, m, l = orc.mx_attn_rows_head(mz, vc, ve, 0, 0, rows, causal, wl.sm_scale, return_ml=True)
    for r, i in enumerate(rows):
        ref, M = _non_online(orc, mz, vc, ve, i, causal, wl.sm_scale, fmt)
        assert m[r] == M
        # the exp2 of the oracle (libm) and numpy's may differ by an ulp: P codes
        # may flip at a block-rounding boundary, so the bound is loose but far
        # below a wrong tile, scale or block
        assert np.abs(out[r] - ref).max() <= 2e-3 * np.abs(ref).max() + 1e-5, (i, np.abs(out[r] - ref).max())


@pytest.mark.parametrize("fmt", list(FMTS))
def test_largest_probability_is_exactly_one(orc, fmt):
    """With the running maximum rounded down, the row's largest p is in
    [1, 1 + 2^-23): its P block takes scale 2^-2 and it dequantizes to exactly
    1.  One key tile (N = 128) and V = the identity, so out[i, j] l = P~_ij.
    Rounded to nearest, the maximum leaves p = 1 - 2^-24 on part of the rows,
    whose block then saturates the element to 0.9375."""
    N = d = 128
    wl = si.make("tiny", N=N, H=1, seed=5)
    q, k = si.bf16_codes(wl.q), si.bf16_codes(wl.k)
    v = np.zeros((1, 1, N, d), np.uint16)
    v[0, 0, np.arange(N), np.arange(N)] = 0x3F80                 # bf16 1.0
    mz = orc.mx_quant_qk(q, k, fmt)
    vc, ve = orc.mx_quant_v(v, fmt)
    assert np.all(orc.mx_dequant(vc[0, 0], np.repeat(ve[0, 0], 32, axis=0), fmt) == np.eye(N))
    rows = np.arange(N)
    out, m, l = orc.mx_attn_rows_head(mz, vc, ve, 0, 0, rows, False, wl.sm_scale, return_ml=True)
    pq = out.astype(np.float64) * l[:, None]
    top = pq.max(axis=1)
    assert np.all(np.abs(top - 1.0) <= 2.0**-22), top[np.abs(top - 1.0) > 2.0**-22]
    # the rounded-down maximum: m <= max S lambda < m + one ulp of m
    S = (orc.mx_dequant(mz["q_c"][0, 0], np.repeat(mz["q_e"][0, 0], 32, axis=1), fmt) @
         orc.mx_dequant(mz["k_c"][0, 0], np.repeat(mz["k_e"][0, 0], 32, axis=1), fmt).T)
    exact = S.astype(np.float32).astype(np.float64).max(axis=1) * np.float64(orc.lam(wl.sm_scale))
    assert np.all(m.astype(np.float64) <= exact)
    assert np.all(np.nextafter(m, np.float32(np.inf)).astype(np.float64) > exact)


def test_fp64_cosine_orders_the_formats(orc):
    """MXFP6 stays close to the INT8/FP8 path against FP64 attention; MXFP4
    (E2M1, one mantissa bit) falls far below it -- the accuracy the pages
    report for MXFP4 lies in between because their inputs differ."""
    wl = si.make("tiny", H=2)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    o6, *_ = orc.mx_attention(q, k, v, False, wl.sm_scale, fmt="mxfp6")
    o4, *_ = orc.mx_attention(q, k, v, False, wl.sm_scale, fmt="mxfp4")
    o8, *_ = orc.attention(q, k, v, False, wl.sm_scale)
    for h in range(2):
        ref = orc.ref64_rows_head(q, k, v, 0, h, np.arange(wl.N), False, wl.sm_scale)
        c6, c4, c8 = _cos(o6[0, h], ref), _cos(o4[0, h], ref), _cos(o8[0, h], ref)
        assert c6 >= 0.997 and c4 < c6 - 0.01 and c8 > c6, (c6, c4, c8)
