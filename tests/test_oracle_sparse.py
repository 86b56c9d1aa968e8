"""Pins of the oracle's block-sparse tile skipping.

A key tile that a query block does not visit contributes nothing: the row's
online softmax runs over the visited tiles only.  Pinned by (1) an all-ones
mask reproducing the dense result bit for bit, (2) each row equal bit for bit
to the dense algorithm run on the compacted operands (only the visited tiles'
quantized keys, scales and values, in order), (3) FP64 softmax attention over
the visited keys computed independently in numpy, (4) rows that visit no key
giving 0, (5) causal masking composing with the tile mask.
"""
import numpy as np
import pytest

import synthetic_inputs as si


def _cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _setup(orc, N, H=1, pv="fp8", seed=5, name="tiny"):
    wl = si.make(name, N=N, H=H, seed=seed)
    q, k, v = (si.bf16_codes(t) for t in (wl.q, wl.k, wl.v))
    z = orc.quant_qk(q, k)
    vq, vs = orc.quant_v(v, pv)
    return wl, q, k, v, z, vq, vs


def _random_mask(B, H, N, keep, seed):
    nb = -(-N // 128)
    rng = np.random.default_rng(seed)
    return (rng.random((B, H, nb, nb)) < keep).astype(np.uint8)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_all_ones_mask_is_dense(orc, pv):
    wl, q, k, v, z, vq, vs = _setup(orc, 700, H=2, pv=pv)
    rows = np.arange(wl.N)
    ones = np.ones((1, 2, 6, 6), np.uint8)
    for causal in (False, True):
        for h in range(2):
            a = orc.attn_rows_head(z, vq, vs, 0, h, rows, causal, wl.sm_scale, pv)
            b = orc.attn_rows_head(z, vq, vs, 0, h, rows, causal, wl.sm_scale, pv, tile_mask=ones)
            assert np.array_equal(a, b)


@pytest.mark.parametrize("pv", ["fp8", "fp16"])
def test_rows_equal_dense_on_compacted_operands(orc, pv):
    wl, q, k, v, z, vq, vs = _setup(orc, 1000, pv=pv, seed=9)  # 8 tiles, the last 104 keys
    mask = _random_mask(1, 1, wl.N, 0.5, seed=3)
    mask[0, 0, 2, :] = 0
    mask[0, 0, 2, 7] = 1          # a block that sees only the ragged last tile
    rows = np.arange(wl.N)
    out = orc.attn_rows_head(z, vq, vs, 0, 0, rows, False, wl.sm_scale, pv, tile_mask=mask)
    for r in range(mask.shape[2]):
        tiles = np.flatnonzero(mask[0, 0, r])
        rr = rows[r * 128:(r + 1) * 128]
        if len(tiles) == 0:
            assert not out[rr].any()
            continue
        keys = np.concatenate([np.arange(t * 128, min(wl.N, t * 128 + 128)) for t in tiles])
        zc = dict(q8=z["q8"], q_scale=z["q_scale"], k8=z["k8"][:, :, keys],
                  k_scale=z["k_scale"][:, :, tiles], k_mean=z["k_mean"], qblk=z["qblk"])
        vqc = np.ascontiguousarray(vq[:, :, keys])
        n = len(keys)
        qsel = rr[rr < wl.N]
        ref = _dense_compacted(orc, zc, vqc, vs, qsel, n, wl.sm_scale, pv)
        assert np.array_equal(out[qsel], ref), r


def _dense_compacted(orc, zc, vqc, vs, qrows, n, sm_scale, pv):
    """Dense oracle over the n compacted keys for query rows qrows: a head of
    exactly n tokens whose key side is the compacted keys and whose first query
    rows are the selected ones (each with its own block's scale); more rows
    than keys are handled in chunks of at most n rows."""
    d = zc["q8"].shape[-1]
    ntile = -(-n // 128)
    k8 = np.ascontiguousarray(zc["k8"][:, :, :n])
    ks = np.ascontiguousarray(zc["k_scale"][:, :, :ntile])
    vq = np.ascontiguousarray(vqc[:, :, :n])
    outs = []
    for c0 in range(0, len(qrows), n):
        sel = qrows[c0:c0 + n]
        m = len(sel)
        q8 = np.zeros((1, 1, n, d), np.int8)
        q8[0, 0, :m] = zc["q8"][0, 0, sel]
        qs = np.zeros((1, 1, n), np.float32)
        qs[0, 0, :m] = zc["q_scale"][0, 0, sel // zc["qblk"]]
        zz = dict(q8=q8, q_scale=qs, k8=k8, k_scale=ks, k_mean=zc["k_mean"], qblk=1)
        outs.append(orc.attn_rows_head(zz, vq, vs, 0, 0, np.arange(m), False, sm_scale, pv))
    return np.concatenate(outs)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_fp64_over_visited_keys(orc, causal):
    wl, q, k, v, z, vq, vs = _setup(orc, 900, H=2, seed=13)
    mask = _random_mask(1, 2, wl.N, 0.6, seed=21)
    for h in range(2):
        mask[0, h, :, 0] = 1      # every block sees tile 0, so every causal row sees a key
    rows = np.arange(wl.N)
    qf = orc.bf16_to_f32(q).reshape(q.shape).astype(np.float64)
    kf = orc.bf16_to_f32(k).reshape(k.shape).astype(np.float64)
    vf = orc.bf16_to_f32(v).reshape(v.shape).astype(np.float64)
    for h in range(2):
        out = orc.attn_rows_head(z, vq, vs, 0, h, rows, causal, wl.sm_scale, "fp8", tile_mask=mask)
        s = qf[0, h] @ kf[0, h].T * wl.sm_scale
        vis = np.repeat(np.repeat(mask[0, h].astype(bool), 128, 0), 128, 1)[:wl.N, :wl.N]
        if causal:
            vis &= np.tril(np.ones((wl.N, wl.N), bool))
        s = np.where(vis, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (p / p.sum(axis=1, keepdims=True)) @ vf[0, h]
        assert _cos(out, ref) >= 0.999, (h, _cos(out, ref))


def test_rows_that_visit_nothing_are_zero(orc):
    wl, q, k, v, z, vq, vs = _setup(orc, 400, seed=17)
    mask = np.ones((1, 1, 4, 4), np.uint8)
    mask[0, 0, 1] = 0
    rows = np.arange(wl.N)
    out, m, l = orc.attn_rows_head(z, vq, vs, 0, 0, rows, False, wl.sm_scale, "fp8",
                                   return_ml=True, tile_mask=mask)
    assert not out[128:256].any() and np.all(l[128:256] == 0) and np.all(np.isinf(m[128:256]))
    assert np.all(l[:128] > 0) and np.all(l[256:] > 0)
    # causal: block 1 skips tile 1 (its diagonal tile) -> its rows still see tile 0
    mask = np.ones((1, 1, 4, 4), np.uint8)
    mask[0, 0, 1, 1] = 0
    out = orc.attn_rows_head(z, vq, vs, 0, 0, rows, True, wl.sm_scale, "fp8", tile_mask=mask)
    dense = orc.attn_rows_head(z, vq, vs, 0, 0, rows, True, wl.sm_scale, "fp8")
    assert np.array_equal(out[:128], dense[:128]) and np.array_equal(out[256:], dense[256:])
    assert not np.array_equal(out[128:256], dense[128:256]) and np.isfinite(out).all()
