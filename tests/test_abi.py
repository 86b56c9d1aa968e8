"""The C ABI without a GPU: the library loads, exports every function that
include/sage.h declares, reports its constants, and rejects invalid arguments
with the documented status codes before anything is launched."""
import ctypes as ct
import math
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")


@pytest.fixture(scope="module")
def sage():
    import quantized_attention_video_02_amd as s
    from quantized_attention_video_02_amd import build as b

    if not os.path.exists(b.LIB_PATH):
        b.build()
    s.lib()
    return s


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(sage_\w+)\s*\(", txt, flags=re.M)))


def test_every_declared_symbol_is_exported(sage):
    names = declared_functions()
    assert set(names) == set(sage.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", sage.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for n in names:
        assert n in exported, n
    assert not any(e.startswith("or_") for e in exported)  # nothing of the oracle


def test_config_matches_the_method_constants(sage):
    import oracle

    for d in (64, 128):
        c = sage.get_config(d)
        assert c["abi_version"] == 1
        assert c["blkq"] == c["blkk"] == oracle.BLK == 128
        assert c["bc"] == oracle.BC == 128 and c["br"] == 256
        assert c["p_scale"] == oracle.P_SCALE == 448.0
        assert np.float32(c["log2_p_scale"]) == np.float32(math.log2(448.0))
        assert c["fp8_format"] == 0
    with pytest.raises(sage.SageError, match="UNSUPPORTED"):
        sage.get_config(96)


def test_quant_sizes(sage):
    s = sage.quant_sizes(2, 3, 300, 64, "fp8")
    nblk, npad = 3, 384
    assert s[sage.BUF_Q8] == s[sage.BUF_K8] == 2 * 3 * npad * 64
    assert s[sage.BUF_QSCALE] == s[sage.BUF_KSCALE] == 2 * 3 * nblk * 4
    assert s[sage.BUF_KMEAN] == s[sage.BUF_VSCALE] == 2 * 3 * 64 * 4
    assert s[sage.BUF_VQ] == 2 * 3 * npad * 64
    assert s[sage.BUF_WS_QK] == 2 * 3 * 1 * 64 * 8
    assert s[sage.BUF_WS_V] == (2 * 3 * 64 + 2 * 3 * 64) * 4
    s16 = sage.quant_sizes(2, 3, 300, 64, "fp16")
    assert s16[sage.BUF_VQ] == 2 * s[sage.BUF_VQ] and s16[sage.BUF_WS_V] == 0
    st = sage.quant_sizes(2, 3, 300, 64, "fp8", q_gran="token")
    assert st[sage.BUF_QSCALE] == 2 * 3 * npad * 4   # one scale per (padded) query row
    assert [st[i] for i in range(sage.NBUF) if i != sage.BUF_QSCALE] == \
        [s[i] for i in range(sage.NBUF) if i != sage.BUF_QSCALE]
    assert sage.quant_sizes(2, 3, 300, 64, "fp8", q_gran="block") == s


def test_qsmooth_sizes(sage):
    qm, bias = sage.qsmooth_sizes(2, 3, 300, 64)
    assert qm == 2 * 3 * 64 * 16 * 4                 # [B][H][d][16 ceil(nblk/16)] fp32
    assert bias == 2 * 3 * 3 * 384 * 4               # [B][H][nblk][N_pad] fp32


def _codes(sage):
    L = sage.lib()
    return L, {L.sage_status_string(c).decode().split(":")[0]: c for c in range(-8, 1)}


A = 0x10000  # a fake, 16-byte-aligned address: never dereferenced (validation fails first)


def test_invalid_arguments_rejected_before_launch(sage):
    L, _ = _codes(sage)
    sz = (ct.c_size_t * sage.NBUF)()
    assert L.sage_quant_sizes(1, 1, 0, 128, 0, sz) == -2
    assert L.sage_quant_sizes(1, 1, 10, 96, 0, sz) == -3
    assert L.sage_quant_sizes(1, 1, 10, 128, 2, sz) == -2
    assert L.sage_quant_sizes(1, 1, 10, 128, 0, None) == -1
    assert L.sage_quant_sizes(70000, 1, 10, 128, 0, sz) == -5
    assert L.sage_quant_sizes(1, 1 << 20, 1 << 20, 128, 0, sz) == -5
    qk = lambda q=A, N=256, d=128, lay=0, ws=A, wsb=1 << 20, q8=A: L.sage_quant_qk(
        q, A, 1, 1, N, d, lay, q8, A, A, A, A, ws, wsb, None)
    assert qk(q=None) == -1
    assert qk(ws=None) == -1
    assert qk(N=-5) == -2
    assert qk(d=32) == -3
    assert qk(lay=2) == -2
    assert qk(q=A + 8) == -4
    assert qk(q8=A + 1) == -4
    assert qk(wsb=16) == -7
    qv = lambda pv=0, ws=A, wsb=1 << 20, v=A: L.sage_quant_v(v, 1, 1, 256, 128, 0, pv, A, A, ws,
                                                              wsb, None)
    assert qv(v=None) == -1
    assert qv(pv=3) == -2
    assert qv(ws=None) == -1
    assert qv(wsb=8) == -7
    assert qv(v=A + 4) == -4
    sz1 = (ct.c_size_t * 9)()
    assert L.sage_quant_sizes(1, 1, 256, 128, 0, sz1) == 0
    need = sz1[7] + sz1[8]
    qkv = lambda v=A, pv=0, ws=A, wsb=need, N=256, vq=A: L.sage_quant_qkv(
        A, A, v, 1, 1, N, 128, 0, pv, A, A, A, A, A, vq, A, ws, wsb, None)
    assert qkv(v=None) == -1
    assert qkv(ws=None) == -1
    assert qkv(pv=2) == -2
    assert qkv(N=0) == -2
    assert qkv(vq=A + 2) == -4
    assert qkv(wsb=need - 1) == -7
    assert qkv(wsb=sz1[7]) == -7  # the V partials need room too
    fwd = lambda causal=0, sm=0.1, pv=0, od=0, out=A, N=256, lay=0: L.sage_attn_fwd(
        A, A, A, A, A, A, 1, 2, N, 128, lay, causal, sm, pv, out, od, None)
    assert fwd(out=None) == -1
    assert fwd(causal=2) == -2
    assert fwd(sm=float("nan")) == -2
    assert fwd(sm=float("inf")) == -2
    assert fwd(sm=0.0) == -2
    assert fwd(sm=-1.0) == -2
    assert fwd(pv=7) == -2
    assert fwd(od=5) == -2
    assert fwd(N=0) == -2
    assert fwd(lay=-1) == -2
    assert fwd(out=A + 2) == -4
    assert L.sage_quant_sizes_ex(1, 1, 10, 128, 0, 2, sz) == -2
    assert L.sage_quant_sizes_ex(1, 1, 10, 128, 0, -1, sz) == -2
    assert L.sage_quant_sizes_ex(1, 1, 10, 128, 0, 1, None) == -1
    qkx = lambda g=1, q=A: L.sage_quant_qk_ex(q, A, 1, 1, 256, 128, 0, g, A, A, A, A, A, A,
                                              1 << 20, None)
    assert qkx(g=2) == -2
    assert qkx(q=None) == -1
    fwdx = lambda g=1, sm=0.1: L.sage_attn_fwd_ex(A, A, A, A, A, A, 1, 2, 256, 128, 0, 0, sm, 0,
                                                  g, A, 0, None)
    assert fwdx(g=3) == -2
    assert fwdx(sm=-2.0) == -2
    sp = lambda tm=A, N=256, g=0: L.sage_attn_fwd_sparse(A, A, A, A, A, A, 1, 2, N, 128, 0, 0, 0.1,
                                                         0, g, tm, A, 0, None)
    assert sp(tm=None) == -1
    assert sp(tm=A + 3) == -4
    assert sp(g=5) == -2
    assert sp(N=2048 * 128 + 1) == -5      # more key tiles than a sparse launch can list
    assert sp(N=2048 * 128, tm=A + 3) == -4   # the size passes; validation stops at alignment
    a_, b_ = ct.c_size_t(), ct.c_size_t()
    assert L.sage_qsmooth_sizes(1, 1, 10, 128, None, ct.byref(b_)) == -1
    assert L.sage_qsmooth_sizes(1, 1, 0, 128, ct.byref(a_), ct.byref(b_)) == -2
    qks = lambda qm=A, g=0, q=A: L.sage_quant_qk_smooth(q, A, 1, 1, 256, 128, 0, g, A, A, A, A, A,
                                                       qm, A, 1 << 20, None)
    assert qks(qm=None) == -1
    assert qks(qm=A + 8) == -4
    assert qks(g=4) == -2
    assert qks(q=None) == -1
    qb = lambda qm=A, sm=0.1, N=256, bias=A, H=1: L.sage_q_smooth_bias(qm, A, A, 1, H, N, 128, 0, sm,
                                                                       bias, None)
    assert qb(qm=None) == -1
    assert qb(bias=None) == -1
    assert qb(sm=0.0) == -2
    assert qb(sm=float("nan")) == -2
    assert qb(bias=A + 4) == -4
    assert qb(N=1 << 20, H=4096) == -5      # the correction alone would be 2^40+ floats
    sm_ = lambda bias=A, tm=None, g=0, N=256: L.sage_attn_fwd_smooth(
        A, A, A, A, A, A, 1, 2, N, 128, 0, 0, 0.1, 0, g, bias, tm, A, 0, None)
    assert sm_(bias=None) == -1
    assert sm_(bias=A + 4) == -4
    assert sm_(g=3) == -2
    assert sm_(tm=A + 3) == -4
    assert sm_(tm=A, N=2048 * 128 + 1) == -5
    dbg = lambda b=0, h=0, row0=0, nrows=4, s=A: L.sage_attn_fwd_debug(
        A, A, A, A, A, A, 1, 2, 256, 128, 0, 0, 0.1, 0, A, 0, b, h, row0, nrows, s, None)
    assert dbg(s=None) == -1
    assert dbg(b=1) == -2
    assert dbg(h=2) == -2
    assert dbg(row0=-1) == -2
    assert dbg(nrows=0) == -2
    assert dbg(row0=250, nrows=7) == -2
    assert dbg(s=A + 4) == -4


def test_backward_arguments_rejected_before_launch(sage):
    L = sage.lib()
    ws = ct.c_size_t()
    assert L.sage_bwd_sizes(1, 1, 256, 128, None) == -1
    assert L.sage_bwd_sizes(1, 1, 0, 128, ct.byref(ws)) == -2
    assert L.sage_bwd_sizes(1, 1, 256, 96, ct.byref(ws)) == -3
    assert L.sage_bwd_sizes(1, 1, 256, 64, ct.byref(ws)) == 0
    assert L.sage_bwd_sizes(70000, 1, 256, 128, ct.byref(ws)) == -5
    # the documented parts, each rounded up to 256 bytes
    B, H, N, d = 2, 3, 300, 128
    assert L.sage_bwd_sizes(B, H, N, d, ct.byref(ws)) == 0
    bh, nblk = B * H, -(-N // 128)
    parts = [bh * 128 * nblk * 4, bh * nblk * 4] + [bh * 128 * nblk * d * 2] * 2 + \
        [bh * nblk * d * 128] * 3 + [bh * nblk * 512 * 4]
    need = sum(-(-p // 256) * 256 for p in parts)
    assert ws.value == need
    bwd = lambda q8=A, lse=A, dq=A, wsp=A, wsb=need, N=N, d=d, lay=0, causal=0, sm=0.1: \
        L.sage_attn_bwd(q8, A, A, A, A, A, A, lse, B, H, N, d, lay, causal, sm, dq, A, A, wsp, wsb,
                        None)
    assert bwd(q8=None) == -1
    assert bwd(lse=None) == -1
    assert bwd(dq=None) == -1
    assert bwd(wsp=None) == -1
    assert bwd(N=0) == -2
    assert bwd(d=96) == -3
    assert bwd(lay=2) == -2
    assert bwd(causal=2) == -2
    for sm in (float("nan"), float("inf"), 0.0, -1.0):
        assert bwd(sm=sm) == -2
    assert bwd(dq=A + 4) == -4
    assert bwd(wsp=A + 16) == -4      # the workspace must be 256-byte aligned
    assert bwd(wsb=need - 1) == -7
    lse = lambda out=A, ls=A, causal=0, sm=0.1, pv=0: L.sage_attn_fwd_lse(
        A, A, A, A, A, A, 1, 2, 256, 128, 0, causal, sm, pv, out, 0, ls, None)
    assert lse(ls=None) == -1
    assert lse(out=None) == -1
    assert lse(causal=2) == -2
    assert lse(sm=0.0) == -2
    assert lse(pv=7) == -2
    assert lse(ls=A + 4) == -4


def test_binding_refuses_host_tensors_and_wrong_operands(sage):
    """The binding passes raw pointers: a host tensor, or an operand of the
    wrong size, is refused before the library is called."""
    import torch

    B, H, N, d = 1, 2, 200, 128
    x = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    for call in (lambda: sage.quant_qk(x, x), lambda: sage.quant_v(x),
                 lambda: sage.quant_qk_mx(x, x), lambda: sage.quant_v_mx(x)):
        with pytest.raises(ValueError, match="one GPU"):
            call()
    nblk = -(-N // 128)
    qz = dict(B=B, H=H, N=N, d=d, layout="HND", q_gran="block",
              q8=torch.zeros((B, H, nblk * 128, d), dtype=torch.int8),
              q_scale=torch.zeros((B, H, nblk)), k8=torch.zeros((B, H, nblk * 128, d), dtype=torch.int8),
              k_scale=torch.zeros((B, H, nblk)))
    vq = torch.zeros((B, H, nblk, d, 128), dtype=torch.uint8)
    vs = torch.zeros((B, H, d))
    lse = torch.zeros((B, H, N))
    with pytest.raises(ValueError, match="one GPU"):
        sage.attn_fwd(qz, vq, vs)
    with pytest.raises(ValueError, match="one GPU"):
        sage.attn_fwd_lse(qz, vq, vs)
    with pytest.raises(ValueError, match="one GPU"):
        sage.attn_bwd(qz, x, x, x, lse)
    mz = dict(B=B, H=H, N=N, d=d, layout="HND", q6=torch.zeros((B, H, nblk * 128, d), dtype=torch.uint8),
              k6=torch.zeros((B, H, nblk * 128, d), dtype=torch.uint8))
    with pytest.raises(ValueError, match="one GPU"):
        sage.attn_fwd_mx(mz, vq)
    # the operand sizes are checked after the device (on GPU tensors, in the
    # GPU parity tests); the output check on its own:
    with pytest.raises(ValueError):
        sage._check_out(torch.zeros((B, H, N, d)), (B, H, N, 64), torch.device("cpu"))


def test_status_strings(sage):
    L = sage.lib()
    names = [L.sage_status_string(c).decode() for c in range(0, -8, -1)]
    assert names[0] == "SAGE_OK" and all(n.startswith("SAGE_ERR_") for n in names[1:])
    assert L.sage_status_string(12345).decode() == "SAGE_ERR_UNKNOWN"


def test_mx4_layout_reader_round_trip():
    """The tests' reader of the E2M1 block layout against a packer written
    from the same header text in the opposite direction."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from sage_layouts import mx4_unpack_blocks

    rng = np.random.default_rng(1)
    vals = rng.integers(0, 16, (5, 32)).astype(np.uint8)
    scales = rng.integers(0, 256, 5).astype(np.uint8)
    raw = np.zeros((5, 32), np.uint8)
    for b in range(5):
        for i in range(16):
            raw[b, i] = vals[b, i] | (vals[b, 16 + i] << 4)   # value i low, 16 + i high
        raw[b, 24] = scales[b]
    c, e, pad = mx4_unpack_blocks(raw)
    assert np.array_equal(c, vals) and np.array_equal(e, scales) and not pad.any()
    raw[0, 20] = 1
    assert mx4_unpack_blocks(raw)[2].any()


def test_mx_format_argument_rejected_before_launch(sage):
    """The _fmt entry points take SAGE_MX_FP6 (6) or SAGE_MX_FP4 (4) only."""
    L = sage.lib()
    p = ct.c_void_p(16)
    for fmt in (0, 5, 8, -4):
        assert L.sage_quant_qk_mx_fmt(p, p, 1, 1, 10, 128, 0, fmt, p, p, p, p, 1 << 20, None) == -2
        assert L.sage_quant_v_mx_fmt(p, 1, 1, 10, 128, 0, fmt, p, None) == -2
        assert L.sage_attn_fwd_mx_fmt(p, p, p, 1, 1, 10, 128, 0, fmt, 0, 0.1, p, 0, None) == -2


def test_mx6_layout_reader_round_trip():
    """The tests' reader of the MX6 block layout against a packer written
    from the same header text in the opposite direction."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from sage_layouts import mx6_unpack_blocks

    rng = np.random.default_rng(0)
    vals = rng.integers(0, 64, (5, 32)).astype(np.uint8)
    scales = rng.integers(0, 256, 5).astype(np.uint8)
    raw = np.zeros((5, 32), np.uint8)
    for b in range(5):
        word = 0
        for i in range(16):
            word |= int(vals[b, i]) << (12 * i)            # element 2i = value i
            word |= int(vals[b, 16 + i]) << (12 * i + 6)   # element 2i + 1 = value 16 + i
        raw[b, :24] = np.frombuffer(word.to_bytes(24, "little"), np.uint8)
        raw[b, 24] = scales[b]
    c, e, pad = mx6_unpack_blocks(raw)
    assert np.array_equal(c, vals) and np.array_equal(e, scales) and not pad.any()
