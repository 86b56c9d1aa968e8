"""HIP graph capture of whole steps.

Every libsage entry point only launches kernels on the caller's stream (no
allocation, copy or memset inside the library; the binding's output and
workspace tensors come from PyTorch's allocator, which serves a capture from
the graph's own pool), so a quantize-and-attend step, or the training
forward and the backward, can be captured once and replayed.  Each replay
must equal the eager result bit for bit, with eager work and
synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import synthetic_inputs as si

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_attention_video_02_amd as s

    s.lib()
    return s


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _replay_and_compare(g, out, fn, eager):
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert torch.equal(a, b), i
        other = fn()                     # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(other, eager):
            assert torch.equal(a, b), i


def _forward_step(sage, wl, path):
    tm = None
    if path == "sparse":
        nblk = -(-wl.N // 128)
        rng = np.random.default_rng(7)
        tm = torch.from_numpy((rng.random((wl.B, wl.H, nblk, nblk)) < 0.6).astype(np.uint8)).cuda()

    def fn():
        if path == "mx":
            return (sage.attn_fwd_mx(sage.quant_qk_mx(wl.q, wl.k), sage.quant_v_mx(wl.v),
                                     sm_scale=wl.sm_scale),)
        pv = "fp16" if path == "fp16" else "fp8"
        qz = sage.quant_qk(wl.q, wl.k, q_gran="token" if path == "token" else "block",
                           q_smooth=path == "qsmooth", sm_scale=wl.sm_scale)
        vq, vs = sage.quant_v(wl.v, pv)
        return (sage.attn_fwd(qz, vq, vs, sm_scale=wl.sm_scale, pv=pv, tile_mask=tm),)
    return fn


@pytest.mark.parametrize("path", ["fp8", "fp16", "token", "sparse", "qsmooth", "mx"])
def test_forward_step_graph_replays_equal_eager(sage, path):
    print(f"[graph] forward {path}", flush=True)
    wl = si.make("tiny", N=700, H=2, device="cuda")
    fn = _forward_step(sage, wl, path)
    eager = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    g, out = _capture(fn)
    _replay_and_compare(g, out, fn, eager)


def test_training_step_graph_replays_equal_eager(sage):
    print("[graph] training forward + backward", flush=True)
    wl = si.make("causal_prefill", B=1, H=2, N=600, device="cuda")
    do = si.output_grad(wl)

    def fn():
        qz = sage.quant_qk(wl.q, wl.k)
        vq, vs = sage.quant_v(wl.v, "fp8")
        o, lse = sage.attn_fwd_lse(qz, vq, vs, causal=True, sm_scale=wl.sm_scale)
        return (o, lse) + tuple(sage.attn_bwd(qz, wl.v, o, do, lse, causal=True, sm_scale=wl.sm_scale))

    eager = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    g, out = _capture(fn)
    _replay_and_compare(g, out, fn, eager)
