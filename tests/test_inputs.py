"""The seeded synthetic workloads: shapes, determinism and the outlier recipe."""
import torch

import synthetic_inputs as si


def test_shapes_and_determinism():
    a = si.make("tiny", N=257)
    b = si.make("tiny", N=257)
    assert a.q.shape == (1, 2, 257, 128) and a.q.dtype == torch.bfloat16
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    c = si.make("tiny", N=257, seed=5)
    assert not torch.equal(a.q, c.q)


def test_offset_recipe_has_per_channel_key_offsets():
    wl = si.make("tiny", N=4096, H=2)
    km = wl.k.float().mean(dim=2)  # per (b, h, channel)
    assert 1.5 < km.std().item() < 4.5  # offsets ~ N(0, 3^2)
    assert wl.q.float().mean(dim=2).abs().max().item() < 0.2


def test_outlier_recipe():
    wl = si.make("outlier", B=1, H=3, N=2000)
    assert wl.outlier_tokens.shape == (1, 3, 10)  # round(0.5% of 2000)
    qn = wl.q.float().norm(dim=-1)
    for h in range(3):
        idx = wl.outlier_tokens[0, h]
        assert len(set(idx.tolist())) == 10
        assert qn[0, h, idx].min() > 5 * qn[0, h].median()
    km = wl.k.float().mean(dim=2).abs()  # exactly one channel per head carries the offset
    assert ((km > 2.0).sum(dim=-1) <= 1).all()
