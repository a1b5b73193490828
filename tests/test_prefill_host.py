"""Host-side checks of the prefill driver's model pieces (CPU tensors): the
rotary embedding depends only on relative position in dot products and
keeps norms; RMSNorm gives unit root-mean-square rows."""

import torch

from token_selection_tsp_amd import prefill


def test_rope_relative_position_and_norm():
    g = torch.Generator().manual_seed(0)
    d = 64
    q = torch.randn(1, 2, d, generator=g, dtype=torch.float64).float()
    k = torch.randn(1, 2, d, generator=g, dtype=torch.float64).float()

    def dot(pq, pk):
        rq = prefill._rope(q, torch.tensor([pq]), 10000.0)
        rk = prefill._rope(k, torch.tensor([pk]), 10000.0)
        return (rq * rk).sum(-1)

    base = dot(5, 2)
    for shift in (0, 1, 17, 1000):
        assert torch.allclose(dot(5 + shift, 2 + shift), base, rtol=1e-4, atol=1e-4)
    assert not torch.allclose(dot(5, 2), dot(9, 2), rtol=1e-3, atol=1e-3)
    r = prefill._rope(q, torch.tensor([123]), 10000.0)
    assert torch.allclose(r.norm(dim=-1), q.norm(dim=-1), rtol=1e-5)
    assert torch.allclose(prefill._rope(q, torch.tensor([0]), 10000.0), q)   # position 0: identity


def test_rms_norm_unit_rows():
    x = torch.randn(7, 256, dtype=torch.float32) * 3.0 + 1.0
    w = torch.ones(256)
    y = prefill._rms(x, w, 1e-6)
    assert torch.allclose(y.pow(2).mean(-1).sqrt(), torch.ones(7), rtol=1e-4)
    w2 = torch.full((256,), 2.0)
    assert torch.allclose(prefill._rms(x, w2, 1e-6), 2 * y, rtol=1e-6)


def test_llama3_8b_shape():
    s = prefill.llama3_8b()
    assert (s.layers, s.hidden, s.heads, s.kv_heads, s.head_dim, s.mlp) == (32, 4096, 32, 8, 128, 14336)
    assert s.heads * s.head_dim == s.hidden and s.heads % s.kv_heads == 0
