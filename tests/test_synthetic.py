"""The seeded input generators: the concentrated-key option produces keys at
the requested cosine to their head's running mean key (the key concentration
of "The Key to Going Linear: Analysis-Driven Transformer Linearization",
appendix B.1, Metric 1), with unit norm; the default keys are not
concentrated."""
import torch

import synthetic


def _running_mean_cos(k):
    k = k.double()
    n = torch.arange(1, k.shape[1] + 1, dtype=torch.float64)[None, :, None, None]
    mean = k.cumsum(1) / n
    return (k * mean).sum(-1) / (k.norm(dim=-1) * mean.norm(dim=-1))


def test_concentrated_keys_cosine_and_norm():
    for cos in (0.8, 0.9, 0.97):
        x = synthetic.gdn_inputs(1, 2000, 2, 128, 64, dtype="f32", seed=5, key_cos=cos)
        c = _running_mean_cos(x["k"])
        assert abs(float(c[:, 200:].mean()) - cos) < 0.01
        assert torch.allclose(x["k"].norm(dim=-1), torch.ones(1, 2000, 2), atol=1e-5)


def test_default_keys_not_concentrated():
    x = synthetic.gdn_inputs(1, 2000, 2, 128, 64, dtype="f32", seed=5)
    assert float(_running_mean_cos(x["k"])[:, 200:].abs().mean()) < 0.1


def test_beta_shift_moves_step_sizes_up():
    lo = synthetic.gdn_inputs(1, 4000, 1, 16, 16, dtype="f32", seed=1)["beta"]
    hi = synthetic.gdn_inputs(1, 4000, 1, 16, 16, dtype="f32", seed=1, beta_shift=3.0)["beta"]
    assert 0.45 < float(lo.mean()) < 0.55 and float(hi.mean()) > 0.9
    assert float(hi.max()) < 1.0
