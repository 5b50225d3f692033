"""Where the oracle's readings meet and leave the one mHC module the image
holds: transformers' DeepseekV4HyperConnection (a library implementation,
used here only as a cross-check on CPU, in fp64).

With its group scales at 1 and hc_eps = 0 the module computes the oracle's
coefficients: the same logit order [pre 4, post 4, mix 16] (reading R4's
split), the RMS scale of the flattened 4C row (R2; the module scales the row
before the projection, the oracle the projection, equal in exact
arithmetic), post = 2 sigmoid, and the Sinkhorn of exp(logits) rows first
(its first row step is a softmax, which is the row division when eps = 0).
It differs in one reading the pages leave open (R4): its decoder layer
consumes the Sinkhorn matrix transposed, output route k = sum_j M[j, k] x_j,
where the oracle takes row j as output route j.  So the oracle's post with M
equals the module's mixing with M^T, and not with M.
"""
import numpy as np
import pytest
import torch

import oracle as O

tfm = pytest.importorskip("transformers.models.deepseek_v4.modeling_deepseek_v4")
cfgm = pytest.importorskip("transformers.models.deepseek_v4.configuration_deepseek_v4")


def module(C, iters, seed=0):
    c = cfgm.DeepseekV4Config(hidden_size=C, hc_mult=4, hc_sinkhorn_iters=iters, hc_eps=0.0, rms_norm_eps=1e-6)
    m = tfm.DeepseekV4HyperConnection(c).double()
    g = torch.Generator().manual_seed(seed)
    with torch.no_grad():
        m.fn.copy_(torch.randn((24, 4 * C), generator=g, dtype=torch.float64) * 0.02)
        m.base.copy_(torch.randn(24, generator=g, dtype=torch.float64) * 0.1)
        m.scale.fill_(1.0)
    return m


def test_coefficients_agree_with_the_module():
    C, T = 256, 12
    m = module(C, iters=20)
    g = torch.Generator().manual_seed(1)
    x = torch.randn((1, T, 4, C), generator=g, dtype=torch.float64).to(torch.bfloat16).double()
    with torch.no_grad():
        post, comb, collapsed = m(x)
    cf = O.coeffs(x[0].numpy(), m.fn.detach().numpy().T, m.base.detach().numpy(), hc_norm_eps=1e-6,
                  hc_post_scale=2.0, sinkhorn_eps=0.0, sinkhorn_iters=20)
    pre_o, post_o, res_o = O.split_coeffs(cf)
    # (the module casts the flattened row to fp32 before its projection, so
    # the agreement is to the coefficient bar, 1e-4 relative)
    assert np.allclose(post[0].numpy(), post_o, rtol=1e-4, atol=0)
    assert np.allclose(comb[0].numpy(), res_o, rtol=1e-4, atol=0)
    # the module's collapsed stream is sum_i pre_i x_i
    assert np.allclose(collapsed[0].numpy(), np.einsum("ti,tic->tc", pre_o, x[0].numpy()), rtol=1e-4, atol=1e-6)


def test_mixing_orientation_differs():
    # oracle: x'_j = sum_i M[j, i] x_i + post_j y; module: x'_k = sum_j M[j, k] x_j + post_k y
    C, T = 256, 5
    rng = np.random.default_rng(2)
    x = O.bf16_round(rng.standard_normal((T, 4, C)))
    y = O.bf16_round(rng.standard_normal((T, C)))
    M = O.sinkhorn(np.exp(rng.standard_normal((T, 4, 4))), 20, 0.0)
    pw = rng.uniform(0, 2, size=(T, 4))

    def module_mix(mat):
        xt = torch.from_numpy(x)[None]
        out = torch.from_numpy(pw)[None].unsqueeze(-1) * torch.from_numpy(y)[None].unsqueeze(-2) + torch.matmul(
            torch.from_numpy(mat)[None].transpose(-1, -2), xt)
        return out[0].numpy()

    ours = O.post_exact(x, y, pw, M)
    assert np.allclose(ours, O.bf16_round(module_mix(np.swapaxes(M, 1, 2))), rtol=0, atol=0.05 * np.abs(ours).max())
    # with M itself the module mixes by columns: another result, since M is not symmetric
    assert np.abs(ours - O.bf16_round(module_mix(M))).max() > 0.1
    # after the last column normalisation the module's output weights (columns) sum to 1
    assert np.allclose(M.sum(axis=1), 1.0, atol=1e-12)
