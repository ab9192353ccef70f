"""Router logits on the bf16 MFMA path (64 tokens and up), against the oracle.

The three tilings of the MFMA router (few tiles: 16 tokens per workgroup with
each wave's K steps loaded in batches; middle: 32 tokens per workgroup with
double-buffered K steps; many tokens: 64 tokens per workgroup) at the Gemma
shape, with and without the per-dimension router scale and the logit bias;
logits within 1e-4 of max|logit| of the oracle's fp64 values (the products
are exact, the fp32 sums in another order).  Ids and weights come from the
same call and are checked under the near-tie rule."""
import numpy as np
import pytest
import torch

import oracle
import parity
from sparse_moe_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("T", [64, 100, 512, 1024, 1056, 2048, 2100])
@pytest.mark.parametrize("scaled", [False, True])
def test_router_logits_mfma(T, scaled):
    from sparse_moe_amd import binding
    spec = synth.LayerSpec("router-T%d" % T, H=2816, E=128, K=8, I=64, T=T, act="bf16",
                           router_std=1 / np.sqrt(2816), seed=51)
    L = synth.make_layer(spec)
    g = np.random.default_rng(53 + T)
    rs = (1.0 + 0.25 * g.standard_normal(spec.H)).astype(np.float32) if scaled else None
    bias = (0.1 * g.standard_normal(spec.E)).astype(np.float32) if scaled else None
    print("case: router logits T=%d scaled=%s" % (T, scaled), flush=True)
    logits = torch.full((T, spec.E), float("nan"), device="cuda")
    ids = torch.full((T, spec.K), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, spec.K), float("nan"), device="cuda")
    binding.moe_router_topk(parity.to_dev(L.x), parity.to_dev(L.w_router), logits, ids, w,
                            r_scale=None if rs is None else parity.to_dev(rs),
                            logit_bias=None if bias is None else parity.to_dev(bias))
    torch.cuda.synchronize()
    ref = oracle.router_logits(L.x, L.w_router, r_scale=rs, bias=bias)
    got = logits.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    print("  -> max|d|/max|ref| = %.2e" % err, flush=True)
    assert err <= 1e-4
    parity.check_routing(L, {"topk_ids": ids.cpu().numpy(), "topk_w": w.cpu().numpy()}, ref)
