"""Plain Q4_0 linear layer through the C ABI (moe_linear_q4_0).

Model card "Gemma 4 26B-A4B it QAT Q4_0 with MTP assistant and vision, NInfer
v3 artifact", table "What is inside": the Q, K and V rows of a block form one
Q4_0 parent, read in place like the experts' matrices.  The pages give no
attention widths; the Gemma-width cases use a synthetic parent of 4224 rows
(three 1408-row parts) over the hidden size 2816.  The oracle is the pinned
plain Q4_0 linear layer; the bar is the same as for the expert outputs.
"""
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


@pytest.mark.parametrize("H,R,T,act", [
    (2816, 4224, 1, "f32"),      # decode, GEMV staged through LDS
    (2816, 4224, 6, "bf16"),     # a few tokens, GEMV with register windows
    (2816, 4224, 5, "f32"),
    (2816, 4224, 130, "bf16"),   # prefill chunk: bf16 MFMA, a ragged second slot tile
    (288, 100, 70, "bf16"),      # odd block count and rows not a multiple of 16: GEMV
    (256, 200, 80, "bf16"),      # rows not a multiple of 16 at T >= 64: GEMV
])
def test_linear_q4_0(H, R, T, act):
    from sparse_moe_amd import binding
    rng = np.random.default_rng(H + R + T)
    spec = synth.LayerSpec("lin", H=H, E=1, K=1, I=32, T=T, act=act, router_std=0.1, seed=R)
    x = synth.activations(spec, T, spec.seed + 5)
    nb = H // 32
    w = np.empty((R, nb, 18), np.uint8)
    w[..., 2:] = rng.integers(0, 256, size=(R, nb, 16), dtype=np.uint8)
    d = np.abs(rng.normal(0.0, 0.02, size=(R, nb))).astype(np.float16)
    w[..., 0:2] = d.view(np.uint8).reshape(R, nb, 2)
    print("linear H=%d R=%d T=%d act=%s" % (H, R, T, act), flush=True)
    y = binding.moe_linear_q4_0(parity.to_dev(x), parity.to_dev(w))
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    rows = np.arange(T) if T <= 8 else np.unique(np.r_[np.arange(0, T, 9), T - 1])
    ref = oracle.linear_q4_0(x[rows], w)
    err = np.max(np.abs(got[rows] - ref))
    assert err <= parity.TOL * np.max(np.abs(ref)), err
