"""The block's dense MLP as an always-on expert (one expert, top-1, weight 1).

Model card "Gemma 4 26B-A4B it QAT Q4_0 with MTP assistant and vision, NInfer
v3 artifact", table "What is inside": the dense MLP's gate and up rows are one
Q4_0 parent, as an expert's are.  The pages give no width for it; these cases
use I = 2112 (three expert widths) at the Gemma hidden size, plus a narrow
ragged one.  The oracle is the pinned per-token expert FFN with expert 0.
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


@pytest.mark.parametrize("H,I,T,act", [
    (2816, 2112, 1, "f32"),     # decode
    (2816, 2112, 8, "bf16"),    # batched decode (GEMV path)
    (2816, 2112, 200, "bf16"),  # prefill chunk (MFMA path)
    (288, 96, 70, "bf16"),      # odd block counts per row
])
def test_dense_mlp(H, I, T, act):
    from sparse_moe_amd import binding
    spec = synth.LayerSpec("dense-H%d-I%d-T%d" % (H, I, T), H=H, E=1, K=1, I=I, T=T, act=act,
                           router_std=1 / np.sqrt(H), seed=31)
    L = synth.make_layer(spec)
    print("dense mlp H=%d I=%d T=%d act=%s" % (H, I, T, act), flush=True)
    out = binding.dense_ffn_q4_0(parity.to_dev(L.x), parity.to_dev(L.w_gate_up[0]),
                                 parity.to_dev(L.w_down[0]))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rows = range(T) if T <= 8 else range(0, T, 7)
    for t in rows:
        _, y = oracle.expert_ffn_token(L.x[t], L.w_gate_up, L.w_down, 0)
        err = np.max(np.abs(got[t] - y))
        assert err <= parity.TOL * np.max(np.abs(y)), (t, err)
