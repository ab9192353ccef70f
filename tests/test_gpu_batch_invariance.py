"""Batch invariance of the decode path at speculative-decoding verification
shapes.

Model card "Gemma 4 26B-A4B it QAT Q4_0 with MTP assistant and vision, NInfer
v3 artifact", sections "Speculative decoding" and "Quality": the model checks
the assistant's drafts in one pass whose logits equal those of plain decoding
bit for bit.  For the routed-MoE layer that means a token's result may not
depend on the batch it is computed in: one request verifying 1 + d tokens,
two or three requests with one draft each, up to eight requests decoding
plainly, or any mix of them.

Every batch below 64 tokens takes the same kernels per token (the per-expert
router GEMV, the Q4_0 GEMV expert FFN, the fixed-order combine), so each
token's router logits, top-K ids and weights and combined output must equal,
bit for bit, those of the same token run alone (T = 1), with the fused routing
call and with the separate router and permutation calls alike.
"""
import numpy as np
import pytest
import torch

import parity
from sparse_moe_amd import synth

pytestmark = pytest.mark.gpu

T_ALL = 63
# (first token, batch size): one request with 1..4 drafts, 2-3 requests with
# one draft each, 8 plain requests, and larger mixed batches up to 63 tokens
BATCHES = [(0, 2), (3, 5), (10, 4), (20, 6), (30, 8), (7, 9), (40, 17), (0, 40), (0, 63)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_token_results_do_not_depend_on_the_batch(act):
    from sparse_moe_amd import binding
    spec = synth.LayerSpec("verify-%s" % act, H=2816, E=128, K=8, I=704, T=T_ALL, act=act,
                           router_std=1 / np.sqrt(2816), seed=21)
    L = synth.make_layer(spec)
    x = parity.to_dev(L.x)
    wr, gu, dn = parity.to_dev(L.w_router), parity.to_dev(L.w_gate_up), parity.to_dev(L.w_down)
    sc = parity.to_dev(L.expert_scale)

    def run(a, n, fused):
        print("batch act=%s first=%d size=%d fused=%s" % (act, a, n, fused), flush=True)
        b = binding.moe_layer(x[a:a + n].contiguous(), wr, gu, dn, spec.K, expert_scale=sc,
                              fused_route=fused)
        torch.cuda.synchronize()
        return {k: getattr(b, k).cpu().numpy() for k in ("logits", "topk_ids", "topk_w", "out")}

    alone = [run(t, 1, True) for t in range(T_ALL)]
    for t in (0, 17, 62):   # the separate routing calls give the same single-token result
        r = run(t, 1, False)
        for k in r:
            assert np.array_equal(_bits(r[k]), _bits(alone[t][k])), (t, k)
    for a, n in BATCHES:
        for fused in (True, False):
            r = run(a, n, fused)
            for i in range(n):
                ref = alone[a + i]
                for k in ("logits", "topk_ids", "topk_w", "out"):
                    assert np.array_equal(_bits(r[k][i]), _bits(ref[k][0])), (a, n, fused, i, k)
