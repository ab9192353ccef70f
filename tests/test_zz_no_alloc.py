"""The no-allocation expert FFN entry point against the workspace one.

moe_expert_ffn_q4_0_noalloc runs the same kernels as moe_expert_ffn_q4_0 with
the library's static per-GPU scratch as its workspace, so its outputs must
equal the workspace entry point's bit for bit.  Two calls in a row on each
path, the second with a smaller input (the scratch keeps the first call's
contents), on the decode GEMV path and on the bf16 MFMA path; the first call's
result is also checked against the oracle on sampled tokens."""
import numpy as np
import pytest
import torch

import parity
from sparse_moe_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _layer_calls(L):
    """Routing through the C ABI, then both FFN entry points on it."""
    from sparse_moe_amd import binding
    spec = L.spec
    T = L.x.shape[0]
    x = parity.to_dev(L.x)
    gu, dn = parity.to_dev(L.w_gate_up), parity.to_dev(L.w_down)
    act = torch.float32 if spec.act == "f32" else torch.bfloat16
    bufs = binding.LayerBuffers(T, spec.H, spec.I, spec.E, spec.K, act)
    binding.moe_router_topk(x, parity.to_dev(L.w_router), bufs.logits, bufs.topk_ids,
                            bufs.topk_w)
    binding.moe_permute(bufs.topk_ids, spec.E, bufs.offsets, bufs.sorted_slots, bufs.slot_pos,
                        bufs.ws_perm)
    binding.moe_expert_ffn_q4_0(x, gu, dn, spec.K, bufs.offsets, bufs.sorted_slots, bufs.y_sorted,
                                bufs.ws_ffn)
    y_na = torch.full_like(bufs.y_sorted, float("nan"))
    binding.moe_expert_ffn_q4_0_noalloc(x, gu, dn, spec.K, bufs.offsets, bufs.sorted_slots, y_na)
    torch.cuda.synchronize()
    return bufs, y_na


@pytest.mark.parametrize("spec_id,T1,T2", [(2, 8, 3), (1, 1, 1), (3, 256, 64)])
def test_noalloc_equals_workspace_entry_point(spec_id, T1, T2):
    spec = synth.SPECS[spec_id]
    for i, T in enumerate((T1, T2)):
        print("case: noalloc %s T=%d (call %d)" % (spec.name, T, i + 1), flush=True)
        L = synth.make_layer(spec, seed=900 + 10 * spec_id + i, T=T)
        bufs, y_na = _layer_calls(L)
        assert torch.equal(y_na, bufs.y_sorted), "no-alloc output differs from the workspace one"
        if i == 0:
            g = {k: getattr(bufs, k).cpu().numpy() for k in
                 ("logits", "topk_ids", "topk_w", "offsets", "sorted_slots", "slot_pos")}
            g["y_sorted"] = y_na.cpu().numpy()
            from sparse_moe_amd import binding
            binding.moe_combine(y_na, bufs.slot_pos, bufs.topk_ids, bufs.topk_w,
                                parity.to_dev(L.expert_scale), out_f32=bufs.out)
            torch.cuda.synchronize()
            g["out"] = bufs.out.cpu().numpy()
            sample = None if T <= 8 else np.unique(np.r_[0, T // 2, T - 1])
            print("  ->", parity.check_layer(L, g, token_sample=sample), flush=True)


def test_noalloc_rejects_more_than_its_scratch():
    from sparse_moe_amd import binding
    spec = synth.SPECS[3]
    x = torch.zeros((4096, spec.H), dtype=torch.bfloat16, device="cuda")
    gu = torch.zeros((spec.E, 2 * spec.I, spec.H // 32, 18), dtype=torch.uint8, device="cuda")
    dn = torch.zeros((spec.E, spec.H, spec.I // 32, 18), dtype=torch.uint8, device="cuda")
    off = torch.zeros(spec.E + 1, dtype=torch.int32, device="cuda")
    ss = torch.zeros(4096 * spec.K, dtype=torch.int32, device="cuda")
    y = torch.zeros((4096 * spec.K, spec.H), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.MoEError, match="MOE_ERR_SCRATCH"):
        binding.moe_expert_ffn_q4_0_noalloc(x, gu, dn, spec.K, off, ss, y)
