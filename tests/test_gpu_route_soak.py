"""Soak test of the fused few-token routing kernel (moe_route for 1..8 tokens).

Its workgroups publish the router logits to the last one through an agent-scope
release increment of a counter in the workspace, and the last one reads them
after an acquire fence, runs top-K and the permutation, and resets the counter.
2,000 calls in a row on one workspace, with fresh seeded activations and a
token count cycling through 1..8, must each equal the separate calls
(moe_router_topk + moe_permute, which hand the logits over through a kernel
boundary) bit for bit; the loop stops at the first difference."""
import numpy as np
import pytest
import torch

from sparse_moe_amd import synth

pytestmark = pytest.mark.gpu

CALLS = 2000


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_fused_routing_soak(act):
    from sparse_moe_amd import binding
    spec = synth.SPECS[1]
    H, E, K = spec.H, spec.E, spec.K
    L = synth.make_layer(spec, seed=901, with_x=False)
    wr = torch.from_numpy(L.w_router).cuda()
    dt = torch.float32 if act == "f32" else torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(902)
    fused = [binding.LayerBuffers(T, H, spec.I, E, K, dt) for T in range(1, 9)]
    sep = [binding.LayerBuffers(T, H, spec.I, E, K, dt) for T in range(1, 9)]
    ws = torch.zeros(binding.moe_route_workspace_bytes(8, K, E), dtype=torch.uint8, device="cuda")
    keys = ("logits", "topk_ids", "topk_w", "offsets", "sorted_slots", "slot_pos")
    print("case: fused routing soak, %d calls, %s" % (CALLS, act), flush=True)
    for i in range(CALLS):
        T = 1 + i % 8
        x = torch.randn((T, H), generator=gen, device="cuda").to(dt)
        f, s = fused[T - 1], sep[T - 1]
        binding.moe_route(x, wr, f.logits, f.topk_ids, f.topk_w, f.offsets, f.sorted_slots,
                          f.slot_pos, ws)
        binding.moe_router_topk(x, wr, s.logits, s.topk_ids, s.topk_w)
        binding.moe_permute(s.topk_ids, E, s.offsets, s.sorted_slots, s.slot_pos, s.ws_perm)
        same = all(torch.equal(getattr(f, k), getattr(s, k)) for k in keys)
        assert same, "call %d (T=%d): fused routing differs from the separate calls" % (i, T)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "counter not left at zero"
    print("  -> %d calls equal" % CALLS, flush=True)
