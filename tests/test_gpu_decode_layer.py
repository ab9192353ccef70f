"""The one-call decode layer (moe_layer_decode) on the GPU.

  * parity with the oracle for 1..8 tokens at the Gemma shape, fp32 and bf16
    activations (routing bit-exact under the near-tie rule, combined output
    within the fp32 bar);
  * bitwise equality with the separate calls (moe_route, moe_expert_ffn_q4_0,
    moe_combine) on the same inputs: logits, ids, weights, permutation and the
    combined output, fp32 and residual + bf16;
  * injected logits, a small shape with other block counts, and K = 16;
  * a 30-layer decode stack (RMSNorm, layer, residual) captured in one HIP
    graph and replayed several times, with eager work between the replays,
    each replay equal to the eager stack bit for bit.

One token at the Gemma shape runs gate/up and down in one launch (down
workgroups wait on a completion counter); every call here also checks that
its timeout flag stayed clear.  Other shapes take two launches.
"""
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


def _dev_layer(L):
    return dict(x=parity.to_dev(L.x), wr=parity.to_dev(L.w_router), gu=parity.to_dev(L.w_gate_up),
                dn=parity.to_dev(L.w_down), sc=parity.to_dev(L.expert_scale),
                bias=None if L.router_bias is None else parity.to_dev(L.router_bias))


ROUTE_KEYS = ("logits", "topk_ids", "topk_w", "offsets", "sorted_slots", "slot_pos")


def _run_both(L, logits_in=None, residual=False):
    """The fused call and the separate calls on the same inputs."""
    from sparse_moe_amd import binding
    d = _dev_layer(L)
    T, H = L.x.shape
    spec = L.spec
    act = torch.float32 if spec.act == "f32" else torch.bfloat16
    li = None if logits_in is None else parity.to_dev(logits_in)
    res = None
    if residual:
        res = parity.to_dev(synth.activations(spec, T, spec.seed + 55))
    outs = {}
    for name in ("fused", "separate"):
        bufs = binding.LayerBuffers(T, H, spec.I, spec.E, spec.K, act)
        for t in (bufs.logits, bufs.topk_w, bufs.out):
            t.fill_(float("nan"))
        for t in (bufs.topk_ids, bufs.offsets, bufs.sorted_slots, bufs.slot_pos):
            t.fill_(-1)
        out_act = torch.full((T, H), float("nan"), dtype=res.dtype, device="cuda") if residual else None
        if name == "fused":
            binding.moe_layer_decode(d["x"], d["wr"], d["gu"], d["dn"], spec.K, expert_scale=d["sc"],
                                     logit_bias=d["bias"], bufs=bufs, logits_in=li,
                                     out_act=out_act, residual=res)
            torch.cuda.synchronize()
            # the one-token one-launch path's completion counter and timeout flag
            ctr = bufs.ws_decode[:8].view(torch.int32).cpu().numpy()
            assert ctr[1] == 0, "the down workgroups timed out waiting for gate/up"
        else:
            binding.moe_layer(d["x"], d["wr"], d["gu"], d["dn"], spec.K, expert_scale=d["sc"],
                              logit_bias=d["bias"], bufs=bufs, logits_in=li, out_act=out_act,
                              residual=res, fused_route=True)
        torch.cuda.synchronize()
        g = {k: getattr(bufs, k).cpu().numpy() for k in ROUTE_KEYS + ("out",)}
        if residual:
            g["out_act"] = out_act.view(torch.int16).cpu().numpy()
        outs[name] = g
    return outs


def _assert_bitwise(outs):
    a, b = outs["fused"], outs["separate"]
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), "%s differs" % k


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_decode_layer_parity_and_bitwise(T, act):
    base = synth.SPECS[1] if act == "f32" else synth.SPECS[2]
    spec = synth.LayerSpec(**{**base.__dict__, "T": T, "name": "decode-layer-T%d-%s" % (T, act)})
    L = synth.make_layer(spec, seed=700 + T)
    print("case: decode layer T=%d %s" % (T, act), flush=True)
    outs = _run_both(L, residual=(T == 3))
    _assert_bitwise(outs)
    g = dict(outs["fused"])
    res = parity.check_layer(L, g, check_y=False)
    print("  ->", res, flush=True)


def test_decode_layer_injected_logits_bitwise():
    spec = synth.SPECS[2]
    L = synth.make_layer(spec, seed=711)
    lg = synth.uniform_logits(spec.T, spec.E, spec.seed)
    print("case: decode layer injected logits", flush=True)
    outs = _run_both(L, logits_in=lg)
    _assert_bitwise(outs)
    parity.check_layer(L, dict(outs["fused"]), logits_in=lg, check_y=False)


@pytest.mark.parametrize("H,I,E,K,T,act", [
    (256, 64, 8, 2, 1, "f32"),       # one token, a shape outside the one-launch path
    (256, 64, 8, 2, 4, "f32"),       # one block pair per down row
    (384, 192, 16, 16, 4, "bf16"),   # K = 16 (64 slots), odd pair counts
    (512, 128, 32, 4, 7, "bf16"),
])
def test_decode_layer_other_shapes(H, I, E, K, T, act):
    spec = synth.LayerSpec("decode-layer-H%d-I%d-E%d-K%d-T%d" % (H, I, E, K, T), H=H, E=E, K=K, I=I,
                           T=T, act=act, router_std=1 / np.sqrt(H), seed=13)
    L = synth.make_layer(spec)
    print("case: decode layer %s" % spec.name, flush=True)
    outs = _run_both(L, residual=True)
    _assert_bitwise(outs)
    parity.check_layer(L, dict(outs["fused"]), check_y=False)


def test_decode_layer_rejects_unsupported_shapes():
    from sparse_moe_amd import binding
    spec = synth.SPECS[2]
    L = synth.make_layer(spec, T=9)
    d = _dev_layer(L)
    with pytest.raises(binding.MoEError, match="MOE_ERR_UNSUPPORTED"):
        binding.moe_layer_decode(d["x"], d["wr"], d["gu"], d["dn"], spec.K, expert_scale=d["sc"])


@pytest.mark.parametrize("T", [1, 4])
def test_decode_stack_graph_replays_equal_eager(T):
    # 30 decode layers (RMSNorm -> layer -> residual, bf16 stream) with distinct
    # weights: a seeded layer and copies with its experts stored in other orders
    from sparse_moe_amd import binding
    spec = synth.SPECS[4]
    H, E, K, I, nl = spec.H, spec.E, spec.K, spec.I, spec.layers
    L = synth.make_layer(spec, seed=synth.stack_layer_seed(0), with_x=False)
    base = _dev_layer(synth.LayerInputs(spec, 0, np.zeros((0, H), np.uint16), L.w_router,
                                        L.router_bias, L.w_gate_up, L.w_down, L.expert_scale))
    rms_w = parity.to_dev(L.rms_w)
    gen = torch.Generator().manual_seed(5)
    layers = []
    for i in range(nl):
        perm = torch.randperm(E, generator=gen).cuda()
        layers.append({k: base[k].index_select(0, perm).contiguous() for k in ("wr", "gu", "dn", "sc", "bias")})
    x0 = parity.to_dev(synth.activations(spec, T, 77))
    xa, xb, xhat = x0.clone(), torch.empty_like(x0), torch.empty_like(x0)
    bufs = binding.LayerBuffers(T, H, I, E, K, torch.bfloat16)

    def stack():
        xin, xout = xa, xb
        xin.copy_(x0)
        for w in layers:
            binding.moe_rmsnorm(xin, rms_w, spec.rms_eps, xhat)
            binding.moe_layer_decode(xhat, w["wr"], w["gu"], w["dn"], K, expert_scale=w["sc"],
                                     logit_bias=w["bias"], bufs=bufs, out_act=xout, residual=xin,
                                     out_f32=False)
            xin, xout = xout, xin
        return xin

    print("case: 30-layer decode graph T=%d" % T, flush=True)
    final = stack()
    torch.cuda.synchronize()
    eager = final.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        stack()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gfinal = stack()
    for rep in range(4):
        final.fill_(0)
        xb.add_(1)                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gfinal, eager), "graph replay %d differs from the eager stack" % rep
    assert torch.isfinite(eager.float()).all()
