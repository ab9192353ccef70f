"""Stack workload: 30 routed-MoE layers over a 512-token bf16 chunk, each
preceded by RMSNorm and followed by the residual add, with a Zipf(1.1) prior on
the router and independently seeded weights per layer.

Every layer runs on the GPU through the C ABI.  On a spread of layers the
GPU's result is compared with the oracle fed the GPU's own layer input
(teacher forcing): the normalised activations within one bf16 rounding, the
routing bit-exactly (near-tie rule), the expert outputs and the combined output
within the fp32 bar on sampled tokens, and the residual output as the RNE
rounding of (input + combined output)."""
import numpy as np
import pytest
import torch

import oracle
import parity
from sparse_moe_amd import synth

pytestmark = pytest.mark.gpu

CHECK_LAYERS = (0, 1, 7, 14, 22, 29)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    return synth.f32_to_bf16_bits(v.astype(np.float32))


def test_stack_30_layers_teacher_forced():
    from sparse_moe_amd import binding
    spec = synth.SPECS[4]
    T, H, E, K, I = spec.T, spec.H, spec.E, spec.K, spec.I
    x = parity.to_dev(synth.activations(spec, T, spec.seed))
    xhat = torch.empty_like(x)
    xnext = torch.empty_like(x)
    bufs = binding.LayerBuffers(T, H, I, E, K, torch.bfloat16)
    pick = np.random.default_rng(44)
    hit = []
    for layer in range(spec.layers):
        L = synth.make_layer(spec, seed=synth.stack_layer_seed(layer), with_x=False)
        rms_w = parity.to_dev(L.rms_w)
        binding.moe_rmsnorm(x, rms_w, spec.rms_eps, xhat)
        binding.moe_layer(xhat, parity.to_dev(L.w_router), parity.to_dev(L.w_gate_up),
                          parity.to_dev(L.w_down), K, expert_scale=parity.to_dev(L.expert_scale),
                          logit_bias=parity.to_dev(L.router_bias), bufs=bufs, residual=x,
                          out_act=xnext)
        torch.cuda.synchronize()
        counts = np.diff(bufs.offsets.cpu().numpy())
        hit.append(int((counts > 0).sum()))
        if layer in CHECK_LAYERS:
            print("stack layer %d: experts hit %d, largest %d" % (layer, hit[-1], counts.max()),
                  flush=True)
            x_in = x.view(torch.int16).cpu().numpy().view(np.uint16)
            xh = xhat.view(torch.int16).cpu().numpy().view(np.uint16)
            # RMSNorm: within one bf16 rounding of the oracle's (RNE from fp64 vs from fp32)
            ref_hat = oracle.rmsnorm(x_in, L.rms_w, spec.rms_eps)
            a, b = bf16_to_f32(xh), bf16_to_f32(ref_hat)
            assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-30), "rmsnorm differs"
            assert np.mean(xh != ref_hat) < 1e-3
            # the layer, teacher-forced at the GPU's normalised input
            L.x = xh
            g = {k: getattr(bufs, k).cpu().numpy() for k in
                 ("logits", "topk_ids", "topk_w", "offsets", "sorted_slots", "slot_pos",
                  "y_sorted", "out")}
            # sampled tokens: random ones plus one routed to the busiest expert
            busy = int(np.argmax(counts))
            ss = g["sorted_slots"]
            t_busy = int(ss[g["offsets"][busy]] // K)
            sample = np.unique(np.concatenate([pick.choice(T, 3, replace=False), [t_busy]]))
            res = parity.check_layer(L, g, token_sample=sample)
            print("  ->", res, flush=True)
            # residual: x_next = RNE(x + out) with out the fp32 combined output
            xn = xnext.view(torch.int16).cpu().numpy().view(np.uint16)
            want = f32_to_bf16_rne(bf16_to_f32(x_in) + g["out"])
            assert np.array_equal(xn[sample], want[sample]), "residual add differs"
        x, xnext = xnext, x
    # the Zipf prior concentrates tokens: far fewer than 128 experts per layer
    assert max(hit) < 128 and min(hit) > 8
    xf = bf16_to_f32(x.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.all(np.isfinite(xf))
