"""Stack workload: 30 routed-MoE layers over a 512-token bf16 chunk, each
preceded by RMSNorm and followed by the residual add, with a Zipf(1.1) prior on
the router and independently seeded weights per layer.

Every layer runs on the GPU through the C ABI.  Every layer's GPU result is
compared with the oracle fed the GPU's own layer input (teacher forcing): the
normalised activations within one bf16 rounding, the routing of all tokens
bit-exactly (near-tie rule), the expert outputs and the combined output within
the fp32 bar on sampled tokens, and the residual output against the oracle's
residual step (bf16 of input + combined output).  Separately, a few tokens run
through all 30 oracle blocks from the same start (no teacher forcing) and the
end-to-end drift of the GPU's final activations is reported."""
import numpy as np
import pytest
import torch

import oracle
import parity
from sparse_moe_amd import synth

pytestmark = pytest.mark.gpu

SAMPLE_PER_LAYER = 5     # random tokens per layer, plus the busiest and quietest experts' tokens
DRIFT_TOKENS = 4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (8 significant bits; normal range)."""
    e = np.frexp(np.maximum(np.abs(v), 2.0 ** -126))[1]
    return np.ldexp(1.0, e - 8)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.timeout(900)
def test_stack_30_layers_teacher_forced_and_drift():
    from sparse_moe_amd import binding
    spec = synth.SPECS[4]
    T, H, E, K, I = spec.T, spec.H, spec.E, spec.K, spec.I
    x0 = synth.activations(spec, T, spec.seed)
    x = parity.to_dev(x0)
    xhat = torch.empty_like(x)
    xnext = torch.empty_like(x)
    bufs = binding.LayerBuffers(T, H, I, E, K, torch.bfloat16)
    pick = np.random.default_rng(44)
    drift_tok = np.sort(pick.choice(T, DRIFT_TOKENS, replace=False))
    x_orc = x0[drift_tok].copy()          # the oracle's own residual stream for those tokens
    diverged = 0                          # (layer, drift token) pairs routed differently
    hit = []
    for layer in range(spec.layers):
        L = synth.make_layer(spec, seed=synth.stack_layer_seed(layer), with_x=False)
        binding.moe_rmsnorm(x, parity.to_dev(L.rms_w), spec.rms_eps, xhat)
        binding.moe_layer(xhat, parity.to_dev(L.w_router), parity.to_dev(L.w_gate_up),
                          parity.to_dev(L.w_down), K, expert_scale=parity.to_dev(L.expert_scale),
                          logit_bias=parity.to_dev(L.router_bias), bufs=bufs, residual=x,
                          out_act=xnext)
        torch.cuda.synchronize()
        counts = np.diff(bufs.offsets.cpu().numpy())
        hit.append(int((counts > 0).sum()))
        x_in, xh, xn = to_bits(x), to_bits(xhat), to_bits(xnext)
        # RMSNorm: within one bf16 rounding of the oracle's (RNE from fp64 vs from fp32)
        ref_hat = oracle.rmsnorm(x_in, L.rms_w, spec.rms_eps)
        a, b = bf16_to_f64(xh), bf16_to_f64(ref_hat)
        assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-30), "rmsnorm differs"
        assert np.mean(xh != ref_hat) < 1e-3
        # the layer, teacher-forced at the GPU's normalised input; sampled tokens:
        # random ones plus the first and last token of the busiest expert and a
        # token of the quietest hit expert
        L.x = xh
        g = {k: getattr(bufs, k).cpu().numpy() for k in
             ("logits", "topk_ids", "topk_w", "offsets", "sorted_slots", "slot_pos",
              "y_sorted", "out")}
        off, ss = g["offsets"], g["sorted_slots"]
        busy = int(np.argmax(counts))
        quiet = int(np.argmin(np.where(counts > 0, counts, T * K + 1)))
        special = [ss[off[busy]] // K, ss[off[busy + 1] - 1] // K, ss[off[quiet]] // K]
        sample = np.unique(np.concatenate([pick.choice(T, SAMPLE_PER_LAYER, replace=False),
                                           special]))
        refs = {}
        res = parity.check_layer(L, g, token_sample=sample, refs=refs)
        # residual: the oracle's step on (GPU input, oracle output); the GPU adds its
        # fp32 output and rounds once, so they agree within one bf16 spacing of the
        # sum plus the output's own tolerance
        want = oracle.residual(x_in[sample], refs["out"][sample])
        out_ref = refs["out"][sample]
        bound = bf16_ulp(bf16_to_f64(want)) + parity.TOL * np.abs(out_ref).max()
        dev = np.abs(bf16_to_f64(xn[sample]) - bf16_to_f64(want))
        assert np.all(dev <= bound), "residual differs from the oracle's by %g" % dev.max()
        # and bit for bit the fp32 sum of the GPU's own input and combined output,
        # rounded to nearest even (every token)
        own = synth.f32_to_bf16_bits(
            (x_in.astype(np.uint32) << 16).view(np.float32) + g["out"].astype(np.float32))
        assert np.array_equal(xn, own), "residual is not RNE(x + out) of the GPU's own out"
        same = float(np.mean(xn[sample] == want))
        assert same > 0.95, "residual: only %.3f of the elements equal the oracle's" % same
        print("stack layer %d: experts hit %d, largest %d, y_err %.2e, out_err %.2e, "
              "residual equal %.4f" % (layer, hit[-1], counts.max(), res["y_err"],
                                       res["out_err"], same), flush=True)
        # the drift tokens through the oracle's own block (no teacher forcing)
        r = oracle.stack_layer(x_orc, L.rms_w, spec.rms_eps, L.w_router, L.w_gate_up, L.w_down,
                               K, scale=L.expert_scale, bias=L.router_bias)
        x_orc = r["x_next"]
        diverged += int((r["ids"] != g["topk_ids"][drift_tok]).any(axis=1).sum())
        x, xnext = xnext, x
    # the Zipf prior concentrates tokens: far fewer than 128 experts per layer
    assert max(hit) < 128 and min(hit) > 8
    xf = bf16_to_f64(to_bits(x))
    assert np.all(np.isfinite(xf))
    ref = bf16_to_f64(x_orc)
    drift = np.abs(xf[drift_tok] - ref).max() / np.abs(ref).max()
    rel_rms = np.sqrt(np.mean((xf[drift_tok] - ref) ** 2) / np.mean(ref ** 2))
    print("end-to-end drift over %d layers, %d tokens (GPU stack vs oracle stack from the same "
          "input): max|d|/max|ref| = %.3e, relative RMS = %.3e; layers where a drift token's "
          "experts differ: %d of %d" % (spec.layers, DRIFT_TOKENS, drift, rel_rms, diverged,
                                       spec.layers * DRIFT_TOKENS), flush=True)
    assert np.all(np.isfinite(ref))
