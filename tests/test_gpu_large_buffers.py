"""Activation buffers of 2 GiB and more on the grouped-GEMM (MFMA) path.

Below 2 GiB the grouped GEMM's direct loads are buffer loads with 32-bit lane
offsets; from 2 GiB on they take 64-bit addresses.  These cases put a bf16
activation buffer just over 2 GiB through the gate/up product (the expert FFN
with 262,240 tokens at H = 4096) and through the down-product kernel (the plain
Q4_0 linear layer at the same size), and compare sampled rows, including rows
that lie past the first 2 GiB, with the oracle token by token.  The tokens are
1,024 seeded rows repeated, so the oracle needs only those rows.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
from sparse_moe_amd import synth

pytestmark = pytest.mark.gpu

H = 4096
T = (1 << 31) // (2 * H) + 96   # bf16 activations just over 2 GiB
BASE = 1024                     # distinct token rows


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs():
    spec = synth.LayerSpec("large", H=H, E=2, K=1, I=64, T=BASE, act="bf16", router_std=0.1,
                           seed=41)
    xs = synth.activations(spec, BASE, spec.seed + 5)          # bf16 bits [BASE, H]
    x = parity.to_dev(xs)
    xb = x.repeat((T + BASE - 1) // BASE, 1)[:T].contiguous()  # row t = row t % BASE
    assert xb.numel() * 2 >= (1 << 31)
    return xs, xb


def _sample():
    # first rows, the middle, and rows whose bytes start past 2 GiB
    past = (1 << 31) // (2 * H)
    return np.unique(np.array([0, 1, BASE - 1, T // 2, past, past + 33, T - 2, T - 1]))


def test_linear_over_2gib():
    from sparse_moe_amd import binding
    xs, xb = _inputs()
    R = 64
    w = synth.q4_0_random(synth.rng(41, 7), 1, R, H)[0]
    print("linear T=%d H=%d R=%d" % (T, H, R), flush=True)
    y = binding.moe_linear_q4_0(xb, parity.to_dev(w))
    torch.cuda.synchronize()
    s = _sample()
    got = y[torch.from_numpy(s).cuda()].cpu().numpy()
    ref = oracle.linear_q4_0(xs[s % BASE], w)
    err = np.max(np.abs(got - ref))
    assert err <= parity.TOL * np.max(np.abs(ref)), err


def test_expert_ffn_over_2gib():
    from sparse_moe_amd import binding
    xs, xb = _inputs()
    E, K, I = 2, 1, 64
    w_gu = synth.q4_0_random(synth.rng(41, 8), E, 2 * I, H)
    w_dn = synth.q4_0_random(synth.rng(41, 9), E, H, I)
    ids = (np.arange(T) % E).astype(np.int32).reshape(T, K)
    off, ss, sp = oracle.permute(ids, E)
    y = torch.empty((T * K, H), dtype=torch.float32, device="cuda")
    nb = binding.moe_expert_ffn_q4_0_workspace_bytes(T, K, H, I, E, binding.act_dtype(xb))
    ws = torch.empty((max(16, nb),), dtype=torch.uint8, device="cuda")
    print("expert FFN T=%d H=%d I=%d E=%d" % (T, H, I, E), flush=True)
    binding.moe_expert_ffn_q4_0(xb, parity.to_dev(w_gu), parity.to_dev(w_dn), K,
                                parity.to_dev(off), parity.to_dev(ss), y, ws)
    torch.cuda.synchronize()
    s = _sample()
    got = y[torch.from_numpy(sp[s].astype(np.int64)).cuda()].cpu().numpy()
    ref = np.stack([oracle.expert_ffn_token(xs[t % BASE], w_gu, w_dn, int(t % E))[1] for t in s])
    err = np.max(np.abs(got - ref))
    assert err <= parity.TOL * np.max(np.abs(ref)), err
