"""Pins of the oracle's number formats and of its Q4_0 block decode.

fp16 / bf16 decoding is checked exhaustively against numpy's float16 and
torch's bfloat16 (library routines); bf16 encoding against torch's fp32 ->
bf16 conversion and against hand-worked ties; the Q4_0 decode against the
hand-built blocks in tests/golden/q4_0_blocks.txt and against identities.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_0_blocks.txt")


def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    # sign of zero
    assert math.copysign(1.0, oracle.f16_to_f64(0x8000)) == -1.0
    # inf / nan scales are flagged as non-finite
    assert math.isinf(oracle.f16_to_f64(0x7C00)) and math.isnan(oracle.f16_to_f64(0x7E00))


def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_encode_matches_torch_on_fp32_values():
    g = np.random.default_rng(1234)
    vals = np.concatenate([
        g.standard_normal(20000).astype(np.float32),
        (g.standard_normal(5000) * 1e-38).astype(np.float32),   # subnormal range
        np.clip(g.standard_normal(5000) * 1e38, -3.4e38, 3.4e38).astype(np.float32),  # near overflow
        # exact midpoints between neighbouring bf16 values (ties -> even)
        (np.arange(1, 5001, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38, 3.4028235e38, 1e-45, -1e-45],
                 dtype=np.float32),
    ])
    ref = _torch_bf16_bits(vals)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_encode_binary64_cases_by_hand():
    # 1 + 2^-8 is the midpoint of 1.0 (0x3F80) and 1 + 2^-7 (0x3F81): ties to even
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    # a hair above the midpoint (not representable in fp32) rounds up
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    # a hair below rounds down
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 - 2.0 ** -40) == 0x3F80
    # 1 + 3*2^-8 is the midpoint of 0x3F81 and 0x3F82: ties to the even 0x3F82
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.f64_to_bf16(-2.5) == 0xC020
    assert oracle.f64_to_bf16(float("inf")) == 0x7F80
    assert oracle.f64_to_bf16(1e39) == 0x7F80            # overflow
    assert oracle.f64_to_bf16(2.0 ** -133) == 0x0001     # smallest subnormal
    assert oracle.f64_to_bf16(2.0 ** -134) == 0x0000     # tie with zero -> even (zero)
    assert oracle.f64_to_bf16(2.0 ** -126) == 0x0080     # smallest normal
    assert (oracle.f64_to_bf16(float("nan")) & 0x7FFF) > 0x7F80


def _golden_blocks():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, rest = line.split(":", 1)
            hexes, vals = rest.split("|")
            blk = np.array([int(h, 16) for h in hexes.split()], dtype=np.uint8)
            exp = np.array([float(v) for v in vals.split()], dtype=np.float64)
            assert blk.size == 18 and exp.size == 32, name
            out.append((name, blk, exp))
    return out


@pytest.mark.parametrize("name,blk,exp", _golden_blocks(), ids=lambda v: v if isinstance(v, str) else "")
def test_q4_0_golden_blocks(name, blk, exp):
    got = oracle.q4_0_decode(blk)
    assert np.array_equal(got, exp), (name, got, exp)


def test_q4_0_identities():
    g = np.random.default_rng(7)
    for _ in range(50):
        dbits = np.float16(abs(g.standard_normal()) * 0.02).view(np.uint16)
        d = float(np.uint16(dbits).view(np.float16))
        lohi = [int(dbits) & 0xFF, int(dbits) >> 8]
        # all codes 8 -> zero
        assert np.all(oracle.q4_0_decode(np.array(lohi + [0x88] * 16, np.uint8)) == 0.0)
        # all codes 0 -> -8 d ; all codes 15 -> 7 d
        assert np.all(oracle.q4_0_decode(np.array(lohi + [0x00] * 16, np.uint8)) == -8 * d)
        assert np.all(oracle.q4_0_decode(np.array(lohi + [0xFF] * 16, np.uint8)) == 7 * d)
        # a single non-8 nibble lands on element j (low) or j+16 (high) only
        j = int(g.integers(16))
        q = int(g.integers(16))
        qs = [0x88] * 16
        qs[j] = 0x80 | q
        v = oracle.q4_0_decode(np.array(lohi + qs, np.uint8))
        want = np.zeros(32)
        want[j] = (q - 8) * d
        assert np.array_equal(v, want)
        qs[j] = (q << 4) | 0x08
        v = oracle.q4_0_decode(np.array(lohi + qs, np.uint8))
        want = np.zeros(32)
        want[j + 16] = (q - 8) * d
        assert np.array_equal(v, want)
    # d = 1.0: the codes decode to the integers -8..7
    for q in range(16):
        v = oracle.q4_0_decode(np.array([0x00, 0x3C] + [q | (q << 4)] * 16, np.uint8))
        assert np.all(v == q - 8)


def test_gelu_tanh_against_torch_and_identities():
    z = np.concatenate([np.linspace(-12, 12, 2001), [0.0, 1e-300, -1e-300, 40.0, -40.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    got = np.array([oracle.gelu_tanh(float(v)) for v in z])
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu_tanh(0.0) == 0.0
    # gelu(z) - gelu(-z) = z for the tanh form (tanh is odd)
    for v in np.linspace(-6, 6, 97):
        assert abs((oracle.gelu_tanh(v) - oracle.gelu_tanh(-v)) - v) <= 1e-14 * max(1.0, abs(v))
    assert abs(oracle.gelu_tanh(40.0) - 40.0) < 1e-12 and abs(oracle.gelu_tanh(-40.0)) < 1e-12
