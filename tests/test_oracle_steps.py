"""Pins of the oracle's layer steps against library routines, closed forms and
brute force on small inputs (router matmul, softmax/top-k, stable sort,
dequantised dense matmuls, RMSNorm), plus invariants."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from sparse_moe_amd import synth


# ---- helpers independent of the oracle -------------------------------------
def act_to_f64(x: np.ndarray) -> np.ndarray:
    """Decode activations with library conversions (numpy / torch)."""
    if x.dtype == np.float32:
        return x.astype(np.float64)
    return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double().numpy()


def dequant_q4_0(q: np.ndarray) -> np.ndarray:
    """Dense fp64 matrices from Q4_0 bytes [..., rows, nb, 18] -> [..., rows, nb*32].
    (The element order is the one the golden blocks pin.)"""
    d = q[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    qs = q[..., 2:].astype(np.int64)
    lo = (qs & 15) - 8
    hi = (qs >> 4) - 8
    vals = np.concatenate([lo, hi], axis=-1).astype(np.float64) * d[..., None]
    return vals.reshape(*q.shape[:-2], q.shape[-2] * 32)


def test_dequant_helper_matches_golden():
    from test_oracle_formats import _golden_blocks
    for name, blk, exp in _golden_blocks():
        got = dequant_q4_0(blk.reshape(1, 1, 18))[0]
        assert np.array_equal(got, exp), name


def tiny(T=4, seed=0, **kw):
    spec = synth.SPECS[0]
    if kw:
        spec = synth.LayerSpec(**{**spec.__dict__, **kw})
    return synth.make_layer(spec, seed=seed, T=T)


# ---- router -----------------------------------------------------------------
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_router_logits_equal_dense_matmul(act):
    L = tiny(T=9, act=act)
    x = act_to_f64(L.x)
    g = np.random.default_rng(3)
    rs = (1 + 0.1 * g.standard_normal(L.spec.H)).astype(np.float32)
    bias = g.standard_normal(L.spec.E).astype(np.float32)
    ref = (x * rs.astype(np.float64)) @ L.w_router.astype(np.float64).T + bias.astype(np.float64)
    got = oracle.router_logits(L.x, L.w_router, r_scale=rs, bias=bias)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    got0 = oracle.router_logits(L.x, L.w_router)
    np.testing.assert_allclose(got0, x @ L.w_router.astype(np.float64).T, rtol=1e-12, atol=1e-12)


def test_router_logits_gemma_shape_subset():
    spec = synth.SPECS[1]
    L = synth.make_layer(spec, T=3)
    ref = act_to_f64(L.x) @ L.w_router.astype(np.float64).T
    np.testing.assert_allclose(oracle.router_logits(L.x, L.w_router), ref, rtol=1e-11, atol=1e-11)


# ---- softmax / top-k --------------------------------------------------------
def test_topk_is_first_k_of_stable_sort_and_weights_are_selected_softmax():
    g = np.random.default_rng(5)
    for E, K in [(8, 2), (128, 8), (16, 16), (256, 16), (5, 1)]:
        l = g.standard_normal((40, E))
        ids, w = oracle.topk_softmax(l, K)
        order = np.argsort(-l, axis=1, kind="stable")[:, :K]
        assert np.array_equal(ids, order)
        ref_w = scipy.special.softmax(np.take_along_axis(l, order, 1), axis=1)
        np.testing.assert_allclose(w, ref_w, rtol=1e-12, atol=1e-15)
        assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-12)
        # weights descend with the logits
        assert np.all(np.diff(w, axis=1) <= 0)


def test_topk_softmax_sums_to_one_full_and_k_equals_e():
    g = np.random.default_rng(6)
    l = g.standard_normal((10, 12)) * 5
    ids, w = oracle.topk_softmax(l, 12)
    assert np.array_equal(ids, np.argsort(-l, axis=1, kind="stable"))
    np.testing.assert_allclose(w, np.take_along_axis(scipy.special.softmax(l, axis=1), ids, 1),
                               rtol=1e-12)
    assert np.all(np.abs(w.sum(1) - 1) <= 1e-12)


def test_topk_ties_lower_index_first():
    l = np.zeros((1, 8))
    ids, w = oracle.topk_softmax(l, 3)
    assert ids.tolist() == [[0, 1, 2]] and np.allclose(w, 1 / 3, rtol=0, atol=1e-15)
    l = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0]])
    ids, _ = oracle.topk_softmax(l, 4)
    assert ids.tolist() == [[1, 2, 4, 3]]


# ---- permutation ------------------------------------------------------------
@pytest.mark.parametrize("T,K,E", [(0, 2, 8), (1, 8, 128), (7, 2, 8), (64, 8, 128), (33, 1, 3),
                                   (100, 4, 1)])
def test_permute_equals_stable_argsort(T, K, E):
    g = np.random.default_rng(T * 1000 + K * 10 + E)
    ids = g.integers(0, E, size=(T, K)).astype(np.int32)
    off, ss, sp = oracle.permute(ids, E)
    flat = ids.ravel()
    assert np.array_equal(ss, np.argsort(flat, kind="stable").astype(np.int32))
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    assert off[-1] == T * K
    assert np.array_equal(sp[ss], np.arange(T * K))
    for e in range(E):
        seg = ss[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# ---- expert FFN -------------------------------------------------------------
def ffn_dense(x64, gu, dn, e, act):
    """Dense reference of one expert with torch fp64 ops (library GELU)."""
    I = gu.shape[1] // 2
    Wgu = dequant_q4_0(gu[e])              # [2I, H]
    Wd = dequant_q4_0(dn[e])               # [H, I]
    g = x64 @ Wgu[:I].T
    u = x64 @ Wgu[I:].T
    h = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy() * u
    if act == "f32":
        h = h.astype(np.float32).astype(np.float64)
    return h, h @ Wd.T


def test_expert_ffn_token_equals_dense_f32():
    L = tiny(T=3)
    x64 = act_to_f64(L.x)
    for t in range(3):
        for e in range(L.spec.E):
            h, y = oracle.expert_ffn_token(L.x[t], L.w_gate_up, L.w_down, e)
            hr, yr = ffn_dense(x64[t], L.w_gate_up, L.w_down, e, "f32")
            np.testing.assert_allclose(h, hr, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(y, yr, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_linear_q4_0_equals_dense_matmul(act):
    # the plain Q4_0 linear layer against whole-matrix decoding and a numpy fp64
    # matmul; ragged row count, several tokens
    L = tiny(T=3)
    rng = np.random.default_rng(9)
    w = L.w_down[1][:37]                         # 37 rows of 2 blocks (H = 64)
    H = w.shape[1] * 32
    x = rng.standard_normal((4, H)).astype(np.float32)
    if act == "bf16":
        x = synth.f32_to_bf16_bits(x)
    y = oracle.linear_q4_0(x, w)
    ref = act_to_f64(x) @ dequant_q4_0(w).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # a single non-zero weight block picks out d * (q - 8) . x of its 32 elements
    w1 = np.zeros((2, H // 32, 18), np.uint8)
    w1[1, 1, 0:2] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    w1[1, 1, 2:] = 0x9A                           # low nibble 10, high nibble 9
    y1 = oracle.linear_q4_0(x, w1)
    xs = act_to_f64(x)[:, 32:64]
    np.testing.assert_allclose(y1[:, 0], 0.0, atol=0)
    np.testing.assert_allclose(y1[:, 1], 0.5 * (2 * xs[:, :16].sum(1) + 1 * xs[:, 16:].sum(1)),
                               rtol=1e-12, atol=1e-12)


def test_expert_ffn_token_bf16_hidden_rounding():
    L = tiny(T=2, act="bf16")
    x64 = act_to_f64(L.x)
    for e in range(L.spec.E):
        h, y = oracle.expert_ffn_token(L.x[0], L.w_gate_up, L.w_down, e)
        hr, _ = ffn_dense(x64[0], L.w_gate_up, L.w_down, e, "none")
        # h is bf16: each value is exactly representable and within half an ulp (<= 2^-8 rel)
        hb = torch.from_numpy(h).float().to(torch.bfloat16).double().numpy()
        assert np.array_equal(hb, h)
        assert np.all(np.abs(h - hr) <= np.abs(hr) * 2.0 ** -8 + 1e-30)
        # y is the dense down product of exactly that h
        Wd = dequant_q4_0(L.w_down[e])
        np.testing.assert_allclose(y, h @ Wd.T, rtol=1e-10, atol=1e-12)


def test_expert_ffn_closed_forms():
    L = tiny(T=1)
    H, I = L.spec.H, L.spec.I
    zero = np.zeros(H, np.float32)
    h, y = oracle.expert_ffn_token(zero, L.w_gate_up, L.w_down, 3)
    assert np.all(h == 0) and np.all(y == 0)
    # unit vector e_j: g_i = Wg[i,j], u_i = Wu[i,j] -> h_i = gelu(Wg[i,j]) Wu[i,j]
    e = 5
    Wgu = dequant_q4_0(L.w_gate_up[e])
    Wd = dequant_q4_0(L.w_down[e])
    for j in (0, 17, 31, 32, H - 1):
        x = np.zeros(H, np.float32)
        x[j] = 1.0
        h, y = oracle.expert_ffn_token(x, L.w_gate_up, L.w_down, e)
        g, u = Wgu[:I, j], Wgu[I:, j]
        c = np.sqrt(2 / np.pi)
        href = (0.5 * g * (1 + np.tanh(c * (g + 0.044715 * g ** 3))) * u).astype(np.float32)
        np.testing.assert_allclose(h, href, rtol=1e-6, atol=0)
        np.testing.assert_allclose(y, Wd @ h, rtol=1e-12, atol=1e-14)


def test_expert_ffn_sorted_layout_matches_per_token():
    L = tiny(T=6)
    K = L.spec.K
    ids = np.random.default_rng(2).integers(0, L.spec.E, size=(6, K)).astype(np.int32)
    off, ss, sp = oracle.permute(ids, L.spec.E)
    y = oracle.expert_ffn(L.x, L.w_gate_up, L.w_down, K, off, ss)
    for p in range(6 * K):
        s = ss[p]
        _, yr = oracle.expert_ffn_token(L.x[s // K], L.w_gate_up, L.w_down, ids.ravel()[s])
        assert np.array_equal(y[p], yr)


# ---- combine ----------------------------------------------------------------
def test_combine_k1_and_linearity():
    g = np.random.default_rng(9)
    T, K, H, E = 5, 3, 64, 6
    ids = g.integers(0, E, size=(T, K)).astype(np.int32)
    off, ss, sp = oracle.permute(ids, E)
    y = g.standard_normal((T * K, H))
    w = scipy.special.softmax(g.standard_normal((T, K)), axis=1)
    sc = (1 + 0.1 * g.standard_normal(E)).astype(np.float32)
    out = oracle.combine(y, sp, ids, w, sc)
    ref = np.einsum("tk,tkh->th", w * sc.astype(np.float64)[ids], y[sp.reshape(T, K)])
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
    # linearity in y
    y2 = g.standard_normal((T * K, H))
    out2 = oracle.combine(y2, sp, ids, w, sc)
    out12 = oracle.combine(2 * y - 3 * y2, sp, ids, w, sc)
    np.testing.assert_allclose(out12, 2 * out - 3 * out2, rtol=1e-12, atol=1e-12)
    # K = 1: out = s_e * y (w = 1)
    ids1 = ids[:, :1].copy()
    off1, ss1, sp1 = oracle.permute(ids1, E)
    y1 = g.standard_normal((T, H))
    out1 = oracle.combine(y1, sp1, ids1, np.ones((T, 1)), sc)
    np.testing.assert_allclose(out1, sc.astype(np.float64)[ids1[:, 0], None] * y1[sp1], rtol=1e-15)


# ---- whole layer against an independent torch fp64 composition -------------
def torch_layer(L, K, logits_in=None):
    x64 = torch.from_numpy(act_to_f64(L.x))
    if logits_in is None:
        logits = x64 @ torch.from_numpy(L.w_router.astype(np.float64)).T
        if L.router_bias is not None:
            logits = logits + torch.from_numpy(L.router_bias.astype(np.float64))
    else:
        logits = torch.from_numpy(logits_in.astype(np.float64))
    p = torch.softmax(logits, dim=-1)
    top_p, top_i = torch.topk(p, K, dim=-1)          # no ties in random data
    w = top_p / top_p.sum(-1, keepdim=True)
    out = torch.zeros_like(x64)
    I = L.w_gate_up.shape[1] // 2
    for e in range(L.w_gate_up.shape[0]):
        Wgu = torch.from_numpy(dequant_q4_0(L.w_gate_up[e]))
        Wd = torch.from_numpy(dequant_q4_0(L.w_down[e]))
        tok, kk = torch.nonzero(top_i == e, as_tuple=True)
        if tok.numel() == 0:
            continue
        xe = x64[tok]
        h = torch.nn.functional.gelu(xe @ Wgu[:I].T, approximate="tanh") * (xe @ Wgu[I:].T)
        # h is materialised in the activation type (fp32, or bf16 via fp32)
        h = h.float().double() if L.x.dtype == np.float32 else h.float().to(torch.bfloat16).double()
        y = h @ Wd.T
        c = w[tok, kk] * float(1) * torch.from_numpy(L.expert_scale.astype(np.float64))[e]
        out.index_add_(0, tok, c[:, None] * y)
    return logits.numpy(), top_i.numpy(), w.numpy(), out.numpy()


def test_tiny_layer_against_torch_composition():
    L = tiny()
    K = L.spec.K
    r = oracle.moe_layer(L.x, L.w_router, L.w_gate_up, L.w_down, K, scale=L.expert_scale)
    logits, ids, w, out = torch_layer(L, K)
    np.testing.assert_allclose(r["logits"], logits, rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["ids"], ids)
    np.testing.assert_allclose(r["w"], w, rtol=1e-12)
    scale = np.abs(out).max()
    assert np.abs(r["out"] - out).max() <= 1e-10 * scale


def test_layer_step_functions_compose_to_layer():
    L = tiny(T=5)
    K = L.spec.K
    r = oracle.moe_layer(L.x, L.w_router, L.w_gate_up, L.w_down, K, scale=L.expert_scale)
    logits = oracle.router_logits(L.x, L.w_router)
    ids, w = oracle.topk_softmax(logits, K)
    off, ss, sp = oracle.permute(ids, L.spec.E)
    y = oracle.expert_ffn(L.x, L.w_gate_up, L.w_down, K, off, ss)
    out = oracle.combine(y, sp, ids, w, L.expert_scale)
    assert np.array_equal(r["ids"], ids) and np.array_equal(r["offsets"], off)
    assert np.array_equal(r["sorted_slots"], ss) and np.array_equal(r["slot_pos"], sp)
    assert np.array_equal(r["out"], out)


def test_injected_logits_mode_and_token_mask():
    L = tiny(T=6)
    K = L.spec.K
    lg = synth.uniform_logits(6, L.spec.E, 11)
    mask = np.array([1, 0, 1, 0, 0, 1], np.uint8)
    r = oracle.moe_layer(L.x, None, L.w_gate_up, L.w_down, K, scale=L.expert_scale,
                         logits_in=lg, token_mask=mask)
    _, ids, w, out = torch_layer(L, K, logits_in=lg)
    assert np.array_equal(r["ids"], ids)
    sel = mask.astype(bool)
    assert np.abs(r["out"][sel] - out[sel]).max() <= 1e-10 * np.abs(out).max()
    assert np.all(np.isnan(r["out"][~sel]))


# ---- RMSNorm / stack ----------------------------------------------------------
def test_rmsnorm_against_torch():
    g = np.random.default_rng(4)
    x = synth.f32_to_bf16_bits(g.standard_normal((7, 256)).astype(np.float32) * 3)
    w = (1 + 0.05 * g.standard_normal(256)).astype(np.float32)
    got = oracle.rmsnorm(x, w, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(act_to_f64(x)), (256,),
                                       weight=torch.from_numpy(w.astype(np.float64)), eps=1e-6)
    refb = ref.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # direct fp64 -> bf16 rounding vs torch's fp64 -> fp32 -> bf16: equal except for
    # double-rounding ties, which are one ulp apart
    diff = np.abs(got.astype(np.int32) - refb.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 1e-3
    # zero rows stay zero (eps keeps the scale finite)
    z = oracle.rmsnorm(np.zeros((1, 256), np.uint16), w, 1e-6)
    assert np.all(z == 0)


# ---- residual add and one block of the stack ----------------------------------
def _bf16_table():
    """Every finite bf16 value (decoded by torch) with its bit pattern, ascending;
    -0 left out so that each value appears once."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = act_to_f64(bits)
    keep = np.isfinite(vals) & (bits != 0x8000)
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], bits[keep][order]


def nearest_even_bf16(s: np.ndarray) -> np.ndarray:
    """Brute force: the bf16 nearest to each binary64 s, ties to the even pattern."""
    vals, bits = _bf16_table()
    i = np.clip(np.searchsorted(vals, s), 1, vals.size - 1)
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = s - lo, hi - s
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((bits[i] & 1) == 0))
    return np.where(pick_hi, bits[i], bits[i - 1]).astype(np.uint16)


def test_residual_is_nearest_even_bf16():
    g = np.random.default_rng(21)
    T, H = 12, 96
    x = synth.f32_to_bf16_bits((g.standard_normal((T, H)) * 2).astype(np.float32))
    out = g.standard_normal((T, H)) * np.exp(g.uniform(-12, 3, size=(T, H)))
    xv = act_to_f64(x)
    # exact ties: out = half a bf16 ulp of x (with x's sign), so x + out lies
    # halfway between two bf16 values
    ulp = np.ldexp(1.0, np.frexp(np.abs(xv))[1] - 8)
    out[0] = np.sign(xv[0]) * ulp[0] / 2
    out[1] = -np.sign(xv[1]) * ulp[1] / 4
    got = oracle.residual(x, out)
    assert np.array_equal(got, nearest_even_bf16(xv + out))
    # out = 0 keeps x; x = 0 gives the rounding of out
    assert np.array_equal(oracle.residual(x, np.zeros((T, H))), x)
    z = np.zeros((T, H), np.uint16)
    assert np.array_equal(oracle.residual(z, out), nearest_even_bf16(out))
    # masked rows are untouched
    m = np.zeros(T, np.uint8)
    m[3] = 1
    r = oracle.residual(x, out, token_mask=m)
    assert np.array_equal(r[3], got[3]) and not r[np.arange(T) != 3].any()


def stack_spec(T=5):
    base = synth.SPECS[4]
    return synth.LayerSpec(**{**base.__dict__, "H": 256, "E": 8, "K": 2, "I": 64, "T": T,
                              "router_std": 1 / 16, "name": "tiny-stack"})


def test_stack_layer_composes_norm_layer_residual():
    spec = stack_spec()
    L = synth.make_layer(spec, seed=31)
    r = oracle.stack_layer(L.x, L.rms_w, spec.rms_eps, L.w_router, L.w_gate_up, L.w_down, spec.K,
                           scale=L.expert_scale, bias=L.router_bias)
    xhat = oracle.rmsnorm(L.x, L.rms_w, spec.rms_eps)
    lay = oracle.moe_layer(xhat, L.w_router, L.w_gate_up, L.w_down, spec.K, scale=L.expert_scale,
                           bias=L.router_bias)
    assert np.array_equal(r["xhat"], xhat)
    assert np.array_equal(r["ids"], lay["ids"])
    assert np.array_equal(r["out"], lay["out"])
    assert np.array_equal(r["x_next"], oracle.residual(L.x, lay["out"]))


def test_stack_layer_against_torch_composition():
    spec = stack_spec(T=6)
    L = synth.make_layer(spec, seed=33)
    r = oracle.stack_layer(L.x, L.rms_w, spec.rms_eps, L.w_router, L.w_gate_up, L.w_down, spec.K,
                           scale=L.expert_scale, bias=L.router_bias)
    x64 = torch.from_numpy(act_to_f64(L.x))
    xh = torch.nn.functional.rms_norm(x64, (spec.H,), weight=torch.from_numpy(
        L.rms_w.astype(np.float64)), eps=spec.rms_eps)
    xhb = xh.float().to(torch.bfloat16)
    L2 = synth.LayerInputs(spec, spec.T, xhb.view(torch.int16).numpy().view(np.uint16).copy(),
                           L.w_router, L.router_bias, L.w_gate_up, L.w_down, L.expert_scale)
    _, ids, _, out = torch_layer(L2, spec.K)
    xn = (x64 + torch.from_numpy(out)).float().to(torch.bfloat16)
    xn = xn.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(r["ids"], ids)
    # torch rounds fp64 -> fp32 -> bf16, the oracle fp64 -> bf16 once: equal
    # except for double-rounding ties, one ulp apart
    diff = np.abs(r["x_next"].astype(np.int32) - xn.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 1e-2


def test_stack_layer_degenerate_inputs():
    spec = stack_spec(T=3)
    L = synth.make_layer(spec, seed=35)
    # x = 0: the norm stays finite (eps), the experts see zeros, so x stays 0
    z = np.zeros_like(L.x)
    r = oracle.stack_layer(z, L.rms_w, spec.rms_eps, L.w_router, L.w_gate_up, L.w_down, spec.K,
                           scale=L.expert_scale, bias=L.router_bias)
    assert not r["xhat"].any() and not r["x_next"].any() and np.all(r["out"] == 0)
    # zero expert scales d: every expert weight is 0, so the block returns x
    gu, dn = L.w_gate_up.copy(), L.w_down.copy()
    gu[..., 0:2] = 0
    dn[..., 0:2] = 0
    r = oracle.stack_layer(L.x, L.rms_w, spec.rms_eps, L.w_router, gu, dn, spec.K,
                           scale=L.expert_scale, bias=L.router_bias)
    assert np.array_equal(r["x_next"], L.x)
