"""Comparison of the HIP path with the CPU oracle (test infrastructure).

Bars:
  * expert ids and permutation (offsets, sorted slots, slot positions):
    bit-exact.  A token is a near-tie when two of its K+1 largest oracle logits
    are closer than NEAR_TIE; its GPU ids are then accepted if they are a valid
    top-K within NEAR_TIE, and the oracle's downstream steps are recomputed
    with the GPU's ids so every output stays comparable.
  * fp32 outputs (expert outputs y, combined out): max|gpu - ref| <= TOL * max|ref|.
  * router logits: max|gpu - ref| <= 1e-4 * max|ref| (fp32 accumulation of an
    fp64-defined sum); top-K weights: |gpu - ref| <= 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = 2e-3
NEAR_TIE = 1e-5


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def run_gpu_layer(L, logits_in=None, bufs=None, fused_route=False):
    """Run the four C-ABI calls on the layer inputs; returns (numpy dict, bufs)."""
    from sparse_moe_amd import binding
    x = to_dev(L.x)
    wr = to_dev(L.w_router)
    gu = to_dev(L.w_gate_up)
    dn = to_dev(L.w_down)
    sc = to_dev(L.expert_scale)
    bias = None if L.router_bias is None else to_dev(L.router_bias)
    li = None if logits_in is None else to_dev(logits_in)
    bufs = binding.moe_layer(x, wr, gu, dn, L.spec.K, expert_scale=sc, logit_bias=bias,
                             logits_in=li, bufs=bufs, fused_route=fused_route)
    torch.cuda.synchronize()
    return {k: getattr(bufs, k).cpu().numpy() for k in
            ("logits", "topk_ids", "topk_w", "offsets", "sorted_slots", "slot_pos", "y_sorted",
             "out")}, bufs


def near_tie_tokens(logits: np.ndarray, K: int) -> np.ndarray:
    s = -np.sort(-logits, axis=1)[:, :K + 1]
    gaps = s[:, :-1] - s[:, 1:]
    return (gaps < NEAR_TIE).any(axis=1)


def valid_topk(logits_row: np.ndarray, ids_row: np.ndarray) -> bool:
    E = logits_row.size
    if len(set(ids_row.tolist())) != ids_row.size or ids_row.min() < 0 or ids_row.max() >= E:
        return False
    sel = logits_row[ids_row]
    rest = np.delete(logits_row, ids_row)
    if rest.size and sel.min() < rest.max() - NEAR_TIE:
        return False
    return bool(np.all(np.diff(sel) <= NEAR_TIE))


def max_rel(gpu: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.abs(ref).max())
    d = float(np.abs(gpu.astype(np.float64) - ref).max())
    return d / scale if scale > 0 else d


def check_routing(L, g: dict, logits_ref: np.ndarray):
    """ids bit-exact (near-ties: valid top-K); returns the effective ids and weights."""
    K = L.spec.K
    ids_ref, _ = oracle.topk_softmax(logits_ref, K)
    ties = near_tie_tokens(logits_ref, K)
    gid = g["topk_ids"]
    exact = ~ties
    bad = np.nonzero((gid[exact] != ids_ref[exact]).any(axis=1))[0]
    assert bad.size == 0, "expert ids differ on %d non-tie tokens, e.g. %s vs %s" % (
        bad.size, gid[exact][bad[0]], ids_ref[exact][bad[0]])
    for t in np.nonzero(ties)[0]:
        assert valid_topk(logits_ref[t], gid[t]), "token %d: invalid near-tie top-K" % t
    ids_eff = np.where(ties[:, None], gid, ids_ref).astype(np.int32)
    w_ref = oracle.topk_weights(logits_ref, ids_eff)
    dw = np.abs(g["topk_w"] - w_ref).max() if w_ref.size else 0.0
    assert dw <= 1e-5, "top-K weights differ by %g" % dw
    return ids_eff, w_ref, int(ties.sum())


def check_layer(L, g: dict, logits_in=None, token_sample=None, refs=None, check_y=True):
    """Full comparison of one layer's GPU outputs against the oracle.

    token_sample: indices of tokens whose expert outputs and combined output the
    oracle computes (None: all tokens).  refs: a dict that receives the oracle's
    combined output ("out", binary64, rows of unsampled tokens NaN) and the
    effective expert ids ("ids")."""
    K, E = L.spec.K, L.spec.E
    if logits_in is None:
        logits_ref = oracle.router_logits(L.x, L.w_router, bias=L.router_bias)
        lr = max_rel(g["logits"], logits_ref)
        assert lr <= 1e-4, "router logits rel err %g" % lr
    else:
        logits_ref = logits_in.astype(np.float64)
    ids_eff, w_ref, nties = check_routing(L, g, logits_ref)
    off, ss, sp = oracle.permute(ids_eff, E)
    assert np.array_equal(g["offsets"], off), "expert offsets differ"
    assert np.array_equal(g["sorted_slots"], ss), "sorted slots differ"
    assert np.array_equal(g["slot_pos"], sp), "slot positions differ"
    T = L.x.shape[0]
    if token_sample is None:
        tmask = np.ones(T, np.uint8)
    else:
        tmask = np.zeros(T, np.uint8)
        tmask[np.asarray(token_sample)] = 1
    smask = np.repeat(tmask, K)
    y_ref = oracle.expert_ffn(L.x, L.w_gate_up, L.w_down, K, off, ss, slot_mask=smask)
    rows = np.nonzero(smask[ss])[0]  # sorted positions of the selected slots
    ye = None
    if check_y:   # (a fused decode layer stores no per-slot expert outputs)
        ye = max_rel(g["y_sorted"][rows], y_ref[rows])
        assert ye <= TOL, "expert outputs rel err %g" % ye
    out_ref = oracle.combine(y_ref, sp, ids_eff, w_ref, L.expert_scale, token_mask=tmask)
    sel = tmask.astype(bool)
    oe = max_rel(g["out"][sel], out_ref[sel])
    assert oe <= TOL, "combined output rel err %g" % oe
    assert np.all(np.isfinite(g["out"])), "non-finite output"
    if refs is not None:
        refs["out"] = out_ref
        refs["ids"] = ids_eff
    return dict(y_err=ye, out_err=oe, near_ties=nties, distinct_experts=int((np.diff(off) > 0).sum()))
