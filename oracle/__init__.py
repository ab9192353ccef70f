"""ctypes front end of the CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does.  It shares no code with the HIP library.  Inputs are numpy arrays in the
layer's storage formats (fp32, bf16 bit patterns as uint16, raw Q4_0 bytes);
outputs are float64 / int32 numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_HDR = os.path.join(_HERE, "moe_oracle.h")
LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C11, -O2, no fast-math, no FMA contraction)."""
    stale = (not os.path.exists(LIB_PATH) or
             os.path.getmtime(LIB_PATH) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)))
    if force or stale:
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-D_DEFAULT_SOURCE", "-O2", "-fno-fast-math", "-ffp-contract=off",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(LIB_PATH)
        p, i32, i64, d = C.c_void_p, C.c_int, C.c_int64, C.c_double
        L.orc_f16_to_f64.argtypes = [C.c_uint16]; L.orc_f16_to_f64.restype = d
        L.orc_bf16_to_f64.argtypes = [C.c_uint16]; L.orc_bf16_to_f64.restype = d
        L.orc_f64_to_bf16.argtypes = [d]; L.orc_f64_to_bf16.restype = C.c_uint16
        L.orc_round_act.argtypes = [d, i32]; L.orc_round_act.restype = d
        L.orc_q4_0_decode.argtypes = [p, p]; L.orc_q4_0_decode.restype = None
        L.orc_gelu_tanh.argtypes = [d]; L.orc_gelu_tanh.restype = d
        L.orc_router_logits.argtypes = [p, i32, i64, i32, p, p, p, i32, p]
        L.orc_topk_softmax.argtypes = [p, i64, i32, i32, p, p]
        L.orc_topk_weights.argtypes = [p, i64, i32, i32, p, p]
        L.orc_permute.argtypes = [p, i64, i32, i32, p, p, p]
        L.orc_expert_ffn_token.argtypes = [p, i32, i32, p, p, i32, i32, p, p]
        L.orc_expert_ffn.argtypes = [p, i32, i64, i32, p, p, i32, i32, i32, p, p, p, p]
        L.orc_linear_q4_0.argtypes = [p, i32, i64, i32, p, i32, p]
        L.orc_combine.argtypes = [p, p, p, p, p, i64, i32, i32, p, p]
        L.orc_rmsnorm.argtypes = [p, i32, p, d, i64, i32, p]
        L.orc_moe_layer.argtypes = [p, i32, i64, i32, p, p, p, p, i32, i32, p, p, i32, p, p,
                                    p, p, p, p, p, p, p]
        L.orc_residual.argtypes = [p, p, i64, i32, p, p]
        L.orc_stack_layer.argtypes = [p, i64, i32, p, d, p, p, i32, i32, p, p, i32, p, p, p, p, p,
                                      p]
        for f in ("orc_residual", "orc_stack_layer", "orc_router_logits", "orc_topk_softmax", "orc_topk_weights", "orc_permute", "orc_expert_ffn_token",
                  "orc_expert_ffn", "orc_linear_q4_0", "orc_combine", "orc_rmsnorm", "orc_moe_layer"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _act(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("activations must be float32 or uint16 (bf16 bits), got %s" % x.dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("%s failed with code %d" % (what, rc))


# ---- scalar helpers -------------------------------------------------------
def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return lib().orc_bf16_to_f64(bits)


def f64_to_bf16(v: float) -> int:
    return lib().orc_f64_to_bf16(v)


def gelu_tanh(z: float) -> float:
    return lib().orc_gelu_tanh(z)


def round_act(v: float, act: int) -> float:
    return lib().orc_round_act(v, act)


def q4_0_decode(block: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(block, dtype=np.uint8)
    assert b.size == 18
    out = np.empty(32, np.float64)
    lib().orc_q4_0_decode(_ptr(b), _ptr(out))
    return out


# ---- steps ----------------------------------------------------------------
def router_logits(x, w_r, r_scale=None, bias=None) -> np.ndarray:
    x = np.ascontiguousarray(x)
    T, H = x.shape
    E = w_r.shape[0]
    w_r = np.ascontiguousarray(w_r, np.float32)
    out = np.empty((T, E), np.float64)
    rs = None if r_scale is None else np.ascontiguousarray(r_scale, np.float32)
    bs = None if bias is None else np.ascontiguousarray(bias, np.float32)
    _check(lib().orc_router_logits(_ptr(x), _act(x), T, H, _ptr(w_r), _ptr(rs), _ptr(bs), E,
                                   _ptr(out)), "orc_router_logits")
    return out


def topk_softmax(logits: np.ndarray, K: int):
    l = np.ascontiguousarray(logits, np.float64)
    T, E = l.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    _check(lib().orc_topk_softmax(_ptr(l), T, E, K, _ptr(ids), _ptr(w)), "orc_topk_softmax")
    return ids, w


def topk_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    l = np.ascontiguousarray(logits, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    T, E = l.shape
    K = ids.shape[1]
    w = np.empty((T, K), np.float64)
    _check(lib().orc_topk_weights(_ptr(l), T, E, K, _ptr(ids), _ptr(w)), "orc_topk_weights")
    return w


def permute(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, np.int32)
    T, K = ids.shape
    off = np.empty(E + 1, np.int32)
    ss = np.empty(T * K, np.int32)
    sp = np.empty(T * K, np.int32)
    _check(lib().orc_permute(_ptr(ids), T, K, E, _ptr(off), _ptr(ss), _ptr(sp)), "orc_permute")
    return off, ss, sp


def expert_ffn_token(x_row, w_gate_up, w_down, e: int):
    """(h [I], y [H]) of one token through expert e."""
    x_row = np.ascontiguousarray(x_row)
    H = x_row.shape[-1]
    I = w_gate_up.shape[1] // 2
    h = np.empty(I, np.float64)
    y = np.empty(H, np.float64)
    _check(lib().orc_expert_ffn_token(_ptr(x_row), _act(x_row), H, _ptr(w_gate_up),
                                      _ptr(w_down), I, e, _ptr(h), _ptr(y)),
           "orc_expert_ffn_token")
    return h, y


def linear_q4_0(x, w) -> np.ndarray:
    """y [T, R] = x [T, H] times the Q4_0 matrix w [R, H/32, 18] (transposed)."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    w = np.ascontiguousarray(w, np.uint8)
    R = w.shape[0]
    assert w.shape[1] * 32 == H and w.shape[2] == 18
    y = np.empty((T, R), np.float64)
    _check(lib().orc_linear_q4_0(_ptr(x), _act(x), T, H, _ptr(w), R, _ptr(y)), "orc_linear_q4_0")
    return y


def expert_ffn(x, w_gate_up, w_down, K: int, offsets, sorted_slots, slot_mask=None):
    x = np.ascontiguousarray(x)
    T, H = x.shape
    E = w_gate_up.shape[0]
    I = w_gate_up.shape[1] // 2
    y = np.full((T * K, H), np.nan, np.float64)
    m = None if slot_mask is None else np.ascontiguousarray(slot_mask, np.uint8)
    _check(lib().orc_expert_ffn(_ptr(x), _act(x), T, H, _ptr(np.ascontiguousarray(w_gate_up)),
                                _ptr(np.ascontiguousarray(w_down)), I, E, K,
                                _ptr(np.ascontiguousarray(offsets, np.int32)),
                                _ptr(np.ascontiguousarray(sorted_slots, np.int32)), _ptr(m),
                                _ptr(y)), "orc_expert_ffn")
    return y


def combine(y_sorted, slot_pos, ids, w, scale=None, token_mask=None) -> np.ndarray:
    ids = np.ascontiguousarray(ids, np.int32)
    T, K = ids.shape
    y = np.ascontiguousarray(y_sorted, np.float64)
    H = y.shape[1]
    out = np.full((T, H), np.nan, np.float64)
    sc = None if scale is None else np.ascontiguousarray(scale, np.float32)
    m = None if token_mask is None else np.ascontiguousarray(token_mask, np.uint8)
    _check(lib().orc_combine(_ptr(y), _ptr(np.ascontiguousarray(slot_pos, np.int32)), _ptr(ids),
                             _ptr(np.ascontiguousarray(w, np.float64)), _ptr(sc), T, K, H, _ptr(m),
                             _ptr(out)), "orc_combine")
    return out


def rmsnorm(x, w, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x)
    T, H = x.shape
    out = np.empty((T, H), np.uint16)
    _check(lib().orc_rmsnorm(_ptr(x), _act(x), _ptr(np.ascontiguousarray(w, np.float32)), eps, T,
                             H, _ptr(out)), "orc_rmsnorm")
    return out


def moe_layer(x, w_r, w_gate_up, w_down, K: int, scale=None, bias=None, r_scale=None,
              logits_in=None, token_mask=None) -> dict:
    """Whole layer; returns dict(logits, ids, w, offsets, sorted_slots, slot_pos, out)."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    E = w_gate_up.shape[0]
    I = w_gate_up.shape[1] // 2
    logits = np.empty((T, E), np.float64)
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    off = np.empty(E + 1, np.int32)
    ss = np.empty(T * K, np.int32)
    sp = np.empty(T * K, np.int32)
    out = np.full((T, H), np.nan, np.float64)
    wr = None if w_r is None else np.ascontiguousarray(w_r, np.float32)
    li = None if logits_in is None else np.ascontiguousarray(logits_in, np.float32)
    sc = None if scale is None else np.ascontiguousarray(scale, np.float32)
    bs = None if bias is None else np.ascontiguousarray(bias, np.float32)
    rs = None if r_scale is None else np.ascontiguousarray(r_scale, np.float32)
    m = None if token_mask is None else np.ascontiguousarray(token_mask, np.uint8)
    _check(lib().orc_moe_layer(_ptr(x), _act(x), T, H, _ptr(wr), _ptr(li), _ptr(rs), _ptr(bs), E,
                               K, _ptr(np.ascontiguousarray(w_gate_up)),
                               _ptr(np.ascontiguousarray(w_down)), I, _ptr(sc), _ptr(m),
                               _ptr(logits), _ptr(ids), _ptr(w), _ptr(off), _ptr(ss), _ptr(sp),
                               _ptr(out)), "orc_moe_layer")
    return dict(logits=logits, ids=ids, w=w, offsets=off, sorted_slots=ss, slot_pos=sp, out=out)


def residual(x_bf16, out, token_mask=None) -> np.ndarray:
    """x_next = bf16(x + out) (bf16 bits as uint16; out binary64)."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    T, H = x.shape
    o = np.ascontiguousarray(out, np.float64)
    assert o.shape == (T, H)
    m = None if token_mask is None else np.ascontiguousarray(token_mask, np.uint8)
    xn = np.zeros((T, H), np.uint16)
    _check(lib().orc_residual(_ptr(x), _ptr(o), T, H, _ptr(m), _ptr(xn)), "orc_residual")
    return xn


def stack_layer(x_bf16, rms_w, eps: float, w_r, w_gate_up, w_down, K: int, scale=None,
                bias=None, token_mask=None) -> dict:
    """One pre-norm block of the stack; returns dict(xhat, ids, out, x_next)."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    T, H = x.shape
    E = w_gate_up.shape[0]
    I = w_gate_up.shape[1] // 2
    xhat = np.zeros((T, H), np.uint16)
    ids = np.zeros((T, K), np.int32)
    out = np.zeros((T, H), np.float64)
    xn = np.zeros((T, H), np.uint16)
    sc = None if scale is None else np.ascontiguousarray(scale, np.float32)
    bs = None if bias is None else np.ascontiguousarray(bias, np.float32)
    m = None if token_mask is None else np.ascontiguousarray(token_mask, np.uint8)
    _check(lib().orc_stack_layer(_ptr(x), T, H, _ptr(np.ascontiguousarray(rms_w, np.float32)),
                                 eps, _ptr(np.ascontiguousarray(w_r, np.float32)), _ptr(bs), E, K,
                                 _ptr(np.ascontiguousarray(w_gate_up)),
                                 _ptr(np.ascontiguousarray(w_down)), I, _ptr(sc), _ptr(m),
                                 _ptr(xhat), _ptr(ids), _ptr(out), _ptr(xn)), "orc_stack_layer")
    return dict(xhat=xhat, ids=ids, out=out, x_next=xn)
