"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function include/sparse_moe.h declares, and rejects bad arguments with
the documented status before enqueueing anything.

Every call below fails validation, so no kernel is launched and the fake
device addresses are never touched."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_moe.h")

binding = pytest.importorskip("sparse_moe_amd.binding")
lib = binding.lib

OK, NULL, SHAPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5
A = C.c_void_p(0x100000)        # 16-byte aligned fake device address (never dereferenced)
B = C.c_void_p(0x200000)
MIS = C.c_void_p(0x100004)      # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.SIGNATURES)
    assert lib.moe_abi_version() == 1


def test_status_strings():
    for s in range(8):
        assert lib.moe_status_string(s) != b"unknown status"
    assert lib.moe_status_string(99) == b"unknown status"


def test_router_validation():
    f = lib.moe_router_topk
    # (x, x_dt, T, H, W_r, r_scale, bias, E, K, logits, ids, w, stream)
    assert f(A, 0, 4, 256, A, None, None, 0, 1, A, A, A, None) == SHAPE        # E = 0
    assert f(A, 0, 4, 256, A, None, None, 8, 9, A, A, A, None) == SHAPE        # K > E
    assert f(A, 0, 4, 256, A, None, None, 300, 2, A, A, A, None) == SHAPE      # E > 256
    assert f(A, 0, 4, 256, A, None, None, 64, 17, A, A, A, None) == SHAPE      # K > 16
    assert f(A, 0, 4, 100, A, None, None, 8, 2, A, A, A, None) == SHAPE        # H % 32
    assert f(A, 0, -1, 256, A, None, None, 8, 2, A, A, A, None) == SHAPE       # T < 0
    assert f(A, 5, 4, 256, A, None, None, 8, 2, A, A, A, None) == UNSUP        # dtype
    assert f(None, 0, 0, 256, None, None, None, 8, 2, None, None, None, None) == OK  # T = 0
    assert f(None, 0, 4, 256, A, None, None, 8, 2, A, A, A, None) == NULL      # x
    assert f(A, 0, 4, 256, A, None, None, 8, 2, None, A, A, None) == NULL      # logits
    assert f(A, 0, 4, 256, A, None, None, 8, 2, A, A, MIS, None) == ALIGN
    assert f(MIS, 0, 4, 256, A, None, None, 8, 2, A, A, A, None) == ALIGN
    assert f(A, 0, 4, 256, A, MIS, None, 8, 2, A, A, A, None) == ALIGN


def test_permute_validation_and_workspace():
    f = lib.moe_permute
    assert lib.moe_permute_workspace_bytes(4, 2, 8) == 0           # one tile: no workspace
    big = lib.moe_permute_workspace_bytes(4096, 8, 128)
    assert big >= (32 * 128 + 32768) * 4 and big % 256 == 0
    assert f(A, 4096, 8, 128, A, A, A, None, 0, None) == WS
    assert f(A, 4096, 8, 128, A, A, A, A, 16, None) == WS
    assert f(A, 4, 2, 8, None, A, A, None, 0, None) == NULL
    assert f(A, 4, 2, 8, A, MIS, A, None, 0, None) == ALIGN
    assert f(A, 4, 9, 8, A, A, A, None, 0, None) == SHAPE
    assert f(None, 0, 2, 8, None, None, None, None, 0, None) == OK
    assert f(A, 2 ** 30, 8, 128, A, A, A, A, 1 << 40, None) == SHAPE   # T*K >= 2^31


def test_route_validation_and_workspace():
    f = lib.moe_route
    assert lib.moe_route_workspace_bytes(1, 8, 128) == 256
    assert lib.moe_route_workspace_bytes(4096, 8, 128) == 256 + lib.moe_permute_workspace_bytes(4096, 8, 128)
    # (x, x_dt, T, H, W_r, r_scale, bias, E, K, logits, ids, w, offsets, sorted, pos, ws, ws_bytes, stream)
    assert f(A, 0, 1, 2816, A, None, None, 128, 8, A, A, A, A, A, A, A, 16, None) == WS
    assert f(A, 0, 1, 2816, A, None, None, 128, 8, A, A, A, A, A, A, None, 256, None) == WS
    assert f(A, 0, 1, 2816, A, None, None, 128, 8, A, A, A, None, A, A, A, 256, None) == NULL
    assert f(A, 0, 1, 2816, A, None, None, 128, 8, A, A, A, A, MIS, A, A, 256, None) == ALIGN
    assert f(A, 0, 1, 2816, A, None, None, 128, 0, A, A, A, A, A, A, A, 256, None) == SHAPE
    assert f(None, 0, 0, 2816, None, None, None, 128, 8, None, None, None, None, None, None, None,
             0, None) == OK


def test_ffn_validation_and_workspace():
    f = lib.moe_expert_ffn_q4_0
    ws = lib.moe_expert_ffn_q4_0_workspace_bytes(4096, 8, 2816, 704, 128, 1)
    assert ws >= 4096 * 8 * 704 * 2
    assert lib.moe_expert_ffn_q4_0_workspace_bytes(4, 2, 250, 64, 8, 0) == 0   # bad H
    # (x, x_dt, T, H, w_gu, w_dn, I, E, K, offsets, sorted, y, ws, ws_bytes, stream)
    assert f(A, 1, 4096, 2816, A, A, 704, 128, 8, A, A, A, A, 16, None) == WS
    assert f(A, 1, 4096, 2816, A, A, 704, 128, 8, A, A, A, None, ws, None) == WS
    assert f(A, 1, 4, 2816, A, A, 700, 128, 8, A, A, A, A, ws, None) == SHAPE   # I % 32
    assert f(A, 1, 4, 8192, A, A, 704, 128, 8, A, A, A, A, ws, None) == SHAPE   # H > max
    assert f(A, 1, 4, 2816, None, A, 704, 128, 8, A, A, A, A, ws, None) == NULL
    assert f(A, 1, 4, 2816, MIS, A, 704, 128, 8, A, A, A, A, ws, None) == ALIGN
    assert f(A, 3, 4, 2816, A, A, 704, 128, 8, A, A, A, A, ws, None) == UNSUP
    assert f(None, 1, 0, 2816, None, None, 704, 128, 8, None, None, None, None, 0, None) == OK


def test_ffn_noalloc_validation():
    f = lib.moe_expert_ffn_q4_0_noalloc
    SCRATCH = 7
    # (x, x_dt, T, H, w_gu, w_dn, I, E, K, offsets, sorted, y, stream)
    assert f(A, 1, 4096, 2816, A, A, 704, 128, 8, A, A, A, None) == SCRATCH   # prefill: too big
    assert f(A, 1, 1024, 2816, A, A, 704, 128, 8, A, A, A, None) == SCRATCH
    assert f(None, 1, 8, 2816, A, A, 704, 128, 8, A, A, A, None) == NULL      # fits, x missing
    assert f(A, 1, 8, 2816, A, A, 700, 128, 8, A, A, A, None) == SHAPE
    assert f(A, 4, 8, 2816, A, A, 704, 128, 8, A, A, A, None) == UNSUP
    assert f(None, 1, 0, 2816, None, None, 704, 128, 8, None, None, None, None) == OK
    # every decode batch below 64 tokens fits; 927 bf16 tokens at the Gemma shape do
    big = lib.moe_expert_ffn_q4_0_workspace_bytes
    assert big(63, 8, 2816, 704, 128, 0) <= 16 << 20
    assert big(927, 8, 2816, 704, 128, 1) <= 16 << 20 < big(928, 8, 2816, 704, 128, 1)


def test_decode_layer_validation_and_workspace():
    f = lib.moe_layer_decode
    ws = lib.moe_layer_decode_workspace_bytes(1, 8, 2816, 704, 128, 0)
    # a 16 KiB header of completion counters, then h [T*K, I]
    assert ws == (16 << 10) + 8 * 704 * 4
    assert lib.moe_layer_decode_workspace_bytes(1, 8, 2800, 704, 128, 0) == 0   # H % 32
    UNS = 4

    def call(x=A, xdt=0, T=1, H=2816, wr=A, E=128, K=8, I=704, ws_=A, wsb=ws, out=A, act=None,
             odt=0, logits=A):
        # (x, x_dt, T, H, W_r, r_scale, bias, E, K, w_gu, w_dn, I, scale, logits, ids, w, off,
        #  sorted, slot_pos, residual, rdt, out_f32, out_act, odt, ws, ws_bytes, stream)
        return f(x, xdt, T, H, wr, None, None, E, K, A, A, I, A, logits, A, A, A, A, A, None, 0,
                 out, act, odt, ws_, wsb, None)
    assert call(T=9) == UNS                  # more than 8 tokens
    assert call(T=8, K=16, E=128) == UNS     # more than 64 slots
    assert call(H=2848) == UNS               # 89 blocks per gate/up row: odd
    assert call(I=736) == UNS                # 23 blocks per down row: odd
    assert call(xdt=3) == UNS
    assert call(T=0, x=None) == OK
    assert call(x=None) == NULL
    assert call(out=None) == NULL             # no output
    assert call(logits=None) == NULL
    assert call(ws_=None) == WS
    assert call(wsb=16) == WS
    assert call(x=MIS) == ALIGN
    assert call(E=300) == SHAPE


def test_combine_and_rmsnorm_validation():
    f = lib.moe_combine
    # (y, slot_pos, ids, w, scale, T, K, H, residual, rdt, out_f32, out_act, odt, stream)
    assert f(A, A, A, A, A, 4, 2, 256, None, 0, None, None, 0, None) == NULL   # no output
    assert f(A, A, None, A, A, 4, 2, 256, None, 0, A, None, 0, None) == NULL   # scale needs ids
    assert f(A, A, A, A, A, 4, 2, 250, None, 0, A, None, 0, None) == SHAPE
    assert f(A, A, A, A, A, 4, 2, 256, None, 0, A, A, 9, None) == UNSUP
    assert f(A, A, A, A, A, 4, 2, 256, MIS, 0, A, None, 0, None) == ALIGN
    assert f(None, None, None, None, None, 0, 2, 256, None, 0, None, None, 0, None) == OK
    g = lib.moe_rmsnorm
    assert g(A, 1, A, C.c_float(1e-6), 4, 100, A, 1, None) == SHAPE
    assert g(A, 1, None, C.c_float(1e-6), 4, 256, A, 1, None) == NULL
    assert g(A, 1, A, C.c_float(-1.0), 4, 256, A, 1, None) == SHAPE
    assert g(A, 1, A, C.c_float(1e-6), 4, 256, MIS, 1, None) == ALIGN
    assert g(None, 1, None, C.c_float(1e-6), 0, 256, None, 1, None) == OK


def test_linear_validation_and_workspace():
    f = lib.moe_linear_q4_0
    small = lib.moe_linear_q4_0_workspace_bytes(4, 2816, 4224, 0)
    assert small == 256 + 256                      # offsets, slot list (GEMV path)
    big = lib.moe_linear_q4_0_workspace_bytes(4096, 2816, 4224, 1)
    assert big >= 256 + 4096 * 4 + 4096 * 2816 * 2 + 4096 * 88 * 4   # + MFMA staging
    assert lib.moe_linear_q4_0_workspace_bytes(4, 250, 16, 0) == 0    # H % 32
    assert lib.moe_linear_q4_0_workspace_bytes(4, 2816, 0, 0) == 0    # no rows
    # (x, x_dt, T, H, W, R, y, ws, ws_bytes, stream)
    assert f(A, 0, 4, 2816, A, 4224, A, A, 16, None) == WS
    assert f(A, 0, 4, 2816, A, 4224, A, None, small, None) == WS
    assert f(A, 0, 4, 2800, A, 4224, A, A, small, None) == SHAPE
    assert f(A, 0, 4, 8192, A, 4224, A, A, small, None) == SHAPE      # H > max
    assert f(A, 0, 4, 2816, A, 70000, A, A, small, None) == SHAPE     # R > max
    assert f(A, 0, 4, 2816, None, 4224, A, A, small, None) == NULL
    assert f(A, 0, 4, 2816, A, 4224, MIS, A, small, None) == ALIGN
    assert f(A, 7, 4, 2816, A, 4224, A, A, small, None) == UNSUP
    assert f(None, 0, 0, 2816, None, 4224, None, None, 0, None) == OK
