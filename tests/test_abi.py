"""CPU checks of the C ABI: the library loads, exports every declared symbol,
derives the same NF4 table as the oracle, and rejects bad arguments before
launching anything (these calls never reach the GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import qlora_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")


@pytest.fixture(scope="module")
def lib():
    from bit_quantized_fine_qlora_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libqlora.so is not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for nm in names:
        assert hasattr(lib, nm), nm


def test_binding_prototypes_cover_header():
    from bit_quantized_fine_qlora_amd import _lib
    assert set(declared_functions()) == set(_lib.PROTOTYPES)


def test_library_table_matches_oracle(lib):
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    lib.qlora_nf4_table(ctypes.cast(lv, ctypes.c_void_p), ctypes.cast(th, ctypes.c_void_p))
    got_q = np.frombuffer(lv, dtype=np.float32)
    got_t = np.frombuffer(th, dtype=np.float32)
    assert np.array_equal(got_q.view(np.uint32), O.NF4_Q.view(np.uint32))
    assert np.array_equal(got_t.view(np.uint32), O.NF4_T.view(np.uint32))


def test_level_tables_match_oracle(lib):
    for qtype, (Q, T) in ((0, (O.NF4_Q, O.NF4_T)), (1, (O.UNIFORM4_Q, O.UNIFORM4_T)),
                          (2, (O.EDGE_MEAN_Q, O.EDGE_MEAN_T)), (3, (O.INT4_Q, O.INT4_T))):
        lv = (ctypes.c_float * 16)()
        th = (ctypes.c_float * 15)()
        assert lib.qlora_level_table(qtype, ctypes.cast(lv, ctypes.c_void_p), ctypes.cast(th, ctypes.c_void_p)) == 0
        assert np.array_equal(np.frombuffer(lv, dtype=np.float32).view(np.uint32), Q.view(np.uint32)), qtype
        assert np.array_equal(np.frombuffer(th, dtype=np.float32).view(np.uint32), T.view(np.uint32)), qtype
    assert lib.qlora_level_table(4, None, None) == -7
    assert lib.qlora_level_table(-1, None, None) == -7


def test_status_strings(lib):
    for st in range(-8, 1):
        assert len(lib.qlora_status_string(st)) >= 2
    assert lib.qlora_version() >= 100


P = ctypes.c_void_p(1 << 20)   # a non-NULL, 16-byte-aligned dummy; never dereferenced on error paths
MIS = ctypes.c_void_p((1 << 20) + 4)


def test_quantize_argument_errors(lib):
    f = lib.qlora_quantize_nf4_dq
    assert f(None, 4, 64, P, P, P, None) == -1
    assert f(P, 4, 60, P, P, P, None) == -2        # n not a multiple of 64
    assert f(P, 0, 64, P, P, P, None) == -2
    assert f(P, -3, 64, P, P, P, None) == -2
    assert f(P, 4, 0, P, P, P, None) == -2
    assert f(MIS, 4, 64, P, P, P, None) == -4
    assert f(P, 1 << 31, 64, P, P, P, None) == -2


def test_level_table_variant_argument_errors(lib):
    assert lib.qlora_quantize_dq(5, P, 4, 64, P, P, P, None) == -7
    assert lib.qlora_quantize_dq(1, P, 4, 60, P, P, P, None) == -2
    assert lib.qlora_quantize_dq(1, None, 4, 64, P, P, P, None) == -1
    assert lib.qlora_dequant_dq(-1, P, P, P, 4, 64, P, None) == -7
    assert lib.qlora_dequant_dq(1, P, P, P, 4, 64, MIS, None) == -4


def test_grouped_quantize_argument_errors(lib):
    from bit_quantized_fine_qlora_amd import _lib
    f = lib.qlora_quantize_dq_grouped

    def arr(*ws):
        a = (_lib.QuantWeight * max(len(ws), 1))()
        for i, (W, m, n, codes) in enumerate(ws):
            a[i] = _lib.QuantWeight(W, m, n, codes, P, P)
        return a
    good = (P, 4, 64, P)
    assert f(4, 1, arr(good), None) == -7                  # unknown qtype first
    assert f(0, 1, None, None) == -1
    assert f(0, 0, arr(good), None) == -7                  # count 1..8
    assert f(0, 9, arr(*[good] * 9), None) == -7
    assert f(0, 2, arr(good, (None, 4, 64, P)), None) == -1
    assert f(0, 2, arr(good, (P, 4, 60, P)), None) == -2   # every weight checked before launch
    assert f(0, 2, arr(good, (P, 4, 64, MIS)), None) == -4
    assert f(3, 2, arr(good, (P, 1 << 31, 64, P)), None) == -2


def test_dequant_argument_errors(lib):
    f = lib.qlora_dequant_nf4_dq
    assert f(P, P, None, 4, 64, P, None) == -1
    assert f(P, P, P, 4, 65, P, None) == -2
    assert f(P, P, P, 4, 64, MIS, None) == -4


def fwd(lib, M=32, n=256, m=256, r=8, s=2.0, x=P, A=P, B=P, h=P, u=None, ws=P, wsb=1 << 30):
    return lib.qlora_linear_fwd(M, n, m, r, s, x, P, P, P, A, B, h, u, ws, wsb, None)


def test_fwd_argument_errors(lib):
    assert fwd(lib, x=None) == -1
    assert fwd(lib, h=None) == -1
    assert fwd(lib, n=100) == -2
    assert fwd(lib, M=0) == -2
    assert fwd(lib, m=-1) == -2
    assert fwd(lib, r=0) == -3
    assert fwd(lib, r=129) == -3
    assert fwd(lib, s=float("inf")) == -7
    assert fwd(lib, s=float("nan")) == -7
    assert fwd(lib, x=MIS) == -4
    assert fwd(lib, u=MIS) == -4
    assert fwd(lib, ws=None) == -5
    need = lib.qlora_workspace_bytes(0, 32, 256, 256, 8)
    assert need > 0
    assert fwd(lib, wsb=need - 1) == -5


def test_bwd_argument_errors(lib):
    f = lib.qlora_linear_bwd

    def call(M=32, n=256, m=256, r=8, s=2.0, g=P, gA=P, gB=P, gx=P, ws=P, wsb=1 << 30):
        return f(M, n, m, r, s, P, g, P, P, P, P, P, None, gx, gA, gB, ws, wsb, None)

    assert call(g=None) == -1
    assert call(gA=None) == -1
    assert call(gB=None) == -1
    assert call(n=32) == -2
    assert call(r=200) == -3
    assert call(gx=MIS) == -4
    need = lib.qlora_workspace_bytes(1, 32, 256, 256, 8)
    assert call(wsb=need - 1) == -5


def test_workspace_sizes(lib):
    assert lib.qlora_workspace_bytes(0, 4096, 4096, 14336, 16) > 0
    assert lib.qlora_workspace_bytes(1, 4096, 4096, 14336, 16) > 0
    # 896 output tiles on 256 CUs: the last 128 tiles run as K halves whose fp32
    # partial sums (256 x 256 each) live in the forward's workspace
    assert lib.qlora_workspace_bytes(0, 4096, 4096, 14336, 16) >= 128 * 256 * 256 * 4
    # few tiles (256 tokens; sized for 256 CUs, the count assumed without a
    # device): the 16 grad_x tiles run as 16 K pieces and the 56 forward tiles
    # as 4, each piece's fp32 sums (256 x 256) in the workspace
    assert lib.qlora_workspace_bytes(1, 256, 4096, 14336, 16) >= 16 * 16 * 256 * 256 * 4
    assert lib.qlora_workspace_bytes(0, 256, 4096, 14336, 16) >= 56 * 4 * 256 * 256 * 4
    # 256 tiles fill the chip exactly: nothing is split
    assert lib.qlora_workspace_bytes(0, 4096, 4096, 4096, 16) < 16 << 20
    assert lib.qlora_workspace_bytes(0, 32, 100, 256, 8) == 0
    assert lib.qlora_workspace_bytes(7, 32, 256, 256, 8) == 0
    assert lib.qlora_workspace_bytes(0, 32, 256, 256, 0) == 0


def test_linear_check_without_hand_off(lib):
    # calls that have no bounded wait are complete by construction: OK with
    # nothing read back (no GPU is touched); bad arguments are rejected first
    f = lib.qlora_linear_check
    assert f(0, 16, 4096, 1024, 16, None, None) == 0       # weight-streaming forward
    assert f(0, 4096, 4096, 4096, 16, None, None) == 0     # 256 tiles: one full round
    assert f(1, 256, 4096, 14336, 16, None, None) == 0     # few tiles: K pieces, no wait
    assert f(3, 4096, 4096, 4096, 16, None, None) == -7    # unknown op
    assert f(0, 4096, 100, 4096, 16, None, None) == -2     # n % 64 != 0
    assert f(0, 4096, 4096, 4096, 0, None, None) == -3     # r = 0
    # this grad_x GEMM (896 tiles) splits its last round: the workspace is needed
    assert f(1, 4096, 14336, 4096, 16, None, None) == -1
    # 16 grad_x tiles over K = 1024 run as two K halves through the hand-off
    assert f(1, 16, 4096, 1024, 16, None, None) == -1


def test_static_forward_rejects_large_layouts(lib):
    # u and the split partials of 262144 tokens at r = 128 need far more than
    # the 64 MiB scratch: refused before anything touches the GPU
    f = lib.qlora_linear_fwd_static
    assert lib.qlora_workspace_bytes(0, 262144, 64, 64, 128) > 64 << 20
    assert f(262144, 64, 64, 128, 1.0, P, P, P, P, P, P, P, None, None) == -5
    # argument errors come first, as for qlora_linear_fwd
    assert f(16, 100, 64, 8, 1.0, P, P, P, P, P, P, P, None, None) == -2
    assert f(16, 64, 64, 8, 1.0, None, P, P, P, P, P, P, None, None) == -1
    assert f(16, 64, 64, 8, 1.0, MIS, P, P, P, P, P, P, None, None) == -4
    assert f(16, 64, 64, 0, 1.0, P, P, P, P, P, P, P, None, None) == -3


def layer_desc(n=256, m=256, r=8, s=2.0, x=1 << 20, h=1 << 20, u=0):
    from bit_quantized_fine_qlora_amd import _lib
    return _lib.LinearLayer(n, m, r, s, x, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, h, u)


def test_grouped_argument_errors(lib):
    from bit_quantized_fine_qlora_amd import _lib
    f = lib.qlora_linear_fwd_grouped
    arr = (_lib.LinearLayer * 3)(layer_desc(), layer_desc(n=512, m=128, r=16), layer_desc(m=1024))
    need = lib.qlora_grouped_workspace_bytes(16, 3, arr)
    assert need > 0
    assert f(16, 3, None, P, 1 << 30, None) == -1
    assert f(16, 0, arr, P, 1 << 30, None) == -7
    assert f(16, 9, arr, P, 1 << 30, None) == -7
    assert f(16, 3, arr, None, 1 << 30, None) == -5
    assert f(16, 3, arr, P, need - 1, None) == -5
    assert f(16, 3, arr, MIS, need, None) == -4
    bad = (_lib.LinearLayer * 2)(layer_desc(), layer_desc(n=100))
    assert f(16, 2, bad, P, 1 << 30, None) == -2
    assert lib.qlora_grouped_workspace_bytes(16, 2, bad) == 0
    bad = (_lib.LinearLayer * 2)(layer_desc(), layer_desc(r=0))
    assert f(16, 2, bad, P, 1 << 30, None) == -3
    bad = (_lib.LinearLayer * 2)(layer_desc(), layer_desc(x=0))
    assert f(16, 2, bad, P, 1 << 30, None) == -1
    bad = (_lib.LinearLayer * 2)(layer_desc(), layer_desc(u=(1 << 20) + 4))
    assert f(16, 2, bad, P, 1 << 30, None) == -4
    # the grouped workspace is the sum of the single-layer ones, each rounded to 256 bytes
    singles = [lib.qlora_workspace_bytes(0, 16, d.n, d.m, d.r) for d in arr]
    assert need == sum((b + 255) // 256 * 256 for b in singles)


def test_dropout_argument_errors(lib):
    from bit_quantized_fine_qlora_amd import _lib
    fwd_ex, bwd_ex = lib.qlora_linear_fwd_ex, lib.qlora_linear_bwd_ex

    def drop(p):
        return ctypes.pointer(_lib.Dropout(p, 7, 0))

    def f(d, x=P):
        return fwd_ex(32, 256, 256, 8, 2.0, x, P, P, P, P, P, P, None, d, P, 1 << 30, None)

    def b(d, ws=P, wsb=1 << 30, gA=P):
        return bwd_ex(32, 256, 256, 8, 2.0, P, P, P, P, P, P, P, None, P, gA, P, d, ws, wsb, None)

    for p in (-0.25, 1.0, 1.5, float("nan"), float("inf")):
        assert f(drop(p)) == -7, p
        assert b(drop(p)) == -7, p
    assert f(None, x=None) == -1
    assert f(drop(0.1), x=None) == -1
    assert b(drop(0.1), gA=None) == -1
    # with the mask on, the backward needs the dropout workspace (one M x n
    # fp32 buffer more than the plain backward)
    plain = lib.qlora_workspace_bytes(1, 32, 256, 256, 8)
    need = lib.qlora_workspace_bytes(2, 32, 256, 256, 8)
    assert need == plain + 32 * 256 * 4
    assert b(drop(0.1), wsb=plain) == -5
    assert b(drop(0.1), wsb=need - 1) == -5
    assert b(drop(0.1), ws=None, wsb=need) == -5
