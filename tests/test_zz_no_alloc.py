"""The allocation-free forward (qlora_linear_fwd_static, through the C ABI)
against the forward with a caller workspace (qlora_linear_fwd).

Where the forward's workspace layout fits the library's scratch the two run
the same kernels on the same layout and must agree bit for bit; a layout
larger than the scratch runs the GEMM without its K-split region and must
agree to the float tolerance.  Calls follow each other with shrinking inputs,
so each one runs on the scratch contents the previous call left behind.
"""

import numpy as np
import pytest
import torch

import qlora_inputs as QI
from parity_utils import assert_close, dev_bf16, f64, host_bits, oracle_full

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import bit_quantized_fine_qlora_amd as lib
    lib._lib.load()
    return lib


def say(msg):
    print(f"[case] {msg}", flush=True)


def layer(Q, M, n, m, r, seed):
    inp = QI.custom_inputs(seed=seed, M=M, n=n, m=m, r=r)
    q = Q.quantize_nf4_dq(torch.from_numpy(inp["W"]).to("cuda"))
    return inp, q, dev_bf16(inp["x"]), dev_bf16(inp["A"]), dev_bf16(inp["B"])


def run_pair(Q, M, n, m, r, s, seed, oracle=True):
    inp, q, x, A, B = layer(Q, M, n, m, r, seed)
    ws = torch.empty(max(Q.workspace_bytes(Q.QLORA_OP_FWD, M, n, m, r), 256), dtype=torch.uint8, device="cuda")
    say(f"static forward M={M} n={n} m={m} r={r} (workspace {ws.numel()} B)")
    h0, u0 = Q.linear_fwd(x, q, A, B, s, workspace=ws)
    h1 = torch.empty_like(h0)
    u1 = torch.empty_like(u0)
    Q.linear_fwd_static(x, q, A, B, s, h1, u1)
    torch.cuda.synchronize()
    Q.linear_check(Q.QLORA_OP_FWD, M, n, m, r, None)
    fits = ws.numel() <= SCRATCH
    if fits:
        assert torch.equal(h0, h1), "h differs from qlora_linear_fwd"
        assert torch.equal(u0, u1), "u differs from qlora_linear_fwd"
    else:
        assert_close(f64(host_bits(h1)), f64(host_bits(h0)), "h against qlora_linear_fwd")
        assert torch.equal(u0, u1), "u differs from qlora_linear_fwd"
    if oracle:
        ref = oracle_full(inp["W"], inp["x"], None, inp["A"], inp["B"], s)
        assert_close(f64(host_bits(h1)), ref["h"], "static h")
        assert_close(u1.cpu().numpy(), ref["u"], "static u")
    return fits


def test_static_forward_shrinking_calls(Q):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # 1: more tiles than CUs with a short last round (K split, counters in the scratch)
    M, n, m = 2304, 512, 8192
    tiles = -(-M // 256) * -(-m // 256)
    say(f"{tiles} tiles on {cus} CUs")
    assert run_pair(Q, M, n, m, 16, 2.0, seed=11)
    # 2: smaller, few tiles (K pieces in the scratch, over the first call's contents)
    assert run_pair(Q, 200, 2048, 3001, 16, 2.0, seed=12)
    # 3: smaller still, the weight-streaming path
    assert run_pair(Q, 16, 1024, 700, 8, 0.5, seed=13)


def test_static_forward_layout_larger_than_scratch(Q):
    # 64 tiles x 4 K pieces fill 64 MiB of K-split planes: with the split
    # partials the layout is larger than the scratch, so the GEMM runs whole
    M, n, m, r = 512, 2048, 8192, 16
    need = Q.workspace_bytes(Q.QLORA_OP_FWD, M, n, m, r)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if need <= SCRATCH:
        pytest.skip(f"layout {need} B fits the scratch on {cus} CUs")
    assert not run_pair(Q, M, n, m, r, 2.0, seed=14, oracle=False)
    # and a smaller call after it, back on the full layout
    assert run_pair(Q, 64, 1024, 1500, 32, 1.0, seed=15)


def test_static_forward_records_no_events(Q):
    # with library profiling switched on, the allocation-free call records no
    # events (creating them would allocate); the workspace call still does
    M, n, m, r = 512, 1024, 1024, 16
    inp, q, x, A, B = layer(Q, M, n, m, r, seed=21)
    h = torch.empty((M, m), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((M, r), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(Q.workspace_bytes(Q.QLORA_OP_FWD, M, n, m, r), 256), dtype=torch.uint8, device="cuda")
    say("static forward with profiling on")
    Q.profile_enable(True)
    try:
        Q.linear_fwd_static(x, q, A, B, 2.0, h, u)
        torch.cuda.synchronize()
        assert Q.profile_query("fwd_gemm") == (0, 0.0)
        assert Q.profile_query("down_proj") == (0, 0.0)
        Q.linear_fwd(x, q, A, B, 2.0, h=h, u=u, workspace=ws)
        torch.cuda.synchronize()
        assert Q.profile_query("fwd_gemm")[0] == 1
    finally:
        Q.profile_enable(False)
    ref = oracle_full(inp["W"], inp["x"], None, inp["A"], inp["B"], 2.0)
    assert_close(f64(host_bits(h)), ref["h"], "h")
