"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bit-exact: quantizer codes, 8-bit constants, c2 and the dequantized bf16
weight.  Within tolerance (relative L2 <= 1e-2 and max-abs <= 2e-2 max|ref|):
h, u, grad_x, grad_A, grad_B.  Small and ragged shapes are checked on every
output; the full-size layers are checked on every quantizer output and on
sampled rows / columns of the float outputs, computed by the oracle.
"""

import numpy as np
import pytest
import torch

import qlora_inputs as QI
from oracle import qlora_oracle as O
from parity_utils import assert_close, dev_bf16, f64, host_bits, oracle_full, sample_indices

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import bit_quantized_fine_qlora_amd as lib
    lib._lib.load()
    return lib


def say(msg):
    print(f"[case] {msg}", flush=True)


def run_gpu(Q, W, x_bits, g_bits, A_bits, B_bits, s, need_bwd=True):
    Wd = torch.from_numpy(W).to("cuda")
    q = Q.quantize_nf4_dq(Wd)
    x, A, B = dev_bf16(x_bits), dev_bf16(A_bits), dev_bf16(B_bits)
    h, u = Q.linear_fwd(x, q, A, B, s)
    out = dict(q=q, h=h, u=u)
    if need_bwd:
        g = dev_bf16(g_bits)
        gx, gA, gB = Q.linear_bwd(x, g, q, A, B, s, u=u)
        out.update(grad_x=gx, grad_A=gA, grad_B=gB, x=x, g=g, A=A, B=B)
    torch.cuda.synchronize()
    return out


def check_quantizer(q, qw):
    assert np.array_equal(q.codes.cpu().numpy(), qw["codes"]), "codes differ"
    assert np.array_equal(q.absmax8.cpu().numpy(), qw["absmax8"]), "absmax8 differ"
    assert np.array_equal(q.c2.cpu().numpy().view(np.uint32), qw["c2"].view(np.uint32)), "c2 differ"


def check_full(Q, W, inp, s, need_bwd=True, label=""):
    ref = oracle_full(W, inp["x"], inp["g"] if need_bwd else None, inp["A"], inp["B"], s)
    say(f"{label} gpu run shape W={W.shape} x={inp['x'].shape} r={inp['A'].shape[0]}")
    got = run_gpu(Q, W, inp["x"], inp["g"], inp["A"], inp["B"], s, need_bwd)
    check_quantizer(got["q"], ref["qw"])
    deq = host_bits(Q.dequant_nf4_dq(got["q"]))
    want = O.dequant_nf4_dq(ref["qw"]["codes"], ref["qw"]["absmax8"], ref["qw"]["c2"], W.size).reshape(W.shape)
    assert np.array_equal(deq, want), "dequantized bf16 weight differs"
    assert_close(f64(host_bits(got["h"])), ref["h"], f"{label} h")
    assert_close(got["u"].cpu().numpy(), ref["u"], f"{label} u")
    if need_bwd:
        assert_close(f64(host_bits(got["grad_x"])), ref["grad_x"], f"{label} grad_x")
        assert_close(f64(host_bits(got["grad_A"])), ref["grad_A"], f"{label} grad_A")
        assert_close(f64(host_bits(got["grad_B"])), ref["grad_B"], f"{label} grad_B")
    return got, ref


# ------------------------------------------------------------------ small

def test_config1_full(Q):
    L = QI.WORKLOADS[1]["layers"][0]
    inp = QI.layer_inputs(1, L)
    got, ref = check_full(Q, inp["W"], inp, L.s, label="config1")
    # u recomputed inside the backward gives the same bits
    say("config1 bwd with u recomputed")
    gx2, gA2, gB2 = Q.linear_bwd(got["x"], got["g"], got["q"], got["A"], got["B"], L.s, u=None)
    torch.cuda.synchronize()
    assert torch.equal(gx2, got["grad_x"]) and torch.equal(gA2, got["grad_A"]) and torch.equal(gB2, got["grad_B"])
    # determinism: a second run gives identical bits
    say("config1 determinism")
    again = run_gpu(Q, inp["W"], inp["x"], inp["g"], inp["A"], inp["B"], L.s)
    for k in ("h", "u", "grad_x", "grad_A", "grad_B"):
        assert torch.equal(again[k], got[k]), k
    # skipping grad_x leaves the adapter gradients unchanged
    _, gA3, gB3 = Q.linear_bwd(got["x"], got["g"], got["q"], got["A"], got["B"], L.s, u=got["u"],
                               need_grad_x=False)
    torch.cuda.synchronize()
    assert torch.equal(gA3, got["grad_A"]) and torch.equal(gB3, got["grad_B"])


RAGGED = [
    # (M, n, m, r, s)
    (17, 192, 200, 5, 1.5),
    (1, 64, 1, 1, 2.0),
    (300, 320, 300, 128, 0.125),
    (600, 1024, 700, 16, 2.0),
    (513, 256, 520, 24, 0.75),
    (64, 128, 72, 64, 0.25),
    (257, 448, 259, 7, 3.0),
    (200, 256, 1000, 32, 1.0),
    (77, 128, 333, 8, 2.0),
    # the single-read g pass sized by M (r % 8 = 0, r <= 32): one 64-token
    # sub-tile per workgroup with more than 8 v partials (the 16-wide planes
    # sum), two sub-tiles at 32 ranks (likewise), one at 24 ranks
    (64, 256, 2100, 16, 2.0),
    (100, 320, 1500, 32, 1.5),
    (40, 256, 300, 24, 0.5),
]


@pytest.mark.parametrize("M,n,m,r,s", RAGGED)
def test_ragged_shapes(Q, M, n, m, r, s):
    inp = QI.custom_inputs(seed=M * 7 + m, M=M, n=n, m=m, r=r)
    check_full(Q, inp["W"], inp, s, label=f"ragged M={M} n={n} m={m} r={r}")


def _random_shapes(count, seed):
    """Seeded shapes over both forward paths: M in 1..640, n a multiple of 64
    up to 1536, m in 1..1200, r in 1..128."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        M = int(rng.integers(1, 33)) if i % 3 == 0 else int(rng.integers(33, 641))
        out.append((M, 64 * int(rng.integers(1, 25)), int(rng.integers(1, 1201)), int(rng.integers(1, 129)),
                    float(rng.choice([0.25, 0.5, 1.0, 2.0, 3.0]))))
    return out


RANDOM_SHAPES = _random_shapes(12, 2026)


@pytest.mark.parametrize("M,n,m,r,s", RANDOM_SHAPES)
def test_random_shapes(Q, M, n, m, r, s):
    inp = QI.custom_inputs(seed=M + 3 * n + 5 * m + 7 * r, M=M, n=n, m=m, r=r)
    check_full(Q, inp["W"], inp, s, label=f"random M={M} n={n} m={m} r={r}")


K_SPLIT = [
    # (M, n, m, r, s): more 256 x 256 output tiles than CUs, with at most half
    # a round left over: those last tiles run as two K halves whose fp32 sums
    # meet in the workspace (ragged edges and two LoRA steps in the second)
    (2304, 512, 8192, 16, 2.0),
    (2400, 640, 7000, 40, 0.5),
]


@pytest.mark.parametrize("M,n,m,r,s", K_SPLIT)
def test_k_split_last_round(Q, M, n, m, r, s):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-M // 256) * -(-m // 256)
    rem = tiles % cus
    if not (tiles > cus and 0 < rem <= cus // 2):
        pytest.skip(f"{tiles} tiles on {cus} CUs: no K split")
    lib = Q._lib.load()
    assert lib.qlora_workspace_bytes(0, M, n, m, r) >= rem * 256 * 256 * 4, "split partials not in the workspace"
    inp = QI.custom_inputs(seed=M + 3 * m + r, M=M, n=n, m=m, r=r)
    got, _ = check_full(Q, inp["W"], inp, s, need_bwd=False, label=f"k-split M={M} n={n} m={m} r={r}")
    say("k-split determinism")
    x, A, B = dev_bf16(inp["x"]), dev_bf16(inp["A"]), dev_bf16(inp["B"])
    ws = torch.empty(Q.workspace_bytes(Q.QLORA_OP_FWD, M, n, m, r), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        h2, u2 = Q.linear_fwd(x, got["q"], A, B, s, workspace=ws)
        torch.cuda.synchronize()
        # no hand-off wait ran out (the give-up word stayed zero)
        Q.linear_check(Q.QLORA_OP_FWD, M, n, m, r, ws)
        assert torch.equal(h2, got["h"]) and torch.equal(u2, got["u"])


FEW_TILES = [
    # (M, n, m, r, s) with at most half as many 256 x 256 output tiles as
    # CUs: every tile runs as P K pieces whose fp32 planes a second pass adds
    # in piece order.  P (forward / grad_x on 256 CUs): 4 / 5 with ragged
    # features (m % 4 != 0, M m odd); 4 / 9 with two LoRA steps in the last
    # piece; 2 / 16 (P = 2: two halves through the K-split hand-off); 8 / 1
    # (too few K steps to split the grad_x GEMM).
    (200, 2048, 3001, 16, 2.0),
    (96, 2048, 5000, 40, 0.5),
    (256, 1024, 8192, 8, 1.0),
    (33, 4096, 512, 16, 2.0),
]


def expected_pieces(M, N, K, cus):
    """K pieces per output tile of the few-tile mode: P = min(CUs / tiles, 16)
    when the tiles fill at most half the CUs, lowered until every piece keeps
    at least 8 K steps of 64.  P = 2 runs as two halves through the K-split
    hand-off (one fp32 plane per tile), P >= 3 as pieces (P planes a tile)."""
    tiles = -(-M // 256) * -(-N // 256)
    if tiles * 2 > cus:
        return 1, tiles
    pc = min(cus // tiles, 16)
    nk = -(-K // 64)
    while pc > 1 and nk // pc < 8:
        pc -= 1
    return pc, tiles


def few_tile_planes(pc):
    """fp32 256 x 256 planes per tile in the workspace of a few-tile GEMM."""
    return 1 if pc == 2 else pc


@pytest.mark.parametrize("M,n,m,r,s", FEW_TILES)
def test_k_pieces_few_tiles(Q, M, n, m, r, s):
    lib = Q._lib.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pf, tf = expected_pieces(M, m, n, cus)      # forward: N = m, K = n
    pb, tb = expected_pieces(M, n, m, cus)      # grad_x: N = n, K = m
    if pf == 1 and pb == 1:
        pytest.skip(f"{tf} / {tb} tiles on {cus} CUs: neither GEMM runs in K pieces")
    # each GEMM that runs in pieces keeps P fp32 planes of 256 x 256 per tile
    # in its workspace (one per tile when the two halves meet by hand-off)
    if pf > 1:
        assert lib.qlora_workspace_bytes(0, M, n, m, r) >= few_tile_planes(pf) * tf * 256 * 256 * 4, \
            "forward K-piece planes missing"
    if pb > 1:
        assert lib.qlora_workspace_bytes(1, M, n, m, r) >= few_tile_planes(pb) * tb * 256 * 256 * 4, \
            "grad_x K-piece planes missing"
    say(f"k-pieces: forward P={pf} ({tf} tiles), grad_x P={pb} ({tb} tiles)")
    inp = QI.custom_inputs(seed=7 * M + m + 11 * r, M=M, n=n, m=m, r=r)
    got, _ = check_full(Q, inp["W"], inp, s, label=f"k-pieces M={M} n={n} m={m} r={r}")
    say("k-pieces determinism")
    ws_f = torch.empty(Q.workspace_bytes(Q.QLORA_OP_FWD, M, n, m, r), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(Q.workspace_bytes(Q.QLORA_OP_BWD, M, n, m, r), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        h2, u2 = Q.linear_fwd(got["x"], got["q"], got["A"], got["B"], s, workspace=ws_f)
        gx2, gA2, gB2 = Q.linear_bwd(got["x"], got["g"], got["q"], got["A"], got["B"], s, u=u2, workspace=ws_b)
        torch.cuda.synchronize()
        # two-half GEMMs: no hand-off wait ran out
        Q.linear_check(Q.QLORA_OP_FWD, M, n, m, r, ws_f)
        Q.linear_check(Q.QLORA_OP_BWD, M, n, m, r, ws_b)
        assert torch.equal(h2, got["h"]) and torch.equal(u2, got["u"])
        assert torch.equal(gx2, got["grad_x"]) and torch.equal(gA2, got["grad_A"]) and torch.equal(gB2, got["grad_B"])


SMALL_M = [
    # (M, n, m, r, s) on the weight-streaming path (M <= 32): K chunks of 2048,
    # 256-k pieces per wave, groups of 128 features
    (16, 4096, 1024, 16, 2.0),
    (1, 64, 33, 1, 1.0),
    (32, 4160, 130, 17, 0.5),
    (15, 2112, 257, 64, 0.25),
    (31, 320, 16, 128, 0.125),
    (16, 6144, 384, 7, 3.0),
    (2, 128, 2000, 32, 2.0),
]


@pytest.mark.parametrize("M,n,m,r,s", SMALL_M)
def test_small_token_path(Q, M, n, m, r, s):
    inp = QI.custom_inputs(seed=M * 11 + n + m, M=M, n=n, m=m, r=r)
    got, _ = check_full(Q, inp["W"], inp, s, label=f"small-M M={M} n={n} m={m} r={r}")
    # the feature-group finishers' wait for u never ran out, and a rerun on
    # the same workspace (its counters left from the last call) gives the same bits
    say("small-M rerun on one workspace")
    ws = torch.empty(Q.workspace_bytes(Q.QLORA_OP_FWD, M, n, m, r), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        h2, u2 = Q.linear_fwd(got["x"], got["q"], got["A"], got["B"], s, workspace=ws)
        torch.cuda.synchronize()
        Q.linear_check(Q.QLORA_OP_FWD, M, n, m, r, ws)
        assert torch.equal(h2, got["h"]) and torch.equal(u2, got["u"])


def grouped_case(Q, M, shapes, seed):
    layers, singles = [], []
    for i, (n, m, r, s) in enumerate(shapes):
        inp = QI.custom_inputs(seed=seed + i, M=M, n=n, m=m, r=r)
        q = Q.quantize_nf4_dq(torch.from_numpy(inp["W"]).to("cuda"))
        x, A, B = dev_bf16(inp["x"]), dev_bf16(inp["A"]), dev_bf16(inp["B"])
        layers.append((x, q, A, B, s))
        singles.append((inp, s))
    say(f"grouped forward M={M} layers={len(shapes)}")
    outs = Q.linear_fwd_grouped(layers)
    torch.cuda.synchronize()
    for (x, q, A, B, s), (h, u), (inp, _) in zip(layers, outs, singles):
        h1, u1 = Q.linear_fwd(x, q, A, B, s)
        torch.cuda.synchronize()
        assert torch.equal(h, h1) and torch.equal(u, u1), "grouped and single-layer results differ"
        W = inp["W"]
        ref = oracle_full(W, inp["x"], None, inp["A"], inp["B"], s)
        assert_close(f64(host_bits(h)), ref["h"], f"grouped h {W.shape}")
        assert_close(u.cpu().numpy(), ref["u"], f"grouped u {W.shape}")


def test_grouped_forward_small_tokens(Q):
    grouped_case(Q, 16, [(4096, 512, 16, 2.0), (1024, 64, 8, 1.0), (2112, 300, 16, 2.0), (256, 1024, 32, 0.5),
                         (64, 16, 1, 4.0), (6144, 128, 64, 0.25), (512, 2048, 16, 2.0)], seed=700)


def test_grouped_forward_large_tokens(Q):
    grouped_case(Q, 72, [(256, 320, 16, 2.0), (512, 64, 8, 1.0)], seed=800)


def test_grouped_full_block_matches_single_layers(Q):
    # the seven layers of the 8B-shaped block at 16 tokens, in one grouped call
    cfg = QI.WORKLOADS[4]
    gen = torch.Generator(device="cuda").manual_seed(4)
    layers = []
    for L in cfg["layers"]:
        W = torch.randn((L.m, L.n), generator=gen, device="cuda", dtype=torch.float32) * L.w_sigma
        q = Q.quantize_nf4_dq(W)
        del W
        x = torch.randn((L.M, L.n), generator=gen, device="cuda").to(torch.bfloat16)
        A = (torch.randn((L.r, L.n), generator=gen, device="cuda") / 16).to(torch.bfloat16)
        B = (torch.randn((L.m, L.r), generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
        layers.append((x, q, A, B, L.s))
    say("grouped 8B block forward")
    outs = Q.linear_fwd_grouped(layers)
    torch.cuda.synchronize()
    for (x, q, A, B, s), (h, u) in zip(layers, outs):
        h1, u1 = Q.linear_fwd(x, q, A, B, s)
        torch.cuda.synchronize()
        # every partial sum (per K chunk, wave quarter and piece) is taken in
        # the same order whatever else shares the launch: identical bits
        assert torch.equal(u, u1), "grouped vs single u"
        assert torch.equal(h, h1), "grouped vs single h"
    # a repeated grouped call gives identical bits
    again = Q.linear_fwd_grouped(layers)
    torch.cuda.synchronize()
    for (h, u), (h2, u2) in zip(outs, again):
        assert torch.equal(h, h2) and torch.equal(u, u2)
    del layers, outs, again
    torch.cuda.empty_cache()


def test_every_e4m3_scale_code(Q):
    # the 8-bit block constants take every finite non-negative E4M3 code
    # (0x00 .. 0x7e, subnormals included) with random codes: the dequantized
    # weight is bit-exact and the forward (16 tokens: weight streaming; 96:
    # tiled GEMM) and backward match the oracle on the same constants
    m, n, r, s = 128, 256, 16, 2.0
    rng = np.random.default_rng(77)
    nblk = m * n // 64
    absmax8 = (np.arange(nblk) % 0x7F).astype(np.uint8)
    c2 = np.array([1.5, 0.75], dtype=np.float32)
    codes = rng.integers(0, 256, size=m * n // 2, dtype=np.uint8)
    q = Q.QuantizedWeight(codes=torch.from_numpy(codes).cuda(), absmax8=torch.from_numpy(absmax8).cuda(),
                          c2=torch.from_numpy(c2).cuda(), m=m, n=n)
    say("dequant with every E4M3 code")
    want = O.dequant_nf4_dq(codes, absmax8, c2, m * n)
    assert np.array_equal(host_bits(Q.dequant_nf4_dq(q)).reshape(-1), want), "dequantized bf16 weight differs"
    Wd = f64(want).reshape(m, n)
    for M in (16, 96):
        inp = QI.custom_inputs(seed=500 + M, M=M, n=n, m=m, r=r)
        x, g, A, B = dev_bf16(inp["x"]), dev_bf16(inp["g"]), dev_bf16(inp["A"]), dev_bf16(inp["B"])
        say(f"every E4M3 code, M={M}")
        h, u = Q.linear_fwd(x, q, A, B, s)
        gx, gA, gB = Q.linear_bwd(x, g, q, A, B, s, u=u)
        torch.cuda.synchronize()
        xf, gf, Af, Bf = f64(inp["x"]), f64(inp["g"]), f64(inp["A"]), f64(inp["B"])
        h_ref, u_ref = O.linear_fwd(xf, Wd, Af, Bf, s)
        bw = O.linear_bwd(xf, gf, Wd, Af, Bf, s, u=u_ref)
        assert_close(f64(host_bits(h)), h_ref, f"M={M} h")
        assert_close(f64(host_bits(gx)), bw["grad_x"], f"M={M} grad_x")
        assert_close(f64(host_bits(gA)), bw["grad_A"], f"M={M} grad_A")
        assert_close(f64(host_bits(gB)), bw["grad_B"], f"M={M} grad_B")


def test_adapter_b_zero(Q):
    # B = 0 (the adapter's initial state): h is the plain dequant GEMM, grad_A is exactly 0
    inp = QI.custom_inputs(seed=3, M=96, n=256, m=320, r=16)
    inp["B"] = np.zeros_like(inp["B"])
    got, ref = check_full(Q, inp["W"], inp, 2.0, label="B=0")
    assert not torch.any(got["grad_A"].float() != 0)


def test_weight_zero_pure_adapter(Q):
    # W0 = 0: every code is 7 with a zero scale, so h = s u B^T and grad_x = s v A alone
    inp = QI.custom_inputs(seed=4, M=80, n=192, m=144, r=8)
    inp["W"] = np.zeros_like(inp["W"])
    inp["B"] = QI.to_bf16_bits(QI.bf16_bits_as_f32(inp["B"]) * 50.0)
    got, ref = check_full(Q, inp["W"], inp, 2.0, label="W0=0")
    assert np.all(O.unpack_codes(got["q"].codes.cpu().numpy(), inp["W"].size) == 7)


def test_zero_blocks_and_partial_group(Q):
    inp = QI.custom_inputs(seed=5, M=40, n=192, m=100, r=4)   # 19200 weights: 1 full + 1 partial group
    W = inp["W"]
    W[3, 64:128] = 0.0                 # one all-zero block
    W[7, :] = 0.0                      # a whole zero row
    W[9, 5] = 0.0                      # an isolated exact zero
    check_full(Q, W, inp, 1.0, label="zero blocks")


def test_quantizer_threshold_boundaries(Q):
    # normalized weights placed exactly on, and one ulp around, every threshold,
    # with random block absmax values; plus tiny and denormal weights
    rng = np.random.default_rng(21)
    nblk = 4096
    W = np.empty((nblk, 64), dtype=np.float32)
    T = O.NF4_T
    for b in range(nblk):
        c = np.float32(np.exp2(rng.uniform(-20, 10)) * (1 + rng.random()))
        t = T[rng.integers(0, 15, size=63)]
        k = rng.integers(-2, 3, size=63)
        tk = (t.view(np.int32) + k.astype(np.int32)).view(np.float32)
        tk = np.where(t == 0, np.float32(0), tk)
        sign = np.where(rng.random(63) < 0.5, -1, 1).astype(np.float32)
        w = (tk * sign * c).astype(np.float32)
        W[b, 0] = c if b % 2 else -c
        W[b, 1:] = np.clip(w, -c, c)
    W[10, 5] = np.float32(1e-40)       # denormal
    W[11, 1:] = np.float32(3e-39)
    W[12, :] = np.float32(1e-38)
    W[13, 1:] = W[13, 1:] * np.float32(1e-30)
    W = W.reshape(256, -1)
    say("threshold boundary quantize")
    q = Q.quantize_nf4_dq(torch.from_numpy(W).to("cuda"))
    torch.cuda.synchronize()
    check_quantizer(q, O.quantize_nf4_dq(W))


# ------------------------------------------------------------------ uniform 4-bit grid

UNIFORM4 = [(64, 256), (333, 192), (14336, 4096)]


@pytest.mark.parametrize("m,n", UNIFORM4)
def test_uniform4_quantizer(Q, m, n):
    # the comparison grid through the same quantizer and dequantizer: bit-exact
    inp = QI.custom_inputs(seed=m + 2 * n, M=1, n=n, m=m, r=1)
    W = inp["W"]
    table = O.uniform4_table()
    say(f"uniform4 quantize {m}x{n}")
    q = Q.quantize_dq(torch.from_numpy(W).cuda(), qtype=Q.QTYPE_UNIFORM4)
    torch.cuda.synchronize()
    qw = O.quantize_nf4_dq(W, table=table)
    check_quantizer(q, qw)
    deq = host_bits(Q.dequant_dq(q, qtype=Q.QTYPE_UNIFORM4)).reshape(-1)
    want = O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size, table=table)
    assert np.array_equal(deq, want), "uniform4 dequantized weight differs"
    if m * n >= 1 << 20:
        # the pages' claim with the GPU kernels: NF4 round trip beats the uniform grid
        w64 = W.reshape(-1).astype(np.float64)
        qn = Q.quantize_dq(torch.from_numpy(W).cuda(), qtype=Q.QTYPE_NF4)
        e_nf4 = np.linalg.norm(f64(host_bits(Q.dequant_dq(qn)).reshape(-1)) - w64) / np.linalg.norm(w64)
        e_uni = np.linalg.norm(f64(deq) - w64) / np.linalg.norm(w64)
        say(f"round-trip rel-L2: nf4 {e_nf4:.5f}, uniform4 {e_uni:.5f}")
        assert e_nf4 < e_uni
        del qn
    del q
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m,n", UNIFORM4)
def test_edge_mean_quantizer(Q, m, n):
    # the edge-mean (quantile-average) table through the same kernels: bit-exact
    inp = QI.custom_inputs(seed=m + 3 * n, M=1, n=n, m=m, r=1)
    W = inp["W"]
    table = O.edge_mean_table()
    say(f"edge-mean quantize {m}x{n}")
    q = Q.quantize_dq(torch.from_numpy(W).cuda(), qtype=Q.QTYPE_EDGE_MEAN4)
    torch.cuda.synchronize()
    qw = O.quantize_nf4_dq(W, table=table)
    check_quantizer(q, qw)
    deq = host_bits(Q.dequant_dq(q, qtype=Q.QTYPE_EDGE_MEAN4)).reshape(-1)
    want = O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size, table=table)
    assert np.array_equal(deq, want), "edge-mean dequantized weight differs"
    del q
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m,n", UNIFORM4)
def test_int4_quantizer(Q, m, n):
    # the INT4 absmax grid through the same kernels: bit-exact codes,
    # constants and dequantized weight (both zeros included)
    inp = QI.custom_inputs(seed=m + 5 * n, M=1, n=n, m=m, r=1)
    W = inp["W"]
    if m == 333:
        W[7, :64] = 0.0            # an all-zero block: every weight takes the -0 level
        W[9, 5] = 0.0              # an exact zero in a normal block
    table = O.int4_table()
    say(f"int4 quantize {m}x{n}")
    q = Q.quantize_dq(torch.from_numpy(W).cuda(), qtype=Q.QTYPE_INT4)
    torch.cuda.synchronize()
    qw = O.quantize_nf4_dq(W, table=table)
    check_quantizer(q, qw)
    deq = host_bits(Q.dequant_dq(q, qtype=Q.QTYPE_INT4)).reshape(-1)
    want = O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], W.size, table=table)
    assert np.array_equal(deq, want), "int4 dequantized weight differs"
    if m * n >= 1 << 20:
        # the pages' comparison with the GPU kernels: NF4 round trip beats INT4
        w64 = W.reshape(-1).astype(np.float64)
        qn = Q.quantize_dq(torch.from_numpy(W).cuda(), qtype=Q.QTYPE_NF4)
        e_nf4 = np.linalg.norm(f64(host_bits(Q.dequant_dq(qn)).reshape(-1)) - w64) / np.linalg.norm(w64)
        e_int4 = np.linalg.norm(f64(deq) - w64) / np.linalg.norm(w64)
        say(f"round-trip rel-L2: nf4 {e_nf4:.5f}, int4 {e_int4:.5f}")
        assert e_nf4 < e_int4
        del qn
    del q
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ grouped quantization

GROUPED_SHAPES = [(256, 256), (203, 4160), (1, 64), (1000, 1024), (17, 960), (64, 256), (333, 192), (4, 4096)]


@pytest.mark.parametrize("qtype", [0, 3])
def test_grouped_quantizer_small(Q, qtype):
    # eight weights in one launch (ragged last groups, a one-block weight, an
    # all-zero block, an exact zero, a subnormal): bit-exact against the
    # oracle and against one call per weight
    table = None if qtype == 0 else O.int4_table()
    Ws = []
    for i, (m, n) in enumerate(GROUPED_SHAPES):
        W = QI.custom_inputs(seed=700 + i, M=1, n=n, m=m, r=1)["W"]
        if i == 1:
            W[0, :64] = 0.0
            W[2, 5] = 0.0
            W[3, 7] = 1e-39
        Ws.append(W)
    dWs = [torch.from_numpy(W).cuda() for W in Ws]
    say(f"grouped quantize qtype {qtype}: {len(Ws)} weights")
    qs = Q.quantize_dq_grouped(dWs, qtype=qtype)
    torch.cuda.synchronize()
    for W, dW, q in zip(Ws, dWs, qs):
        qw = O.quantize_nf4_dq(W, table=table)
        check_quantizer(q, qw)
        one = Q.quantize_dq(dW, qtype=qtype)
        assert torch.equal(one.codes, q.codes) and torch.equal(one.absmax8, q.absmax8)
        assert torch.equal(one.c2.view(torch.int32), q.c2.view(torch.int32))
    # fewer weights into the same outputs: the same bits again
    again = Q.quantize_dq_grouped(dWs[:3], qtype=qtype, outs=qs[:3])
    torch.cuda.synchronize()
    for W, q in zip(Ws[:3], again):
        qw = O.quantize_nf4_dq(W, table=table)
        check_quantizer(q, qw)


def test_grouped_quantizer_8b_block(Q):
    # the 8B-shaped block's seven weights in one launch = one call per weight,
    # bit for bit (the single-weight path is checked against the oracle at
    # these sizes elsewhere); the k weight also against the oracle directly
    layers = QI.WORKLOADS[4]["layers"]
    gen = torch.Generator(device="cuda").manual_seed(44)
    dWs = [torch.randn((L.m, L.n), generator=gen, device="cuda").mul_(L.w_sigma) for L in layers]
    say("grouped quantize 8B block (7 weights)")
    qs = Q.quantize_dq_grouped(dWs)
    torch.cuda.synchronize()
    for L, dW, q in zip(layers, dWs, qs):
        one = Q.quantize_nf4_dq(dW)
        assert torch.equal(one.codes, q.codes), L.name
        assert torch.equal(one.absmax8, q.absmax8), L.name
        assert torch.equal(one.c2.view(torch.int32), q.c2.view(torch.int32)), L.name
        del one
    k = [i for i, L in enumerate(layers) if L.name == "k"][0]
    check_quantizer(qs[k], O.quantize_nf4_dq(dWs[k].cpu().numpy()))
    del qs, dWs
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ adapter merge

def bf16_order(bits):
    b = np.asarray(bits).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def check_merge(got_bits, want_bits, what):
    # the kernel's fp32 sum differs from the exact one by far less than half a
    # bf16 unit, so its rounding is the exact one or a neighbour
    d = np.abs(bf16_order(got_bits) - bf16_order(want_bits))
    assert d.max() <= 1, f"{what}: {int(d.max())} bf16 units off"
    assert np.mean(d == 0) >= 0.99, f"{what}: only {np.mean(d == 0):.4f} exact"


MERGE = [
    # (m, n, r, s)
    (256, 256, 8, 2.0),
    (333, 192, 5, 0.5),
    (64, 640, 128, 0.25),
    (1, 64, 1, 1.0),
    (100, 128, 32, 3.0),
]


@pytest.mark.parametrize("m,n,r,s", MERGE)
def test_merge_adapter(Q, m, n, r, s):
    inp = QI.custom_inputs(seed=7 * m + n + r, M=1, n=n, m=m, r=r)
    qw = O.quantize_nf4_dq(inp["W"])   # oracle codes, uploaded as the kernel's input
    q = Q.QuantizedWeight(codes=torch.from_numpy(qw["codes"]).cuda(), absmax8=torch.from_numpy(qw["absmax8"]).cuda(),
                          c2=torch.from_numpy(qw["c2"]).cuda(), m=m, n=n)
    Wd_bits = O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], m * n)
    A, B = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    say(f"merge m={m} n={n} r={r}")
    got = host_bits(Q.merge_adapter(q, A, B, s)).reshape(m, n)
    check_merge(got, O.merge_adapter(Wd_bits, inp["A"], inp["B"], s, m, n), f"merge {m}x{n} r={r}")
    # a zero adapter (B = 0, or s = 0) leaves the dequantized weight bit for bit
    got0 = host_bits(Q.merge_adapter(q, A, torch.zeros_like(B), s)).reshape(-1)
    assert np.array_equal(got0, Wd_bits), "merge with B = 0 differs from W'"
    got1 = host_bits(Q.merge_adapter(q, A, B, 0.0)).reshape(-1)
    assert np.array_equal(got1, Wd_bits), "merge with s = 0 differs from W'"


def test_merge_adapter_full_size_gate(Q):
    # the gate projection of the 8B-shaped block (14336 x 4096, r = 16), rows sampled
    L = QI.WORKLOADS[2]["layers"][0]
    inp = QI.layer_inputs(2, L, tensors=("W", "A", "B"))
    say(f"merge full size {L.m}x{L.n}: oracle quantize")
    qw = O.quantize_nf4_dq(inp["W"])
    q = Q.QuantizedWeight(codes=torch.from_numpy(qw["codes"]).cuda(), absmax8=torch.from_numpy(qw["absmax8"]).cuda(),
                          c2=torch.from_numpy(qw["c2"]).cuda(), m=L.m, n=L.n)
    A, B = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    say("merge full size: gpu")
    Wm = Q.merge_adapter(q, A, B, L.s)
    rows = sample_indices(L.m, 128, 4242)
    got = host_bits(Wm[torch.from_numpy(rows).cuda()])
    Wr_bits = O.bf16_bits_rne_f64(O.dequant_rows(qw, L.m, L.n, rows)).reshape(-1)
    want = O.merge_adapter(Wr_bits, inp["A"], inp["B"][rows], L.s, len(rows), L.n)
    check_merge(got, want, "merge full-size gate (sampled rows)")
    del Wm, q
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ full size

def oracle_rows_for(W, rows):
    """W'[rows] from the oracle's own quantization of the whole weight."""
    m, n = W.shape
    qw = O.quantize_nf4_dq(W)
    return qw, O.dequant_rows(qw, m, n, rows)


def full_layer_case(Q, cfg, layer, need_bwd):
    L = layer
    say(f"config{cfg} {L.name} {L.m}x{L.n} M={L.M} r={L.r}: drawing inputs")
    inp = QI.layer_inputs(cfg, L, tensors=("W", "x", "g", "A", "B") if need_bwd else ("W", "x", "A", "B"))
    W = inp["W"]
    say(f"config{cfg} {L.name}: gpu quantize/fwd/bwd")
    got = run_gpu(Q, W, inp["x"], inp.get("g"), inp["A"], inp["B"], L.s, need_bwd)
    say(f"config{cfg} {L.name}: oracle quantize")
    qw = O.quantize_nf4_dq(W)
    check_quantizer(got["q"], qw)
    rows = sample_indices(L.m, 96, 1000 * cfg + L.index)
    toks = sample_indices(L.M, 48, 2000 * cfg + L.index)
    cols = sample_indices(L.n, 96, 3000 * cfg + L.index)
    Wr = O.dequant_rows(qw, L.m, L.n, rows)
    deq = Q.dequant_nf4_dq(got["q"])
    deq_rows = host_bits(deq[torch.from_numpy(rows).cuda()])
    assert np.array_equal(f64(deq_rows), Wr), "dequantized rows differ"
    del deq
    x = f64(inp["x"])
    A = f64(inp["A"])
    B = f64(inp["B"])
    u_t = x[toks] @ A.T
    h_ref = x[toks] @ Wr.T + L.s * (u_t @ B[rows].T)
    h_got = f64(host_bits(got["h"][torch.from_numpy(toks).cuda()][:, torch.from_numpy(rows).cuda()]))
    assert_close(h_got, h_ref, f"config{cfg} {L.name} h (sampled)")
    assert_close(got["u"][torch.from_numpy(toks).cuda()].cpu().numpy(), u_t, f"config{cfg} {L.name} u (sampled)")
    if not need_bwd:
        return
    say(f"config{cfg} {L.name}: oracle backward on samples")
    g = f64(inp["g"])
    Wc = O.dequant_cols(qw, L.m, L.n, cols)
    v = g @ B
    u = x @ A.T
    gx_ref = g[toks] @ Wc + L.s * (v[toks] @ A[:, cols])
    gA_ref = L.s * (v.T @ x[:, cols])
    gB_ref = L.s * (g[:, rows].T @ u)
    tc, cc, rc = (torch.from_numpy(a).cuda() for a in (toks, cols, rows))
    assert_close(f64(host_bits(got["grad_x"][tc][:, cc])), gx_ref, f"config{cfg} {L.name} grad_x (sampled)")
    assert_close(f64(host_bits(got["grad_A"][:, cc])), gA_ref, f"config{cfg} {L.name} grad_A (sampled)")
    assert_close(f64(host_bits(got["grad_B"][rc])), gB_ref, f"config{cfg} {L.name} grad_B (sampled)")


FULL = [(2, L) for L in QI.WORKLOADS[2]["layers"]] + [(3, L) for L in QI.WORKLOADS[3]["layers"]] \
    + [(4, L) for L in QI.WORKLOADS[4]["layers"]] + [(5, L) for L in QI.WORKLOADS[5]["layers"]]


@pytest.mark.parametrize("cfg,layer", FULL, ids=[f"cfg{c}-{L.name}" for c, L in FULL])
def test_full_size_layer(Q, cfg, layer):
    full_layer_case(Q, cfg, layer, need_bwd=QI.WORKLOADS[cfg]["backward"])
    torch.cuda.empty_cache()
