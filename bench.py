"""Benchmark of the QLoRA adapted-linear hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input, already
resident in HBM, on the 70B-shaped transformer block (hidden 8192, FFN
28672, 64 query / 8 KV heads of dim 128; q 8192x8192, k and v 1024x8192,
o 8192x8192, gate and up 28672x8192, down 8192x28672), 8192 tokens (batch 8
x seq 1024), LoRA r = 64, alpha = 16 on all seven projections:
  - quantize the seven frozen weights (NF4 + double quantization), in one
    grouped launch;
  - forward of every layer (u = x A^T, h = x W'^T + s u B^T);
  - backward of every layer, in reverse order (grad_x, grad_A, grad_B).
Every layer has its own independent x and upstream gradient g.

value = algorithmic forward + backward flops of the seven layers per step
(2.855e13) / step time, the quantizer's time included in the step.  The
timed steps run with the library's kernel timing off; per-kernel times come
from a separate pass, layer by layer, with HIP events recorded on the stream
the library launches on.  Prints one JSON line.

Besides the timed steps (and outside them) it also measures, each with HIP
events on the stream the library launches on:
  - the block's forward pass alone, backward pass alone and quantization;
  - the 8B-shaped gate projection (14336 x 4096, 4096 tokens, r = 16) and
    down projection (4096 x 14336, 4096 tokens, r = 64): forward, backward,
    forward + backward and quantize;
  - the small-token regime: the forward of all seven layers of the
    8B-shaped block at 16 tokens in one grouped call, and the quantization of
    the block's seven weights in one grouped call (one call per weight
    beside it), both against the HBM peak;
  - the adapter merge W_merged = bf16(W' + s B A) of the gate projection,
    against the HBM peak;
  - the adapter optimizer step (Adam, decoupled weight decay) over the
    adapters of a 32-layer 8B-shaped model at r = 16 (448 tensors, 41.9 M
    parameters, 28 bytes each), against the HBM peak, and over one block's
    adapters with the optimizer state in pinned host memory;
  - LoRA dropout on the gate projection, against the plain passes;
  - the quantizer on the uniform 4-bit comparison grid and the edge-mean
    table: round-trip relative error of the gate weight through the GPU
    kernels, and the uniform quantizer's time.
For the HBM-bound measurements the caches are flushed before every
repetition by reading 1 GiB (a read evicts the working set cleanly; a write
flush would leave dirty lines whose write-back lands in the timed kernel).
Inputs are drawn on the device with torch's generator from the same
distributions as the seeded parity inputs (they are timed, not compared).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SPIN_CYCLES = 2_000_000   # torch.cuda._sleep before a timed call: ~1 ms at the shader clock
BF16_PEAK_TFLOPS = 2500.0

# HBM bytes per launch of the dominant GEMM kernels, from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE runs of this script (KiB per dispatch), scaled by
# what the same counters read for a plain 1 GiB device copy (FETCH_SIZE x
# 2.0, WRITE_SIZE x 1.0; see profiles/).  Keyed by "layer/kernel" of the
# 70B-block step.  Valid only for the GEMM sources they were taken on (the
# kernel and the header it includes): reported as null once either changes.
# The counters count the L2's requests to the memory fabric, so bytes served
# by the last-level cache (MALL) are included: an upper bound on HBM bytes.
# The k and v forwards run every tile as two K halves: their writes are h
# plus one fp32 half-sum per tile.
GEMM_SRC = [os.path.join(ROOT, "bit_quantized_fine_qlora_amd", "csrc", f) for f in ("gemm_linear.hip", "qlora_common.h")]
GEMM_TRAFFIC = {
    "src_sha1": "283b6faedb84f1f83fab3cd6ceb33c5641383d8a",
    "q/fwd_gemm": {"fetch": 1297956352, "write": 134244224},
    "k/fwd_gemm": {"fetch": 584374315, "write": 50344448},
    "v/fwd_gemm": {"fetch": 584374699, "write": 50345301},
    "o/fwd_gemm": {"fetch": 1296410965, "write": 134267733},
    "gate/fwd_gemm": {"fetch": 4822930475, "write": 469998379},
    "up/fwd_gemm": {"fetch": 4836978048, "write": 469906688},
    "down/fwd_gemm": {"fetch": 4462792747, "write": 134226005},
    "down/dgrad_gemm": {"fetch": 4603999957, "write": 469812011},
    "up/dgrad_gemm": {"fetch": 4383820459, "write": 134230101},
    "gate/dgrad_gemm": {"fetch": 4383888896, "write": 134230528},
    "o/dgrad_gemm": {"fetch": 1278466347, "write": 134239104},
    "v/dgrad_gemm": {"fetch": 191499520, "write": 134444587},
    "k/dgrad_gemm": {"fetch": 191376171, "write": 134419883},
    "q/dgrad_gemm": {"fetch": 1278483968, "write": 134250923},
}


def gemm_traffic(key):
    import hashlib
    h = hashlib.sha1()
    try:
        for path in GEMM_SRC:
            with open(path, "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    digest = h.hexdigest()
    if digest != GEMM_TRAFFIC["src_sha1"] or key not in GEMM_TRAFFIC:
        return None
    t = GEMM_TRAFFIC[key]
    return int(t["fetch"] + t["write"])


def fwd_flops(M, n, m, r):
    return 2 * M * m * n + 2 * M * r * (m + n)


def bwd_flops(M, n, m, r):
    return 2 * M * m * n + 4 * M * r * (m + n)


def quant_bytes(m, n):
    numel = m * n
    return 4 * numel + numel // 2 + numel // 64 + 4 * ((numel // 64 + 255) // 256)


def small_forward_bytes(layers, M):
    """Algorithmic bytes of a small-token forward: packed weight + x + A + B + h."""
    tot = 0
    for L in layers:
        numel = L.m * L.n
        tot += numel // 2 + numel // 64 + 4 * ((numel // 64 + 255) // 256)
        tot += 2 * (M * L.n + L.r * L.n + L.m * L.r + M * L.m)
    return tot


def timed_us(fn, reps, flush=None):
    """Median and min of `reps` event-timed calls of fn (after one untimed call).
    The GPU is kept busy before the start event (by the flush read, or by a
    spin kernel), so that the host has queued all of fn's launches before the
    GPU reaches the start event: the time is the kernels', not the host's
    launch gaps."""
    import torch
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush.sum()
        else:
            torch.cuda._sleep(SPIN_CYCLES)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def small_token_block(Q, dev, reps):
    """Forward of the 8B-shaped block (7 layers, 16 tokens) and quantization of its weights."""
    import torch

    import qlora_inputs as QI
    cfg = QI.WORKLOADS[4]
    gen = torch.Generator(device=dev).manual_seed(4)
    Ws, layers = [], []
    for L in cfg["layers"]:
        W = torch.randn((L.m, L.n), generator=gen, device=dev, dtype=torch.float32) * L.w_sigma
        q = Q.quantize_nf4_dq(W)
        x = torch.randn((L.M, L.n), generator=gen, device=dev).to(torch.bfloat16)
        A = (torch.randn((L.r, L.n), generator=gen, device=dev) / 16).to(torch.bfloat16)
        B = (torch.randn((L.m, L.r), generator=gen, device=dev) * 0.01).to(torch.bfloat16)
        Ws.append((W, q))
        layers.append((x, q, A, B, L.s))
    M = cfg["layers"][0].M
    grouped = Q.GroupedForward(layers)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    fb = small_forward_bytes(cfg["layers"], M)
    med, mn = timed_us(grouped.run, reps, flush)
    qbytes = sum(quant_bytes(L.m, L.n) for L in cfg["layers"])

    dWs, qs = [W for W, _ in Ws], [q for _, q in Ws]

    def quant_all():
        Q.quantize_dq_grouped(dWs, outs=qs)

    def quant_each():
        for W, q in Ws:
            Q.quantize_nf4_dq(W, out=q)

    qmed, qmn = timed_us(quant_all, max(3, reps // 2), flush)
    qmed1, _ = timed_us(quant_each, max(3, reps // 2), flush)
    return {
        "forward": {"workload": "8B-shaped block: q,k,v,o,gate,up,down, 16 tokens, r=16, one grouped call",
                    "us": round(med, 2), "us_min": round(mn, 2), "bytes": fb,
                    "GB/s": round(fb / (med * 1e-6) / 1e9, 1), "hbm_frac": round(fb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "quantize": {"workload": "the block's seven fp32 weights (218,103,808 params), one grouped call",
                     "us": round(qmed, 2), "bytes": qbytes,
                     "GB/s": round(qbytes / (qmed * 1e-6) / 1e9, 1),
                     "hbm_frac": round(qbytes / (qmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "us_one_call_per_weight": round(qmed1, 2)},
        "cache_flush": "1 GiB read before every repetition",
    }


def merge_bytes(m, n, r):
    """Packed weight read, adapter read, merged bf16 weight written."""
    numel = m * n
    return numel // 2 + numel // 64 + 4 * ((numel // 64 + 255) // 256) + 2 * (r * n + m * r) + 2 * numel


def level_table_variants(Q, W, q, reps):
    """Round-trip error of the gate weight through quantize + dequant for NF4, the
    uniform grid, the edge-mean table and the INT4 absmax grid."""
    import torch
    w = W.double()
    out = {}
    for name, qtype in (("nf4", Q.QTYPE_NF4), ("uniform4", Q.QTYPE_UNIFORM4), ("edge_mean4", Q.QTYPE_EDGE_MEAN4),
                        ("int4", Q.QTYPE_INT4)):
        qq = Q.quantize_dq(W, qtype=qtype)
        d = Q.dequant_dq(qq, qtype=qtype).double()
        out[name] = {"roundtrip_rel_l2": round(float(torch.linalg.norm(d - w) / torch.linalg.norm(w)), 6)}
        del qq, d
    qu = Q.alloc_quantized(q.m, q.n, W.device)
    med, _ = timed_us(lambda: Q.quantize_dq(W, qtype=Q.QTYPE_UNIFORM4, out=qu), reps)
    qb = quant_bytes(q.m, q.n)
    out["uniform4"].update({"quantize_us": round(med, 2), "GB/s": round(qb / (med * 1e-6) / 1e9, 1)})
    out["workload"] = f"gate weight {q.m}x{q.n}, N(0, 0.02^2)"
    out["timing"] = "back-to-back launches, no cache flush (the 235 MB weight partly stays in the 256 MB MALL)"
    return out


def adapter_merge(Q, q, A, B, s, reps):
    """W_merged = bf16(W' + s B A) of one layer, cold caches."""
    import torch
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=q.codes.device)
    med, mn = timed_us(lambda: Q.merge_adapter(q, A, B, s), reps, flush)
    r = A.shape[0]
    mb = merge_bytes(q.m, q.n, r)
    return {"workload": f"gate projection {q.m}x{q.n}, r={r}", "us": round(med, 2), "us_min": round(mn, 2),
            "bytes": mb, "GB/s": round(mb / (med * 1e-6) / 1e9, 1),
            "hbm_frac": round(mb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "cache_flush": "1 GiB read before every repetition"}


ADAM_BYTES_PER_PARAM = 28  # fp32 weight, moments read + written, bf16 grad read, bf16 copy written


def adapter_adam(Q, dev, reps):
    """One Adam step over all adapters of a 32-layer 8B-shaped model, state in HBM;
    and over one block's adapters with the state in pinned host memory."""
    import torch

    import qlora_inputs as QI
    layers = QI.WORKLOADS[4]["layers"]
    shapes = []
    for _ in range(32):
        for L in layers:
            shapes += [L.r * L.n, L.m * L.r]

    def make(counts, host):
        kw = dict(pin_memory=True) if host else dict(device=dev)
        ts = []
        for c in counts:
            p = torch.empty(c, dtype=torch.float32, **kw)
            p.normal_(0, 0.02) if not host else p.copy_(torch.randn(c) * 0.02)
            m = torch.zeros(c, dtype=torch.float32, **kw)
            v = torch.zeros(c, dtype=torch.float32, **kw)
            g = (torch.randn(c, device=dev) * 1e-3).to(torch.bfloat16)
            p16 = torch.empty(c, dtype=torch.bfloat16, device=dev)
            ts.append((p, p16, g, m, v))
        return ts

    out = {}
    ts = make(shapes, False)
    nparam = sum(shapes)
    step = [0]
    plan = [Q.AdamStep(ts)]

    def run():
        step[0] += 1
        plan[0].run(2e-4, 0.9, 0.999, 1e-8, 0.01, step=step[0])

    med, mn = timed_us(run, reps)
    b = nparam * ADAM_BYTES_PER_PARAM
    out["hbm_state"] = {"workload": "Adam step, adapters of 32 layers x 7 projections (r=16), state in HBM",
                        "params": nparam, "tensors": len(shapes), "us": round(med, 2), "us_min": round(mn, 2),
                        "bytes": b, "GB/s": round(b / (med * 1e-6) / 1e9, 1),
                        "hbm_frac": round(b / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del ts
    plan[0] = None
    torch.cuda.empty_cache()
    block = shapes[:14]
    plan[0] = Q.AdamStep(make(block, True))
    step[0] = 0
    med, mn = timed_us(run, max(3, reps // 2))
    nb = sum(block)
    out["host_state"] = {"workload": "Adam step, one block's adapters (14 tensors), weights and moments in pinned "
                                     "host memory, gradient and bf16 copy in HBM",
                         "params": nb, "us": round(med, 2), "GB/s": round(nb * ADAM_BYTES_PER_PARAM / (med * 1e-6) / 1e9, 1)}
    return out


def dropout_passes(Q, x, g, q, A, B, s, h, u, out, ws_f, plain, reps):
    """Forward and backward with dropout p = 0.05 on the adapter input, against
    the plain passes; the fp32 adapter term of grad_x as its own kernel."""
    import torch
    M, n = x.shape
    m, r = q.m, A.shape[0]
    drop = (0.05, 1234, 0)
    ws_bd = torch.empty(Q.workspace_bytes(Q.QLORA_OP_BWD_DROPOUT, M, n, m, r), dtype=torch.uint8, device=x.device)
    fwd = lambda: Q.linear_fwd(x, q, A, B, s, h=h, u=u, workspace=ws_f, dropout=drop)  # noqa: E731
    bwd = lambda: Q.linear_bwd(x, g, q, A, B, s, u=u, out=out, workspace=ws_bd, dropout=drop)  # noqa: E731
    fwd_med, _ = timed_us(fwd, reps)
    bwd_med, _ = timed_us(bwd, reps)
    Q.profile_enable(True)
    for _ in range(reps):
        torch.cuda._sleep(SPIN_CYCLES)
        bwd()
    torch.cuda.synchronize()
    Q.profile_enable(False)
    kern = {}
    for name in ("dropout_term", "dgrad_gemm", "down_proj", "token_grad", "gpass"):
        cnt, tot = Q.profile_query(name)
        if cnt:
            kern[name] = round(tot * 1e3 / cnt, 2)
    # dropout term: v (M r fp32) and A (r n bf16) read, M n fp32 written
    tb = M * r * 4 + r * n * 2 + M * n * 4
    du = kern.get("dropout_term", 0.0)
    return {"workload": f"gate projection {m}x{n}, {M} tokens, r={r}, p=0.05",
            "forward_us": round(fwd_med, 2), "backward_us": round(bwd_med, 2),
            "forward_vs_plain": round(fwd_med / plain["forward"]["us"], 3),
            "backward_vs_plain": round(bwd_med / plain["backward"]["us"], 3),
            "kernels_us": kern,
            "dropout_term": {"bytes": tb, "GB/s": round(tb / (du * 1e-6) / 1e9, 1) if du else None}}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return None


def cpu_baseline(cfg, layers, tokens):
    """Time the oracle (float64 numpy) on a bounded sample of the workload:
    for each of `layers` in turn, the whole weight's quantization and
    dequantization, then its forward and backward on the first `tokens`
    tokens (all of them by default)."""
    import qlora_inputs as QI
    from oracle import qlora_oracle as O

    dt = 0.0
    flops = 0
    for L in layers:
        inp = QI.layer_inputs(cfg, L, M=tokens)
        t0 = time.perf_counter()
        qw = O.quantize_nf4_dq(inp["W"])
        Wd = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], L.m * L.n)).reshape(L.m, L.n)
        x = O.bf16_bits_to_float64(inp["x"])
        g = O.bf16_bits_to_float64(inp["g"])
        A = O.bf16_bits_to_float64(inp["A"])
        B = O.bf16_bits_to_float64(inp["B"])
        h, u = O.linear_fwd(x, Wd, A, B, L.s)
        O.linear_bwd(x, g, Wd, A, B, L.s, u=u)
        dt += time.perf_counter() - t0
        flops += fwd_flops(tokens, L.n, L.m, L.r) + bwd_flops(tokens, L.n, L.m, L.r)
        del inp, qw, Wd, x, g, A, B, h, u
    threads = blas_threads()
    names = ", ".join(f"{L.name} {L.m}x{L.n}" for L in layers)
    M = layers[0].M
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads) if threads else (os.cpu_count() or 1),
        "kind": "oracle",
        "sample": (f"70B block, projections {names}: for each, quantize the whole weight, dequantize it, then " +
                   (f"fwd + bwd of all {M} tokens" if tokens == M else f"fwd + bwd for {tokens} of the {M} tokens") +
                   f", float64 numpy; {dt:.2f} s; value = sample fwd+bwd flops / time (quantize and dequantize "
                   f"included)"),
        "blas_threads": threads,
        "os_cpu_count": os.cpu_count(),
        "seconds": round(dt, 2),
    }


GEMM_KERNELS = ("fwd_gemm", "dgrad_gemm")
KERNELS = ("quantize", "fwd_gemm", "dgrad_gemm", "down_proj", "gpass", "token_grad", "transpose")


def gemm_launch_flops(kernel, M, n, m, r):
    """Algorithmic flops of one GEMM launch: the dense product plus the LoRA
    term it carries as extra K steps (u B^T or v A)."""
    if kernel == "fwd_gemm":
        return 2 * M * m * n + 2 * M * m * r
    return 2 * M * n * m + 2 * M * n * r


class LayerSet:
    """Device tensors of one workload's layers (drawn on the device), with one
    forward and one backward workspace shared by all of them."""

    def __init__(self, Q, dev, layers, seed, backward=True):
        import torch
        gen = torch.Generator(device=dev).manual_seed(seed)
        self.Q, self.dev, self.layers = Q, dev, layers
        self.t = []
        wf = wb = 256
        for L in layers:
            M, n, m, r = L.M, L.n, L.m, L.r
            W = torch.randn((m, n), generator=gen, device=dev, dtype=torch.float32).mul_(L.w_sigma)
            d = dict(L=L, W=W, q=Q.alloc_quantized(m, n, dev),
                     x=torch.randn((M, n), generator=gen, device=dev).to(torch.bfloat16),
                     A=torch.randn((r, n), generator=gen, device=dev).div_(16).to(torch.bfloat16),
                     B=torch.randn((m, r), generator=gen, device=dev).mul_(0.01).to(torch.bfloat16),
                     h=torch.empty((M, m), dtype=torch.bfloat16, device=dev),
                     u=torch.empty((M, r), dtype=torch.float32, device=dev))
            if backward:
                d["g"] = torch.randn((M, m), generator=gen, device=dev).to(torch.bfloat16)
                d["out"] = (torch.empty((M, n), dtype=torch.bfloat16, device=dev),
                            torch.empty((r, n), dtype=torch.bfloat16, device=dev),
                            torch.empty((m, r), dtype=torch.bfloat16, device=dev))
                wb = max(wb, Q.workspace_bytes(Q.QLORA_OP_BWD, M, n, m, r))
            wf = max(wf, Q.workspace_bytes(Q.QLORA_OP_FWD, M, n, m, r))
            self.t.append(d)
        self.ws_f = torch.empty(wf, dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty(wb, dtype=torch.uint8, device=dev) if backward else None
        self.quantize()

    def quantize_one(self, d):
        self.Q.quantize_nf4_dq(d["W"], out=d["q"])

    def fwd_one(self, d):
        L = d["L"]
        self.Q.linear_fwd(d["x"], d["q"], d["A"], d["B"], L.s, h=d["h"], u=d["u"], workspace=self.ws_f)

    def bwd_one(self, d):
        L = d["L"]
        self.Q.linear_bwd(d["x"], d["g"], d["q"], d["A"], d["B"], L.s, u=d["u"], out=d["out"], workspace=self.ws_b)

    def quantize(self):
        # the layers' weights in one launch (at most 8 per call)
        for i in range(0, len(self.t), 8):
            ds = self.t[i:i + 8]
            self.Q.quantize_dq_grouped([d["W"] for d in ds], outs=[d["q"] for d in ds])

    def forward(self):
        for d in self.t:
            self.fwd_one(d)

    def backward(self):
        for d in reversed(self.t):
            self.bwd_one(d)

    def step(self):
        self.quantize()
        self.forward()
        self.backward()

    def flops(self):
        return sum(fwd_flops(L.M, L.n, L.m, L.r) + bwd_flops(L.M, L.n, L.m, L.r) for L in self.layers)

    def kernel_times(self, reps):
        """Per layer: average duration of every library kernel over `reps`
        forward + backward calls of that layer (HIP events on the launch
        stream), the quantizer's too; checks that no K-split wait ran out.
        A spin kernel ahead of each call keeps the host ahead of the GPU, so
        that no event pair spans a gap in the host's launches."""
        import torch
        Q = self.Q
        out = {}
        for d in self.t:
            L = d["L"]
            Q.profile_enable(True)
            for _ in range(reps):
                torch.cuda._sleep(SPIN_CYCLES)
                self.quantize_one(d)
                self.fwd_one(d)
                self.bwd_one(d)
            torch.cuda.synchronize()
            Q.profile_enable(False)
            Q.linear_check(Q.QLORA_OP_FWD, L.M, L.n, L.m, L.r, self.ws_f)
            Q.linear_check(Q.QLORA_OP_BWD, L.M, L.n, L.m, L.r, self.ws_b)
            kern = {}
            for name in KERNELS:
                cnt, tot = Q.profile_query(name)
                if cnt:
                    kern[name] = {"launches_per_call": cnt // reps, "us_per_call": round(tot * 1e3 / reps, 2)}
                    if name in GEMM_KERNELS:
                        us = tot * 1e3 / cnt
                        f = gemm_launch_flops(name, L.M, L.n, L.m, L.r)
                        kern[name].update({"avg_us": round(us, 2), "flop": f,
                                           "TFLOP/s": round(f / (us * 1e-6) / 1e12, 1),
                                           "mfma_frac": round(f / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)})
            out[L.name] = kern
        return out


def small_layer(Q, dev, reps):
    """The 256 x 256 layer at 32 tokens (r = 8): absolute GPU times of the
    quantizer, forward and backward (launch latency dominates, so no
    roofline fraction), and the oracle's times for the same layer on the
    host: float64 numpy (median of 5) and the pure-Python loop forward (one
    run, one core)."""
    import numpy as np
    import torch
    import qlora_inputs as QI
    from oracle import qlora_oracle as O

    L = QI.WORKLOADS[1]["layers"][0]
    ls = LayerSet(Q, dev, [L], seed=1)
    d = ls.t[0]
    out = {"workload": f"single {L.m}x{L.n} layer, {L.M} tokens, r={L.r}, alpha={L.alpha:g}"}
    for nm, fn in (("quantize", lambda: ls.quantize_one(d)), ("forward", lambda: ls.fwd_one(d)),
                   ("backward", lambda: ls.bwd_one(d))):
        med, mn = timed_us(fn, reps)
        out[nm + "_us"] = round(med, 2)
        out[nm + "_us_min"] = round(mn, 2)
    del ls, d
    inp = QI.layer_inputs(1, L)
    x = O.bf16_bits_to_float64(inp["x"])
    g = O.bf16_bits_to_float64(inp["g"])
    A = O.bf16_bits_to_float64(inp["A"])
    B = O.bf16_bits_to_float64(inp["B"])
    ts = {"quantize": [], "forward": [], "backward": []}
    for _ in range(5):
        t0 = time.perf_counter()
        qw = O.quantize_nf4_dq(inp["W"])
        t1 = time.perf_counter()
        Wd = O.bf16_bits_to_float64(O.dequant_nf4_dq(qw["codes"], qw["absmax8"], qw["c2"], L.m * L.n)).reshape(L.m, L.n)
        t2 = time.perf_counter()
        h, u = O.linear_fwd(x, Wd, A, B, L.s)
        t3 = time.perf_counter()
        O.linear_bwd(x, g, Wd, A, B, L.s, u=u)
        t4 = time.perf_counter()
        ts["quantize"].append(t1 - t0)
        ts["forward"].append(t3 - t1)
        ts["backward"].append(t4 - t3)
    oracle = {k + "_us": round(float(np.median(v)) * 1e6, 1) for k, v in ts.items()}
    t0 = time.perf_counter()
    O.linear_fwd_loops(x, Wd, A, B, L.s)
    oracle["forward_python_loops_us"] = round((time.perf_counter() - t0) * 1e6, 1)
    oracle["note"] = ("oracle on the host: float64 numpy, median of 5 (forward includes the dequantization); "
                      "the loop forward is pure Python on one core")
    out["oracle"] = oracle
    torch.cuda.empty_cache()
    return out


def vendor_gemm(dev, layers, reps):
    """Context for the fused GEMM's rate: the ROCm vendor library's plain bf16
    GEMM (torch.matmul, no dequantization, no LoRA term) on the forward
    shapes of the block's projections, beside the fused forward GEMM's time
    from the per-layer pass.  Not part of the path and not a roofline."""
    import torch
    out = {"note": "torch.matmul on plain bf16 operands (x @ W^T, W already bf16); the fused kernel also "
                   "dequantizes W and adds the LoRA term"}
    for name, (M, m, n) in (("q", (8192, 8192, 8192)), ("gate", (8192, 28672, 8192)), ("down", (8192, 8192, 28672))):
        a = torch.randn(M, n, device=dev, dtype=torch.bfloat16)
        w = torch.randn(m, n, device=dev, dtype=torch.bfloat16)
        med, _ = timed_us(lambda: a @ w.t(), reps)
        row = {"shape": f"M {M}, N {m}, K {n}", "us": round(med, 1),
               "TFLOP/s": round(2 * M * m * n / (med * 1e-6) / 1e12, 1)}
        fused = layers.get(name, {}).get("fwd_gemm")
        if fused:
            row["fused_fwd_gemm_us"] = fused["avg_us"]
        out[name] = row
        del a, w
    torch.cuda.empty_cache()
    return out


def gate_sections(Q, dev, reps):
    """The 8B gate projection (14336 x 4096, 4096 tokens, r = 16): forward,
    backward and their kernels, the dropout passes, the adapter merge and the
    level-table round trips."""
    import torch
    import qlora_inputs as QI
    gate = LayerSet(Q, dev, QI.WORKLOADS[2]["layers"], seed=2)
    out = {"gate_8B": layer_passes(gate, reps)}
    d = gate.t[0]
    L = d["L"]
    out["gate_8B"]["kernels"] = gate.kernel_times(5)[L.name]
    out["dropout"] = dropout_passes(Q, d["x"], d["g"], d["q"], d["A"], d["B"], L.s, d["h"], d["u"], d["out"],
                                    gate.ws_f, out["gate_8B"], reps)
    out["adapter_merge"] = adapter_merge(Q, d["q"], d["A"], d["B"], L.s, reps)
    out["level_tables"] = level_table_variants(Q, d["W"], d["q"], reps)
    del gate, d
    torch.cuda.empty_cache()
    return out


def layer_passes(ls, reps):
    """Forward, backward and forward + backward of one layer (median of reps)."""
    d = ls.t[0]
    L = d["L"]
    fwd, _ = timed_us(lambda: ls.fwd_one(d), reps)
    bwd, _ = timed_us(lambda: ls.bwd_one(d), reps)
    both, _ = timed_us(lambda: (ls.fwd_one(d), ls.bwd_one(d)), reps)
    qt, _ = timed_us(lambda: ls.quantize_one(d), reps)
    ff, bf = fwd_flops(L.M, L.n, L.m, L.r), bwd_flops(L.M, L.n, L.m, L.r)
    qb = quant_bytes(L.m, L.n)
    return {
        "workload": f"{L.name} projection {L.m}x{L.n}, {L.M} tokens, r={L.r}, alpha={L.alpha:g}",
        "forward": {"us": round(fwd, 2), "TFLOP/s": round(ff / (fwd * 1e-6) / 1e12, 1),
                    "mfma_frac": round(ff / (fwd * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "backward": {"us": round(bwd, 2), "TFLOP/s": round(bf / (bwd * 1e-6) / 1e12, 1),
                     "mfma_frac": round(bf / (bwd * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "fwd_bwd": {"us": round(both, 2), "TFLOP/s": round((ff + bf) / (both * 1e-6) / 1e12, 1),
                    "mfma_frac": round((ff + bf) / (both * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "quantize": {"us": round(qt, 2), "GB/s": round(qb / (qt * 1e-6) / 1e9, 1),
                     "hbm_frac": round(qb / (qt * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "timing": "back-to-back, no cache flush"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--profile-reps", type=int, default=3, help="per-layer calls timed kernel by kernel")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the measurements outside the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--small-only", action="store_true",
                    help="only run the small-token section (for profiling it alone)")
    ap.add_argument("--gate-only", action="store_true",
                    help="only run the gate-projection sections (for profiling them alone)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_fine_qlora_amd as Q
    import qlora_inputs as QI

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 3}))
        return

    if args.small_only:
        print(json.dumps({"small_tokens": small_token_block(Q, dev, max(args.steps, 3))}), flush=True)
        return
    if args.gate_only:
        print(json.dumps(gate_sections(Q, dev, max(args.steps, 3))), flush=True)
        return

    cfg = 5
    blk = LayerSet(Q, dev, QI.WORKLOADS[cfg]["layers"], seed=cfg)
    M, r, s = blk.layers[0].M, blk.layers[0].r, blk.layers[0].s
    for _ in range(args.warmup):
        blk.step()
    torch.cuda.synchronize()
    print(f"[bench] 70B block: {args.warmup} warm-up steps done", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    for _ in range(args.steps):
        blk.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    flops = blk.flops()
    value = flops / (ms * 1e-3) / 1e12
    print(f"[bench] 70B block: {args.steps} timed steps, {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # per-layer kernel times (a separate pass with the library's HIP events)
    layers = blk.kernel_times(args.profile_reps)
    gemms = [(f"{nm}/{k}", v) for nm, kk in layers.items() for k, v in kk.items() if k in GEMM_KERNELS]
    dom_key, dom = max(gemms, key=lambda kv: kv[1]["avg_us"])
    achieved = dom["flop"] / (dom["avg_us"] * 1e-6) / 1e12
    roofline = {"kernel": dom_key, "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": gemm_traffic(dom_key),
                "per_launch_flop": dom["flop"], "avg_us": dom["avg_us"]}
    gemm_flop = sum(v["flop"] * v["launches_per_call"] for _, v in gemms)
    gemm_us = sum(v["us_per_call"] for _, v in gemms)
    print(f"[bench] per-layer kernel times done", file=sys.stderr, flush=True)

    out = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s and NF4 weight GB/s (% of roofline), 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "70B-shaped block (q 8192x8192, k/v 1024x8192, o 8192x8192, gate/up 28672x8192, "
                               "down 8192x28672) NF4+DQ, 8192 tokens, r=64, alpha=16 on all seven: quantize + "
                               "fwd + bwd of the seven layers per step",
                   "M": M, "r": r, "s": s, "layers": len(blk.layers), "step_flop": flops},
        "roofline": roofline,
        "block_gemms": {"flop": gemm_flop, "us": round(gemm_us, 1),
                        "TFLOP/s": round(gemm_flop / (gemm_us * 1e-6) / 1e12, 1),
                        "mfma_frac": round(gemm_flop / (gemm_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                        "note": "all 14 GEMM launches of a step, summed from the per-layer kernel times"},
        "layers": layers,
    }
    if not args.no_extra:
        fwd, _ = timed_us(blk.forward, 5)
        bwd, _ = timed_us(blk.backward, 5)
        ff = sum(fwd_flops(L.M, L.n, L.m, L.r) for L in blk.layers)
        bf = sum(bwd_flops(L.M, L.n, L.m, L.r) for L in blk.layers)
        qb = sum(quant_bytes(L.m, L.n) for L in blk.layers)
        qt, qmin = timed_us(blk.quantize, 5)
        out["block_passes"] = {
            "forward": {"us": round(fwd, 1), "TFLOP/s": round(ff / (fwd * 1e-6) / 1e12, 1)},
            "backward": {"us": round(bwd, 1), "TFLOP/s": round(bf / (bwd * 1e-6) / 1e12, 1)},
            "fwd_bwd_without_quantize_us": round(fwd + bwd, 1),
            "fwd_bwd_without_quantize_TFLOP/s": round((ff + bf) / ((fwd + bwd) * 1e-6) / 1e12, 1),
            "quantize": {"us": round(qt, 1), "bytes": qb, "GB/s": round(qb / (qt * 1e-6) / 1e9, 1),
                         "hbm_frac": round(qb / (qt * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "note": "the seven fp32 weights (3.42 GB, larger than the caches), back to back"},
        }
        print(f"[bench] block passes done", file=sys.stderr, flush=True)
    del blk
    torch.cuda.empty_cache()
    if not args.no_extra:
        out["vendor_bf16_gemm"] = vendor_gemm(dev, layers, 10)
        print(f"[bench] vendor GEMM context done", file=sys.stderr, flush=True)

    if not args.no_extra:
        out.update(gate_sections(Q, dev, 10))
        print(f"[bench] gate projection done", file=sys.stderr, flush=True)
        down = LayerSet(Q, dev, QI.WORKLOADS[3]["layers"], seed=3)
        out["down_8B"] = layer_passes(down, 10)
        out["down_8B"]["kernels"] = down.kernel_times(5)[down.layers[0].name]
        del down
        torch.cuda.empty_cache()
        print(f"[bench] down projection done", file=sys.stderr, flush=True)
        out["adapter_adam"] = adapter_adam(Q, dev, 10)
        torch.cuda.empty_cache()
        out["small_tokens"] = small_token_block(Q, dev, 10)
        out["small_layer"] = small_layer(Q, dev, 20)
        print(f"[bench] extras done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, QI.WORKLOADS[cfg]["layers"][:4], args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
