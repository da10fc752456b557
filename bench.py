"""Benchmark of the QLoRA adapted-linear hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input, already
resident in HBM: quantize the frozen weight (NF4 + double quantization),
forward (u = x A^T, h = x W'^T + s u B^T), backward (grad_x, grad_A,
grad_B).  Workload: the Llama-3.1-8B-shaped gate projection, W0 14336 x
4096, 4096 tokens (batch 4 x seq 1024), LoRA r = 16, alpha = 32.

value = algorithmic forward + backward flops per step / step time (TFLOP/s),
the quantizer's time included in the step.  Prints one JSON line.

Besides the timed steps (and outside them) it also measures, each with HIP
events on the stream the library launches on:
  - the forward alone and the backward alone of the same layer;
  - the small-token regime: the forward of all seven layers of the
    8B-shaped block at 16 tokens in one grouped call, and the quantization of
    the block's seven weights, both against the HBM peak;
  - the adapter merge W_merged = bf16(W' + s B A) of the gate projection,
    against the HBM peak;
  - the adapter optimizer step (Adam, decoupled weight decay) over the
    adapters of a 32-layer 8B-shaped model at r = 16 (448 tensors, 41.9 M
    parameters, 28 bytes each), against the HBM peak, and over one block's
    adapters with the optimizer state in pinned host memory;
  - the quantizer on the uniform 4-bit comparison grid: round-trip relative
    error of the gate weight through the GPU kernels for NF4 and for the
    uniform grid, and the uniform quantizer's time.
For the HBM-bound measurements the caches are flushed before every
repetition by reading 1 GiB (a read evicts the working set cleanly; a write
flush would leave dirty lines whose write-back lands in the timed kernel).
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
BF16_PEAK_TFLOPS = 2500.0

# HBM bytes per launch of the GEMM kernels on this workload, from rocprofv3
# --pmc FETCH_SIZE and WRITE_SIZE runs of this script (KiB per dispatch),
# scaled by what the same counters read for a plain 1 GiB device copy
# (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0; see profiles/).  Valid only for the
# GEMM sources they were taken on (the kernel and the header it includes):
# reported as null once either changes.
GEMM_SRC = [os.path.join(ROOT, "bit_quantized_fine_qlora_amd", "csrc", f) for f in ("gemm_linear.hip", "qlora_common.h")]
GEMM_TRAFFIC = {
    "src_sha1": "8eb9791ff195d4a04166db0f7f98cbbb2a90ef00",
    "fwd_gemm": {"fetch": 2 * 295420.0 * 1024, "write": 147509.0 * 1024},
    "dgrad_gemm": {"fetch": 2 * 198148.0 * 1024, "write": 32801.0 * 1024},
}


def gemm_traffic(kernel):
    import hashlib
    h = hashlib.sha1()
    try:
        for path in GEMM_SRC:
            with open(path, "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    digest = h.hexdigest()
    if digest != GEMM_TRAFFIC["src_sha1"] or kernel not in GEMM_TRAFFIC:
        return None
    t = GEMM_TRAFFIC[kernel]
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
    """Median and min of `reps` event-timed calls of fn (after one untimed call)."""
    import torch
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush.sum()
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

    def quant_all():
        for W, q in Ws:
            Q.quantize_nf4_dq(W, out=q)

    qmed, qmn = timed_us(quant_all, max(3, reps // 2), flush)
    return {
        "forward": {"workload": "8B-shaped block: q,k,v,o,gate,up,down, 16 tokens, r=16, one grouped call",
                    "us": round(med, 2), "us_min": round(mn, 2), "bytes": fb,
                    "GB/s": round(fb / (med * 1e-6) / 1e9, 1), "hbm_frac": round(fb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "quantize": {"workload": "the block's seven fp32 weights (218,103,808 params)",
                     "us": round(qmed, 2), "bytes": qbytes,
                     "GB/s": round(qbytes / (qmed * 1e-6) / 1e9, 1),
                     "hbm_frac": round(qbytes / (qmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "cache_flush": "1 GiB read before every repetition",
    }


def merge_bytes(m, n, r):
    """Packed weight read, adapter read, merged bf16 weight written."""
    numel = m * n
    return numel // 2 + numel // 64 + 4 * ((numel // 64 + 255) // 256) + 2 * (r * n + m * r) + 2 * numel


def level_table_variants(Q, W, q, reps):
    """Round-trip error of the gate weight through quantize + dequant for NF4, the
    uniform grid and the edge-mean table."""
    import torch
    w = W.double()
    out = {}
    for name, qtype in (("nf4", Q.QTYPE_NF4), ("uniform4", Q.QTYPE_UNIFORM4), ("edge_mean4", Q.QTYPE_EDGE_MEAN4)):
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


def cpu_baseline(cfg, layer, tokens):
    """Time the oracle (float64 numpy) on a bounded sample of the workload."""
    import numpy as np

    import qlora_inputs as QI
    from oracle import qlora_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    L = layer
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
    dt = time.perf_counter() - t0
    flops = fwd_flops(tokens, L.n, L.m, L.r) + bwd_flops(tokens, L.n, L.m, L.r)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"quantize the full {L.m}x{L.n} weight + fwd + bwd for {tokens} of the {L.M} tokens, "
                   f"float64 numpy; {dt:.2f} s; value = sample fwd+bwd flops / time"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the measurements outside the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
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

    cfg = 2
    L = QI.WORKLOADS[cfg]["layers"][0]
    M, n, m, r, s = L.M, L.n, L.m, L.r, L.s
    inp = QI.layer_inputs(cfg, L)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    W = torch.from_numpy(inp["W"]).to(dev)
    x, g, A, B = (dev_bf16(inp[k]) for k in ("x", "g", "A", "B"))
    q = Q.alloc_quantized(m, n, dev)
    h = torch.empty((M, m), dtype=torch.bfloat16, device=dev)
    u = torch.empty((M, r), dtype=torch.float32, device=dev)
    gx = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
    gA = torch.empty((r, n), dtype=torch.bfloat16, device=dev)
    gB = torch.empty((m, r), dtype=torch.bfloat16, device=dev)
    ws_f = torch.empty(Q.workspace_bytes(Q.QLORA_OP_FWD, M, n, m, r), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(Q.workspace_bytes(Q.QLORA_OP_BWD, M, n, m, r), dtype=torch.uint8, device=dev)

    def step():
        Q.quantize_nf4_dq(W, out=q)
        Q.linear_fwd(x, q, A, B, s, h=h, u=u, workspace=ws_f)
        Q.linear_bwd(x, g, q, A, B, s, u=u, out=(gx, gA, gB), workspace=ws_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    Q.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    Q.profile_enable(False)

    ms = (t1 - t0) * 1e3 / args.steps
    flops = fwd_flops(M, n, m, r) + bwd_flops(M, n, m, r)
    value = flops / (ms * 1e-3) / 1e12

    kern = {}
    for name in ("quantize", "fwd_gemm", "dgrad_gemm", "down_proj", "gpass", "token_grad", "transpose"):
        cnt, tot = Q.profile_query(name)
        if cnt:
            kern[name] = {"launches": cnt, "avg_us": tot * 1e3 / cnt}

    per_launch = {
        "fwd_gemm": 2 * M * m * n + 2 * M * m * r,
        "dgrad_gemm": 2 * M * n * m + 2 * M * n * r,
    }
    dom = max(per_launch, key=lambda k: kern.get(k, {}).get("avg_us", 0.0))
    dom_us = kern[dom]["avg_us"]
    achieved = per_launch[dom] / (dom_us * 1e-6) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": gemm_traffic(dom)}
    qb = quant_bytes(m, n)
    quant = {"avg_us": round(kern["quantize"]["avg_us"], 2),
             "GB/s": round(qb / (kern["quantize"]["avg_us"] * 1e-6) / 1e9, 1),
             "hbm_frac": round(qb / (kern["quantize"]["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    other = {k: {"launches": v["launches"], "avg_us": round(v["avg_us"], 2)} for k, v in kern.items()}

    extra = {}
    if not args.no_extra:
        fwd_med, _ = timed_us(lambda: Q.linear_fwd(x, q, A, B, s, h=h, u=u, workspace=ws_f), 10)
        bwd_med, _ = timed_us(lambda: Q.linear_bwd(x, g, q, A, B, s, u=u, out=(gx, gA, gB), workspace=ws_b), 10)
        extra["passes"] = {
            "forward": {"us": round(fwd_med, 2), "TFLOP/s": round(fwd_flops(M, n, m, r) / (fwd_med * 1e-6) / 1e12, 1)},
            "backward": {"us": round(bwd_med, 2), "TFLOP/s": round(bwd_flops(M, n, m, r) / (bwd_med * 1e-6) / 1e12, 1)},
        }

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
        "config": {"workload": "gate projection W0 14336x4096 NF4+DQ, 4096 tokens, r=16, alpha=32: "
                               "quantize + fwd + bwd per step",
                   "M": M, "n": n, "m": m, "r": r, "s": s},
        "roofline": roofline,
        "quantize": quant,
        "kernels": other,
    }
    out.update(extra)
    if not args.no_extra:
        out["dropout"] = dropout_passes(Q, x, g, q, A, B, s, h, u, (gx, gA, gB), ws_f, extra["passes"], 10)
        out["adapter_merge"] = adapter_merge(Q, q, A, B, s, 10)
        out["adapter_adam"] = adapter_adam(Q, dev, 10)
        out["level_tables"] = level_table_variants(Q, W, q, 10)
        del W, x, g, A, B, h, gx, ws_f, ws_b
        torch.cuda.empty_cache()
        out["small_tokens"] = small_token_block(Q, dev, 10)
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, L, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
