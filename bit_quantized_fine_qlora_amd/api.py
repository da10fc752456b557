"""Torch-facing binding of the QLoRA library.

Only marshals tensors into pointers and sizes and passes the current HIP
stream; every step of the computation runs in the HIP kernels of
libqlora.so.  Torch supplies device memory (outputs and workspaces).
"""

from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib

QLORA_OP_FWD = 0
QLORA_OP_BWD = 1
QLORA_OP_BWD_DROPOUT = 2


@dataclasses.dataclass
class QuantizedWeight:
    """NF4 + double-quantized m x n weight: codes, absmax8 (E4M3) and c2."""
    codes: torch.Tensor     # uint8 [m*n/2]
    absmax8: torch.Tensor   # uint8 [m*n/64]
    c2: torch.Tensor        # float32 [ceil(m*n/16384)]
    m: int
    n: int

    def nbytes(self) -> int:
        return self.codes.numel() + self.absmax8.numel() + 4 * self.c2.numel()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, shape, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


QTYPE_NF4 = 0
QTYPE_UNIFORM4 = 1
QTYPE_EDGE_MEAN4 = 2
QTYPE_INT4 = 3


def level_table(qtype: int = QTYPE_NF4):
    """(levels[16], thresholds[15]) of a level table as the library derived them (host)."""
    lib = _lib.load()
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _lib.check(lib.qlora_level_table(int(qtype), ctypes.cast(lv, ctypes.c_void_p), ctypes.cast(th, ctypes.c_void_p)),
               "qlora_level_table")
    return list(lv), list(th)


def quantize_dq(W: torch.Tensor, qtype: int = QTYPE_NF4, out: QuantizedWeight | None = None) -> QuantizedWeight:
    """Blockwise 4-bit quantization with double quantization on a chosen level table."""
    m, n = W.shape
    _need(W, torch.float32, (m, n), "W")
    q = out if out is not None else alloc_quantized(m, n, W.device)
    st = _lib.load().qlora_quantize_dq(int(qtype), _ptr(W), m, n, _ptr(q.codes), _ptr(q.absmax8), _ptr(q.c2),
                                       _stream(W.device))
    _lib.check(st, "qlora_quantize_dq")
    return q


def quantize_dq_grouped(Ws, qtype: int = QTYPE_NF4, outs=None):
    """Quantize several fp32 weights in one launch, each as quantize_dq would.

    Ws: sequence of up to 8 m x n fp32 tensors on one device; outs: matching
    QuantizedWeights to write, or None to allocate.  Returns the list of
    QuantizedWeights.
    """
    if not Ws:
        return []
    dev = Ws[0].device
    arr = (_lib.QuantWeight * len(Ws))()
    qs = []
    for i, W in enumerate(Ws):
        m, n = W.shape
        _need(W, torch.float32, (m, n), "W")
        if W.device != dev:
            raise ValueError("quantize_dq_grouped: all weights must be on one device")
        q = outs[i] if outs is not None else alloc_quantized(m, n, dev)
        arr[i] = _lib.QuantWeight(_ptr(W), m, n, _ptr(q.codes), _ptr(q.absmax8), _ptr(q.c2))
        qs.append(q)
    st = _lib.load().qlora_quantize_dq_grouped(int(qtype), len(Ws), arr, _stream(dev))
    _lib.check(st, "qlora_quantize_dq_grouped")
    return qs


def dequant_dq(q: QuantizedWeight, qtype: int = QTYPE_NF4) -> torch.Tensor:
    out = torch.empty((q.m, q.n), dtype=torch.bfloat16, device=q.codes.device)
    st = _lib.load().qlora_dequant_dq(int(qtype), _ptr(q.codes), _ptr(q.absmax8), _ptr(q.c2), q.m, q.n, _ptr(out),
                                      _stream(q.codes.device))
    _lib.check(st, "qlora_dequant_dq")
    return out


def nf4_table():
    """(levels[16], thresholds[15]) as the library derived them (host)."""
    lib = _lib.load()
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    lib.qlora_nf4_table(ctypes.cast(lv, ctypes.c_void_p), ctypes.cast(th, ctypes.c_void_p))
    return list(lv), list(th)


def workspace_bytes(op: int, M: int, n: int, m: int, r: int) -> int:
    return int(_lib.load().qlora_workspace_bytes(op, M, n, m, r))


def alloc_quantized(m: int, n: int, device="cuda") -> QuantizedWeight:
    numel = m * n
    return QuantizedWeight(
        codes=torch.empty(numel // 2, dtype=torch.uint8, device=device),
        absmax8=torch.empty(numel // 64, dtype=torch.uint8, device=device),
        c2=torch.empty((numel // 64 + 255) // 256, dtype=torch.float32, device=device),
        m=m, n=n)


def quantize_nf4_dq(W: torch.Tensor, out: QuantizedWeight | None = None) -> QuantizedWeight:
    m, n = W.shape
    _need(W, torch.float32, (m, n), "W")
    q = out if out is not None else alloc_quantized(m, n, W.device)
    st = _lib.load().qlora_quantize_nf4_dq(_ptr(W), m, n, _ptr(q.codes), _ptr(q.absmax8), _ptr(q.c2),
                                           _stream(W.device))
    _lib.check(st, "qlora_quantize_nf4_dq")
    return q


def dequant_nf4_dq(q: QuantizedWeight) -> torch.Tensor:
    out = torch.empty((q.m, q.n), dtype=torch.bfloat16, device=q.codes.device)
    st = _lib.load().qlora_dequant_nf4_dq(_ptr(q.codes), _ptr(q.absmax8), _ptr(q.c2), q.m, q.n, _ptr(out),
                                          _stream(q.codes.device))
    _lib.check(st, "qlora_dequant_nf4_dq")
    return out


class AdamStep:
    """Prepared optimizer step over a fixed list of adapter tensors.

    tensors: list of (param fp32, param_bf16 bf16 or None, grad bf16, exp_avg fp32, exp_avg_sq fp32), each
    contiguous with the same number of elements, on the GPU or (param and moments) in pinned host memory.
    The tensor table is marshalled once; run() launches the step.
    """

    def __init__(self, tensors):
        self._keep = list(tensors)
        self._arr = (_lib.AdamTensor * len(self._keep))()
        self._dev = None
        for i, (p, p16, g, m, v) in enumerate(self._keep):
            n = p.numel()
            if p.dtype != torch.float32 or m.dtype != torch.float32 or v.dtype != torch.float32:
                raise TypeError("param, exp_avg and exp_avg_sq must be float32")
            if g.dtype != torch.bfloat16 or (p16 is not None and p16.dtype != torch.bfloat16):
                raise TypeError("grad and param_bf16 must be bfloat16")
            named = [(p, "param"), (g, "grad"), (m, "exp_avg"), (v, "exp_avg_sq")]
            if p16 is not None:
                named.append((p16, "param_bf16"))
            for t, nm in named:
                if t.numel() != n or not t.is_contiguous():
                    raise ValueError(f"{nm}: expected {n} contiguous elements")
            if g.is_cuda:
                self._dev = g.device
            self._arr[i] = _lib.AdamTensor(n, p.data_ptr(), p16.data_ptr() if p16 is not None else None,
                                           g.data_ptr(), m.data_ptr(), v.data_ptr())

    def run(self, lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
            weight_decay: float = 0.0, step: int = 1) -> None:
        st = _lib.load().qlora_adam_step(self._arr, len(self._keep), float(lr), float(beta1), float(beta2),
                                         float(eps), float(weight_decay), int(step), _stream(self._dev))
        _lib.check(st, "qlora_adam_step")


def adam_step(tensors, lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
              weight_decay: float = 0.0, step: int = 1) -> None:
    """Adam step with decoupled weight decay on adapter tensors, in place (see AdamStep)."""
    AdamStep(tensors).run(lr, beta1, beta2, eps, weight_decay, step)


def merge_adapter(q: QuantizedWeight, A: torch.Tensor, B: torch.Tensor, s: float) -> torch.Tensor:
    """bf16(W' + s B A): the adapter folded into the dequantized weight (m x n bf16)."""
    r = A.shape[0]
    _need(A, torch.bfloat16, (r, q.n), "A")
    _need(B, torch.bfloat16, (q.m, r), "B")
    out = torch.empty((q.m, q.n), dtype=torch.bfloat16, device=q.codes.device)
    st = _lib.load().qlora_merge_adapter(_ptr(q.codes), _ptr(q.absmax8), _ptr(q.c2), q.m, q.n, r, float(s),
                                         _ptr(A), _ptr(B), _ptr(out), _stream(q.codes.device))
    _lib.check(st, "qlora_merge_adapter")
    return out


def _workspace(op, M, n, m, r, device, workspace):
    need = workspace_bytes(op, M, n, m, r)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def _dropout(dropout):
    """(p, seed, offset) or None -> a qlora_dropout pointer (None: plain layer)."""
    if dropout is None:
        return None
    p, seed, offset = dropout
    return ctypes.pointer(_lib.Dropout(float(p), int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1)))


def linear_fwd(x: torch.Tensor, q: QuantizedWeight, A: torch.Tensor, B: torch.Tensor, s: float,
               h: torch.Tensor | None = None, u: torch.Tensor | None = None, want_u: bool = True,
               workspace: torch.Tensor | None = None, dropout=None):
    """h = x W'^T + s (x A^T) B^T.  Returns (h bf16 [M, m], u fp32 [M, r] or None).

    dropout: (p, seed, offset) for dropout on the adapter input (the adapter
    reads x * keep / (1 - p)), or None.
    """
    M, n = x.shape
    m = q.m
    r = A.shape[0]
    _need(x, torch.bfloat16, (M, q.n), "x")
    _need(A, torch.bfloat16, (r, q.n), "A")
    _need(B, torch.bfloat16, (m, r), "B")
    if h is None:
        h = torch.empty((M, m), dtype=torch.bfloat16, device=x.device)
    if u is None and want_u:
        u = torch.empty((M, r), dtype=torch.float32, device=x.device)
    ws = _workspace(QLORA_OP_FWD, M, n, m, r, x.device, workspace)
    if dropout is None:
        st = _lib.load().qlora_linear_fwd(M, n, m, r, float(s), _ptr(x), _ptr(q.codes), _ptr(q.absmax8),
                                          _ptr(q.c2), _ptr(A), _ptr(B), _ptr(h), _ptr(u), _ptr(ws), ws.numel(),
                                          _stream(x.device))
        _lib.check(st, "qlora_linear_fwd")
    else:
        st = _lib.load().qlora_linear_fwd_ex(M, n, m, r, float(s), _ptr(x), _ptr(q.codes), _ptr(q.absmax8),
                                             _ptr(q.c2), _ptr(A), _ptr(B), _ptr(h), _ptr(u), _dropout(dropout),
                                             _ptr(ws), ws.numel(), _stream(x.device))
        _lib.check(st, "qlora_linear_fwd_ex")
    return h, u


def linear_fwd_static(x: torch.Tensor, q: QuantizedWeight, A: torch.Tensor, B: torch.Tensor, s: float,
                      h: torch.Tensor, u: torch.Tensor | None = None):
    """qlora_linear_fwd_static: the forward with the library's own device scratch
    (no workspace).  h (and u, if wanted) must be given: nothing is allocated."""
    M, n = x.shape
    m = q.m
    r = A.shape[0]
    _need(x, torch.bfloat16, (M, q.n), "x")
    _need(A, torch.bfloat16, (r, q.n), "A")
    _need(B, torch.bfloat16, (m, r), "B")
    _need(h, torch.bfloat16, (M, m), "h")
    if u is not None:
        _need(u, torch.float32, (M, r), "u")
    st = _lib.load().qlora_linear_fwd_static(M, n, m, r, float(s), _ptr(x), _ptr(q.codes), _ptr(q.absmax8),
                                             _ptr(q.c2), _ptr(A), _ptr(B), _ptr(h), _ptr(u), _stream(x.device))
    _lib.check(st, "qlora_linear_fwd_static")
    return h, u


class GroupedForward:
    """A reusable grouped forward: outputs, descriptors and workspace are made once.

    layers: sequence of (x, q, A, B, s) as for linear_fwd, all with the same
    token count M.  run() launches the forward of every layer (one launch
    pair for M <= 32) and returns the list of (h, u) output tensors.
    """

    def __init__(self, layers):
        if not layers:
            raise ValueError("no layers")
        self.M = layers[0][0].shape[0]
        self.device = layers[0][0].device
        self.keep = list(layers)
        self.descs = (_lib.LinearLayer * len(layers))()
        self.outs = []
        for i, (x, q, A, B, s) in enumerate(layers):
            r = A.shape[0]
            _need(x, torch.bfloat16, (self.M, q.n), "x")
            _need(A, torch.bfloat16, (r, q.n), "A")
            _need(B, torch.bfloat16, (q.m, r), "B")
            h = torch.empty((self.M, q.m), dtype=torch.bfloat16, device=self.device)
            u = torch.empty((self.M, r), dtype=torch.float32, device=self.device)
            self.outs.append((h, u))
            self.descs[i] = _lib.LinearLayer(q.n, q.m, r, float(s), x.data_ptr(), q.codes.data_ptr(),
                                             q.absmax8.data_ptr(), q.c2.data_ptr(), A.data_ptr(), B.data_ptr(),
                                             h.data_ptr(), u.data_ptr())
        need = _lib.load().qlora_grouped_workspace_bytes(self.M, len(layers), self.descs)
        if need == 0:
            raise ValueError("invalid grouped forward arguments")
        self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)

    def run(self):
        st = _lib.load().qlora_linear_fwd_grouped(self.M, len(self.keep), self.descs, _ptr(self.workspace),
                                                  self.workspace.numel(), _stream(self.device))
        _lib.check(st, "qlora_linear_fwd_grouped")
        return self.outs


def linear_fwd_grouped(layers):
    """Forward of several layers sharing the token count M, in one call.

    layers: sequence of (x, q, A, B, s) as for linear_fwd.  Returns a list of
    (h, u) pairs.  For M <= 32 all layers are streamed by one launch.
    """
    if not layers:
        return []
    return GroupedForward(layers).run()


def linear_bwd(x: torch.Tensor, g: torch.Tensor, q: QuantizedWeight, A: torch.Tensor, B: torch.Tensor, s: float,
               u: torch.Tensor | None = None, need_grad_x: bool = True, out=None,
               workspace: torch.Tensor | None = None, dropout=None):
    """Returns (grad_x bf16 [M, n] or None, grad_A bf16 [r, n], grad_B bf16 [m, r]).

    dropout: the forward's (p, seed, offset), or None; u, when given, is the
    forward's u (with the mask).
    """
    M, n = x.shape
    m = q.m
    r = A.shape[0]
    _need(x, torch.bfloat16, (M, q.n), "x")
    _need(g, torch.bfloat16, (M, m), "g")
    _need(A, torch.bfloat16, (r, n), "A")
    _need(B, torch.bfloat16, (m, r), "B")
    if u is not None:
        _need(u, torch.float32, (M, r), "u")
    if out is None:
        gx = torch.empty((M, n), dtype=torch.bfloat16, device=x.device) if need_grad_x else None
        gA = torch.empty((r, n), dtype=torch.bfloat16, device=x.device)
        gB = torch.empty((m, r), dtype=torch.bfloat16, device=x.device)
    else:
        gx, gA, gB = out
    if dropout is None:
        ws = _workspace(QLORA_OP_BWD, M, n, m, r, x.device, workspace)
        st = _lib.load().qlora_linear_bwd(M, n, m, r, float(s), _ptr(x), _ptr(g), _ptr(q.codes), _ptr(q.absmax8),
                                          _ptr(q.c2), _ptr(A), _ptr(B), _ptr(u), _ptr(gx), _ptr(gA), _ptr(gB),
                                          _ptr(ws), ws.numel(), _stream(x.device))
        _lib.check(st, "qlora_linear_bwd")
    else:
        ws = _workspace(QLORA_OP_BWD_DROPOUT, M, n, m, r, x.device, workspace)
        st = _lib.load().qlora_linear_bwd_ex(M, n, m, r, float(s), _ptr(x), _ptr(g), _ptr(q.codes),
                                             _ptr(q.absmax8), _ptr(q.c2), _ptr(A), _ptr(B), _ptr(u), _ptr(gx),
                                             _ptr(gA), _ptr(gB), _dropout(dropout), _ptr(ws), ws.numel(),
                                             _stream(x.device))
        _lib.check(st, "qlora_linear_bwd_ex")
    return gx, gA, gB


def linear_check(op: int, M: int, n: int, m: int, r: int, workspace: torch.Tensor | None) -> None:
    """Raise if the last call of `op` on `workspace` had a bounded wait run out
    (qlora_linear_check; synchronizes the current stream).  workspace None with
    the forward op: the scratch of linear_fwd_static."""
    dev = workspace.device if workspace is not None else None
    st = _lib.load().qlora_linear_check(int(op), M, n, m, r, _ptr(workspace), _stream(dev))
    _lib.check(st, "qlora_linear_check")


def profile_enable(on: bool = True) -> None:
    _lib.check(_lib.load().qlora_profile_enable(1 if on else 0), "qlora_profile_enable")


def profile_query(name: str):
    """(launches, total_ms) of a kernel recorded while profiling was on."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _lib.check(_lib.load().qlora_profile_query(name.encode(), ctypes.byref(n), ctypes.byref(ms)),
               "qlora_profile_query")
    return int(n.value), float(ms.value)
