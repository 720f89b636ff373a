"""Python front end of the library: device copies of a layer's weights and thin
wrappers around the C entry points.

torch provides device memory and the current stream only; every computation
happens in libqsmoe.so's HIP kernels (argument marshalling here, nothing else).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import ExpertsC, LayerC, QTensorC, RouterC, check


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _to_device(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def _bits_tensor(x: torch.Tensor) -> torch.Tensor:
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"activations must be bf16 (or its int16 bit pattern), got {x.dtype}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("activations must be a contiguous device tensor")
    return x


class DeviceQTensor:
    """A stacked quantised projection resident on the device."""

    def __init__(self, fmt: str, bits: int, group: int, rows: int, cols: int, codes: torch.Tensor,
                 scales: torch.Tensor, biases: Optional[torch.Tensor]):
        self.fmt, self.bits, self.group, self.rows, self.cols = fmt, bits, group, rows, cols
        self.codes, self.scales, self.biases = codes, scales, biases
        self.num_experts = codes.shape[0]
        fmt_c = {"affine": _lib.MOE_FMT_AFFINE, "mxfp4": _lib.MOE_FMT_MXFP4, "mxfp8": _lib.MOE_FMT_MXFP8}[fmt]
        self.c = QTensorC(fmt_c, bits, group, rows, cols,
                          self.num_experts, codes.data_ptr(), scales.data_ptr(),
                          biases.data_ptr() if biases is not None else None)

    @classmethod
    def from_host(cls, q, device) -> "DeviceQTensor":
        """From an object with spec.{fmt,bits,group}, rows, cols, codes, scales, biases (numpy)."""
        return cls(q.spec.fmt, q.spec.bits, q.spec.group, q.rows, q.cols, _to_device(q.codes, device),
                   _to_device(q.scales, device), None if q.biases is None else _to_device(q.biases, device))

    def clone(self) -> "DeviceQTensor":
        return DeviceQTensor(self.fmt, self.bits, self.group, self.rows, self.cols, self.codes.clone(),
                             self.scales.clone(), None if self.biases is None else self.biases.clone())

    def nbytes_per_expert(self) -> int:
        b = (self.codes[0].numel() * 4 + self.scales[0].numel() * self.scales.element_size())
        if self.biases is not None:
            b += self.biases[0].numel() * 2
        return b


class DeviceExperts:
    def __init__(self, gate: DeviceQTensor, up: DeviceQTensor, down: DeviceQTensor):
        self.gate, self.up, self.down = gate, up, down
        self.c = ExpertsC(gate.c, up.c, down.c)

    @classmethod
    def from_host(cls, ew, device) -> "DeviceExperts":
        return cls(DeviceQTensor.from_host(ew.gate, device), DeviceQTensor.from_host(ew.up, device),
                   DeviceQTensor.from_host(ew.down, device))

    def clone(self) -> "DeviceExperts":
        return DeviceExperts(self.gate.clone(), self.up.clone(), self.down.clone())

    def nbytes_per_expert(self) -> int:
        return sum(q.nbytes_per_expert() for q in (self.gate, self.up, self.down))


class DeviceLayer:
    """Router, routed experts and optional shared expert of one MoE layer."""

    def __init__(self, route: str, top_k: int, wr: torch.Tensor, bias: Optional[torch.Tensor],
                 tid2eid: Optional[torch.Tensor], routed: DeviceExperts, shared: Optional[DeviceExperts],
                 routed_scale: float = 1.0):
        self.route, self.top_k = route, top_k
        self.wr, self.bias, self.tid2eid = wr, bias, tid2eid
        self.routed, self.shared = routed, shared
        self.E, self.d = wr.shape
        self.I = routed.gate.rows
        self.vocab = 0 if tid2eid is None else tid2eid.shape[0]
        self.router_c = RouterC(_lib.MOE_ROUTE_HASH if route == "hash" else _lib.MOE_ROUTE_TOPK, self.E, top_k,
                                self.d, self.vocab, wr.data_ptr(), bias.data_ptr() if bias is not None else None,
                                tid2eid.data_ptr() if tid2eid is not None else None, routed_scale)
        self._shared_c = shared.c if shared is not None else None
        self.c = LayerC(self.router_c, routed.c,
                        ctypes.pointer(self._shared_c) if shared is not None else ctypes.POINTER(ExpertsC)())

    @classmethod
    def from_host(cls, layer, device="cuda", routed=None) -> "DeviceLayer":
        """From a host layer (cfg.route, cfg.top_k, wr, bias, tid2eid, routed, shared as numpy)."""
        cfg = layer.cfg
        r = routed if routed is not None else DeviceExperts.from_host(layer.routed, device)
        sh = DeviceExperts.from_host(layer.shared, device) if layer.shared is not None else None
        return cls(cfg.route, cfg.top_k, _to_device(layer.wr, device),
                   None if layer.bias is None or cfg.route == "hash" else _to_device(layer.bias, device),
                   None if layer.tid2eid is None else _to_device(layer.tid2eid, device), r, sh)

    def clone(self) -> "DeviceLayer":
        """An independent device copy of every weight (same values, new memory)."""
        c = lambda t: None if t is None else t.clone()
        return DeviceLayer(self.route, self.top_k, c(self.wr), c(self.bias), c(self.tid2eid), self.routed.clone(),
                           None if self.shared is None else self.shared.clone(), self.router_c.routed_scale)

    # -- workspace ---------------------------------------------------------
    def workspace_size(self, max_tokens: int) -> int:
        n = _lib.load().moe_workspace_size(ctypes.byref(self.c), max_tokens)
        if n == 0:
            raise _lib.MoeError(_lib.MOE_ERR_INVALID_ARG, "moe_workspace_size")
        return n

    def workspace(self, max_tokens: int) -> torch.Tensor:
        ws = torch.empty(self.workspace_size(max_tokens), dtype=torch.uint8, device=self.wr.device)
        workspace_init(ws)
        return ws

    def workspace_layout(self, T: int) -> dict:
        """moe_workspace_layout: byte offsets of moe_forward's intermediates in
        the workspace for T tokens (0: not written), plus 'total' and 'fused'."""
        out = _lib.WsLayoutC()
        check(_lib.load().moe_workspace_layout(ctypes.byref(self.c), T, ctypes.byref(out)), "moe_workspace_layout")
        return {name: getattr(out, name) for name, _ in _lib.WsLayoutC._fields_}


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    check(_lib.load().moe_workspace_init(_ptr(ws), ws.numel(), _stream(stream)), "moe_workspace_init")


def device_error(ws: torch.Tensor, stream=None) -> int:
    code = ctypes.c_int32(0)
    check(_lib.load().moe_device_error(_ptr(ws), ctypes.byref(code), _stream(stream)), "moe_device_error")
    return code.value


def router_logits(layer: DeviceLayer, x: torch.Tensor, stream=None) -> torch.Tensor:
    x = _bits_tensor(x)
    T = x.shape[0]
    out = torch.empty((T, layer.E), dtype=torch.float32, device=x.device)
    check(_lib.load().moe_router_logits(ctypes.byref(layer.router_c), _ptr(x), T, _ptr(out), _stream(stream)),
          "moe_router_logits")
    return out


def route(layer: DeviceLayer, x: torch.Tensor, token_ids: Optional[torch.Tensor] = None,
          ws: Optional[torch.Tensor] = None, stream=None):
    x = _bits_tensor(x)
    T, k = x.shape[0], layer.top_k
    if ws is None:
        ws = layer.workspace(T)
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    check(_lib.load().moe_route(ctypes.byref(layer.router_c), _ptr(x), _ptr(token_ids), T, _ptr(ids), _ptr(w),
                                _ptr(ws), ws.numel(), _stream(stream)), "moe_route")
    return ids, w


def quantize_affine(w: torch.Tensor, bits: int, group: int, err: Optional[torch.Tensor] = None, stream=None):
    """Plain min/max affine quantisation of bf16 weights [rows][cols] (moe_quantize_affine):
    returns (codes uint32 [rows][cols*bits/32], scales fp16, biases fp16 [rows][cols/group])
    as device tensors (the fp16 ones as int16 bit patterns)."""
    w = _bits_tensor(w)
    rows, cols = w.shape
    codes = torch.empty((rows, cols * bits // 32), dtype=torch.int32, device=w.device)
    scales = torch.empty((rows, cols // group), dtype=torch.int16, device=w.device)
    biases = torch.empty_like(scales)
    check(_lib.load().moe_quantize_affine(_ptr(w), rows, cols, bits, group, _ptr(codes), _ptr(scales), _ptr(biases),
                                          None if err is None else _ptr(err), _stream(stream)), "moe_quantize_affine")
    return codes, scales, biases


def mhc_sinkhorn(logits: torch.Tensor, iters: int = 10, eps: float = 0.0, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """mHC mix matrices (moe_mhc_sinkhorn): logits fp32 [T][n][n] -> fp32 [T][n][n]."""
    if logits.dtype != torch.float32 or not logits.is_cuda or not logits.is_contiguous() or logits.dim() != 3:
        raise ValueError("logits must be a contiguous fp32 device tensor [T][n][n]")
    T, n, n2 = logits.shape
    if n != n2:
        raise ValueError("mix matrices must be square")
    out = torch.empty_like(logits) if out is None else out
    check(_lib.load().moe_mhc_sinkhorn(_ptr(logits), T, n, iters, eps, _ptr(out), _stream(stream)),
          "moe_mhc_sinkhorn")
    return out


def permute(ids: torch.Tensor, num_experts: int, ws: torch.Tensor, stream=None):
    T, k = ids.shape
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=ids.device)
    perm = torch.empty(T * k, dtype=torch.int32, device=ids.device)
    check(_lib.load().moe_permute(_ptr(ids), T, k, num_experts, _ptr(offsets), _ptr(perm), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_permute")
    return offsets, perm


def expert_ffn(layer: DeviceLayer, x: torch.Tensor, offsets: torch.Tensor, perm: torch.Tensor,
               ws: torch.Tensor, stream=None):
    x = _bits_tensor(x)
    T, k, d = x.shape[0], layer.top_k, layer.d
    y_slot = torch.empty((T * k, d), dtype=torch.float32, device=x.device)
    y_sh = torch.empty((T, d), dtype=torch.float32, device=x.device) if layer.shared is not None else None
    sh = ctypes.byref(layer._shared_c) if layer.shared is not None else None
    check(_lib.load().moe_expert_ffn(ctypes.byref(layer.routed.c), sh, _ptr(x), T, k, _ptr(offsets), _ptr(perm),
                                     _ptr(y_slot), _ptr(y_sh), _ptr(ws), ws.numel(), _stream(stream)),
          "moe_expert_ffn")
    return y_slot, y_sh


def combine(y_slot: torch.Tensor, w: torch.Tensor, y_shared: Optional[torch.Tensor], out_dtype: str = "bf16",
            stream=None) -> torch.Tensor:
    T, k = w.shape
    d = y_slot.shape[1]
    f32 = out_dtype == "f32"
    out = torch.empty((T, d), dtype=torch.float32 if f32 else torch.bfloat16, device=y_slot.device)
    check(_lib.load().moe_combine(_ptr(y_slot), _ptr(w), _ptr(y_shared), T, k, d,
                                  _lib.MOE_OUT_F32 if f32 else _lib.MOE_OUT_BF16, _ptr(out), _stream(stream)),
          "moe_combine")
    return out


def forward(layer: DeviceLayer, x: torch.Tensor, token_ids: Optional[torch.Tensor] = None,
            out_dtype: str = "bf16", ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    x = _bits_tensor(x)
    T = x.shape[0]
    if ws is None:
        ws = layer.workspace(T)
    if out is None:
        f32 = out_dtype == "f32"
        out = torch.empty((T, layer.d), dtype=torch.float32 if f32 else torch.bfloat16, device=x.device)
    else:  # a given output buffer decides the output type
        if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (T, layer.d):
            raise ValueError(f"out must be float32 or bfloat16 of shape ({T}, {layer.d})")
        f32 = out.dtype == torch.float32
    check(_lib.load().moe_forward(ctypes.byref(layer.c), _ptr(x), _ptr(token_ids), T,
                                  _lib.MOE_OUT_F32 if f32 else _lib.MOE_OUT_BF16, _ptr(out), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_forward")
    return out


def forward_noalloc(layer: DeviceLayer, x: torch.Tensor, token_ids: Optional[torch.Tensor], out: torch.Tensor,
                    stream=None) -> torch.Tensor:
    """moe_forward_noalloc: moe_forward on the library's own per-GPU workspace
    (no workspace argument; calls on one GPU must not overlap in time). The
    output type follows `out` (float32 or bfloat16)."""
    x = _bits_tensor(x)
    f32 = out.dtype == torch.float32
    check(_lib.load().moe_forward_noalloc(ctypes.byref(layer.c), _ptr(x), _ptr(token_ids), x.shape[0],
                                          _lib.MOE_OUT_F32 if f32 else _lib.MOE_OUT_BF16, _ptr(out),
                                          _stream(stream)), "moe_forward_noalloc")
    return out


def forward_probed(layer: DeviceLayer, x: torch.Tensor, token_ids: Optional[torch.Tensor], out: torch.Tensor,
                   ws: torch.Tensor, events, stream=None):
    """moe_forward with a (start, stop) event pair per kernel, timestamped by
    the dispatch itself: kernel i runs between events[2i] and events[2i+1].
    Returns the kernels' names. ``events`` are torch.cuda.Event(enable_timing=True),
    already created on the device (record them once first)."""
    x = _bits_tensor(x)
    n = len(events)
    evs = (ctypes.c_void_p * n)(*[ctypes.c_void_p(e.cuda_event) for e in events])
    names = (ctypes.c_char_p * n)()
    count = ctypes.c_int32(0)
    f32 = out.dtype == torch.float32
    check(_lib.load().moe_forward_probed(ctypes.byref(layer.c), _ptr(x), _ptr(token_ids), x.shape[0],
                                         _lib.MOE_OUT_F32 if f32 else _lib.MOE_OUT_BF16, _ptr(out), _ptr(ws),
                                         ws.numel(), _stream(stream), evs, n, names, ctypes.byref(count)),
          "moe_forward_probed")
    return [names[i].decode() for i in range(count.value)]


def ws_region(ws: torch.Tensor, offset: int, dtype: torch.dtype, shape) -> torch.Tensor:
    """A view of `shape` elements of `dtype` at byte `offset` of a workspace
    (for reading the intermediates moe_workspace_layout locates)."""
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.tensor([], dtype=dtype).element_size()
    if offset <= 0 or offset + nbytes > ws.numel():
        raise ValueError(f"region [{offset}, {offset + nbytes}) outside the workspace")
    return ws[offset:offset + nbytes].view(dtype).view(*shape)


def probe_stream(buf: torch.Tensor, mode: int, sink: Optional[torch.Tensor] = None, stream=None) -> None:
    """moe_probe_stream over all of `buf` (a contiguous device tensor):
    mode 0 dense read, 1 the first 32 bytes of every 128-byte line, 2 write.
    Reads need `sink`: 2048 int32 words on the device (one per workgroup)."""
    check(_lib.load().moe_probe_stream(_ptr(buf), buf.numel() * buf.element_size(), mode, _ptr(sink),
                                       _stream(stream)), "moe_probe_stream")


def probe_mfma(workgroups: int, iters: int, out: torch.Tensor, stream=None) -> None:
    """moe_probe_mfma into `out` (int64 [5] on the device, zeroed by the caller)."""
    check(_lib.load().moe_probe_mfma(workgroups, iters, _ptr(out), _stream(stream)), "moe_probe_mfma")


@dataclass
class Intermediates:
    ids: torch.Tensor
    w: torch.Tensor
    offsets: torch.Tensor
    perm: torch.Tensor
    y_slot: torch.Tensor
    y_shared: Optional[torch.Tensor]
    out: torch.Tensor


def forward_staged(layer: DeviceLayer, x: torch.Tensor, token_ids: Optional[torch.Tensor] = None,
                   out_dtype: str = "f32", ws: Optional[torch.Tensor] = None, stream=None) -> Intermediates:
    """The four entry points called one after another, keeping every intermediate."""
    T = x.shape[0]
    if ws is None:
        ws = layer.workspace(T)
    ids, w = route(layer, x, token_ids, ws, stream)
    offsets, perm = permute(ids, layer.E, ws, stream)
    y_slot, y_sh = expert_ffn(layer, x, offsets, perm, ws, stream)
    out = combine(y_slot, w, y_sh, out_dtype, stream)
    return Intermediates(ids, w, offsets, perm, y_slot, y_sh, out)
