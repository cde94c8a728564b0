"""Thin ctypes binding over libq4moe.so (the C ABI in include/q4moe.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels.  The
library must be built (``python -m quantized_moe_decode_affine_amd.build``);
loading fails with an error otherwise, and there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq4moe.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
OUT_F32, OUT_BF16, OUT_BF16_RESIDUAL = 0, 1, 2  # residual: bf16(x + y), moe_ffn_decode only
OP_GEMV, OP_GEMM, OP_ROUTE, OP_PERMUTE, OP_FFN_DECODE, OP_FFN_PREFILL, OP_LMHEAD, OP_FFN_DECODE_BATCH = range(8)

EXPORTS = ("q4_gemv", "q4_gemm", "moe_route_topk", "moe_route_topk_q8", "moe_permute", "moe_ffn_decode", "moe_ffn_decode_noalloc",
           "moe_ffn_decode_batch",
           "moe_ffn_prefill", "lmhead_argmax", "q4moe_pack_group_major", "q4moe_workspace_bytes", "q4moe_strerror")


class Q4Error(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


class q4moe_matrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("count", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("reserved", ctypes.c_int32), ("codes_gm", ctypes.c_void_p)]


class q4moe_layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("router", ctypes.c_void_p),
                ("gate", q4moe_matrix), ("up", q4moe_matrix), ("down", q4moe_matrix),
                ("sh_gate", q4moe_matrix), ("sh_up", q4moe_matrix), ("sh_down", q4moe_matrix),
                ("router_q8", q4moe_matrix), ("sh_gate_w", ctypes.c_void_p)]


_lib = None


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    """Load libq4moe.so (once) and declare the entry points; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m quantized_moe_decode_affine_amd.build` "
                           "(the HIP library is the only implementation)")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    pm, pl = ctypes.POINTER(q4moe_matrix), ctypes.POINTER(q4moe_layer)
    sigs = {
        "q4_gemv": [pm, vp, vp, ctypes.c_int, vp],
        "q4_gemm": [pm, vp, i64, vp, ctypes.c_int, vp, sz, vp],
        "moe_route_topk": [vp, i32, i32, vp, i64, i32, vp, vp, vp, sz, vp],
        "moe_route_topk_q8": [pm, vp, i64, i32, vp, vp, vp, sz, vp],
        "moe_permute": [vp, i64, i32, i32, vp, vp, vp, vp, sz, vp],
        "moe_ffn_decode": [pl, vp, vp, ctypes.c_int, vp, vp, vp, sz, vp],
        "moe_ffn_decode_noalloc": [pl, vp, vp, ctypes.c_int, vp, vp, vp],
        "moe_ffn_decode_batch": [pl, vp, i64, vp, ctypes.c_int, vp, vp, vp, sz, vp],
        "moe_ffn_prefill": [pl, vp, i64, vp, ctypes.c_int, vp, sz, vp],
        "lmhead_argmax": [pm, vp, i64, vp, vp, vp, sz, vp],
        "q4moe_pack_group_major": [pm, vp, vp],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.q4moe_workspace_bytes.argtypes = [ctypes.c_int, pl, pm, i64]
    lib.q4moe_workspace_bytes.restype = sz
    lib.q4moe_strerror.argtypes = [ctypes.c_int]
    lib.q4moe_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise Q4Error(fn, status, load_library().q4moe_strerror(status).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


# --------------------------------------------------------------- device data --

def _dev(a: np.ndarray, device) -> torch.Tensor:
    """A numpy array of raw bits -> device tensor of the same bytes (uint32 -> int32, uint16 -> int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> a torch.bfloat16 device tensor."""
    return _dev(bits, device).view(torch.bfloat16)


class DeviceQ4:
    """An affine matrix (or a stack of them) resident on the device: 4-bit codes, or 8-bit
    codes when the code words per row hold 4 columns each (k is taken from the groups)."""

    def __init__(self, codes: np.ndarray, scales: np.ndarray, biases: np.ndarray, device="cuda"):
        if codes.ndim == 2:
            codes, scales, biases = codes[None], scales[None], biases[None]
        self.count, self.n, words = codes.shape
        self.k = scales.shape[-1] * 64
        if words * 8 == self.k:
            self.bits = 4
        elif words * 4 == self.k:
            self.bits = 8
        else:
            raise ValueError(f"{words} code words per row do not hold {self.k} columns at 4 or 8 bits")
        self.codes = _dev(codes, device)
        self.scales = _dev(scales, device)
        self.biases = _dev(biases, device)
        self.codes_gm = None
        self.struct = q4moe_matrix(self.codes.data_ptr(), self.scales.data_ptr(), self.biases.data_ptr(),
                                   self.count, self.n, self.k, self.bits, 0)

    def pack_group_major(self) -> None:
        """Add the group-major copy of the codes that the prefill GEMMs read (4-bit only)."""
        if self.bits != 4 or self.codes_gm is not None:
            return
        self.codes_gm = torch.empty_like(self.codes)
        _check("q4moe_pack_group_major", load_library().q4moe_pack_group_major(
            ctypes.byref(self.struct), _ptr(self.codes_gm), _stream()))
        self.struct.codes_gm = self.codes_gm.data_ptr()

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.biases))


class DeviceLayer:
    """MoE layer weights on the device plus the C descriptor that points at them."""

    def __init__(self, layer, device="cuda"):
        self.hidden, self.inter = layer.hidden, layer.inter
        self.n_experts, self.top_k = layer.n_experts, layer.top_k
        self.router = _dev(layer.router, device)
        self.gate = DeviceQ4(layer.gate.codes, layer.gate.scales, layer.gate.biases, device)
        self.up = DeviceQ4(layer.up.codes, layer.up.scales, layer.up.biases, device)
        self.down = DeviceQ4(layer.down.codes, layer.down.scales, layer.down.biases, device)
        self.has_shared = layer.has_shared
        if layer.has_shared:
            self.sh = [DeviceQ4(m.codes, m.scales, m.biases, device) for m in (layer.sh_gate, layer.sh_up, layer.sh_down)]
        else:
            self.sh = []
        rq8 = getattr(layer, "router_q8", None)
        self.router_q8 = DeviceQ4(*rq8, device=device) if rq8 is not None else None
        gw = getattr(layer, "sh_gate_w", None)
        self.sh_gate_w = _dev(gw, device) if gw is not None else None
        self._describe()

    def _describe(self) -> None:
        sh = [m.struct for m in self.sh] if self.has_shared else [q4moe_matrix() for _ in range(3)]
        new = q4moe_layer(self.hidden, self.inter, self.n_experts, self.top_k, self.router.data_ptr(),
                          self.gate.struct, self.up.struct, self.down.struct, *sh,
                          self.router_q8.struct if self.router_q8 is not None else q4moe_matrix(),
                          self.sh_gate_w.data_ptr() if self.sh_gate_w is not None else None)
        if hasattr(self, "struct"):  # rewritten in place: references taken to it stay current
            ctypes.memmove(ctypes.addressof(self.struct), ctypes.addressof(new), ctypes.sizeof(new))
        else:
            self.struct = new

    def pack_group_major(self) -> None:
        """Give every 4-bit expert matrix its group-major copy (moe_ffn_prefill reads those;
        the decode calls keep reading the row-major codes).  Doubles the 4-bit code memory."""
        for m in (self.gate, self.up, self.down, *self.sh):
            m.pack_group_major()
        self._describe()

    @property
    def nbytes(self) -> int:
        total = self.gate.nbytes + self.up.nbytes + self.down.nbytes + sum(m.nbytes for m in self.sh)
        return total + (self.router_q8.nbytes if self.router_q8 is not None else self.router.numel() * 2)


# ---------------------------------------------------------------- workspaces --

def workspace_bytes(op: int, layer: Optional[DeviceLayer] = None, W: Optional[DeviceQ4] = None,
                    rows: int = 0) -> int:
    lib = load_library()
    return lib.q4moe_workspace_bytes(op, ctypes.byref(layer.struct) if layer else None,
                                     ctypes.byref(W.struct) if W else None, rows)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled device byte buffer (torch's allocator returns 256-byte aligned blocks).

    Zero-filled because the decode workspace holds arrival counters and phase
    flags, and the LM-head workspace an arrival counter, that must be zero before
    their first use (each call leaves them ready for the next); the other
    operations do not care."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _out(shape, out_dtype, device, out=None):
    if out is not None:
        return out
    return torch.empty(shape, dtype=torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, device=device)


# --------------------------------------------------------------- entry points --

def q4_gemv(W: DeviceQ4, x: torch.Tensor, out_dtype: int = OUT_F32, out: Optional[torch.Tensor] = None):
    y = _out((W.count * W.n,), out_dtype, x.device, out)
    _check("q4_gemv", load_library().q4_gemv(ctypes.byref(W.struct), _ptr(x), _ptr(y), out_dtype, _stream()))
    return y


def q4_gemm(W: DeviceQ4, X: torch.Tensor, out_dtype: int = OUT_F32, out=None, ws: Optional[torch.Tensor] = None):
    m = X.shape[0]
    Y = _out((m, W.count * W.n), out_dtype, X.device, out)
    need = workspace_bytes(OP_GEMM, W=W, rows=m)
    ws = ws if ws is not None else workspace(need, X.device)
    _check("q4_gemm", load_library().q4_gemm(ctypes.byref(W.struct), _ptr(X), m, _ptr(Y), out_dtype, _ptr(ws),
                                             ws.numel(), _stream()))
    return Y


def moe_route_topk(router: torch.Tensor, X: torch.Tensor, top_k: int, ws: Optional[torch.Tensor] = None):
    E, H = router.shape
    T = X.shape[0]
    ids = torch.empty((T, top_k), dtype=torch.int32, device=X.device)
    w = torch.empty((T, top_k), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(load_library().q4moe_workspace_bytes(
            OP_ROUTE, ctypes.byref(q4moe_layer(H, 0, E, top_k)), None, T), X.device)
    _check("moe_route_topk", load_library().moe_route_topk(_ptr(router), E, H, _ptr(X), T, top_k, _ptr(ids),
                                                           _ptr(w), _ptr(ws), ws.numel(), _stream()))
    return ids, w


def moe_route_topk_q8(router_q8: DeviceQ4, X: torch.Tensor, top_k: int, ws: Optional[torch.Tensor] = None):
    """Top-k routing through an affine-Q8 router matrix (n_experts x hidden, 8-bit codes)."""
    E = router_q8.n
    T = X.shape[0]
    ids = torch.empty((T, top_k), dtype=torch.int32, device=X.device)
    w = torch.empty((T, top_k), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(load_library().q4moe_workspace_bytes(
            OP_ROUTE, ctypes.byref(q4moe_layer(router_q8.k, 0, E, top_k)), None, T), X.device)
    _check("moe_route_topk_q8", load_library().moe_route_topk_q8(ctypes.byref(router_q8.struct), _ptr(X), T, top_k,
                                                                 _ptr(ids), _ptr(w), _ptr(ws), ws.numel(), _stream()))
    return ids, w


def gpu_routing(layer: DeviceLayer, X: torch.Tensor):
    """The layer's routing of the rows X through its own router (bf16 or 8-bit)."""
    if layer.router_q8 is not None:
        return moe_route_topk_q8(layer.router_q8, X, layer.top_k)
    return moe_route_topk(layer.router, X, layer.top_k)


def moe_permute(ids: torch.Tensor, n_experts: int, ws: Optional[torch.Tensor] = None):
    T, k = ids.shape
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=ids.device)
    rows = torch.empty(T * k, dtype=torch.int32, device=ids.device)
    inv = torch.empty(T * k, dtype=torch.int32, device=ids.device)
    if ws is None:
        ws = workspace(load_library().q4moe_workspace_bytes(
            OP_PERMUTE, ctypes.byref(q4moe_layer(0, 0, n_experts, k)), None, T), ids.device)
    _check("moe_permute", load_library().moe_permute(_ptr(ids), T, k, n_experts, _ptr(offsets), _ptr(rows),
                                                     _ptr(inv), _ptr(ws), ws.numel(), _stream()))
    return offsets, rows, inv


# Byte offset of the decode workspace's abandoned-wait counter (include/q4moe.h, moe_ffn_decode).
DECODE_TIMEOUT_OFFSET = 2048


class DecodeTimeout(RuntimeError):
    """A decode launch gave up waiting for a value another workgroup publishes; its result is wrong."""


def decode_timeouts(ws: torch.Tensor) -> int:
    """The abandoned-wait counter of a decode workspace (synchronises with the device)."""
    return int(ws[DECODE_TIMEOUT_OFFSET:DECODE_TIMEOUT_OFFSET + 4].view(torch.int32).item())


def check_decode_workspace(ws: torch.Tensor) -> None:
    """Raise DecodeTimeout when any decode call that used `ws` abandoned a wait."""
    n = decode_timeouts(ws)
    if n:
        raise DecodeTimeout(f"{n} bounded wait(s) inside moe_ffn_decode gave up: the outputs written since the "
                            f"workspace was zeroed are wrong (were all workgroups resident at once?)")


def moe_ffn_decode(layer: DeviceLayer, x: torch.Tensor, out_dtype: int = OUT_F32, out=None,
                   ids_out: Optional[torch.Tensor] = None, w_out: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None):
    """One decode step through the layer.  With a workspace of its own (ws None) the call
    synchronises and raises DecodeTimeout if the launch abandoned a wait; a caller that passes
    `ws` checks it with check_decode_workspace when it synchronises."""
    y = _out((layer.hidden,), out_dtype, x.device, out)
    own = ws is None
    if own:
        ws = workspace(workspace_bytes(OP_FFN_DECODE, layer), x.device)
    _check("moe_ffn_decode", load_library().moe_ffn_decode(ctypes.byref(layer.struct), _ptr(x), _ptr(y), out_dtype,
                                                           _ptr(ids_out), _ptr(w_out), _ptr(ws), ws.numel(),
                                                           _stream()))
    if own:
        check_decode_workspace(ws)
    return y


def moe_ffn_decode_noalloc(layer: DeviceLayer, x: torch.Tensor, out_dtype: int = OUT_F32, out=None,
                           ids_out: Optional[torch.Tensor] = None, w_out: Optional[torch.Tensor] = None):
    """moe_ffn_decode on the library's fixed scratch array (no workspace, nothing allocated
    by the call; `out` must be given for that)."""
    y = _out((layer.hidden,), out_dtype, x.device, out)
    _check("moe_ffn_decode_noalloc", load_library().moe_ffn_decode_noalloc(
        ctypes.byref(layer.struct), _ptr(x), _ptr(y), out_dtype, _ptr(ids_out), _ptr(w_out), _stream()))
    return y


def moe_ffn_decode_batch(layer: DeviceLayer, X: torch.Tensor, out_dtype: int = OUT_F32, out=None,
                         ids_out: Optional[torch.Tensor] = None, w_out: Optional[torch.Tensor] = None,
                         ws: Optional[torch.Tensor] = None):
    B = X.shape[0]
    Y = _out((B, layer.hidden), out_dtype, X.device, out)
    if ws is None:
        ws = workspace(workspace_bytes(OP_FFN_DECODE_BATCH, layer, rows=B), X.device)
    _check("moe_ffn_decode_batch", load_library().moe_ffn_decode_batch(
        ctypes.byref(layer.struct), _ptr(X), B, _ptr(Y), out_dtype, _ptr(ids_out), _ptr(w_out), _ptr(ws),
        ws.numel(), _stream()))
    return Y


def moe_ffn_prefill(layer: DeviceLayer, X: torch.Tensor, out_dtype: int = OUT_F32, out=None,
                    ws: Optional[torch.Tensor] = None):
    T = X.shape[0]
    Y = _out((T, layer.hidden), out_dtype, X.device, out)
    if ws is None:
        ws = workspace(workspace_bytes(OP_FFN_PREFILL, layer, rows=T), X.device)
    _check("moe_ffn_prefill", load_library().moe_ffn_prefill(ctypes.byref(layer.struct), _ptr(X), T, _ptr(Y),
                                                             out_dtype, _ptr(ws), ws.numel(), _stream()))
    return Y


def lmhead_argmax(W: DeviceQ4, X: torch.Tensor, ws: Optional[torch.Tensor] = None, with_max: bool = True):
    B = X.shape[0]
    ids = torch.empty(B, dtype=torch.int32, device=X.device)
    mx = torch.empty(B, dtype=torch.float32, device=X.device) if with_max else None
    if ws is None:
        ws = workspace(workspace_bytes(OP_LMHEAD, W=W, rows=B), X.device)
    _check("lmhead_argmax", load_library().lmhead_argmax(ctypes.byref(W.struct), _ptr(X), B, _ptr(ids), _ptr(mx),
                                                         _ptr(ws), ws.numel(), _stream()))
    return ids, mx
