"""Python binding of the MI355X EXL3 library (libexl3.so, C ABI in include/exl3.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  The library
must have been built (``python -m gemm_exl3_linear_amd.build`` or
``__graft_entry__.build()``); importing this package does not load it, the
first call does, and a missing library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libexl3.so")
HEADER_PATH = os.path.join(ROOT, "include", "exl3.h")

EXL3_OK = 0
EXL3_E_INVALID = 1
EXL3_E_UNSUPPORTED = 2
EXL3_E_WORKSPACE = 3
EXL3_E_HIP = 4
EXL3_F16 = 0
EXL3_F32 = 1
CODEBOOK_MUL1 = 2
MAX_TOPK = 16
MAX_MULTI = 8
SCRATCH_BYTES = 32 << 20  # EXL3_SCRATCH_BYTES


class Exl3Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


class _Weight(ctypes.Structure):
    _fields_ = [("trellis", ctypes.c_void_p), ("suh", ctypes.c_void_p), ("svh", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("k", ctypes.c_int32), ("n", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("codebook", ctypes.c_int32)]


class _Arena(ctypes.Structure):
    _fields_ = [("trellis", ctypes.c_void_p), ("suh", ctypes.c_void_p), ("svh", ctypes.c_void_p),
                ("experts", ctypes.c_int32), ("slots", ctypes.c_int32), ("k", ctypes.c_int32),
                ("n", ctypes.c_int32), ("bits", ctypes.c_int32), ("codebook", ctypes.c_int32)]


class _Widths(ctypes.Structure):
    _fields_ = [("bits_host", ctypes.c_void_p), ("bits", ctypes.c_void_p), ("offsets", ctypes.c_void_p)]


_lib = None


def header_functions() -> list[str]:
    """Names of the functions include/exl3.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(exl3_[a-z_0-9]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """Load libexl3.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m gemm_exl3_linear_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.exl3_abi_version.restype = i32
    L.exl3_abi_version.argtypes = []
    L.exl3_status_str.restype = ctypes.c_char_p
    L.exl3_status_str.argtypes = [i32]
    L.exl3_reconstruct.restype = i32
    L.exl3_reconstruct.argtypes = [ctypes.POINTER(_Weight), vp, vp]
    L.exl3_hadamard.restype = i32
    L.exl3_hadamard.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, vp]
    L.exl3_linear_workspace_size.restype = sz
    L.exl3_linear_workspace_size.argtypes = [ctypes.POINTER(_Weight), i64]
    L.exl3_linear.restype = i32
    L.exl3_linear.argtypes = [ctypes.POINTER(_Weight), vp, i64, i64, vp, i64, i32, vp, sz, vp]
    L.exl3_linear_no_workspace.restype = i32
    L.exl3_linear_no_workspace.argtypes = [ctypes.POINTER(_Weight), vp, i64, i64, vp, i64, i32, vp]
    L.exl3_reconstruct_int8.restype = i32
    L.exl3_reconstruct_int8.argtypes = [ctypes.POINTER(_Weight), vp, vp]
    L.exl3_linear_int8_workspace_size.restype = sz
    L.exl3_linear_int8_workspace_size.argtypes = [ctypes.POINTER(_Weight), i64]
    L.exl3_linear_int8.restype = i32
    L.exl3_linear_int8.argtypes = [ctypes.POINTER(_Weight), vp, i64, i64, vp, i64, i32, vp, sz, vp]
    L.exl3_linear_multi_workspace_size.restype = sz
    L.exl3_linear_multi_workspace_size.argtypes = [ctypes.POINTER(ctypes.POINTER(_Weight)), i32, i64]
    L.exl3_linear_multi.restype = i32
    L.exl3_linear_multi.argtypes = [ctypes.POINTER(ctypes.POINTER(_Weight)), i32, vp, i64, i64,
                                    ctypes.POINTER(vp), ctypes.POINTER(i64), i32, vp, sz, vp]
    L.exl3_grouped_experts_workspace_size.restype = sz
    L.exl3_grouped_experts_workspace_size.argtypes = [ctypes.POINTER(_Arena), ctypes.POINTER(_Arena), i64, i32]
    L.exl3_grouped_experts.restype = i32
    L.exl3_grouped_experts.argtypes = [ctypes.POINTER(_Arena), ctypes.POINTER(_Arena), vp, vp, vp, i64, i32,
                                       vp, vp, sz, vp]
    Wp = ctypes.POINTER(_Widths)
    L.exl3_grouped_experts_mixed_workspace_size.restype = sz
    L.exl3_grouped_experts_mixed_workspace_size.argtypes = [ctypes.POINTER(_Arena), Wp, ctypes.POINTER(_Arena),
                                                            Wp, i64, i32]
    L.exl3_grouped_experts_mixed.restype = i32
    L.exl3_grouped_experts_mixed.argtypes = [ctypes.POINTER(_Arena), Wp, ctypes.POINTER(_Arena), Wp, vp, vp, vp,
                                             i64, i32, vp, vp, sz, vp]
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().exl3_status_str(int(status)).decode()


def abi_version() -> int:
    return int(lib().exl3_abi_version())


def _check(status: int, what: str):
    if status != EXL3_OK:
        raise Exl3Error(status, what)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


# ---------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------
@dataclass
class Exl3Weight:
    """One EXL3 tensor on the GPU: trellis int16/uint16 [k/16, n/16, 16*bits],
    suh fp16 [k], svh fp16 [n], optional bias fp16 [n]."""
    trellis: "object"
    suh: "object"
    svh: "object"
    bits: int
    bias: Optional["object"] = None
    codebook: int = CODEBOOK_MUL1

    @property
    def k(self) -> int:
        return int(self.trellis.shape[0]) * 16

    @property
    def n(self) -> int:
        return int(self.trellis.shape[1]) * 16

    def _c(self) -> _Weight:
        return _Weight(_ptr(self.trellis), _ptr(self.suh), _ptr(self.svh), _ptr(self.bias),
                       self.k, self.n, int(self.bits), int(self.codebook))

    @staticmethod
    def from_numpy(trellis, suh, svh, bits, bias=None, device="cuda"):
        import torch
        t = torch.from_numpy(trellis.view("int16").copy()).to(device)
        s1 = torch.from_numpy(suh.astype("float16")).to(device)
        s2 = torch.from_numpy(svh.astype("float16")).to(device)
        b = None if bias is None else torch.from_numpy(bias.astype("float16")).to(device)
        return Exl3Weight(t, s1, s2, bits, b)


@dataclass
class Exl3Arena:
    """Packed expert arena on the GPU: trellis [E, slots, k/16, n/16, 16*bits],
    suh fp16 [E, slots, k], svh fp16 [E, slots, n]."""
    trellis: "object"
    suh: "object"
    svh: "object"
    bits: int
    codebook: int = CODEBOOK_MUL1

    @property
    def experts(self) -> int:
        return int(self.trellis.shape[0])

    @property
    def slots(self) -> int:
        return int(self.trellis.shape[1])

    @property
    def k(self) -> int:
        return int(self.trellis.shape[2]) * 16

    @property
    def n(self) -> int:
        return int(self.trellis.shape[3]) * 16

    def _c(self) -> _Arena:
        return _Arena(_ptr(self.trellis), _ptr(self.suh), _ptr(self.svh), self.experts, self.slots,
                      self.k, self.n, int(self.bits), int(self.codebook))

    @staticmethod
    def from_numpy(arena: dict, device="cuda"):
        import torch
        return Exl3Arena(torch.from_numpy(arena["trellis"].view("int16").copy()).to(device),
                         torch.from_numpy(arena["suh"].astype("float16")).to(device),
                         torch.from_numpy(arena["svh"].astype("float16")).to(device),
                         int(arena["bits"]))


@dataclass
class Exl3MixedArena:
    """Expert arena with a width per expert on the GPU: trellis int16/uint16
    [total words] with expert e's slots at word offsets[e] on, widths int32
    [E] both on the host (``bits_host``, a ctypes array the record points to)
    and on the GPU (``bits``), offsets int64 [E] on the GPU, suh fp16
    [E, slots, k], svh fp16 [E, slots, n]."""
    trellis: "object"
    suh: "object"
    svh: "object"
    bits: "object"
    offsets: "object"
    bits_host: "object"
    codebook: int = CODEBOOK_MUL1

    @property
    def experts(self) -> int:
        return int(self.suh.shape[0])

    @property
    def slots(self) -> int:
        return int(self.suh.shape[1])

    @property
    def k(self) -> int:
        return int(self.suh.shape[2])

    @property
    def n(self) -> int:
        return int(self.svh.shape[2])

    def _c(self) -> _Arena:
        return _Arena(_ptr(self.trellis), _ptr(self.suh), _ptr(self.svh), self.experts, self.slots,
                      self.k, self.n, 0, int(self.codebook))

    def _w(self) -> _Widths:
        return _Widths(ctypes.addressof(self.bits_host), _ptr(self.bits), _ptr(self.offsets))

    @staticmethod
    def from_numpy(arena: dict, device="cuda"):
        """Packs the per-expert trellis arrays (entry e [slots, k/16, n/16,
        16*bits[e]]) one after the other into one allocation."""
        import numpy as np
        import torch
        widths = [int(b) for b in arena["bits"]]
        sizes = [int(t.size) for t in arena["trellis"]]
        offsets = np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)
        flat = np.concatenate([np.ascontiguousarray(t).reshape(-1) for t in arena["trellis"]])
        host = (ctypes.c_int32 * len(widths))(*widths)
        return Exl3MixedArena(torch.from_numpy(flat.view("int16").copy()).to(device),
                              torch.from_numpy(arena["suh"].astype("float16")).to(device),
                              torch.from_numpy(arena["svh"].astype("float16")).to(device),
                              torch.tensor(widths, dtype=torch.int32, device=device),
                              torch.from_numpy(offsets).to(device), host)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def exl3_reconstruct(w: Exl3Weight, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((w.k, w.n), dtype=torch.float16, device=w.trellis.device)
    cw = w._c()
    _check(lib().exl3_reconstruct(ctypes.byref(cw), _ptr(out), _stream(stream)), "exl3_reconstruct")
    return out


def exl3_hadamard(x, sign_before=None, sign_after=None, out=None, stream=None):
    import torch
    assert x.dim() == 2 and x.stride(1) == 1
    dtype = {torch.float16: EXL3_F16, torch.float32: EXL3_F32}[x.dtype]
    if out is None:
        out = torch.empty_like(x)
    rows, dim = x.shape
    _check(lib().exl3_hadamard(_ptr(x), _ptr(out), dtype, rows, dim, x.stride(0), out.stride(0),
                               _ptr(sign_before), _ptr(sign_after), _stream(stream)), "exl3_hadamard")
    return out


def exl3_linear_workspace_size(w: Exl3Weight, m: int) -> int:
    cw = w._c()
    return int(lib().exl3_linear_workspace_size(ctypes.byref(cw), int(m)))


def _ydt(dtype) -> int:
    import torch
    if dtype == torch.float16:
        return EXL3_F16
    if dtype == torch.float32:
        return EXL3_F32
    raise ValueError(f"output dtype {dtype} is not fp16 or fp32")


def exl3_linear(x, w: Exl3Weight, out_dtype=None, out=None, workspace=None, stream=None):
    import torch
    assert x.dim() == 2 and x.dtype == torch.float16 and x.stride(1) == 1
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.n), dtype=out_dtype or torch.float16, device=x.device)
    ydt = _ydt(out.dtype)
    cw = w._c()
    if workspace is None:  # a caller's workspace is checked against the size by the library
        need = int(lib().exl3_linear_workspace_size(ctypes.byref(cw), int(m)))
        if need:  # scratch only: no clearing needed
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().exl3_linear(ctypes.byref(cw), _ptr(x), m, x.stride(0), _ptr(out), out.stride(0), ydt,
                             _ptr(workspace), wsb, _stream(stream)), "exl3_linear")
    return out


def exl3_linear_no_workspace(x, w: Exl3Weight, out, stream=None):
    """exl3_linear_no_workspace: exl3_linear with the library's own device
    array as workspace; the caller passes the output (nothing is allocated
    here or in the library)."""
    import torch
    assert x.dim() == 2 and x.dtype == torch.float16 and x.stride(1) == 1
    assert out.dim() == 2 and out.shape[0] == x.shape[0]
    cw = w._c()
    _check(lib().exl3_linear_no_workspace(ctypes.byref(cw), _ptr(x), x.shape[0], x.stride(0), _ptr(out),
                                          out.stride(0), _ydt(out.dtype), _stream(stream)),
           "exl3_linear_no_workspace")
    return out


def exl3_reconstruct_int8(w: Exl3Weight, out=None, stream=None):
    """int8 weights W_q [k, n] of the int8 prefill (exl3_reconstruct_int8)."""
    import torch
    if out is None:
        out = torch.empty((w.k, w.n), dtype=torch.int8, device=w.trellis.device)
    cw = w._c()
    _check(lib().exl3_reconstruct_int8(ctypes.byref(cw), _ptr(out), _stream(stream)),
           "exl3_reconstruct_int8")
    return out


def exl3_linear_int8_workspace_size(w: Exl3Weight, m: int) -> int:
    cw = w._c()
    return int(lib().exl3_linear_int8_workspace_size(ctypes.byref(cw), int(m)))


def exl3_linear_int8(x, w: Exl3Weight, out_dtype=None, out=None, workspace=None, stream=None):
    """The int8 prefill linear (exl3_linear_int8): x fp16 [m, k] -> y [m, n]."""
    import torch
    assert x.dim() == 2 and x.dtype == torch.float16 and x.stride(1) == 1
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.n), dtype=out_dtype or torch.float16, device=x.device)
    ydt = _ydt(out.dtype)
    cw = w._c()
    if workspace is None:
        need = int(lib().exl3_linear_int8_workspace_size(ctypes.byref(cw), int(m)))
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().exl3_linear_int8(ctypes.byref(cw), _ptr(x), m, x.stride(0), _ptr(out), out.stride(0),
                                  ydt, _ptr(workspace), wsb, _stream(stream)), "exl3_linear_int8")
    return out


def _weight_array(ws):
    """ctypes array of pointers to the tensors' C records (records kept alive)."""
    recs = [w._c() for w in ws]
    arr = (ctypes.POINTER(_Weight) * len(recs))(*[ctypes.pointer(r) for r in recs])
    return arr, recs


def exl3_linear_multi_workspace_size(ws, m: int) -> int:
    arr, _recs = _weight_array(ws)
    return int(lib().exl3_linear_multi_workspace_size(arr, len(ws), int(m)))


def exl3_linear_multi(x, ws, out_dtype=None, outs=None, workspace=None, stream=None):
    """y[i] = exl3_linear(x, ws[i]) for tensors that share the input x (same k)."""
    import torch
    assert x.dim() == 2 and x.dtype == torch.float16 and x.stride(1) == 1
    m = x.shape[0]
    if outs is None:
        outs = [torch.empty((m, w.n), dtype=out_dtype or torch.float16, device=x.device) for w in ws]
    ydt = _ydt(outs[0].dtype)
    arr, _recs = _weight_array(ws)
    if workspace is None:
        need = int(lib().exl3_linear_multi_workspace_size(arr, len(ws), int(m)))
        if need:  # scratch only: no clearing needed
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    yp = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    ld = (ctypes.c_int64 * len(outs))(*[o.stride(0) for o in outs])
    _check(lib().exl3_linear_multi(arr, len(ws), _ptr(x), m, x.stride(0), yp, ld, ydt, _ptr(workspace), wsb,
                                   _stream(stream)), "exl3_linear_multi")
    return outs


def exl3_grouped_experts_workspace_size(gate_up: Exl3Arena, down: Exl3Arena, t: int, topk: int) -> int:
    a, b = gate_up._c(), down._c()
    return int(lib().exl3_grouped_experts_workspace_size(ctypes.byref(a), ctypes.byref(b), int(t), int(topk)))


def exl3_grouped_experts(x, topk_ids, topk_weights, gate_up: Exl3Arena, down: Exl3Arena, out=None,
                         workspace=None, stream=None):
    import torch
    assert x.dtype == torch.float16 and x.is_contiguous()
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous()
    assert topk_weights.dtype == torch.float32 and topk_weights.is_contiguous()
    t, topk = topk_ids.shape
    if out is None:
        out = torch.empty((t, down.n), dtype=torch.float32, device=x.device)
    a, b = gate_up._c(), down._c()
    if workspace is None:
        need = int(lib().exl3_grouped_experts_workspace_size(ctypes.byref(a), ctypes.byref(b), int(t), int(topk)))
        if need:
            workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().exl3_grouped_experts(ctypes.byref(a), ctypes.byref(b), _ptr(x), _ptr(topk_ids),
                                      _ptr(topk_weights), t, topk, _ptr(out), _ptr(workspace), wsb,
                                      _stream(stream)), "exl3_grouped_experts")
    return out


def exl3_grouped_experts_mixed_workspace_size(gate_up: Exl3MixedArena, down: Exl3MixedArena, t: int,
                                              topk: int) -> int:
    a, b = gate_up._c(), down._c()
    wa, wb = gate_up._w(), down._w()
    return int(lib().exl3_grouped_experts_mixed_workspace_size(ctypes.byref(a), ctypes.byref(wa), ctypes.byref(b),
                                                               ctypes.byref(wb), int(t), int(topk)))


def exl3_grouped_experts_mixed(x, topk_ids, topk_weights, gate_up: Exl3MixedArena, down: Exl3MixedArena,
                               out=None, workspace=None, stream=None):
    """exl3_grouped_experts over arenas whose experts each have their own width."""
    import torch
    assert x.dtype == torch.float16 and x.is_contiguous()
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous()
    assert topk_weights.dtype == torch.float32 and topk_weights.is_contiguous()
    t, topk = topk_ids.shape
    if out is None:
        out = torch.empty((t, down.n), dtype=torch.float32, device=x.device)
    a, b = gate_up._c(), down._c()
    wa, wb = gate_up._w(), down._w()
    if workspace is None:
        need = int(lib().exl3_grouped_experts_mixed_workspace_size(ctypes.byref(a), ctypes.byref(wa),
                                                                   ctypes.byref(b), ctypes.byref(wb), int(t),
                                                                   int(topk)))
        if need:
            workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().exl3_grouped_experts_mixed(ctypes.byref(a), ctypes.byref(wa), ctypes.byref(b), ctypes.byref(wb),
                                            _ptr(x), _ptr(topk_ids), _ptr(topk_weights), t, topk, _ptr(out),
                                            _ptr(workspace), wsb, _stream(stream)), "exl3_grouped_experts_mixed")
    return out
