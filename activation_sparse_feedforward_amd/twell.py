"""Thin ctypes binding of libtwell (include/twell.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libtwell.so.  The binding checks what a raw pointer cannot carry -- that each
tensor lives on the GPU, is contiguous, has the expected dtype and is large
enough for the descriptor -- so that no kernel is ever handed a host pointer
or an undersized buffer.  If libtwell.so is missing the import of this module
still works, but every call raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass
from typing import NamedTuple, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtwell.so")

TWELL_OK, TWELL_EINVAL, TWELL_EUNSUPPORTED, TWELL_EHIP, TWELL_ESCRATCH = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 128 << 20  # TWELL_NOALLOC_SCRATCH_BYTES
TWELL_FP32, TWELL_BF16 = 0, 1

EXPORTED = ("twell_sizes", "twell_pack", "twell_pack_classic", "twell_ffn_fwd", "twell_ffn_fwd_hybrid",
            "twell_ffn_bwd", "twell_dense_ffn_fwd", "twell_status_str", "twell_ffn_fwd_hybrid_noalloc")


class TwellError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: status {code} ({status_str(code)})")
        self.code = code


class CDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("slots", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class CAct(ctypes.Structure):
    _fields_ = [("count", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("val", ctypes.c_void_p)]


class CRoute(ctypes.Structure):
    _fields_ = [("ell_rows", ctypes.c_void_p), ("dense_rows", ctypes.c_void_p), ("n_rows", ctypes.c_void_p),
                ("row_kind", ctypes.c_void_p), ("max_dense_rows", ctypes.c_int64)]


class CSizes(ctypes.Structure):
    _fields_ = [("count", ctypes.c_size_t), ("idx", ctypes.c_size_t), ("val", ctypes.c_size_t),
                ("ws_dense_fwd", ctypes.c_size_t), ("ws_hybrid", ctypes.c_size_t), ("ws_bwd", ctypes.c_size_t),
                ("ws_pack_classic", ctypes.c_size_t)]


_lib = None


def library() -> ctypes.CDLL:
    """Load libtwell.so once; raise if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m activation_sparse_feedforward_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, ST = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        D = ctypes.POINTER(CDesc)
        R = ctypes.POINTER(CRoute)
        sig = {
            "twell_sizes": (ST, [D, I64, ctypes.POINTER(CSizes)]),
            "twell_ffn_fwd_hybrid": (ST, [D, P, P, CAct, P, P, P, R, P, SZ, P]),
            "twell_ffn_fwd_hybrid_noalloc": (ST, [D, P, P, CAct, P, P, P, R, P]),
            "twell_ffn_bwd": (ST, [D, P, CAct, R, P, P, P, P, ctypes.c_float, P, P, P, P, P, SZ, P]),
            "twell_pack": (ST, [D, P, P, CAct, P, P, P]),
            "twell_pack_classic": (ST, [D, P, P, CAct, P, SZ, P]),
            "twell_ffn_fwd": (ST, [D, P, CAct, P, P, P, P]),
            "twell_dense_ffn_fwd": (ST, [D, P, P, P, P, P, P, SZ, P]),
            "twell_status_str": (ctypes.c_char_p, [ST]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib = lib
    return _lib


def status_str(code: int) -> str:
    return library().twell_status_str(int(code)).decode()


# ----------------------------------------------------------------------------- descriptor
@dataclass(frozen=True)
class Desc:
    T: int
    d_model: int
    d_ff: int
    tile_n: int
    slots: int
    dtype: str  # "fp32" | "bf16"

    @property
    def n_t(self) -> int:
        return self.d_ff // self.tile_n

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def c(self) -> CDesc:
        return CDesc(int(self.T), int(self.d_model), int(self.d_ff), int(self.tile_n), int(self.slots),
                     TWELL_BF16 if self.dtype == "bf16" else TWELL_FP32)

    def with_T(self, T: int) -> "Desc":
        return Desc(T, self.d_model, self.d_ff, self.tile_n, self.slots, self.dtype)


class Act(NamedTuple):
    """The three TwELL planes as device tensors."""
    count: torch.Tensor  # int32 [T, n_t]
    idx: torch.Tensor    # uint8 [T, n_t, C]
    val: torch.Tensor    # dtype [T, n_t, C]


class Route(NamedTuple):
    """Row routing of the hybrid format as device tensors."""
    ell_rows: torch.Tensor    # int32 [T]
    dense_rows: torch.Tensor  # int32 [max_dense_rows]
    n_rows: torch.Tensor      # int32 [3]: n_ell, n_dense, dense rows over the cap
    row_kind: torch.Tensor    # uint8 [T]: 1 = dense fallback

    @property
    def max_dense_rows(self) -> int:
        return int(self.dense_rows.numel())


# The entry points below share one C struct and one size table per descriptor
# (the library only reads the struct): at small batches the host cost of a
# call, not the kernels, sets the pace of a step.
@functools.lru_cache(maxsize=256)
def _cdesc(desc: Desc) -> CDesc:
    return desc.c()


@functools.lru_cache(maxsize=256)
def _sizes(desc: Desc, max_dense_rows: int) -> dict:
    out = CSizes()
    st = library().twell_sizes(ctypes.byref(_cdesc(desc)), ctypes.c_int64(max_dense_rows), ctypes.byref(out))
    if st != TWELL_OK:
        raise TwellError("twell_sizes", st)
    return {k: int(getattr(out, k)) for k, _ in CSizes._fields_}


def sizes(desc: Desc, max_dense_rows: int = 0) -> dict:
    return dict(_sizes(desc, int(max_dense_rows)))


def alloc_act(desc: Desc, device="cuda") -> Act:
    return Act(torch.empty((desc.T, desc.n_t), dtype=torch.int32, device=device),
               torch.empty((desc.T, desc.n_t, desc.slots), dtype=torch.uint8, device=device),
               torch.empty((desc.T, desc.n_t, desc.slots), dtype=desc.torch_dtype, device=device))


def alloc_route(desc: Desc, max_dense_rows: int, device="cuda") -> Route:
    return Route(torch.empty(max(desc.T, 1), dtype=torch.int32, device=device),
                 torch.empty(max_dense_rows, dtype=torch.int32, device=device),
                 torch.zeros(3, dtype=torch.int32, device=device),
                 torch.empty(max(desc.T, 1), dtype=torch.uint8, device=device))


# ----------------------------------------------------------------------------- checks
def _ptr(t: Optional[torch.Tensor], name: str, nbytes: int, dtype: Optional[torch.dtype] = None) -> int:
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.nbytes < nbytes:
        raise ValueError(f"{name}: {t.nbytes} bytes, need {nbytes}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _act(desc: Desc, act: Act) -> CAct:
    sz = _sizes(desc, 0)
    return CAct(_ptr(act.count, "count", sz["count"], torch.int32),
                _ptr(act.idx, "idx", sz["idx"], torch.uint8),
                _ptr(act.val, "val", sz["val"], desc.torch_dtype))


def _route(desc: Desc, route: Route) -> CRoute:
    cap = route.max_dense_rows
    return CRoute(_ptr(route.ell_rows, "ell_rows", desc.T * 4, torch.int32),
                  _ptr(route.dense_rows, "dense_rows", cap * 4, torch.int32) if cap else 0,
                  _ptr(route.n_rows, "n_rows", 12, torch.int32),
                  _ptr(route.row_kind, "row_kind", desc.T, torch.uint8), cap)


def _check(fn: str, st: int):
    if st != TWELL_OK:
        raise TwellError(fn, st)


# ----------------------------------------------------------------------------- entry points
def twell_pack(desc: Desc, x, w_gate_t, act: Act, stats=None, gate_dbg=None, stream=None):
    """Gate GEMM + ReLU + TwELL pack in one dispatch (see include/twell.h)."""
    e = 2 if desc.dtype == "bf16" else 4
    dt = desc.torch_dtype
    _check("twell_pack", library().twell_pack(
        ctypes.byref(_cdesc(desc)), _ptr(x, "x", desc.T * desc.d_model * e, dt),
        _ptr(w_gate_t, "w_gate_t", desc.d_ff * desc.d_model * e, dt), _act(desc, act),
        _ptr(stats, "stats", 16, torch.int64), _ptr(gate_dbg, "gate_dbg", desc.T * desc.d_ff * e, dt),
        _stream(stream)))


def twell_pack_classic(desc: Desc, x, w_gate_t, act: Act, ws, stream=None):
    """Baseline: dense gate GEMM writing ReLU(g) to ws, then a conversion kernel
    to the same TwELL planes (see include/twell.h)."""
    e = 2 if desc.dtype == "bf16" else 4
    dt = desc.torch_dtype
    need = _sizes(desc, 0)["ws_pack_classic"]
    _check("twell_pack_classic", library().twell_pack_classic(
        ctypes.byref(_cdesc(desc)), _ptr(x, "x", desc.T * desc.d_model * e, dt),
        _ptr(w_gate_t, "w_gate_t", desc.d_ff * desc.d_model * e, dt), _act(desc, act), _ptr(ws, "ws", need),
        ctypes.c_size_t(ws.numel() * ws.element_size() if ws is not None else 0), _stream(stream)))


def twell_ffn_fwd(desc: Desc, x, act: Act, w_up_t, w_down, y, stream=None):
    """Fused TwELL up + down projection: one fused kernel, dispatched once per
    generation of resident workgroups for large batches (see include/twell.h)."""
    e = 2 if desc.dtype == "bf16" else 4
    dt = desc.torch_dtype
    _check("twell_ffn_fwd", library().twell_ffn_fwd(
        ctypes.byref(_cdesc(desc)), _ptr(x, "x", desc.T * desc.d_model * e, dt), _act(desc, act),
        _ptr(w_up_t, "w_up_t", desc.d_ff * desc.d_model * e, dt),
        _ptr(w_down, "w_down", desc.d_ff * desc.d_model * e, dt),
        _ptr(y, "y", desc.T * desc.d_model * e, dt), _stream(stream)))


def twell_ffn_fwd_hybrid(desc: Desc, x, w_gate_t, act: Act, w_up_t, w_down, y, route: Route, ws, stream=None):
    """Router + fused TwELL path on ELL rows + dense MFMA fallback on dense rows."""
    e = 2 if desc.dtype == "bf16" else 4
    dt = desc.torch_dtype
    need = _sizes(desc, route.max_dense_rows)["ws_hybrid"]
    cr = _route(desc, route)
    _check("twell_ffn_fwd_hybrid", library().twell_ffn_fwd_hybrid(
        ctypes.byref(_cdesc(desc)), _ptr(x, "x", desc.T * desc.d_model * e, dt),
        _ptr(w_gate_t, "w_gate_t", desc.d_ff * desc.d_model * e, dt), _act(desc, act),
        _ptr(w_up_t, "w_up_t", desc.d_ff * desc.d_model * e, dt),
        _ptr(w_down, "w_down", desc.d_ff * desc.d_model * e, dt),
        _ptr(y, "y", desc.T * desc.d_model * e, dt), ctypes.byref(cr), _ptr(ws, "ws", need),
        ctypes.c_size_t(ws.numel() * ws.element_size() if ws is not None else 0), _stream(stream)))


def twell_ffn_fwd_hybrid_noalloc(desc: Desc, x, w_gate_t, act: Act, w_up_t, w_down, y, route: Route,
                                 stream=None):
    """twell_ffn_fwd_hybrid with the library's static device scratch as its
    workspace: allocates nothing (see include/twell.h for the size limit and
    the rule that calls on one device must not overlap)."""
    e = 2 if desc.dtype == "bf16" else 4
    dt = desc.torch_dtype
    cr = _route(desc, route)
    _check("twell_ffn_fwd_hybrid_noalloc", library().twell_ffn_fwd_hybrid_noalloc(
        ctypes.byref(_cdesc(desc)), _ptr(x, "x", desc.T * desc.d_model * e, dt),
        _ptr(w_gate_t, "w_gate_t", desc.d_ff * desc.d_model * e, dt), _act(desc, act),
        _ptr(w_up_t, "w_up_t", desc.d_ff * desc.d_model * e, dt),
        _ptr(w_down, "w_down", desc.d_ff * desc.d_model * e, dt),
        _ptr(y, "y", desc.T * desc.d_model * e, dt), ctypes.byref(cr), _stream(stream)))


def twell_ffn_bwd(desc: Desc, x, act: Act, route: Route, w_gate_t, w_up_t, w_down, dy, l1_coef: float,
                  dx, dw_gate_t, dw_up_t, dw_down, ws, stream=None):
    """Backward of the hybrid-format FFN with the L1 activation penalty (see include/twell.h)."""
    e = 2 if desc.dtype == "bf16" else 4
    dt = desc.torch_dtype
    need = _sizes(desc, route.max_dense_rows)["ws_bwd"]
    cr = _route(desc, route)
    wbytes = desc.d_ff * desc.d_model
    _check("twell_ffn_bwd", library().twell_ffn_bwd(
        ctypes.byref(_cdesc(desc)), _ptr(x, "x", desc.T * desc.d_model * e, dt), _act(desc, act), ctypes.byref(cr),
        _ptr(w_gate_t, "w_gate_t", wbytes * e, dt), _ptr(w_up_t, "w_up_t", wbytes * e, dt),
        _ptr(w_down, "w_down", wbytes * e, dt), _ptr(dy, "dy", desc.T * desc.d_model * e, dt),
        ctypes.c_float(l1_coef), _ptr(dx, "dx", desc.T * desc.d_model * e, dt),
        _ptr(dw_gate_t, "dw_gate_t", wbytes * 4, torch.float32), _ptr(dw_up_t, "dw_up_t", wbytes * 4, torch.float32),
        _ptr(dw_down, "dw_down", wbytes * 4, torch.float32), _ptr(ws, "ws", need),
        ctypes.c_size_t(ws.numel() * ws.element_size() if ws is not None else 0), _stream(stream)))


def twell_dense_ffn_fwd(desc: Desc, x, w_gate_t, w_up_t, w_down, y, ws, stream=None):
    """The library's dense MFMA FFN (gate|up GEMM with ReLU*u epilogue, then down)."""
    e = 2 if desc.dtype == "bf16" else 4
    dt = desc.torch_dtype
    need = _sizes(desc, 0)["ws_dense_fwd"]
    _check("twell_dense_ffn_fwd", library().twell_dense_ffn_fwd(
        ctypes.byref(_cdesc(desc)), _ptr(x, "x", desc.T * desc.d_model * e, dt),
        _ptr(w_gate_t, "w_gate_t", desc.d_ff * desc.d_model * e, dt),
        _ptr(w_up_t, "w_up_t", desc.d_ff * desc.d_model * e, dt),
        _ptr(w_down, "w_down", desc.d_ff * desc.d_model * e, dt),
        _ptr(y, "y", desc.T * desc.d_model * e, dt), _ptr(ws, "ws", need),
        ctypes.c_size_t(ws.numel() * ws.element_size() if ws is not None else 0), _stream(stream)))
