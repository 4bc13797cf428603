"""Q2_K quantised decode for AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``libq2kdecode.so`` (declared in
``include/q2k_decode.h``). Each function has the name of its C entry point
and only marshals arguments: torch tensors in, device pointers and the
current HIP stream out. Every step runs in the library's HIP kernels; there
is no CPU fallback. A missing library raises on first use.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq2kdecode.so")

Q2K_OK = 0
ERROR_NAMES = {-1: "Q2K_EINVAL", -2: "Q2K_ESHAPE", -3: "Q2K_ESPACE", -4: "Q2K_EALIGN",
               -5: "Q2K_ELAUNCH", -6: "Q2K_EDEVICE"}
MAX_M = 8
BLOCK_BYTES = 84
BLOCK_WEIGHTS = 256

# (name, restype, argtypes) of every exported symbol of the header.
_VP, _I32, _I64, _SZ, _F32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                              ctypes.c_float)
SIGNATURES = {
    "q2k_abi_version": (_I32, []),
    "q2k_last_error": (ctypes.c_char_p, []),
    "q2k_set_product_kernel": (_I32, [_I32]),
    "q2k_product_kernel": (_I32, [_I32, _I32, _I32]),
    "q8_1_rows_bytes": (_SZ, [_I32, _I32]),
    "q8_1_rows": (_I32, [_VP, _I64, _VP, _SZ, _I32, _I32, _VP]),
    "q2k_mmvq": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _VP]),
    "q8_1_q2k_mmvq": (_I32, [_VP, _VP, _I64, _VP, _SZ, _VP, _I32, _I32, _I32, _VP]),
    "q2k_mmvq_pair": (_I32, [_VP, _VP, _I32, _VP, _VP, _I32, _VP, _I32, _I32, _VP]),
    "q8_1_q2k_mmvq_pair": (_I32, [_VP, _VP, _I32, _VP, _VP, _I32, _VP, _I64, _VP, _SZ, _I32, _I32,
                                  _VP]),
    "q2k_mmvq_experts": (_I32, [ctypes.POINTER(ctypes.c_void_p), _I32, _I64, _I32, _VP, _I32,
                                _VP, _I32, _VP, _I32, _I32, _I32, _VP, _VP]),
    "q8_1_q2k_mmvq_experts": (_I32, [ctypes.POINTER(ctypes.c_void_p), _I32, _I64, _I32, _VP, _I32,
                                     _VP, _I64, _VP, _SZ, _VP, _I32, _I32, _I32, _VP, _VP]),
    "q8_1_q2k_mmvq_experts_swiglu": (_I32, [ctypes.POINTER(ctypes.c_void_p), _I64, _I32, _VP, _I32,
                                            _VP, _VP, _SZ, _VP, _VP, _VP, _SZ, _I32, _I32, _VP, _VP]),
    "swiglu_q2k_mmvq_experts": (_I32, [ctypes.POINTER(ctypes.c_void_p), _I32, _I64, _I32, _VP,
                                       _I32, _VP, _VP, _VP, _SZ, _VP, _I32, _I32, _VP, _VP]),
    "q2k_mmvq_grouped": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _I32, _VP]),
    "q2k_mmq": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _VP]),
    "q2k_gemv_bf16": (_I32, [_VP, _VP, _I64, _VP, _I32, _I32, _I32, _VP]),
    "swiglu_q8_1_rows": (_I32, [_VP, _VP, _VP, _VP, _SZ, _I32, _I32, _VP]),
    "q2k_dequant_rows": (_I32, [_VP, _I64, _VP, _I32, _VP, _VP, _VP]),
    "q2k_dequant_rows_q8_1": (_I32, [_VP, _I64, _VP, _I32, _VP, _VP, _SZ, _VP, _VP]),
    "engram_gate": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _F32, _VP]),
    "engram_rows_q8_1": (_I32, [_VP, _I64, _VP, _VP, _VP, _I32, _I32, _I32, _I64, _VP, _I64, _VP, _I64,
                                _I32, _VP, _I64, _VP, _VP, _VP, _SZ, _VP, _VP]),
    "q2k_block_dots": (_I32, [_VP, _VP, _VP, _I32, _I32, _I32, _VP]),
    "engram_step_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "engram_step_noalloc": (_I32, [_VP, _I64, _VP, _VP, _VP, _I32, _I32, _I32, _I64, _VP, _I64, _VP, _I64,
                                   _I32, _VP, _I64, _VP, _VP, _VP, _I32, _I32, _F32, _VP, _VP]),
    "engram_step": (_I32, [_VP, _I64, _VP, _VP, _VP, _I32, _I32, _I32, _I64, _VP, _I64, _VP, _I64, _I32,
                           _VP, _I64, _VP, _VP, _VP, _I32, _I32, _F32, _VP, _SZ, _VP, _VP]),
    "engram_hash": (_I32, [_VP, _I64, _VP, _VP, _VP, _I32, _I32, _I32, _I64, _VP, _I64, _VP, _I32,
                           _I64, _VP, _VP, _VP]),
}

_lib: Optional[ctypes.CDLL] = None


class Q2KError(RuntimeError):
    """A non-zero status from the library, with its code and message."""

    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libq2kdecode.so (built in-tree); raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m q2_quantized_decode_amd.build`"
                " (hipcc, gfx950). There is no CPU fallback.")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, code: int) -> None:
    if code != Q2K_OK:
        msg = lib().q2k_last_error()
        raise Q2KError(fn, code, msg.decode() if msg else "")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda) tensor, got {t.device}")
    return t.data_ptr()


def _contig(t: torch.Tensor, name: str) -> int:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _dev(t, name)


def q2k_abi_version() -> int:
    return int(lib().q2k_abi_version())


KERNEL_AUTO, KERNEL_MATRIX_CORES, KERNEL_PACKED_DOTS = 0, 1, 2


def q2k_set_product_kernel(choice: int) -> int:
    """Process-wide product kernel choice (speed only: every choice returns
    the same bits); returns the previous one."""
    r = int(lib().q2k_set_product_kernel(choice))
    if r < 0:
        _check("q2k_set_product_kernel", r)
    return r


def q2k_product_kernel(n: int, k: int, m: int) -> int:
    """KERNEL_MATRIX_CORES or KERNEL_PACKED_DOTS: the kernel a single-matrix
    product of this shape runs under the current choice."""
    r = int(lib().q2k_product_kernel(n, k, m))
    if r < 0:
        _check("q2k_product_kernel", r)
    return r


def q8_1_rows_bytes(m: int, k: int) -> int:
    return int(lib().q8_1_rows_bytes(m, k))


def q8_1_rows(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q8_1 rows of a bf16 [m, k] tensor (row stride any multiple of 8)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a bf16 [m, k] tensor with unit column stride")
    m, k = x.shape
    need = q8_1_rows_bytes(m, k)
    if out is None:
        out = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check("q8_1_rows", lib().q8_1_rows(_dev(x, "x"), x.stride(0), _contig(out, "out"),
                                        out.numel(), m, k, _stream()))
    return out


def q2k_mmvq(w: torch.Tensor, xq: torch.Tensor, n: int, k: int, m: int,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """f32 [m, n] = Q2_K w [n, k] times q8_1 rows xq [m, k]."""
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check("q2k_mmvq", lib().q2k_mmvq(_contig(w, "w"), _contig(xq, "xq"), _contig(out, "out"),
                                      n, k, m, _stream()))
    return out


def q8_1_q2k_mmvq(w: torch.Tensor, x: torch.Tensor, n: int, k: int,
                  xq: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """q8_1 rows of bf16 x [m, k] into xq, then f32 [m, n] = w [n, k] times
    them: one call (one launch for a single token). Returns (y, xq)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a bf16 [m, k] tensor with unit column stride")
    m = x.shape[0]
    need = q8_1_rows_bytes(m, k)
    if xq is None:
        xq = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check("q8_1_q2k_mmvq", lib().q8_1_q2k_mmvq(
        _contig(w, "w"), _dev(x, "x"), x.stride(0), _contig(xq, "xq"), xq.numel(),
        _contig(out, "out"), n, k, m, _stream()))
    return out, xq


def q2k_mmvq_pair(wa: torch.Tensor, na: int, wb: torch.Tensor, nb: int, xq: torch.Tensor,
                  k: int, m: int, ya: Optional[torch.Tensor] = None,
                  yb: Optional[torch.Tensor] = None):
    """Two Q2_K matrices against the same q8_1 rows, one launch."""
    if ya is None:
        ya = torch.empty((m, na), dtype=torch.float32, device=wa.device)
    if yb is None:
        yb = torch.empty((m, nb), dtype=torch.float32, device=wb.device)
    _check("q2k_mmvq_pair", lib().q2k_mmvq_pair(
        _contig(wa, "wa"), _contig(ya, "ya"), na, _contig(wb, "wb"), _contig(yb, "yb"), nb,
        _contig(xq, "xq"), k, m, _stream()))
    return ya, yb


def q8_1_q2k_mmvq_pair(wa: torch.Tensor, na: int, wb: torch.Tensor, nb: int, x: torch.Tensor, k: int,
                       xq: Optional[torch.Tensor] = None, ya: Optional[torch.Tensor] = None,
                       yb: Optional[torch.Tensor] = None):
    """q8_1 rows of bf16 x [m, k] into xq, then the pair on them in one call.
    Returns (ya, yb, xq)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a bf16 [m, k] tensor with unit column stride")
    m = x.shape[0]
    need = q8_1_rows_bytes(m, k)
    if xq is None:
        xq = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if ya is None:
        ya = torch.empty((m, na), dtype=torch.float32, device=wa.device)
    if yb is None:
        yb = torch.empty((m, nb), dtype=torch.float32, device=wb.device)
    _check("q8_1_q2k_mmvq_pair", lib().q8_1_q2k_mmvq_pair(
        _contig(wa, "wa"), _contig(ya, "ya"), na, _contig(wb, "wb"), _contig(yb, "yb"), nb,
        _dev(x, "x"), x.stride(0), _contig(xq, "xq"), xq.numel(), k, m, _stream()))
    return ya, yb, xq


def q2k_mmvq_experts(bases: Sequence[torch.Tensor], expert_stride_bytes: int, n_experts: int,
                     ids: torch.Tensor, xq: torch.Tensor, x_per_id: bool, n: int, k: int,
                     m: int, out: Optional[torch.Tensor] = None,
                     err_flag: Optional[torch.Tensor] = None,
                     base_ptrs: Optional[Sequence[int]] = None) -> torch.Tensor:
    """f32 [n_bases, n_ids, m, n] for the expert ids in ``ids`` (int32, device).

    ``bases`` are the expert sets (expert e at byte e * expert_stride_bytes);
    ``base_ptrs`` may give explicit device addresses inside them instead."""
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    n_ids = ids.numel()
    ptrs = list(base_ptrs) if base_ptrs is not None else [_contig(b, "base") for b in bases]
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    if out is None:
        out = torch.empty((len(ptrs), n_ids, m, n), dtype=torch.float32, device=ids.device)
    flag = 0 if err_flag is None else _contig(err_flag, "err_flag")
    _check("q2k_mmvq_experts", lib().q2k_mmvq_experts(
        arr, len(ptrs), expert_stride_bytes, n_experts, _contig(ids, "ids"), n_ids,
        _contig(xq, "xq"), 1 if x_per_id else 0, _contig(out, "out"), n, k, m, flag or None,
        _stream()))
    return out


def q8_1_q2k_mmvq_experts(bases: Sequence[torch.Tensor], expert_stride_bytes: int, n_experts: int,
                          ids: torch.Tensor, x: torch.Tensor, n: int, k: int,
                          xq: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                          err_flag: Optional[torch.Tensor] = None):
    """q8_1 of the shared bf16 input x [m, k] into xq, then the expert batch
    on it (x_per_id = 0); one launch for one token. Returns (y, xq)."""
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a bf16 [m, k] tensor with unit column stride")
    m = x.shape[0]
    n_ids = ids.numel()
    ptrs = [_contig(b, "base") for b in bases]
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    need = q8_1_rows_bytes(m, k)
    if xq is None:
        xq = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((len(ptrs), n_ids, m, n), dtype=torch.float32, device=ids.device)
    flag = 0 if err_flag is None else _contig(err_flag, "err_flag")
    _check("q8_1_q2k_mmvq_experts", lib().q8_1_q2k_mmvq_experts(
        arr, len(ptrs), expert_stride_bytes, n_experts, _contig(ids, "ids"), n_ids, _dev(x, "x"),
        x.stride(0), _contig(xq, "xq"), xq.numel(), _contig(out, "out"), n, k, m, flag or None,
        _stream()))
    return out, xq


def q8_1_q2k_mmvq_experts_swiglu(bases: Sequence[torch.Tensor], expert_stride_bytes: int,
                                 n_experts: int, ids: torch.Tensor, x: torch.Tensor, n: int, k: int,
                                 xq: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                                 h: Optional[torch.Tensor] = None, hq: Optional[torch.Tensor] = None,
                                 want_h: bool = False, err_flag: Optional[torch.Tensor] = None):
    """Gate and up (bases = [gate set, up set]) of one bf16 token x [1, k],
    then the bf16 SwiGLU of the two result sets and its q8_1 rows: one
    launch where the shapes allow. Returns (y [2, n_ids, 1, n], xq, h or
    None, hq); hq feeds q2k_mmvq_experts(..., x_per_id=True)."""
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    if len(bases) != 2:
        raise ValueError("bases must be the gate and up expert sets")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[0] != 1 or x.stride(1) != 1:
        raise ValueError("x must be a bf16 [1, k] tensor with unit column stride")
    n_ids = ids.numel()
    ptrs = [_contig(b, "base") for b in bases]
    arr = (ctypes.c_void_p * 2)(*ptrs)
    need = q8_1_rows_bytes(1, k)
    if xq is None:
        xq = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((2, n_ids, 1, n), dtype=torch.float32, device=ids.device)
    if h is None and want_h:
        h = torch.empty((n_ids, n), dtype=torch.bfloat16, device=ids.device)
    hneed = q8_1_rows_bytes(n_ids, n)
    if hq is None:
        hq = torch.empty(max(hneed, 16), dtype=torch.uint8, device=ids.device)
    flag = 0 if err_flag is None else _contig(err_flag, "err_flag")
    _check("q8_1_q2k_mmvq_experts_swiglu", lib().q8_1_q2k_mmvq_experts_swiglu(
        arr, expert_stride_bytes, n_experts, _contig(ids, "ids"), n_ids, _dev(x, "x"),
        _contig(xq, "xq"), xq.numel(), _contig(out, "out"), _contig(h, "h") if h is not None else None,
        _contig(hq, "hq"), hq.numel(), n, k, flag or None, _stream()))
    return out, xq, h, hq


def swiglu_q2k_mmvq_experts(bases: Sequence[torch.Tensor], expert_stride_bytes: int, n_experts: int,
                            ids: torch.Tensor, g: torch.Tensor, u: torch.Tensor, n: int,
                            hq: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                            err_flag: Optional[torch.Tensor] = None):
    """h = bf16 SwiGLU of the f32 gate and up rows g, u [n_ids, k], its q8_1
    rows into hq, then the per-id expert product on them; one launch where
    the shapes allow. Returns (y [n_bases, n_ids, 1, n], hq)."""
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    if g.dtype != torch.float32 or u.dtype != torch.float32 or g.shape != u.shape or g.dim() != 2:
        raise ValueError("g and u must be f32 [n_ids, k] of one shape")
    n_ids, k = g.shape
    if n_ids != ids.numel():
        raise ValueError("g and u need one row per id")
    ptrs = [_contig(b, "base") for b in bases]
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    need = q8_1_rows_bytes(n_ids, k)
    if hq is None:
        hq = torch.empty(max(need, 16), dtype=torch.uint8, device=g.device)
    if out is None:
        out = torch.empty((len(ptrs), n_ids, 1, n), dtype=torch.float32, device=g.device)
    flag = 0 if err_flag is None else _contig(err_flag, "err_flag")
    _check("swiglu_q2k_mmvq_experts", lib().swiglu_q2k_mmvq_experts(
        arr, len(ptrs), expert_stride_bytes, n_experts, _contig(ids, "ids"), n_ids,
        _contig(g, "g"), _contig(u, "u"), _contig(hq, "hq"), hq.numel(), _contig(out, "out"), n, k,
        flag or None, _stream()))
    return out, hq


def q2k_mmq(w: torch.Tensor, xq: torch.Tensor, n: int, k: int, m: int,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """f32 [m, n] for any number of tokens m (up to 4096)."""
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check("q2k_mmq", lib().q2k_mmq(_contig(w, "w"), _contig(xq, "xq"), _contig(out, "out"), n, k, m,
                                    _stream()))
    return out


def q2k_mmvq_grouped(w: torch.Tensor, xq: torch.Tensor, groups: int, rows_per_group: int, k: int,
                     m: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """f32 [m, groups * rows_per_group]: row g*R + r of ``w`` against elements
    g*k .. g*k+k-1 of each q8_1 row (rows of width groups * k)."""
    if out is None:
        out = torch.empty((m, groups * rows_per_group), dtype=torch.float32, device=w.device)
    _check("q2k_mmvq_grouped", lib().q2k_mmvq_grouped(
        _contig(w, "w"), _contig(xq, "xq"), _contig(out, "out"), groups, rows_per_group, k, m,
        _stream()))
    return out


def q2k_gemv_bf16(w: torch.Tensor, x: torch.Tensor, n: int, k: int,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """f32 [m, n]: Q2_K [n, k] against bf16 x [m, k] (not quantised)."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a bf16 [m, k] tensor with unit column stride")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check("q2k_gemv_bf16", lib().q2k_gemv_bf16(_contig(w, "w"), _dev(x, "x"), x.stride(0),
                                                _contig(out, "out"), n, k, m, _stream()))
    return out


def swiglu_q8_1_rows(g: torch.Tensor, u: torch.Tensor, h: Optional[torch.Tensor] = None,
                     hq: Optional[torch.Tensor] = None, want_h: bool = True):
    """h = bf16(silu(g) * u) and its q8_1 rows; g, u f32 [rows, k]."""
    if g.dtype != torch.float32 or u.dtype != torch.float32 or g.shape != u.shape or g.dim() != 2:
        raise ValueError("g and u must be f32 [rows, k] of one shape")
    rows, k = g.shape
    if h is None and want_h:
        h = torch.empty((rows, k), dtype=torch.bfloat16, device=g.device)
    need = q8_1_rows_bytes(rows, k)
    if hq is None:
        hq = torch.empty(max(need, 16), dtype=torch.uint8, device=g.device)
    hp = _contig(h, "h") if h is not None else None
    _check("swiglu_q8_1_rows", lib().swiglu_q8_1_rows(
        _contig(g, "g"), _contig(u, "u"), hp, _contig(hq, "hq"), hq.numel(), rows, k, _stream()))
    return h, hq


def q2k_dequant_rows(table: torch.Tensor, n_table_rows: int, ids: Optional[torch.Tensor],
                     n_rows: int, out: Optional[torch.Tensor] = None,
                     err_flag: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [n_rows, 256] rows of a Q2_K table, gathered by int64 ``ids``."""
    if ids is not None and ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    if out is None:
        out = torch.empty((n_rows, BLOCK_WEIGHTS), dtype=torch.bfloat16, device=table.device)
    idp = _contig(ids, "ids") if ids is not None else None
    flag = _contig(err_flag, "err_flag") if err_flag is not None else None
    _check("q2k_dequant_rows", lib().q2k_dequant_rows(
        _contig(table, "table"), n_table_rows, idp, n_rows, _contig(out, "out"), flag, _stream()))
    return out


def q2k_dequant_rows_q8_1(table: torch.Tensor, n_table_rows: int, ids: Optional[torch.Tensor],
                          n_rows: int, xq: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, want_rows: bool = False,
                          err_flag: Optional[torch.Tensor] = None):
    """Gathered rows as one q8_1 row of width 256 * n_rows (and, with
    ``want_rows`` or ``out``, their bf16 [n_rows, 256] values)."""
    if ids is not None and ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    if out is None and want_rows:
        out = torch.empty((n_rows, BLOCK_WEIGHTS), dtype=torch.bfloat16, device=table.device)
    need = q8_1_rows_bytes(1, n_rows * BLOCK_WEIGHTS)
    if xq is None:
        xq = torch.empty(max(need, 16), dtype=torch.uint8, device=table.device)
    idp = _contig(ids, "ids") if ids is not None else None
    op = _contig(out, "out") if out is not None else None
    flag = _contig(err_flag, "err_flag") if err_flag is not None else None
    _check("q2k_dequant_rows_q8_1", lib().q2k_dequant_rows_q8_1(
        _contig(table, "table"), n_table_rows, idp, n_rows, op, _contig(xq, "xq"), xq.numel(), flag,
        _stream()))
    return xq, out


def engram_gate(h: torch.Tensor, kv: torch.Tensor, qk: torch.Tensor, eps: float) -> torch.Tensor:
    """In place on the f32 stream h [t, hc, dim]; kv f32 [t, (hc+1)*dim]; qk [hc, dim]."""
    if h.dtype != torch.float32 or kv.dtype != torch.float32 or qk.dtype != torch.float32:
        raise ValueError("h, kv and qk must be f32")
    if h.dim() != 3:
        raise ValueError("h must be [t, hc, dim]")
    t, hc, dim = h.shape
    _check("engram_gate", lib().engram_gate(_contig(h, "h"), _contig(kv, "kv"), _contig(qk, "qk"),
                                            t, hc, dim, float(eps), _stream()))
    return h


def _hash_tables(token_map: torch.Tensor, multipliers: torch.Tensor, primes: torch.Tensor,
                 offsets: torch.Tensor, cache: torch.Tensor):
    """Dtypes and shapes of the engram hash tables: multipliers int64
    [n_layers, max_ngram], primes int64 [n_layers, max_ngram - 1, n_heads],
    offsets int64 with one entry per prime. The kernels index these arrays
    from (n_layers, max_ngram, n_heads), so a mis-shaped table would read
    past its allocation: refused here. Returns (n_layers, max_ngram, n_heads)."""
    for name, t in (("token_map", token_map), ("multipliers", multipliers), ("primes", primes),
                    ("offsets", offsets), ("cache", cache)):
        if t.dtype != torch.int64:
            raise ValueError(f"{name} must be int64")
    if multipliers.dim() != 2 or primes.dim() != 3:
        raise ValueError("multipliers must be [n_layers, max_ngram] and primes "
                         "[n_layers, max_ngram - 1, n_heads]")
    n_layers, max_ngram = multipliers.shape
    if primes.shape[0] != n_layers or primes.shape[1] != max_ngram - 1:
        raise ValueError(f"primes {tuple(primes.shape)} does not match multipliers "
                         f"{tuple(multipliers.shape)}")
    if offsets.numel() != primes.numel():
        raise ValueError("offsets must hold one entry per prime")
    return n_layers, max_ngram, primes.shape[2]


def _engram_step_buffers(table: torch.Tensor, n_table_rows: int, wkv: torch.Tensor, qk: torch.Tensor,
                         h: torch.Tensor, token: torch.Tensor, cols: int):
    """Sizes of the engram step's buffers against its shapes (the kernels
    read table rows below n_table_rows, the whole wkv [(hc+1)*dim, cols*256]
    and qk [hc, dim])."""
    if token.dtype != torch.int32 or token.numel() < 1:
        raise ValueError("token must be int32 with one element")
    if h.dtype != torch.float32 or h.dim() != 3 or h.shape[0] != 1:
        raise ValueError("h must be f32 [1, hc, dim]")
    _, hc, dim = h.shape
    if table.numel() * table.element_size() < n_table_rows * BLOCK_BYTES:
        raise ValueError(f"table holds fewer than n_table_rows = {n_table_rows} blocks")
    if wkv.numel() * wkv.element_size() != (hc + 1) * dim * cols * BLOCK_BYTES:
        raise ValueError(f"wkv must be Q2_K [(hc+1)*dim, {cols * BLOCK_WEIGHTS}] for hc = {hc}, dim = {dim}")
    if qk.dtype != torch.float32 or qk.numel() != hc * dim:
        raise ValueError("qk must be f32 [hc, dim]")
    return hc, dim


def engram_hash(token_map: torch.Tensor, multipliers: torch.Tensor, primes: torch.Tensor,
                offsets: torch.Tensor, pad_id: int, cache: torch.Tensor, ids: torch.Tensor,
                start_pos: int, out: Optional[torch.Tensor] = None,
                err_flag: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int64 [n_layers, seqlen, (max_ngram-1)*n_heads] engram row ids for the
    int32 token ids at positions start_pos.. (the int64 ``cache`` is updated)."""
    n_layers, max_ngram, n_heads = _hash_tables(token_map, multipliers, primes, offsets, cache)
    if ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    cols = (max_ngram - 1) * n_heads
    seqlen = ids.numel()
    if out is None:
        out = torch.empty((n_layers, seqlen, cols), dtype=torch.int64, device=ids.device)
    flag = 0 if err_flag is None else _contig(err_flag, "err_flag")
    _check("engram_hash", lib().engram_hash(
        _contig(token_map, "token_map"), token_map.numel(), _contig(multipliers, "multipliers"),
        _contig(primes, "primes"), _contig(offsets, "offsets"), n_layers, max_ngram, n_heads,
        pad_id, _contig(cache, "cache"), cache.numel(), _contig(ids, "ids"), seqlen, start_pos,
        _contig(out, "out"), flag or None, _stream()))
    return out


def engram_rows_q8_1(token_map: torch.Tensor, multipliers: torch.Tensor, primes: torch.Tensor,
                     offsets: torch.Tensor, pad_id: int, cache: torch.Tensor, token: torch.Tensor,
                     pos: int, layer: int, table: torch.Tensor, n_table_rows: int,
                     xq: Optional[torch.Tensor] = None, ids_out: Optional[torch.Tensor] = None,
                     rows_out: Optional[torch.Tensor] = None,
                     err_flag: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode token (int32 ``token`` [1] at position ``pos``): hashed layer
    ``layer``'s row ids, their gather and dequantisation, and q8_1 of the rows
    viewed as one row, in one launch. Returns xq."""
    n_layers, max_ngram, n_heads = _hash_tables(token_map, multipliers, primes, offsets, cache)
    if token.dtype != torch.int32:
        raise ValueError("token must be int32")
    cols = (max_ngram - 1) * n_heads
    if table.numel() * table.element_size() < n_table_rows * BLOCK_BYTES:
        raise ValueError(f"table holds fewer than n_table_rows = {n_table_rows} blocks")
    need = q8_1_rows_bytes(1, cols * BLOCK_WEIGHTS)
    if xq is None:
        xq = torch.empty(max(need, 16), dtype=torch.uint8, device=table.device)
    opt = lambda t, n: _contig(t, n) if t is not None else None
    _check("engram_rows_q8_1", lib().engram_rows_q8_1(
        _contig(token_map, "token_map"), token_map.numel(), _contig(multipliers, "multipliers"),
        _contig(primes, "primes"), _contig(offsets, "offsets"), n_layers, max_ngram, n_heads, pad_id,
        _contig(cache, "cache"), cache.numel(), _contig(token, "token"), pos, layer,
        _contig(table, "table"), n_table_rows, opt(ids_out, "ids_out"), opt(rows_out, "rows_out"),
        _contig(xq, "xq"), xq.numel(), opt(err_flag, "err_flag"), _stream()))
    return xq


def q2k_block_dots(w: torch.Tensor, xq: torch.Tensor, n: int, k: int, m: int,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int32 [m, n, k/32, 2]: the exact (I, M) sums of the integer stage of the
    product of m tokens (q2k_mmvq up to 8 tokens, q2k_mmq past 8)."""
    if out is None:
        out = torch.empty((m, n, k // 32, 2), dtype=torch.int32, device=w.device)
    _check("q2k_block_dots", lib().q2k_block_dots(_contig(w, "w"), _contig(xq, "xq"),
                                                  _contig(out, "out"), n, k, m, _stream()))
    return out


def engram_step_workspace_bytes(max_ngram: int, n_heads: int, hc: int, dim: int) -> int:
    return int(lib().engram_step_workspace_bytes(max_ngram, n_heads, hc, dim))


def engram_step(token_map: torch.Tensor, multipliers: torch.Tensor, primes: torch.Tensor,
                offsets: torch.Tensor, pad_id: int, cache: torch.Tensor, token: torch.Tensor, pos: int,
                layer: int, table: torch.Tensor, n_table_rows: int, wkv: torch.Tensor, qk: torch.Tensor,
                h: torch.Tensor, eps: float, workspace: Optional[torch.Tensor] = None,
                err_flag: Optional[torch.Tensor] = None):
    """One decode token through the engram step: row ids of hashed layer
    ``layer``, gather + dequant + q8_1, the wkv projection into kv and the
    gate on h [1, hc, dim] in place. Returns (h, workspace); the workspace
    starts with kv f32 [(hc+1)*dim]."""
    n_layers, max_ngram, n_heads = _hash_tables(token_map, multipliers, primes, offsets, cache)
    hc, dim = _engram_step_buffers(table, n_table_rows, wkv, qk, h, token, (max_ngram - 1) * n_heads)
    need = engram_step_workspace_bytes(max_ngram, n_heads, hc, dim)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=h.device)
    flag = _contig(err_flag, "err_flag") if err_flag is not None else None
    _check("engram_step", lib().engram_step(
        _contig(token_map, "token_map"), token_map.numel(), _contig(multipliers, "multipliers"),
        _contig(primes, "primes"), _contig(offsets, "offsets"), n_layers, max_ngram, n_heads, pad_id,
        _contig(cache, "cache"), cache.numel(), _contig(token, "token"), pos, layer,
        _contig(table, "table"), n_table_rows, _contig(wkv, "wkv"), _contig(qk, "qk"), _contig(h, "h"),
        hc, dim, float(eps), _contig(workspace, "workspace"), workspace.numel(), flag, _stream()))
    return h, workspace


def engram_step_noalloc(token_map: torch.Tensor, multipliers: torch.Tensor, primes: torch.Tensor,
                        offsets: torch.Tensor, pad_id: int, cache: torch.Tensor, token: torch.Tensor,
                        pos: int, layer: int, table: torch.Tensor, n_table_rows: int, wkv: torch.Tensor,
                        qk: torch.Tensor, h: torch.Tensor, eps: float,
                        err_flag: Optional[torch.Tensor] = None) -> torch.Tensor:
    """engram_step with the library's own device array as its workspace (no
    allocation anywhere in the call); h [1, hc, dim] updated in place."""
    n_layers, max_ngram, n_heads = _hash_tables(token_map, multipliers, primes, offsets, cache)
    hc, dim = _engram_step_buffers(table, n_table_rows, wkv, qk, h, token, (max_ngram - 1) * n_heads)
    flag = _contig(err_flag, "err_flag") if err_flag is not None else None
    _check("engram_step_noalloc", lib().engram_step_noalloc(
        _contig(token_map, "token_map"), token_map.numel(), _contig(multipliers, "multipliers"),
        _contig(primes, "primes"), _contig(offsets, "offsets"), n_layers, max_ngram, n_heads, pad_id,
        _contig(cache, "cache"), cache.numel(), _contig(token, "token"), pos, layer,
        _contig(table, "table"), n_table_rows, _contig(wkv, "wkv"), _contig(qk, "qk"), _contig(h, "h"),
        hc, dim, float(eps), flag, _stream()))
    return h
