"""Python binding of libmoe with the C ABI's names.

Argument marshalling only: tensors are passed as device pointers, the stream
is torch's current HIP stream, and every step of the layer runs in the HIP
kernels of libmoe.  Element types: torch.float32 (MOE_F32) or torch.bfloat16
(MOE_BF16); indices int32; routing weights float32.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import MoeDispatch, MoeForwardViews, MoeShape, MoeSizes, check, lib

_DT = {torch.float32: _lib.MOE_F32, torch.bfloat16: _lib.MOE_BF16}
_TORCH_DT = {v: k for k, v in _DT.items()}


@dataclasses.dataclass(frozen=True)
class Shape:
    T: int
    d: int
    E: int
    k: int
    F: int
    capacity: int = 0
    dtype: torch.dtype = torch.bfloat16
    tile_rows: int = 0  # 0: the library chooses
    weight_layout: int = 0  # 0: row-major expert weights; 1: blocked 16-row order (moe_pack_blocked16)

    def c(self) -> MoeShape:
        return MoeShape(self.T, self.d, self.E, self.k, self.F, self.capacity, _DT[self.dtype], self.tile_rows,
                        self.weight_layout)


def _p(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def query(shape: Shape) -> MoeSizes:
    out = MoeSizes()
    check("moe_query", lib().moe_query(ctypes.byref(shape.c()), ctypes.byref(out)))
    return out


def workspace_size(shape: Shape) -> int:
    """Bytes of workspace moe_forward needs (moe_workspace_size)."""
    n = ctypes.c_size_t()
    check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(shape.c()), ctypes.byref(n)))
    return n.value


class Dispatch:
    """Device buffer holding one moe_dispatch_t's arrays, with tensor views."""

    def __init__(self, shape: Shape, device="cuda", c: Optional[MoeDispatch] = None,
                 owner: Optional[torch.Tensor] = None):
        self.shape = shape
        if c is None:
            sz = query(shape)
            self.buf = torch.empty(sz.dispatch_bytes + 256, dtype=torch.uint8, device=device)
            base = (self.buf.data_ptr() + 255) // 256 * 256
            c = MoeDispatch()
            check("moe_dispatch_carve",
                  lib().moe_dispatch_carve(ctypes.byref(shape.c()), base, sz.dispatch_bytes, ctypes.byref(c)))
        else:
            self.buf = owner
        self.c = c

    def _view(self, name: str, n: int, dtype=torch.int32) -> torch.Tensor:
        ptr = getattr(self.c, name)
        off = ptr - self.buf.data_ptr()
        esz = torch.tensor([], dtype=dtype).element_size()
        return self.buf[off:off + n * esz].view(dtype)

    def arrays(self) -> dict:
        s, E, Tk = self.shape, self.shape.E, self.shape.T * self.shape.k
        R = query(s).rows
        mt = self.c.max_tiles
        return {
            "counts": self._view("counts", E),
            "offsets": self._view("offsets", E + 1),
            "spill_counts": self._view("spill_counts", E),
            "spill_offsets": self._view("spill_offsets", E + 1),
            "row_of": self._view("row_of", Tk),
            "token_of": self._view("token_of", R),
            "tile_off": self._view("tile_off", 2 * (E + 1)).view(2, E + 1),
            "tile_map": self._view("tile_map", 2 * mt * 4).view(2, mt, 4),
            "n_tiles": self._view("n_tiles", 2),
            "err_flags": self._view("err_flags", 1),
        }


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer whose data pointer is 256-byte aligned."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moe_route(shape: Shape, x, w_router, bias, topk_ids, topk_w, stream=None):
    check("moe_route", lib().moe_route(ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(topk_ids),
                                       _p(topk_w), _stream(stream)))


def moe_permute(shape: Shape, x, topk_ids, disp: Dispatch, x_perm, ws, stream=None):
    check("moe_permute", lib().moe_permute(ctypes.byref(shape.c()), _p(x), _p(topk_ids), ctypes.byref(disp.c),
                                           _p(x_perm), _p(ws), ws.numel(), _stream(stream)))


def moe_ffn_gate_up(shape: Shape, x_perm, w_gate, w_up, disp: Dispatch, pass_idx: int, h, stream=None):
    check("moe_ffn_gate_up", lib().moe_ffn_gate_up(ctypes.byref(shape.c()), _p(x_perm), _p(w_gate), _p(w_up),
                                                   ctypes.byref(disp.c), pass_idx, _p(h), _stream(stream)))


def moe_ffn_gate_up_gather(shape: Shape, x, w_gate, w_up, disp: Dispatch, pass_idx: int, h, stream=None):
    check("moe_ffn_gate_up_gather", lib().moe_ffn_gate_up_gather(
        ctypes.byref(shape.c()), _p(x), _p(w_gate), _p(w_up), ctypes.byref(disp.c), pass_idx, _p(h),
        _stream(stream)))


LAYOUT_ROWS = 0
LAYOUT_BLOCKED16 = 1
# pass argument of the grouped GEMM calls: both passes of the capacity mode in one launch
PASS_BOTH = 2


def moe_pack_blocked16(src, dst=None, stream=None):
    """Re-store a [..., rows, K] weight tensor (rows % 16 == 0, K * itemsize % 64 == 0)
    in the blocked 16-row order; returns dst (allocated like src if None)."""
    if dst is None:
        dst = torch.empty_like(src)
    if src.shape != dst.shape or src.dtype != dst.dtype:
        raise ValueError("dst must match src")
    rows = src.shape[-2]
    row_bytes = src.shape[-1] * src.element_size()
    matrices = src.numel() // (src.shape[-1] * rows)
    check("moe_pack_blocked16", lib().moe_pack_blocked16(_p(src), _p(dst), matrices, rows, row_bytes,
                                                         _stream(stream)))
    return dst


def moe_ffn_gate_up_fp8(shape: Shape, x, w_gate, w_up, s_gate, s_up, disp: Dispatch, pass_idx: int, h,
                        stream=None):
    """Gate+up with E4M3 weight codes (uint8 [E,F,d]) and per-channel fp32 scales [E,F]."""
    check("moe_ffn_gate_up_fp8", lib().moe_ffn_gate_up_fp8(
        ctypes.byref(shape.c()), _p(x), _p(w_gate), _p(w_up), _p(s_gate), _p(s_up), ctypes.byref(disp.c),
        pass_idx, _p(h), _stream(stream)))


def moe_ffn_down_fp8(shape: Shape, h, w_down, s_down, disp: Dispatch, pass_idx: int, y_perm, stream=None):
    """Down projection with E4M3 weight codes (uint8 [E,d,F]) and per-channel fp32 scales [E,d]."""
    check("moe_ffn_down_fp8", lib().moe_ffn_down_fp8(ctypes.byref(shape.c()), _p(h), _p(w_down), _p(s_down),
                                                     ctypes.byref(disp.c), pass_idx, _p(y_perm),
                                                     _stream(stream)))


def moe_ffn_down(shape: Shape, h, w_down, disp: Dispatch, pass_idx: int, y_perm, stream=None):
    check("moe_ffn_down", lib().moe_ffn_down(ctypes.byref(shape.c()), _p(h), _p(w_down), ctypes.byref(disp.c),
                                             pass_idx, _p(y_perm), _stream(stream)))


def moe_grouped_ffn(shape: Shape, x_perm, w_gate, w_up, w_down, disp: Dispatch, h, y_perm, stream=None):
    check("moe_grouped_ffn", lib().moe_grouped_ffn(ctypes.byref(shape.c()), _p(x_perm), _p(w_gate), _p(w_up),
                                                   _p(w_down), ctypes.byref(disp.c), _p(h), _p(y_perm),
                                                   _stream(stream)))


def moe_combine(shape: Shape, y_perm, topk_w, disp: Dispatch, out, stream=None):
    check("moe_combine", lib().moe_combine(ctypes.byref(shape.c()), _p(y_perm), _p(topk_w), ctypes.byref(disp.c),
                                           _p(out), _stream(stream)))


@dataclasses.dataclass
class ForwardViews:
    disp: Dispatch
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    x_perm: Optional[torch.Tensor]  # None: moe_forward reads x through token_of
    h: torch.Tensor
    y_perm: torch.Tensor


def _ws_view(ws: torch.Tensor, ptr: int, n: int, dtype) -> torch.Tensor:
    off = ptr - ws.data_ptr()
    esz = torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + n * esz].view(dtype)


def _forward_views(shape: Shape, v, ws, topk_ids, topk_w) -> ForwardViews:
    R = query(shape).rows
    Tk = shape.T * shape.k
    s = shape
    ids = topk_ids if topk_ids is not None else _ws_view(ws, v.topk_ids, Tk, torch.int32).view(s.T, s.k)
    wts = topk_w if topk_w is not None else _ws_view(ws, v.topk_w, Tk, torch.float32).view(s.T, s.k)
    return ForwardViews(
        disp=Dispatch(shape, c=v.disp, owner=ws),
        topk_ids=ids, topk_w=wts,
        x_perm=None,
        h=_ws_view(ws, v.h, R * s.F, s.dtype).view(R, s.F),
        y_perm=_ws_view(ws, v.y_perm, R * s.d, s.dtype).view(R, s.d),
    )


def moe_forward(shape: Shape, x, w_router, bias, topk_ids, topk_w, w_gate, w_up, w_down, out, ws,
                stream=None) -> ForwardViews:
    """The whole layer; returns views of the intermediates inside `ws`."""
    v = MoeForwardViews()
    check("moe_forward", lib().moe_forward(ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(topk_ids),
                                           _p(topk_w), _p(w_gate), _p(w_up), _p(w_down), _p(out), _p(ws),
                                           ws.numel(), ctypes.byref(v), _stream(stream)))
    return _forward_views(shape, v, ws, topk_ids, topk_w)


def moe_forward_fp8(shape: Shape, x, w_router, bias, topk_ids, topk_w, w_gate, w_up, w_down, s_gate, s_up,
                    s_down, out, ws, stream=None) -> ForwardViews:
    """The whole layer with E4M3 expert weight codes and per-channel fp32 scales."""
    v = MoeForwardViews()
    check("moe_forward_fp8", lib().moe_forward_fp8(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(topk_ids), _p(topk_w), _p(w_gate), _p(w_up),
        _p(w_down), _p(s_gate), _p(s_up), _p(s_down), _p(out), _p(ws), ws.numel(), ctypes.byref(v),
        _stream(stream)))
    return _forward_views(shape, v, ws, topk_ids, topk_w)


def moe_forward_noalloc(shape: Shape, x, w_router, bias, topk_ids, topk_w, w_gate, w_up, w_down, out,
                        stream=None) -> MoeForwardViews:
    """The whole layer with the library's own device scratch array instead of a
    workspace (for callers that cannot allocate); returns the raw views struct
    (device addresses inside that array, valid until the next call)."""
    v = MoeForwardViews()
    check("moe_forward_noalloc", lib().moe_forward_noalloc(
        ctypes.byref(shape.c()), _p(x), _p(w_router), _p(bias), _p(topk_ids), _p(topk_w), _p(w_gate), _p(w_up),
        _p(w_down), _p(out), ctypes.byref(v), _stream(stream)))
    return v
