"""Binding of libmoe_peaks: measurement probes of the achievable HBM streaming
rate and bf16 matrix-core throughput (the ceilings a roofline of the expert
GEMMs is drawn against).  Argument marshalling only; the probes run as HIP
kernels in libmoe_peaks.so.  Declarations and exact result definitions are in
include/moe_peaks.h."""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_peaks.so")
EXPORTED = ["moe_peak_read", "moe_peak_copy", "moe_peak_mfma"]

MFMA_FLOPS = 16 * 16 * 32 * 2  # one v_mfma_f32_16x16x32_bf16
MFMA_CHAINS = 8                 # per wavefront, per round
MFMA_WAVES = 4                  # per workgroup

_lib = None
_lock = threading.Lock()


def lib():
    """The loaded libmoe_peaks (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                import torch  # noqa: F401  (binds the library to torch's HIP runtime)
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with `python -m grouped_gemm_gemv_amd.build`")
                l = ctypes.CDLL(LIB_PATH)
                p, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
                f = ctypes.c_float
                for name, args in {"moe_peak_read": [p, sz, p, i, i, p], "moe_peak_copy": [p, p, sz, i, i, p],
                                   "moe_peak_mfma": [f, f, i, p, i, p]}.items():
                    fn = getattr(l, name)
                    fn.argtypes = args
                    fn.restype = ctypes.c_int
                _lib = l
    return _lib


def _check(name: str, status: int) -> None:
    if status != 0:
        raise RuntimeError(f"{name}: status {status} ({'invalid argument' if status == 1 else 'HIP error'})")


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


NONTEMPORAL = 1  # flags bit 0
REGIONS = 2      # flags bit 1


def moe_peak_read(buf, sink, blocks: int, flags: int = 0, stream=None) -> None:
    """Streaming read of the whole of `buf` (a contiguous device tensor);
    sink: int32 device tensor of `blocks` words (per-workgroup XOR)."""
    assert buf.is_contiguous() and sink.numel() >= blocks
    _check("moe_peak_read", lib().moe_peak_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                                sink.data_ptr(), blocks, flags, _stream(stream)))


def moe_peak_copy(src, dst, blocks: int, flags: int = 0, stream=None) -> None:
    """dst <- src (contiguous device tensors of the same byte size)."""
    nb = src.numel() * src.element_size()
    assert src.is_contiguous() and dst.is_contiguous() and dst.numel() * dst.element_size() == nb
    _check("moe_peak_copy", lib().moe_peak_copy(src.data_ptr(), dst.data_ptr(), nb, blocks, flags,
                                                _stream(stream)))


def moe_peak_mfma(a: float, b: float, iters: int, sink, blocks: int, stream=None) -> float:
    """Matrix-core loop; sink: float32 device tensor of 4*blocks values.
    Returns the FLOPs launched."""
    assert sink.numel() >= MFMA_WAVES * blocks
    _check("moe_peak_mfma", lib().moe_peak_mfma(a, b, iters, sink.data_ptr(), blocks, _stream(stream)))
    return float(blocks) * MFMA_WAVES * MFMA_CHAINS * iters * MFMA_FLOPS
