"""Binding of libqsa_calib.so (include/qsa_calibrate.h): the streaming-read and dense bf16
MFMA kernels that the QSA kernels' measured rates are reported against.  Measurement
infrastructure only; the QSA path does not use it.  Argument marshalling only.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_LIB_PATH = os.path.join(_HERE, "libqsa_calib.so")
SIGNATURES = {
    "qsa_calib_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_void_p]),
    "qsa_calib_mfma_bf16": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]),
    "qsa_calib_mfma_sink_floats": (ctypes.c_int, [ctypes.c_int]),
}
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(CALIB_LIB_PATH):
            raise RuntimeError(f"{CALIB_LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_37_amd.build`")
        h = ctypes.CDLL(CALIB_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _lib = h
    return _lib


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def stream_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    """Enqueue one read of every byte of ``buf`` (contiguous, GPU)."""
    st = lib().qsa_calib_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                     ctypes.c_void_p(sink.data_ptr()), blocks, _stream(buf.device))
    if st != 0:
        raise RuntimeError(f"qsa_calib_stream_read failed with status {st}")


def mfma_bf16(iters: int, blocks: int, sink: torch.Tensor) -> float:
    """Enqueue one dense bf16 MFMA loop; returns its flop count."""
    fl = ctypes.c_double(0.0)
    st = lib().qsa_calib_mfma_bf16(iters, blocks, ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.byref(fl), _stream(sink.device))
    if st != 0:
        raise RuntimeError(f"qsa_calib_mfma_bf16 failed with status {st}")
    return fl.value


def sink_floats(blocks: int) -> int:
    return lib().qsa_calib_mfma_sink_floats(blocks)


def _best_of(fn, reps: int) -> float:
    """Shortest of ``reps`` event-timed runs of fn() on the current stream, in ms."""
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b)
        best = t if best is None else min(best, t)
    return best


def measure_read_gbs(dev, mib: int = 4096, reps: int = 5) -> dict:
    """Sustained HBM read rate: one read of a ``mib`` MiB buffer (larger than the 256 MB
    last-level cache), best of ``reps``."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * 8
    buf = torch.ones(mib * 2**20 // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(blocks, dtype=torch.int32, device=dev)
    stream_read(buf, sink, blocks)  # warm-up
    torch.cuda.synchronize()
    ms = _best_of(lambda: stream_read(buf, sink, blocks), reps)
    nbytes = buf.numel() * 4
    del buf
    return {"kernel": "qsa_calib_stream_read", "bytes": nbytes, "ms": round(ms, 4),
            "GB/s": round(nbytes / (ms / 1e3) / 1e9, 1), "workgroups": blocks}


def measure_mfma_tflops(dev, iters: int = 50000, reps: int = 5) -> dict:
    """Sustained dense bf16 matrix rate: v_mfma_f32_32x32x16_bf16 back to back on every SIMD
    (two waves each), best of ``reps``."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus
    sink = torch.empty(sink_floats(blocks), dtype=torch.float32, device=dev)
    mfma_bf16(100, blocks, sink)  # warm-up
    torch.cuda.synchronize()
    flops = [0.0]

    def run():
        flops[0] = mfma_bf16(iters, blocks, sink)

    ms = _best_of(run, reps)
    return {"kernel": "qsa_calib_mfma_bf16", "flops": flops[0], "ms": round(ms, 4),
            "TFLOP/s": round(flops[0] / (ms / 1e3) / 1e12, 1), "workgroups": blocks}
