"""Binding of libmcpeak (include/mc_peak.h): the in-run ceilings the benchmark reports its
rooflines against -- bf16 matrix-core throughput and HBM streaming-read bandwidth -- and the
copy kernel that HBM byte counters are scaled by.  Not part of the Memory Caching path."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmcpeak.so")
_lib = None


def load(path: str = LIB_PATH):
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError("libmcpeak.so not found at %s; build it with "
                          "`python -m chunked_linear_attention_segment_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.mcpeak_mfma_out_floats.restype = I
        lib.mcpeak_mfma_out_floats.argtypes = [I]
        lib.mcpeak_mfma_flops.restype = ctypes.c_double
        lib.mcpeak_mfma_flops.argtypes = [I, I]
        lib.mcpeak_mfma.restype = I
        lib.mcpeak_mfma.argtypes = [I, I, P, P]
        lib.mcpeak_stream_out_words.restype = I
        lib.mcpeak_stream_out_words.argtypes = [I]
        lib.mcpeak_stream_read.restype = I
        lib.mcpeak_stream_read.argtypes = [P, S, I, P, P]
        lib.mcpeak_copy.restype = I
        lib.mcpeak_copy.argtypes = [P, P, S, I, P]
        _lib = lib
    return _lib


def _timed(launch, reps, stream):
    """Mean duration in ms of `reps` launches, with events on the launch stream."""
    import torch
    launch()  # warm-up
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        launch()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]


def mfma_bf16_tflops(n_blocks=4096, iters=2048, reps=5):
    """Measured dense bf16 matrix-core throughput (TFLOP/s), median of `reps` launches."""
    import torch
    lib = load()
    out = torch.empty(lib.mcpeak_mfma_out_floats(n_blocks), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()

    def launch():
        if lib.mcpeak_mfma(n_blocks, iters, out.data_ptr(), s.cuda_stream) != 0:
            raise RuntimeError("mcpeak_mfma failed")
    ms = _timed(launch, reps, s)
    return lib.mcpeak_mfma_flops(n_blocks, iters) / (ms / 1e3) / 1e12


def hbm_read_gbs(gib=4, n_blocks=16384, reps=5):
    """Measured HBM streaming-read bandwidth (GB/s) over a `gib` GiB buffer (each of the
    `n_blocks` workgroups reads one contiguous 1/n_blocks of it)."""
    import torch
    lib = load()
    n = gib << 30
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(lib.mcpeak_stream_out_words(n_blocks), dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()

    def launch():
        if lib.mcpeak_stream_read(buf.data_ptr(), n, n_blocks, out.data_ptr(), s.cuda_stream):
            raise RuntimeError("mcpeak_stream_read failed")
    ms = _timed(launch, reps, s)
    del buf
    return n / (ms / 1e3) / 1e9


def copy(src, dst, n_bytes, n_blocks=8192, stream=None):
    import torch
    s = stream or torch.cuda.current_stream()
    if load().mcpeak_copy(src.data_ptr(), dst.data_ptr(), n_bytes, n_blocks, s.cuda_stream):
        raise RuntimeError("mcpeak_copy failed")
