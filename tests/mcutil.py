"""Shared helpers for the GPU parity tests (device transfer and the error metric)."""
import numpy as np

# max relative error bars: fp32 inputs, and bf16 inputs with fp32 accumulation
TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(a, dtype="f32"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_np(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy() if t.dtype != torch.int32 else \
        t.detach().cpu().numpy()


def slice_rel_err(got, ref, lead=2):
    """max over leading (b, h) slices of max|got - ref| / max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.reshape(int(np.prod(got.shape[:lead])), -1)
    r = ref.reshape(g.shape)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


def announce(msg):
    print(msg, flush=True)
