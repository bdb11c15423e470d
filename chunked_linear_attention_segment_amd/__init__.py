"""Memory Caching (MC) over a linear-attention memory on MI355X: Python binding of libmc.

The binding only marshals arguments: every step of the path runs in the HIP kernels of
``libmc.so`` (built by ``python -m chunked_linear_attention_segment_amd.build``).  There is
no fallback: if the library is missing, loading raises.

Entry points (same names and arguments as include/mc.h; tensors are torch tensors on the
GPU, host scalars are Python ints or one-element int32 numpy arrays):
    mc_abi_version, mc_status_str, mc_workspace_bytes,
    mc_scan_prefill, mc_grm_readout, mc_ssc_readout, mc_decode_step,
    mc_scan_prefill_segs, mc_grm_readout_segs, mc_grm_prefill_segs, mc_ssc_readout_segs,
    mc_scan_prefill_swla,
    mc_grm_backward, mc_decode_step_noalloc
plus helpers that allocate outputs / workspaces with torch (memory plumbing only).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MC_LIB names another build of the same library (e.g. one with host-side sanitizers)
LIB_PATH = os.environ.get("MC_LIB") or os.path.join(_HERE, "libmc.so")

MC_OK, MC_ERR_NULL, MC_ERR_DIMS, MC_ERR_UNSUPPORTED = 0, 1, 2, 3
MC_ERR_ALIGN, MC_ERR_WORKSPACE, MC_ERR_HIP, MC_ERR_CAPACITY, MC_ERR_SCRATCH = 4, 5, 6, 7, 8
MC_NOALLOC_SCRATCH_BYTES = 64 << 20
MC_F32, MC_BF16 = 0, 1
MC_PHI_IDENTITY, MC_PHI_ELU1 = 0, 1
MC_OP_PREFILL, MC_OP_GRM, MC_OP_SSC, MC_OP_DECODE, MC_OP_GRM_BACKWARD, MC_OP_SCAN_SEGS, \
    MC_OP_GRM_SEGS, MC_OP_SSC_SEGS, MC_OP_GRM_PREFILL_SEGS = 0, 1, 2, 3, 4, 5, 6, 7, 8

EXPORTED = ["mc_abi_version", "mc_status_str", "mc_workspace_bytes", "mc_scan_prefill",
            "mc_grm_readout", "mc_ssc_readout", "mc_decode_step", "mc_scan_prefill_segs",
            "mc_grm_readout_segs", "mc_grm_prefill_segs", "mc_ssc_readout_segs",
            "mc_scan_prefill_swla",
            "mc_grm_backward", "mc_decode_step_noalloc"]
MC_MAX_SEGS = 512


class McDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "H", "L", "d_k", "d_v", "d_g", "seg_len", "x_heads", "dtype", "phi")]


class McError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, mc_status_str(status), status))


_lib = None


def load(path: str = LIB_PATH):
    """Load libmc.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError("libmc.so not found at %s; build it with "
                          "`python -m chunked_linear_attention_segment_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, D = ctypes.c_void_p, ctypes.POINTER(McDims)
        lib.mc_abi_version.restype = ctypes.c_int
        lib.mc_status_str.restype = ctypes.c_char_p
        lib.mc_status_str.argtypes = [ctypes.c_int]
        lib.mc_workspace_bytes.restype = ctypes.c_size_t
        lib.mc_workspace_bytes.argtypes = [D, ctypes.c_int, ctypes.c_int32, ctypes.c_int32]
        lib.mc_scan_prefill.restype = ctypes.c_int
        lib.mc_scan_prefill.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.mc_grm_readout.restype = ctypes.c_int
        lib.mc_grm_readout.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P,
                                       ctypes.c_size_t, P]
        lib.mc_ssc_readout.restype = ctypes.c_int
        lib.mc_ssc_readout.argtypes = [D, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P, P,
                                       P, ctypes.c_size_t, P]
        lib.mc_scan_prefill_segs.restype = ctypes.c_int
        lib.mc_scan_prefill_segs.argtypes = [D, P, ctypes.c_int32, P, P, P, P, P, P, P, P, P,
                                             ctypes.c_size_t, P]
        lib.mc_grm_readout_segs.restype = ctypes.c_int
        lib.mc_grm_readout_segs.argtypes = [D, P, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P,
                                            ctypes.c_size_t, P]
        lib.mc_grm_prefill_segs.restype = ctypes.c_int
        lib.mc_grm_prefill_segs.argtypes = [D, P, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P,
                                            P, ctypes.c_size_t, P]
        lib.mc_ssc_readout_segs.restype = ctypes.c_int
        lib.mc_ssc_readout_segs.argtypes = [D, P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P,
                                            P, P, P, P, P, ctypes.c_size_t, P]
        lib.mc_scan_prefill_swla.restype = ctypes.c_int
        lib.mc_scan_prefill_swla.argtypes = [D, P, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P,
                                             P, P]
        lib.mc_grm_backward.restype = ctypes.c_int
        lib.mc_grm_backward.argtypes = [D] + [P] * 15 + [ctypes.c_size_t, P]
        lib.mc_decode_step.restype = ctypes.c_int
        lib.mc_decode_step.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P, P,
                                       ctypes.c_size_t, P]
        lib.mc_decode_step_noalloc.restype = ctypes.c_int
        lib.mc_decode_step_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int32,
                                               P, P]
        _lib = lib
    return _lib


def make_dims(B, H, L, d_k, d_v, d_g, seg_len, x_heads=1, dtype="bf16", phi="identity"):
    dt = {"f32": MC_F32, "bf16": MC_BF16}.get(dtype, dtype)
    ph = {"identity": MC_PHI_IDENTITY, "elu1": MC_PHI_ELU1}.get(phi, phi)
    return McDims(B, H, L, d_k, d_v, d_g, seg_len, x_heads, dt, ph)


def _p(t):
    """Device (or host) address of a tensor / numpy array / raw int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    return _p(ws), ws.numel() * ws.element_size()


def _check(rc, where):
    if rc != MC_OK:
        raise McError(rc, where)


def mc_abi_version() -> int:
    return load().mc_abi_version()


def mc_status_str(status: int) -> str:
    return load().mc_status_str(int(status)).decode()


def mc_workspace_bytes(dims: McDims, op: int, top_k: int = 0, n_cap: int = 0) -> int:
    return int(load().mc_workspace_bytes(ctypes.byref(dims), int(op), int(top_k), int(n_cap)))


def mc_scan_prefill(dims, Q, K, V, X, M, M_lo, P, O_on, ws=None, stream=None):
    w, wb = _ws(ws)
    _check(load().mc_scan_prefill(ctypes.byref(dims), _p(Q), _p(K), _p(V), _p(X), _p(M),
                                  _p(M_lo), _p(P), _p(O_on), w, wb, _stream(stream)),
           "mc_scan_prefill")


def mc_grm_readout(dims, Q, K, V, U, X, M, M_lo, P, O_on, Y, gamma=None, ws=None,
                   stream=None):
    w, wb = _ws(ws)
    _check(load().mc_grm_readout(ctypes.byref(dims), _p(Q), _p(K), _p(V), _p(U), _p(X), _p(M),
                                 _p(M_lo), _p(P), _p(O_on), _p(Y), _p(gamma), w, wb,
                                 _stream(stream)),
           "mc_grm_readout")


def mc_ssc_readout(dims, top_k, Q, K, V, U, X, M, M_lo, P, O_on, Y, idx, ws=None, stream=None):
    w, wb = _ws(ws)
    _check(load().mc_ssc_readout(ctypes.byref(dims), int(top_k), _p(Q), _p(K), _p(V), _p(U),
                                 _p(X), _p(M), _p(M_lo), _p(P), _p(O_on), _p(Y), _p(idx), w,
                                 wb, _stream(stream)),
           "mc_ssc_readout")


def _offsets(seg_off):
    off = np.ascontiguousarray(np.asarray(seg_off, dtype=np.int32))
    return off, off.shape[0] - 1


def mc_scan_prefill_segs(dims, seg_off, Q, K, V, X, M, M_lo, P, O_on, ws=None, stream=None):
    """seg_off: host offsets 0 = o_0 < ... < o_n = L (segment i = [o_i, o_{i+1})); ws:
    mc_workspace_bytes(dims, MC_OP_SCAN_SEGS, n) bytes (see workspace_segs)."""
    off, n = _offsets(seg_off)
    w, wb = _ws(ws)
    _check(load().mc_scan_prefill_segs(ctypes.byref(dims), off.ctypes.data, n, _p(Q), _p(K),
                                       _p(V), _p(X), _p(M), _p(M_lo), _p(P), _p(O_on), w, wb,
                                       _stream(stream)),
           "mc_scan_prefill_segs")


def workspace_segs(dims, n_seg, device="cuda"):
    """Workspace of mc_scan_prefill_segs for n_seg segments (None when none is needed)."""
    import torch
    nb = mc_workspace_bytes(dims, MC_OP_SCAN_SEGS, n_seg)
    return torch.empty(nb, dtype=torch.uint8, device=device) if nb else None


def mc_grm_readout_segs(dims, seg_off, Q, U, X, M, M_lo, P, O_on, Y, gamma=None, ws=None,
                        stream=None):
    off, n = _offsets(seg_off)
    w, wb = _ws(ws)
    _check(load().mc_grm_readout_segs(ctypes.byref(dims), off.ctypes.data, n, _p(Q), _p(U),
                                      _p(X), _p(M), _p(M_lo), _p(P), _p(O_on), _p(Y),
                                      _p(gamma), w, wb, _stream(stream)),
           "mc_grm_readout_segs")


def mc_grm_prefill_segs(dims, seg_off, Q, K, V, U, X, M, M_lo, P, Y, gamma=None, ws=None,
                        stream=None):
    """The whole GRM prefill over the segments [seg_off[i], seg_off[i+1]) in one call; ws:
    mc_workspace_bytes(dims, MC_OP_GRM_PREFILL_SEGS, n) bytes."""
    off, n = _offsets(seg_off)
    w, wb = _ws(ws)
    _check(load().mc_grm_prefill_segs(ctypes.byref(dims), off.ctypes.data, n, _p(Q), _p(K),
                                      _p(V), _p(U), _p(X), _p(M), _p(M_lo), _p(P), _p(Y),
                                      _p(gamma), w, wb, _stream(stream)),
           "mc_grm_prefill_segs")


def mc_ssc_readout_segs(dims, seg_off, top_k, Q, U, X, M, M_lo, P, O_on, Y, idx, ws=None,
                        stream=None):
    """SSC read over the segments [seg_off[i], seg_off[i+1]); O_on from mc_scan_prefill_segs;
    ws: mc_workspace_bytes(dims, MC_OP_SSC_SEGS, top_k, n) bytes."""
    off, n = _offsets(seg_off)
    w, wb = _ws(ws)
    _check(load().mc_ssc_readout_segs(ctypes.byref(dims), off.ctypes.data, n, int(top_k),
                                      _p(Q), _p(U), _p(X), _p(M), _p(M_lo), _p(P), _p(O_on),
                                      _p(Y), _p(idx), w, wb, _stream(stream)),
           "mc_ssc_readout_segs")


def mc_scan_prefill_swla(dims, seg_off, alpha, beta, lam, Q, K, V, X, M, M_lo, P, O_on,
                         stream=None):
    """SWLA write path (window 2).  seg_off None = segments of dims.seg_len; alpha, beta, lam
    are [B,H,L] fp32 device tensors."""
    if seg_off is None:
        off, n = None, 0
    else:
        off, n = _offsets(seg_off)
    _check(load().mc_scan_prefill_swla(ctypes.byref(dims), None if off is None else off.ctypes.data,
                                       n, _p(alpha), _p(beta), _p(lam), _p(Q), _p(K), _p(V),
                                       _p(X), _p(M), _p(M_lo), _p(P), _p(O_on), _stream(stream)),
           "mc_scan_prefill_swla")


def mc_grm_backward(dims, Q, K, V, U, X, M, M_lo, P, dY, dQ, dK, dV, dU, dX, ws=None,
                    stream=None):
    w, wb = _ws(ws)
    _check(load().mc_grm_backward(ctypes.byref(dims), _p(Q), _p(K), _p(V), _p(U), _p(X), _p(M),
                                  _p(M_lo), _p(P), _p(dY), _p(dQ), _p(dK), _p(dV), _p(dU),
                                  _p(dX), w, wb, _stream(stream)),
           "mc_grm_backward")


def grm_backward(dims, Q, K, V, U, X, M, M_lo, P, dY, stream=None):
    """Gradients of the GRM prefill with fresh fp32 outputs: dict dQ, dK, dV, dU, dX."""
    import torch
    dev = Q.device
    f = dict(dtype=torch.float32, device=dev)
    B, H, L = dims.B, dims.H, dims.L
    out = {"dQ": torch.empty((B, H, L, dims.d_k), **f), "dK": torch.empty((B, H, L, dims.d_k), **f),
           "dV": torch.empty((B, H, L, dims.d_v), **f), "dU": torch.empty((B, H, L, dims.d_g), **f),
           "dX": torch.empty((B, dims.x_heads, L, dims.d_g), **f)}
    ws = workspace(dims, MC_OP_GRM_BACKWARD, device=dev)
    mc_grm_backward(dims, Q, K, V, U, X, M, M_lo, P, dY, out["dQ"], out["dK"], out["dV"],
                    out["dU"], out["dX"], ws=ws, stream=stream)
    return out


def mc_decode_step(dims, q, k, v, u, x, M_on, xsum_on, count_on, M_cache, P_cache, n_cached,
                   n_cap, y, ws=None, stream=None):
    """count_on and n_cached are one-element int32 numpy arrays, updated in place.  u=None
    reads the plain mean of the memories (memory caching applied after pre-training)."""
    assert isinstance(count_on, np.ndarray) and count_on.dtype == np.int32
    assert isinstance(n_cached, np.ndarray) and n_cached.dtype == np.int32
    w, wb = _ws(ws)
    _check(load().mc_decode_step(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(u), _p(x),
                                 _p(M_on), _p(xsum_on), count_on.ctypes.data, _p(M_cache),
                                 _p(P_cache), n_cached.ctypes.data, int(n_cap), _p(y), w, wb,
                                 _stream(stream)),
           "mc_decode_step")


def mc_decode_step_noalloc(dims, q, k, v, u, x, M_on, xsum_on, count_on, M_cache, P_cache,
                           n_cached, n_cap, y, stream=None):
    """mc_decode_step with the library's fixed per-GPU scratch instead of a workspace."""
    assert isinstance(count_on, np.ndarray) and count_on.dtype == np.int32
    assert isinstance(n_cached, np.ndarray) and n_cached.dtype == np.int32
    _check(load().mc_decode_step_noalloc(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(u), _p(x),
                                         _p(M_on), _p(xsum_on), count_on.ctypes.data,
                                         _p(M_cache), _p(P_cache), n_cached.ctypes.data,
                                         int(n_cap), _p(y), _stream(stream)),
           "mc_decode_step_noalloc")


# ---- allocation helpers (torch is only memory plumbing here) ----------------------------

def torch_dtype(dims):
    import torch
    return torch.bfloat16 if dims.dtype == MC_BF16 else torch.float32


def workspace(dims, op, top_k=0, n_cap=0, device="cuda"):
    import torch
    n = mc_workspace_bytes(dims, op, top_k, n_cap)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def alloc_prefill(dims, device="cuda", online=True):
    """Output buffers of mc_scan_prefill: M, M_lo, P, O_on (None unless `online`)."""
    import torch
    NS = (dims.L + dims.seg_len - 1) // dims.seg_len
    M = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.float32, device=device)
    M_lo = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.bfloat16,
                       device=device)
    P = torch.empty((dims.B, dims.x_heads, NS, dims.d_g), dtype=torch.float32, device=device)
    O_on = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch.float32,
                       device=device) if online else None
    return M, M_lo, P, O_on


def prefill_grm(dims, Q, K, V, U, X, want_gamma=False, online=True, stream=None):
    """scan + GRM read with freshly allocated outputs; returns a dict of tensors.
    online=False skips the O_on round trip (the read forms the online term itself)."""
    import torch
    M, M_lo, P, O_on = alloc_prefill(dims, Q.device, online)
    mc_scan_prefill(dims, Q, K, V, X, M, M_lo, P, O_on, stream=stream)
    Y = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch_dtype(dims), device=Q.device)
    NS = M.shape[2]
    G = torch.empty((dims.B, dims.H, dims.L, NS), dtype=torch.float32,
                    device=Q.device) if want_gamma else None
    ws = workspace(dims, MC_OP_GRM, device=Q.device)
    mc_grm_readout(dims, Q, K, V, U, X, M, M_lo, P, O_on, Y, G, ws=ws, stream=stream)
    out = {"Y": Y, "M": M, "M_lo": M_lo, "P": P, "O_on": O_on}
    if want_gamma:
        out["gamma"] = G
    return out


def prefill_grm_segs(dims, seg_off, Q, K, V, U, X, want_gamma=False, stream=None):
    """scan + GRM read over the segments [seg_off[i], seg_off[i+1]) with fresh outputs."""
    import torch
    NS = len(seg_off) - 1
    dev = Q.device
    M = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.float32, device=dev)
    M_lo = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.bfloat16,
                       device=dev)
    P = torch.empty((dims.B, dims.x_heads, NS, dims.d_g), dtype=torch.float32, device=dev)
    O_on = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch.float32, device=dev)
    mc_scan_prefill_segs(dims, seg_off, Q, K, V, X, M, M_lo, P, O_on,
                         ws=workspace_segs(dims, NS, device=dev), stream=stream)
    Y = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch_dtype(dims), device=dev)
    G = torch.empty((dims.B, dims.H, dims.L, NS), dtype=torch.float32,
                    device=dev) if want_gamma else None
    ws = workspace(dims, MC_OP_GRM_SEGS, top_k=NS, device=dev)
    mc_grm_readout_segs(dims, seg_off, Q, U, X, M, M_lo, P, O_on, Y, G, ws=ws, stream=stream)
    out = {"Y": Y, "M": M, "M_lo": M_lo, "P": P, "O_on": O_on}
    if want_gamma:
        out["gamma"] = G
    return out


def prefill_grm_segs_onecall(dims, seg_off, Q, K, V, U, X, want_gamma=False, stream=None):
    """mc_grm_prefill_segs with fresh outputs (no O_on is handed over)."""
    import torch
    NS = len(seg_off) - 1
    dev = Q.device
    M = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.float32, device=dev)
    M_lo = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.bfloat16,
                       device=dev)
    P = torch.empty((dims.B, dims.x_heads, NS, dims.d_g), dtype=torch.float32, device=dev)
    Y = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch_dtype(dims), device=dev)
    G = torch.empty((dims.B, dims.H, dims.L, NS), dtype=torch.float32,
                    device=dev) if want_gamma else None
    ws = workspace(dims, MC_OP_GRM_PREFILL_SEGS, top_k=NS, device=dev)
    mc_grm_prefill_segs(dims, seg_off, Q, K, V, U, X, M, M_lo, P, Y, G, ws=ws, stream=stream)
    out = {"Y": Y, "M": M, "M_lo": M_lo, "P": P}
    if want_gamma:
        out["gamma"] = G
    return out


def prefill_grm_swla(dims, alpha, beta, lam, Q, K, V, U, X, seg_off=None, want_gamma=False,
                     stream=None):
    """SWLA scan + GRM read (constant segments, or the given offsets) with fresh outputs."""
    import torch
    dev = Q.device
    NS = (len(seg_off) - 1) if seg_off is not None else (dims.L + dims.seg_len - 1) // dims.seg_len
    M = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.float32, device=dev)
    M_lo = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.bfloat16,
                       device=dev)
    P = torch.empty((dims.B, dims.x_heads, NS, dims.d_g), dtype=torch.float32, device=dev)
    O_on = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch.float32, device=dev)
    mc_scan_prefill_swla(dims, seg_off, alpha, beta, lam, Q, K, V, X, M, M_lo, P, O_on,
                         stream=stream)
    Y = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch_dtype(dims), device=dev)
    G = torch.empty((dims.B, dims.H, dims.L, NS), dtype=torch.float32,
                    device=dev) if want_gamma else None
    ws = workspace(dims, MC_OP_GRM if seg_off is None else MC_OP_GRM_SEGS, top_k=NS,
                   device=dev)
    if seg_off is None:
        mc_grm_readout(dims, Q, None, None, U, X, M, M_lo, P, O_on, Y, G, ws=ws, stream=stream)
    else:
        mc_grm_readout_segs(dims, seg_off, Q, U, X, M, M_lo, P, O_on, Y, G, ws=ws,
                            stream=stream)
    out = {"Y": Y, "M": M, "M_lo": M_lo, "P": P, "O_on": O_on}
    if want_gamma:
        out["gamma"] = G
    return out


def prefill_ssc_segs(dims, seg_off, top_k, Q, K, V, U, X, stream=None):
    """scan + SSC read over the segments [seg_off[i], seg_off[i+1]) with fresh outputs."""
    import torch
    NS = len(seg_off) - 1
    dev = Q.device
    M = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.float32, device=dev)
    M_lo = torch.empty((dims.B, dims.H, NS, dims.d_v, dims.d_k), dtype=torch.bfloat16,
                       device=dev)
    P = torch.empty((dims.B, dims.x_heads, NS, dims.d_g), dtype=torch.float32, device=dev)
    O_on = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch.float32, device=dev)
    mc_scan_prefill_segs(dims, seg_off, Q, K, V, X, M, M_lo, P, O_on,
                         ws=workspace_segs(dims, NS, device=dev), stream=stream)
    Y = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch_dtype(dims), device=dev)
    idx = torch.empty((dims.B, dims.H, dims.L, top_k), dtype=torch.int32, device=dev)
    ws = workspace(dims, MC_OP_SSC_SEGS, top_k=top_k, n_cap=NS, device=dev)
    mc_ssc_readout_segs(dims, seg_off, top_k, Q, U, X, M, M_lo, P, O_on, Y, idx, ws=ws,
                        stream=stream)
    return {"Y": Y, "idx": idx, "M": M, "M_lo": M_lo, "P": P, "O_on": O_on}


def prefill_ssc(dims, top_k, Q, K, V, U, X, online=True, stream=None):
    import torch
    M, M_lo, P, O_on = alloc_prefill(dims, Q.device, online)
    mc_scan_prefill(dims, Q, K, V, X, M, M_lo, P, O_on, stream=stream)
    Y = torch.empty((dims.B, dims.H, dims.L, dims.d_v), dtype=torch_dtype(dims), device=Q.device)
    idx = torch.empty((dims.B, dims.H, dims.L, top_k), dtype=torch.int32, device=Q.device)
    ws = workspace(dims, MC_OP_SSC, top_k=top_k, device=Q.device)
    mc_ssc_readout(dims, top_k, Q, K, V, U, X, M, M_lo, P, O_on, Y, idx, ws=ws, stream=stream)
    return {"Y": Y, "idx": idx, "M": M, "M_lo": M_lo, "P": P, "O_on": O_on}
