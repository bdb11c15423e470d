"""fp64 CPU oracle for Memory Caching over a linear-attention memory.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the benchmark's
CPU-baseline leg, never by the product package.  It shares no code with the HIP path.

The arithmetic lives in ``mc_oracle.c`` (plain C, fp64, OpenMP over (b, h)); this module
only builds it with gcc and marshals numpy arrays.  The functions follow, per token, the
recurrence and read of the Memory Caching paper (§3 Eq. 4b, §3.1 Eq. 7-10) and the Sparse
Selective Caching / Memory Soup formulas of the gitcode explainer (§3.3, §3.4), and the
sliding-window linear-attention memory of the paper's SWLA paragraph (Eq. 28-29); the C file
cites each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mc_oracle.c")
_LIB = os.path.join(_HERE, "libmc_oracle.so")

GRM, SSC, RESIDUAL, SOUP, AVERAGE = 0, 1, 2, 3, 4
_MODES = {"grm": GRM, "ssc": SSC, "residual": RESIDUAL, "soup": SOUP, "average": AVERAGE}


def build(force: bool = False) -> str:
    """Compile mc_oracle.c into libmc_oracle.so with gcc (IEEE fp64, no contraction).
    MC_ORACLE_LIB names a library built elsewhere from the same source (e.g. with sanitizers),
    which is then used as it is."""
    if os.environ.get("MC_ORACLE_LIB"):
        return os.environ["MC_ORACLE_LIB"]
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared",
               "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        lib.mco_prefill.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P, P, P, P,
                                    ctypes.c_int64, P, P, P, P, P, P, ctypes.c_int, P,
                                    ctypes.c_int32, P, P, P]
        lib.mco_prefill.restype = ctypes.c_int
        lib.mco_decode_step.argtypes = [P, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P,
                                        ctypes.c_int32, P, P]
        lib.mco_decode_step.restype = ctypes.c_int
        lib.mco_grm_backward.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int, P,
                                         ctypes.c_int64]
        lib.mco_grm_backward.restype = ctypes.c_int
        lib.mco_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().mco_max_threads())


def prefill(Q, K, V, U, X, seg_len: int, phi: str = "identity", mode: str = "grm",
            top_k: int = 0, rows=None, want_states: bool = False, want_online: bool = False,
            want_gamma: bool = False, n_threads: int = 0, seg_offsets=None,
            swla=None) -> dict:
    """Evaluate the MC read for every token (or only ``rows``) of every (b, h).

    Q, K [B,H,L,dk]; V [B,H,L,dv]; U [B,H,L,dg]; X [B,xh,L,dg] (xh = 1 or H).
    Segments have length seg_len, or are [seg_offsets[i], seg_offsets[i+1]) when
    seg_offsets (0 = o_0 < o_1 < ... < o_N = L) is given (seg_len is then ignored).
    swla = (alpha, beta, lam), each [B,H,L]: the SWLA memory of window 2 (Memory Caching
    paper, Eq. 28) in place of the linear-attention update.
    Returns a dict with 'Y' [B,H,n_rows,dv] and, on request, 'M' [B,H,NS,dv,dk],
    'P' [B,xh,NS,dg], 'O_on' [B,H,L,dv], 'gamma' [B,H,n_rows,NS], 'idx' [B,H,n_rows,top_k].
    """
    Q, K, V, U, X = (_f64(a) for a in (Q, K, V, U, X))
    B, H, L, dk = Q.shape
    dv = V.shape[-1]
    dg = U.shape[-1]
    xh = X.shape[1]
    assert K.shape == Q.shape and V.shape[:3] == (B, H, L) and U.shape[:3] == (B, H, L)
    assert X.shape == (B, xh, L, dg)
    off = None
    if seg_offsets is not None:
        off = np.ascontiguousarray(np.asarray(seg_offsets, dtype=np.int32))
        C = 0
        NS = off.shape[0] - 1
    else:
        C = int(seg_len)
        NS = (L + C - 1) // C
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        nr = rows.shape[0]
    else:
        nr = L
    m = _MODES[mode]
    gates = [None, None, None]
    if swla is not None:
        gates = [_f64(g) for g in swla]
        assert all(g.shape == (B, H, L) for g in gates)
    dims = np.array([B, H, L, dk, dv, dg, C, xh, 1 if phi in ("elu1", "elu+1") else 0],
                    dtype=np.int32)
    out = {"Y": np.zeros((B, H, nr, dv))}
    M = np.zeros((B, H, NS, dv, dk)) if want_states else None
    P = np.zeros((B, xh, NS, dg)) if want_states else None
    O = np.zeros((B, H, L, dv)) if want_online else None
    G = np.zeros((B, H, nr, NS)) if want_gamma else None
    I = np.full((B, H, nr, max(top_k, 1)), -1, dtype=np.int32) if m == SSC else None
    rc = _load().mco_prefill(_ptr(dims), m, int(top_k), _ptr(Q), _ptr(K), _ptr(V), _ptr(U),
                             _ptr(X), _ptr(rows), int(nr), _ptr(out["Y"]), _ptr(M), _ptr(P),
                             _ptr(O), _ptr(G), _ptr(I), int(n_threads), _ptr(off),
                             int(NS if off is not None else 0), *(_ptr(g) for g in gates))
    if rc != 0:
        raise ValueError("mco_prefill failed with code %d" % rc)
    if want_states:
        out["M"], out["P"] = M, P
    if want_online:
        out["O_on"] = O
    if want_gamma:
        out["gamma"] = G
    if I is not None:
        out["idx"] = I
    return out


class DecodeState:
    """Host-side fp64 decode state: online memory, x sum, counters and the cache."""

    def __init__(self, M_on, xsum, count, M_cache, P_cache, n_cached):
        self.M_on = _f64(M_on).copy()
        self.xsum = _f64(xsum).copy()
        self.count = np.array([count], dtype=np.int32)
        self.M_cache = _f64(M_cache).copy()
        self.P_cache = _f64(P_cache).copy()
        self.n_cached = np.array([n_cached], dtype=np.int32)

    @property
    def n_cap(self) -> int:
        return self.M_cache.shape[2]


def decode_step(state: DecodeState, q, k, v, u, x, seg_len: int, phi: str = "identity",
                mode: str = "grm", want_gamma: bool = False):
    """One decode step; updates ``state`` in place and returns y [B,H,dv] (and gamma)."""
    q, k, v, u, x = (_f64(a) for a in (q, k, v, u, x))
    B, H, dk = q.shape
    dv = v.shape[-1]
    dg = u.shape[-1]
    xh = x.shape[1]
    dims = np.array([B, H, dk, dv, dg, int(seg_len), xh,
                     1 if phi in ("elu1", "elu+1") else 0], dtype=np.int32)
    y = np.zeros((B, H, dv))
    G = np.zeros((B, H, state.n_cap + 1)) if want_gamma else None
    rc = _load().mco_decode_step(_ptr(dims), _MODES[mode], _ptr(q), _ptr(k), _ptr(v), _ptr(u),
                                 _ptr(x), _ptr(state.M_on), _ptr(state.xsum),
                                 _ptr(state.count), _ptr(state.M_cache), _ptr(state.P_cache),
                                 _ptr(state.n_cached), int(state.n_cap), _ptr(y), _ptr(G))
    if rc != 0:
        raise ValueError("mco_decode_step failed with code %d" % rc)
    return (y, G) if want_gamma else y


def grm_backward(Q, K, V, U, X, dY, seg_len: int, phi: str = "identity",
                 n_threads: int = 0, rows=None) -> dict:
    """Gradients of the GRM prefill (constant segments of seg_len) for the upstream gradient
    dY [B,H,L,dv]: 'dQ', 'dK' [B,H,L,dk], 'dV' [B,H,L,dv], 'dU' [B,H,L,dg], 'dX' [B,xh,L,dg]
    (heads summed when X is shared).  With rows, only 'dQ' and 'dU' at those rows."""
    Q, K, V, U, X, dY = (_f64(a) for a in (Q, K, V, U, X, dY))
    B, H, L, dk = Q.shape
    dv, dg, xh = V.shape[-1], U.shape[-1], X.shape[1]
    assert dY.shape == V.shape
    dims = np.array([B, H, L, dk, dv, dg, int(seg_len), xh,
                     1 if phi in ("elu1", "elu+1") else 0], dtype=np.int32)
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        nr = rows.shape[0]
        out = {"dQ": np.zeros((B, H, nr, dk)), "dU": np.zeros((B, H, nr, dg))}
        ext = [None, None, None]
    else:
        nr = L
        out = {"dQ": np.zeros(Q.shape), "dK": np.zeros(K.shape), "dV": np.zeros(V.shape),
               "dU": np.zeros(U.shape), "dX": np.zeros(X.shape)}
        ext = [out["dK"], out["dV"], out["dX"]]
    rc = _load().mco_grm_backward(_ptr(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(U), _ptr(X),
                                  _ptr(dY), _ptr(out["dQ"]), _ptr(ext[0]), _ptr(ext[1]),
                                  _ptr(out["dU"]), _ptr(ext[2]), int(n_threads), _ptr(rows),
                                  int(nr))
    if rc != 0:
        raise ValueError("mco_grm_backward failed with code %d" % rc)
    return out


def log_segments(L: int) -> list:
    """Offsets of the logarithmic segmentation of a length-L sequence (gitcode explainer §4.2:
    L in binary, one segment per non-zero bit, of that power-of-two length, largest first;
    37 -> 32, 4, 1).  Returns [0, o_1, ..., L]."""
    assert L >= 1
    off = [0]
    for b in range(int(L).bit_length() - 1, -1, -1):
        if (L >> b) & 1:
            off.append(off[-1] + (1 << b))
    return off
