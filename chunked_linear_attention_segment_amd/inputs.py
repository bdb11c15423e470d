"""Seeded synthetic inputs for the Memory Caching prefill / decode workloads.

This module only draws random numbers and rounds them to the storage dtype; it holds
none of the method's arithmetic.  It serves both the HIP path and the CPU oracle, which
receive exactly the same values (bf16 values are carried here as float32 arrays whose
entries are exactly representable in bf16).

Recipes (shapes follow the workloads of the Memory Caching paper's experiments: context
lengths up to 64K, segment lengths 64..512, head dim 64/128):
  "proj"   x ~ N(0,1) [B,L,d_in] shared by the heads; per head W_q, W_k, W_v, W_u ~
           N(0, 1/d_in); q, k, v, u = x W (the input projections of Eq. 4a / Eq. 10).
  "l2norm" q, k ~ N(0,1) then L2-normalised per token per head; v ~ N(0,1);
           x ~ N(0,1) shared; u = x W_u with W_u ~ N(0, 1/d_in).
Draw order for a seed: x, then W_q, W_k, W_v, W_u (proj) or q, k, v, W_u (l2norm).
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d_k: int
    d_v: int
    d_g: int
    seg_len: int
    phi: str = "identity"       # "identity" | "elu1"
    dtype: str = "bf16"         # "f32" | "bf16"
    x_heads: int = 1            # 1: X shared by heads; H: per-head X
    recipe: str = "proj"        # "proj" | "l2norm"
    top_k: int = 0              # SSC only
    op: str = "grm"             # "grm" | "ssc" | "decode"
    # decode only
    n_cached: int = 0
    count_on: int = 0


WORKLOADS = {
    "grm_f32_L512": Workload("grm_f32_L512", 1, 1, 512, 64, 64, 64, 64, "identity", "f32"),
    "grm_bf16_L4K_elu": Workload("grm_bf16_L4K_elu", 4, 16, 4096, 128, 128, 128, 256, "elu1"),
    "ssc_bf16_L16K_k4": Workload("ssc_bf16_L16K_k4", 2, 16, 16384, 128, 128, 128, 256,
                                 "identity", top_k=4, op="ssc"),
    "grm_bf16_L64K": Workload("grm_bf16_L64K", 1, 32, 65536, 128, 128, 128, 512, "identity",
                              recipe="l2norm"),
    "decode_bf16_64x32_n256": Workload("decode_bf16_64x32_n256", 64, 32, 1, 128, 128, 128, 256,
                                       "identity", op="decode", n_cached=256, count_on=100,
                                       recipe="l2norm"),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite inputs: u + 0x8000 never wraps (the largest finite pattern is 0xFF7FFFFF)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def _l2n(a: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.einsum("...i,...i->...", a, a, dtype=np.float32))[..., None]
    return a / np.maximum(n, np.float32(1e-30))


def make_prefill(w: Workload, seed: int = 0, L: int | None = None, B: int | None = None,
                 H: int | None = None) -> dict:
    """Q, K [B,H,L,dk]; V [B,H,L,dv]; U [B,H,L,dg]; X [B,xh,L,dg] as float32 arrays.

    L, B, H may override the workload's sizes (same recipe, smaller draw)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    rng = np.random.default_rng(seed)
    din = w.d_g
    xh = 1 if w.x_heads == 1 else H
    x = rng.standard_normal((B, xh, L, din), dtype=np.float32)
    sd = np.float32(1.0 / np.sqrt(din))
    if w.recipe == "proj":
        Wq = rng.standard_normal((H, din, w.d_k), dtype=np.float32) * sd
        Wk = rng.standard_normal((H, din, w.d_k), dtype=np.float32) * sd
        Wv = rng.standard_normal((H, din, w.d_v), dtype=np.float32) * sd
        Wu = rng.standard_normal((H, din, w.d_g), dtype=np.float32) * sd
        q = np.empty((B, H, L, w.d_k), dtype=np.float32)
        k = np.empty((B, H, L, w.d_k), dtype=np.float32)
        v = np.empty((B, H, L, w.d_v), dtype=np.float32)
        u = np.empty((B, H, L, w.d_g), dtype=np.float32)
        for h in range(H):
            xb = x[:, 0 if xh == 1 else h]
            q[:, h], k[:, h], v[:, h], u[:, h] = xb @ Wq[h], xb @ Wk[h], xb @ Wv[h], xb @ Wu[h]
    elif w.recipe == "l2norm":
        q = _l2n(rng.standard_normal((B, H, L, w.d_k), dtype=np.float32))
        k = _l2n(rng.standard_normal((B, H, L, w.d_k), dtype=np.float32))
        v = rng.standard_normal((B, H, L, w.d_v), dtype=np.float32)
        Wu = rng.standard_normal((H, din, w.d_g), dtype=np.float32) * sd
        u = np.empty((B, H, L, w.d_g), dtype=np.float32)
        for h in range(H):
            xb = x[:, 0 if xh == 1 else h]
            u[:, h] = xb @ Wu[h]
    else:
        raise ValueError(w.recipe)
    return {"Q": _store(q, w.dtype), "K": _store(k, w.dtype), "V": _store(v, w.dtype),
            "U": _store(u, w.dtype), "X": _store(x, w.dtype)}


def make_decode(w: Workload, seed: int = 0, B: int | None = None, H: int | None = None,
                n_cap: int | None = None, n_cached: int | None = None,
                count_on: int | None = None) -> dict:
    """Host-side decode inputs (small sizes; the full-size cache is drawn on the device).

    Cache (stored in the workload dtype): M^(i) ~ N(0, C/d) (a sum of C products of unit-norm k and
    N(0,1) v); P_i ~ N(0, 1/C); online M_on ~ N(0, c/d) fp32 and x sum ~ N(0, c) for
    c = count_on tokens already in the online segment.  New token: q, k unit-norm,
    v, x ~ N(0,1), u = x W_u with W_u ~ N(0, 1/d)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    n = w.n_cached if n_cached is None else n_cached
    cap = (n + 2) if n_cap is None else n_cap
    cnt = w.count_on if count_on is None else count_on
    C, dk, dv, dg = w.seg_len, w.d_k, w.d_v, w.d_g
    xh = 1 if w.x_heads == 1 else H
    rng = np.random.default_rng(seed)
    Mc = np.zeros((B, H, cap, dv, dk), dtype=np.float32)
    Mc[:, :, :n] = rng.standard_normal((B, H, n, dv, dk), dtype=np.float32) * np.float32(
        np.sqrt(C / dk))
    Mc = _store(Mc, w.dtype)
    Pc = np.zeros((B, xh, cap, dg), dtype=np.float32)
    Pc[:, :, :n] = rng.standard_normal((B, xh, n, dg), dtype=np.float32) * np.float32(
        1.0 / np.sqrt(C))
    M_on = rng.standard_normal((B, H, dv, dk), dtype=np.float32) * np.float32(
        np.sqrt(max(cnt, 0) / dk))
    xsum = rng.standard_normal((B, xh, dg), dtype=np.float32) * np.float32(np.sqrt(max(cnt, 0)))
    if cnt == 0:
        M_on[:] = 0
        xsum[:] = 0
    x = rng.standard_normal((B, xh, dg), dtype=np.float32)
    q = _l2n(rng.standard_normal((B, H, dk), dtype=np.float32))
    k = _l2n(rng.standard_normal((B, H, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, dv), dtype=np.float32)
    Wu = rng.standard_normal((H, dg, dg), dtype=np.float32) * np.float32(1.0 / np.sqrt(dg))
    u = np.empty((B, H, dg), dtype=np.float32)
    for h in range(H):
        u[:, h] = x[:, 0 if xh == 1 else h] @ Wu[h]
    st = w.dtype
    return {"q": _store(q, st), "k": _store(k, st), "v": _store(v, st), "u": _store(u, st),
            "x": _store(x, st), "M_on": M_on, "xsum": xsum, "count": cnt,
            "M_cache": Mc, "P_cache": Pc, "n_cached": n}


def make_prefill_device(w: Workload, seed: int = 0, device="cuda", L: int | None = None,
                        B: int | None = None, H: int | None = None) -> dict:
    """The same recipes drawn on the device with a seeded torch generator (for the
    full-size workloads, whose host draw would take minutes).  Returns torch tensors in the
    storage dtype.  The random stream differs from make_prefill's; each caller uses one
    generator for both the GPU path and the oracle (which receives copies of these)."""
    import torch
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    din = w.d_g
    xh = 1 if w.x_heads == 1 else H
    sd = 1.0 / float(np.sqrt(din))
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def randn(*shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)

    x = randn(B, xh, L, din)
    out = {}
    if w.recipe == "proj":
        Ws = [randn(H, din, n) * sd for n in (w.d_k, w.d_k, w.d_v, w.d_g)]
        for name, Wm in zip(("Q", "K", "V", "U"), Ws):
            t = torch.empty((B, H, L, Wm.shape[-1]), dtype=dt, device=device)
            for h in range(H):
                t[:, h] = (x[:, 0 if xh == 1 else h] @ Wm[h]).to(dt)
            out[name] = t
    elif w.recipe == "l2norm":
        for name, n in (("Q", w.d_k), ("K", w.d_k)):
            t = torch.empty((B, H, L, n), dtype=dt, device=device)
            for h in range(H):
                a = randn(B, L, n)
                t[:, h] = (a / a.norm(dim=-1, keepdim=True).clamp_min(1e-30)).to(dt)
            out[name] = t
        V = torch.empty((B, H, L, w.d_v), dtype=dt, device=device)
        for h in range(H):
            V[:, h] = randn(B, L, w.d_v).to(dt)
        out["V"] = V
        Wu = randn(H, din, w.d_g) * sd
        U = torch.empty((B, H, L, w.d_g), dtype=dt, device=device)
        for h in range(H):
            U[:, h] = (x[:, 0 if xh == 1 else h] @ Wu[h]).to(dt)
        out["U"] = U
    else:
        raise ValueError(w.recipe)
    out["X"] = x.to(dt)
    return out


def make_decode_device(w: Workload, seed: int = 0, device="cuda", n_cap: int | None = None) -> dict:
    """Full-size decode state and token drawn on the device (recipe of make_decode).
    The state cache M [B,H,n_cap,dv,dk] is drawn slice by slice in the storage dtype."""
    import torch
    B, H, C, dk, dv, dg = w.B, w.H, w.seg_len, w.d_k, w.d_v, w.d_g
    n = w.n_cached
    cap = (n + 2) if n_cap is None else n_cap
    cnt = w.count_on
    xh = 1 if w.x_heads == 1 else H
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def randn(*shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)

    Mc = torch.zeros((B, H, cap, dv, dk), dtype=dt, device=device)
    sc = float(np.sqrt(C / dk))
    for b in range(B):
        for h in range(H):
            Mc[b, h, :n] = (randn(n, dv, dk) * sc).to(dt)
    Pc = torch.zeros((B, xh, cap, dg), dtype=torch.float32, device=device)
    Pc[:, :, :n] = randn(B, xh, n, dg) * float(1.0 / np.sqrt(C))
    M_on = randn(B, H, dv, dk) * float(np.sqrt(max(cnt, 0) / dk))
    xsum = randn(B, xh, dg) * float(np.sqrt(max(cnt, 0)))
    if cnt == 0:
        M_on.zero_()
        xsum.zero_()
    x = randn(B, xh, dg)
    q = randn(B, H, dk)
    q = q / q.norm(dim=-1, keepdim=True)
    k = randn(B, H, dk)
    k = k / k.norm(dim=-1, keepdim=True)
    v = randn(B, H, dv)
    Wu = randn(H, dg, dg) * float(1.0 / np.sqrt(dg))
    u = torch.empty((B, H, dg), dtype=torch.float32, device=device)
    for h in range(H):
        u[:, h] = x[:, 0 if xh == 1 else h] @ Wu[h]
    return {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "u": u.to(dt), "x": x.to(dt),
            "M_on": M_on.contiguous(), "xsum": xsum.contiguous(), "count": cnt,
            "M_cache": Mc, "P_cache": Pc, "n_cached": n, "n_cap": cap}


# SWLA gates (the Memory Caching paper's sliding-window linear attention, window 2): the
# decay alpha_t and the window weights beta_t (previous token) and lam_t (current token), one
# value per token per head.  The pages do not say how a model forms them; uniform draws with
# a decay close to 1 (a long horizon) and window weights of either sign around 1 stand in.
SWLA_RANGES = {"alpha": (0.9, 1.0), "beta": (-0.5, 1.0), "lam": (0.25, 1.25)}


def make_swla_gates(B: int, H: int, L: int, seed: int = 0, ranges=None) -> dict:
    """alpha, beta, lam [B,H,L] float32 (host draw, numpy PCG64)."""
    rg = dict(SWLA_RANGES, **(ranges or {}))
    rng = np.random.default_rng(seed)
    return {k: rng.uniform(rg[k][0], rg[k][1], (B, H, L)).astype(np.float32)
            for k in ("alpha", "beta", "lam")}


def make_swla_gates_device(B: int, H: int, L: int, seed: int = 0, device="cuda",
                           ranges=None) -> dict:
    """The same gates drawn on the device with a seeded torch generator (full sizes)."""
    import torch
    rg = dict(SWLA_RANGES, **(ranges or {}))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = {}
    for k in ("alpha", "beta", "lam"):
        lo, hi = rg[k]
        out[k] = torch.rand((B, H, L), generator=g, device=device, dtype=torch.float32) * \
            (hi - lo) + lo
    return out


def make_upstream_grad(B: int, H: int, L: int, d_v: int, seed: int = 0,
                       dtype: str = "f32") -> np.ndarray:
    """dY [B,H,L,d_v] ~ N(0,1), the gradient of a loss with respect to the read's output,
    stored in the input dtype (float32 array of bf16-representable values for bf16)."""
    rng = np.random.default_rng(seed)
    return _store(rng.standard_normal((B, H, L, d_v), dtype=np.float32), dtype)
