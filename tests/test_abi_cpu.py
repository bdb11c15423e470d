"""C-ABI contract checks that need no GPU.

libmc validates every argument before its first HIP call, so each error path can be
exercised here with fake (never dereferenced) device addresses.  No call in this file
passes validation, so no kernel is ever launched.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import chunked_linear_attention_segment_amd as mc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "mc.h")

A = 0x7f0000000000  # an aligned fake device address (never dereferenced)
MIS = A + 4         # a misaligned one


def _declared():
    txt = open(HDR).read()
    return sorted(set(re.findall(r"^\s*(?:mc_status|int|const char\*|size_t)\s+(mc_\w+)\(", txt,
                                 re.M)))


def test_library_exports_every_declared_symbol():
    lib = mc.load()
    names = _declared()
    assert set(names) == set(mc.EXPORTED)
    for n in names:
        assert hasattr(lib, n)
    out = subprocess.run(["nm", "-D", "--defined-only", mc.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (mc_\w+)$", out, re.M))
    assert set(names) <= exported


def test_version_and_status_strings():
    assert mc.mc_abi_version() == 1
    for s in range(9):
        assert isinstance(mc.mc_status_str(s), str) and mc.mc_status_str(s)


def dims(**kw):
    base = dict(B=1, H=2, L=1024, d_k=128, d_v=128, d_g=128, seg_len=256, x_heads=1,
                dtype="bf16", phi="identity")
    base.update(kw)
    return mc.make_dims(**base)


def scan(d, **ptr):
    p = dict(Q=A, K=A, V=A, X=A, M=A, M_lo=A, P=A, O_on=A)
    p.update(ptr)
    return mc.load().mc_scan_prefill(ctypes.byref(d), p["Q"], p["K"], p["V"], p["X"], p["M"],
                                     p["M_lo"], p["P"], p["O_on"], None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), mc.MC_ERR_DIMS), (dict(H=-1), mc.MC_ERR_DIMS), (dict(L=0), mc.MC_ERR_DIMS),
    (dict(seg_len=0), mc.MC_ERR_DIMS), (dict(x_heads=3), mc.MC_ERR_DIMS),
    (dict(d_k=96), mc.MC_ERR_UNSUPPORTED), (dict(d_v=32), mc.MC_ERR_UNSUPPORTED),
    (dict(d_g=12), mc.MC_ERR_UNSUPPORTED), (dict(d_g=512), mc.MC_ERR_UNSUPPORTED),
    (dict(dtype=7), mc.MC_ERR_UNSUPPORTED), (dict(phi=5), mc.MC_ERR_UNSUPPORTED),
])
def test_scan_rejects_bad_dims(kw, code):
    assert scan(dims(**kw)) == code


def test_scan_null_and_alignment():
    assert mc.load().mc_scan_prefill(None, A, A, A, A, A, A, A, A, None, 0, None) == mc.MC_ERR_NULL
    for name in ("Q", "K", "V", "X", "M", "P"):
        assert scan(dims(), **{name: None}) == mc.MC_ERR_NULL
        assert scan(dims(), **{name: MIS}) == mc.MC_ERR_ALIGN
    assert scan(dims(), O_on=MIS) == mc.MC_ERR_ALIGN           # optional, but checked
    assert scan(dims(), M_lo=None) == mc.MC_ERR_NULL          # bf16 needs the operand copy
    assert scan(dims(dtype="f32"), M_lo=MIS) == mc.MC_ERR_ALIGN


def grm(d, ws_bytes, **ptr):
    p = dict(Q=A, K=A, V=A, U=A, X=A, M=A, M_lo=A, P=A, O_on=A, Y=A, gamma=None, ws=A)
    p.update(ptr)
    return mc.load().mc_grm_readout(ctypes.byref(d), p["Q"], p["K"], p["V"], p["U"], p["X"],
                                    p["M"], p["M_lo"], p["P"], p["O_on"], p["Y"], p["gamma"],
                                    p["ws"], ws_bytes, None)


def test_grm_workspace_and_pointers():
    d = dims()
    need = mc.mc_workspace_bytes(d, mc.MC_OP_GRM)
    assert need >= 4 * 2 * 1024
    assert grm(d, need - 1) == mc.MC_ERR_WORKSPACE
    assert grm(d, need, ws=None) == mc.MC_ERR_WORKSPACE
    assert grm(d, need, Y=None) == mc.MC_ERR_NULL
    assert grm(d, need, M_lo=None) == mc.MC_ERR_NULL            # bf16 reads M_lo
    assert grm(dims(dtype="f32"), need, M=None) == mc.MC_ERR_NULL  # fp32 reads M
    assert grm(d, need, gamma=MIS) == mc.MC_ERR_ALIGN
    assert grm(dims(L=-5), need) == mc.MC_ERR_DIMS
    # without O_on the online term is formed from K and V, which are then required
    assert grm(d, need, O_on=None, K=None) == mc.MC_ERR_NULL
    assert grm(d, need, O_on=None, V=None) == mc.MC_ERR_NULL
    assert grm(d, need, O_on=None, K=MIS) == mc.MC_ERR_ALIGN


def test_read_workspace_regions():
    # the bf16 MFMA read forms the online term in-kernel and takes the online logit from
    # fp32 prefix sums of X; the generic kernels (fp32, or a gate width the MFMA read does not
    # take) stage the online read and the online logits instead
    d = dims()
    B, H, L, dv, dg, xh = d.B, d.H, d.L, d.d_v, d.d_g, d.x_heads
    aon = 4 * B * H * L
    bf = mc.mc_workspace_bytes(d, mc.MC_OP_GRM)
    assert bf >= aon + 4 * B * xh * L * dg
    for gen in (dims(dtype="f32"), dims(d_g=24), dims(d_g=256)):
        assert mc.mc_workspace_bytes(gen, mc.MC_OP_GRM) >= aon + 4 * B * H * L * dv
    # d_k = d_v = 128: the gate runs as its own pass and writes its softmax numerators per
    # read tile of 256 tokens (bf16 [B,H,tiles,NS,256]) plus the online weight and 1/l per token
    g = dims(d_k=128, d_v=128)
    NS, T = -(-g.L // g.seg_len), -(-g.L // 256)
    assert mc.mc_workspace_bytes(g, mc.MC_OP_GRM) >= (
        4 * g.B * g.H * g.L + 4 * g.B * g.x_heads * g.L * g.d_g
        + 2 * g.B * g.H * T * NS * 256 + 8 * g.B * g.H * g.L)


def test_ssc_arguments():
    d = dims()
    lib = mc.load()
    need = mc.mc_workspace_bytes(d, mc.MC_OP_SSC, 4)
    # the SSC read adds fp64 segment sums of X to the prefix sums (its gate stays in the read)
    B, L, xh, dg = d.B, d.L, d.x_heads, d.d_g
    NS = -(-L // d.seg_len)
    assert need >= 4 * B * xh * L * dg + 8 * B * xh * NS * dg

    def call(k, ws_bytes, idx=A):
        return lib.mc_ssc_readout(ctypes.byref(d), k, A, A, A, A, A, A, A, A, A, A, idx, A,
                                  ws_bytes, None)
    assert call(0, need) == mc.MC_ERR_DIMS
    assert call(17, need) == mc.MC_ERR_UNSUPPORTED
    assert call(4, need, idx=None) == mc.MC_ERR_NULL
    assert call(4, need - 8) == mc.MC_ERR_WORKSPACE


def test_decode_arguments_and_capacity():
    d = dims(L=1)
    lib = mc.load()
    C = d.seg_len
    n_cap = 8
    need = mc.mc_workspace_bytes(d, mc.MC_OP_DECODE, 0, n_cap)
    assert need > 0

    def call(count, n, cap=n_cap, ws_bytes=need, y=A):
        cnt = np.array([count], np.int32)
        nc = np.array([n], np.int32)
        rc = lib.mc_decode_step(ctypes.byref(d), A, A, A, A, A, A, A, cnt.ctypes.data, A, A,
                                nc.ctypes.data, cap, y, A, ws_bytes, None)
        return rc, int(cnt[0]), int(nc[0])
    assert call(C - 1, n_cap) == (mc.MC_ERR_CAPACITY, C - 1, n_cap)  # unchanged on error
    assert call(C, 0)[0] == mc.MC_ERR_DIMS
    assert call(-1, 0)[0] == mc.MC_ERR_DIMS
    assert call(3, n_cap + 1)[0] == mc.MC_ERR_DIMS
    assert call(3, 2, ws_bytes=need - 1)[0] == mc.MC_ERR_WORKSPACE
    assert call(3, 2, y=None)[0] == mc.MC_ERR_NULL
    assert call(3, 2, y=MIS)[0] == mc.MC_ERR_ALIGN


def test_decode_noalloc_arguments():
    # the same validation as mc_decode_step (no workspace argument), plus the limit of the
    # fixed scratch buffer: 64 x 32 heads of d_v = 128 hold up to 496 cached states
    lib = mc.load()

    def call(d, count, n, cap, y=A):
        cnt = np.array([count], np.int32)
        nc = np.array([n], np.int32)
        rc = lib.mc_decode_step_noalloc(ctypes.byref(d), A, A, A, A, A, A, A, cnt.ctypes.data,
                                        A, A, nc.ctypes.data, cap, y, None)
        return rc, int(cnt[0]), int(nc[0])
    d = dims(L=1)
    C = d.seg_len
    assert call(d, C - 1, 8, 8) == (mc.MC_ERR_CAPACITY, C - 1, 8)
    assert call(d, C, 0, 8)[0] == mc.MC_ERR_DIMS
    assert call(d, 3, 9, 8)[0] == mc.MC_ERR_DIMS
    assert call(d, 3, 2, 8, y=None)[0] == mc.MC_ERR_NULL
    assert call(d, 3, 2, 8, y=MIS)[0] == mc.MC_ERR_ALIGN
    big = dims(B=64, H=32, L=1)
    assert mc.mc_workspace_bytes(big, mc.MC_OP_DECODE, 0, 496) <= mc.MC_NOALLOC_SCRATCH_BYTES
    assert mc.mc_workspace_bytes(big, mc.MC_OP_DECODE, 0, 497) > mc.MC_NOALLOC_SCRATCH_BYTES
    assert call(big, 3, 497, 600) == (mc.MC_ERR_SCRATCH, 3, 497)  # unchanged on error
    assert call(big, 3, 496, 600, y=MIS)[0] == mc.MC_ERR_ALIGN


def test_workspace_sizes_scale_with_inputs():
    small = mc.mc_workspace_bytes(dims(L=512), mc.MC_OP_GRM)
    big = mc.mc_workspace_bytes(dims(L=4096), mc.MC_OP_GRM)
    assert big >= 8 * small - 256
    assert mc.mc_workspace_bytes(dims(B=0), mc.MC_OP_GRM) == 0
    assert mc.mc_workspace_bytes(dims(), mc.MC_OP_PREFILL) == 0


def test_segment_offsets_are_validated():
    # arbitrary boundaries: host offsets 0 = o_0 < ... < o_n = L, at most MC_MAX_SEGS segments
    d = dims(L=1000)
    lib = mc.load()
    ws = mc.mc_workspace_bytes(d, mc.MC_OP_GRM)

    def scan(off, **kw):
        off = np.ascontiguousarray(np.asarray(off, dtype=np.int32))
        p = dict(Q=A, K=A, V=A, X=A, M=A, M_lo=A, P=A, O_on=A)
        p.update(kw)
        nb = mc.mc_workspace_bytes(d, mc.MC_OP_SCAN_SEGS, max(1, off.shape[0] - 1))
        return lib.mc_scan_prefill_segs(ctypes.byref(d), off.ctypes.data, off.shape[0] - 1,
                                        p["Q"], p["K"], p["V"], p["X"], p["M"], p["M_lo"],
                                        p["P"], p["O_on"], p.get("ws", A), p.get("wsb", nb),
                                        None)

    def read(off, ws_bytes=ws, **kw):
        off = np.ascontiguousarray(np.asarray(off, dtype=np.int32))
        p = dict(Q=A, U=A, X=A, M=A, M_lo=A, P=A, O_on=A, Y=A, gamma=None, ws=A)
        p.update(kw)
        return lib.mc_grm_readout_segs(ctypes.byref(d), off.ctypes.data, off.shape[0] - 1,
                                       p["Q"], p["U"], p["X"], p["M"], p["M_lo"], p["P"],
                                       p["O_on"], p["Y"], p["gamma"], p["ws"], ws_bytes, None)
    good = [0, 512, 768, 896, 960, 992, 1000]
    for bad in ([0, 512, 512, 1000], [1, 512, 1000], [0, 512, 999], [0, 600, 500, 1000], [0]):
        assert scan(bad) == mc.MC_ERR_DIMS, bad
        assert read(bad) == mc.MC_ERR_DIMS, bad
    many = list(range(0, 1000, 1)) + [1000]  # 1000 segments > MC_MAX_SEGS
    assert scan(many) == mc.MC_ERR_UNSUPPORTED
    assert read(many) == mc.MC_ERR_UNSUPPORTED
    assert lib.mc_scan_prefill_segs(ctypes.byref(d), None, 2, A, A, A, A, A, A, A, A, A, 0,
                                    None) == mc.MC_ERR_NULL
    # bf16: long segments are scanned as pieces whose states take workspace
    nb = mc.mc_workspace_bytes(d, mc.MC_OP_SCAN_SEGS, len(good) - 1)
    assert nb >= 2 * 4 * d.B * d.H * (len(good) - 1 + 2) * d.d_v * d.d_k
    assert scan(good, ws=None) == mc.MC_ERR_WORKSPACE
    assert scan(good, wsb=nb - 1) == mc.MC_ERR_WORKSPACE
    assert mc.mc_workspace_bytes(dims(L=1000, dtype="f32"), mc.MC_OP_SCAN_SEGS, 6) == 0
    # the read's workspace for n_seg segments holds the gate pass's buffers (bf16, d = 128),
    # which grow with n_seg; without them (the constant-length size) the read forms the gate
    # in-kernel, so either size is accepted and less than the read's own buffers is not
    g6 = mc.mc_workspace_bytes(d, mc.MC_OP_GRM_SEGS, 6)
    g64 = mc.mc_workspace_bytes(d, mc.MC_OP_GRM_SEGS, 64)
    aon = 4 * d.B * d.H * d.L
    assert g64 > g6 > aon + 4 * d.B * d.x_heads * d.L * d.d_g
    assert g64 - g6 >= 2 * d.B * d.H * ((d.L + 255) // 256) * 256 * (64 - 6)
    assert mc.mc_workspace_bytes(d, mc.MC_OP_GRM_SEGS, 0) == 0
    assert mc.mc_workspace_bytes(d, mc.MC_OP_GRM_SEGS, mc.MC_MAX_SEGS + 1) == 0
    assert read(good, ws_bytes=0) == mc.MC_ERR_WORKSPACE
    assert read(good, ws=None, ws_bytes=g6) == mc.MC_ERR_WORKSPACE
    assert read(good, ws_bytes=aon) == mc.MC_ERR_WORKSPACE
    assert scan(good, M_lo=None) == mc.MC_ERR_NULL        # bf16 writes the bf16 copy
    assert scan(good, X=MIS) == mc.MC_ERR_ALIGN
    assert read(good, O_on=None) == mc.MC_ERR_NULL        # the read takes the scan's O_on
    assert read(good, Y=MIS) == mc.MC_ERR_ALIGN


def test_prefill_segs_one_call_arguments():
    # the one-call prefill over offsets: validation as the two calls it replaces, no O_on
    # argument; its workspace holds the scan's pieces, the memories before them (or O_on) and
    # the read's buffers
    d = dims(L=1000)
    lib = mc.load()
    good = [0, 512, 768, 896, 960, 992, 1000]
    n = len(good) - 1
    need = mc.mc_workspace_bytes(d, mc.MC_OP_GRM_PREFILL_SEGS, n)
    assert need >= (mc.mc_workspace_bytes(d, mc.MC_OP_SCAN_SEGS, n)
                    + mc.mc_workspace_bytes(d, mc.MC_OP_GRM_SEGS, n)
                    + 4 * d.B * d.H * d.L * d.d_v)
    assert mc.mc_workspace_bytes(d, mc.MC_OP_GRM_PREFILL_SEGS, 0) == 0
    assert mc.mc_workspace_bytes(d, mc.MC_OP_GRM_PREFILL_SEGS, mc.MC_MAX_SEGS + 1) == 0

    def call(off, ws_bytes=need, **kw):
        off = np.ascontiguousarray(np.asarray(off, dtype=np.int32))
        p = dict(Q=A, K=A, V=A, U=A, X=A, M=A, M_lo=A, P=A, Y=A, gamma=None, ws=A)
        p.update(kw)
        return lib.mc_grm_prefill_segs(ctypes.byref(d), off.ctypes.data, off.shape[0] - 1,
                                       p["Q"], p["K"], p["V"], p["U"], p["X"], p["M"],
                                       p["M_lo"], p["P"], p["Y"], p["gamma"], p["ws"],
                                       ws_bytes, None)
    for bad in ([0, 512, 512, 1000], [1, 512, 1000], [0, 512, 999], [0]):
        assert call(bad) == mc.MC_ERR_DIMS, bad
    assert call(list(range(1000)) + [1000]) == mc.MC_ERR_UNSUPPORTED
    assert call(good, K=None) == mc.MC_ERR_NULL
    assert call(good, M=None) == mc.MC_ERR_NULL
    assert call(good, M_lo=None) == mc.MC_ERR_NULL
    assert call(good, ws_bytes=need - 1) == mc.MC_ERR_WORKSPACE
    assert call(good, ws=None) == mc.MC_ERR_WORKSPACE
    assert call(good, gamma=MIS) == mc.MC_ERR_ALIGN


def test_ssc_segment_offsets_arguments():
    # the SSC read over arbitrary boundaries: offsets validated as for the GRM read, top_k as
    # for mc_ssc_readout, O_on required; its workspace holds the online logits, the fp64
    # means of the n_seg segments and, for the routed read (bf16, d = 128), the tiles' pairs
    d = dims(L=1000)
    lib = mc.load()
    good = [0, 512, 768, 896, 960, 992, 1000]
    n = len(good) - 1
    need = mc.mc_workspace_bytes(d, mc.MC_OP_SSC_SEGS, 4, n)
    T = -(-d.L // 256)
    assert need >= (4 * d.B * d.H * d.L + 8 * d.B * d.x_heads * d.d_g * n
                    + 2 * 4 * d.B * d.H * T * 256 * 4 + 2 * d.B * d.H * n * d.d_v * d.d_k)
    assert mc.mc_workspace_bytes(d, mc.MC_OP_SSC_SEGS, 4, 64) > need
    assert mc.mc_workspace_bytes(d, mc.MC_OP_SSC_SEGS, 0, n) == 0
    assert mc.mc_workspace_bytes(d, mc.MC_OP_SSC_SEGS, 17, n) == 0
    assert mc.mc_workspace_bytes(d, mc.MC_OP_SSC_SEGS, 4, 0) == 0
    assert mc.mc_workspace_bytes(d, mc.MC_OP_SSC_SEGS, 4, mc.MC_MAX_SEGS + 1) == 0
    # fp32 runs the generic read: no routing tables
    f = dims(L=1000, dtype="f32")
    assert (mc.mc_workspace_bytes(f, mc.MC_OP_SSC_SEGS, 4, n)
            < mc.mc_workspace_bytes(d, mc.MC_OP_SSC_SEGS, 4, n))

    def call(off, k=4, ws_bytes=need, **kw):
        off = np.ascontiguousarray(np.asarray(off, dtype=np.int32))
        p = dict(Q=A, U=A, X=A, M=A, M_lo=A, P=A, O_on=A, Y=A, idx=A, ws=A)
        p.update(kw)
        return lib.mc_ssc_readout_segs(ctypes.byref(d), off.ctypes.data, off.shape[0] - 1, k,
                                       p["Q"], p["U"], p["X"], p["M"], p["M_lo"], p["P"],
                                       p["O_on"], p["Y"], p["idx"], p["ws"], ws_bytes, None)
    for bad in ([0, 512, 512, 1000], [1, 512, 1000], [0, 512, 999], [0]):
        assert call(bad) == mc.MC_ERR_DIMS, bad
    assert call(list(range(1000)) + [1000]) == mc.MC_ERR_UNSUPPORTED
    assert call(good, k=0) == mc.MC_ERR_DIMS
    assert call(good, k=17) == mc.MC_ERR_UNSUPPORTED
    assert call(good, idx=None) == mc.MC_ERR_NULL
    assert call(good, O_on=None) == mc.MC_ERR_NULL
    assert call(good, M_lo=None) == mc.MC_ERR_NULL        # bf16 reads the bf16 copy
    assert call(good, ws_bytes=need - 1) == mc.MC_ERR_WORKSPACE
    assert call(good, ws=None) == mc.MC_ERR_WORKSPACE
    assert call(good, Y=MIS) == mc.MC_ERR_ALIGN
    assert lib.mc_ssc_readout_segs(ctypes.byref(d), None, 2, 4, A, A, A, A, A, A, A, A, A, A,
                                   need, None) == mc.MC_ERR_NULL


def test_swla_scan_arguments():
    # SWLA write path: gates and O_on required, offsets optional and validated like the
    # segment-offset calls; every check happens before any HIP call
    d = dims(L=1000)
    lib = mc.load()

    def scan(off=None, **kw):
        p = dict(alpha=A, beta=A, lam=A, Q=A, K=A, V=A, X=A, M=A, M_lo=A, P=A, O_on=A)
        p.update(kw)
        o = None if off is None else np.ascontiguousarray(np.asarray(off, dtype=np.int32))
        return lib.mc_scan_prefill_swla(ctypes.byref(d), None if o is None else o.ctypes.data,
                                        0 if o is None else o.shape[0] - 1, p["alpha"],
                                        p["beta"], p["lam"], p["Q"], p["K"], p["V"], p["X"],
                                        p["M"], p["M_lo"], p["P"], p["O_on"], None)
    for g in ("alpha", "beta", "lam", "O_on", "Q", "M"):
        assert scan(**{g: None}) == mc.MC_ERR_NULL, g
    assert scan(M_lo=None) == mc.MC_ERR_NULL
    assert scan(beta=MIS) == mc.MC_ERR_ALIGN
    assert scan([0, 400, 400, 1000]) == mc.MC_ERR_DIMS
    assert scan([0, 400, 999]) == mc.MC_ERR_DIMS
    assert scan(list(range(0, 1000)) + [1000]) == mc.MC_ERR_UNSUPPORTED
    bad = dims(L=1000)
    bad.seg_len = 0
    assert lib.mc_scan_prefill_swla(ctypes.byref(bad), None, 0, A, A, A, A, A, A, A, A, A, A,
                                    A, None) == mc.MC_ERR_DIMS


def test_backward_arguments():
    d = dims()
    lib = mc.load()
    need = mc.mc_workspace_bytes(d, mc.MC_OP_GRM_BACKWARD)
    B, H, L, dk, dv = d.B, d.H, d.L, d.d_k, d.d_v
    NS = -(-L // d.seg_len)
    # online read and its transpose, dgamma per (token, segment), dM per segment, 3 per token
    assert need >= 4 * B * H * L * (dv + dk + NS + 3) + 4 * B * H * NS * dv * dk

    def call(ws_bytes=need, **kw):
        p = dict(Q=A, K=A, V=A, U=A, X=A, M=A, M_lo=A, P=A, dY=A, dQ=A, dK=A, dV=A, dU=A, dX=A,
                 ws=A)
        p.update(kw)
        return lib.mc_grm_backward(ctypes.byref(d), *(p[k] for k in (
            "Q", "K", "V", "U", "X", "M", "M_lo", "P", "dY", "dQ", "dK", "dV", "dU", "dX",
            "ws")), ws_bytes, None)
    for k in ("Q", "K", "V", "U", "X", "P", "dY", "dQ", "dK", "dV", "dU", "dX", "M_lo"):
        assert call(**{k: None}) == mc.MC_ERR_NULL, k
    assert call(ws_bytes=need - 1) == mc.MC_ERR_WORKSPACE
    assert call(dX=MIS) == mc.MC_ERR_ALIGN
    # bf16 reads only the bf16 states: M = NULL passes the pointer checks (the call then stops
    # at the misaligned dX); fp32 reads only M, so there M = NULL is an error
    assert call(M=None, dX=MIS) == mc.MC_ERR_ALIGN
    d.dtype = mc.MC_F32
    need = mc.mc_workspace_bytes(d, mc.MC_OP_GRM_BACKWARD)
    assert call(ws_bytes=need, M=None) == mc.MC_ERR_NULL
    assert call(ws_bytes=need, M_lo=None, dX=MIS) == mc.MC_ERR_ALIGN
