"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Bars (max over (b, h) slices of max|gpu - oracle| / max|oracle|): 1e-4 for fp32 inputs,
2e-2 for bf16 inputs with fp32 accumulation; SSC indices must match exactly.
Small cases span several tiles and segments and include ragged tails (L % C != 0,
L % 32 != 0), a single partial segment, C = 1, per-head X and both head widths.
"""
import numpy as np
import pytest

import oracle
from chunked_linear_attention_segment_amd.inputs import (WORKLOADS, Workload, make_prefill,
                                                         make_swla_gates, make_upstream_grad)
from mcutil import TOL, announce, slice_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunked_linear_attention_segment_amd as mc  # noqa: E402


def _dims(w: Workload, L=None, B=None, H=None):
    return mc.make_dims(B if B is not None else w.B, H if H is not None else w.H,
                        L if L is not None else w.L, w.d_k, w.d_v, w.d_g, w.seg_len,
                        1 if w.x_heads == 1 else (H if H is not None else w.H), w.dtype, w.phi)


SMALL = {
    "f32_L512_d64_C64": (WORKLOADS["grm_f32_L512"], {}),
    "bf16_elu_L1024_C256": (WORKLOADS["grm_bf16_L4K_elu"], dict(B=1, H=2, L=1024)),
    "bf16_elu_ragged_L1000": (WORKLOADS["grm_bf16_L4K_elu"], dict(B=2, H=2, L=1000)),
    "bf16_l2norm_L4096_C512": (WORKLOADS["grm_bf16_L64K"], dict(B=1, H=2, L=4096)),
    "bf16_single_partial_segment": (WORKLOADS["grm_bf16_L4K_elu"], dict(B=1, H=2, L=200)),
    "bf16_C16_d64_L300": (Workload("x", 1, 2, 300, 64, 64, 64, 16, "identity", "bf16"), {}),
    "f32_dk128_dv64_C48_L333": (Workload("x", 2, 2, 333, 128, 64, 96, 48, "elu1", "f32"), {}),
    "bf16_dk64_dv128_xheadsH": (Workload("x", 1, 3, 640, 64, 128, 64, 128, "identity", "bf16",
                                         x_heads=3), {}),
    "f32_C1_L40": (Workload("x", 1, 2, 40, 64, 64, 32, 1, "identity", "f32"), {}),
    # more cached states than the read keeps weights for at once (128): the gate takes the
    # max over every logit first and the weights are refreshed in the middle of the read
    "bf16_C16_150_segments": (Workload("x", 1, 2, 2400, 64, 64, 128, 16, "identity", "bf16"),
                              {}),
    # d = 128: the 512-token read with the gate pass; many segments per tile, ragged tail,
    # more cached states than one tile of weights rows, elu+1
    "bf16_d128_C48_ragged_L700": (Workload("x", 1, 2, 700, 128, 128, 128, 48, "elu1", "bf16"),
                                  {}),
    "bf16_d128_C16_150_segments": (Workload("x", 1, 2, 2400, 128, 128, 128, 16, "identity",
                                            "bf16"), {}),
    # degenerate sizes: one token; one-token segments on the MFMA path
    "bf16_d128_L1": (Workload("x", 1, 2, 1, 128, 128, 128, 64, "identity", "bf16"), {}),
    "f32_d64_L1": (Workload("x", 1, 1, 1, 64, 64, 64, 64, "identity", "f32"), {}),
    "bf16_d128_C1_L80_elu": (Workload("x", 1, 2, 80, 128, 128, 64, 1, "elu1", "bf16"), {}),
    "bf16_d128_C512_L1536_elu": (Workload("x", 2, 3, 1536, 128, 128, 64, 512, "elu1", "bf16"),
                                 {}),
}


def _run_grm(w, kw, seed=0, online=True):
    inp = make_prefill(w, seed=seed, **kw)
    d = _dims(w, **kw)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    out = mc.prefill_grm(d, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"], want_gamma=True,
                         online=online)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], seg_len=w.seg_len,
                         phi=w.phi, mode="grm", want_states=True, want_online=True,
                         want_gamma=True)
    return out, ref


@pytest.mark.parametrize("online", [True, False], ids=["with_O_on", "fused_online"])
@pytest.mark.parametrize("name", list(SMALL))
def test_grm_prefill_small(name, online):
    w, kw = SMALL[name]
    announce("grm parity %s online=%s" % (name, online))
    out, ref = _run_grm(w, kw, online=online)
    tol = TOL[w.dtype]
    errs = {
        "Y": slice_rel_err(to_np(out["Y"]), ref["Y"]),
        "M": slice_rel_err(to_np(out["M"]), ref["M"]),
        "P": slice_rel_err(to_np(out["P"]), ref["P"]),
        "gamma": slice_rel_err(to_np(out["gamma"]), ref["gamma"]),
    }
    if online:
        errs["O_on"] = slice_rel_err(to_np(out["O_on"]), ref["O_on"])
    if w.dtype == "bf16":
        errs["M_lo"] = slice_rel_err(to_np(out["M_lo"]), ref["M"])
    announce("  errors %s" % errs)
    for k, e in errs.items():
        assert e <= tol, (k, e)


SSC_SMALL = {
    "bf16_L2048_C128_k4": (Workload("x", 1, 2, 2048, 128, 128, 128, 128, "identity", "bf16",
                                    top_k=4, op="ssc"), {}),
    "bf16_ragged_L1500_C64_k3": (Workload("x", 2, 2, 1500, 128, 128, 128, 64, "elu1", "bf16",
                                          top_k=3, op="ssc"), {}),
    "f32_L512_C32_k2_d64": (Workload("x", 1, 2, 512, 64, 64, 64, 32, "identity", "f32",
                                     top_k=2, op="ssc"), {}),
    "bf16_k_ge_N": (Workload("x", 1, 2, 512, 128, 128, 128, 64, "identity", "bf16", top_k=9,
                             op="ssc"), {}),
    # more candidate segments than the SSC read keeps weights for at once (96)
    "bf16_C16_120_segments_k5": (Workload("x", 1, 2, 1920, 64, 64, 64, 16, "elu1", "bf16",
                                          top_k=5, op="ssc"), {}),
    # d_k != d_v: with the online term given, the read kernel that forms the gate itself is
    # not used at d_v = 128 (the generic read is)
    "bf16_dk64_dv128_k3": (Workload("x", 1, 2, 1024, 64, 128, 64, 128, "identity", "bf16",
                                    top_k=3, op="ssc"), {}),
}


@pytest.mark.parametrize("online", [True, False], ids=["with_O_on", "fused_online"])
@pytest.mark.parametrize("name", list(SSC_SMALL))
def test_ssc_prefill_small(name, online):
    w, kw = SSC_SMALL[name]
    announce("ssc parity %s online=%s" % (name, online))
    inp = make_prefill(w, seed=1, **kw)
    d = _dims(w, **kw)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    out = mc.prefill_ssc(d, w.top_k, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"],
                         online=online)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], seg_len=w.seg_len,
                         phi=w.phi, mode="ssc", top_k=w.top_k)
    np.testing.assert_array_equal(to_np(out["idx"]), ref["idx"])
    e = slice_rel_err(to_np(out["Y"]), ref["Y"])
    announce("  Y error %.3g" % e)
    assert e <= TOL[w.dtype]


def test_ssc_ties_choose_lowest_index():
    """Duplicated segments give exactly equal router scores; the lower index must win."""
    w = Workload("x", 1, 2, 1024, 128, 128, 128, 64, "identity", "bf16", top_k=2, op="ssc")
    inp = make_prefill(w, seed=3)
    for src, dst in ((0, 3), (0, 7), (2, 9)):
        inp["X"][:, :, dst * 64:(dst + 1) * 64] = inp["X"][:, :, src * 64:(src + 1) * 64]
    d = _dims(w)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    out = mc.prefill_ssc(d, w.top_k, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"])
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], seg_len=64,
                         mode="ssc", top_k=2)
    got = to_np(out["idx"])
    np.testing.assert_array_equal(got, ref["idx"])
    late = (np.arange(1024) // 64 >= 4)[None, None, :]
    sel0 = (got == 0).any(-1)
    sel3 = (got == 3).any(-1)
    assert not np.any(sel3 & ~sel0 & late)   # 3 never wins over its equal, lower twin
    assert np.any(sel0 & ~sel3 & late)       # the tie at the k-th place did occur


def test_grm_deterministic():
    w, kw = SMALL["bf16_elu_L1024_C256"]
    inp = make_prefill(w, seed=5, **kw)
    d = _dims(w, **kw)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    for online in (True, False):
        a = mc.prefill_grm(d, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"], online=online)
        b = mc.prefill_grm(d, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"], online=online)
        assert torch.equal(a["Y"], b["Y"]) and torch.equal(a["M"], b["M"])


def test_ssc_routed_read_deterministic():
    """The routed SSC read adds every token's terms in a fixed order (the online term, then
    the selected states by ascending index), so two calls give identical bits."""
    w, kw = SSC_SMALL["bf16_L2048_C128_k4"]
    announce("ssc determinism")
    inp = make_prefill(w, seed=6, **kw)
    d = _dims(w, **kw)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    for online in (True, False):
        a = mc.prefill_ssc(d, w.top_k, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"],
                           online=online)
        b = mc.prefill_ssc(d, w.top_k, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"],
                           online=online)
        assert torch.equal(a["Y"], b["Y"]) and torch.equal(a["idx"], b["idx"])


# ---- decode -------------------------------------------------------------------------------

def _decode_case(w, B, H, n, cnt, cap, seed):
    from chunked_linear_attention_segment_amd.inputs import make_decode
    inp = make_decode(w, seed=seed, B=B, H=H, n_cap=cap, n_cached=n, count_on=cnt)
    d = mc.make_dims(B, H, 1, w.d_k, w.d_v, w.d_g, w.seg_len, 1, w.dtype, w.phi)
    return inp, d


def _gpu_decode_state(inp, dtype):
    dev = {k: to_dev(inp[k], dtype) for k in ("q", "k", "v", "u", "x")}
    dev["M_on"] = to_dev(inp["M_on"])
    dev["xsum"] = to_dev(inp["xsum"])
    dev["M_cache"] = to_dev(inp["M_cache"], dtype)
    dev["P_cache"] = to_dev(inp["P_cache"])
    return dev


# n spans: no cached state, one short run, several runs with a ragged last one
@pytest.mark.parametrize("dtype,phi,n,cnt,C,dk,dv", [("bf16", "identity", 7, 3, 16, 128, 128),
                                                     ("f32", "elu1", 5, 0, 8, 128, 128),
                                                     ("bf16", "identity", 0, 2, 16, 128, 128),
                                                     ("f32", "identity", 40, 6, 8, 128, 128),
                                                     ("bf16", "elu1", 19, 13, 16, 64, 128),
                                                     ("bf16", "identity", 45, 5, 8, 64, 64),
                                                     ("f32", "identity", 33, 4, 8, 128, 64)])
def test_decode_step_small(dtype, phi, n, cnt, C, dk, dv):
    w = Workload("x", 2, 3, 1, dk, dv, 128, C, phi, dtype, op="decode")
    cap = n + 3
    inp, d = _decode_case(w, 2, 3, n, cnt, cap, seed=11)
    dev = _gpu_decode_state(inp, dtype)
    st = oracle.DecodeState(inp["M_on"], inp["xsum"], cnt, inp["M_cache"], inp["P_cache"], n)
    count = np.array([cnt], np.int32)
    ncached = np.array([n], np.int32)
    ws = mc.workspace(d, mc.MC_OP_DECODE, n_cap=cap)
    # several steps in a row, crossing a segment boundary (emission) when C - cnt <= steps
    for step in range(C - cnt + 2):
        y = torch.empty((2, 3, dv), dtype=mc.torch_dtype(d), device="cuda")
        if step > 0:  # a fresh token each step
            rng = np.random.default_rng(100 + step)
            for key in ("q", "k", "v", "u", "x"):
                arr = rng.standard_normal(inp[key].shape).astype(np.float32)
                if dtype == "bf16":
                    from chunked_linear_attention_segment_amd.inputs import round_bf16
                    arr = round_bf16(arr)
                inp[key] = arr
                dev[key] = to_dev(arr, dtype)
        mc.mc_decode_step(d, dev["q"], dev["k"], dev["v"], dev["u"], dev["x"], dev["M_on"],
                          dev["xsum"], count, dev["M_cache"], dev["P_cache"], ncached, cap, y,
                          ws=ws)
        torch.cuda.synchronize()
        yref = oracle.decode_step(st, inp["q"], inp["k"], inp["v"], inp["u"], inp["x"],
                                  seg_len=C, phi=phi)
        assert int(count[0]) == int(st.count[0]) and int(ncached[0]) == int(st.n_cached[0])
        e = slice_rel_err(to_np(y), yref)
        assert e <= TOL[dtype], (step, e)
        assert slice_rel_err(to_np(dev["M_on"]), st.M_on) <= 1e-5 or np.all(st.M_on == 0)
        nn = int(ncached[0])
        if nn:
            assert slice_rel_err(to_np(dev["M_cache"])[:, :, :nn], st.M_cache[:, :, :nn],
                                 lead=3) <= TOL[dtype]
            assert slice_rel_err(to_np(dev["P_cache"])[:, :, :nn], st.P_cache[:, :, :nn],
                                 lead=3) <= 1e-5
        # the oracle keeps full precision; feed it the cache the GPU holds so the
        # next step compares reads, not the rounding of an emitted bf16 state
        st.M_cache = to_np(dev["M_cache"]).copy()


@pytest.mark.parametrize("dtype,n,cnt,C", [("bf16", 37, 5, 8), ("f32", 0, 3, 8),
                                            ("bf16", 9, 14, 16)])
def test_decode_average_small(dtype, n, cnt, C):
    """Post-training decode (u = NULL): the plain mean of the memories, several steps in a
    row across a segment boundary, against the oracle's average mode."""
    w = Workload("x", 2, 3, 1, 128, 128, 128, C, "identity", dtype, op="decode")
    cap = n + 3
    inp, d = _decode_case(w, 2, 3, n, cnt, cap, seed=31)
    dev = _gpu_decode_state(inp, dtype)
    st = oracle.DecodeState(inp["M_on"], inp["xsum"], cnt, inp["M_cache"], inp["P_cache"], n)
    count = np.array([cnt], np.int32)
    ncached = np.array([n], np.int32)
    ws = mc.workspace(d, mc.MC_OP_DECODE, n_cap=cap)
    for step in range(C - cnt + 1):
        announce("decode average %s n=%d step %d" % (dtype, int(ncached[0]), step))
        if step > 0:
            rng = np.random.default_rng(200 + step)
            for key in ("q", "k", "v", "x"):
                arr = rng.standard_normal(inp[key].shape).astype(np.float32)
                if dtype == "bf16":
                    from chunked_linear_attention_segment_amd.inputs import round_bf16
                    arr = round_bf16(arr)
                inp[key] = arr
                dev[key] = to_dev(arr, dtype)
        y = torch.empty((2, 3, 128), dtype=mc.torch_dtype(d), device="cuda")
        mc.mc_decode_step(d, dev["q"], dev["k"], dev["v"], None, dev["x"], dev["M_on"],
                          dev["xsum"], count, dev["M_cache"], dev["P_cache"], ncached, cap, y,
                          ws=ws)
        torch.cuda.synchronize()
        yref = oracle.decode_step(st, inp["q"], inp["k"], inp["v"], inp["u"], inp["x"],
                                  seg_len=C, mode="average")
        assert int(count[0]) == int(st.count[0]) and int(ncached[0]) == int(st.n_cached[0])
        assert slice_rel_err(to_np(y), yref) <= TOL[dtype]
        nn = int(ncached[0])
        if nn:
            assert slice_rel_err(to_np(dev["P_cache"])[:, :, :nn], st.P_cache[:, :, :nn],
                                 lead=3) <= 1e-5
        st.M_cache = to_np(dev["M_cache"]).copy()


def test_prefill_then_decode_matches_longer_prefill():
    """Prefill L tokens, hand the trailing partial segment to decode, step one token:
    equals row L of a prefill over L+1 tokens (bf16, identity)."""
    w = Workload("x", 1, 2, 1, 128, 128, 128, 64, "identity", "bf16")
    L = 191  # 2 full segments + 63 tokens: the decode step completes segment 2 (emission)
    inp = make_prefill(w, seed=21, L=L + 1)
    d = mc.make_dims(1, 2, L, 128, 128, 128, 64, 1, "bf16", "identity")
    dev = {k: to_dev(v[:, :, :L], "bf16") for k, v in inp.items()}
    pre = mc.prefill_grm(d, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"])
    cap = 4
    nfull, cnt = divmod(L, 64)
    Mc = torch.zeros((1, 2, cap, 128, 128), dtype=torch.bfloat16, device="cuda")
    Mc[:, :, :nfull] = pre["M_lo"][:, :, :nfull]
    Pc = torch.zeros((1, 1, cap, 128), dtype=torch.float32, device="cuda")
    Pc[:, :, :nfull] = pre["P"][:, :, :nfull]
    M_on = pre["M"][:, :, nfull].contiguous()
    xsum = (pre["P"][:, :, nfull] * cnt).contiguous()
    tok = {k: to_dev(v[:, :, L], "bf16") for k, v in inp.items()}
    y = torch.empty((1, 2, 128), dtype=torch.bfloat16, device="cuda")
    count = np.array([cnt], np.int32)
    ncached = np.array([nfull], np.int32)
    dd = mc.make_dims(1, 2, 1, 128, 128, 128, 64, 1, "bf16", "identity")
    mc.mc_decode_step(dd, tok["Q"], tok["K"], tok["V"], tok["U"], tok["X"], M_on, xsum, count,
                      Mc, Pc, ncached, cap, y, ws=mc.workspace(dd, mc.MC_OP_DECODE, n_cap=cap))
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], seg_len=64,
                         want_states=True)
    assert slice_rel_err(to_np(y), ref["Y"][:, :, L]) <= 2e-2
    assert int(ncached[0]) == 3 and int(count[0]) == 0
    assert slice_rel_err(to_np(Mc[:, :, 2]), ref["M"][:, :, 2]) <= 2e-2
    assert slice_rel_err(to_np(Pc[:, :, 2]), ref["P"][:, :, 2]) <= 1e-5


# Arbitrary segment boundaries (mc_scan_prefill_segs / mc_grm_readout_segs) against the
# oracle's seg_offsets mode: the logarithmic segmentation, random boundaries (including
# one-token segments), and boundaries at multiples of C (the constant-length read).
def _random_offsets(L, n, seed):
    cuts = np.sort(np.random.default_rng(seed).choice(np.arange(1, L), n - 1, replace=False))
    return [0] + cuts.tolist() + [L]


SEG_CASES = {
    "bf16_log_L1000_d128": (Workload("x", 1, 2, 1000, 128, 128, 128, 1, "identity", "bf16"),
                            "log"),
    "f32_log_L777_d64_elu": (Workload("x", 2, 2, 777, 64, 64, 32, 1, "elu1", "f32"), "log"),
    "bf16_random_L900_d128_elu": (Workload("x", 1, 3, 900, 128, 128, 64, 1, "elu1", "bf16"),
                                  "random"),
    "f32_random_L300_d64_xheadsH": (Workload("x", 1, 2, 300, 64, 128, 64, 1, "identity", "f32",
                                             x_heads=2), "random"),
    "bf16_multiples_of_64_L640": (Workload("x", 1, 2, 640, 128, 64, 128, 1, "identity",
                                           "bf16"), "c64"),
    "bf16_max_512_segments_L1100": (Workload("x", 1, 2, 1100, 128, 128, 128, 1, "identity",
                                             "bf16"), "max"),
    # segments longer than a scan piece (512 tokens): scanned as pieces, then combined
    "bf16_long_segments_L2100": (Workload("x", 1, 2, 2100, 128, 128, 128, 1, "identity", "bf16"),
                                 "long"),
    "bf16_long_segments_d64_elu_xheadsH": (Workload("x", 1, 2, 1700, 64, 64, 64, 1, "elu1",
                                                    "bf16", x_heads=2), "long"),
    # 511 one-token segments and one of 1589: no piece table fits, so the one call forms O_on
    # in its workspace instead of walking the long segment in the read
    "bf16_512_segments_one_long_L2100": (Workload("x", 1, 2, 2100, 128, 128, 128, 1,
                                                  "identity", "bf16"), "max_long"),
}


@pytest.mark.parametrize("calls", ["two_calls", "one_call"])
@pytest.mark.parametrize("name", list(SEG_CASES))
def test_grm_segment_offsets(name, calls):
    # two calls: the scan hands O_on to the read; one call (mc_grm_prefill_segs): bf16 d = 128
    # forms the online term in the read over the scan's pieces, other sizes go through O_on
    w, kind = SEG_CASES[name]
    if kind == "log":
        off = oracle.log_segments(w.L)
    elif kind == "random":
        off = _random_offsets(w.L, 23, seed=5)
        off = sorted(set(off + [off[1] + 1]))  # a one-token segment
    elif kind == "max":
        off = _random_offsets(w.L, mc.MC_MAX_SEGS, seed=6)  # the most segments a call takes
    elif kind == "long":
        off = [0, 1500, 1600, w.L]  # 3 pieces, 1 piece, 1 or 2 pieces
    elif kind == "max_long":
        off = list(range(0, mc.MC_MAX_SEGS)) + [w.L]
    else:
        off = list(range(0, w.L, 64)) + [w.L]
    announce("grm segment offsets %s (%s): %d segments" % (name, calls, len(off) - 1))
    inp = make_prefill(w, seed=3)
    d = _dims(w)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    run = mc.prefill_grm_segs if calls == "two_calls" else mc.prefill_grm_segs_onecall
    out = run(d, off, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"], want_gamma=True)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], seg_len=1,
                         phi=w.phi, mode="grm", want_states=True, want_online=True,
                         want_gamma=True, seg_offsets=off)
    tol = TOL[w.dtype]
    keys = ("Y", "M", "P", "gamma") + (("O_on",) if "O_on" in out else ())
    errs = {k: slice_rel_err(to_np(out[k]), ref[k]) for k in keys}
    announce("  errors %s" % errs)
    for k, e in errs.items():
        assert e <= tol, (k, e)


# The SSC read over arbitrary boundaries (mc_ssc_readout_segs): bf16 d = 128 runs the routed
# read, the rest the generic read restricted to the selections; indices bit-exact.
SSC_SEG_CASES = {
    "bf16_log_L1000_d128_k3": (Workload("x", 1, 2, 1000, 128, 128, 128, 1, "identity", "bf16",
                                        top_k=3, op="ssc"), "log"),
    "bf16_random_L900_d128_elu_k4": (Workload("x", 2, 2, 900, 128, 128, 64, 1, "elu1", "bf16",
                                              top_k=4, op="ssc"), "random"),
    "bf16_max_512_segments_L1100_k8": (Workload("x", 1, 2, 1100, 128, 128, 128, 1, "identity",
                                                "bf16", top_k=8, op="ssc"), "max"),
    "bf16_long_segments_L2100_k2": (Workload("x", 1, 2, 2100, 128, 128, 128, 1, "identity",
                                             "bf16", top_k=2, op="ssc"), "long"),
    "bf16_multiples_of_64_L1024_k16": (Workload("x", 1, 2, 1024, 128, 128, 128, 1, "elu1",
                                                "bf16", top_k=16, op="ssc"), "c64"),
    "f32_random_L300_d64_xheadsH_k2": (Workload("x", 1, 2, 300, 64, 64, 64, 1, "identity",
                                                "f32", x_heads=2, top_k=2, op="ssc"), "random"),
    "bf16_dk64_dv128_log_L777_k16": (Workload("x", 1, 2, 777, 64, 128, 64, 1, "elu1", "bf16",
                                              top_k=16, op="ssc"), "log"),
}


@pytest.mark.parametrize("name", list(SSC_SEG_CASES))
def test_ssc_segment_offsets(name):
    w, kind = SSC_SEG_CASES[name]
    if kind == "log":
        off = oracle.log_segments(w.L)
    elif kind == "random":
        off = _random_offsets(w.L, 23, seed=7)
        off = sorted(set(off + [off[1] + 1]))  # a one-token segment
    elif kind == "max":
        off = _random_offsets(w.L, mc.MC_MAX_SEGS, seed=8)
    elif kind == "long":
        off = [0, 1500, 1600, w.L]
    else:
        off = list(range(0, w.L, 64)) + [w.L]
    announce("ssc segment offsets %s: %d segments" % (name, len(off) - 1))
    inp = make_prefill(w, seed=4)
    d = _dims(w)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    out = mc.prefill_ssc_segs(d, off, w.top_k, dev["Q"], dev["K"], dev["V"], dev["U"],
                              dev["X"])
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], seg_len=1,
                         phi=w.phi, mode="ssc", top_k=w.top_k, seg_offsets=off)
    np.testing.assert_array_equal(to_np(out["idx"]), ref["idx"])
    e = slice_rel_err(to_np(out["Y"]), ref["Y"])
    announce("  Y error %.3g" % e)
    assert e <= TOL[w.dtype]


def test_ssc_segment_offsets_at_multiples_of_C_match_constant_read():
    # boundaries every C tokens select exactly what the constant-length SSC read selects
    w = Workload("x", 1, 2, 1000, 128, 128, 128, 64, "identity", "bf16", top_k=4, op="ssc")
    off = list(range(0, w.L, w.seg_len)) + [w.L]
    announce("ssc offsets at multiples of %d vs the constant read" % w.seg_len)
    inp = make_prefill(w, seed=9)
    d = _dims(w)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    a = mc.prefill_ssc_segs(d, off, w.top_k, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"])
    b = mc.prefill_ssc(d, w.top_k, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"])
    torch.cuda.synchronize()
    assert torch.equal(a["idx"], b["idx"])
    e = slice_rel_err(to_np(a["Y"]), to_np(b["Y"]))
    announce("  Y difference %.3g" % e)
    assert e <= TOL[w.dtype]


def test_grm_segment_offsets_in_kernel_gate():
    # The offsets read given only the constant-length workspace (MC_OP_GRM) forms the gate
    # in-kernel instead of running the gate pass over the offsets; both against the oracle.
    w = Workload("x", 1, 2, 1000, 128, 128, 128, 1, "identity", "bf16")
    off = oracle.log_segments(w.L)
    announce("grm segment offsets, in-kernel gate: %d segments" % (len(off) - 1))
    inp = make_prefill(w, seed=4)
    d = _dims(w)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    NS = len(off) - 1
    M = torch.empty((1, 2, NS, 128, 128), dtype=torch.float32, device="cuda")
    M_lo = torch.empty((1, 2, NS, 128, 128), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((1, 1, NS, 128), dtype=torch.float32, device="cuda")
    O_on = torch.empty((1, 2, w.L, 128), dtype=torch.float32, device="cuda")
    mc.mc_scan_prefill_segs(d, off, dev["Q"], dev["K"], dev["V"], dev["X"], M, M_lo, P, O_on,
                            ws=mc.workspace_segs(d, NS))
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], seg_len=1,
                         phi=w.phi, mode="grm", seg_offsets=off)
    outs = {}
    for op in (mc.MC_OP_GRM, mc.MC_OP_GRM_SEGS):
        Y = torch.empty((1, 2, w.L, 128), dtype=torch.bfloat16, device="cuda")
        ws = mc.workspace(d, op, top_k=NS)
        mc.mc_grm_readout_segs(d, off, dev["Q"], dev["U"], dev["X"], M, M_lo, P, O_on, Y,
                               None, ws=ws)
        torch.cuda.synchronize()
        outs[op] = to_np(Y)
        e = slice_rel_err(outs[op], ref["Y"])
        announce("  workspace op %d: Y error %.3g" % (op, e))
        assert e <= TOL["bf16"], (op, e)


# SWLA memory (window 2) under GRM: the MFMA scan for constant bf16 segments, the generic scan
# for fp32 and for offsets; the read takes the online term from O_on.
SWLA_CASES = {
    "bf16_d128_C256_L700": (Workload("x", 1, 3, 700, 128, 128, 128, 256, "identity", "bf16"),
                            None, None),
    "bf16_d64_C48_L300_elu": (Workload("x", 2, 2, 300, 64, 64, 64, 48, "elu1", "bf16"),
                              None, None),
    "bf16_d128_C128_strong_decay": (Workload("x", 1, 2, 512, 128, 128, 128, 128, "identity",
                                             "bf16"), None, {"alpha": (0.0, 0.2)}),
    "bf16_d128_C192_alpha_0_or_1": (Workload("x", 1, 2, 600, 128, 128, 64, 192, "identity",
                                             "bf16"), None, "binary"),
    "bf16_d128v64_C64_L200": (Workload("x", 1, 2, 200, 128, 64, 128, 64, "elu1", "bf16"),
                              None, None),
    "f32_d64_C64_L300": (Workload("x", 1, 2, 300, 64, 64, 64, 64, "identity", "f32"), None,
                         None),
    "bf16_log_L1000_d128": (Workload("x", 1, 2, 1000, 128, 128, 128, 1, "identity", "bf16"),
                            "log", None),
    "f32_random_L500_d128_xheadsH": (Workload("x", 1, 2, 500, 128, 128, 64, 1, "elu1", "f32",
                                              x_heads=2), "random", None),
}


@pytest.mark.parametrize("name", list(SWLA_CASES))
def test_swla_grm(name):
    w, seg, gate_kind = SWLA_CASES[name]
    off = None
    if seg == "log":
        off = oracle.log_segments(w.L)
    elif seg == "random":
        off = _random_offsets(w.L, 17, seed=9)
    inp = make_prefill(w, seed=4)
    B, H = inp["Q"].shape[:2]
    if gate_kind == "binary":  # decay switched fully off or on, token by token
        g = make_swla_gates(B, H, w.L, seed=6)
        g["alpha"] = (g["alpha"] > 0.95).astype(np.float32)
    else:
        g = make_swla_gates(B, H, w.L, seed=6, ranges=gate_kind)
    announce("swla %s: %s segments" % (name, "constant" if off is None else len(off) - 1))
    d = _dims(w)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    gd = {k: to_dev(v) for k, v in g.items()}
    out = mc.prefill_grm_swla(d, gd["alpha"], gd["beta"], gd["lam"], dev["Q"], dev["K"],
                              dev["V"], dev["U"], dev["X"], seg_off=off, want_gamma=True)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], seg_len=w.seg_len,
                         phi=w.phi, mode="grm", want_states=True, want_online=True,
                         want_gamma=True, seg_offsets=off,
                         swla=(g["alpha"], g["beta"], g["lam"]))
    tol = TOL[w.dtype]
    errs = {k: slice_rel_err(to_np(out[k]), ref[k]) for k in ("Y", "M", "P", "O_on", "gamma")}
    announce("  errors %s" % errs)
    for k, e in errs.items():
        assert e <= tol, (k, e)


# Backward of the GRM prefill: every gradient (fp32 outputs) against the oracle's, from the
# states and means the forward wrote.
BWD_CASES = {
    "f32_d64_C32_L200": Workload("x", 1, 2, 200, 64, 64, 64, 32, "identity", "f32"),
    "f32_d128_C64_L300_elu_xheadsH": Workload("x", 1, 2, 300, 128, 128, 64, 64, "elu1", "f32",
                                              x_heads=2),
    "bf16_d128_C256_L700": Workload("x", 1, 3, 700, 128, 128, 128, 256, "identity", "bf16"),
    "bf16_d128v64_C48_L333_elu": Workload("x", 2, 2, 333, 128, 64, 64, 48, "elu1", "bf16"),
    "bf16_d64_C16_L640_many_segments": Workload("x", 1, 2, 640, 64, 64, 32, 16, "identity",
                                                "bf16"),
    # bf16 with d_k = d_v = 128: the MFMA backward (swapped read, dgamma and dM on MFMA)
    "bf16_d128_C48_L500_elu": Workload("x", 2, 2, 500, 128, 128, 64, 48, "elu1", "bf16"),
    "bf16_d128_C512_L1536": Workload("x", 1, 2, 1536, 128, 128, 128, 512, "identity", "bf16"),
    "bf16_d128_C16_L640_xheadsH": Workload("x", 1, 2, 640, 128, 128, 32, 16, "identity", "bf16",
                                           x_heads=2),
    # degenerate sizes: one token; one-token segments; one segment (no cached state)
    "bf16_d128_L1": Workload("x", 1, 2, 1, 128, 128, 128, 64, "identity", "bf16"),
    "bf16_d128_C1_L48_elu": Workload("x", 1, 2, 48, 128, 128, 64, 1, "elu1", "bf16"),
    "f32_d64_single_segment_L100": Workload("x", 1, 2, 100, 64, 64, 64, 256, "identity", "f32"),
}


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_grm_backward(name):
    w = BWD_CASES[name]
    announce("grm backward %s" % name)
    inp = make_prefill(w, seed=8)
    B, H = inp["Q"].shape[:2]
    dY = make_upstream_grad(B, H, w.L, w.d_v, seed=9, dtype=w.dtype)
    d = _dims(w)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    fwd = mc.prefill_grm(d, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"], online=False)
    got = mc.grm_backward(d, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"], fwd["M"],
                          fwd["M_lo"], fwd["P"], to_dev(dY, w.dtype))
    torch.cuda.synchronize()
    ref = oracle.grm_backward(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], dY,
                              seg_len=w.seg_len, phi=w.phi)
    tol = TOL[w.dtype]
    errs = {k: slice_rel_err(to_np(got[k]), ref[k]) for k in ("dQ", "dK", "dV", "dU", "dX")}
    announce("  errors %s" % errs)
    for k, e in errs.items():
        assert e <= tol, (k, e)


def test_grm_backward_bf16_reads_only_bf16_states():
    """The bf16 backward takes the cached states from their bf16 copy alone: M = NULL is a valid
    call (the header's contract for bf16), and its gradients match the oracle."""
    w = BWD_CASES["bf16_d128_C256_L700"]
    announce("grm backward bf16 with M = NULL")
    inp = make_prefill(w, seed=8)
    B, H = inp["Q"].shape[:2]
    dY = make_upstream_grad(B, H, w.L, w.d_v, seed=9, dtype=w.dtype)
    d = _dims(w)
    dev = {k: to_dev(v, w.dtype) for k, v in inp.items()}
    fwd = mc.prefill_grm(d, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"], online=False)
    got = mc.grm_backward(d, dev["Q"], dev["K"], dev["V"], dev["U"], dev["X"], None,
                          fwd["M_lo"], fwd["P"], to_dev(dY, w.dtype))
    torch.cuda.synchronize()
    ref = oracle.grm_backward(inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], dY,
                              seg_len=w.seg_len, phi=w.phi)
    for k in ("dQ", "dK", "dV", "dU", "dX"):
        e = slice_rel_err(to_np(got[k]), ref[k])
        assert e <= TOL[w.dtype], (k, e)
