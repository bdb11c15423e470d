"""GPU parity at the full workload sizes, in the launch configuration the benchmark times
(scan, then the read with the online term formed inside it: O_on = NULL).

The GPU computes every head and token; the fp64 oracle recomputes sampled heads on the
host -- the full-length scan of each, and the read at sampled rows (every segment
boundary, the first and last tokens and seeded random rows; every row for SSC indices).
Bars as in the small-case tests: max|gpu - oracle| / max|oracle| per (b, h) slice,
2e-2 for bf16 inputs with fp32 accumulation; SSC indices exact.
"""
import numpy as np
import pytest

import oracle
from chunked_linear_attention_segment_amd.inputs import (WORKLOADS, make_decode_device,
                                                         make_prefill_device,
                                                         make_swla_gates_device,
                                                         make_upstream_grad)
from mcutil import TOL, announce, slice_rel_err, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunked_linear_attention_segment_amd as mc  # noqa: E402


def _dims(w):
    return mc.make_dims(w.B, w.H, w.L, w.d_k, w.d_v, w.d_g, w.seg_len, 1, w.dtype, w.phi)


def _sample_rows(L, C, n_random, seed):
    r = set(range(min(8, L))) | set(range(max(0, L - 8), L))
    for s in range(0, L, C):
        r |= {t for t in (s - 1, s, s + 1, s + C // 2) if 0 <= t < L}
    r |= set(np.random.default_rng(seed).integers(0, L, n_random).tolist())
    return np.array(sorted(r), dtype=np.int32)


def _head(inp, b, h):
    """One (b, h) slice of the device inputs as host fp64 arrays of batch and head 1."""
    out = {}
    for k in ("Q", "K", "V", "U"):
        out[k] = inp[k][b:b + 1, h:h + 1].to(torch.float64).cpu().numpy()
    out["X"] = inp["X"][b:b + 1].to(torch.float64).cpu().numpy()
    return out


@pytest.mark.parametrize("name,heads", [("grm_bf16_L4K_elu", [(0, 0), (3, 15), (1, 6)]),
                                        ("grm_bf16_L64K", [(0, 0), (0, 31)])])
def test_grm_full_size(name, heads):
    w = WORKLOADS[name]
    announce("full-size GRM %s: B=%d H=%d L=%d C=%d" % (name, w.B, w.H, w.L, w.seg_len))
    inp = make_prefill_device(w, seed=0)
    d = _dims(w)
    out = mc.prefill_grm(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], online=False)
    torch.cuda.synchronize()
    assert torch.isfinite(out["Y"].float()).all()
    rows = _sample_rows(w.L, w.seg_len, 256, seed=7)
    for b, h in heads:
        hin = _head(inp, b, h)
        ref = oracle.prefill(hin["Q"], hin["K"], hin["V"], hin["U"], hin["X"],
                             seg_len=w.seg_len, phi=w.phi, rows=rows, want_states=True)
        errs = {
            "Y": slice_rel_err(to_np(out["Y"][b:b + 1, h:h + 1, rows]), ref["Y"]),
            "M": slice_rel_err(to_np(out["M"][b:b + 1, h:h + 1]), ref["M"]),
            "M_lo": slice_rel_err(to_np(out["M_lo"][b:b + 1, h:h + 1]), ref["M"]),
            "P": slice_rel_err(to_np(out["P"][b:b + 1]), ref["P"]),
        }
        announce("  (b=%d, h=%d) %d rows: %s" % (b, h, len(rows), errs))
        assert errs["Y"] <= TOL["bf16"] and errs["M_lo"] <= TOL["bf16"] and errs["P"] <= 1e-4
        # with phi = identity the bf16 operands of the state contraction are the inputs
        # themselves (exact products, fp32 sums); elu+1 features are rounded to bf16 first
        assert errs["M"] <= (1e-4 if w.phi == "identity" else TOL["bf16"])


def test_ssc_full_size():
    # every head: the oracle runs the full SSC read of all 2 x 16 heads (one per thread), so
    # the indices of every token of every head are compared exactly, and Y everywhere
    w = WORKLOADS["ssc_bf16_L16K_k4"]
    announce("full-size SSC: B=%d H=%d L=%d C=%d k=%d" % (w.B, w.H, w.L, w.seg_len, w.top_k))
    inp = make_prefill_device(w, seed=0)
    d = _dims(w)
    out = mc.prefill_ssc(d, w.top_k, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"],
                         online=False)
    torch.cuda.synchronize()
    host = {k: v.to(torch.float64).cpu().numpy() for k, v in inp.items()}
    ref = oracle.prefill(host["Q"], host["K"], host["V"], host["U"], host["X"],
                         seg_len=w.seg_len, phi=w.phi, mode="ssc", top_k=w.top_k)
    got_idx = to_np(out["idx"])
    n_bad = int((got_idx != ref["idx"]).any(axis=-1).sum())
    announce("  %d x %d heads, %d tokens each: %d tokens with differing indices"
             % (w.B, w.H, w.L, n_bad))
    np.testing.assert_array_equal(got_idx, ref["idx"])
    e = slice_rel_err(to_np(out["Y"]), ref["Y"])
    announce("  Y error %.3g (max over heads)" % e)
    assert e <= TOL["bf16"]
    del inp, out, host, ref
    torch.cuda.empty_cache()


def test_ssc_segment_offsets_full_size():
    # the SSC workload's shape with random boundaries, as many segments as its constant length
    # gives (mc_scan_prefill_segs + mc_ssc_readout_segs, the routed read); every head against
    # the oracle, indices of every token exactly
    w = WORKLOADS["ssc_bf16_L16K_k4"]
    n = -(-w.L // w.seg_len)
    cuts = np.sort(np.random.default_rng(21).choice(np.arange(1, w.L), n - 1, replace=False))
    off = [0] + cuts.tolist() + [w.L]
    announce("full-size SSC with offsets: B=%d H=%d L=%d, %d segments, k=%d"
             % (w.B, w.H, w.L, n, w.top_k))
    inp = make_prefill_device(w, seed=2)
    d = mc.make_dims(w.B, w.H, w.L, w.d_k, w.d_v, w.d_g, 1, w.x_heads, w.dtype, w.phi)
    out = mc.prefill_ssc_segs(d, off, w.top_k, inp["Q"], inp["K"], inp["V"], inp["U"],
                              inp["X"])
    torch.cuda.synchronize()
    host = {k: v.to(torch.float64).cpu().numpy() for k, v in inp.items()}
    ref = oracle.prefill(host["Q"], host["K"], host["V"], host["U"], host["X"], seg_len=1,
                         phi=w.phi, mode="ssc", top_k=w.top_k, seg_offsets=off)
    got_idx = to_np(out["idx"])
    n_bad = int((got_idx != ref["idx"]).any(axis=-1).sum())
    announce("  %d tokens with differing indices" % n_bad)
    np.testing.assert_array_equal(got_idx, ref["idx"])
    e = slice_rel_err(to_np(out["Y"]), ref["Y"])
    announce("  Y error %.3g (max over heads)" % e)
    assert e <= TOL["bf16"]
    del inp, out, host, ref
    torch.cuda.empty_cache()


def test_decode_full_size():
    """One step of the 64-sequence x 32-head, 256-cached-state workload (no emission), then
    a step that closes the online segment (emission into slot 256) on the same cache."""
    w = WORKLOADS["decode_bf16_64x32_n256"]
    announce("full-size decode: B=%d H=%d n_cached=%d count_on=%d" % (w.B, w.H, w.n_cached,
                                                                       w.count_on))
    di = make_decode_device(w, seed=0)
    cap = di["n_cap"]
    d = mc.make_dims(w.B, w.H, 1, w.d_k, w.d_v, w.d_g, w.seg_len, 1, w.dtype, w.phi)
    ws = mc.workspace(d, mc.MC_OP_DECODE, n_cap=cap)
    sample = [(0, 0), (63, 31), (17, 5)]

    def host_state(b, h, count):
        return oracle.DecodeState(
            di["M_on"][b:b + 1, h:h + 1].double().cpu().numpy(),
            di["xsum"][b:b + 1].double().cpu().numpy(), count,
            di["M_cache"][b:b + 1, h:h + 1].double().cpu().numpy(),
            di["P_cache"][b:b + 1].double().cpu().numpy(), int(nc[0]))

    def tok(b, h):
        return [di[k][b:b + 1, h:h + 1].double().cpu().numpy() for k in ("q", "k", "v", "u")] + \
               [di["x"][b:b + 1].double().cpu().numpy()]

    # the second step continues from the online state the first one left
    for count in (w.count_on, w.seg_len - 1):
        nc = np.array([w.n_cached], np.int32)
        cnt = np.array([count], np.int32)
        states = {bh: host_state(*bh, count) for bh in sample}
        y = torch.empty((w.B, w.H, w.d_v), dtype=torch.bfloat16, device="cuda")
        mc.mc_decode_step(d, di["q"], di["k"], di["v"], di["u"], di["x"], di["M_on"], di["xsum"],
                          cnt, di["M_cache"], di["P_cache"], nc, cap, y, ws=ws)
        torch.cuda.synchronize()
        emitted = count + 1 == w.seg_len
        assert int(nc[0]) == w.n_cached + emitted and int(cnt[0]) == (0 if emitted else count + 1)
        for (b, h), st in states.items():
            yref = oracle.decode_step(st, *tok(b, h), seg_len=w.seg_len, phi=w.phi)
            e = slice_rel_err(to_np(y[b:b + 1, h:h + 1]), yref)
            announce("  count_on=%d (b=%d, h=%d): y error %.3g" % (count, b, h, e))
            assert e <= TOL["bf16"]
            if emitted:
                got = to_np(di["M_cache"][b:b + 1, h:h + 1, w.n_cached])
                assert slice_rel_err(got, st.M_cache[:, :, w.n_cached], lead=2) <= TOL["bf16"]
                assert slice_rel_err(to_np(di["P_cache"][b:b + 1, :, w.n_cached]),
                                     st.P_cache[:, :, w.n_cached], lead=2) <= 1e-5
                assert float(di["M_on"][b, h].abs().max()) == 0.0
            else:
                assert slice_rel_err(to_np(di["M_on"][b:b + 1, h:h + 1]), st.M_on) <= 1e-5
    del di
    torch.cuda.empty_cache()


@pytest.mark.parametrize("calls", ["two_calls", "one_call"])
def test_log_segments_full_size(calls):
    # the logarithmic segmentation at the L=64K workload's shape, L = 65535 (16 segments):
    # mc_scan_prefill_segs + mc_grm_readout_segs, and mc_grm_prefill_segs as the benchmark
    # times it (the read forms the online term over the 512-token pieces of the long segments)
    w = WORKLOADS["grm_bf16_L64K"]
    L = 65535
    off = oracle.log_segments(L)
    announce("full-size log segmentation (%s): H=%d L=%d, %d segments"
             % (calls, w.H, L, len(off) - 1))
    inp = make_prefill_device(w, seed=0, L=L)
    d = mc.make_dims(w.B, w.H, L, w.d_k, w.d_v, w.d_g, 1, 1, w.dtype, w.phi)
    run = mc.prefill_grm_segs if calls == "two_calls" else mc.prefill_grm_segs_onecall
    out = run(d, off, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"])
    torch.cuda.synchronize()
    assert torch.isfinite(out["Y"].float()).all()
    # segment boundaries, the ends and starts of the 512-token pieces of the longest segment,
    # seeded random rows
    rows = np.unique(np.concatenate([np.array(off[1:-1]) - 1, np.array(off[1:-1]),
                                     np.arange(511, off[1], 512), np.arange(512, off[1], 512),
                                     np.random.default_rng(11).integers(0, L, 200)])
                     ).astype(np.int32)
    for b, h in [(0, 0), (0, 17)]:
        hin = _head(inp, b, h)
        ref = oracle.prefill(hin["Q"], hin["K"], hin["V"], hin["U"], hin["X"], seg_len=1,
                             phi=w.phi, rows=rows, want_states=True, seg_offsets=off)
        errs = {"Y": slice_rel_err(to_np(out["Y"][b:b + 1, h:h + 1, rows]), ref["Y"]),
                "M": slice_rel_err(to_np(out["M"][b:b + 1, h:h + 1]), ref["M"]),
                "P": slice_rel_err(to_np(out["P"][b:b + 1]), ref["P"])}
        announce("  (b=%d, h=%d) %d rows: %s" % (b, h, len(rows), errs))
        assert errs["Y"] <= TOL["bf16"] and errs["M"] <= 1e-4 and errs["P"] <= 1e-4


def test_swla_full_size():
    # SWLA memory at the L=64K workload's shape (C = 512), as the benchmark times it:
    # mc_scan_prefill_swla (MFMA scan) + mc_grm_readout with the scan's online read
    w = WORKLOADS["grm_bf16_L64K"]
    announce("full-size SWLA: H=%d L=%d C=%d" % (w.H, w.L, w.seg_len))
    inp = make_prefill_device(w, seed=0)
    g = make_swla_gates_device(w.B, w.H, w.L, seed=1)
    d = mc.make_dims(w.B, w.H, w.L, w.d_k, w.d_v, w.d_g, w.seg_len, 1, w.dtype, w.phi)
    out = mc.prefill_grm_swla(d, g["alpha"], g["beta"], g["lam"], inp["Q"], inp["K"], inp["V"],
                              inp["U"], inp["X"])
    torch.cuda.synchronize()
    assert torch.isfinite(out["Y"].float()).all()
    C = w.seg_len
    rows = np.unique(np.concatenate([np.arange(C - 1, w.L, C), np.arange(0, w.L, C) + 63,
                                     np.random.default_rng(12).integers(0, w.L, 200)])
                     ).astype(np.int32)
    for b, h in [(0, 0), (0, 23)]:
        hin = _head(inp, b, h)
        gates = tuple(g[k][b:b + 1, h:h + 1].double().cpu().numpy()
                      for k in ("alpha", "beta", "lam"))
        ref = oracle.prefill(hin["Q"], hin["K"], hin["V"], hin["U"], hin["X"], seg_len=C,
                             phi=w.phi, rows=rows, want_states=True, swla=gates)
        errs = {"Y": slice_rel_err(to_np(out["Y"][b:b + 1, h:h + 1, rows]), ref["Y"]),
                "M": slice_rel_err(to_np(out["M"][b:b + 1, h:h + 1]), ref["M"]),
                "P": slice_rel_err(to_np(out["P"][b:b + 1]), ref["P"])}
        announce("  (b=%d, h=%d) %d rows: %s" % (b, h, len(rows), errs))
        assert errs["Y"] <= TOL["bf16"] and errs["M"] <= TOL["bf16"] and errs["P"] <= 1e-4
    del inp, out
    torch.cuda.empty_cache()


def _backward_inputs(w, seed):
    inp = make_prefill_device(w, seed=seed)
    dY = torch.from_numpy(make_upstream_grad(w.B, w.H, w.L, w.d_v, seed=seed + 1,
                                             dtype=w.dtype)).cuda().to(torch.bfloat16)
    d = _dims(w)
    fwd = mc.prefill_grm(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], online=False)
    got = mc.grm_backward(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], fwd["M"],
                          fwd["M_lo"], fwd["P"], dY)
    torch.cuda.synchronize()
    return inp, dY, fwd, got


def test_backward_full_size_L4K():
    # every gradient of every head of the L=4K workload (B=4, H=16, C=256, elu+1) against
    # the oracle, in the launch configuration the benchmark times
    w = WORKLOADS["grm_bf16_L4K_elu"]
    announce("full-size backward %s: B=%d H=%d L=%d C=%d" % (w.name, w.B, w.H, w.L, w.seg_len))
    inp, dY, fwd, got = _backward_inputs(w, seed=2)
    host = {k: v.to(torch.float64).cpu().numpy() for k, v in inp.items()}
    ref = oracle.grm_backward(host["Q"], host["K"], host["V"], host["U"], host["X"],
                              dY.to(torch.float64).cpu().numpy(), seg_len=w.seg_len, phi=w.phi)
    errs = {k: slice_rel_err(to_np(got[k]), ref[k]) for k in ("dQ", "dK", "dV", "dU", "dX")}
    announce("  errors %s" % errs)
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)
    del inp, dY, fwd, got
    torch.cuda.empty_cache()


def test_backward_full_size_L64K():
    # the L=64K workload: per-token gradients (dQ, dU) at sampled rows of two heads against
    # the oracle, and for the whole input Euler's identity for the inputs Y is linear in
    # (V, and with phi = identity Q and K): sum(dV*V) = sum(dQ*Q) = sum(dK*K) = sum(dY*Y)
    w = WORKLOADS["grm_bf16_L64K"]
    announce("full-size backward %s: H=%d L=%d C=%d" % (w.name, w.H, w.L, w.seg_len))
    inp, dY, fwd, got = _backward_inputs(w, seed=3)
    assert all(torch.isfinite(v).all() for v in got.values())
    Y = torch.empty((w.B, w.H, w.L, w.d_v), dtype=torch.bfloat16, device="cuda")
    d = _dims(w)
    mc.mc_grm_readout(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], fwd["M"],
                      fwd["M_lo"], fwd["P"], None, Y, None,
                      ws=mc.workspace(d, mc.MC_OP_GRM), stream=None)
    torch.cuda.synchronize()

    def dot(a, b):
        return float((a.double() * b.double()).sum())
    ref = dot(dY, Y)
    # rounding errors (bf16 Y and states) enter every term with its own sign, so the scale of
    # the deviation is the root of the summed squares, not the sum of magnitudes
    scale = float(((dY.double() * Y.double()) ** 2).sum().sqrt())
    for k, x in (("dV", inp["V"]), ("dQ", inp["Q"]), ("dK", inp["K"])):
        e = abs(dot(got[k], x) - ref) / scale
        announce("  sum(%s*%s) = %.6g, sum(dY*Y) = %.6g, deviation / rms scale %.3g"
                 % (k, k[1:], dot(got[k], x), ref, e))
        assert e <= TOL["bf16"], (k, e)
    rows = _sample_rows(w.L, w.seg_len, 128, seed=13)
    for b, h in [(0, 0), (0, 29)]:
        hin = _head(inp, b, h)
        r = oracle.grm_backward(hin["Q"], hin["K"], hin["V"], hin["U"], hin["X"],
                                dY[b:b + 1, h:h + 1].to(torch.float64).cpu().numpy(),
                                seg_len=w.seg_len, phi=w.phi, rows=rows)
        errs = {k: slice_rel_err(to_np(got[k][b:b + 1, h:h + 1, rows]), r[k]) for k in ("dQ", "dU")}
        announce("  (b=%d, h=%d) %d rows: %s" % (b, h, len(rows), errs))
        for k, e in errs.items():
            assert e <= TOL["bf16"], (k, e)
    del inp, dY, fwd, got, Y
    torch.cuda.empty_cache()


def test_backward_split_dm_walk():
    # The dM / dP walk cuts the token axis into ranges of 128 chunks of 64 tokens (8192
    # tokens); each group of four cached segments gets one workgroup per range that holds
    # some of its later tokens, and their partial sums are added into dM and dP.  At
    # L = 20480, C = 512 the first four groups span 3 ranges, the next four 2, so every
    # gradient, compared element by element with the oracle, depends on the split sums.  The
    # fp32 states are not passed (M = NULL): the bf16 call reads only their bf16 copy.
    from chunked_linear_attention_segment_amd.inputs import Workload
    w = Workload("bwd_split", 1, 2, 20480, 128, 128, 128, 512, "identity", "bf16",
                 recipe="l2norm")
    items = [len({c // 128 for c in range((i0 + 1) * w.seg_len // 64, -(-w.L // 64))})
             for i0 in range(0, 40, 4)]
    assert items == [3, 3, 3, 3, 2, 2, 2, 2, 1, 1]
    announce("backward, split dM walk: B=%d H=%d L=%d C=%d" % (w.B, w.H, w.L, w.seg_len))
    inp = make_prefill_device(w, seed=4)
    dY = torch.from_numpy(make_upstream_grad(w.B, w.H, w.L, w.d_v, seed=5,
                                             dtype=w.dtype)).cuda().to(torch.bfloat16)
    d = _dims(w)
    fwd = mc.prefill_grm(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], online=False)
    got = mc.grm_backward(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], None,
                          fwd["M_lo"], fwd["P"], dY)
    torch.cuda.synchronize()
    host = {k: v.to(torch.float64).cpu().numpy() for k, v in inp.items()}
    ref = oracle.grm_backward(host["Q"], host["K"], host["V"], host["U"], host["X"],
                              dY.to(torch.float64).cpu().numpy(), seg_len=w.seg_len, phi=w.phi)
    errs = {k: slice_rel_err(to_np(got[k]), ref[k]) for k in ("dQ", "dK", "dV", "dU", "dX")}
    announce("  errors %s" % errs)
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)
    # two calls sum the split partials in different orders; they agree to fp32 rounding
    again = mc.grm_backward(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], None,
                            fwd["M_lo"], fwd["P"], dY)
    torch.cuda.synchronize()
    for k in ("dK", "dV", "dX"):
        assert slice_rel_err(to_np(again[k]), to_np(got[k])) <= 1e-4, k
    del inp, dY, fwd, got, again
    torch.cuda.empty_cache()
