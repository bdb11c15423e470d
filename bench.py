"""Benchmark of the Memory Caching hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--only LEG]

A step is one GRM prefill of the L=64K workload (B=1, H=32, d=128, segment 512, bf16
inputs, fp32 accumulation): mc_scan_prefill (per-segment scan: cached states and means)
followed by mc_grm_readout (online read inside each segment, gate, gamma-weighted read of
every cached state), with all inputs resident in HBM.  Prints one JSON line; `value` is
prefill tokens/s over the K timed steps (wall clock between two synchronisations).  The same
line carries the other workloads (the L=512 fp32 and L=4K bf16 GRM prefills, the L=16K SSC
prefill, the decode step of the 64x32-sequence, 256-cached-state workload, the logarithmic
segmentation, the SWLA memory, the backward), the roofline of the dominant kernel and the
fp64 oracle's CPU rate.  Per-call times are HIP events on the launch stream; the reported
figure is their median.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
METRIC = "MC-GRM prefill tokens/s (L=64K,H=32,d=128); decode cached-state HBM GB/s"


def readout_flops(B, H, L, C, dk, dv, dg, online=True):
    """Algorithmic FLOPs of the GRM read of one prefill: per (b,h), every token of segment s
    reads s cached states (2*dk*dv each) and forms s+1 gate logits (2*dg each); when the read
    also forms the online term (online=True: O_on = NULL), each token adds 2*(dk+dv) per key
    of its segment up to itself (causal pairs only)."""
    N = -(-L // C)
    read = 0
    gate = 0
    pairs = 0
    for s in range(N):
        n_tok = min(C, L - s * C)
        read += n_tok * s * 2 * dk * dv
        gate += n_tok * (s + 1) * 2 * dg
        pairs += n_tok * (n_tok + 1) // 2
    return B * H * (read + gate + (pairs * 2 * (dk + dv) if online else 0))


def scan_flops(B, H, L, C, dk, dv):
    """State emit (2*dk*dv per token) + causal online read inside each segment
    (2*dk + 2*dv per token pair r <= t in the same segment)."""
    N = -(-L // C)
    pairs = 0
    for s in range(N):
        n = min(C, L - s * C)
        pairs += n * (n + 1) // 2
    return B * H * (L * 2 * dk * dv + pairs * 2 * (dk + dv))


def decode_bytes(B, H, n, dk, dv, dg, elt):
    """Algorithmic HBM bytes of one decode step: every cached state once, the online state
    read and written, the cached means once per sequence."""
    return B * H * n * dk * dv * elt + B * H * dk * dv * 4 * 2 + B * n * dg * 4


def step_flops(B, H, L, C, dk, dv, dg):
    """Algorithmic FLOPs of a whole GRM prefill step (scan + read with the online term formed
    in the read): the state emit (2*dk*dv per token) plus readout_flops(online=True)."""
    return B * H * L * 2 * dk * dv + readout_flops(B, H, L, C, dk, dv, dg, online=True)


def ssc_step_work(B, H, L, C, d, dg, k):
    """Algorithmic FLOPs and HBM bytes of an SSC prefill step: the state emit, the online term
    (2*(dk+dv) per causal pair of a segment), s+1 gate logits per token and the top-k read
    (2*d*d per selected state, min(k, s) of them); bytes: Q, K, V, U read and Y written once
    (bf16), X read once per sequence, the fp32 and bf16 states, the means and the indices
    written."""
    N = -(-L // C)
    pairs = read = gate = 0
    for s in range(N):
        n = min(C, L - s * C)
        pairs += n * (n + 1) // 2
        read += n * min(k, s) * 2 * d * d
        gate += n * (s + 1) * 2 * dg
    fl = B * H * (L * 2 * d * d + pairs * 4 * d + gate + read)
    by = B * H * L * (2 * d * 2 + 2 * d + 2 * dg + 2 * d + 4 * k) + B * L * dg * 2 + \
        B * H * N * d * d * 6 + B * N * dg * 4
    return fl, by


def timed_calls(fns, steps, warmup, stream):
    """Run the callables in order `warmup` times, then `steps` times with a HIP event pair
    around each on `stream`; returns, per callable, the list of event times (ms) and the wall
    time of the timed steps (ms per step)."""
    import torch
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in fns] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        for j, f in enumerate(fns):
            ev[i][j][0].record(stream)
            f()
            ev[i][j][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return [[ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(steps)]
            for j in range(len(fns))], wall


def med(x):
    return float(np.median(np.asarray(x)))


# The sources each stored traffic figure depends on (the call's kernels and what they include)
CALL_SOURCES = {
    "grm_readout": ["abi.cpp", "common.cuh", "mc_internal.h", "gate.hip", "read_mfma.hip",
                    "readout.hip"],
    "decode_step": ["abi.cpp", "common.cuh", "mc_internal.h", "decode.hip"],
    "ssc_readout": ["abi.cpp", "common.cuh", "mc_internal.h", "readout.hip", "ssc_gather.hip"],
}
# the kernels of each call, by name fragment, as rocprofv3 lists them
CALL_KERNELS = {
    "grm_readout": ["xps_kernel", "xps_group_kernel", "pfrag_kernel", "gate_w_kernel",
                    "grm_read_kernel"],
    "decode_step": ["decode_read_kernel", "decode_combine_kernel"],
    "ssc_readout": ["aon_kernel", "seg_mean64_kernel", "ssc_select", "frag_states_kernel",
                    "ssc_gather_kernel"],
}


def src_hash(files):
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(ROOT, "chunked_linear_attention_segment_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(call: str, workload: str):
    """HBM bytes per call from the committed rocprofv3 counter summary, if it was taken on the
    call's current kernel sources (else None).  The value is a stored profile figure, not a
    measurement of this run; the JSON line says so next to it."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
        ent = rec.get(call, {}).get(workload)
        if ent and ent.get("src_hash") == src_hash(CALL_SOURCES[call]):
            return ent["bytes_per_launch"]
    except Exception:
        return None
    return None


def counters_summary(root: str, calib_mib: int) -> None:
    """Write profiles/traffic.json from rocprofv3 counter runs under `root`: one directory per
    (counter, run) named fetch_<run> / write_<run>, runs prefill, decode, ssc and calib (the
    copy kernel of calib_mib MiB).  Per kernel, the mean FETCH_SIZE / WRITE_SIZE (KiB) per
    dispatch, scaled by what the copy kernel reads for its known bytes; per call, the sum over
    its kernels (each runs once per call)."""
    import csv
    import glob

    def per_kernel(run):
        disp = {}
        for f in glob.glob(os.path.join(root, run, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                k = disp.setdefault(r["Kernel_Name"], {})
                k[r["Dispatch_Id"]] = k.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return {n: sum(v.values()) / len(v) for n, v in disp.items()}

    n = calib_mib << 20
    cf, cw = per_kernel("fetch_calib"), per_kernel("write_calib")
    copy = [k for k in cf if "copy16" in k][0]
    fetch_factor, write_factor = n / (cf[copy] * 1024), n / (cw[copy] * 1024)
    out = {"calibration": {"kernel": "libmcpeak copy16_kernel, %d MiB read + %d MiB written"
                           % (calib_mib, calib_mib),
                           "fetch_factor": fetch_factor, "write_factor": write_factor}}
    for call, run, workload in (("grm_readout", "prefill", "grm_bf16_L64K"),
                                ("decode_step", "decode", "decode_bf16_64x32_n256"),
                                ("ssc_readout", "ssc", "ssc_bf16_L16K_k4")):
        f, w = per_kernel("fetch_" + run), per_kernel("write_" + run)
        kern = {}
        for name in f:
            if any(frag in name for frag in CALL_KERNELS[call]) and name in w:
                short = name.replace("(anonymous namespace)::", "").split("(")[0]
                short = short.replace("void ", "")
                kern[short] = {"fetch_kib": f[name], "write_kib": w[name],
                               "bytes": f[name] * 1024 * fetch_factor + w[name] * 1024 * write_factor}
        out[call] = {workload: {"kernels": kern,
                                "bytes_per_launch": sum(k["bytes"] for k in kern.values()),
                                "src_hash": src_hash(CALL_SOURCES[call])}}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


TRAFFIC_SOURCE = ("stored, not measured in this run: profiles/traffic.json (rocprofv3 FETCH_SIZE "
                  "and WRITE_SIZE per launch, scaled by a copy kernel of known size), used only "
                  "while the kernel sources hash to the value recorded there")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-peak", action="store_true",
                    help="skip the in-run ceilings (bf16 MFMA loop, HBM streaming read)")
    ap.add_argument("--cpu-rows", type=int, default=32768)
    ap.add_argument("--online", choices=["scan", "fused"], default="fused",
                    help="where the online read M_t^(s) phi(q_t) is formed: written by the scan "
                         "and read back (scan), or inside the gated read from K and V (fused)")
    ap.add_argument("--no-segs", action="store_true",
                    help="skip the logarithmic-segmentation prefill line")
    ap.add_argument("--no-swla", action="store_true",
                    help="skip the SWLA-memory prefill line")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward (training) lines")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the L=512 fp32, L=4K bf16 and L=16K SSC prefill lines")
    ap.add_argument("--only", choices=["all", "prefill", "small", "ssc", "decode", "segs", "swla",
                                       "backward"],
                    default="all",
                    help="profiling aid: run only one workload (the JSON line then lacks the "
                         "other part)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="profiling aid: copy a MIB-sized device buffer 3 times and exit (the "
                         "reference kernel for scaling HBM byte counters)")
    ap.add_argument("--counters-summary", metavar="DIR",
                    help="write profiles/traffic.json from the rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE runs under DIR (fetch_<run>, write_<run> for prefill, "
                         "decode, ssc and calib, the copy kernel of --calibrate-copy MiB) and "
                         "exit")
    args = ap.parse_args()
    if args.counters_summary:
        counters_summary(args.counters_summary, args.calibrate_copy or 1024)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import chunked_linear_attention_segment_amd as mc
    from chunked_linear_attention_segment_amd.inputs import (WORKLOADS, make_decode_device,
                                                             make_prefill_device)

    torch.cuda.set_device(0)
    dev = "cuda"
    if args.calibrate_copy:
        from chunked_linear_attention_segment_amd import peak
        n = args.calibrate_copy << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            peak.copy(a, b, n)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return
    if args.only in ("small", "ssc", "decode", "segs", "swla", "backward"):
        rec = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup}
        {"small": run_small, "ssc": run_ssc, "decode": run_decode, "segs": run_log_segments,
         "swla": run_swla, "backward": run_backward}[args.only](args, rec, dev)
        print(json.dumps(rec), flush=True)
        return
    w = WORKLOADS["grm_bf16_L64K"]
    B, H, L, C, dk, dv, dg = w.B, w.H, w.L, w.seg_len, w.d_k, w.d_v, w.d_g
    d = mc.make_dims(B, H, L, dk, dv, dg, C, 1, w.dtype, w.phi)
    inp = make_prefill_device(w, seed=0, device=dev)
    M, M_lo, P, O_on = mc.alloc_prefill(d, dev, online=(args.online == "scan"))
    Y = torch.empty((B, H, L, dv), dtype=torch.bfloat16, device=dev)
    ws = mc.workspace(d, mc.MC_OP_GRM, device=dev)
    stream = torch.cuda.current_stream()

    def scan():
        mc.mc_scan_prefill(d, inp["Q"], inp["K"], inp["V"], inp["X"], M, M_lo, P, O_on,
                           stream=stream)

    def read():
        mc.mc_grm_readout(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], M, M_lo, P, O_on,
                          Y, None, ws=ws, stream=stream)

    # K timed steps between two synchronisations (wall clock: `value`), with a HIP event pair
    # around each call on the launch stream (per-call medians: the roofline)
    (scan_t, read_t), ms_per_step = timed_calls([scan, read], args.steps, args.warmup, stream)
    scan_ms, read_ms = med(scan_t), med(read_t)
    tokens_per_s = B * L / (ms_per_step / 1e3)

    fl_read = readout_flops(B, H, L, C, dk, dv, dg, online=(args.online == "fused"))
    fl_step = step_flops(B, H, L, C, dk, dv, dg)
    achieved = fl_read / (read_ms / 1e3) / 1e12
    traffic = load_traffic("grm_readout", w.name)
    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded device draw: q,k unit-norm, v,x ~ N(0,1), u = x W_u)",
        "config": {"workload": w.name, "B": B, "H": H, "L": L, "d_k": dk, "d_v": dv, "d_g": dg,
                   "seg_len": C, "phi": w.phi, "online_read": args.online,
                   "steps_timed": "mc_scan_prefill + mc_grm_readout"},
        "kernels_ms": {"mc_scan_prefill": round(scan_ms, 4), "mc_grm_readout": round(read_ms, 4),
                       "statistic": "median of %d HIP-event pairs on the launch stream"
                                    % args.steps,
                       "mc_grm_readout_mean": round(float(np.mean(read_t)), 4)},
        "roofline": {"kernel": "mc_grm_readout (prefix sums, gate pass, gamma-weighted read)",
                     "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "traffic_source": TRAFFIC_SOURCE,
                     "algorithmic_flops": fl_read,
                     "step": {"what": "whole step (scan + read), wall clock",
                              "algorithmic_flops": fl_step,
                              "achieved": round(fl_step / (ms_per_step / 1e3) / 1e12, 2)}},
    }
    del M, M_lo, P, O_on, Y, ws, inp
    torch.cuda.empty_cache()

    if not args.no_small and args.only == "all":
        run_small(args, rec, dev)
        run_ssc(args, rec, dev)

    if not args.no_decode and args.only == "all":
        run_decode(args, rec, dev)

    if not args.no_segs and args.only == "all":
        run_log_segments(args, rec, dev)

    if not args.no_swla and args.only == "all":
        run_swla(args, rec, dev)

    if not args.no_backward and args.only == "all":
        run_backward(args, rec, dev)

    if not args.no_peak and args.only == "all":
        measured_peaks(rec)

    if not args.no_cpu and args.only == "all":
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(rec), flush=True)


def measured_peaks(rec):
    """The same rooflines against ceilings measured in this run on this GPU: a bf16 MFMA
    loop from registers on every CU, and a 4 GiB streaming read."""
    from chunked_linear_attention_segment_amd import peak
    mf = peak.mfma_bf16_tflops()
    bw = peak.hbm_read_gbs()
    r = rec["roofline"]
    r["measured_peak"] = round(mf, 1)
    r["frac_of_measured"] = round(r["achieved"] / mf, 4)
    st = r.get("step")
    if st:
        st["frac_of_measured"] = round(st["achieved"] / mf, 4)
    if "decode" in rec:
        rd = rec["decode"]["roofline"]
        rd["measured_peak"] = round(bw, 1)
        rd["frac_of_measured"] = round(rd["achieved"] / bw, 4)
    for leg in rec.get("small", {}).values():
        rl = leg["roofline"]
        if rl["bound"] == "mfma":
            rl["measured_peak"] = round(mf, 1)
            rl["frac_of_measured"] = round(rl["achieved"] / mf, 4)
    if "ssc" in rec:
        rl = rec["ssc"]["roofline"]
        t_min = max(rl["algorithmic_flops"] / (mf * 1e12), rl["algorithmic_bytes"] / (bw * 1e9))
        rl["frac_of_measured"] = round(t_min / (rec["ssc"]["ms_per_step"] / 1e3), 4)
    rec["measured_peaks"] = {"mfma_bf16_tflops": round(mf, 1), "hbm_read_gbs": round(bw, 1),
                             "how": "libmcpeak: 4096 WGs x 4 waves of back-to-back "
                                    "v_mfma_f32_32x32x16_bf16; 4 GiB streaming read"}


def run_small(args, rec, dev):
    """The L=512 fp32 GRM prefill (B=1, H=1, d=64, segment 64; on the fp32 vector kernels, a
    latency-bound size) and the L=4K bf16 GRM prefill (B=4, H=16, d=128, segment 256, elu+1),
    each as scan + read with the online term formed in the read; tokens/s of the step and the
    roofline of the read call (bf16 MFMA) or of the step (fp32 vector units)."""
    import torch

    import chunked_linear_attention_segment_amd as mc
    from chunked_linear_attention_segment_amd.inputs import WORKLOADS, make_prefill_device
    stream = torch.cuda.current_stream()
    out = {}
    for name in ("grm_f32_L512", "grm_bf16_L4K_elu"):
        w = WORKLOADS[name]
        B, H, L, C, dk, dv, dg = w.B, w.H, w.L, w.seg_len, w.d_k, w.d_v, w.d_g
        d = mc.make_dims(B, H, L, dk, dv, dg, C, 1, w.dtype, w.phi)
        inp = make_prefill_device(w, seed=0, device=dev)
        M, M_lo, P, O_on = mc.alloc_prefill(d, dev, online=False)
        Y = torch.empty((B, H, L, dv), dtype=mc.torch_dtype(d), device=dev)
        ws = mc.workspace(d, mc.MC_OP_GRM, device=dev)

        def scan():
            mc.mc_scan_prefill(d, inp["Q"], inp["K"], inp["V"], inp["X"], M, M_lo, P, O_on,
                               stream=stream)

        def read():
            mc.mc_grm_readout(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], M, M_lo, P,
                              O_on, Y, None, ws=ws, stream=stream)
        steps = max(args.steps, 20)
        (scan_t, read_t), ms = timed_calls([scan, read], steps, args.warmup, stream)
        fl_read = readout_flops(B, H, L, C, dk, dv, dg, online=True)
        fl_step = step_flops(B, H, L, C, dk, dv, dg)
        if w.dtype == "bf16":
            tf = fl_read / (med(read_t) / 1e3) / 1e12
            roof = {"kernel": "mc_grm_readout", "bound": "mfma", "achieved": round(tf, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / PEAK_BF16_TFLOPS, 4), "algorithmic_flops": fl_read}
        else:
            tf = fl_step / (ms / 1e3) / 1e12
            roof = {"kernel": "whole step (fp32 vector kernels)", "bound": "alu",
                    "achieved": round(tf, 4), "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / PEAK_FP32_TFLOPS, 6), "algorithmic_flops": fl_step}
        out[name] = {"metric": "prefill tokens/s", "value": round(B * L / (ms / 1e3), 1),
                     "unit": "tokens/s", "ms_per_step": round(ms, 4), "steps": steps,
                     "config": {"B": B, "H": H, "L": L, "d_k": dk, "d_v": dv, "d_g": dg,
                                "seg_len": C, "phi": w.phi, "dtype": w.dtype},
                     "kernels_ms": {"mc_scan_prefill": round(med(scan_t), 4),
                                    "mc_grm_readout": round(med(read_t), 4)},
                     "roofline": roof}
        del inp, M, M_lo, P, O_on, Y, ws
        torch.cuda.empty_cache()
    rec["small"] = out


def run_ssc(args, rec, dev):
    """The L=16K SSC prefill (B=2, H=16, d=128, segment 256, top-4): mc_scan_prefill (the
    states and the online term O_on) + mc_ssc_readout (selection, routing of the (token,
    segment) pairs, and the read of the selected states only), inputs resident; tokens/s, and
    the fraction of the binding roofline max(algorithmic FLOPs / MFMA peak, algorithmic bytes /
    HBM bandwidth) (HBM at this size)."""
    import torch

    import chunked_linear_attention_segment_amd as mc
    from chunked_linear_attention_segment_amd.inputs import WORKLOADS, make_prefill_device
    stream = torch.cuda.current_stream()
    w = WORKLOADS["ssc_bf16_L16K_k4"]
    B, H, L, C, dk, dv, dg, k = w.B, w.H, w.L, w.seg_len, w.d_k, w.d_v, w.d_g, w.top_k
    d = mc.make_dims(B, H, L, dk, dv, dg, C, 1, w.dtype, w.phi)
    inp = make_prefill_device(w, seed=0, device=dev)
    M, M_lo, P, O_on = mc.alloc_prefill(d, dev, online=True)
    Y = torch.empty((B, H, L, dv), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((B, H, L, k), dtype=torch.int32, device=dev)
    ws = mc.workspace(d, mc.MC_OP_SSC, top_k=k, device=dev)

    def scan():
        mc.mc_scan_prefill(d, inp["Q"], inp["K"], inp["V"], inp["X"], M, M_lo, P, O_on,
                           stream=stream)

    def read():
        mc.mc_ssc_readout(d, k, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], M, M_lo, P,
                          O_on, Y, idx, ws=ws, stream=stream)
    (scan_t, read_t), ms = timed_calls([scan, read], args.steps, args.warmup, stream)
    fl, by = ssc_step_work(B, H, L, C, dk, dg, k)
    t_min = max(fl / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
    rec["ssc"] = {"workload": w.name, "metric": "SSC prefill tokens/s",
                  "value": round(B * L / (ms / 1e3), 1), "unit": "tokens/s",
                  "ms_per_step": round(ms, 4), "top_k": k,
                  "steps_timed": "mc_scan_prefill + mc_ssc_readout",
                  "kernels_ms": {"mc_scan_prefill": round(med(scan_t), 4),
                                 "mc_ssc_readout": round(med(read_t), 4)},
                  "roofline": {"bound": "hbm" if by / PEAK_HBM_GBS / 1e9 > fl / PEAK_BF16_TFLOPS / 1e12
                               else "mfma",
                               "what": "whole step against max(FLOPs / 2.5 PFLOP/s, bytes / 8 TB/s)",
                               "achieved": round(by / (ms / 1e3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(t_min / (ms / 1e3), 4),
                               "algorithmic_flops": fl, "algorithmic_bytes": by,
                               "traffic_readout": load_traffic("ssc_readout", w.name),
                               "traffic_source": TRAFFIC_SOURCE}}
    # the same shape over random segment boundaries, as many segments as the constant length
    # gives: mc_scan_prefill_segs + mc_ssc_readout_segs (the routed read with the offsets)
    NS = -(-L // C)
    cuts = np.sort(np.random.default_rng(21).choice(np.arange(1, L), NS - 1, replace=False))
    off = [0] + cuts.tolist() + [L]
    ds = mc.make_dims(B, H, L, dk, dv, dg, 1, 1, w.dtype, w.phi)
    wss = mc.workspace_segs(ds, NS, device=dev)
    wsr = mc.workspace(ds, mc.MC_OP_SSC_SEGS, top_k=k, n_cap=NS, device=dev)

    def scan_segs():
        mc.mc_scan_prefill_segs(ds, off, inp["Q"], inp["K"], inp["V"], inp["X"], M, M_lo, P,
                                O_on, ws=wss, stream=stream)

    def read_segs():
        mc.mc_ssc_readout_segs(ds, off, k, inp["Q"], inp["U"], inp["X"], M, M_lo, P, O_on, Y,
                               idx, ws=wsr, stream=stream)
    (scan_s, read_s), ms_s = timed_calls([scan_segs, read_segs], args.steps, args.warmup, stream)
    rec["ssc_offsets"] = {"workload": "%s shape, %d random segment boundaries" % (w.name, NS),
                          "metric": "SSC prefill tokens/s",
                          "value": round(B * L / (ms_s / 1e3), 1), "unit": "tokens/s",
                          "ms_per_step": round(ms_s, 4), "top_k": k,
                          "steps_timed": "mc_scan_prefill_segs + mc_ssc_readout_segs",
                          "kernels_ms": {"mc_scan_prefill_segs": round(med(scan_s), 4),
                                         "mc_ssc_readout_segs": round(med(read_s), 4)}}
    del inp, M, M_lo, P, O_on, Y, idx, ws, wss, wsr
    torch.cuda.empty_cache()


def run_decode(args, rec, dev):
    import torch

    import chunked_linear_attention_segment_amd as mc
    from chunked_linear_attention_segment_amd.inputs import WORKLOADS, make_decode_device
    stream = torch.cuda.current_stream()
    if True:
        wd = WORKLOADS["decode_bf16_64x32_n256"]
        dd = mc.make_dims(wd.B, wd.H, 1, wd.d_k, wd.d_v, wd.d_g, wd.seg_len, 1, wd.dtype, wd.phi)
        di = make_decode_device(wd, seed=0, device=dev)
        cap = di["n_cap"]
        wsd = mc.workspace(dd, mc.MC_OP_DECODE, n_cap=cap, device=dev)
        yd = torch.empty((wd.B, wd.H, wd.d_v), dtype=torch.bfloat16, device=dev)
        M_on0 = di["M_on"].clone()
        xs0 = di["xsum"].clone()

        def dstep(u):
            # the online state is restored before each timed step so every step does identical
            # work; u=None is the post-training (uniform-weight) read
            cnt = np.array([wd.count_on], np.int32)
            nc = np.array([wd.n_cached], np.int32)
            mc.mc_decode_step(dd, di["q"], di["k"], di["v"], u, di["x"], di["M_on"],
                              di["xsum"], cnt, di["M_cache"], di["P_cache"], nc, cap, yd, ws=wsd,
                              stream=stream)

        def timed(u):
            for _ in range(args.warmup):
                di["M_on"].copy_(M_on0)
                di["xsum"].copy_(xs0)
                dstep(u)
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for i in range(args.steps):
                di["M_on"].copy_(M_on0)
                di["xsum"].copy_(xs0)
                ev[i][0].record(stream)
                dstep(u)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            return med([a.elapsed_time(b) for a, b in ev])

        dms = timed(di["u"])
        ams = timed(None)
        by = decode_bytes(wd.B, wd.H, wd.n_cached, wd.d_k, wd.d_v, wd.d_g, 2)
        by_avg = by - wd.B * wd.n_cached * wd.d_g * 4  # no means are read
        gbs = by / (dms / 1e3) / 1e9
        rec["decode"] = {"workload": wd.name, "metric": "decode cached-state HBM GB/s",
                         "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(dms, 4),
                         "tokens_per_s": round(wd.B / (dms / 1e3), 1),
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(gbs / PEAK_HBM_GBS, 4),
                                      "traffic": load_traffic("decode_step", wd.name),
                                      "algorithmic_bytes": by},
                         "average_read": {"what": "post-training read (u = NULL: uniform weights)",
                                          "ms_per_step": round(ams, 4),
                                          "value": round(by_avg / (ams / 1e3) / 1e9, 1),
                                          "unit": "GB/s"}}
        del di, wsd, yd
        torch.cuda.empty_cache()


def run_log_segments(args, rec, dev):
    """The logarithmic segmentation (one segment per set bit of L, largest first) of the L=64K
    workload's shape at L = 65535 (16 segments of 32768 .. 1 tokens): mc_grm_prefill_segs, the
    one-call prefill (the MFMA scan of the states with the 32768-token segment as pieces, the
    gate pass, and the MFMA read forming the online term over the pieces), inputs resident,
    tokens/s; the two-call form (mc_scan_prefill_segs writing O_on + mc_grm_readout_segs)
    timed beside it."""
    import torch

    import chunked_linear_attention_segment_amd as mc
    from chunked_linear_attention_segment_amd.inputs import WORKLOADS, make_prefill_device
    w = WORKLOADS["grm_bf16_L64K"]
    L = 65535
    off = [0]
    for b in range(L.bit_length() - 1, -1, -1):
        if (L >> b) & 1:
            off.append(off[-1] + (1 << b))
    NS = len(off) - 1
    B, H, dk, dv, dg = w.B, w.H, w.d_k, w.d_v, w.d_g
    d = mc.make_dims(B, H, L, dk, dv, dg, 1, 1, w.dtype, w.phi)
    inp = make_prefill_device(w, seed=0, device=dev, L=L)
    M = torch.empty((B, H, NS, dv, dk), dtype=torch.float32, device=dev)
    M_lo = torch.empty((B, H, NS, dv, dk), dtype=torch.bfloat16, device=dev)
    P = torch.empty((B, 1, NS, dg), dtype=torch.float32, device=dev)
    O_on = torch.empty((B, H, L, dv), dtype=torch.float32, device=dev)
    Y = torch.empty((B, H, L, dv), dtype=torch.bfloat16, device=dev)
    ws = mc.workspace(d, mc.MC_OP_GRM_SEGS, top_k=NS, device=dev)
    wss = mc.workspace_segs(d, NS, device=dev)
    ws1 = mc.workspace(d, mc.MC_OP_GRM_PREFILL_SEGS, top_k=NS, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        mc.mc_grm_prefill_segs(d, off, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], M,
                               M_lo, P, Y, None, ws=ws1, stream=stream)

    def step2():
        mc.mc_scan_prefill_segs(d, off, inp["Q"], inp["K"], inp["V"], inp["X"], M, M_lo, P,
                                O_on, ws=wss, stream=stream)
        mc.mc_grm_readout_segs(d, off, inp["Q"], inp["U"], inp["X"], M, M_lo, P, O_on, Y,
                               None, ws=ws, stream=stream)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return med([a.elapsed_time(b) for a, b in ev])
    ms = timed(step)
    ms2 = timed(step2)
    # algorithmic FLOPs: per token, the state update and online read (4 dk dv), the reads of
    # the completed segments before its own (2 dk dv each) and s + 1 gate logits (2 dg each);
    # algorithmic bytes: Q, K, V, U read and Y written once (bf16), X once per sequence, the
    # states (fp32 + bf16) and means written.  At about 77 FLOP per byte the step is below the
    # bf16 ridge (2.5 PFLOP/s / 8 TB/s), so its roofline is HBM.
    fl = 0
    for s in range(NS):
        n = off[s + 1] - off[s]
        fl += n * (4 * dk * dv + s * 2 * dk * dv + (s + 1) * 2 * dg)
    fl *= B * H
    by = B * H * L * (2 * dk * 2 + 2 * dv * 2 + 2 * dg) + B * L * dg * 2 + \
        B * H * NS * dv * dk * 6 + B * NS * dg * 4
    gbs = by / (ms / 1e3) / 1e9
    rec["log_segments"] = {
        "workload": "grm_bf16_L64K shape at L=65535, logarithmic segmentation (%d segments)"
                    % NS,
        "metric": "prefill tokens/s", "value": round(B * L / (ms / 1e3), 1), "unit": "tokens/s",
        "ms_per_step": round(ms, 4),
        "steps_timed": "mc_grm_prefill_segs",
        "two_calls_ms_per_step": round(ms2, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": by, "algorithmic_flops": fl}}
    del inp, M, M_lo, P, O_on, Y, ws, wss, ws1
    torch.cuda.empty_cache()


def run_swla(args, rec, dev):
    """The SWLA memory (window 2) at the L=64K workload's shape: mc_scan_prefill_swla (the
    decayed scan on MFMA, which also writes the online read) + mc_grm_readout taking that
    online read; inputs and gates resident, tokens/s.  Rooflines: the read against bf16 MFMA
    (its algorithmic FLOPs without the online term, which the scan forms), the scan against
    HBM (its algorithmic bytes)."""
    import torch

    import chunked_linear_attention_segment_amd as mc
    from chunked_linear_attention_segment_amd.inputs import (WORKLOADS, make_prefill_device,
                                                             make_swla_gates_device)
    w = WORKLOADS["grm_bf16_L64K"]
    B, H, L, C, dk, dv, dg = w.B, w.H, w.L, w.seg_len, w.d_k, w.d_v, w.d_g
    d = mc.make_dims(B, H, L, dk, dv, dg, C, 1, w.dtype, w.phi)
    inp = make_prefill_device(w, seed=0, device=dev)
    g = make_swla_gates_device(B, H, L, seed=1, device=dev)
    M, M_lo, P, O_on = mc.alloc_prefill(d, dev, online=True)
    Y = torch.empty((B, H, L, dv), dtype=torch.bfloat16, device=dev)
    ws = mc.workspace(d, mc.MC_OP_GRM, device=dev)
    stream = torch.cuda.current_stream()

    def scan():
        mc.mc_scan_prefill_swla(d, None, g["alpha"], g["beta"], g["lam"], inp["Q"], inp["K"],
                                inp["V"], inp["X"], M, M_lo, P, O_on, stream=stream)

    def read():
        mc.mc_grm_readout(d, inp["Q"], None, None, inp["U"], inp["X"], M, M_lo, P, O_on, Y,
                          None, ws=ws, stream=stream)
    for _ in range(args.warmup):
        scan()
        read()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        scan()
        e[1].record(stream)
        read()
        e[2].record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    scan_ms = med([e[0].elapsed_time(e[1]) for e in ev])
    read_ms = med([e[1].elapsed_time(e[2]) for e in ev])
    fl_read = readout_flops(B, H, L, C, dk, dv, dg, online=False)
    tf = fl_read / (read_ms / 1e3) / 1e12
    NS = -(-L // C)
    # scan bytes: Q, K, V (bf16) and the three gates read; O_on (fp32), the states (fp32 and
    # bf16) and the means written; X read once for the means
    sbytes = B * H * L * (2 * dk * 2 + 2 * dv + 3 * 4 + 4 * dv) + B * H * NS * dv * dk * 6 + \
        B * L * dg * 2 + B * NS * dg * 4
    gbs = sbytes / (scan_ms / 1e3) / 1e9
    rec["swla"] = {
        "workload": "grm_bf16_L64K shape with the SWLA memory (window 2, per-token decay and "
                    "window weights)",
        "metric": "prefill tokens/s", "value": round(B * L / (ms / 1e3), 1), "unit": "tokens/s",
        "ms_per_step": round(ms, 4),
        "steps_timed": "mc_scan_prefill_swla + mc_grm_readout (online read from the scan)",
        "kernels_ms": {"mc_scan_prefill_swla": round(scan_ms, 4),
                       "mc_grm_readout": round(read_ms, 4)},
        "roofline": {"kernel": "mc_grm_readout", "bound": "mfma", "achieved": round(tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "algorithmic_flops": fl_read},
        "scan_roofline": {"kernel": "mc_scan_prefill_swla", "bound": "hbm",
                          "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": sbytes}}
    del inp, g, M, M_lo, P, O_on, Y, ws
    torch.cuda.empty_cache()


def backward_flops(B, H, L, C, dk, dv, dg):
    """Algorithmic FLOPs of the GRM prefill's backward: per (token, cached state read) the
    state read for dgamma, the dq term and the dM term (2*dk*dv each) and the gate logit, du
    and dP terms (2*dg each); per (token, key) pair of the online segment the recomputed
    online read, its dq term and the dv and dk terms (2*(dk+dv) each); per token the cached
    states' gradients applied to k and v (2*dk*dv each)."""
    N = -(-L // C)
    per_state = 0
    pairs = 0
    for s in range(N):
        n = min(C, L - s * C)
        per_state += n * s
        pairs += n * (n + 1) // 2
    return B * H * (per_state * (3 * 2 * dk * dv + 3 * 2 * dg) + pairs * 4 * 2 * (dk + dv)
                    + L * 2 * 2 * dk * dv)


def run_backward(args, rec, dev):
    """The backward of the GRM prefill (training) at the L=4K workload and the L=64K
    workload's shape: forward once, then mc_grm_backward timed with HIP events on its stream
    (inputs, states and dY resident).  tokens/s of the backward alone; algorithmic FLOPs
    against the peak of the units its dense contractions run on."""
    import torch

    import chunked_linear_attention_segment_amd as mc
    from chunked_linear_attention_segment_amd.inputs import (WORKLOADS, make_prefill_device,
                                                             make_upstream_grad)
    out = {}
    for name in ("grm_bf16_L4K_elu", "grm_bf16_L64K"):
        w = WORKLOADS[name]
        B, H, L, C, dk, dv, dg = w.B, w.H, w.L, w.seg_len, w.d_k, w.d_v, w.d_g
        d = mc.make_dims(B, H, L, dk, dv, dg, C, 1, w.dtype, w.phi)
        inp = make_prefill_device(w, seed=0, device=dev)
        dY = torch.from_numpy(make_upstream_grad(B, H, L, dv, seed=1, dtype=w.dtype)).to(
            dev).to(torch.bfloat16)
        fwd = mc.prefill_grm(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], online=False)
        f = dict(dtype=torch.float32, device=dev)
        g = [torch.empty((B, H, L, dk), **f), torch.empty((B, H, L, dk), **f),
             torch.empty((B, H, L, dv), **f), torch.empty((B, H, L, dg), **f),
             torch.empty((B, 1, L, dg), **f)]
        ws = mc.workspace(d, mc.MC_OP_GRM_BACKWARD, device=dev)
        stream = torch.cuda.current_stream()

        def step():
            mc.mc_grm_backward(d, inp["Q"], inp["K"], inp["V"], inp["U"], inp["X"], fwd["M"],
                               fwd["M_lo"], fwd["P"], dY, *g, ws=ws, stream=stream)
        steps = max(1, min(args.steps, 3 if L > 8192 else args.steps))
        for _ in range(min(args.warmup, 1)):
            step()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        ms = med([a.elapsed_time(b) for a, b in ev])
        fl = backward_flops(B, H, L, C, dk, dv, dg)
        tf = fl / (ms / 1e3) / 1e12
        # bf16 with d_k = d_v = 128 runs the dense contractions on MFMA; other shapes on the
        # fp32 vector units
        mfma = w.dtype == "bf16" and dk == 128 and dv == 128
        peak = PEAK_BF16_TFLOPS if mfma else 157.3
        out[name] = {"ms_per_step": round(ms, 3), "tokens_per_s": round(B * L / (ms / 1e3), 1),
                     "steps": steps,
                     "roofline": {"bound": "mfma" if mfma else "alu", "achieved": round(tf, 2),
                                  "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                                  "algorithmic_flops": fl}}
        del inp, dY, fwd, g, ws
        torch.cuda.empty_cache()
    rec["backward"] = {"what": "mc_grm_backward: gradients of Q, K, V, U, X (fp32) from dY",
                       "metric": "backward tokens/s", "workloads": out}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, rows_sample):
    """The fp64 oracle on every host core this process may run on, on a bounded sample of the
    same workload: a group of heads (at most one per thread) runs the full-length scan and
    evaluates `rows_sample` evenly spaced rows; a second run with one row gives the scan's fixed
    cost, and the per-row cost is extrapolated to all L rows and all heads."""
    import torch

    import oracle
    from chunked_linear_attention_segment_amd.inputs import make_prefill_device

    cores = len(os.sched_getaffinity(0))
    Hs = min(cores, w.H)
    inp = make_prefill_device(w, seed=0, device="cuda", H=Hs)
    host = {k: v.to(torch.float64).cpu().numpy() for k, v in inp.items()}
    del inp
    L = w.L
    rows = np.linspace(0, L - 1, rows_sample).astype(np.int32)
    rows = np.unique(rows)
    t0 = time.perf_counter()
    oracle.prefill(host["Q"], host["K"], host["V"], host["U"], host["X"], seg_len=w.seg_len,
                   phi=w.phi, rows=np.array([L - 1], np.int32), n_threads=cores)
    t_scan = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.prefill(host["Q"], host["K"], host["V"], host["U"], host["X"], seg_len=w.seg_len,
                   phi=w.phi, rows=rows, n_threads=cores)
    t_rows = time.perf_counter() - t0
    per_row = max(t_rows - t_scan, 0.0) / len(rows)
    t_full_group = t_scan + per_row * L          # Hs heads, all L rows
    t_full = t_full_group * (w.H / Hs) * w.B
    return {"value": round(w.B * L / t_full, 2), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "threads": "OpenMP, %d threads (every core in this process's affinity set)" % cores,
            "sample": "%d of %d heads, full-length scan, %d evenly spaced rows of %d; scan "
                      "%.2fs + rows %.2fs, extrapolated linearly in rows and heads"
                      % (Hs, w.H, len(rows), L, t_scan, t_rows - t_scan)}


if __name__ == "__main__":
    main()
