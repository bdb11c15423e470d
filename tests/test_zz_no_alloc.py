"""mc_decode_step_noalloc (the decode step on the library's fixed per-GPU scratch buffer)
against mc_decode_step (the same kernels on a caller workspace), through the C ABI.

Two calls in a row on the same GPU, the second on a smaller input (fewer sequences, heads and
cached states), so it runs on a scratch buffer that still holds the first call's partial
softmaxes.  Both entry points run the same kernels on the same inputs, so every output --
y, the online state, the x sum, the emitted cache slot and mean, the host counters -- must
be identical.  One oracle head per call pins the shared result to the definition as well.
"""
import numpy as np
import pytest

import oracle
from chunked_linear_attention_segment_amd.inputs import Workload, make_decode_device
from mcutil import TOL, announce, slice_rel_err, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import chunked_linear_attention_segment_amd as mc  # noqa: E402

# (workload, seed): the first closes its online segment (emission into slot n_cached), the
# second is smaller and does not
CALLS = [
    (Workload("noalloc_a", 16, 8, 1, 128, 128, 128, 64, "identity", "bf16", recipe="l2norm",
              op="decode", n_cached=40, count_on=63), 21),
    (Workload("noalloc_b", 3, 2, 1, 128, 128, 128, 64, "elu1", "bf16", recipe="l2norm",
              op="decode", n_cached=9, count_on=10), 22),
]


def _clone(di):
    return {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in di.items()}


def test_noalloc_decode_matches_workspace_entry_point():
    for w, seed in CALLS:
        announce("noalloc decode: B=%d H=%d n_cached=%d count_on=%d phi=%s"
                 % (w.B, w.H, w.n_cached, w.count_on, w.phi))
        di = make_decode_device(w, seed=seed)
        cap = di["n_cap"]
        d = mc.make_dims(w.B, w.H, 1, w.d_k, w.d_v, w.d_g, w.seg_len, 1, w.dtype, w.phi)
        host = {"M_on": di["M_on"][:1, :1].double().cpu().numpy(),
                "xsum": di["xsum"][:1].double().cpu().numpy(),
                "M_cache": di["M_cache"][:1, :1].double().cpu().numpy(),
                "P_cache": di["P_cache"][:1].double().cpu().numpy()}
        ref_state = _clone(di)
        ref_cnt = np.array([w.count_on], np.int32)
        ref_nc = np.array([w.n_cached], np.int32)
        y_ref = torch.empty((w.B, w.H, w.d_v), dtype=torch.bfloat16, device="cuda")
        mc.mc_decode_step(d, di["q"], di["k"], di["v"], di["u"], di["x"], ref_state["M_on"],
                          ref_state["xsum"], ref_cnt, ref_state["M_cache"],
                          ref_state["P_cache"], ref_nc, cap, y_ref,
                          ws=mc.workspace(d, mc.MC_OP_DECODE, n_cap=cap))
        cnt = np.array([w.count_on], np.int32)
        nc = np.array([w.n_cached], np.int32)
        y = torch.empty((w.B, w.H, w.d_v), dtype=torch.bfloat16, device="cuda")
        mc.mc_decode_step_noalloc(d, di["q"], di["k"], di["v"], di["u"], di["x"], di["M_on"],
                                  di["xsum"], cnt, di["M_cache"], di["P_cache"], nc, cap, y)
        torch.cuda.synchronize()
        emitted = w.count_on + 1 == w.seg_len
        assert (int(cnt[0]), int(nc[0])) == (int(ref_cnt[0]), int(ref_nc[0]))
        assert int(nc[0]) == w.n_cached + emitted
        assert torch.equal(y, y_ref)
        for k in ("M_on", "xsum", "M_cache", "P_cache"):
            assert torch.equal(di[k], ref_state[k]), k
        # head (0, 0) against the oracle
        st = oracle.DecodeState(host["M_on"], host["xsum"], w.count_on, host["M_cache"],
                                host["P_cache"], w.n_cached)
        tok = [di[k][:1, :1].double().cpu().numpy() for k in ("q", "k", "v", "u")] + \
              [di["x"][:1].double().cpu().numpy()]
        yref = oracle.decode_step(st, *tok, seg_len=w.seg_len, phi=w.phi)
        e = slice_rel_err(to_np(y[:1, :1]), yref)
        announce("  identical to the workspace entry point; head (0,0) vs oracle %.3g" % e)
        assert e <= TOL["bf16"]
        del di, ref_state, y, y_ref
    torch.cuda.empty_cache()
