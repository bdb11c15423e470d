"""Pins for the fp64 oracle: each checks it against something other than itself.

Every test here runs on the CPU.  The pins are chosen so that a plausible slip in the
oracle (a dropped term, a wrong sign or index, a transposed operand, read-before-update,
an off-by-one segment, the wrong pool) fails at least one of them:

  worked examples   hand-derived values (tests/golden/*.json)
  N = 1             plain causal linear attention (the RNN end point of the segmentation)
  residual          ungated residual memory collapses to plain linear attention for matrix
                    memory (the sum of the segment states is the full state)
  SSC, k >= N-1     equals GRM
  brute force       token-pair form y_t = sum_{r<=t} gamma_t^{seg(r)} (q_t.k_r) v_r, L <= 64
  C = 1             softmax attention with queries u, keys x (torch SDPA)
  segment-constant  block-causal softmax attention over segment keys (torch SDPA)
  U = 0             uniform gate: y_t = LA_t / (s+1)
  soup              Memory Soup equals GRM for linear memory
  invariants        simplex gate, linearity in V, head independence, causality
  decode            prefill(L) + one decode step == last row of prefill(L+1)
  decode, average   LA read / (number of memories); equals the gated step with u = 0
  variable segments brute force with arbitrary boundaries; multiples of C equal the
                    constant-length path; log segmentation of 37 is 32, 4, 1 (the pages' example)
  SWLA              unit gates give the linear-attention memory; token-pair brute force with
                    gate products; alpha = 0 is a two-token window; constant decay is masked
                    attention; soup = GRM
  backward          central differences of the forward oracle (every coordinate); torch
                    autograd of an independent token-pair form
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _phi(z, phi):
    return z if phi == "identity" else np.where(z > 0, z + 1.0, np.exp(np.minimum(z, 0.0)))


def _causal_la(Q, K, V, phi="identity"):
    """Textbook causal unnormalised linear attention, attention form, per (b, h)."""
    qh, kh = _phi(Q, phi), _phi(K, phi)
    L = Q.shape[-2]
    S = qh @ np.swapaxes(kh, -1, -2)
    S = S * np.tril(np.ones((L, L)))
    return S @ V


def _rand(B, H, L, dk, dv, dg, xh=1, seed=0, scale_u=1.0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, L, dk))
    K = rng.standard_normal((B, H, L, dk))
    V = rng.standard_normal((B, H, L, dv))
    U = rng.standard_normal((B, H, L, dg)) * scale_u
    X = rng.standard_normal((B, xh, L, dg))
    return Q, K, V, U, X


def _scalar_case(fix):
    def val(z):
        return {"ln2": math.log(2.0), "ln3": math.log(3.0)}.get(z, z) if isinstance(z, str) else z
    inp = fix["inputs"]
    arr = lambda n: np.array([float(val(z)) for z in inp[n]]).reshape(1, 1, -1, 1)
    return arr("q"), arr("k"), arr("v"), arr("u"), arr("x")


def test_golden_grm_worked_example():
    fix = json.load(open(os.path.join(GOLD, "grm_worked_example.json")))
    q, k, v, u, x = _scalar_case(fix)
    out = oracle.prefill(q, k, v, u, x, seg_len=2, mode="grm", want_states=True)
    np.testing.assert_allclose(out["Y"].ravel(), fix["expected_y"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["M"].ravel(), fix["expected_states"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["P"].ravel(), fix["expected_means"], rtol=0, atol=1e-14)


def test_golden_ssc_tie_worked_example():
    fix = json.load(open(os.path.join(GOLD, "ssc_tie_worked_example.json")))
    q, k, v, u, x = _scalar_case(fix)
    ssc = oracle.prefill(q, k, v, u, x, seg_len=2, mode="ssc", top_k=1)
    np.testing.assert_allclose(ssc["Y"].ravel(), fix["expected_y_ssc"], rtol=0, atol=1e-14)
    assert ssc["idx"][0, 0].tolist() == fix["expected_idx_ssc"]
    grm = oracle.prefill(q, k, v, u, x, seg_len=2, mode="grm")
    np.testing.assert_allclose(grm["Y"].ravel(), fix["expected_y_grm"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("phi", ["identity", "elu1"])
def test_single_segment_is_linear_attention(phi):
    Q, K, V, U, X = _rand(2, 3, 40, 8, 6, 5, seed=1)
    out = oracle.prefill(Q, K, V, U, X, seg_len=40, phi=phi)
    np.testing.assert_allclose(out["Y"], _causal_la(Q, K, V, phi), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C", [1, 3, 8, 16])
def test_residual_collapses_to_linear_attention(C):
    Q, K, V, U, X = _rand(1, 2, 48, 6, 7, 4, seed=2)
    out = oracle.prefill(Q, K, V, U, X, seg_len=C, mode="residual")
    np.testing.assert_allclose(out["Y"], _causal_la(Q, K, V), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("C,k", [(8, 7), (8, 9), (16, 2)])
def test_ssc_with_all_segments_equals_grm(C, k):
    Q, K, V, U, X = _rand(1, 2, 64, 5, 5, 6, seed=3)
    N = 64 // C
    grm = oracle.prefill(Q, K, V, U, X, seg_len=C, mode="grm", want_gamma=True)
    ssc = oracle.prefill(Q, K, V, U, X, seg_len=C, mode="ssc", top_k=k, want_gamma=True)
    if k >= N - 1:
        np.testing.assert_array_equal(ssc["Y"], grm["Y"])
        np.testing.assert_array_equal(ssc["gamma"], grm["gamma"])
        s = np.arange(64) // C
        for t in range(64):
            exp = list(range(min(s[t], k))) + [-1] * (k - min(s[t], k))
            assert ssc["idx"][0, 0, t].tolist() == exp
    else:
        assert not np.allclose(ssc["Y"], grm["Y"])


def _brute(Q, K, V, U, X, C, phi="identity", mode="grm", top_k=0, off=None):
    """Token-pair evaluation with no states: y_t = sum_{r<=t} w_{t,seg(r)} (q_t.k_r) v_r.
    Segments have length C, or are [off[i], off[i+1]) when off is given."""
    B, H, L, _ = Q.shape
    xh = X.shape[1]
    qh, kh = _phi(Q, phi), _phi(K, phi)
    if off is None:
        off = list(range(0, L, C)) + [L]
    seg = np.searchsorted(np.asarray(off), np.arange(L), side="right") - 1
    Y = np.zeros(V.shape)
    IDX = []
    for b in range(B):
        for h in range(H):
            x = X[b, 0 if xh == 1 else h]
            means = [x[off[i]:off[i + 1]].mean(axis=0) for i in range(len(off) - 1)]
            for t in range(L):
                s = int(seg[t])
                scores = [float(U[b, h, t] @ means[i]) for i in range(s)]
                online = float(U[b, h, t] @ x[off[s]:t + 1].mean(axis=0))
                if mode == "ssc":
                    order = sorted(range(s), key=lambda i: (-scores[i], i))
                    chosen = sorted(order[:top_k])
                    IDX.append(chosen + [-1] * (top_k - len(chosen)))
                else:
                    chosen = list(range(s))
                logits = np.array([scores[i] for i in chosen] + [online])
                w = torch.softmax(torch.tensor(logits, dtype=torch.float64), 0).numpy()
                weight = dict(zip(chosen + [s], w))
                for r in range(t + 1):
                    g = weight.get(int(seg[r]), 0.0)
                    Y[b, h, t] += g * float(qh[b, h, t] @ kh[b, h, r]) * V[b, h, r]
    return Y, IDX


@pytest.mark.parametrize("L,C,phi,xh", [(64, 8, "identity", 1), (60, 16, "elu1", 2),
                                        (37, 5, "identity", 2), (48, 4, "elu1", 1)])
def test_brute_force_grm(L, C, phi, xh):
    Q, K, V, U, X = _rand(1, 2, L, 4, 3, 5, xh=xh, seed=4)
    out = oracle.prefill(Q, K, V, U, X, seg_len=C, phi=phi, mode="grm")
    Yb, _ = _brute(Q, K, V, U, X, C, phi)
    np.testing.assert_allclose(out["Y"], Yb, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("L,C,k", [(64, 4, 3), (63, 8, 2), (40, 4, 1)])
def test_brute_force_ssc(L, C, k):
    Q, K, V, U, X = _rand(1, 2, L, 4, 3, 5, seed=5, scale_u=3.0)
    out = oracle.prefill(Q, K, V, U, X, seg_len=C, mode="ssc", top_k=k)
    Yb, Ib = _brute(Q, K, V, U, X, C, mode="ssc", top_k=k)
    np.testing.assert_allclose(out["Y"], Yb, rtol=1e-11, atol=1e-11)
    np.testing.assert_array_equal(out["idx"].reshape(-1, k), np.array(Ib))


def _sdpa(q, k, v, mask):
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.tensor(mask), scale=1.0).numpy()


def test_segment_length_one_is_softmax_attention():
    """C = 1, q = k = e1: y_t = sum_{i<=t} softmax_i(<u_t, x_i>) v_i (causal SDPA, scale 1)."""
    L, d = 50, 6
    rng = np.random.default_rng(6)
    U = rng.standard_normal((1, 1, L, d))
    X = rng.standard_normal((1, 1, L, d))
    V = rng.standard_normal((1, 1, L, 4))
    e1 = np.zeros((1, 1, L, 3))
    e1[..., 0] = 1.0
    out = oracle.prefill(e1, e1, V, U, X, seg_len=1)
    ref = _sdpa(U, X, V, np.tril(np.ones((L, L), dtype=bool)))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-12)


def test_segment_constant_pool_is_block_causal_attention():
    """x constant inside each segment, q = k = e1, v non-zero only at segment starts:
    y_t = sum_{i<=s} softmax_i(<u_t, c_i>) v_{iC}.  Pins the segment means and the
    online prefix mean (its divisor is the count of tokens seen)."""
    C, N, d = 8, 6, 5
    L = C * N
    rng = np.random.default_rng(7)
    c = rng.standard_normal((N, d))
    X = np.repeat(c, C, axis=0).reshape(1, 1, L, d)
    U = rng.standard_normal((1, 1, L, d)) * 2
    V = np.zeros((1, 1, L, 3))
    vs = rng.standard_normal((N, 3))
    V[0, 0, ::C] = vs
    e1 = np.zeros((1, 1, L, 2))
    e1[..., 0] = 1.0
    out = oracle.prefill(e1, e1, V, U, X, seg_len=C)
    mask = np.arange(N)[None, :] <= (np.arange(L) // C)[:, None]
    ref = _sdpa(U, c.reshape(1, 1, N, d), vs.reshape(1, 1, N, 3), mask)
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-12)


def test_zero_gate_input_gives_uniform_weights():
    Q, K, V, U, X = _rand(1, 2, 45, 4, 4, 4, seed=8)
    C = 6
    out = oracle.prefill(Q, K, V, 0 * U, X, seg_len=C, want_gamma=True)
    s = np.arange(45) // C
    np.testing.assert_allclose(out["Y"], _causal_la(Q, K, V) / (s + 1)[None, None, :, None],
                               rtol=1e-12, atol=1e-12)
    g = out["gamma"][0, 0]
    for t in range(45):
        np.testing.assert_allclose(g[t, :s[t] + 1], 1.0 / (s[t] + 1), rtol=1e-14)
        assert np.all(g[t, s[t] + 1:] == 0)


def test_first_segment_reads_only_online_memory():
    Q, K, V, U, X = _rand(1, 1, 32, 4, 4, 4, seed=9)
    out = oracle.prefill(Q, K, V, U, X, seg_len=16, want_online=True)
    np.testing.assert_array_equal(out["Y"][0, 0, :16], out["O_on"][0, 0, :16])
    np.testing.assert_allclose(out["O_on"][..., :16, :], _causal_la(Q, K, V)[..., :16, :],
                               rtol=1e-12, atol=1e-12)


def test_memory_soup_equals_grm_for_linear_memory():
    Q, K, V, U, X = _rand(2, 2, 40, 5, 4, 3, seed=10)
    grm = oracle.prefill(Q, K, V, U, X, seg_len=8, mode="grm")
    soup = oracle.prefill(Q, K, V, U, X, seg_len=8, mode="soup")
    np.testing.assert_allclose(soup["Y"], grm["Y"], rtol=1e-12, atol=1e-12)


def test_states_and_means_are_segment_sums():
    Q, K, V, U, X = _rand(1, 2, 30, 3, 4, 5, xh=2, seed=11)
    C = 8
    out = oracle.prefill(Q, K, V, U, X, seg_len=C, want_states=True)
    for i in range(4):
        sl = slice(i * C, min((i + 1) * C, 30))
        np.testing.assert_allclose(out["M"][:, :, i],
                                   np.swapaxes(V[:, :, sl], -1, -2) @ K[:, :, sl], rtol=1e-12)
        np.testing.assert_allclose(out["P"][:, :, i], X[:, :, sl].mean(axis=2), rtol=1e-12)


def test_gate_is_on_the_simplex_and_rows_subset_matches():
    Q, K, V, U, X = _rand(2, 2, 50, 4, 4, 4, seed=12, scale_u=5)
    full = oracle.prefill(Q, K, V, U, X, seg_len=7, want_gamma=True)
    g = full["gamma"]
    assert np.all(g >= 0) and np.all(g <= 1)
    np.testing.assert_allclose(g.sum(-1), 1.0, rtol=1e-13)
    rows = np.array([0, 6, 7, 20, 49])
    part = oracle.prefill(Q, K, V, U, X, seg_len=7, rows=rows, want_gamma=True)
    np.testing.assert_array_equal(part["Y"], full["Y"][:, :, rows])
    np.testing.assert_array_equal(part["gamma"], full["gamma"][:, :, rows])


def test_linear_in_values_and_heads_independent():
    Q, K, V, U, X = _rand(1, 3, 33, 4, 4, 4, xh=3, seed=13)
    V2 = np.random.default_rng(14).standard_normal(V.shape)
    y1 = oracle.prefill(Q, K, V, U, X, seg_len=5)["Y"]
    y2 = oracle.prefill(Q, K, V2, U, X, seg_len=5)["Y"]
    y12 = oracle.prefill(Q, K, 2 * V - 3 * V2, U, X, seg_len=5)["Y"]
    np.testing.assert_allclose(y12, 2 * y1 - 3 * y2, rtol=1e-11, atol=1e-11)
    perm = [2, 0, 1]
    yp = oracle.prefill(Q[:, perm], K[:, perm], V[:, perm], U[:, perm], X[:, perm], seg_len=5)["Y"]
    np.testing.assert_array_equal(yp, y1[:, perm])


def test_causal():
    Q, K, V, U, X = _rand(1, 1, 40, 4, 4, 4, seed=15)
    base = oracle.prefill(Q, K, V, U, X, seg_len=8)["Y"]
    t0 = 21
    Q2, K2, V2, U2, X2 = (a.copy() for a in (Q, K, V, U, X))
    for a in (Q2, K2, V2, U2, X2):
        a[..., t0 + 1:, :] += 10.0
    pert = oracle.prefill(Q2, K2, V2, U2, X2, seg_len=8)["Y"]
    np.testing.assert_array_equal(pert[..., :t0 + 1, :], base[..., :t0 + 1, :])
    assert not np.allclose(pert[..., t0 + 1:, :], base[..., t0 + 1:, :])


def test_ssc_ties_pick_lowest_index():
    C, L = 4, 32
    Q, K, V, U, X = _rand(1, 1, L, 4, 4, 4, seed=16)
    X[..., 8:12, :] = X[..., 0:4, :]   # segment 2 duplicates segment 0 (equal scores)
    X[..., 20:24, :] = X[..., 0:4, :]  # and segment 5
    U[..., 24:, :] = X[..., 0:4, :].mean(axis=2, keepdims=True) * 50  # make them win
    out = oracle.prefill(Q, K, V, U, X, seg_len=C, mode="ssc", top_k=1)
    assert np.all(out["idx"][0, 0, 24:, 0] == 0)
    out2 = oracle.prefill(Q, K, V, U, X, seg_len=C, mode="ssc", top_k=2)
    assert np.all(out2["idx"][0, 0, 24:] == [0, 2])


@pytest.mark.parametrize("L,C", [(20, 8), (23, 8), (15, 8), (16, 4)])
def test_prefill_then_decode_equals_longer_prefill(L, C):
    B, H, dk, dv, dg = 2, 2, 4, 3, 5
    Q, K, V, U, X = _rand(B, H, L + 1, dk, dv, dg, seed=17)
    full = oracle.prefill(Q, K, V, U, X, seg_len=C, mode="grm", want_states=True)
    pre = oracle.prefill(Q[:, :, :L], K[:, :, :L], V[:, :, :L], U[:, :, :L], X[:, :, :L],
                         seg_len=C, want_states=True)
    nfull, cnt = divmod(L, C)
    cap = nfull + 2
    Mc = np.zeros((B, H, cap, dv, dk))
    Pc = np.zeros((B, 1, cap, dg))
    Mc[:, :, :nfull] = pre["M"][:, :, :nfull]
    Pc[:, :, :nfull] = pre["P"][:, :, :nfull]
    M_on = pre["M"][:, :, nfull] if cnt else np.zeros((B, H, dv, dk))
    xsum = pre["P"][:, :, nfull] * cnt if cnt else np.zeros((B, 1, dg))
    st = oracle.DecodeState(M_on, xsum.reshape(B, 1, dg), cnt, Mc, Pc, nfull)
    y = oracle.decode_step(st, Q[:, :, L], K[:, :, L], V[:, :, L], U[:, :, L], X[:, :, L],
                           seg_len=C)
    np.testing.assert_allclose(y, full["Y"][:, :, L], rtol=1e-12, atol=1e-12)
    if (L + 1) % C == 0:
        assert st.n_cached[0] == nfull + 1 and st.count[0] == 0
        np.testing.assert_allclose(st.M_cache[:, :, nfull], full["M"][:, :, nfull], rtol=1e-12)
        np.testing.assert_allclose(st.P_cache[:, :, nfull], full["P"][:, :, nfull], rtol=1e-12)
        assert np.all(st.M_on == 0) and np.all(st.xsum == 0)
    else:
        assert st.n_cached[0] == nfull and st.count[0] == cnt + 1


def test_decode_residual_is_linear_attention_read():
    B, H, dk, dv, dg, C = 1, 2, 4, 4, 3, 4
    rng = np.random.default_rng(18)
    n = 3
    Mc = np.zeros((B, H, 5, dv, dk))
    Mc[:, :, :n] = rng.standard_normal((B, H, n, dv, dk))
    st = oracle.DecodeState(rng.standard_normal((B, H, dv, dk)), rng.standard_normal((B, 1, dg)),
                            1, Mc, rng.standard_normal((B, 1, 5, dg)), n)
    q, k = rng.standard_normal((B, H, dk)), rng.standard_normal((B, H, dk))
    v, u, x = rng.standard_normal((B, H, dv)), rng.standard_normal((B, H, dg)), rng.standard_normal((B, 1, dg))
    total = Mc[:, :, :n].sum(2) + st.M_on + v[..., :, None] * k[..., None, :]
    y = oracle.decode_step(st, q, k, v, u, x, seg_len=C, mode="residual")
    np.testing.assert_allclose(y, np.einsum("bhcr,bhr->bhc", total, q), rtol=1e-12)


@pytest.mark.parametrize("L,C", [(20, 8), (23, 8), (15, 8)])
def test_decode_average_is_linear_attention_over_memory_count(L, C):
    """Post-training decode (uniform weights over the n cached memories and the online one):
    the memories of a prefilled sequence sum to its full linear-attention state, so the
    step's output is the attention-form linear-attention read of token L divided by the
    number of memories; with u = 0 the gated step gives the same weights."""
    B, H, dk, dv, dg = 2, 2, 4, 3, 5
    Q, K, V, U, X = _rand(B, H, L + 1, dk, dv, dg, seed=23)
    pre = oracle.prefill(Q[:, :, :L], K[:, :, :L], V[:, :, :L], U[:, :, :L], X[:, :, :L],
                         seg_len=C, want_states=True)
    nfull, cnt = divmod(L, C)
    cap = nfull + 2

    def state():
        Mc = np.zeros((B, H, cap, dv, dk))
        Pc = np.zeros((B, 1, cap, dg))
        Mc[:, :, :nfull] = pre["M"][:, :, :nfull]
        Pc[:, :, :nfull] = pre["P"][:, :, :nfull]
        M_on = pre["M"][:, :, nfull].copy() if cnt else np.zeros((B, H, dv, dk))
        xsum = (pre["P"][:, :, nfull] * cnt).reshape(B, 1, dg) if cnt else np.zeros((B, 1, dg))
        return oracle.DecodeState(M_on, xsum, cnt, Mc, Pc, nfull)

    tok = [A[:, :, L] for A in (Q, K, V, U, X)]
    st = state()
    y = oracle.decode_step(st, *tok, seg_len=C, mode="average")
    la = _causal_la(Q, K, V)[:, :, L]
    np.testing.assert_allclose(y, la / (nfull + 1), rtol=1e-11, atol=1e-12)
    st0 = state()
    y0 = oracle.decode_step(st0, tok[0], tok[1], tok[2], np.zeros_like(tok[3]), tok[4],
                            seg_len=C, mode="grm")
    np.testing.assert_allclose(y, y0, rtol=1e-12, atol=1e-13)
    # the cache bookkeeping is that of the gated step
    np.testing.assert_array_equal(st.n_cached, st0.n_cached)
    np.testing.assert_allclose(st.M_cache, st0.M_cache, rtol=0, atol=0)
    np.testing.assert_allclose(st.P_cache, st0.P_cache, rtol=0, atol=0)


@pytest.mark.parametrize("off,phi,xh", [([0, 3, 4, 11, 20, 29], "identity", 1),
                                        ([0, 1, 2, 3, 13, 14, 29], "elu1", 2),
                                        ([0, 29], "identity", 1)])
def test_brute_force_variable_segments(off, phi, xh):
    L = off[-1]
    Q, K, V, U, X = _rand(1, 2, L, 4, 3, 5, xh=xh, seed=41, scale_u=2.0)
    out = oracle.prefill(Q, K, V, U, X, seg_len=0, phi=phi, mode="grm", seg_offsets=off,
                         want_states=True)
    Yb, _ = _brute(Q, K, V, U, X, 0, phi, off=off)
    np.testing.assert_allclose(out["Y"], Yb, rtol=1e-11, atol=1e-11)
    # states and means are the per-segment sums and means
    x = X[:, :, :, :]
    for i in range(len(off) - 1):
        a, b_ = off[i], off[i + 1]
        kh = _phi(K[:, :, a:b_], phi)
        np.testing.assert_allclose(out["M"][:, :, i],
                                   np.einsum("bhtc,bhtr->bhcr", V[:, :, a:b_], kh), rtol=1e-12)
        np.testing.assert_allclose(out["P"][:, :, i], x[:, :, a:b_].mean(axis=2), rtol=1e-12)
    ssc = oracle.prefill(Q, K, V, U, X, seg_len=0, phi=phi, mode="ssc", top_k=2, seg_offsets=off)
    Ys, Is = _brute(Q, K, V, U, X, 0, phi, mode="ssc", top_k=2, off=off)
    np.testing.assert_allclose(ssc["Y"], Ys, rtol=1e-11, atol=1e-11)
    np.testing.assert_array_equal(ssc["idx"].reshape(-1, 2), np.array(Is))


@pytest.mark.parametrize("L,C", [(64, 8), (37, 5)])
def test_offsets_at_multiples_of_C_equal_constant_segments(L, C):
    Q, K, V, U, X = _rand(2, 2, L, 4, 3, 5, seed=42)
    off = list(range(0, L, C)) + [L]
    a = oracle.prefill(Q, K, V, U, X, seg_len=C, want_states=True, want_gamma=True,
                       want_online=True)
    b = oracle.prefill(Q, K, V, U, X, seg_len=0, seg_offsets=off, want_states=True,
                       want_gamma=True, want_online=True)
    for key in ("Y", "M", "P", "gamma", "O_on"):
        np.testing.assert_array_equal(a[key], b[key])


def test_log_segments_worked_example():
    fix = json.load(open(os.path.join(GOLD, "log_segments_worked_example.json")))
    for case in fix["cases"]:
        assert oracle.log_segments(case["L"]) == case["offsets"]
    for L in range(1, 300):
        off = oracle.log_segments(L)
        lens = np.diff(off)
        assert off[0] == 0 and off[-1] == L and len(lens) == bin(L).count("1")
        assert all(int(n) & (int(n) - 1) == 0 for n in lens) and list(lens) == sorted(lens)[::-1]


# ---- SWLA memory of window 2 (Memory Caching paper, SWLA paragraph, Eq. 26-29) ----

def _swla_gates(B, H, L, seed, alpha_lo=0.5):
    rng = np.random.default_rng(seed)
    alpha = rng.uniform(alpha_lo, 1.0, (B, H, L))
    beta = rng.uniform(-0.5, 1.0, (B, H, L))
    lam = rng.uniform(0.2, 1.2, (B, H, L))
    return alpha, beta, lam


def _swla_weight(alpha, beta, lam, a, t, r):
    """Weight of v_r k_r^T in the memory after token t, both in the segment starting at a:
    it was written with lam_r at step r and with beta_{r+1} at step r+1 (its second slot in
    the window), and every later step multiplied it by that step's alpha."""
    assert a <= r <= t
    w = lam[r] * np.prod(alpha[r + 1:t + 1])
    if r + 1 <= t:
        w += beta[r + 1] * np.prod(alpha[r + 2:t + 1])
    return w


def _brute_swla(Q, K, V, U, X, off, gates, phi="identity"):
    """Token-pair form of Eq. 29 with the Eq. 28 memory: no recurrence, every (t, r) weight
    written as products of the gates.  Returns Y, the cached states and the online read."""
    B, H, L, dk = Q.shape
    dv = V.shape[-1]
    xh = X.shape[1]
    qh, kh = _phi(Q, phi), _phi(K, phi)
    seg = np.searchsorted(np.asarray(off), np.arange(L), side="right") - 1
    NS = len(off) - 1
    Y = np.zeros(V.shape)
    O = np.zeros(V.shape)
    M = np.zeros((B, H, NS, dv, dk))
    for b in range(B):
        for h in range(H):
            al, be, la = (g[b, h] for g in gates)
            x = X[b, 0 if xh == 1 else h]
            means = [x[off[i]:off[i + 1]].mean(axis=0) for i in range(NS)]
            for i in range(NS):
                a, e = off[i], off[i + 1] - 1
                for r in range(a, e + 1):
                    M[b, h, i] += _swla_weight(al, be, la, a, e, r) * np.outer(V[b, h, r], kh[b, h, r])
            for t in range(L):
                s = int(seg[t])
                a = off[s]
                logits = [float(U[b, h, t] @ means[i]) for i in range(s)]
                logits.append(float(U[b, h, t] @ x[a:t + 1].mean(axis=0)))
                g = torch.softmax(torch.tensor(logits, dtype=torch.float64), 0).numpy()
                for r in range(a, t + 1):
                    O[b, h, t] += (_swla_weight(al, be, la, a, t, r)
                                   * float(qh[b, h, t] @ kh[b, h, r]) * V[b, h, r])
                Y[b, h, t] = g[s] * O[b, h, t]
                for i in range(s):
                    Y[b, h, t] += g[i] * (M[b, h, i] @ qh[b, h, t])
    return Y, M, O


def test_swla_unit_gates_are_the_linear_attention_memory():
    # alpha = 1, beta = 0, lam = 1 turns Eq. 28 into the linear-attention update (c = 1)
    B, H, L = 2, 2, 45
    Q, K, V, U, X = _rand(B, H, L, 4, 3, 5, seed=51)
    one, zero = np.ones((B, H, L)), np.zeros((B, H, L))
    for mode, k in (("grm", 0), ("ssc", 2)):
        a = oracle.prefill(Q, K, V, U, X, seg_len=8, mode=mode, top_k=k, want_states=True,
                           want_online=True)
        b = oracle.prefill(Q, K, V, U, X, seg_len=8, mode=mode, top_k=k, want_states=True,
                           want_online=True, swla=(one, zero, one))
        for key in a:
            np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("L,C,off,phi,xh", [(40, 8, None, "identity", 1),
                                            (37, 6, None, "elu1", 2),
                                            (29, 0, [0, 1, 3, 11, 12, 29], "identity", 1)])
def test_brute_force_swla(L, C, off, phi, xh):
    B, H = 1, 2
    Q, K, V, U, X = _rand(B, H, L, 4, 3, 5, xh=xh, seed=52, scale_u=2.0)
    gates = _swla_gates(B, H, L, seed=53)
    out = oracle.prefill(Q, K, V, U, X, seg_len=C, phi=phi, seg_offsets=off, want_states=True,
                         want_online=True, swla=gates)
    o = off if off is not None else list(range(0, L, C)) + [L]
    Yb, Mb, Ob = _brute_swla(Q, K, V, U, X, o, gates, phi)
    np.testing.assert_allclose(out["O_on"], Ob, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(out["M"], Mb, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(out["Y"], Yb, rtol=1e-11, atol=1e-11)


def test_swla_without_carry_is_a_two_token_window():
    # alpha = 0 keeps only the window: M_t = beta_t v_{t-1} k_{t-1}^T + lam_t v_t k_t^T, and
    # the segment's first token has no previous token to write
    B, H, L, C = 1, 3, 30, 7
    Q, K, V, U, X = _rand(B, H, L, 4, 3, 5, seed=54)
    _, beta, lam = _swla_gates(B, H, L, seed=55)
    out = oracle.prefill(Q, K, V, U, X, seg_len=C, want_online=True, want_states=True,
                         swla=(np.zeros((B, H, L)), beta, lam))
    for h in range(H):
        for t in range(L):
            exp = lam[0, h, t] * float(Q[0, h, t] @ K[0, h, t]) * V[0, h, t]
            if t % C:
                exp = exp + beta[0, h, t] * float(Q[0, h, t] @ K[0, h, t - 1]) * V[0, h, t - 1]
            np.testing.assert_allclose(out["O_on"][0, h, t], exp, rtol=1e-12, atol=1e-12)
        for i in range((L + C - 1) // C):
            e = min(L, (i + 1) * C) - 1
            exp = lam[0, h, e] * np.outer(V[0, h, e], K[0, h, e])
            if e % C:
                exp = exp + beta[0, h, e] * np.outer(V[0, h, e - 1], K[0, h, e - 1])
            np.testing.assert_allclose(out["M"][0, h, i], exp, rtol=1e-12, atol=1e-12)


def test_swla_constant_decay_one_segment_is_decayed_attention():
    # beta = 0, lam = 1, alpha = a, one segment: y_t = sum_{r<=t} a^(t-r) (q_t.k_r) v_r, the
    # attention form with a decay mask
    B, H, L, a = 1, 2, 33, 0.93
    Q, K, V, U, X = _rand(B, H, L, 4, 3, 5, seed=56)
    gates = (np.full((B, H, L), a), np.zeros((B, H, L)), np.ones((B, H, L)))
    out = oracle.prefill(Q, K, V, U, X, seg_len=L, swla=gates)
    t = np.arange(L)
    D = np.where(t[:, None] >= t[None, :], a ** (t[:, None] - t[None, :]).clip(0), 0.0)
    exp = (Q @ np.swapaxes(K, -1, -2) * D) @ V
    np.testing.assert_allclose(out["Y"], exp, rtol=1e-11, atol=1e-11)


def test_swla_soup_equals_grm():
    # SWLA is a linear memory, so its Memory Soup and GRM variants coincide (the remark after
    # Eq. 29)
    B, H, L = 1, 2, 36
    Q, K, V, U, X = _rand(B, H, L, 4, 3, 5, seed=57)
    gates = _swla_gates(B, H, L, seed=58)
    a = oracle.prefill(Q, K, V, U, X, seg_len=6, mode="grm", swla=gates)
    b = oracle.prefill(Q, K, V, U, X, seg_len=6, mode="soup", swla=gates)
    np.testing.assert_allclose(a["Y"], b["Y"], rtol=1e-12, atol=1e-12)


# ---- backward of the GRM prefill: gradients of sum(Y * dY) ----

def _loss(Q, K, V, U, X, dY, C, phi):
    return float((oracle.prefill(Q, K, V, U, X, seg_len=C, phi=phi)["Y"] * dY).sum())


@pytest.mark.parametrize("L,C,phi,xh", [(13, 4, "identity", 1), (11, 3, "elu1", 2),
                                        (9, 9, "identity", 2)])
def test_backward_matches_finite_differences(L, C, phi, xh):
    # central differences of the forward oracle, every coordinate of every input
    B, H = 1, 2
    Q, K, V, U, X = _rand(B, H, L, 3, 2, 3, xh=xh, seed=61, scale_u=1.5)
    dY = np.random.default_rng(62).standard_normal(V.shape)
    got = oracle.grm_backward(Q, K, V, U, X, dY, seg_len=C, phi=phi)
    eps = 1e-6
    for name, arr in (("dQ", Q), ("dK", K), ("dV", V), ("dU", U), ("dX", X)):
        num = np.zeros(arr.shape)
        for ix in np.ndindex(arr.shape):
            keep = arr[ix]
            arr[ix] = keep + eps
            fp = _loss(Q, K, V, U, X, dY, C, phi)
            arr[ix] = keep - eps
            fm = _loss(Q, K, V, U, X, dY, C, phi)
            arr[ix] = keep
            num[ix] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(got[name], num, rtol=1e-6, atol=1e-7, err_msg=name)


def _torch_brute_grm(Q, K, V, U, X, C, phi):
    """Token-pair form of the GRM read in torch (no states): differentiable by autograd."""
    B, H, L, _ = Q.shape
    xh = X.shape[1]
    f = (lambda z: z) if phi == "identity" else (lambda z: torch.where(z > 0, z + 1.0, torch.exp(torch.clamp(z, max=0.0))))
    qh, kh = f(Q), f(K)
    seg = [t // C for t in range(L)]
    NS = (L + C - 1) // C
    rows = []
    for b in range(B):
        for h in range(H):
            x = X[b, 0 if xh == 1 else h]
            means = [x[i * C:min(L, (i + 1) * C)].mean(0) for i in range(NS)]
            ys = []
            for t in range(L):
                s = seg[t]
                logits = [U[b, h, t] @ means[i] for i in range(s)]
                logits.append(U[b, h, t] @ x[s * C:t + 1].mean(0))
                g = torch.softmax(torch.stack(logits), 0)
                y = 0.0
                for r in range(t + 1):
                    y = y + g[seg[r]] * (qh[b, h, t] @ kh[b, h, r]) * V[b, h, r]
                ys.append(y)
            rows.append(torch.stack(ys))
    return torch.stack(rows).reshape(B, H, L, -1)


@pytest.mark.parametrize("L,C,phi,xh", [(24, 8, "identity", 1), (19, 5, "elu1", 2)])
def test_backward_matches_autograd_of_token_pair_form(L, C, phi, xh):
    B, H = 1, 2
    Q, K, V, U, X = _rand(B, H, L, 4, 3, 5, xh=xh, seed=63, scale_u=1.5)
    dY = np.random.default_rng(64).standard_normal(V.shape)
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (Q, K, V, U, X)]
    Y = _torch_brute_grm(*ts, C, phi)
    (Y * torch.tensor(dY)).sum().backward()
    got = oracle.grm_backward(Q, K, V, U, X, dY, seg_len=C, phi=phi)
    for name, t in zip(("dQ", "dK", "dV", "dU", "dX"), ts):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=1e-10, atol=1e-11,
                                   err_msg=name)


def test_backward_rows_are_the_full_gradients_at_those_rows():
    B, H, L, C = 1, 2, 30, 7
    Q, K, V, U, X = _rand(B, H, L, 4, 3, 5, seed=65)
    dY = np.random.default_rng(66).standard_normal(V.shape)
    full = oracle.grm_backward(Q, K, V, U, X, dY, seg_len=C, phi="elu1")
    rows = [0, 6, 7, 13, 29]
    part = oracle.grm_backward(Q, K, V, U, X, dY, seg_len=C, phi="elu1", rows=rows)
    np.testing.assert_array_equal(part["dQ"], full["dQ"][:, :, rows])
    np.testing.assert_array_equal(part["dU"], full["dU"][:, :, rows])
