"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Nothing here calls the GPU library.  Each test checks the oracle against
something other than itself: hand-worked values, closed forms, invariants the
recurrence must satisfy, a library routine, or an independent chunked
formulation.  Together they are chosen so that a plausible slip in the oracle
(a dropped decay, decay after the write, a read before the write, a wrong
sign, a transposed state, a misplaced A_log or dt_bias, a wrong varlen
offset) fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

from kda_testutil import bf16_tensor, rand_inputs
from oracle import kda_oracle, kda_oracle_np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_both(inp, scale, lb, **kw):
    """Run the C oracle and the numpy twin; check they agree; return C's."""
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], scale,
            inp["A_log"], inp["dt_bias"], lb)
    o1, f1 = kda_oracle(*args, initial_state=inp.get("initial_state"),
                        cu_seqlens=inp.get("cu_seqlens"), **kw)
    o2, f2 = kda_oracle_np(*args, initial_state=inp.get("initial_state"),
                           cu_seqlens=inp.get("cu_seqlens"))
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13)
    assert np.allclose(f1, f2, rtol=1e-12, atol=1e-13)
    return o1, f1


# --------------------------------------------------------------------------
# hand-worked values
# --------------------------------------------------------------------------

def _golden_cases():
    with open(os.path.join(GOLDEN, "handworked_small_heads.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_handworked(case):
    K, V = case["K"], case["V"]
    T = len(case["q"])
    shape = lambda a, d: bf16_tensor(np.array(a, dtype=np.float32).reshape(1, T, 1, d))
    inp = dict(
        q=shape(case["q"], K), k=shape(case["k"], K), v=shape(case["v"], V),
        g=shape(case["g"], K),
        beta=bf16_tensor(np.array(case["beta_logit"], dtype=np.float32).reshape(1, T, 1)),
        A_log=torch.tensor([case["A_log"]], dtype=torch.float32),
        dt_bias=torch.tensor([case["dt_bias"]], dtype=torch.float32),
        initial_state=None)
    if case["initial_state"] is not None:
        inp["initial_state"] = torch.tensor(case["initial_state"], dtype=torch.float32).reshape(1, 1, V, K)
    out, fin = run_both(inp, case["scale"], case["lower_bound"])
    np.testing.assert_allclose(out.reshape(T, V), np.array(case["out"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(fin.reshape(V, K), np.array(case["final_state"]), rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def _sign_gates(rng, B, T, H, K):
    """Gate logits of +-100: sigmoid is then 1 or 0 to double precision, so
    each token's decay per channel is exactly e^lb or 1."""
    s = rng.integers(0, 2, size=(B, T, H, K))
    return s, bf16_tensor(np.where(s == 1, 100.0, -100.0).astype(np.float32))


def test_zero_beta_is_pure_decay():
    """beta = 0 removes every write: final = diag(e^{G_L}) S0 and
    o_t = scale (diag(e^{G_t}) S0)^T q_t, with G the per-channel gate sum."""
    rng = np.random.default_rng(1)
    B, T, H, K, V, lb, scale = 2, 23, 2, 8, 6, -1.7, 0.37
    inp = rand_inputs(B, T, H, K, V, seed=3, init=torch.float32)
    s, inp["g"] = _sign_gates(rng, B, T, H, K)
    inp["A_log"] = torch.zeros(H)
    inp["dt_bias"] = torch.zeros(H, K)
    inp["beta"] = bf16_tensor(np.full((B, T, H), -8192.0, dtype=np.float32))
    out, fin = run_both(inp, scale, lb)
    q = inp["q"].double().numpy()
    S0 = inp["initial_state"].double().numpy()  # [B,H,V,K]
    cnt = np.cumsum(s, axis=1)                    # [B,T,H,K]
    for b in range(B):
        for h in range(H):
            decay = np.exp(lb * cnt[b, :, h, :])  # [T,K]
            ref_o = scale * np.einsum("tk,vk,tk->tv", decay, S0[b, h], q[b, :, h, :])
            np.testing.assert_allclose(out[b, :, h], ref_o, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(fin[b, h], S0[b, h] * decay[-1][None, :],
                                       rtol=1e-12, atol=1e-15)


def test_zero_beta_without_state_is_zero():
    inp = rand_inputs(1, 19, 2, 8, 8, seed=4)
    inp["beta"] = bf16_tensor(np.full((1, 19, 2), -8192.0, dtype=np.float32))
    out, fin = run_both(inp, 0.5, -5.0)
    assert not out.any() and not fin.any()


def test_one_hot_keys_reduce_to_gla():
    """Distinct one-hot keys make S^T k_t = 0 before each write, so the state
    is a gated linear attention sum:
    o_t = scale sum_{s<=t} beta_s q_t[i_s] e^{G_t[i_s]-G_s[i_s]} v_s."""
    rng = np.random.default_rng(5)
    B, T, H, K, V, lb, scale = 1, 12, 2, 16, 5, -2.3, 0.8
    inp = rand_inputs(B, T, H, K, V, seed=6)
    idx = np.stack([rng.permutation(K)[:T] for _ in range(H)], axis=1)  # [T,H]
    kk = np.zeros((B, T, H, K), dtype=np.float32)
    for t in range(T):
        for h in range(H):
            kk[0, t, h, idx[t, h]] = 1.0
    inp["k"] = bf16_tensor(kk)
    s, inp["g"] = _sign_gates(rng, B, T, H, K)
    inp["A_log"] = torch.zeros(H)
    inp["dt_bias"] = torch.zeros(H, K)
    out, fin = run_both(inp, scale, lb)
    q = inp["q"].double().numpy()[0]
    v = inp["v"].double().numpy()[0]
    beta = expit(inp["beta"].double().numpy()[0])
    G = lb * np.cumsum(s[0], axis=0)  # [T,H,K]
    for h in range(H):
        for t in range(T):
            ref = np.zeros(V)
            for u in range(t + 1):
                i = idx[u, h]
                ref += beta[u, h] * q[t, h, i] * math.exp(G[t, h, i] - G[u, h, i]) * v[u, h]
            np.testing.assert_allclose(out[0, t, h], scale * ref, rtol=1e-12, atol=1e-14)


def test_repeated_key_with_full_beta_overwrites_row():
    """The same one-hot key e_i every token with beta = 1 makes row i of S
    equal v_t after token t, while the other rows only decay."""
    rng = np.random.default_rng(7)
    B, T, H, K, V, lb, scale, i = 1, 9, 1, 8, 4, -0.9, 1.25, 3
    inp = rand_inputs(B, T, H, K, V, seed=8, init=torch.float32)
    kk = np.zeros((B, T, H, K), dtype=np.float32)
    kk[..., i] = 1.0
    inp["k"] = bf16_tensor(kk)
    inp["beta"] = bf16_tensor(np.full((B, T, H), 100.0, dtype=np.float32))
    s, inp["g"] = _sign_gates(rng, B, T, H, K)
    inp["A_log"] = torch.zeros(H)
    inp["dt_bias"] = torch.zeros(H, K)
    out, fin = run_both(inp, scale, lb)
    S0 = inp["initial_state"].double().numpy()[0, 0].T  # S[k, v]
    q = inp["q"].double().numpy()[0, :, 0]
    v = inp["v"].double().numpy()[0, :, 0]
    G = lb * np.cumsum(s[0, :, 0], axis=0)
    for t in range(T):
        S = np.exp(G[t])[:, None] * S0
        S[i] = v[t]
        np.testing.assert_allclose(out[0, t, 0], scale * S.T @ q[t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], S.T, rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------
# the gate: A_log, dt_bias, lower_bound
# --------------------------------------------------------------------------

def test_gate_value_matches_library_sigmoid():
    """One token, beta = 0, unit state: final[v][k] = exp(lb * expit(x_k))
    with x = exp(A_log) (g + dt_bias); expit is scipy's logistic."""
    rng = np.random.default_rng(9)
    H, K, V, lb = 3, 8, 2, -4.2
    inp = rand_inputs(1, 1, H, K, V, seed=10)
    inp["beta"] = bf16_tensor(np.full((1, 1, H), -8192.0, dtype=np.float32))
    S0 = np.ones((1, H, V, K), dtype=np.float32)
    inp["initial_state"] = torch.from_numpy(S0)
    inp["A_log"] = torch.from_numpy(rng.normal(size=H).astype(np.float32))
    _, fin = run_both(inp, 1.0, lb)
    g = inp["g"].double().numpy()[0, 0]
    x = np.exp(inp["A_log"].double().numpy())[:, None] * (g + inp["dt_bias"].double().numpy())
    ref = np.exp(lb * expit(x))  # [H,K]
    np.testing.assert_allclose(fin[0], np.broadcast_to(ref[:, None, :], (H, V, K)), rtol=1e-13)


def test_A_log_multiplies_the_biased_gate():
    """exp(A_log) = 2 with g = x/2 equals A_log = 0 with g = x."""
    B, T, H, K, V = 1, 20, 2, 8, 8
    inp = rand_inputs(B, T, H, K, V, seed=11, init=torch.float32)
    half = np.round(np.random.default_rng(12).normal(size=(B, T, H, K)) * 8) / 16
    inp["dt_bias"] = torch.zeros(H, K)
    a = dict(inp, g=bf16_tensor(half.astype(np.float32)),
             A_log=torch.full((H,), math.log(2.0), dtype=torch.float32))
    b = dict(inp, g=bf16_tensor((2 * half).astype(np.float32)), A_log=torch.zeros(H))
    oa, fa = run_both(a, 0.7, -3.0)
    ob, fb = run_both(b, 0.7, -3.0)
    # float32(ln 2) differs from ln 2 by < 3e-8 relative
    np.testing.assert_allclose(oa, ob, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(fa, fb, rtol=1e-6, atol=1e-7)


def test_dt_bias_is_per_head_and_channel():
    """Moving a per-(head, channel) offset from g into dt_bias[h, k] leaves
    the result unchanged bit for bit."""
    B, T, H, K, V = 2, 7, 3, 8, 4
    inp = rand_inputs(B, T, H, K, V, seed=13)
    off = np.round(np.random.default_rng(14).normal(size=(H, K)) * 4) / 4
    a = dict(inp, g=bf16_tensor(np.broadcast_to(off, (B, T, H, K)).astype(np.float32)),
             dt_bias=torch.zeros(H, K))
    b = dict(inp, g=bf16_tensor(np.zeros((B, T, H, K), np.float32)),
             dt_bias=torch.from_numpy(off.astype(np.float32)))
    oa, fa = run_both(a, 0.3, -2.0)
    ob, fb = run_both(b, 0.3, -2.0)
    assert np.array_equal(oa, ob) and np.array_equal(fa, fb)


def test_missing_gate_params_mean_zero():
    """A_log = None acts as A_log = 0 and dt_bias = None as dt_bias = 0."""
    inp = rand_inputs(1, 17, 2, 8, 8, seed=15)
    a = dict(inp, A_log=None, dt_bias=None)
    b = dict(inp, A_log=torch.zeros(2), dt_bias=torch.zeros(2, 8))
    oa, fa = run_both(a, 0.5, -5.0)
    ob, fb = run_both(b, 0.5, -5.0)
    assert np.array_equal(oa, ob) and np.array_equal(fa, fb)


def test_zero_lower_bound_ignores_the_gate():
    """lb = 0 gives decay 1 whatever g is (the ungated delta rule)."""
    inp = rand_inputs(1, 21, 2, 8, 8, seed=16, init=torch.float32)
    other = dict(inp, g=(inp["g"].float() * 3 + 1).bfloat16())
    oa, fa = run_both(inp, 0.5, 0.0)
    ob, fb = run_both(other, 0.5, 0.0)
    assert np.array_equal(oa, ob) and np.array_equal(fa, fb)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_split_sequence_chains_through_the_state():
    """Running [0,T1) then [T1,T) from final(T1) equals one pass."""
    B, T, H, K, V, T1 = 2, 45, 2, 16, 8, 19
    inp = rand_inputs(B, T, H, K, V, seed=17, init=torch.float32)
    args = lambda d, sl: (d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["g"][:, sl],
                          d["beta"][:, sl], 0.6, d["A_log"], d["dt_bias"], -5.0)
    o, f = kda_oracle(*args(inp, slice(None)), initial_state=inp["initial_state"])
    o1, f1 = kda_oracle(*args(inp, slice(0, T1)), initial_state=inp["initial_state"])
    o2, f2 = kda_oracle(*args(inp, slice(T1, None)), initial_state=f1.astype(np.float32))
    # the hand-off rounds the state to float32 once
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=0, atol=1e-7)
    np.testing.assert_allclose(f2, f, rtol=0, atol=1e-7)


def test_packed_sequences_equal_separate_runs():
    lens = [5, 16, 1, 0, 33]
    H, K, V = 2, 8, 8
    inp = rand_inputs(1, 0, H, K, V, seed=18, varlen=lens, init=torch.bfloat16)
    o, f = run_both(inp, 0.4, -5.0)
    cu = inp["cu_seqlens"].numpy()
    for n in range(len(lens)):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        on, fn = kda_oracle(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], inp["g"][:, sl],
                            inp["beta"][:, sl], 0.4, inp["A_log"], inp["dt_bias"], -5.0,
                            initial_state=inp["initial_state"][n:n + 1])
        assert np.array_equal(on[0], o[0, sl])
        assert np.array_equal(fn[0], f[n])
    # a zero-length sequence hands its initial state straight through
    np.testing.assert_array_equal(f[3], inp["initial_state"][3].double().numpy())


def test_power_of_two_scaling_is_exact():
    """(out, final) is linear in (S0, v); scaling both by 2 is exact."""
    inp = rand_inputs(2, 25, 2, 8, 8, seed=19, init=torch.float32)
    o, f = run_both(inp, 0.5, -5.0)
    d = dict(inp, v=(inp["v"].float() * 2).bfloat16(), initial_state=inp["initial_state"] * 2)
    o2, f2 = run_both(d, 0.5, -5.0)
    assert np.array_equal(o2, 2 * o) and np.array_equal(f2, 2 * f)


def test_superposition_in_state_and_values():
    rng = np.random.default_rng(20)
    B, T, H, K, V = 1, 30, 2, 8, 8
    inp = rand_inputs(B, T, H, K, V, seed=21)
    grid = lambda shape: (rng.integers(-32, 33, size=shape) / 16).astype(np.float32)
    va, vb = grid((B, T, H, V)), grid((B, T, H, V))
    sa, sb = grid((B, H, V, K)), grid((B, H, V, K))
    run = lambda vv, ss: run_both(dict(inp, v=bf16_tensor(vv), initial_state=torch.from_numpy(ss)),
                                  0.5, -5.0)
    oa, fa = run(va, sa)
    ob, fb = run(vb, sb)
    oc, fc = run(va + vb, sa + sb)
    np.testing.assert_allclose(oc, oa + ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fc, fa + fb, rtol=0, atol=1e-12)


def test_scale_is_linear_in_output_only():
    inp = rand_inputs(1, 13, 2, 8, 8, seed=22, init=torch.float32)
    o1, f1 = run_both(inp, 0.25, -5.0)
    o2, f2 = run_both(inp, 1.0, -5.0)
    assert np.array_equal(4 * o1, o2) and np.array_equal(f1, f2)


def test_head_permutation():
    B, T, H, K, V = 2, 14, 4, 8, 8
    inp = rand_inputs(B, T, H, K, V, seed=23, init=torch.float32)
    perm = torch.tensor([2, 0, 3, 1])
    p = dict(q=inp["q"][:, :, perm], k=inp["k"][:, :, perm], v=inp["v"][:, :, perm],
             g=inp["g"][:, :, perm], beta=inp["beta"][:, :, perm], A_log=inp["A_log"][perm],
             dt_bias=inp["dt_bias"][perm], initial_state=inp["initial_state"][:, perm])
    o, f = run_both(inp, 0.5, -5.0)
    op, fp = run_both(p, 0.5, -5.0)
    assert np.array_equal(op, o[:, :, perm.numpy()]) and np.array_equal(fp, f[:, perm.numpy()])


def test_thread_count_and_chain_subset_do_not_change_results():
    inp = rand_inputs(2, 40, 3, 16, 16, seed=24, init=torch.bfloat16)
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 0.5, inp["A_log"],
            inp["dt_bias"], -5.0)
    o1, f1 = kda_oracle(*args, initial_state=inp["initial_state"], threads=1)
    o8, f8 = kda_oracle(*args, initial_state=inp["initial_state"], threads=8)
    assert np.array_equal(o1, o8) and np.array_equal(f1, f8)
    sub = kda_oracle(*args, initial_state=inp["initial_state"], chains=[(1, 2), (0, 1)])
    assert np.array_equal(sub[0][0], o1[1, :, 2]) and np.array_equal(sub[0][1], f1[1, 2])
    assert np.array_equal(sub[1][0], o1[0, :, 1]) and np.array_equal(sub[1][1], f1[0, 1])


# --------------------------------------------------------------------------
# an independent chunked (WY) formulation of the same recurrence
# --------------------------------------------------------------------------

def neumann_inverse(L):
    """(I - L)^-1 for strictly lower-triangular 16x16 L as the product
    (I+L)(I+L^2)(I+L^4)(I+L^8), exact because L^16 = 0 (chunk-size page,
    'Efficient 16x16 Matrix Inversion')."""
    n = L.shape[0]
    I = np.eye(n)
    out = I.copy()
    P = L.copy()
    for _ in range(4):
        out = out @ (I + P)
        P = P @ P
    return out


def test_neumann_product_is_the_inverse():
    rng = np.random.default_rng(25)
    for _ in range(5):
        L = np.tril(rng.normal(size=(16, 16)) * 0.3, -1)
        np.testing.assert_allclose(neumann_inverse(L), np.linalg.inv(np.eye(16) - L),
                                   rtol=1e-10, atol=1e-12)


def chunked_wy(q, k, v, a, beta, scale, S0, C=16):
    """Chunk-of-C evaluation: per chunk, G = cumsum(a), K~ = k e^G,
    K^ = k e^-G, Q~ = scale q e^G, Kbar = k e^(G_C - G); A = diag(beta) K~ K^T
    strictly lower, P = Q~ K^T lower, T = (I + A)^-1, W = T diag(beta) K~,
    U~ = T diag(beta) V; U = U~ - W S; O = Q~ S + P U; S <- e^G_C S + Kbar^T U."""
    L = q.shape[0]
    S = S0.copy()
    out = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(c0 + C, L))
        n = sl.stop - sl.start
        G = np.cumsum(a[sl], axis=0)
        Kt, Kh = k[sl] * np.exp(G), k[sl] * np.exp(-G)
        Qt = scale * q[sl] * np.exp(G)
        Kb = k[sl] * np.exp(G[-1] - G)
        A = np.tril(beta[sl, None] * (Kt @ Kh.T), -1)
        P = np.tril(Qt @ Kh.T)
        Tm = neumann_inverse(-A) if n == C else np.linalg.inv(np.eye(n) + A)
        W = Tm @ (beta[sl, None] * Kt)
        U = Tm @ (beta[sl, None] * v[sl]) - W @ S
        out[sl] = Qt @ S + P @ U
        S = np.exp(G[-1])[:, None] * S + Kb.T @ U
    return out, S


@pytest.mark.parametrize("lb,T", [(-5.0, 53), (-3.0, 64), (0.0, 31), (-5.0, 7)])
def test_token_loop_equals_chunked_form(lb, T):
    B, H, K, V = 1, 2, 32, 16
    inp = rand_inputs(B, T, H, K, V, seed=26, init=torch.float32)
    o, f = kda_oracle(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], 0.3,
                      inp["A_log"], inp["dt_bias"], lb, initial_state=inp["initial_state"])
    g = inp["g"].double().numpy()[0]
    x = np.exp(inp["A_log"].double().numpy())[None, :, None] * (g + inp["dt_bias"].double().numpy())
    a = lb * expit(x)  # [T,H,K]
    beta = expit(inp["beta"].double().numpy()[0])
    for h in range(H):
        oc, Sc = chunked_wy(inp["q"].double().numpy()[0, :, h], inp["k"].double().numpy()[0, :, h],
                            inp["v"].double().numpy()[0, :, h], a[:, h], beta[:, h], 0.3,
                            inp["initial_state"].double().numpy()[0, h].T)
        np.testing.assert_allclose(o[0, :, h], oc, rtol=0, atol=1e-12)
        np.testing.assert_allclose(f[0, h], Sc.T, rtol=0, atol=1e-12)
