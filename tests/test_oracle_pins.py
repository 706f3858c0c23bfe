"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

Each test computes its expectation by a route that shares nothing with the
oracle's token loop (printed values, closed forms, explicit matrix products,
direct double sums, invariants), so that a dropped term, a wrong sign, a
transposed operand, a decay on the wrong axis or a readout taken before the
write fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(x, axis=-1):
    return x / np.linalg.norm(x, axis=axis, keepdims=True)


def _rand_inputs(rng, T, H, dk, dv, g_scale=1.0):
    q = _unit(rng.standard_normal((T, H, dk)))
    k = _unit(rng.standard_normal((T, H, dk)))
    v = rng.standard_normal((T, H, dv))
    g = -g_scale * rng.random((T, H, dk))
    beta = rng.random((T, H))
    return q, k, v, g, beta


# --------------------------------------------------------------------------
# P1: worked example -- Hybrid Attention, "KDA: don't write the same
# information twice": prediction 2, target 6, beta 0.5 -> 4 along the key.
# --------------------------------------------------------------------------
def test_p1_worked_delta_example(oracle_mod):
    ex = json.load(open(os.path.join(GOLDEN, "worked_delta_example.json")))
    rng = np.random.default_rng(11)
    dk = 6
    kk = _unit(rng.standard_normal(dk))
    S0 = (ex["prediction"] * kk)[:, None]          # S0^T k = prediction
    q = kk[None, None, :]
    k = kk[None, None, :]
    v = np.array([[[ex["target"]]]])
    g = np.zeros((1, 1, dk))
    beta = np.array([[ex["beta"]]])
    o, S = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0[None, None])
    assert o[0, 0, 0] == pytest.approx(ex["result"], abs=1e-14)
    assert float(S[0, 0, :, 0] @ kk) == pytest.approx(ex["result"], abs=1e-14)
    # the component orthogonal to k is untouched by the write
    w = _unit(rng.standard_normal(dk) - (rng.standard_normal(dk) @ kk) * kk)
    w = _unit(w - (w @ kk) * kk)
    assert abs(float(S[0, 0, :, 0] @ w)) < 1e-14


# --------------------------------------------------------------------------
# P2: beta = 1 with a unit key and no decay stores v exactly along k
# (neuralmasteryai.com section 3); the readout uses the state after the
# write (kimi-k3-course lesson 2), so q = k reads back v.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dk,dv", [(4, 4), (5, 3), (16, 16)])
def test_p2_exact_recall_after_write(oracle_mod, dk, dv):
    rng = np.random.default_rng(dk * 10 + dv)
    T, H = 9, 2
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    # last token: beta = 1, g = 0, q = k
    beta[-1] = 1.0
    g[-1] = 0.0
    q[-1] = k[-1]
    o, S = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0)
    np.testing.assert_allclose(o[-1], v[-1], atol=1e-13)
    for h in range(H):
        np.testing.assert_allclose(S[0, h].T @ k[-1, h], v[-1, h], atol=1e-13)


# --------------------------------------------------------------------------
# P3: with the delta term removed, no decay and beta = 1 the recurrence is
# linear attention, o_t = sum_{i<=t} (q_t . k_i) v_i (neuralmasteryai.com
# section 2, the regrouped sum).  Computed here as a direct double sum.
# --------------------------------------------------------------------------
def test_p3_linear_attention_double_sum(oracle_mod):
    rng = np.random.default_rng(3)
    T, H, dk, dv = 12, 3, 5, 7
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = np.zeros((T, H, dk))
    beta = np.ones((T, H))
    o, S = oracle_mod.prefill(q, k, v, g, beta, delta=False)
    ref = np.zeros_like(o)
    for t in range(T):
        for h in range(H):
            for i in range(t + 1):
                ref[t, h] += float(q[t, h] @ k[i, h]) * v[i, h]
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    for h in range(H):
        np.testing.assert_allclose(S[0, h], sum(np.outer(k[i, h], v[i, h]) for i in range(T)),
                                   atol=1e-12)


# P3b: gated linear write (delta removed, decay and beta kept) has the closed
# form S_t = Diag(e^{G_t}) S0 + sum_{i<=t} Diag(e^{G_t - G_i}) beta_i k_i v_i^T
# with G the inclusive per-channel cumulative log-decay.
def test_p3b_gated_linear_closed_form(oracle_mod):
    rng = np.random.default_rng(4)
    T, H, dk, dv = 10, 2, 6, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0, delta=False,
                              scale=0.7)
    G = np.cumsum(g, axis=0)
    for h in range(H):
        for t in range(T):
            St = np.exp(G[t, h])[:, None] * S0[0, h]
            for i in range(t + 1):
                St = St + np.exp(G[t, h] - G[i, h])[:, None] * beta[i, h] * np.outer(k[i, h], v[i, h])
            np.testing.assert_allclose(o[t, h], 0.7 * St.T @ q[t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, atol=1e-12)


# --------------------------------------------------------------------------
# P4: pure decay.  beta = 0 removes every write, so S_T = Diag(e^{sum g}) S0
# and o_t = S0^T (e^{G_t} * q_t): the decay scales key-channel ROWS
# (Understanding Kimi K3's attention, symbol table; neuralmasteryai.com
# section 5).  dk != dv makes a decay on the wrong axis fail to match.
# --------------------------------------------------------------------------
def test_p4_pure_decay_rows(oracle_mod):
    rng = np.random.default_rng(5)
    T, H, dk, dv = 8, 2, 6, 4
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=2.0)
    beta[:] = 0.0
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0)
    G = np.cumsum(g, axis=0)
    for h in range(H):
        np.testing.assert_allclose(S[0, h], np.exp(G[-1, h])[:, None] * S0[0, h], rtol=1e-14, atol=0)
        for t in range(T):
            np.testing.assert_allclose(o[t, h], S0[0, h].T @ (np.exp(G[t, h]) * q[t, h]),
                                       rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# P5: the product form (I - b k k^T) Diag(a) S + b k v^T and the gradient-
# descent form D S - b grad L(D S), grad L(X) = k (X^T k - v)^T
# (Understanding Kimi K3's attention), evaluated with explicit matrices.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", ["product", "gradient"])
def test_p5_equivalent_forms(oracle_mod, form):
    rng = np.random.default_rng(6)
    T, H, dk, dv = 11, 2, 5, 4
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0, scale=1.3)
    for h in range(H):
        St = S0[0, h].copy()
        for t in range(T):
            kk, vv, b = k[t, h], v[t, h], beta[t, h]
            D = np.diag(np.exp(g[t, h]))
            if form == "product":
                St = (np.eye(dk) - b * np.outer(kk, kk)) @ D @ St + b * np.outer(kk, vv)
            else:
                X = D @ St
                St = X - b * np.outer(kk, X.T @ kk - vv)
            np.testing.assert_allclose(o[t, h], 1.3 * St.T @ q[t, h], atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, atol=1e-12)


# --------------------------------------------------------------------------
# P6: brute force on tiny inputs, from the unrolled sum
#   S_t = Phi_t..Phi_1 S0 + sum_s Phi_t..Phi_{s+1} b_s k_s v_s^T,
#   Phi_t = (I - b_t k_t k_t^T) Diag(a_t),
# over a packed batch whose sequences restart from their own S0.
# --------------------------------------------------------------------------
def test_p6_brute_force_unrolled_packed(oracle_mod):
    rng = np.random.default_rng(7)
    lens = [3, 0, 5, 1, 8]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, H, dk, dv = int(cu[-1]), 2, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=1.5)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    o, S = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu)
    for n in range(len(lens)):
        for h in range(H):
            a, b_ = int(cu[n]), int(cu[n + 1])
            Phi = [(np.eye(dk) - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(g[t, h]))
                   for t in range(a, b_)]
            for t in range(a, b_):
                # Phi_t ... Phi_a applied to S0, then each write carried forward
                prod_all = np.eye(dk)
                for s in range(a, t + 1):
                    prod_all = Phi[s - a] @ prod_all
                St = prod_all @ S0[n, h]
                for s in range(a, t + 1):
                    P = np.eye(dk)
                    for r in range(s + 1, t + 1):
                        P = Phi[r - a] @ P
                    St = St + P @ (beta[s, h] * np.outer(k[s, h], v[s, h]))
                np.testing.assert_allclose(o[t, h], St.T @ q[t, h], atol=1e-13)
            if b_ == a:
                np.testing.assert_array_equal(S[n, h], S0[n, h])
            else:
                np.testing.assert_allclose(S[n, h], St, atol=1e-13)


# --------------------------------------------------------------------------
# P7: the toy memory demo of neuralmasteryai.com section 3 (d = 64, 20
# pairs, then key 0 rewritten): printed relative errors for linear attention
# and for the delta rule.  Inputs are drawn in the order the page describes.
# --------------------------------------------------------------------------
def test_p7_toy_demo_printed_errors(oracle_mod):
    ex = json.load(open(os.path.join(GOLDEN, "toy_delta_vs_linear.json")))
    rng = np.random.default_rng(ex["seed"])
    d, n = ex["d"], ex["pairs"]
    keys = []
    for _ in range(n):
        x = rng.standard_normal(d)
        keys.append(x / np.linalg.norm(x))
    vals = [rng.standard_normal(d) for _ in range(n)]
    new_val = rng.standard_normal(d)
    rk, pk = ex["rewrite_key"], ex["probe_key"]
    K = np.array(keys + [keys[rk]])[:, None, :]
    V = np.array(vals + [new_val])[:, None, :]
    T = K.shape[0]
    g = np.zeros((T, 1, d))
    beta = np.ones((T, 1))

    def rel(S, key, target):
        return np.linalg.norm(S.T @ key - target) / np.linalg.norm(target)

    for name, delta in (("linear_attention", False), ("delta_rule", True)):
        _, S = oracle_mod.prefill(K, K, V, g, beta, delta=delta)
        S = S[0, 0]
        got = (round(rel(S, keys[rk], new_val), ex["decimals"]),
               round(rel(S, keys[pk], vals[pk]), ex["decimals"]))
        want = (ex[name]["rewritten_key_error"], ex[name]["probe_key_error"])
        assert got == pytest.approx(want, abs=1e-9), name


# --------------------------------------------------------------------------
# P8: with unit keys, beta in [0,1], g <= 0 and v = 0 every step is a
# contraction, so ||S_t||_F never grows (the erase factor has eigenvalues 1
# and 1 - beta; the fade has entries in (0, 1]).
# --------------------------------------------------------------------------
def test_p8_contraction_invariant(oracle_mod):
    rng = np.random.default_rng(8)
    N, H, dk, dv = 3, 4, 8, 6
    S = rng.standard_normal((N, H, dk, dv))
    prev = np.linalg.norm(S, axis=(2, 3))
    for _ in range(20):
        q = _unit(rng.standard_normal((N, H, dk)))
        k = _unit(rng.standard_normal((N, H, dk)))
        v = np.zeros((N, H, dv))
        g = -rng.random((N, H, dk))
        beta = rng.random((N, H))
        _, S = oracle_mod.decode_step(q, k, v, g, beta, S)
        cur = np.linalg.norm(S, axis=(2, 3))
        assert np.all(cur <= prev * (1 + 1e-15))
        prev = cur


# --------------------------------------------------------------------------
# P9: the update is affine in (S, v), so outputs and states superpose.
# --------------------------------------------------------------------------
def test_p9_superposition(oracle_mod):
    rng = np.random.default_rng(9)
    T, H, dk, dv = 14, 2, 5, 6
    q, k, v1, g, beta = _rand_inputs(rng, T, H, dk, dv)
    v2 = rng.standard_normal((T, H, dv))
    S0 = rng.standard_normal((1, H, dk, dv))
    o12, S12 = oracle_mod.prefill(q, k, v1 + v2, g, beta, initial_state=S0)
    o1, S1 = oracle_mod.prefill(q, k, v1, g, beta, initial_state=S0)
    o2, S2 = oracle_mod.prefill(q, k, v2, g, beta)
    np.testing.assert_allclose(o12, o1 + o2, atol=1e-12)
    np.testing.assert_allclose(S12, S1 + S2, atol=1e-12)


# --------------------------------------------------------------------------
# P10: entry points agree -- decode step == prefill of one token; a split
# prefill resumed from the carried state == the whole prefill (the prefix
# reuse of the Inside Kimi K3 page needs exactly this); packing == separate.
# --------------------------------------------------------------------------
def test_p10_decode_equals_prefill_one_token(oracle_mod):
    rng = np.random.default_rng(10)
    N, H, dk, dv = 3, 2, 5, 4
    q, k, v, g, beta = _rand_inputs(rng, N, H, dk, dv)   # one token per sequence
    S0 = rng.standard_normal((N, H, dk, dv))
    od, Sd = oracle_mod.decode_step(q, k, v, g, beta, S0, scale=0.5)
    cu = np.arange(N + 1, dtype=np.int64)
    op, Sp = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu, scale=0.5)
    np.testing.assert_array_equal(od, op)
    np.testing.assert_array_equal(Sd, Sp)


def test_p10_split_resume_and_packing(oracle_mod):
    rng = np.random.default_rng(12)
    T1, T2, H, dk, dv = 7, 9, 2, 4, 5
    q, k, v, g, beta = _rand_inputs(rng, T1 + T2, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, S = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0)
    oa, Sa = oracle_mod.prefill(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], initial_state=S0)
    ob, Sb = oracle_mod.prefill(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], initial_state=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(Sb, S, rtol=0, atol=1e-15)
    # packed = separate
    cu = np.array([0, T1, T1 + T2], dtype=np.int64)
    S0p = np.concatenate([S0, Sa])
    op, Sp = oracle_mod.prefill(q, k, v, g, beta, initial_state=S0p, cu_seqlens=cu)
    np.testing.assert_array_equal(op[:T1], oa)
    np.testing.assert_array_equal(op[T1:], oracle_mod.prefill(
        q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], initial_state=Sa)[0])
    np.testing.assert_array_equal(Sp[1], Sb[0])


def test_oracle_rejects_bad_cu(oracle_mod):
    q = np.zeros((4, 1, 2)); v = np.zeros((4, 1, 2)); beta = np.zeros((4, 1))
    with pytest.raises(ValueError):
        oracle_mod.prefill(q, q, v, q, beta, cu_seqlens=np.array([0, 3, 2, 4]))


# --------------------------------------------------------------------------
# P11: state checkpoints at token boundaries (prefix reuse restores the KDA
# state at a token boundary: Inside Kimi K3, "Sequence mixing").  With
# beta = 0 the state after t tokens of a sequence is exp(sum of its first t
# g rows) applied to the key rows of its initial state, so every checkpoint
# has a closed form; a boundary off by one token changes the exponent.
# --------------------------------------------------------------------------
def test_p11_checkpoints_pure_decay_closed_form(oracle_mod):
    rng = np.random.default_rng(13)
    lengths = [10, 0, 25, 15, 4]
    interval = 5
    T, H, dk, dv = sum(lengths), 2, 3, 4
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=0.7)
    beta[:] = 0.0
    N = len(lengths)
    S0 = rng.standard_normal((N, H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    ck, first = oracle_mod.prefill_checkpoints(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu,
                                               interval=interval)
    assert list(first) == [0, 2, 2, 7, 10, 10]
    assert ck.shape == (10, H, dk, dv)
    for n in range(N):
        for j in range(lengths[n] // interval):
            t = (j + 1) * interval
            G = g[cu[n]:cu[n] + t].sum(axis=0)  # [H, dk]
            for h in range(H):
                np.testing.assert_allclose(ck[first[n] + j, h], np.exp(G[h])[:, None] * S0[n, h],
                                           rtol=1e-13, atol=0)


def test_p11b_last_checkpoint_is_final_state(oracle_mod):
    rng = np.random.default_rng(14)
    lengths = [12, 8]
    T, H, dk, dv = sum(lengths), 1, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    cu = np.array([0, 12, 20], dtype=np.int64)
    ck, first = oracle_mod.prefill_checkpoints(q, k, v, g, beta, cu_seqlens=cu, interval=4)
    _, S = oracle_mod.prefill(q, k, v, g, beta, cu_seqlens=cu)
    assert list(first) == [0, 3, 5]
    np.testing.assert_array_equal(ck[2], S[0])
    np.testing.assert_array_equal(ck[4], S[1])


# --------------------------------------------------------------------------
# P12: the fused input preparation (Understanding Kimi K3's attention: q, k
# L2-normalised in the symbol table; g = g_min Sigmoid(e^{A_h} z) with
# g_min = -5 in the gate equation).  Special values of the logistic pin the
# sign, the e^{A_h} factor and g_min; rescaling q and k per (token, head) by
# positive factors must change nothing; the gate's inverse must give back a
# chosen g through the already pinned recurrence.
# --------------------------------------------------------------------------
def test_p12a_gate_special_values(oracle_mod):
    ln3 = np.log(3.0)
    z = np.array([0.0, ln3, -ln3, ln3 / 2, 60.0, -60.0]).reshape(6, 1, 1)
    a = np.array([0.0])
    g = oracle_mod.gate(z, a)[:, 0, 0]
    np.testing.assert_allclose(g[:4], [-2.5, -3.75, -1.25, -5.0 / (1 + 3 ** -0.5)], rtol=1e-15)
    assert abs(g[4] + 5.0) <= 1e-20 and -1e-20 <= g[5] <= 0.0  # the limits g_min and 0
    # e^{A_h}: A = ln 2 doubles the logit
    g2 = oracle_mod.gate(np.full((1, 1, 1), ln3 / 2), np.array([np.log(2.0)]))
    np.testing.assert_allclose(g2[0, 0, 0], -3.75, rtol=1e-15)
    # one A per head, broadcast over tokens and channels
    g3 = oracle_mod.gate(np.zeros((2, 3, 4)) + ln3, np.log(np.array([1.0, 2.0, 0.5])))
    np.testing.assert_allclose(g3[:, 1, :], -5.0 / (1 + 1 / 9.0), rtol=1e-15)
    np.testing.assert_allclose(g3[:, 2, :], -5.0 / (1 + 3 ** -0.5), rtol=1e-15)


def test_p12b_l2norm_scale_invariance_and_zero(oracle_mod):
    rng = np.random.default_rng(15)
    T, H, dk, dv = 9, 2, 5, 3
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    z = rng.standard_normal((T, H, dk))
    a = rng.standard_normal(H) * 0.3
    beta = rng.random((T, H))
    o1, S1 = oracle_mod.prefill_fused(q, k, v, z, a, beta)
    cq = np.exp(rng.standard_normal((T, H, 1)))
    ck = np.exp(rng.standard_normal((T, H, 1)))
    o2, S2 = oracle_mod.prefill_fused(q * cq, k * ck, v, z, a, beta)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-14)
    n = np.linalg.norm(oracle_mod.l2norm(q), axis=-1)
    np.testing.assert_allclose(n, 1.0, rtol=1e-15)
    q0 = q.copy(); q0[4, 1] = 0.0
    o3, _ = oracle_mod.prefill_fused(q0, k, v, z, a, beta)
    assert np.all(o3[4, 1] == 0.0)


def test_p12c_inverse_gate_matches_plain_prefill(oracle_mod):
    rng = np.random.default_rng(16)
    T, H, dk, dv = 11, 2, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=4.0)
    g = np.clip(g, -4.99, -1e-3)
    a = np.array([0.4, -0.7])
    z = -np.log(-5.0 / g - 1.0) / np.exp(a)[None, :, None]   # Sigmoid^{-1}(g / g_min) / e^{A}
    of, Sf = oracle_mod.prefill_fused(q, k, v, z, a, beta)
    op, Sp = oracle_mod.prefill(q, k, v, g, beta)
    np.testing.assert_allclose(of, op, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(Sf, Sp, rtol=1e-10, atol=1e-13)


# --------------------------------------------------------------------------
# P13: the output gate Sigmoid(gate) * RMSNorm(o) (Understanding Kimi K3's
# attention, output equation).  A constant row normalises to its sign; a
# one-hot row of length d has RMS |a| / sqrt(d) (a sum in place of the mean
# fails); Sigmoid(0) = 1/2 and Sigmoid(ln 3) = 3/4; the weight acts per
# channel; eps enters under the root.
# --------------------------------------------------------------------------
def test_p13_output_gate_closed_forms(oracle_mod):
    d = 8
    w = np.arange(1, d + 1, dtype=np.float64) / 4.0
    o = np.full((2, 1, d), -3.0)
    gate = np.zeros((2, 1, d))
    y = oracle_mod.output_gate(o, gate, w, 0.0)
    np.testing.assert_allclose(y, np.broadcast_to(-0.5 * w, y.shape), rtol=1e-15)
    oh = np.zeros((1, 1, d)); oh[0, 0, 3] = 2.5
    g3 = np.full((1, 1, d), np.log(3.0))
    y = oracle_mod.output_gate(oh, g3, w, 0.0)
    expect = np.zeros(d); expect[3] = np.sqrt(d) * w[3] * 0.75
    np.testing.assert_allclose(y[0, 0], expect, rtol=1e-14, atol=0)
    # eps under the root: row (1, 1, ..., 1) with eps = 3 -> 1 / sqrt(1 + 3) = 1/2
    y = oracle_mod.output_gate(np.ones((1, 1, d)), np.full((1, 1, d), 50.0), np.ones(d), 3.0)
    np.testing.assert_allclose(y, 0.5, rtol=1e-15)
    # zero row with eps > 0 stays zero
    assert np.all(oracle_mod.output_gate(np.zeros((1, 1, d)), np.zeros((1, 1, d)), w, 1e-6) == 0.0)


# --------------------------------------------------------------------------
# P14: the backward oracle against central finite differences of the forward
# oracle (itself pinned by P1-P10), for every input of a tiny packed batch with
# an initial state, an output gradient and a final-state gradient.  The
# chunkwise form's gradients are checked against the token recurrence's
# ("Hybrid Attention", section "But isn't a recurrent update sequential?");
# these are the recurrence's.  seg_len = 2 makes the backward recompute the
# forward from stored states at every other token.
# --------------------------------------------------------------------------
def _bwd_case(rng, lengths, H, dk, dv):
    T = sum(lengths)
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=1.5)
    N = len(lengths)
    S0 = 0.5 * rng.standard_normal((N, H, dk, dv))
    d_o = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((N, H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return [q, k, v, g, beta, S0], d_o, dST, cu


@pytest.mark.parametrize("seg_len", [2, 0])
def test_p14_backward_finite_differences(oracle_mod, seg_len):
    rng = np.random.default_rng(21)
    inputs, d_o, dST, cu = _bwd_case(rng, [5, 0, 3], 2, 3, 2)
    scale = 0.7

    def loss(args):
        o, S = oracle_mod.prefill(*args[:5], initial_state=args[5], cu_seqlens=cu, scale=scale)
        return float(np.sum(d_o * o) + np.sum(dST * S))

    grads = oracle_mod.prefill_backward(*inputs[:5], d_o, initial_state=inputs[5], d_final_state=dST,
                                        cu_seqlens=cu, scale=scale, seg_len=seg_len)
    h = 1e-6
    for idx, (x, gx) in enumerate(zip(inputs, grads)):
        fd = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            saved = x[pos]
            x[pos] = saved + h
            lp = loss(inputs)
            x[pos] = saved - h
            lm = loss(inputs)
            x[pos] = saved
            fd[pos] = (lp - lm) / (2 * h)
        assert gx.shape == x.shape
        np.testing.assert_allclose(gx, fd, rtol=0, atol=1e-7 * max(1.0, np.max(np.abs(fd)))), idx


# --------------------------------------------------------------------------
# P15: the same gradients by torch's fp64 autograd through a plain loop over
# the product form S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T, o = scale
# S_t^T q (Understanding Kimi K3's attention, state-update and readout
# equations), at lengths that cross the backward's 64-token segments, with
# an empty sequence and a one-token one.
# --------------------------------------------------------------------------
def test_p15_backward_matches_autograd(oracle_mod):
    import torch
    rng = np.random.default_rng(22)
    lengths = [150, 0, 70, 1]
    H, dk, dv = 2, 6, 5
    inputs, d_o, dST, cu = _bwd_case(rng, lengths, H, dk, dv)
    scale = 0.9
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in inputs]
    q, k, v, g, beta, S0 = ts
    eye = torch.eye(dk, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    for n in range(len(lengths)):
        for h in range(H):
            S = S0[n, h]
            for t in range(int(cu[n]), int(cu[n + 1])):
                kk = k[t, h]
                S = (eye - beta[t, h] * torch.outer(kk, kk)) @ (torch.exp(g[t, h])[:, None] * S) \
                    + beta[t, h] * torch.outer(kk, v[t, h])
                loss = loss + torch.dot(torch.tensor(d_o[t, h]), scale * (S.T @ q[t, h]))
            loss = loss + torch.sum(torch.tensor(dST[n, h]) * S)
    loss.backward()
    grads = oracle_mod.prefill_backward(*inputs[:5], d_o, initial_state=inputs[5], d_final_state=dST,
                                        cu_seqlens=cu, scale=scale)
    for t, gx in zip(ts, grads):
        ref = t.grad.numpy()
        np.testing.assert_allclose(gx, ref, rtol=0, atol=1e-11 * max(1.0, np.max(np.abs(ref))))
