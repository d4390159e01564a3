"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics (CPU only).

Each test checks the oracle against something other than itself: printed worked examples,
closed forms, exact rational brute force, invariants and special cases that reduce to a
second, independently printed statement of the loop or to library routines.
"""

import math
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def _scalar_run(S0, v, beta, alpha, n, lib=None):
    """d_k = d_v = 1, k = q = 1, scale 1, the same (v, beta, alpha) repeated n times."""
    q = np.ones((n, 1, 1)); k = np.ones((n, 1, 1)); vv = np.full((n, 1, 1), v)
    g = np.full((n, 1), math.log(alpha)); b = np.full((n, 1), beta)
    o, fin, _ = oracle.recurrence(q, k, vv, g, b, [0, n], 1.0,
                                  initial_state=np.full((1, 1, 1, 1), S0), lib=lib)
    return o[:, 0, 0], fin[0, 0, 0, 0]


# ---------------------------------------------------------------------------------------
# 1. the pages' worked scalar examples
# ---------------------------------------------------------------------------------------

def test_golden_scalar_examples():
    rows = _read_golden("scalar_delta_rule.txt")
    assert len(rows) == 2
    for row in rows:
        name, S0, v, beta, alpha, outs = [x.strip() for x in row.split("|")]
        expect = [float(x) for x in outs.split()]
        o, fin = _scalar_run(float(S0), float(v), float(beta), float(alpha), len(expect))
        if alpha == "1.0":
            # no decay: exact in binary floating point
            assert list(o) == expect, name
        else:
            np.testing.assert_allclose(o, expect, rtol=0, atol=1e-14, err_msg=name)
        assert fin == o[-1]


def test_scalar_examples_discriminate_orderings():
    """The decayed example separates the two printed orderings of the update.

    Correcting the undecayed memory (alpha*S + beta*(v - S)) gives 0.5*6 + 0.5*(10-6) = 5,
    not the page's 6.5; reading the output before the update gives 6, not 8.
    """
    S0, v, beta, alpha = 6.0, 10.0, 0.5, 0.5
    undecayed_correction = alpha * S0 + beta * (v - S0)
    assert undecayed_correction == 5.0
    o, _ = _scalar_run(S0, v, beta, alpha, 1)
    assert abs(o[0] - 6.5) < 1e-14 and abs(o[0] - undecayed_correction) > 1


# ---------------------------------------------------------------------------------------
# 2. closed form for a repeated (k, v, alpha, beta) with |k| = 1
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("alpha,beta", [(1.0, 0.5), (0.5, 0.5), (0.9, 0.3), (0.97, 0.99)])
def test_closed_form_repeated_pair(alpha, beta):
    rng = np.random.default_rng(5)
    d_k, d_v, n = 6, 4, 60
    kk = rng.standard_normal(d_k); kk /= np.linalg.norm(kk)
    vv = rng.standard_normal(d_v)
    S0 = rng.standard_normal((d_v, d_k))
    q = np.tile(kk, (n, 1, 1)); k = np.tile(kk, (n, 1, 1)); v = np.tile(vv, (n, 1, 1))
    g = np.full((n, 1), math.log(alpha)); b = np.full((n, 1), beta)
    _, _, traj = oracle.recurrence(q, k, v, g, b, [0, n], 1.0,
                                   initial_state=S0[None, None], want_traj=True)
    rho = alpha * (1 - beta)
    x_star = beta * vv / (1 - rho)
    for t in range(n):
        expect = x_star + rho ** (t + 1) * (S0 @ kk - x_star)
        np.testing.assert_allclose(traj[0, t] @ kk, expect, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------
# 3. exact rational brute force (unrolled products) on tiny packed batches
# ---------------------------------------------------------------------------------------

_UNIT_KEYS3 = [(Fraction(3, 5), Fraction(4, 5), Fraction(0)),
               (Fraction(0), Fraction(5, 13), Fraction(12, 13)),
               (Fraction(2, 3), Fraction(1, 3), Fraction(2, 3)),
               (Fraction(2, 7), Fraction(-3, 7), Fraction(6, 7)),
               (Fraction(-1, 3), Fraction(2, 3), Fraction(2, 3)),
               (Fraction(0), Fraction(-1), Fraction(0))]


def _rational_case(seed, seq_lens, h_qk, h_v, d_k=3, d_v=2):
    """Random rational inputs with unit keys; returns Fraction lists and float64 arrays."""
    rng = np.random.default_rng(seed)
    T = sum(seq_lens)
    fr = lambda: Fraction(int(rng.integers(-9, 10)), int(rng.integers(1, 8)))
    k = [[list(_UNIT_KEYS3[int(rng.integers(len(_UNIT_KEYS3)))]) for _ in range(h_qk)]
         for _ in range(T)]
    q = [[[fr() for _ in range(d_k)] for _ in range(h_qk)] for _ in range(T)]
    v = [[[fr() for _ in range(d_v)] for _ in range(h_v)] for _ in range(T)]
    alpha = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(h_v)] for _ in range(T)]
    beta = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(h_v)] for _ in range(T)]
    S0 = [[[[fr() for _ in range(d_k)] for _ in range(d_v)] for _ in range(h_v)]
          for _ in range(len(seq_lens))]
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, S0=S0)


@pytest.mark.parametrize("seed,seq_lens,h_qk,h_v", [
    (1, [8], 1, 1),
    (2, [3, 5], 1, 2),
    (3, [0, 4, 4], 2, 4),
    (4, [1, 7], 2, 2),
])
def test_brute_force_exact(seed, seq_lens, h_qk, h_v):
    d_k, d_v = 3, 2              # non-square state: a transposed S fails
    c = _rational_case(seed, seq_lens, h_qk, h_v, d_k, d_v)
    scale = Fraction(1, 2)
    cu = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int64)
    f = lambda x: np.array(x, dtype=object).astype(np.float64)
    o, fin, _ = oracle.recurrence(
        f(c["q"]), f(c["k"]), f(c["v"]),
        np.log(f(c["alpha"])), f(c["beta"]), cu, float(scale), initial_state=f(c["S0"]))
    group = h_v // h_qk
    for n in range(len(seq_lens)):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for h in range(h_v):
            j = h // group       # V head h reads QK head h // (h_v / h_qk)
            sl = range(t0, t1)
            states, outs = brute.unrolled_chain(
                c["S0"][n][h], [c["q"][t][j] for t in sl], [c["k"][t][j] for t in sl],
                [c["v"][t][h] for t in sl], [c["alpha"][t][h] for t in sl],
                [c["beta"][t][h] for t in sl], scale)
            final = states[-1] if states else c["S0"][n][h]
            np.testing.assert_allclose(fin[n, h], f(final), rtol=1e-13, atol=1e-14)
            for i, t in enumerate(sl):
                np.testing.assert_allclose(o[t, h], f(outs[i]), rtol=1e-13, atol=1e-14)


def test_brute_force_forms_agree_exactly():
    """The rank-1 per-token form equals the multiplied-out transition form, exactly."""
    c = _rational_case(11, [6], 1, 1)
    args = (c["S0"][0][0], [x[0] for x in c["q"]], [x[0] for x in c["k"]],
            [x[0] for x in c["v"]], [x[0] for x in c["alpha"]], [x[0] for x in c["beta"]],
            Fraction(3, 4))
    s1, o1 = brute.unrolled_chain(*args)
    s2, o2 = brute.rank1_chain(*args)
    assert s1 == s2 and o1 == o2


# ---------------------------------------------------------------------------------------
# 4-5. per-step identity and state-norm bound along a trajectory
# ---------------------------------------------------------------------------------------

def _traj_case(T=96, d=16, beta_one=False, seed=3):
    x = workloads.make_prefill([T], h_qk=1, h_v=1, d_k=d, d_v=d, io_dtype="bf16",
                               with_initial_state=True, seed=seed, state_std=0.5)
    q, k, v = x.as_f64("q"), x.as_f64("k"), x.as_f64("v")
    beta = np.ones_like(x.as_f64("beta")) if beta_one else x.as_f64("beta")
    g = x.as_f64("g")
    S0 = x.as_f64("initial_state")
    _, _, traj = oracle.recurrence(q, k, v, g, beta, x.cu_seqlens, x.scale,
                                   initial_state=S0, want_traj=True)
    prev = np.concatenate([S0[0], traj[0, :-1]], axis=0)   # S_{t-1}
    return q[:, 0], k[:, 0], v[:, 0], np.exp(g[:, 0]), beta[:, 0], prev, traj[0]


def test_per_step_identity():
    """S_t k_t = alpha(1 - beta |k|^2) S_{t-1} k_t + beta |k|^2 v_t at every step."""
    q, k, v, a, b, prev, cur = _traj_case()
    for t in range(len(a)):
        kk = k[t] @ k[t]      # bf16 keys are only near-unit
        lhs = cur[t] @ k[t]
        rhs = a[t] * (1 - b[t] * kk) * (prev[t] @ k[t]) + b[t] * kk * v[t]
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-13)


def test_beta_one_stores_value():
    """beta = 1 with a unit key writes v exactly at that key: S_t k_t = v_t."""
    d = 4
    rng = np.random.default_rng(8)
    keys = np.array([[1, 0, 0, 0], [0, 0.6, 0.8, 0], [0.5, 0.5, 0.5, 0.5]], dtype=np.float64)
    T = len(keys)
    v = rng.standard_normal((T, 1, d))
    g = np.log(np.array([[0.3], [0.9], [0.5]]))
    _, _, traj = oracle.recurrence(keys[:, None], keys[:, None], v, g, np.ones((T, 1)),
                                   [0, T], 1.0, initial_state=rng.standard_normal((1, 1, d, d)),
                                   want_traj=True)
    for t in range(T):
        np.testing.assert_allclose(traj[0, t] @ keys[t], v[t, 0], rtol=0, atol=1e-15)


def test_state_norm_bound():
    """|S_t|_F <= alpha_t |S_{t-1}|_F + beta_t |v_t| |k_t| for beta |k|^2 in [0, 2]."""
    q, k, v, a, b, prev, cur = _traj_case(T=200, d=32, seed=9)
    assert np.all(b * np.sum(k * k, axis=1) <= 2)
    for t in range(len(a)):
        lhs = np.linalg.norm(cur[t])
        rhs = a[t] * np.linalg.norm(prev[t]) + b[t] * np.linalg.norm(v[t]) * np.linalg.norm(k[t])
        assert lhs <= rhs * (1 + 1e-12), t


# ---------------------------------------------------------------------------------------
# 6. state size does not grow with the number of tokens
# ---------------------------------------------------------------------------------------

def test_golden_state_vs_cache_sizes():
    vals = dict(row.split() for row in _read_golden("state_vs_cache.txt"))
    state_numbers = int(vals["state_numbers"])
    per_token, tokens = int(vals["cache_per_token"]), int(vals["tokens"])
    assert per_token * tokens == int(vals["cache_at_tokens"])
    d = int(math.isqrt(state_numbers))          # a 16 x 16 state holds 256 numbers
    sizes = []
    for T in (1, 64, tokens, 4096):
        x = workloads.make_prefill([T], h_qk=1, h_v=1, d_k=d, d_v=d, seed=T)
        _, fin, _ = oracle.recurrence(x.as_f64("q"), x.as_f64("k"), x.as_f64("v"),
                                      x.as_f64("g"), x.as_f64("beta"), x.cu_seqlens, x.scale)
        sizes.append(fin[0, 0].size)
        assert np.all(np.isfinite(fin))
    assert sizes == [state_numbers] * 4


def test_golden_head_shape_matches_workloads():
    vals = dict(row.split() for row in _read_golden("gdn_heads.txt"))
    assert int(vals["v_heads"]) == workloads.H_V
    assert int(vals["qk_heads"]) == workloads.H_QK
    assert int(vals["head_dim"]) == workloads.D_HEAD


# ---------------------------------------------------------------------------------------
# 7. special cases
# ---------------------------------------------------------------------------------------

def test_beta_zero_is_pure_decay():
    x = workloads.make_prefill([40], h_qk=2, h_v=4, d_k=8, d_v=6, io_dtype="f32",
                               with_initial_state=True, seed=4)
    g = x.as_f64("g")
    S0 = x.as_f64("initial_state")
    o, fin, _ = oracle.recurrence(x.as_f64("q"), x.as_f64("k"), x.as_f64("v"), g,
                                  np.zeros_like(g), x.cu_seqlens, x.scale, initial_state=S0)
    cum = np.exp(np.cumsum(g, axis=0))          # [T][h_v]
    np.testing.assert_allclose(fin[0], cum[-1][:, None, None] * S0[0], rtol=1e-13)
    q = x.as_f64("q")
    for h in range(4):
        expect = x.scale * cum[:, h, None] * (q[:, h // 2] @ S0[0, h].T)
        np.testing.assert_allclose(o[:, h], expect, rtol=1e-12, atol=1e-15)


def _product_form(Q, K, V, beta, S0):
    """States and read-outs of one chain at alpha = 1 from the transition-matrix product
    (not from the per-token rank-1 update): with M_t = I - beta_t k_t k_t^T,
        S_t = S_0 M_1 ... M_t + sum_{s <= t} beta_s v_s k_s^T M_{s+1} ... M_t,
    every S_t formed from scratch by numpy matrix products, and o_t = S_t q_t."""
    T, d_k = K.shape
    Ms = [np.eye(d_k) - beta[t] * np.outer(K[t], K[t]) for t in range(T)]
    outs, S = [], None
    for t in range(T):
        P = np.eye(d_k)
        S = np.zeros_like(S0)
        for s in range(t, -1, -1):          # P = M_{s+1} ... M_t, built from the right
            S = S + beta[s] * np.outer(V[s], K[s]) @ P
            P = Ms[s] @ P
        S = S + S0 @ P
        outs.append(S @ Q[t])
    return np.stack(outs), S


def test_alpha_one_matches_product_form():
    """At alpha = 1 (no decay) the oracle equals the transition-matrix product form of the
    update, at a float size (T = 50, d_k = 12, d_v = 10) beyond the exact brute force."""
    x = workloads.make_prefill([50], h_qk=1, h_v=1, d_k=12, d_v=10, io_dtype="f32",
                               with_initial_state=True, seed=12)
    q, k, v, b = x.as_f64("q"), x.as_f64("k"), x.as_f64("v"), x.as_f64("beta")
    s0 = x.as_f64("initial_state")
    o, fin, _ = oracle.recurrence(q, k, v, np.zeros_like(b), b, x.cu_seqlens, 1.0,
                                  initial_state=s0)
    o_ref, S = _product_form(q[:, 0], k[:, 0], v[:, 0], b[:, 0], s0[0, 0])
    np.testing.assert_allclose(o[:, 0], o_ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-11, atol=1e-13)


def test_chaining_and_varlen_and_zero_length():
    """Two halves through the returned state equal the whole; packed equals separate;
    an empty sequence returns its initial state."""
    x = workloads.make_prefill([37, 0, 70], h_qk=2, h_v=4, d_k=8, d_v=8, io_dtype="f32",
                               with_initial_state=True, seed=21)
    a = {n: x.as_f64(n) for n in ("q", "k", "v", "g", "beta", "initial_state")}
    o, fin, _ = oracle.recurrence(a["q"], a["k"], a["v"], a["g"], a["beta"], x.cu_seqlens,
                                  x.scale, initial_state=a["initial_state"])
    np.testing.assert_array_equal(fin[1], a["initial_state"][1])
    t0 = 37
    for split in (1, 30, 69):
        sl1, sl2 = slice(t0, t0 + split), slice(t0 + split, t0 + 70)
        o1, f1, _ = oracle.recurrence(*(a[n][sl1] for n in ("q", "k", "v", "g", "beta")),
                                      [0, split], x.scale, initial_state=a["initial_state"][2:3])
        o2, f2, _ = oracle.recurrence(*(a[n][sl2] for n in ("q", "k", "v", "g", "beta")),
                                      [0, 70 - split], x.scale, initial_state=f1)
        np.testing.assert_allclose(np.concatenate([o1, o2]), o[t0:t0 + 70], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(f2[0], fin[2], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------------------
# 8. front end against library routines
# ---------------------------------------------------------------------------------------

def _front_end_torch(mixed, w, cu, h_qk, h_v, d_k, d_v, q_scale):
    """Independent statement with torch library routines (CPU, float64): depthwise conv1d
    with (K-1) zeros of left padding per sequence, F.silu, F.normalize (eps 1e-12)."""
    x = torch.from_numpy(mixed)
    W = torch.from_numpy(w)
    C, K = W.shape
    outs = []
    for n in range(len(cu) - 1):
        seg = x[cu[n]:cu[n + 1]].T[None]                    # [1][C][T_n]
        if seg.shape[-1] == 0:
            continue
        y = torch.nn.functional.conv1d(torch.nn.functional.pad(seg, (K - 1, 0)), W[:, None, :],
                                       groups=C)
        outs.append(torch.nn.functional.silu(y[0].T))
    z = torch.cat(outs)
    T = z.shape[0]
    nq = h_qk * d_k
    q = torch.nn.functional.normalize(z[:, :nq].reshape(T, h_qk, d_k), dim=-1) * q_scale
    k = torch.nn.functional.normalize(z[:, nq:2 * nq].reshape(T, h_qk, d_k), dim=-1)
    v = z[:, 2 * nq:].reshape(T, h_v, d_v)
    return q.numpy(), k.numpy(), v.numpy()


@pytest.mark.parametrize("seq_lens", [[10], [0, 1, 3, 10], [2, 2, 5]])
def test_front_end_matches_torch(seq_lens):
    h_qk, h_v, d_k, d_v = 2, 4, 8, 8
    fe = workloads.make_frontend(seq_lens, h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v, seed=31)
    mixed = workloads.bf16_bits_to_f32(fe.mixed).astype(np.float64)
    w = fe.conv_weight.astype(np.float64)
    q, k, v = oracle.conv_prep(mixed, w, fe.cu_seqlens, h_qk, h_v, d_k, d_v, fe.q_scale)
    qr, kr, vr = _front_end_torch(mixed, w, fe.cu_seqlens, h_qk, h_v, d_k, d_v, fe.q_scale)
    for a, b in ((q, qr), (k, kr), (v, vr)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_front_end_closed_forms():
    """Only the current-token tap set: z = silu(x); normalised heads have unit norm."""
    h_qk, h_v, d = 1, 2, 4
    fe = workloads.make_frontend([5, 3], h_qk=h_qk, h_v=h_v, d_k=d, d_v=d, seed=2)
    mixed = workloads.bf16_bits_to_f32(fe.mixed).astype(np.float64)
    w = np.zeros_like(fe.conv_weight, dtype=np.float64)
    w[:, -1] = 1.0
    q, k, v = oracle.conv_prep(mixed, w, fe.cu_seqlens, h_qk, h_v, d, d, 0.25)
    silu = mixed / (1 + np.exp(-mixed))
    np.testing.assert_allclose(v.reshape(8, -1), silu[:, 2 * d:], rtol=1e-15)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 0.25, rtol=1e-14)
    # history only: tap 0 sees the token three back, zero at each sequence start
    w2 = np.zeros_like(w)
    w2[:, 0] = 1.0
    _, _, v2 = oracle.conv_prep(mixed, w2, fe.cu_seqlens, h_qk, h_v, d, d, 1.0)
    v2 = v2.reshape(8, -1)
    assert np.all(v2[0:3] == 0) and np.all(v2[5:8] == 0)
    np.testing.assert_allclose(v2[3:5], silu[0:2, 2 * d:], rtol=1e-15)


# ---------------------------------------------------------------------------------------
# per-channel form (one decay per value channel, correction from the state before the
# decay: the code panel of section "01 . GatedDeltaNet(config)" of the Evolving Transformer)
# ---------------------------------------------------------------------------------------

def _channel_rational_case(seed, seq_lens, h_qk, h_v, d_k=3, d_v=2):
    c = _rational_case(seed, seq_lens, h_qk, h_v, d_k, d_v)
    rng = np.random.default_rng(seed + 1000)
    T = sum(seq_lens)
    c["alpha_rows"] = [[[Fraction(int(rng.integers(1, 9)), 8) for _ in range(d_v)] for _ in range(h_v)]
                       for _ in range(T)]
    return c


def _channel_brute_pass(seed, seq_lens, h_qk, h_v, lib=None):
    c = _channel_rational_case(seed, seq_lens, h_qk, h_v)
    scale = Fraction(1, 2)
    cu = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int64)
    f = lambda x: np.array(x, dtype=object).astype(np.float64)
    o, fin, _ = oracle.recurrence_channel(
        f(c["q"]), f(c["k"]), f(c["v"]), np.log(f(c["alpha_rows"])), f(c["beta"]), cu,
        float(scale), initial_state=f(c["S0"]), lib=lib)
    group = h_v // h_qk
    for n in range(len(seq_lens)):
        sl = range(int(cu[n]), int(cu[n + 1]))
        for h in range(h_v):
            j = h // group
            states, outs = brute.unrolled_chain_channel(
                c["S0"][n][h], [c["q"][t][j] for t in sl], [c["k"][t][j] for t in sl],
                [c["v"][t][h] for t in sl], [c["alpha_rows"][t][h] for t in sl],
                [c["beta"][t][h] for t in sl], scale)
            final = states[-1] if states else c["S0"][n][h]
            if not np.allclose(fin[n, h], f(final), rtol=1e-13, atol=1e-14):
                return False
            if len(sl) and not np.allclose(o[list(sl), h], f(outs), rtol=1e-13, atol=1e-14):
                return False
    return True


@pytest.mark.parametrize("seed,seq_lens,h_qk,h_v", [(21, [6], 1, 1), (22, [0, 3, 5], 1, 2),
                                                    (23, [4, 2], 2, 4)])
def test_channel_form_brute_force_exact(seed, seq_lens, h_qk, h_v):
    """Against the row-by-row unrolled product (exact rationals; d_k = 3, d_v = 2)."""
    assert _channel_brute_pass(seed, seq_lens, h_qk, h_v)


def test_channel_form_alpha_one_is_the_main_form():
    """With every decay 1 the two forms are one rule (decay first or not makes no difference)."""
    x = workloads.make_prefill([30, 7], h_qk=2, h_v=4, d_k=8, d_v=6, io_dtype="f32",
                               with_initial_state=True, seed=31)
    q, k, v, b = x.as_f64("q"), x.as_f64("k"), x.as_f64("v"), x.as_f64("beta")
    S0 = x.as_f64("initial_state")
    o1, f1, _ = oracle.recurrence(q, k, v, np.zeros_like(b), b, x.cu_seqlens, x.scale, initial_state=S0)
    o2, f2, _ = oracle.recurrence_channel(q, k, v, np.zeros(b.shape + (6,)), b, x.cu_seqlens,
                                          x.scale, initial_state=S0)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(f2, f1, rtol=1e-13, atol=1e-15)


def test_channel_form_equal_decays_map_onto_the_main_form():
    """With one decay a for every channel, a S + b (v - S k) k^T is the main form's
    a S + b' (v' - a S k) k^T at b' = b / a and v' = a v: the correction is taken from the
    state before the decay in one form and after it in the other."""
    x = workloads.make_prefill([25], h_qk=1, h_v=2, d_k=8, d_v=6, io_dtype="f32",
                               with_initial_state=True, seed=32)
    q, k, v, b, g = x.as_f64("q"), x.as_f64("k"), x.as_f64("v"), x.as_f64("beta"), x.as_f64("g")
    S0 = x.as_f64("initial_state")
    a = np.exp(g)                                   # [T][h_v]
    o1, f1, _ = oracle.recurrence_channel(q, k, v, np.repeat(g[:, :, None], 6, axis=2), b,
                                          x.cu_seqlens, x.scale, initial_state=S0)
    o2, f2, _ = oracle.recurrence(q, k, v * a[:, :, None], g, b / a, x.cu_seqlens, x.scale,
                                  initial_state=S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(f1, f2, rtol=1e-11, atol=1e-14)


def test_channel_form_beta_zero_is_row_decay():
    """beta = 0: row i of the state is scaled by the running product of its own decays (a
    decay applied to columns instead, or with the wrong channel index, fails this)."""
    x = workloads.make_prefill([20], h_qk=1, h_v=2, d_k=7, d_v=5, io_dtype="f32",
                               with_initial_state=True, seed=33)
    rng = np.random.default_rng(33)
    g = -np.abs(rng.standard_normal((20, 2, 5))) * 0.1
    S0 = x.as_f64("initial_state")
    q = x.as_f64("q")
    o, fin, _ = oracle.recurrence_channel(q, x.as_f64("k"), x.as_f64("v"), g,
                                          np.zeros((20, 2)), x.cu_seqlens, x.scale, initial_state=S0)
    cum = np.exp(np.cumsum(g, axis=0))              # [T][h_v][d_v]
    np.testing.assert_allclose(fin[0], cum[-1][:, :, None] * S0[0], rtol=1e-13)
    for h in range(2):
        expect = x.scale * cum[:, h, :] * (q[:, 0] @ S0[0, h].T)
        np.testing.assert_allclose(o[:, h], expect, rtol=1e-12, atol=1e-15)


_CH_MUTATIONS = {
    "channel: correction from the decayed state": ("const double ci = b * (vt[i] - u[i]);",
                                                   "const double ci = b * (vt[i] - ai * u[i]);"),
    "channel: decay by key channel": ("for (int j = 0; j < d_k; ++j) Si[j] = ai * Si[j] + ci * kt[j];",
                                      "for (int j = 0; j < d_k; ++j) Si[j] = exp(gt[j % d_v]) * Si[j] + ci * kt[j];"),
    "channel: no decay": ("const double ai = exp(gt[i]);", "const double ai = 1.0;"),
    "channel: read-out before the update": ("/* read-out after the update */\n        if (o) {",
                                            "/* mutated */\n        if (0) {"),
}


@pytest.fixture(scope="module")
def channel_mutant_libs():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")).read()
    libs = {}
    with tempfile.TemporaryDirectory() as td:
        for name, (a, b) in _CH_MUTATIONS.items():
            assert src.count(a) == 1, name
            path = os.path.join(td, "c%d.c" % len(libs))
            with open(path, "w") as f:
                f.write(src.replace(a, b))
            so = path[:-2] + ".so"
            subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                                   path, "-o", so, "-lm"])
            libs[name] = oracle.load_library(so)
        yield libs


@pytest.mark.parametrize("name", sorted(_CH_MUTATIONS))
def test_channel_pins_catch_planted_mistake(channel_mutant_libs, name):
    assert not _channel_brute_pass(22, [0, 3, 5], 1, 2, lib=channel_mutant_libs[name]), name


# ---------------------------------------------------------------------------------------
# planted mistakes: each plausible slip in the oracle fails at least one pin above
# ---------------------------------------------------------------------------------------

_MUTATIONS = {
    "correct against undecayed state": ("c = b * (vt[i] - a * u[i]);", "c = b * (vt[i] - u[i]);"),
    "no decay on the state": ("= a * S[(ptrdiff_t)i * d_k + j] + c * kt[j];",
                              "= S[(ptrdiff_t)i * d_k + j] + c * kt[j];"),
    "read-out before the update": ("/* o = scale * S q, read after the update */\n        if (o) {",
                                   "/* mutated */\n        if (0) {"),
    "transposed state in S k": ("s += S[(ptrdiff_t)i * d_k + j] * kt[j];",
                                "s += S[(ptrdiff_t)j * d_v + i] * kt[j];"),
    "wrong head mapping": ("const int j = h / (J->h_v / J->h_qk);", "const int j = h % J->h_qk;"),
    "scale dropped": ("ot[i] = scale * s;", "ot[i] = s;"),
}


@pytest.fixture(scope="module")
def mutant_libs():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")).read()
    libs = {}
    with tempfile.TemporaryDirectory() as td:
        for name, (a, b) in _MUTATIONS.items():
            assert src.count(a) == 1, name
            path = os.path.join(td, "m%d.c" % len(libs))
            with open(path, "w") as f:
                f.write(src.replace(a, b))
            so = path[:-2] + ".so"
            subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                                   path, "-o", so, "-lm"])
            libs[name] = oracle.load_library(so)
        yield libs


def _pins_pass(lib):
    o, _ = _scalar_run(6.0, 10.0, 0.5, 1.0, 3, lib=lib)
    if list(o) != [8.0, 9.0, 9.5]:
        return False
    o, _ = _scalar_run(6.0, 10.0, 0.5, 0.5, 1, lib=lib)
    if abs(o[0] - 6.5) > 1e-14:
        return False
    c = _rational_case(3, [0, 4, 4], 2, 4)
    cu = np.array([0, 0, 4, 8], dtype=np.int64)
    f = lambda x: np.array(x, dtype=object).astype(np.float64)
    o, fin, _ = oracle.recurrence(f(c["q"]), f(c["k"]), f(c["v"]), np.log(f(c["alpha"])),
                                  f(c["beta"]), cu, 0.5, initial_state=f(c["S0"]), lib=lib)
    for n in (1, 2):
        for h in range(4):
            sl = range(int(cu[n]), int(cu[n + 1]))
            states, outs = brute.unrolled_chain(
                c["S0"][n][h], [c["q"][t][h // 2] for t in sl], [c["k"][t][h // 2] for t in sl],
                [c["v"][t][h] for t in sl], [c["alpha"][t][h] for t in sl],
                [c["beta"][t][h] for t in sl], Fraction(1, 2))
            if not np.allclose(fin[n, h], f(states[-1]), rtol=1e-12, atol=1e-14):
                return False
            if not np.allclose(o[list(sl), h], f(outs), rtol=1e-12, atol=1e-14):
                return False
    return True


def test_pins_pass_on_the_oracle():
    assert _pins_pass(None)


@pytest.mark.parametrize("name", sorted(_MUTATIONS))
def test_pins_catch_planted_mistake(mutant_libs, name):
    assert not _pins_pass(mutant_libs[name]), name


# ---------------------------------------------------------------------------------------
# output epilogue: per-head RMS norm with the zero-centred scale (1 + w), then the gate
# ---------------------------------------------------------------------------------------

def _norm_pins(lib=None):
    """Every pin of gated_rmsnorm; returns the names of those that fail."""
    fails = []
    gr = lambda o, z, w, eps, gate: oracle.gated_rmsnorm(np.array(o, dtype=np.float64),
                                                        np.array(z, dtype=np.float64),
                                                        np.array(w, dtype=np.float64),
                                                        eps=eps, gate=gate, lib=lib)
    # worked by hand: x = (3, 4) has mean square 12.5, so x / rms = (3, 4) / sqrt(12.5)
    ref = np.array([3.0, 4.0]) / np.sqrt(12.5)
    out = gr([[[3.0, 4.0]]], [[[60.0, 60.0]]], [0.0, 0.0], 0.0, oracle.GATE_SIGMOID)[0, 0]
    if not np.allclose(out, ref, rtol=1e-14, atol=0):
        fails.append("hand example, gate open")
    # sigmoid(0) = 1/2; SiLU(0) = 0
    out = gr([[[3.0, 4.0]]], [[[0.0, 0.0]]], [0.0, 0.0], 0.0, oracle.GATE_SIGMOID)[0, 0]
    if not np.allclose(out, ref / 2, rtol=1e-14, atol=0):
        fails.append("sigmoid(0) = 1/2")
    out = gr([[[3.0, 4.0]]], [[[0.0, 0.0]]], [0.0, 0.0], 0.0, oracle.GATE_SILU)[0, 0]
    if not np.all(out == 0.0):
        fails.append("silu(0) = 0")
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly; SiLU multiplies by z. A constant
    # vector has rms equal to its value, so y = 1 and out is the gate itself.
    z = [np.log(3.0), -np.log(3.0)]
    out = gr([[[2.0, 2.0]]], [[z]], [0.0, 0.0], 0.0, oracle.GATE_SIGMOID)[0, 0]
    if not np.allclose(out, [0.75, 0.25], rtol=1e-14, atol=0):
        fails.append("sigmoid(+-ln 3)")
    out = gr([[[2.0, 2.0]]], [[z]], [0.0, 0.0], 0.0, oracle.GATE_SILU)[0, 0]
    if not np.allclose(out, [0.75 * np.log(3.0), -0.25 * np.log(3.0)], rtol=1e-14, atol=0):
        fails.append("silu(+-ln 3)")
    # zero-centred scale: weight w multiplies by (1 + w), so w = 0 is the identity scale
    out = gr([[[3.0, 4.0]]], [[[60.0, 60.0]]], [1.0, -0.5], 0.0, oracle.GATE_SIGMOID)[0, 0]
    if not np.allclose(out, ref * np.array([2.0, 0.5]), rtol=1e-14, atol=0):
        fails.append("scale 1 + w")
    # one head at a time: heads with proportional values give equal outputs (eps = 0), and
    # a change in one head leaves the other alone
    out = gr([[[3.0, 4.0], [30.0, 40.0]]], np.full((1, 2, 2), 60.0), [0.0, 0.0], 0.0,
             oracle.GATE_SIGMOID)[0]
    if not (np.allclose(out[0], ref, rtol=1e-14, atol=0) and np.allclose(out[1], ref, rtol=1e-14, atol=0)):
        fails.append("per-head norm")
    # closed form with eps: mean(out^2) = ms / (ms + eps) for an open gate and w = 0
    rng = np.random.Generator(np.random.PCG64(160))
    o = rng.standard_normal((5, 3, 128)) * 0.05
    eps = 1e-3
    out = gr(o, np.full(o.shape, 60.0), np.zeros(128), eps, oracle.GATE_SIGMOID)
    ms = np.mean(o * o, axis=-1)
    if not np.allclose(np.mean(out * out, axis=-1), ms / (ms + eps), rtol=1e-12, atol=0):
        fails.append("mean square with eps")
    # scale invariance without eps
    w = rng.standard_normal(128) * 0.1
    zz = rng.standard_normal(o.shape)
    b = gr(o * 37.0, zz, w, 0.0, oracle.GATE_SILU)
    c = gr(o, zz, w, 0.0, oracle.GATE_SILU)
    if not np.allclose(b, c, rtol=1e-12, atol=1e-15):
        fails.append("scale invariance")
    # all-zero read-out with eps > 0: zero out, no NaN
    out = gr(np.zeros((1, 1, 128)), np.ones((1, 1, 128)), np.zeros(128), 1e-6, oracle.GATE_SIGMOID)
    if not np.all(out == 0.0):
        fails.append("zero read-out")
    return fails


def test_gated_rmsnorm_pins():
    assert _norm_pins() == []


def test_gated_rmsnorm_rejects_unknown_gate():
    with pytest.raises(ValueError):
        oracle.gated_rmsnorm(np.ones((1, 1, 4)), np.ones((1, 1, 4)), np.zeros(4), gate=2)


_NORM_MUTATIONS = {
    "norm: sum instead of mean": ("    ms /= d_v;\n", "    ms /= 1;\n"),
    "norm: weight without the zero-centred 1": ("* (1.0 + weight[i]);", "* (weight[i]);"),
    "norm: no square root": ("const double inv_rms = 1.0 / sqrt(ms + eps);",
                             "const double inv_rms = 1.0 / (ms + eps);"),
    "norm: over all heads of a row": ("const size_t base = ((size_t)r * h_v + h) * d_v;",
                                      "const size_t base = ((size_t)r * h_v + 0) * d_v + (size_t)h * 0;"),
    "gate: sign of the sigmoid": ("const double sig = 1.0 / (1.0 + exp(-zi));",
                                  "const double sig = 1.0 / (1.0 + exp(zi));"),
    "gate: sigmoid and SiLU swapped": ("out[base + i] = y * (gate == 0 ? sig : zi * sig);",
                                       "out[base + i] = y * (gate == 1 ? sig : zi * sig);"),
    "norm of the gated read-out": ("for (int i = 0; i < d_v; ++i) ms += o[base + i] * o[base + i];",
                                   "for (int i = 0; i < d_v; ++i) { const double gz = 1.0 / (1.0 + exp(-z[base + i])); "
                                   "ms += o[base + i] * gz * o[base + i] * gz; }"),
}


@pytest.fixture(scope="module")
def norm_mutant_libs():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")).read()
    libs = {}
    with tempfile.TemporaryDirectory() as td:
        for name, (a, b) in _NORM_MUTATIONS.items():
            assert src.count(a) == 1, name
            path = os.path.join(td, "n%d.c" % len(libs))
            with open(path, "w") as f:
                f.write(src.replace(a, b))
            so = path[:-2] + ".so"
            subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                                   path, "-o", so, "-lm"])
            libs[name] = oracle.load_library(so)
        yield libs


@pytest.mark.parametrize("name", sorted(_NORM_MUTATIONS))
def test_norm_pins_catch_planted_mistake(norm_mutant_libs, name):
    assert _norm_pins(lib=norm_mutant_libs[name]) != [], name
