"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each pin checks the oracle against something it does not compute itself: a value
worked by hand (tests/golden), a closed form, an invariant of the mathematics, a
special case that reduces to a library routine, or brute force on tiny inputs.
``test_planted_mistakes`` plants plausible mistakes in the oracle and checks that at
least one pin catches each of them.
"""
import json
import math
import os
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import kvx_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _orthonormal(rng, n, c):
    q, _ = np.linalg.qr(rng.standard_normal((n, c)))
    return q


# ------------------------------------------------------------------------- budget

def pin_budget_golden():
    for case in _golden("budget.json")["cases"]:
        assert O.budget(case["T"], case["pct"]) == case["k"], case


def pin_budget_ceiling():
    for T in range(0, 300):
        for pct in range(0, 101):
            want = math.ceil(Fraction(pct * T, 100))
            assert O.budget(T, pct) == want


# ------------------------------------------------------------------------- mapper

def pin_map_identity():
    rng = _rng(1)
    x = rng.standard_normal((9, 16))
    z = O.map_latent(x, np.eye(16))
    assert np.array_equal(z, x)


def pin_map_orthogonal_roundtrip():
    """Orthogonal shared projection + the matching per-layer reconstruction returns the
    source KV split into layer blocks (an orthogonal mapper reproduces its input)."""
    rng = _rng(2)
    L, H_kv, d_h = 3, 2, 4
    d_t = 2 * H_kv * d_h
    d = L * d_t
    x = rng.standard_normal((11, d))
    Q = _orthonormal(rng, d, d)
    z = O.map_latent(x, Q)                          # z = x Q^T
    w_l = np.stack([Q.T[l * d_t:(l + 1) * d_t] for l in range(L)])
    K, V, Y = O.reconstruct(z, w_l, H_kv, d_h)
    for l in range(L):
        blk = x[:, l * d_t:(l + 1) * d_t]
        assert np.abs(Y[l] - blk).max() < 1e-12
        assert np.abs(K[l].reshape(11, -1) - blk[:, :H_kv * d_h]).max() < 1e-12
        assert np.abs(V[l].reshape(11, -1) - blk[:, H_kv * d_h:]).max() < 1e-12


def pin_map_linearity():
    rng = _rng(3)
    w = rng.standard_normal((5, 12))
    a, b = rng.standard_normal((4, 12)), rng.standard_normal((4, 12))
    lhs = O.map_latent(2.0 * a - 3.0 * b, w)
    rhs = 2.0 * O.map_latent(a, w) - 3.0 * O.map_latent(b, w)
    assert np.abs(lhs - rhs).max() < 1e-12
    # a non-square mapper: each latent entry is one weight row dotted with the input
    for i in range(4):
        for j in range(5):
            assert abs(O.map_latent(a, w)[i, j] - sum(a[i, c] * w[j, c] for c in range(12))) < 1e-12


def pin_reconstruct_block_identity():
    """w_l = identity picks latent columns: K head h of layer 0 is z[:, h*d_h:(h+1)*d_h],
    V heads follow the K heads."""
    rng = _rng(4)
    H_kv, d_h = 2, 3
    d_t = 2 * H_kv * d_h
    z = rng.standard_normal((5, d_t))
    w_l = np.stack([np.eye(d_t), np.eye(d_t)[::-1]])
    K, V, _ = O.reconstruct(z, w_l, H_kv, d_h)
    for h in range(H_kv):
        assert np.array_equal(K[0][:, h], z[:, h * d_h:(h + 1) * d_h])
        assert np.array_equal(V[0][:, h], z[:, (H_kv + h) * d_h:(H_kv + h + 1) * d_h])
    # layer 1 reverses the columns
    assert np.array_equal(V[1][:, H_kv - 1, ::-1], z[:, :d_h])


# ------------------------------------------------------------------------- score

def pin_score_hand():
    g = _golden("score_hand.json")
    u = np.array(g["u"])
    Y = np.array(g["y"])
    assert abs(O.rank_disagreement(Y, u)[0] - g["score"]) < 1e-12


def pin_score_in_span_zero():
    rng = _rng(5)
    L, d_t, c, N = 3, 10, 4, 7
    u = np.stack([_orthonormal(rng, d_t, c) for _ in range(L)])
    Y = np.stack([rng.standard_normal((N, c)) @ u[l].T for l in range(L)])
    s = O.rank_disagreement(Y, u)
    assert np.all(np.abs(s) <= 1e-12 * np.sum(Y * Y, axis=(0, 2)))


def pin_score_complement_full():
    rng = _rng(6)
    L, d_t, c, N = 2, 8, 3, 6
    s_full = []
    u = []
    Y = []
    for _ in range(L):
        q = _orthonormal(rng, d_t, d_t)
        u.append(q[:, :c])
        Y.append(rng.standard_normal((N, d_t - c)) @ q[:, c:].T)   # orthogonal to span(U)
    u, Y = np.stack(u), np.stack(Y)
    s = O.rank_disagreement(Y, u)
    want = np.sum(Y * Y, axis=(0, 2))
    assert np.abs(s - want).max() <= 1e-12 * want.max()


def pin_score_empty_basis():
    rng = _rng(7)
    Y = rng.standard_normal((2, 5, 6))
    s = O.rank_disagreement(Y, np.zeros((2, 6, 0)))
    assert np.abs(s - np.sum(Y * Y, axis=(0, 2))).max() < 1e-12


def pin_score_homogeneous_equivariant():
    rng = _rng(8)
    L, d_t, c, N = 2, 8, 3, 9
    u = np.stack([_orthonormal(rng, d_t, c) for _ in range(L)])
    Y = rng.standard_normal((L, N, d_t))
    s = O.rank_disagreement(Y, u)
    assert np.abs(O.rank_disagreement(2.5 * Y, u) - 6.25 * s).max() < 1e-11 * s.max()
    perm = rng.permutation(N)
    assert np.abs(O.rank_disagreement(Y[:, perm], u) - s[perm]).max() < 1e-12 * s.max()


def pin_score_least_squares():
    """The residual outside span(U) equals the least-squares residual of fitting y by U's
    columns (library routine), so the energies agree."""
    rng = _rng(9)
    L, d_t, c, N = 2, 9, 4, 5
    u = np.stack([_orthonormal(rng, d_t, c) for _ in range(L)])
    Y = rng.standard_normal((L, N, d_t))
    want = np.zeros(N)
    for l in range(L):
        coef, *_ = np.linalg.lstsq(u[l], Y[l].T, rcond=None)
        res = Y[l].T - u[l] @ coef
        want += np.sum(res * res, axis=0)
    assert np.abs(O.rank_disagreement(Y, u) - want).max() < 1e-12 * want.max()


def pin_score_latent_identity():
    """For a linear bias-free mapper the score is a quadratic form of the latent:
    s_t = z_t^T A z_t with A = sum_l R_l^T R_l, R_l = (I - U_l U_l^T) W_l."""
    rng = _rng(10)
    L, H_kv, d_h, r, c, N = 3, 2, 4, 6, 5, 8
    d_t = 2 * H_kv * d_h
    w_l = rng.standard_normal((L, d_t, r))
    u = np.stack([_orthonormal(rng, d_t, c) for _ in range(L)])
    z = rng.standard_normal((N, r))
    _, _, Y = O.reconstruct(z, w_l, H_kv, d_h)
    s = O.rank_disagreement(Y, u)
    A = np.zeros((r, r))
    for l in range(L):
        R = w_l[l] - u[l] @ (u[l].T @ w_l[l])
        A += R.T @ R
    s2 = np.einsum("ti,ij,tj->t", z, A, z)
    assert np.abs(s - s2).max() <= 1e-12 * s.max()


# ------------------------------------------------------------------------- select

def pin_select_brute_force():
    rng = _rng(11)
    for trial in range(40):
        T = int(rng.integers(1, 40))
        s = rng.integers(0, 5, size=T).astype(float) * (1 if trial % 2 else 0.5)
        for k in range(T + 1):
            S, C = O.select(s, k)
            order = sorted(range(T), key=lambda t: (-s[t], t))
            assert list(S) == sorted(order[:k])
            assert list(C) == sorted(order[k:])


def pin_select_all_equal():
    s = np.full(20, 3.0)
    S, C = O.select(s, 6)
    assert list(S) == list(range(6)) and list(C) == list(range(6, 20))


def pin_select_signed_zero():
    s = np.array([-0.0, 0.0, -0.0, 0.0, 1.0, -1.0])
    S, _ = O.select(s, 3)          # 1.0 first, then the two lowest-index zeros
    assert list(S) == [0, 1, 4]


def pin_select_extremes():
    s = np.arange(10.0)[::-1]
    S, C = O.select(s, 0)
    assert len(S) == 0 and list(C) == list(range(10))
    S, C = O.select(s, 10)
    assert list(S) == list(range(10)) and len(C) == 0


def pin_select_planted():
    """Positions whose source KV is scaled by 3 score 9x (homogeneity) and must be
    selected whenever their count fits the budget."""
    rng = _rng(12)
    T, d, r, L, H_kv, d_h, c = 60, 256, 64, 2, 2, 16, 16
    d_t = 2 * H_kv * d_h
    x = rng.standard_normal((T, d))
    planted = rng.choice(T, size=7, replace=False)
    x[planted] *= 3.0
    w_s = rng.standard_normal((r, d)) / 16
    w_l = rng.standard_normal((L, d_t, r)) / 8
    u = np.stack([_orthonormal(rng, d_t, c) for _ in range(L)])
    _, _, Y = O.reconstruct(O.map_latent(x, w_s), w_l, H_kv, d_h)
    s = O.rank_disagreement(Y, u)
    S, _ = O.select(s, O.budget(T, 30))
    assert set(planted.tolist()) <= set(S.tolist())


# ------------------------------------------------------------------------- rope / recompute

def pin_rope_zero_position():
    rng = _rng(13)
    x = rng.standard_normal((3, 5, 8))
    assert np.array_equal(O.rope(x, np.zeros((3, 5)), 10000.0), x)


def pin_rope_d2_closed_form():
    """d_h = 2 has one pair at frequency 1: a plane rotation by the position itself."""
    for p in (1, 7, 1000):
        out = O.rope(np.array([[0.3, -1.1]]), np.array([p]), 10000.0)[0]
        want = [0.3 * math.cos(p) + 1.1 * math.sin(p), -1.1 * math.cos(p) + 0.3 * math.sin(p)]
        assert np.abs(out - want).max() < 1e-12


def pin_rope_d4_pairs():
    """d_h = 4: pairs are (0, 2) at frequency 1 and (1, 3) at frequency base^(-1/2)."""
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    out = O.rope(x, np.array([1]), 10000.0)[0]
    a0, a1 = 1.0, 0.01
    want = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
            3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    assert np.abs(out - want).max() < 1e-12


def pin_rope_norm_and_relative():
    rng = _rng(14)
    q, k = rng.standard_normal(16), rng.standard_normal(16)
    for m, n in ((5, 2), (300, 17), (16383, 9000)):
        rq = O.rope(q[None], np.array([m]), 10000.0)[0]
        rk = O.rope(k[None], np.array([n]), 10000.0)[0]
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-12
        rel = O.rope(q[None], np.array([m - n]), 10000.0)[0]
        assert abs(rq @ rk - rel @ k) < 1e-10


def pin_reconstruct_rotated_matrix_form():
    """Rotated translated keys: every key head of every layer times the block-diagonal plane
    rotation of its row's position (pair (j, j + d_h/2) by the angle p * base^(-2j/d_h)), built
    here as explicit 2x2 matrices; V and the mapped vectors as the plain reconstruction."""
    rng = _rng(70)
    H_kv, d_h, L, r, N = 2, 6, 3, 5, 7
    z = rng.standard_normal((N, r))
    w_l = rng.standard_normal((L, 2 * H_kv * d_h, r))
    pos = np.array([0, 3, 1, 40, 7, 1000, 2])
    K, V, Y = O.reconstruct_rotated(z, w_l, H_kv, d_h, pos, 100.0)
    Y_plain = np.stack([z @ w_l[l].T for l in range(L)])
    assert np.abs(Y - Y_plain).max() < 1e-12
    assert np.abs(V - Y_plain[:, :, H_kv * d_h:].reshape(L, N, H_kv, d_h)).max() < 1e-12
    K_plain = Y_plain[:, :, :H_kv * d_h].reshape(L, N, H_kv, d_h)
    half = d_h // 2
    for t in range(N):
        R = np.zeros((d_h, d_h))
        for j in range(half):
            a = pos[t] * 100.0 ** (-2.0 * j / d_h)
            R[j, j], R[j, j + half] = math.cos(a), -math.sin(a)
            R[j + half, j], R[j + half, j + half] = math.sin(a), math.cos(a)
        want = K_plain[:, t] @ R.T
        assert np.abs(K[:, t] - want).max() < 1e-10


def pin_qknorm_head_norms():
    """Each normalised head has squared norm d_h * ms / (ms + eps) with unit gains (ms its mean
    square before normalising), at every position (the rotation keeps norms); with eps = 0 the
    heads do not change when the hidden rows are scaled; v is the plain projection."""
    rng = _rng(72)
    H_q, H_kv, d_h, D, n = 2, 1, 6, 10, 5
    x = rng.standard_normal((n, D))
    w = rng.standard_normal(((H_q + 2 * H_kv) * d_h, D))
    pos = np.array([0, 5, 17, 300, 2])
    ones = np.ones(d_h)
    eps = 0.25
    q, k, v = O.recompute_qkv_qknorm(x, w, pos, H_q, H_kv, d_h, 10000.0, ones, ones, eps)
    raw = x @ w.T
    rq = raw[:, :H_q * d_h].reshape(n, H_q, d_h)
    rk = raw[:, H_q * d_h:(H_q + H_kv) * d_h].reshape(n, H_kv, d_h)
    for got, r in ((q, rq), (k, rk)):
        ms = np.mean(r * r, axis=-1)
        assert np.abs(np.sum(got * got, axis=-1) - d_h * ms / (ms + eps)).max() < 1e-10
    assert np.abs(v - raw[:, (H_q + H_kv) * d_h:].reshape(n, H_kv, d_h)).max() < 1e-12
    q1, k1, _ = O.recompute_qkv_qknorm(x, w, pos, H_q, H_kv, d_h, 10000.0, ones, ones, 0.0)
    q3, k3, _ = O.recompute_qkv_qknorm(3.0 * x, w, pos, H_q, H_kv, d_h, 10000.0, ones, ones, 0.0)
    assert np.abs(q1 - q3).max() < 1e-10 and np.abs(k1 - k3).max() < 1e-10


def pin_qknorm_gain_before_rotation():
    """The gains act before the rotation: a head's norm does not depend on its position even with
    uneven gains, and at position 0 a gain that keeps one channel keeps only that channel."""
    rng = _rng(73)
    H_q, H_kv, d_h, D = 1, 1, 8, 9
    x = np.repeat(rng.standard_normal((1, D)), 3, axis=0)
    w = rng.standard_normal(((H_q + 2 * H_kv) * d_h, D))
    g = rng.uniform(0.2, 3.0, d_h)
    q, k, _ = O.recompute_qkv_qknorm(x, w, np.array([0, 9, 4000]), H_q, H_kv, d_h, 10000.0, g, g[::-1], 1e-6)
    for t in (q, k):
        nrm = np.linalg.norm(t, axis=-1)
        assert np.abs(nrm - nrm[0]).max() < 1e-10
    e = np.zeros(d_h)
    e[3] = 2.0
    q0, _, _ = O.recompute_qkv_qknorm(x[:1], w, np.array([0]), H_q, H_kv, d_h, 10000.0, e, g, 1e-6)
    assert np.count_nonzero(np.abs(q0) > 1e-14) == 1 and abs(q0[0, 0, 3]) > 0


def pin_recompute_identity_weights():
    """w_qkv made of identity blocks returns the hidden rows themselves (q, k rotated)."""
    rng = _rng(15)
    H_q, H_kv, d_h = 2, 1, 4
    D = H_q * d_h
    x = rng.standard_normal((6, D))
    w = np.concatenate([np.eye(D), np.eye(D)[:H_kv * d_h], np.eye(D)[H_kv * d_h:2 * H_kv * d_h]])
    pos = np.array([0, 3, 4, 9, 10, 20])
    q, k, v = O.recompute_qkv(x, w, pos, H_q, H_kv, d_h, 10000.0)
    assert np.abs(q - O.rope(x.reshape(6, H_q, d_h), pos[:, None], 10000.0)).max() < 1e-12
    assert np.abs(k[:, 0] - O.rope(x[:, :d_h], pos, 10000.0)).max() < 1e-12
    assert np.array_equal(v[:, 0], x[:, d_h:2 * d_h])


# ------------------------------------------------------------------------- attention

def pin_attention_hand():
    g = _golden("attention_hand.json")
    q = np.array(g["q"])[None, None]
    K = np.array(g["K"])[:, None]
    V = np.array(g["V"])[:, None]
    o, lse = O.sparse_causal_attention(q, K, V, np.array([g["pos"]]))
    assert np.abs(o[0, 0] - g["o"]).max() < 1e-12
    assert abs(lse[0, 0] - g["lse"]) < 1e-12


def _sdpa_causal(q, K, V):
    """Library routine: torch's scaled_dot_product_attention, causal, float64 CPU.
    q [T, H_q, d], K/V [T, H_kv, d]; KV heads repeated g times (head h reads h // g)."""
    g = q.shape[1] // K.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(K, g, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(V, g, axis=1)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()


def pin_attention_full_is_causal_sdpa():
    rng = _rng(16)
    T, H_q, H_kv, d_h = 23, 6, 2, 8
    q = rng.standard_normal((T, H_q, d_h))
    K = rng.standard_normal((T, H_kv, d_h))
    V = rng.standard_normal((T, H_kv, d_h))
    o, lse = O.sparse_causal_attention(q, K, V, np.arange(T))
    assert np.abs(o - _sdpa_causal(q, K, V)).max() < 1e-12
    # log-sum-exp against scipy's routine
    from scipy.special import logsumexp
    g = H_q // H_kv
    for i in (0, 5, T - 1):
        for h in range(H_q):
            ref = logsumexp(K[:i + 1, h // g] @ q[i, h] / math.sqrt(d_h))
            assert abs(lse[i, h] - ref) < 1e-12


def pin_attention_special_cases():
    rng = _rng(17)
    T, H_q, H_kv, d_h = 12, 4, 2, 4
    q = rng.standard_normal((3, H_q, d_h))
    K = rng.standard_normal((T, H_kv, d_h))
    V = rng.standard_normal((T, H_kv, d_h))
    o, _ = O.sparse_causal_attention(q, K, V, np.array([0, 5, 11]))
    # the first position sees only itself
    assert np.abs(o[0] - np.repeat(V[0], 2, axis=0)).max() < 1e-12
    # constant values give the constant back
    Vc = np.broadcast_to(np.array([1.0, -2.0, 0.5, 3.0]), (T, H_kv, d_h)).copy()
    oc, _ = O.sparse_causal_attention(q, K, Vc, np.array([0, 5, 11]))
    assert np.abs(oc - Vc[0, 0]).max() < 1e-12
    # GQA equals MHA over KV heads repeated g times
    om, _ = O.sparse_causal_attention(q, np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1),
                                      np.array([0, 5, 11]))
    assert np.abs(o - om).max() < 1e-12


# ------------------------------------------------------------------------- end to end

def _tiny_problem(seed, T=20):
    rng = _rng(seed)
    L_t, H_q, H_kv, d_h, r, D, c = 2, 4, 2, 4, 6, 8, 3
    d_t = 2 * H_kv * d_h
    d_src = 24
    return dict(
        x_src=rng.standard_normal((T, d_src)), w_s=rng.standard_normal((r, d_src)) / 5,
        w_l=rng.standard_normal((L_t, d_t, r)) / 2.5,
        u=np.stack([_orthonormal(rng, d_t, c) for _ in range(L_t)]),
        x_l=rng.standard_normal((L_t, T, D)),
        w_qkv=rng.standard_normal((L_t, (H_q + 2 * H_kv) * d_h, D)) / 3,
        H_q=H_q, H_kv=H_kv, d_h=d_h)


def pin_handoff_zero_budget():
    p = _tiny_problem(18)
    out = O.handoff_request(pct=0, **p)
    assert len(out["S"]) == 0 and out["O"].shape[1] == 0
    assert np.array_equal(out["K"], out["K_tr"]) and np.array_equal(out["V"], out["V_tr"])


def pin_handoff_full_budget_is_prefill():
    """A 100% budget recomputes every position, so the cache is the target's own K/V and
    the outputs equal plain causal attention over the target's own Q/K/V."""
    p = _tiny_problem(19)
    out = O.handoff_request(pct=100, **p)
    T = p["x_src"].shape[0]
    H_q, H_kv, d_h = p["H_q"], p["H_kv"], p["d_h"]
    for l in range(p["w_l"].shape[0]):
        qkv = p["x_l"][l] @ p["w_qkv"][l].T
        q = qkv[:, :H_q * d_h].reshape(T, H_q, d_h)
        k = qkv[:, H_q * d_h:(H_q + H_kv) * d_h].reshape(T, H_kv, d_h)
        v = qkv[:, (H_q + H_kv) * d_h:].reshape(T, H_kv, d_h)
        # rotary embedding by explicit 2x2 rotations of each (j, j + d_h/2) pair
        def rot(a):
            b = a.copy()
            for t in range(T):
                for j in range(d_h // 2):
                    ang = t * 10000.0 ** (-2.0 * j / d_h)
                    x1, x2 = a[t, :, j], a[t, :, j + d_h // 2]
                    b[t, :, j] = x1 * math.cos(ang) - x2 * math.sin(ang)
                    b[t, :, j + d_h // 2] = x2 * math.cos(ang) + x1 * math.sin(ang)
            return b
        q, k = rot(q), rot(k)
        assert np.abs(out["K"][l] - k).max() < 1e-12
        assert np.abs(out["V"][l] - v).max() < 1e-12
        assert np.abs(out["O"][l] - _sdpa_causal(q, k, v)).max() < 1e-12


def pin_handoff_partial_budget_mixed_cache():
    """At a partial budget the mixed cache holds translated K/V off the selected set and
    recomputed K/V on it; every selected query attends to both kinds."""
    p = _tiny_problem(20)
    out = O.handoff_request(pct=30, **p)
    S, C = out["S"], out["C"]
    assert len(S) == O.budget(20, 30) and sorted(set(S) | set(C)) == list(range(20))
    assert np.array_equal(out["K"][:, C], out["K_tr"][:, C])
    assert not np.allclose(out["K"][:, S], out["K_tr"][:, S])
    # the last selected query's output changes if a translated entry it sees changes
    l, i = 0, len(S) - 1
    Kp = out["K"][l].copy()
    j = int(C[C < S[i]][0])
    Kp[j] += 1.0
    q, _, _ = O.recompute_qkv(p["x_l"][l][S], p["w_qkv"][l], S, p["H_q"], p["H_kv"], p["d_h"], 10000.0)
    o2, _ = O.sparse_causal_attention(q[i:i + 1], Kp, out["V"][l], S[i:i + 1])
    assert np.abs(o2[0] - out["O"][l, i]).max() > 1e-6


# ------------------------------------------------------------------------- layer chaining

def pin_rmsnorm_hand():
    """[3, 4, 0, 0]: mean square 25/4, rms 2.5; with gain [1, 2, 3, 4] -> [1.2, 3.2, 0, 0]."""
    y = O.rmsnorm(np.array([[3.0, 4.0, 0.0, 0.0]]), np.array([1.0, 2.0, 3.0, 4.0]), 0.0)
    assert np.abs(y - np.array([[1.2, 3.2, 0.0, 0.0]])).max() < 1e-15
    # eps enters under the root: [1, 1] with eps 3 -> 1 / sqrt(1 + 3) = 0.5
    assert np.abs(O.rmsnorm(np.ones((1, 2)), np.ones(2), 3.0) - 0.5).max() < 1e-15


def pin_rmsnorm_invariants():
    rng = _rng(41)
    x = rng.standard_normal((5, 12))
    g = rng.uniform(0.5, 2.0, 12)
    y = O.rmsnorm(x, g, 0.0)
    assert np.abs(O.rmsnorm(7.5 * x, g, 0.0) - y).max() < 1e-13      # scale invariant
    assert np.abs(np.mean((y / g) ** 2, axis=1) - 1.0).max() < 1e-13  # unit rms before the gain


def pin_silu_closed_form():
    assert O.silu(np.array([0.0]))[0] == 0.0
    # sigmoid(ln 3) = 3/4
    assert abs(O.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    x = _rng(42).standard_normal(50) * 4
    assert np.abs(O.silu(x) - O.silu(-x) - x).max() < 1e-13          # x s(x) + x s(-x) = x


def _layer_loops(x, S, K, V, w, H_q, H_kv, d_h, base, eps):
    """One decoder layer written element by element (independent of the vectorised oracle)."""
    n, D = x.shape
    F = w["w_gate"].shape[0]
    g = H_q // H_kv
    def norm(row, gain):
        ms = sum(v * v for v in row) / len(row)
        return [row[j] / math.sqrt(ms + eps) * gain[j] for j in range(len(row))]
    def rot(vec, p):
        out = list(vec)
        for j in range(d_h // 2):
            a = p * base ** (-2.0 * j / d_h)
            x1, x2 = vec[j], vec[j + d_h // 2]
            out[j] = x1 * math.cos(a) - x2 * math.sin(a)
            out[j + d_h // 2] = x2 * math.cos(a) + x1 * math.sin(a)
        return out
    Km, Vm = K.copy(), V.copy()
    qs = []
    for i in range(n):
        h = norm(list(x[i]), w["gamma_in"])
        row = [sum(w["w_qkv"][c][j] * h[j] for j in range(D)) for c in range((H_q + 2 * H_kv) * d_h)]
        p = int(S[i])
        qs.append([rot(row[hh * d_h:(hh + 1) * d_h], p) for hh in range(H_q)])
        for hk in range(H_kv):
            Km[p, hk] = rot(row[(H_q + hk) * d_h:(H_q + hk + 1) * d_h], p)
            Vm[p, hk] = row[(H_q + H_kv + hk) * d_h:(H_q + H_kv + hk + 1) * d_h]
    out = np.zeros_like(x)
    for i in range(n):
        p = int(S[i])
        o = []
        for hh in range(H_q):
            kv = hh // g
            lg = [sum(qs[i][hh][d] * Km[j, kv, d] for d in range(d_h)) / math.sqrt(d_h) for j in range(p + 1)]
            m = max(lg)
            e = [math.exp(v - m) for v in lg]
            tot = sum(e)
            o += [sum(e[j] / tot * Vm[j, kv, d] for j in range(p + 1)) for d in range(d_h)]
        x1 = [x[i][c] + sum(w["w_o"][c][j] * o[j] for j in range(H_q * d_h)) for c in range(D)]
        h2 = norm(x1, w["gamma_post"])
        a = []
        for f in range(F):
            gt = sum(w["w_gate"][f][j] * h2[j] for j in range(D))
            up = sum(w["w_up"][f][j] * h2[j] for j in range(D))
            a.append(gt / (1.0 + math.exp(-gt)) * up)
        out[i] = [x1[c] + sum(w["w_down"][c][f] * a[f] for f in range(F)) for c in range(D)]
    return out, Km, Vm


def _tiny_layers(seed, L, D, F, H_q, H_kv, d_h):
    rng = _rng(seed)
    return [dict(gamma_in=rng.uniform(0.5, 1.5, D), w_qkv=rng.standard_normal(((H_q + 2 * H_kv) * d_h, D)) / 2,
                 w_o=rng.standard_normal((D, H_q * d_h)) / 2, gamma_post=rng.uniform(0.5, 1.5, D),
                 w_gate=rng.standard_normal((F, D)) / 2, w_up=rng.standard_normal((F, D)) / 2,
                 w_down=rng.standard_normal((D, F)) / 2) for _ in range(L)]


def pin_target_layer_brute_force():
    rng = _rng(43)
    T, D, F, H_q, H_kv, d_h = 7, 6, 5, 4, 2, 4
    S = np.array([1, 3, 4, 6])
    x = rng.standard_normal((len(S), D))
    K, V = rng.standard_normal((T, H_kv, d_h)), rng.standard_normal((T, H_kv, d_h))
    w = _tiny_layers(44, 1, D, F, H_q, H_kv, d_h)[0]
    got, Kg, Vg, _, _ = O.target_layer(x, S, K, V, w, H_q, H_kv, d_h, 10000.0, 1e-6)
    want, Kw, Vw = _layer_loops(x, S, K, V, w, H_q, H_kv, d_h, 10000.0, 1e-6)
    assert np.abs(got - want).max() < 1e-11
    assert np.abs(Kg - Kw).max() < 1e-12 and np.abs(Vg - Vw).max() < 1e-12


def pin_target_layer_zero_weights_pass_through():
    """With W_o = 0 and W_down = 0 both residual branches vanish: the rows pass unchanged,
    and the cache and outputs are those of the plain recompute of rmsnorm(x)."""
    rng = _rng(45)
    T, D, F, H_q, H_kv, d_h = 9, 8, 6, 4, 2, 4
    S = np.array([0, 2, 5, 8])
    x = rng.standard_normal((len(S), D))
    K, V = rng.standard_normal((T, H_kv, d_h)), rng.standard_normal((T, H_kv, d_h))
    w = _tiny_layers(46, 1, D, F, H_q, H_kv, d_h)[0]
    w["w_o"][:] = 0.0
    w["w_down"][:] = 0.0
    out, Km, Vm, Oo, _ = O.target_layer(x, S, K, V, w, H_q, H_kv, d_h, 10000.0, 1e-6)
    assert np.array_equal(out, x)
    h = O.rmsnorm(x, w["gamma_in"], 1e-6)
    q, kk, vv = O.recompute_qkv(h, w["w_qkv"], S, H_q, H_kv, d_h, 10000.0)
    K2, V2 = O.scatter(K, V, S, kk, vv)
    assert np.array_equal(Km, K2) and np.array_equal(Vm, V2)
    assert np.abs(Oo - O.sparse_causal_attention(q, K2, V2, S)[0]).max() == 0.0


def pin_chained_full_budget_is_dense_forward():
    """Selecting every position turns the chained layers into the target's own forward pass:
    each layer's cache is its own rotated K/V and each layer's rows follow from dense
    causal attention (compared with torch's scaled-dot-product attention)."""
    rng = _rng(47)
    T, D, F, H_q, H_kv, d_h, L = 6, 8, 10, 4, 2, 4, 2
    layers = _tiny_layers(48, L, D, F, H_q, H_kv, d_h)
    x0 = rng.standard_normal((T, D))
    S = np.arange(T)
    K_tr = rng.standard_normal((L, T, H_kv, d_h))
    V_tr = rng.standard_normal((L, T, H_kv, d_h))
    out = O.chained_layers(x0, S, K_tr, V_tr, layers, H_q, H_kv, d_h)
    x = x0
    for l, w in enumerate(layers):
        ms = np.mean(x * x, axis=1, keepdims=True)
        h = x / np.sqrt(ms + 1e-6) * w["gamma_in"]
        qkv = h @ w["w_qkv"].T
        q = qkv[:, :H_q * d_h].reshape(T, H_q, d_h)
        k = qkv[:, H_q * d_h:(H_q + H_kv) * d_h].reshape(T, H_kv, d_h)
        v = qkv[:, (H_q + H_kv) * d_h:].reshape(T, H_kv, d_h)
        ang = np.arange(T)[:, None, None] * 10000.0 ** (-2.0 * np.arange(d_h // 2) / d_h)
        c, s_ = np.cos(ang), np.sin(ang)
        rot = lambda a: np.concatenate([a[..., :d_h // 2] * c - a[..., d_h // 2:] * s_,
                                        a[..., d_h // 2:] * c + a[..., :d_h // 2] * s_], -1)
        q, k = rot(q), rot(k)
        assert np.abs(out["K"][l] - k).max() < 1e-12 and np.abs(out["V"][l] - v).max() < 1e-12
        o = _sdpa_causal(q, k, v)
        x1 = x + o.reshape(T, -1) @ w["w_o"].T
        h2 = x1 / np.sqrt(np.mean(x1 * x1, axis=1, keepdims=True) + 1e-6) * w["gamma_post"]
        gt = h2 @ w["w_gate"].T
        x = x1 + ((gt * torch.sigmoid(torch.from_numpy(gt)).numpy()) * (h2 @ w["w_up"].T)) @ w["w_down"].T
        assert np.abs(out["X"][l + 1] - x).max() < 1e-10, l


def pin_argmax_ties_lowest():
    assert O.argmax_lowest(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert list(O.argmax_lowest(np.array([[0.0, 0.0], [-1.0, -2.0]]))) == [0, 0]


def pin_lm_head_hand():
    """rmsnorm([3, 4], gain 1) = [3, 4] / sqrt(12.5); against w rows e1, e2, e1 + e2."""
    x = np.array([[3.0, 4.0]])
    w = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    r = math.sqrt(12.5)
    assert np.abs(O.lm_head(x, np.ones(2), w, 0.0) - np.array([[3 / r, 4 / r, 7 / r]])).max() < 1e-15


def pin_first_token_full_budget_is_last_dense_row():
    """After a 100% budget the cache is the target's own, and the first-token step for the
    last position reproduces the dense forward's last row: its logits are the LM head of
    that row, and its rewritten cache rows are unchanged."""
    rng = _rng(49)
    T, D, F, H_q, H_kv, d_h, L, Vv = 6, 8, 10, 4, 2, 4, 2, 11
    layers = _tiny_layers(50, L, D, F, H_q, H_kv, d_h)
    x0 = rng.standard_normal((T, D))
    full = O.chained_layers(x0, np.arange(T), rng.standard_normal((L, T, H_kv, d_h)),
                            rng.standard_normal((L, T, H_kv, d_h)), layers, H_q, H_kv, d_h)
    g = rng.uniform(0.5, 1.5, D)
    w_lm = rng.standard_normal((Vv, D))
    logits, tok, K, V = O.first_token(x0[T - 1], T - 1, full["K"], full["V"], layers, g, w_lm, H_q, H_kv, d_h)
    last = full["X"][-1][T - 1]
    want = (last / np.sqrt(np.mean(last ** 2) + 1e-6) * g) @ w_lm.T
    assert np.abs(logits - want).max() < 1e-10
    assert tok == int(np.argmax(want))
    assert np.abs(K - full["K"]).max() < 1e-12 and np.abs(V - full["V"]).max() < 1e-12


def pin_score_normalized_angle():
    """One layer, d_t = 2, span(U) the first axis: a vector at angle a to that axis scores sin^2(a)
    whatever its length; a second layer adds its energies to both sums."""
    u = np.array([[[1.0], [0.0]]])
    for a, rad in ((0.0, 2.0), (0.3, 1.0), (math.pi / 4, 5.0), (1.2, 0.01), (math.pi / 2, 3.0)):
        Y = np.array([[[rad * math.cos(a), rad * math.sin(a)]]])
        assert abs(O.rank_disagreement_normalized(Y, u)[0] - math.sin(a) ** 2) < 1e-12
    u2 = np.stack([u[0], u[0]])
    Y2 = np.array([[[3.0, 4.0]], [[0.0, 0.0]]])          # second layer empty: same as one layer
    assert abs(O.rank_disagreement_normalized(Y2, u2)[0] - 16.0 / 25.0) < 1e-12
    Y3 = np.array([[[3.0, 4.0]], [[1.0, 0.0]]])          # (16) / (25 + 1)
    assert abs(O.rank_disagreement_normalized(Y3, u2)[0] - 16.0 / 26.0) < 1e-12
    assert O.rank_disagreement_normalized(np.zeros((2, 1, 2)), u2)[0] == 0.0


def pin_score_normalized_bounds_and_scale():
    rng = _rng(71)
    L, N, d_t, c = 3, 40, 8, 3
    Y = rng.standard_normal((L, N, d_t))
    u = np.stack([np.linalg.qr(rng.standard_normal((d_t, c)))[0] for _ in range(L)])
    s = O.rank_disagreement_normalized(Y, u)
    assert np.all(s >= 0) and np.all(s <= 1)
    scale = rng.uniform(0.1, 10.0, N)                    # per-token scaling leaves the share alone
    assert np.abs(O.rank_disagreement_normalized(Y * scale[None, :, None], u) - s).max() < 1e-12
    # in-span tokens score 0, tokens orthogonal to every span score 1
    Yin = np.stack([rng.standard_normal((N, c)) @ u[l].T for l in range(L)])
    assert np.abs(O.rank_disagreement_normalized(Yin, u)).max() < 1e-12
    Yout = np.stack([Y[l] - (Y[l] @ u[l]) @ u[l].T for l in range(L)])
    assert np.abs(O.rank_disagreement_normalized(Yout, u) - 1.0).max() < 1e-12


def pin_score_gap_hand():
    # scores 5, 3, 3, 1 (shuffled): the gap after the k-th largest, relative to it, worked by hand
    s = np.array([3.0, 1.0, 5.0, 3.0])
    assert O.score_gap(s, 1) == pytest.approx(2.0 / 5.0, abs=1e-15)   # 5 vs 3
    assert O.score_gap(s, 2) == 0.0                                   # 3 vs 3: a tie at the boundary
    assert O.score_gap(s, 3) == pytest.approx(2.0 / 3.0, abs=1e-15)   # 3 vs 1
    assert O.score_gap(s, 0) == math.inf and O.score_gap(s, 4) == math.inf
    # a negative k-th score divides by its magnitude; a zero one leaves the plain difference
    assert O.score_gap(np.array([-4.0, -3.0]), 1) == pytest.approx(1.0 / 3.0, abs=1e-15)   # -3 vs -4
    assert O.score_gap(np.array([0.0, -0.25]), 1) == 0.25
    # the gap does not depend on the order of the positions
    rng = _rng(77)
    t = rng.standard_normal(50)
    assert O.score_gap(t, 17) == O.score_gap(t[rng.permutation(50)], 17)


# ------------------------------------------------------------------------- fitting

def _planted_pair(seed, n, d, L, d_t, r, noise=0.0):
    """Source KV x [n, d] with per-channel scales, a planted rank-r map W [L d_t, d] and the
    target KV y = x W^T (+ noise) of all L layers, layer-major."""
    rng = _rng(seed)
    x = rng.standard_normal((n, d)) * rng.uniform(0.5, 2.0, d)
    W = rng.standard_normal((L * d_t, r)) @ (rng.standard_normal((r, d)) / math.sqrt(d))
    y = x @ W.T + noise * rng.standard_normal((n, L * d_t))
    return x, y, W


def _principal_sines(a, b):
    """Sines of the principal angles between the column spans of a and b (equal dimensions):
    the singular values of the part of b's orthonormal basis outside a's span (accurate for
    small angles, unlike 1 - cos^2)."""
    qa, _ = np.linalg.qr(a)
    qb, _ = np.linalg.qr(b)
    return np.linalg.svd(qb - qa @ (qa.T @ qb), compute_uv=False)


def pin_fit_recovers_planted_map():
    # a noise-free rank-5 map, more calibration positions than source channels, no ridge term:
    # the fitted composite map (reconstruction times projection) is the planted map
    x, y, W = _planted_pair(60, n=120, d=24, L=3, d_t=10, r=5)
    w_s, w_l = O.fit_mapper(x, y, 5, 0.0, 3)
    assert w_s.shape == (5, 24) and w_l.shape == (3, 10, 5)
    comp = w_l.reshape(30, 5) @ w_s
    assert np.abs(comp - W).max() <= 1e-10 * np.abs(W).max()


def pin_fit_reduced_rank_residual():
    # no ridge term: the rank-r fit's residual is the least-squares residual plus the energy of
    # the fitted values' discarded singular directions (Pythagoras + Eckart-Young); the fitted
    # values are formed here from an orthonormal basis of x's columns (QR), their singular
    # values from the eigenvalues of their Gram matrix
    x, y, _ = _planted_pair(61, n=80, d=20, L=2, d_t=12, r=6, noise=0.3)
    r = 6
    w_s, w_l = O.fit_mapper(x, y, r, 0.0, 2)
    comp = w_l.reshape(24, r) @ w_s
    q, _ = np.linalg.qr(x)
    yhat = q @ (q.T @ y)
    sig2 = np.sort(np.linalg.eigvalsh(yhat.T @ yhat))[::-1]
    want = np.sum((y - yhat) ** 2) + np.sum(sig2[r:])
    got = np.sum((x @ comp.T - y) ** 2)
    assert abs(got - want) <= 1e-9 * want


def pin_fit_ridge_normal_equations():
    # full rank (r = all outputs): the composite is the ridge solution itself, which satisfies
    # the normal equations (x^T x + lam I) B = x^T y
    x, y, _ = _planted_pair(62, n=30, d=40, L=2, d_t=6, r=3, noise=0.5)
    lam = 2.5
    w_s, w_l = O.fit_mapper(x, y, 12, lam, 2)
    comp = w_l.reshape(12, 12) @ w_s                     # [L d_t, d] = B^T
    lhs = (x.T @ x + lam * np.eye(40)) @ comp.T
    assert np.abs(lhs - x.T @ y).max() <= 1e-9 * np.abs(x.T @ y).max()


def pin_fit_invariances():
    # orthonormal reconstruction columns; the composite scales with y and ignores the order of
    # the calibration positions
    x, y, _ = _planted_pair(63, n=50, d=16, L=3, d_t=8, r=4, noise=0.2)
    w_s, w_l = O.fit_mapper(x, y, 4, 0.7, 3)
    V = w_l.reshape(24, 4)
    assert np.abs(V.T @ V - np.eye(4)).max() <= 1e-12
    comp = V @ w_s
    w_s2, w_l2 = O.fit_mapper(x, 3.0 * y, 4, 0.7, 3)
    assert np.abs(w_l2.reshape(24, 4) @ w_s2 - 3.0 * comp).max() <= 1e-10 * np.abs(comp).max()
    perm = _rng(64).permutation(50)
    w_s3, w_l3 = O.fit_mapper(x[perm], y[perm], 4, 0.7, 3)
    assert np.abs(w_l3.reshape(24, 4) @ w_s3 - comp).max() <= 1e-10 * np.abs(comp).max()


def pin_calibration_planted_span():
    # every mapped calibration vector lies in a planted 3-dim subspace P of each layer: the
    # basis spans exactly P (principal angles 0)
    rng = _rng(65)
    L, d_t, r, n, c = 2, 12, 6, 40, 3
    z = rng.standard_normal((n, r)) * np.array([3.0, 2.0, 1.5, 1.0, 0.7, 0.4])
    P = [np.linalg.qr(rng.standard_normal((d_t, c)))[0] for _ in range(L)]
    w_l = np.stack([P[l] @ rng.standard_normal((c, r)) for l in range(L)])
    u = O.calibration_basis(z, w_l, c)
    for l in range(L):
        assert np.abs(u[l].T @ u[l] - np.eye(c)).max() <= 1e-12
        assert _principal_sines(u[l], P[l]).max() <= 1e-10


def pin_calibration_energy_is_discarded_spectrum():
    # summed over the calibration positions, the rank-disagreement score of the mapped KV
    # equals the energy of each layer's discarded singular directions (Eckart-Young); the
    # singular values come from the eigenvalues of the d_t x d_t Gram matrix
    rng = _rng(66)
    L, d_t, r, n, c = 3, 10, 7, 30, 4
    z = rng.standard_normal((n, r)) * rng.uniform(0.3, 3.0, r)
    w_l = rng.standard_normal((L, d_t, r))
    u = O.calibration_basis(z, w_l, c)
    _, _, Y = O.reconstruct(z, w_l, 1, d_t // 2)
    total = np.sum(O.rank_disagreement(Y, u))
    want = 0.0
    for l in range(L):
        m = w_l[l] @ z.T
        ev = np.sort(np.linalg.eigvalsh(m @ m.T))[::-1]
        want += np.sum(ev[c:])
    assert abs(total - want) <= 1e-9 * want


# ------------------------------------------------------------------------- direct scoring of a stored cache, per-layer sets

def _split_kv(y, H_kv, d_h):
    """[L, T, 2 H_kv d_h] rows in the reconstruction's channel order -> stored K, V [L, T, H_kv, d_h]."""
    L, T = y.shape[:2]
    hd = H_kv * d_h
    return y[..., :hd].reshape(L, T, H_kv, d_h), y[..., hd:].reshape(L, T, H_kv, d_h)


def pin_layer_disagreement_closed_forms():
    """Layer by layer, with each layer's own basis (the first c columns of a full orthogonal
    matrix Q_l): a stored vector inside span(U_l) scores 0, one built from Q_l's other columns
    scores its squared norm, and their sum scores the second part only.  The same stored vector in
    two layers scores 0 in the layer whose span holds it and the squared norm of its coordinates
    on the other layer's remaining columns there.  A basis of K channels only ignores K and scores
    all of V (the K heads come first in the stored vector)."""
    rng = _rng(80)
    L, T, H_kv, d_h, c = 2, 5, 2, 4, 3
    d_t = 2 * H_kv * d_h
    Q = np.stack([np.linalg.qr(rng.standard_normal((d_t, d_t)))[0] for _ in range(L)])
    u = Q[:, :, :c]
    a = rng.standard_normal((L, T, c))
    b = rng.standard_normal((L, T, d_t - c))
    inside = np.einsum("ldc,ltc->ltd", Q[:, :, :c], a)
    outside = np.einsum("ldc,ltc->ltd", Q[:, :, c:], b)
    E_in = O.layer_disagreement(*_split_kv(inside, H_kv, d_h), u)
    E_out = O.layer_disagreement(*_split_kv(outside, H_kv, d_h), u)
    E_sum = O.layer_disagreement(*_split_kv(inside + outside, H_kv, d_h), u)
    want = np.sum(b * b, axis=2)
    assert E_in.shape == (L, T) and np.abs(E_in).max() < 1e-24 + 1e-12 * np.sum(a * a)
    assert np.abs(E_out - want).max() <= 1e-12 * want.max()
    assert np.abs(E_sum - want).max() <= 1e-12 * want.max()
    # one vector in both layers, inside layer 0's span
    y = np.stack([inside[0], inside[0]])
    E = O.layer_disagreement(*_split_kv(y, H_kv, d_h), u)
    other = np.einsum("dc,td->tc", Q[1, :, c:], inside[0])
    assert np.abs(E[0]).max() <= 1e-12 * np.sum(inside[0] ** 2)
    assert np.abs(E[1] - np.sum(other ** 2, axis=1)).max() <= 1e-12 * np.sum(inside[0] ** 2)
    assert E[1].min() > 1e-3
    # a basis of the first c K channels
    e = np.zeros((1, d_t, c))
    e[0, np.arange(c), np.arange(c)] = 1.0
    yk = np.zeros((1, T, d_t))
    yk[0, :, :c] = rng.standard_normal((T, c))
    yk[0, :, H_kv * d_h:] = rng.standard_normal((T, H_kv * d_h))
    Ek = O.layer_disagreement(*_split_kv(yk, H_kv, d_h), e)
    assert np.abs(Ek[0] - np.sum(yk[0, :, H_kv * d_h:] ** 2, axis=1)).max() <= 1e-12 * np.sum(yk ** 2)


def pin_layer_disagreement_sums_to_score():
    """Scored from the translated cache the reconstruction writes, the layers' energies add up to
    the rank-disagreement score of the same mapped vectors."""
    rng = _rng(81)
    L, T, r, H_kv, d_h, c = 3, 11, 6, 2, 4, 5
    d_t = 2 * H_kv * d_h
    z = rng.standard_normal((T, r))
    w_l = rng.standard_normal((L, d_t, r))
    u = np.stack([_orthonormal(rng, d_t, c) for _ in range(L)])
    K, V, Y = O.reconstruct(z, w_l, H_kv, d_h)
    E = O.layer_disagreement(K, V, u)
    s = O.rank_disagreement(Y, u)
    assert E.shape == (L, T) and (E >= 0).all()
    assert np.abs(E.sum(axis=0) - s).max() <= 1e-12 * s.max()


def pin_select_per_layer_hand():
    """Every layer its own top-k, ties to the lower position (worked by hand)."""
    E = np.array([[3.0, 1.0, 2.0, 2.0, 0.0],
                  [0.0, 5.0, 5.0, 1.0, 7.0],
                  [1.0, 1.0, 1.0, 1.0, 1.0]])
    S, C = O.select_per_layer(E, 2)
    assert S.tolist() == [[0, 2], [1, 4], [0, 1]]
    assert C.tolist() == [[1, 3, 4], [0, 2, 3], [2, 3, 4]]
    S0, C0 = O.select_per_layer(E, 0)
    assert S0.shape == (3, 0) and C0.tolist() == [[0, 1, 2, 3, 4]] * 3


def _layer_sets_case(rng, L, T, H_q, H_kv, d_h, D, same_layers=False):
    d_src, r, c = 10, 2 * H_kv * d_h * L, 3
    d_t = 2 * H_kv * d_h
    x_src = rng.standard_normal((T, d_src))
    w_s = rng.standard_normal((r, d_src))
    w_l = rng.standard_normal((L, d_t, r))
    u = np.stack([_orthonormal(rng, d_t, c) for _ in range(L)])
    if same_layers:
        w_l[:] = w_l[0]
        u[:] = u[0]
    x_l = rng.standard_normal((L, T, D))
    w_qkv = rng.standard_normal((L, (H_q + 2 * H_kv) * d_h, D))
    return x_src, w_s, w_l, u, x_l, w_qkv


def pin_layer_sets_hand():
    """Each layer recomputes the positions of its own largest energies: layer l's reconstruction
    reads only block l of the latent, so energies planted in block 0 at positions 1 and 4 and in
    block 1 at 2 and 7 select {1, 4} in layer 0 and {2, 7} in layer 1 (a set shared by both
    layers, from the summed score, would be {1, 2})."""
    L, T, H_kv, d_h = 2, 8, 1, 2
    d_t = 2 * H_kv * d_h
    z = np.full((T, L * d_t), 1e-3)
    z[1, 0], z[4, 1], z[2, d_t], z[7, d_t + 2] = 10.0, 9.5, 9.7, 9.0
    w_l = np.zeros((L, d_t, L * d_t))
    for l in range(L):
        w_l[l][:, l * d_t:(l + 1) * d_t] = np.eye(d_t)
    u = np.zeros((L, d_t, 0))                   # empty calibration span: the energy is the squared norm
    H_q, D = 2, 4
    rng = _rng(82)
    out = O.handoff_request_layer_sets(z, np.eye(L * d_t), w_l, u, rng.standard_normal((L, T, D)),
                                       rng.standard_normal((L, (H_q + 2 * H_kv) * d_h, D)), 25, H_q, H_kv, d_h)
    assert out["S"].tolist() == [[1, 4], [2, 7]]
    assert out["C"].tolist() == [[0, 2, 3, 5, 6, 7], [0, 1, 3, 4, 5, 6]]


def pin_layer_sets_shared_when_layers_agree():
    """With every layer's reconstruction and basis equal, every layer's energies are the same, so
    every layer's set is the shared set of the summed score and the variant's cache and outputs
    are the plain handoff's."""
    rng = _rng(83)
    L, T, H_q, H_kv, d_h, D = 3, 30, 4, 2, 4, 12
    args = _layer_sets_case(rng, L, T, H_q, H_kv, d_h, D, same_layers=True)
    a = O.handoff_request_layer_sets(*args, 30, H_q, H_kv, d_h)
    b = O.handoff_request(*args, 30, H_q, H_kv, d_h)
    for l in range(L):
        assert a["S"][l].tolist() == b["S"].tolist()
    for key in ("K", "V", "O", "LSE"):
        assert np.abs(a[key] - b[key]).max() <= 1e-12 * np.abs(b[key]).max(), key


def pin_layer_sets_complement_and_layer_order():
    """Layer l writes recomputed K/V only at its own set: its complement rows keep the translated
    values, and its set's rows change.  Reordering the layers (weights, bases, inputs) reorders the
    energies, sets, cache and outputs the same way."""
    rng = _rng(84)
    L, T, H_q, H_kv, d_h, D = 3, 30, 4, 2, 4, 12
    args = _layer_sets_case(rng, L, T, H_q, H_kv, d_h, D)
    out = O.handoff_request_layer_sets(*args, 30, H_q, H_kv, d_h)
    assert any(out["S"][0].tolist() != out["S"][l].tolist() for l in range(1, L))
    for l in range(L):
        Cl, Sl = out["C"][l], out["S"][l]
        assert np.array_equal(out["K"][l][Cl], out["K_tr"][l][Cl])
        assert np.array_equal(out["V"][l][Cl], out["V_tr"][l][Cl])
        assert np.abs(out["K"][l][Sl] - out["K_tr"][l][Sl]).min(axis=(1, 2)).max() > 0
    perm = np.array([2, 0, 1])
    x_src, w_s, w_l, u, x_l, w_qkv = args
    po = O.handoff_request_layer_sets(x_src, w_s, w_l[perm], u[perm], x_l[perm], w_qkv[perm], 30, H_q, H_kv, d_h)
    assert np.array_equal(po["S"], out["S"][perm])
    for key in ("E", "K", "V", "O", "LSE"):
        assert np.abs(po[key] - out[key][perm]).max() <= 1e-12 * np.abs(out[key]).max(), key


# ------------------------------------------------------------------------- page-granular selection

def pin_page_selection_hand():
    """Worked by hand: T = 10, pages of 4 ([0,4), [4,8), [8,10)); the short last page competes
    with its two positions' sum."""
    s = np.array([1.0, 0.0, 0.0, 1.0, 0.5, 0.5, 0.5, 0.0, 3.0, 0.2])
    ps = O.page_scores(s, 4)
    assert np.allclose(ps, [2.0, 1.5, 3.2], rtol=0, atol=1e-15)
    S, C, P = O.select_pages(ps, 10, 4, 2)
    assert P.tolist() == [0, 2] and S.tolist() == [0, 1, 2, 3, 8, 9] and C.tolist() == [4, 5, 6, 7]
    S1, C1, P1 = O.select_pages(ps, 10, 4, 1)
    assert P1.tolist() == [2] and S1.tolist() == [8, 9] and len(C1) == 8
    # equal page scores: the lower page
    S2, _, P2 = O.select_pages(np.array([1.0, 1.0, 1.0]), 10, 4, 1)
    assert P2.tolist() == [0] and S2.tolist() == [0, 1, 2, 3]


def pin_page_selection_unit_pages():
    """Pages of one position are positions: the page scores are the scores and the selection is
    the position selection with the same count."""
    rng = _rng(90)
    for T in (1, 7, 64, 300):
        s = rng.standard_normal(T)
        ps = O.page_scores(s, 1)
        assert np.array_equal(ps, s)
        for k in (0, 1, T // 3, T):
            S, C, P = O.select_pages(ps, T, 1, k)
            S0, C0 = O.select(s, k)
            assert np.array_equal(S, S0) and np.array_equal(C, C0) and np.array_equal(P, S0)


def pin_page_selection_whole_pages():
    """Every selected set is a union of whole pages inside [0, T) (the last one possibly short),
    with |S| = k_pages * page_size less the last page's shortfall when it is chosen; the page
    scores add up to the total score; a page made to dominate is chosen."""
    rng = _rng(91)
    for T, ps_, kp in ((100, 16, 3), (37, 8, 2), (64, 16, 4), (5, 16, 1)):
        s = rng.uniform(0, 1, T)
        pg = O.page_scores(s, ps_)
        assert len(pg) == -(-T // ps_) and abs(pg.sum() - s.sum()) <= 1e-12 * s.sum()
        S, C, P = O.select_pages(pg, T, ps_, kp)
        assert np.array_equal(np.sort(np.concatenate([S, C])), np.arange(T))
        short = (-T) % ps_ if (len(pg) - 1) in P.tolist() else 0
        assert len(S) == kp * ps_ - short
        for j in P:
            assert set(range(j * ps_, min((j + 1) * ps_, T))) <= set(S.tolist())
        s2 = s.copy()
        last = len(pg) - 1
        s2[last * ps_] = 1e6
        _, _, P2 = O.select_pages(O.page_scores(s2, ps_), T, ps_, kp)
        assert last in P2.tolist()


PINS = {name: fn for name, fn in globals().items() if name.startswith("pin_")}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name]()


# ------------------------------------------------------------------------- planted mistakes

def _mut_rope_sign(x, pos, base):
    d_h = x.shape[-1]
    h = d_h // 2
    ang = O.rope_angles(pos, d_h, base)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * np.cos(ang) + x2 * np.sin(ang), x2 * np.cos(ang) - x1 * np.sin(ang)], -1)


def _mut_rope_interleaved(x, pos, base):
    d_h = x.shape[-1]
    ang = O.rope_angles(pos, d_h, base)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * np.cos(ang) - x2 * np.sin(ang)
    out[..., 1::2] = x2 * np.cos(ang) + x1 * np.sin(ang)
    return out


def _mut_attn_factory(scale_fn=None, exclusive=False, gqa_mod=False):
    def attn(q, K, V, pos):
        n, H_q, d_h = q.shape
        H_kv = K.shape[1]
        g = H_q // H_kv
        Oo = np.zeros((n, H_q, d_h))
        lse = np.zeros((n, H_q))
        for i in range(n):
            p = int(pos[i]) + (0 if exclusive else 1)
            p = max(p, 1)
            for h in range(H_q):
                kv = h % H_kv if gqa_mod else h // g
                lg = (K[:p, kv] @ q[i, h]) * (scale_fn(d_h) if scale_fn else 1 / math.sqrt(d_h))
                e = np.exp(lg - lg.max())
                Oo[i, h] = (e / e.sum()) @ V[:p, kv]
                lse[i, h] = lg.max() + math.log(e.sum())
        return Oo, lse
    return attn


def _mut_select_high_index(s, k):
    T = s.shape[0]
    order = np.lexsort((-np.arange(T), -s))
    return np.sort(order[:k]), np.sort(order[k:])


def _mut_score_projection(Y, u):
    s = np.zeros(Y.shape[1])
    for l in range(Y.shape[0]):
        p = Y[l] @ u[l]
        s += np.sum(p * p, axis=1)
    return s


def _mut_score_one_layer(Y, u):
    res = Y[0] - (Y[0] @ u[0]) @ u[0].T
    return np.sum(res * res, axis=1)


def _mut_map_no_transpose(x, w):
    return x @ w if w.shape[0] == x.shape[1] else x @ w.T[:, ::-1]


def _mut_reconstruct_kv_swapped(z, w_l, H_kv, d_h):
    K, V, Y = RECONSTRUCT(z, w_l, H_kv, d_h)
    return V, K, Y


def _mut_budget_floor(T, pct):
    return pct * T // 100


RECONSTRUCT = O.reconstruct


def _mut_rmsnorm_no_root(x, gamma, eps):
    return x / (np.mean(x * x, axis=-1, keepdims=True) + eps) * gamma


def _mut_rmsnorm_sum(x, gamma, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * gamma


def _mut_silu_sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _mut_mlp_gate_up_swapped(x, w_gate, w_up, w_down):
    return (O_SILU(x @ w_up.T) * (x @ w_gate.T)) @ w_down.T


def _mut_layer_no_residual(x_rows, S, K, V, w, H_q, H_kv, d_h, base, eps):
    x2, K2, V2, Oo, lse = TARGET_LAYER(x_rows, S, K, V, w, H_q, H_kv, d_h, base, eps)
    return x2 - x_rows, K2, V2, Oo, lse


O_SILU = O.silu
TARGET_LAYER = O.target_layer


def _mut_lm_head_no_norm(x, gamma, w_lm, eps):
    return (x * gamma) @ w_lm.T


def _mut_argmax_highest(logits):
    a = np.asarray(logits)
    return a.shape[-1] - 1 - np.argmax(a[..., ::-1], axis=-1)

def _mut_scatter_kv_swapped(K, V, S, k_new, v_new):
    return SCATTER(K, V, S, v_new, k_new)


def _mut_scatter_shifted(K, V, S, k_new, v_new):
    return SCATTER(K, V, np.minimum(np.asarray(S) + 1, K.shape[0] - 1), k_new, v_new)


def _mut_recompute_v_rotated(x_rows, w_qkv, pos, H_q, H_kv, d_h, base):
    q, k, v = RECOMPUTE(x_rows, w_qkv, pos, H_q, H_kv, d_h, base)
    return q, k, O.rope(v, np.asarray(pos)[:, None], base)


def _mut_recompute_rank_positions(x_rows, w_qkv, pos, H_q, H_kv, d_h, base):
    return RECOMPUTE(x_rows, w_qkv, np.arange(len(pos)), H_q, H_kv, d_h, base)


def _mut_chained_from_input(x0_rows, S, K_tr, V_tr, layers, H_q, H_kv, d_h, base=10000.0, eps=1e-6):
    out = CHAINED(x0_rows, S, K_tr, V_tr, layers[:1], H_q, H_kv, d_h, base, eps)
    for l in range(1, len(layers)):
        o = CHAINED(x0_rows, S, K_tr[l:l + 1], V_tr[l:l + 1], layers[l:l + 1], H_q, H_kv, d_h, base, eps)
        for key in ("K", "V", "O", "LSE"):
            out[key] = np.concatenate([out[key], o[key]])
        out["X"] = np.concatenate([out["X"], o["X"][1:]])
    return out


def _mut_first_token_one_layer(x0_last, p_last, K, V, layers, gamma_final, w_lm, H_q, H_kv, d_h,
                               base=10000.0, eps=1e-6):
    logits, tok, K1, V1 = FIRST_TOKEN(x0_last, p_last, K[:1], V[:1], layers[:1], gamma_final, w_lm,
                                      H_q, H_kv, d_h, base, eps)
    return logits, tok, np.concatenate([K1, K[1:]]), np.concatenate([V1, V[1:]])


def _mut_score_gap_wrong_neighbour(s, k):
    T = s.shape[0]
    if k == 0 or k == T:
        return math.inf
    srt = np.sort(s)[::-1]
    return float((srt[k - 2] - srt[k - 1]) / abs(srt[k - 1])) if k >= 2 else float(srt[0] - srt[1]) / abs(srt[0])


FIT = O.fit_mapper
def _mut_fit_on_targets(x, y, r, lam, L):
    # singular vectors of the targets instead of the fitted values
    n, d = x.shape
    m = y.shape[1]
    B = np.linalg.lstsq(np.vstack([x, math.sqrt(lam) * np.eye(d)]), np.vstack([y, np.zeros((d, m))]), rcond=None)[0]
    V = np.linalg.svd(y, full_matrices=False)[2][:r].T
    return (B @ V).T, V.reshape(L, m // L, r)


def _mut_fit_no_ridge(x, y, r, lam, L):
    return FIT(x, y, r, 0.0, L)


def _mut_fit_trailing(x, y, r, lam, L):
    n, d = x.shape
    m = y.shape[1]
    B = np.linalg.lstsq(np.vstack([x, math.sqrt(lam) * np.eye(d)]), np.vstack([y, np.zeros((d, m))]), rcond=None)[0]
    vt = np.linalg.svd(x @ B, full_matrices=False)[2]
    V = vt[-r:].T
    return (B @ V).T, V.reshape(L, m // L, r)


def _mut_calibration_trailing(z, w_l, c):
    L, d_t, _ = w_l.shape
    return np.stack([np.linalg.svd(w_l[l] @ z.T, full_matrices=False)[0][:, -c:] for l in range(L)])


def _mut_calibration_no_latent(z, w_l, c):
    L, d_t, _ = w_l.shape
    return np.stack([np.linalg.svd(w_l[l], full_matrices=False)[0][:, :c] for l in range(L)])


SCATTER = O.scatter
RECOMPUTE = O.recompute_qkv
CHAINED = O.chained_layers
FIRST_TOKEN = O.first_token

def _mut_reconstruct_rotated_v(z, w_l, H_kv, d_h, pos, base):
    K, V, Y = O.reconstruct(z, w_l, H_kv, d_h)
    return K, O.rope(V, np.asarray(pos)[None, :, None], base), Y


def _mut_reconstruct_rotated_row_index(z, w_l, H_kv, d_h, pos, base):
    K, V, Y = O.reconstruct(z, w_l, H_kv, d_h)
    return O.rope(K, np.arange(len(pos))[None, :, None], base), V, Y


def _mut_normalized_by_span(Y, u):
    outside = O.rank_disagreement(Y, u)
    inside = np.sum(Y * Y, axis=(0, 2)) - outside
    return np.where(inside > 0, outside / np.where(inside > 0, inside, 1.0), 0.0)


def _mut_normalized_mean_of_layers(Y, u):
    L = Y.shape[0]
    acc = np.zeros(Y.shape[1])
    for l in range(L):
        tot = np.sum(Y[l] * Y[l], axis=1)
        res = O.rank_disagreement(Y[l:l + 1], u[l:l + 1])
        acc += np.where(tot > 0, res / np.where(tot > 0, tot, 1.0), 0.0)
    return acc / L


def _mut_qknorm_gain_after_rope(x_rows, w_qkv, pos, H_q, H_kv, d_h, base, q_gain, k_gain, eps):
    q, k, v = O.recompute_qkv(x_rows, w_qkv, pos, H_q, H_kv, d_h, base)
    return (O.rmsnorm(q, np.ones(d_h), eps) * q_gain, O.rmsnorm(k, np.ones(d_h), eps) * k_gain, v)


def _mut_qknorm_over_all_heads(x_rows, w_qkv, pos, H_q, H_kv, d_h, base, q_gain, k_gain, eps):
    qkv = x_rows @ w_qkv.T
    n = x_rows.shape[0]
    q = O.rmsnorm(qkv[:, :H_q * d_h], np.tile(q_gain, H_q), eps).reshape(n, H_q, d_h)
    k = O.rmsnorm(qkv[:, H_q * d_h:(H_q + H_kv) * d_h], np.tile(k_gain, H_kv), eps).reshape(n, H_kv, d_h)
    v = qkv[:, (H_q + H_kv) * d_h:].reshape(n, H_kv, d_h)
    return O.rope(q, np.asarray(pos)[:, None], base), O.rope(k, np.asarray(pos)[:, None], base), v


_ORIG = {name: getattr(O, name) for name in ("layer_disagreement", "select_per_layer", "page_scores",
                                             "select_pages")}


def _mut_page_score_max(s, page_size):
    T = s.shape[0]
    return np.array([np.max(s[j * page_size:min((j + 1) * page_size, T)]) for j in range(-(-T // page_size))])


def _mut_page_last_full(ps, T, page_size, k_pages):
    P, _ = O.select(ps, k_pages)
    S = np.sort(np.concatenate([np.arange(j * page_size, (j + 1) * page_size) for j in P])) if len(P) else \
        np.zeros(0, dtype=np.int64)
    C = np.setdiff1d(np.arange(T), S)
    return S.astype(np.int64), C.astype(np.int64), P


def _mut_page_ties_high(ps, T, page_size, k_pages):
    return _ORIG["select_pages"](ps + 1e-9 * np.arange(len(ps)), T, page_size, k_pages)


def _mut_direct_v_then_k(K, V, u):
    L, T = K.shape[:2]
    E = np.zeros((L, T))
    for l in range(L):
        y = np.concatenate([V[l].reshape(T, -1), K[l].reshape(T, -1)], axis=1)
        res = y - (y @ u[l]) @ u[l].T
        E[l] = np.sum(res * res, axis=1)
    return E


def _mut_direct_first_basis(K, V, u):
    return _ORIG["layer_disagreement"](K, V, np.stack([u[0]] * u.shape[0]))


def _mut_per_layer_summed(E, k):
    return _ORIG["select_per_layer"](np.stack([E.sum(axis=0)] * E.shape[0]), k)


def _mut_per_layer_first_set(E, k):
    return _ORIG["select_per_layer"](np.stack([E[0]] * E.shape[0]), k)


MUTANTS = {
    "rope_sign": ("rope", _mut_rope_sign),
    "rope_interleaved": ("rope", _mut_rope_interleaved),
    "attn_no_scale": ("sparse_causal_attention", _mut_attn_factory(scale_fn=lambda d: 1.0)),
    "attn_exclusive_causal": ("sparse_causal_attention", _mut_attn_factory(exclusive=True)),
    "attn_gqa_modulo": ("sparse_causal_attention", _mut_attn_factory(gqa_mod=True)),
    "select_ties_high_index": ("select", _mut_select_high_index),
    "score_projection_energy": ("rank_disagreement", _mut_score_projection),
    "score_one_layer": ("rank_disagreement", _mut_score_one_layer),
    "normalized_by_span_energy": ("rank_disagreement_normalized", _mut_normalized_by_span),
    "normalized_mean_of_layer_shares": ("rank_disagreement_normalized", _mut_normalized_mean_of_layers),
    "map_untransposed": ("map_latent", _mut_map_no_transpose),
    "reconstruct_kv_swapped": ("reconstruct", _mut_reconstruct_kv_swapped),
    "reconstruct_rotated_v": ("reconstruct_rotated", _mut_reconstruct_rotated_v),
    "reconstruct_rotated_row_index": ("reconstruct_rotated", _mut_reconstruct_rotated_row_index),
    "budget_floor": ("budget", _mut_budget_floor),
    "rmsnorm_no_root": ("rmsnorm", _mut_rmsnorm_no_root),
    "rmsnorm_sum_not_mean": ("rmsnorm", _mut_rmsnorm_sum),
    "silu_is_sigmoid": ("silu", _mut_silu_sigmoid),
    "mlp_gate_up_swapped": ("swiglu_mlp", _mut_mlp_gate_up_swapped),
    "layer_no_residual": ("target_layer", _mut_layer_no_residual),
    "lm_head_no_norm": ("lm_head", _mut_lm_head_no_norm),
    "argmax_ties_highest": ("argmax_lowest", _mut_argmax_highest),
    "scatter_kv_swapped": ("scatter", _mut_scatter_kv_swapped),
    "scatter_shifted": ("scatter", _mut_scatter_shifted),
    "recompute_v_rotated": ("recompute_qkv", _mut_recompute_v_rotated),
    "qknorm_gain_after_rope": ("recompute_qkv_qknorm", _mut_qknorm_gain_after_rope),
    "qknorm_over_all_heads": ("recompute_qkv_qknorm", _mut_qknorm_over_all_heads),
    "recompute_rank_positions": ("recompute_qkv", _mut_recompute_rank_positions),
    "chained_from_input": ("chained_layers", _mut_chained_from_input),
    "first_token_one_layer": ("first_token", _mut_first_token_one_layer),
    "score_gap_wrong_neighbour": ("score_gap", _mut_score_gap_wrong_neighbour),
    "fit_svd_of_targets": ("fit_mapper", _mut_fit_on_targets),
    "fit_no_ridge": ("fit_mapper", _mut_fit_no_ridge),
    "fit_trailing_directions": ("fit_mapper", _mut_fit_trailing),
    "calibration_trailing_directions": ("calibration_basis", _mut_calibration_trailing),
    "calibration_without_latents": ("calibration_basis", _mut_calibration_no_latent),
    "direct_score_v_then_k": ("layer_disagreement", _mut_direct_v_then_k),
    "direct_score_first_basis": ("layer_disagreement", _mut_direct_first_basis),
    "layer_sets_from_summed_score": ("select_per_layer", _mut_per_layer_summed),
    "layer_sets_first_layer_everywhere": ("select_per_layer", _mut_per_layer_first_set),
    "page_score_max": ("page_scores", _mut_page_score_max),
    "page_last_counted_full": ("select_pages", _mut_page_last_full),
    "page_ties_high": ("select_pages", _mut_page_ties_high),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistakes(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for name, pin in PINS.items():
        if name == "pin_budget_ceiling" and attr != "budget":
            continue
        try:
            pin()
        except AssertionError:          # a crash is not a catch: the pin must see a wrong value
            caught.append(name)
    assert caught, f"no pin caught the planted mistake {mutant}"
