"""GPU parity of the mapper fit and of the calibration subspaces (kvx_fit_mapper,
kvx_fit_calibration) against the oracle's fit_mapper and calibration_basis.

The factorization is unique only up to a rotation of the latent, so what is compared is what the
handoff uses: the composite map (reconstruction times projection), the mapped KV of the
calibration positions, the span of the reconstruction columns (principal angles) and their
orthonormality; for the calibration, the span of every layer's basis and its orthonormality.
The oracle runs in float64 on exactly the values the device read (the stored x and y, and for
the calibration the device's own stored z and w_l).

Inputs (synth.calibration_pair): a planted rank-r relation with a spectral step after the first
c directions and 5% noise; the cases span fewer and more calibration positions than source
channels, the ridge term, ragged sizes (n = 130, 200: a partial last 64-block in every blocked
fp64 factorization), r above one 64-block (96), c = r, and a single target layer.

Tolerances.  fp32 storage: the device forms the two Gram matrices in fp32 (relative error about
1e-6 of their entries); the ridge solve moves H = I - lam C^-1 by at most |dG| / lam, so with the
ridge values here every compared quantity stays below 1e-4; the bar is 1e-3.  bf16 storage: the
fitted weights are rounded to bf16 (2^-9 relative per element, about 3e-3 on the composite map
and the mapped KV), bar 1e-2 (2e-2 for the sines of the reconstruction span).  The calibration
subspaces are computed in fp64 from the stored z and w_l on both sides and stored in fp32: bar
1e-4 for both dtypes.  Each case first checks, on the oracle, that the ridge term matters (the
fit at lam / 2 differs by more than five times the bar) and that the subspaces are well defined
(a gap after the r-th and c-th singular values), so that the bars can tell a wrong fit apart.
"""
import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from helpers import f64
from oracle import kvx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (name, dtype, n, d_src, L_t, d_t, r, c, lam)
CASES = [
    ("f32_under", torch.float32, 384, 512, 4, 128, 96, 24, 50.0),
    ("bf16_under", torch.bfloat16, 384, 512, 4, 128, 96, 24, 50.0),
    ("bf16_over", torch.bfloat16, 512, 256, 2, 256, 64, 16, 60.0),
    ("f32_ragged", torch.float32, 130, 96, 3, 40, 40, 10, 5.0),
    ("bf16_ragged_c_eq_r", torch.bfloat16, 200, 128, 1, 192, 40, 40, 30.0),
]
ITERS = 30


def _sines(a, b):
    """Sines of the principal angles between the column spans of a and b (equal dimensions)."""
    qa, _ = np.linalg.qr(a)
    qb, _ = np.linalg.qr(b)
    return np.linalg.svd(qb - qa @ (qa.T @ qb), compute_uv=False)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("name,dtype,n,d_src,L_t,d_t,r,c,lam", CASES, ids=[c[0] for c in CASES])
def test_fit_matches_oracle(name, dtype, n, d_src, L_t, d_t, r, c, lam):
    print(f"fit case {name}", flush=True)
    m = L_t * d_t
    x, y = synth.calibration_pair(n, d_src, L_t, d_t, r, seed=700 + n, strong=c, dtype=dtype, device=DEV)
    x64, y64 = f64(x), f64(y)

    o_ws, o_wl = O.fit_mapper(x64, y64, r, lam, L_t)
    o_comp = o_wl.reshape(m, r) @ o_ws
    bar = 1e-3 if dtype == torch.float32 else 1e-2
    # preconditions on the oracle: the ridge term matters, the rank-r subspace is well separated
    h_ws, h_wl = O.fit_mapper(x64, y64, r, lam / 2, L_t)
    assert _rel(h_wl.reshape(m, r) @ h_ws, o_comp) > 5 * bar
    sv = np.linalg.svd(x64 @ o_comp.T, compute_uv=False)
    assert sv[r] < 0.5 * sv[r - 1] if r < len(sv) else True

    w_s, w_l = kvx.fit_mapper(x, y, L_t, r, lam, iters=ITERS)
    torch.cuda.synchronize()
    assert w_s.shape == (r, d_src) and w_l.shape == (L_t, d_t, r)
    g_ws, g_wl = f64(w_s), f64(w_l)
    assert np.isfinite(g_ws).all() and np.isfinite(g_wl).all()
    V = g_wl.reshape(m, r)
    comp = V @ g_ws
    print(f"  composite {_rel(comp, o_comp):.2e}  span sine {_sines(V, o_wl.reshape(m, r)).max():.2e}", flush=True)
    assert _rel(comp, o_comp) <= bar, f"composite map {_rel(comp, o_comp):.3e}"
    assert _rel(x64 @ comp.T, x64 @ o_comp.T) <= bar, "mapped KV"
    sin_bar = 1e-3 if dtype == torch.float32 else 2e-2
    assert _sines(V, o_wl.reshape(m, r)).max() <= sin_bar, "reconstruction span"
    assert np.abs(V.T @ V - np.eye(r)).max() <= (1e-4 if dtype == torch.float32 else 1e-2)

    # calibration subspaces from the device's own latents and reconstructions
    z = kvx.map_latent(x, w_s)
    u = kvx.fit_calibration(z, w_l, c, iters=ITERS)
    torch.cuda.synchronize()
    assert u.shape == (L_t, d_t, c) and u.dtype == torch.float32
    z64 = f64(z)
    o_u = O.calibration_basis(z64, g_wl, c)
    g_u = f64(u)
    for l in range(L_t):
        sv = np.linalg.svd(g_wl[l] @ z64.T, compute_uv=False)
        if c < len(sv):
            assert sv[c] < 0.75 * sv[c - 1], "calibration subspace not separated"
        assert _sines(g_u[l], o_u[l]).max() <= 1e-4, f"layer {l} calibration span"
        assert np.abs(g_u[l].T @ g_u[l] - np.eye(c)).max() <= 1e-5


def test_fit_feeds_scoring():
    """The fitted weights and subspaces go straight into the scoring: the device's scores of the
    calibration positions under them equal the oracle's rank disagreement of the same stored
    values (relative 1e-5, the bar of the scoring parity test)."""
    n, d_src, L_t, d_t, r, c = 256, 256, 2, 128, 64, 16
    H_kv, d_h = 1, 64
    print("fit feeds scoring", flush=True)
    x, y = synth.calibration_pair(n, d_src, L_t, d_t, r, seed=777, strong=c, dtype=torch.bfloat16, device=DEV)
    w_s, w_l = kvx.fit_mapper(x, y, L_t, r, 10.0)
    z = kvx.map_latent(x, w_s)
    u = kvx.fit_calibration(z, w_l, c)
    op = kvx.score_prepare(w_l, u)
    batch = kvx.Batch.for_budgets([n], [20], DEV)
    scores, _, _ = kvx.score_select(z, op, batch, [20])
    torch.cuda.synchronize()
    _, _, Y = O.reconstruct(f64(z), f64(w_l), H_kv, d_h)
    s_ref = O.rank_disagreement(Y, f64(u))
    err = np.max(np.abs(f64(scores) - s_ref) / s_ref)
    assert err <= 1e-5, f"max relative score error {err:.2e}"
