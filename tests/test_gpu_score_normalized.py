"""GPU parity of the normalized score (kvx_score_select_normalized): the energy of each token's
mapped KV outside the calibration subspaces over the energy of all of it, against the oracle's
rank_disagreement_normalized on the same stored latent, reconstruction weights and subspaces.

Both quadratic forms run on the score GEMM (hi/lo bf16 operators, or fp32), each sum accurate to
about 1e-6 relative, so the ratio is held to 1e-5 relative (plus 1e-7 absolute for shares near 0).
The selection is the exact top-k of the returned scores (ties to the lower position) and equals
the oracle's outside a 1e-5 band around the k-th score.  Cases: bf16 and fp32, one request and a
batch of three with different budgets, a request longer than the select kernel keeps in LDS.
"""
import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from cross_model_kv_amd.workloads import TINY_F32
from helpers import band_check, f64
from oracle import kvx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small(name, **kw):
    base = dict(name=name, dtype="bf16", T=3000, L_s=2, H_s=2, d_hs=64, r=128, L_t=3, H_q=8, H_kv=2,
                d_h=128, D=256, c=64, pct=30)
    base.update(kw)
    return TINY_F32.shrink(**base)


CASES = {
    "bf16-one": small("bf16-one"),
    "bf16-batched": small("bf16-batched", n_req=3, t_min=200, t_max=3000, pct_choices=(20, 30, 40), r=192),
    "bf16-long": small("bf16-long", T=40000, L_t=2, r=128),
    "f32-batched": small("f32-batched", dtype="f32", n_req=2, t_min=100, t_max=900, pct_choices=(30, 40)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_score_normalized(name):
    wl = CASES[name]
    print(f"[score normalized] {name}", flush=True)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    inp = synth.generate(wl, 91, DEV)
    batch = kvx.Batch.for_budgets(inp.lengths, inp.pcts, DEV)
    z = synth.latent(batch.n_tokens, wl.r, 91, dtype=dt, device=DEV)
    op = kvx.score_prepare(inp.w_l, inp.u)
    op_tot = kvx.score_prepare(inp.w_l, inp.u[:, :, :0])
    scores, sel, rest = kvx.score_select_normalized(z, op, op_tot, batch, inp.pcts)
    torch.cuda.synchronize()
    s = f64(scores)
    _, _, Y = O.reconstruct(f64(z), f64(inp.w_l), wl.H_kv, wl.d_h)
    s_ref = O.rank_disagreement_normalized(Y, f64(inp.u))
    assert np.all(np.abs(s - s_ref) <= 1e-5 * s_ref + 1e-7), f"max error {np.abs(s - s_ref).max():.2e}"
    assert s_ref.min() > 0.05 and s_ref.max() < 0.99          # shares well inside (0, 1) here
    sel_h, rest_h = sel.cpu().numpy(), rest.cpu().numpy()
    cs, cr = batch.cu_sel, [c - k for c, k in zip(batch.cu_tokens, batch.cu_sel)]
    for b, T in enumerate(inp.lengths):
        rows = slice(batch.cu_tokens[b], batch.cu_tokens[b + 1])
        k = O.budget(T, inp.pcts[b])
        S_own, C_own = O.select(s[rows].astype(np.float32).astype(np.float64), k)
        assert np.array_equal(sel_h[cs[b]:cs[b + 1]], S_own) and np.array_equal(rest_h[cr[b]:cr[b + 1]], C_own)
        band_check(sel_h[cs[b]:cs[b + 1]], s_ref[rows], k, 1e-5)
