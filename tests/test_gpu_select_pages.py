"""GPU parity of page-granular selection (kvx_select_pages) against the oracle's page_scores and
select_pages, and of a handoff that recomputes whole pages against the oracle's downstream steps.

The page scores are fp32 sums of fp32 scores in position order on the device and fp64 sums in the
oracle: they agree to within page_size * 2^-24 of the sum of the page's |scores| (bar 1e-6 relative
to that sum, page_size <= 64).  The pages are then chosen from the device's own page scores on
both sides (bit-exact: pages, positions, counts), and the oracle's choice from its fp64 page scores
agrees outside the band of page scores within that bar of the k-th.

Cases: page sizes 1 (the position selection itself), 3 and 16, requests shorter than a page, an
exact multiple of the page size and ragged ones, budgets 0%, 30%, 40% and 100%, scores with many
exact ties (page scores tie too) and a request of 40,000 positions (more pages than the select kernel
keeps in LDS at page size 1).
"""
import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from cross_model_kv_amd.handoff import Handoff
from cross_model_kv_amd.workloads import TINY_F32
from helpers import assert_close, band_check, f64, min_row_cosine, oracle_downstream
from oracle import kvx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (name, lengths, pcts, page_size, score kind)
CASES = [
    ("ps16-ragged", [100, 7, 64, 333], [30, 40, 100, 30], 16, "normal"),
    ("ps3-ties", [50, 51, 2, 90], [30, 0, 40, 30], 3, "ties"),
    ("ps1-positions", [200, 17], [30, 40], 1, "normal"),
    ("ps16-long", [40000], [30], 16, "normal"),
    ("ps1-long", [40000], [40], 1, "ties"),
    ("ps16-empty-requests", [0, 40, 0, 17], [30, 40, 30, 100], 16, "normal"),
]


def _scores(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "ties":
        return rng.integers(0, 4, n).astype(np.float32)
    return rng.standard_normal(n).astype(np.float32) ** 2


@pytest.mark.parametrize("name,lengths,pcts,ps,kind", CASES, ids=[c[0] for c in CASES])
def test_select_pages_matches_oracle(name, lengths, pcts, ps, kind):
    print(f"[select pages] {name}", flush=True)
    batch = kvx.Batch.for_budgets(lengths, [0] * len(lengths), DEV)
    s = _scores(kind, batch.n_tokens, 81)
    scores = torch.from_numpy(s).to(DEV)
    sel, rest, sb, pscore, psel = kvx.select_pages(scores, batch, ps, pcts)
    torch.cuda.synchronize()
    sel_h, rest_h, pscore_h, psel_h = sel.cpu().numpy(), rest.cpu().numpy(), f64(pscore), psel.cpu().numpy()
    po = kp0 = 0
    for b, T in enumerate(lengths):
        sr = s[batch.cu_tokens[b]:batch.cu_tokens[b + 1]].astype(np.float64)
        n_p = -(-T // ps)
        k_p = O.budget(n_p, pcts[b])
        ref_ps = O.page_scores(sr, ps)
        dev_ps = pscore_h[po:po + n_p]
        mag = O.page_scores(np.abs(sr), ps)
        assert np.all(np.abs(dev_ps - ref_ps) <= 1e-6 * mag), f"request {b} page scores"
        # the device's own page scores decide on both sides
        S, C, P = O.select_pages(dev_ps, T, ps, k_p)
        assert sb.cu_sel[b + 1] - sb.cu_sel[b] == len(S)
        assert np.array_equal(psel_h[kp0:kp0 + k_p], P)
        assert np.array_equal(sel_h[sb.cu_sel[b]:sb.cu_sel[b + 1]], S)
        r0 = batch.cu_tokens[b] - sb.cu_sel[b]
        assert np.array_equal(rest_h[r0:r0 + len(C)], C)
        if 0 < k_p < n_p:
            tau = np.sort(ref_ps)[::-1][k_p - 1]
            if tau > 0:
                band_check(P, ref_ps, k_p, 2e-6 * mag.max() / tau)
        if ps == 1:                                   # pages of one position: the position selection
            S0, _ = O.select(dev_ps, O.budget(T, pcts[b]))
            assert np.array_equal(S, S0)
        po += n_p
        kp0 += k_p


def test_page_handoff_against_oracle():
    """map -> score -> whole pages of 16 -> reconstruct the other pages -> recompute the pages'
    positions and attend, compared with the oracle's recompute, scatter and attention on the
    device's set; the short last page is selected."""
    wl = TINY_F32.shrink(name="pages", dtype="bf16", T=250, L_s=2, H_s=2, d_hs=64, r=128, L_t=2, H_q=8, H_kv=2,
                         d_h=128, D=256, c=32, pct=30)
    print("[select pages] handoff", flush=True)
    inp = synth.generate(wl, 82, DEV)
    h = Handoff(inp, DEV)
    h.cache.k.zero_()                                   # rows no step writes read as zeros
    h.cache.v.zero_()
    h.map()
    h.select()                                          # the position scores (its selection unused)
    scores = h.scores.clone()
    scores[wl.T - 3] = scores.max() * 100.0             # make the short last page [240, 250) win
    sel, rest, sb, _, psel = kvx.select_pages(scores, h.batch, 16, [wl.pct])
    assert int(psel[-1]) == (wl.T - 1) // 16 and sb.total_sel == 16 * (len(psel) - 1) + wl.T % 16
    kvx.reconstruct(h.z, inp.w_l, wl.H_kv, wl.d_h, sb, h.cache, rows=rest)
    torch.cuda.synchronize()
    K_tr = np.stack([f64(h.cache.k[l]) for l in range(wl.L_t)])
    V_tr = np.stack([f64(h.cache.v[l]) for l in range(wl.L_t)])
    S = sel.cpu().numpy().astype(np.int64)
    outs = [kvx.recompute_attn(l, inp.x_l[l], inp.w_qkv[l], wl.H_q, wl.H_kv, wl.d_h, h.rope, sb, sel, h.cache)
            for l in range(wl.L_t)]
    torch.cuda.synchronize()
    # the oracle's translated values on the complement (the device's selected rows were not
    # written by the reconstruction; the oracle's own values stand in there before the scatter)
    K_or, V_or, _ = O.reconstruct(f64(h.z), f64(inp.w_l), wl.H_kv, wl.d_h)
    C = rest.cpu().numpy()
    assert_close(K_tr[:, C], K_or[:, C], 1e-2, "translated K")
    K_tr[:, S], V_tr[:, S] = K_or[:, S], V_or[:, S]
    K, V, O_ref, _ = oracle_downstream(K_tr, V_tr, f64(inp.x_l), f64(inp.w_qkv), S, wl.H_q, wl.H_kv, wl.d_h,
                                       wl.rope_base)
    o = np.stack([f64(x) for x in outs])
    assert min_row_cosine(o.reshape(-1, wl.d_h), O_ref.reshape(-1, wl.d_h)) >= 0.999
    assert_close(o, O_ref, 2e-2, "attention out")
    assert_close(np.stack([f64(h.cache.k[l]) for l in range(wl.L_t)]), K, 2e-2, "K cache")
