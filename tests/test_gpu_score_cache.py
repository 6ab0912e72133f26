"""GPU parity of the direct scoring of a stored cache (kvx_score_cache, kvx_score_cache_select)
and of per-layer selection sets (kvx_select_topk_layers) against the oracle's layer_disagreement,
select and select_per_layer, and of the handoff with per-layer sets against the oracle's
downstream steps.

The oracle reads exactly what the device read: the stored cache rows (bf16 or fp32, widened to
fp64) of every scored layer at every position's slot, and the fp32 bases.

Tolerances.  The energy of layer l at position t is |y|^2 - |U^T y|^2.  bf16: the products y u run
on the matrix cores with u split into two bf16 halves (together u to about 2^-17 relative) and fp32
accumulation over d_t terms, |y|^2 in fp32 from the same values, so the error stays below about
1e-5 |y|^2; the bar is 3e-5 |y|^2 per layer and position (and the sum of those for the summed
score).  fp32: every step in fp32, bar 1e-5 |y|^2.  Where floating point decides the sets, the
device's own scores decide them on both sides (bit-exact), and the oracle's sets must agree
outside the band of scores within twice the bar of the k-th.

Cases: contiguous and paged caches, one request and a batch of three with different budgets, a
scored layer range that starts past layer 0, c below one 256-direction tile and c over two (a
partial second tile), a basis that holds most of the energy (|E| a few percent of |y|^2), and the
16K workload's full shape (64 layers, 16384 positions, d_t = 2048, c = 512) checked on sampled
positions.
"""
import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from cross_model_kv_amd.handoff import Handoff
from cross_model_kv_amd.workloads import QWEN_8B_32B_16K, TINY_F32
from helpers import band_check, f64, oracle_downstream, slots_of, assert_close, min_row_cosine
from oracle import kvx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small(name, **kw):
    base = dict(name=name, dtype="bf16", T=700, L_s=2, H_s=2, d_hs=64, r=128, L_t=3, H_q=8, H_kv=2,
                d_h=128, D=256, c=40, pct=30)
    base.update(kw)
    return TINY_F32.shrink(**base)


# (workload, layer0, n_layers)
CASES = {
    "bf16-one-c40": (small("bf16-one-c40"), 1, 2),
    "bf16-c264-two-tiles": (small("bf16-c264", c=264, T=900), 0, 3),
    "bf16-mostly-inside": (small("bf16-inside", c=112, T=300, L_t=2), 0, 2),
    "bf16-batched-paged": (small("bf16-batched-paged", H_q=16, H_kv=4, d_h=64, c=64, n_req=3, t_min=80, t_max=700,
                                 pct_choices=(20, 30, 40), paged=True, page_size=16), 0, 3),
    "f32-batched": (TINY_F32.shrink(name="f32-batched", L_t=3, n_req=2, t_min=60, t_max=300, pct_choices=(20, 40)),
                    1, 2),
}


def _stored_rows(cache, layers, batch, lengths, page_table, positions=None):
    """Stored K and V [n_layers, n, H_kv, d_h] (fp64) of the batch's positions (or the listed global
    rows) in the given layers, in batch row order."""
    pt = page_table.cpu().numpy() if page_table is not None else None
    sl = np.concatenate([slots_of(b, T, batch.cu_tokens, pt) for b, T in enumerate(lengths)])
    if positions is not None:
        sl = sl[positions]
    idx = torch.as_tensor(sl, device=cache.k.device)
    K = np.stack([f64(cache.k[l][idx]) for l in layers])
    V = np.stack([f64(cache.v[l][idx]) for l in layers])
    return K, V


def _setup(wl, seed, mostly_inside=False, lengths=None, pcts=None):
    inp = synth.generate(wl, seed, DEV, lengths=lengths, pcts=pcts)
    h = Handoff(inp, DEV)
    h.map()
    kvx.reconstruct(h.z, inp.w_l, wl.H_kv, wl.d_h, h.batch, h.cache)          # every position
    u = inp.u
    if mostly_inside:
        # the bases of the mapped vectors' own dominant directions: most of each vector's energy
        # lies inside the span, so the energy outside is a small difference of large numbers
        d_t = 2 * wl.H_kv * wl.d_h
        us = []
        for l in range(wl.L_t):
            Y = f64(inp.w_l[l]) @ f64(h.z).T
            us.append(np.linalg.svd(Y, full_matrices=False)[0][:, :wl.c])
        u = torch.from_numpy(np.stack(us).astype(np.float32)).to(DEV)
        assert u.shape == (wl.L_t, d_t, wl.c)
    torch.cuda.synchronize()
    return inp, h, u


# requests of length 0 among others (lengths, budgets)
EMPTY = ([0, 257, 0, 64], [30, 30, 40, 100])


@pytest.mark.parametrize("name", list(CASES) + ["bf16-empty-requests"])
def test_score_cache_matches_oracle(name):
    lengths = pcts = None
    if name == "bf16-empty-requests":
        wl, l0, n = small("bf16-empty", n_req=4, t_min=1, t_max=300, pct_choices=(30,)), 0, 3
        lengths, pcts = EMPTY
    else:
        wl, l0, n = CASES[name]
    print(f"[score cache] {name}", flush=True)
    inp, h, u = _setup(wl, 71, mostly_inside=name == "bf16-mostly-inside", lengths=lengths, pcts=pcts)
    dt = kvx.BF16 if wl.dtype == "bf16" else kvx.F32
    op = kvx.score_cache_prepare(u[l0:l0 + n].contiguous(), dt)
    energy = kvx.score_cache(h.cache, l0, wl.H_kv, wl.d_h, op, h.batch)
    scores, sel, rest = kvx.score_cache_select(h.cache, l0, wl.H_kv, wl.d_h, op, h.batch, inp.pcts)
    sel_l, rest_l = kvx.select_topk_layers(energy.contiguous(), h.batch)
    torch.cuda.synchronize()

    K, V = _stored_rows(h.cache, range(l0, l0 + n), h.batch, inp.lengths, inp.page_table)
    E_ref = O.layer_disagreement(K, V, f64(u[l0:l0 + n]))
    yy = np.sum(K.reshape(n, len(K[0]), -1) ** 2, axis=2) + np.sum(V.reshape(n, len(V[0]), -1) ** 2, axis=2)
    bar = 3e-5 if wl.dtype == "bf16" else 1e-5
    E = f64(energy)
    err = np.abs(E - E_ref) / yy
    print(f"  max |dE| / |y|^2 = {err.max():.2e}; E / |y|^2 in [{(E_ref / yy).min():.3f}, {(E_ref / yy).max():.3f}]",
          flush=True)
    assert err.max() <= bar
    if name == "bf16-mostly-inside":
        assert (E_ref / yy).max() < 0.1                 # the case really is a small difference
    s = f64(scores)
    s_ref = E_ref.sum(axis=0)
    assert np.all(np.abs(s - s_ref) <= bar * yy.sum(axis=0))
    # the summed score is the layer sum of the returned energies (fixed order, fp32)
    assert np.abs(s - E.sum(axis=0)).max() <= 1e-6 * s.max()

    sel_h, rest_h = sel.cpu().numpy(), rest.cpu().numpy()
    sl_h, rl_h = sel_l.cpu().numpy(), rest_l.cpu().numpy()
    cs, cr = h.batch.cu_sel, [c - k for c, k in zip(h.batch.cu_tokens, h.batch.cu_sel)]
    for b, T in enumerate(inp.lengths):
        rows = slice(h.batch.cu_tokens[b], h.batch.cu_tokens[b + 1])
        k = O.budget(T, inp.pcts[b])
        # summed score: the device's sets are the exact top-k of its scores, and the oracle's
        # outside the band
        S_own, C_own = O.select(s[rows], k)
        assert np.array_equal(sel_h[cs[b]:cs[b + 1]], S_own) and np.array_equal(rest_h[cr[b]:cr[b + 1]], C_own)
        if 0 < k < T:
            tau = np.sort(s_ref[rows])[::-1][k - 1]
            band_check(sel_h[cs[b]:cs[b + 1]], s_ref[rows], k, 2 * bar * yy.sum(axis=0)[rows].max() / tau)
        # per-layer sets: every layer's own top-k of its energies
        S_l, C_l = O.select_per_layer(E[:, rows], k)
        assert np.array_equal(sl_h[:, cs[b]:cs[b + 1]], S_l) and np.array_equal(rl_h[:, cr[b]:cr[b + 1]], C_l)
        for j in range(n):
            if 0 < k < T:
                tau = np.sort(E_ref[j, rows])[::-1][k - 1]
                band_check(sl_h[j, cs[b]:cs[b + 1]], E_ref[j, rows], k, 2 * bar * yy[j, rows].max() / tau)


def test_score_cache_full_shape_sampled():
    """The 16K workload's shape: 64 layers of 16384 positions, H_kv = 8, d_h = 128, c = 512, in the
    launch the bench times; the oracle on 48 sampled positions (first, last and random)."""
    wl = QWEN_8B_32B_16K
    L, N, d_t = wl.L_t, wl.T, 2 * wl.H_kv * wl.d_h
    print("[score cache] full shape", flush=True)
    k = synth.cache_fill((L, N, wl.H_kv, wl.d_h), 72, device=DEV)
    v = synth.cache_fill((L, N, wl.H_kv, wl.d_h), 73, device=DEV)
    cache = kvx.Cache(k, v, L, N)
    rng = np.random.default_rng(74)
    u = torch.from_numpy(np.stack([synth.orthonormal_basis(rng, d_t, wl.c) for _ in range(L)]).astype(np.float32))
    u = u.to(DEV)
    batch = kvx.Batch.for_budgets([N], [wl.pct], DEV)
    op = kvx.score_cache_prepare(u, kvx.BF16)
    energy = kvx.score_cache(cache, 0, wl.H_kv, wl.d_h, op, batch)
    scores, sel, rest = kvx.score_cache_select(cache, 0, wl.H_kv, wl.d_h, op, batch, [wl.pct])
    torch.cuda.synchronize()
    pos = np.unique(np.concatenate([[0, 1, 255, 256, N - 1], rng.choice(N, 43, replace=False)]))
    idx = torch.as_tensor(pos, device=DEV)
    K = np.stack([f64(k[l][idx]) for l in range(L)])
    V = np.stack([f64(v[l][idx]) for l in range(L)])
    E_ref = O.layer_disagreement(K, V, f64(u))
    yy = np.sum(K.reshape(L, len(pos), -1) ** 2, axis=2) + np.sum(V.reshape(L, len(pos), -1) ** 2, axis=2)
    E = f64(energy[:, idx])
    err = np.abs(E - E_ref) / yy
    print(f"  max |dE| / |y|^2 = {err.max():.2e} over {len(pos)} positions x {L} layers", flush=True)
    assert err.max() <= 3e-5
    s = f64(scores)
    assert np.all(np.abs(s[pos] - E_ref.sum(axis=0)) <= 3e-5 * yy.sum(axis=0))
    S_own, C_own = O.select(s, O.budget(N, wl.pct))
    assert np.array_equal(sel.cpu().numpy(), S_own) and np.array_equal(rest.cpu().numpy(), C_own)


def test_layer_sets_handoff_against_oracle():
    """The handoff with per-layer sets: every position translated, each layer scored from its own
    stored K/V, its own top-k recomputed (kvx_recompute_attn with that layer's set), compared with
    the oracle's recompute, scatter and attention on the device's sets (bf16 tolerances of the
    end-to-end tests); the sets differ between layers."""
    wl = small("layer-sets", T=640, L_t=3, c=64, pct=30)
    print("[score cache] layer-set handoff", flush=True)
    inp, h, u = _setup(wl, 75)
    op = kvx.score_cache_prepare(u.contiguous(), kvx.BF16)
    energy = kvx.score_cache(h.cache, 0, wl.H_kv, wl.d_h, op, h.batch)
    sel_l, _ = kvx.select_topk_layers(energy.contiguous(), h.batch)
    torch.cuda.synchronize()
    K_tr = np.stack([f64(h.cache.k[l]) for l in range(wl.L_t)])
    V_tr = np.stack([f64(h.cache.v[l]) for l in range(wl.L_t)])
    S = sel_l.cpu().numpy().astype(np.int64)
    assert any(not np.array_equal(S[0], S[l]) for l in range(1, wl.L_t))
    outs = [kvx.recompute_attn(l, inp.x_l[l], inp.w_qkv[l], wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch,
                               sel_l[l].contiguous(), h.cache) for l in range(wl.L_t)]
    torch.cuda.synchronize()
    for l in range(wl.L_t):
        Kl, Vl, O_ref, _ = oracle_downstream(K_tr[l:l + 1], V_tr[l:l + 1], f64(inp.x_l[l:l + 1]),
                                             f64(inp.w_qkv[l:l + 1]), S[l], wl.H_q, wl.H_kv, wl.d_h, wl.rope_base)
        o = f64(outs[l])[None]
        assert min_row_cosine(o.reshape(-1, wl.d_h), O_ref.reshape(-1, wl.d_h)) >= 0.999
        assert_close(o, O_ref, 2e-2, f"layer {l} attention out")
        assert_close(f64(h.cache.k[l])[None], Kl, 2e-2, f"layer {l} K cache")
        # rows outside the layer's set keep the translated values exactly
        C = np.setdiff1d(np.arange(wl.T), S[l])
        assert np.array_equal(f64(h.cache.k[l])[C], K_tr[l][C]) and np.array_equal(f64(h.cache.v[l])[C], V_tr[l][C])
