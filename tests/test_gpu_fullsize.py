"""Parity at the full workload sizes, in the call sequence bench.py times, on sampled outputs.

For every large workload (0.6B->14B-, 8B->32B-, 8B->70B-shaped, the 16-request paged batch and a
131,072-position context with the 8B->32B shapes)
one whole handoff runs on the GPU, then the fp64 oracle recomputes sampled outputs one by one
from the generated inputs:

* latent rows, scores of sampled positions, translated cache rows of sampled complement
  positions and recomputed K/V rows of sampled selected positions (bf16 storage: 2e-2);
* the selected sets: sizes, ascending order, disjoint cover of the positions, and exactly the
  top-k of the returned scores (ties to the lower position);
* attention outputs of early selected queries end to end (the oracle rebuilds the mixed cache
  prefix from the inputs), min row cosine 0.999;
* attention of late selected queries stage-wise: one layer's cache is refilled with a seeded
  stand-in and recomputed for a seeded selected set, so the oracle needs only that layer.
"""
import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth, workloads
from cross_model_kv_amd.handoff import Handoff
from helpers import assert_close, f64, logical, min_row_cosine, rel_norm
from oracle import kvx_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda:0"
# a long context: the 8B->32B head shapes, latent and hidden sizes at 131,072 positions, with two
# source and two target layers so the inputs stay a few GB (select runs past its LDS key copy,
# the last query blocks walk 2048 key tiles)
LONG = workloads.ALL["8B-to-32B-shape-T16384"].shrink(name="8B-to-32B-heads-T131072-2-layers", T=131072,
                                                      L_s=2, L_t=2, pct=2)
WORKLOADS = dict(workloads.ALL, **{LONG.name: LONG})
LARGE = ["0.6B-to-14B-shape-T4096", "8B-to-32B-shape-T16384", "8B-to-70B-shape-T8192", "batched-16req-paged16",
         LONG.name]
SEEDS = {"0.6B-to-14B-shape-T4096": 2, "8B-to-32B-shape-T16384": 3, "8B-to-70B-shape-T8192": 4,
         "batched-16req-paged16": 5, LONG.name: 6}


def say(msg):
    print(msg, flush=True)


def _rows(t, idx):
    return f64(t[torch.as_tensor(np.asarray(idx), device=t.device)])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", LARGE)
def test_fullsize_sampled(name):
    wl = WORKLOADS[name]
    seed = SEEDS[name]
    say(f"[fullsize] {name} seed {seed}: generating inputs")
    inp = synth.generate(wl, seed, DEV)
    h = Handoff(inp, DEV)
    say(f"[fullsize] {name}: running the handoff")
    h.run()
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    cu, cs = inp.cu_tokens, h.batch.cu_sel
    n_req = len(inp.lengths)
    reqs = [0] if n_req == 1 else sorted(rng.choice(n_req, 2, replace=False).tolist())
    layers = sorted(rng.choice(wl.L_t, 2, replace=False).tolist())
    pt = inp.page_table.cpu().numpy() if wl.paged else None
    sel_all, rest_all, scores = h.S.cpu().numpy(), h.C.cpu().numpy(), f64(h.scores)

    # selected sets: sizes, order, cover, exact top-k of the returned scores
    for b in range(n_req):
        T, k = inp.lengths[b], O.budget(inp.lengths[b], inp.pcts[b])
        S = sel_all[cs[b]:cs[b + 1]]
        C = rest_all[cu[b] - cs[b]:cu[b + 1] - cs[b + 1]]
        assert len(S) == k and np.all(np.diff(S) > 0) and np.all(np.diff(C) > 0)
        assert np.array_equal(np.sort(np.concatenate([S, C])), np.arange(T))
        S_own, _ = O.select(scores[cu[b]:cu[b + 1]].astype(np.float32).astype(np.float64), k)
        assert np.array_equal(S, S_own)

    w_s = f64(inp.w_s)
    w_l = f64(inp.w_l)
    u = f64(inp.u)
    for b in reqs:
        T = inp.lengths[b]
        S = sel_all[cs[b]:cs[b + 1]]
        C = rest_all[cu[b] - cs[b]:cu[b + 1] - cs[b + 1]]
        say(f"[fullsize] {name}: request {b} (T={T}, k={len(S)}), layers {layers}")
        # latent rows and scores of sampled positions (oracle from the source KV)
        pos = np.sort(rng.choice(T, 12, replace=False))
        z_ref = O.map_latent(_rows(inp.x_src, cu[b] + pos), w_s)
        assert_close(_rows(h.z, cu[b] + pos), z_ref, 2e-2, "latent rows")
        _, _, Y = O.reconstruct(z_ref, w_l, wl.H_kv, wl.d_h)
        s_ref = O.rank_disagreement(Y, u)
        err = np.max(np.abs(scores[cu[b] + pos] - s_ref) / s_ref)
        say(f"   score rel err (bf16 latent vs fp64) {err:.2e}")
        assert err <= 1e-2
        # translated rows at sampled complement positions
        pc = np.sort(rng.choice(C, 8, replace=False))
        zc = O.map_latent(_rows(inp.x_src, cu[b] + pc), w_s)
        Kt, Vt, _ = O.reconstruct(zc, w_l, wl.H_kv, wl.d_h)
        for l in layers:
            Kg = logical(h.cache.k, l, b, T, cu, pt, wl.page_size)
            Vg = logical(h.cache.v, l, b, T, cu, pt, wl.page_size)
            assert_close(Kg[pc], Kt[l], 2e-2, "translated K")
            assert_close(Vg[pc], Vt[l], 2e-2, "translated V")
        # recomputed rows at sampled selected positions, and early queries end to end
        ps = np.sort(rng.choice(S, 8, replace=False))
        for l in layers:
            wq = f64(inp.w_qkv[l])
            _, kk, vv = O.recompute_qkv(_rows(inp.x_l[l], cu[b] + ps), wq, ps, wl.H_q, wl.H_kv, wl.d_h,
                                        wl.rope_base)
            Kg = logical(h.cache.k, l, b, T, cu, pt, wl.page_size)
            Vg = logical(h.cache.v, l, b, T, cu, pt, wl.page_size)
            assert_close(Kg[ps], kk, 2e-2, "recomputed K")
            assert_close(Vg[ps], vv, 2e-2, "recomputed V")
            # early queries: rebuild the mixed cache prefix [0, P] from the inputs
            early = np.nonzero(S < 600)[0][:6]
            if len(early) == 0:
                continue
            P = int(S[early[-1]]) + 1
            z_pre = O.map_latent(_rows(inp.x_src, cu[b] + np.arange(P)), w_s)
            Kp, Vp, _ = O.reconstruct(z_pre, w_l[l:l + 1], wl.H_kv, wl.d_h)
            Sp = S[S < P]
            q, k2, v2 = O.recompute_qkv(_rows(inp.x_l[l], cu[b] + Sp), wq, Sp, wl.H_q, wl.H_kv, wl.d_h,
                                        wl.rope_base)
            Km, Vm = O.scatter(Kp[0], Vp[0], Sp, k2, v2)
            o_ref, _ = O.sparse_causal_attention(q[early], Km, Vm, Sp[early])
            o = _rows(h.out[l], cs[b] + early)
            cos = min_row_cosine(o, o_ref)
            say(f"   layer {l}: early queries {Sp[early].tolist()} min cosine {cos:.6f}")
            assert cos >= 0.999
            assert_close(o, o_ref, 2e-2, "attention (early queries)")

    # late queries, stage-wise: refill one layer with a stand-in and recompute a seeded set
    b = reqs[-1]
    T = inp.lengths[b]
    l = layers[-1]
    k = O.budget(T, inp.pcts[b])
    S_list = []
    for bb in range(n_req):
        Tb = inp.lengths[bb]
        S_list.append(synth.random_subset(Tb, O.budget(Tb, inp.pcts[bb]), seed + 100 + bb))
    sel = torch.from_numpy(np.concatenate(S_list).astype(np.int32)).to(DEV)
    shape = (h.cache.k.shape[1], wl.H_kv, wl.d_h)
    h.cache.k[l].copy_(synth.cache_fill(shape, seed + 7, dtype=torch.bfloat16, device=DEV))
    h.cache.v[l].copy_(synth.cache_fill(shape, seed + 8, dtype=torch.bfloat16, device=DEV))
    K0 = logical(h.cache.k, l, b, T, cu, pt, wl.page_size)
    V0 = logical(h.cache.v, l, b, T, cu, pt, wl.page_size)
    out = kvx.recompute_attn(l, inp.x_l[l], inp.w_qkv[l], wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch, sel, h.cache)
    torch.cuda.synchronize()
    S = S_list[b]
    say(f"[fullsize] {name}: stage-wise recompute of layer {l}, request {b}, late queries")
    q, kk, vv = O.recompute_qkv(_rows(inp.x_l[l], cu[b] + S), f64(inp.w_qkv[l]), S, wl.H_q, wl.H_kv, wl.d_h,
                                wl.rope_base)
    Km, Vm = O.scatter(K0, V0, S, kk, vv)
    late = np.arange(len(S) - 4, len(S))
    o_ref, _ = O.sparse_causal_attention(q[late], Km, Vm, S[late])
    o = _rows(out, cs[b] + late)
    cos = min_row_cosine(o, o_ref)
    say(f"   late queries {S[late].tolist()} min cosine {cos:.6f} normwise {rel_norm(o, o_ref):.2e}")
    assert cos >= 0.999
    assert_close(o, o_ref, 2e-2, "attention (late queries)")
    Kg = logical(h.cache.k, l, b, T, cu, pt, wl.page_size)
    assert_close(Kg[S[late]], kk[late], 2e-2, "recomputed K (late)")
    del h, inp, out
    torch.cuda.empty_cache()
