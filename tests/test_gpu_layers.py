"""Several target layers in one call (kvx_recompute_attn_layers and its two launches).

The grouped projection reads every layer's own input rows and weights and writes every
layer's q rows and cache layer; the attention launch runs the layers' workgroups one layer
after another.  Neither splits its work, so each layer's results must equal, bit for bit,
the same entry point called for that layer alone (n_layers = 1), and the attention must equal
kvx_sparse_attention of that layer without a workspace.  Any mistake in the per-layer offsets
(input rows, weights, q rows, cache layer, outputs, log-sum-exps) breaks the equality; the
end-to-end handoff tests compare the outputs of this path with the oracle (Handoff.run).
Cases: contiguous and paged caches, one and several requests, a layer range that starts past
layer 0, g = 4 and 5, d_h 64 and 128, fp32 (the single-layer kernels, layer by layer).
"""
import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from cross_model_kv_amd.handoff import Handoff
from cross_model_kv_amd.workloads import TINY_F32
from helpers import assert_close, f64, min_row_cosine, oracle_downstream
from oracle import kvx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small(name, **kw):
    base = dict(name=name, dtype="bf16", T=640, L_s=2, H_s=2, d_hs=64, r=128, L_t=5, H_q=8, H_kv=2,
                d_h=128, D=256, c=64, pct=30)
    base.update(kw)
    return TINY_F32.shrink(**base)


CASES = {
    "bf16-contig": small("bf16-contig"),
    "bf16-g5-d64": small("bf16-g5-d64", H_q=10, d_h=64, T=500, pct=40),
    "bf16-batched-paged": small("bf16-batched-paged", H_q=16, H_kv=4, n_req=3, t_min=80, t_max=700,
                                pct_choices=(20, 30, 40), paged=True, page_size=16),
    "f32-batched": TINY_F32.shrink(name="f32-batched", L_t=4, n_req=2, t_min=60, t_max=300,
                                   pct_choices=(20, 40)),
}


def _prepared(wl, seed):
    inp = synth.generate(wl, seed, DEV)
    h = Handoff(inp, DEV)
    h.cache.k.zero_()                          # slots no step writes compare equal
    h.cache.v.zero_()
    h.map()
    h.select()
    h.reconstruct()
    return inp, h


@pytest.mark.parametrize("name", list(CASES))
def test_layers_equal_single_layer_calls(name):
    wl = CASES[name]
    print(f"[layers] {name}", flush=True)
    inp, h = _prepared(wl, 61)
    k = h.batch.total_sel
    S = h.S
    l0, n = 1, wl.L_t - 1                     # a range that starts past layer 0
    # (a) all n layers in one call
    out_a = torch.zeros((n, k, wl.H_q, wl.d_h), dtype=inp.x_l.dtype, device=DEV)
    lse_a = torch.zeros((n, k, wl.H_q), dtype=torch.float32, device=DEV)
    kvx.recompute_attn_layers(l0, inp.x_l[l0:l0 + n], inp.w_qkv[l0:l0 + n], wl.H_q, wl.H_kv, wl.d_h, h.rope,
                              h.batch, S, h.cache, out=out_a, lse=lse_a)
    torch.cuda.synchronize()
    cache_a = (h.cache.k.clone(), h.cache.v.clone())
    # (b) the same entry point one layer at a time, on a fresh translated cache
    _, h2 = _prepared(wl, 61)
    assert torch.equal(h2.S, S)
    out_b = torch.zeros_like(out_a)
    lse_b = torch.zeros_like(lse_a)
    for j in range(n):
        kvx.recompute_attn_layers(l0 + j, inp.x_l[l0 + j:l0 + j + 1], inp.w_qkv[l0 + j:l0 + j + 1], wl.H_q,
                                  wl.H_kv, wl.d_h, h2.rope, h2.batch, S, h2.cache, out=out_b[j:j + 1],
                                  lse=lse_b[j:j + 1])
    torch.cuda.synchronize()
    assert torch.equal(h2.cache.k, cache_a[0]) and torch.equal(h2.cache.v, cache_a[1]), "cache"
    assert torch.equal(out_a, out_b), "attention outputs"
    assert torch.equal(lse_a, lse_b), "log-sum-exps"
    if wl.dtype == "bf16":
        # (c) the two launches apart, and the attention of each layer through the single-layer
        # entry point without a workspace, on the q rows of the grouped projection
        _, h3 = _prepared(wl, 61)
        qkv = kvx.qkv_rope_scatter_layers(l0, inp.x_l[l0:l0 + n], inp.w_qkv[l0:l0 + n], wl.H_q, wl.H_kv, wl.d_h,
                                          h3.rope, h3.batch, S, h3.cache)
        out_c = torch.zeros_like(out_a)
        kvx.sparse_attention_layers(l0, qkv, wl.H_q, wl.H_kv, wl.d_h, h3.rope, h3.batch, S, h3.cache, out_c)
        out_d = torch.zeros_like(out_a)
        lse_d = torch.zeros_like(lse_a)
        for j in range(n):
            kvx.sparse_attention(l0 + j, qkv[j], wl.H_q, wl.H_kv, wl.d_h, h3.rope, h3.batch, S, h3.cache, out_d[j],
                                 lse_d[j], split=False)
        torch.cuda.synchronize()
        assert torch.equal(h3.cache.k, cache_a[0]) and torch.equal(h3.cache.v, cache_a[1])
        assert torch.equal(out_c, out_a) and torch.equal(out_d, out_a) and torch.equal(lse_d, lse_a)
    else:
        # fp32: the single-layer entry point gives the same values
        _, h4 = _prepared(wl, 61)
        out_e = torch.zeros_like(out_a)
        for j in range(n):
            kvx.recompute_attn(l0 + j, inp.x_l[l0 + j], inp.w_qkv[l0 + j], wl.H_q, wl.H_kv, wl.d_h, h4.rope,
                               h4.batch, S, h4.cache, out=out_e[j])
        torch.cuda.synchronize()
        assert torch.equal(h4.cache.k, cache_a[0]) and torch.equal(h4.cache.v, cache_a[1])
        assert torch.equal(out_e, out_a)


def test_layers_against_oracle():
    """One request, all layers in one call, compared with the oracle's downstream steps on the
    device's own selection (bf16 tolerances of the end-to-end tests)."""
    wl = CASES["bf16-contig"]
    print("[layers] oracle", flush=True)
    inp, h = _prepared(wl, 62)
    K_tr = np.stack([f64(h.cache.k[l]) for l in range(wl.L_t)])
    V_tr = np.stack([f64(h.cache.v[l]) for l in range(wl.L_t)])
    S = h.S.cpu().numpy()
    out = kvx.recompute_attn_layers(0, inp.x_l, inp.w_qkv, wl.H_q, wl.H_kv, wl.d_h, h.rope, h.batch, h.S, h.cache)
    torch.cuda.synchronize()
    K, V, O_ref, _ = oracle_downstream(K_tr, V_tr, f64(inp.x_l), f64(inp.w_qkv), S, wl.H_q, wl.H_kv, wl.d_h,
                                       wl.rope_base)
    o = f64(out[:, :len(S)])
    assert min_row_cosine(o.reshape(-1, wl.d_h), O_ref.reshape(-1, wl.d_h)) >= 0.999
    assert_close(o, O_ref, 2e-2, "attention out")
    assert_close(np.stack([f64(h.cache.k[l]) for l in range(wl.L_t)]), K, 2e-2, "K cache")
