"""GPU parity of the chained target layers (through the C ABI) against the fp64 oracle.

The building blocks (RMS norm, output projection + residual, SiLU-gated MLP) are checked
alone, over ragged tiles and the split-along-K path; a layer with zero residual branches
must pass its rows through bit for bit; and whole chained handoffs (map, select,
reconstruct, then every layer on the selected rows) are compared with the oracle's
chained layers run on the GPU's selected set.  Tolerances as for the handoff: bf16
storage 2e-2 relative (normwise and max-abs per tensor), attention rows minimum cosine
0.999.
"""
import math

import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from cross_model_kv_amd.handoff import ChainedHandoff
from cross_model_kv_amd.workloads import TINY_F32
from helpers import assert_close, f64, logical, min_row_cosine, rel_norm
from oracle import kvx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def normal(shape, seed, std=1.0):
    n = int(np.prod(shape))
    return (synth.latent(n // shape[-1], shape[-1], seed, dtype=torch.float32, device=DEV) * std).to(torch.bfloat16)


# ------------------------------------------------------------------------------ building blocks

@pytest.mark.parametrize("n,D", [(37, 256), (300, 5120), (5, 16384)])
def test_rmsnorm(n, D):
    say(f"[chain] rmsnorm n={n} D={D}")
    x = normal((n, D), 91, 3.0)
    gamma = (synth.latent(1, D, 92, dtype=torch.float32, device=DEV)[0] * 0.2 + 1.0).to(torch.bfloat16)
    y = kvx.rmsnorm(x, gamma, 1e-6)
    x2 = x.clone()
    kvx.rmsnorm(x2, gamma, 1e-6, y=x2)          # in place
    torch.cuda.synchronize()
    assert_close(f64(y), O.rmsnorm(f64(x), f64(gamma), 1e-6), 1e-2, "rmsnorm")
    assert torch.equal(y, x2)


@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (64, 4096, 4096), (1, 520, 1024), (5, 4096, 4096)])
def test_linear_residual(M, N, K):
    say(f"[chain] linear+residual M={M} N={N} K={K}")
    a, w, r = normal((M, K), 93), normal((N, K), 94, 1 / math.sqrt(K)), normal((M, N), 95)
    out = kvx.linear_residual(a, w, r)
    r2 = r.clone()
    kvx.linear_residual(a, w, r2, out=r2)       # in place: out is the residual
    torch.cuda.synchronize()
    assert_close(f64(out), f64(r) + f64(a) @ f64(w).T, 2e-2, "linear + residual")
    assert torch.equal(out, r2)


@pytest.mark.parametrize("M,D,F", [(300, 512, 776), (64, 4096, 512), (2, 512, 776), (16, 1024, 2048)])
def test_swiglu(M, D, F):
    say(f"[chain] swiglu M={M} D={D} F={F}")
    x, wg, wu = normal((M, D), 96), normal((F, D), 97, 1 / math.sqrt(D)), normal((F, D), 98, 1 / math.sqrt(D))
    h = kvx.swiglu(x, wg, wu)
    h2 = kvx.swiglu(x, wg, wu)
    torch.cuda.synchronize()
    ref = O.silu(f64(x) @ f64(wg).T) * (f64(x) @ f64(wu).T)
    assert_close(f64(h), ref, 2e-2, "gated MLP rows")
    assert torch.equal(h, h2)


def test_split_paths_engaged():
    """The second shape of each GEMM test above takes the split-along-K path."""
    import ctypes
    b = ctypes.c_size_t()
    assert kvx.lib().kvx_linear_residual_workspace(kvx.BF16, 64, 4096, 4096, ctypes.byref(b)) == 0 and b.value > 0
    assert kvx.lib().kvx_swiglu_workspace(kvx.BF16, 64, 4096, 512, ctypes.byref(b)) == 0 and b.value > 0


# ------------------------------------------------------------------------------ whole layers

def small(name, **kw):
    base = dict(name=name, dtype="bf16", T=384, L_s=2, H_s=2, d_hs=64, r=128, L_t=3, H_q=8, H_kv=2,
                d_h=128, D=256, c=64, pct=30, F=512)
    base.update(kw)
    return TINY_F32.shrink(**base)


CHAIN_CASES = {
    "chain-g4-d128": small("chain-g4-d128"),
    "chain-g4-d64": small("chain-g4-d64", d_h=64, F=768, T=300),
    "chain-g8-batched-paged": small("chain-g8-batched-paged", H_q=16, H_kv=2, n_req=3, t_min=60, t_max=500,
                                    pct_choices=(20, 30, 40), paged=True, F=640, L_t=2),
    # wide rows: every projection of the layer has few tiles and is split along K
    "chain-wide-D": small("chain-wide-D", D=2048, F=4096, T=500, pct=40, L_t=2),
}


def _layer_dicts(inp, cw, wl):
    return [dict(gamma_in=f64(cw.gamma_in[l]), w_qkv=f64(inp.w_qkv[l]), w_o=f64(cw.w_o[l]),
                 gamma_post=f64(cw.gamma_post[l]), w_gate=f64(cw.w_gate[l]), w_up=f64(cw.w_up[l]),
                 w_down=f64(cw.w_down[l])) for l in range(wl.L_t)]


@pytest.mark.parametrize("name", sorted(CHAIN_CASES))
def test_chained_handoff(name):
    wl = CHAIN_CASES[name]
    seed = 31
    say(f"[chain] handoff {name}")
    inp = synth.generate(wl, seed, DEV)
    cw = synth.chain_weights(wl, seed, DEV)
    h = ChainedHandoff(inp, cw, DEV)
    h.run()
    torch.cuda.synchronize()
    layers = _layer_dicts(inp, cw, wl)
    cu, cs = h.batch.cu_tokens, h.batch.cu_sel
    pt = inp.page_table.cpu().numpy() if wl.paged else None
    S_all = h.S.cpu().numpy()
    x_rows = f64(h.x)
    for b, T in enumerate(inp.lengths):
        S = S_all[cs[b]:cs[b + 1]]
        if len(S) == 0:
            continue
        z = O.map_latent(f64(inp.x_src[cu[b]:cu[b + 1]]), f64(inp.w_s))
        K_tr, V_tr, _ = O.reconstruct(z, f64(inp.w_l), wl.H_kv, wl.d_h)
        ref = O.chained_layers(f64(inp.x_l[0, cu[b]:cu[b + 1]])[S], S, K_tr, V_tr, layers, wl.H_q, wl.H_kv,
                               wl.d_h, wl.rope_base, wl.norm_eps)
        for l in range(wl.L_t):
            o = f64(h.out[l, cs[b]:cs[b + 1]])
            cos = min_row_cosine(o, ref["O"][l])
            say(f"  request {b} (T={T}, k={len(S)}) layer {l}: attention min cosine {cos:.6f}")
            assert cos >= 0.999
            assert_close(o, ref["O"][l], 2e-2, f"attention rows, layer {l}")
            Kg = logical(h.cache.k, l, b, T, cu, pt, wl.page_size)
            Vg = logical(h.cache.v, l, b, T, cu, pt, wl.page_size)
            assert_close(Kg[S], ref["K"][l][S], 2e-2, f"recomputed K, layer {l}")
            assert_close(Vg[S], ref["V"][l][S], 2e-2, f"recomputed V, layer {l}")
        xo = x_rows[cs[b]:cs[b + 1]]
        say(f"  request {b}: final rows normwise {rel_norm(xo, ref['X'][-1]):.2e}")
        assert_close(xo, ref["X"][-1], 2e-2, "final rows")


def test_layer_pass_through_bitexact():
    """W_o = 0 and W_down = 0: the rows leave the layer unchanged bit for bit, and the cache
    and attention rows equal those of the separate calls on the normalised rows."""
    wl = CHAIN_CASES["chain-g4-d128"]
    say("[chain] pass-through layer")
    inp = synth.generate(wl, 33, DEV)
    cw = synth.chain_weights(wl, 33, DEV)
    batch = kvx.Batch.for_budgets(inp.lengths, inp.pcts, DEV)
    S = synth.random_subset(inp.lengths[0], batch.n_sel[0], 33)
    sel = torch.from_numpy(S).to(DEV)
    N = batch.n_tokens
    k0 = synth.cache_fill((wl.L_t, N, wl.H_kv, wl.d_h), 34, device=DEV)
    v0 = synth.cache_fill((wl.L_t, N, wl.H_kv, wl.d_h), 35, device=DEV)
    c1 = kvx.Cache(k0.clone(), v0.clone(), wl.L_t, N)
    c2 = kvx.Cache(k0.clone(), v0.clone(), wl.L_t, N)
    rope = kvx.rope_table(wl.rope_base, wl.d_h, max(inp.lengths), DEV)
    zero_o, zero_down = torch.zeros_like(cw.w_o[0]), torch.zeros_like(cw.w_down[0])
    w = kvx.LayerWeights(cw.gamma_in[0], inp.w_qkv[0], zero_o, cw.gamma_post[0], cw.w_gate[0], cw.w_up[0], zero_down)
    x = kvx.gather_rows(inp.x_l[0], batch, sel)
    x_in = x.clone()
    o1 = torch.empty((len(S), wl.H_q, wl.d_h), dtype=torch.bfloat16, device=DEV)
    kvx.target_layer(0, x, w, wl.F, wl.H_q, wl.H_kv, wl.d_h, wl.norm_eps, rope, batch, sel, c1, attn_out=o1)
    # the same steps through the separate calls: normalised rows placed at their batch rows
    xn = kvx.rmsnorm(x_in, cw.gamma_in[0], wl.norm_eps)
    x_full = torch.zeros((N, wl.D), dtype=torch.bfloat16, device=DEV)
    x_full[sel.long()] = xn
    qkv = kvx.qkv_rope_scatter(0, x_full, inp.w_qkv[0], wl.H_q, wl.H_kv, wl.d_h, rope, batch, sel, c2)
    o2 = torch.empty_like(o1)
    kvx.sparse_attention(0, qkv, wl.H_q, wl.H_kv, wl.d_h, rope, batch, sel, c2, o2)
    torch.cuda.synchronize()
    assert torch.equal(x, x_in), "rows changed"
    assert torch.equal(x_in, inp.x_l[0][sel.long()]), "gathered rows differ"  # one request: rows = positions
    assert torch.equal(c1.k, c2.k) and torch.equal(c1.v, c2.v), "caches differ"
    assert torch.equal(o1, o2), "attention rows differ"


# ------------------------------------------------------------------------------ first token

@pytest.mark.parametrize("M,N,K", [(1, 5000, 1024), (3, 2048, 4096), (16, 1000, 25600), (17, 520, 512),
                                   (300, 520, 512)])
def test_linear(M, N, K):
    """Plain projection, including the few-row shapes of the first-token step (up to 16 rows:
    the weight-streaming kernel, every output tile reduced with the usual epilogue)."""
    say(f"[first token] linear M={M} N={N} K={K}")
    a, w = normal((M, K), 101), normal((N, K), 102, 1 / math.sqrt(K))
    out = kvx.linear(a, w)
    out2 = kvx.linear(a, w)
    torch.cuda.synchronize()
    assert_close(f64(out), f64(a) @ f64(w).T, 2e-2, "linear")
    assert torch.equal(out, out2)


def test_argmax_ties_lowest():
    """Exact decisions on the stored values: ties (including many equal maxima) go to the
    lowest index; compared with the brute-force argmax of the same bf16 values."""
    say("[first token] argmax")
    rng = np.random.default_rng(103)
    rows = [rng.standard_normal(5000), np.zeros(777), np.full(300, -3.0), rng.integers(-3, 4, 4096).astype(float)]
    for r in rows:
        x = torch.tensor(r, dtype=torch.float32).to(torch.bfloat16).to(DEV)[None, :]
        got = int(kvx.argmax(x).cpu()[0])
        vals = x.float().cpu().numpy()[0]
        assert got == int(np.argmax(vals)), (got, int(np.argmax(vals)))


FT_CASES = {
    "ft-g4-d128": small("ft-g4-d128", vocab=1000),
    "ft-g8-batched-paged": small("ft-g8-batched-paged", H_q=16, H_kv=2, n_req=3, t_min=60, t_max=500,
                                 pct_choices=(20, 30, 40), paged=True, F=640, L_t=2, vocab=2048),
}


@pytest.mark.parametrize("name", sorted(FT_CASES))
def test_first_token(name):
    """Chained handoff, then the first-token step: logits and the last position's cache rows
    match the oracle; the token is the argmax of the GPU's own logits (an exact decision)
    and its oracle logit lies within the bf16 tolerance of the oracle's maximum."""
    wl = FT_CASES[name]
    seed = 41
    say(f"[first token] {name}")
    inp = synth.generate(wl, seed, DEV)
    cw = synth.chain_weights(wl, seed, DEV)
    h = ChainedHandoff(inp, cw, DEV)
    h.run()
    h.prepare_first_token()
    h.first_token()
    torch.cuda.synchronize()
    layers = _layer_dicts(inp, cw, wl)
    cu, cs = h.batch.cu_tokens, h.batch.cu_sel
    pt = inp.page_table.cpu().numpy() if wl.paged else None
    S_all = h.S.cpu().numpy()
    logits = f64(h.logits)
    tokens = h.token.cpu().numpy()
    for b, T in enumerate(inp.lengths):
        S = S_all[cs[b]:cs[b + 1]]
        z = O.map_latent(f64(inp.x_src[cu[b]:cu[b + 1]]), f64(inp.w_s))
        K_tr, V_tr, _ = O.reconstruct(z, f64(inp.w_l), wl.H_kv, wl.d_h)
        if len(S):
            ch = O.chained_layers(f64(inp.x_l[0, cu[b]:cu[b + 1]])[S], S, K_tr, V_tr, layers, wl.H_q, wl.H_kv,
                                  wl.d_h, wl.rope_base, wl.norm_eps)
            K_m, V_m = ch["K"], ch["V"]
        else:
            K_m, V_m = K_tr, V_tr
        ref_logits, ref_tok, K_f, V_f = O.first_token(f64(inp.x_l[0, cu[b] + T - 1]), T - 1, K_m, V_m, layers,
                                                      f64(cw.gamma_final), f64(cw.w_lm), wl.H_q, wl.H_kv, wl.d_h,
                                                      wl.rope_base, wl.norm_eps)
        say(f"  request {b} (T={T}): logits normwise {rel_norm(logits[b], ref_logits):.2e}, token {tokens[b]} "
            f"(oracle {ref_tok})")
        assert_close(logits[b], ref_logits, 2e-2, "first-token logits")
        assert tokens[b] == int(np.argmax(logits[b])), "token is not the argmax of the stored logits"
        span = ref_logits.max() - ref_logits.min()
        assert ref_logits.max() - ref_logits[tokens[b]] <= 2e-2 * span
        for l in range(wl.L_t):
            Kg = logical(h.cache.k, l, b, T, cu, pt, wl.page_size)
            Vg = logical(h.cache.v, l, b, T, cu, pt, wl.page_size)
            assert_close(Kg[T - 1], K_f[l][T - 1], 2e-2, f"last position K, layer {l}")
            assert_close(Vg[T - 1], V_f[l][T - 1], 2e-2, f"last position V, layer {l}")
