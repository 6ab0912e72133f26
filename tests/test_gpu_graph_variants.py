"""The variant entry points captured in a HIP graph replay bit for bit: direct scoring of the stored
cache (per layer and summed, with its selection), per-layer selection sets, the normalized score
with its selection, the reconstruction with rotated keys and the QK-norm projection.

None of them allocates, copies or synchronises, so one capture records them all.  Each replay is
checked against the eager run, with eager work and synchronisations between the replays; the
outputs are cleared with a fill kernel (not a memset node) before each replay.  The eager results
are pinned to the oracle by the variants' own parity tests.
"""
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from cross_model_kv_amd.handoff import Handoff
from cross_model_kv_amd.workloads import TINY_F32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_variants_graph_replay():
    wl = TINY_F32.shrink(name="graph-variants", dtype="bf16", T=640, L_s=2, H_s=2, d_hs=64, r=128, L_t=3, H_q=8,
                         H_kv=2, d_h=128, D=256, c=64, pct=30, n_req=2, t_min=200, t_max=640, pct_choices=(30, 40))
    print("[graph] variants", flush=True)
    inp = synth.generate(wl, 23, DEV)
    h = Handoff(inp, DEV)
    h.cache.k.zero_()
    h.cache.v.zero_()
    h.map()
    kvx.reconstruct(h.z, inp.w_l, wl.H_kv, wl.d_h, h.batch, h.cache)          # every position
    b = h.batch
    N, K = b.n_tokens, b.total_sel
    L = wl.L_t
    op_c = kvx.score_cache_prepare(inp.u, kvx.BF16)
    op = kvx.score_prepare(inp.w_l, inp.u)
    op_tot = kvx.score_prepare(inp.w_l, inp.u[:, :, :0])
    cache2 = kvx.Cache.empty(L, N, wl.H_kv, wl.d_h, torch.bfloat16, DEV)
    cache2.k.zero_()
    cache2.v.zero_()
    gq = torch.linspace(0.5, 1.5, wl.d_h, device=DEV)
    gk = torch.linspace(1.5, 0.5, wl.d_h, device=DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    bufs = {
        "energy": torch.empty((L, N), **f32), "lsel": torch.empty((L, K), **i32), "lrest": torch.empty((L, N - K), **i32),
        "cs": torch.empty(N, **f32), "csel": torch.empty(K, **i32), "crest": torch.empty(N - K, **i32),
        "ns": torch.empty(N, **f32), "nsel": torch.empty(K, **i32), "nrest": torch.empty(N - K, **i32),
        "qkv": torch.empty((K, (wl.H_q + 2 * wl.H_kv) * wl.d_h), dtype=torch.bfloat16, device=DEV),
    }
    ws_c = torch.empty(4 * L * N + 4096, dtype=torch.uint8, device=DEV)
    ws_n = torch.empty(4 * 2 * N * 4 + 4096, dtype=torch.uint8, device=DEV)

    def run():
        kvx.score_cache(h.cache, 0, wl.H_kv, wl.d_h, op_c, b, energy=bufs["energy"], ws=ws_c)
        kvx.select_topk_layers(bufs["energy"], b, out=(bufs["lsel"], bufs["lrest"]))
        kvx.score_cache_select(h.cache, 0, wl.H_kv, wl.d_h, op_c, b, inp.pcts, ws=ws_c,
                               out=(bufs["cs"], bufs["csel"], bufs["crest"]))
        kvx.score_select_normalized(h.z, op, op_tot, b, inp.pcts, ws=ws_n, out=(bufs["ns"], bufs["nsel"], bufs["nrest"]))
        kvx.reconstruct(h.z, inp.w_l, wl.H_kv, wl.d_h, b, cache2, rope=h.rope)
        kvx.qkv_rope_scatter_qknorm(0, inp.x_l[0], inp.w_qkv[0], wl.H_q, wl.H_kv, wl.d_h, gq, gk, 1e-6, h.rope, b,
                                    bufs["nsel"], cache2, bufs["qkv"])

    outs = list(bufs.values()) + [cache2.k, cache2.v]
    for t in outs:                     # parts no call writes (the k and v columns of qkv) read as zeros
        t.zero_()
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    names = list(bufs) + ["cache2.k", "cache2.v"]
    for rep in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(names, outs, ref):
            assert torch.equal(t, r), (rep, name)
        run()                          # eager work between replays
        torch.cuda.synchronize()
