"""A whole handoff captured in a HIP graph (through torch's graph API) replays bit for bit.

No entry point allocates, copies or synchronises, so map, select, reconstruct and every layer's
fused projection and attention can be recorded once and replayed.  Each replay is checked
against the eager run, with eager work and synchronisations between the replays; the outputs
are cleared with a fill kernel (not a memset node) before each replay.  The eager result itself
is pinned to the oracle by the end-to-end parity tests."""
import pytest
import torch

from cross_model_kv_amd import synth
from cross_model_kv_amd.handoff import Handoff
from cross_model_kv_amd.workloads import TINY_F32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    "bf16-g4-d128": TINY_F32.shrink(name="graph-bf16", dtype="bf16", T=640, L_s=2, H_s=2, d_hs=64, r=128, L_t=3,
                                    H_q=8, H_kv=2, d_h=128, D=256, c=64, pct=30),
    "bf16-g8-batched-paged": TINY_F32.shrink(name="graph-paged", dtype="bf16", T=384, L_s=2, H_s=2, d_hs=64, r=128,
                                             L_t=2, H_q=16, H_kv=2, d_h=128, D=256, c=64, pct=30, n_req=3, t_min=60,
                                             t_max=900, pct_choices=(20, 30, 40), paged=True, page_size=16),
    "f32-tiny": TINY_F32,
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_handoff_graph_replay(name):
    wl = CASES[name]
    print(f"[graph] {name}", flush=True)
    inp = synth.generate(wl, 21, DEV)
    h = Handoff(inp, DEV)
    h.cache.k.zero_()                  # slots past a request's end (paged pools) are never written
    h.cache.v.zero_()
    h.run()
    torch.cuda.synchronize()
    ref = {"out": h.out.clone(), "lse": h.lse.clone(), "sel": h.S.clone(), "scores": h.scores.clone(),
           "k": h.cache.k.clone(), "v": h.cache.v.clone()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        h.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (h.out, h.lse, h.scores, h.cache.k, h.cache.v):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.out, ref["out"]), rep
        assert torch.equal(h.lse, ref["lse"]), rep
        assert torch.equal(h.S, ref["sel"]), rep
        assert torch.equal(h.scores, ref["scores"]), rep
        assert torch.equal(h.cache.k, ref["k"]) and torch.equal(h.cache.v, ref["v"]), rep
        h.run()                        # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(h.out, ref["out"]), rep
