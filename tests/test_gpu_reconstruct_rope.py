"""GPU parity of the reconstruction with rotated translated keys (kvx_reconstruct_rope) against
the oracle's reconstruct_rotated: the reading of the pages in which the mapper's keys carry no
rotary phase, so each translated key is rotated at its own position as recomputed keys are.

Cases: one request and a batch of three, contiguous and paged (16-token pages), d_h 128 and 64,
complement rows and all rows, and H_kv = 3 at d_h = 64 (the key/value boundary of a layer falls
inside one wave's 128 output columns, and the last column tile is half empty).  Checks: the keys
within the bf16 bar (2e-2 normwise and max-abs, per request and tensor: the value is rounded to
bf16 once before the rotation and once after, like the fused projection), the values bit for bit
equal to kvx_reconstruct's, the paged cache equal to the contiguous one, and rows outside the list
untouched.  fp32 (the reconstruction, then the keys rotated in place): bar 1e-4, with d_h 64 and 96
(no lane layout ties the fp32 path to 64 or 128).
"""
import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from cross_model_kv_amd.workloads import TINY_F32
from helpers import assert_close, f64, logical
from oracle import kvx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small(name, **kw):
    base = dict(name=name, dtype="bf16", T=420, L_s=2, H_s=2, d_hs=64, r=128, L_t=3, H_q=8, H_kv=2,
                d_h=128, D=256, c=64, pct=30)
    base.update(kw)
    return TINY_F32.shrink(**base)


CASES = {
    "d128-one-request": small("d128-one-request"),
    "d64-hkv3-batched-paged": small("d64-hkv3-batched-paged", d_h=64, H_kv=3, H_q=6, n_req=3, t_min=40,
                                    t_max=600, pct_choices=(20, 40), paged=True, page_size=16),
    "d128-batched-paged": small("d128-batched-paged", H_kv=4, H_q=16, n_req=3, t_min=100, t_max=500,
                                pct_choices=(30,), paged=True, page_size=16),
    "f32-d64-batched-paged": small("f32-d64-batched-paged", dtype="f32", d_h=64, H_kv=2, H_q=8, n_req=2, t_min=60,
                                   t_max=300, pct_choices=(30,), paged=True, page_size=16),
    "f32-d96-one-request": small("f32-d96-one-request", dtype="f32", d_h=96, H_kv=1, H_q=4),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("all_rows", [False, True], ids=["complement", "all-rows"])
def test_reconstruct_rope(name, all_rows):
    wl = CASES[name]
    print(f"[reconstruct_rope] {name} all_rows={all_rows}", flush=True)
    inp = synth.generate(wl, 81, DEV)
    batch = kvx.Batch.for_budgets(inp.lengths, inp.pcts, DEV)
    N = batch.n_tokens
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    bar = 1e-4 if wl.dtype == "f32" else 2e-2
    z = synth.latent(N, wl.r, 81, dtype=dt, device=DEV)
    S_list = [synth.random_subset(t, k, 81 + b) for b, (t, k) in enumerate(zip(inp.lengths, batch.n_sel))]
    C_list = [np.setdiff1d(np.arange(t), S) for t, S in zip(inp.lengths, S_list)]
    rest = None if all_rows else torch.from_numpy(np.concatenate(C_list).astype(np.int32)).to(DEV)
    rope = kvx.rope_table(wl.rope_base, wl.d_h, max(inp.lengths), DEV)
    shape = (wl.L_t, N, wl.H_kv, wl.d_h)
    cont = kvx.Cache(torch.full(shape, 7.0, dtype=dt, device=DEV),
                     torch.full(shape, 7.0, dtype=dt, device=DEV), wl.L_t, N)
    plain = kvx.Cache(torch.full(shape, 7.0, dtype=dt, device=DEV),
                      torch.full(shape, 7.0, dtype=dt, device=DEV), wl.L_t, N)
    kvx.reconstruct(z, inp.w_l, wl.H_kv, wl.d_h, batch, cont, rows=rest, rope=rope)
    kvx.reconstruct(z, inp.w_l, wl.H_kv, wl.d_h, batch, plain, rows=rest)
    pt = None
    if wl.paged:
        n_slots = inp.n_pages * wl.page_size
        ps = (wl.L_t, n_slots, wl.H_kv, wl.d_h)
        paged = kvx.Cache(torch.full(ps, 7.0, dtype=dt, device=DEV),
                          torch.full(ps, 7.0, dtype=dt, device=DEV), wl.L_t, n_slots,
                          page_table=inp.page_table, page_size=wl.page_size)
        kvx.reconstruct(z, inp.w_l, wl.H_kv, wl.d_h, batch, paged, rows=rest, rope=rope)
        pt = inp.page_table.cpu().numpy()
    torch.cuda.synchronize()
    assert torch.equal(cont.v, plain.v), "values differ from the plain reconstruction"
    for b, T in enumerate(inp.lengths):
        rows = np.arange(T) if all_rows else C_list[b]
        K = np.stack([logical(cont.k, l, b, T, batch.cu_tokens) for l in range(wl.L_t)])
        if wl.paged:
            Kp = np.stack([logical(paged.k, l, b, T, batch.cu_tokens, pt, wl.page_size) for l in range(wl.L_t)])
            Vp = np.stack([logical(paged.v, l, b, T, batch.cu_tokens, pt, wl.page_size) for l in range(wl.L_t)])
            V = np.stack([logical(cont.v, l, b, T, batch.cu_tokens) for l in range(wl.L_t)])
            assert np.array_equal(K, Kp) and np.array_equal(V, Vp), "paged and contiguous layouts differ"
        if not all_rows:
            assert np.all(K[:, S_list[b]] == 7.0), "selected rows were written"
        zb = f64(z[batch.cu_tokens[b]:batch.cu_tokens[b + 1]])
        K_ref, _, _ = O.reconstruct_rotated(zb, f64(inp.w_l), wl.H_kv, wl.d_h, np.arange(T), wl.rope_base)
        assert_close(K[:, rows], K_ref[:, rows], bar, f"rotated keys, request {b}")
        # the rotation moved them: the plain keys are far from the rotated ones past position 0
        K_plain = np.stack([logical(plain.k, l, b, T, batch.cu_tokens) for l in range(wl.L_t)])
        late = rows[rows > 8]
        assert np.linalg.norm(K[:, late] - K_plain[:, late]) > 0.1 * np.linalg.norm(K_plain[:, late])
