"""Paged caches of every page-size class against the same data laid out contiguously and
against the oracle.

The attention looks pages up three ways: one wave-uniform page-table read per 1 KB load block
(power-of-two pages holding at least one block's keys), a per-lane lookup in the page table
staged in LDS (other page sizes, and a request's last tile), and a per-lane lookup in HBM (tables
longer than the LDS copy).  The fused projection writes k and v through the same slot map.
Sizes 1, 3, 4, 8, 16, 24 and 64 with d_h 64 and 128 reach every one of these paths; page size 1
with a 2300-token request gives a table longer than the LDS copy."""
import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth
from helpers import f64, logical, min_row_cosine, rel_norm, slots_of
from oracle import kvx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H_Q, H_KV = 16, 2
LENGTHS = [37, 700, 2300]
PCTS = [30, 40, 20]
CASES = [(ps, dh) for dh in (128, 64) for ps in (1, 3, 4, 8, 16, 24, 64)]


def layouts(page_size, d_h, batch, seed):
    """The same random keys and values as a paged cache and as a contiguous one."""
    pt, n_pages = synth.page_table_for(LENGTHS, page_size, seed)
    n_slots = n_pages * page_size
    shape = (1, n_slots, H_KV, d_h)
    kp = synth.cache_fill(shape, seed + 1, device=DEV)
    vp = synth.cache_fill(shape, seed + 2, device=DEV)
    ptn = pt.numpy()
    slots = np.concatenate([slots_of(b, T, batch.cu_tokens, ptn, page_size) for b, T in enumerate(LENGTHS)])
    idx = torch.as_tensor(slots, device=DEV).long()
    paged = kvx.Cache(kp, vp, 1, n_slots, pt.to(DEV), page_size)
    cont = kvx.Cache(kp[:, idx].contiguous(), vp[:, idx].contiguous(), 1, batch.n_tokens)
    return paged, cont, ptn


def selection(batch, seed):
    S_list = [synth.random_subset(T, k, seed + b) for b, (T, k) in enumerate(zip(LENGTHS, batch.n_sel))]
    return S_list, torch.from_numpy(np.concatenate(S_list).astype(np.int32)).to(DEV)


@pytest.mark.parametrize("page_size,d_h", CASES)
def test_attention_page_sizes(page_size, d_h):
    print(f"[pages] attention page_size={page_size} d_h={d_h}", flush=True)
    batch = kvx.Batch.for_budgets(LENGTHS, PCTS, DEV)
    paged, cont, ptn = layouts(page_size, d_h, batch, 40)
    S_list, sel = selection(batch, 50)
    rope = kvx.rope_table(1e6, d_h, max(LENGTHS), DEV)
    qkv = synth.latent(batch.total_sel, (H_Q + 2 * H_KV) * d_h, 60, device=DEV)
    k = batch.total_sel
    outs = {}
    for name, cache in (("paged", paged), ("contiguous", cont)):
        for split in (True, False):
            o = torch.empty((k, H_Q, d_h), dtype=torch.bfloat16, device=DEV)
            lse = torch.empty((k, H_Q), dtype=torch.float32, device=DEV)
            kvx.sparse_attention(0, qkv, H_Q, H_KV, d_h, rope, batch, sel, cache, o, lse, split=split)
            outs[(name, split)] = (o, lse)
    torch.cuda.synchronize()
    for split in (True, False):     # the layouts change only the load addresses
        assert torch.equal(outs[("paged", split)][0], outs[("contiguous", split)][0]), f"split={split}"
        assert torch.equal(outs[("paged", split)][1], outs[("contiguous", split)][1]), f"split={split}"
    q_all = f64(qkv[:, :H_Q * d_h]).reshape(k, H_Q, d_h)
    cs = batch.cu_sel
    for b, T in enumerate(LENGTHS):
        S = S_list[b]
        if len(S) == 0:
            continue
        K0 = logical(paged.k, 0, b, T, batch.cu_tokens, ptn, page_size)
        V0 = logical(paged.v, 0, b, T, batch.cu_tokens, ptn, page_size)
        q = O.rope(q_all[cs[b]:cs[b + 1]], S[:, None], 1e6)
        o_ref, lse_ref = O.sparse_causal_attention(q, K0, V0, S)
        for split in (True, False):
            o, lse = outs[("paged", split)]
            o = f64(o[cs[b]:cs[b + 1]])
            assert min_row_cosine(o, o_ref) >= 0.999, (b, split)
            assert rel_norm(o, o_ref) < 2e-2, (b, split)
            assert np.abs(f64(lse[cs[b]:cs[b + 1]]) - lse_ref).max() < 2e-2, (b, split)


@pytest.mark.parametrize("page_size,d_h", [(1, 128), (3, 64), (24, 128), (64, 64)])
def test_fused_projection_page_sizes(page_size, d_h):
    """The fused projection writes the same rotated k and v through the paged slot map as
    through the contiguous one, and leaves every other slot untouched."""
    print(f"[pages] projection page_size={page_size} d_h={d_h}", flush=True)
    D = 256
    batch = kvx.Batch.for_budgets(LENGTHS, PCTS, DEV)
    paged, cont, ptn = layouts(page_size, d_h, batch, 70)
    k_before = paged.k.clone()
    S_list, sel = selection(batch, 80)
    rope = kvx.rope_table(1e6, d_h, max(LENGTHS), DEV)
    x = synth.latent(batch.n_tokens, D, 90, device=DEV)
    w = (synth.latent((H_Q + 2 * H_KV) * d_h, D, 91, device=DEV).float() / D ** 0.5).to(torch.bfloat16)
    q1 = kvx.qkv_rope_scatter(0, x, w, H_Q, H_KV, d_h, rope, batch, sel, paged)
    q2 = kvx.qkv_rope_scatter(0, x, w, H_Q, H_KV, d_h, rope, batch, sel, cont)
    torch.cuda.synchronize()
    qc = H_Q * d_h
    assert torch.equal(q1[:, :qc], q2[:, :qc])
    for b, T in enumerate(LENGTHS):
        sl = torch.as_tensor(slots_of(b, T, batch.cu_tokens, ptn, page_size), device=DEV).long()
        rows = slice(batch.cu_tokens[b], batch.cu_tokens[b + 1])
        assert torch.equal(paged.k[0, sl], cont.k[0, rows]), b
        assert torch.equal(paged.v[0, sl], cont.v[0, rows]), b
        # positions outside the selection keep their translated values
        keep = np.setdiff1d(np.arange(T), S_list[b])
        kp = torch.as_tensor(keep, device=DEV).long()
        assert torch.equal(paged.k[0, sl[kp]], k_before[0, sl[kp]]), b
