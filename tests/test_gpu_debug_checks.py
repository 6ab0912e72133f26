"""KVX_DEBUG: the device index lists the kernels trust are checked before anything is launched.

With KVX_DEBUG=1 an unsorted or out-of-range selected list, an unsorted complement list, a
page mapped twice and device prefix arrays that differ from the host copies must each
return KVX_ERR_INVALID, and the outputs must stay untouched (nothing was enqueued).  Every
bad input here stays inside the buffers even if it were launched (an out-of-range position
is the first position of the next request, whose slots and rotary angles exist), so a
broken check shows up as a failed assertion, not as a fault.  Valid inputs under KVX_DEBUG
give the same results as without it.
"""
import ctypes

import numpy as np
import pytest
import torch

from cross_model_kv_amd import kvx, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H_Q, H_KV, D_H, D = 8, 2, 128, 256
LENGTHS = [300, 260]
PCT = 30
SENTINEL = 7.0


def say(msg):
    print(msg, flush=True)


def setup(paged=False):
    batch = kvx.Batch.for_budgets(LENGTHS, [PCT] * len(LENGTHS), DEV)
    S_list = [synth.random_subset(t, k, 70 + b) for b, (t, k) in enumerate(zip(LENGTHS, batch.n_sel))]
    if paged:
        pt, n_pages = synth.page_table_for(LENGTHS, 16, 71)
        n_slots = n_pages * 16
        pt = pt.to(DEV)
    else:
        pt, n_slots = None, batch.n_tokens
    shape = (1, n_slots, H_KV, D_H)
    cache = kvx.Cache(synth.cache_fill(shape, 72, device=DEV), synth.cache_fill(shape, 73, device=DEV), 1, n_slots,
                      pt, 16)
    qkv = synth.latent(batch.total_sel, (H_Q + 2 * H_KV) * D_H, 74, device=DEV)
    x = synth.latent(batch.n_tokens, D, 75, device=DEV)
    w = (synth.latent((H_Q + 2 * H_KV) * D_H, D, 76, dtype=torch.float32, device=DEV) / 16.0).to(torch.bfloat16)
    rope = kvx.rope_table(10000.0, D_H, max(LENGTHS) + 8, DEV)
    return batch, S_list, cache, qkv, x, w, rope


def to_dev(S_list):
    return torch.from_numpy(np.concatenate(S_list).astype(np.int32)).to(DEV)


def attention(batch, sel, cache, qkv, rope):
    out = torch.full((batch.total_sel, H_Q, D_H), SENTINEL, dtype=torch.bfloat16, device=DEV)
    kvx.sparse_attention(0, qkv, H_Q, H_KV, D_H, rope, batch, sel, cache, out)
    return out


def expect_invalid(fn, what):
    with pytest.raises(kvx.KvxError) as e:
        fn()
    assert e.value.code == -1, f"{what}: {e.value}"
    say(f"  {what}: {e.value}")


def test_debug_rejects_bad_selected_lists(monkeypatch):
    monkeypatch.setenv("KVX_DEBUG", "1")
    batch, S_list, cache, qkv, x, w, rope = setup()
    say("[debug] selected lists")
    k0 = len(S_list[0])
    bad = []
    unsorted = [S_list[0].copy(), S_list[1]]
    unsorted[0][[3, 4]] = unsorted[0][[4, 3]]
    bad.append(("unsorted sel", to_dev(unsorted)))
    repeated = [S_list[0].copy(), S_list[1]]
    repeated[0][5] = repeated[0][4]
    bad.append(("repeated sel", to_dev(repeated)))
    past_end = [S_list[0].copy(), S_list[1]]
    past_end[0][k0 - 1] = LENGTHS[0]          # one past request 0's end: request 1's first slot
    bad.append(("sel past the request's end", to_dev(past_end)))
    for what, sel in bad:
        out = torch.full((batch.total_sel, H_Q, D_H), SENTINEL, dtype=torch.bfloat16, device=DEV)
        k_before, v_before = cache.k.clone(), cache.v.clone()
        expect_invalid(lambda: kvx.sparse_attention(0, qkv, H_Q, H_KV, D_H, rope, batch, sel, cache, out),
                       what + " (sparse_attention)")
        expect_invalid(lambda: kvx.recompute_attn(0, x, w, H_Q, H_KV, D_H, rope, batch, sel, cache, out=out),
                       what + " (recompute_attn)")
        expect_invalid(lambda: kvx.qkv_rope_scatter(0, x, w, H_Q, H_KV, D_H, rope, batch, sel, cache),
                       what + " (qkv_rope_scatter)")
        expect_invalid(lambda: kvx.rope_scatter(0, qkv, H_Q, H_KV, D_H, rope, batch, sel, cache),
                       what + " (rope_scatter)")
        expect_invalid(lambda: kvx.gather_rows(x, batch, sel), what + " (gather_rows)")
        torch.cuda.synchronize()
        assert torch.all(out == SENTINEL), f"{what}: output written"
        assert torch.equal(cache.k, k_before) and torch.equal(cache.v, v_before), f"{what}: cache written"


def test_debug_rejects_bad_complement_list(monkeypatch):
    monkeypatch.setenv("KVX_DEBUG", "1")
    batch, S_list, cache, qkv, x, w, rope = setup()
    say("[debug] complement list")
    C_list = [np.setdiff1d(np.arange(t), S).astype(np.int32) for t, S in zip(LENGTHS, S_list)]
    C_list[1] = C_list[1][::-1].copy()
    rows = to_dev(C_list)
    z = synth.latent(batch.n_tokens, 128, 77, device=DEV)
    w_l = (synth.latent(2 * H_KV * D_H, 128, 78, dtype=torch.float32, device=DEV) / 11.3).to(torch.bfloat16)[None]
    k_before = cache.k.clone()
    expect_invalid(lambda: kvx.reconstruct(z, w_l, H_KV, D_H, batch, cache, rows=rows), "descending rows")
    torch.cuda.synchronize()
    assert torch.equal(cache.k, k_before), "cache written"


def test_debug_rejects_page_mapped_twice(monkeypatch):
    monkeypatch.setenv("KVX_DEBUG", "1")
    batch, S_list, cache, qkv, x, w, rope = setup(paged=True)
    say("[debug] page table")
    pt = cache.page_table.clone()
    pt[1, 2] = pt[0, 0]                       # request 1's third page is request 0's first
    twice = kvx.Cache(cache.k, cache.v, 1, cache.c.n_slots, pt, 16)
    sel = to_dev(S_list)
    out = torch.full((batch.total_sel, H_Q, D_H), SENTINEL, dtype=torch.bfloat16, device=DEV)
    expect_invalid(lambda: kvx.sparse_attention(0, qkv, H_Q, H_KV, D_H, rope, batch, sel, twice, out),
                   "page mapped twice")
    torch.cuda.synchronize()
    assert torch.all(out == SENTINEL)


def test_debug_rejects_prefix_mismatch(monkeypatch):
    monkeypatch.setenv("KVX_DEBUG", "1")
    batch, S_list, cache, qkv, x, w, rope = setup()
    say("[debug] prefix arrays")
    sel = to_dev(S_list)
    bad = kvx.Batch(LENGTHS, batch.n_sel, DEV)
    bad.d_sel[1] -= 1                         # device copy differs from the host copy
    out = torch.full((batch.total_sel, H_Q, D_H), SENTINEL, dtype=torch.bfloat16, device=DEV)
    expect_invalid(lambda: kvx.sparse_attention(0, qkv, H_Q, H_KV, D_H, rope, bad, sel, cache, out),
                   "device cu_sel differs")
    torch.cuda.synchronize()
    assert torch.all(out == SENTINEL)


@pytest.mark.parametrize("paged", [False, True])
def test_debug_accepts_valid_inputs(monkeypatch, paged):
    batch, S_list, cache, qkv, x, w, rope = setup(paged)
    sel = to_dev(S_list)
    say(f"[debug] valid inputs ({'paged' if paged else 'contiguous'})")
    ref = attention(batch, sel, cache, qkv, rope)
    monkeypatch.setenv("KVX_DEBUG", "1")
    got = attention(batch, sel, cache, qkv, rope)
    monkeypatch.setenv("KVX_DEBUG", "0")
    torch.cuda.synchronize()
    assert torch.equal(ref, got)
    assert not torch.any(got == SENTINEL)
