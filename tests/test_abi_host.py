"""Host-only checks of the C ABI (no GPU needed): the library loads, exports every symbol
include/kvx.h declares, computes the budget, and rejects bad arguments on the host before
any GPU work (every call below fails validation, so nothing reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

from cross_model_kv_amd import kvx
from oracle import kvx_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -4
A16 = ctypes.c_void_p(0x10000)           # aligned fake device address (never dereferenced)
A16B = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)           # misaligned fake address


def declared_symbols():
    with open(os.path.join(ROOT, "include", "kvx.h")) as f:
        return sorted(set(re.findall(r"^KVX_API[^(]*?\b(kvx_\w+)\s*\(", f.read(), flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 13
    lib = kvx.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert kvx.version().startswith("kvx")


def test_budget_matches_oracle():
    for T in range(0, 2000, 7):
        for pct in (0, 1, 20, 30, 33, 40, 99, 100):
            assert kvx.budget(T, pct) == O.budget(T, pct)
    assert kvx.lib().kvx_budget(10, 101) == -1
    assert kvx.lib().kvx_budget(-1, 30) == -1
    assert b"pct" in kvx.lib().kvx_last_error()


class FakeBatch:
    def __init__(self, lengths, ks, dev_ptrs=True):
        n = len(lengths)
        self.cu_t = [0]
        self.cu_s = [0]
        for t, k in zip(lengths, ks):
            self.cu_t.append(self.cu_t[-1] + t)
            self.cu_s.append(self.cu_s[-1] + k)
        self.h_t = (ctypes.c_int32 * (n + 1))(*self.cu_t)
        self.h_s = (ctypes.c_int32 * (n + 1))(*self.cu_s)
        self.c = kvx._Batch(n, self.h_t, self.h_s, 0x30000 if dev_ptrs else None, 0x40000 if dev_ptrs else None)


def cache(layout=0, n_layers=2, n_slots=1000, page_size=16, max_pages=8, k=A16, v=A16B, page_table=0x50000):
    return kvx._Cache(layout, k.value if k is not None else None, v.value if v is not None else None, n_layers,
                      n_slots, page_size, max_pages, page_table)


def status(code, expect, needle=None):
    assert code == expect, (code, kvx.lib().kvx_last_error())
    if needle:
        assert needle.encode() in kvx.lib().kvx_last_error(), kvx.lib().kvx_last_error()


def test_map_latent_validation():
    L = kvx.lib()
    status(L.kvx_map_latent(None, 7, A16, A16, A16, 10, 64, 8, None, 0), UNSUPPORTED, "dtype")
    status(L.kvx_map_latent(None, 1, None, A16, A16, 10, 64, 8, None, 0), INVALID, "x_src")
    status(L.kvx_map_latent(None, 1, MIS, A16, A16, 10, 64, 8, None, 0), INVALID, "aligned")
    status(L.kvx_map_latent(None, 1, A16, A16, A16, -1, 64, 8, None, 0), INVALID, "n")
    status(L.kvx_map_latent(None, 1, A16, A16, A16, 10, 0, 8, None, 0), INVALID, "positive")
    status(L.kvx_map_latent(None, 1, A16, A16, A16, 10, 100, 8, None, 0), INVALID, "d_src % 64")
    status(L.kvx_map_latent(None, 1, A16, A16, A16, 10, 64, 12, None, 0), INVALID, "r % 8")
    # too few output tiles to fill the GPU: the product is split along d_src and needs a workspace
    need = ctypes.c_size_t()
    assert L.kvx_map_latent_workspace(1, 4096, 57344, 1024, ctypes.byref(need)) == 0 and need.value > 0
    status(L.kvx_map_latent(None, 1, A16, A16, A16, 4096, 57344, 1024, None, 0), WORKSPACE, "workspace")
    status(L.kvx_map_latent(None, 1, A16, A16, A16, 4096, 57344, 1024, A16, need.value - 1), WORKSPACE, "workspace")
    assert L.kvx_map_latent_workspace(0, 4096, 57344, 1024, ctypes.byref(need)) == 0 and need.value == 0


def test_score_prepare_validation():
    L = kvx.lib()
    b = ctypes.c_size_t()
    status(L.kvx_score_prepare_workspace(8, 16, 17, ctypes.byref(b)), INVALID)
    assert L.kvx_score_prepare_workspace(8, 16, 4, ctypes.byref(b)) == 0 and b.value > 0
    status(L.kvx_score_prepare(None, 1, A16, A16, 2, 8, 16, 4, A16, None, 0), WORKSPACE)
    status(L.kvx_score_prepare(None, 1, A16, A16, 2, 8, 16, 4, A16, A16, 1), WORKSPACE)
    status(L.kvx_score_prepare(None, 1, A16, None, 2, 8, 16, 4, A16, A16, 1 << 20), INVALID, "u")
    status(L.kvx_score_prepare(None, 1, A16, A16, 0, 8, 16, 4, A16, A16, 1 << 20), INVALID)
    status(L.kvx_score_prepare(None, 1, A16, A16, 2, 8, 16, 20, A16, A16, 1 << 20), INVALID, "calibration")


def test_fit_validation():
    """The mapper and calibration fits check ranks, alignment, lambda, iteration count and
    workspace before any device work."""
    L = kvx.lib()
    b = ctypes.c_size_t()
    # (dtype, n, d_src, L_t, d_t, r)
    status(L.kvx_fit_mapper_workspace(1, 64, 128, 2, 64, 65, ctypes.byref(b)), INVALID, "must not exceed n")
    status(L.kvx_fit_mapper_workspace(1, 256, 32, 2, 64, 40, ctypes.byref(b)), INVALID, "d_src")
    status(L.kvx_fit_mapper_workspace(1, 60, 128, 2, 64, 16, ctypes.byref(b)), INVALID, "n % 8")
    status(L.kvx_fit_mapper_workspace(1, 64, 100, 2, 64, 16, ctypes.byref(b)), INVALID, "d_src % 64")
    status(L.kvx_fit_mapper_workspace(7, 64, 128, 2, 64, 16, ctypes.byref(b)), UNSUPPORTED, "dtype")
    status(L.kvx_fit_mapper_workspace(1, 64, 128, 0, 64, 16, ctypes.byref(b)), INVALID, "positive")
    assert L.kvx_fit_mapper_workspace(0, 60, 100, 3, 10, 16, ctypes.byref(b)) == 0 and b.value > 60 * 60 * 8
    need = ctypes.c_size_t()
    assert L.kvx_fit_mapper_workspace(1, 64, 128, 2, 64, 16, ctypes.byref(need)) == 0
    fit = lambda x=A16, lam=1.0, iters=10, ws=A16, wsb=need.value: L.kvx_fit_mapper(
        None, 1, x, A16, 64, 128, 2, 64, 16, ctypes.c_double(lam), iters, A16, A16B, ws, wsb)
    status(fit(x=None), INVALID, "x")
    status(fit(x=MIS), INVALID, "aligned")
    status(fit(lam=0.0), INVALID, "lambda")
    status(fit(lam=float("inf")), INVALID, "lambda")
    status(fit(lam=float("nan")), INVALID, "lambda")
    status(fit(iters=0), INVALID, "iters")
    status(fit(ws=None), WORKSPACE)
    status(fit(wsb=need.value - 1), WORKSPACE)
    # (n, L_t, d_t, r, c)
    status(L.kvx_fit_calibration_workspace(64, 2, 32, 16, 17, ctypes.byref(b)), INVALID, "must not exceed")
    status(L.kvx_fit_calibration_workspace(8, 2, 32, 16, 9, ctypes.byref(b)), INVALID, "must not exceed")
    assert L.kvx_fit_calibration_workspace(64, 2, 32, 16, 8, ctypes.byref(need)) == 0 and need.value > 0
    cal = lambda z=A16, u=A16B, iters=10, ws=A16, wsb=need.value: L.kvx_fit_calibration(
        None, 1, z, A16, 64, 2, 32, 16, 8, iters, u, ws, wsb)
    status(cal(z=None), INVALID, "z")
    status(cal(u=MIS), INVALID, "aligned")
    status(cal(iters=20000), INVALID, "iters")
    status(cal(wsb=need.value - 1), WORKSPACE)


def test_batch_validation():
    L = kvx.lib()
    bad = FakeBatch([10, 5], [3, 6])                      # k > T
    status(L.kvx_select_topk(None, A16, ctypes.byref(bad.c), A16, A16), INVALID, "selects")
    nodev = FakeBatch([10], [3], dev_ptrs=False)
    status(L.kvx_select_topk(None, A16, ctypes.byref(nodev.c), A16, A16), INVALID, "device")
    empty = kvx._Batch(0, None, None, None, None)
    status(L.kvx_select_topk(None, A16, ctypes.byref(empty), A16, A16), INVALID, "n_req")
    ok = FakeBatch([10], [3])
    status(L.kvx_select_topk(None, None, ctypes.byref(ok.c), A16, A16), INVALID, "scores")
    status(L.kvx_select_topk(None, A16, ctypes.byref(ok.c), None, A16), INVALID, "sel")
    status(L.kvx_select_topk(None, A16, None, A16, A16), INVALID, "batch")


def test_score_select_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    pct = (ctypes.c_int32 * 2)(30, 30)
    need = ctypes.c_size_t()
    assert L.kvx_score_select_workspace(1, 128, 150, ctypes.byref(need)) == 0
    args = lambda p, r=128, ws=A16, wsb=need.value: (None, 1, A16, A16, r, ctypes.byref(bt.c), p, A16, A16,
                                                     A16, ws, wsb)
    status(L.kvx_score_select(*args(pct, r=96)), INVALID, "r % 64")
    status(L.kvx_score_select(*args(None)), INVALID, "budget_pct")
    status(L.kvx_score_select(*args((ctypes.c_int32 * 2)(30, 40))), INVALID, "budget")
    status(L.kvx_score_select(*args((ctypes.c_int32 * 2)(30, 130))), INVALID, "outside")
    status(L.kvx_score_select(*args(pct, ws=None)), WORKSPACE)
    status(L.kvx_score_select(*args(pct, wsb=need.value - 1)), WORKSPACE)


def test_score_select_noalloc_validation():
    """The no-allocation variant validates like kvx_score_select and refuses, before touching
    the device, a batch whose scratch exceeds the fixed array it uses."""
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    pct = (ctypes.c_int32 * 2)(30, 30)
    args = lambda p, r=128, b=bt: (None, 1, A16, A16, r, ctypes.byref(b.c), p, A16, A16, A16)
    status(L.kvx_score_select_noalloc(*args(pct, r=96)), INVALID, "r % 64")
    status(L.kvx_score_select_noalloc(*args(None)), INVALID, "budget_pct")
    status(L.kvx_score_select_noalloc(*args((ctypes.c_int32 * 2)(30, 40))), INVALID, "budget")
    # bf16 scratch is 4 * N * ceil(r / 256) bytes: r = 1024 and N = 2^20 + 64 is over 16 MiB
    big_T = (1 << 20) + 64
    big = FakeBatch([big_T], [kvx.budget(big_T, 30)])
    status(L.kvx_score_select_noalloc(*args((ctypes.c_int32 * 1)(30), r=1024, b=big)), WORKSPACE, "scratch")


def test_score_select_normalized_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    pct = (ctypes.c_int32 * 2)(30, 30)
    need = ctypes.c_size_t()
    one = ctypes.c_size_t()
    assert L.kvx_score_select_normalized_workspace(1, 128, 150, ctypes.byref(need)) == 0
    assert L.kvx_score_select_workspace(1, 128, 150, ctypes.byref(one)) == 0 and need.value == 2 * one.value
    args = lambda opt=A16B, ws=A16, wsb=need.value: (None, 1, A16, A16, opt, 128, ctypes.byref(bt.c), pct, A16,
                                                      A16, A16, ws, wsb)
    status(L.kvx_score_select_normalized(*args(opt=None)), INVALID, "op_total")
    status(L.kvx_score_select_normalized(*args(ws=None)), WORKSPACE)
    status(L.kvx_score_select_normalized(*args(wsb=need.value - 1)), WORKSPACE)


def test_score_cache_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    pct = (ctypes.c_int32 * 2)(30, 30)
    c = cache(n_layers=3)
    # prepare: shapes of the packed basis
    status(L.kvx_score_cache_prepare(None, 1, A16, 2, 192, 16, A16B), INVALID, "d_t % 128")
    status(L.kvx_score_cache_prepare(None, 1, A16, 2, 256, 12, A16B), INVALID, "c % 8")
    status(L.kvx_score_cache_prepare(None, 1, A16, 2, 256, 300, A16B), INVALID, "c <= d_t")
    status(L.kvx_score_cache_prepare(None, 1, None, 2, 256, 16, A16B), INVALID, "u")
    status(L.kvx_score_cache_prepare(None, 3, A16, 2, 256, 16, A16B), UNSUPPORTED, "dtype")
    # workspace: bf16 one partial per 256 directions and layer, fp32 one per layer
    b16, b32 = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.kvx_score_cache_workspace(1, 2, 300, 150, ctypes.byref(b16)) == 0 and b16.value == -(-2 * 2 * 150 * 4 // 256) * 256
    assert L.kvx_score_cache_workspace(0, 2, 300, 150, ctypes.byref(b32)) == 0 and b32.value == -(-2 * 150 * 4 // 256) * 256
    need = ctypes.c_size_t()
    assert L.kvx_score_cache_workspace(1, 2, 64, 150, ctypes.byref(need)) == 0

    def call(dt=1, l0=0, n=2, H_kv=2, d_h=64, op=A16B, cc=64, cch=c, energy=A16, ws=A16, wsb=None):
        return L.kvx_score_cache(None, dt, ctypes.byref(cch), l0, n, H_kv, d_h, op, cc, ctypes.byref(bt.c), energy,
                                 ws, need.value if wsb is None else wsb)
    status(call(l0=2), INVALID, "outside the cache")
    status(call(n=0), INVALID, "n_layers")
    status(call(H_kv=1, d_h=40), INVALID, "% 64")
    status(call(cc=12), INVALID, "c % 8")
    status(call(cc=257), INVALID, "c must be in")
    status(call(op=None), INVALID, "op")
    status(call(energy=None), INVALID, "energy")
    status(call(ws=None), WORKSPACE)
    status(call(wsb=need.value - 1), WORKSPACE)
    status(call(cch=cache(n_layers=3, n_slots=100)), INVALID, "n_slots")
    status(call(dt=0, H_kv=64, d_h=80), INVALID, "d_t <= 8192")
    # the summed score and its selection: budgets as in kvx_score_select
    bad = (ctypes.c_int32 * 2)(30, 40)
    sargs = lambda p=pct, wsb=need.value: (None, 1, ctypes.byref(c), 0, 2, 2, 64, A16B, 64, ctypes.byref(bt.c), p,
                                           A16, A16, A16, A16, wsb)
    status(L.kvx_score_cache_select(*sargs(p=bad)), INVALID, "budget")
    status(L.kvx_score_cache_select(*sargs(p=None)), INVALID, "budget_pct")
    status(L.kvx_score_cache_select(*sargs(wsb=need.value - 1)), WORKSPACE)
    # per-layer selection
    status(L.kvx_select_topk_layers(None, A16, 0, ctypes.byref(bt.c), A16, A16), INVALID, "n_layers")
    status(L.kvx_select_topk_layers(None, None, 2, ctypes.byref(bt.c), A16, A16), INVALID, "scores")
    status(L.kvx_select_topk_layers(None, A16, 2, ctypes.byref(bt.c), None, A16), INVALID, "sel")


def test_select_pages_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    pg = FakeBatch([7, 4], [3, 2])              # ceil(100 / 16) = 7, ceil(50 / 16) = 4
    bad = FakeBatch([7, 3], [3, 2])
    one = FakeBatch([7], [3])
    args = lambda ps=16, pages=pg, cu=A16: (None, A16, ctypes.byref(bt.c), ps, ctypes.byref(pages.c), A16, A16,
                                            A16B, cu, A16, A16B)
    status(L.kvx_select_pages(*args(ps=0)), INVALID, "page_size")
    status(L.kvx_select_pages(*args(pages=bad)), INVALID, "pages")
    status(L.kvx_select_pages(*args(pages=one)), INVALID, "requests")
    status(L.kvx_select_pages(*args(ps=8)), INVALID, "pages of 8")
    status(L.kvx_select_pages(*args(cu=None)), INVALID, "cu_sel")


def test_reconstruct_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    c = cache()
    status(L.kvx_reconstruct(None, 1, A16, A16, 2, 96, 2, 64, ctypes.byref(bt.c), None, ctypes.byref(c)),
           INVALID, "r % 64")
    small = cache(n_slots=100)
    status(L.kvx_reconstruct(None, 1, A16, A16, 2, 128, 2, 64, ctypes.byref(bt.c), None, ctypes.byref(small)),
           INVALID, "n_slots")
    few = cache(n_layers=1)
    status(L.kvx_reconstruct(None, 1, A16, A16, 2, 128, 2, 64, ctypes.byref(bt.c), None, ctypes.byref(few)),
           INVALID, "n_layers")
    paged = cache(layout=1, n_slots=16 * 20, max_pages=3)   # 100 positions need 7 pages
    status(L.kvx_reconstruct(None, 1, A16, A16, 2, 128, 2, 64, ctypes.byref(bt.c), None, ctypes.byref(paged)),
           INVALID, "max_pages")
    nopt = cache(layout=1, n_slots=16 * 20, page_table=None)
    status(L.kvx_reconstruct(None, 1, A16, A16, 2, 128, 2, 64, ctypes.byref(bt.c), None, ctypes.byref(nopt)),
           INVALID, "page_table")
    badlayout = cache(layout=5)
    status(L.kvx_reconstruct(None, 1, A16, A16, 2, 128, 2, 64, ctypes.byref(bt.c), None,
                             ctypes.byref(badlayout)), INVALID, "layout")
    status(L.kvx_reconstruct(None, 1, A16, A16, 2, 128, 2, 64, ctypes.byref(bt.c), MIS, ctypes.byref(c)),
           INVALID, "rows")


def test_reconstruct_rope_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    c = cache()
    args = lambda dt=1, d_h=64, rope=A16B, max_pos=100: (None, dt, A16, A16, 2, 128, 2, d_h, rope, max_pos,
                                                          ctypes.byref(bt.c), None, ctypes.byref(c))
    status(L.kvx_reconstruct_rope(*args(d_h=96)), UNSUPPORTED, "d_h")
    status(L.kvx_reconstruct_rope(*args(dt=0, d_h=96, rope=None)), INVALID, "rope")   # fp32: any d_h % 8 == 0
    status(L.kvx_reconstruct_rope(*args(rope=None)), INVALID, "rope")
    status(L.kvx_reconstruct_rope(*args(max_pos=99)), INVALID, "positions")


def test_rope_table_validation():
    L = kvx.lib()
    status(L.kvx_rope_table(None, 10000.0, 7, 10, A16), INVALID, "even")
    status(L.kvx_rope_table(None, 10000.0, 64, 0, A16), INVALID, "max_pos")
    status(L.kvx_rope_table(None, -1.0, 64, 10, A16), INVALID, "base")
    status(L.kvx_rope_table(None, 10000.0, 64, 10, None), INVALID, "table")


def test_recompute_attn_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    c = cache()
    need = ctypes.c_size_t()
    assert L.kvx_recompute_attn_workspace(1, ctypes.byref(bt.c), 256, 8, 2, 64, ctypes.byref(need)) == 0
    assert need.value >= 45 * 12 * 64 * 2

    def call(dtype=1, layer=0, D=256, H_q=8, H_kv=2, d_h=64, max_pos=100, cc=c, ws=A16, wsb=None):
        return L.kvx_recompute_attn(None, dtype, layer, A16, A16, D, H_q, H_kv, d_h, A16, max_pos,
                                    ctypes.byref(bt.c), A16, ctypes.byref(cc), A16, None, ws,
                                    need.value if wsb is None else wsb)
    status(call(d_h=96), UNSUPPORTED, "d_h")
    status(call(H_q=9), INVALID, "multiple")
    status(call(H_q=34, H_kv=2), UNSUPPORTED, "> 16")
    status(call(H_q=18, H_kv=2, wsb=0), WORKSPACE)      # g = 9 is supported (padded 8-wave blocks)
    status(call(D=100), INVALID, "D % 64")
    status(call(max_pos=99), INVALID, "rope")
    status(call(layer=2), INVALID, "layer")
    status(call(ws=None), WORKSPACE)
    status(call(wsb=need.value - 1), WORKSPACE)
    status(call(dtype=3), UNSUPPORTED, "dtype")


def test_qkv_rope_scatter_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    c = cache()
    need = ctypes.c_size_t()
    assert L.kvx_qkv_project_workspace(1, ctypes.byref(bt.c), 4096, 8, 2, 64, ctypes.byref(need)) == 0
    assert need.value > 0, "a few rows over a wide D split along D"

    def call(dtype=1, layer=0, D=4096, H_q=8, H_kv=2, d_h=64, max_pos=100, cc=c, ws=A16, wsb=None, qkv=A16):
        return L.kvx_qkv_rope_scatter(None, dtype, layer, A16, A16, D, H_q, H_kv, d_h, A16, max_pos,
                                      ctypes.byref(bt.c), A16, ctypes.byref(cc), qkv, ws,
                                      need.value if wsb is None else wsb)
    status(call(d_h=96), UNSUPPORTED, "d_h")
    status(call(H_q=9), INVALID, "multiple")
    status(call(D=100), INVALID, "D % 64")
    status(call(max_pos=99), INVALID, "rope")
    status(call(layer=2), INVALID, "layer")
    status(call(qkv=None), INVALID, "qkv")
    status(call(ws=None), WORKSPACE)
    status(call(wsb=need.value - 1), WORKSPACE)
    status(call(dtype=3), UNSUPPORTED, "dtype")


def test_qknorm_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    c = cache(n_layers=1)
    args = lambda dt=1, gq=A16, eps=1e-6, d_h=128: (None, dt, 0, A16, A16, 256, 8, 2, d_h, gq, A16B,
                                                    ctypes.c_float(eps), A16, 100, ctypes.byref(bt.c), A16,
                                                    ctypes.byref(c), A16)
    status(L.kvx_qkv_rope_scatter_qknorm(*args(gq=None)), INVALID, "gain")
    status(L.kvx_qkv_rope_scatter_qknorm(*args(dt=0, gq=None)), INVALID, "gain")
    status(L.kvx_qkv_rope_scatter_qknorm(*args(eps=-1.0)), INVALID, "eps")
    status(L.kvx_qkv_rope_scatter_qknorm(*args(d_h=96)), UNSUPPORTED, "d_h")


def test_chaining_validation():
    L = kvx.lib()
    bt = FakeBatch([100, 50], [30, 15])
    c = cache()
    # gather / rmsnorm
    status(L.kvx_gather_rows(None, 0, A16, 64, ctypes.byref(bt.c), A16, A16B), UNSUPPORTED, "BF16 only")
    status(L.kvx_gather_rows(None, 1, A16, 60, ctypes.byref(bt.c), A16, A16B), INVALID, "multiple of 8")
    status(L.kvx_gather_rows(None, 1, A16, 64, ctypes.byref(bt.c), None, A16B), INVALID, "sel")
    status(L.kvx_rmsnorm(None, 1, A16, A16B, 1e-6, 4, 20000, A16), INVALID, "D")
    status(L.kvx_rmsnorm(None, 1, A16, A16B, -1.0, 4, 64, A16), INVALID, "eps")
    status(L.kvx_rmsnorm(None, 1, A16, MIS, 1e-6, 4, 64, A16), INVALID, "gamma")
    # linear + residual, gated MLP
    need = ctypes.c_size_t()
    assert L.kvx_linear_residual_workspace(1, 64, 4096, 4096, ctypes.byref(need)) == 0
    assert need.value > 0, "a few rows over a wide K split along K"
    status(L.kvx_linear_residual(None, 1, A16, A16, A16, A16, 64, 4096, 100, A16, need.value), INVALID, "K")
    status(L.kvx_linear_residual(None, 1, A16, A16, A16, A16, 64, 4096, 4096, None, 0), WORKSPACE)
    status(L.kvx_linear_residual(None, 1, A16, A16, A16, A16, 64, 4096, 4096, A16, need.value - 1), WORKSPACE)
    status(L.kvx_swiglu(None, 1, A16, A16, A16, A16, 64, 100, 256, None, 0), INVALID, "D")
    status(L.kvx_swiglu(None, 1, A16, A16, A16, A16, 64, 256, 12, None, 0), INVALID, "F")
    status(L.kvx_swiglu(None, 1, A16, None, A16, A16, 64, 256, 256, None, 0), INVALID, "w_gate")
    # the whole layer
    assert L.kvx_target_layer_workspace(1, ctypes.byref(bt.c), 256, 512, 8, 2, 64, ctypes.byref(need)) == 0
    assert need.value >= 45 * (256 + 12 * 64 + 8 * 64 + 512) * 2
    W = kvx._LayerWeights(*([A16.value] * 7))
    Wbad = kvx._LayerWeights(*([A16.value] * 5 + [None, A16.value]))

    def call(dtype=1, layer=0, D=256, F=512, H_q=8, H_kv=2, d_h=64, eps=1e-6, w=W, ws=A16, wsb=None, max_pos=100):
        return L.kvx_target_layer(None, dtype, layer, A16, ctypes.byref(w), D, F, H_q, H_kv, d_h, eps, A16, max_pos,
                                  ctypes.byref(bt.c), A16, ctypes.byref(c), None, None, ws,
                                  need.value if wsb is None else wsb)
    status(call(dtype=0), UNSUPPORTED, "BF16 only")
    status(call(d_h=96), UNSUPPORTED, "d_h")
    status(call(D=100), INVALID, "D")
    status(call(F=100), INVALID, "F")
    status(call(eps=-1.0), INVALID, "eps")
    status(call(w=Wbad), INVALID, "w_up")
    status(call(max_pos=99), INVALID, "rope")
    status(call(layer=2), INVALID, "layer")
    status(call(ws=None), WORKSPACE)
    status(call(wsb=need.value - 16), WORKSPACE)
