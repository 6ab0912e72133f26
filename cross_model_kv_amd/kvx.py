"""Thin Python binding of libkvx (ctypes).

Argument marshalling only: every step of the handoff runs in the HIP kernels behind the C
ABI in include/kvx.h.  PyTorch supplies device memory and the current stream.  There is
no fallback: if libkvx.so is missing or was built for another GPU, calls fail loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvx.so")

F32, BF16 = 0, 1
CONTIGUOUS, PAGED = 0, 1
STATUS = {0: "KVX_OK", -1: "KVX_ERR_INVALID", -2: "KVX_ERR_UNSUPPORTED", -3: "KVX_ERR_HIP",
          -4: "KVX_ERR_WORKSPACE"}


class KvxError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(code, code)}: {msg}")
        self.code = code


class _Batch(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32),
                ("cu_tokens_h", ctypes.POINTER(ctypes.c_int32)),
                ("cu_sel_h", ctypes.POINTER(ctypes.c_int32)),
                ("cu_tokens_d", ctypes.c_void_p),
                ("cu_sel_d", ctypes.c_void_p)]


class _Cache(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32),
                ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p),
                ("n_layers", ctypes.c_int32),
                ("n_slots", ctypes.c_int64),
                ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32),
                ("page_table", ctypes.c_void_p)]


class _LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gamma_in", "w_qkv", "w_o", "gamma_post", "w_gate", "w_up", "w_down")]


_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "kvx_last_error": ([], ctypes.c_char_p),
    "kvx_version": ([], ctypes.c_char_p),
    "kvx_budget": ([_I32, _I32], _I32),
    "kvx_map_latent_workspace": ([_I32, _I64, _I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "kvx_map_latent": ([_P, _I32, _P, _P, _P, _I64, _I32, _I32, _P, _SZ], _I32),
    "kvx_score_prepare_workspace": ([_I32, _I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "kvx_score_prepare": ([_P, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ], _I32),
    "kvx_select_topk": ([_P, _P, ctypes.POINTER(_Batch), _P, _P], _I32),
    "kvx_score_select_workspace": ([_I32, _I32, _I64, ctypes.POINTER(_SZ)], _I32),
    "kvx_score_select": ([_P, _I32, _P, _P, _I32, ctypes.POINTER(_Batch), ctypes.POINTER(_I32), _P, _P,
                          _P, _P, _SZ], _I32),
    "kvx_score_select_noalloc": ([_P, _I32, _P, _P, _I32, ctypes.POINTER(_Batch), ctypes.POINTER(_I32), _P, _P,
                                  _P], _I32),
    "kvx_score_select_normalized_workspace": ([_I32, _I32, ctypes.c_int64, ctypes.POINTER(_SZ)], _I32),
    "kvx_score_select_normalized": ([_P, _I32, _P, _P, _P, _I32, ctypes.POINTER(_Batch), ctypes.POINTER(_I32), _P,
                                     _P, _P, _P, _SZ], _I32),
    "kvx_score_cache_prepare": ([_P, _I32, _P, _I32, _I32, _I32, _P], _I32),
    "kvx_score_cache_workspace": ([_I32, _I32, _I32, _I64, ctypes.POINTER(_SZ)], _I32),
    "kvx_score_cache": ([_P, _I32, ctypes.POINTER(_Cache), _I32, _I32, _I32, _I32, _P, _I32, ctypes.POINTER(_Batch),
                         _P, _P, _SZ], _I32),
    "kvx_score_cache_select": ([_P, _I32, ctypes.POINTER(_Cache), _I32, _I32, _I32, _I32, _P, _I32,
                                ctypes.POINTER(_Batch), ctypes.POINTER(_I32), _P, _P, _P, _P, _SZ], _I32),
    "kvx_select_topk_layers": ([_P, _P, _I32, ctypes.POINTER(_Batch), _P, _P], _I32),
    "kvx_select_pages": ([_P, _P, ctypes.POINTER(_Batch), _I32, ctypes.POINTER(_Batch), _P, _P, _P, _P, _P, _P],
                         _I32),
    "kvx_fit_mapper_workspace": ([_I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "kvx_fit_mapper": ([_P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, ctypes.c_double, _I32, _P, _P, _P, _SZ],
                       _I32),
    "kvx_fit_calibration_workspace": ([_I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "kvx_fit_calibration": ([_P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ], _I32),
    "kvx_qkv_rope_scatter_qknorm": ([_P, _I32, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _P, ctypes.c_float, _P,
                                     _I32, ctypes.POINTER(_Batch), _P, ctypes.POINTER(_Cache), _P], _I32),
    "kvx_reconstruct_rope": ([_P, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, ctypes.POINTER(_Batch), _P,
                              ctypes.POINTER(_Cache)], _I32),
    "kvx_reconstruct": ([_P, _I32, _P, _P, _I32, _I32, _I32, _I32, ctypes.POINTER(_Batch), _P,
                         ctypes.POINTER(_Cache)], _I32),
    "kvx_rope_table": ([_P, ctypes.c_double, _I32, _I32, _P], _I32),
    "kvx_recompute_attn_workspace": ([_I32, ctypes.POINTER(_Batch), _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)],
                                     _I32),
    "kvx_qkv_project_workspace": ([_I32, ctypes.POINTER(_Batch), _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)],
                                  _I32),
    "kvx_recompute_attn": ([_P, _I32, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I32,
                            ctypes.POINTER(_Batch), _P, ctypes.POINTER(_Cache), _P, _P, _P, _SZ], _I32),
    "kvx_qkv_project": ([_P, _I32, _P, _P, _I32, _I32, _I32, _I32, ctypes.POINTER(_Batch), _P, _P, _P, _SZ],
                        _I32),
    "kvx_recompute_attn_layers_workspace": ([_I32, ctypes.POINTER(_Batch), _I32, _I32, _I32, _I32, _I32,
                                             ctypes.POINTER(_SZ)], _I32),
    "kvx_recompute_attn_layers": ([_P, _I32, _I32, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I32,
                                   ctypes.POINTER(_Batch), _P, ctypes.POINTER(_Cache), _P, _P, _P, _SZ], _I32),
    "kvx_qkv_rope_scatter_layers": ([_P, _I32, _I32, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I32,
                                     ctypes.POINTER(_Batch), _P, ctypes.POINTER(_Cache), _P], _I32),
    "kvx_sparse_attention_layers": ([_P, _I32, _I32, _I32, _P, _I32, _I32, _I32, _P, _I32, ctypes.POINTER(_Batch),
                                     _P, ctypes.POINTER(_Cache), _P, _P], _I32),
    "kvx_rope_scatter": ([_P, _I32, _I32, _P, _I32, _I32, _I32, _P, _I32, ctypes.POINTER(_Batch), _P,
                          ctypes.POINTER(_Cache)], _I32),
    "kvx_qkv_rope_scatter": ([_P, _I32, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, ctypes.POINTER(_Batch),
                              _P, ctypes.POINTER(_Cache), _P, _P, _SZ], _I32),
    "kvx_sparse_attention_workspace": ([_I32, ctypes.POINTER(_Batch), _I32, _I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "kvx_sparse_attention": ([_P, _I32, _I32, _P, _I32, _I32, _I32, _P, _I32, ctypes.POINTER(_Batch), _P,
                              ctypes.POINTER(_Cache), _P, _P, _P, _SZ], _I32),
    "kvx_gather_rows": ([_P, _I32, _P, _I32, ctypes.POINTER(_Batch), _P, _P], _I32),
    "kvx_rmsnorm": ([_P, _I32, _P, _P, ctypes.c_float, _I64, _I32, _P], _I32),
    "kvx_linear_residual_workspace": ([_I32, _I64, _I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "kvx_linear_residual": ([_P, _I32, _P, _P, _P, _P, _I64, _I32, _I32, _P, _SZ], _I32),
    "kvx_swiglu_workspace": ([_I32, _I64, _I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "kvx_swiglu": ([_P, _I32, _P, _P, _P, _P, _I64, _I32, _I32, _P, _SZ], _I32),
    "kvx_linear_workspace": ([_I32, _I64, _I32, _I32, ctypes.POINTER(_SZ)], _I32),
    "kvx_linear": ([_P, _I32, _P, _P, _P, _I64, _I32, _I32, _P, _SZ], _I32),
    "kvx_argmax": ([_P, _I32, _P, _I64, _I32, _P], _I32),
    "kvx_target_layer_workspace": ([_I32, ctypes.POINTER(_Batch), _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(_SZ)],
                                   _I32),
    "kvx_target_layer": ([_P, _I32, _I32, _P, ctypes.POINTER(_LayerWeights), _I32, _I32, _I32, _I32, _I32,
                          ctypes.c_float, _P, _I32, ctypes.POINTER(_Batch), _P, ctypes.POINTER(_Cache), _P, _P, _P,
                          _SZ], _I32),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvx.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def _check(fn: str, code: int):
    if code != 0:
        raise KvxError(fn, code, lib().kvx_last_error().decode())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def version() -> str:
    return lib().kvx_version().decode()


def budget(T: int, pct: int) -> int:
    k = lib().kvx_budget(T, pct)
    if k < 0:
        raise KvxError("kvx_budget", -1, lib().kvx_last_error().decode())
    return k


class Batch:
    """Ragged batch descriptor: request lengths and selected counts, host and device copies."""

    def __init__(self, lengths: Sequence[int], n_sel: Sequence[int], device):
        self.lengths = [int(t) for t in lengths]
        self.n_sel = [int(k) for k in n_sel]
        self.cu_tokens = [0]
        self.cu_sel = [0]
        for t, k in zip(self.lengths, self.n_sel):
            self.cu_tokens.append(self.cu_tokens[-1] + t)
            self.cu_sel.append(self.cu_sel[-1] + k)
        n = len(self.lengths)
        self._h_tok = (ctypes.c_int32 * (n + 1))(*self.cu_tokens)
        self._h_sel = (ctypes.c_int32 * (n + 1))(*self.cu_sel)
        self.d_tok = torch.tensor(self.cu_tokens, dtype=torch.int32, device=device)
        self.d_sel = torch.tensor(self.cu_sel, dtype=torch.int32, device=device)
        self.c = _Batch(n, self._h_tok, self._h_sel, self.d_tok.data_ptr(), self.d_sel.data_ptr())

    @classmethod
    def for_budgets(cls, lengths: Sequence[int], pcts: Sequence[int], device) -> "Batch":
        return cls(lengths, [budget(t, p) for t, p in zip(lengths, pcts)], device)

    @property
    def n_req(self) -> int:
        return len(self.lengths)

    @property
    def n_tokens(self) -> int:
        return self.cu_tokens[-1]

    @property
    def total_sel(self) -> int:
        return self.cu_sel[-1]

    @property
    def total_rest(self) -> int:
        return self.n_tokens - self.total_sel


class Cache:
    """Target K/V cache of all layers, contiguous [L][slots][H_kv][d_h] or paged."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, n_layers: int, n_slots: int,
                 page_table: Optional[torch.Tensor] = None, page_size: int = 16):
        self.k, self.v, self.page_table = k, v, page_table
        paged = page_table is not None
        self.c = _Cache(PAGED if paged else CONTIGUOUS, k.data_ptr(), v.data_ptr(), n_layers, n_slots,
                        page_size if paged else 0, page_table.shape[1] if paged else 0,
                        page_table.data_ptr() if paged else None)

    @classmethod
    def empty(cls, n_layers: int, n_slots: int, H_kv: int, d_h: int, dtype, device,
              page_table: Optional[torch.Tensor] = None, page_size: int = 16) -> "Cache":
        shape = (n_layers, n_slots, H_kv, d_h)
        k = torch.empty(shape, dtype=dtype, device=device)
        v = torch.empty(shape, dtype=dtype, device=device)
        return cls(k, v, n_layers, n_slots, page_table, page_size)


def map_latent_workspace(dtype: int, n: int, d_src: int, r: int) -> int:
    b = _SZ()
    _check("kvx_map_latent_workspace", lib().kvx_map_latent_workspace(dtype, n, d_src, r, ctypes.byref(b)))
    return b.value


def map_latent(x_src: torch.Tensor, w_s: torch.Tensor, z: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    n, d_src = x_src.shape
    r = w_s.shape[0]
    dt = _dtype(x_src)
    if z is None:
        z = torch.empty((n, r), dtype=x_src.dtype, device=x_src.device)
    need = map_latent_workspace(dt, n, d_src, r)
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=x_src.device)
    _check("kvx_map_latent", lib().kvx_map_latent(_stream(x_src.device), dt, _ptr(x_src), _ptr(w_s), _ptr(z), n,
                                                  d_src, r, _ptr(ws) if need else None, ws.numel() if need else 0))
    return z


def score_prepare(w_l: torch.Tensor, u: torch.Tensor) -> torch.Tensor:
    L_t, d_t, r = w_l.shape
    c = u.shape[2]
    dt = _dtype(w_l)
    ws_bytes = _SZ()
    _check("kvx_score_prepare_workspace", lib().kvx_score_prepare_workspace(r, d_t, c, ctypes.byref(ws_bytes)))
    ws = torch.empty(ws_bytes.value, dtype=torch.uint8, device=w_l.device)
    op = (torch.empty((r, 2 * r), dtype=torch.bfloat16, device=w_l.device) if dt == BF16
          else torch.empty((r, r), dtype=torch.float32, device=w_l.device))
    _check("kvx_score_prepare", lib().kvx_score_prepare(_stream(w_l.device), dt, _ptr(w_l),
                                                        _ptr(u) if c > 0 else None, L_t, r, d_t, c,
                                                        _ptr(op), _ptr(ws), ws_bytes.value))
    return op


def select_topk(scores: torch.Tensor, batch: Batch, out=None):
    dev = scores.device
    if out is None:
        sel = torch.empty(max(batch.total_sel, 1), dtype=torch.int32, device=dev)
        rest = torch.empty(max(batch.total_rest, 1), dtype=torch.int32, device=dev)
    else:
        sel, rest = out
    _check("kvx_select_topk", lib().kvx_select_topk(_stream(dev), _ptr(scores), ctypes.byref(batch.c),
                                                    _ptr(sel), _ptr(rest)))
    return sel[:batch.total_sel], rest[:batch.total_rest]


def score_select_workspace(dtype: int, r: int, n: int) -> int:
    b = _SZ()
    _check("kvx_score_select_workspace", lib().kvx_score_select_workspace(dtype, r, n, ctypes.byref(b)))
    return b.value


def score_select(z: torch.Tensor, op: torch.Tensor, batch: Batch, pcts: Sequence[int],
                 ws: Optional[torch.Tensor] = None, out=None):
    dev = z.device
    r = z.shape[1]
    dt = _dtype(z)
    need = score_select_workspace(dt, r, batch.n_tokens)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if out is None:
        scores = torch.empty(batch.n_tokens, dtype=torch.float32, device=dev)
        sel = torch.empty(max(batch.total_sel, 1), dtype=torch.int32, device=dev)
        rest = torch.empty(max(batch.total_rest, 1), dtype=torch.int32, device=dev)
    else:
        scores, sel, rest = out
    pct = (ctypes.c_int32 * batch.n_req)(*[int(p) for p in pcts])
    _check("kvx_score_select", lib().kvx_score_select(_stream(dev), dt, _ptr(z), _ptr(op), r,
                                                      ctypes.byref(batch.c), pct, _ptr(scores), _ptr(sel),
                                                      _ptr(rest), _ptr(ws), need))
    return scores, sel[:batch.total_sel], rest[:batch.total_rest]


def score_cache_prepare(u: torch.Tensor, dtype: int) -> torch.Tensor:
    """Calibration bases u [n_layers][d_t][c] fp32 packed for the direct scoring of a cache of
    storage dtype `dtype` (BF16 or F32)."""
    L, d_t, c = u.shape
    op = (torch.empty((L, c, 2 * d_t), dtype=torch.bfloat16, device=u.device) if dtype == BF16
          else torch.empty((L, d_t, c), dtype=torch.float32, device=u.device))
    _check("kvx_score_cache_prepare", lib().kvx_score_cache_prepare(_stream(u.device), dtype, _ptr(u), L, d_t, c,
                                                                    _ptr(op)))
    return op


def _score_cache_ws(dt: int, n_layers: int, c: int, n: int, ws, dev):
    b = _SZ()
    _check("kvx_score_cache_workspace", lib().kvx_score_cache_workspace(dt, n_layers, c, n, ctypes.byref(b)))
    if ws is None or ws.numel() < b.value:
        ws = torch.empty(max(b.value, 16), dtype=torch.uint8, device=dev)
    return ws


def _op_shape(op: torch.Tensor):
    """(n_layers, c) of a packed basis."""
    return (op.shape[0], op.shape[1]) if op.dtype == torch.bfloat16 else (op.shape[0], op.shape[2])


def score_cache(cache: Cache, layer0: int, H_kv: int, d_h: int, op: torch.Tensor, batch: Batch,
                energy: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Energy outside the calibration subspace of every position's stored K/V, per scored layer:
    [n_layers][N] fp32 for the layers [layer0, layer0 + n_layers) of `cache`."""
    dev = cache.k.device
    dt = _dtype(cache.k)
    n_layers, c = _op_shape(op)
    if energy is None:
        energy = torch.empty((n_layers, max(batch.n_tokens, 1)), dtype=torch.float32, device=dev)
    ws = _score_cache_ws(dt, n_layers, c, batch.n_tokens, ws, dev)
    _check("kvx_score_cache", lib().kvx_score_cache(_stream(dev), dt, ctypes.byref(cache.c), layer0, n_layers, H_kv,
                                                    d_h, _ptr(op), c, ctypes.byref(batch.c), _ptr(energy), _ptr(ws),
                                                    ws.numel()))
    return energy[:, :batch.n_tokens]


def score_cache_select(cache: Cache, layer0: int, H_kv: int, d_h: int, op: torch.Tensor, batch: Batch,
                       pcts: Sequence[int], ws: Optional[torch.Tensor] = None, out=None):
    """Scores summed over the scored layers' stored K/V and their top-budget selection."""
    dev = cache.k.device
    dt = _dtype(cache.k)
    n_layers, c = _op_shape(op)
    ws = _score_cache_ws(dt, n_layers, c, batch.n_tokens, ws, dev)
    if out is None:
        scores = torch.empty(max(batch.n_tokens, 1), dtype=torch.float32, device=dev)
        sel = torch.empty(max(batch.total_sel, 1), dtype=torch.int32, device=dev)
        rest = torch.empty(max(batch.total_rest, 1), dtype=torch.int32, device=dev)
    else:
        scores, sel, rest = out
    pct = (ctypes.c_int32 * batch.n_req)(*[int(p) for p in pcts])
    _check("kvx_score_cache_select", lib().kvx_score_cache_select(
        _stream(dev), dt, ctypes.byref(cache.c), layer0, n_layers, H_kv, d_h, _ptr(op), c, ctypes.byref(batch.c), pct,
        _ptr(scores), _ptr(sel), _ptr(rest), _ptr(ws), ws.numel()))
    return scores[:batch.n_tokens], sel[:batch.total_sel], rest[:batch.total_rest]


def select_topk_layers(scores: torch.Tensor, batch: Batch, out=None):
    """Every layer's own top-k: scores [n_layers][N] -> sel [n_layers][K], rest [n_layers][N - K]."""
    dev = scores.device
    n_layers = scores.shape[0]
    if out is None:
        sel = torch.empty((n_layers, max(batch.total_sel, 1)), dtype=torch.int32, device=dev)
        rest = torch.empty((n_layers, max(batch.total_rest, 1)), dtype=torch.int32, device=dev)
    else:
        sel, rest = out
    assert scores.is_contiguous() and scores.shape[1] == batch.n_tokens
    assert sel.shape[1] == batch.total_sel or batch.total_sel == 0
    assert rest.shape[1] == batch.total_rest or batch.total_rest == 0
    _check("kvx_select_topk_layers", lib().kvx_select_topk_layers(_stream(dev), _ptr(scores), n_layers,
                                                                  ctypes.byref(batch.c), _ptr(sel), _ptr(rest)))
    return sel[:, :batch.total_sel], rest[:, :batch.total_rest]


def select_pages(scores: torch.Tensor, batch: Batch, page_size: int, pcts: Sequence[int]):
    """Whole pages of page_size positions by the sum of their scores; request b keeps
    kvx_budget(ceil(T_b / page_size), pcts[b]) pages.  The selected count depends on the data (a
    short last page), so this call waits for the device to read it.  Returns (sel, rest, sel_batch,
    page_scores, sel_pages): sel_batch is the batch of the positions with the selected counts."""
    dev = scores.device
    n_pages = [-(-t // page_size) for t in batch.lengths]
    pages = Batch.for_budgets(n_pages, pcts, dev)
    page_scores = torch.empty(max(pages.n_tokens, 1), dtype=torch.float32, device=dev)
    sel_pages = torch.empty(max(pages.total_sel, 1), dtype=torch.int32, device=dev)
    rest_pages = torch.empty(max(pages.total_rest, 1), dtype=torch.int32, device=dev)
    cu_sel = torch.empty(batch.n_req + 1, dtype=torch.int32, device=dev)
    sel = torch.empty(max(pages.total_sel * page_size, 1), dtype=torch.int32, device=dev)
    rest = torch.empty(max(batch.n_tokens, 1), dtype=torch.int32, device=dev)
    _check("kvx_select_pages", lib().kvx_select_pages(_stream(dev), _ptr(scores), ctypes.byref(batch.c), page_size,
                                                      ctypes.byref(pages.c), _ptr(page_scores), _ptr(sel_pages),
                                                      _ptr(rest_pages), _ptr(cu_sel), _ptr(sel), _ptr(rest)))
    cu = cu_sel.cpu().tolist()
    counts = [cu[b + 1] - cu[b] for b in range(batch.n_req)]
    sel_batch = Batch(batch.lengths, counts, dev)
    return (sel[:cu[-1]], rest[:batch.n_tokens - cu[-1]], sel_batch, page_scores[:pages.n_tokens],
            sel_pages[:pages.total_sel])


def score_select_normalized(z: torch.Tensor, op: torch.Tensor, op_total: torch.Tensor, batch: Batch,
                            pcts: Sequence[int], ws: Optional[torch.Tensor] = None, out=None):
    """Scores as shares (outside energy over total energy) and their top-budget selection."""
    dev = z.device
    r = z.shape[1]
    dt = _dtype(z)
    b = _SZ()
    _check("kvx_score_select_normalized_workspace",
           lib().kvx_score_select_normalized_workspace(dt, r, batch.n_tokens, ctypes.byref(b)))
    need = b.value
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if out is None:
        scores = torch.empty(batch.n_tokens, dtype=torch.float32, device=dev)
        sel = torch.empty(max(batch.total_sel, 1), dtype=torch.int32, device=dev)
        rest = torch.empty(max(batch.total_rest, 1), dtype=torch.int32, device=dev)
    else:
        scores, sel, rest = out
    pct = (ctypes.c_int32 * batch.n_req)(*[int(p) for p in pcts])
    _check("kvx_score_select_normalized", lib().kvx_score_select_normalized(
        _stream(dev), dt, _ptr(z), _ptr(op), _ptr(op_total), r, ctypes.byref(batch.c), pct, _ptr(scores), _ptr(sel),
        _ptr(rest), _ptr(ws), ws.numel()))
    return scores, sel[:batch.total_sel], rest[:batch.total_rest]


def score_select_noalloc(z: torch.Tensor, op: torch.Tensor, batch: Batch, pcts: Sequence[int], out=None):
    """kvx_score_select with the library's fixed scratch instead of a workspace (no allocation
    in the library; out = (scores, sel, rest) avoids the allocations here as well)."""
    dev = z.device
    r = z.shape[1]
    if out is None:
        scores = torch.empty(batch.n_tokens, dtype=torch.float32, device=dev)
        sel = torch.empty(max(batch.total_sel, 1), dtype=torch.int32, device=dev)
        rest = torch.empty(max(batch.total_rest, 1), dtype=torch.int32, device=dev)
    else:
        scores, sel, rest = out
    pct = (ctypes.c_int32 * batch.n_req)(*[int(p) for p in pcts])
    _check("kvx_score_select_noalloc", lib().kvx_score_select_noalloc(_stream(dev), _dtype(z), _ptr(z), _ptr(op), r,
                                                                      ctypes.byref(batch.c), pct, _ptr(scores),
                                                                      _ptr(sel), _ptr(rest)))
    return scores, sel[:batch.total_sel], rest[:batch.total_rest]


def fit_mapper(x: torch.Tensor, y: torch.Tensor, L_t: int, r: int, lam: float, iters: int = 30):
    """Closed-form fit of the factorized mapper to paired calibration KV: x [n, d_src], y [n, L_t * d_t]
    (layer-major).  Returns w_s [r, d_src] and w_l [L_t, d_t, r] in x's dtype."""
    n, d_src = x.shape
    d_t = y.shape[1] // L_t
    dt = _dtype(x)
    b = _SZ()
    _check("kvx_fit_mapper_workspace", lib().kvx_fit_mapper_workspace(dt, n, d_src, L_t, d_t, r, ctypes.byref(b)))
    ws = torch.empty(b.value, dtype=torch.uint8, device=x.device)
    w_s = torch.empty((r, d_src), dtype=x.dtype, device=x.device)
    w_l = torch.empty((L_t, d_t, r), dtype=x.dtype, device=x.device)
    _check("kvx_fit_mapper", lib().kvx_fit_mapper(_stream(x.device), dt, _ptr(x), _ptr(y), n, d_src, L_t, d_t, r,
                                                  float(lam), iters, _ptr(w_s), _ptr(w_l), _ptr(ws), b.value))
    return w_s, w_l


def fit_calibration(z: torch.Tensor, w_l: torch.Tensor, c: int, iters: int = 30) -> torch.Tensor:
    """Calibration subspaces: u [L_t, d_t, c] fp32 from the calibration latents z [n, r] and w_l [L_t, d_t, r]."""
    n, r = z.shape
    L_t, d_t, _ = w_l.shape
    b = _SZ()
    _check("kvx_fit_calibration_workspace", lib().kvx_fit_calibration_workspace(n, L_t, d_t, r, c, ctypes.byref(b)))
    ws = torch.empty(b.value, dtype=torch.uint8, device=z.device)
    u = torch.empty((L_t, d_t, c), dtype=torch.float32, device=z.device)
    _check("kvx_fit_calibration", lib().kvx_fit_calibration(_stream(z.device), _dtype(z), _ptr(z), _ptr(w_l), n, L_t,
                                                            d_t, r, c, iters, _ptr(u), _ptr(ws), b.value))
    return u


def reconstruct(z: torch.Tensor, w_l: torch.Tensor, H_kv: int, d_h: int, batch: Batch, cache: Cache,
                rows: Optional[torch.Tensor] = None, rope: Optional[torch.Tensor] = None):
    """Translated K/V of the listed rows (all rows when rows is None) into every layer's cache;
    with a rotary table the keys are rotated at their positions (kvx_reconstruct_rope)."""
    L_t, _, r = w_l.shape
    if rows is None:
        rp = None                                   # every position
    elif rows.numel() == 0:
        rp = _ptr(_placeholder(z.device))           # an empty list: nothing to reconstruct
    else:
        rp = _ptr(rows)
    if rope is not None:
        _check("kvx_reconstruct_rope", lib().kvx_reconstruct_rope(
            _stream(z.device), _dtype(z), _ptr(z), _ptr(w_l), L_t, r, H_kv, d_h, _ptr(rope), rope.shape[0],
            ctypes.byref(batch.c), rp, ctypes.byref(cache.c)))
        return
    _check("kvx_reconstruct", lib().kvx_reconstruct(_stream(z.device), _dtype(z), _ptr(z), _ptr(w_l), L_t, r,
                                                    H_kv, d_h, ctypes.byref(batch.c), rp,
                                                    ctypes.byref(cache.c)))


_placeholders = {}


def _placeholder(device) -> torch.Tensor:
    key = str(device)
    if key not in _placeholders:
        _placeholders[key] = torch.zeros(4, dtype=torch.int32, device=device)
    return _placeholders[key]


def rope_table(base: float, d_h: int, max_pos: int, device) -> torch.Tensor:
    t = torch.empty((max_pos, d_h // 2, 2), dtype=torch.float32, device=device)
    _check("kvx_rope_table", lib().kvx_rope_table(_stream(device), float(base), d_h, max_pos, _ptr(t)))
    return t


def recompute_attn_workspace(dtype: int, batch: Batch, D: int, H_q: int, H_kv: int, d_h: int) -> int:
    b = _SZ()
    _check("kvx_recompute_attn_workspace",
           lib().kvx_recompute_attn_workspace(dtype, ctypes.byref(batch.c), D, H_q, H_kv, d_h, ctypes.byref(b)))
    return b.value


def qkv_project_workspace(dtype: int, batch: Batch, D: int, H_q: int, H_kv: int, d_h: int) -> int:
    b = _SZ()
    _check("kvx_qkv_project_workspace",
           lib().kvx_qkv_project_workspace(dtype, ctypes.byref(batch.c), D, H_q, H_kv, d_h, ctypes.byref(b)))
    return b.value


def recompute_attn(layer: int, x_l: torch.Tensor, w_qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int,
                   rope: torch.Tensor, batch: Batch, sel: torch.Tensor, cache: Cache,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None):
    dev = x_l.device
    dt = _dtype(x_l)
    D = x_l.shape[1]
    need = recompute_attn_workspace(dt, batch, D, H_q, H_kv, d_h)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((max(batch.total_sel, 1), H_q, d_h), dtype=x_l.dtype, device=dev)
    _check("kvx_recompute_attn", lib().kvx_recompute_attn(
        _stream(dev), dt, layer, _ptr(x_l), _ptr(w_qkv), D, H_q, H_kv, d_h, _ptr(rope), rope.shape[0],
        ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None, ctypes.byref(cache.c),
        _ptr(out), _ptr(lse), _ptr(ws), ws.numel()))
    return out[:batch.total_sel]


def qkv_project(x_l: torch.Tensor, w_qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int, batch: Batch,
                sel: torch.Tensor, qkv: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    dev = x_l.device
    dt = _dtype(x_l)
    D = x_l.shape[1]
    n_qkv = (H_q + 2 * H_kv) * d_h
    if qkv is None:
        qkv = torch.empty((max(batch.total_sel, 1), n_qkv), dtype=x_l.dtype, device=dev)
    need = qkv_project_workspace(dt, batch, D, H_q, H_kv, d_h)
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("kvx_qkv_project", lib().kvx_qkv_project(_stream(dev), dt, _ptr(x_l), _ptr(w_qkv), D,
                                                    H_q, H_kv, d_h, ctypes.byref(batch.c),
                                                    _ptr(sel) if sel.numel() else None, _ptr(qkv),
                                                    _ptr(ws) if need else None, ws.numel() if need else 0))
    return qkv


def rope_scatter(layer: int, qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int, rope: torch.Tensor, batch: Batch,
                 sel: torch.Tensor, cache: Cache):
    _check("kvx_rope_scatter", lib().kvx_rope_scatter(_stream(qkv.device), _dtype(qkv), layer, _ptr(qkv), H_q, H_kv,
                                                      d_h, _ptr(rope), rope.shape[0], ctypes.byref(batch.c),
                                                      _ptr(sel) if sel.numel() else None, ctypes.byref(cache.c)))


def qkv_rope_scatter(layer: int, x_l: torch.Tensor, w_qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int,
                     rope: torch.Tensor, batch: Batch, sel: torch.Tensor, cache: Cache,
                     qkv: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Steps 1-3 in one call: q rows into qkv (its k/v columns stay unwritten), rotated k and v
    into the cache.  Returns qkv."""
    dev = x_l.device
    dt = _dtype(x_l)
    D = x_l.shape[1]
    n_qkv = (H_q + 2 * H_kv) * d_h
    if qkv is None:
        qkv = torch.empty((max(batch.total_sel, 1), n_qkv), dtype=x_l.dtype, device=dev)
    need = qkv_project_workspace(dt, batch, D, H_q, H_kv, d_h)
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("kvx_qkv_rope_scatter", lib().kvx_qkv_rope_scatter(
        _stream(dev), dt, layer, _ptr(x_l), _ptr(w_qkv), D, H_q, H_kv, d_h, _ptr(rope), rope.shape[0],
        ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None, ctypes.byref(cache.c), _ptr(qkv),
        _ptr(ws) if need else None, ws.numel() if need else 0))
    return qkv


def qkv_rope_scatter_qknorm(layer: int, x_l: torch.Tensor, w_qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int,
                            q_gain: torch.Tensor, k_gain: torch.Tensor, eps: float, rope: torch.Tensor, batch: Batch,
                            sel: torch.Tensor, cache: Cache, qkv: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Steps 1-3 with q and k normalised per head before the rotation (QK-norm); returns qkv."""
    dev = x_l.device
    D = x_l.shape[1]
    n_qkv = (H_q + 2 * H_kv) * d_h
    if qkv is None:
        qkv = torch.empty((max(batch.total_sel, 1), n_qkv), dtype=x_l.dtype, device=dev)
    _check("kvx_qkv_rope_scatter_qknorm", lib().kvx_qkv_rope_scatter_qknorm(
        _stream(dev), _dtype(x_l), layer, _ptr(x_l), _ptr(w_qkv), D, H_q, H_kv, d_h, _ptr(q_gain), _ptr(k_gain),
        float(eps), _ptr(rope), rope.shape[0], ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None,
        ctypes.byref(cache.c), _ptr(qkv)))
    return qkv


def sparse_attention_workspace(dtype: int, batch: Batch, H_q: int, H_kv: int, d_h: int) -> int:
    b = _SZ()
    _check("kvx_sparse_attention_workspace",
           lib().kvx_sparse_attention_workspace(dtype, ctypes.byref(batch.c), H_q, H_kv, d_h, ctypes.byref(b)))
    return b.value


def sparse_attention(layer: int, qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int, rope: torch.Tensor,
                     batch: Batch, sel: torch.Tensor, cache: Cache, out: torch.Tensor,
                     lse: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, split: bool = True):
    """Causal attention of the selected queries; with split=False no workspace is passed and
    the keys of a query block are never cut into chunks."""
    dt = _dtype(qkv)
    need = sparse_attention_workspace(dt, batch, H_q, H_kv, d_h) if split else 0
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=qkv.device)
    _check("kvx_sparse_attention", lib().kvx_sparse_attention(
        _stream(qkv.device), dt, layer, _ptr(qkv), H_q, H_kv, d_h, _ptr(rope), rope.shape[0],
        ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None, ctypes.byref(cache.c), _ptr(out), _ptr(lse),
        _ptr(ws) if need else None, ws.numel() if need else 0))
    return out


def recompute_attn_layers_workspace(dtype: int, batch: Batch, D: int, H_q: int, H_kv: int, d_h: int,
                                    n_layers: int) -> int:
    b = _SZ()
    _check("kvx_recompute_attn_layers_workspace",
           lib().kvx_recompute_attn_layers_workspace(dtype, ctypes.byref(batch.c), D, H_q, H_kv, d_h, n_layers,
                                                     ctypes.byref(b)))
    return b.value


def recompute_attn_layers(l0: int, x: torch.Tensor, w_qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int,
                          rope: torch.Tensor, batch: Batch, sel: torch.Tensor, cache: Cache,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvx_recompute_attn of layers l0 .. l0 + n - 1 in one call: x [n, N, D], w_qkv [n, n_qkv, D];
    returns out [n, total_sel, H_q, d_h]."""
    dev = x.device
    dt = _dtype(x)
    n, _, D = x.shape
    need = recompute_attn_layers_workspace(dt, batch, D, H_q, H_kv, d_h, n)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((n, max(batch.total_sel, 1), H_q, d_h), dtype=x.dtype, device=dev)
    _check("kvx_recompute_attn_layers", lib().kvx_recompute_attn_layers(
        _stream(dev), dt, l0, n, _ptr(x), _ptr(w_qkv), D, H_q, H_kv, d_h, _ptr(rope), rope.shape[0],
        ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None, ctypes.byref(cache.c), _ptr(out), _ptr(lse),
        _ptr(ws), ws.numel()))
    return out


def qkv_rope_scatter_layers(l0: int, x: torch.Tensor, w_qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int,
                            rope: torch.Tensor, batch: Batch, sel: torch.Tensor, cache: Cache,
                            qkv: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Steps 1-3 of layers l0 .. l0 + n - 1 in one launch; returns qkv [n, total_sel, n_qkv] (q columns)."""
    dev = x.device
    n, _, D = x.shape
    n_qkv = (H_q + 2 * H_kv) * d_h
    if qkv is None:
        qkv = torch.empty((n, max(batch.total_sel, 1), n_qkv), dtype=x.dtype, device=dev)
    _check("kvx_qkv_rope_scatter_layers", lib().kvx_qkv_rope_scatter_layers(
        _stream(dev), _dtype(x), l0, n, _ptr(x), _ptr(w_qkv), D, H_q, H_kv, d_h, _ptr(rope), rope.shape[0],
        ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None, ctypes.byref(cache.c), _ptr(qkv)))
    return qkv


def sparse_attention_layers(l0: int, qkv: torch.Tensor, H_q: int, H_kv: int, d_h: int, rope: torch.Tensor,
                            batch: Batch, sel: torch.Tensor, cache: Cache, out: torch.Tensor,
                            lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal attention of layers l0 .. l0 + n - 1 in one launch: qkv [n, total_sel, n_qkv],
    out [n, total_sel, H_q, d_h], lse [n, total_sel, H_q] or None."""
    n = qkv.shape[0]
    _check("kvx_sparse_attention_layers", lib().kvx_sparse_attention_layers(
        _stream(qkv.device), _dtype(qkv), l0, n, _ptr(qkv), H_q, H_kv, d_h, _ptr(rope), rope.shape[0],
        ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None, ctypes.byref(cache.c), _ptr(out), _ptr(lse)))
    return out


# ------------------------------------------------------------------------------ layer chaining

def gather_rows(src: torch.Tensor, batch: Batch, sel: torch.Tensor, dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dst[i] = src[cu_tokens[b] + sel[i]]: the compact selected rows of a batch."""
    D = src.shape[1]
    if dst is None:
        dst = torch.empty((max(batch.total_sel, 1), D), dtype=src.dtype, device=src.device)
    _check("kvx_gather_rows", lib().kvx_gather_rows(_stream(src.device), _dtype(src), _ptr(src), D,
                                                    ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None,
                                                    _ptr(dst)))
    return dst


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    n, D = x.shape
    if y is None:
        y = torch.empty_like(x)
    _check("kvx_rmsnorm", lib().kvx_rmsnorm(_stream(x.device), _dtype(x), _ptr(x), _ptr(gamma), eps, n, D, _ptr(y)))
    return y


def _ws(need: int, ws: Optional[torch.Tensor], device):
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return (_ptr(ws), ws.numel()) if need else (None, 0)


def linear_residual(a: torch.Tensor, w: torch.Tensor, resid: torch.Tensor, out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = resid + a w^T (out may be resid)."""
    M, K = a.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty_like(resid)
    b = _SZ()
    _check("kvx_linear_residual_workspace", lib().kvx_linear_residual_workspace(_dtype(a), M, N, K, ctypes.byref(b)))
    wp, wn = _ws(b.value, ws, a.device)
    _check("kvx_linear_residual", lib().kvx_linear_residual(_stream(a.device), _dtype(a), _ptr(a), _ptr(w),
                                                            _ptr(resid), _ptr(out), M, N, K, wp, wn))
    return out


def swiglu(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, h: Optional[torch.Tensor] = None,
           ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h = silu(x w_gate^T) * (x w_up^T)."""
    M, D = x.shape
    F = w_gate.shape[0]
    if h is None:
        h = torch.empty((M, F), dtype=x.dtype, device=x.device)
    b = _SZ()
    _check("kvx_swiglu_workspace", lib().kvx_swiglu_workspace(_dtype(x), M, D, F, ctypes.byref(b)))
    wp, wn = _ws(b.value, ws, x.device)
    _check("kvx_swiglu", lib().kvx_swiglu(_stream(x.device), _dtype(x), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(h),
                                          M, D, F, wp, wn))
    return h


class LayerWeights:
    """Device weights of one chained target layer (bf16, output-major)."""

    def __init__(self, gamma_in, w_qkv, w_o, gamma_post, w_gate, w_up, w_down):
        self.tensors = (gamma_in, w_qkv, w_o, gamma_post, w_gate, w_up, w_down)
        self.c = _LayerWeights(*[t.data_ptr() for t in self.tensors])


def target_layer_workspace(dtype: int, batch: Batch, D: int, F: int, H_q: int, H_kv: int, d_h: int) -> int:
    b = _SZ()
    _check("kvx_target_layer_workspace",
           lib().kvx_target_layer_workspace(dtype, ctypes.byref(batch.c), D, F, H_q, H_kv, d_h, ctypes.byref(b)))
    return b.value


def target_layer(layer: int, x: torch.Tensor, w: LayerWeights, F: int, H_q: int, H_kv: int, d_h: int, eps: float,
                 rope: torch.Tensor, batch: Batch, sel: torch.Tensor, cache: Cache,
                 attn_out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One chained target layer on the compact selected rows x (updated in place)."""
    D = x.shape[1]
    dt = _dtype(x)
    need = target_layer_workspace(dt, batch, D, F, H_q, H_kv, d_h)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check("kvx_target_layer", lib().kvx_target_layer(
        _stream(x.device), dt, layer, _ptr(x), ctypes.byref(w.c), D, F, H_q, H_kv, d_h, eps, _ptr(rope),
        rope.shape[0], ctypes.byref(batch.c), _ptr(sel) if sel.numel() else None, ctypes.byref(cache.c),
        _ptr(attn_out), _ptr(lse), _ptr(ws), ws.numel()))
    return x


def linear_workspace(dtype: int, M: int, N: int, K: int) -> int:
    b = _SZ()
    _check("kvx_linear_workspace", lib().kvx_linear_workspace(dtype, M, N, K, ctypes.byref(b)))
    return b.value


def linear(a: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None,
           ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = a w^T."""
    M, K = a.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    b = _SZ()
    _check("kvx_linear_workspace", lib().kvx_linear_workspace(_dtype(a), M, N, K, ctypes.byref(b)))
    wp, wn = _ws(b.value, ws, a.device)
    _check("kvx_linear", lib().kvx_linear(_stream(a.device), _dtype(a), _ptr(a), _ptr(w), _ptr(out), M, N, K, wp, wn))
    return out


def argmax(logits: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index of each row's largest logit (ties to the lowest index), int32."""
    n, V = logits.shape
    if out is None:
        out = torch.empty(max(n, 1), dtype=torch.int32, device=logits.device)
    _check("kvx_argmax", lib().kvx_argmax(_stream(logits.device), _dtype(logits), _ptr(logits), n, V, _ptr(out)))
    return out[:n]
