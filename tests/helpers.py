"""Test-side helpers: conversions, logical views of a (paged) cache, error metrics."""
from __future__ import annotations

import numpy as np
import torch


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a stored tensor to float64 on the host."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def slots_of(b: int, T: int, cu_tokens, page_table: np.ndarray = None, page_size: int = 16) -> np.ndarray:
    """Cache slots of positions 0..T-1 of request b (contiguous or paged layout)."""
    p = np.arange(T)
    if page_table is None:
        return cu_tokens[b] + p
    return page_table[b, p // page_size] * page_size + p % page_size


def logical(cache_t: torch.Tensor, layer: int, b: int, T: int, cu_tokens, page_table=None,
            page_size=16) -> np.ndarray:
    """Request b's [T, H_kv, d_h] view of one layer of a cache tensor [L][slots][H_kv][d_h]."""
    sl = slots_of(b, T, cu_tokens, page_table, page_size)
    return f64(cache_t[layer][torch.as_tensor(sl, device=cache_t.device)])


def rel_norm(a: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / den) if den > 0 else float(np.linalg.norm(a))


def rel_max(a: np.ndarray, ref: np.ndarray) -> float:
    den = np.abs(ref).max()
    return float(np.abs(a - ref).max() / den) if den > 0 else float(np.abs(a).max())


def min_row_cosine(a: np.ndarray, ref: np.ndarray) -> float:
    a = a.reshape(-1, a.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    num = (a * ref).sum(-1)
    den = np.linalg.norm(a, axis=-1) * np.linalg.norm(ref, axis=-1)
    return float((num / den).min())


def assert_close(a, ref, tol, what):
    """Relative error per tensor: normwise and max-abs, both within tol."""
    rn, rm = rel_norm(a, ref), rel_max(a, ref)
    assert rn <= tol and rm <= tol, f"{what}: normwise {rn:.3e}, max {rm:.3e} > {tol:.1e}"
    return rn, rm


def band_check(S_gpu, s_ora: np.ndarray, k: int, eps: float):
    """Selected sets agree outside the band |s - tau| <= eps * tau around the oracle's k-th
    score.  Returns (band size, symmetric difference size, oracle relative gap)."""
    from oracle import kvx_oracle as O
    S_ora, _ = O.select(s_ora, k)
    if k == 0 or k == len(s_ora):
        assert set(S_gpu) == set(S_ora.tolist())
        return 0, 0, float("inf")
    tau = np.sort(s_ora)[::-1][k - 1]
    band = set(np.nonzero(np.abs(s_ora - tau) <= eps * abs(tau))[0].tolist())
    a, b = set(int(x) for x in S_gpu), set(S_ora.tolist())
    assert a - band == b - band, f"selection differs outside the band: {sorted((a ^ b) - band)[:10]}"
    return len(band), len(a ^ b), O.score_gap(s_ora, k)


def oracle_downstream(K_tr: np.ndarray, V_tr: np.ndarray, x_l: np.ndarray, w_qkv: np.ndarray, S: np.ndarray,
                      H_q: int, H_kv: int, d_h: int, base: float):
    """The oracle's recompute, scatter and attention steps on a given selected set S (the GPU's
    own set, so that both sides attend with the same queries).  K_tr, V_tr [L_t, T, H_kv, d_h]
    is the oracle's translated cache, x_l [L_t, T, D].  Returns the mixed cache K, V and the
    outputs O [L_t, k, H_q, d_h], LSE [L_t, k, H_q]."""
    from oracle import kvx_oracle as O
    S = np.asarray(S, dtype=np.int64)
    L = K_tr.shape[0]
    K, V = K_tr.copy(), V_tr.copy()
    out = np.zeros((L, len(S), H_q, d_h))
    lse = np.zeros((L, len(S), H_q))
    for l in range(L):
        q, kk, vv = O.recompute_qkv(x_l[l][S], w_qkv[l], S, H_q, H_kv, d_h, base)
        K[l], V[l] = O.scatter(K[l], V[l], S, kk, vv)
        if len(S):
            out[l], lse[l] = O.sparse_causal_attention(q, K[l], V[l], S)
    return K, V, out, lse
