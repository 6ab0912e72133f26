"""Seeded synthetic inputs for the cross-model KV handoff.

Real source/target checkpoints, real source KV caches and calibration data are not
available, so every input here is drawn from a seeded generator with the shapes of
the workloads in ``workloads.py``:

* source KV ``x_src`` [N, d_src]: N(0,1) times one U(0.5, 2) factor per channel
  (the factor stands in for outlier channels), channel order (layer, K/V, head, dim);
* ``w_s`` [r, d_src] ~ N(0, 1/d_src); ``w_l`` [L_t, d_t, r] ~ N(0, 1/r);
  ``w_qkv`` [L_t, (H_q + 2 H_kv) d_h, D] ~ N(0, 1/D)  (weights are stored output-major,
  i.e. row j holds the weights that produce output j);
* calibration bases ``u`` [L_t, d_t, c]: Q factor of the QR of an N(0,1) matrix,
  computed in float64 with diag(R) > 0, stored float32;
* target hidden inputs ``x_l`` [L_t, N, D] ~ N(0,1);
* batched serving: lengths log-uniform in [t_min, t_max] rounded to an integer,
  budgets uniform over the workload's choices, pages assigned by a random permutation
  of a pool of sum(ceil(T_i / page_size)) pages.

Sub-seeds come from ``numpy.random.SeedSequence(seed).spawn(10)`` in a fixed order.
Small tensors are drawn on the host with numpy (PCG64); tensors of a full-size
workload are drawn on the device with ``torch.Generator`` seeded from the same
sub-seed.  This module computes nothing of the method itself.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from .workloads import Workload

_SUBSEEDS = ("scales", "x_src", "w_s", "w_l", "u", "x_l", "w_qkv", "lengths", "budgets", "pages")

# host generation below this many stored elements, device generation above it
HOST_LIMIT = 1 << 27


def _subseeds(seed: int):
    return dict(zip(_SUBSEEDS, np.random.SeedSequence(seed).spawn(len(_SUBSEEDS))))


def _torch_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def storage_dtype(wl: Workload) -> torch.dtype:
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


@dataclass
class Inputs:
    wl: Workload
    lengths: List[int]          # T_i per request
    pcts: List[int]             # budget percent per request
    x_src: torch.Tensor         # [N, d_src]
    w_s: torch.Tensor           # [r, d_src]
    w_l: torch.Tensor           # [L_t, d_t, r]
    u: torch.Tensor             # [L_t, d_t, c] float32
    x_l: torch.Tensor           # [L_t, N, D]
    w_qkv: torch.Tensor         # [L_t, n_qkv, D]
    page_table: Optional[torch.Tensor]  # [n_req, max_pages] int32 (paged workloads)
    n_pages: int

    @property
    def n_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def cu_tokens(self) -> List[int]:
        out = [0]
        for t in self.lengths:
            out.append(out[-1] + t)
        return out


def draw_lengths_budgets(wl: Workload, seed: int):
    """Per-request lengths and budget percents (one request unless the workload is batched)."""
    ss = _subseeds(seed)
    if not wl.batched:
        return [wl.T], [wl.pct]
    rl = np.random.Generator(np.random.PCG64(ss["lengths"]))
    lo, hi = math.log(wl.t_min), math.log(wl.t_max)
    lengths = [int(round(math.exp(v))) for v in rl.uniform(lo, hi, size=wl.n_req)]
    rb = np.random.Generator(np.random.PCG64(ss["budgets"]))
    pcts = [int(wl.pct_choices[i]) for i in rb.integers(0, len(wl.pct_choices), size=wl.n_req)]
    return lengths, pcts


def page_table_for(lengths: List[int], page_size: int, seed: int):
    """Random page assignment; unused table entries are 0 and are never read."""
    ss = _subseeds(seed)
    need = [(t + page_size - 1) // page_size for t in lengths]
    n_pages = int(sum(need))
    perm = np.random.Generator(np.random.PCG64(ss["pages"])).permutation(n_pages).astype(np.int32)
    max_pages = max(need)
    table = np.zeros((len(lengths), max_pages), dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return torch.from_numpy(table), n_pages


def orthonormal_basis(rng: np.random.Generator, n: int, c: int) -> np.ndarray:
    """Q factor of an N(0,1) n-by-c matrix with the sign of each column fixed by diag(R) > 0."""
    if c == 0:
        return np.zeros((n, 0))
    q, r = np.linalg.qr(rng.standard_normal((n, c)))
    return q * np.where(np.diag(r) < 0, -1.0, 1.0)[None, :]


def _host_normal(ss, shape, std=1.0):
    rng = np.random.Generator(np.random.PCG64(ss))
    return rng.standard_normal(size=shape) * std


def generate(wl: Workload, seed: int, device="cpu", where: str = "auto",
             lengths: Optional[List[int]] = None, pcts: Optional[List[int]] = None) -> Inputs:
    """Draw every input of the handoff for workload ``wl``; tensors land on ``device``.
    ``lengths`` / ``pcts`` replace the drawn request lengths and budgets (ragged edge cases)."""
    ss = _subseeds(seed)
    if lengths is None:
        lengths, pcts = draw_lengths_budgets(wl, seed)
    else:
        lengths, pcts = [int(t) for t in lengths], [int(p) for p in pcts]
    N = int(sum(lengths))
    dt = storage_dtype(wl)
    dev = torch.device(device)
    total = N * wl.d_src + wl.L_t * N * wl.D + wl.L_t * wl.n_qkv * wl.D
    on_host = where == "host" or (where == "auto" and (total <= HOST_LIMIT or dev.type == "cpu"))

    # per-channel scales are always drawn on the host (d_src values)
    scales = np.random.Generator(np.random.PCG64(ss["scales"])).uniform(0.5, 2.0, size=wl.d_src)

    # calibration bases: float64 QR on the host, one sub-stream per layer
    ru = np.random.Generator(np.random.PCG64(ss["u"]))
    u = np.stack([orthonormal_basis(ru, wl.d_t, wl.c) for _ in range(wl.L_t)]).astype(np.float32)
    u_t = torch.from_numpy(u).to(dev)

    if on_host:
        def host(name, shape, std=1.0):
            return torch.from_numpy(_host_normal(ss[name], shape, std).astype(np.float32))
        x_src = (host("x_src", (N, wl.d_src)) * torch.from_numpy(scales.astype(np.float32))[None, :])
        w_s = host("w_s", (wl.r, wl.d_src), 1.0 / math.sqrt(wl.d_src))
        w_l = host("w_l", (wl.L_t, wl.d_t, wl.r), 1.0 / math.sqrt(wl.r))
        x_l = host("x_l", (wl.L_t, N, wl.D))
        w_qkv = host("w_qkv", (wl.L_t, wl.n_qkv, wl.D), 1.0 / math.sqrt(wl.D))
        x_src, w_s, w_l, x_l, w_qkv = (t.to(dt).to(dev) for t in (x_src, w_s, w_l, x_l, w_qkv))
    else:
        def dev_normal(name, shape, std=1.0, per_layer=False, col_scale=None):
            g = torch.Generator(device=dev)
            g.manual_seed(_torch_seed(ss[name]))
            out = torch.empty(shape, dtype=dt, device=dev)
            rows = out.view(-1, shape[-1])
            chunk = max(1, (1 << 26) // shape[-1])
            for i in range(0, rows.shape[0], chunk):
                blk = torch.randn((min(chunk, rows.shape[0] - i), shape[-1]), generator=g,
                                  device=dev, dtype=torch.float32)
                if std != 1.0:
                    blk.mul_(std)
                if col_scale is not None:
                    blk.mul_(col_scale)
                rows[i:i + blk.shape[0]].copy_(blk)
            return out
        cs = torch.from_numpy(scales.astype(np.float32)).to(dev)[None, :]
        x_src = dev_normal("x_src", (N, wl.d_src), col_scale=cs)
        w_s = dev_normal("w_s", (wl.r, wl.d_src), 1.0 / math.sqrt(wl.d_src))
        w_l = dev_normal("w_l", (wl.L_t, wl.d_t, wl.r), 1.0 / math.sqrt(wl.r))
        x_l = dev_normal("x_l", (wl.L_t, N, wl.D))
        w_qkv = dev_normal("w_qkv", (wl.L_t, wl.n_qkv, wl.D), 1.0 / math.sqrt(wl.D))

    page_table, n_pages = None, 0
    if wl.paged:
        page_table, n_pages = page_table_for(lengths, wl.page_size, seed)
        page_table = page_table.to(dev)
    return Inputs(wl, lengths, pcts, x_src, w_s, w_l, u_t, x_l, w_qkv, page_table, n_pages)


# ---------------------------------------------------------------------------------
# chained target layers: the weights of the rest of each target layer
# ---------------------------------------------------------------------------------

@dataclass
class ChainWeights:
    gamma_in: torch.Tensor      # [L_t, D]       U(0.5, 1.5)
    w_o: torch.Tensor           # [L_t, D, H_q d_h] ~ N(0, 1/(H_q d_h))
    gamma_post: torch.Tensor    # [L_t, D]       U(0.5, 1.5)
    w_gate: torch.Tensor        # [L_t, F, D]    ~ N(0, 1/D)
    w_up: torch.Tensor          # [L_t, F, D]    ~ N(0, 1/D)
    w_down: torch.Tensor        # [L_t, D, F]    ~ N(0, 1/F)
    gamma_final: Optional[torch.Tensor] = None   # [D]      U(0.5, 1.5)   (vocab > 0)
    w_lm: Optional[torch.Tensor] = None          # [V, D]   ~ N(0, 1/D)


_CHAIN_SUBSEEDS = ("gamma_in", "w_o", "gamma_post", "w_gate", "w_up", "w_down", "gamma_final", "w_lm")


def chain_weights(wl: Workload, seed: int, device="cpu", where: str = "auto") -> ChainWeights:
    """Weights of the chained layers of workload ``wl`` (bf16), and the final norm and
    vocabulary projection when the workload has a vocabulary.  Sub-seeds come from
    ``SeedSequence([seed, 404]).spawn(8)`` so the handoff's own inputs are unchanged."""
    if wl.F <= 0:
        raise ValueError(f"workload {wl.name} has no MLP width")
    ss = dict(zip(_CHAIN_SUBSEEDS, np.random.SeedSequence([seed, 404]).spawn(len(_CHAIN_SUBSEEDS))))
    dev = torch.device(device)
    L, D, F, HD = wl.L_t, wl.D, wl.F, wl.H_q * wl.d_h
    total = L * (D * HD + 3 * F * D)
    on_host = where == "host" or (where == "auto" and (total <= HOST_LIMIT or dev.type == "cpu"))

    def gains(name):
        rng = np.random.Generator(np.random.PCG64(ss[name]))
        return torch.from_numpy(rng.uniform(0.5, 1.5, size=(L, D)).astype(np.float32)).to(torch.bfloat16).to(dev)

    def normal(name, shape, std):
        if on_host:
            return torch.from_numpy((_host_normal(ss[name], shape) * std).astype(np.float32)).to(torch.bfloat16).to(dev)
        g = torch.Generator(device=dev)
        g.manual_seed(_torch_seed(ss[name]))
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        rows = out.view(-1, shape[-1])
        chunk = max(1, (1 << 26) // shape[-1])
        for i in range(0, rows.shape[0], chunk):
            blk = torch.randn((min(chunk, rows.shape[0] - i), shape[-1]), generator=g, device=dev,
                              dtype=torch.float32)
            rows[i:i + blk.shape[0]].copy_(blk.mul_(std))
        return out

    cw = ChainWeights(gains("gamma_in"), normal("w_o", (L, D, HD), 1.0 / math.sqrt(HD)), gains("gamma_post"),
                      normal("w_gate", (L, F, D), 1.0 / math.sqrt(D)), normal("w_up", (L, F, D), 1.0 / math.sqrt(D)),
                      normal("w_down", (L, D, F), 1.0 / math.sqrt(F)))
    if wl.vocab > 0:
        rng = np.random.Generator(np.random.PCG64(ss["gamma_final"]))
        cw.gamma_final = torch.from_numpy(rng.uniform(0.5, 1.5, size=D).astype(np.float32)).to(torch.bfloat16).to(dev)
        cw.w_lm = normal("w_lm", (wl.vocab, D), 1.0 / math.sqrt(D))
    return cw


# ---------------------------------------------------------------------------------
# stage inputs: seeded stand-ins for the upstream results of a single stage
# ---------------------------------------------------------------------------------

def latent(n: int, r: int, seed: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """A stand-in latent [n, r] ~ N(0,1) for stage-wise score / reconstruct checks."""
    ss = np.random.SeedSequence([seed, 101])
    if n * r <= HOST_LIMIT:
        return torch.from_numpy(_host_normal(ss, (n, r)).astype(np.float32)).to(dtype).to(device)
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(ss))
    return torch.randn((n, r), generator=g, device=device, dtype=torch.float32).to(dtype)


def cache_fill(shape, seed: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """A stand-in translated cache (N(0,1)) for stage-wise recompute checks."""
    ss = np.random.SeedSequence([seed, 202])
    n = int(np.prod(shape))
    if n <= HOST_LIMIT:
        return torch.from_numpy(_host_normal(ss, shape).astype(np.float32)).to(dtype).to(device)
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(ss))
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    chunk = 1 << 26
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        flat[i:i + m].copy_(torch.randn(m, generator=g, device=device, dtype=torch.float32))
    return out


def random_subset(T: int, k: int, seed: int) -> np.ndarray:
    """k distinct positions of [0, T), ascending (a stand-in selected set)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 303])))
    return np.sort(rng.choice(T, size=k, replace=False)).astype(np.int32)


def adversarial_scores(kind: str, T: int, seed: int) -> np.ndarray:
    """Score vectors built to stress a top-k selection (ties, signed zeros, 1-ulp gaps)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 404])))
    if kind == "equal":
        return np.full(T, 1.5, dtype=np.float32)
    if kind == "few_values":          # many ties everywhere, including at any boundary
        return rng.integers(0, 4, size=T).astype(np.float32)
    if kind == "signed_zeros":        # +0.0 and -0.0 mixed with a few positives/negatives
        v = np.where(rng.random(T) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        idx = rng.choice(T, size=max(1, T // 8), replace=False)
        v[idx] = rng.standard_normal(len(idx)).astype(np.float32)
        return v
    if kind == "ulp":                 # values a few ulps apart around 1.0
        steps = rng.integers(-3, 4, size=T).astype(np.float32)
        return (np.float32(1.0) + steps * np.float32(2.0 ** -23)).astype(np.float32)
    if kind == "normal":
        return rng.standard_normal(T).astype(np.float32)
    if kind == "positive":
        return np.abs(rng.standard_normal(T)).astype(np.float32) * 100
    raise ValueError(kind)


def calibration_pair(n: int, d_src: int, L_t: int, d_t: int, r: int, seed: int, strong: int, noise: float = 0.05,
                     dtype=torch.float32, device="cpu"):
    """Paired calibration KV with a planted linear relation, for fitting the mapper.

    x [n, d_src]: N(0,1) times one U(0.5, 2) factor per channel (as ``x_src``);
    y [n, L_t d_t] = x Q diag(s) P^T + N(0, noise^2), with Q [d_src, r] orthonormal columns,
    P the stack of L_t independent [d_t, r] orthonormal blocks (one per layer, so every layer
    sees all r directions) and s_j = 1 for the first ``strong`` directions and 0.3 for the rest
    (a spectral step that separates the top ``strong`` directions of each layer).
    Drawn in float64 on the host, returned in ``dtype`` (y computed before rounding)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 505])))
    x = rng.standard_normal((n, d_src)) * rng.uniform(0.5, 2.0, d_src)[None, :]
    q = orthonormal_basis(rng, d_src, r)
    p = np.vstack([orthonormal_basis(rng, d_t, r) for _ in range(L_t)])
    s = np.where(np.arange(r) < strong, 1.0, 0.3)
    y = (x @ q) * s[None, :] @ p.T + noise * rng.standard_normal((n, L_t * d_t))
    cast = lambda a: torch.from_numpy(a.astype(np.float32)).to(dtype).to(device)
    return cast(x), cast(y)
