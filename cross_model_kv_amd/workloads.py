"""Workload shapes for the cross-model KV handoff.

Each workload fixes the source-KV shape, the latent rank of the factorized mapper,
the target attention shape, the calibration rank and the recompute budget.  The
shapes follow the model pairs that the PANORAMA abstract (Qwen3 8B to 32B at 16K
tokens) and the RaReCache abstract (Qwen3-0.6B to 14B at a 30% budget, Llama3-8B
to 70B at 40%) report on; the tiny one is a small fp32 case for exact checks.  The MLP
widths F and vocabulary sizes of the chained variant are those of the named target models'
public configurations (Qwen3-14B F 17408, Qwen3-32B F 25600, both 151936 tokens; Llama-3-70B F 28672,
128256 tokens); the pages do not print them.

This module only holds sizes.  It does no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16": storage type of activations and weights
    T: int                     # positions per request (ignored when lengths are drawn)
    L_s: int                   # source layers
    H_s: int                   # source KV heads
    d_hs: int                  # source head dim
    r: int                     # latent rank
    L_t: int                   # target layers
    H_q: int                   # target query heads
    H_kv: int                  # target KV heads
    d_h: int                   # target head dim
    D: int                     # target hidden size
    c: int                     # calibration rank per layer
    pct: int                   # recompute budget in percent
    rope_base: float = 10000.0
    n_req: int = 1
    # batched serving: lengths drawn log-uniform in [t_min, t_max], budgets from pct_choices
    t_min: int = 0
    t_max: int = 0
    pct_choices: Tuple[int, ...] = ()
    paged: bool = False
    page_size: int = 16
    # chained target layers (MLP after the attention): intermediate width of the gated MLP
    # and the RMS-norm epsilon; F = 0 means the workload has no chained variant
    F: int = 0
    norm_eps: float = 1e-6
    # first-token step: vocabulary size of the target (0: no first-token variant)
    vocab: int = 0

    @property
    def d_src(self) -> int:
        return 2 * self.L_s * self.H_s * self.d_hs

    @property
    def d_t(self) -> int:
        return 2 * self.H_kv * self.d_h

    @property
    def g(self) -> int:
        return self.H_q // self.H_kv

    @property
    def n_qkv(self) -> int:
        return (self.H_q + 2 * self.H_kv) * self.d_h

    @property
    def batched(self) -> bool:
        return self.n_req > 1 or bool(self.pct_choices)

    def shrink(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY_F32 = Workload(
    name="tiny-fp32-T256", dtype="f32", T=256, L_s=4, H_s=2, d_hs=64, r=128,
    L_t=4, H_q=8, H_kv=2, d_h=64, D=512, c=64, pct=30)

QWEN_0P6B_14B = Workload(
    name="0.6B-to-14B-shape-T4096", dtype="bf16", T=4096, L_s=28, H_s=8, d_hs=128,
    r=1024, L_t=40, H_q=40, H_kv=8, d_h=128, D=5120, c=512, pct=30, F=17408, vocab=151936)

QWEN_8B_32B_16K = Workload(
    name="8B-to-32B-shape-T16384", dtype="bf16", T=16384, L_s=36, H_s=8, d_hs=128,
    r=1024, L_t=64, H_q=64, H_kv=8, d_h=128, D=5120, c=512, pct=30, F=25600, vocab=151936)

LLAMA_8B_70B = Workload(
    name="8B-to-70B-shape-T8192", dtype="bf16", T=8192, L_s=32, H_s=8, d_hs=128,
    r=1536, L_t=80, H_q=64, H_kv=8, d_h=128, D=8192, c=768, pct=40, F=28672, vocab=128256)

BATCHED_16 = Workload(
    name="batched-16req-paged16", dtype="bf16", T=0, L_s=36, H_s=8, d_hs=128,
    r=1024, L_t=64, H_q=64, H_kv=8, d_h=128, D=5120, c=512, pct=30,
    n_req=16, t_min=1024, t_max=16384, pct_choices=(20, 30, 40), paged=True, page_size=16, F=25600, vocab=151936)

ALL = {w.name: w for w in (TINY_F32, QWEN_0P6B_14B, QWEN_8B_32B_16K, LLAMA_8B_70B, BATCHED_16)}
