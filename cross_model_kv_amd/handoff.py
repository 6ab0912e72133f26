"""One cross-model KV handoff on the GPU: buffers and the call order of the C ABI.

map_latent -> score_select -> reconstruct(complement rows) -> recompute_attn_layers over
chunks of target layers.  Selection runs before reconstruction because the score needs only
the latent; the selected rows are then left for the recomputation to write, so reconstruction
computes the complement only (the translated values it would write there are overwritten
before anything reads them).  Every layer recomputes from its own given input rows, so the
layers are independent and a chunk of them runs as one projection launch and one attention
launch (chunks sized so that their q rows stay within LAYER_WS_BYTES).  No arithmetic
happens here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import kvx
from .synth import ChainWeights, Inputs


LAYER_WS_BYTES = 1 << 30      # q rows of one chunk of layers


def layer_chunks(L: int, per_layer_bytes: int):
    """Chunks [(l0, n)] covering L layers: as few as keep n * per_layer_bytes <= LAYER_WS_BYTES,
    with sizes as equal as possible."""
    lc = max(1, min(L, LAYER_WS_BYTES // max(per_layer_bytes, 1)))
    n_chunks = -(-L // lc)
    sizes = [L // n_chunks + (1 if i < L % n_chunks else 0) for i in range(n_chunks)]
    return [(sum(sizes[:i]), n) for i, n in enumerate(sizes)]


class Handoff:
    def __init__(self, inp: Inputs, device="cuda", keep_all_outputs: bool = True):
        wl = inp.wl
        self.inp = inp
        self.wl = wl
        self.device = torch.device(device)
        dt = inp.x_src.dtype
        self.batch = kvx.Batch.for_budgets(inp.lengths, inp.pcts, self.device)
        N = self.batch.n_tokens
        # one-time preparations per model pair (not part of a handoff)
        self.op = kvx.score_prepare(inp.w_l, inp.u)
        self.rope = kvx.rope_table(wl.rope_base, wl.d_h, max(inp.lengths), self.device)
        # buffers
        self.z = torch.empty((N, wl.r), dtype=dt, device=self.device)
        self.scores = torch.empty(N, dtype=torch.float32, device=self.device)
        self.sel = torch.empty(max(self.batch.total_sel, 1), dtype=torch.int32, device=self.device)
        self.rest = torch.empty(max(self.batch.total_rest, 1), dtype=torch.int32, device=self.device)
        self.ws_map = torch.empty(max(kvx.map_latent_workspace(kvx._dtype(self.z), N, wl.d_src, wl.r), 16),
                                  dtype=torch.uint8, device=self.device)
        self.ws_score = torch.empty(max(kvx.score_select_workspace(kvx._dtype(self.z), wl.r, N), 16),
                                    dtype=torch.uint8, device=self.device)
        self.ws_attn = torch.empty(max(kvx.recompute_attn_workspace(kvx._dtype(self.z), self.batch, wl.D, wl.H_q,
                                                                    wl.H_kv, wl.d_h), 16),
                                   dtype=torch.uint8, device=self.device)
        if wl.paged:
            n_slots = inp.n_pages * wl.page_size
            self.cache = kvx.Cache.empty(wl.L_t, n_slots, wl.H_kv, wl.d_h, dt, self.device,
                                         page_table=inp.page_table, page_size=wl.page_size)
        else:
            self.cache = kvx.Cache.empty(wl.L_t, N, wl.H_kv, wl.d_h, dt, self.device)
        dti = kvx._dtype(self.z)
        per_layer = kvx.recompute_attn_layers_workspace(dti, self.batch, wl.D, wl.H_q, wl.H_kv, wl.d_h, 1)
        self.chunks = layer_chunks(wl.L_t, per_layer)
        lc = max(n for _, n in self.chunks)
        self.ws_layers_bytes = max(per_layer * lc, 16)
        self.ws_layers = None          # allocated on first use
        self.keep_all = keep_all_outputs
        n_out = wl.L_t if keep_all_outputs else lc
        k = max(self.batch.total_sel, 1)
        self.out = torch.empty((n_out, k, wl.H_q, wl.d_h), dtype=dt, device=self.device)
        self.lse = torch.empty((n_out, k, wl.H_q), dtype=torch.float32, device=self.device)

    # the four stages ------------------------------------------------------------------
    def map(self):
        kvx.map_latent(self.inp.x_src, self.inp.w_s, self.z, self.ws_map)

    def select(self):
        kvx.score_select(self.z, self.op, self.batch, self.inp.pcts, ws=self.ws_score,
                         out=(self.scores, self.sel, self.rest))

    def reconstruct(self, all_rows: bool = False):
        rows = None if all_rows else self.rest[:self.batch.total_rest]
        kvx.reconstruct(self.z, self.inp.w_l, self.wl.H_kv, self.wl.d_h, self.batch, self.cache, rows=rows)

    def recompute(self, layer: int):
        """One layer through the single-layer entry point (output slot 0 unless all are kept)."""
        wl = self.wl
        slot = layer if self.keep_all else 0
        kvx.recompute_attn(layer, self.inp.x_l[layer], self.inp.w_qkv[layer], wl.H_q, wl.H_kv, wl.d_h,
                           self.rope, self.batch, self.sel[:self.batch.total_sel], self.cache,
                           out=self.out[slot], lse=self.lse[slot], ws=self.ws_attn)

    def recompute_layers(self, l0: int, n: int):
        """Layers l0 .. l0 + n - 1 in one call (outputs at their layers, or slots 0 .. n - 1).  A
        chunk of one layer takes the single-layer entry point, whose workspace lets it split
        the last round of projection tiles and the keys of too few query blocks."""
        wl = self.wl
        if n == 1:
            slot = l0 if self.keep_all else 0
            kvx.recompute_attn(l0, self.inp.x_l[l0], self.inp.w_qkv[l0], wl.H_q, wl.H_kv, wl.d_h, self.rope,
                               self.batch, self.sel[:self.batch.total_sel], self.cache, out=self.out[slot],
                               lse=self.lse[slot], ws=self.ws_attn)
            return
        s0 = l0 if self.keep_all else 0
        if self.ws_layers is None:
            self.ws_layers = torch.empty(self.ws_layers_bytes, dtype=torch.uint8, device=self.device)
        kvx.recompute_attn_layers(l0, self.inp.x_l[l0:l0 + n], self.inp.w_qkv[l0:l0 + n], wl.H_q, wl.H_kv, wl.d_h,
                                  self.rope, self.batch, self.sel[:self.batch.total_sel], self.cache,
                                  out=self.out[s0:s0 + n], lse=self.lse[s0:s0 + n], ws=self.ws_layers)

    def run(self, all_rows: bool = False):
        self.map()
        self.select()
        self.reconstruct(all_rows)
        for l0, n in self.chunks:
            self.recompute_layers(l0, n)

    # views --------------------------------------------------------------------------
    @property
    def S(self) -> torch.Tensor:
        return self.sel[:self.batch.total_sel]

    @property
    def C(self) -> torch.Tensor:
        return self.rest[:self.batch.total_rest]


class ChainedHandoff(Handoff):
    """The handoff with the selected rows continuing through every target layer: after each
    layer's recomputed attention, its output projection, norms and gated MLP run on the same
    rows, and layer l+1 recomputes its Q/K/V from layer l's output rows (kvx_target_layer).
    Layer 0 starts from the target's input rows at the selected positions."""

    def __init__(self, inp: Inputs, cw: ChainWeights, device="cuda", keep_all_outputs: bool = True):
        super().__init__(inp, device, keep_all_outputs)
        wl = self.wl
        self.cw = cw
        k = max(self.batch.total_sel, 1)
        self.x = torch.empty((k, wl.D), dtype=inp.x_l.dtype, device=self.device)
        self.layers = [kvx.LayerWeights(cw.gamma_in[l], inp.w_qkv[l], cw.w_o[l], cw.gamma_post[l], cw.w_gate[l],
                                        cw.w_up[l], cw.w_down[l]) for l in range(wl.L_t)]
        need = kvx.target_layer_workspace(kvx._dtype(self.x), self.batch, wl.D, wl.F, wl.H_q, wl.H_kv, wl.d_h)
        self.ws_layer = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device)

    def start_rows(self):
        kvx.gather_rows(self.inp.x_l[0], self.batch, self.S, self.x)

    def chain_layer(self, layer: int):
        wl = self.wl
        slot = layer if self.keep_all else 0
        kvx.target_layer(layer, self.x, self.layers[layer], wl.F, wl.H_q, wl.H_kv, wl.d_h, wl.norm_eps, self.rope,
                         self.batch, self.S, self.cache, attn_out=self.out[slot], lse=self.lse[slot],
                         ws=self.ws_layer)

    def run(self, all_rows: bool = False):
        self.map()
        self.select()
        self.reconstruct(all_rows)
        self.start_rows()
        for l in range(self.wl.L_t):
            self.chain_layer(l)

    # first token --------------------------------------------------------------------
    def prepare_first_token(self):
        """Buffers of the first-token step: a one-row-per-request batch at the last prompt
        positions, the row buffer, logits and tokens."""
        wl, dev = self.wl, self.device
        if self.cw.w_lm is None:
            raise ValueError("workload has no vocabulary")
        lengths = self.batch.lengths
        self.last_batch = kvx.Batch(lengths, [1] * len(lengths), dev)
        self.last_sel = torch.tensor([t - 1 for t in lengths], dtype=torch.int32, device=dev)
        n = len(lengths)
        self.x_last = torch.empty((n, wl.D), dtype=self.x.dtype, device=dev)
        self.xn_last = torch.empty_like(self.x_last)
        self.logits = torch.empty((n, wl.vocab), dtype=self.x.dtype, device=dev)
        self.token = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
        dt = kvx._dtype(self.x)
        need = max(kvx.target_layer_workspace(dt, self.last_batch, wl.D, wl.F, wl.H_q, wl.H_kv, wl.d_h),
                   kvx.linear_workspace(dt, n, wl.vocab, wl.D))
        self.ws_last = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def first_token(self):
        """The last prompt position through every layer over the mixed cache, then the
        final norm, the vocabulary projection and the argmax."""
        wl = self.wl
        kvx.gather_rows(self.inp.x_l[0], self.last_batch, self.last_sel, self.x_last)
        for l in range(wl.L_t):
            kvx.target_layer(l, self.x_last, self.layers[l], wl.F, wl.H_q, wl.H_kv, wl.d_h, wl.norm_eps, self.rope,
                             self.last_batch, self.last_sel, self.cache, ws=self.ws_last)
        kvx.rmsnorm(self.x_last, self.cw.gamma_final, wl.norm_eps, y=self.xn_last)
        kvx.linear(self.xn_last, self.cw.w_lm, self.logits, self.ws_last)
        kvx.argmax(self.logits, self.token)
