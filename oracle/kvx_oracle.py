"""Plain float64 CPU oracle of the cross-model KV handoff.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the bench's CPU-baseline leg
are the only callers; the product path (the HIP library and its binding) never
imports, calls or runs anything here.  It shares no code with the HIP path.

What it follows, step by step (page titles as printed on the pages):

* "PANORAMA: Cross-Model KV Sharing via Contextual Recomputation", abstract:
  the mapper is factorized into one shared source projection, which turns each prompt
  position's source KV into a compact latent, and a layer-specific target
  reconstruction of each target layer's K/V from that latent; a small subset of
  important target positions is then recomputed so that it attends over the full KV
  cache the mapper produced.
* RaReCache abstract (the CacheReforge card and the arxivdaily page): each token is
  scored by the energy of its mapped KV in output directions that the calibration
  data supports weakly, and a fixed share of positions (30% or 40%) is recomputed.

Readings taken where the pages are silent (each stated where it is used):
linear bias-free mapper; calibration subspace given as an orthonormal basis per
layer, with weak support by the calibration data read as lying outside its span; score = sum over target
layers of the squared residual of the concatenated [K | V] vector; budget
k = ceil(pct * T / 100); ties go to the lower position; rotate-half RoPE with base
10000 applied only to recomputed q and k at their true positions; all selected K/V
of a layer are written before any selected query attends; inclusive causal mask,
scale 1/sqrt(d_h), KV head = h // (H_q / H_kv).

Target layer chaining (the selected rows continuing through the rest of each target
layer, so that layer l+1's recomputed rows come from layer l's output): the pages name
the model pairs (Qwen3 and Llama targets) but not their blocks; the reading here is the
plain pre-norm decoder layer those families share - RMS normalisation with a per-channel
gain, the recomputed attention, an output projection and a residual add, a second RMS
normalisation, a SiLU-gated MLP and a second residual add - with no norm on q or k.

Variants (unranked on the pages' list of next steps, each its own function): the score as a share
of the token's energy, the keys of a mapper without rotary phase, QK-norm on the recomputed q and
k, the score taken directly from a stored cache layer by layer, per-layer selection sets, and
selection of whole pages of positions.

Fitting (before the path): the mapper is fitted in closed form to paired calibration KV of the
two models - reduced-rank ridge regression, the rank-r least-squares map from source KV to the
target KV of all layers, factored into the shared projection and the per-layer reconstructions -
and each layer's calibration subspace is the span of the top left singular vectors of the mapped
calibration KV.

Every function takes float64 numpy arrays (exact upcasts of the stored values) and
computes its result by its plain definition.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np


# ------------------------------------------------------------------------------------
# budget
# ------------------------------------------------------------------------------------

def budget(T: int, pct: int) -> int:
    """Number of positions to recompute: ceil(pct * T / 100) in integer arithmetic.

    RaReCache abstract: a fixed share of the positions (30%, also 40%) is recomputed.
    The count is rounded up so the budget is never under-spent.
    """
    if not (0 <= pct <= 100) or T < 0:
        raise ValueError("budget: need 0 <= pct <= 100 and T >= 0")
    return (pct * T + 99) // 100


# ------------------------------------------------------------------------------------
# mapper: shared source projection, then layer-specific reconstruction
# ------------------------------------------------------------------------------------

def map_latent(x_src: np.ndarray, w_s: np.ndarray) -> np.ndarray:
    """Shared source projection (PANORAMA abstract): z_t = W_s x_t for every position.

    x_src [N, d_src] (source K and V of all source layers concatenated per position),
    w_s [r, d_src] stored output-major.  Returns the latent Z [N, r].
    """
    return x_src @ w_s.T


def reconstruct(z: np.ndarray, w_l: np.ndarray, H_kv: int, d_h: int):
    """Layer-specific target reconstruction (PANORAMA abstract): y_{t,l} = W_l z_t.

    w_l [L_t, d_t, r] stored output-major; the first H_kv*d_h outputs of a layer are its
    K heads and the rest its V heads, head-major.  Returns the translated cache
    K, V [L_t, N, H_kv, d_h] and the mapped vectors Y [L_t, N, d_t].
    """
    L = w_l.shape[0]
    N = z.shape[0]
    Y = np.stack([z @ w_l[l].T for l in range(L)])
    K = Y[:, :, :H_kv * d_h].reshape(L, N, H_kv, d_h)
    V = Y[:, :, H_kv * d_h:].reshape(L, N, H_kv, d_h)
    return K, V, Y


def reconstruct_rotated(z: np.ndarray, w_l: np.ndarray, H_kv: int, d_h: int, pos: np.ndarray,
                        base: float):
    """The reconstruction for a mapper whose keys carry no rotary phase (the other reading of
    whether translated K is cache-ready; the pages do not say): every translated key head is
    rotated at its own position, as recomputed keys are, and V is left as it is.
    pos [N] is each row's position in its request.  Returns K, V [L_t, N, H_kv, d_h], Y."""
    K, V, Y = reconstruct(z, w_l, H_kv, d_h)
    return rope(K, np.asarray(pos)[None, :, None], base), V, Y


# ------------------------------------------------------------------------------------
# rank-disagreement score and top-budget selection
# ------------------------------------------------------------------------------------

def rank_disagreement(Y: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Score of every position (RaReCache abstract: the rank-disagreement score).

    The energy of a token's mapped KV in directions the calibration data supports
    weakly, read as: the squared norm of the part of y_{t,l} outside span(U_l), summed
    over the target layers.  Y [L_t, N, d_t], u [L_t, d_t, c] with orthonormal columns.
    The residual is formed explicitly: R = Y - (Y U) U^T.
    """
    L, N, _ = Y.shape
    s = np.zeros(N)
    for l in range(L):
        proj = (Y[l] @ u[l]) @ u[l].T
        res = Y[l] - proj
        s += np.sum(res * res, axis=1)
    return s


def rank_disagreement_normalized(Y: np.ndarray, u: np.ndarray) -> np.ndarray:
    """The score as a share instead of an energy (an unranked variant of the RaReCache abstract's
    score; the pages do not say which): the energy of a token's mapped KV outside the calibration
    subspaces divided by the energy of all of its mapped KV, both summed over the target layers,
    so the score lies in [0, 1] and does not grow with the size of the vectors.  A token whose
    mapped KV is zero in every layer scores 0.  Y [L_t, N, d_t], u [L_t, d_t, c]."""
    outside = rank_disagreement(Y, u)
    total = np.sum(Y * Y, axis=(0, 2))
    out = np.zeros_like(outside)
    nz = total > 0
    out[nz] = outside[nz] / total[nz]
    return out


def layer_disagreement(K: np.ndarray, V: np.ndarray, u: np.ndarray) -> np.ndarray:
    """The rank-disagreement energy scored directly from a stored target cache, layer by layer
    (an unranked variant of the RaReCache abstract's score, for a mapper that is not linear, whose
    cache has no latent form): for layer l and position t, the squared norm of the part of the
    stored vector y = [K heads | V heads] (head-major, the order reconstruct splits) outside
    span(U_l).  K, V [L_t, T, H_kv, d_h] as stored, u [L_t, d_t, c] with orthonormal columns.
    Returns E [L_t, T]; its sum over the layers is the summed score of those stored values."""
    L, T = K.shape[0], K.shape[1]
    E = np.zeros((L, T))
    for l in range(L):
        y = np.concatenate([K[l].reshape(T, -1), V[l].reshape(T, -1)], axis=1)
        res = y - (y @ u[l]) @ u[l].T
        E[l] = np.sum(res * res, axis=1)
    return E


def select_per_layer(E: np.ndarray, k: int):
    """Per-layer selection sets (an unranked variant): every layer takes its own k positions of
    largest energy E[l], with select's rule for ties.  Returns S [L_t, k] and C [L_t, T - k],
    each row ascending."""
    sets = [select(E[l], k) for l in range(E.shape[0])]
    T = E.shape[1]
    S = np.array([s for s, _ in sets], dtype=np.int64).reshape(E.shape[0], k)
    C = np.array([c for _, c in sets], dtype=np.int64).reshape(E.shape[0], T - k)
    return S, C


def select(s: np.ndarray, k: int):
    """The k positions with the largest score; ties go to the lower position.

    Sort by the key (-s_t, t) and take the first k.  Returns (S, C): the selected set and
    its complement, both ascending.  -0.0 and +0.0 compare equal here, as numbers.
    """
    T = s.shape[0]
    if not (0 <= k <= T):
        raise ValueError("select: need 0 <= k <= T")
    order = np.lexsort((np.arange(T), -s))
    S = np.sort(order[:k]).astype(np.int64)
    C = np.sort(order[k:]).astype(np.int64)
    return S, C


# ------------------------------------------------------------------------------------
# contextual recomputation of the selected positions
# ------------------------------------------------------------------------------------

def page_scores(s: np.ndarray, page_size: int) -> np.ndarray:
    """Page-granular scoring (an unranked variant, after the block-rounded repair sets of the PatchKV
    abstract on the CacheReforge card): a request's positions fall into pages of page_size
    consecutive positions, page j holding [j * page_size, min((j + 1) * page_size, T)) (the last
    page may be short); a page's score is the sum of its positions' scores."""
    T = s.shape[0]
    n_pages = -(-T // page_size)
    return np.array([np.sum(s[j * page_size:min((j + 1) * page_size, T)]) for j in range(n_pages)])


def select_pages(ps: np.ndarray, T: int, page_size: int, k_pages: int):
    """The k_pages pages of largest page score (select's rule: ties to the lower page), recomputed
    whole.  Returns (S, C, P): the selected positions and their complement (ascending, inside
    [0, T)) and the selected pages (ascending).  |S| is k_pages * page_size less the shortfall of
    the last page when that page is selected."""
    P, _ = select(ps, k_pages)
    chosen = np.zeros(T, dtype=bool)
    for j in P:
        chosen[j * page_size:min((j + 1) * page_size, T)] = True
    t = np.arange(T)
    return t[chosen].astype(np.int64), t[~chosen].astype(np.int64), P


def rope_angles(pos: np.ndarray, d_h: int, base: float) -> np.ndarray:
    """Angles pos * base**(-2j/d_h) for j < d_h/2, in float64; shape pos.shape + (d_h/2,)."""
    j = np.arange(d_h // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / d_h)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half rotary embedding at positions ``pos``.

    x [..., d_h] with ``pos`` broadcast over the leading axes; pair (j, j + d_h/2) is
    rotated by the angle of frequency j.
    """
    d_h = x.shape[-1]
    half = d_h // 2
    ang = rope_angles(pos, d_h, base)
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def recompute_qkv(x_rows: np.ndarray, w_qkv: np.ndarray, pos: np.ndarray,
                  H_q: int, H_kv: int, d_h: int, base: float):
    """Target Q/K/V of the selected positions (PANORAMA abstract, contextual recompute).

    x_rows [k, D] are the target layer's hidden inputs at the selected positions,
    w_qkv [(H_q + 2 H_kv) d_h, D] stored output-major with rows [Q heads | K heads |
    V heads].  q and k are rotated at their true positions; v is not.
    """
    qkv = x_rows @ w_qkv.T
    n = x_rows.shape[0]
    q = qkv[:, :H_q * d_h].reshape(n, H_q, d_h)
    k = qkv[:, H_q * d_h:(H_q + H_kv) * d_h].reshape(n, H_kv, d_h)
    v = qkv[:, (H_q + H_kv) * d_h:].reshape(n, H_kv, d_h)
    pos = np.asarray(pos)
    q = rope(q, pos[:, None], base)
    k = rope(k, pos[:, None], base)
    return q, k, v


def recompute_qkv_qknorm(x_rows: np.ndarray, w_qkv: np.ndarray, pos: np.ndarray, H_q: int, H_kv: int,
                         d_h: int, base: float, q_gain: np.ndarray, k_gain: np.ndarray, eps: float):
    """recompute_qkv for a target whose layers normalise q and k per head before the rotation
    (QK-norm, an unranked variant: one of the target families the pages name uses it, the pages
    do not describe the block): every q head and every k head is RMS-normalised over its d_h
    channels with its own per-channel gain (q_gain, k_gain [d_h], shared by the heads of the
    layer), then rotated at its true position; v is left as it is."""
    qkv = x_rows @ w_qkv.T
    n = x_rows.shape[0]
    q = qkv[:, :H_q * d_h].reshape(n, H_q, d_h)
    k = qkv[:, H_q * d_h:(H_q + H_kv) * d_h].reshape(n, H_kv, d_h)
    v = qkv[:, (H_q + H_kv) * d_h:].reshape(n, H_kv, d_h)
    pos = np.asarray(pos)
    q = rope(rmsnorm(q, q_gain, eps), pos[:, None], base)
    k = rope(rmsnorm(k, k_gain, eps), pos[:, None], base)
    return q, k, v


def scatter(K: np.ndarray, V: np.ndarray, S: np.ndarray, k_new: np.ndarray, v_new: np.ndarray):
    """Mixed cache: recomputed K/V replace the translated ones at the selected positions."""
    K = K.copy()
    V = V.copy()
    K[S] = k_new
    V[S] = v_new
    return K, V


def sparse_causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, pos: np.ndarray):
    """Causal attention of the selected queries over the full (mixed) cache.

    q [k, H_q, d_h] at positions ``pos``; K, V [T, H_kv, d_h].  Query (i, h) attends to
    keys j <= pos[i] of KV head h // (H_q / H_kv) with weights
    softmax(q . K_j / sqrt(d_h)).  Returns O [k, H_q, d_h] and the natural-log
    log-sum-exp of the scaled logits, LSE [k, H_q].
    """
    n, H_q, d_h = q.shape
    H_kv = K.shape[1]
    g = H_q // H_kv
    O = np.zeros((n, H_q, d_h))
    lse = np.zeros((n, H_q))
    scale = 1.0 / math.sqrt(d_h)
    for i in range(n):
        p = int(pos[i])
        for h in range(H_q):
            kv = h // g
            logits = (K[:p + 1, kv, :] @ q[i, h]) * scale
            m = logits.max()
            e = np.exp(logits - m)
            tot = e.sum()
            w = e / tot
            assert abs(w.sum() - 1.0) <= 1e-12
            O[i, h] = w @ V[:p + 1, kv, :]
            lse[i, h] = m + math.log(tot)
    return O, lse


# ------------------------------------------------------------------------------------
# the whole handoff, one request at a time
# ------------------------------------------------------------------------------------

def handoff_request(x_src: np.ndarray, w_s: np.ndarray, w_l: np.ndarray, u: np.ndarray,
                    x_l: np.ndarray, w_qkv: np.ndarray, pct: int, H_q: int, H_kv: int,
                    d_h: int, base: float = 10000.0) -> Dict[str, np.ndarray]:
    """One request: map -> score -> select -> recompute + scatter -> attend, per layer.

    x_src [T, d_src], x_l [L_t, T, D], w_qkv [L_t, n_qkv, D].  Returns the latent Z, the
    translated cache (K_tr, V_tr), the scores s, the sets S and C, the mixed cache
    (K, V) [L_t, T, H_kv, d_h] and the attention outputs O [L_t, k, H_q, d_h], LSE.
    """
    T = x_src.shape[0]
    L = w_l.shape[0]
    z = map_latent(x_src, w_s)
    K_tr, V_tr, Y = reconstruct(z, w_l, H_kv, d_h)
    s = rank_disagreement(Y, u)
    k = budget(T, pct)
    S, C = select(s, k)
    K = K_tr.copy()
    V = V_tr.copy()
    O = np.zeros((L, k, H_q, d_h))
    LSE = np.zeros((L, k, H_q))
    for l in range(L):
        q, kk, vv = recompute_qkv(x_l[l][S], w_qkv[l], S, H_q, H_kv, d_h, base)
        K[l], V[l] = scatter(K[l], V[l], S, kk, vv)
        O[l], LSE[l] = sparse_causal_attention(q, K[l], V[l], S)
    return dict(z=z, K_tr=K_tr, V_tr=V_tr, s=s, S=S, C=C, K=K, V=V, O=O, LSE=LSE)


def handoff_request_layer_sets(x_src: np.ndarray, w_s: np.ndarray, w_l: np.ndarray, u: np.ndarray,
                               x_l: np.ndarray, w_qkv: np.ndarray, pct: int, H_q: int, H_kv: int,
                               d_h: int, base: float = 10000.0) -> Dict[str, np.ndarray]:
    """One request with per-layer selection sets, scored directly from the stored cache (the two
    unranked variants together): map, translate every position of every layer, score each layer
    from its own stored K/V (layer_disagreement), and let layer l recompute its own top-k set S_l,
    scatter there and attend with the queries of S_l.  The budget k is the same for every layer.
    Returns z, the translated cache (K_tr, V_tr), E [L_t, T], S [L_t, k], C [L_t, T - k], the
    mixed cache (K, V) and O [L_t, k, H_q, d_h], LSE [L_t, k, H_q] (row i of layer l is S[l][i])."""
    T = x_src.shape[0]
    L = w_l.shape[0]
    z = map_latent(x_src, w_s)
    K_tr, V_tr, _ = reconstruct(z, w_l, H_kv, d_h)
    E = layer_disagreement(K_tr, V_tr, u)
    k = budget(T, pct)
    S, C = select_per_layer(E, k)
    K = K_tr.copy()
    V = V_tr.copy()
    O = np.zeros((L, k, H_q, d_h))
    LSE = np.zeros((L, k, H_q))
    for l in range(L):
        q, kk, vv = recompute_qkv(x_l[l][S[l]], w_qkv[l], S[l], H_q, H_kv, d_h, base)
        K[l], V[l] = scatter(K[l], V[l], S[l], kk, vv)
        if k:
            O[l], LSE[l] = sparse_causal_attention(q, K[l], V[l], S[l])
    return dict(z=z, K_tr=K_tr, V_tr=V_tr, E=E, S=S, C=C, K=K, V=V, O=O, LSE=LSE)


# ------------------------------------------------------------------------------------
# target layer chaining: the rest of the target layer on the selected rows
# ------------------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square normalisation of every row, then a per-channel gain:
    y = x / sqrt(mean_j(x_j^2) + eps) * gamma."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def swiglu_mlp(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """SiLU-gated MLP: W_down (silu(W_gate x) * (W_up x)).  w_gate, w_up [F, D] and
    w_down [D, F], stored output-major."""
    return (silu(x @ w_gate.T) * (x @ w_up.T)) @ w_down.T


def target_layer(x_rows: np.ndarray, S: np.ndarray, K: np.ndarray, V: np.ndarray, w: Dict[str, np.ndarray],
                 H_q: int, H_kv: int, d_h: int, base: float, eps: float):
    """One pre-norm decoder layer of the target, run on the selected rows only.

    x_rows [k, D] is the residual stream at the selected positions S (ascending), K, V
    [T, H_kv, d_h] the layer's translated cache.  w holds gamma_in [D], w_qkv, w_o
    [D, H_q d_h], gamma_post [D], w_gate, w_up [F, D], w_down [D, F].  Steps:
    h = rmsnorm(x); q, k, v from h (rotated at the true positions); all k, v written
    into the cache; attention of the selected queries over the mixed cache;
    x1 = x + O W_o^T; x2 = x1 + mlp(rmsnorm(x1)).  Returns x2, the mixed cache K, V,
    the attention output O [k, H_q, d_h] and its LSE.
    """
    n = x_rows.shape[0]
    h = rmsnorm(x_rows, w["gamma_in"], eps)
    q, kk, vv = recompute_qkv(h, w["w_qkv"], S, H_q, H_kv, d_h, base)
    K, V = scatter(K, V, S, kk, vv)
    O, lse = sparse_causal_attention(q, K, V, S)
    x1 = x_rows + O.reshape(n, H_q * d_h) @ w["w_o"].T
    x2 = x1 + swiglu_mlp(rmsnorm(x1, w["gamma_post"], eps), w["w_gate"], w["w_up"], w["w_down"])
    return x2, K, V, O, lse


def chained_layers(x0_rows: np.ndarray, S: np.ndarray, K_tr: np.ndarray, V_tr: np.ndarray,
                   layers: Sequence[Dict[str, np.ndarray]], H_q: int, H_kv: int, d_h: int,
                   base: float = 10000.0, eps: float = 1e-6) -> Dict[str, np.ndarray]:
    """The selected rows through every target layer in turn: layer l+1 takes layer l's
    output rows.  x0_rows [k, D] are the target's input rows at the selected positions,
    K_tr, V_tr [L_t, T, H_kv, d_h] the translated cache.  Returns the final rows X, the
    mixed cache K, V, and O, LSE per layer."""
    L = len(layers)
    x = x0_rows
    K = K_tr.copy()
    V = V_tr.copy()
    n = x0_rows.shape[0]
    O = np.zeros((L, n, H_q, d_h))
    LSE = np.zeros((L, n, H_q))
    X = np.zeros((L + 1,) + x0_rows.shape)
    X[0] = x
    for l in range(L):
        x, K[l], V[l], O[l], LSE[l] = target_layer(x, S, K[l], V[l], layers[l], H_q, H_kv, d_h, base, eps)
        X[l + 1] = x
    return dict(X=X, K=K, V=V, O=O, LSE=LSE)


# ------------------------------------------------------------------------------------
# first token after the handoff
# ------------------------------------------------------------------------------------

def lm_head(x: np.ndarray, gamma: np.ndarray, w_lm: np.ndarray, eps: float) -> np.ndarray:
    """Logits of rows x: the final RMS normalisation, then the vocabulary projection
    w_lm [V, D] (output-major)."""
    return rmsnorm(x, gamma, eps) @ w_lm.T


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Index of the largest logit of every row; ties go to the lowest index."""
    return np.argmax(logits, axis=-1)


def first_token(x0_last: np.ndarray, p_last: int, K: np.ndarray, V: np.ndarray,
                layers: Sequence[Dict[str, np.ndarray]], gamma_final: np.ndarray, w_lm: np.ndarray,
                H_q: int, H_kv: int, d_h: int, base: float = 10000.0, eps: float = 1e-6):
    """The first target token after a handoff (the time-to-first-token step).

    The last prompt position p_last runs through every target layer as a single recomputed
    row over the layer's mixed cache K[l], V[l] [T, H_kv, d_h] (its own k, v recomputed and
    written there), starting from the target's input row x0_last [D]; its final row is
    normalised and projected onto the vocabulary.  Returns the logits [V], the token (the
    argmax, ties to the lowest index) and the updated cache.
    """
    S = np.array([p_last])
    x = x0_last[None, :]
    K = K.copy()
    V = V.copy()
    for l, w in enumerate(layers):
        x, K[l], V[l], _, _ = target_layer(x, S, K[l], V[l], w, H_q, H_kv, d_h, base, eps)
    logits = lm_head(x, gamma_final, w_lm, eps)[0]
    return logits, int(argmax_lowest(logits)), K, V


# ------------------------------------------------------------------------------------
# fitting the mapper and the calibration subspaces from paired calibration data
# ------------------------------------------------------------------------------------

def fit_mapper(x: np.ndarray, y: np.ndarray, r: int, lam: float, L: int):
    """Closed-form least-squares fit of the factorized mapper (PANORAMA abstract: the mapper
    is factorized into one shared source projection and a layer-specific reconstruction, and is
    first fitted for translation alone; RaReCache abstract: closed-form linear maps translate
    KV between models).

    Read here as reduced-rank ridge regression: the rank-r linear map B_r from source KV to the
    target KV of all layers that minimises ||x B_r - y||^2 among maps in the row space of the
    ridge solution.  x [n, d_src] source KV of n calibration positions; y [n, L * d_t] the
    target K|V of the same positions, layer-major (layer l is columns l*d_t .. (l+1)*d_t).
    Steps: the ridge least-squares map B = argmin ||x B - y||^2 + lam ||B||^2 (solved as an
    ordinary least-squares problem on x stacked over sqrt(lam) I); the fitted values x B; their
    top-r right singular vectors V [L * d_t, r]; then B_r = B V V^T, factored as the shared
    projection w_s = (B V)^T [r, d_src] and the per-layer reconstructions w_l = V's rows of
    layer l [L, d_t, r].  The factorization is unique up to a rotation of the latent.
    """
    n, d = x.shape
    m = y.shape[1]
    xa = np.vstack([x, math.sqrt(lam) * np.eye(d)])
    ya = np.vstack([y, np.zeros((d, m))])
    B = np.linalg.lstsq(xa, ya, rcond=None)[0]
    _, _, vt = np.linalg.svd(x @ B, full_matrices=False)
    V = vt[:r].T
    w_s = (B @ V).T
    w_l = V.reshape(L, m // L, r)
    return w_s, w_l


def calibration_basis(z: np.ndarray, w_l: np.ndarray, c: int) -> np.ndarray:
    """Calibration subspace of every target layer (RaReCache abstract: output directions the
    calibration data supports): U_l = the top-c left singular vectors of the mapped calibration
    KV, the d_t x n matrix whose column t is w_l z_t.  z [n, r] latents of the calibration
    positions, w_l [L, d_t, r].  Returns u [L, d_t, c] (orthonormal columns)."""
    L, d_t, _ = w_l.shape
    u = np.zeros((L, d_t, c))
    for l in range(L):
        left, _, _ = np.linalg.svd(w_l[l] @ z.T, full_matrices=False)
        u[l] = left[:, :c]
    return u


def score_gap(s: np.ndarray, k: int) -> float:
    """Relative gap between the k-th and (k+1)-th largest scores (inf when k is 0 or T)."""
    T = s.shape[0]
    if k == 0 or k == T:
        return math.inf
    srt = np.sort(s)[::-1]
    tau = srt[k - 1]
    return float((srt[k - 1] - srt[k]) / abs(tau)) if tau != 0 else float(srt[k - 1] - srt[k])
