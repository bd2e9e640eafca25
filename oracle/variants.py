"""Attention variants: sliding window, logit soft cap, attention sinks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product package
never imports this module.

What is computed, and where the pages state it:

* The article "FlashInfer" (section "Custom attention templates") lists
  sliding windows, attention sinks and logit soft caps among the choices a
  model makes around the query-key product, which FlashInfer's template
  specialises. It names them and gives no formula.
* Everything else (exact softmax attention, the attention state (O, LSE), the
  empty row giving O = 0 and LSE = -inf, the paged cache walk) is as in
  ``attention.py`` (article "FlashInfer", sections "Attention states",
  "Extreme-negative-logit correction", "Block-sparse cache representation").

Readings taken where the pages are silent:

* Sliding window, ``window_left`` = W (W < 0: no window). A query at absolute
  position p in its request's KV (prefill: p = i + L - Q for query token i of
  Q, with L keys; decode: p = L - 1) sees key t only if t >= p - W; with the
  causal mask it also needs t <= p, so it sees at most W + 1 keys.
* Logit soft cap, ``soft_cap`` = c (c <= 0: off). The scaled logit
  x = sm_scale * q.k of every key is replaced by c * tanh(x / c) before the
  mask and the softmax; masked keys stay excluded.
* Attention sink, ``sinks`` = sigma[h] per query head (None: none). A virtual
  key whose (already final) logit is sigma[h] and whose value is the zero
  vector joins every row's softmax:
      Z = exp(sigma) + sum_{t visible} exp(x_t),
      O = sum_t exp(x_t) v_t / Z,  LSE = ln Z.
  So a row that sees no key gets O = 0 and LSE = sigma; sigma = -inf is the
  same as no sink. The sink enters once per row, whatever the split of the
  keys: the state with the sink is the merge of the keys' state with the
  state (0, sigma).
"""

from __future__ import annotations

import numpy as np

from .attention import NEG_INF, decode_bits, gather_request_kv, request_kv_len


def capped_logits(x: np.ndarray, soft_cap: float) -> np.ndarray:
    """c * tanh(x / c) for soft_cap c > 0; x unchanged otherwise."""
    c = float(soft_cap)
    if c > 0.0:
        return c * np.tanh(np.asarray(x, dtype=np.float64) / c)
    return np.asarray(x, dtype=np.float64)


def window_visible(qo_len: int, kv_len: int, window_left: int, causal: bool) -> np.ndarray:
    """Mask [Q, L]: query i (position p = i + L - Q) sees key t iff
    t >= p - W (when W >= 0) and t <= p (when causal)."""
    i = np.arange(qo_len)[:, None]
    t = np.arange(kv_len)[None, :]
    p = i + (kv_len - qo_len)
    vis = np.ones((qo_len, kv_len), dtype=bool)
    if causal:
        vis &= t <= p
    if window_left >= 0:
        vis &= t >= p - int(window_left)
    return vis


def variant_state(q, k, v, sm_scale: float, visible=None, soft_cap: float = 0.0,
                  sink: float | None = None):
    """State (O [R, Dv], LSE [R]) of rows q [R, D] over keys k [L, D] / values v [L, Dv]
    with the soft cap and the sink of the module docstring, float64.

    ``visible`` [R, L] (bool, None: all). ``sink`` is one logit shared by the rows
    (they belong to one query head), or None.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R = q.shape[0]
    L = k.shape[0]
    Dv = v.shape[1] if v.ndim == 2 else q.shape[1]
    sig = NEG_INF if sink is None else float(sink)
    O = np.zeros((R, Dv), dtype=np.float64)
    LSE = np.full((R,), NEG_INF, dtype=np.float64)
    if R == 0:
        return O, LSE
    if visible is None:
        visible = np.ones((R, L), dtype=bool)
    x = capped_logits((q @ k.T) * float(sm_scale), soft_cap) if L > 0 else np.zeros((R, 0))
    x = np.where(visible, x, NEG_INF)                   # masked keys: -inf
    # the reference point of each row: the largest term, the sink included
    row_max = x.max(axis=1) if L > 0 else np.full((R,), NEG_INF)
    m = np.maximum(row_max, sig)
    live = m > NEG_INF
    mu = np.where(live, m, 0.0)
    w = np.exp(x - mu[:, None])                         # exp(-inf) = 0
    z = w.sum(axis=1) + np.exp(sig - mu)
    if L > 0:
        O[live] = (w[live] @ v) / z[live, None]
    LSE[live] = mu[live] + np.log(z[live])
    return O, LSE


def batch_decode_variant(q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, dtype: str,
                         sm_scale: float, window_left: int = -1, soft_cap: float = 0.0,
                         sinks=None, requests=None):
    """Paged batch decode (one query token per request, at position L_b - 1) with
    the variants. Shapes as ``attention.batch_decode``; ``sinks`` [Hq] or None."""
    qf = decode_bits(q, dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    P = k_cache.shape[1]
    O = np.zeros((B, Hq, D), dtype=np.float64)
    LSE = np.full((B, Hq), NEG_INF)
    for b in (range(B) if requests is None else requests):
        L = request_kv_len(kv_indptr, last_page_len, b, P)
        vis = window_visible(1, L, window_left, causal=True)
        for g in range(Hkv):
            k, v = gather_request_kv(k_cache, v_cache, dtype, kv_indptr, kv_indices,
                                     last_page_len, b, g)
            for h in range(g * G, (g + 1) * G):
                sink = None if sinks is None else float(sinks[h])
                o, s = variant_state(qf[b, h][None, :], k, v, sm_scale, vis, soft_cap, sink)
                O[b, h], LSE[b, h] = o[0], s[0]
    return O, LSE


def batch_prefill_variant(q, k_cache, v_cache, qo_indptr, kv_indptr, kv_indices, last_page_len,
                          dtype: str, sm_scale: float, causal: bool, window_left: int = -1,
                          soft_cap: float = 0.0, sinks=None, requests=None, heads=None):
    """Paged batch prefill with the variants. Shapes as ``attention.batch_prefill``."""
    qf = decode_bits(q, dtype)
    N, Hq, D = qf.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    P = k_cache.shape[1]
    O = np.zeros((N, Hq, D), dtype=np.float64)
    LSE = np.full((N, Hq), NEG_INF)
    B = len(qo_indptr) - 1
    head_list = list(range(Hq)) if heads is None else list(heads)
    for b in (range(B) if requests is None else requests):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        L = request_kv_len(kv_indptr, last_page_len, b, P)
        vis = window_visible(q1 - q0, L, window_left, causal)
        kv_by_head = {}
        for h in head_list:
            g = h // G
            if g not in kv_by_head:
                kv_by_head[g] = gather_request_kv(k_cache, v_cache, dtype, kv_indptr,
                                                  kv_indices, last_page_len, b, g)
            k, v = kv_by_head[g]
            sink = None if sinks is None else float(sinks[h])
            O[q0:q1, h], LSE[q0:q1, h] = variant_state(qf[q0:q1, h], k, v, sm_scale, vis,
                                                       soft_cap, sink)
    return O, LSE
