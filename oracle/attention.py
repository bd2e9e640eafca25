"""fp64 attention states over a paged KV cache: the oracle's arithmetic.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product package
never imports this module.

What is computed, and where the FlashInfer pages state it:

* Exact attention. For one query row q and the visible keys/values of one KV
  head, the output is softmax(scale * q k^T) v and the state carries the
  log-sum-exp of the scaled logits next to it. The pages describe the flash
  kernels as exact attention with a running maximum (article "FlashInfer",
  sections "Correctness and numerical behavior" and
  "Extreme-negative-logit correction"); exact attention *is* this definition,
  so the oracle writes the definition out with true max subtraction in fp64.
* Attention state and merge. Attention over part of the cache is an
  (output, log-sum-exp) pair; states of disjoint parts merge into the state of
  their union by rescaling with the log-sum-exp values, since the partial
  outputs cannot simply be averaged (article "FlashInfer", section
  "Attention states"; docs index "flashinfer.cascade" > "Merge Attention
  States").
* Fully masked rows. A row that sees no key has output 0 and log-sum-exp -inf,
  and no finite sentinel stands in for -inf (article "FlashInfer", section
  "Extreme-negative-logit correction").
* Paged cache. Keys and values live in fixed-size pages that need not be
  contiguous; a page table lists each request's pages (article "FlashInfer",
  section "Block-sparse cache representation"; docs index "KV-Cache Layout in
  FlashInfer" > "Page Table Layout", "Layout: NHD/HND").
* Cascade. A shared prefix is evaluated separately from each request's suffix
  and the two states are merged (article "FlashInfer", section
  "Attention states"; docs index "Cascade Attention"). Its plain definition is
  attention over the concatenated prefix + suffix tokens, which is what
  ``cascade_decode`` computes.

Readings taken where the pages are silent:

* The log-sum-exp is the natural log of sum exp(scale * q.k) over visible keys.
* GQA: query head h reads KV head h // G with G = num_qo_heads // num_kv_heads.
* The causal mask is aligned bottom-right: query i (0-based within a request
  of Q query tokens and L keys) sees key t iff t <= i + L - Q.
* Page table: request b owns pages kv_indices[kv_indptr[b]:kv_indptr[b+1]];
  its KV length is (n_b - 1) * page_size + last_page_len[b] when n_b > 0 and 0
  otherwise; token t lives in page kv_indices[kv_indptr[b] + t // P] at slot
  t % P. Page memory is NHD: [page, slot, kv_head, head_dim].
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# dtype decoding (exact): fp16/bf16 values arrive as uint16 bit patterns.
# ----------------------------------------------------------------------------
def decode_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored values to float64 exactly.

    ``dtype`` is "f16" or "bf16" (``x`` holds uint16 bit patterns), or "f32" /
    "f64" (``x`` holds floats). Every fp16 and bf16 value is exactly
    representable in float64, so this step adds no error.
    """
    if dtype == "f16":
        return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # a bf16 value is the upper 16 bits of the float32 with the same value
        u32 = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u32.view(np.float32).astype(np.float64)
    if dtype in ("f32", "f64"):
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# page-table walk
# ----------------------------------------------------------------------------
def request_kv_len(kv_indptr, last_page_len, b: int, page_size: int) -> int:
    """KV length of request b: (n_b - 1) * P + last_page_len[b], or 0 when n_b = 0."""
    n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
    if n == 0:
        return 0
    return (n - 1) * page_size + int(last_page_len[b])


def request_token_pages(kv_indptr, kv_indices, last_page_len, b: int, page_size: int):
    """(page id, slot) of each logical token t = 0 .. L_b - 1 of request b."""
    L = request_kv_len(kv_indptr, last_page_len, b, page_size)
    t = np.arange(L, dtype=np.int64)
    pages = np.asarray(kv_indices, dtype=np.int64)[int(kv_indptr[b]) + t // page_size]
    slots = t % page_size
    return pages, slots


def gather_request_kv(k_cache, v_cache, dtype: str, kv_indptr, kv_indices, last_page_len,
                      b: int, kv_head: int):
    """Keys and values [L_b, D] (float64) of request b for one KV head.

    ``k_cache`` / ``v_cache`` are NHD page pools [num_pages, P, Hkv, D].
    """
    page_size = k_cache.shape[1]
    pages, slots = request_token_pages(kv_indptr, kv_indices, last_page_len, b, page_size)
    k = decode_bits(k_cache[pages, slots, kv_head, :], dtype)
    v = decode_bits(v_cache[pages, slots, kv_head, :], dtype)
    return k, v


# ----------------------------------------------------------------------------
# the attention state of a set of query rows over one KV head
# ----------------------------------------------------------------------------
def attention_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
                    visible: np.ndarray | None = None):
    """State (O [R, D], LSE [R]) of rows q [R, D] over keys k [L, D], values v [L, D].

    ``visible`` [R, L] (bool) says which keys each row may see (None: all).
    For a row with a non-empty visible set A:
        s_t = scale * sum_d q_d k_{t,d},  m = max_A s,  w_t = exp(s_t - m),
        O = sum_A w_t v_t / sum_A w_t,     LSE = m + ln(sum_A w_t).
    A row with an empty visible set gets O = 0 and LSE = -inf.
    All arithmetic is float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R, D = q.shape
    L = k.shape[0]
    if visible is None:
        visible = np.ones((R, L), dtype=bool)
    O = np.zeros((R, v.shape[1] if v.ndim == 2 else D), dtype=np.float64)
    LSE = np.full((R,), NEG_INF, dtype=np.float64)
    if L == 0 or R == 0:
        return O, LSE
    s = (q @ k.T) * float(sm_scale)                      # [R, L] scaled logits
    nonempty = visible.any(axis=1)
    s_vis = np.where(visible, s, NEG_INF)                # masked logits are -inf
    m = np.where(nonempty, s_vis.max(axis=1), 0.0)       # row max over visible keys
    w = np.exp(s_vis - m[:, None])                       # exp(-inf) = 0 for masked keys
    l = w.sum(axis=1)
    O[nonempty] = (w[nonempty] @ v) / l[nonempty, None]
    LSE[nonempty] = m[nonempty] + np.log(l[nonempty])
    return O, LSE


def causal_visible(qo_len: int, kv_len: int) -> np.ndarray:
    """Bottom-right causal mask [Q, L]: query i sees key t iff t <= i + L - Q."""
    i = np.arange(qo_len)[:, None]
    t = np.arange(kv_len)[None, :]
    return t <= i + (kv_len - qo_len)


# ----------------------------------------------------------------------------
# operations
# ----------------------------------------------------------------------------
def single_decode(q, k, v, dtype: str, sm_scale: float):
    """One query token over a contiguous NHD cache.

    q [Hq, D], k / v [L, Hkv, D] (stored values, see ``decode_bits``).
    Returns O [Hq, D] and LSE [Hq] in float64.
    """
    qf = decode_bits(q, dtype)
    kf = decode_bits(k, dtype)
    vf = decode_bits(v, dtype)
    Hq = qf.shape[0]
    Hkv = kf.shape[1]
    G = Hq // Hkv
    O = np.zeros(qf.shape, dtype=np.float64)
    LSE = np.full((Hq,), NEG_INF)
    for g in range(Hkv):
        rows = slice(g * G, (g + 1) * G)
        O[rows], LSE[rows] = attention_state(qf[rows], kf[:, g, :], vf[:, g, :], sm_scale)
    return O, LSE


def batch_decode(q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, dtype: str,
                 sm_scale: float, requests=None):
    """One query token per request over a paged cache.

    q [B, Hq, D]; caches [num_pages, P, Hkv, D]. Returns O [B, Hq, D] and
    LSE [B, Hq] (float64). ``requests`` limits the work to a subset of b (the
    other rows stay O = 0, LSE = -inf) so that full-size workloads can be
    sampled.
    """
    qf = decode_bits(q, dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Hq, D), dtype=np.float64)
    LSE = np.full((B, Hq), NEG_INF)
    for b in (range(B) if requests is None else requests):
        for g in range(Hkv):
            k, v = gather_request_kv(k_cache, v_cache, dtype, kv_indptr, kv_indices,
                                     last_page_len, b, g)
            rows = slice(g * G, (g + 1) * G)
            O[b, rows], LSE[b, rows] = attention_state(qf[b, rows], k, v, sm_scale)
    return O, LSE


def batch_prefill(q, k_cache, v_cache, qo_indptr, kv_indptr, kv_indices, last_page_len,
                  dtype: str, sm_scale: float, causal: bool, requests=None, heads=None):
    """Many query tokens per request (ragged q) over a paged cache.

    q [sum_b Q_b, Hq, D] with request b's tokens at rows
    qo_indptr[b] .. qo_indptr[b+1]-1. With ``causal`` the mask is bottom-right
    aligned (``causal_visible``). Returns O [sum Q, Hq, D], LSE [sum Q, Hq]
    in float64. ``requests`` / ``heads`` restrict the work for sampling.
    """
    qf = decode_bits(q, dtype)
    N, Hq, D = qf.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    page_size = k_cache.shape[1]
    O = np.zeros((N, Hq, D), dtype=np.float64)
    LSE = np.full((N, Hq), NEG_INF)
    B = len(qo_indptr) - 1
    head_list = list(range(Hq)) if heads is None else list(heads)
    for b in (range(B) if requests is None else requests):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        Q = q1 - q0
        L = request_kv_len(kv_indptr, last_page_len, b, page_size)
        vis = causal_visible(Q, L) if causal else None
        kv_by_head = {}
        for h in head_list:
            g = h // G
            if g not in kv_by_head:
                kv_by_head[g] = gather_request_kv(k_cache, v_cache, dtype, kv_indptr,
                                                  kv_indices, last_page_len, b, g)
            k, v = kv_by_head[g]
            O[q0:q1, h], LSE[q0:q1, h] = attention_state(qf[q0:q1, h], k, v, sm_scale, vis)
    return O, LSE


def merge_states(v, s):
    """Merge K attention states per row.

    v [n, K, H, D], s [n, K, H] (natural-log LSE). For each (n, h):
        s* = max_k s_k;  if s* = -inf the result is (0, -inf);
        w_k = exp(s_k - s*);  O = sum_k w_k v_k / sum_k w_k;  LSE = s* + ln sum_k w_k.
    Returns (O [n, H, D], LSE [n, H]) in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    s_star = s.max(axis=1)                                  # [n, H]
    live = s_star > NEG_INF
    base = np.where(live, s_star, 0.0)
    w = np.exp(s - base[:, None, :])                        # exp(-inf) = 0
    wsum = w.sum(axis=1)                                    # [n, H]
    O = np.zeros(v.shape[:1] + v.shape[2:], dtype=np.float64)
    num = (w[..., None] * v).sum(axis=1)                    # [n, H, D]
    O[live] = num[live] / wsum[live][:, None]
    LSE = np.full(s_star.shape, NEG_INF)
    LSE[live] = s_star[live] + np.log(wsum[live])
    return O, LSE


def merge_state(va, sa, vb, sb):
    """Merge two states: (va [n,H,D], sa [n,H]) and (vb, sb) -> (O, LSE), float64."""
    v = np.stack([np.asarray(va, np.float64), np.asarray(vb, np.float64)], axis=1)
    s = np.stack([np.asarray(sa, np.float64), np.asarray(sb, np.float64)], axis=1)
    return merge_states(v, s)


def cascade_decode(q, k_cache, v_cache, prefix_indices, prefix_last_page_len,
                   suffix_indptr, suffix_indices, suffix_last_page_len, dtype: str,
                   sm_scale: float, requests=None):
    """Decode where every request sees one shared prefix followed by its own suffix.

    The plain definition: attention of q[b] over the concatenation of the
    prefix tokens (pages ``prefix_indices``, last page holding
    ``prefix_last_page_len`` tokens) and request b's suffix tokens (page table
    ``suffix_indptr`` / ``suffix_indices`` / ``suffix_last_page_len``).
    Returns O [B, Hq, D], LSE [B, Hq] in float64.
    """
    qf = decode_bits(q, dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    pre_indptr = np.array([0, len(prefix_indices)], dtype=np.int64)
    pre_lpl = np.array([prefix_last_page_len], dtype=np.int64)
    O = np.zeros((B, Hq, D), dtype=np.float64)
    LSE = np.full((B, Hq), NEG_INF)
    pre_kv = [gather_request_kv(k_cache, v_cache, dtype, pre_indptr, prefix_indices, pre_lpl, 0, g)
              for g in range(Hkv)]
    for b in (range(B) if requests is None else requests):
        for g in range(Hkv):
            ks, vs = gather_request_kv(k_cache, v_cache, dtype, suffix_indptr, suffix_indices,
                                       suffix_last_page_len, b, g)
            k = np.concatenate([pre_kv[g][0], ks], axis=0)
            v = np.concatenate([pre_kv[g][1], vs], axis=0)
            rows = slice(g * G, (g + 1) * G)
            O[b, rows], LSE[b, rows] = attention_state(qf[b, rows], k, v, sm_scale)
    return O, LSE
