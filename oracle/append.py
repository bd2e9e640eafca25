"""Appending new K/V rows into a paged cache: the oracle's placement rule.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product package
never imports this module.

What is computed, and where the pages state it:

* The operation itself, writing new K/V tensors into the paged KV cache, is
  named in the docs index, section "flashinfer.page" > "Append new K/V tensors
  to Paged KV-Cache".
* Where token t of request b lives is the page walk of the paged cache
  (article "FlashInfer", section "Block-sparse cache representation"; docs
  index "KV-Cache Layout in FlashInfer" > "Page Table Layout"): page
  kv_indices[kv_indptr[b] + t // P], slot t % P, NHD page memory
  [page, slot, kv_head, head_dim].

Readings taken where the pages are silent:

* Each appended row names its request b and its position t in that request.
* The page table already describes the cache after the append, so the KV
  length L_b counts the appended tokens; the usual append puts request b's
  A_b new tokens at positions L_b - A_b .. L_b - 1 (``append_positions``).
* A row whose b is outside [0, B), whose t is outside [0, L_b), or whose page
  index t // P is not below the request's page count is not written; nothing
  but the named (page, slot) rows changes.
"""

from __future__ import annotations

import numpy as np


def append_positions(append_indptr, kv_indptr, last_page_len, page_size: int):
    """(batch index, position) of every appended row when request b's
    A_b = append_indptr[b+1] - append_indptr[b] new tokens are its last A_b
    tokens: row append_indptr[b] + i goes to position L_b - A_b + i."""
    B = len(kv_indptr) - 1
    nnz = int(append_indptr[B])
    batch = np.zeros(nnz, dtype=np.int32)
    pos = np.zeros(nnz, dtype=np.int32)
    for b in range(B):
        n_pages = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        L = (n_pages - 1) * page_size + int(last_page_len[b]) if n_pages > 0 else 0
        A = int(append_indptr[b + 1]) - int(append_indptr[b])
        if A > L:
            raise ValueError(f"request {b} appends {A} tokens but holds only {L}")
        for i in range(A):
            batch[int(append_indptr[b]) + i] = b
            pos[int(append_indptr[b]) + i] = L - A + i
    return batch, pos


def append_paged_kv(k_cache, v_cache, append_k, append_v, batch_indices, positions,
                    kv_indptr, kv_indices, last_page_len):
    """Copies of the pools k_cache / v_cache [num_pages, P, Hkv, D] with appended
    row n (append_k[n], append_v[n], each [Hkv, D]) written at the page and slot
    of position positions[n] of request batch_indices[n]. Values are copied as
    stored (bit patterns), so the placement is exact."""
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    P = k.shape[1]
    B = len(kv_indptr) - 1
    for n in range(len(batch_indices)):
        b, t = int(batch_indices[n]), int(positions[n])
        if not 0 <= b < B or t < 0:
            continue
        n_pages = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        if n_pages <= 0:
            continue
        L = (n_pages - 1) * P + int(last_page_len[b])
        if t >= L or t // P >= n_pages:
            continue
        page = int(kv_indices[int(kv_indptr[b]) + t // P])
        slot = t % P
        k[page, slot] = append_k[n]
        v[page, slot] = append_v[n]
    return k, v
