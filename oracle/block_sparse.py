"""Block-sparse attention: the oracle's definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product package
never imports this module.

What is computed, and where the pages state it:

* The operation is named in the docs index, "flashinfer.sparse" >
  "BlockSparseAttentionWrapper", and the article "FlashInfer" (section
  "Block-sparse cache representation") describes a cache organisation as a
  block-sparse structure over which exact attention runs.
* Exact attention and its state (output, log-sum-exp), with O = 0 and
  LSE = -inf for a row that sees nothing: ``attention_state`` in
  ``attention.py`` (article "FlashInfer", sections "Attention states" and
  "Extreme-negative-logit correction").

Readings taken where the pages are silent:

* The mask is a BSR matrix over blocks of R query tokens and C key tokens:
  query token i sees key t iff block t // C is listed for block row i // R;
  there is no causal mask. The last query / key block may be shorter.
* Q is [N_q, Hq, D], K and V are dense [N_kv, Hkv, D]; query head h reads KV
  head h // (Hq / Hkv).
"""

from __future__ import annotations

import numpy as np

from .attention import attention_state, decode_bits


def block_mask(bsr_indptr, bsr_indices, num_qo_tokens: int, num_kv_tokens: int, R: int,
               C: int) -> np.ndarray:
    """visible [N_q, N_kv]: query token i sees key t iff block t // C is in row i // R."""
    vis = np.zeros((num_qo_tokens, num_kv_tokens), dtype=bool)
    for i in range(len(bsr_indptr) - 1):
        r0, r1 = i * R, min((i + 1) * R, num_qo_tokens)
        for e in range(int(bsr_indptr[i]), int(bsr_indptr[i + 1])):
            j = int(bsr_indices[e])
            vis[r0:r1, j * C:min((j + 1) * C, num_kv_tokens)] = True
    return vis


def block_sparse_attention(q, k, v, dtype: str, bsr_indptr, bsr_indices, R: int, C: int,
                           sm_scale: float):
    """States (O [N_q, Hq, D], LSE [N_q, Hq]) of block-sparse attention, float64."""
    qf = decode_bits(q, dtype)
    kf = decode_bits(k, dtype)
    vf = decode_bits(v, dtype)
    Nq, Hq, D = qf.shape
    Nkv, Hkv = kf.shape[0], kf.shape[1]
    G = Hq // Hkv
    vis = block_mask(bsr_indptr, bsr_indices, Nq, Nkv, R, C)
    O = np.zeros((Nq, Hq, D))
    LSE = np.zeros((Nq, Hq))
    for h in range(Hq):
        g = h // G
        O[:, h], LSE[:, h] = attention_state(qf[:, h], kf[:, g], vf[:, g], sm_scale, visible=vis)
    return O, LSE
