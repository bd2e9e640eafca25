"""Seeded synthetic workloads for paged-KV attention.

This module only draws inputs: request lengths, page tables and N(0,1) values
rounded to fp16 / bf16 bit patterns. It holds none of the attention
arithmetic, imports nothing from the HIP path or from the oracle, and serves
both sides: the same arrays feed the GPU library and the fp64 oracle.

Recipe (for every workload):
  * rng = numpy.random.default_rng(seed);
  * draw order: request lengths, then one permutation of the page pool, then
    q, then the K pool, then the V pool;
  * values are float32 standard normals rounded to the storage dtype with
    round-to-nearest-even (the returned arrays hold the uint16 bit patterns);
  * the page pool holds ceil(1.25 * pages needed) pages; request b takes the
    next n_b pages of the permutation, in request order;
  * lengths are uniform integers with both ends included;
  * pool pages no request uses, and slots past last_page_len in each request's
    last page, hold N(0,1) values, or NaN when ``canary=True`` (a read of any
    of them poisons the result).
The K / V pools are drawn in chunks so that multi-GB pools fit in host memory.
"""

from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

F16_NAN = np.uint16(0x7E00)
BF16_NAN = np.uint16(0x7FC0)
_CHUNK = 1 << 24


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array -> uint16 bit patterns of the nearest fp16 / bf16 (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
        out = rounded.astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            out[nan] = BF16_NAN
        return out
    raise ValueError(dtype)


def nan_bits(dtype: str) -> np.uint16:
    return F16_NAN if dtype == "f16" else BF16_NAN


def normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws rounded to ``dtype``, drawn in fixed-size chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = round_bits(rng.standard_normal(e - s, dtype=np.float32), dtype)
    return out.reshape(shape)


@dataclass
class PagedKV:
    """A paged KV cache plus page table (NHD pages [num_pages, P, Hkv, D])."""
    k_cache: np.ndarray
    v_cache: np.ndarray
    kv_indptr: np.ndarray        # int32 [B+1]
    kv_indices: np.ndarray       # int32 [nnz pages]
    last_page_len: np.ndarray    # int32 [B]
    page_size: int

    @property
    def kv_lens(self) -> np.ndarray:
        n = np.diff(self.kv_indptr.astype(np.int64))
        return np.where(n > 0, (n - 1) * self.page_size + self.last_page_len, 0).astype(np.int64)


@dataclass
class Workload:
    kind: str                    # "single_decode" | "decode" | "prefill" | "cascade"
    dtype: str                   # "f16" | "bf16"
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    sm_scale: float
    q: np.ndarray                # uint16 bits
    kv: PagedKV | None = None
    k: np.ndarray | None = None  # single decode: contiguous [L, Hkv, D]
    v: np.ndarray | None = None
    qo_indptr: np.ndarray | None = None
    causal: bool = False
    # cascade: shared prefix page list (+ last page length); suffix table is ``kv``
    prefix_indices: np.ndarray | None = None
    prefix_last_page_len: int = 0
    meta: dict = field(default_factory=dict)


def _page_counts(kv_lens, P):
    return np.array([(int(L) + P - 1) // P for L in kv_lens], dtype=np.int64)


def _last_page_len(kv_lens, P):
    return np.array([0 if L == 0 else int(L) - (int(L) + P - 1) // P * P + P for L in kv_lens],
                    dtype=np.int32)


def _fill_pool(rng, num_pages, P, Hkv, D, dtype):
    return normal_bits(rng, (num_pages, P, Hkv, D), dtype)


def _poison_unused(cache, used_pages, tail_slots, dtype):
    """NaN into unused pages and into (page, slot) tails past last_page_len."""
    nan = nan_bits(dtype)
    mask = np.ones(cache.shape[0], dtype=bool)
    mask[used_pages] = False
    cache[mask] = nan
    for page, first_free in tail_slots:
        cache[page, first_free:] = nan


def make_paged(rng, kv_lens, P, Hkv, D, dtype, q_shape, pool_factor=1.25, canary=False,
               extra_pages_front=0):
    """Draw a page pool for requests of ``kv_lens`` and q; returns (PagedKV, q, extra).

    ``extra_pages_front`` pages are taken from the permutation before the
    requests' pages (the cascade's shared prefix) and returned as ``extra``.
    """
    n = _page_counts(kv_lens, P)
    need = int(n.sum()) + extra_pages_front
    pool = max(1, math.ceil(pool_factor * need))
    perm = rng.permutation(pool).astype(np.int32)
    extra = perm[:extra_pages_front]
    indices = perm[extra_pages_front:need]
    indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(n)
    lpl = _last_page_len(kv_lens, P)
    q = normal_bits(rng, q_shape, dtype)
    k_cache = _fill_pool(rng, pool, P, Hkv, D, dtype)
    v_cache = _fill_pool(rng, pool, P, Hkv, D, dtype)
    kv = PagedKV(k_cache, v_cache, indptr, indices, lpl, P)
    return kv, q, extra


def canary_tails(kv: PagedKV, dtype: str, extra_pages=(), extra_last_len=None):
    """Poison unused pool pages and the slots past each last_page_len with NaN."""
    used = np.concatenate([kv.kv_indices.astype(np.int64), np.asarray(extra_pages, np.int64)])
    tails = []
    for b in range(len(kv.last_page_len)):
        p0, p1 = int(kv.kv_indptr[b]), int(kv.kv_indptr[b + 1])
        if p1 > p0 and kv.last_page_len[b] < kv.page_size:
            tails.append((int(kv.kv_indices[p1 - 1]), int(kv.last_page_len[b])))
    if len(extra_pages) and extra_last_len is not None and extra_last_len < kv.page_size:
        tails.append((int(extra_pages[-1]), int(extra_last_len)))
    for cache in (kv.k_cache, kv.v_cache):
        _poison_unused(cache, used, tails, dtype)


# ----------------------------------------------------------------------------
# the five workloads, at full size and at reduced sizes for quick parity tests
# ----------------------------------------------------------------------------
def single_decode(seed=173000, kv_len=1024, num_qo_heads=32, num_kv_heads=32, head_dim=128,
                  dtype="f16"):
    """One query token, contiguous NHD k / v [kv_len, Hkv, D]; draws q, then k, then v."""
    rng = np.random.default_rng(seed)
    q = normal_bits(rng, (num_qo_heads, head_dim), dtype)
    k = normal_bits(rng, (kv_len, num_kv_heads, head_dim), dtype)
    v = normal_bits(rng, (kv_len, num_kv_heads, head_dim), dtype)
    return Workload("single_decode", dtype, num_qo_heads, num_kv_heads, head_dim,
                    1.0 / math.sqrt(head_dim), q, k=k, v=v, meta={"seed": seed, "kv_len": kv_len})


def batch_decode(seed=173001, batch=64, kv_min=512, kv_max=4096, num_qo_heads=32,
                 num_kv_heads=8, head_dim=128, page_size=16, dtype="f16", canary=False,
                 kv_lens=None):
    """One query token per request over a paged cache with uniform random lengths."""
    rng = np.random.default_rng(seed)
    if kv_lens is None:
        kv_lens = rng.integers(kv_min, kv_max + 1, size=batch)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    kv, q, _ = make_paged(rng, kv_lens, page_size, num_kv_heads, head_dim, dtype,
                          (len(kv_lens), num_qo_heads, head_dim))
    if canary:
        canary_tails(kv, dtype)
    return Workload("decode", dtype, num_qo_heads, num_kv_heads, head_dim,
                    1.0 / math.sqrt(head_dim), q, kv=kv,
                    meta={"seed": seed, "kv_lens": kv_lens})


def batch_prefill(seed=173002, batch=16, qo_min=128, qo_max=1024, prefix_min=0,
                  prefix_max=2048, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                  page_size=16, dtype="bf16", causal=True, canary=False, qo_lens=None,
                  prefix_lens=None):
    """Ragged query tokens appended after a cached prefix; kv_len = prefix + qo_len."""
    rng = np.random.default_rng(seed)
    if qo_lens is None:
        qo_lens = rng.integers(qo_min, qo_max + 1, size=batch)
    if prefix_lens is None:
        prefix_lens = rng.integers(prefix_min, prefix_max + 1, size=len(qo_lens))
    qo_lens = np.asarray(qo_lens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    kv_lens = qo_lens + prefix_lens
    qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    kv, q, _ = make_paged(rng, kv_lens, page_size, num_kv_heads, head_dim, dtype,
                          (int(qo_lens.sum()), num_qo_heads, head_dim))
    if canary:
        canary_tails(kv, dtype)
    return Workload("prefill", dtype, num_qo_heads, num_kv_heads, head_dim,
                    1.0 / math.sqrt(head_dim), q, kv=kv, qo_indptr=qo_indptr, causal=causal,
                    meta={"seed": seed, "qo_lens": qo_lens, "kv_lens": kv_lens})


def cascade(seed=173003, batch=128, prefix_len=8192, suffix_min=64, suffix_max=1024,
            num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype="f16",
            canary=False, suffix_lens=None):
    """Decode requests sharing one prefix page list, each with its own suffix pages.

    Prefix and suffix pages come from one pool permutation: the prefix takes
    the first ceil(prefix_len / P) pages, then the suffixes in request order.
    """
    rng = np.random.default_rng(seed)
    if suffix_lens is None:
        suffix_lens = rng.integers(suffix_min, suffix_max + 1, size=batch)
    suffix_lens = np.asarray(suffix_lens, dtype=np.int64)
    n_prefix = (prefix_len + page_size - 1) // page_size
    kv, q, prefix_pages = make_paged(rng, suffix_lens, page_size, num_kv_heads, head_dim, dtype,
                                     (len(suffix_lens), num_qo_heads, head_dim),
                                     extra_pages_front=n_prefix)
    prefix_lpl = 0 if prefix_len == 0 else prefix_len - (n_prefix - 1) * page_size
    if canary:
        canary_tails(kv, dtype, prefix_pages, prefix_lpl)
    return Workload("cascade", dtype, num_qo_heads, num_kv_heads, head_dim,
                    1.0 / math.sqrt(head_dim), q, kv=kv, prefix_indices=prefix_pages.copy(),
                    prefix_last_page_len=prefix_lpl,
                    meta={"seed": seed, "prefix_len": prefix_len, "suffix_lens": suffix_lens})


def long_decode(seed=173004, batch=4, kv_len=131072, num_qo_heads=64, num_kv_heads=8,
                head_dim=128, page_size=64, dtype="bf16", canary=False):
    """Long-context decode: every request has the same (long) KV length."""
    w = batch_decode(seed=seed, batch=batch, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                     head_dim=head_dim, page_size=page_size, dtype=dtype, canary=canary,
                     kv_lens=np.full(batch, kv_len, dtype=np.int64))
    w.meta["kv_len"] = kv_len
    return w


@dataclass
class AppendWorkload:
    """New K/V rows to write into a paged cache whose page table already covers them."""
    kind = "append"              # (class attribute, not a field)
    dtype: str
    kv: PagedKV                  # page table after the append; pools as they are before it
    append_k: np.ndarray         # [nnz, Hkv, D] bit patterns
    append_v: np.ndarray
    append_indptr: np.ndarray    # int32 [B+1]: request b appends rows append_indptr[b]..[b+1]-1
    meta: dict = field(default_factory=dict)


def append_kv(seed=173002, batch=16, new_min=128, new_max=1024, prefix_min=0, prefix_max=2048,
              num_kv_heads=8, head_dim=128, page_size=16, dtype="bf16", canary=False,
              new_lens=None, prefix_lens=None):
    """The K/V of a prefill step's new tokens, appended after each request's cached prefix.

    With the default seed the lengths are those of the causal prefill workload
    (new tokens = its query tokens; same draws, same order). Draw order:
    new lengths, prefix lengths, pool permutation, K pool, V pool, appended K
    rows, appended V rows. With ``canary`` the unused pool pages, the slots past
    each last_page_len and the slots the append will write hold NaN.
    """
    rng = np.random.default_rng(seed)
    if new_lens is None:
        new_lens = rng.integers(new_min, new_max + 1, size=batch)
    if prefix_lens is None:
        prefix_lens = rng.integers(prefix_min, prefix_max + 1, size=len(new_lens))
    new_lens = np.asarray(new_lens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    kv_lens = new_lens + prefix_lens
    kv, _, _ = make_paged(rng, kv_lens, page_size, num_kv_heads, head_dim, dtype,
                          (0, num_kv_heads, head_dim))
    nnz = int(new_lens.sum())
    append_k = normal_bits(rng, (nnz, num_kv_heads, head_dim), dtype)
    append_v = normal_bits(rng, (nnz, num_kv_heads, head_dim), dtype)
    append_indptr = np.zeros(len(new_lens) + 1, dtype=np.int32)
    append_indptr[1:] = np.cumsum(new_lens)
    if canary:
        canary_tails(kv, dtype)
        nan = nan_bits(dtype)
        for b in range(len(kv_lens)):
            for t in range(int(prefix_lens[b]), int(kv_lens[b])):
                page = kv.kv_indices[kv.kv_indptr[b] + t // page_size]
                kv.k_cache[page, t % page_size] = nan
                kv.v_cache[page, t % page_size] = nan
    return AppendWorkload(dtype, kv, append_k, append_v, append_indptr,
                          meta={"seed": seed, "new_lens": new_lens, "prefix_lens": prefix_lens})


# Full-size workloads, in the order they are numbered in the tests and bench.
FULL = {
    0: lambda **kw: single_decode(seed=173000, **kw),
    1: lambda **kw: batch_decode(seed=173001, **kw),
    2: lambda **kw: batch_prefill(seed=173002, **kw),
    3: lambda **kw: cascade(seed=173003, **kw),
    4: lambda **kw: long_decode(seed=173004, **kw),
}

# Reduced sizes that the oracle finishes in seconds yet still span several
# tiles, several chunks and ragged tails.
SMALL = {
    0: lambda **kw: single_decode(seed=173100, kv_len=1000, **kw),
    1: lambda **kw: batch_decode(seed=173101, batch=8, kv_min=1, kv_max=700, **kw),
    2: lambda **kw: batch_prefill(seed=173102, batch=4, qo_min=1, qo_max=300, prefix_min=0,
                                  prefix_max=400, **kw),
    3: lambda **kw: cascade(seed=173103, batch=6, prefix_len=1000, suffix_min=1, suffix_max=200,
                            **kw),
    4: lambda **kw: long_decode(seed=173104, batch=2, kv_len=9000, **kw),
}


@dataclass
class BlockSparseWorkload:
    """Queries, dense keys / values and a BSR block mask over them."""
    kind = "block_sparse"        # (class attribute, not a field)
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    sm_scale: float
    q: np.ndarray                # [N_q, Hq, D] bit patterns
    k: np.ndarray                # [N_kv, Hkv, D]
    v: np.ndarray
    bsr_indptr: np.ndarray       # int32 [num_block_rows + 1]
    bsr_indices: np.ndarray      # int32, ascending within each block row
    row_block: int
    col_block: int
    meta: dict = field(default_factory=dict)


def block_sparse(seed=173006, num_qo_tokens=8192, num_kv_tokens=8192, row_block=64, col_block=64,
                 density=0.25, num_qo_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                 diagonal=True, empty_rows=()):
    """A random block mask: each (block row, key block) pair is kept with probability
    ``density`` (and the diagonal block always when ``diagonal``); block rows listed in
    ``empty_rows`` keep nothing. Draw order: the mask (one uniform per block pair, row
    major), q, k, v."""
    rng = np.random.default_rng(seed)
    mb = (num_qo_tokens + row_block - 1) // row_block
    nb = (num_kv_tokens + col_block - 1) // col_block
    keep = rng.random((mb, nb)) < density
    if diagonal:
        for i in range(min(mb, nb)):
            keep[i, i] = True
    for i in empty_rows:
        keep[i, :] = False
    indptr = np.zeros(mb + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(keep.sum(axis=1))
    indices = np.nonzero(keep)[1].astype(np.int32)        # row-major: ascending within a row
    q = normal_bits(rng, (num_qo_tokens, num_qo_heads, head_dim), dtype)
    k = normal_bits(rng, (num_kv_tokens, num_kv_heads, head_dim), dtype)
    v = normal_bits(rng, (num_kv_tokens, num_kv_heads, head_dim), dtype)
    return BlockSparseWorkload(dtype, num_qo_heads, num_kv_heads, head_dim,
                               1.0 / math.sqrt(head_dim), q, k, v, indptr, indices, row_block,
                               col_block, meta={"seed": seed, "density": density})


@dataclass
class PodWorkload:
    """A mixed batch: prefill requests and decode requests whose page tables point
    into one shared page pool (``prefill.kv`` and ``decode.kv`` hold the same pool
    arrays)."""
    kind = "pod"                 # (class attribute, not a field)
    prefill: Workload
    decode: Workload
    meta: dict = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.prefill.dtype


def pod(seed=173007, p_batch=16, qo_min=128, qo_max=1024, prefix_min=0, prefix_max=2048,
        d_batch=64, kv_min=512, kv_max=4096, num_qo_heads=32, num_kv_heads=8, head_dim=128,
        page_size=16, dtype="bf16", causal=True, canary=False, qo_lens=None, prefix_lens=None,
        d_lens=None):
    """The causal prefill workload's requests and the batch decode workload's requests
    in one batch over one pool. Draw order: prefill query lengths, prefixes, decode
    lengths, the pool (prefill requests' pages first), prefill q, K pool, V pool,
    decode q."""
    rng = np.random.default_rng(seed)
    if qo_lens is None:
        qo_lens = rng.integers(qo_min, qo_max + 1, size=p_batch)
    if prefix_lens is None:
        prefix_lens = rng.integers(prefix_min, prefix_max + 1, size=len(qo_lens))
    if d_lens is None:
        d_lens = rng.integers(kv_min, kv_max + 1, size=d_batch)
    qo_lens = np.asarray(qo_lens, dtype=np.int64)
    prefix_lens = np.asarray(prefix_lens, dtype=np.int64)
    d_lens = np.asarray(d_lens, dtype=np.int64)
    p_lens = qo_lens + prefix_lens
    Bp = len(qo_lens)
    kv, q_p, _ = make_paged(rng, np.concatenate([p_lens, d_lens]), page_size, num_kv_heads,
                            head_dim, dtype, (int(qo_lens.sum()), num_qo_heads, head_dim))
    q_d = normal_bits(rng, (len(d_lens), num_qo_heads, head_dim), dtype)
    if canary:
        canary_tails(kv, dtype)
    cut = int(kv.kv_indptr[Bp])
    kv_p = PagedKV(kv.k_cache, kv.v_cache, kv.kv_indptr[:Bp + 1].copy(), kv.kv_indices[:cut].copy(),
                   kv.last_page_len[:Bp].copy(), page_size)
    kv_d = PagedKV(kv.k_cache, kv.v_cache, (kv.kv_indptr[Bp:] - cut).astype(np.int32),
                   kv.kv_indices[cut:].copy(), kv.last_page_len[Bp:].copy(), page_size)
    qo_indptr = np.zeros(Bp + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    scale = 1.0 / math.sqrt(head_dim)
    wp = Workload("prefill", dtype, num_qo_heads, num_kv_heads, head_dim, scale, q_p, kv=kv_p,
                  qo_indptr=qo_indptr, causal=causal,
                  meta={"seed": seed, "qo_lens": qo_lens, "kv_lens": p_lens})
    wd = Workload("decode", dtype, num_qo_heads, num_kv_heads, head_dim, scale, q_d, kv=kv_d,
                  meta={"seed": seed, "kv_lens": d_lens})
    return PodWorkload(wp, wd, meta={"seed": seed})
