"""Inputs with every logit below -5e4 that still vary by O(1) from key to key.

The FlashInfer article (section "Extreme-negative-logit correction") reports
that a finite "minus infinity" of -5e4 silently zeroed rows whose logits all
lay below it. These helpers turn the usual seeded N(0, 1) workloads into such
inputs (on the host, before upload); every value stays exactly representable
in fp16 and bf16:
  * q[..., 0] = 768 and k[..., 0] = -768 (every raw score gets -768^2);
  * q[..., 1] = 8 and k[token, :, 1] = a ramp from -16 to 16 over the
    request's logical positions (quarter steps), so later keys score higher
    and the running maximum moves;
  * every other element is rounded to a multiple of 1/4.
Every product and partial sum of a raw score is then a multiple of 1/16 below
2^20 in magnitude, so fp32 scores are exact in any summation order, and the
logits are ~-52137 +- 15 (natural-log units).

No attention arithmetic here: only value placement.
"""

import numpy as np

from paged_kv_cache_173_amd import workloads as wl

A = 768.0
LOGIT_CEILING = -5e4


def _float(bits, dtype):
    """uint16 fp16 / bf16 bit patterns -> float64 (exact)."""
    bits = np.asarray(bits, np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _quarter(x):
    return np.round(np.asarray(x, np.float64) * 4.0) / 4.0


def _bits(x, dtype):
    return wl.round_bits(np.asarray(x, np.float32), dtype)


def extreme_q(q_bits, dtype):
    """q with the large first component, the ramp weight and quarter-step values."""
    x = _quarter(_float(q_bits, dtype))
    x[..., 0] = A
    x[..., 1] = 8.0
    out = _bits(x, dtype)
    assert np.array_equal(_float(out, dtype), x, equal_nan=True)   # exactly representable
    return out


def _ramp(t, n):
    """Quarter-step ramp from -16 (t = 0) to 16 (t = n - 1)."""
    return _quarter(-16.0 + 32.0 * t / max(n - 1, 1))


def extreme_rows(k_bits, dtype, ramp=None):
    """K rows [..., D] with -A in component 0, quarter-step values elsewhere and, if given,
    the ramp values in component 1 (ramp broadcasts over the leading axes)."""
    x = _quarter(_float(k_bits, dtype))
    x[..., 0] = -A
    if ramp is not None:
        x[..., 1] = ramp
    out = _bits(x, dtype)
    assert np.array_equal(_float(out, dtype), x, equal_nan=True)   # (NaN canaries stay NaN)
    return out


def extreme_paged(kv, dtype, requests_lens, extra=None):
    """Rewrite a page pool in place: K rows get -A and quarter values everywhere (so a
    wrong page would still be extreme), the ramp goes into the used tokens of each request
    by logical position; V rows are rounded to quarter steps. ``extra`` = (pages, length)
    of a further page list (the cascade's prefix) that gets its own ramp."""
    P = kv.page_size
    kc = kv.k_cache.astype(np.uint16)
    vc = kv.v_cache.astype(np.uint16)
    kc = extreme_rows(kc, dtype)
    vc = _bits(_quarter(_float(vc, dtype)), dtype)
    x = _float(kc, dtype)

    def put(pages, L):
        for j, page in enumerate(pages):
            t = j * P + np.arange(P)
            n = int(min(P, L - j * P))
            if n <= 0:
                break
            x[page, :n, :, 1] = _ramp(t[:n], L)[:, None]

    for b, L in enumerate(requests_lens):
        put(kv.kv_indices[kv.kv_indptr[b]:kv.kv_indptr[b + 1]], int(L))
    if extra is not None:
        put(*extra)
    kv.k_cache = _bits(x, dtype)
    assert np.array_equal(_float(kv.k_cache, dtype), x, equal_nan=True)
    kv.v_cache = vc


