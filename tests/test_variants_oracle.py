"""Pins of the variant oracle (sliding window, logit soft cap, attention sinks).

Each pin checks the oracle against something other than its own formula:
closed forms built from exact identities (tanh(atanh(1/2)) = 1/2 with
atanh(1/2) = ln(3)/2), reductions to the already-pinned plain attention
(``oracle.attention_state`` / ``batch_prefill`` / ``batch_decode``), a sink
written out as an explicit extra key with a zero value row, the merge identity
of attention states, and brute-force slicing instead of masking. A planted
mistake test shows that the plausible slips fail at least one pin.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import variants as ov
from paged_kv_cache_173_amd import workloads as wl

LN3 = math.log(3.0)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- soft cap
def test_soft_cap_closed_form_two_keys():
    """c = 2 ln 3 and a scaled logit of c * atanh(1/2) = (ln 3)^2 cap to exactly ln 3;
    a second key with logit 0 stays 0. Weights 3 : 1, so O = (3 v1 + v2) / 4 and
    LSE = ln 4. sm_scale = 1/2, so a cap applied before the scale gives a different
    value (ln 3 * tanh(ln 3) = 0.879...)."""
    c = 2.0 * LN3
    scale = 0.5
    q = np.array([[1.0, 0.0]])
    k = np.array([[2.0 * LN3 * LN3, 0.0], [0.0, 5.0]])      # q.k = 2 (ln 3)^2 and 0
    v = np.array([[1.0, 0.0, 2.0], [0.0, 1.0, -2.0]])
    O, LSE = ov.variant_state(q, k, v, scale, soft_cap=c)
    assert np.allclose(O[0], [0.75, 0.25, 1.0], rtol=0, atol=1e-14)
    assert abs(LSE[0] - math.log(4.0)) < 1e-14


def test_soft_cap_saturates_to_uniform():
    """Scaled logits far above the cap all cap to c (within c * 2e-17): uniform
    weights, O = mean of v, LSE = c + ln n."""
    rng = np.random.default_rng(1)
    c = 3.0
    q = np.array([[1.0] + [0.0] * 7])
    k = np.zeros((5, 8))
    k[:, 0] = [200.0, 300.0, 250.0, 1000.0, 180.0]           # scale 0.5: logits >= 90 = 30c
    v = _rand(rng, 5, 8)
    O, LSE = ov.variant_state(q, k, v, 0.5, soft_cap=c)
    assert np.allclose(O[0], v.mean(axis=0), rtol=0, atol=1e-13)
    assert abs(LSE[0] - (c + math.log(5))) < 1e-13


def test_soft_cap_large_cap_is_plain_attention():
    """c -> infinity recovers the plain (pinned) attention state."""
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 6, 16), _rand(rng, 40, 16), _rand(rng, 40, 16)
    vis = rng.random((6, 40)) < 0.7
    O0, L0 = oracle.attention_state(q, k, v, 0.3, vis)
    O1, L1 = ov.variant_state(q, k, v, 0.3, vis, soft_cap=1e9)
    assert np.allclose(O1, O0, rtol=0, atol=1e-12) and np.allclose(L1, L0, rtol=0, atol=1e-12)


def test_soft_cap_bounds_every_logit():
    """Capped logits lie in (-c, c): with n visible keys, |LSE - ln n| < c."""
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 8, 32) * 30, _rand(rng, 50, 32) * 30, _rand(rng, 50, 32)
    _, LSE = ov.variant_state(q, k, v, 1.0, soft_cap=2.5)
    assert np.all(np.abs(LSE - math.log(50)) < 2.5)


# ---------------------------------------------------------------- sinks
def test_sink_closed_form():
    """One key with scaled logit ln 3 and a sink of logit 0: Z = 3 + 1, so
    O = 3/4 v and LSE = ln 4."""
    q = np.array([[LN3, 0.0]])
    k = np.array([[1.0, 7.0]])
    v = np.array([[4.0, -8.0]])
    O, LSE = ov.variant_state(q, k, v, 1.0, sink=0.0)
    assert np.allclose(O[0], [3.0, -6.0], rtol=0, atol=1e-14)
    assert abs(LSE[0] - math.log(4.0)) < 1e-14


def test_sink_is_an_extra_key_with_zero_value():
    """The sink equals one more key, whose scaled logit is sigma and whose value row
    is zero, in the plain (pinned) attention state: one row at a time, the key
    k* = q * sigma / (scale |q|^2) has scale * q.k* = sigma up to rounding."""
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 5, 16), _rand(rng, 30, 16), _rand(rng, 30, 16)
    scale = 0.25
    for sigma in (-3.0, 0.0, 1.7, 9.0):
        O, LSE = ov.variant_state(q, k, v, scale, sink=sigma)
        for r in range(5):
            ks = q[r] * sigma / (scale * float(q[r] @ q[r]))
            k2 = np.vstack([k, ks[None, :]])
            v2 = np.vstack([v, np.zeros((1, 16))])
            o_ref, l_ref = oracle.attention_state(q[r:r + 1], k2, v2, scale)
            assert np.allclose(O[r], o_ref[0], rtol=0, atol=1e-12)
            assert abs(LSE[r] - l_ref[0]) < 1e-12


def test_sink_is_a_merge_with_the_state_zero_sigma():
    """State with the sink = merge of the keys' state with (0, sigma) (pinned merge)."""
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 7, 16), _rand(rng, 25, 16), _rand(rng, 25, 16)
    vis = rng.random((7, 25)) < 0.5
    vis[3] = False                                            # a row that sees nothing
    sigma = 0.8
    O, LSE = ov.variant_state(q, k, v, 0.4, vis, sink=sigma)
    Ok, Lk = oracle.attention_state(q, k, v, 0.4, vis)
    Om, Lm = oracle.merge_state(Ok[:, None, :], Lk[:, None], np.zeros_like(Ok)[:, None, :],
                                np.full((7, 1), sigma))
    assert np.allclose(O, Om[:, 0], rtol=0, atol=1e-12)
    assert np.allclose(LSE, Lm[:, 0], rtol=0, atol=1e-12)


def test_sink_on_an_empty_row_and_minus_inf_sink():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 3, 8), _rand(rng, 10, 8), _rand(rng, 10, 8)
    none = np.zeros((3, 10), dtype=bool)
    O, LSE = ov.variant_state(q, k, v, 1.0, none, sink=-1.25)
    assert np.all(O == 0) and np.all(LSE == -1.25)
    O, LSE = ov.variant_state(q, k, v, 1.0, none, sink=None)
    assert np.all(O == 0) and np.all(LSE == -np.inf)
    # sigma = -inf is no sink at all
    O1, L1 = ov.variant_state(q, k, v, 1.0, sink=-np.inf)
    O0, L0 = oracle.attention_state(q, k, v, 1.0)
    assert np.array_equal(O1, O0) and np.array_equal(L1, L0)


# ---------------------------------------------------------------- window
def test_window_mask_brute_force():
    """Entry by entry: p = i + L - Q, visible iff p - W <= t (<= p when causal)."""
    for Q, L, W in [(1, 9, 3), (5, 12, 0), (4, 4, 2), (7, 3, 1), (6, 20, 100)]:
        for causal in (True, False):
            m = ov.window_visible(Q, L, W, causal)
            for i in range(Q):
                p = i + L - Q
                for t in range(L):
                    want = t >= p - W and (t <= p or not causal)
                    assert m[i, t] == want


def test_window_zero_returns_own_value():
    """W = 0 with the causal mask: query i sees only key p = i + L - Q, so
    O = v_p and LSE = scale * q.k_p (rows with p < 0 see nothing)."""
    rng = np.random.default_rng(7)
    Q, L = 6, 10
    q, k, v = _rand(rng, Q, 16), _rand(rng, L, 16), _rand(rng, L, 16)
    O, LSE = ov.variant_state(q, k, v, 0.5, ov.window_visible(Q, L, 0, True))
    for i in range(Q):
        p = i + L - Q
        assert np.allclose(O[i], v[p], rtol=0, atol=1e-14)
        assert abs(LSE[i] - 0.5 * float(q[i] @ k[p])) < 1e-13


def test_window_equals_slicing():
    """A windowed causal row equals plain attention over the slice k[p-W .. p]."""
    rng = np.random.default_rng(8)
    Q, L, W = 9, 40, 7
    q, k, v = _rand(rng, Q, 16), _rand(rng, L, 16), _rand(rng, L, 16)
    O, LSE = ov.variant_state(q, k, v, 0.3, ov.window_visible(Q, L, W, True), soft_cap=0.0)
    for i in range(Q):
        p = i + L - Q
        lo = max(0, p - W)
        o_ref, l_ref = oracle.attention_state(q[i:i + 1], k[lo:p + 1], v[lo:p + 1], 0.3)
        assert np.allclose(O[i], o_ref[0], rtol=0, atol=1e-13) and abs(LSE[i] - l_ref[0]) < 1e-13


# ---------------------------------------------------------------- batch forms
def test_batch_forms_reduce_to_the_plain_ones():
    """No variant: identical to the pinned batch decode / prefill; a window wider
    than every request is no window."""
    w = wl.batch_decode(seed=11, batch=5, kv_min=1, kv_max=90, num_qo_heads=8,
                        num_kv_heads=2, page_size=16, dtype="f16")
    kv = w.kv
    O0, L0 = oracle.batch_decode(w.q, kv.k_cache, kv.v_cache, kv.kv_indptr, kv.kv_indices,
                                 kv.last_page_len, "f16", 0.1)
    for W in (-1, 500):
        O1, L1 = ov.batch_decode_variant(w.q, kv.k_cache, kv.v_cache, kv.kv_indptr,
                                         kv.kv_indices, kv.last_page_len, "f16", 0.1,
                                         window_left=W)
        assert np.allclose(O1, O0, rtol=0, atol=1e-14) and np.allclose(L1, L0, rtol=0, atol=1e-14)
    p = wl.batch_prefill(seed=12, batch=3, qo_min=1, qo_max=40, prefix_max=30, num_qo_heads=4,
                         num_kv_heads=2, page_size=16, dtype="bf16")
    kv = p.kv
    for causal in (True, False):
        O0, L0 = oracle.batch_prefill(p.q, kv.k_cache, kv.v_cache, p.qo_indptr, kv.kv_indptr,
                                      kv.kv_indices, kv.last_page_len, "bf16", 0.2, causal)
        O1, L1 = ov.batch_prefill_variant(p.q, kv.k_cache, kv.v_cache, p.qo_indptr, kv.kv_indptr,
                                          kv.kv_indices, kv.last_page_len, "bf16", 0.2, causal,
                                          window_left=10_000)
        assert np.allclose(O1, O0, rtol=0, atol=1e-14) and np.allclose(L1, L0, rtol=0, atol=1e-14)


def test_batch_decode_window_is_the_last_w_plus_one_tokens():
    """Decode with window W equals plain single decode over each request's last
    W + 1 tokens (a brute-force gather, no mask)."""
    w = wl.batch_decode(seed=13, batch=4, kv_min=1, kv_max=70, num_qo_heads=4,
                        num_kv_heads=1, page_size=3, dtype="bf16")
    kv = w.kv
    W = 9
    O, LSE = ov.batch_decode_variant(w.q, kv.k_cache, kv.v_cache, kv.kv_indptr, kv.kv_indices,
                                     kv.last_page_len, "bf16", 0.15, window_left=W)
    for b in range(4):
        L = int(kv.kv_lens[b])
        toks = range(max(0, L - 1 - W), L)
        pages = [int(kv.kv_indices[kv.kv_indptr[b] + t // 3]) for t in toks]
        k = np.stack([kv.k_cache[p_, t % 3] for p_, t in zip(pages, toks)])
        v = np.stack([kv.v_cache[p_, t % 3] for p_, t in zip(pages, toks)])
        o_ref, l_ref = oracle.single_decode(w.q[b], k, v, "bf16", 0.15)
        assert np.allclose(O[b], o_ref, rtol=0, atol=1e-13) and np.allclose(LSE[b], l_ref, atol=1e-13)


# ---------------------------------------------------------------- planted mistakes
@pytest.mark.parametrize("mistake", ["cap_before_scale", "clamp_not_tanh", "cap_missing_div",
                                     "sink_with_value", "window_off_by_one"])
def test_planted_mistakes_fail_a_pin(monkeypatch, mistake):
    """Each plausible slip, planted in a copy of the oracle's arithmetic, fails a pin."""
    real_cap = ov.capped_logits
    real_vis = ov.window_visible
    if mistake == "cap_before_scale":
        def bad_state(q, k, v, sm_scale, visible=None, soft_cap=0.0, sink=None):
            x = real_cap(np.asarray(q) @ np.asarray(k).T, soft_cap) * sm_scale
            return _state_from_logits(x, v, visible, sink)
        monkeypatch.setattr(ov, "variant_state", bad_state)
        with pytest.raises(AssertionError):
            test_soft_cap_closed_form_two_keys()
        return
    if mistake == "clamp_not_tanh":
        monkeypatch.setattr(ov, "capped_logits",
                            lambda x, c: np.clip(x, -c, c) if c > 0 else np.asarray(x, float))
        with pytest.raises(AssertionError):
            test_soft_cap_closed_form_two_keys()
        return
    if mistake == "cap_missing_div":
        monkeypatch.setattr(ov, "capped_logits",
                            lambda x, c: c * np.tanh(x) if c > 0 else np.asarray(x, float))
        with pytest.raises(AssertionError):
            test_soft_cap_large_cap_is_plain_attention()
        return
    if mistake == "sink_with_value":
        def bad_state(q, k, v, sm_scale, visible=None, soft_cap=0.0, sink=None):
            # the sink's weight lands on the first value row instead of a zero row
            O, LSE = real_state(q, k, v, sm_scale, visible, soft_cap, sink)
            if sink is not None and np.asarray(k).shape[0] > 0:
                O = O + np.exp(sink - LSE)[:, None] * np.asarray(v)[0][None, :]
            return O, LSE
        real_state = ov.variant_state
        monkeypatch.setattr(ov, "variant_state", bad_state)
        with pytest.raises(AssertionError):
            test_sink_closed_form()
        return
    if mistake == "window_off_by_one":
        monkeypatch.setattr(ov, "window_visible",
                            lambda Q, L, W, causal: real_vis(Q, L, W + 1 if W >= 0 else W, causal))
        with pytest.raises(AssertionError):
            test_window_zero_returns_own_value()
        return


def _state_from_logits(x, v, visible, sink):
    x = np.asarray(x, float)
    R, L = x.shape
    if visible is None:
        visible = np.ones((R, L), dtype=bool)
    x = np.where(visible, x, -np.inf)
    sig = -np.inf if sink is None else sink
    m = np.maximum(x.max(axis=1), sig)
    w = np.exp(x - m[:, None])
    z = w.sum(axis=1) + np.exp(sig - m)
    return (w @ np.asarray(v, float)) / z[:, None], m + np.log(z)
