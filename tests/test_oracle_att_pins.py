"""Pins of the oracle's windowed decode attention to facts fixed by the pages
and by mathematics, none of which re-types its formula:

  - closed forms: one visible row returns that row's V exactly; equal scores
    return the mean of the visible V rows; two rows give
    v1 + (v2 - v1) * sigmoid(s2 - s1), worked with Python's math module; a row
    whose score dominates returns its V;
  - the window of the pull request "GQA support sliding_window_cache"
    ("Design": results identical to a full-length cache; the CPU follow-up: rows
    older than the window are masked): rows outside [L - W, L) change nothing,
    and the windowed cache gives exactly what a full-length cache gives with
    the same local window;
  - the ring-buffer page ("Sliding-window ring buffer"): slot order does not
    change the scores, so permuting the visible rows changes nothing beyond
    rounding;
  - GQA head grouping (the roadmap's "Phase 1"): query head h reads KV head
    h / (Hq / Hkv), checked with KV heads of distinct constant V;
  - no overflow for huge scores; bad lengths flagged, empty windows zero.

SWRT_ORACLE_LIB may name another build of the oracle (the mutation test uses
this to check that planted mistakes fail here).
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
from oracle import XF_BF16, XF_F32

F32 = XF_F32


@pytest.fixture(scope="module")
def orc() -> oracle.Oracle:
    path = os.environ.get("SWRT_ORACLE_LIB")
    return oracle.Oracle(path) if path else oracle.get()


def case(g, B=3, Hq=8, Hkv=2, C=16, D=8):
    q = g.standard_normal((B, Hq, D)).astype(np.float32)
    k = g.standard_normal((B, Hkv, C, D)).astype(np.float32)
    v = g.standard_normal((B, Hkv, C, D)).astype(np.float32)
    return q, k, v


def test_one_visible_row_is_that_rows_v(orc):
    g = np.random.default_rng(1)
    q, k, v = case(g)
    L = np.array([1, 9, 16])
    out, f = orc.window_attention(q, k, v, L, 1, 0.7, F32)  # W = 1: only row L - 1
    assert f == 0
    for b in range(3):
        for h in range(8):
            np.testing.assert_array_equal(out[b, h], v[b, h // 4, L[b] - 1].astype(np.float64))


def test_equal_scores_average_the_window(orc):
    g = np.random.default_rng(2)
    q, k, v = case(g)
    q[:] = 0.0
    L = np.array([3, 16, 10])
    W = 6
    out, _ = orc.window_attention(q, k, v, L, W, 1.0, F32)
    for b in range(3):
        lo = max(0, L[b] - W)
        for h in range(8):
            want = v[b, h // 4, lo:L[b]].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(out[b, h], want, rtol=1e-13, atol=1e-15)


def test_two_rows_closed_form(orc):
    """Two query heads of one KV head, each with its own query: B = 1, D = 2."""
    q = np.float32([[[1.0, 2.0], [-1.0, 0.5]]])
    k = np.float32([[[[0.5, -1.0], [2.0, 0.25]]]])
    v = np.float32([[[[3.0, -1.0], [-2.0, 4.0]]]])
    scale = 0.75
    out, _ = orc.window_attention(q, k, v, [2], 8, scale, F32)
    # head 0 scores: 0.5 - 2 = -1.5 and 2 + 0.5 = 2.5; head 1: -0.5 - 0.5 = -1 and -2 + 0.125
    for h, (s1, s2) in enumerate(((-1.5, 2.5), (-1.0, -1.875))):
        sig = 1.0 / (1.0 + math.exp(-(scale * s2 - scale * s1)))
        want = [3.0 + (-2.0 - 3.0) * sig, -1.0 + (4.0 - -1.0) * sig]
        np.testing.assert_allclose(out[0, h], want, rtol=1e-14)


def test_dominant_score_and_no_overflow(orc):
    g = np.random.default_rng(3)
    q, k, v = case(g, B=1, Hq=2, Hkv=1, C=8, D=4)
    k[0, 0, 5] = q[0, 0] * 1e3  # row 5's score is huge for head 0
    out, _ = orc.window_attention(q, k, v, [8], 8, 1.0, F32)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out[0, 0], v[0, 0, 5], rtol=1e-12)


def test_rows_outside_the_window_change_nothing(orc):
    g = np.random.default_rng(4)
    q, k, v = case(g)
    L = np.array([16, 7, 12])
    W = 5
    base, _ = orc.window_attention(q, k, v, L, W, 0.4, F32)
    k2, v2 = k.copy(), v.copy()
    for b in range(3):
        lo = max(0, L[b] - W)
        k2[b, :, :lo] = g.standard_normal(k2[b, :, :lo].shape)
        v2[b, :, :lo] = 1e6
        k2[b, :, L[b]:] = 1e3
        v2[b, :, L[b]:] = -1e6
    out, _ = orc.window_attention(q, k2, v2, L, W, 0.4, F32)
    np.testing.assert_array_equal(out, base)
    # and the window is exactly W rows: moving its lower edge changes the result
    k3 = k.copy()
    k3[0, :, L[0] - W] += 3.0
    assert not np.array_equal(orc.window_attention(q, k3, v, L, W, 0.4, F32)[0], base)


def test_windowed_cache_equals_full_cache(orc):
    """A windowed cache holding the last L = min(T, C) tokens gives exactly the
    full-length cache's result under the same local window."""
    g = np.random.default_rng(5)
    B, Hq, Hkv, D, Tmax, C, W = 2, 4, 2, 8, 40, 12, 10
    q = g.standard_normal((B, Hq, D)).astype(np.float32)
    kf = g.standard_normal((B, Hkv, Tmax, D)).astype(np.float32)
    vf = g.standard_normal((B, Hkv, Tmax, D)).astype(np.float32)
    T = np.array([33, 7])
    full, _ = orc.window_attention(q, kf, vf, T, W, 0.3, F32)
    kw = np.zeros((B, Hkv, C, D), np.float32)
    vw = np.zeros((B, Hkv, C, D), np.float32)
    L = np.minimum(T, C)
    for b in range(B):
        kw[b, :, :L[b]] = kf[b, :, T[b] - L[b]:T[b]]
        vw[b, :, :L[b]] = vf[b, :, T[b] - L[b]:T[b]]
    win, _ = orc.window_attention(q, kw, vw, L, W, 0.3, F32)
    np.testing.assert_array_equal(win, full)


def test_slot_order_does_not_matter(orc):
    g = np.random.default_rng(6)
    q, k, v = case(g, C=10)
    L = np.array([10, 10, 10])
    base, _ = orc.window_attention(q, k, v, L, 10, 0.5, F32)
    perm = g.permutation(10)
    out, _ = orc.window_attention(q, k[:, :, perm], v[:, :, perm], L, 10, 0.5, F32)
    np.testing.assert_allclose(out, base, rtol=1e-12, atol=1e-14)


def test_query_heads_read_their_kv_head(orc):
    g = np.random.default_rng(7)
    q, k, v = case(g, Hq=12, Hkv=3)
    for kv in range(3):
        v[:, kv] = kv + 1.0
    out, _ = orc.window_attention(q, k, v, [16, 5, 9], 16, 0.9, F32)
    for h in range(12):
        np.testing.assert_allclose(out[:, h], h // 4 + 1.0, rtol=1e-14)


def test_bf16_elements_decode_exactly(orc):
    """bf16 q/k/v: the same as float32 arrays holding the decoded values."""
    g = np.random.default_rng(8)
    q, k, v = case(g)
    bits = [(a.view(np.uint32) >> 16).astype(np.uint16) for a in (q, k, v)]
    dec = [(b_.astype(np.uint32) << 16).view(np.float32) for b_ in bits]
    L = np.array([16, 4, 11])
    a, _ = orc.window_attention(*bits, L, 7, 0.6, XF_BF16)
    b, _ = orc.window_attention(*dec, L, 7, 0.6, F32)
    np.testing.assert_array_equal(a, b)


def test_bad_and_empty_lengths(orc):
    g = np.random.default_rng(9)
    q, k, v = case(g)
    out = np.full((3, 8, 8), 7.0)
    out, f = orc.window_attention(q, k, v, [0, 17, -1], 4, 1.0, F32, out=out)
    assert f == oracle.FLAG_BAD_LENGTHS
    np.testing.assert_array_equal(out[0], 0.0)
    np.testing.assert_array_equal(out[1:], 7.0)
