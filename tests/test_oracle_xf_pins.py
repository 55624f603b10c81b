"""Pins of the oracle's fused-append transform: RoPE on K at the absolute
position, then conversion or affine quantization into the cache's element type.

None of these checks re-types the oracle's arithmetic. They use:
  - library roundings: torch's float32 -> bfloat16 and numpy's float32 ->
    float16 conversions (round to nearest even), numpy's float16 -> float32
    decoding, and Python's round-half-even;
  - closed forms of a rotation: a one-hot pair (1, 0) turns into (cos, sin) and
    (0, 1) into (-sin, cos), read straight from the tables at the position the
    pull request "GQA support sliding_window_cache" prescribes (the absolute
    one, "Summary of Changes"), and elements past the rotary dimension, and V,
    pass unchanged;
  - invariants: a rotation keeps each pair's length, turning back by the
    negated angle restores the input, scores depend only on the distance of
    the two positions, and the interleaved layout is a permutation of the
    half-split one;
  - the quantization statements of the onnx-light how-to "Persistent
    input/output feedback" (section "Optional heterogeneous paged KV"): ties
    round to even, codes saturate, a non-saturated reconstruction is within
    half a scale, and the end-to-end fixture's parameters (components
    +/-0.173 * step, scale 0.01, zero points 0 and 128);
  - reductions to functions pinned elsewhere: with nothing to rotate or
    convert, the fused append and the fused TensorScatter are the plain ones.

SWRT_ORACLE_LIB may name another build of the oracle (the mutation test uses
this to check that planted mistakes fail here).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import XF_BF16, XF_F16, XF_F32, XF_INT8, XF_UINT8, Transform

NP = {XF_F32: np.float32, XF_F16: np.float16, XF_BF16: np.uint16, XF_INT8: np.int8,
      XF_UINT8: np.uint8}


@pytest.fixture(scope="module")
def orc() -> oracle.Oracle:
    path = os.environ.get("SWRT_ORACLE_LIB")
    return oracle.Oracle(path) if path else oracle.get()


def row_out(orc, x: Transform, t, pos, row):
    out = np.zeros(row.size * oracle.XF_BYTES[x.out_type] // np.dtype(NP[x.out_type]).itemsize,
                   NP[x.out_type])
    assert orc.xf_row(x, t, pos, np.ascontiguousarray(row), out) == oracle.OK
    return out


def rope_tables(max_pos, rot, base=10000.0):
    """cos / sin of p * base^(-2j/rot), evaluated in float64, stored as float32."""
    j = np.arange(rot // 2)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * j / rot)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def random_tables(g, max_pos, rot):
    ang = g.uniform(-math.pi, math.pi, size=(max_pos, rot // 2))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def finite_f32(g, n):
    bits = g.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    return v[~np.isnan(v)]


# -- element conversions ------------------------------------------------------
def test_bf16_output_rounds_like_torch(orc):
    g = np.random.default_rng(1)
    v = finite_f32(g, 20000)
    # exact ties: the dropped half is 0x8000, with an even and an odd kept half
    ties = (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000, 0x00018000],
                     np.uint32)).view(np.float32)
    v = np.concatenate([v, ties, np.float32([0.0, -0.0, np.inf, -np.inf, 1e-45])])
    got = row_out(orc, Transform(XF_F32, XF_BF16), 1, 0, v)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    nan = row_out(orc, Transform(XF_F32, XF_BF16), 1, 0, np.float32([np.nan, -np.nan]))
    np.testing.assert_array_equal(nan, [0x7FC0, 0x7FC0])  # canonical quiet NaN


def test_f16_output_rounds_like_numpy(orc):
    g = np.random.default_rng(2)
    parts = [finite_f32(g, 5000),
             g.uniform(-70000, 70000, 5000).astype(np.float32),      # overflow boundary
             (g.uniform(-1, 1, 5000) * 2.0**-14).astype(np.float32),  # subnormal range
             (g.uniform(-1, 1, 5000) * 2.0**-24).astype(np.float32)]  # below the smallest
    # exact ties between neighbouring float16 values, normal and subnormal
    h = g.integers(0, 0x7BFF, size=3000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    parts.append(((lo + hi) / 2).astype(np.float32))
    parts.append(np.float32([65504.0, 65519.99, 65520.0, -65520.0, 2.0**-25, 3 * 2.0**-26]))
    v = np.concatenate(parts)
    got = row_out(orc, Transform(XF_F32, XF_F16), 1, 0, v)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16)
    np.testing.assert_array_equal(got.view(np.uint16), want.view(np.uint16))
    nan = row_out(orc, Transform(XF_F32, XF_F16), 1, 0, np.float32([np.nan]))
    assert nan.view(np.uint16)[0] == 0x7E00


def test_float32_nan_is_canonical(orc):
    """Any NaN, whatever its sign and payload, is stored as 0x7FC00000."""
    nans = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF, 0x7FA12345], np.uint32)
    got = row_out(orc, Transform(XF_F32, XF_F32), 1, 0, nans.view(np.float32))
    np.testing.assert_array_equal(got.view(np.uint32), [0x7FC00000] * 5)
    h = row_out(orc, Transform(XF_F16, XF_F32), 1, 0, np.uint16([0xFE01, 0x7C01]).view(np.float16))
    np.testing.assert_array_equal(h.view(np.uint32), [0x7FC00000] * 2)
    # a NaN made by the rotation itself (inf * 0) as well
    cos, sin = np.float32([[0.0]]), np.float32([[1.0]])
    r = row_out(orc, Transform(XF_F32, XF_F32, cos, sin, 2), 0, 0, np.float32([np.inf, 0.0]))
    assert r.view(np.uint32)[0] == 0x7FC00000


def test_inputs_decode_exactly(orc):
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = row_out(orc, Transform(XF_F16, XF_F32), 1, 0, every.view(np.float16))
    want = every.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    np.testing.assert_array_equal(f16[~nan], want[~nan])
    assert np.isnan(f16[nan]).all()
    bf = row_out(orc, Transform(XF_BF16, XF_F32), 1, 0, every)
    want = (every.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(want)
    np.testing.assert_array_equal(bf.view(np.uint32)[~nan], want.view(np.uint32)[~nan])
    assert np.isnan(bf[nan]).all()


# -- rotation -----------------------------------------------------------------
def pairs(D, rot, interleaved):
    h = rot // 2
    return [(2 * j, 2 * j + 1) if interleaved else (j, j + h) for j in range(h)]


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("D,rot", [(16, 16), (20, 12)])
def test_one_hot_pairs_read_the_tables(orc, interleaved, D, rot):
    """(1, 0) -> (cos, sin) and (0, 1) -> (-sin, cos) at table row pos, column j."""
    g = np.random.default_rng(D + rot + interleaved)
    cos, sin = random_tables(g, 50, rot)
    x = Transform(XF_F32, XF_F32, cos, sin, rot, interleaved)
    for pos in (0, 7, 49):
        for j, (i0, i1) in enumerate(pairs(D, rot, interleaved)):
            for which, (e0, e1) in ((i0, (cos[pos, j], sin[pos, j])),
                                    (i1, (-sin[pos, j], cos[pos, j]))):
                v = np.zeros(D, np.float32)
                v[which] = 1.0
                out = row_out(orc, x, 0, pos, v)
                want = np.zeros(D, np.float32)
                want[i0], want[i1] = e0, e1
                np.testing.assert_array_equal(out, want)
        for i in range(rot, D):  # past the rotary dimension: unchanged
            v = np.zeros(D, np.float32)
            v[i] = 3.0
            np.testing.assert_array_equal(row_out(orc, x, 0, pos, v), v)
    v = g.standard_normal(D).astype(np.float32)
    np.testing.assert_array_equal(row_out(orc, x, 1, 9, v), v)  # V is never rotated


def test_rotation_keeps_pair_lengths_and_turns_back(orc):
    g = np.random.default_rng(3)
    D = 64
    cos, sin = rope_tables(4096, D)
    fwd = Transform(XF_F32, XF_F32, cos, sin, D)
    back = Transform(XF_F32, XF_F32, cos, -sin, D)
    u = 2.0**-24
    for pos in (0, 1, 100, 4095):
        v = g.standard_normal(D).astype(np.float32)
        r = row_out(orc, fwd, 0, pos, v).astype(np.float64)
        for i0, i1 in pairs(D, D, False):
            n0 = math.hypot(float(v[i0]), float(v[i1]))
            n1 = math.hypot(r[i0], r[i1])
            c2s2 = float(cos[pos, i0]) ** 2 + float(sin[pos, i0]) ** 2
            assert abs(n1 - n0 * math.sqrt(c2s2)) <= 8 * u * n0 + 1e-30
        w = row_out(orc, back, 0, pos, r.astype(np.float32)).astype(np.float64)
        assert np.abs(w - v).max() <= 16 * u * np.abs(v).max()


def test_scores_depend_on_distance_only(orc):
    g = np.random.default_rng(4)
    D = 64
    cos, sin = rope_tables(20000, D)
    x = Transform(XF_F32, XF_F32, cos, sin, D)
    q = g.standard_normal(D).astype(np.float32)
    k = g.standard_normal(D).astype(np.float32)
    scale = float(np.linalg.norm(q) * np.linalg.norm(k))
    for p, pk, shift in ((10, 3, 100), (500, 499, 7000), (130, 0, 19000 - 130)):
        a = np.dot(row_out(orc, x, 0, p, q).astype(np.float64),
                   row_out(orc, x, 0, pk, k).astype(np.float64))
        b = np.dot(row_out(orc, x, 0, p + shift, q).astype(np.float64),
                   row_out(orc, x, 0, pk + shift, k).astype(np.float64))
        assert abs(a - b) <= 2e-4 * scale


def test_interleaved_is_a_permutation_of_half_split(orc):
    g = np.random.default_rng(5)
    D, rot = 24, 16
    cos, sin = random_tables(g, 20, rot)
    half = Transform(XF_F32, XF_F32, cos, sin, rot, False)
    inter = Transform(XF_F32, XF_F32, cos, sin, rot, True)
    perm = np.arange(D)  # interleaved slot of each half-split element
    for j, ((h0, h1), (i0, i1)) in enumerate(zip(pairs(D, rot, False), pairs(D, rot, True))):
        perm[h0], perm[h1] = i0, i1
    for pos in (0, 11, 19):
        v = g.standard_normal(D).astype(np.float32)
        w = np.empty_like(v)
        w[perm] = v
        np.testing.assert_array_equal(row_out(orc, inter, 0, pos, w)[perm],
                                      row_out(orc, half, 0, pos, v))


def test_half_precision_inputs_and_outputs_rotate_in_float(orc):
    """bf16 in, rotated, bf16 out equals: decode, rotate in float32, round
    with torch (the one-step pins above fix each part)."""
    g = np.random.default_rng(6)
    D = 32
    cos, sin = rope_tables(300, D)
    v = torch.from_numpy(g.standard_normal(D).astype(np.float32)).to(torch.bfloat16)
    bits = v.view(torch.int16).numpy().view(np.uint16)
    f = row_out(orc, Transform(XF_BF16, XF_F32, cos, sin, D), 0, 123, bits)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(row_out(orc, Transform(XF_BF16, XF_BF16, cos, sin, D), 0, 123,
                                          bits), want)


# -- quantization -------------------------------------------------------------
def test_ties_round_to_even(orc):
    ks = np.arange(-6, 7)
    y = ((ks + 0.5) * 0.25).astype(np.float32)  # y / 0.25 = k + 0.5 exactly
    got = row_out(orc, Transform(XF_F32, XF_INT8, scale=(0.25, 0.25)), 1, 0, y)
    np.testing.assert_array_equal(got, [round(k + 0.5) for k in ks])


def test_saturation_nan_and_zero_points(orc):
    y = np.float32([0.0, 1e6, -1e6, np.inf, -np.inf, np.nan, 1.26, -1.29])
    i8 = row_out(orc, Transform(XF_F32, XF_INT8, scale=(0.01, 0.01)), 1, 0, y)
    np.testing.assert_array_equal(i8, [0, 127, -128, 127, -128, 0, 126, -128])
    u8 = row_out(orc, Transform(XF_F32, XF_UINT8, scale=(0.01, 0.01), zero_point=(128, 128)), 1,
                 0, y)
    np.testing.assert_array_equal(u8, [128, 255, 0, 255, 0, 128, 254, 0])
    zp = row_out(orc, Transform(XF_F32, XF_INT8, scale=(1.0, 1.0), zero_point=(-3, -3)), 1, 0,
                 np.float32([0.0, 2.0, 200.0]))
    np.testing.assert_array_equal(zp, [-3, -1, 127])


@pytest.mark.parametrize("out,zp", [(XF_INT8, 0), (XF_INT8, 17), (XF_UINT8, 128)])
def test_reconstruction_within_half_a_scale(orc, out, zp):
    g = np.random.default_rng(7 + zp)
    s = np.float32(0.037)
    lo, hi = (-128, 127) if out == XF_INT8 else (0, 255)
    y = g.uniform((lo - zp) * float(s), (hi - zp) * float(s), 4000).astype(np.float32)
    q = row_out(orc, Transform(XF_F32, out, scale=(s, s), zero_point=(zp, zp)), 1, 0, y)
    err = np.abs((q.astype(np.float64) - zp) * float(s) - y.astype(np.float64))
    assert (err <= float(s) / 2 + np.abs(y) * 2.0**-22).all()


def test_fixture_parameters_of_the_pages(orc):
    """Components +/-0.173 * step (steps 1..4) at scale 0.01: INT8 zero point
    0 and UINT8 zero point 128 (the end-to-end fixture's table)."""
    vals = [Fraction(sign * 173 * step, 1000) for step in (1, 2, 3, 4) for sign in (1, -1)]
    codes = [round(v / Fraction(1, 100)) for v in vals]  # exact: none is a tie
    y = np.float32([float(v) for v in vals])
    i8 = row_out(orc, Transform(XF_F32, XF_INT8, scale=(0.01, 0.01)), 1, 0, y)
    u8 = row_out(orc, Transform(XF_F32, XF_UINT8, scale=(0.01, 0.01), zero_point=(128, 128)), 1,
                 0, y)
    np.testing.assert_array_equal(i8, codes)
    np.testing.assert_array_equal(u8, [c + 128 for c in codes])


def test_k_and_v_use_their_own_parameters(orc):
    y = np.float32([1.0, -1.0, 0.3])
    x = Transform(XF_F32, XF_UINT8, scale=(0.5, 0.25), zero_point=(10, 100))
    np.testing.assert_array_equal(row_out(orc, x, 0, 0, y), [12, 8, 11])
    np.testing.assert_array_equal(row_out(orc, x, 1, 0, y), [104, 96, 101])


def test_bad_transforms_rejected(orc):
    row = np.zeros(8, np.float32)
    out = np.zeros(8, np.int8)
    cos, sin = rope_tables(4, 8)
    for bad in (Transform(XF_INT8, XF_INT8), Transform(XF_F32, 9),
                Transform(XF_F32, XF_INT8, scale=(0.0, 1.0)),
                Transform(XF_F32, XF_INT8, scale=(1.0, np.inf)),
                Transform(XF_F32, XF_INT8, zero_point=(128, 0)),
                Transform(XF_F32, XF_INT8, cos, sin, 7),
                Transform(XF_F32, XF_INT8, cos, sin, 10)):
        assert orc.xf_row(bad, 0, 0, row, out) == oracle.E_INVALID_ARG
    ok = Transform(XF_F32, XF_INT8, cos, sin, 8)
    assert orc.xf_row(ok, 0, 3, row, out) == oracle.OK
    assert orc.xf_row(ok, 0, 4, row, out) == oracle.E_INVALID_ARG  # past the tables


# -- fused windowed append ----------------------------------------------------
def _window_case(g, B, H, C, S, D, in_type):
    new_shape = (B, H, S, D)
    if in_type == XF_BF16:
        new = [torch.from_numpy(g.standard_normal(new_shape).astype(np.float32))
               .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16) for _ in range(2)]
    else:
        new = [g.standard_normal(new_shape).astype(NP[in_type]) for _ in range(2)]
    return new


@pytest.mark.parametrize("in_type", [XF_F32, XF_F16, XF_BF16])
@pytest.mark.parametrize("S", [1, 3])
def test_window_identity_transform_is_the_plain_append(orc, in_type, S):
    g = np.random.default_rng(10 + S + in_type)
    B, H, C, D = 5, 2, 8, 6
    kn, vn = _window_case(g, B, H, C, S, D, in_type)
    T = np.array([1, 5, 8, 9, 30]) + S - 1
    L = orc.kv_seq_lengths(T - 1, S, C)
    k0 = g.integers(0, 255, (B, H, C, D * kn.itemsize), dtype=np.uint8)
    v0 = g.integers(0, 255, (B, H, C, D * kn.itemsize), dtype=np.uint8)
    st = [np.zeros((B, H, C + S, D * kn.itemsize), np.uint8) for _ in range(4)] if S > 1 else \
        [None] * 4
    k1, v1, k2, v2 = k0.copy(), v0.copy(), k0.copy(), v0.copy()
    f1 = orc.kv_window_append_xf(Transform(in_type, in_type), k1, v1, kn, vn,
                                 (H * S * D, S * D, D), S, L.cache_past, L.evict, L.past,
                                 st[0], st[1])
    f2 = orc.kv_window_append_strided(k2, v2, kn, vn, (H * S * D, S * D, D), S, L.cache_past,
                                      L.evict, st[2], st[3], elem_bits=kn.itemsize * 8,
                                      head_dim=D)
    assert f1 == f2 == 0
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)
    if S > 1:
        np.testing.assert_array_equal(st[0], st[2])


@pytest.mark.parametrize("out_type", [XF_BF16, XF_INT8, XF_UINT8])
@pytest.mark.parametrize("S", [1, 4])
def test_window_rows_are_transformed_at_absolute_positions(orc, out_type, S):
    """The appended rows are the transform of the new rows at position
    P + s (absolute: far beyond the capacity), K rotated and V not; every
    other byte of the step is the plain step's."""
    g = np.random.default_rng(20 + S + out_type)
    B, H, C, D = 4, 3, 8, 8
    cos, sin = rope_tables(6000, 8)
    x = Transform(XF_BF16, out_type, cos, sin, 8, False, (0.02, 0.03), (0, 0) if
                  out_type != XF_UINT8 else (120, 130))
    kn, vn = _window_case(g, B, H, C, S, D, XF_BF16)
    T = np.array([2, 9, 4000, 5990]) + S - 1
    L = orc.kv_seq_lengths(T - 1, S, C)
    es = oracle.XF_BYTES[out_type]
    k0 = g.integers(0, 255, (B, H, C, D * es), dtype=np.uint8)
    v0 = g.integers(0, 255, (B, H, C, D * es), dtype=np.uint8)
    k1, v1 = k0.copy(), v0.copy()
    st = [np.zeros((B, H, C + S, D * es), np.uint8) for _ in range(2)] if S > 1 else [None] * 2
    assert orc.kv_window_append_xf(x, k1, v1, kn, vn, (H * S * D, S * D, D), S, L.cache_past,
                                   L.evict, L.past, st[0], st[1]) == 0
    # the same step on rows transformed one at a time
    rows = [np.zeros((B, H, S, D * es), np.uint8) for _ in range(2)]
    for t, new in enumerate((kn, vn)):
        for b in range(B):
            for h in range(H):
                for s in range(S):
                    rows[t][b, h, s] = row_out(orc, x, t, int(L.past[b]) + s,
                                               new[b, h, s]).view(np.uint8)
    k2, v2 = k0.copy(), v0.copy()
    st2 = [np.zeros_like(st[0]) for _ in range(2)] if S > 1 else [None] * 2
    assert orc.kv_window_append(k2, v2, rows[0], rows[1], L.cache_past, L.evict, st2[0], st2[1],
                                elem_bits=8) == 0
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)
    assert L.past[3] > 5000  # positions far past the capacity were rotated


def test_window_position_out_of_tables_skips_the_entry(orc):
    g = np.random.default_rng(30)
    B, H, C, D, S = 3, 2, 8, 4, 2
    cos, sin = rope_tables(100, 4)
    x = Transform(XF_F32, XF_INT8, cos, sin, 4, True, (0.1, 0.1))
    kn, vn = _window_case(g, B, H, C, S, D, XF_F32)
    past = np.array([10, 99, 98])  # entry 1 needs rows 99 and 100: one past the tables
    lp = np.array([3, 8, 8], np.int32)
    ev = np.array([0, 2, 2], np.int32)
    k = g.integers(-128, 127, (B, H, C, D), dtype=np.int8)
    v = g.integers(-128, 127, (B, H, C, D), dtype=np.int8)
    k0, v0 = k.copy(), v.copy()
    st = [np.zeros((B, H, C + S, D), np.int8) for _ in range(2)]
    f = orc.kv_window_append_xf(x, k, v, kn, vn, (H * S * D, S * D, D), S, lp, ev, past,
                                st[0], st[1])
    assert f == oracle.FLAG_ROPE_RANGE
    np.testing.assert_array_equal(k[1], k0[1])
    np.testing.assert_array_equal(v[1], v0[1])
    assert not np.array_equal(k[2], k0[2])  # the last in-range positions were written
    # bad lengths are reported as such, before the positions are looked at
    lp[1] = 9
    f = orc.kv_window_append_xf(x, k, v, kn, vn, (H * S * D, S * D, D), S, lp, ev, past,
                                st[0], st[1])
    assert f == oracle.FLAG_BAD_LENGTHS


# -- fused TensorScatter ------------------------------------------------------
@pytest.mark.parametrize("mode", ["linear", "circular"])
def test_scatter_identity_transform_is_plain_tensorscatter(orc, mode):
    g = np.random.default_rng(40)
    B, H, M, S, D = 3, 2, 7, 3, 5
    past = g.standard_normal((B, H, M, D)).astype(np.float16)
    upd = g.standard_normal((B, H, S, D)).astype(np.float16)
    w = np.array([0, 4, 9 if mode == "circular" else 2])
    for t in (0, 1):
        present = np.empty_like(past)
        st, f = orc.tensor_scatter_xf(Transform(XF_F16, XF_F16), t, present, past, upd, w, mode)
        want, fw = orc.tensor_scatter(past, upd, w, axis=-2, mode=mode)
        assert st == 0 and f == fw == 0
        np.testing.assert_array_equal(present, want)


def test_scatter_positions_are_absolute_before_the_wrap(orc):
    g = np.random.default_rng(41)
    B, H, M, S, D = 2, 2, 6, 3, 8
    cos, sin = random_tables(g, 64, 8)
    x = Transform(XF_F32, XF_F32, cos, sin, 8)
    past = np.zeros((B, H, M, D), np.float32)
    upd = np.zeros((B, H, S, D), np.float32)
    upd[..., 0] = 1.0  # one-hot on the first element of pair 0
    w = np.array([17, 40])  # ring positions 17.. and 40..: slots (w + s) mod 6
    present = past.copy()
    st, f = orc.tensor_scatter_xf(x, 0, present, present, upd, w, "circular")
    assert st == 0 and f == 0
    for b in range(B):
        for s in range(S):
            row = present[b, 0, (w[b] + s) % M]
            assert row[0] == cos[w[b] + s, 0] and row[4] == sin[w[b] + s, 0]


def test_scatter_position_out_of_tables_keeps_past(orc):
    g = np.random.default_rng(42)
    B, H, M, S, D = 3, 1, 30, 2, 4
    cos, sin = rope_tables(20, 4)
    x = Transform(XF_F32, XF_UINT8, cos, sin, 4, False, (0.1, 0.1), (128, 128))
    past = g.integers(0, 255, (B, H, M, D), dtype=np.uint8)
    upd = g.standard_normal((B, H, S, D)).astype(np.float32)
    # entry 1: positions 19, 20 (the tables end at 19); entry 2: rows 29, 30 of 30
    w = np.array([3, 19, 29])
    present = np.zeros_like(past)
    st, f = orc.tensor_scatter_xf(x, 1, present, past, upd, w, "linear")
    assert st == 0 and f == oracle.FLAG_ROPE_RANGE | oracle.FLAG_LINEAR_OOB
    np.testing.assert_array_equal(present[1:], past[1:])
    assert not np.array_equal(present[0], past[0])


# -- per-channel parameters and the fp8 target ----------------------------------
# The pull request "GQA support sliding_window_cache" (comment-only follow-up)
# gives the quantized cache's per-channel scales the shape (kv_num_heads, 1,
# head_size), the singleton dimension flattened: element i of a row of KV
# head h takes entry h * head_size + i.

def _codes(orc, x, t, head, rows):
    """Rows [n, D] of in_type through the transform as KV head ``head``."""
    D = rows.shape[1]
    out = np.zeros((len(rows), D), NP.get(x.out_type, np.uint8))
    for i, r in enumerate(rows):
        assert orc.xf_row(x, t, 0, np.ascontiguousarray(r), out[i], head=head) == oracle.OK
    return out


@pytest.mark.parametrize("out_type", [XF_INT8, XF_UINT8, oracle.XF_FP8_E4M3])
def test_per_channel_tables_of_one_value_are_the_scalar(orc, out_type):
    """Tables holding one value everywhere give exactly the scalar
    transform's bytes, through the windowed append and TensorScatter."""
    g = np.random.default_rng(60)
    B, H, C, S, D = 3, 2, 8, 2, 6
    zp = (0, 0) if out_type != XF_UINT8 else (120, 131)
    sc = (0.05, 0.02)
    xs = Transform(XF_F32, out_type, scale=sc, zero_point=zp)
    tabs = tuple(np.full((H, D), v, np.float32) for v in sc)
    ztabs = tuple(np.full((H, D), v, np.int32) for v in zp) if out_type != oracle.XF_FP8_E4M3 \
        else (None, None)
    xc = Transform(XF_F32, out_type, scale=(1.0, 1.0), zero_point=(0, 0) if ztabs[0] is not None
                   else zp, channel_scale=tabs, channel_zero_point=ztabs)
    kn, vn = (g.standard_normal((B, H, S, D)).astype(np.float32) * 3 for _ in range(2))
    T = np.array([2, 9, 30]) + S - 1
    L = orc.kv_seq_lengths(T - 1, S, C)
    base = g.integers(0, 255, (B, H, C, D), dtype=np.uint8)
    outs = []
    for x in (xs, xc):
        k, v = base.copy(), base.copy()
        st = [np.zeros((B, H, C + S, D), np.uint8) for _ in range(2)]
        assert orc.kv_window_append_xf(x, k, v, kn, vn, (H * S * D, S * D, D), S, L.cache_past,
                                       L.evict, L.past, st[0], st[1]) == 0
        pres = base.copy()
        code, f = orc.tensor_scatter_xf(x, 1, pres, pres, vn, np.array([1, 0, 5]), "linear")
        assert code == 0 and f == 0
        outs.append((k, v, st[0], pres))
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("out_type,lo,hi", [(XF_INT8, -128, 127), (XF_UINT8, 0, 255)])
def test_per_channel_reconstruction_within_half_of_each_channels_scale(orc, out_type, lo, hi):
    g = np.random.default_rng(61)
    H, D, n = 3, 16, 40
    tab = (2.0 ** g.uniform(-8, -2, (H, D))).astype(np.float32)
    ztab = g.integers(lo + 20, hi - 20, (H, D)).astype(np.int32)
    x = Transform(XF_F32, out_type, channel_scale=(tab, tab), channel_zero_point=(ztab, ztab))
    for h in range(H):
        rows = (g.uniform(-1, 1, (n, D)) * tab[h] * 60).astype(np.float32)
        codes = _codes(orc, x, 1, h, rows).astype(np.int64)
        rec = (codes - ztab[h]) * tab[h].astype(np.float64)
        inside = (codes > lo) & (codes < hi)
        assert inside.mean() > 0.8
        assert (np.abs(rec - rows)[inside] <= tab[h][None, :].repeat(n, 0)[inside] / 2 + 1e-12).all()


def test_per_channel_channels_and_heads_are_independent(orc):
    """Changing one channel's scale of one head changes only that element of
    that head's rows (K and V alike); a head reads its own table row."""
    g = np.random.default_rng(62)
    H, D = 3, 8
    tab = np.full((H, D), 0.05, np.float32)
    rows = (g.standard_normal((20, D)) * 2).astype(np.float32)
    x0 = Transform(XF_F32, XF_INT8, channel_scale=(tab, tab))
    ref = [[_codes(orc, x0, t, h, rows) for h in range(H)] for t in range(2)]
    tab2 = tab.copy()
    tab2[1, 5] = 0.2
    x1 = Transform(XF_F32, XF_INT8, channel_scale=(tab2, tab))
    for t in range(2):
        for h in range(H):
            got = _codes(orc, x1, t, h, rows)
            changed = np.argwhere((got != ref[t][h]).any(axis=0)).ravel().tolist()
            assert changed == ([5] if (t, h) == (0, 1) else [])
    # per-head constant tables equal the scalar transform of that head's value
    tab3 = np.repeat(np.array([[0.01], [0.1], [0.03]], np.float32), D, axis=1)
    x3 = Transform(XF_F32, XF_INT8, channel_scale=(tab3, tab3))
    for h in range(H):
        xs = Transform(XF_F32, XF_INT8, scale=(float(tab3[h, 0]),) * 2)
        np.testing.assert_array_equal(_codes(orc, x3, 0, h, rows), _codes(orc, xs, 0, 0, rows))


def test_per_channel_scatter_reads_the_head_of_prefix_index_one(orc):
    """TensorScatter of [B, H, M, D] caches: rows of prefix (b, h) use table
    row h; a rank-5 cache takes no tables."""
    g = np.random.default_rng(63)
    B, H, M, S, D = 2, 3, 6, 2, 4
    tab = (2.0 ** g.uniform(-6, -2, (H, D))).astype(np.float32)
    x = Transform(XF_F32, XF_INT8, channel_scale=(tab, tab))
    upd = g.standard_normal((B, H, S, D)).astype(np.float32)
    past = np.zeros((B, H, M, D), np.int8)
    pres = past.copy()
    w = np.array([1, 3])
    code, f = orc.tensor_scatter_xf(x, 0, pres, pres, upd, w, "linear")
    assert code == 0 and f == 0
    for b in range(B):
        for h in range(H):
            want = _codes(orc, x, 0, h, upd[b, h])
            np.testing.assert_array_equal(pres[b, h, w[b]:w[b] + S], want)
    p5 = np.zeros((B, 1, H, M, D), np.int8)
    code, _ = orc.tensor_scatter_xf(x, 0, p5, p5, upd[:, None], w, "linear")
    assert code == oracle.E_INVALID_ARG


def _e4m3_decode_torch(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_fp8_every_code_round_trips(orc):
    """All 256 E4M3 codes, decoded by torch's float8_e4m3fn: each finite one
    encodes back to itself (scale 1), the two NaNs to the positive NaN."""
    codes = np.arange(256, dtype=np.uint8)
    vals = _e4m3_decode_torch(codes)
    x = Transform(XF_F32, oracle.XF_FP8_E4M3)
    got = _codes(orc, x, 0, 0, vals.reshape(32, 8)).view(np.uint8).ravel()
    finite = ~np.isnan(vals)
    np.testing.assert_array_equal(got[finite], codes[finite])
    assert (got[~finite] == 0x7F).all() and finite.sum() == 254


def test_fp8_rounds_like_torch_and_saturates(orc):
    """Inside the range torch's float32 -> float8_e4m3fn conversion (nearest
    even) gives the same codes, exact midpoints included; beyond +-448 and
    at the infinities the code saturates to +-448; NaN is 0x7F."""
    g = np.random.default_rng(64)
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    v = _e4m3_decode_torch(codes).astype(np.float64)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)  # exact in binary32
    rnd = (g.uniform(-463.9, 463.9, 4000) * 2.0 ** g.integers(-14, 1, 4000)).astype(np.float32)
    vals = np.concatenate([mids, -mids, rnd, [2.0 ** -10, 3 * 2.0 ** -10, -0.0, 0.0]]).astype(np.float32)
    vals = vals[: len(vals) // 8 * 8]
    x = Transform(XF_F32, oracle.XF_FP8_E4M3)
    got = _codes(orc, x, 0, 0, vals.reshape(-1, 8)).view(np.uint8).ravel()
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, want)
    big = np.array([448.0, 449.0, 463.9, 464.0, 1e30, np.inf, -500.0, -np.inf], np.float32)
    got = _codes(orc, x, 0, 0, big[None]).view(np.uint8).ravel()
    assert list(got) == [0x7E] * 6 + [0xFE] * 2
    nan = np.full((1, 8), np.nan, np.float32)
    assert (_codes(orc, x, 0, 0, nan).view(np.uint8) == 0x7F).all()


def test_fp8_applies_the_scale_first(orc):
    """The fp8 code of y is that of fl(y / scale), per channel too; a zero
    point is refused."""
    g = np.random.default_rng(65)
    rows = g.standard_normal((10, 8)).astype(np.float32) * 5
    tab = (2.0 ** g.uniform(-3, 3, (2, 8))).astype(np.float32)
    x = Transform(XF_F32, oracle.XF_FP8_E4M3, channel_scale=(tab, tab))
    for h in range(2):
        got = _codes(orc, x, 1, h, rows).view(np.uint8)
        want = torch.from_numpy((rows / tab[h]).astype(np.float32)).to(torch.float8_e4m3fn)
        np.testing.assert_array_equal(got, want.view(torch.uint8).numpy())
    bad = Transform(XF_F32, oracle.XF_FP8_E4M3, zero_point=(1, 0))
    out = np.zeros(8, np.uint8)
    assert orc.xf_row(bad, 0, 0, rows[0], out) == oracle.E_INVALID_ARG
    bad2 = Transform(XF_F32, XF_F32, channel_scale=(tab, None))  # no scale for a float target
    assert orc.xf_row(bad2, 0, 0, rows[0], np.zeros(8, np.float32)) == oracle.E_INVALID_ARG


@pytest.mark.parametrize("out_type", [XF_INT8, oracle.XF_FP8_E4M3])
def test_per_channel_window_rows_use_their_heads_tables(orc, out_type):
    """The windowed append with per-channel tables: the appended rows of KV
    head h are the rows transformed with table row h, the rest is the plain
    step."""
    g = np.random.default_rng(66)
    B, H, C, S, D = 3, 3, 8, 2, 8
    tab = [(2.0 ** g.uniform(-6, -1, (H, D))).astype(np.float32) for _ in range(2)]
    z = None if out_type == oracle.XF_FP8_E4M3 else \
        tuple(g.integers(-20, 20, (H, D)).astype(np.int32) for _ in range(2))
    x = Transform(XF_F32, out_type, channel_scale=tuple(tab),
                  channel_zero_point=z if z is not None else (None, None))
    kn, vn = (g.standard_normal((B, H, S, D)).astype(np.float32) for _ in range(2))
    T = np.array([2, 9, 30]) + S - 1
    L = orc.kv_seq_lengths(T - 1, S, C)
    base = g.integers(0, 255, (B, H, C, D), dtype=np.uint8)
    k1, v1 = base.copy(), base.copy()
    st = [np.zeros((B, H, C + S, D), np.uint8) for _ in range(2)]
    assert orc.kv_window_append_xf(x, k1, v1, kn, vn, (H * S * D, S * D, D), S, L.cache_past,
                                   L.evict, L.past, st[0], st[1]) == 0
    rows = [np.zeros((B, H, S, D), np.uint8) for _ in range(2)]
    for t, new in enumerate((kn, vn)):
        for b in range(B):
            for h in range(H):
                rows[t][b, h] = _codes(orc, x, t, h, new[b, h]).view(np.uint8)
    k2, v2 = base.copy(), base.copy()
    st2 = [np.zeros_like(st[0]) for _ in range(2)]
    assert orc.kv_window_append(k2, v2, rows[0], rows[1], L.cache_past, L.evict, st2[0], st2[1],
                                elem_bits=8) == 0
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)


def test_nan_quotient_takes_the_saturated_zero_point(orc):
    """Per-channel tables are data: a scale that makes y / scale NaN (a NaN
    scale, or 0 / 0) gives the zero point like a NaN input does, and a zero
    point outside the code range saturates; a zero scale on a nonzero y gives
    an infinite quotient and so a saturated code."""
    D = 8
    tab = np.float32([np.nan, 0.0, 0.0, 0.5, 0.5, 0.5, -0.5, np.inf])[None]
    z = np.int32([3, 4, 5, 300, -300, 7, 0, 9])[None]
    x = Transform(XF_F32, XF_INT8, channel_scale=(tab, tab), channel_zero_point=(z, z))
    row = np.float32([1.0, 0.0, 2.0, np.nan, np.nan, 1.0, 1.0, 5.0])[None]
    got = _codes(orc, x, 0, 0, row).astype(np.int64).ravel()
    assert list(got) == [3, 4, 127, 127, -128, 9, -2, 9]
