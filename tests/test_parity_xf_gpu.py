"""GPU parity of the fused append (RoPE on K at the absolute position, then
conversion or affine quantization into the cache's dtype) against the CPU
oracle, byte for byte.

Every float operation of the transform is fixed (binary32, one rounding per
product and sum, correctly rounded division, round half to even), so the
rounded elements and the quantized codes are unique and the tolerance is 0:
whole caches, staging buffers and flag words are compared as bytes. Inputs
mix ordinary values with infinities, NaNs, huge and subnormal values and
exact rounding ties; positions run far past the capacity.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_ring_tensor_amd as swrt
from sliding_window_ring_tensor_amd import workloads as wl
from sliding_window_ring_tensor_amd.decode_step import ModelDecodeStep
from tests.test_parity_gpu import DEV, Guarded, flag_word, hb, say

pytestmark = pytest.mark.gpu

FLOAT_IN = [torch.float32, torch.float16, torch.bfloat16]
OUT = [torch.float32, torch.float16, torch.bfloat16, torch.int8, torch.uint8,
       torch.float8_e4m3fn]
ORC_TYPE = {torch.float32: oracle.XF_F32, torch.float16: oracle.XF_F16,
            torch.bfloat16: oracle.XF_BF16, torch.int8: oracle.XF_INT8,
            torch.uint8: oracle.XF_UINT8, torch.float8_e4m3fn: oracle.XF_FP8_E4M3}
BYTE_OUT = (torch.int8, torch.uint8, torch.float8_e4m3fn)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    swrt.lib()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def new_rows(g, shape, dtype) -> torch.Tensor:
    """Host rows: mostly N(0, 2) values, with specials mixed in."""
    n = int(np.prod(shape))
    if dtype in (torch.float16, torch.bfloat16):
        v = torch.from_numpy(g.standard_normal(n).astype(np.float32) * 2).to(dtype)
        bits = v.view(torch.int16)
        raw = torch.from_numpy(g.integers(-32768, 32767, size=n, dtype=np.int16))
        pick = torch.from_numpy(g.random(n) < 0.1)
        bits = torch.where(pick, raw, bits)  # every 16-bit pattern can appear
        return bits.view(dtype).reshape(shape)
    v = g.standard_normal(n).astype(np.float32) * 2
    special = np.float32([np.inf, -np.inf, np.nan, 1e30, -1e30, 1e-40, -0.0, 65520.0,
                          1.00390625, 2.5 * 0.02, 3.5 * 0.01])
    idx = g.integers(0, n, size=max(1, n // 10))
    v[idx] = special[g.integers(0, len(special), size=idx.size)]
    return torch.from_numpy(v).reshape(shape)


def tables(positions, rot):
    return wl.rope_tables(positions, rot)


def channel_tables(g, H, D, out, special=False):
    """Per-channel (scales, zero points) for K and V, [H, D] each: scales of
    2^U[-8, -3), zero points inside the code range (None for fp8 and float
    targets). special: some entries zero, negative, NaN or huge, some zero
    points out of range (the tables are data; both sides apply the formula)."""
    if out not in BYTE_OUT:
        return (None, None), (None, None)
    sc = [(2.0 ** g.uniform(-8, -3, (H, D))).astype(np.float32) for _ in range(2)]
    zp = [None, None]
    if out != torch.float8_e4m3fn:
        lo, hi = (-128, 127) if out == torch.int8 else (0, 255)
        zp = [g.integers(lo, hi, (H, D), endpoint=True).astype(np.int32) for _ in range(2)]
    if special:
        for a in sc:
            a.flat[::7] = np.float32([0.0, -0.03, np.nan, 3e38, np.inf, 1e-30, -0.0])[
                np.arange(len(a.flat[::7])) % 7]
        for z in zp:
            if z is not None:
                z.flat[::5] = np.int32([-1000, 1000, 300, -300])[np.arange(len(z.flat[::5])) % 4]
    return tuple(sc), tuple(zp)


def make_xf(rot_mode, D, positions, out, zp=(0, 0), channels=None):
    """(device Transform, oracle Transform) for rot_mode None / 'half' / 'inter'.
    channels: per-channel tables as channel_tables returns them."""
    rot = 0 if rot_mode is None else (D if rot_mode == "half" else D - 4)
    cos = sin = None
    if rot:
        cos, sin = tables(positions, rot)
    if out == torch.uint8 and zp == (0, 0):
        zp = (128, 120)
    (ks, vs), (kz, vz) = channels if channels is not None else ((None, None), (None, None))
    dv = lambda a: None if a is None else torch.from_numpy(a).to(DEV)  # noqa: E731
    dev = swrt.Transform(None if cos is None else cos.to(DEV), None if sin is None else sin.to(DEV),
                         rot_mode == "inter", 0.02, 0.01, *zp, dv(ks), dv(vs), dv(kz), dv(vz))
    return dev, lambda in_dt, out_dt: oracle.Transform(
        ORC_TYPE[in_dt], ORC_TYPE[out_dt], None if cos is None else cos.numpy(),
        None if sin is None else sin.numpy(), rot, rot_mode == "inter", (0.02, 0.01), zp,
        (ks, vs), (kz, vz))


def host_np(t: torch.Tensor) -> np.ndarray:
    """A numpy array the oracle can take (bf16 as raw uint16, fp8 as uint8)."""
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
    return t.numpy().copy()


# ---------------------------------------------------------------------------
# TensorScatter with the transform
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rot_mode", [None, "half", "inter"])
@pytest.mark.parametrize("out", OUT, ids=str)
@pytest.mark.parametrize("inp", FLOAT_IN, ids=str)
def test_scatter_xf_every_conversion(orc, inp, out, rot_mode):
    say("scatter xf", inp, out, rot_mode)
    g = wl.rng(100 * FLOAT_IN.index(inp) + 10 * OUT.index(out) + [None, "half", "inter"].index(rot_mode))
    B, H, M, S, D = 3, 2, 40, 3, 20
    xd, xo = make_xf(rot_mode, D, 300, out)
    for mode, w in (("linear", [0, 17, 37]), ("circular", [5, 39, 250])):
        w = np.array(w, np.int64)
        pasts = [wl.host_payload(g, (B, H, M, D), out, raw_bits=True) for _ in range(2)]
        upds = [new_rows(g, (B, H, S, D), inp) for _ in range(2)]
        for in_place in (True, False):
            dp = [Guarded(p, seed=i) for i, p in enumerate(pasts)]
            du = [u.to(DEV) for u in upds]
            outs = [p.t for p in dp] if in_place else [Guarded(None, p.shape, out, seed=9 + i)
                                                        for i, p in enumerate(pasts)]
            flags = flag_word()
            swrt.tensor_scatter_xf([p.t for p in dp], du, [0, 1], torch.from_numpy(w).to(DEV),
                                   xd, mode=mode,
                                   outs=outs if in_place else [o.t for o in outs], flags=flags)
            torch.cuda.synchronize()
            for t in range(2):
                want = host_np(pasts[t])
                st, f = orc.tensor_scatter_xf(xo(inp, out), t, want, want, host_np(upds[t]), w,
                                              mode)
                assert st == 0 and f == flags.item() == 0
                got = dp[t].t if in_place else outs[t].t
                np.testing.assert_array_equal(hb(got), want.view(np.uint8).reshape(hb(got).shape))
                dp[t].check("past")
                if not in_place:
                    outs[t].check("present")


@pytest.mark.parametrize("special", [False, True])
@pytest.mark.parametrize("out", BYTE_OUT, ids=str)
def test_scatter_xf_per_channel(orc, out, special):
    """Per-channel scales (and zero points) [H, D]: rows of cache head h read
    table row h; rank 3 caches read one row. special: zero, negative, NaN and
    huge scales, zero points out of range -- data both sides put through the
    same formula."""
    say("scatter xf per channel", out, special)
    g = wl.rng(150 + BYTE_OUT.index(out) + 10 * special)
    for shape in ((3, 4, 40, 24), (5, 33, 16)):
        H = shape[1] if len(shape) == 4 else 1
        D, S = shape[-1], 3
        ch = channel_tables(g, H, D, out, special)
        xd, xo = make_xf("half", D, 300, out, channels=ch)
        w = np.array([0, 17, 30, 1, 9][:shape[0]], np.int64)
        ushape = shape[:-2] + (S, D)
        pasts = [wl.host_payload(g, shape, out, raw_bits=True) for _ in range(2)]
        upds = [new_rows(g, ushape, torch.float32) for _ in range(2)]
        dp = [p.to(DEV) for p in pasts]
        flags = flag_word()
        swrt.tensor_scatter_xf(dp, [u.to(DEV) for u in upds], [0, 1], torch.from_numpy(w).to(DEV),
                               xd, outs=dp, flags=flags)
        torch.cuda.synchronize()
        for t in range(2):
            want = host_np(pasts[t])
            st, f = orc.tensor_scatter_xf(xo(torch.float32, out), t, want, want, host_np(upds[t]),
                                          w, "linear")
            assert st == 0 and f == flags.item() == 0
            np.testing.assert_array_equal(hb(dp[t]), want.view(np.uint8).reshape(hb(dp[t]).shape))


def test_scatter_xf_position_range_and_linear_bounds(orc):
    g = wl.rng(11)
    B, H, M, S, D = 4, 2, 30, 2, 8
    xd, xo = make_xf("half", D, 20, torch.int8)
    past = wl.host_payload(g, (B, H, M, D), torch.int8, raw_bits=True)
    upd = new_rows(g, (B, H, S, D), torch.float32)
    w = np.array([3, 19, 29, -1], np.int64)  # in range, past the tables, past M, negative
    d = past.to(DEV)
    flags = flag_word()
    swrt.tensor_scatter_xf([d], [upd.to(DEV)], [0], torch.from_numpy(w).to(DEV), xd, outs=[d],
                           flags=flags)
    want = host_np(past)
    st, f = orc.tensor_scatter_xf(xo(torch.float32, torch.int8), 0, want, want, host_np(upd), w)
    torch.cuda.synchronize()
    assert st == 0 and f == flags.item() == swrt.FLAG_ROPE_RANGE | swrt.FLAG_LINEAR_OOB
    np.testing.assert_array_equal(hb(d), want.view(np.uint8))


# ---------------------------------------------------------------------------
# windowed append with the transform
# ---------------------------------------------------------------------------
def _window_case(orc, g, B, H, C, S, D, inp, out, rot_mode, T, n_layers=1, phase_split=False,
                 strides_bsnh=False, positions=9000, stage_step=False, channels=None):
    """stage_step: the lengths and the stage phase in one launch, then the
    commit. channels: per-channel tables (channel_tables)."""
    xd, xo = make_xf(rot_mode, D, positions, out, channels=channels)
    sk = (np.asarray(T) - 1).astype(np.int32)
    lens = swrt.kv_seq_lengths(torch.from_numpy(sk).to(DEV), S, C)
    L = orc.kv_seq_lengths(sk, S, C)
    kc = [wl.host_payload(g, (B, H, C, D), out, raw_bits=True) for _ in range(n_layers)]
    vc = [wl.host_payload(g, (B, H, C, D), out, raw_bits=True) for _ in range(n_layers)]
    # new rows: contiguous BNSH, or contiguous BSNH seen as [B, H, S, D]
    base_shape = (B, S, H, D) if strides_bsnh else (B, H, S, D)
    kb = [new_rows(g, base_shape, inp) for _ in range(n_layers)]
    vb = [new_rows(g, base_shape, inp) for _ in range(n_layers)]
    view = (lambda t: t.transpose(1, 2)) if strides_bsnh else (lambda t: t)
    ks = [wl.host_payload(g, (B, H, C + S, D), out, raw_bits=True) for _ in range(n_layers)]
    vs = [wl.host_payload(g, (B, H, C + S, D), out, raw_bits=True) for _ in range(n_layers)]
    dk = [Guarded(t, seed=1 + i) for i, t in enumerate(kc)]
    dv = [Guarded(t, seed=40 + i) for i, t in enumerate(vc)]
    dks = [Guarded(t, seed=80 + i) for i, t in enumerate(ks)] if S > 1 else None
    dvs = [Guarded(t, seed=120 + i) for i, t in enumerate(vs)] if S > 1 else None
    flags = flag_word()
    dkn = [view(t.to(DEV)) for t in kb]
    dvn = [view(t.to(DEV)) for t in vb]
    phases = ("stage", "commit") if ((phase_split or stage_step) and S > 1) else ("all",)
    if stage_step:
        got = swrt.kv_window_stage_step_xf([t.t for t in dk], [t.t for t in dv], dkn, dvn,
                                           torch.from_numpy(sk).to(DEV), [t.t for t in dks],
                                           [t.t for t in dvs], xd, flags=flags)
        lens = got
        phases_run = ("commit",)
        for x, y in zip(got, (L.total, L.past, L.cache_past, L.cache_total, L.evict)):
            np.testing.assert_array_equal(x.cpu().numpy(), y)
    else:
        phases_run = phases
    for ph in phases_run:
        swrt.kv_window_append_xf([t.t for t in dk], [t.t for t in dv], dkn, dvn, lens.cache_past,
                                 lens.evict, lens.past, xd,
                                 k_stagings=None if dks is None else [t.t for t in dks],
                                 v_stagings=None if dvs is None else [t.t for t in dvs],
                                 phase=ph, flags=flags)
    torch.cuda.synchronize()
    fl = L.flags if stage_step else 0  # the lengths' own flag comes from the same launch
    for i in range(n_layers):
        hk, hv = host_np(kc[i]), host_np(vc[i])
        hks, hvs = (host_np(ks[i]), host_np(vs[i])) if S > 1 else (None, None)
        knn, vnn = host_np(kb[i]), host_np(vb[i])  # the buffers, read through the strides
        strides = tuple(view(kb[i]).stride()[:3])
        for ph in phases:
            fl |= orc.kv_window_append_xf(
                xo(inp, out), hk, hv, knn, vnn, strides, S, L.cache_past, L.evict, L.past, hks,
                hvs, {"all": oracle.PHASE_ALL, "stage": oracle.PHASE_STAGE,
                      "commit": oracle.PHASE_COMMIT}[ph])
        np.testing.assert_array_equal(hb(dk[i].t), hk.view(np.uint8).reshape(hb(dk[i].t).shape))
        np.testing.assert_array_equal(hb(dv[i].t), hv.view(np.uint8).reshape(hb(dv[i].t).shape))
        if S > 1:
            np.testing.assert_array_equal(hb(dks[i].t),
                                          hks.view(np.uint8).reshape(hb(dks[i].t).shape))
            np.testing.assert_array_equal(hb(dvs[i].t),
                                          hvs.view(np.uint8).reshape(hb(dvs[i].t).shape))
        for t in (dk[i], dv[i]) + ((dks[i], dvs[i]) if S > 1 else ()):
            t.check("window buffer")
    assert flags.item() == fl
    return fl


@pytest.mark.parametrize("rot_mode", [None, "half", "inter"])
@pytest.mark.parametrize("out", OUT, ids=str)
@pytest.mark.parametrize("inp", [torch.float32, torch.bfloat16], ids=str)
def test_window_xf_decode(orc, inp, out, rot_mode):
    say("window xf S=1", inp, out, rot_mode)
    g = wl.rng(21 + OUT.index(out))
    T = [1, 5, 16, 17, 4000, 8999, 9001, 700]  # 9001: the position leaves the tables
    f = _window_case(orc, g, 8, 2, 16, 1, 12, inp, out, rot_mode, T, n_layers=2)
    assert (f == swrt.FLAG_ROPE_RANGE) == (rot_mode is not None)


@pytest.mark.parametrize("phase_split", [False, True])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.int8, torch.float32], ids=str)
def test_window_xf_staged(orc, out, phase_split):
    say("window xf staged", out, phase_split)
    g = wl.rng(31)
    T = [3, 10, 40, 41, 2000, 8990, 9003, 60]  # 9003: P + S past the tables
    f = _window_case(orc, g, 8, 2, 24, 7, 16, torch.bfloat16, out, "half", T, n_layers=2,
                     phase_split=phase_split, strides_bsnh=True)
    assert f == swrt.FLAG_ROPE_RANGE


@pytest.mark.parametrize("out", [torch.bfloat16, torch.int8, torch.uint8], ids=str)
def test_window_xf_stage_step(orc, out):
    """The lengths and the fused stage phase in one launch, then the fused commit."""
    say("window xf stage step", out)
    g = wl.rng(33)
    T = [3, 10, 40, 41, 2000, 8990, 9003, 60]  # 3: T < S; 9003: P + S past the tables
    f = _window_case(orc, g, 8, 2, 24, 7, 16, torch.bfloat16, out, "half", T, n_layers=2,
                     strides_bsnh=True, stage_step=True)
    assert f == swrt.FLAG_ROPE_RANGE | swrt.FLAG_BAD_SEQLEN


@pytest.mark.parametrize("S,C", [(1, 128), (1, 16), (5, 24)], ids=str)
@pytest.mark.parametrize("out", BYTE_OUT, ids=str)
def test_window_xf_per_channel(orc, out, S, C):
    """The windowed append with per-channel tables: in place (one slice per
    workgroup, and slices sharing a workgroup at C = 16) and staged, with
    rotation, special table entries included."""
    say("window xf per channel", out, S, C)
    g = wl.rng(160 + BYTE_OUT.index(out) + S + C)
    B, H, D = 6, 4, 64
    T = g.integers(1, 3 * C, size=B)
    T[:2] = [C, C + 1]
    ch = channel_tables(g, H, D, out, special=True)
    _window_case(orc, g, B, H, C, S, D, torch.bfloat16, out, "half", T, positions=8 * C,
                 channels=ch, n_layers=2)


def fused_slices_per_group(C, row_bytes, D):
    """The launch's split of a 512-thread workgroup into subgroups for a fused
    append (host arithmetic): a subgroup of 512 / spw lanes holds a whole
    shift at four 16-byte words a lane and one element of the row a lane."""
    row_words = -(-row_bytes // 16)
    spw = 1
    while spw < 4 and (C - 1) * row_words <= (512 // (2 * spw)) * 4 and \
            row_words <= 512 // (2 * spw) and D <= 512 // (2 * spw):
        spw *= 2
    return spw


@pytest.mark.parametrize("case", ["group2", "group4", "wide_rows", "odd_words"])
def test_window_xf_shapes(orc, case):
    """Slices shared by 2 or 4 subgroups (int8 rows of 64 and 32 bytes), rows
    wider than one pass of the workgroup, and 2-byte copy words."""
    g = wl.rng(41)
    B, H, C, D, out, rot = {"group2": (6, 3, 200, 64, torch.int8, "half"),
                            "group4": (6, 3, 64, 32, torch.uint8, "inter"),
                            "wide_rows": (2, 2, 3, 2304, torch.float32, "half"),
                            "odd_words": (5, 2, 9, 6, torch.bfloat16, "inter")}[case]
    if case.startswith("group"):
        assert fused_slices_per_group(C, D, D) == int(case[-1])
    say("window xf", case)
    T = g.integers(1, 4 * C, size=B)
    T[:2] = [C, C + 1]
    _window_case(orc, g, B, H, C, 1, D, torch.bfloat16, out, rot, T, positions=8 * C)


def test_window_xf_bad_lengths_before_positions(orc):
    g = wl.rng(51)
    B, H, C, S, D = 4, 2, 8, 1, 8
    xd, xo = make_xf("half", D, 50, torch.int8)
    kc = wl.host_payload(g, (B, H, C, D), torch.int8, raw_bits=True)
    vc = wl.host_payload(g, (B, H, C, D), torch.int8, raw_bits=True)
    kn, vn = new_rows(g, (B, H, S, D), torch.float32), new_rows(g, (B, H, S, D), torch.float32)
    lp = np.array([3, 9, 8, 8], np.int32)    # entry 1: Lp > C
    ev = np.array([0, 0, 1, 1], np.int32)
    past = np.array([3, 49, 49, 50], np.int64)  # entry 3: position 50 leaves the tables
    dk, dv = kc.to(DEV), vc.to(DEV)
    flags = flag_word()
    swrt.kv_window_append_xf([dk], [dv], [kn.to(DEV)], [vn.to(DEV)], torch.from_numpy(lp).to(DEV),
                             torch.from_numpy(ev).to(DEV), torch.from_numpy(past).to(DEV), xd,
                             flags=flags)
    hk, hv = host_np(kc), host_np(vc)
    f = orc.kv_window_append_xf(xo(torch.float32, torch.int8), hk, hv, host_np(kn), host_np(vn),
                                (H * S * D, S * D, D), S, lp, ev, past)
    torch.cuda.synchronize()
    assert f == flags.item() == swrt.FLAG_BAD_LENGTHS | swrt.FLAG_ROPE_RANGE
    np.testing.assert_array_equal(hb(dk), hk.view(np.uint8))
    np.testing.assert_array_equal(hb(dv), hv.view(np.uint8))


@pytest.mark.parametrize("D", [192, 1040])
def test_xf_wide_rows_in_shared_workgroups(orc, D):
    """A slice small enough to share a workgroup (C = 4) with an appended row
    wider than a quarter workgroup's lanes (int8, D = 192: two slices a
    workgroup then; D = 1040: one, a few elements a lane): the launch keeps a
    lane per element of the row for every slice, in the windowed append and
    in the one-launch step."""
    B, H, C = 3, 2, 4
    # host arithmetic: 16-byte words per row, and the subgroup split that the
    # plain copy alone would choose (four slices of 128 lanes, fewer than D)
    row_words = D // 16
    spw = 1
    while spw < 4 and (C - 1) * row_words <= (512 // (2 * spw)) * 2 and \
            row_words <= 512 // (2 * spw):
        spw *= 2
    assert spw == 4 and D > 512 // spw
    g = wl.rng(45)
    T = np.array([1, 4, 5, 9, 2, 3])[:B]
    say("window xf wide rows in shared workgroups", D)
    _window_case(orc, g, B, H, C, 1, D, torch.bfloat16, torch.int8, "half", T, positions=64)
    xd, xo = make_xf("half", D, 64, torch.int8)
    sk = (T - 1).astype(np.int32)
    wc = [wl.host_payload(g, (B, H, C, D), torch.int8, raw_bits=True) for _ in range(2)]
    wn = [new_rows(g, (B, H, 1, D), torch.bfloat16) for _ in range(2)]
    dc, dn = [t.to(DEV) for t in wc], [t.to(DEV) for t in wn]
    flags = flag_word()
    swrt.kv_decode_step_xf([dc[0]], [dc[1]], [dn[0]], [dn[1]], torch.from_numpy(sk).to(DEV), [],
                           [], [], [], None, xd, flags=flags)
    L = orc.kv_seq_lengths(sk, 1, C)
    hc = [host_np(t) for t in wc]
    f = orc.kv_window_append_xf(xo(torch.bfloat16, torch.int8), hc[0], hc[1], host_np(wn[0]),
                                host_np(wn[1]), (H * D, D, D), 1, L.cache_past, L.evict, L.past)
    torch.cuda.synchronize()
    assert f == flags.item() == 0
    for x, y in zip(dc, hc):
        np.testing.assert_array_equal(hb(x), y.view(np.uint8))


# ---------------------------------------------------------------------------
# the one-launch decode step with the transform
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["base", "drift"])
@pytest.mark.parametrize("out,D,chan", [(torch.int8, 64, False), (torch.bfloat16, 64, False),
                                        (torch.uint8, 32, False), (torch.float32, 512, False),
                                        (torch.float16, 6, False),
                                        (torch.float8_e4m3fn, 64, False),
                                        (torch.int8, 64, True), (torch.uint8, 32, True),
                                        (torch.float8_e4m3fn, 64, True)], ids=str)
def test_decode_step_xf(orc, out, D, chan, layout):
    """One launch against the three fused calls and against the oracle
    (chan: per-channel scales and zero points)."""
    say("decode step xf", out, D, chan, layout)
    g = wl.rng(61 + D)
    B, H, M, nw, nf = 12, 2, 300, 2, 2
    W = 64
    C = W if layout == "base" else W + 16
    xd, xo = make_xf("half" if D % 4 == 0 else "inter", D, 2000, out,
                     channels=channel_tables(g, H, D, out) if chan else None)
    T = g.integers(1, 1900, size=B)
    T[:4] = [C, C + 1, 2001, 1]  # 2001: past the tables
    sk = (T - 1).astype(np.int32)
    wi = ((T - 1) % M).astype(np.int64)
    mk = lambda shape, dt: wl.host_payload(g, shape, dt, raw_bits=True) if dt == out \
        else new_rows(g, shape, dt)  # noqa: E731
    host = ([mk((B, H, C, D), out) for _ in range(2 * nw)], [mk((B, H, 1, D), torch.bfloat16)
                                                            for _ in range(2 * nw)],
            [mk((B, H, M, D), out) for _ in range(2 * nf)], [mk((B, H, 1, D), torch.bfloat16)
                                                            for _ in range(2 * nf)])
    window = None if layout == "base" else W
    results = []
    for fused in (True, False):
        wc, wn, fc, fn = [[t.to(DEV) for t in grp] for grp in host]
        sk_d, wi_d = torch.from_numpy(sk).to(DEV), torch.from_numpy(wi).to(DEV)
        flags = flag_word()
        if fused:
            lens = swrt.kv_decode_step_xf(wc[:nw], wc[nw:], wn[:nw], wn[nw:], sk_d, fc[:nf],
                                          fc[nf:], fn[:nf], fn[nf:], wi_d, xd, window=window,
                                          flags=flags)
        else:
            lens = swrt.kv_seq_lengths(sk_d, 1, C, window=window, flags=flags)
            swrt.kv_window_append_xf(wc[:nw], wc[nw:], wn[:nw], wn[nw:], lens.cache_past,
                                     lens.evict, lens.past, xd, flags=flags)
            swrt.tensor_scatter_xf(fc, fn, [0] * nf + [1] * nf, wi_d, xd, outs=fc, flags=flags)
        torch.cuda.synchronize()
        results.append(([hb(t) for t in (*wc, *fc, *lens)], flags.item()))
    (a, fa), (b3, fb) = results
    assert fa == fb
    for x, y in zip(a, b3):
        np.testing.assert_array_equal(x, y)
    L = orc.kv_seq_lengths(sk, 1, C) if window is None else orc.kv_seq_lengths_drift(sk, 1, C, W)
    wc, wn, fc, fn = [[host_np(t) for t in grp] for grp in host]
    f = 0
    for i in range(nw):
        f |= orc.kv_window_append_xf(xo(torch.bfloat16, out), wc[i], wc[nw + i], wn[i],
                                     wn[nw + i], (H * D, D, D), 1, L.cache_past, L.evict, L.past)
    for i in range(2 * nf):
        st, fl = orc.tensor_scatter_xf(xo(torch.bfloat16, out), i // nf, fc[i], fc[i], fn[i], wi)
        assert st == 0
        f |= fl
    assert fa == f == swrt.FLAG_ROPE_RANGE
    for x, y in zip(a, [*wc, *fc]):
        np.testing.assert_array_equal(x, y.view(np.uint8).reshape(x.shape))


def test_workload7_full_size(orc):
    """The fused-append model step at full size, in the launch configuration
    the benchmark times: one launch against three, whole windowed caches and
    two whole full layers; the oracle on every windowed layer and on the
    written row of every full cache."""
    spec = wl.workload7()
    say("workload 7 full size")
    a = ModelDecodeStep(spec, DEV, set_id=0)
    b = ModelDecodeStep(spec, DEV, set_id=0)
    win_before = [host_np(t) for t in a.buffers.win_k + a.buffers.win_v]
    a.run_fused()
    b.run_three()
    torch.cuda.synchronize()
    assert a.buffers.flags.item() == b.buffers.flags.item() == 0
    for x, y in zip(a.buffers.win_k + a.buffers.win_v, b.buffers.win_k + b.buffers.win_v):
        assert torch.equal(x, y)
    for x, y in zip(a.buffers.full_k[:2] + a.buffers.full_v[:2],
                    b.buffers.full_k[:2] + b.buffers.full_v[:2]):
        assert torch.equal(x, y)
    for x, y in zip(a.buffers.lengths, b.buffers.lengths):
        assert torch.equal(x, y)
    xd = a.buffers.xf
    xo = oracle.Transform(oracle.XF_BF16, oracle.XF_INT8, xd.cos.cpu().numpy(),
                          xd.sin.cpu().numpy(), spec.rotary_dim, False,
                          (spec.k_scale, spec.v_scale), (0, 0))
    L = orc.kv_seq_lengths(spec.seqlens_k, 1, spec.window)
    nw = len(spec.windowed_layers)
    for i in range(nw):
        hk, hv = win_before[i], win_before[nw + i]
        assert orc.kv_window_append_xf(xo, hk, hv, host_np(a.buffers.win_kn[i]),
                                       host_np(a.buffers.win_vn[i]),
                                       (spec.kv_heads * spec.head_dim, spec.head_dim,
                                        spec.head_dim), 1, L.cache_past, L.evict, L.past) == 0
        np.testing.assert_array_equal(host_np(a.buffers.win_k[i]), hk)
        np.testing.assert_array_equal(host_np(a.buffers.win_v[i]), hv)
    T = spec.total_lens
    rows = torch.arange(spec.batch, device=DEV)
    for t, (caches, news) in enumerate(((a.buffers.full_k, a.buffers.full_kn),
                                        (a.buffers.full_v, a.buffers.full_vn))):
        for c, n in zip(caches, news):
            got = c[rows, :, torch.from_numpy(T - 1).to(DEV)].cpu().numpy()  # [B, H, D]
            hn = host_np(n)
            for bb in range(spec.batch):
                for h in range(spec.kv_heads):
                    want = np.zeros(spec.head_dim, np.int8)
                    assert orc.xf_row(xo, t, int(T[bb] - 1), hn[bb, h, 0], want) == 0
                    np.testing.assert_array_equal(got[bb, h], want)
