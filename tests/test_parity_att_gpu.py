"""GPU parity of the windowed decode attention against the float64 oracle.

The kernels compute in binary32 and the oracle in float64, so outputs agree
within the tolerance of tests/att_bound.py, per batch entry and query head:
the forward error of any binary32 streaming evaluation of the definition
(the precision the onnx-light-cpu roadmap's "Phase 1" prescribes), fixed from
the definition and not from the kernels' order of operations, plus the
output's own rounding for 16-bit outputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_ring_tensor_amd as swrt
from sliding_window_ring_tensor_amd import workloads as wl
from sliding_window_ring_tensor_amd.decode_step import ModelDecodeStep
from tests.att_bound import window_tolerance, with_output_rounding
from tests.test_parity_gpu import DEV, flag_word, say

pytestmark = pytest.mark.gpu
ORC = {torch.float32: oracle.XF_F32, torch.float16: oracle.XF_F16,
       torch.bfloat16: oracle.XF_BF16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    swrt.lib()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def host_np(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def decoded(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def bound(q, k, v, L, W, scale, out_dtype, ref):
    """The per-(b, h) tolerance of tests/att_bound.py, broadcast over D."""
    qd, kd, vd = decoded(q), decoded(k), decoded(v)
    B, Hq, D = qd.shape
    G = Hq // kd.shape[1]
    tol = np.zeros((B, Hq, 1))
    for b in range(B):
        r0, r1 = max(0, int(L[b]) - W), int(L[b])
        if r1 <= r0:
            continue
        for h in range(Hq):
            tol[b, h] = window_tolerance(qd[b, h], kd[b, h // G, r0:r1], vd[b, h // G, r0:r1],
                                         scale)
    return with_output_rounding(tol, ref, out_dtype)


def check(orc, qs, ks, vs, L, W, scale, outs, out_dtype):
    worst = 0.0
    for q, k, v, o in zip(qs, ks, vs, outs):
        ref, f = orc.window_attention(host_np(q), host_np(k), host_np(v), L, W, scale, ORC[q.dtype])
        got = decoded(o)
        tol = bound(q, k, v, L, W, scale, out_dtype, ref)
        err = np.abs(got - ref)
        assert (err <= tol).all(), f"max err/tol {np.max(err / tol):.3g}"
        worst = max(worst, float(np.max(err / tol)))
    return worst


def make(g, B, Hq, Hkv, C, D, dtype, n_layers=2, qscale=1.0):
    f = lambda shape, s=1.0: torch.from_numpy(  # noqa: E731
        (g.standard_normal(shape) * s).astype(np.float32)).to(dtype)
    qs = [f((B, Hq, D), qscale) for _ in range(n_layers)]
    ks = [f((B, Hkv, C, D)) for _ in range(n_layers)]
    vs = [f((B, Hkv, C, D)) for _ in range(n_layers)]
    return qs, ks, vs


SHAPES = [  # (dtype, D, Hq, Hkv): every lanes-per-row width and group size
    (torch.bfloat16, 32, 16, 16), (torch.bfloat16, 32, 32, 2),
    (torch.bfloat16, 64, 8, 8), (torch.bfloat16, 64, 16, 8), (torch.bfloat16, 64, 16, 4),
    (torch.bfloat16, 64, 64, 8), (torch.bfloat16, 64, 32, 2),
    (torch.bfloat16, 128, 64, 8), (torch.bfloat16, 256, 16, 4),
    (torch.bfloat16, 128, 32, 2), (torch.bfloat16, 256, 16, 1),  # group 16, matrix cores only
    (torch.float16, 32, 8, 1), (torch.float16, 64, 64, 8), (torch.float16, 128, 8, 4),
    (torch.float16, 256, 32, 2),
    (torch.float32, 16, 4, 2), (torch.float32, 64, 64, 8), (torch.float32, 128, 8, 8),
    # matrix cores, any group: 7 and 12 heads, and 20 and 32 (two waves per window)
    (torch.bfloat16, 64, 14, 2), (torch.float16, 32, 24, 2), (torch.bfloat16, 128, 40, 2),
    (torch.bfloat16, 64, 64, 2),
    # matrix cores, head_dim 96 and 192 (12- and 24-byte V chunks per lane)
    (torch.bfloat16, 96, 16, 2), (torch.float16, 192, 8, 8),
]


@pytest.mark.parametrize("out_same", [False, True], ids=["f32_out", "same_out"])
@pytest.mark.parametrize("dtype,D,Hq,Hkv", SHAPES, ids=lambda x: str(x))
def test_window_attention_shapes(orc, dtype, D, Hq, Hkv, out_same):
    say("window attention", dtype, D, Hq, Hkv, out_same)
    g = wl.rng(D * 1000 + Hq * 10 + Hkv)
    B, C = 6, 40
    qs, ks, vs = make(g, B, Hq, Hkv, C, D, dtype)
    L = np.array([0, 1, 7, 33, 40, 40], np.int32)
    odt = dtype if out_same else torch.float32
    for W in (40, 9, 1):
        flags = flag_word()
        outs = swrt.window_attention([t.to(DEV) for t in qs], [t.to(DEV) for t in ks],
                                     [t.to(DEV) for t in vs], torch.from_numpy(L).to(DEV), W,
                                     out_dtype=odt, flags=flags)
        torch.cuda.synchronize()
        assert flags.item() == 0
        worst = check(orc, qs, ks, vs, L, W, D ** -0.5, outs, odt)
        say("  W", W, "worst err/tol", round(worst, 4))
        for o in outs:  # the empty window gives zeros
            assert (o[0] == 0).all()


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 64, 32, 4), (torch.float16, 128, 8, 8),
                                           (torch.bfloat16, 32, 16, 16), (torch.bfloat16, 64, 96, 4),
                                           (torch.bfloat16, 96, 32, 8)],
                         ids=str)
def test_many_windows_one_wave_each(orc, dtype, D, Hq, Hkv):
    """Enough (layer, b, kv head) windows that each takes one wave (the
    matrix-core kernel's other launch shape), ragged lengths and windows."""
    say("window attention, many windows", dtype, D, Hq, Hkv)
    g = wl.rng(D + Hq + Hkv)
    n_layers, B, C = 2, 2048 // Hkv, 48
    qs, ks, vs = make(g, B, Hq, Hkv, C, D, dtype, n_layers=n_layers)
    L = g.integers(0, C + 1, size=B).astype(np.int32)
    L[:4] = [0, 1, 17, C]
    for W in (C, 21):
        outs = swrt.window_attention([t.to(DEV) for t in qs], [t.to(DEV) for t in ks],
                                     [t.to(DEV) for t in vs], torch.from_numpy(L).to(DEV), W,
                                     out_dtype=torch.float32)
        torch.cuda.synchronize()
        worst = check(orc, qs, ks, vs, L, W, D ** -0.5, outs, torch.float32)
        say("  W", W, "worst err/tol", round(worst, 4))


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 64, 8, 2), (torch.float16, 128, 32, 2),
                                           (torch.float32, 64, 4, 1)], ids=str)
def test_long_windows(orc, dtype, D, Hq, Hkv):
    """Windows of up to 1000 rows (63 tiles): many blocks per wave, the tiles
    split over four waves and merged, a window shorter than the cache, a
    partial last tile."""
    say("window attention, long windows", dtype, D, Hq, Hkv)
    g = wl.rng(5000 + D + Hq)
    B, C = 6, 1000
    qs, ks, vs = make(g, B, Hq, Hkv, C, D, dtype, n_layers=1, qscale=0.3)
    L = np.array([0, 1, 999, 1000, 517, 16], np.int32)
    for W in (1000, 700, 17):
        outs = swrt.window_attention([t.to(DEV) for t in qs], [t.to(DEV) for t in ks],
                                     [t.to(DEV) for t in vs], torch.from_numpy(L).to(DEV), W,
                                     out_dtype=torch.float32)
        torch.cuda.synchronize()
        worst = check(orc, qs, ks, vs, L, W, D ** -0.5, outs, torch.float32)
        say("  W", W, "worst err/tol", round(worst, 4))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_eight_byte_aligned_operands(orc, dtype):
    """16-bit operands that are 8- but not 16-byte aligned take the VALU
    kernel; same results within the bound."""
    g = wl.rng(11)
    B, Hq, Hkv, C, D = 5, 16, 4, 40, 64
    qs, ks, vs = make(g, B, Hq, Hkv, C, D, dtype, n_layers=1)

    def shifted(t):  # the same values at an address 8 bytes past a 16-byte boundary
        buf = torch.empty(t.numel() + 4, dtype=dtype, device=DEV)
        v = buf[4:].view(t.shape)
        v.copy_(t.to(DEV))
        assert v.data_ptr() % 16 == 8
        return v
    L = np.array([40, 3, 0, 39, 16], np.int32)
    outs = swrt.window_attention([shifted(qs[0])], [shifted(ks[0])], [shifted(vs[0])],
                                 torch.from_numpy(L).to(DEV), 24, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(orc, qs, ks, vs, L, 24, D ** -0.5, outs, torch.float32)


def test_large_scores_stay_finite(orc):
    g = wl.rng(7)
    B, Hq, Hkv, C, D = 4, 16, 2, 128, 64
    qs, ks, vs = make(g, B, Hq, Hkv, C, D, torch.bfloat16, n_layers=1, qscale=40.0)
    L = np.array([128, 64, 3, 100], np.int32)
    outs = swrt.window_attention([t.to(DEV) for t in qs], [t.to(DEV) for t in ks],
                                 [t.to(DEV) for t in vs], torch.from_numpy(L).to(DEV), 128,
                                 out_dtype=torch.float32, scale=1.0)
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    check(orc, qs, ks, vs, L, 128, 1.0, outs, torch.float32)


def test_bad_lengths_leave_outputs(orc):
    g = wl.rng(8)
    B, Hq, Hkv, C, D = 3, 8, 2, 16, 64
    qs, ks, vs = make(g, B, Hq, Hkv, C, D, torch.bfloat16, n_layers=1)
    L = np.array([17, 5, -1], np.int32)
    out = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device=DEV)
    flags = flag_word()
    swrt.window_attention([qs[0].to(DEV)], [ks[0].to(DEV)], [vs[0].to(DEV)],
                          torch.from_numpy(L).to(DEV), 16, outs=[out], flags=flags)
    torch.cuda.synchronize()
    assert flags.item() == swrt.FLAG_BAD_LENGTHS
    assert (out[0] == 7).all() and (out[2] == 7).all()
    ref, _ = orc.window_attention(host_np(qs[0][1:2]), host_np(ks[0][1:2]), host_np(vs[0][1:2]),
                                  L[1:2], 16, D ** -0.5, oracle.XF_BF16)
    np.testing.assert_allclose(out[1].cpu().numpy(), ref[0], atol=1e-4)


@pytest.mark.parametrize("layout", ["base", "drift"])
def test_attention_after_the_decode_step(orc, layout):
    """The path end to end: the one-launch step appends the new token, then
    attention reads the windows it left, against the oracle on the same
    appended caches."""
    g = wl.rng(9)
    B, Hq, Hkv, D, W = 8, 32, 4, 64, 64
    C = W if layout == "base" else W + 16
    T = g.integers(1, 3 * C, size=B)
    T[:3] = [1, C, C + 1]
    sk = torch.from_numpy((T - 1).astype(np.int32)).to(DEV)
    kc = torch.randn(B, Hkv, C, D, device=DEV).to(torch.bfloat16)
    vc = torch.randn(B, Hkv, C, D, device=DEV).to(torch.bfloat16)
    kn = torch.randn(B, Hkv, 1, D, device=DEV).to(torch.bfloat16)
    vn = torch.randn(B, Hkv, 1, D, device=DEV).to(torch.bfloat16)
    q = torch.randn(B, Hq, D, device=DEV).to(torch.bfloat16)
    lens = swrt.kv_decode_step([kc], [vc], [kn], [vn], sk, [], [], torch.empty(0, dtype=torch.int64,
                               device=DEV), window=None if layout == "base" else W)
    outs = swrt.window_attention([q], [kc], [vc], lens.cache_total, W, out_dtype=torch.float32)
    torch.cuda.synchronize()
    L = lens.cache_total.cpu().numpy()
    assert (L == np.minimum(T, C)).all() if layout == "base" else ((L >= np.minimum(T, W)) &
                                                                   (L <= C)).all()
    check(orc, [q.cpu()], [kc.cpu()], [vc.cpu()], L, W, D ** -0.5, outs, torch.float32)
    # the appended token is the last resident row: its V is what W = 1 returns
    one = swrt.window_attention([q], [kc], [vc], lens.cache_total, 1, out_dtype=torch.float32)[0]
    vrow = vn[:, :, 0].float().cpu().numpy()  # [B, Hkv, D]
    for b in range(B):
        np.testing.assert_array_equal(one[b].cpu().numpy(), vrow[b][np.arange(Hq) // (Hq // Hkv)])


def test_workload8_full_size(orc):
    """Attention over the 12 windowed layers of the model step, in the launch
    configuration the benchmark times (every layer compared)."""
    spec = wl.workload8()
    say("workload 8 full size")
    st = ModelDecodeStep(spec, DEV, set_id=0)
    st.run_fused()  # the step's append, then its attention
    outs = st.attention()
    torch.cuda.synchronize()
    b = st.buffers
    L = b.lengths.cache_total.cpu().numpy()
    worst = check(orc, [t.cpu() for t in b.win_q], [t.cpu() for t in b.win_k],
                  [t.cpu() for t in b.win_v], L, spec.window, spec.head_dim ** -0.5, outs,
                  torch.bfloat16)
    say("  worst err/tol", round(worst, 4))
