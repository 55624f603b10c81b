"""GPU parity of the paged caches against the oracle.

Conversion (swrt_paged_quantize) and append (swrt_paged_append, sealed
blocks; swrt_paged_append_open, the open-page extension) decide every byte in
binary32 on both sides: whole arenas, descriptor tables and block tables are
compared byte for byte. Attention (swrt_paged_attention) reduces in fp32
against the oracle's float64 and is held, per batch entry and query head, to
the tolerance of tests/att_bound.py (the forward error of any binary32
streaming evaluation of the definition, affine elements decoded with one
rounding), plus the output's own rounding for 16-bit outputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_ring_tensor_amd as swrt
from sliding_window_ring_tensor_amd import workloads as wl
from tests.att_bound import window_tolerance, with_output_rounding
from tests.test_parity_gpu import DEV, flag_word, say

pytestmark = pytest.mark.gpu
F32, F16, BF16, I8, U8, I4, U4, I2, U2 = 1, 2, 3, 4, 5, 6, 7, 8, 9
ALL_FORMATS = [F32, F16, BF16, I8, U8, I4, U4, I2, U2]
QT = {torch.float32: oracle.XF_F32, torch.float16: oracle.XF_F16, torch.bfloat16: oracle.XF_BF16}
RANGES = {I8: (-128, 127), U8: (0, 255), I4: (-8, 7), U4: (0, 15), I2: (-2, 1), U2: (0, 3)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    swrt.lib()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def otable(case) -> np.ndarray:
    t = np.zeros(case.n_pages, oracle.PAGE_DTYPE)
    for f in wl.PAGE_FIELDS:
        t[f] = case.fields[f]
    return t


def upload(case, table=None) -> swrt.PagedCache:
    tb = swrt.page_table(case.fields) if table is None else table.view(swrt.PAGE_DTYPE)
    return swrt.PagedCache.upload(tb, case.page_ptr, case.page_ids, case.arena, DEV)


def random_format(g, formats=ALL_FORMATS):
    def pick(s, i, n):
        kf, vf = (int(f) for f in g.choice(formats, 2))
        ks, vs = (float(np.float32(x)) for x in g.uniform(0.01, 0.3, 2))
        kz = int(g.integers(*RANGES[kf], endpoint=True)) if kf in RANGES else 0
        vz = int(g.integers(*RANGES[vf], endpoint=True)) if vf in RANGES else 0
        return (kf, vf, ks if kf in RANGES else 1.0, vs if vf in RANGES else 1.0, kz, vz)
    return pick


def decode_rows(arena, page, D, kv):
    """float64 values of a page's valid rows (numpy bit unpacking, for the bound)."""
    fmt = int(page[kv + "_format"])
    bits = oracle.PAGE_BITS[fmt]
    n, off = int(page["length"]), int(page[kv + "_offset"])
    raw = arena[off:off + n * D * bits // 8]
    if fmt == F32:
        return raw.view(np.float32).astype(np.float64).reshape(n, D)
    if fmt == F16:
        return raw.view(np.float16).astype(np.float64).reshape(n, D)
    if fmt == BF16:
        return (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64) \
            .reshape(n, D)
    codes = (np.unpackbits(raw, bitorder="little").reshape(-1, bits) *
             (1 << np.arange(bits))).sum(axis=1).astype(np.int64)
    if fmt in (I8, I4, I2):
        codes = np.where(codes >= 1 << (bits - 1), codes - (1 << bits), codes)
    return ((codes - int(page[kv + "_zero_point"])) * float(page[kv + "_scale"])).reshape(n, D)


def bound(case, tb, q, Hkv, left_window, scale, out_dtype, ref):
    qd = q.detach().cpu().to(torch.float64).numpy()
    B, Hq, D = qd.shape
    G = Hq // Hkv
    tol = np.zeros((B, Hq, 1))
    for b in range(B):
        for g in range(Hkv):
            s = b * Hkv + g
            ids = case.page_ids[case.page_ptr[s]:case.page_ptr[s + 1]]
            if len(ids) == 0:
                continue
            # the stream's pages are contiguous from token 0 (valid cases
            # only): decode just those the window reaches
            ends = tb[ids]["start"] + tb[ids]["length"]
            T = int(ends[-1])
            r0 = 0 if left_window < 0 else max(0, T - 1 - left_window)
            vis = ids[ends > r0]
            first = int(tb[vis[0]]["start"])
            k = np.concatenate([decode_rows(case.arena, tb[i], D, "k") for i in vis])[r0 - first:]
            v = np.concatenate([decode_rows(case.arena, tb[i], D, "v") for i in vis])[r0 - first:]
            for h in range(g * G, (g + 1) * G):
                tol[b, h] = window_tolerance(qd[b, h], k, v, scale, paged=True)
    return with_output_rounding(tol, ref, out_dtype)


def q_host(q: torch.Tensor) -> np.ndarray:
    t = q.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def run_attention(orc, case, q, Hkv, left_window, out_dtype, scale=None, tb=None, formats=None):
    D = q.shape[2]
    sc = D ** -0.5 if scale is None else scale
    cache = upload(case) if tb is None else swrt.PagedCache.upload(tb, case.page_ptr,
                                                                   case.page_ids, case.arena, DEV)
    flags = flag_word()
    out = swrt.paged_attention([q.to(DEV)], [cache], left_window, Hkv, scale=sc,
                               out_dtype=out_dtype, flags=flags, formats=formats)[0]
    torch.cuda.synchronize()
    tbo = otable(case) if tb is None else tb
    ref, f = orc.paged_attention(q_host(q), QT[q.dtype], case.arena, tbo, case.page_ptr,
                                 case.page_ids, left_window, Hkv, sc)
    return out, ref, int(flags.item()), f, tbo


SHAPES = [  # (q dtype, D, Hq, Hkv)
    (torch.bfloat16, 64, 16, 2), (torch.bfloat16, 32, 8, 8), (torch.bfloat16, 128, 16, 1),
    (torch.bfloat16, 256, 4, 4), (torch.float16, 64, 32, 2), (torch.float32, 64, 8, 4),
    (torch.float32, 32, 3, 1), (torch.bfloat16, 64, 12, 4),
    # groups of 7, and of 20 and 34 heads (two and three waves per stream)
    (torch.bfloat16, 64, 14, 2), (torch.bfloat16, 64, 40, 2), (torch.float32, 32, 34, 1),
]


@pytest.mark.parametrize("left_window", [-1, 0, 7, 40])
@pytest.mark.parametrize("qdt,D,Hq,Hkv", SHAPES, ids=str)
def test_paged_attention_mixed_formats(orc, qdt, D, Hq, Hkv, left_window):
    """Pages of every format (random per page, K and V apart), sealed partial
    pages, shuffled arena, ragged streams (empty, one token, many pages)."""
    say("paged attention", qdt, D, Hq, Hkv, left_window)
    g = wl.rng(D * 100 + Hq * 10 + Hkv + left_window)
    B = 3
    T = g.integers(1, 90, size=B * Hkv)
    T[0] = 0
    T[-1] = 1
    streams = [wl.page_split(g, int(t), int(g.choice([4, 16, 32])), sealed=0.3) for t in T]
    case = wl.paged_case(g, D, streams, random_format(g))
    q = torch.from_numpy(g.uniform(-1, 1, (B, Hq, D)).astype(np.float32)).to(qdt)
    for odt in (torch.float32, qdt):
        out, ref, fg, fo, tb = run_attention(orc, case, q, Hkv, left_window, odt)
        assert fg == fo == 0
        got = out.detach().cpu().to(torch.float64).numpy()
        tol = bound(case, tb, q, Hkv, left_window, D ** -0.5, odt, ref)
        err = np.abs(got - ref)
        assert (err <= tol).all(), f"max err/tol {np.max(err / tol):.3g}"
        say("  out", odt, "worst err/tol", round(float(np.max(err / tol)), 4))
        G = Hq // Hkv
        assert (out[0, :G] == 0).all()  # the empty stream


@pytest.mark.parametrize("formats", [None, (BF16, I8)], ids=["any", "bf16-int8"])
@pytest.mark.parametrize("left_window", [-1, 63, 64, 150])
@pytest.mark.parametrize("qdt", [torch.bfloat16, torch.float32], ids=str)
def test_paged_attention_windows_over_many_pages(orc, qdt, left_window, formats):
    """Windows that reach more than 64 pages (pages of 1 to 3 tokens): the
    kernel walks a stream's pages 64 at a time from the last one back, so
    these streams take two to seven groups, with the window's first page at
    and around a group boundary; for any format and in the build for bf16
    and int8 pages (whose staging buffers carry over from group to group)."""
    say("paged attention, many pages", qdt, left_window, formats)
    g = wl.rng(900 + left_window)
    D, Hq, Hkv, B = 64, 8, 2, 3
    T = g.integers(100, 400, size=B * Hkv)
    T[0] = 64  # a window of 64 one-token pages: exactly one group
    T[1] = 65
    caps = [1, 1, 2, 3, 1, 2]
    streams = [wl.page_split(g, int(t), c, sealed=0.2) for t, c in zip(T, caps)]
    assert max(len(s) for s in streams) > 128
    case = wl.paged_case(g, D, streams, random_format(g) if formats is None
                         else random_format(g, list(formats)))
    q = torch.from_numpy(g.uniform(-1, 1, (B, Hq, D)).astype(np.float32)).to(qdt)
    out, ref, fg, fo, tb = run_attention(orc, case, q, Hkv, left_window, torch.float32,
                                         formats=formats)
    assert fg == fo == 0
    got = out.detach().cpu().to(torch.float64).numpy()
    tol = bound(case, tb, q, Hkv, left_window, D ** -0.5, torch.float32, ref)
    err = np.abs(got - ref)
    assert (err <= tol).all(), f"max err/tol {np.max(err / tol):.3g}"
    say("  worst err/tol", round(float(np.max(err / tol)), 4))


@pytest.mark.parametrize("head", [(64, torch.bfloat16), (32, torch.float32), (128, torch.bfloat16)],
                         ids=["d64-bf16q", "d32-f32q", "d128-bf16q"])
@pytest.mark.parametrize("zero_points", ["zero", "any"])
@pytest.mark.parametrize("formats", [(BF16, I8), (BF16, I8, U8, I4, U4, I2, U2)], ids=str)
def test_paged_attention_declared_formats(orc, formats, zero_points, head):
    """A declared page-format set runs the kernel built for it: bf16 and int8
    only (the lean build; at head_dim 64 with a bf16 query it runs five waves
    per SIMD), or every staged format but f16 (without the f32 and f16
    paths). On pages of the declared formats it gives the same bytes as the
    build for any format (the same tile code runs) and meets the oracle's
    bound; int8 pages of zero point 0 take the decode without the
    subtraction, others the general one. A page of an undeclared format makes
    its stream fail its checks (BAD_PAGES, outputs untouched), and the other
    streams' outputs stay those of the unrestricted call."""
    say("paged attention, declared formats", formats, zero_points, head)
    D, qdt = head
    g = wl.rng(77 + len(formats) + (zero_points == "zero") + D)
    B, Hq, Hkv, lw = 3, 16, 2, 40
    T = g.integers(20, 90, size=B * Hkv)
    streams = [wl.page_split(g, int(t), int(g.choice([4, 16])), sealed=0.2) for t in T]
    pick = random_format(g, list(formats))

    def fmt(s, i, n):
        kf, vf, ks, vs, kz, vz = pick(s, i, n)
        if zero_points == "zero" or g.integers(0, 2):
            kz = vz = 0
        return kf, vf, ks, vs, kz, vz
    case = wl.paged_case(g, D, streams, fmt)
    q = torch.from_numpy(g.uniform(-1, 1, (B, Hq, D)).astype(np.float32)).to(qdt)
    cache = upload(case)
    outs = {}
    for decl in (None, formats):
        flags = flag_word()
        outs[decl] = swrt.paged_attention([q.to(DEV)], [cache], lw, Hkv, out_dtype=torch.float32,
                                          flags=flags, formats=decl)[0]
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
    assert torch.equal(outs[None], outs[formats])
    tb = otable(case)
    ref, fo = orc.paged_attention(q_host(q), QT[q.dtype], case.arena, tb, case.page_ptr,
                                  case.page_ids, lw, Hkv, D ** -0.5)
    assert fo == 0
    got = outs[formats].cpu().to(torch.float64).numpy()
    tol = bound(case, tb, q, Hkv, lw, D ** -0.5, torch.float32, ref)
    assert (np.abs(got - ref) <= tol).all()
    # the same streams with stream 1's last page in f16 (K and V) and stream
    # 4's in f32 (V): valid pages, outside the declared set
    def fmt2(s, i, n):
        kf, vf, ks, vs, kz, vz = fmt(s, i, n)
        if i == n - 1 and s == 1:
            return F16, F16, 1.0, 1.0, 0, 0
        if i == n - 1 and s == 4:
            return kf, F32, ks, 1.0, kz, 0
        return kf, vf, ks, vs, kz, vz
    case2 = wl.paged_case(g, D, streams, fmt2)
    cache = upload(case2)
    flags = flag_word()
    full = swrt.paged_attention([q.to(DEV)], [cache], lw, Hkv, out_dtype=torch.float32,
                                flags=flags)[0]
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    out = torch.full((B, Hq, D), 7.0, device=DEV)
    flags = flag_word()
    swrt.paged_attention([q.to(DEV)], [cache], lw, Hkv, outs=[out], flags=flags, formats=formats)
    torch.cuda.synchronize()
    assert int(flags.item()) == swrt.FLAG_BAD_PAGES
    G = Hq // Hkv
    bad = np.zeros((B, Hq), bool)
    for s_ in (1, 4):
        b, kv = divmod(s_, Hkv)
        bad[b, kv * G:(kv + 1) * G] = True
    got, badt = out.cpu(), torch.from_numpy(bad)
    assert (got[badt] == 7.0).all()
    assert torch.equal(got[~badt], full.cpu()[~badt])


@pytest.mark.parametrize("left_window", [-1, 0, 5, 40])
@pytest.mark.parametrize("D,Hq,Hkv,qdt", [(64, 16, 2, torch.bfloat16), (64, 16, 4, torch.float32),
                                          (32, 8, 8, torch.bfloat16), (128, 16, 2, torch.bfloat16)],
                         ids=str)
def test_paged_attention_bf16_int8_build_tiles(orc, D, Hq, Hkv, qdt, left_window):
    """The build for bf16 and int8 pages (declared) on pages of 4 to 48 rows:
    several tiles in one page (the loop's advance within a page), partial
    tiles, K and V formats apart, any zero points, ragged and empty streams;
    within the oracle's bound, for fp32 and 16-bit outputs."""
    say("paged attention, bf16 + int8 build", D, Hq, Hkv, qdt, left_window)
    g = wl.rng(500 + D + Hq * 3 + Hkv * 7 + left_window)
    B = 3
    T = g.integers(1, 130, size=B * Hkv)
    T[0] = 0
    T[-1] = 17
    streams = [wl.page_split(g, int(t), int(g.choice([4, 16, 32, 48])), sealed=0.3) for t in T]
    case = wl.paged_case(g, D, streams, random_format(g, [BF16, I8]))
    q = torch.from_numpy(g.uniform(-1, 1, (B, Hq, D)).astype(np.float32)).to(qdt)
    cache = upload(case)
    tb = otable(case)
    ref, fo = orc.paged_attention(q_host(q), QT[qdt], case.arena, tb, case.page_ptr,
                                  case.page_ids, left_window, Hkv, D ** -0.5)
    assert fo == 0
    for odt in (torch.float32, torch.bfloat16):
        flags = flag_word()
        out = swrt.paged_attention([q.to(DEV)], [cache], left_window, Hkv, out_dtype=odt,
                                   flags=flags, formats=(BF16, I8))[0]
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        got = out.cpu().to(torch.float64).numpy()
        tol = bound(case, tb, q, Hkv, left_window, D ** -0.5, odt, ref)
        err = np.abs(got - ref)
        assert (err <= tol).all(), f"max err/tol {np.max(err / tol):.3g}"
        say("  out", odt, "worst err/tol", round(float(np.max(err / tol)), 4))
        G = Hq // Hkv
        assert (out[0, :G] == 0).all()  # the empty stream


def test_paged_attention_bad_pages_flag_and_skip(orc):
    g = wl.rng(60)
    D, B, Hq, Hkv = 64, 2, 4, 2
    streams = [wl.page_split(g, 40, 16) for _ in range(B * Hkv)]
    case = wl.paged_case(g, D, streams, lambda s, i, n: (BF16, I8, 1.0, 0.05, 0, 0))
    q = torch.from_numpy(g.uniform(-1, 1, (B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
    good, ref, fg, fo, tb = run_attention(orc, case, q, Hkv, 9, torch.float32)
    assert fg == fo == 0
    cases = []
    # stream 0: its first page is outside a 10-token window; wreck it: not read
    t1 = tb.copy()
    t1[case.page_ids[0]]["length"] = 0
    t1[case.page_ids[0]]["k_offset"] = 1 << 40
    cases.append((t1, 0))
    # stream 1: last page starts one token late (contiguity)
    t2 = tb.copy()
    t2[case.page_ids[case.page_ptr[2] - 1]]["start"] += 1
    cases.append((t2, oracle.FLAG_BAD_PAGES))
    # stream 2: a visible page's payload runs past the arena
    t3 = tb.copy()
    t3[case.page_ids[case.page_ptr[3] - 1]]["v_offset"] = len(case.arena) - 16
    cases.append((t3, oracle.FLAG_BAD_PAGES))
    # stream 3: a visible page with a zero scale; and a misaligned offset
    t4 = tb.copy()
    t4[case.page_ids[case.page_ptr[4] - 1]]["v_scale"] = 0.0
    cases.append((t4, oracle.FLAG_BAD_PAGES))
    for t, want in cases:
        cache = swrt.PagedCache.upload(t, case.page_ptr, case.page_ids, case.arena, DEV)
        out = torch.full((B, Hq, D), 7.0, device=DEV)
        flags = flag_word()
        swrt.paged_attention([q.to(DEV)], [cache], 9, Hkv, outs=[out], flags=flags)
        torch.cuda.synchronize()
        refo, fo = orc.paged_attention(q_host(q), oracle.XF_BF16, case.arena, t, case.page_ptr,
                                       case.page_ids, 9, Hkv, D ** -0.5,
                                       out=np.full((B, Hq, D), 7.0))
        assert int(flags.item()) == fo == want
        got = out.cpu().numpy()
        same = refo == 7.0
        assert (got[same] == 7.0).all()
        np.testing.assert_allclose(got[~same], refo[~same], atol=1e-4)
    # the library's layout rule (not the pages'): a payload offset that is not
    # a multiple of 16 makes the page invalid for the kernels; the oracle,
    # which follows the pages, reads it
    t5 = tb.copy()
    pid = case.page_ids[case.page_ptr[4] - 1]
    t5[pid]["k_offset"] += 8
    cache = swrt.PagedCache.upload(t5, case.page_ptr, case.page_ids, case.arena, DEV)
    out = torch.full((B, Hq, D), 7.0, device=DEV)
    flags = flag_word()
    swrt.paged_attention([q.to(DEV)], [cache], 9, Hkv, outs=[out], flags=flags)
    torch.cuda.synchronize()
    _, fo = orc.paged_attention(q_host(q), oracle.XF_BF16, case.arena, t5, case.page_ptr,
                                case.page_ids, 9, Hkv, D ** -0.5)
    assert fo == 0 and int(flags.item()) == swrt.FLAG_BAD_PAGES
    got = out.cpu().numpy()
    assert (got[1, 2:] == 7.0).all()  # stream 3 = (b 1, kv head 1): its heads untouched
    np.testing.assert_allclose(got[0], good.cpu().numpy()[0], atol=1e-4)
    # an id out of range among the visible pages, and page_ptr past page_ids
    for mut in ("id", "ptr"):
        ids, ptr = case.page_ids.copy(), case.page_ptr.copy()
        if mut == "id":
            ids[case.page_ptr[1] - 1] = case.n_pages
        else:
            ptr[-1] = len(ids) + 1
        cache = swrt.PagedCache.upload(tb, ptr, ids, case.arena, DEV)
        flags = flag_word()
        swrt.paged_attention([q.to(DEV)], [cache], 9, Hkv, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == swrt.FLAG_BAD_PAGES


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (68, 2)])
def test_paged_attention_several_layers_sharing_a_block_table(orc, Hq, Hkv):
    """Three layers on one block table. Each layer's workgroups start at a
    multiple of 8: with 8 (stream, chunk) items a layer, or 24 at three
    chunks a stream (34 heads a group), the later layers begin after idle
    padding workgroups, and a stream's chunks straddle workgroups."""
    say("paged layers on one table", Hq, Hkv)
    g = wl.rng(61)
    D, B, n = 64, 4, 3
    streams = [wl.page_split(g, int(t), 16, 0.2) for t in g.integers(1, 200, B * Hkv)]
    # one block table (the same layout and formats), each layer its own payload bytes
    cases = [wl.paged_case(wl.rng(70), D, streams, random_format(wl.rng(71)),
                           payload_rng=wl.rng(72 + i)) for i in range(n)]
    for c in cases[1:]:
        assert all((c.fields[f] == cases[0].fields[f]).all() for f in wl.PAGE_FIELDS)
    table = swrt.PagedCache.upload(swrt.page_table(cases[0].fields), cases[0].page_ptr,
                                   cases[0].page_ids, cases[0].arena, DEV)
    caches = [swrt.PagedCache(torch.from_numpy(c.arena).to(DEV), table.pages, table.page_ptr,
                              table.page_ids) for c in cases]
    qs = [torch.from_numpy(g.uniform(-1, 1, (B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
          for _ in range(n)]
    flags = flag_word()
    outs = swrt.paged_attention([q.to(DEV) for q in qs], caches, 30, Hkv, out_dtype=torch.float32,
                                flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    tb = otable(cases[0])
    for i in range(n):
        ref, f = orc.paged_attention(q_host(qs[i]), oracle.XF_BF16, cases[i].arena, tb,
                                     cases[0].page_ptr, cases[0].page_ids, 30, Hkv, D ** -0.5)
        err = np.abs(outs[i].cpu().numpy() - ref)
        tol = bound(wl.PagedCase(D, cases[0].fields, cases[0].page_ptr, cases[0].page_ids,
                                 cases[i].arena, 0), tb, qs[i], Hkv, 30, D ** -0.5,
                    torch.float32, ref)
        assert (err <= tol).all()


# -- conversion -----------------------------------------------------------------------

@pytest.mark.parametrize("kf,vf", [(I8, U4), (I2, U2), (F16, BF16), (F32, I4), (U8, F32),
                                   (BF16, I8), (I4, I4)])
def test_paged_quantize_bytes_equal_the_oracle(orc, kf, vf):
    say("paged quantize", kf, vf)
    g = wl.rng(62 + kf * 10 + vf)
    D = 64
    streams = [wl.page_split(g, int(t), 16, 0.3) for t in g.integers(1, 100, 12)]
    case = wl.paged_case(g, D, streams, random_format(g), spare_bytes=1 << 20)
    tb = otable(case)
    sel = np.sort(g.choice(case.n_pages, size=max(1, case.n_pages // 3), replace=False)).astype(np.int32)
    base = case.free_offset
    dst, off = [], base
    for pid in sel:
        for f in (kf, vf):
            dst.append(off)
            nb = int(tb[pid]["capacity"]) * D * oracle.PAGE_BITS[f] // 8
            off += -(-nb // 16) * 16 + int(g.integers(0, 3)) * 16
    ks, vs = 0.0375, 0.011
    kz = (RANGES[kf][0] + RANGES[kf][1] + 1) // 2 if kf in RANGES else 0
    vz = RANGES[vf][0] if vf in RANGES else 0
    st, ar, pout = orc.paged_quantize(case.arena, tb, sel, dst, base, len(case.arena), kf, ks, kz,
                                      vf, vs, vz, D)
    assert st == oracle.OK
    cache = upload(case)
    flags = flag_word()
    blocks = torch.from_numpy(sel).to(DEV)
    dsts = torch.from_numpy(np.array(dst, np.int64)).to(DEV)
    for in_place in (False, True):
        c = upload(case)
        out = swrt.paged_quantize(c, blocks, dsts, base, len(case.arena), kf, ks, kz, vf, vs, vz, D,
                                  pages_out=c.pages if in_place else None, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        np.testing.assert_array_equal(c.arena.cpu().numpy(), ar)
        assert out.cpu().numpy().tobytes() == pout.tobytes()
    # attention over the converted cache equals the oracle's within the bound
    q = torch.from_numpy(g.uniform(-1, 1, (3, 8, D)).astype(np.float32)).to(torch.bfloat16)
    newcase = wl.PagedCase(D, {f: pout[f] for f in wl.PAGE_FIELDS}, case.page_ptr, case.page_ids,
                           ar, 0)
    o, ref, fg, fo, _ = run_attention(orc, newcase, q, 4, -1, torch.float32, tb=pout)
    assert fg == fo == 0
    tol = bound(newcase, pout, q, 4, -1, D ** -0.5, torch.float32, ref)
    assert (np.abs(o.cpu().numpy() - ref) <= tol).all()


def test_paged_quantize_rejects_and_writes_nothing(orc):
    g = wl.rng(63)
    D = 32
    case = wl.paged_case(g, D, [wl.page_split(g, 40, 8) for _ in range(2)],
                         lambda s, i, n: (BF16, BF16, 1.0, 1.0, 0, 0), spare_bytes=4096)
    base, end = case.free_offset, len(case.arena)
    tb = otable(case)
    good = dict(blocks=[0, 1], dst=[base, base + 128, base + 256, base + 384], fb=base, fe=end)
    bads = [dict(blocks=[1, 1]), dict(blocks=[1, 0]), dict(blocks=[0, case.n_pages]),
            dict(dst=[base, base + 100, base + 256, base + 384]),
            dict(dst=[base + 16, base, base + 256, base + 384]),    # out of order
            dict(fb=base - 16, dst=[base - 16, base + 128, base + 256, base + 384]),
            dict(fe=base + 400)]
    for kw in bads:
        a = {**good, **kw}
        st, _, _ = orc.paged_quantize(case.arena, tb, a["blocks"], a["dst"], a["fb"], a["fe"],
                                      I8, 0.1, 0, I8, 0.1, 0, D)
        assert st == oracle.E_INVALID_ARG, kw
        c = upload(case)
        flags = flag_word()
        out = swrt.paged_quantize(c, torch.tensor(a["blocks"], dtype=torch.int32, device=DEV),
                                  torch.tensor(a["dst"], dtype=torch.int64, device=DEV), a["fb"],
                                  a["fe"], I8, 0.1, 0, I8, 0.1, 0, D, pages_out=c.pages,
                                  flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == swrt.FLAG_BAD_PAGES, kw
        np.testing.assert_array_equal(c.arena.cpu().numpy(), case.arena)
        assert out.cpu().numpy().tobytes() == tb.tobytes()
    # the library's layout rule: destinations at multiples of 16 (the oracle,
    # which follows the pages, accepts this request)
    dst = [base, base + 264, base + 520, base + 776]  # 256-byte payloads, three off by 8
    st, _, _ = orc.paged_quantize(case.arena, tb, [0, 1], dst, base, end, I8, 0.1, 0, I8, 0.1, 0,
                                  D)
    assert st == oracle.OK
    c = upload(case)
    flags = flag_word()
    out = swrt.paged_quantize(c, torch.tensor([0, 1], dtype=torch.int32, device=DEV),
                              torch.tensor(dst, dtype=torch.int64, device=DEV), base, end, I8, 0.1,
                              0, I8, 0.1, 0, D, pages_out=c.pages, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == swrt.FLAG_BAD_PAGES
    np.testing.assert_array_equal(c.arena.cpu().numpy(), case.arena)
    assert out.cpu().numpy().tobytes() == tb.tobytes()
    # a bad page anywhere in the table stops everything, selected or not
    t = tb.copy()
    t[case.n_pages - 1]["capacity"] = 0
    c = swrt.PagedCache.upload(t, case.page_ptr, case.page_ids, case.arena, DEV)
    flags = flag_word()
    swrt.paged_quantize(c, torch.tensor([0], dtype=torch.int32, device=DEV),
                        torch.tensor([base, base + 128], dtype=torch.int64, device=DEV), base, end,
                        I8, 0.1, 0, I8, 0.1, 0, D, pages_out=c.pages, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == swrt.FLAG_BAD_PAGES
    np.testing.assert_array_equal(c.arena.cpu().numpy(), case.arena)


# -- append ---------------------------------------------------------------------------

@pytest.mark.parametrize("new_dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_paged_append_open_equals_the_oracle(orc, new_dtype):
    """The open-page extension."""
    g = wl.rng(64)
    D, S = 64, 24
    T = g.integers(0, 50, S)
    T[0], T[1] = 0, 16  # a stream without pages; one whose only page is full
    streams = [wl.page_split(g, int(t), 16 if i == 1 else int(g.choice([4, 8, 16])), 0.3)
               for i, t in enumerate(T)]
    streams[1] = [(16, 16)]
    case = wl.paged_case(g, D, streams, random_format(g))
    tb = otable(case)
    kn = torch.from_numpy(g.uniform(-2, 2, (S, D)).astype(np.float32)).to(new_dtype)
    vn = torch.from_numpy(g.uniform(-2, 2, (S, D)).astype(np.float32)).to(new_dtype)
    ar, pout, fo = orc.paged_append_open(case.arena, tb, case.page_ptr, case.page_ids,
                                         q_host(kn), q_host(vn), QT[new_dtype], D)
    c = upload(case)
    flags = flag_word()
    swrt.paged_append_open([c], [kn.to(DEV)], [vn.to(DEV)], flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == fo
    assert fo == swrt.FLAG_BAD_PAGES | swrt.FLAG_PAGE_FULL
    np.testing.assert_array_equal(c.arena.cpu().numpy(), ar)
    assert c.table().tobytes() == pout.tobytes()


def test_paged_append_open_shared_table_grows_once_then_attention_sees_it(orc):
    g = wl.rng(65)
    D, B, Hkv, n = 64, 2, 4, 3
    S = B * Hkv
    streams = [wl.page_split(g, int(t), 16) for t in g.integers(1, 60, S)]
    cases = [wl.paged_case(wl.rng(80), D, streams, lambda s, i, m: (BF16, BF16, 1.0, 1.0, 0, 0),
                           payload_rng=wl.rng(90 + i)) for i in range(n)]
    table = swrt.PagedCache.upload(swrt.page_table(cases[0].fields), cases[0].page_ptr,
                                   cases[0].page_ids, cases[0].arena, DEV)
    caches = [swrt.PagedCache(torch.from_numpy(c.arena).to(DEV), table.pages, table.page_ptr,
                              table.page_ids) for c in cases]
    kn = [torch.from_numpy(g.uniform(-1, 1, (S, D)).astype(np.float32)).to(torch.bfloat16)
          for _ in range(n)]
    vn = [torch.from_numpy(g.uniform(-1, 1, (S, D)).astype(np.float32)).to(torch.bfloat16)
          for _ in range(n)]
    full = int((cases[0].fields["length"] == cases[0].fields["capacity"])[
        cases[0].page_ids[cases[0].page_ptr[1:] - 1]].sum())
    flags = flag_word()
    swrt.paged_append_open(caches, [k.to(DEV) for k in kn], [v.to(DEV) for v in vn], flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == (swrt.FLAG_PAGE_FULL if full else 0)
    tb0 = otable(cases[0])
    for i in range(n):
        ar, pout, _ = orc.paged_append_open(cases[i].arena, tb0, cases[0].page_ptr,
                                            cases[0].page_ids, q_host(kn[i]), q_host(vn[i]),
                                            oracle.XF_BF16, D)
        np.testing.assert_array_equal(caches[i].arena.cpu().numpy(), ar)
        assert table.table().tobytes() == pout.tobytes()  # grew once, not n times
    # attention with a zero left window returns each appended V exactly
    q = torch.from_numpy(g.uniform(-1, 1, (B, 8, D)).astype(np.float32)).to(torch.bfloat16)
    outs = swrt.paged_attention([q.to(DEV)] * n, caches, 0, Hkv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    last = cases[0].page_ids[cases[0].page_ptr[1:] - 1]
    lengths0 = cases[0].fields["length"][last]
    caps = cases[0].fields["capacity"][last]
    for i in range(n):
        for s in range(S):
            if lengths0[s] == caps[s]:
                continue
            got = outs[i][s // Hkv, (s % Hkv) * 2:(s % Hkv) * 2 + 2].cpu().numpy()
            want = vn[i][s].float().cpu().numpy()
            np.testing.assert_array_equal(got, np.stack([want, want]))


def slotted_upload(case, stride: int, extra_pages: int, table=None, arena=None):
    """The case as a slotted block table on the device with ``extra_pages``
    free descriptors after its pages; returns (cache, host descriptors,
    page_count, page_ids)."""
    n = len(case.page_ptr) - 1
    count = np.diff(case.page_ptr).astype(np.int32)
    ids = np.full(n * stride, -1, np.int32)
    for s in range(n):
        ids[s * stride:s * stride + count[s]] = case.page_ids[case.page_ptr[s]:case.page_ptr[s + 1]]
    base = otable(case) if table is None else table
    tb = np.zeros(len(base) + extra_pages, oracle.PAGE_DTYPE)
    tb[:len(base)] = base
    ar = case.arena if arena is None else arena
    cache = swrt.PagedCache.upload(tb.view(swrt.PAGE_DTYPE), None, ids, ar, DEV,
                                   page_count=count, page_stride=stride)
    return cache, tb, count, ids


def sealed_both(orc, cache, tb, count, ids, arena, kn, vn, first, free, fmt):
    """The sealed append on the device and in the oracle; returns the flags of
    both and the oracle's (arena, descriptors, count, ids)."""
    kf, ks, kz, vf, vs, vz = fmt
    NS, S, D = kn.shape
    flags = flag_word()
    swrt.paged_append([cache], [kn.to(DEV)], [vn.to(DEV)], first_id=first, free_begin=free,
                      free_end=cache.arena.numel(), k_format=kf, k_scale=ks, k_zero_point=kz,
                      v_format=vf, v_scale=vs, v_zero_point=vz, flags=flags)
    st, ar, pout, cnt, ids2, fo, written = orc.paged_append(
        arena, tb, count, cache.page_stride, ids, q_host(kn), q_host(vn), QT[kn.dtype], S, D, D,
        first, free, len(arena), kf, ks, kz, vf, vs, vz)
    assert st == oracle.OK
    torch.cuda.synchronize()
    return int(flags.item()), fo, (ar, pout, cnt, ids2), written


@pytest.mark.parametrize("S", [1, 4])
@pytest.mark.parametrize("new_dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_paged_sealed_append_equals_the_oracle(orc, new_dtype, S):
    """One new block per stream in every target format pair: arena,
    descriptors and the slotted block table byte for byte; streams that are
    empty, have no free slot, or whose last block is bad are handled as the
    oracle handles them; no byte outside the new blocks changes."""
    g = wl.rng(70 + S)
    D, NS = 64, 24
    T = g.integers(0, 60, NS)
    T[0] = 0
    streams = [wl.page_split(g, int(t), int(g.choice([4, 8, 16])), 0.3) for t in T]
    stride = max(len(st) for st in streams) + 1
    streams[1] = [(4, 4)] * stride  # every slot in use
    streams[2] = [(3, 4), (2, 4)]
    case = wl.paged_case(g, D, streams, random_format(g), spare_bytes=NS * S * D * 4 * 2 + 4096)
    tbase = otable(case)
    tbase[case.page_ids[case.page_ptr[3] - 1]]["capacity"] = 0  # stream 2: a bad last block
    for fmt in [(I8, 0.05, 3, U4, 0.25, 8), (BF16, 1.0, 0, F32, 1.0, 0), (I2, 0.5, -1, U2, 0.3, 2),
                (F16, 1.0, 0, I4, 0.125, -2), (U8, 0.02, 128, BF16, 1.0, 0)]:
        say("paged sealed append", new_dtype, S, fmt)
        cache, tb, count, ids = slotted_upload(case, stride, NS, table=tbase)
        kn = torch.from_numpy(g.uniform(-2, 2, (NS, S, D)).astype(np.float32)).to(new_dtype)
        vn = torch.from_numpy(g.uniform(-2, 2, (NS, S, D)).astype(np.float32)).to(new_dtype)
        free = case.free_offset + 16
        fg, fo, (ar, pout, cnt, ids2), written = sealed_both(orc, cache, tb, count, ids,
                                                             case.arena, kn, vn, case.n_pages,
                                                             free, fmt)
        assert fg == fo == swrt.FLAG_BAD_PAGES | swrt.FLAG_PAGE_FULL
        np.testing.assert_array_equal(cache.arena.cpu().numpy(), ar)
        assert cache.table().tobytes() == pout.tobytes()
        np.testing.assert_array_equal(cache.page_count.cpu().numpy(), cnt)
        np.testing.assert_array_equal(cache.page_ids.cpu().numpy(), ids2)
        bits = oracle.PAGE_BITS[fmt[0]] + oracle.PAGE_BITS[fmt[3]]
        assert list(cnt - count) == [1] + [0, 0] + [1] * (NS - 3)  # streams 1 and 2 skipped
        assert written == (NS - 2) * S * D * bits // 8
        # nothing outside the new payloads changed
        keep = np.ones(len(ar), bool)
        keep[free:free + NS * S * D * bits // 8] = False
        np.testing.assert_array_equal(ar[keep], case.arena[keep])


def test_paged_sealed_decode_loop_shared_table_then_attention(orc):
    """Layers sharing one slotted block table take a one-token block per
    stream and step (the descriptors and the table grow once per step, every
    arena gets its rows); attention then reads the old pages and every new
    block: a zero left window returns each stream's last V exactly, a wide one
    stays within the attention bound of the oracle."""
    g = wl.rng(75)
    D, B, Hkv, Hq, n, steps = 64, 2, 4, 8, 3, 5
    NS = B * Hkv
    streams = [wl.page_split(g, int(t), 16) for t in g.integers(1, 60, NS)]
    stride = max(len(st) for st in streams) + steps
    spare = steps * NS * 2 * D * 2
    cases = [wl.paged_case(wl.rng(80), D, streams, lambda s, i, m: (BF16, BF16, 1.0, 1.0, 0, 0),
                           payload_rng=wl.rng(90 + i), spare_bytes=spare) for i in range(n)]
    base, tb, count, ids = slotted_upload(cases[0], stride, steps * NS)
    caches = [swrt.PagedCache(torch.from_numpy(c.arena).to(DEV), base.pages, None, base.page_ids,
                              base.page_count, stride) for c in cases]
    arenas = [c.arena.copy() for c in cases]
    first, free = cases[0].n_pages, cases[0].free_offset
    for step in range(steps):
        kn = [torch.from_numpy(g.uniform(-1, 1, (NS, 1, D)).astype(np.float32)).to(torch.bfloat16)
              for _ in range(n)]
        vn = [torch.from_numpy(g.uniform(-1, 1, (NS, 1, D)).astype(np.float32)).to(torch.bfloat16)
              for _ in range(n)]
        flags = flag_word()
        swrt.paged_append(caches, [k.to(DEV) for k in kn], [v.to(DEV) for v in vn],
                          first_id=first, free_begin=free, free_end=len(arenas[0]),
                          k_format=BF16, v_format=BF16, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        for i in range(n):
            st, arenas[i], tb_i, cnt, ids_i, fo, w = orc.paged_append(
                arenas[i], tb, count, stride, ids, q_host(kn[i]), q_host(vn[i]), oracle.XF_BF16,
                1, D, D, first, free, len(arenas[i]), BF16, 1.0, 0, BF16, 1.0, 0)
            assert st == oracle.OK and fo == 0
            np.testing.assert_array_equal(caches[i].arena.cpu().numpy(), arenas[i])
        tb, count, ids = tb_i, cnt, ids_i
        assert base.table().tobytes() == tb.tobytes()  # grew once, not n times
        np.testing.assert_array_equal(base.page_count.cpu().numpy(), count)
        np.testing.assert_array_equal(base.page_ids.cpu().numpy(), ids)
        first += NS
        free += w
    q = torch.from_numpy(g.uniform(-1, 1, (B, Hq, D)).astype(np.float32)).to(torch.bfloat16)
    outs = swrt.paged_attention([q.to(DEV)] * n, caches, 0, Hkv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for i in range(n):
        for s in range(NS):
            got = outs[i][s // Hkv, (s % Hkv) * G:(s % Hkv + 1) * G].cpu().numpy()
            want = vn[i][s, 0].float().cpu().numpy()
            np.testing.assert_array_equal(got, np.stack([want] * G))
    flags = flag_word()
    outs = swrt.paged_attention([q.to(DEV)] * n, caches, 40, Hkv, out_dtype=torch.float32,
                                flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    ptr = np.concatenate([[0], np.cumsum(count)]).astype(np.int32)
    flat = np.concatenate([ids[s * stride:s * stride + count[s]] for s in range(NS)])
    for i in range(n):
        ref, f = orc.paged_attention(q_host(q), oracle.XF_BF16, arenas[i], tb, None, ids, 40, Hkv,
                                     D ** -0.5, page_count=count, page_stride=stride)
        ref2, _ = orc.paged_attention(q_host(q), oracle.XF_BF16, arenas[i], tb, ptr, flat, 40,
                                      Hkv, D ** -0.5)
        assert f == 0
        np.testing.assert_array_equal(ref, ref2)  # the two table forms agree
        case = wl.PagedCase(D, {}, ptr, flat, arenas[i], 0)
        tol = bound(case, tb, q, Hkv, 40, D ** -0.5, torch.float32, ref)
        assert (np.abs(outs[i].cpu().numpy() - ref) <= tol).all()


def test_paged_sealed_append_layout_rule(orc):
    """The library's layout rule: payload rows of 16-byte blocks. Rows of 8
    bytes (int2, head_dim 32) and a free region off a 16-byte boundary are
    refused at the boundary (the oracle, which follows the pages, takes them);
    two tokens per block make the int2 payload 16 bytes again."""
    g = wl.rng(76)
    D, NS = 32, 4
    case = wl.paged_case(g, D, [wl.page_split(g, 5, 4) for _ in range(NS)],
                         lambda s, i, n: (BF16, BF16, 1.0, 1.0, 0, 0), spare_bytes=4096)
    cache, tb, count, ids = slotted_upload(case, 4, NS)
    kn = torch.zeros((NS, 1, D), dtype=torch.bfloat16, device=DEV)
    free = case.free_offset
    for kw in (dict(v_format=I2, v_scale=0.5), dict(free_begin=free + 8)):
        a = dict(first_id=case.n_pages, free_begin=free, free_end=len(case.arena),
                 k_format=BF16, v_format=BF16)
        a.update(kw)
        with pytest.raises(swrt.SwrtError) as e:
            swrt.paged_append([cache], [kn], [kn], **a)
        assert e.value.status == swrt.E_UNSUPPORTED
        st = orc.paged_append(case.arena, tb, count, 4, ids, q_host(kn), q_host(kn),
                              oracle.XF_BF16, 1, D, D, a["first_id"], a["free_begin"],
                              a["free_end"], a["k_format"], 1.0, 0, a["v_format"],
                              a.get("v_scale", 1.0), 0)[0]
        assert st == oracle.OK
    kn2 = torch.zeros((NS, 2, D), dtype=torch.bfloat16, device=DEV)
    swrt.paged_append([cache], [kn2], [kn2], first_id=case.n_pages, free_begin=free,
                      free_end=len(case.arena), k_format=BF16, v_format=I2, v_scale=0.5)
    torch.cuda.synchronize()
    assert list(cache.page_count.cpu().numpy()) == list(count + 1)


def test_workload9_full_size(orc):
    """The paged decode step at full size in the launch configuration the
    benchmark times: attention over all 12 layers (every output compared),
    then the cooling conversion of every stream's oldest hot page in one layer,
    one sealed append into every stream of every layer (bytes compared) and
    attention again over the grown table."""
    from sliding_window_ring_tensor_amd.paged_step import PagedDecodeStep
    spec = wl.workload9()
    say("workload 9 full size")
    st = PagedDecodeStep(spec, DEV, set_id=0, spare_bytes=2 << 20)
    st.attention()
    torch.cuda.synchronize()
    assert int(st.flags.item()) == 0
    tb = st.table_host.view(oracle.PAGE_DTYPE)
    case = wl.PagedCase(spec.head_dim, st.fields, st.page_ptr_host, st.page_ids_host, None, 0)
    worst = 0.0
    for i in range(spec.layers):
        arena = st.arenas[i].cpu().numpy()
        ref, f = orc.paged_attention(q_host(st.qs[i]), oracle.XF_BF16, arena, tb,
                                     st.page_ptr_host, st.page_ids_host, spec.left_window,
                                     spec.kv_heads, spec.head_dim ** -0.5)
        assert f == 0
        case.arena = arena
        tol = bound(case, tb, st.qs[i], spec.kv_heads, spec.left_window, spec.head_dim ** -0.5,
                    torch.bfloat16, ref)
        err = np.abs(st.outs[i].float().cpu().numpy() - ref)
        assert (err <= tol).all(), f"layer {i}: max err/tol {np.max(err / tol):.3g}"
        worst = max(worst, float(np.max(err / tol)))
    say("  attention worst err/tol", round(worst, 4))
    # cooling: the oldest hot page of every stream, bf16 -> int8, in layer 3
    blocks, dst, cool_bytes = st.cooling_selection()
    arena = st.arenas[3].cpu().numpy()
    code, ar, pout = orc.paged_quantize(arena, tb, blocks, dst, st.layout_bytes, len(arena),
                                        spec.cold_format, spec.k_scale, 0, spec.cold_format,
                                        spec.v_scale, 0, spec.head_dim)
    assert code == oracle.OK
    flags = flag_word()
    out = swrt.paged_quantize(st.caches[3], torch.from_numpy(blocks).to(DEV),
                              torch.from_numpy(dst).to(DEV), st.layout_bytes, len(arena),
                              spec.cold_format, spec.k_scale, 0, spec.cold_format, spec.v_scale, 0,
                              spec.head_dim, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    np.testing.assert_array_equal(st.arenas[3].cpu().numpy(), ar)
    assert out.cpu().numpy().tobytes() == pout.tobytes()
    # sealed append: one new one-token block per stream, every layer, one
    # slotted block table; attention then reads the new blocks too
    NS = spec.batch * spec.kv_heads
    count = np.diff(st.page_ptr_host).astype(np.int32)
    stride = int(count.max()) + 1
    ids = np.full(NS * stride, -1, np.int32)
    for s_ in range(NS):
        ids[s_ * stride:s_ * stride + count[s_]] = \
            st.page_ids_host[st.page_ptr_host[s_]:st.page_ptr_host[s_ + 1]]
    tb2 = np.zeros(len(tb) + NS, oracle.PAGE_DTYPE)
    tb2[:len(tb)] = tb
    base = swrt.PagedCache.upload(tb2.view(swrt.PAGE_DTYPE), None, ids, st.arenas[0], DEV,
                                  page_count=count, page_stride=stride)
    caches = [swrt.PagedCache(a, base.pages, None, base.page_ids, base.page_count, stride)
              for a in st.arenas]
    free = st.layout_bytes + (-(-cool_bytes // 16)) * 16
    kn = [wl.device_payload((NS, 1, spec.head_dim), torch.bfloat16, 9, 300 + i, DEV)
          for i in range(spec.layers)]
    vn = [wl.device_payload((NS, 1, spec.head_dim), torch.bfloat16, 9, 400 + i, DEV)
          for i in range(spec.layers)]
    before = [a.cpu().numpy() for a in st.arenas]
    flags = flag_word()
    swrt.paged_append(caches, kn, vn, first_id=len(tb), free_begin=free,
                      free_end=len(before[0]), k_format=spec.hot_format,
                      v_format=spec.hot_format, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    for i in (0, 7, 11):
        code, ar, pout, cnt, ids2, f, _ = orc.paged_append(
            before[i], tb2, count, stride, ids, q_host(kn[i]), q_host(vn[i]), oracle.XF_BF16, 1,
            spec.head_dim, spec.head_dim, len(tb), free, len(before[i]), spec.hot_format, 1.0, 0,
            spec.hot_format, 1.0, 0)
        assert code == oracle.OK and f == 0
        np.testing.assert_array_equal(st.arenas[i].cpu().numpy(), ar)
        assert base.table().tobytes() == pout.tobytes()
        np.testing.assert_array_equal(base.page_count.cpu().numpy(), cnt)
        np.testing.assert_array_equal(base.page_ids.cpu().numpy(), ids2)
    flags = flag_word()
    outs = swrt.paged_attention(st.qs, caches, spec.left_window, spec.kv_heads, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    ptr = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    flat = np.concatenate([ids2[s_ * stride:s_ * stride + cnt[s_]] for s_ in range(NS)])
    for i in (0, 11):
        arena = st.arenas[i].cpu().numpy()
        ref, f = orc.paged_attention(q_host(st.qs[i]), oracle.XF_BF16, arena, pout, None, ids2,
                                     spec.left_window, spec.kv_heads, spec.head_dim ** -0.5,
                                     page_count=cnt, page_stride=stride)
        assert f == 0
        case = wl.PagedCase(spec.head_dim, {}, ptr, flat, arena, 0)
        tol = bound(case, pout, st.qs[i], spec.kv_heads, spec.left_window,
                    spec.head_dim ** -0.5, torch.bfloat16, ref)
        err = np.abs(outs[i].float().cpu().numpy() - ref)
        assert (err <= tol).all(), f"after the append, layer {i}: max err/tol {np.max(err / tol):.3g}"
