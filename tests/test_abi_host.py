"""C-ABI checks that need no GPU.

- libswrt.so loads and exports every function include/swrt.h declares;
- the header's constants agree with the Python binding and (by value) with
  the oracle's own constants;
- host validation rejects bad arguments with the documented status before
  anything is launched;
- the multiply-shift divider used by the kernels' index math is exact.

The validation calls pass made-up, never dereferenced addresses. They only run
where no GPU is visible, so a validation bug can never turn into a launch on a
real device; the GPU suite repeats the interesting rejections with real
buffers.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest
import torch

import oracle
import sliding_window_ring_tensor_amd as swrt
from sliding_window_ring_tensor_amd import build as swrt_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swrt.h")

no_gpu_visible = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                    reason="made-up addresses are only passed with no GPU visible")


@pytest.fixture(scope="session")
def L():
    if not os.path.exists(swrt.LIBRARY):
        swrt_build.build()
    return swrt.lib()


def _header():
    return open(HEADER).read()


def test_exports_every_declared_function(L):
    declared = set(re.findall(r"^(?:int|const char \*)\s*(swrt_\w+)\s*\(", _header(), re.M))
    assert {"swrt_tensor_scatter", "swrt_tensor_scatter_batched", "swrt_kv_seq_lengths", "swrt_kv_window_append",
            "swrt_kv_window_append_layers", "swrt_kv_decode_step", "swrt_kv_seq_lengths_drift",
            "swrt_kv_window_append_xf", "swrt_tensor_scatter_xf", "swrt_kv_decode_step_xf",
            "swrt_window_attention", "swrt_paged_attention", "swrt_paged_quantize",
            "swrt_paged_append", "swrt_paged_append_open", "swrt_kv_window_append_noalloc",
            "swrt_status_string",
            "swrt_abi_version"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", swrt.LIBRARY], check=True,
                         capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (swrt_\w+)", out))
    assert declared <= exported, declared - exported
    for name in declared:
        assert hasattr(L, name)


def test_constants_agree():
    defs = dict(re.findall(r"#define (SWRT_\w+) (\d+)u?", _header()))
    assert int(defs["SWRT_ABI_VERSION"]) == swrt.ABI_VERSION
    py = {"SWRT_OK": swrt.OK, "SWRT_E_INVALID_ARG": swrt.E_INVALID_ARG,
          "SWRT_E_UNSUPPORTED": swrt.E_UNSUPPORTED, "SWRT_E_LAUNCH": swrt.E_LAUNCH,
          "SWRT_FLAG_LINEAR_OOB": swrt.FLAG_LINEAR_OOB, "SWRT_FLAG_BAD_SEQLEN": swrt.FLAG_BAD_SEQLEN,
          "SWRT_FLAG_BAD_LENGTHS": swrt.FLAG_BAD_LENGTHS, "SWRT_MODE_LINEAR": swrt.MODE_LINEAR,
          "SWRT_MODE_CIRCULAR": swrt.MODE_CIRCULAR, "SWRT_PHASE_STAGE": swrt.PHASE_STAGE,
          "SWRT_PHASE_COMMIT": swrt.PHASE_COMMIT, "SWRT_PHASE_ALL": swrt.PHASE_ALL,
          "SWRT_MAX_LAYERS": swrt.MAX_LAYERS, "SWRT_MAX_BATCHED": swrt.MAX_BATCHED,
          "SWRT_FLAG_ROPE_RANGE": swrt.FLAG_ROPE_RANGE,
          "SWRT_XF_F32": swrt.XF_TYPES[torch.float32], "SWRT_XF_F16": swrt.XF_TYPES[torch.float16],
          "SWRT_XF_BF16": swrt.XF_TYPES[torch.bfloat16], "SWRT_XF_INT8": swrt.XF_TYPES[torch.int8],
          "SWRT_XF_UINT8": swrt.XF_TYPES[torch.uint8],
          "SWRT_XF_INT4": swrt.PAGE_FORMATS["int4"], "SWRT_XF_UINT4": swrt.PAGE_FORMATS["uint4"],
          "SWRT_XF_INT2": swrt.PAGE_FORMATS["int2"], "SWRT_XF_UINT2": swrt.PAGE_FORMATS["uint2"],
          "SWRT_FLAG_BAD_PAGES": swrt.FLAG_BAD_PAGES, "SWRT_FLAG_PAGE_FULL": swrt.FLAG_PAGE_FULL}
    for k, v in py.items():
        assert int(defs[k]) == v, k
    # the oracle defines its own values; they must mean the same bits
    assert oracle.FLAG_LINEAR_OOB == swrt.FLAG_LINEAR_OOB
    assert oracle.FLAG_BAD_SEQLEN == swrt.FLAG_BAD_SEQLEN
    assert oracle.FLAG_BAD_LENGTHS == swrt.FLAG_BAD_LENGTHS
    assert oracle.FLAG_ROPE_RANGE == swrt.FLAG_ROPE_RANGE
    assert (oracle.XF_F32, oracle.XF_F16, oracle.XF_BF16, oracle.XF_INT8, oracle.XF_UINT8) == \
        tuple(swrt.XF_TYPES[t] for t in (torch.float32, torch.float16, torch.bfloat16, torch.int8,
                                          torch.uint8))
    # the two transform structs have the same field layout
    assert [f[0] for f in oracle.RowXf._fields_] == [f[0] for f in swrt.RowTransform._fields_]
    assert ctypes.sizeof(oracle.RowXf) == ctypes.sizeof(swrt.RowTransform)
    # page formats, flags and the descriptor layout
    assert {k: oracle_v for k, oracle_v in (("int4", oracle.XF_INT4), ("uint4", oracle.XF_UINT4),
                                            ("int2", oracle.XF_INT2), ("uint2", oracle.XF_UINT2))} \
        == {k: swrt.PAGE_FORMATS[k] for k in ("int4", "uint4", "int2", "uint2")}
    assert (oracle.FLAG_BAD_PAGES, oracle.FLAG_PAGE_FULL) == (swrt.FLAG_BAD_PAGES, swrt.FLAG_PAGE_FULL)
    assert oracle.PAGE_DTYPE == swrt.PAGE_DTYPE and swrt.PAGE_DTYPE.itemsize == 64
    assert ctypes.sizeof(swrt.PagedLayer) == 88
    assert (oracle.MODE_LINEAR, oracle.MODE_CIRCULAR) == (swrt.MODE_LINEAR, swrt.MODE_CIRCULAR)
    assert (oracle.PHASE_STAGE, oracle.PHASE_COMMIT, oracle.PHASE_ALL) == \
        (swrt.PHASE_STAGE, swrt.PHASE_COMMIT, swrt.PHASE_ALL)


def test_status_strings(L):
    for code in (0, 1, 2, 3, 99, -1):
        assert isinstance(L.swrt_status_string(code), bytes)
    assert L.swrt_status_string(0) == b"ok"
    assert L.swrt_abi_version() == swrt.ABI_VERSION


def test_binding_refuses_cpu_tensors():
    t = torch.zeros(2, 3, 4)
    with pytest.raises(swrt.SwrtError):
        swrt.tensor_scatter(t, t[:, :1].contiguous(), None, axis=1)


def test_binding_checks_batch_and_staging_counts():
    """Host-side checks of the bindings, before any device work: seqlens_k must
    hold one entry per batch entry and there is one staging buffer per layer."""
    B, H, C, S, D = 3, 2, 8, 4, 16
    z = lambda *shape: torch.zeros(*shape, dtype=torch.bfloat16)  # noqa: E731
    kc, kn, ks = z(B, H, C, D), z(B, H, S, D), z(B, H, C + S, D)
    sk = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(swrt.SwrtError, match="one entry per batch entry"):
        swrt.prepare_kv_window_stage_step([kc], [kc], [kn], [kn], sk[:2], [ks], [ks])
    with pytest.raises(swrt.SwrtError, match="one entry per batch entry"):
        swrt.prepare_kv_decode_step([kc], [kc], [kn[:, :, :1]], [kn[:, :, :1]], sk[:1], [], [],
                                    None)
    with pytest.raises(swrt.SwrtError, match="staging buffer per layer"):
        swrt.prepare_kv_window_stage_step([kc, kc], [kc, kc], [kn, kn], [kn, kn], sk, [ks],
                                          [ks])
    with pytest.raises(swrt.SwrtError, match="staging buffer per layer"):
        swrt.prepare_kv_window_append_layers([kc, kc], [kc, kc], [kn, kn], [kn, kn],
                                             sk, sk, k_stagings=[ks], v_stagings=[ks])


def test_binding_checks_tensor_scatter_shapes():
    """Host-side checks of the TensorScatter bindings ([TS] Inputs): the update
    matches past on every axis but the sequence axis, write_indices holds one
    int64 index per batch entry and the flag word is int32. The library only
    sees past's shape, so a narrower update or a short index vector would
    otherwise be read past its end on the device."""
    past = torch.zeros(2, 3, 16, 8, dtype=torch.float32)
    upd = torch.zeros(2, 3, 4, 8, dtype=torch.float32)
    wi = torch.zeros(2, dtype=torch.int64)
    fl = torch.zeros(1, dtype=torch.int32)
    for bad in (torch.zeros(2, 3, 4, 4), torch.zeros(2, 2, 4, 8), torch.zeros(1, 3, 4, 8)):
        with pytest.raises(swrt.SwrtError, match="must match past"):
            swrt.prepare_tensor_scatter(past, bad, wi, axis=2)
        with pytest.raises(swrt.SwrtError, match="must match past"):
            swrt.prepare_tensor_scatter_batched([past], [bad], wi, axis=-2)
    for bad in (wi[:1], torch.zeros(3, dtype=torch.int64), torch.zeros(2, dtype=torch.int32),
                torch.zeros(2, 1, dtype=torch.int64)):
        with pytest.raises(swrt.SwrtError, match="one index per batch entry"):
            swrt.prepare_tensor_scatter(past, upd, bad, axis=2)
    for bad in (torch.zeros(1, dtype=torch.int64), torch.zeros(0, dtype=torch.int32)):
        with pytest.raises(swrt.SwrtError, match="int32 tensor with at least one element"):
            swrt.prepare_tensor_scatter(past, upd, wi, axis=2, flags=bad)
    # the fused form: [..., S, head_dim] updates, the same index and flag checks
    xf = swrt.Transform()
    kc = torch.zeros(2, 3, 16, 8, dtype=torch.bfloat16)
    ku = torch.zeros(2, 3, 4, 8, dtype=torch.bfloat16)
    with pytest.raises(swrt.SwrtError, match="other dims"):
        swrt.prepare_tensor_scatter_xf([kc], [ku[:, :2]], [0], wi, xf)
    with pytest.raises(swrt.SwrtError, match="one index per batch entry"):
        swrt.prepare_tensor_scatter_xf([kc], [ku], [0], wi[:1], xf)
    with pytest.raises(swrt.SwrtError, match="int32 tensor with at least one element"):
        swrt.prepare_tensor_scatter_xf([kc], [ku], [0], wi, xf, flags=fl.to(torch.int64))
    # a well-formed call gets as far as the device check (CPU tensors here)
    with pytest.raises(swrt.SwrtError, match="GPU only"):
        swrt.prepare_tensor_scatter(past, upd, wi, axis=2, flags=fl)


def test_fastdiv_exact(tmp_path):
    exe = str(tmp_path / "fastdiv_check")
    subprocess.run([swrt_build.HIPCC, "-x", "hip", f"--offload-arch={swrt_build.ARCH}", "-O2",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "fastdiv_check.cpp"), "-o", exe],
                   check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout


# ---------------------------------------------------------------------------
# host validation (made-up addresses, never dereferenced)
# ---------------------------------------------------------------------------

A, B_, C_, D_ = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000, 0x40_0000_0000
I64 = ctypes.c_int64


def _shape(*d):
    return (I64 * len(d))(*d)


def _ts(L, present=A, past=A, update=B_, wi=None, shape=(2, 3, 16, 8), rank=None, axis=-2,
        S=2, mode=0, bits=32, flags=None):
    rank = len(shape) if rank is None else rank
    return L.swrt_tensor_scatter(present, past, update, wi, _shape(*shape), rank, axis, S, mode,
                                 bits, flags, None)


@no_gpu_visible
def test_tensor_scatter_rejects(L):
    INV, UNS, OK = swrt.E_INVALID_ARG, swrt.E_UNSUPPORTED, swrt.OK
    assert _ts(L, shape=(2, 3, 16, 8), rank=1) == INV
    assert _ts(L, shape=(2,) * 9) == INV
    for axis in (0, 4, -5, -4):
        assert _ts(L, axis=axis) == INV
    assert _ts(L, mode=2) == INV
    for bits in (0, 12, 256):
        assert _ts(L, bits=bits) == INV
    assert _ts(L, S=17) == INV and _ts(L, S=-1) == INV
    assert _ts(L, shape=(2, -3, 16, 8)) == INV
    assert _ts(L, shape=(2, 3, 16, 3), bits=4) == UNS                   # 1.5-byte rows
    assert _ts(L, present=0, past=0) == INV
    assert _ts(L, update=0) == INV
    assert _ts(L, present=A + 2, past=A + 2) == INV                     # fp32 misaligned
    assert _ts(L, update=A + 64) == INV                                 # update inside present
    assert _ts(L, present=A, past=A + 256) == INV                       # present overlaps past
    assert _ts(L, wi=A + 8) == INV                                      # indices inside present
    assert _ts(L, wi=B_ + 4 * 2 * 3 * 2 * 8 + 4) == INV                 # misaligned int64
    # no-ops return OK without launching
    assert _ts(L, shape=(0, 3, 16, 8)) == OK
    assert _ts(L, shape=(2, 3, 16, 0)) == OK
    assert _ts(L, S=0) == OK                                            # in place, empty update
    # batched: mixing in-place and out-of-place tensors, too many tensors, a
    # present shared by two tensors
    V = ctypes.c_void_p
    shp = _shape(2, 3, 16, 8)
    st = L.swrt_tensor_scatter_batched(2, (V * 2)(A, C_), (V * 2)(A, D_), (V * 2)(B_, B_), None,
                                       shp, 4, -2, 2, 0, 32, None, None)
    assert st == INV
    many = (V * 65)(*([A] * 65))
    assert L.swrt_tensor_scatter_batched(65, many, many, many, None, shp, 4, -2, 2, 0, 32, None,
                                         None) == INV
    st = L.swrt_tensor_scatter_batched(2, (V * 2)(A, A), (V * 2)(A, A), (V * 2)(B_, B_), None,
                                       shp, 4, -2, 2, 0, 32, None, None)
    assert st == INV


def _lens(L, sk=A, batch=4, S=1, C=8, T=B_, P=B_ + 0x1000, Lp=C_, Lt=C_ + 0x1000, E=D_, W=None):
    return L.swrt_kv_seq_lengths(sk, batch, S, C, T, P, Lp, Lt, E, W, None, None)


@no_gpu_visible
def test_kv_seq_lengths_rejects(L):
    INV = swrt.E_INVALID_ARG
    assert _lens(L, batch=-1) == INV
    assert _lens(L, S=0) == INV and _lens(L, C=0) == INV
    assert _lens(L, sk=0) == INV and _lens(L, Lp=0) == INV and _lens(L, E=0) == INV
    assert _lens(L, sk=A + 2) == INV and _lens(L, T=B_ + 4) == INV
    assert _lens(L, Lt=C_ + 8) == INV                                   # overlaps Lp
    assert _lens(L, E=A) == INV                                         # overlaps seqlens_k
    assert _lens(L, batch=0) == swrt.OK
    assert _lens(L, W=D_ + 0x1004) == INV                               # work prefix: 8-byte
    assert _lens(L, W=D_ + 8) == INV                                    # overlaps E
    assert _lens(L, W=D_ + 0x1000) in (swrt.OK, swrt.E_LAUNCH)          # [batch + 1] int64
    drift = L.swrt_kv_seq_lengths_drift
    assert drift(A, 4, 1, 8, 0, B_, B_ + 0x1000, C_, C_ + 0x1000, D_, None, None, None) == INV
    assert drift(A, 4, 1, 8, 9, B_, B_ + 0x1000, C_, C_ + 0x1000, D_, None, None, None) == INV
    assert drift(A, 0, 1, 8, 5, B_, B_ + 0x1000, C_, C_ + 0x1000, D_, None, None,
                 None) == swrt.OK


def _win(L, kc=A, vc=A + 0x1000_0000, kn=B_, vn=B_ + 0x1000_0000, strides=None, ks=None, vs=None,
         lp=D_, ev=D_ + 0x1000, batch=2, H=2, C=8, S=1, D=16, bits=16, phase=3):
    strides = (I64 * 3)(*(strides or (H * S * D, S * D, D)))
    return L.swrt_kv_window_append(kc, vc, kn, vn, strides, ks, vs, lp, ev, batch, H, C, S, D,
                                   bits, phase, None, None)


@no_gpu_visible
def test_kv_window_append_noalloc_rejects(L):
    """The no-alloc variant refuses a staging buffer beyond half its array, and
    bad arguments, before touching the device."""
    INV, UNS = swrt.E_INVALID_ARG, swrt.E_UNSUPPORTED
    assert swrt.NOALLOC_STAGING_BYTES == 128 << 20

    def na(B=2, H=2, C=8, S=4, D=16, bits=16):
        st = (I64 * 3)(H * S * D, S * D, D)
        return L.swrt_kv_window_append_noalloc(A, A + 0x1000_0000, B_, B_ + 0x1000_0000, st, D_,
                                               D_ + 0x1000, B, H, C, S, D, bits, None, None)
    assert na(C=0) == INV and na(S=0) == INV and na(B=-1) == INV and na(bits=24) == INV
    # (C + S) * D * 2 bytes per slice: 64 MiB + 1 slice row past half the array
    assert na(B=1, H=1, C=4096, S=2, D=8192 + 64) == UNS
    assert na(B=64, H=64, C=4096, S=64, D=128) == UNS
    assert na(B=2**20, H=2**20, C=2**20, S=2, D=128) == UNS  # overflows 64-bit bytes
    assert na(B=0) == swrt.OK or na(B=0) == swrt.E_LAUNCH


@no_gpu_visible
def test_kv_window_append_rejects(L):
    INV, UNS = swrt.E_INVALID_ARG, swrt.E_UNSUPPORTED
    assert _win(L, C=0) == INV and _win(L, S=0) == INV
    assert _win(L, batch=-1) == INV and _win(L, H=-1) == INV and _win(L, D=-1) == INV
    assert _win(L, bits=24) == INV
    assert _win(L, S=4, phase=0, ks=C_, vs=C_ + 0x1000_0000) == INV
    assert _win(L, S=4, phase=4, ks=C_, vs=C_ + 0x1000_0000) == INV
    assert _win(L, S=4) == INV                                          # staging missing
    assert _win(L, strides=(-1, 16, 16)) == INV
    assert _win(L, bits=4, D=3) == UNS                                  # odd 4-bit row
    assert _win(L, kc=0) == INV and _win(L, lp=0) == INV
    assert _win(L, vc=A + 64) == INV                                    # K and V caches overlap
    assert _win(L, kn=A + 32) == INV                                    # new rows inside a cache
    assert _win(L, S=4, ks=A + 512, vs=C_) == INV                       # staging inside a cache
    assert _win(L, S=4, ks=C_, vs=C_ + 64) == INV                       # staging buffers overlap
    assert _win(L, kc=A + 1) == INV                                     # bf16 misaligned
    assert _win(L, lp=A + 16) == INV                                    # lengths inside a cache
    assert _win(L, batch=0) == swrt.OK and _win(L, H=0) == swrt.OK and _win(L, D=0) == swrt.OK
    arr = (ctypes.c_void_p * 33)(*([A] * 33))
    st = L.swrt_kv_window_append_layers(33, arr, arr, arr, arr, (I64 * 3)(32, 16, 16), None, None,
                                        D_, D_ + 0x1000, 2, 2, 8, 1, 16, 16, 3, None, None)
    assert st == INV
    # the same cache in two layers
    kcs = (ctypes.c_void_p * 2)(A, A)
    vcs = (ctypes.c_void_p * 2)(A + 0x1000_0000, A + 0x2000_0000)
    kns = (ctypes.c_void_p * 2)(B_, B_)
    st = L.swrt_kv_window_append_layers(2, kcs, vcs, kns, kns, (I64 * 3)(32, 16, 16), None, None,
                                        D_, D_ + 0x1000, 2, 2, 8, 1, 16, 16, 3, None, None)
    assert st == INV


@no_gpu_visible
def test_kv_decode_step_rejects(L):
    INV = swrt.E_INVALID_ARG
    V = ctypes.c_void_p

    def call(nw=1, nf=1, wk=A, wv=A + 0x1000_0000, fc=C_, sk=D_, C=8, M=16, batch=2, lens=None,
             W=None):
        arr = lambda *p: (V * len(p))(*p)  # noqa: E731
        return L.swrt_kv_decode_step(nw, arr(wk), arr(wv), arr(B_), arr(B_ + 0x1000),
                                     (I64 * 3)(32, 16, 16), sk, C, C if W is None else W, None,
                                     None, lens, None, None,
                                     nf, arr(fc), arr(B_ + 0x2000), D_ + 0x1000, M, batch, 2, 16,
                                     16, None, None)
    assert call(nw=33) == INV and call(nf=65) == INV and call(nw=-1) == INV
    assert call(C=0) == INV and call(batch=-1) == INV
    assert call(sk=0) == INV                                   # windowed layers need seqlens_k
    assert call(fc=A + 64) == INV                              # full cache inside a windowed one
    assert call(M=0) == INV                                    # S = 1 > M
    assert call(lens=D_ + 4) == INV                            # length output inside seqlens_k
    assert call(sk=D_ + 2) == INV                              # misaligned seqlens_k
    assert call(W=0) == INV and call(W=9) == INV               # window outside [1, C]
    assert call(nw=0, nf=0) == swrt.OK                         # nothing to do


@no_gpu_visible
def test_kv_window_stage_step_rejects(L):
    INV = swrt.E_INVALID_ARG
    V = ctypes.c_void_p

    def call(nl=1, kc=A, ks=C_, sk=D_, C=8, S=3, batch=2, cp=D_ + 0x1000, ev=D_ + 0x2000,
             W=None, tot=None):
        arr = lambda *p: (V * len(p))(*p)  # noqa: E731
        return L.swrt_kv_window_stage_step(nl, arr(kc), arr(A + 0x1000_0000), arr(B_),
                                           arr(B_ + 0x1000), (I64 * 3)(96, 48, 16), arr(ks),
                                           arr(C_ + 0x1000_0000), sk, C, C if W is None else W,
                                           tot, None, cp, None, ev, batch, 2, S, 16, 16, None,
                                           None)
    assert call(nl=33) == INV and call(nl=-1) == INV
    assert call(S=1) == INV                                    # one row has no stage phase
    assert call(C=0) == INV and call(batch=-1) == INV
    assert call(sk=0) == INV                                   # seqlens_k required
    assert call(cp=0) == INV and call(ev=0) == INV             # the commit reads Lp and E
    assert call(W=0) == INV and call(W=9) == INV               # window outside [1, C]
    assert call(ks=A + 64) == INV                              # staging inside a cache
    assert call(cp=D_ + 4) == INV                              # length output inside seqlens_k
    assert call(tot=D_ + 0x3004) == INV                        # misaligned int64 output
    assert call(batch=0) == swrt.OK                            # nothing to do
    arr = lambda *p: (V * len(p))(*p)  # noqa: E731
    assert L.swrt_kv_window_stage_step_xf(1, arr(A), arr(A + 0x1000_0000), arr(B_),
                                          arr(B_ + 0x1000), (I64 * 3)(96, 48, 16), arr(C_),
                                          arr(C_ + 0x1000_0000), D_, 8, 8, None, D_ + 0x3000,
                                          D_ + 0x1000, None, D_ + 0x2000, 2, 2, 3, 16, None, None,
                                          None) == INV                 # no transform


def _xf(in_type=1, out_type=4, cos=None, sin=None, max_pos=0, rot=0, scale=(0.5, 0.5), zp=(0, 0)):
    x = swrt.RowTransform()
    x.in_type, x.out_type = in_type, out_type
    x.cos_table, x.sin_table = cos, sin
    x.max_position, x.rotary_dim = max_pos, rot
    x.scale[0], x.scale[1] = scale
    x.zero_point[0], x.zero_point[1] = zp
    return x


@no_gpu_visible
def test_fused_append_rejects(L):
    """Bad transforms and buffers are refused before any launch; good ones get
    as far as the launch (which fails here: no GPU is visible, and these
    made-up addresses are never dereferenced)."""
    INV, V = swrt.E_INVALID_ARG, ctypes.c_void_p
    launched = (swrt.OK, swrt.E_LAUNCH)
    arr = lambda *p: (V * len(p))(*p)  # noqa: E731

    def win(x, kc=A, kn=B_, S=1, D=16, strides=None, past=D_ + 0x2000):
        st = (I64 * 3)(*(strides or (2 * S * D, S * D, D)))
        return L.swrt_kv_window_append_xf(1, arr(kc), arr(kc + 0x1000_0000), arr(kn),
                                          arr(kn + 0x1000_0000), st, None, None, D_, D_ + 0x1000,
                                          past, 2, 2, 8, S, D, 3,
                                          None if x is None else ctypes.byref(x), None, None)
    tab = C_
    ok = _xf(cos=tab, sin=tab + 0x1000, max_pos=64, rot=16)
    assert win(None) == INV                                              # no transform
    assert win(_xf(in_type=4)) == INV                                    # int8 new rows
    assert win(_xf(out_type=9)) == INV
    assert win(_xf(scale=(0.0, 1.0))) == INV and win(_xf(scale=(1.0, float("inf")))) == INV
    assert win(_xf(scale=(float("nan"), 1.0))) == INV
    assert win(_xf(zp=(128, 0))) == INV and win(_xf(out_type=5, zp=(0, -1))) == INV
    assert win(_xf(cos=tab, sin=None, max_pos=64, rot=16)) == INV      # one table only
    assert win(_xf(cos=tab, sin=tab + 0x1000, max_pos=0, rot=16)) == INV
    assert win(_xf(cos=tab, sin=tab + 0x1000, max_pos=64, rot=15)) == INV
    assert win(_xf(cos=tab, sin=tab + 0x1000, max_pos=64, rot=18)) == INV  # > head_dim
    assert win(_xf(cos=tab + 2, sin=tab + 0x1000, max_pos=64, rot=16)) == INV  # misaligned
    assert win(_xf(cos=A + 64, sin=tab + 0x1000, max_pos=64, rot=16)) == INV   # table in a cache
    assert win(ok, past=0) == INV and win(ok, past=D_ + 0x2004) == INV   # past_lens
    assert win(ok, kn=B_ + 2) == INV                                     # f32 rows misaligned
    assert win(ok) in launched and win(ok, kn=B_ + 4) in launched       # element alignment
    assert win(_xf(in_type=3, out_type=3)) in launched
    # the fp8 target and per-channel tables [kv_heads, head_dim]
    assert win(_xf(out_type=10, scale=(0.5, 0.25))) in launched
    assert win(_xf(out_type=10, zp=(1, 0))) == INV                     # fp8 has no zero point

    def chan(out_type=4, cs=(None, None), cz=(None, None), **kw):
        x = _xf(out_type=out_type, **kw)
        x.channel_scale[0], x.channel_scale[1] = cs
        x.channel_zero_point[0], x.channel_zero_point[1] = cz
        return x
    tabs = (D_ + 0x4000, D_ + 0x5000)
    assert win(chan(cs=tabs, cz=tabs)) in launched                       # int8, both tables
    assert win(chan(out_type=10, cs=tabs)) in launched                  # fp8 scales
    assert win(chan(out_type=10, cz=tabs)) == INV                       # fp8: no zero points
    assert win(chan(out_type=3, cs=tabs)) == INV                        # bf16: no scales
    assert win(chan(cs=(D_ + 0x4002, None))) == INV                     # misaligned table
    assert win(chan(cs=(A + 64, None))) == INV                          # table inside a cache

    def ts(x, rank=4, tensors=(0, 1), n=2, mode=0):
        shape = _shape(*{4: (2, 3, 16, 8), 3: (2, 16, 8), 2: (2, 16)}[rank])
        t = (ctypes.c_int * 2)(*tensors)
        return L.swrt_tensor_scatter_xf(n, arr(A, A + 0x1000_0000), arr(A, A + 0x1000_0000),
                                        arr(B_, B_ + 0x1000_0000), t, None, shape, rank, 2, mode,
                                        None if x is None else ctypes.byref(x), None, None)
    assert ts(None) == INV and ts(ok, rank=2) == INV and ts(ok, tensors=(0, 2)) == INV
    assert ts(_xf(cos=tab, sin=tab + 0x1000, max_pos=64, rot=10)) == INV  # > head_dim 8
    assert ts(_xf()) in launched and ts(_xf(), mode=1) in launched
    assert ts(chan(cs=tabs)) in launched and ts(chan(cs=tabs), rank=3) in launched

    def ts5(x):
        shape = _shape(2, 2, 3, 16, 8)
        t = (ctypes.c_int * 2)(0, 1)
        return L.swrt_tensor_scatter_xf(2, arr(A, A + 0x1000_0000), arr(A, A + 0x1000_0000),
                                        arr(B_, B_ + 0x1000_0000), t, None, shape, 5, 2, 0,
                                        ctypes.byref(x), None, None)
    assert ts5(_xf()) in launched and ts5(chan(cs=tabs)) == INV         # rank 5: no tables

    def dec(x, nfl=1):
        return L.swrt_kv_decode_step_xf(1, arr(A), arr(A + 0x1000_0000), arr(B_),
                                        arr(B_ + 0x1000), (I64 * 3)(32, 16, 16), D_, 8, 8, None,
                                        None, None, None, None, nfl, arr(C_ + 0x10_0000),
                                        arr(C_ + 0x20_0000), arr(B_ + 0x2000), arr(B_ + 0x3000),
                                        D_ + 0x1000, 16, 2, 2, 16,
                                        None if x is None else ctypes.byref(x), None, None)
    assert dec(None) == INV and dec(_xf(), nfl=33) == INV and dec(_xf(), nfl=-1) == INV
    assert dec(_xf()) in launched


@no_gpu_visible
def test_window_attention_rejects(L):
    INV, UNS, V = swrt.E_INVALID_ARG, swrt.E_UNSUPPORTED, ctypes.c_void_p
    launched = (swrt.OK, swrt.E_LAUNCH)
    arr = lambda *p: (V * len(p))(*p)  # noqa: E731

    def att(q=A, k=B_, v=C_, out=D_, lens=D_ + 0x10_0000, W=8, B=2, Hq=8, Hkv=2, Cap=16, D=64,
            scale=0.125, et=3, ot=3, n=1):
        return L.swrt_window_attention(n, arr(q), arr(k), arr(v), arr(out), lens, W, B, Hq, Hkv,
                                       Cap, D, scale, et, ot, None, None)
    assert att() in launched
    assert att(W=0) == INV and att(Cap=0) == INV and att(Hkv=0) == INV and att(B=-1) == INV
    assert att(Hq=6, Hkv=4) == INV                           # not a multiple
    assert att(Hq=6, Hkv=2) in launched                      # group of 3: the matrix-core kernel
    assert att(Hq=64, Hkv=2) in launched                     # group of 32: two waves per window
    assert att(Hq=6, Hkv=2, et=1, ot=1) == UNS               # group of 3 on the VALU kernel
    assert att(D=24) == UNS and att(D=40) == UNS             # 48-, 80-byte rows
    assert att(D=96) in launched and att(D=192) in launched  # matrix cores: head_dim 96, 192
    assert att(D=96, q=A + 8) == UNS                         # the VALU kernel: 192-byte rows
    assert att(Hq=32, Hkv=2, D=128) in launched              # 16-bit: the matrix-core kernel
    assert att(Hq=32, Hkv=2, D=128, q=A + 8) == UNS          # 8-byte aligned: the VALU kernel,
    assert att(Hq=32, Hkv=2, D=64, et=1, ot=1) == UNS        # as for fp32: group 16 x 256 B
    assert att(et=4) == INV and att(ot=5) == INV             # no integer attention
    assert att(scale=float("nan")) == INV and att(scale=float("inf")) == INV
    assert att(q=A + 4) == INV and att(k=B_ + 2) == INV      # 8-byte alignment
    assert att(out=B_ + 64) == INV                           # output inside a cache
    assert att(lens=0) == INV and att(n=33) == INV
    assert att(n=0) == swrt.OK and att(B=0) == swrt.OK


@no_gpu_visible
def test_paged_rejects(L):
    """Host-side checks of the paged entry points (nothing is launched)."""
    INV, UNS = swrt.E_INVALID_ARG, swrt.E_UNSUPPORTED
    launched = (swrt.OK, swrt.E_LAUNCH)

    def layer(**kw):
        f = dict(q=A, out=D_, arena=B_, arena_bytes=4096, pages=C_, n_pages=4,
                 page_ptr=C_ + 0x1000, page_ids=C_ + 0x2000, n_ids=4, page_count=None,
                 page_stride=0)
        f.update(kw)
        return swrt.PagedLayer(*[f[n] for n, _ in swrt.PagedLayer._fields_])

    def att(layers=None, lw=-1, B=2, Hq=8, Hkv=2, D=64, scale=0.125, qt=3, ot=3, n=1, fm=0):
        arr = (swrt.PagedLayer * n)(*([layer()] * n if layers is None else layers))
        return L.swrt_paged_attention(n, ctypes.cast(arr, ctypes.c_void_p), lw, B, Hq, Hkv, D,
                                      scale, qt, ot, fm, None, None)
    assert att() in launched
    # the declared page formats: bits 1 .. 9 (either kernel build), nothing else
    assert att(fm=(1 << 3) | (1 << 4)) in launched and att(fm=0x3FE) in launched
    assert att(fm=1) == INV and att(fm=1 << 10) == INV
    assert att(D=48) == UNS and att(D=512) == UNS           # head_dim
    assert att(Hq=64, Hkv=2) in launched                    # a group of 32: two waves per stream
    assert att(Hq=6, Hkv=4) == INV and att(qt=4) == INV and att(ot=9) == INV
    assert att(scale=float("nan")) == INV and att(n=33) == INV
    assert att(layers=[layer(arena_bytes=4100)]) == INV     # not a multiple of 16
    assert att(layers=[layer(arena=B_ + 8)]) == INV         # arena alignment
    assert att(layers=[layer(q=A + 8)]) == INV              # query alignment
    assert att(layers=[layer(out=B_ + 64)]) == INV          # output inside the arena
    assert att(layers=[layer(page_ptr=None)]) == INV
    assert att(n=0) == swrt.OK and att(B=0) == swrt.OK

    def quant(arena=B_, ab=4096, pin=C_, n=4, bl=C_ + 0x2000, nb=1, dst=C_ + 0x3000, fb=2048,
              fe=4096, pout=C_, kf=4, ks=0.1, kz=0, vf=4, vs=0.1, vz=0, D=64, flags=D_ + 0x100000):
        return L.swrt_paged_quantize(arena, ab, pin, n, bl, nb, dst, fb, fe, pout, kf, ks, kz, vf,
                                     vs, vz, D, flags, None)
    assert quant() in launched
    assert quant(kf=10) == INV and quant(ks=0.0) == INV and quant(kz=200) == INV
    assert quant(vf=9, vz=4) == INV                         # uint2 zero point past 3
    assert quant(fb=5000) == INV and quant(fe=8192) == INV and quant(fb=3000, fe=2000) == INV
    assert quant(flags=None) == INV                         # the flag word is required
    assert quant(D=40) == INV and quant(nb=5) == INV
    assert quant(pout=B_ + 16) == INV                       # descriptors inside the arena

    def app(layers=None, n=1, S=8, D=64, nt=3):
        arr = (swrt.PagedLayer * n)(*([layer()] * n if layers is None else layers))
        kn = (ctypes.c_void_p * n)(*[D_ + 0x200000 * (i + 1) for i in range(n)])
        vn = (ctypes.c_void_p * n)(*[D_ + 0x200000 * (i + 1) + 0x100000 for i in range(n)])
        return L.swrt_paged_append_open(n, ctypes.cast(arr, ctypes.c_void_p), kn, vn, nt, S, D,
                                        None, None)
    assert app() in launched
    three = [layer(arena=B_ + 0x10000 * i) for i in range(3)]
    assert app(layers=three, n=3) in launched               # three arenas, one block table
    assert app(n=3) == INV                                  # one arena written by three layers
    assert app(layers=[three[0], layer(arena=B_ + 0x20000, page_ids=C_ + 0x5000)], n=2) == INV
    assert app(D=40) == INV and app(nt=4) == INV and app(n=33) == INV
    assert app(layers=[layer(arena_bytes=4104)]) == INV
    # slotted rows: page_count with a stride (page_ptr unused)
    slot = dict(page_ptr=None, page_count=C_ + 0x1000, page_stride=2, n_ids=16)
    assert att(layers=[layer(**slot)]) in launched
    assert att(layers=[layer(**{**slot, "page_stride": 0})]) == INV
    assert att(layers=[layer(page_ptr=None)]) == INV           # no table at all

    def seal(layers=None, n=1, NS=8, S=1, D=64, nt=3, first=8, fb=1024, fe=4096, kf=3, ks=1.0,
             kz=0, vf=4, vs=0.1, vz=0):
        arr = (swrt.PagedLayer * n)(*([layer(**sl)] * n if layers is None else layers))
        kn = (ctypes.c_void_p * n)(*[D_ + 0x200000 * (i + 1) for i in range(n)])
        vn = (ctypes.c_void_p * n)(*[D_ + 0x200000 * (i + 1) + 0x100000 for i in range(n)])
        return L.swrt_paged_append(n, ctypes.cast(arr, ctypes.c_void_p), kn, vn, nt, NS, S, D,
                                   first, fb, fe, kf, ks, kz, vf, vs, vz, None, None)
    sl = dict(page_ptr=None, page_count=C_ + 0x1000, page_stride=2, n_ids=16, n_pages=16)
    assert seal() in launched
    assert seal(first=9) == INV and seal(first=-1) == INV    # new ids past the descriptors
    assert seal(fe=1024 + 8 * 192 - 16) == INV                # room for seven streams only
    assert seal(fb=5000, fe=5000) == INV                      # free region past the arena
    assert seal(NS=9, first=0) == INV                         # slots past page_ids
    assert seal(S=0) == INV and seal(nt=4) == INV and seal(kf=10) == INV and seal(vs=0.0) == INV
    assert seal(vz=128) == INV                                # int8 zero point
    assert seal(layers=[layer(**{**sl, "page_count": None, "page_ptr": C_ + 0x1000})]) == INV
    assert seal(D=40) == UNS and seal(D=8) == UNS             # head_dim: 16-byte blocks
    assert seal(fb=1032) == UNS                               # free region not 16-byte aligned
    assert seal(D=32, vf=8) == UNS                            # int2 rows of 8 bytes
    assert seal(D=32, vf=8, S=2) in launched                  # two of them: 16 bytes
    three = [layer(**{**sl, "arena": B_ + 0x10000 * i}) for i in range(3)]
    assert seal(layers=three, n=3) in launched                # three arenas, one block table
    assert seal(n=3) == INV                                   # one arena written by three layers
    part = layer(**{**sl, "arena": B_ + 0x20000, "page_ids": C_ + 0x5000})
    assert seal(layers=[three[0], part], n=2) == INV          # partly shared table
    other = layer(**{**sl, "arena": B_ + 0x30000, "arena_bytes": 8192})
    assert seal(layers=[three[0], other], n=2) == INV         # shared table, arenas of two sizes
    assert seal(NS=0) == swrt.OK and seal(n=0) == swrt.OK
