"""Plain CPU oracle for the sliding-window KV-cache update path.

TEST INFRASTRUCTURE ONLY. The test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only code allowed to import this
package. The product package never imports it, and this package imports
nothing from the product package.

The arithmetic lives in ``swrt_oracle.c`` (plain C, scalar loops, one memcpy per
row); this module only compiles it with gcc and marshals numpy buffers through
ctypes. Page citations are in that file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "swrt_oracle.c")
LIBRARY = os.path.join(HERE, "libswrt_oracle.so")

OK = 0
E_INVALID_ARG = 1
E_UNSUPPORTED = 2
FLAG_LINEAR_OOB = 1
FLAG_BAD_SEQLEN = 2
FLAG_BAD_LENGTHS = 4
MODE_LINEAR = 0
MODE_CIRCULAR = 1
PHASE_STAGE = 1
PHASE_COMMIT = 2
PHASE_ALL = 3
FLAG_ROPE_RANGE = 8
# element types of the row transform
XF_F32, XF_F16, XF_BF16, XF_INT8, XF_UINT8 = 1, 2, 3, 4, 5
XF_FP8_E4M3 = 10
XF_BYTES = {XF_F32: 4, XF_F16: 2, XF_BF16: 2, XF_INT8: 1, XF_UINT8: 1, XF_FP8_E4M3: 1}
# page formats beyond those: sub-byte affine codes; bits per element of every format
XF_INT4, XF_UINT4, XF_INT2, XF_UINT2 = 6, 7, 8, 9
PAGE_BITS = {XF_F32: 32, XF_F16: 16, XF_BF16: 16, XF_INT8: 8, XF_UINT8: 8, XF_INT4: 4,
             XF_UINT4: 4, XF_INT2: 2, XF_UINT2: 2}
FLAG_BAD_PAGES = 16
FLAG_PAGE_FULL = 32
# the C struct orc_page, 64 bytes
PAGE_DTYPE = np.dtype([("start", "<i8"), ("length", "<i4"), ("capacity", "<i4"),
                       ("k_offset", "<i8"), ("v_offset", "<i8"), ("k_format", "<i4"),
                       ("v_format", "<i4"), ("k_scale", "<f4"), ("v_scale", "<f4"),
                       ("k_zero_point", "<i4"), ("v_zero_point", "<i4"), ("reserved", "<i4", (2,))])
assert PAGE_DTYPE.itemsize == 64


def build(source: str = SOURCE, out: str = LIBRARY, extra: tuple = ()) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    # -ffp-contract=off: every float operation of the row transform is rounded
    # on its own, as its definition states
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror",
           "-shared", "-fPIC", *extra, source, "-o", out, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    return out


class OracleError(RuntimeError):
    pass


class RowXf(ctypes.Structure):
    """The C struct orc_row_xf."""
    _fields_ = [("in_type", ctypes.c_int), ("out_type", ctypes.c_int),
                ("cos_table", ctypes.c_void_p), ("sin_table", ctypes.c_void_p),
                ("max_position", ctypes.c_int64), ("rotary_dim", ctypes.c_int64),
                ("interleaved", ctypes.c_int), ("scale", ctypes.c_float * 2),
                ("zero_point", ctypes.c_int32 * 2), ("channel_scale", ctypes.c_void_p * 2),
                ("channel_zero_point", ctypes.c_void_p * 2)]


@dataclass
class Transform:
    """A row transform: RoPE tables (float32 [max_position, rotary_dim/2], or
    None), element types and the K / V affine parameters."""
    in_type: int
    out_type: int
    cos: np.ndarray | None = None
    sin: np.ndarray | None = None
    rotary_dim: int = 0
    interleaved: bool = False
    scale: tuple = (1.0, 1.0)
    zero_point: tuple = (0, 0)
    # per-channel parameters [kv_heads, head_dim] for K and V (None: the scalar)
    channel_scale: tuple = (None, None)
    channel_zero_point: tuple = (None, None)

    def c(self) -> RowXf:
        x = RowXf()
        x.in_type, x.out_type = self.in_type, self.out_type
        if self.cos is not None:
            self.cos = np.ascontiguousarray(self.cos, dtype=np.float32)
            self.sin = np.ascontiguousarray(self.sin, dtype=np.float32)
            x.cos_table, x.sin_table = self.cos.ctypes.data, self.sin.ctypes.data
            x.max_position = self.cos.shape[0]
        x.rotary_dim = self.rotary_dim
        x.interleaved = int(self.interleaved)
        x.scale[0], x.scale[1] = self.scale
        x.zero_point[0], x.zero_point[1] = self.zero_point
        self.channel_scale = tuple(None if a is None else np.ascontiguousarray(a, np.float32)
                                   for a in self.channel_scale)
        self.channel_zero_point = tuple(None if a is None else np.ascontiguousarray(a, np.int32)
                                        for a in self.channel_zero_point)
        for k in range(2):
            a, z = self.channel_scale[k], self.channel_zero_point[k]
            x.channel_scale[k] = None if a is None else a.ctypes.data
            x.channel_zero_point[k] = None if z is None else z.ctypes.data
        return x


def _ptr(a):
    if a is None:
        return None
    return ctypes.c_void_p(a.ctypes.data)


@dataclass
class Lengths:
    total: np.ndarray        # T, int64
    past: np.ndarray         # P, int64
    cache_past: np.ndarray   # Lp, int32
    cache_total: np.ndarray  # L, int32
    evict: np.ndarray        # E, int32
    flags: int
    work: np.ndarray | None = None  # exclusive prefix of each entry's rows, int64 [B + 1]


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(path)
        vp, i64, i32, u32p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.POINTER(ctypes.c_uint32)
        lib.orc_tensor_scatter.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, u32p]
        lib.orc_tensor_scatter.restype = ctypes.c_int
        lib.orc_kv_seq_lengths.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, u32p]
        lib.orc_kv_seq_lengths.restype = ctypes.c_int
        lib.orc_kv_seq_lengths_drift.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                                 u32p]
        lib.orc_kv_seq_lengths_drift.restype = ctypes.c_int
        lib.orc_kv_window_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             i64, i64, i64, i64, i64, i32, ctypes.c_uint, u32p]
        lib.orc_kv_window_append.restype = ctypes.c_int
        xfp = ctypes.POINTER(RowXf)
        lib.orc_xf_row.argtypes = [xfp, i32, i64, i64, vp, vp, i64]
        lib.orc_xf_row.restype = ctypes.c_int
        lib.orc_kv_window_append_xf.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                                i64, i64, i64, ctypes.c_uint, xfp, u32p]
        lib.orc_kv_window_append_xf.restype = ctypes.c_int
        lib.orc_tensor_scatter_xf.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, xfp, u32p]
        lib.orc_tensor_scatter_xf.restype = ctypes.c_int
        lib.orc_window_attention.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                             ctypes.c_double, i32, u32p]
        lib.orc_window_attention.restype = ctypes.c_int
        f32 = ctypes.c_float
        lib.orc_paged_attention.argtypes = [vp, i32, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp,
                                            i64, i64, i64, i64, i64, ctypes.c_double, u32p]
        lib.orc_paged_attention.restype = ctypes.c_int
        lib.orc_paged_quantize.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, vp, i32, f32,
                                           ctypes.c_int32, i32, f32, ctypes.c_int32, i64]
        lib.orc_paged_quantize.restype = ctypes.c_int
        i32v = ctypes.c_int32
        lib.orc_paged_append.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, i32, i64, i64,
                                         i64, i64, i64, i64, i64, i32, f32, i32v, i32, f32, i32v,
                                         u32p, ctypes.POINTER(ctypes.c_int64)]
        lib.orc_paged_append.restype = ctypes.c_int
        lib.orc_paged_append_open.argtypes = [vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, vp, i32,
                                              i64, i64, u32p]
        lib.orc_paged_append_open.restype = ctypes.c_int
        self.lib = lib

    # -- TensorScatter ----------------------------------------------------
    def tensor_scatter_raw(self, present, past, update, write_indices, shape, axis,
                           seq_len, mode, elem_bits):
        """Byte-level call. Buffers are C-contiguous numpy arrays (any dtype);
        ``shape`` is the logical shape of past. Returns (status, flags)."""
        shp = np.ascontiguousarray(np.asarray(shape, dtype=np.int64))
        wi = None if write_indices is None else np.ascontiguousarray(write_indices, dtype=np.int64)
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_tensor_scatter(_ptr(present), _ptr(past), _ptr(update), _ptr(wi),
                                         _ptr(shp), len(shape), axis, seq_len, mode, elem_bits,
                                         ctypes.byref(flags))
        return st, flags.value

    def tensor_scatter(self, past: np.ndarray, update: np.ndarray, write_indices=None,
                       axis: int = -2, mode: str = "linear", in_place: bool = False,
                       elem_bits: int | None = None):
        """present = TensorScatter(past, update, write_indices). Returns (present, flags).
        With in_place=True, ``past`` itself is updated and returned."""
        past = np.ascontiguousarray(past) if not in_place else past
        assert past.flags.c_contiguous
        update = np.ascontiguousarray(update)
        ax = axis + past.ndim if axis < 0 else axis
        seq_len = update.shape[ax] if update.ndim == past.ndim else 0
        present = past if in_place else np.empty_like(past)
        bits = elem_bits or past.dtype.itemsize * 8
        st, flags = self.tensor_scatter_raw(present, past, update, write_indices, past.shape,
                                            axis, seq_len,
                                            MODE_CIRCULAR if mode == "circular" else MODE_LINEAR,
                                            bits)
        if st != OK:
            raise OracleError(f"orc_tensor_scatter status {st}")
        return present, flags

    # -- lengths ----------------------------------------------------------
    def kv_seq_lengths(self, seqlens_k, seq_len: int, capacity: int) -> Lengths:
        sk = np.ascontiguousarray(seqlens_k, dtype=np.int32)
        B = sk.shape[0]
        T = np.zeros(B, np.int64)
        P = np.zeros(B, np.int64)
        Lp = np.zeros(B, np.int32)
        L = np.zeros(B, np.int32)
        E = np.zeros(B, np.int32)
        W = np.zeros(B + 1, np.int64)
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_kv_seq_lengths(_ptr(sk), B, seq_len, capacity, _ptr(T), _ptr(P),
                                         _ptr(Lp), _ptr(L), _ptr(E), _ptr(W), ctypes.byref(flags))
        if st != OK:
            raise OracleError(f"orc_kv_seq_lengths status {st}")
        return Lengths(T, P, Lp, L, E, flags.value, W)

    def kv_seq_lengths_drift(self, seqlens_k, seq_len: int, capacity: int,
                             window: int) -> Lengths:
        sk = np.ascontiguousarray(seqlens_k, dtype=np.int32)
        B = sk.shape[0]
        T = np.zeros(B, np.int64)
        P = np.zeros(B, np.int64)
        Lp = np.zeros(B, np.int32)
        L = np.zeros(B, np.int32)
        E = np.zeros(B, np.int32)
        W = np.zeros(B + 1, np.int64)
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_kv_seq_lengths_drift(_ptr(sk), B, seq_len, capacity, window, _ptr(T),
                                               _ptr(P), _ptr(Lp), _ptr(L), _ptr(E), _ptr(W),
                                               ctypes.byref(flags))
        if st != OK:
            raise OracleError(f"orc_kv_seq_lengths_drift status {st}")
        return Lengths(T, P, Lp, L, E, flags.value, W)

    def kv_seq_lengths_status(self, seqlens_k, seq_len, capacity) -> int:
        sk = np.ascontiguousarray(seqlens_k, dtype=np.int32)
        B = sk.shape[0]
        out = [np.zeros(B, t) for t in (np.int64, np.int64, np.int32, np.int32, np.int32)]
        out.append(np.zeros(B + 1, np.int64))
        flags = ctypes.c_uint32(0)
        return self.lib.orc_kv_seq_lengths(_ptr(sk), B, seq_len, capacity,
                                           *[_ptr(o) for o in out], ctypes.byref(flags))

    # -- windowed step ----------------------------------------------------
    def kv_window_append(self, k_cache, v_cache, k_new, v_new, cache_past_lens, evict_counts,
                         k_staging=None, v_staging=None, phase: int = PHASE_ALL,
                         elem_bits: int | None = None):
        """In-place windowed step on numpy buffers: caches [B,H,C,D], new rows
        [B,H,S,D], staging [B,H,C+S,D] (S > 1). Returns the flags."""
        B, H, C, D = k_cache.shape
        S = k_new.shape[2]
        return self.kv_window_append_strided(k_cache, v_cache, np.ascontiguousarray(k_new),
                                             np.ascontiguousarray(v_new), (H * S * D, S * D, D),
                                             S, cache_past_lens, evict_counts, k_staging,
                                             v_staging, phase, elem_bits)

    def kv_window_append_strided(self, k_cache, v_cache, k_new, v_new, new_strides, seq_len,
                                 cache_past_lens, evict_counts, k_staging=None,
                                 v_staging=None, phase: int = PHASE_ALL,
                                 elem_bits: int | None = None, head_dim: int | None = None):
        B, H, C = k_cache.shape[:3]
        D = head_dim if head_dim is not None else k_cache.shape[3]
        bits = elem_bits or k_cache.dtype.itemsize * 8
        ns = np.ascontiguousarray(np.asarray(new_strides, dtype=np.int64))
        lp = np.ascontiguousarray(cache_past_lens, dtype=np.int32)
        ev = np.ascontiguousarray(evict_counts, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_kv_window_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new),
                                           _ptr(v_new), _ptr(ns), _ptr(k_staging),
                                           _ptr(v_staging), _ptr(lp), _ptr(ev), B, H, C,
                                           seq_len, D, bits, phase, ctypes.byref(flags))
        if st != OK:
            raise OracleError(f"orc_kv_window_append status {st}")
        return flags.value


    # -- fused append: RoPE + conversion / quantization -------------------
    def xf_row(self, x: Transform, t: int, pos: int, row: np.ndarray, out: np.ndarray,
               head: int = 0) -> int:
        """One row of KV head ``head`` through the transform (row: head_dim
        elements of in_type, out: head_dim elements of out_type, both
        contiguous). Returns the status."""
        D = out.size
        if x.in_type in (XF_F32, XF_F16, XF_BF16) and x.out_type in XF_BYTES:
            assert row.nbytes == D * XF_BYTES[x.in_type] and out.nbytes == D * XF_BYTES[x.out_type]
        return self.lib.orc_xf_row(ctypes.byref(x.c()), t, head, pos, _ptr(row), _ptr(out), D)

    def kv_window_append_xf(self, x: Transform, k_cache, v_cache, k_new, v_new, new_strides,
                            seq_len, cache_past_lens, evict_counts, past_lens, k_staging=None,
                            v_staging=None, phase: int = PHASE_ALL) -> int:
        """Windowed step whose new rows pass through ``x`` first. Caches
        [B, H, C, row] hold D out_type elements per row (any numpy dtype; D
        follows from the row bytes), new rows of in_type are addressed by
        ``new_strides`` (elements). Returns the flags."""
        B, H, C = k_cache.shape[:3]
        D = k_cache.shape[3] * k_cache.itemsize // XF_BYTES[x.out_type]  # elements per row
        ns = np.ascontiguousarray(np.asarray(new_strides, dtype=np.int64))
        lp = np.ascontiguousarray(cache_past_lens, dtype=np.int32)
        ev = np.ascontiguousarray(evict_counts, dtype=np.int32)
        pl = np.ascontiguousarray(past_lens, dtype=np.int64)
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_kv_window_append_xf(_ptr(k_cache), _ptr(v_cache), _ptr(k_new),
                                              _ptr(v_new), _ptr(ns), _ptr(k_staging),
                                              _ptr(v_staging), _ptr(lp), _ptr(ev), _ptr(pl), B,
                                              H, C, seq_len, D, phase, ctypes.byref(x.c()),
                                              ctypes.byref(flags))
        if st != OK:
            raise OracleError(f"orc_kv_window_append_xf status {st}")
        return flags.value

    def tensor_scatter_xf(self, x: Transform, t: int, present, past, update, write_indices,
                          mode: str = "linear"):
        """TensorScatter along axis -2 whose update rows pass through ``x``
        (t = 0: K, rotated; 1: V). present / past [..., M, row] hold D out_type
        elements per row, update [..., S, row'] D in_type elements (any numpy
        dtypes). Returns (status, flags)."""
        shp = np.asarray(past.shape, dtype=np.int64)
        shp[-1] = past.shape[-1] * past.itemsize // XF_BYTES[x.out_type]  # elements per row
        assert update.shape[-1] * update.itemsize == shp[-1] * XF_BYTES[x.in_type]
        wi = None if write_indices is None else np.ascontiguousarray(write_indices, dtype=np.int64)
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_tensor_scatter_xf(_ptr(present), _ptr(past), _ptr(update), _ptr(wi),
                                            _ptr(shp), past.ndim, update.shape[-2],
                                            MODE_CIRCULAR if mode == "circular" else MODE_LINEAR,
                                            t, ctypes.byref(x.c()), ctypes.byref(flags))
        return st, flags.value


    # -- windowed decode attention -----------------------------------------
    def window_attention(self, q, k_cache, v_cache, cache_total_lens, window: int,
                         scale: float, elem_type: int, out: np.ndarray | None = None):
        """float64 attention of q [B, Hq, D] over caches [B, Hkv, C, D] (any numpy
        arrays holding elem_type elements; D follows from the row bytes).
        Returns (out [B, Hq, D] float64, flags)."""
        es = XF_BYTES[elem_type]
        B, Hkv, C = k_cache.shape[:3]
        D = k_cache.shape[3] * k_cache.itemsize // es
        Hq = q.shape[1]
        if out is None:
            out = np.zeros((B, Hq, D), np.float64)
        L = np.ascontiguousarray(cache_total_lens, dtype=np.int32)
        qc, kc, vc = (np.ascontiguousarray(a) for a in (q, k_cache, v_cache))  # alive for the call
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_window_attention(_ptr(qc), _ptr(kc), _ptr(vc), _ptr(out), _ptr(L), window,
                                           B, Hq, Hkv, C, D, scale, elem_type, ctypes.byref(flags))
        if st != OK:
            raise OracleError(f"orc_window_attention status {st}")
        return out, flags.value


    # -- paged caches -----------------------------------------------------------
    def paged_attention(self, q, q_type: int, arena, pages, page_ptr, page_ids, left_window: int,
                        kv_heads: int, scale: float, out: np.ndarray | None = None,
                        page_count=None, page_stride: int = 0):
        """float64 attention of q [B, Hq, D] (q_type elements) over the paged
        caches; returns (out [B, Hq, D] float64, flags). The block table is
        compressed rows (page_ptr) or, with page_count, slotted rows of
        page_stride slots per stream."""
        B, Hq = q.shape[:2]
        D = q.shape[2] * q.itemsize // XF_BYTES[q_type]
        if out is None:
            out = np.zeros((B, Hq, D), np.float64)
        qc = np.ascontiguousarray(q)
        ar = np.ascontiguousarray(arena, dtype=np.uint8)
        pg = np.ascontiguousarray(pages, dtype=PAGE_DTYPE)
        ptr = None if page_ptr is None else np.ascontiguousarray(page_ptr, dtype=np.int32)
        cnt = None if page_count is None else np.ascontiguousarray(page_count, dtype=np.int32)
        ids = np.ascontiguousarray(page_ids, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_paged_attention(_ptr(qc), q_type, _ptr(ar), ar.nbytes, _ptr(pg), len(pg),
                                          _ptr(ptr), _ptr(cnt), page_stride, _ptr(ids), len(ids),
                                          _ptr(out), left_window, B, Hq, kv_heads, D, scale,
                                          ctypes.byref(flags))
        if st != OK:
            raise OracleError(f"orc_paged_attention status {st}")
        return out, flags.value

    def paged_quantize(self, arena, pages, blocks, dst_offsets, free_begin: int, free_end: int,
                       k_format: int, k_scale: float, k_zero_point: int, v_format: int,
                       v_scale: float, v_zero_point: int, head_dim: int):
        """QuantizePagedCache on copies: returns (status, arena, pages_out)."""
        ar = np.array(arena, dtype=np.uint8, copy=True)
        pg = np.ascontiguousarray(pages, dtype=PAGE_DTYPE)
        pout = pg.copy()
        bl = np.ascontiguousarray(blocks, dtype=np.int32)
        dst = np.ascontiguousarray(dst_offsets, dtype=np.int64)
        st = self.lib.orc_paged_quantize(_ptr(ar), ar.nbytes, _ptr(pg), len(pg), _ptr(bl), len(bl),
                                         _ptr(dst), free_begin, free_end, _ptr(pout), k_format,
                                         k_scale, k_zero_point, v_format, v_scale, v_zero_point,
                                         head_dim)
        return st, ar, pout

    def paged_append(self, arena, pages, page_count, page_stride: int, page_ids, k_new, v_new,
                     new_type: int, seq_len: int, k_head_dim: int, v_head_dim: int, first_id: int,
                     free_begin: int, free_end: int, k_format: int, k_scale: float,
                     k_zero_point: int, v_format: int, v_scale: float, v_zero_point: int):
        """Sealed-block append on copies (one new block of seq_len tokens per
        stream): returns (status, arena, pages, page_count, page_ids, flags,
        payload bytes written)."""
        ar = np.array(arena, dtype=np.uint8, copy=True)
        pg = np.array(pages, dtype=PAGE_DTYPE, copy=True)
        cnt = np.array(page_count, dtype=np.int32, copy=True)
        ids = np.array(page_ids, dtype=np.int32, copy=True)
        kn, vn = np.ascontiguousarray(k_new), np.ascontiguousarray(v_new)
        flags = ctypes.c_uint32(0)
        written = ctypes.c_int64(0)
        st = self.lib.orc_paged_append(_ptr(ar), ar.nbytes, _ptr(pg), len(pg), _ptr(cnt),
                                       page_stride, _ptr(ids), len(ids), _ptr(kn), _ptr(vn),
                                       new_type, len(cnt), seq_len, k_head_dim, v_head_dim,
                                       first_id, free_begin, free_end, k_format, k_scale,
                                       k_zero_point, v_format, v_scale, v_zero_point,
                                       ctypes.byref(flags), ctypes.byref(written))
        return st, ar, pg, cnt, ids, flags.value, written.value

    def paged_append_open(self, arena, pages, page_ptr, page_ids, k_new, v_new, new_type: int,
                          head_dim: int, page_count=None, page_stride: int = 0):
        """Open-page append on copies (each stream's token into its last page):
        returns (arena, pages, flags)."""
        ar = np.array(arena, dtype=np.uint8, copy=True)
        pg = np.array(pages, dtype=PAGE_DTYPE, copy=True)
        ptr = None if page_ptr is None else np.ascontiguousarray(page_ptr, dtype=np.int32)
        cnt = None if page_count is None else np.ascontiguousarray(page_count, dtype=np.int32)
        ids = np.ascontiguousarray(page_ids, dtype=np.int32)
        kn, vn = np.ascontiguousarray(k_new), np.ascontiguousarray(v_new)
        n_streams = len(cnt) if cnt is not None else len(ptr) - 1
        flags = ctypes.c_uint32(0)
        st = self.lib.orc_paged_append_open(_ptr(ar), ar.nbytes, _ptr(pg), len(pg), _ptr(ptr),
                                            _ptr(cnt), page_stride, _ptr(ids), len(ids), _ptr(kn),
                                            _ptr(vn), new_type, n_streams, head_dim,
                                            ctypes.byref(flags))
        if st != OK:
            raise OracleError(f"orc_paged_append_open status {st}")
        return ar, pg, flags.value


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``swrt_oracle.c`` in this directory (built on first use)."""
    global _default
    if _default is None:
        if (not os.path.exists(LIBRARY)
                or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        _default = Oracle(LIBRARY)
    return _default
