"""MI355X (gfx950) KV-cache updates for sliding-window / ring caches.

A thin ctypes binding over ``libswrt.so`` (C-ABI in ``include/swrt.h``). The
functions here only marshal torch tensors (device pointers, shapes, strides,
the current stream) into the C entry points of the same names; every step of
the update runs in the library's HIP kernels. If the library has not been
built, every call raises ``SwrtError``: there is no fallback.

Operations (pages: ONNX operator "TensorScatter"; Core AI model zoo
"Stateful decode & KV cache"; onnxruntime pull request "GQA support
sliding_window_cache"):

    tensor_scatter(past, update, write_indices, axis=-2, mode="linear", out=None)
    tensor_scatter_batched(pasts, updates, write_indices, ...)  # one shape, one launch
    kv_seq_lengths(seqlens_k, seq_len, capacity)
    kv_window_append(k_cache, v_cache, k_new, v_new, cache_past_lens, evict_counts,
                     k_staging=None, v_staging=None, phase="all")
    kv_window_append_layers(...)   # several layers sharing shapes and lengths
    kv_decode_step(...)            # lengths + windowed layers + full layers, one launch

Fused appends (``Transform``: RoPE on K at the absolute position, then
conversion or affine INT8 / UINT8 quantization into the cache's dtype):

    kv_window_append_xf(...), tensor_scatter_xf(...), kv_decode_step_xf(...)

Decode attention over the windowed caches (every query head over the last W
resident rows of its KV head):

    window_attention(qs, k_caches, v_caches, cache_total_lens, window, ...)

Paged caches (onnx-light how-to "Persistent input/output feedback", section
"Optional heterogeneous paged KV"; ``PagedCache``: one layer's arena, page
descriptors and block table on the device):

    paged_attention(qs, caches, left_window, kv_heads, ...)
    paged_quantize(cache, blocks, dst_offsets, free_begin, free_end, ...)
    paged_append(caches, k_news, v_news, ...)

Every function has a ``prepare_*`` twin returning a ``PreparedCall``: the
arguments are checked and marshalled once, and each call of the object only
adds the current stream. Decode loops use it to keep host cost per step small.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import NamedTuple, Sequence

import numpy as np
import torch

__all__ = [
    "SwrtError", "PreparedCall", "WindowLengths", "library_path", "lib",
    "tensor_scatter", "tensor_scatter_batched", "kv_seq_lengths", "kv_window_append",
    "kv_window_append_layers", "kv_window_stage_step", "kv_decode_step",
    "prepare_tensor_scatter", "prepare_tensor_scatter_batched", "prepare_kv_seq_lengths",
    "prepare_kv_window_append_layers", "prepare_kv_window_stage_step", "prepare_kv_decode_step",
    "Transform", "kv_window_append_xf", "tensor_scatter_xf", "kv_decode_step_xf",
    "prepare_kv_window_append_xf", "prepare_tensor_scatter_xf", "prepare_kv_decode_step_xf",
    "kv_window_stage_step_xf", "prepare_kv_window_stage_step_xf",
    "window_attention", "prepare_window_attention",
    "PagedCache", "PAGE_DTYPE", "PAGE_FORMATS", "page_table", "paged_attention",
    "prepare_paged_attention", "paged_quantize", "paged_append", "prepare_paged_append",
    "FLAG_BAD_PAGES", "FLAG_PAGE_FULL",
    "OK", "E_INVALID_ARG", "E_UNSUPPORTED", "E_LAUNCH",
    "FLAG_LINEAR_OOB", "FLAG_BAD_SEQLEN", "FLAG_BAD_LENGTHS", "FLAG_ROPE_RANGE",
    "PHASE_STAGE", "PHASE_COMMIT", "PHASE_ALL",
]

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libswrt.so")

# values of include/swrt.h
OK, E_INVALID_ARG, E_UNSUPPORTED, E_LAUNCH = 0, 1, 2, 3
FLAG_LINEAR_OOB, FLAG_BAD_SEQLEN, FLAG_BAD_LENGTHS, FLAG_ROPE_RANGE = 1, 2, 4, 8
FLAG_BAD_PAGES, FLAG_PAGE_FULL = 16, 32
MODE_LINEAR, MODE_CIRCULAR = 0, 1
PHASE_STAGE, PHASE_COMMIT, PHASE_ALL = 1, 2, 3
MAX_LAYERS = 32
MAX_BATCHED = 64
ABI_VERSION = 10

_PHASES = {"stage": PHASE_STAGE, "commit": PHASE_COMMIT, "all": PHASE_ALL}
_MODES = {"linear": MODE_LINEAR, "circular": MODE_CIRCULAR}


class SwrtError(RuntimeError):
    """A libswrt call failed (or the library is missing)."""

    def __init__(self, msg: str, status: int | None = None):
        super().__init__(msg)
        self.status = status


_lib: ctypes.CDLL | None = None

# element types of a row transform (include/swrt.h SWRT_XF_*)
XF_TYPES = {torch.float32: 1, torch.float16: 2, torch.bfloat16: 3, torch.int8: 4,
            torch.uint8: 5, torch.float8_e4m3fn: 10}


class RowTransform(ctypes.Structure):
    """The C struct swrt_row_transform."""
    _fields_ = [("in_type", ctypes.c_int), ("out_type", ctypes.c_int),
                ("cos_table", ctypes.c_void_p), ("sin_table", ctypes.c_void_p),
                ("max_position", ctypes.c_int64), ("rotary_dim", ctypes.c_int64),
                ("interleaved", ctypes.c_int), ("scale", ctypes.c_float * 2),
                ("zero_point", ctypes.c_int32 * 2), ("channel_scale", ctypes.c_void_p * 2),
                ("channel_zero_point", ctypes.c_void_p * 2)]


@dataclass
class Transform:
    """Row transform of a fused append: K rows turn by RoPE at their absolute
    position (when ``cos``/``sin`` are given: float32 [max_position,
    rotary_dim / 2] device tables), then every element is written in the
    cache's dtype: float32 / float16 / bfloat16 rounded to nearest even, an
    int8 / uint8 affine code round(y / scale) + zero_point (ties to even,
    saturated), or a float8_e4m3fn code of y / scale (nearest even,
    saturating at +-448), with the K or V scale and zero point -- the scalars,
    or per channel the [kv_heads, head_dim] device tables
    ``k_channel_scale`` / ``v_channel_scale`` (float32) and
    ``k_channel_zero_point`` / ``v_channel_zero_point`` (int32)."""
    cos: torch.Tensor | None = None
    sin: torch.Tensor | None = None
    interleaved: bool = False
    k_scale: float = 1.0
    v_scale: float = 1.0
    k_zero_point: int = 0
    v_zero_point: int = 0
    k_channel_scale: torch.Tensor | None = None
    v_channel_scale: torch.Tensor | None = None
    k_channel_zero_point: torch.Tensor | None = None
    v_channel_zero_point: torch.Tensor | None = None

    def channel_tables(self) -> tuple:
        return (self.k_channel_scale, self.v_channel_scale, self.k_channel_zero_point,
                self.v_channel_zero_point)

    def c(self, in_dtype: torch.dtype, out_dtype: torch.dtype, heads: int | None = None,
          head_dim: int | None = None) -> RowTransform:
        if in_dtype not in (torch.float32, torch.float16, torch.bfloat16):
            raise SwrtError("new rows must be float32, float16 or bfloat16")
        if out_dtype not in XF_TYPES:
            raise SwrtError("caches of a fused append must be float32, float16, bfloat16, int8, "
                            "uint8 or float8_e4m3fn")
        x = RowTransform()
        x.in_type, x.out_type = XF_TYPES[in_dtype], XF_TYPES[out_dtype]
        if (self.cos is None) != (self.sin is None):
            raise SwrtError("give both rotary tables or neither")
        if self.cos is not None:
            for t in (self.cos, self.sin):
                _contig("rotary table", t)
                if t.dtype != torch.float32 or t.dim() != 2 or t.shape != self.cos.shape:
                    raise SwrtError("rotary tables must be float32 [max_position, rotary_dim/2]")
            x.cos_table, x.sin_table = self.cos.data_ptr(), self.sin.data_ptr()
            x.max_position = self.cos.shape[0]
            x.rotary_dim = 2 * self.cos.shape[1]
        x.interleaved = int(self.interleaved)
        x.scale[0], x.scale[1] = self.k_scale, self.v_scale
        x.zero_point[0], x.zero_point[1] = self.k_zero_point, self.v_zero_point
        for k, (sc, zp) in enumerate(((self.k_channel_scale, self.k_channel_zero_point),
                                      (self.v_channel_scale, self.v_channel_zero_point))):
            for name, t, dt in (("channel scale", sc, torch.float32),
                                ("channel zero point", zp, torch.int32)):
                if t is None:
                    continue
                _contig(name, t)
                if t.dtype != dt or (heads is not None and tuple(t.shape) != (heads, head_dim)):
                    raise SwrtError(f"{name} tables must be {dt} [kv_heads, head_dim]"
                                    + (f" = [{heads}, {head_dim}]" if heads is not None else ""))
            x.channel_scale[k] = None if sc is None else sc.data_ptr()
            x.channel_zero_point[k] = None if zp is None else zp.data_ptr()
        return x

    def tables(self) -> tuple:
        """Every device tensor the transform reads."""
        return (self.cos, self.sin, *self.channel_tables())


def library_path() -> str:
    return LIBRARY


def lib() -> ctypes.CDLL:
    """The loaded libswrt.so; raises SwrtError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise SwrtError(f"{LIBRARY} is missing: build it with "
                        "`python -m sliding_window_ring_tensor_amd.build`")
    L = ctypes.CDLL(LIBRARY)
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint
    vpp = ctypes.POINTER(ctypes.c_void_p)
    L.swrt_tensor_scatter.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, vp]
    L.swrt_tensor_scatter_batched.argtypes = [i32, vpp, vpp, vpp, vp, vp, i32, i32, i64, i32,
                                              i32, vp, vp]
    L.swrt_kv_seq_lengths.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.swrt_kv_seq_lengths_drift.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                            vp]
    L.swrt_kv_window_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                        i32, i32, u32, vp, vp]
    L.swrt_kv_window_append_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                i32, i32, vp, vp]
    L.swrt_kv_window_append_layers.argtypes = [i32, vpp, vpp, vpp, vpp, vp, vpp, vpp, vp, vp,
                                               i32, i32, i32, i32, i32, i32, u32, vp, vp]
    L.swrt_kv_window_stage_step.argtypes = [i32, vpp, vpp, vpp, vpp, vp, vpp, vpp, vp, i32, i32,
                                             vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    L.swrt_kv_decode_step.argtypes = [i32, vpp, vpp, vpp, vpp, vp, vp, i32, i32, vp, vp, vp, vp,
                                      vp, i32, vpp, vpp, vp, i32, i32, i32, i32, i32, vp, vp]
    xfp = ctypes.POINTER(RowTransform)
    L.swrt_kv_window_append_xf.argtypes = [i32, vpp, vpp, vpp, vpp, vp, vpp, vpp, vp, vp, vp,
                                           i32, i32, i32, i32, i32, u32, xfp, vp, vp]
    L.swrt_kv_window_stage_step_xf.argtypes = [i32, vpp, vpp, vpp, vpp, vp, vpp, vpp, vp, i32,
                                                i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, xfp,
                                                vp, vp]
    L.swrt_tensor_scatter_xf.argtypes = [i32, vpp, vpp, vpp, vp, vp, vp, i32, i64, i32, xfp, vp,
                                         vp]
    L.swrt_kv_decode_step_xf.argtypes = [i32, vpp, vpp, vpp, vpp, vp, vp, i32, i32, vp, vp, vp,
                                         vp, vp, i32, vpp, vpp, vpp, vpp, vp, i32, i32, i32, i32,
                                         xfp, vp, vp]
    L.swrt_window_attention.argtypes = [i32, vpp, vpp, vpp, vpp, vp, i32, i32, i32, i32, i32,
                                        i32, ctypes.c_float, i32, i32, vp, vp]
    f32 = ctypes.c_float
    L.swrt_paged_attention.argtypes = [i32, vp, i64, i32, i32, i32, i32, f32, i32, i32, u32, vp,
                                       vp]
    L.swrt_paged_quantize.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, vp, i32, f32,
                                      ctypes.c_int32, i32, f32, ctypes.c_int32, i32, vp, vp]
    i32v = ctypes.c_int32
    L.swrt_paged_append.argtypes = [i32, vp, vpp, vpp, i32, i32, i32, i32, i64, i64, i64, i32,
                                    f32, i32v, i32, f32, i32v, vp, vp]
    L.swrt_paged_append_open.argtypes = [i32, vp, vpp, vpp, i32, i32, i32, vp, vp]
    for name in ("swrt_tensor_scatter", "swrt_tensor_scatter_batched", "swrt_kv_seq_lengths",
                 "swrt_kv_seq_lengths_drift",
                 "swrt_kv_window_append", "swrt_kv_window_append_layers",
                 "swrt_kv_window_stage_step", "swrt_kv_decode_step",
                 "swrt_kv_window_append_xf", "swrt_kv_window_stage_step_xf",
                 "swrt_tensor_scatter_xf", "swrt_kv_decode_step_xf",
                 "swrt_window_attention", "swrt_paged_attention", "swrt_paged_quantize",
                 "swrt_paged_append", "swrt_paged_append_open",
                 "swrt_kv_window_append_noalloc", "swrt_abi_version"):
        getattr(L, name).restype = ctypes.c_int
    L.swrt_status_string.argtypes = [ctypes.c_int]
    L.swrt_status_string.restype = ctypes.c_char_p
    if L.swrt_abi_version() != ABI_VERSION:
        raise SwrtError("libswrt ABI version mismatch")
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != OK:
        msg = lib().swrt_status_string(status).decode()
        raise SwrtError(f"{what}: {msg} (status {status})", status)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _flags_ptr(flags: torch.Tensor | None):
    """The flag word's address: an int32 tensor of at least one element (the
    library ORs 32-bit flag bits into its first element)."""
    if flags is None:
        return None
    if flags.dtype != torch.int32 or flags.numel() < 1:
        raise SwrtError("flags must be an int32 tensor with at least one element")
    return ctypes.c_void_p(flags.data_ptr())


def _ptrs(ts: Sequence[torch.Tensor] | None):
    if ts is None:
        return None
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _device_of(*ts: torch.Tensor | None) -> torch.device:
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise SwrtError(f"tensors must share one device, got {sorted(map(str, devs))}")
    dev = devs.pop()
    if dev.type != "cuda":
        raise SwrtError(f"libswrt runs on the GPU only; got a tensor on {dev}")
    return dev


def _bits(t: torch.Tensor) -> int:
    return t.element_size() * 8


def _check_write_indices(write_indices: torch.Tensor | None, batch: int) -> None:
    """write_indices: None (all zeros) or a dense int64 [batch] tensor."""
    if write_indices is None:
        return
    _contig("write_indices", write_indices)
    if write_indices.dtype != torch.int64 or tuple(write_indices.shape) != (batch,):
        raise SwrtError(f"write_indices must be int64 [{batch}] (one index per batch entry), "
                        f"got {write_indices.dtype} {tuple(write_indices.shape)}")


def _contig(name: str, t: torch.Tensor) -> None:
    if not t.is_contiguous():
        raise SwrtError(f"{name} must be contiguous (it is never copied)")


class PreparedCall:
    """One library call with its arguments marshalled; calling it enqueues the
    call on the current stream of the tensors' device. It keeps the tensors it
    points at alive."""

    def __init__(self, fn, args: tuple, device: torch.device, what: str, keep: tuple, result=None):
        self._fn, self._args, self._dev, self._what = fn, args, device, what
        self._keep, self.result = keep, result

    def __call__(self):
        with torch.cuda.device(self._dev):
            st = self._fn(*self._args, ctypes.c_void_p(
                torch.cuda.current_stream(self._dev).cuda_stream))
        _check(st, self._what)
        return self.result


# ---------------------------------------------------------------------------
# TensorScatter
# ---------------------------------------------------------------------------

def prepare_tensor_scatter_batched(pasts: Sequence[torch.Tensor],
                                   updates: Sequence[torch.Tensor],
                                   write_indices: torch.Tensor | None = None, *, axis: int = -2,
                                   mode: str = "linear",
                                   outs: Sequence[torch.Tensor] | None = None,
                                   flags: torch.Tensor | None = None,
                                   _single: bool = False) -> PreparedCall:
    n = len(pasts)
    if len(updates) != n or not 1 <= n <= MAX_BATCHED:
        raise SwrtError(f"need 1..{MAX_BATCHED} (past, update) pairs")
    p0, u0 = pasts[0], updates[0]
    presents = [torch.empty_like(p) for p in pasts] if outs is None else list(outs)
    rank = p0.dim()
    ax = axis + rank if axis < 0 else axis
    if not 0 <= ax < rank or u0.dim() != rank:
        raise SwrtError(f"axis {axis} out of range for rank {rank}")
    # [TS] Inputs: update is past's shape with the sequence axis replaced by S,
    # and write_indices holds one index per batch entry
    if any(u0.shape[d] != p0.shape[d] for d in range(rank) if d != ax):
        raise SwrtError(f"update {tuple(u0.shape)} must match past {tuple(p0.shape)} "
                        f"except on axis {axis}")
    _check_write_indices(write_indices, p0.shape[0])
    _flags_ptr(flags)
    dev = _device_of(*pasts, *updates, *presents, write_indices, flags)
    for p, u, o in zip(pasts, updates, presents):
        for name, t in (("past", p), ("update", u), ("out", o)):
            _contig(name, t)
        if p.shape != p0.shape or o.shape != p0.shape or u.shape != u0.shape or \
                len({p.dtype, u.dtype, o.dtype, p0.dtype}) != 1:
            raise SwrtError("every past/out must share one shape, every update another, "
                            "and all one dtype")
    shape = (ctypes.c_int64 * rank)(*p0.shape)
    L = lib()
    keep = (*pasts, *updates, *presents, write_indices, flags)
    if _single:
        args = (_ptr(presents[0]), _ptr(p0), _ptr(u0), _ptr(write_indices), shape, rank, axis,
                u0.shape[ax], _MODES[mode], _bits(p0), _flags_ptr(flags))
        return PreparedCall(L.swrt_tensor_scatter, args, dev, "tensor_scatter", keep,
                            presents[0])
    args = (n, _ptrs(presents), _ptrs(pasts), _ptrs(updates), _ptr(write_indices), shape, rank,
            axis, u0.shape[ax], _MODES[mode], _bits(p0), _flags_ptr(flags))
    return PreparedCall(L.swrt_tensor_scatter_batched, args, dev, "tensor_scatter_batched", keep,
                        presents)


def prepare_tensor_scatter(past, update, write_indices=None, *, axis=-2, mode="linear", out=None,
                           flags=None) -> PreparedCall:
    if update.dtype != past.dtype or update.dim() != past.dim():
        raise SwrtError("update must have past's dtype and rank")
    return prepare_tensor_scatter_batched([past], [update], write_indices, axis=axis, mode=mode,
                                          outs=None if out is None else [out], flags=flags,
                                          _single=True)


def tensor_scatter(past: torch.Tensor, update: torch.Tensor,
                   write_indices: torch.Tensor | None = None, *, axis: int = -2,
                   mode: str = "linear", out: torch.Tensor | None = None,
                   flags: torch.Tensor | None = None) -> torch.Tensor:
    """present = TensorScatter(past, update, write_indices; axis, mode).

    ``out=past`` updates the cache in place (only the target rows are written);
    otherwise a new (or the given) ``out`` receives past with the update rows.
    ``write_indices``: int64 [batch] on the device, or None for zeros.
    ``flags``: optional int32 device word that receives FLAG_* bits.
    """
    return prepare_tensor_scatter(past, update, write_indices, axis=axis, mode=mode, out=out,
                                  flags=flags)()


def tensor_scatter_batched(pasts: Sequence[torch.Tensor], updates: Sequence[torch.Tensor],
                           write_indices: torch.Tensor | None = None, *, axis: int = -2,
                           mode: str = "linear", outs: Sequence[torch.Tensor] | None = None,
                           flags: torch.Tensor | None = None) -> list:
    """TensorScatter on several caches of one shape sharing write_indices, in one
    launch. ``outs=pasts`` updates every cache in place."""
    return prepare_tensor_scatter_batched(pasts, updates, write_indices, axis=axis, mode=mode,
                                          outs=outs, flags=flags)()


# ---------------------------------------------------------------------------
# windowed step: lengths
# ---------------------------------------------------------------------------

class WindowLengths(NamedTuple):
    total: torch.Tensor        # T  = seqlens_k + 1            int64 [B]
    past: torch.Tensor         # P  = max(0, T - S)            int64 [B]
    cache_past: torch.Tensor   # Lp = min(P, C)                int32 [B]
    cache_total: torch.Tensor  # L  = Lp + S - E = min(T, C)   int32 [B]
    evict: torch.Tensor        # E  = max(0, Lp + S - C)       int32 [B]


def _new_lengths(B: int, dev) -> WindowLengths:
    return WindowLengths(*(torch.empty(B, dtype=dt, device=dev) for dt in
                           (torch.int64, torch.int64, torch.int32, torch.int32, torch.int32)))


def _check_seqlens(seqlens_k: torch.Tensor, batch: int | None = None) -> None:
    _contig("seqlens_k", seqlens_k)
    if seqlens_k.dtype != torch.int32 or seqlens_k.dim() != 1:
        raise SwrtError("seqlens_k must be a 1-D int32 tensor")
    if batch is not None and seqlens_k.shape[0] != batch:
        raise SwrtError(f"seqlens_k must hold one entry per batch entry ({batch})")


def _lengths_out(out: WindowLengths | None, B: int, dev) -> WindowLengths:
    """The length arrays to write: new ones, or the caller's after a check."""
    if out is None:
        return _new_lengths(B, dev)
    for t, dt in zip(out, (torch.int64, torch.int64, torch.int32, torch.int32, torch.int32)):
        _contig("lengths", t)
        if t.dtype != dt or t.shape != (B,):
            raise SwrtError("out must be WindowLengths of [B] tensors (int64 total and past, "
                            "int32 cache_past, cache_total and evict)")
    return out


def prepare_kv_seq_lengths(seqlens_k: torch.Tensor, seq_len: int, capacity: int, *,
                           window: int | None = None, out: WindowLengths | None = None,
                           work_offsets: torch.Tensor | None = None,
                           flags: torch.Tensor | None = None) -> PreparedCall:
    _check_seqlens(seqlens_k)
    B = seqlens_k.shape[0]
    if work_offsets is not None:
        _contig("work_offsets", work_offsets)
        if work_offsets.dtype != torch.int64 or tuple(work_offsets.shape) != (B + 1,):
            raise SwrtError(f"work_offsets must be int64 [{B + 1}]")
    _flags_ptr(flags)
    dev = _device_of(seqlens_k, work_offsets, flags)
    out = _lengths_out(out, B, dev)
    tail = (_ptr(out.total), _ptr(out.past), _ptr(out.cache_past), _ptr(out.cache_total),
            _ptr(out.evict), _ptr(work_offsets), _flags_ptr(flags))
    if window is None:
        fn, args, what = lib().swrt_kv_seq_lengths, (_ptr(seqlens_k), B, seq_len, capacity,
                                                     *tail), "kv_seq_lengths"
    else:
        fn, args, what = lib().swrt_kv_seq_lengths_drift, (_ptr(seqlens_k), B, seq_len, capacity,
                                                           window, *tail), "kv_seq_lengths_drift"
    return PreparedCall(fn, args, dev, what, (seqlens_k, *out, work_offsets, flags), out)


def kv_seq_lengths(seqlens_k: torch.Tensor, seq_len: int, capacity: int, *,
                   window: int | None = None, out: WindowLengths | None = None,
                   work_offsets: torch.Tensor | None = None,
                   flags: torch.Tensor | None = None) -> WindowLengths:
    """Lengths of one windowed step for every batch entry, computed on the device.
    With ``window`` (W <= capacity) the drifting layout's lengths: the append
    point drifts and a whole gap of C - W + 1 rows is reclaimed at once.
    ``work_offsets`` (int64 [B + 1], optional) receives the exclusive prefix
    of the rows each entry's step writes."""
    return prepare_kv_seq_lengths(seqlens_k, seq_len, capacity, window=window, out=out,
                                  work_offsets=work_offsets, flags=flags)()


# ---------------------------------------------------------------------------
# windowed step: shift + append / stage + commit
# ---------------------------------------------------------------------------

def _new_strides(k_new: torch.Tensor, v_new: torch.Tensor):
    if k_new.dim() != 4 or k_new.shape != v_new.shape or k_new.stride() != v_new.stride():
        raise SwrtError("k_new and v_new must be [B, H, S, D] views with equal strides")
    if k_new.shape[3] > 1 and k_new.stride(3) != 1:
        raise SwrtError("head_dim of the new rows must be contiguous")
    return (ctypes.c_int64 * 3)(*k_new.stride()[:3])


def _check_layers(k_caches, v_caches, k_news, v_news, new_dtype: torch.dtype | None = None):
    """new_dtype: the new rows' dtype when it differs from the caches' (fused append)."""
    n = len(k_caches)
    if not (len(v_caches) == len(k_news) == len(v_news) == n) or not 1 <= n <= MAX_LAYERS:
        raise SwrtError(f"need 1..{MAX_LAYERS} layers with one tensor of each kind")
    kc = k_caches[0]
    if kc.dim() != 4:
        raise SwrtError("caches must be [B, H, C, D]")
    B, H, C, D = kc.shape
    S = k_news[0].shape[2]
    for t in (*k_caches, *v_caches):
        _contig("cache", t)
        if t.shape != kc.shape or t.dtype != kc.dtype:
            raise SwrtError("all caches must share shape and dtype")
    nd = kc.dtype if new_dtype is None else new_dtype
    for a, b in zip(k_news, v_news):
        if a.shape != (B, H, S, D) or b.shape != (B, H, S, D) or a.dtype != nd \
                or b.dtype != nd or a.stride() != k_news[0].stride() \
                or b.stride() != k_news[0].stride():
            raise SwrtError("new rows must be [B, H, S, D] in one dtype (the caches' unless "
                            "fused) and one stride pattern")
    return n, B, H, C, D, S, _new_strides(k_news[0], v_news[0])


def prepare_kv_window_append_layers(k_caches, v_caches, k_news, v_news, cache_past_lens,
                                    evict_counts, *, k_stagings=None, v_stagings=None,
                                    phase: str = "all", flags: torch.Tensor | None = None,
                                    _single: bool = False) -> PreparedCall:
    n, B, H, C, D, S, strides = _check_layers(k_caches, v_caches, k_news, v_news)
    kc = k_caches[0]
    everything = [*k_caches, *v_caches, *k_news, *v_news, cache_past_lens, evict_counts, flags]
    if S > 1:
        _check_stagings(k_stagings, v_stagings, n, B, H, C, S, D, kc.dtype)
        everything += [*k_stagings, *v_stagings]
    else:
        k_stagings = v_stagings = None
    dev = _device_of(*everything)
    for t in (cache_past_lens, evict_counts):
        _contig("lengths", t)
        if t.dtype != torch.int32 or t.shape != (B,):
            raise SwrtError("cache_past_lens and evict_counts must be int32 [B]")
    L = lib()
    if _single:
        args = (_ptr(kc), _ptr(v_caches[0]), _ptr(k_news[0]), _ptr(v_news[0]), strides,
                None if k_stagings is None else _ptr(k_stagings[0]),
                None if v_stagings is None else _ptr(v_stagings[0]),
                _ptr(cache_past_lens), _ptr(evict_counts), B, H, C, S, D, _bits(kc),
                _PHASES[phase], _flags_ptr(flags))
        return PreparedCall(L.swrt_kv_window_append, args, dev, "kv_window_append",
                            tuple(everything))
    args = (n, _ptrs(k_caches), _ptrs(v_caches), _ptrs(k_news), _ptrs(v_news), strides,
            _ptrs(k_stagings), _ptrs(v_stagings), _ptr(cache_past_lens), _ptr(evict_counts),
            B, H, C, S, D, _bits(kc), _PHASES[phase], _flags_ptr(flags))
    return PreparedCall(L.swrt_kv_window_append_layers, args, dev, "kv_window_append_layers",
                        tuple(everything))


def kv_window_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                     v_new: torch.Tensor, cache_past_lens: torch.Tensor,
                     evict_counts: torch.Tensor, *, k_staging: torch.Tensor | None = None,
                     v_staging: torch.Tensor | None = None, phase: str = "all",
                     flags: torch.Tensor | None = None) -> None:
    """One windowed step on caches [B, H, C, D] (in place).

    ``k_new``/``v_new`` are [B, H, S, D] views (BNSH, or BSNH transposed) with
    head_dim contiguous. ``cache_past_lens``/``evict_counts`` come from
    ``kv_seq_lengths`` with the same S and C. S > 1 needs staging buffers
    [B, H, C + S, D]; ``phase`` picks "stage", "commit" or "all".
    """
    prepare_kv_window_append_layers(
        [k_cache], [v_cache], [k_new], [v_new], cache_past_lens, evict_counts,
        k_stagings=None if k_staging is None else [k_staging],
        v_stagings=None if v_staging is None else [v_staging], phase=phase, flags=flags,
        _single=True)()


NOALLOC_STAGING_BYTES = 128 << 20  # SWRT_NOALLOC_STAGING_BYTES


def prepare_kv_window_append_noalloc(k_cache, v_cache, k_new, v_new, cache_past_lens,
                                     evict_counts, *,
                                     flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``kv_window_append_noalloc``."""
    n, B, H, C, D, S, strides = _check_layers([k_cache], [v_cache], [k_new], [v_new])
    for t in (cache_past_lens, evict_counts):
        _contig("lengths", t)
        if t.dtype != torch.int32 or t.shape != (B,):
            raise SwrtError("cache_past_lens and evict_counts must be int32 [B]")
    _flags_ptr(flags)
    everything = (k_cache, v_cache, k_new, v_new, cache_past_lens, evict_counts, flags)
    dev = _device_of(*everything)
    args = (_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), strides,
            _ptr(cache_past_lens), _ptr(evict_counts), B, H, C, S, D, _bits(k_cache),
            _flags_ptr(flags))
    return PreparedCall(lib().swrt_kv_window_append_noalloc, args, dev,
                        "kv_window_append_noalloc", everything)


def kv_window_append_noalloc(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                             v_new: torch.Tensor, cache_past_lens: torch.Tensor,
                             evict_counts: torch.Tensor, *,
                             flags: torch.Tensor | None = None) -> None:
    """``kv_window_append`` (phase "all") that allocates nothing: an S > 1
    step stages through the library's own per-GPU device array of
    NOALLOC_STAGING_BYTES (calls that overlap on one GPU race on it)."""
    prepare_kv_window_append_noalloc(k_cache, v_cache, k_new, v_new, cache_past_lens,
                                     evict_counts, flags=flags)()


def kv_window_append_layers(k_caches: Sequence[torch.Tensor], v_caches: Sequence[torch.Tensor],
                            k_news: Sequence[torch.Tensor], v_news: Sequence[torch.Tensor],
                            cache_past_lens: torch.Tensor, evict_counts: torch.Tensor, *,
                            k_stagings: Sequence[torch.Tensor] | None = None,
                            v_stagings: Sequence[torch.Tensor] | None = None,
                            phase: str = "all", flags: torch.Tensor | None = None) -> None:
    """The windowed step for several layers that share B, H, C, D, S and the
    lengths (e.g. every windowed layer of a model), in one launch per phase."""
    prepare_kv_window_append_layers(k_caches, v_caches, k_news, v_news, cache_past_lens,
                                    evict_counts, k_stagings=k_stagings, v_stagings=v_stagings,
                                    phase=phase, flags=flags)()


def _check_stagings(k_stagings, v_stagings, n: int, B: int, H: int, C: int, S: int, D: int,
                    dtype):
    if k_stagings is None or v_stagings is None:
        raise SwrtError("S > 1 needs k_staging and v_staging [B, H, C + S, D]")
    if len(k_stagings) != n or len(v_stagings) != n:
        raise SwrtError("one K and one V staging buffer per layer")
    for t in (*k_stagings, *v_stagings):
        _contig("staging", t)
        if t.shape != (B, H, C + S, D) or t.dtype != dtype:
            raise SwrtError("staging must be [B, H, C + S, D] with the caches' dtype")


def prepare_kv_window_stage_step(k_caches, v_caches, k_news, v_news, seqlens_k, k_stagings,
                                 v_stagings, *, window: int | None = None,
                                 out: WindowLengths | None = None,
                                 flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``kv_window_stage_step``."""
    n, B, H, C, D, S, strides = _check_layers(k_caches, v_caches, k_news, v_news)
    if S < 2:
        raise SwrtError("a staged step appends S >= 2 rows")
    _check_seqlens(seqlens_k, B)
    kc = k_caches[0]
    _check_stagings(k_stagings, v_stagings, n, B, H, C, S, D, kc.dtype)
    dev = _device_of(*k_caches, *v_caches, *k_news, *v_news, seqlens_k, *k_stagings,
                     *v_stagings, flags)
    out = _lengths_out(out, B, dev)
    args = (n, _ptrs(k_caches), _ptrs(v_caches), _ptrs(k_news), _ptrs(v_news), strides,
            _ptrs(k_stagings), _ptrs(v_stagings), _ptr(seqlens_k), C,
            C if window is None else window, _ptr(out.total), _ptr(out.past), _ptr(out.cache_past),
            _ptr(out.cache_total), _ptr(out.evict), B, H, S, D, _bits(kc), _flags_ptr(flags))
    keep = (*k_caches, *v_caches, *k_news, *v_news, seqlens_k, *k_stagings, *v_stagings, *out,
            flags)
    return PreparedCall(lib().swrt_kv_window_stage_step, args, dev, "kv_window_stage_step", keep,
                        out)


def kv_window_stage_step(k_caches, v_caches, k_news, v_news, seqlens_k, k_stagings, v_stagings,
                         *, window: int | None = None, out: WindowLengths | None = None,
                         flags: torch.Tensor | None = None) -> WindowLengths:
    """The lengths of a staged windowed step (S >= 2) and its stage phase for
    every layer, in one launch. Same bytes as kv_seq_lengths followed by
    kv_window_append_layers(phase="stage"); finish the step with
    kv_window_append_layers(phase="commit") on the returned lengths' cache_past
    and evict. With ``window`` the lengths are the drifting layout's."""
    return prepare_kv_window_stage_step(k_caches, v_caches, k_news, v_news, seqlens_k, k_stagings,
                                        v_stagings, window=window, out=out, flags=flags)()


# ---------------------------------------------------------------------------
# whole decode step in one launch
# ---------------------------------------------------------------------------

def prepare_kv_decode_step(win_k: Sequence[torch.Tensor], win_v: Sequence[torch.Tensor],
                           win_k_new: Sequence[torch.Tensor], win_v_new: Sequence[torch.Tensor],
                           seqlens_k: torch.Tensor, full_caches: Sequence[torch.Tensor],
                           full_new: Sequence[torch.Tensor], write_indices: torch.Tensor, *,
                           window: int | None = None, out: WindowLengths | None = None,
                           flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``kv_decode_step``."""
    n, B, H, C, D, S, strides = _check_layers(win_k, win_v, win_k_new, win_v_new)
    if S != 1:
        raise SwrtError("a decode step appends one row (S = 1)")
    _check_seqlens(seqlens_k, B)
    nf = len(full_caches)
    if len(full_new) != nf or not 0 <= nf <= MAX_BATCHED:
        raise SwrtError(f"need 0..{MAX_BATCHED} full caches, each with its new rows")
    M = full_caches[0].shape[2] if nf else 1
    for c, u in zip(full_caches, full_new):
        _contig("full cache", c)
        _contig("full-cache new rows", u)
        if c.shape != (B, H, M, D) or u.shape != (B, H, 1, D) or c.dtype != win_k[0].dtype \
                or u.dtype != win_k[0].dtype:
            raise SwrtError("full caches must be [B, H, M, D] and their new rows [B, H, 1, D], "
                            "in the windowed caches' dtype")
    if nf:
        _contig("write_indices", write_indices)
        if write_indices.dtype != torch.int64 or write_indices.shape != (B,):
            raise SwrtError("write_indices must be int64 [B]")
    dev = _device_of(*win_k, *win_v, *win_k_new, *win_v_new, seqlens_k, *full_caches,
                     *full_new, write_indices, flags)
    out = _lengths_out(out, B, dev)
    args = (n, _ptrs(win_k), _ptrs(win_v), _ptrs(win_k_new), _ptrs(win_v_new), strides,
            _ptr(seqlens_k), C, C if window is None else window, _ptr(out.total), _ptr(out.past),
            _ptr(out.cache_past),
            _ptr(out.cache_total), _ptr(out.evict), nf, _ptrs(full_caches) if nf else None,
            _ptrs(full_new) if nf else None, _ptr(write_indices) if nf else None, M, B, H, D,
            _bits(win_k[0]), _flags_ptr(flags))
    keep = (*win_k, *win_v, *win_k_new, *win_v_new, seqlens_k, *full_caches, *full_new,
            write_indices, *out, flags)
    return PreparedCall(lib().swrt_kv_decode_step, args, dev, "kv_decode_step", keep, out)


def kv_decode_step(win_k, win_v, win_k_new, win_v_new, seqlens_k, full_caches, full_new,
                   write_indices, *, window: int | None = None, out: WindowLengths | None = None,
                   flags: torch.Tensor | None = None) -> WindowLengths:
    """Every KV-cache update of one decode step in one launch: the lengths of
    the windowed layers from ``seqlens_k`` (returned), the in-place shift and
    append of every windowed layer's K and V, and the linear TensorScatter of
    one new row at ``write_indices`` into every full cache. Same bytes as
    kv_seq_lengths + kv_window_append_layers + tensor_scatter_batched; with
    ``window`` the windowed layers use the drifting layout."""
    return prepare_kv_decode_step(win_k, win_v, win_k_new, win_v_new, seqlens_k, full_caches,
                                  full_new, write_indices, window=window, out=out,
                                  flags=flags)()


# ---------------------------------------------------------------------------
# fused appends: RoPE on K at the absolute position + conversion / quantization
# ---------------------------------------------------------------------------

def prepare_kv_window_append_xf(k_caches, v_caches, k_news, v_news, cache_past_lens,
                                evict_counts, past_lens, xf: Transform, *, k_stagings=None,
                                v_stagings=None, phase: str = "all",
                                flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``kv_window_append_xf``."""
    n, B, H, C, D, S, strides = _check_layers(k_caches, v_caches, k_news, v_news,
                                              new_dtype=k_news[0].dtype)
    kc = k_caches[0]
    x = xf.c(k_news[0].dtype, kc.dtype, H, D)
    everything = [*k_caches, *v_caches, *k_news, *v_news, cache_past_lens, evict_counts,
                  past_lens, flags, *xf.tables()]
    if S > 1:
        _check_stagings(k_stagings, v_stagings, n, B, H, C, S, D, kc.dtype)
        everything += [*k_stagings, *v_stagings]
    else:
        k_stagings = v_stagings = None
    dev = _device_of(*everything)
    for t in (cache_past_lens, evict_counts):
        _contig("lengths", t)
        if t.dtype != torch.int32 or t.shape != (B,):
            raise SwrtError("cache_past_lens and evict_counts must be int32 [B]")
    _contig("past_lens", past_lens)
    if past_lens.dtype != torch.int64 or past_lens.shape != (B,):
        raise SwrtError("past_lens must be int64 [B]")
    args = (n, _ptrs(k_caches), _ptrs(v_caches), _ptrs(k_news), _ptrs(v_news), strides,
            _ptrs(k_stagings), _ptrs(v_stagings), _ptr(cache_past_lens), _ptr(evict_counts),
            _ptr(past_lens), B, H, C, S, D, _PHASES[phase], ctypes.byref(x), _flags_ptr(flags))
    return PreparedCall(lib().swrt_kv_window_append_xf, args, dev, "kv_window_append_xf",
                        (*everything, x))


def kv_window_append_xf(k_caches, v_caches, k_news, v_news, cache_past_lens, evict_counts,
                        past_lens, xf: Transform, *, k_stagings=None, v_stagings=None,
                        phase: str = "all", flags: torch.Tensor | None = None) -> None:
    """``kv_window_append_layers`` whose new rows (float32 / float16 /
    bfloat16 [B, H, S, D] views) pass through ``xf`` on their way into caches
    of any transform dtype: row s of entry b at absolute position
    past_lens[b] + s (``past_lens`` = the lengths' ``past``). An entry whose
    positions leave the rotary tables is flagged FLAG_ROPE_RANGE and left
    untouched."""
    prepare_kv_window_append_xf(k_caches, v_caches, k_news, v_news, cache_past_lens, evict_counts,
                                past_lens, xf, k_stagings=k_stagings, v_stagings=v_stagings,
                                phase=phase, flags=flags)()


def prepare_kv_window_stage_step_xf(k_caches, v_caches, k_news, v_news, seqlens_k, k_stagings,
                                    v_stagings, xf: Transform, *, window: int | None = None,
                                    out: WindowLengths | None = None,
                                    flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``kv_window_stage_step_xf``."""
    n, B, H, C, D, S, strides = _check_layers(k_caches, v_caches, k_news, v_news,
                                              new_dtype=k_news[0].dtype)
    if S < 2:
        raise SwrtError("a staged step appends S >= 2 rows")
    _check_seqlens(seqlens_k, B)
    kc = k_caches[0]
    x = xf.c(k_news[0].dtype, kc.dtype, H, D)
    _check_stagings(k_stagings, v_stagings, n, B, H, C, S, D, kc.dtype)
    dev = _device_of(*k_caches, *v_caches, *k_news, *v_news, seqlens_k, *k_stagings,
                     *v_stagings, flags, *xf.tables())
    out = _lengths_out(out, B, dev)
    args = (n, _ptrs(k_caches), _ptrs(v_caches), _ptrs(k_news), _ptrs(v_news), strides,
            _ptrs(k_stagings), _ptrs(v_stagings), _ptr(seqlens_k), C,
            C if window is None else window, _ptr(out.total), _ptr(out.past), _ptr(out.cache_past),
            _ptr(out.cache_total), _ptr(out.evict), B, H, S, D, ctypes.byref(x), _flags_ptr(flags))
    keep = (*k_caches, *v_caches, *k_news, *v_news, seqlens_k, *k_stagings, *v_stagings, *out,
            flags, *xf.tables(), x)
    return PreparedCall(lib().swrt_kv_window_stage_step_xf, args, dev, "kv_window_stage_step_xf",
                        keep, out)


def kv_window_stage_step_xf(k_caches, v_caches, k_news, v_news, seqlens_k, k_stagings,
                            v_stagings, xf: Transform, *, window: int | None = None,
                            out: WindowLengths | None = None,
                            flags: torch.Tensor | None = None) -> WindowLengths:
    """``kv_window_stage_step`` whose new rows pass through ``xf`` at absolute
    positions past + s: the lengths and the fused stage phase in one launch.
    Finish with kv_window_append_xf(phase="commit") on the returned lengths'
    cache_past, evict and past."""
    return prepare_kv_window_stage_step_xf(k_caches, v_caches, k_news, v_news, seqlens_k,
                                           k_stagings, v_stagings, xf, window=window, out=out,
                                           flags=flags)()


def prepare_tensor_scatter_xf(pasts: Sequence[torch.Tensor], updates: Sequence[torch.Tensor],
                              tensors: Sequence[int], write_indices: torch.Tensor | None,
                              xf: Transform, *, mode: str = "linear",
                              outs: Sequence[torch.Tensor] | None = None,
                              flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``tensor_scatter_xf``."""
    n = len(pasts)
    if len(updates) != n or len(tensors) != n or not 1 <= n <= MAX_BATCHED:
        raise SwrtError(f"need 1..{MAX_BATCHED} (past, update, tensor) triples")
    p0, u0 = pasts[0], updates[0]
    presents = [torch.empty_like(p) for p in pasts] if outs is None else list(outs)
    x = xf.c(u0.dtype, p0.dtype, p0.shape[1] if p0.dim() == 4 else 1, p0.shape[-1])
    if p0.dim() < 3:
        raise SwrtError("a fused TensorScatter needs rank >= 3 ([..., M, head_dim])")
    if u0.dim() != p0.dim() or u0.shape[:-2] != p0.shape[:-2] or u0.shape[-1] != p0.shape[-1]:
        raise SwrtError("updates must be [..., S, head_dim] with the caches' other dims")
    _check_write_indices(write_indices, p0.shape[0])
    _flags_ptr(flags)
    dev = _device_of(*pasts, *updates, *presents, write_indices, flags, *xf.tables())
    for p, u, o in zip(pasts, updates, presents):
        for name, t in (("past", p), ("update", u), ("out", o)):
            _contig(name, t)
        if p.shape != p0.shape or o.shape != p0.shape or u.shape != u0.shape or \
                p.dtype != p0.dtype or o.dtype != p0.dtype or u.dtype != u0.dtype:
            raise SwrtError("every past/out must share one shape and dtype, every update too")
    rank = p0.dim()
    shape = (ctypes.c_int64 * rank)(*p0.shape)
    tens = (ctypes.c_int * n)(*[int(t) for t in tensors])
    args = (n, _ptrs(presents), _ptrs(pasts), _ptrs(updates), tens, _ptr(write_indices), shape,
            rank, u0.shape[-2], _MODES[mode], ctypes.byref(x), _flags_ptr(flags))
    keep = (*pasts, *updates, *presents, write_indices, flags, *xf.tables(), x, tens, shape)
    return PreparedCall(lib().swrt_tensor_scatter_xf, args, dev, "tensor_scatter_xf", keep,
                        presents)


def tensor_scatter_xf(pasts, updates, tensors, write_indices, xf: Transform, *,
                      mode: str = "linear", outs=None, flags=None) -> list:
    """TensorScatter along axis -2 (caches [..., M, head_dim]) whose update
    rows pass through ``xf``: row s of batch entry b at absolute position
    write_indices[b] + s (before the circular wrap). ``tensors[i]`` is 0 for a
    K cache (rotated) and 1 for a V cache. ``outs=pasts`` updates in place."""
    return prepare_tensor_scatter_xf(pasts, updates, tensors, write_indices, xf, mode=mode,
                                     outs=outs, flags=flags)()


def prepare_kv_decode_step_xf(win_k, win_v, win_k_new, win_v_new, seqlens_k, full_k, full_v,
                              full_k_new, full_v_new, write_indices, xf: Transform, *,
                              window: int | None = None, out: WindowLengths | None = None,
                              flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``kv_decode_step_xf``."""
    n, B, H, C, D, S, strides = _check_layers(win_k, win_v, win_k_new, win_v_new,
                                              new_dtype=win_k_new[0].dtype)
    if S != 1:
        raise SwrtError("a decode step appends one row (S = 1)")
    _check_seqlens(seqlens_k, B)
    nf = len(full_k)
    if not (len(full_v) == len(full_k_new) == len(full_v_new) == nf) or \
            not 0 <= nf <= MAX_BATCHED // 2:
        raise SwrtError(f"need 0..{MAX_BATCHED // 2} full layers, each with K, V and new rows")
    cdt, ndt = win_k[0].dtype, win_k_new[0].dtype
    x = xf.c(ndt, cdt, H, D)
    M = full_k[0].shape[2] if nf else 1
    for c in (*full_k, *full_v):
        _contig("full cache", c)
        if c.shape != (B, H, M, D) or c.dtype != cdt:
            raise SwrtError("full caches must be [B, H, M, D] in the windowed caches' dtype")
    for u in (*full_k_new, *full_v_new):
        _contig("full-cache new rows", u)
        if u.shape != (B, H, 1, D) or u.dtype != ndt:
            raise SwrtError("full-cache new rows must be [B, H, 1, D] in the new rows' dtype")
    if nf:
        _contig("write_indices", write_indices)
        if write_indices.dtype != torch.int64 or write_indices.shape != (B,):
            raise SwrtError("write_indices must be int64 [B]")
    dev = _device_of(*win_k, *win_v, *win_k_new, *win_v_new, seqlens_k, *full_k, *full_v,
                     *full_k_new, *full_v_new, write_indices, flags, *xf.tables())
    out = _lengths_out(out, B, dev)
    args = (n, _ptrs(win_k), _ptrs(win_v), _ptrs(win_k_new), _ptrs(win_v_new), strides,
            _ptr(seqlens_k), C, C if window is None else window, _ptr(out.total), _ptr(out.past),
            _ptr(out.cache_past), _ptr(out.cache_total), _ptr(out.evict), nf,
            _ptrs(full_k) if nf else None, _ptrs(full_v) if nf else None,
            _ptrs(full_k_new) if nf else None, _ptrs(full_v_new) if nf else None,
            _ptr(write_indices) if nf else None, M, B, H, D, ctypes.byref(x), _flags_ptr(flags))
    keep = (*win_k, *win_v, *win_k_new, *win_v_new, seqlens_k, *full_k, *full_v, *full_k_new,
            *full_v_new, write_indices, *out, flags, *xf.tables(), x)
    return PreparedCall(lib().swrt_kv_decode_step_xf, args, dev, "kv_decode_step_xf", keep, out)


def kv_decode_step_xf(win_k, win_v, win_k_new, win_v_new, seqlens_k, full_k, full_v, full_k_new,
                      full_v_new, write_indices, xf: Transform, *, window: int | None = None,
                      out: WindowLengths | None = None,
                      flags: torch.Tensor | None = None) -> WindowLengths:
    """``kv_decode_step`` with the row transform fused into every write: new
    rows (float32 / float16 / bfloat16) of the windowed layers at position
    T - 1, of the full layers (K and V caches given separately) at
    write_indices[b]; every cache in the transform's output dtype."""
    return prepare_kv_decode_step_xf(win_k, win_v, win_k_new, win_v_new, seqlens_k, full_k,
                                     full_v, full_k_new, full_v_new, write_indices, xf,
                                     window=window, out=out, flags=flags)()


# ---------------------------------------------------------------------------
# decode attention over the windowed caches
# ---------------------------------------------------------------------------

def prepare_window_attention(qs: Sequence[torch.Tensor], k_caches: Sequence[torch.Tensor],
                             v_caches: Sequence[torch.Tensor], cache_total_lens: torch.Tensor,
                             window: int, *, scale: float | None = None,
                             out_dtype: torch.dtype | None = None,
                             outs: Sequence[torch.Tensor] | None = None,
                             flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``window_attention``."""
    n = len(qs)
    if not (len(k_caches) == len(v_caches) == n) or not 1 <= n <= MAX_LAYERS:
        raise SwrtError(f"need 1..{MAX_LAYERS} layers with q, K and V each")
    kc = k_caches[0]
    if kc.dim() != 4 or qs[0].dim() != 3:
        raise SwrtError("caches must be [B, Hkv, C, D] and queries [B, Hq, D]")
    B, Hkv, C, D = kc.shape
    Hq = qs[0].shape[1]
    dt = kc.dtype
    if dt not in (torch.float32, torch.float16, torch.bfloat16):
        raise SwrtError("attention takes float32, float16 or bfloat16 caches")
    odt = out_dtype if out_dtype is not None else (outs[0].dtype if outs else dt)
    outs = [torch.empty((B, Hq, D), dtype=odt, device=kc.device) for _ in range(n)] \
        if outs is None else list(outs)
    for t in (*k_caches, *v_caches):
        _contig("cache", t)
        if t.shape != kc.shape or t.dtype != dt:
            raise SwrtError("all caches must share shape and dtype")
    for t in qs:
        _contig("q", t)
        if t.shape != (B, Hq, D) or t.dtype != dt:
            raise SwrtError("queries must be [B, Hq, D] in the caches' dtype")
    for t in outs:
        _contig("out", t)
        if t.shape != (B, Hq, D) or t.dtype != odt or odt not in XF_TYPES or \
                odt in (torch.int8, torch.uint8):
            raise SwrtError("outputs must be [B, Hq, D] float32, float16 or bfloat16")
    _contig("cache_total_lens", cache_total_lens)
    if cache_total_lens.dtype != torch.int32 or cache_total_lens.shape != (B,):
        raise SwrtError("cache_total_lens must be int32 [B]")
    dev = _device_of(*qs, *k_caches, *v_caches, *outs, cache_total_lens, flags)
    sc = D ** -0.5 if scale is None else float(scale)
    args = (n, _ptrs(qs), _ptrs(k_caches), _ptrs(v_caches), _ptrs(outs), _ptr(cache_total_lens),
            window, B, Hq, Hkv, C, D, sc, XF_TYPES[dt], XF_TYPES[odt], _flags_ptr(flags))
    keep = (*qs, *k_caches, *v_caches, *outs, cache_total_lens, flags)
    return PreparedCall(lib().swrt_window_attention, args, dev, "window_attention", keep, outs)


def window_attention(qs, k_caches, v_caches, cache_total_lens, window: int, *,
                     scale: float | None = None, out_dtype: torch.dtype | None = None,
                     outs=None, flags=None) -> list:
    """One-token decode attention of every layer's queries [B, Hq, D] over
    its windowed caches [B, Hkv, C, D]: each query head h attends the last
    ``window`` resident rows [max(0, L - W), L) of KV head h // (Hq // Hkv),
    L = ``cache_total_lens`` (the lengths' ``cache_total``). fp32 softmax and
    accumulation; ``scale`` defaults to 1 / sqrt(D). Returns the outputs."""
    return prepare_window_attention(qs, k_caches, v_caches, cache_total_lens, window,
                                    scale=scale, out_dtype=out_dtype, outs=outs, flags=flags)()


# ---------------------------------------------------------------------------
# paged caches
# ---------------------------------------------------------------------------
# page formats (include/swrt.h SWRT_XF_*)
PAGE_FORMATS = {"f32": 1, "f16": 2, "bf16": 3, "int8": 4, "uint8": 5, "int4": 6, "uint4": 7,
                "int2": 8, "uint2": 9}
# the C struct swrt_page, 64 bytes
PAGE_DTYPE = np.dtype([("start", "<i8"), ("length", "<i4"), ("capacity", "<i4"),
                       ("k_offset", "<i8"), ("v_offset", "<i8"), ("k_format", "<i4"),
                       ("v_format", "<i4"), ("k_scale", "<f4"), ("v_scale", "<f4"),
                       ("k_zero_point", "<i4"), ("v_zero_point", "<i4"), ("reserved", "<i4", (2,))])
_Q_TYPES = {torch.float32: 1, torch.float16: 2, torch.bfloat16: 3}


class PagedLayer(ctypes.Structure):
    """The C struct swrt_paged_layer."""
    _fields_ = [("q", ctypes.c_void_p), ("out", ctypes.c_void_p), ("arena", ctypes.c_void_p),
                ("arena_bytes", ctypes.c_int64), ("pages", ctypes.c_void_p),
                ("n_pages", ctypes.c_int64), ("page_ptr", ctypes.c_void_p),
                ("page_ids", ctypes.c_void_p), ("n_ids", ctypes.c_int64),
                ("page_count", ctypes.c_void_p), ("page_stride", ctypes.c_int64)]


def page_table(fields: dict) -> np.ndarray:
    """swrt_page descriptors (host, PAGE_DTYPE) from per-field arrays."""
    n = len(fields["start"])
    t = np.zeros(n, PAGE_DTYPE)
    for name in PAGE_DTYPE.names:
        if name in fields:
            t[name] = fields[name]
    return t


@dataclass
class PagedCache:
    """One layer's paged cache on the device: ``arena`` (uint8, every page
    payload), ``pages`` (uint8 [n_pages * 64]: the swrt_page descriptors) and
    a block table naming each stream's pages in token order through
    ``page_ids`` (int32), in one of two forms:

    - compressed rows: ``page_ptr`` (int32 [streams + 1]); stream s owns
      page_ids[page_ptr[s]:page_ptr[s + 1]];
    - slotted rows: ``page_count`` (int32 [streams]) and ``page_stride``;
      stream s owns the page_stride slots from s * page_stride and uses the
      first page_count[s]. The sealed append grows this form.

    Several layers may share pages and the block table (one arena each)."""
    arena: torch.Tensor
    pages: torch.Tensor
    page_ptr: torch.Tensor | None
    page_ids: torch.Tensor
    page_count: torch.Tensor | None = None
    page_stride: int = 0

    @staticmethod
    def upload(table: np.ndarray, page_ptr, page_ids, arena, device, page_count=None,
               page_stride: int = 0) -> "PagedCache":
        def dev(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(device)
        pages = torch.from_numpy(np.ascontiguousarray(table, PAGE_DTYPE).view(np.uint8)).to(device)
        ar = arena if isinstance(arena, torch.Tensor) else dev(arena, np.uint8)
        return PagedCache(ar, pages, None if page_ptr is None else dev(page_ptr, np.int32),
                          dev(page_ids, np.int32),
                          None if page_count is None else dev(page_count, np.int32), page_stride)

    @property
    def n_pages(self) -> int:
        return self.pages.numel() // PAGE_DTYPE.itemsize

    @property
    def slotted(self) -> bool:
        return self.page_count is not None

    def n_streams(self) -> int:
        return self.page_count.numel() if self.slotted else self.page_ptr.numel() - 1

    def tensors(self) -> tuple:
        """The device tensors of the cache (arena and block table)."""
        return tuple(t for t in (self.arena, self.pages, self.page_ptr, self.page_ids,
                                 self.page_count) if t is not None)

    def table(self) -> np.ndarray:
        """The descriptors, copied to the host."""
        return self.pages.cpu().numpy().view(PAGE_DTYPE).copy()

    def _check(self):
        if (self.page_ptr is None) == (self.page_count is None):
            raise SwrtError("a block table is either page_ptr (compressed rows) or page_count "
                            "(slotted rows)")
        for name, t, dt in (("arena", self.arena, torch.uint8), ("pages", self.pages, torch.uint8),
                            ("page_ptr", self.page_ptr, torch.int32),
                            ("page_ids", self.page_ids, torch.int32),
                            ("page_count", self.page_count, torch.int32)):
            if t is None:
                continue
            _contig(name, t)
            if t.dtype != dt or t.dim() != 1:
                raise SwrtError(f"{name} must be a 1-D {dt} tensor")
        if self.pages.numel() % PAGE_DTYPE.itemsize:
            raise SwrtError("pages must hold whole 64-byte descriptors")
        if self.slotted and self.page_stride < 1:
            raise SwrtError("slotted rows need page_stride >= 1")

    def layer(self, q=None, out=None) -> PagedLayer:
        return PagedLayer(_ptr(q), _ptr(out), _ptr(self.arena), self.arena.numel(),
                          _ptr(self.pages), self.n_pages, _ptr(self.page_ptr),
                          _ptr(self.page_ids), self.page_ids.numel(), _ptr(self.page_count),
                          self.page_stride if self.slotted else 0)


def _formats_mask(formats) -> int:
    """The page-format set as the library's bit mask (None: any format)."""
    if formats is None:
        return 0
    mask = 0
    for f in formats:
        code = PAGE_FORMATS.get(f, f) if isinstance(f, str) else int(f)
        if code not in PAGE_FORMATS.values():
            raise SwrtError(f"unknown page format {f!r}")
        mask |= 1 << code
    return mask


def prepare_paged_attention(qs: Sequence[torch.Tensor], caches: Sequence[PagedCache],
                            left_window: int, kv_heads: int, *, scale: float | None = None,
                            out_dtype: torch.dtype | None = None,
                            outs: Sequence[torch.Tensor] | None = None,
                            flags: torch.Tensor | None = None,
                            formats=None) -> PreparedCall:
    """See ``paged_attention``."""
    n = len(qs)
    if len(caches) != n or not 1 <= n <= MAX_LAYERS:
        raise SwrtError(f"need 1..{MAX_LAYERS} layers with a query and a cache each")
    q0 = qs[0]
    if q0.dim() != 3 or q0.dtype not in _Q_TYPES:
        raise SwrtError("queries must be [B, Hq, D] float32, float16 or bfloat16")
    B, Hq, D = q0.shape
    odt = out_dtype if out_dtype is not None else (outs[0].dtype if outs else q0.dtype)
    if odt not in _Q_TYPES:
        raise SwrtError("outputs are float32, float16 or bfloat16")
    outs = [torch.empty((B, Hq, D), dtype=odt, device=q0.device) for _ in range(n)] \
        if outs is None else list(outs)
    for q, o, c in zip(qs, outs, caches):
        _contig("q", q)
        _contig("out", o)
        if q.shape != q0.shape or q.dtype != q0.dtype or o.shape != q0.shape or o.dtype != odt:
            raise SwrtError("every query [B, Hq, D] of one dtype, every output of another")
        c._check()
        if c.n_streams() != B * kv_heads:
            raise SwrtError("the block table must hold batch * kv_heads streams")
    _flags_ptr(flags)
    dev = _device_of(*qs, *outs, *(t for c in caches for t in c.tensors()), flags)
    layers = (PagedLayer * n)(*[c.layer(q, o) for c, q, o in zip(caches, qs, outs)])
    sc = D ** -0.5 if scale is None else float(scale)
    args = (n, ctypes.cast(layers, ctypes.c_void_p), int(left_window), B, Hq, kv_heads, D, sc,
            _Q_TYPES[q0.dtype], _Q_TYPES[odt], _formats_mask(formats), _flags_ptr(flags))
    keep = (layers, *qs, *outs, *caches, flags)
    return PreparedCall(lib().swrt_paged_attention, args, dev, "paged_attention", keep, outs)


def paged_attention(qs, caches, left_window: int, kv_heads: int, *, scale: float | None = None,
                    out_dtype: torch.dtype | None = None, outs=None, flags=None,
                    formats=None) -> list:
    """One-token decode attention of every layer's queries [B, Hq, D] over its
    paged cache: query head h of entry b reads stream b * kv_heads + h //
    (Hq // kv_heads) over its last ``left_window`` + 1 tokens (all for a
    negative value), decoding each page's format. ``formats`` (names of
    PAGE_FORMATS or their codes; None: any) declares the formats the visible
    pages may have: a page of another format fails its checks (BAD_PAGES for
    its stream), and a set without f32 and f16 runs the leaner kernel.
    Returns the outputs."""
    return prepare_paged_attention(qs, caches, left_window, kv_heads, scale=scale,
                                   out_dtype=out_dtype, outs=outs, flags=flags,
                                   formats=formats)()


def paged_quantize(cache: PagedCache, blocks: torch.Tensor, dst_offsets: torch.Tensor,
                   free_begin: int, free_end: int, k_format: int, k_scale: float,
                   k_zero_point: int, v_format: int, v_scale: float, v_zero_point: int,
                   head_dim: int, *, pages_out: torch.Tensor | None = None,
                   flags: torch.Tensor) -> torch.Tensor:
    """QuantizePagedCache: convert the selected pages (``blocks`` int32,
    strictly ascending) into the target formats at ``dst_offsets`` (int64
    [2 n]: K0, V0, K1, ...) inside the arena's free region [free_begin,
    free_end); returns the new descriptor table (``pages_out``, which may be
    ``cache.pages``). ``flags`` (int32 device word, BAD_PAGES clear) receives
    FLAG_BAD_PAGES when a check fails; then nothing is written."""
    cache._check()
    out = torch.empty_like(cache.pages) if pages_out is None else pages_out
    for name, t, dt in (("blocks", blocks, torch.int32), ("dst_offsets", dst_offsets, torch.int64)):
        _contig(name, t)
        if t.dtype != dt or t.dim() != 1:
            raise SwrtError(f"{name} must be a 1-D {dt} tensor")
    if dst_offsets.numel() != 2 * blocks.numel() or out.shape != cache.pages.shape:
        raise SwrtError("dst_offsets needs two entries per block; pages_out the table's size")
    if flags is None:
        raise SwrtError("paged_quantize needs a flag word")
    dev = _device_of(cache.arena, cache.pages, blocks, dst_offsets, out, flags)
    with torch.cuda.device(dev):
        st = lib().swrt_paged_quantize(
            _ptr(cache.arena), cache.arena.numel(), _ptr(cache.pages), cache.n_pages,
            _ptr(blocks), blocks.numel(), _ptr(dst_offsets), int(free_begin), int(free_end),
            _ptr(out), int(k_format), float(k_scale), int(k_zero_point), int(v_format),
            float(v_scale), int(v_zero_point), int(head_dim), _flags_ptr(flags),
            ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    _check(st, "paged_quantize")
    return out


def prepare_paged_append(caches: Sequence[PagedCache], k_news: Sequence[torch.Tensor],
                         v_news: Sequence[torch.Tensor], *, first_id: int, free_begin: int,
                         free_end: int, k_format: int, v_format: int, k_scale: float = 1.0,
                         k_zero_point: int = 0, v_scale: float = 1.0, v_zero_point: int = 0,
                         flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``paged_append``."""
    n = len(caches)
    if len(k_news) != n or len(v_news) != n or not 1 <= n <= MAX_LAYERS:
        raise SwrtError(f"need 1..{MAX_LAYERS} layers with a cache and new K and V rows each")
    k0 = k_news[0]
    if k0.dim() != 3 or k0.dtype not in _Q_TYPES:
        raise SwrtError("new rows must be [streams, S, D] float32, float16 or bfloat16")
    NS, S, D = k0.shape
    for c, k, v in zip(caches, k_news, v_news):
        c._check()
        if not c.slotted:
            raise SwrtError("the sealed append grows slotted block tables (page_count)")
        _contig("k_new", k)
        _contig("v_new", v)
        if k.shape != k0.shape or v.shape != k0.shape or k.dtype != k0.dtype or v.dtype != k0.dtype:
            raise SwrtError("every new row tensor [streams, S, D] of one dtype")
        if c.n_streams() != NS:
            raise SwrtError("page_count must hold one entry per stream")
    _flags_ptr(flags)
    dev = _device_of(*k_news, *v_news, *(t for c in caches for t in c.tensors()), flags)
    layers = (PagedLayer * n)(*[c.layer() for c in caches])
    args = (n, ctypes.cast(layers, ctypes.c_void_p), _ptrs(k_news), _ptrs(v_news),
            _Q_TYPES[k0.dtype], NS, S, D, int(first_id), int(free_begin), int(free_end),
            int(k_format), float(k_scale), int(k_zero_point), int(v_format), float(v_scale),
            int(v_zero_point), _flags_ptr(flags))
    keep = (layers, *caches, *k_news, *v_news, flags)
    return PreparedCall(lib().swrt_paged_append, args, dev, "paged_append", keep)


def paged_append(caches, k_news, v_news, *, first_id: int, free_begin: int, free_end: int,
                 k_format: int, v_format: int, k_scale: float = 1.0, k_zero_point: int = 0,
                 v_scale: float = 1.0, v_zero_point: int = 0, flags=None) -> None:
    """Sealed-block append: each stream's new K and V rows ([streams, S, D])
    become one new block of S tokens, descriptor ``first_id + s``, payload in
    the arena's free region from ``free_begin`` (K then V, stream after
    stream), formats and scalar parameters as given; the stream's next slot
    of the (slotted) block table names it. Earlier blocks are never written."""
    prepare_paged_append(caches, k_news, v_news, first_id=first_id, free_begin=free_begin,
                         free_end=free_end, k_format=k_format, v_format=v_format,
                         k_scale=k_scale, k_zero_point=k_zero_point, v_scale=v_scale,
                         v_zero_point=v_zero_point, flags=flags)()


def prepare_paged_append_open(caches: Sequence[PagedCache], k_news: Sequence[torch.Tensor],
                              v_news: Sequence[torch.Tensor], *,
                              flags: torch.Tensor | None = None) -> PreparedCall:
    """See ``paged_append_open``."""
    n = len(caches)
    if len(k_news) != n or len(v_news) != n or not 1 <= n <= MAX_LAYERS:
        raise SwrtError(f"need 1..{MAX_LAYERS} layers with a cache and new K and V rows each")
    k0 = k_news[0]
    if k0.dim() != 2 or k0.dtype not in _Q_TYPES:
        raise SwrtError("new rows must be [streams, D] float32, float16 or bfloat16")
    S, D = k0.shape
    for c, k, v in zip(caches, k_news, v_news):
        c._check()
        _contig("k_new", k)
        _contig("v_new", v)
        if k.shape != k0.shape or v.shape != k0.shape or k.dtype != k0.dtype or v.dtype != k0.dtype:
            raise SwrtError("every new row tensor [streams, D] of one dtype")
        if c.n_streams() != S:
            raise SwrtError("the block table must hold one stream per new row")
    _flags_ptr(flags)
    dev = _device_of(*k_news, *v_news, *(t for c in caches for t in c.tensors()), flags)
    layers = (PagedLayer * n)(*[c.layer() for c in caches])
    args = (n, ctypes.cast(layers, ctypes.c_void_p), _ptrs(k_news), _ptrs(v_news),
            _Q_TYPES[k0.dtype], S, D, _flags_ptr(flags))
    keep = (layers, *caches, *k_news, *v_news, flags)
    return PreparedCall(lib().swrt_paged_append_open, args, dev, "paged_append_open", keep)


def paged_append_open(caches, k_news, v_news, *, flags=None) -> None:
    """The open-page extension: each stream's new K and V rows ([streams, D])
    into its last page, encoded in the page's formats; the page grows by one
    row (once per distinct block table)."""
    prepare_paged_append_open(caches, k_news, v_news, flags=flags)()
