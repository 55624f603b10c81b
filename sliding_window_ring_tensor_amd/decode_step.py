"""One whole-model decode step of KV-cache updates (one launch, or three).

A model whose layers alternate between windowed attention (a window-sized
cache, pull request "GQA support sliding_window_cache", section "Design") and
full attention (a max-length cache updated by TensorScatter in linear mode at
write index T - 1, ONNX operator page "TensorScatter"). At every decode step
each layer receives one new K row and one new V row per (batch, kv-head):

  1. kv_seq_lengths           once for all windowed layers (they share the
                              running lengths): seqlens_k -> Lp, E;
  2. kv_window_append_layers  every windowed layer's K and V: shift by E and
                              append at Lp - E, in place (S = 1), one launch;
  3. tensor_scatter_batched   every full layer's K and V: write row T - 1,
                              in place, one launch;

or all three in one launch (kv_decode_step, the default), which writes the
same bytes. With a fused-append workload (spec.new_dtype set) the new rows
pass through the row transform on their way in (kv_window_append_xf,
tensor_scatter_xf, kv_decode_step_xf): K rotated at position T - 1, every
row converted or quantized into the caches' dtype. The buffers are plain torch tensors on one device; the step only
issues library calls (marshalled once) on the current stream, so it can be
captured in a graph.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import sliding_window_ring_tensor_amd as swrt
from sliding_window_ring_tensor_amd import workloads as wl


@dataclass
class StepBuffers:
    win_k: list      # windowed K caches [B, H, W, D]
    win_v: list
    win_kn: list     # new rows [B, H, 1, D]
    win_vn: list
    full_k: list     # full caches [B, H, M, D]
    full_v: list
    full_kn: list
    full_vn: list
    seqlens_k: torch.Tensor      # int32 [B], T - 1
    write_indices: torch.Tensor  # int64 [B], T - 1
    lengths: swrt.WindowLengths  # outputs of kv_seq_lengths
    flags: torch.Tensor          # int32 [1]
    xf: swrt.Transform | None = None  # fused append
    win_q: list | None = None         # decode attention: queries [B, Hq, D] per windowed layer
    win_out: list | None = None       # and its outputs


class ModelDecodeStep:
    """The KV-cache updates of one decode step of a windowed/full layer stack."""

    def __init__(self, spec: wl.ModelStep, device, set_id: int = 0, raw_bits: bool = False,
                 fill: bool = True):
        self.spec = spec
        self.device = torch.device(device)
        B, H, D, W, M = spec.batch, spec.kv_heads, spec.head_dim, spec.window, spec.max_seq
        dt = spec.dtype
        ndt = spec.new_dtype or dt  # new rows
        seed = spec.seed * 100 + set_id

        def buf(shape, bid):
            t = ndt if shape[2] == 1 else dt
            if fill:
                return wl.payload(shape, t, seed, bid, self.device, raw_bits and t == dt)
            return torch.empty(shape, dtype=t, device=self.device)

        nw, nf = len(spec.windowed_layers), len(spec.full_layers)
        self.buffers = StepBuffers(
            win_k=[buf((B, H, W, D), 10 * i + 0) for i in range(nw)],
            win_v=[buf((B, H, W, D), 10 * i + 1) for i in range(nw)],
            win_kn=[buf((B, H, 1, D), 10 * i + 2) for i in range(nw)],
            win_vn=[buf((B, H, 1, D), 10 * i + 3) for i in range(nw)],
            full_k=[buf((B, H, M, D), 1000 + 10 * i + 0) for i in range(nf)],
            full_v=[buf((B, H, M, D), 1000 + 10 * i + 1) for i in range(nf)],
            full_kn=[buf((B, H, 1, D), 1000 + 10 * i + 2) for i in range(nf)],
            full_vn=[buf((B, H, 1, D), 1000 + 10 * i + 3) for i in range(nf)],
            seqlens_k=torch.from_numpy(spec.seqlens_k).to(self.device),
            write_indices=torch.from_numpy(spec.write_indices).to(self.device),
            lengths=swrt.WindowLengths(*(torch.zeros(B, dtype=t, device=self.device) for t in (
                torch.int64, torch.int64, torch.int32, torch.int32, torch.int32))),
            flags=torch.zeros(1, dtype=torch.int32, device=self.device),
        )
        if spec.q_heads:
            self.buffers.win_q = [buf((B, spec.q_heads, 1, D), 500 + i).view(B, spec.q_heads, D)
                                  for i in range(nw)]
            self.buffers.win_out = [torch.empty((B, spec.q_heads, D), dtype=dt, device=self.device)
                                    for _ in range(nw)]
        if spec.new_dtype is not None:
            cos = sin = None
            if spec.rotary_dim:
                cos, sin = wl.rope_tables(spec.rope_positions, spec.rotary_dim,
                                          device=self.device)
            self.buffers.xf = swrt.Transform(cos, sin, False, spec.k_scale, spec.v_scale)

    # -- the step ---------------------------------------------------------
    def _prepared(self):
        if getattr(self, "_calls", None) is None and self.buffers.xf is not None:
            b, s = self.buffers, self.spec
            nf = len(b.full_k)
            self._calls = {
                "lengths": swrt.prepare_kv_seq_lengths(b.seqlens_k, 1, s.window, out=b.lengths,
                                                       flags=b.flags),
                "windowed": swrt.prepare_kv_window_append_xf(
                    b.win_k, b.win_v, b.win_kn, b.win_vn, b.lengths.cache_past, b.lengths.evict,
                    b.lengths.past, b.xf, flags=b.flags),
                "full": swrt.prepare_tensor_scatter_xf(
                    b.full_k + b.full_v, b.full_kn + b.full_vn, [0] * nf + [1] * nf,
                    b.write_indices, b.xf, outs=b.full_k + b.full_v, flags=b.flags),
                "fused": swrt.prepare_kv_decode_step_xf(
                    b.win_k, b.win_v, b.win_kn, b.win_vn, b.seqlens_k, b.full_k, b.full_v,
                    b.full_kn, b.full_vn, b.write_indices, b.xf, out=b.lengths, flags=b.flags),
            }
        if getattr(self, "_calls", None) is None:
            b, s = self.buffers, self.spec
            caches = b.full_k + b.full_v
            self._calls = {
                "lengths": swrt.prepare_kv_seq_lengths(b.seqlens_k, 1, s.window, out=b.lengths,
                                                       flags=b.flags),
                "windowed": swrt.prepare_kv_window_append_layers(
                    b.win_k, b.win_v, b.win_kn, b.win_vn, b.lengths.cache_past, b.lengths.evict,
                    flags=b.flags),
                "full": swrt.prepare_tensor_scatter_batched(
                    caches, b.full_kn + b.full_vn, b.write_indices, axis=2, mode="linear",
                    outs=caches, flags=b.flags),
                "fused": swrt.prepare_kv_decode_step(
                    b.win_k, b.win_v, b.win_kn, b.win_vn, b.seqlens_k, caches,
                    b.full_kn + b.full_vn, b.write_indices, out=b.lengths, flags=b.flags),
            }
        return self._calls

    def attention(self):
        """Decode attention of every windowed layer over its window (after
        the step has appended and written the lengths); returns the outputs."""
        if getattr(self, "_att", None) is None:
            b, s = self.buffers, self.spec
            self._att = swrt.prepare_window_attention(b.win_q, b.win_k, b.win_v,
                                                      b.lengths.cache_total, s.window,
                                                      outs=b.win_out, flags=b.flags)
        return self._att()

    def attention_bytes(self) -> int:
        """Bytes the attention must move: the visible K and V rows of every
        windowed layer read once, the queries read and the outputs written."""
        s = self.spec
        es = torch.empty((), dtype=s.dtype).element_size()
        L = np.minimum(s.total_lens.astype(np.int64), s.window)  # W = C: every resident row
        rows = int(L.sum()) * s.kv_heads
        nw = len(s.windowed_layers)
        return nw * (2 * rows * s.head_dim * es + 2 * s.batch * s.q_heads * s.head_dim * es)

    def lengths(self):
        self._prepared()["lengths"]()

    def windowed(self):
        self._prepared()["windowed"]()

    def full(self):
        self._prepared()["full"]()

    def run_three(self):
        """The step as three launches: lengths, windowed layers, full layers."""
        c = self._prepared()
        c["lengths"]()
        c["windowed"]()
        c["full"]()

    def run_fused(self):
        """The step as one launch (swrt_kv_decode_step)."""
        self._prepared()["fused"]()

    def run(self, fused: bool = True):
        if fused:
            self.run_fused()
        else:
            self.run_three()

    # -- accounting -------------------------------------------------------
    def algorithmic_bytes(self) -> dict:
        """Bytes the method must move in one step: every byte read once and
        written once. Windowed slice with E = 1: the Lp - 1 shifted rows, each
        read and written, and the appended row (read as a new row, written as
        a cache row); with E = 0: the appended row. Full cache: the written
        row. A fused append also reads each batch entry's table row once (cos
        and sin)."""
        s = self.spec
        row = s.head_dim * torch.empty((), dtype=s.dtype).element_size()
        new_row = s.head_dim * torch.empty((), dtype=s.new_dtype or s.dtype).element_size()
        T = s.total_lens.astype(np.int64)
        P = T - 1
        Lp = np.minimum(P, s.window)
        E = np.maximum(0, Lp + 1 - s.window)
        per_slice = 2 * row * E * (Lp - E) + row + new_row
        windowed = int(per_slice.sum()) * s.kv_heads * 2 * len(s.windowed_layers)
        full = (row + new_row) * s.batch * s.kv_heads * 2 * len(s.full_layers)
        tables = s.batch * s.rotary_dim * 4 if s.new_dtype is not None else 0
        return {"windowed": windowed, "full": full, "tables": tables,
                "lengths": s.batch * (4 + 8 + 8 + 4 * 3), "total": windowed + full + tables}
