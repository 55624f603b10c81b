"""A decode step over paged caches (onnx-light how-to "Persistent
input/output feedback", section "Optional heterogeneous paged KV").

Every layer keeps its K/V pages in its own arena; one block table (page
descriptors, page_ptr, page_ids) serves all layers. A step is

  1. paged_append      each stream's new K and V rows as a new sealed block
                       (on a slotted copy of the table; the benchmark times
                       attention over a fixed cache, since appends grow it);
  2. paged_attention   every layer's 64 query heads over the visible tokens
                       of their KV head's stream, pages decoded in their own
                       formats (cold pages int8, the last two bf16), one
                       launch for all layers;

and, every ``block`` steps, paged_quantize turns the page that has just left
the hot set into the cold format (QuantizePagedCache on selected blocks).
The buffers are plain torch tensors on one device; the calls are marshalled
once and issued on the current stream.
"""
from __future__ import annotations

import numpy as np
import torch

import sliding_window_ring_tensor_amd as swrt
from sliding_window_ring_tensor_amd import workloads as wl


class PagedDecodeStep:
    def __init__(self, spec: wl.PagedStep, device, set_id: int = 0, spare_bytes: int = 0):
        self.spec, self.device = spec, torch.device(device)
        fields, ptr, ids, arena_bytes, visible = wl.paged_step_layout(spec)
        self.fields, self.page_ptr_host, self.page_ids_host = fields, ptr, ids
        self.layout_bytes, self.visible_pages = arena_bytes, visible
        self.table_host = swrt.page_table(fields)
        s = spec
        total = arena_bytes + spare_bytes
        total += (-total) % 2
        seed = s.seed * 100 + set_id
        # payload: U[-1, 1) bf16 values; an int8 page reads their bytes as codes
        self.arenas = [wl.device_payload((total // 2,), torch.bfloat16, seed, 10 + i, self.device)
                       .view(torch.uint8) for i in range(s.layers)]
        base = swrt.PagedCache.upload(self.table_host, ptr, ids, self.arenas[0], self.device)
        self.caches = [swrt.PagedCache(a, base.pages, base.page_ptr, base.page_ids)
                       for a in self.arenas]
        B, Hq, D = s.batch, s.q_heads, s.head_dim
        self.qs = [wl.device_payload((B, Hq, D), torch.bfloat16, seed, 100 + i, self.device)
                   for i in range(s.layers)]
        self.outs = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device=self.device)
                     for _ in range(s.layers)]
        self.flags = torch.zeros(1, dtype=torch.int32, device=self.device)
        self._att = None

    def attention(self):
        if self._att is None:
            s = self.spec
            self._att = swrt.prepare_paged_attention(self.qs, self.caches, s.left_window,
                                                     s.kv_heads, outs=self.outs, flags=self.flags,
                                                     formats=(s.hot_format, s.cold_format))
        return self._att()

    def visible(self):
        """Per stream: (page index, first row, rows) of every page the window
        reaches, from the host copy of the layout."""
        s = self.spec
        out = []
        st, ln = self.fields["start"], self.fields["length"]
        for k in range(len(self.page_ptr_host) - 1):
            p0, p1 = self.page_ptr_host[k], self.page_ptr_host[k + 1]
            T = int(st[p1 - 1] + ln[p1 - 1]) if p1 > p0 else 0
            r0 = max(0, T - 1 - s.left_window) if s.left_window >= 0 else 0
            pages = []
            for i in range(p0, p1):
                if st[i] + ln[i] > r0:
                    first = max(0, r0 - int(st[i]))
                    pages.append((i, first, int(ln[i]) - first))
            out.append(pages)
        return out

    def attention_bytes(self) -> int:
        """Bytes the attention must move per step: every visible token's K
        and V row in its page's format, each visible page's descriptor (64 B)
        and id (4 B), each stream's two page_ptr entries, the queries read and
        the outputs written, for every layer."""
        s = self.spec
        per_layer = 0
        for pages in self.visible():
            per_layer += 8
            for i, _first, n in pages:
                kb = s.head_dim * wl.FORMAT_BITS[int(self.fields["k_format"][i])] // 8
                vb = s.head_dim * wl.FORMAT_BITS[int(self.fields["v_format"][i])] // 8
                per_layer += n * (kb + vb) + 64 + 4
        per_layer += 2 * s.batch * s.q_heads * s.head_dim * 2
        return s.layers * per_layer

    def cooling_selection(self):
        """The page each stream's hot set lets go next (its oldest hot page,
        for streams with more than one page), with destinations in the arena's
        spare room after the layout: (blocks, dst_offsets, bytes)."""
        s = self.spec
        rows = s.block * s.head_dim * wl.FORMAT_BITS[s.cold_format] // 8
        step = -(-rows // 16) * 16
        blocks = []
        for k in range(len(self.page_ptr_host) - 1):
            p0, p1 = self.page_ptr_host[k], self.page_ptr_host[k + 1]
            if p1 - p0 >= s.hot_pages:
                blocks.append(p1 - s.hot_pages)  # the oldest hot page
        blocks = np.array(sorted(blocks), np.int32)
        dst = self.layout_bytes + np.arange(2 * len(blocks), dtype=np.int64) * step
        return blocks, dst, 2 * len(blocks) * step
