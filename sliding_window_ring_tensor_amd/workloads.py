"""Seeded synthetic inputs for the KV-cache update workloads.

This module only draws inputs: shapes, seeded random payloads, write indices
and lengths. It holds none of the update arithmetic, so both the GPU path's
tests and the CPU oracle's checks can take their inputs from it.

Recipe (shared by tests and benchmark):
  - index and length draws: numpy Generator(PCG64(seed)), seed = workload number;
  - payloads: U[-1, 1) fp32 rounded to the payload dtype by torch (round to
    nearest even), or uniform random bytes for the raw-bits variants (every
    NaN / Inf / fp8 encoding appears). Host payloads come from
    PCG64(seed * 1000 + buffer id); large ones are drawn on their device with
    a torch generator seeded from (seed, buffer id), since a 12 GiB host draw
    would dominate every run.

Workloads (sizes and distributions):
  1  TensorScatter linear, fp32 past [2,2,16,8], update [2,2,3,8],
     write_indices ~ U{0..13}, axis -2.
  2  TensorScatter circular, bf16 cache [8,8,4096,128]; step A update S=1,
     step B update S=512, each with its own write_indices ~ U{0..4095}.
  3  windowed decode S=1, K/V bf16 [32,8,128,64], seqlens_k ~ U{1..8192}.
  4  windowed step S=256 through staging, K/V bf16 [4,8,4096,128], past
     length P ~ U{0..16384}, seqlens_k = P + 255.
  5  whole-model decode step: 24 layers, even layers windowed (K/V [64,8,128,64])
     and odd layers full linear TensorScatter caches (K/V [64,8,8192,64]); new
     rows [64,8,1,64]; total length T ~ U{1..8192} shared by all layers;
     windowed seqlens_k = T - 1, full write index T - 1; bf16 or fp8 e4m3fn.
  6  workload 5 as a loop of 200 consecutive decode steps (the benchmark
     builds it from workload 5's draws).
  7  workload 5 with the fused append: new rows bf16 [64,8,1,64] (U[-1,1)),
     caches int8 (random bytes); K rows rotated at position T - 1 with
     rotary_dim 64 (half-split pairs, tables cos/sin of p * 10000^(-2j/64),
     8192 positions); K scale 0.02, V scale 0.01, zero points 0.
  8  workload 5 followed by decode attention over its 12 windowed layers:
     queries bf16 [64, 64, 64] per layer (64 query heads on 8 KV heads, the
     CPU follow-up's head layout), window W = 128 = C, scale 1/8.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {
    "fp32": torch.float32,
    "bf16": torch.bfloat16,
    "fp16": torch.float16,
    "fp8_e4m3fn": torch.float8_e4m3fn,
    "fp8_e5m2": torch.float8_e5m2,
    "fp64": torch.float64,
    "int8": torch.int8,
    "uint8": torch.uint8,
    "int16": torch.int16,
    "int32": torch.int32,
    "int64": torch.int64,
    "bool": torch.bool,
    "complex64": torch.complex64,
    "complex128": torch.complex128,
}

_FLOATS = (torch.float32, torch.bfloat16, torch.float16, torch.float8_e4m3fn,
           torch.float8_e5m2, torch.float64)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def host_payload(g: np.random.Generator, shape, dtype: torch.dtype,
                 raw_bits: bool = False) -> torch.Tensor:
    """Host tensor of `shape`: U[-1,1) rounded to `dtype`, or random bytes."""
    n = int(np.prod(shape)) if len(shape) else 1
    if n == 0:
        return torch.empty(shape, dtype=dtype)
    if raw_bits or dtype not in _FLOATS:
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        raw = torch.from_numpy(g.integers(0, 256, size=nbytes, dtype=np.uint8))
        if dtype == torch.bool:
            raw = raw & 1  # a bool byte must hold 0 or 1
        return raw.view(dtype).reshape(shape).clone()
    vals = torch.from_numpy(g.uniform(-1.0, 1.0, size=n).astype(np.float32))
    if dtype == torch.float64:
        vals = torch.from_numpy(g.uniform(-1.0, 1.0, size=n))
    return vals.to(dtype).reshape(shape)


def device_payload(shape, dtype: torch.dtype, seed: int, buffer_id: int,
                   device, raw_bits: bool = False) -> torch.Tensor:
    """Payload drawn on `device` with a torch generator seeded by (seed, buffer_id)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + buffer_id)
    elem = torch.empty((), dtype=dtype).element_size()
    if int(np.prod(shape)) == 0:
        return torch.empty(shape, dtype=dtype, device=device)
    if raw_bits or dtype not in _FLOATS:
        n = int(np.prod(shape)) * elem
        raw = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=gen, device=device)
        if dtype == torch.bool:
            raw &= 1
        return raw.view(dtype).reshape(shape)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    step = 1 << 26
    for i in range(0, flat.numel(), step):  # bounded fp32 temporaries
        m = min(step, flat.numel() - i)
        tmp = torch.rand(m, generator=gen, device=device, dtype=torch.float32)
        flat[i:i + m] = (tmp * 2.0 - 1.0).to(dtype)
    return out


# --------------------------------------------------------------------------
# workload descriptions (host draws of everything except large payloads)
# --------------------------------------------------------------------------

@dataclass
class ScatterCase:
    name: str
    shape: tuple            # past / present shape
    seq_len: int            # S (update's size on axis)
    axis: int
    mode: str               # "linear" | "circular"
    dtype: torch.dtype
    write_indices: np.ndarray | None  # int64 [shape[0]] or None
    seed: int
    buffer_id: int = 0

    @property
    def update_shape(self):
        s = list(self.shape)
        s[self.axis] = self.seq_len
        return tuple(s)


@dataclass
class WindowCase:
    name: str
    batch: int
    kv_heads: int
    capacity: int
    seq_len: int
    head_dim: int
    dtype: torch.dtype
    seqlens_k: np.ndarray   # int32 [batch]
    seed: int
    buffer_id: int = 0


@dataclass
class ModelStep:
    """Workload 5: windowed layers (even) and full TensorScatter layers (odd)."""
    layers: int
    batch: int
    kv_heads: int
    head_dim: int
    window: int
    max_seq: int
    dtype: torch.dtype
    total_lens: np.ndarray          # T, int64 [batch]
    seqlens_k: np.ndarray           # T - 1, int32 [batch]
    write_indices: np.ndarray       # T - 1, int64 [batch]
    seed: int
    windowed_layers: list = field(default_factory=list)
    full_layers: list = field(default_factory=list)
    # fused append (new rows in new_dtype; caches in dtype), else None
    new_dtype: torch.dtype | None = None
    rotary_dim: int = 0
    rope_positions: int = 0
    k_scale: float = 1.0
    v_scale: float = 1.0
    # decode attention over the windowed layers (0: none)
    q_heads: int = 0


def workload1() -> ScatterCase:
    g = rng(1)
    w = g.integers(0, 13, endpoint=True, size=2).astype(np.int64)
    return ScatterCase("tensor_scatter_linear_fp32_2x2x16x8_s3", (2, 2, 16, 8), 3, 2,
                       "linear", torch.float32, w, seed=1)


def payload(shape, dtype: torch.dtype, seed: int, buffer_id: int, device="cpu",
            raw_bits: bool = False) -> torch.Tensor:
    """Payload for buffer `buffer_id` of workload `seed`: drawn on the host from
    PCG64(seed * 1000 + buffer_id) when device is the CPU, else on the device."""
    if torch.device(device).type == "cpu":
        return host_payload(rng(seed * 1000 + buffer_id), shape, dtype, raw_bits)
    return device_payload(shape, dtype, seed, buffer_id, device, raw_bits)


def scatter_payloads(case: ScatterCase, device="cpu", raw_bits: bool = False):
    """(past, update) of a TensorScatter case."""
    past = payload(case.shape, case.dtype, case.seed, 10 * case.buffer_id, device, raw_bits)
    upd = payload(case.update_shape, case.dtype, case.seed, 10 * case.buffer_id + 1, device,
                  raw_bits)
    return past, upd


def window_payloads(case: WindowCase, device="cpu", raw_bits: bool = False,
                    staging: bool = False):
    """(k_cache, v_cache, k_new, v_new[, k_staging, v_staging]) of a windowed case."""
    B, H, C, S, D = case.batch, case.kv_heads, case.capacity, case.seq_len, case.head_dim
    base = 10 * case.buffer_id
    out = [payload((B, H, C, D), case.dtype, case.seed, base + 0, device, raw_bits),
           payload((B, H, C, D), case.dtype, case.seed, base + 1, device, raw_bits),
           payload((B, H, S, D), case.dtype, case.seed, base + 2, device, raw_bits),
           payload((B, H, S, D), case.dtype, case.seed, base + 3, device, raw_bits)]
    if staging:
        out += [payload((B, H, C + S, D), case.dtype, case.seed, base + 4, device, raw_bits),
                payload((B, H, C + S, D), case.dtype, case.seed, base + 5, device, raw_bits)]
    return tuple(out)


def workload2() -> tuple[ScatterCase, ScatterCase]:
    g = rng(2)
    wa = g.integers(0, 4096, size=8).astype(np.int64)
    wb = g.integers(0, 4096, size=8).astype(np.int64)
    shape = (8, 8, 4096, 128)
    a = ScatterCase("tensor_scatter_circular_bf16_8x8x4096x128_s1", shape, 1, 2,
                    "circular", torch.bfloat16, wa, seed=2, buffer_id=1)
    b = ScatterCase("tensor_scatter_circular_bf16_8x8x4096x128_s512", shape, 512, 2,
                    "circular", torch.bfloat16, wb, seed=2, buffer_id=2)
    return a, b


def workload3() -> WindowCase:
    g = rng(3)
    sk = g.integers(1, 8192, endpoint=True, size=32).astype(np.int32)
    return WindowCase("window_decode_bf16_32x8x128x64_s1", 32, 8, 128, 1, 64,
                      torch.bfloat16, sk, seed=3)


def workload4() -> tuple[WindowCase, np.ndarray]:
    g = rng(4)
    past = g.integers(0, 16384, endpoint=True, size=4).astype(np.int64)
    sk = (past + 255).astype(np.int32)
    return (WindowCase("window_stage_bf16_4x8x4096x128_s256", 4, 8, 4096, 256, 128,
                       torch.bfloat16, sk, seed=4), past)


def workload5(dtype: torch.dtype = torch.bfloat16) -> ModelStep:
    g = rng(5)
    T = g.integers(1, 8192, endpoint=True, size=64).astype(np.int64)
    step = ModelStep(layers=24, batch=64, kv_heads=8, head_dim=64, window=128, max_seq=8192,
                     dtype=dtype, total_lens=T, seqlens_k=(T - 1).astype(np.int32),
                     write_indices=(T - 1).astype(np.int64), seed=5)
    step.windowed_layers = [i for i in range(24) if i % 2 == 0]
    step.full_layers = [i for i in range(24) if i % 2 == 1]
    return step


def workload7() -> ModelStep:
    step = workload5(torch.int8)
    step.seed = 7
    step.new_dtype = torch.bfloat16
    step.rotary_dim = 64
    step.rope_positions = 8192
    step.k_scale, step.v_scale = 0.02, 0.01
    return step


def workload8() -> ModelStep:
    step = workload5(torch.bfloat16)
    step.seed = 8
    step.q_heads = 64
    return step


def rope_tables(positions: int, rotary_dim: int, base: float = 10000.0, device="cpu"):
    """Rotary tables (inputs of the fused append): cos and sin of
    p * base^(-2j / rotary_dim) for p < positions, j < rotary_dim / 2,
    evaluated in float64 and stored as float32 [positions, rotary_dim / 2]."""
    j = np.arange(rotary_dim // 2)
    ang = np.arange(positions)[:, None] * base ** (-2.0 * j / rotary_dim)[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)).to(device),
            torch.from_numpy(np.sin(ang).astype(np.float32)).to(device))


def stratified_seqlens(g: np.random.Generator, batch: int, capacity: int, seq_len: int,
                       hi: int = 8192) -> np.ndarray:
    """seqlens_k with both regimes forced: half the entries leave the window
    partly filled (total length <= capacity), half make it full."""
    lo_part = g.integers(seq_len - 1, max(seq_len - 1, capacity - 1), endpoint=True,
                         size=batch // 2)
    hi_part = g.integers(capacity, hi, endpoint=True, size=batch - batch // 2)
    sk = np.concatenate([lo_part, hi_part])
    g.shuffle(sk)
    return sk.astype(np.int32)


# ---------------------------------------------------------------------------
# paged caches
# ---------------------------------------------------------------------------
# bits per element of each page format, by its C-ABI value (layout only: what a
# page occupies; the formats' arithmetic lives in the kernels and the oracle)
FORMAT_BITS = {1: 32, 2: 16, 3: 16, 4: 8, 5: 8, 6: 4, 7: 4, 8: 2, 9: 2}
_DENSE = {1: torch.float32, 2: torch.float16, 3: torch.bfloat16}
PAGE_FIELDS = ("start", "length", "capacity", "k_offset", "v_offset", "k_format", "v_format",
               "k_scale", "v_scale", "k_zero_point", "v_zero_point")


@dataclass
class PagedCase:
    """Streams of pages in one arena: descriptor fields as arrays (one entry per
    page, in arena order), each stream's page ids in token order (CSR), and the
    arena bytes."""
    head_dim: int
    fields: dict
    page_ptr: np.ndarray
    page_ids: np.ndarray
    arena: np.ndarray
    free_offset: int  # first byte past every page payload (spare room follows)

    @property
    def n_pages(self) -> int:
        return len(self.fields["start"])

    def totals(self) -> np.ndarray:
        """Tokens per stream (the sum of its pages' lengths)."""
        out = np.zeros(len(self.page_ptr) - 1, np.int64)
        for s in range(len(out)):
            ids = self.page_ids[self.page_ptr[s]:self.page_ptr[s + 1]]
            out[s] = int(self.fields["length"][ids].sum())
        return out


def paged_case(g: np.random.Generator, head_dim: int, streams, page_format, *,
               spare_bytes: int = 0, align: int = 16,
               payload_rng: np.random.Generator | None = None) -> PagedCase:
    """A paged cache: ``streams`` lists, per stream, its pages as (length,
    capacity) in token order; ``page_format(stream, page, n_pages)`` gives a
    page's (k_format, v_format, k_scale, v_scale, k_zero_point, v_zero_point).
    Pages sit in the arena in a shuffled order at ``align``-byte offsets; dense
    payloads hold U[-1, 1) values rounded to their type, affine payloads
    uniform random bytes (every row of the capacity is filled, valid or not),
    drawn from ``payload_rng`` when given (the same layout with other bytes)."""
    recs = []
    for s, pages in enumerate(streams):
        start = 0
        for i, (length, cap) in enumerate(pages):
            kf, vf, ks, vs, kz, vz = page_format(s, i, len(pages))
            recs.append(dict(stream=s, index=i, start=start, length=length, capacity=cap,
                             k_format=kf, v_format=vf, k_scale=ks, v_scale=vs,
                             k_zero_point=kz, v_zero_point=vz))
            start += length
    order = g.permutation(len(recs))
    off = 0
    chunks = []
    pg = g if payload_rng is None else payload_rng

    def place(fmt, cap):
        nonlocal off
        nbytes = cap * head_dim * FORMAT_BITS[fmt] // 8
        o = off
        if fmt in _DENSE:
            vals = torch.from_numpy(pg.uniform(-1, 1, size=cap * head_dim).astype(np.float32))
            raw = vals.to(_DENSE[fmt]).view(torch.uint8).numpy()
        else:
            raw = pg.integers(0, 256, size=nbytes, dtype=np.uint8)
        chunks.append((o, raw))
        off += -(-nbytes // align) * align
        return o

    for j in order:
        r = recs[j]
        r["k_offset"] = place(r["k_format"], r["capacity"])
        r["v_offset"] = place(r["v_format"], r["capacity"])
    arena = np.zeros(off + spare_bytes, np.uint8)
    for o, raw in chunks:
        arena[o:o + len(raw)] = raw
    placed = [recs[j] for j in order]  # descriptor i is the i-th page in the arena
    fields = {f: np.array([r[f] for r in placed],
                          dtype=np.float32 if f.endswith("scale") else np.int64)
              for f in PAGE_FIELDS}
    ptr = np.zeros(len(streams) + 1, np.int32)
    ids = []
    for s, pages in enumerate(streams):
        mine = sorted((r["index"], i) for i, r in enumerate(placed) if r["stream"] == s)
        ids.extend(i for _, i in mine)
        ptr[s + 1] = len(ids)
    return PagedCase(head_dim, fields, ptr, np.array(ids, np.int32), arena, off)


def page_split(g: np.random.Generator, tokens: int, capacity: int, sealed: float = 0.0):
    """Pages of ``capacity`` rows holding ``tokens`` tokens in order: full pages,
    except that with probability ``sealed`` a page is closed early (a sealed
    partial page) and the last page holds the remainder."""
    pages, left = [], tokens
    while left > 0:
        n = min(left, capacity)
        if sealed and n > 1 and g.random() < sealed:
            n = int(g.integers(1, n))
        pages.append((n, capacity))
        left -= n
    return pages


@dataclass
class PagedStep:
    """A decode step over paged caches: every layer's streams (batch entry,
    KV head) hold T tokens of their batch entry in pages of ``block`` tokens,
    contiguous from zero; one block table serves every layer (each layer its
    own arena). The last ``hot_pages`` pages of a stream are ``hot_format``,
    older ones ``cold_format`` with scales ``k_scale`` / ``v_scale`` and zero
    points 0. Pages the window never reaches keep descriptors but share one
    placeholder payload (nothing reads it), so the arena holds only what the
    window can see."""
    layers: int
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    block: int
    left_window: int
    total_lens: np.ndarray
    hot_pages: int = 2
    hot_format: int = 3      # bf16
    cold_format: int = 4     # int8
    k_scale: float = 0.02
    v_scale: float = 0.01
    seed: int = 9


def workload9() -> PagedStep:
    g = rng(9)
    T = g.integers(1, 8192, endpoint=True, size=64).astype(np.int64)
    return PagedStep(layers=12, batch=64, kv_heads=8, q_heads=64, head_dim=64, block=16,
                     left_window=127, total_lens=T)


def paged_step_layout(step: PagedStep, align: int = 16):
    """Descriptor fields, page_ptr, page_ids and the arena size of a PagedStep
    (stream-major page order). Returns (fields, page_ptr, page_ids,
    arena_bytes, visible_pages)."""
    D, blk = step.head_dim, step.block
    rows = {f: blk * D * FORMAT_BITS[f] // 8 for f in (step.hot_format, step.cold_format)}
    placeholder = -(-max(rows.values()) // align) * align
    off = placeholder  # [0, placeholder): the shared payload of unreachable pages
    cols = {f: [] for f in PAGE_FIELDS}
    ptr = [0]
    visible = 0
    for b in range(step.batch):
        T = int(step.total_lens[b])
        n = -(-T // blk)
        r0 = max(0, T - 1 - step.left_window) if step.left_window >= 0 else 0
        first_visible = r0 // blk
        for _g in range(step.kv_heads):
            for i in range(n):
                start, length = i * blk, min(blk, T - i * blk)
                fmt = step.hot_format if i >= n - step.hot_pages else step.cold_format
                affine = fmt not in _DENSE
                if i >= first_visible:
                    ko = off
                    off += -(-rows[fmt] // align) * align
                    vo = off
                    off += -(-rows[fmt] // align) * align
                    visible += 1
                else:
                    ko = vo = 0
                for f, v in (("start", start), ("length", length), ("capacity", blk),
                             ("k_offset", ko), ("v_offset", vo), ("k_format", fmt),
                             ("v_format", fmt), ("k_scale", step.k_scale if affine else 1.0),
                             ("v_scale", step.v_scale if affine else 1.0), ("k_zero_point", 0),
                             ("v_zero_point", 0)):
                    cols[f].append(v)
            ptr.append(len(cols["start"]))
    fields = {f: np.array(v, dtype=np.float32 if f.endswith("scale") else np.int64)
              for f, v in cols.items()}
    n_pages = len(fields["start"])
    return fields, np.array(ptr, np.int32), np.arange(n_pages, dtype=np.int32), off, visible
