"""Benchmark: KV-cache update effective HBM GB/s and us per decode step.

Workload (one "step"): the KV-cache updates of one whole-model decode step of a
24-layer model whose even layers use a windowed cache (K/V [64, 8, 128, 64],
capacity 128) and whose odd layers use a full linear cache updated by
TensorScatter (K/V [64, 8, 8192, 64]); batch 64, 8 KV heads, head_dim 64, total
lengths T ~ U{1..8192} shared by all layers; bf16 (or --dtype fp8_e4m3fn).
A step is one launch of kv_decode_step (default), or with --form three the
three-call composition: kv_seq_lengths, kv_window_append_layers (all 12
windowed layers, in place) and tensor_scatter_batched (all 24 full caches).
Both forms are timed in every run; --form picks the one `value` reports.
--workload 7 is the same step with the fused append: bf16 new rows, K rotated
at its absolute position, int8 caches (kv_decode_step_xf, or the three xf
calls).

Measurement
  - value: algorithmic bytes of a step / time of a step, from K steps bracketed
    by torch.cuda.synchronize(), issued eagerly with arguments marshalled once
    (with --timing graph: replayed as one HIP graph per buffer set; on this
    ROCm a graph launch costs a few microseconds more than a kernel launch).
  - Infinity Cache: every buffer set is independent and --sets sets (default
    3, over 512 MB of windowed caches touched between two uses of one set)
    are visited round robin, so no step finds its data in the 256 MB cache.
  - roofline: the dominant kernel (the one-launch step; with --form three the
    window shift + append of the 12 layers) launched back to back (buffer sets
    round robin) in blocks, each between one pair of HIP events on the launch
    stream; achieved = its algorithmic bytes / its median launch duration.
  - every time is the median over blocks of steps (up to 10 blocks of at
    least 20 steps; one block when K < 40).
  - cpu_baseline: the CPU oracle on the same step, host copies of the same
    inputs, for a bounded time: on every host core this process may use
    (independent (layer, batch chunk) slices on a thread pool; `value`), and
    on one thread; with the CPU model.

One JSON line on stdout; progress on stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published peak

# HBM bytes per launch of the dominant kernel from two rocprofv3 counter passes
# (FETCH_SIZE, WRITE_SIZE), each scaled by what the counter reads for a 1 GiB
# copy; valid only for the kernel source they were taken on (its hash).
MEASURED_TRAFFIC = {
    ("bf16", "decode_step_kernel", "7c60268bc4021eab"): {"read": 196_791_383,
                                                         "written": 196_860_370},
    ("fp8_e4m3fn", "decode_step_kernel", "7c60268bc4021eab"): {"read": 99_418_076,
                                                               "written": 98_589_539},
    ("bf16->int8", "decode_step_kernel", "7c60268bc4021eab"): {"read": 101_391_803,
                                                               "written": 98_796_627},
    ("bf16", "window_in_place", "7baab05ee8cf426a"): {"read": 195_192_247, "written": 196_015_224},
    ("bf16", "window_attention_mfma", "3277255b340464c2"): {"read": 202_197_650,
        "written": 6_291_431},
    ("bf16+int8", "paged_attention_kernel", "2558684f894e20c2"): {"read": 127_909_170,
        "written": 6_291_448},
}
_CSRC = "sliding_window_ring_tensor_amd/csrc/"
KERNEL_SOURCES = {
    "window_in_place": ("kv_window.hip", "window_device.hpp", "xf_device.hpp", "swrt_device.hpp"),
    "decode_step_kernel": ("decode_step.hip", "window_device.hpp", "scatter_device.hpp",
                           "xf_device.hpp", "swrt_device.hpp"),
    "paged_attention_kernel": ("paged.hip", "att_device.hpp", "xf_device.hpp", "swrt_device.hpp",
                               "../build.py"),
    # the attention kernel's code also depends on a code-generation flag of the build
    "window_attention_mfma": ("window_attention.hip", "att_device.hpp", "xf_device.hpp",
                              "swrt_device.hpp", "../build.py"),
}


def kernel_source_hash(kernel: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, _CSRC + rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_threads() -> int:
    """The host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(step, seconds: float, threads: int = 1):
    """The oracle as it stands on host copies of buffer set 0: one step is the
    oracle's lengths call, then its windowed step on every windowed layer and
    its TensorScatter on every full cache. With threads > 1 the independent
    (windowed layer, batch chunk) slices, and per batch chunk the full caches'
    scatters, are spread over a pool of host threads (the oracle's ctypes calls
    release the interpreter lock): the batch partition of the CPU follow-up's
    thread-pool MoveKvCacheRows."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    orc = oracle.get()
    spec, b = step.spec, step.buffers
    D, H = spec.head_dim, spec.kv_heads

    def host(t):
        return t.detach().cpu().contiguous().view(torch.uint8).numpy()

    wk = [host(t).copy() for t in b.win_k]
    wv = [host(t).copy() for t in b.win_v]
    wkn, wvn = [host(t) for t in b.win_kn], [host(t) for t in b.win_vn]
    row = D * torch.empty((), dtype=spec.dtype).element_size()
    # full caches: only the written rows are ever touched; their prior content
    # does not change the oracle's work, so they are left uninitialised
    nf = len(spec.full_layers)
    full = [np.empty((spec.batch, H, spec.max_seq, row), np.uint8) for _ in range(2 * nf)]
    fnew = [host(t) for t in b.full_kn + b.full_vn]
    sk, wi = spec.seqlens_k, spec.write_indices
    xo = None
    if b.xf is not None:  # the fused append's transform, as the oracle takes it
        types = {torch.bfloat16: oracle.XF_BF16, torch.float16: oracle.XF_F16,
                 torch.float32: oracle.XF_F32, torch.int8: oracle.XF_INT8,
                 torch.uint8: oracle.XF_UINT8}
        x = b.xf
        xo = oracle.Transform(types[spec.new_dtype], types[spec.dtype],
                              None if x.cos is None else x.cos.cpu().numpy(),
                              None if x.sin is None else x.sin.cpu().numpy(),
                              0 if x.cos is None else 2 * x.cos.shape[1], x.interleaved,
                              (x.k_scale, x.v_scale), (x.k_zero_point, x.v_zero_point))
    bits = row * 8 // D
    # about two parts per thread: each windowed layer split into a few batch
    # chunks, and every full cache's (cheap) scatter of one chunk in one part;
    # finer parts cost more in pool hand-offs than they gain
    chunks = max(1, min(spec.batch, -(-2 * threads // max(1, len(wk))))) if threads > 1 else 1
    edges = [spec.batch * c // chunks for c in range(chunks + 1)]

    def window_part(i, b0, b1, L):
        if xo is None:
            orc.kv_window_append_strided(wk[i][b0:b1], wv[i][b0:b1], wkn[i][b0:b1],
                                         wvn[i][b0:b1], (H * D, D, D), 1, L.cache_past[b0:b1],
                                         L.evict[b0:b1], elem_bits=bits, head_dim=D)
        else:
            orc.kv_window_append_xf(xo, wk[i][b0:b1], wv[i][b0:b1], wkn[i][b0:b1],
                                    wvn[i][b0:b1], (H * D, D, D), 1, L.cache_past[b0:b1],
                                    L.evict[b0:b1], L.past[b0:b1])

    def full_part(b0, b1):
        for i in range(len(full)):
            c, u = full[i][b0:b1], fnew[i][b0:b1]
            if xo is None:
                orc.tensor_scatter_raw(c, c, u, wi[b0:b1], (b1 - b0, H, spec.max_seq, D), 2, 1,
                                       0, bits)
            else:
                orc.tensor_scatter_xf(xo, i // nf, c, c, u, wi[b0:b1])

    pool = ThreadPoolExecutor(max_workers=threads) if threads > 1 else None

    def one_step():
        L = orc.kv_seq_lengths(sk, 1, spec.window)
        parts = [(window_part, (i, edges[c], edges[c + 1], L)) for i in range(len(wk))
                 for c in range(chunks)]
        parts += [(full_part, (edges[c], edges[c + 1])) for c in range(chunks)]
        if pool is None:
            for fn, a in parts:
                fn(*a)
        else:
            for f in [pool.submit(fn, *a) for fn, a in parts]:
                f.result()

    try:
        return _time_steps(one_step, seconds)
    finally:
        if pool is not None:
            pool.shutdown()


def _time_steps(one_step, seconds: float):
    """One untimed step (the host pages of the written rows are mapped on
    first touch), then steps until `seconds` have passed."""
    one_step()
    n, t0 = 0, time.perf_counter()
    while True:
        one_step()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return n, el


def _reps(K: int) -> int:
    """Timed blocks per measurement: blocks of at least 20 steps (a block's
    first launch and its closing synchronization stay a small share), up to
    10 of them, whose median is reported."""
    return max(1, min(10, K // 20))


def _median(xs):
    return float(np.median(np.asarray(xs)))


def _timers(stream, K, W):
    """eager wall clock, event-timed device time and graph replay of fn(set),
    each a list of per-step times, one per block of K // _reps(K) steps."""
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    torch.cuda._sleep(1_000_000)
    s1.record(stream)
    torch.cuda.synchronize()
    cycles_per_s = 1_000_000 / (s0.elapsed_time(s1) * 1e-3)
    R = _reps(K)
    n = K // R

    def eager(fn, n_sets):
        for i in range(W):
            fn(i % n_sets)
        torch.cuda.synchronize()
        out = []
        for r in range(R):
            t0 = time.perf_counter()
            for i in range(n):
                fn((r * n + i) % n_sets)
            torch.cuda.synchronize()
            out.append((time.perf_counter() - t0) / n)
        return out

    def device(fn, n_sets, host_s):
        out = []
        for r in range(R):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(int(cycles_per_s * min(2.0, 2.0 * n * host_s + 0.05)))
            a.record(stream)
            for i in range(n):
                fn((r * n + i) % n_sets)
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) * 1e-3 / n)
        return out

    def graph(fn, n_sets):
        graphs = []
        for i in range(n_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                fn(i)
            graphs.append(g)
        for i in range(W):
            graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        out = []
        for r in range(R):
            t0 = time.perf_counter()
            for i in range(n):
                graphs[(r * n + i) % n_sets].replay()
            torch.cuda.synchronize()
            out.append((time.perf_counter() - t0) / n)
        return out

    return eager, device, graph


def other_workload(args, dev):
    """Workloads 1-4: same timing method as the decode step, one JSON line."""
    import sliding_window_ring_tensor_amd as swrt
    from sliding_window_ring_tensor_amd import workloads as wl

    K, W, n = args.steps, args.warmup, args.workload
    sets, calls, desc = [], [], ""
    if n in (1, 2):
        cases = [wl.workload1()] if n == 1 else list(wl.workload2())
        c0 = cases[0]
        es = torch.empty((), dtype=c0.dtype).element_size()
        row = int(np.prod(c0.shape[c0.axis + 1:])) * es
        O = int(np.prod(c0.shape[:c0.axis]))
        step_bytes = sum(2 * O * c.seq_len * row for c in cases)
        touched = step_bytes
        n_sets = 64 if n == 1 else int(np.ceil(512e6 / touched)) + 1
        for k in range(n_sets):
            cache = wl.payload(c0.shape, c0.dtype, c0.seed, 1000 + 10 * k, dev)
            seq = []
            for c in cases:
                upd = wl.payload(c.update_shape, c.dtype, c.seed, 1000 + 10 * k + 1 + c.buffer_id, dev)
                wi = torch.from_numpy(c.write_indices).to(dev)
                seq.append(swrt.prepare_tensor_scatter(cache, upd, wi, axis=c.axis, mode=c.mode,
                                                       out=cache))
            calls.append(seq)
        desc = " then ".join(c.name for c in cases)
    elif n == 3:
        c = wl.workload3()
        es = torch.empty((), dtype=c.dtype).element_size()
        row = c.head_dim * es
        T = c.seqlens_k.astype(np.int64) + 1
        Lp = np.minimum(T - 1, c.capacity)
        E = np.maximum(0, Lp + 1 - c.capacity)
        step_bytes = int((2 * row * (E * (Lp - E) + 1)).sum()) * c.kv_heads * 2
        n_sets = int(np.ceil(512e6 / step_bytes)) + 1
        for k in range(n_sets):
            c.buffer_id = 10 + k
            kc, vc, kn, vn = wl.window_payloads(c, device=dev)
            sk = torch.from_numpy(c.seqlens_k).to(dev)
            calls.append([swrt.prepare_kv_decode_step([kc], [vc], [kn], [vn], sk, [], [], None)])
        desc = c.name + " (lengths + shift/append in one launch)"
    else:
        c, _ = wl.workload4()
        es = torch.empty((), dtype=c.dtype).element_size()
        row = c.head_dim * es
        T = c.seqlens_k.astype(np.int64) + 1
        S, C = c.seq_len, c.capacity
        Lp = np.minimum(np.maximum(T - S, 0), C)
        E = np.maximum(0, Lp + S - C)
        L = Lp + S - E
        stage = 2 * row * (Lp + S)
        commit = 2 * row * np.where(E > 0, L, S)
        step_bytes = int((stage + commit).sum()) * c.kv_heads * 2
        n_sets = int(np.ceil(512e6 / step_bytes)) + 1
        for k in range(n_sets):
            c.buffer_id = 10 + k
            kc, vc, kn, vn, ks, vs = wl.window_payloads(c, device=dev, staging=True)
            sk = torch.from_numpy(c.seqlens_k).to(dev)
            lens = swrt.kv_seq_lengths(sk, S, C)
            calls.append([swrt.prepare_kv_window_stage_step([kc], [vc], [kn], [vn], sk, [ks], [vs],
                                                            out=lens),
                          swrt.prepare_kv_window_append_layers(
                              [kc], [vc], [kn], [vn], lens.cache_past, lens.evict,
                              k_stagings=[ks], v_stagings=[vs], phase="commit")])
        desc = c.name + " (lengths and stage in one launch, then commit: two launches)"
    torch.cuda.synchronize()

    def step(i):
        for call in calls[i]:
            call()

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        eager, device, graph = _timers(stream, K, W)
        t0 = time.perf_counter()
        for i in range(W):
            step(i % len(calls))
        torch.cuda.synchronize()
        host_s = (time.perf_counter() - t0) / max(W, 1)
        eager_v = eager(step, len(calls))
        device_v = device(step, len(calls), host_s)
        graph_v = graph(step, len(calls))
        parts = {}
        if n == 2:  # each TensorScatter step of the workload on its own
            for j, c in enumerate(cases):
                pb = 2 * O * c.seq_len * row
                dv = device(lambda i, j=j: calls[i][j](), len(calls), host_s)
                ds = _median(dv)
                parts[c.name] = {"bytes": pb, "device_us": round(ds * 1e6, 3),
                                 "device_gbs": round(pb / ds / 1e9, 1),
                                 "device_pct_of_hbm_peak": round(100 * pb / ds / 1e9 / HBM_PEAK_GBS,
                                                                 2)}
    eager_s, device_s, graph_s = _median(eager_v), _median(device_v), _median(graph_v)
    out = {
        "metric": "KV-cache update effective HBM GB/s (% of peak) and us per decode step",
        "value": round(step_bytes / eager_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(eager_s * 1e3, 5),
        "us_per_step": round(eager_s * 1e6, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": str(c0.dtype if n in (1, 2) else c.dtype).replace("torch.", ""),
        "data": "synthetic",
        "config": {"workload": f"workload {n}: {desc}", "bytes_per_step": step_bytes,
                   "cache_defeat": f"{len(calls)} independent buffer sets round robin"},
        "device_us_per_step": round(device_s * 1e6, 3),
        "device_gbs": round(step_bytes / device_s / 1e9, 1),
        "device_pct_of_hbm_peak": round(100 * step_bytes / device_s / 1e9 / HBM_PEAK_GBS, 2),
        "graph_us_per_step": round(graph_s * 1e6, 2),
        "timing": f"medians of {len(eager_v)} blocks of {args.steps // len(eager_v)} steps",
    }
    if parts:
        out["steps_alone"] = parts
    print(json.dumps(out))


def drift_loop(args, dev):
    """Workload 6: K consecutive decode steps of workload 5's model, T
    advancing by one per step, windowed caches of capacity W + slack under the
    drifting layout, against the same loop at capacity W (compaction every
    step). Bytes come from the lengths the kernels returned."""
    import sliding_window_ring_tensor_amd as swrt
    from sliding_window_ring_tensor_amd import workloads as wl

    spec = wl.workload5(wl.DTYPES[args.dtype])
    K, W, n_sets = args.steps, args.warmup, 3
    B, H, D, Wn, M = spec.batch, spec.kv_heads, spec.head_dim, spec.window, spec.max_seq
    es = torch.empty((), dtype=spec.dtype).element_size()
    row = D * es
    nw, nf = len(spec.windowed_layers), len(spec.full_layers)
    steps_per_set = (K + W) // n_sets + 2
    res = {}
    for label, cap in (("drift", Wn + args.slack), ("base", Wn)):
        log(f"{label}: capacity {cap}, window {Wn}")
        calls, outs = [], []
        for i in range(n_sets):
            seed = spec.seed * 100 + 50 + i
            buf = lambda shape, bid: wl.payload(shape, spec.dtype, seed, bid, dev)  # noqa: E731
            wk = [buf((B, H, cap, D), 10 * j) for j in range(nw)]
            wv = [buf((B, H, cap, D), 10 * j + 1) for j in range(nw)]
            wkn = [buf((B, H, 1, D), 10 * j + 2) for j in range(nw)]
            wvn = [buf((B, H, 1, D), 10 * j + 3) for j in range(nw)]
            fc = [buf((B, H, M, D), 1000 + j) for j in range(2 * nf)]
            fn = [buf((B, H, 1, D), 2000 + j) for j in range(2 * nf)]
            # set i's j-th step appends token T0 + j (T0 the drawn lengths, kept below M)
            T0 = np.minimum(spec.total_lens, M - steps_per_set)
            Ts = T0[None, :] + np.arange(steps_per_set)[:, None]
            sk = torch.from_numpy((Ts - 1).astype(np.int32)).to(dev)
            wi = torch.from_numpy((Ts - 1).astype(np.int64)).to(dev)
            lens = [swrt.WindowLengths(*(torch.zeros(B, dtype=t, device=dev) for t in (
                torch.int64, torch.int64, torch.int32, torch.int32, torch.int32)))
                for _ in range(steps_per_set)]
            calls.append([swrt.prepare_kv_decode_step(wk, wv, wkn, wvn, sk[j], fc, fn, wi[j],
                                                      window=Wn, out=lens[j])
                          for j in range(steps_per_set)])
            outs.append(lens)
        torch.cuda.synchronize()
        order = [(k % n_sets, k // n_sets) for k in range(W + K)]
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for s_, j in order[:W]:
                calls[s_][j]()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s_, j in order[W:]:
                calls[s_][j]()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / K
        byts = 0
        for s_, j in order[W:]:
            L = outs[s_][j]
            Lp = L.cache_past.cpu().numpy().astype(np.int64)
            E = L.evict.cpu().numpy().astype(np.int64)
            byts += int((2 * row * (np.where(E > 0, Lp - E, 0) + 1)).sum()) * H * 2 * nw
            byts += 2 * row * B * H * 2 * nf
        compactions = sum(int((outs[s_][j].evict > 0).sum().item()) for s_, j in order[W:])
        res[label] = {"capacity": cap, "us_per_step": wall * 1e6, "bytes_per_step": byts / K,
                      "compacting_entries_per_step": compactions / K}
        del calls, outs
        torch.cuda.empty_cache()
    d, b = res["drift"], res["base"]
    out = {
        "metric": "KV-cache update effective HBM GB/s (% of peak) and us per decode step",
        "value": round(d["bytes_per_step"] / d["us_per_step"] / 1e3, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(d["us_per_step"] / 1e3, 5),
        "us_per_step": round(d["us_per_step"], 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"workload 6: workload 5's decode loop, {K} consecutive steps, "
                               f"windowed caches C = {d['capacity']} = W + {args.slack} under "
                               f"the drifting layout (gap {d['capacity'] - Wn + 1})",
                   "cache_defeat": f"{n_sets} independent buffer sets round robin"},
        "drift": {k: round(v, 3) for k, v in d.items()},
        "base_layout_same_loop": {k: round(v, 3) for k, v in b.items()},
        "speedup_vs_base_layout": round(b["us_per_step"] / d["us_per_step"], 3),
    }
    print(json.dumps(out))


def copy_reference(dev, stream):
    """Achievable reference: 1 GiB device-to-device copies (GB/s moved), by
    torch and by the library's own copy engine (TensorScatter out of place,
    S = 0, which is also the counters' calibration kernel)."""
    import sliding_window_ring_tensor_amd as swrt

    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)

    def copy_gbs(fn, n=10):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return 2 * (1 << 30) * n / (a.elapsed_time(b) * 1e-3) / 1e9

    torch_copy = copy_gbs(lambda: dst.copy_(src))
    s3, d3 = src.view(1, 1 << 26, 16), dst.view(1, 1 << 26, 16)
    swrt_copy = copy_gbs(lambda: swrt.tensor_scatter(s3, s3[:, :0], None, axis=1, out=d3))
    del src, dst, s3, d3
    return torch_copy, swrt_copy


def attention_bench(args, dev):
    """Workload 8: decode attention over the 12 windowed layers of the model
    step (window_attention, one launch), after the step's append; K launches
    round robin over the buffer sets."""
    import oracle
    import sliding_window_ring_tensor_amd as swrt  # noqa: F401
    from sliding_window_ring_tensor_amd import workloads as wl
    from sliding_window_ring_tensor_amd.decode_step import ModelDecodeStep

    spec = wl.workload8()
    K, W = args.steps, args.warmup
    log(f"allocating {args.sets} buffer sets ...")
    steps = [ModelDecodeStep(spec, dev, set_id=i) for i in range(args.sets)]
    for st in steps:  # the step's append writes the windows and their lengths
        st.run_fused()
    torch.cuda.synchronize()
    byts = steps[0].attention_bytes()
    stream = torch.cuda.Stream()
    eager, device, _ = _timers(stream, K, W)
    with torch.cuda.stream(stream):
        log(f"timing {K} attention launches ...")
        att_s = _median(eager(lambda i: steps[i].attention(), len(steps)))
        att_dev = _median(device(lambda i: steps[i].attention(), len(steps), att_s))
        log(f"timing {K} steps of append + attention ...")
        both_s = _median(eager(lambda i: (steps[i].run_fused(), steps[i].attention()),
                               len(steps)))
        torch_copy, swrt_copy = copy_reference(dev, stream)
    flags = [int(st.buffers.flags.item()) for st in steps]
    if any(flags):
        raise SystemExit(f"device flags raised during the benchmark: {flags}")
    value = byts / att_s / 1e9
    achieved = byts / att_dev / 1e9
    meas = MEASURED_TRAFFIC.get(("bf16", "window_attention_mfma",
                                 kernel_source_hash("window_attention_mfma")))
    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s ...")
        orc = oracle.get()
        b = steps[0].buffers

        def host(t):
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

        qs, ks, vs = ([host(t) for t in ts] for ts in (b.win_q, b.win_k, b.win_v))
        L = b.lengths.cache_total.cpu().numpy()

        def one_step():
            for q, k, v in zip(qs, ks, vs):
                orc.window_attention(q, k, v, L, spec.window, spec.head_dim ** -0.5,
                                     oracle.XF_BF16)

        n, el = _time_steps(one_step, args.cpu_seconds)
        cpu = {"value": round(byts * n / el / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{n} attention steps (12 layers) on host copies of buffer set 0, "
                         f"one thread, float64, {el:.1f} s",
               "us_per_step": round(el / n * 1e6, 1)}
    out = {
        "metric": "KV-cache update effective HBM GB/s (% of peak) and us per decode step",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(att_s * 1e3, 5), "us_per_step": round(att_s * 1e6, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"workload 8: decode attention over the {len(spec.windowed_layers)} "
                               f"windowed layers of the model step, B={spec.batch}, "
                               f"Hq={spec.q_heads}, Hkv={spec.kv_heads}, D={spec.head_dim}, "
                               f"C=W={spec.window}, lengths min(T, C) of T~U[1,8192] seed 8, "
                               f"bf16 in and out, fp32 softmax",
                   "bytes_per_step": byts,
                   "form": "one launch per step (window_attention, all windowed layers)",
                   "cache_defeat": f"{args.sets} independent buffer sets round robin"},
        "roofline": {"bound": "hbm", "kernel": "window_attention_mfma: 12 layers, one launch",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if meas is None else meas["read"] + meas["written"],
                     "bytes_per_launch": byts, "median_launch_us": round(att_dev * 1e6, 3)},
        "cpu_baseline": cpu,
        "append_plus_attention_us_per_step": round(both_s * 1e6, 2),
        "copy_reference_gbs": {"torch_copy": round(torch_copy, 1),
                               "swrt_tensor_scatter_copy": round(swrt_copy, 1)},
    }
    print(json.dumps(out))


def paged_bench(args, dev):
    """Workload 9: paged decode attention over 12 layers sharing one block
    table (int8 cold pages, bf16 hot pages, left window 127), one launch per
    step, K launches round robin over the buffer sets; then the cooling
    conversion of every stream's oldest hot page in one layer (in place)."""
    import oracle
    import sliding_window_ring_tensor_amd as swrt
    from sliding_window_ring_tensor_amd import workloads as wl
    from sliding_window_ring_tensor_amd.paged_step import PagedDecodeStep

    spec = wl.workload9()
    K, W = args.steps, args.warmup
    log(f"allocating {args.sets} buffer sets ...")
    steps = [PagedDecodeStep(spec, dev, set_id=i, spare_bytes=1 << 20) for i in range(args.sets)]
    torch.cuda.synchronize()
    byts = steps[0].attention_bytes()
    stream = torch.cuda.Stream()
    eager, device, _ = _timers(stream, K, W)
    with torch.cuda.stream(stream):
        log(f"timing {K} paged attention launches ...")
        att_s = _median(eager(lambda i: steps[i].attention(), len(steps)))
        att_dev = _median(device(lambda i: steps[i].attention(), len(steps), att_s))
        torch_copy, swrt_copy = copy_reference(dev, stream)
        # the cooling conversion, in place on copies of each set's table
        blocks, dst, conv_written = steps[0].cooling_selection()
        bl = torch.from_numpy(blocks).to(dev)
        ds = torch.from_numpy(dst).to(dev)
        tables = [st.caches[0].pages.clone() for st in steps]
        conv = [swrt.PagedCache(st.arenas[0], t, st.caches[0].page_ptr, st.caches[0].page_ids)
                for st, t in zip(steps, tables)]
        cflags = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in steps]

        def convert(i):
            tables[i].copy_(steps[i].caches[0].pages)  # the unconverted table again
            swrt.paged_quantize(conv[i], bl, ds, steps[i].layout_bytes,
                                steps[i].arenas[0].numel(), spec.cold_format, spec.k_scale, 0,
                                spec.cold_format, spec.v_scale, 0, spec.head_dim,
                                pages_out=tables[i], flags=cflags[i])
        log(f"timing {K} conversions ...")
        conv_s = _median(eager(convert, len(steps)))
    flags = [int(st.flags.item()) for st in steps] + [int(f.item()) for f in cflags]
    if any(flags):
        raise SystemExit(f"device flags raised during the benchmark: {flags}")
    value = byts / att_s / 1e9
    achieved = byts / att_dev / 1e9
    meas = MEASURED_TRAFFIC.get(("bf16+int8", "paged_attention_kernel",
                                 kernel_source_hash("paged_attention_kernel")))
    rows_bf16 = spec.block * spec.head_dim * 2
    conv_read = 2 * len(blocks) * rows_bf16 + steps[0].table_host.nbytes + 16 * len(blocks) + \
        4 * len(blocks)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s ...")
        orc = oracle.get()
        st = steps[0]
        arenas = [a.cpu().numpy() for a in st.arenas]
        qs = [q.cpu().view(torch.int16).numpy().view(np.uint16) for q in st.qs]
        tb = st.table_host.view(oracle.PAGE_DTYPE)

        def one_step():
            for a, q in zip(arenas, qs):
                orc.paged_attention(q, oracle.XF_BF16, a, tb, st.page_ptr_host, st.page_ids_host,
                                    spec.left_window, spec.kv_heads, spec.head_dim ** -0.5)

        n, el = _time_steps(one_step, args.cpu_seconds)
        cpu = {"value": round(byts * n / el / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"{n} paged attention steps (12 layers) on host copies of buffer set 0, "
                         f"one thread, float64, {el:.1f} s",
               "us_per_step": round(el / n * 1e6, 1)}
    out = {
        "metric": "KV-cache update effective HBM GB/s (% of peak) and us per decode step",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(att_s * 1e3, 5), "us_per_step": round(att_s * 1e6, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+int8", "data": "synthetic",
        "config": {"workload": f"workload 9: paged decode attention over {spec.layers} layers "
                               f"sharing one block table, B={spec.batch}, Hq={spec.q_heads}, "
                               f"Hkv={spec.kv_heads}, D={spec.head_dim}, pages of {spec.block} "
                               f"tokens ({steps[0].visible_pages} visible of "
                               f"{len(steps[0].page_ids_host)}), left window "
                               f"{spec.left_window}, T~U[1,8192] seed 9, cold pages int8 "
                               f"(scales {spec.k_scale}/{spec.v_scale}), last {spec.hot_pages} "
                               f"pages bf16, bf16 queries and outputs",
                   "bytes_per_step": byts,
                   "form": "one launch per step (paged_attention, all layers)",
                   "cache_defeat": f"{args.sets} independent buffer sets round robin"},
        "roofline": {"bound": "hbm", "kernel": "paged_attention_kernel: 12 layers, one launch",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if meas is None else meas["read"] + meas["written"],
                     "bytes_per_launch": byts, "median_launch_us": round(att_dev * 1e6, 3)},
        "cpu_baseline": cpu,
        "cooling_conversion": {"pages": int(len(blocks)), "us_per_call": round(conv_s * 1e6, 2),
                               "bytes_read": int(conv_read), "bytes_written": int(conv_written),
                               "form": "one layer, in place: validate the whole table, convert "
                                       "bf16 -> int8, publish the selected descriptors "
                                       "(plus a 10 MB table restore per call)"},
        "copy_reference_gbs": {"torch_copy": round(torch_copy, 1),
                               "swrt_tensor_scatter_copy": round(swrt_copy, 1)},
    }
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp8_e4m3fn"])
    ap.add_argument("--sets", type=int, default=3, help="independent buffer sets, round robin")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds of CPU oracle work per leg (all host cores, then one thread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--form", default="fused", choices=["fused", "three"],
                    help="one launch per step (default) or the three-call composition")
    ap.add_argument("--timing", default="eager", choices=["eager", "graph"],
                    help="the timed loop `value` reports (both are measured)")
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9],
                    help="5: the whole-model decode step (default); 1-4: the other workloads; "
                         "6: workload 5's decode loop with drifting windowed caches "
                         "(capacity W + --slack); 7: workload 5 with the fused append (bf16 "
                         "rows, RoPE on K, int8 caches); 8: decode attention over workload 5's "
                         "windowed layers; 9: paged decode attention (int8 cold pages, bf16 hot "
                         "pages) and the cooling conversion; one line each, for the design notes")
    ap.add_argument("--slack", type=int, default=16, help="workload 6: capacity - window")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no cross-GPU step (every (b, h) "
              "slice is independent); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import sliding_window_ring_tensor_amd as swrt
    from sliding_window_ring_tensor_amd import workloads as wl
    from sliding_window_ring_tensor_amd.decode_step import ModelDecodeStep

    if not os.path.exists(swrt.LIBRARY):
        from sliding_window_ring_tensor_amd import build as swrt_build
        swrt_build.build()
    swrt.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == 6:
        return drift_loop(args, dev)
    if args.workload == 8:
        return attention_bench(args, dev)
    if args.workload == 9:
        return paged_bench(args, dev)
    if args.workload not in (5, 7):
        return other_workload(args, dev)
    xf = args.workload == 7
    spec = wl.workload7() if xf else wl.workload5(wl.DTYPES[args.dtype])
    dtype_label = "bf16->int8" if xf else args.dtype
    log(f"allocating {args.sets} buffer sets ...")
    steps = [ModelDecodeStep(spec, dev, set_id=i) for i in range(args.sets)]
    acct = steps[0].algorithmic_bytes()
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    K, W = args.steps, args.warmup
    R = _reps(K)  # timed blocks, medians reported
    NB = K // R
    fused = args.form == "fused"
    with torch.cuda.stream(stream):
        def graph_time(fn):
            """K steps replayed as graphs (one per buffer set), wall clock
            between two synchronizations."""
            for st in steps:
                fn(st)  # warm the launch path before capture
            torch.cuda.synchronize()
            graphs = []
            for st in steps:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    fn(st)
                graphs.append(g)
            for i in range(W):
                graphs[i % len(graphs)].replay()
            torch.cuda.synchronize()
            out = []
            for r in range(R):
                t0 = time.perf_counter()
                for i in range(NB):
                    graphs[(r * NB + i) % len(graphs)].replay()
                torch.cuda.synchronize()
                out.append((time.perf_counter() - t0) / NB)
            return out

        def eager_time(fn):
            """K steps issued from the host (arguments marshalled once), wall
            clock between two synchronizations, per block of NB steps."""
            for i in range(W):
                fn(steps[i % len(steps)])
            torch.cuda.synchronize()
            out = []
            for r in range(R):
                t0 = time.perf_counter()
                for i in range(NB):
                    fn(steps[(r * NB + i) % len(steps)])
                torch.cuda.synchronize()
                out.append((time.perf_counter() - t0) / NB)
            return out

        log(f"timing {K} eager steps, one launch per step ...")
        eager_fused_v = eager_time(lambda st: st.run_fused())
        log(f"timing {K} eager steps, three launches per step ...")
        eager_three_v = eager_time(lambda st: st.run_three())
        log(f"timing {K} graph-replayed steps, one launch per step ...")
        graph_fused_v = graph_time(lambda st: st.run_fused())
        log(f"timing {K} graph-replayed steps, three launches per step ...")
        graph_three_v = graph_time(lambda st: st.run_three())
        eager_fused_s, eager_three_s = _median(eager_fused_v), _median(eager_three_v)
        graph_fused_s, graph_three_s = _median(graph_fused_v), _median(graph_three_v)

        # ---- kernels alone: HIP events ----
        # The host needs longer to issue a launch than the GPU to run it. A
        # sleep kernel issued first keeps the GPU busy while the host queues
        # a whole timed block, so one pair of events on the launch stream
        # brackets back-to-back kernel execution, not host gaps.
        t0 = time.perf_counter()
        for i in range(W):
            steps[i % len(steps)].run_three()
        torch.cuda.synchronize()
        host_step_s = (time.perf_counter() - t0) / max(W, 1)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        torch.cuda._sleep(1_000_000)
        s1.record(stream)
        torch.cuda.synchronize()
        cycles_per_s = 1_000_000 / (s0.elapsed_time(s1) * 1e-3)

        def events_block(fn):
            out = []
            for r in range(R):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(int(cycles_per_s * min(2.0, 2.0 * NB * host_step_s + 0.05)))
                a.record(stream)
                for i in range(NB):
                    fn(steps[(r * NB + i) % len(steps)])
                b.record(stream)
                torch.cuda.synchronize()
                out.append(a.elapsed_time(b) * 1e-3 / NB)
            return out

        log(f"timing {K} launches of the one-launch step ...")
        fused_mean_s = _median(events_block(lambda st: st.run_fused()))
        log(f"timing {K} launches of the window kernel alone ...")
        win_mean_s = _median(events_block(lambda st: st.windowed()))
        log(f"timing {K} three-launch steps ...")
        three_eager_s = _median(events_block(lambda st: st.run_three()))

        torch_copy, swrt_copy = copy_reference(dev, stream)

    flags = [int(st.buffers.flags.item()) for st in steps]
    if any(flags):
        raise SystemExit(f"device flags raised during the benchmark: {flags}")
    if args.timing == "eager":
        step_s = eager_fused_s if fused else eager_three_s
    else:
        step_s = graph_fused_s if fused else graph_three_s
    value = acct["total"] / step_s / 1e9
    fx = " with the fused append (RoPE on K, int8 quantization)" if xf else ""
    if fused:
        kname, kbytes, kmean = "decode_step_kernel", acct["total"], fused_mean_s
        kdesc = ("decode_step_kernel: the whole step in one launch (lengths, 12 windowed layers, "
                 f"24 full caches){fx}")
    else:
        kname, kbytes, kmean = "window_in_place", acct["windowed"], win_mean_s
        kdesc = f"window_in_place: 12 windowed layers, K and V, one launch{fx}"
    achieved = kbytes / kmean / 1e9
    meas = MEASURED_TRAFFIC.get((dtype_label, kname, kernel_source_hash(kname)))
    traffic = None if meas is None else meas["read"] + meas["written"]

    cpu = None
    if not args.no_cpu_baseline:
        nt = host_threads()
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s on {nt} threads ...")
        n, el = cpu_baseline(steps[0], args.cpu_seconds, threads=nt)
        log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s on one thread ...")
        n1, el1 = cpu_baseline(steps[0], args.cpu_seconds, threads=1)
        cpu = {"value": round(acct["total"] * n / el / 1e9, 4), "unit": "GB/s", "cores": nt,
               "kind": "oracle",
               "sample": f"{n} whole-model decode steps of the same workload (host copies of "
                         f"buffer set 0), (layer, batch chunk) slices over {nt} threads, "
                         f"{el:.1f} s",
               "us_per_step": round(el / n * 1e6, 1),
               "cpu_model": cpu_model(),
               "single_thread": {"value": round(acct["total"] * n1 / el1 / 1e9, 4),
                                 "unit": "GB/s", "cores": 1,
                                 "us_per_step": round(el1 / n1 * 1e6, 1),
                                 "sample": f"{n1} steps, one thread, {el1:.1f} s"}}

    out = {
        "metric": "KV-cache update effective HBM GB/s (% of peak) and us per decode step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(step_s * 1e3, 5),
        "us_per_step": round(step_s * 1e6, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label,
        "data": "synthetic",
        "config": {
            "workload": f"whole-model decode-step KV-cache update, {spec.layers} layers "
                        f"({len(spec.windowed_layers)} windowed C={spec.window}, "
                        f"{len(spec.full_layers)} full linear TensorScatter max_seq={spec.max_seq}), "
                        f"B={spec.batch}, H_kv={spec.kv_heads}, D={spec.head_dim}, "
                        f"T~U[1,8192] seed {spec.seed}" + (
                            f"; fused append: bf16 new rows, K rotated at position T-1 "
                            f"(rotary_dim {spec.rotary_dim}), int8 caches, K scale "
                            f"{spec.k_scale}, V scale {spec.v_scale}" if xf else ""),
            "bytes_per_step": acct["total"],
            "form": ("one launch per step (kv_decode_step_xf)" if xf else
                     "one launch per step (kv_decode_step)") if fused else
                    ("three launches per step (kv_seq_lengths, kv_window_append_xf, "
                     "tensor_scatter_xf)" if xf else
                     "three launches per step (kv_seq_lengths, kv_window_append_layers, "
                     "tensor_scatter_batched)"),
            "timing": ("eager: library calls with arguments marshalled once, steps between "
                       "two synchronizations" if args.timing == "eager" else
                       "HIP graph replay, one graph per buffer set") +
                      f"; medians of {R} blocks of {NB} steps",
            "cache_defeat": f"{args.sets} independent buffer sets round robin",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kdesc,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": kbytes,
            "median_launch_us": round(kmean * 1e6, 3),
        },
        "cpu_baseline": cpu,
        "one_launch": {"graph_us_per_step": round(graph_fused_s * 1e6, 2),
                       "eager_us_per_step": round(eager_fused_s * 1e6, 2),
                       "events_us_per_launch": round(fused_mean_s * 1e6, 2)},
        "three_launches": {"graph_us_per_step": round(graph_three_s * 1e6, 2),
                           "eager_us_per_step": round(eager_three_s * 1e6, 2),
                           "events_us_per_step": round(three_eager_s * 1e6, 2),
                           "window_kernel_us": round(win_mean_s * 1e6, 3),
                           "window_kernel_gbs": round(acct["windowed"] / win_mean_s / 1e9, 1)},
        "copy_reference_gbs": {"torch_copy": round(torch_copy, 1),
                               "swrt_tensor_scatter_copy": round(swrt_copy, 1)},
        "env": {"gpu": torch.cuda.get_device_name(dev), "torch": torch.__version__,
                "hip": torch.version.hip, "host": platform.node()},
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
