"""The windowed append that allocates nothing (swrt_kv_window_append_noalloc)
against the allocating entry point (swrt_kv_window_append with torch-owned
staging buffers): every output byte equal, on two calls in a row through the
C-ABI, the second with a smaller input, and the first again after it (the
shared staging array keeps the previous call's bytes)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sliding_window_ring_tensor_amd as swrt
from sliding_window_ring_tensor_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    swrt.lib()


def _case(g, B, H, C, S, D, dtype, bsnh=False):
    sk = g.integers(0, 3 * C, size=B).astype(np.int32)
    sk[: min(B, 3)] = [S - 1, C - 1, C + S][: min(B, 3)]
    kc, vc = (wl.host_payload(g, (B, H, C, D), dtype, raw_bits=True) for _ in range(2))
    shape = (B, S, H, D) if bsnh else (B, H, S, D)
    kn, vn = (wl.host_payload(g, shape, dtype, raw_bits=True) for _ in range(2))
    return sk, kc, vc, kn, vn


def _run(case, S, C, bsnh, noalloc):
    sk, kc, vc, kn, vn = case
    k, v = kc.to(DEV), vc.to(DEV)
    view = (lambda t: t.to(DEV).transpose(1, 2)) if bsnh else (lambda t: t.to(DEV))
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    lens = swrt.kv_seq_lengths(torch.from_numpy(sk).to(DEV), S, C)
    if noalloc:
        swrt.kv_window_append_noalloc(k, v, view(kn), view(vn), lens.cache_past, lens.evict,
                                      flags=flags)
    else:
        B, H, _, D = k.shape
        ks = torch.empty((B, H, C + S, D), dtype=k.dtype, device=DEV)
        vs = torch.empty_like(ks)
        swrt.kv_window_append(k, v, view(kn), view(vn), lens.cache_past, lens.evict,
                              k_staging=ks, v_staging=vs, flags=flags)
    torch.cuda.synchronize()
    return k.cpu().view(torch.uint8), v.cpu().view(torch.uint8), int(flags.item())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.int8], ids=str)
def test_noalloc_equals_the_allocating_call_twice(dtype):
    g = wl.rng(990)
    big = (6, 4, 96, 24, 128, False)   # staging 2 x 6*4*120*128 elements
    small = (3, 2, 40, 5, 64, True)    # then a smaller step, BSNH new rows
    cases = [(p, _case(g, *p[:5], dtype, bsnh=p[5])) for p in (big, small, big)]
    for (B, H, C, S, D, bsnh), case in cases:
        print("noalloc", dtype, B, H, C, S, D, bsnh, flush=True)
        a = _run(case, S, C, bsnh, noalloc=True)
        b = _run(case, S, C, bsnh, noalloc=False)
        assert a[2] == b[2] == 0
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        # and the step did move rows (not a vacuous comparison)
        assert not torch.equal(a[0], case[1].view(torch.uint8))


def test_noalloc_decode_and_limit():
    """S = 1 runs in place (no staging at all); a step whose staging exceeds
    half the array is refused before anything is launched."""
    g = wl.rng(991)
    B, H, C, D = 5, 3, 16, 64
    case = _case(g, B, H, C, 1, D, torch.bfloat16)
    a = _run(case, 1, C, False, noalloc=True)
    b = _run(case, 1, C, False, noalloc=False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # [1, 1, C + S, D] bf16 with (C + S) * D * 2 > 64 MiB
    C2, S2, D2 = 4096, 2, 8192 + 64
    k = torch.zeros((1, 1, C2, D2), dtype=torch.bfloat16, device=DEV)
    kn = torch.zeros((1, 1, S2, D2), dtype=torch.bfloat16, device=DEV)
    lens = swrt.kv_seq_lengths(torch.tensor([S2 - 1], dtype=torch.int32, device=DEV), S2, C2)
    with pytest.raises(swrt.SwrtError) as e:
        swrt.kv_window_append_noalloc(k, k.clone(), kn, kn.clone(), lens.cache_past, lens.evict)
    assert e.value.status == swrt.E_UNSUPPORTED
