"""Tagged-row token histories for replay checks of windowed and ring caches.

Every row of every buffer carries a tag that names where it came from: a new
token row holds (tensor, b, h, token index), an initial cache row holds a
negative "never written" mark unique to its (tensor, b, h, row). A cache state
can then be checked against the invariant of the pull request "GQA support
sliding_window_cache" (section "Design"): the cache holds the L = min(T, C)
most recent tokens, contiguously, at rows [0, L).

Rows are int32 quadruples, optionally widened to D > 4 columns by repeating a
mix of the tag, so that a row-level mistake shows in every column.
"""
from __future__ import annotations

import numpy as np

TAG_COLS = 4


def token_rows(tensor: int, b: int, h: int, tokens, D: int = TAG_COLS) -> np.ndarray:
    """[len(tokens), D] int32 rows for token indices `tokens` of (tensor, b, h)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.empty((tokens.size, D), dtype=np.int32)
    base = np.stack([np.full(tokens.size, tensor), np.full(tokens.size, b),
                     np.full(tokens.size, h), tokens], axis=1)
    for c in range(D):
        out[:, c] = base[:, c % 4] if c < 4 else (base[:, c % 4] * 7919 + c) % (1 << 30)
    return out


def initial_rows(tensor: int, b: int, h: int, n: int, D: int = TAG_COLS) -> np.ndarray:
    """Never-written rows: token field -1 - row, so no token ever matches."""
    return token_rows(tensor, b, h, -1 - np.arange(n), D)


def new_block(B: int, H: int, T_before: np.ndarray, S: int, D: int = TAG_COLS):
    """K and V new rows [B,H,S,D] holding tokens T_before[b] .. T_before[b]+S-1."""
    k = np.empty((B, H, S, D), np.int32)
    v = np.empty((B, H, S, D), np.int32)
    for b in range(B):
        toks = np.arange(T_before[b], T_before[b] + S)
        for h in range(H):
            k[b, h] = token_rows(0, b, h, toks, D)
            v[b, h] = token_rows(1, b, h, toks, D)
    return k, v


def fresh_cache(B: int, H: int, rows: int, D: int = TAG_COLS, tensors=(0, 1)):
    """K and V buffers of never-written rows; `tensors` picks the tag ids
    (0, 1 for caches; e.g. 2, 3 for staging buffers)."""
    k = np.empty((B, H, rows, D), np.int32)
    v = np.empty((B, H, rows, D), np.int32)
    for b in range(B):
        for h in range(H):
            k[b, h] = initial_rows(tensors[0], b, h, rows, D)
            v[b, h] = initial_rows(tensors[1], b, h, rows, D)
    return k, v


def windowed_state(B: int, H: int, C: int, T: np.ndarray, D: int = TAG_COLS):
    """A cache that satisfies the invariant for totals T (rows >= L hold marks)."""
    k, v = fresh_cache(B, H, C, D)
    for b in range(B):
        L = min(int(T[b]), C)
        toks = np.arange(T[b] - L, T[b])
        for h in range(H):
            k[b, h, :L] = token_rows(0, b, h, toks, D)
            v[b, h, :L] = token_rows(1, b, h, toks, D)
    return k, v


def check_window(k, v, T: np.ndarray, C: int, before_k=None, before_v=None):
    """Assert the window invariant for totals T; rows >= L must equal `before_*`."""
    B, H, _, D = k.shape
    for b in range(B):
        L = min(int(T[b]), C)
        toks = np.arange(T[b] - L, T[b])
        for h in range(H):
            np.testing.assert_array_equal(k[b, h, :L], token_rows(0, b, h, toks, D),
                                          err_msg=f"K window b={b} h={h} T={T[b]}")
            np.testing.assert_array_equal(v[b, h, :L], token_rows(1, b, h, toks, D),
                                          err_msg=f"V window b={b} h={h} T={T[b]}")
            if before_k is not None:
                np.testing.assert_array_equal(k[b, h, L:], before_k[b, h, L:],
                                              err_msg=f"K tail b={b} h={h}")
                np.testing.assert_array_equal(v[b, h, L:], before_v[b, h, L:],
                                              err_msg=f"V tail b={b} h={h}")


# Step schedules (new tokens per step) for replays, after the scenario list of
# the windowed-cache test suites described in the same pull request and its CPU
# follow-up: prompt shorter / longer than the capacity followed by decode,
# chunked prefill, eviction boundaries, many decode steps at small capacity.
def schedules(C: int) -> dict:
    return {
        "short_prompt_then_decode": [max(2, C // 3)] + [1] * (C + 5),
        "long_prompt_then_decode": [2 * C + 3] + [1] * 6,
        "chunked_prefill": [6, 6, 6, 6, 6, 1, 1, 1],
        "prompt_equals_capacity": [C, 1, 1, 1],
        "prompt_capacity_minus_one": [C - 1, 1, 1, 1],
        "prompt_capacity_plus_one": [C + 1, 1, 1],
        "decode_from_empty": [1] * (2 * C + 3),
        "chunk_larger_than_capacity": [3, C + 5, 1, 2 * C, 1],
        "chunk_equals_capacity": [1, C, C, 1],
    }
