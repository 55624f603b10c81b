/*
 * swrt.h -- C-ABI of libswrt.so: sliding-window / ring KV-cache updates on
 * AMD Instinct MI355X (gfx950).
 *
 * Three operations, each one or two kernel launches on the caller's stream:
 *
 *   swrt_tensor_scatter    ONNX operator "TensorScatter" (ai.onnx, since
 *                          version 24): write an update block into a
 *                          fixed-capacity cache along the sequence axis at a
 *                          per-batch write index, linear or circular. The
 *                          circular mode is also the ring-buffer write "slot =
 *                          position mod W" of the Core AI model zoo page
 *                          "Stateful decode & KV cache", section
 *                          "Sliding-window ring buffer".
 *   swrt_kv_seq_lengths    onnxruntime pull request "GQA support
 *                          sliding_window_cache", section "Design": the
 *                          absolute and cache-relative lengths and per-batch
 *                          eviction counts of one windowed step, derived on the
 *                          device from seqlens_k.
 *   swrt_kv_window_append  same page, section "Design": shift the resident
 *                          window left by E rows and write the S new rows after
 *                          it, for K and V in one launch; in place when S = 1,
 *                          through a C+S staging cache with copy-back when S > 1.
 * plus batched forms of the last two and of TensorScatter (several layers or
 * caches per launch), swrt_kv_decode_step (all of a decode step at once) and
 * swrt_kv_window_stage_step (the lengths and the stage phase at once),
 * and *_xf forms that fuse the row transform of the append into the write:
 * RoPE on K at the absolute position and conversion or affine quantization
 * into the cache's element type (swrt_row_transform below), and
 * swrt_window_attention, the decode attention that reads the windowed caches.
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer. The library allocates nothing,
 *     frees nothing, keeps no pointer after returning and holds no state, so
 *     calls on disjoint buffers may come from any host thread.
 *   - Streams: work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream). Nothing synchronises; buffers must stay alive until the stream
 *     work ends. No call reads device memory on the host, so every call can be
 *     captured into a HIP graph.
 *   - Layout: dense row-major buffers only (strided new-token rows excepted).
 *     Payload is moved as raw bits: any element type of the given width
 *     round-trips bit-exactly (NaN payloads, -0, fp8 encodings included).
 *   - Synchronous errors: a non-zero status is returned and nothing is
 *     launched. SWRT_E_INVALID_ARG for a null required pointer, a bad rank,
 *     axis, mode, phase or element width, a negative size, S > M (TensorScatter),
 *     C < 1, a pointer not aligned to its element (element size, capped at 8
 *     bytes), or overlapping buffers (other than present == past).
 *     SWRT_E_UNSUPPORTED for a row that does not end on a byte (4-bit elements, odd row length) and
 *     for sizes beyond the limits stated below. SWRT_E_LAUNCH when the HIP
 *     launch itself fails.
 *   - Data-dependent problems are reported asynchronously: bits are OR-ed into
 *     the optional device word *d_flags (may be NULL) and the affected batch
 *     entry is handled as stated per entry point.
 */
#ifndef SWRT_H
#define SWRT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWRT_ABI_VERSION 10

/* synchronous status codes */
#define SWRT_OK 0
#define SWRT_E_INVALID_ARG 1
#define SWRT_E_UNSUPPORTED 2
#define SWRT_E_LAUNCH 3

/* asynchronous flags (OR-ed into *d_flags) */
#define SWRT_FLAG_LINEAR_OOB 1u   /* linear write index < 0 or > M - S        */
#define SWRT_FLAG_BAD_SEQLEN 2u   /* seqlens_k[b] < 0 or seqlens_k[b] + 1 < S */
#define SWRT_FLAG_BAD_LENGTHS 4u  /* (Lp, E) not a step that fits (C, S)      */
#define SWRT_FLAG_ROPE_RANGE 8u   /* a rotary position outside the tables     */
#define SWRT_FLAG_BAD_PAGES 16u   /* a page table or page descriptor failed   */
#define SWRT_FLAG_PAGE_FULL 32u   /* a paged append found its page full       */

/* TensorScatter mode attribute */
#define SWRT_MODE_LINEAR 0
#define SWRT_MODE_CIRCULAR 1

/* phases of a multi-token (S > 1) windowed step */
#define SWRT_PHASE_STAGE 1u   /* seed staging[0..Lp) and write staging[Lp..Lp+S) */
#define SWRT_PHASE_COMMIT 2u  /* copy the surviving window back into the cache   */
#define SWRT_PHASE_ALL 3u     /* STAGE, then COMMIT                              */

#define SWRT_MAX_RANK 8

/*
 * swrt_tensor_scatter -- TensorScatter (ONNX operator page "TensorScatter":
 * description, pseudocode, Inputs, Outputs, Attributes).
 *
 *   present[(*prefix, j(b, s)), :] = update[(*prefix, s), :]
 *   for every prefix index `prefix` over shape[0..axis) (b = prefix[0]) and
 *   every s < S, with j = w_b + s (linear) or (w_b + s) mod M (circular,
 *   floor modulo, so negative w_b wraps too); M = shape[axis]. Every other row
 *   of present equals past.
 *
 * present        device, same shape as past. present == past updates in place
 *                (only the target rows are written); otherwise present is
 *                written in full (past rows plus update rows) and must not
 *                overlap past.
 * past           device, dense row-major `shape`.
 * update         device, dense, `shape` with shape[axis] replaced by seq_len.
 *                Must not overlap present.
 * write_indices  device int64[shape[0]], or NULL for all zeros.
 * shape          host int64[rank]; every dim >= 0.
 * rank           2 .. SWRT_MAX_RANK.
 * axis           sequence axis; negative counts from the end; after that it
 *                must lie in [1, rank) (the batch axis 0 is not allowed).
 * seq_len        S, 0 <= S <= M. S = 0 (or any zero dim) is a no-op apart from
 *                the out-of-place copy.
 * mode           SWRT_MODE_LINEAR or SWRT_MODE_CIRCULAR.
 * elem_bits      4, 8, 16, 32, 64 or 128; 4-bit needs an even row length
 *                (product of shape[axis+1..rank)).
 * d_flags        device uint32 or NULL. SWRT_FLAG_LINEAR_OOB when a linear
 *                w_b < 0 or w_b + S > M: every row of that batch entry keeps
 *                past's value (no partial write).
 * Limits: sizes must fit int64 bytes, and the words one call moves (update
 * bytes in place, present bytes otherwise, over a copy word of up to 16
 * bytes: the widest that divides the row and every address) must stay below
 * 2^31, i.e. up to 32 GiB per call with 16-byte rows.
 */
int swrt_tensor_scatter(void *present, const void *past, const void *update,
                        const int64_t *write_indices, const int64_t *shape,
                        int rank, int axis, int64_t seq_len, int mode,
                        int elem_bits, uint32_t *d_flags, void *stream);

/*
 * swrt_tensor_scatter_batched -- swrt_tensor_scatter on n_tensors caches that
 * share shape, axis, S, mode, element width and write_indices, in one launch
 * (e.g. the K and V caches of every full-attention layer of a model at one
 * decode step).
 *
 * n_tensors            0 .. SWRT_MAX_BATCHED.
 * presents, pasts,
 * updates              host arrays of n_tensors device pointers, each as in
 *                      swrt_tensor_scatter. Either every presents[t] equals
 *                      pasts[t] (in place) or none does. No present may
 *                      overlap any other buffer of the call; updates and
 *                      pasts may be shared.
 * The other arguments and the flag word are shared by all tensors.
 */
#define SWRT_MAX_BATCHED 64
int swrt_tensor_scatter_batched(int n_tensors, void *const *presents,
                                const void *const *pasts,
                                const void *const *updates,
                                const int64_t *write_indices,
                                const int64_t *shape, int rank, int axis,
                                int64_t seq_len, int mode, int elem_bits,
                                uint32_t *d_flags, void *stream);

/*
 * swrt_kv_seq_lengths -- lengths of one windowed GQA step (pull request "GQA
 * support sliding_window_cache", section "Design", and the follow-up that
 * moves the end-pointer arithmetic to 64 bits and clamps the past length).
 *
 * For each b < batch, in 64-bit arithmetic:
 *   T  = seqlens_k[b] + 1          absolute total length after the step
 *   P  = max(0, T - S)             absolute past length
 *   Lp = min(P, C)                 rows resident before the step
 *   E  = max(0, Lp + S - C)        rows evicted by the step
 *   L  = Lp + S - E  (= min(T, C)) rows resident after the step
 *
 * seqlens_k        device int32[batch] (total length minus one).
 * batch            >= 0 (0 is a no-op).
 * seq_len          S >= 1, new tokens in this step.
 * capacity         C >= 1, rows per (b, h) in the cache.
 * total_lens       device int64[batch] or NULL: T.
 * past_lens        device int64[batch] or NULL: P.
 * cache_past_lens  device int32[batch], required: Lp.
 * cache_total_lens device int32[batch] or NULL: L.
 * evict_counts     device int32[batch], required: E.
 * work_offsets     device int64[batch + 1] or NULL: the exclusive prefix over
 *                  the batch of the rows each entry's step writes,
 *                  r_b = (E_b > 0 ? Lp_b - E_b : 0) + 1 for S = 1 (shifted rows
 *                  and the appended one) and Lp_b + S for S > 1 (staged rows):
 *                  work_offsets[0] = 0, work_offsets[b + 1] = work_offsets[b] +
 *                  r_b, the total last. A flat grid sized for the worst case
 *                  can map its tiles to (entry, row) from it without a host
 *                  round trip. 64-bit (the total reaches batch * (C + S)).
 *                  Computed by one workgroup scanning the batch (wave prefix by
 *                  lane shuffles, waves joined through LDS).
 * d_flags          device uint32 or NULL. SWRT_FLAG_BAD_SEQLEN when
 *                  seqlens_k[b] < 0 or T < S; P is then clamped to 0 and the
 *                  other values follow from it.
 * Output buffers must not overlap seqlens_k or each other.
 */
int swrt_kv_seq_lengths(const int32_t *seqlens_k, int batch, int seq_len,
                        int capacity, int64_t *total_lens, int64_t *past_lens,
                        int32_t *cache_past_lens, int32_t *cache_total_lens,
                        int32_t *evict_counts, int64_t *work_offsets, uint32_t *d_flags,
                        void *stream);

/*
 * swrt_kv_seq_lengths_drift -- lengths of one windowed step under the
 * drifting layout of the same pull request's CPU follow-up ("Key design
 * decisions: Drifting layout"). Resident tokens live at rows [0, end) with
 * gap = C - W + 1 and end(x) = x while x <= C, else
 * x - gap * ceil((x - C) / gap), so W <= end <= C: a whole gap of rows is
 * reclaimed at once, once every gap decode steps, and the other steps only
 * append. With T and P as in swrt_kv_seq_lengths:
 *   Lp = end(P), L = end(T), E = Lp + S - L.
 * The window W (1 <= W <= C, else SWRT_E_INVALID_ARG) is the attention
 * window the last W tokens of which stay resident; W = C gives exactly the
 * values of swrt_kv_seq_lengths. Every other argument as there (work_offsets
 * counts a whole gap's shift when the step compacts). The (Lp, E) pairs feed
 * swrt_kv_window_append unchanged.
 */
int swrt_kv_seq_lengths_drift(const int32_t *seqlens_k, int batch, int seq_len,
                              int capacity, int window, int64_t *total_lens,
                              int64_t *past_lens, int32_t *cache_past_lens,
                              int32_t *cache_total_lens, int32_t *evict_counts,
                              int64_t *work_offsets, uint32_t *d_flags, void *stream);

/*
 * swrt_kv_window_append -- one windowed cache step for K and V (pull request
 * "GQA support sliding_window_cache", section "Design": the invariant that
 * the cache holds the L = min(T, C) most recent tokens at rows [0, L), the
 * shift cache[E..Lp) -> cache[0..Lp-E), the write of the new tokens to
 * cache[Lp-E .. Lp-E+S), in-place decode for S = 1 and the C+S staging cache
 * for S > 1).
 *
 * S = 1 (in place, phase ignored): for every (tensor, b, h)
 *     cache[0 .. Lp-E) <- old cache[E .. Lp)   (E is 0 or 1; a whole gap
 *                                               under the drifting layout)
 *     cache[Lp-E]      <- new[b, h, 0]
 * S > 1:
 *   STAGE:  staging[0 .. Lp)    <- cache[0 .. Lp)
 *           staging[Lp .. Lp+S) <- new[b, h, 0 .. S)
 *   COMMIT: cache[0 .. L)       <- staging[E .. E+L)
 *           (when E = 0 only rows [Lp, L) are copied: rows [0, Lp) of staging
 *           hold what STAGE seeded, and the caller must not change them
 *           between the phases; attention may read staging in between.)
 * Cache rows [L, C) and staging rows [Lp+S, C+S) are never written.
 *
 * k_cache, v_cache     device [batch, kv_heads, capacity, head_dim], distinct,
 *                      non-overlapping.
 * k_new, v_new         device; row (b, h, s) starts at element
 *                      b*new_strides[0] + h*new_strides[1] + s*new_strides[2]
 *                      and its head_dim elements are contiguous (BNSH and BSNH
 *                      both fit). Must not overlap any cache or staging buffer.
 * new_strides          host int64[3], element strides for b, h, s (>= 0).
 * k_staging, v_staging device [batch, kv_heads, capacity + seq_len, head_dim];
 *                      required when S > 1, ignored (may be NULL) when S = 1.
 * cache_past_lens,
 * evict_counts         device int32[batch]: Lp and E from swrt_kv_seq_lengths
 *                      (or swrt_kv_seq_lengths_drift) with the same S and C.
 * batch, kv_heads      >= 0 (0 is a no-op). head_dim >= 0.
 * capacity             C >= 1. seq_len S >= 1 (S > C is allowed when S > 1).
 * elem_bits            4, 8, 16, 32, 64 or 128 (4-bit: even head_dim and
 *                      even strides).
 * phase                SWRT_PHASE_STAGE, _COMMIT or _ALL when S > 1.
 * d_flags              device uint32 or NULL. SWRT_FLAG_BAD_LENGTHS when the
 *                      pair is not a step that fits (Lp < 0, Lp > C, E < 0,
 *                      or L = Lp + S - E outside [1, C]): that batch entry is
 *                      left untouched (cache and staging).
 * Limits: batch * kv_heads * 2 slices and (capacity + seq_len) * head_dim *
 * elem_bits / 128 vectors per slice must each stay below 2^31.
 */
int swrt_kv_window_append(void *k_cache, void *v_cache, const void *k_new,
                          const void *v_new, const int64_t *new_strides,
                          void *k_staging, void *v_staging,
                          const int32_t *cache_past_lens,
                          const int32_t *evict_counts, int batch, int kv_heads,
                          int capacity, int seq_len, int head_dim,
                          int elem_bits, unsigned phase, uint32_t *d_flags,
                          void *stream);

/*
 * swrt_kv_window_append_noalloc -- for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * swrt_kv_window_append with phase SWRT_PHASE_ALL and no staging arguments.
 * S = 1 runs in place as there. For S > 1 the two [batch, kv_heads,
 * capacity + seq_len, head_dim] staging buffers are carved from the
 * library's own device array of SWRT_NOALLOC_STAGING_BYTES bytes, which every
 * GPU the library runs on holds until the process ends (K's at its start, V's
 * at the next 256-byte boundary). The call allocates and frees nothing;
 * its first call on a device looks the array's address up with that device
 * current (the caller makes the stream's device current, as for any HIP
 * call). Every call on one GPU shares that GPU's array, so calls that overlap
 * in time on one GPU (other streams, other host threads) race; calls on
 * different GPUs do not. SWRT_E_UNSUPPORTED when one staging buffer exceeds
 * SWRT_NOALLOC_STAGING_BYTES / 2 (it is then refused before anything is
 * launched). Every other argument, check and result as swrt_kv_window_append.
 */
#define SWRT_NOALLOC_STAGING_BYTES (128ll << 20)
int swrt_kv_window_append_noalloc(void *k_cache, void *v_cache, const void *k_new,
                                  const void *v_new, const int64_t *new_strides,
                                  const int32_t *cache_past_lens, const int32_t *evict_counts,
                                  int batch, int kv_heads, int capacity, int seq_len,
                                  int head_dim, int elem_bits, uint32_t *d_flags, void *stream);

/*
 * swrt_kv_window_append_layers -- swrt_kv_window_append for several layers at
 * once (the pull request's Design section applied to every windowed layer of
 * a model in one launch per phase, as for a whole-model decode step whose
 * windowed layers share batch, heads, capacity, head_dim and lengths).
 *
 * n_layers             1 .. SWRT_MAX_LAYERS.
 * k_caches, v_caches,
 * k_news, v_news       host arrays of n_layers device pointers, each as in
 *                      swrt_kv_window_append. New rows of all layers share
 *                      new_strides and may be shared between layers.
 * k_stagings,
 * v_stagings           host arrays of n_layers device pointers, required when
 *                      S > 1 (NULL otherwise).
 * Every other argument, the lengths and the flag word are shared by all
 * layers and mean what they mean for swrt_kv_window_append. No cache or
 * staging buffer may overlap any other buffer of any layer.
 */
#define SWRT_MAX_LAYERS 32
int swrt_kv_window_append_layers(int n_layers, void *const *k_caches,
                                 void *const *v_caches,
                                 const void *const *k_news,
                                 const void *const *v_news,
                                 const int64_t *new_strides,
                                 void *const *k_stagings,
                                 void *const *v_stagings,
                                 const int32_t *cache_past_lens,
                                 const int32_t *evict_counts, int batch,
                                 int kv_heads, int capacity, int seq_len,
                                 int head_dim, int elem_bits, unsigned phase,
                                 uint32_t *d_flags, void *stream);

/*
 * swrt_kv_window_stage_step -- the lengths and the STAGE phase of a windowed
 * step with S >= 2 new rows (pull request "GQA support sliding_window_cache",
 * section "Design": the lengths of the step and the C+S staging cache) in
 * one launch. It writes exactly the bytes of
 *
 *   swrt_kv_seq_lengths_drift(seqlens_k, batch, seq_len, capacity, window,
 *                       total_lens, past_lens, cache_past_lens,
 *                       cache_total_lens, evict_counts)
 *                       (window == capacity: exactly swrt_kv_seq_lengths)
 *   swrt_kv_window_append_layers(n_layers, ..., k_stagings, v_stagings,
 *                       cache_past_lens, evict_counts, batch, kv_heads,
 *                       capacity, seq_len, head_dim, elem_bits,
 *                       SWRT_PHASE_STAGE, ...)
 *
 * with the stage part deriving each entry's Lp from seqlens_k itself (so the
 * pair is always one the step accepts: no SWRT_FLAG_BAD_LENGTHS). The step is
 * finished by swrt_kv_window_append_layers with SWRT_PHASE_COMMIT and the
 * cache_past_lens and evict_counts written here; attention may read the
 * staging buffers in between.
 *
 * n_layers             0 .. SWRT_MAX_LAYERS (0: the lengths alone); the
 *                      caches, new rows, strides and staging buffers as for
 *                      swrt_kv_window_append_layers.
 * seqlens_k            device int32[batch], required when batch > 0.
 * capacity, window     C >= 1 and 1 <= W <= C, as for
 *                      swrt_kv_seq_lengths_drift (W = C: the base layout).
 * total_lens .. evict_counts
 *                      device outputs as for swrt_kv_seq_lengths;
 *                      cache_past_lens and evict_counts are required (the
 *                      commit reads them), the others may be NULL.
 * seq_len              S >= 2 (S = 1 has no staging phase: see
 *                      swrt_kv_decode_step).
 * d_flags              SWRT_FLAG_BAD_SEQLEN (lengths clamped, step
 *                      proceeds), as for swrt_kv_seq_lengths.
 * No written buffer may overlap any other buffer of the call. Limits as for
 * swrt_kv_window_append.
 */
int swrt_kv_window_stage_step(int n_layers, void *const *k_caches,
                              void *const *v_caches, const void *const *k_news,
                              const void *const *v_news,
                              const int64_t *new_strides,
                              void *const *k_stagings, void *const *v_stagings,
                              const int32_t *seqlens_k, int capacity, int window,
                              int64_t *total_lens, int64_t *past_lens,
                              int32_t *cache_past_lens, int32_t *cache_total_lens,
                              int32_t *evict_counts, int batch, int kv_heads,
                              int seq_len, int head_dim, int elem_bits,
                              uint32_t *d_flags, void *stream);

/*
 * swrt_kv_decode_step -- every KV-cache update of one decode step (S = 1) of a
 * model with windowed layers (pull request "GQA support sliding_window_cache",
 * section "Design") and full-length layers (ONNX operator page "TensorScatter",
 * linear mode), in one launch. It writes exactly the bytes of
 *
 *   swrt_kv_seq_lengths_drift(seqlens_k, batch, 1, capacity, window,
 *                       total_lens, past_lens, cache_past_lens,
 *                       cache_total_lens, evict_counts)
 *                       (window == capacity: exactly swrt_kv_seq_lengths)
 *   swrt_kv_window_append_layers(n_window_layers, win_*, win_new_strides,
 *                       Lp, E, batch, kv_heads, capacity, 1, head_dim, ...)
 *   swrt_tensor_scatter_batched(n_full, full_caches, full_caches, full_new,
 *                       write_indices, {batch, kv_heads, max_seq, head_dim},
 *                       rank 4, axis 2, S = 1, SWRT_MODE_LINEAR, ...)
 *
 * with the windowed part deriving each entry's (Lp, E) from seqlens_k itself.
 *
 * n_window_layers      0 .. SWRT_MAX_LAYERS; win_* as for
 *                      swrt_kv_window_append_layers (caches [B, H, C, D], new
 *                      rows [B, H, 1, D] by win_new_strides, host int64[3]).
 * seqlens_k            device int32[batch]; required when there are windowed
 *                      layers or length outputs.
 * capacity             C >= 1 of the windowed caches.
 * window               W, 1 <= W <= C: the drifting layout's window (see
 *                      swrt_kv_seq_lengths_drift); W = C is the base layout.
 * total_lens .. evict_counts
 *                      optional device outputs as for swrt_kv_seq_lengths
 *                      (any may be NULL).
 * n_full               0 .. SWRT_MAX_BATCHED full caches [B, H, max_seq, D],
 *                      updated in place; full_new: their new rows, dense
 *                      [B, H, 1, D]; write_indices: device int64[batch].
 * batch, kv_heads, head_dim, elem_bits: shared by every cache.
 * d_flags              SWRT_FLAG_BAD_SEQLEN (lengths clamped, step proceeds)
 *                      and SWRT_FLAG_LINEAR_OOB (that batch entry of every full
 *                      cache keeps its rows), as for the three calls.
 * No written buffer may overlap any other buffer of the call.
 */
int swrt_kv_decode_step(int n_window_layers, void *const *win_k_caches,
                        void *const *win_v_caches, const void *const *win_k_new,
                        const void *const *win_v_new,
                        const int64_t *win_new_strides,
                        const int32_t *seqlens_k, int capacity, int window,
                        int64_t *total_lens, int64_t *past_lens,
                        int32_t *cache_past_lens, int32_t *cache_total_lens,
                        int32_t *evict_counts, int n_full,
                        void *const *full_caches, const void *const *full_new,
                        const int64_t *write_indices, int max_seq, int batch,
                        int kv_heads, int head_dim, int elem_bits,
                        uint32_t *d_flags, void *stream);

/*
 * ---------------------------------------------------------------------------
 * Fused append: the row transform (pull request "GQA support
 * sliding_window_cache", "Summary of Changes": the KV append writes at the
 * cache-relative offset while RoPE keeps the absolute position, bounded by
 * its own maximum position rather than the capacity; onnx-light how-to
 * "Persistent input/output feedback", section "Optional heterogeneous paged
 * KV": affine INT8 / UINT8 codes with FLOAT scales and scalar parameters on
 * append, ties rounded to even, codes saturated).
 *
 * Per-channel parameters (same pull request, comment-only follow-up: the
 * quantized cache's per-channel scale has shape (kv_num_heads, 1, head_size),
 * its singleton dimension flattened): element e of a row of KV head h takes
 * scale channel_scale[t][h * head_dim + e] and zero point
 * channel_zero_point[t][h * head_dim + e] (t = 0 for K, 1 for V) instead of
 * the scalar when that table is given.
 *
 * Every new row (head_dim elements of in_type) is read as binary32. A K row
 * (never a V row) is rotated when tables are given: each pair (x0, x1) --
 * elements (j, j + rotary_dim/2), or (2j, 2j+1) when interleaved -- becomes
 *   x0' = x0*c - x1*s,  x1' = x1*c + x0*s,  c = cos_table[pos][j], s = sin_table[pos][j],
 * each product and sum one binary32 operation rounded to nearest even (no
 * fused multiply-add); elements from rotary_dim on pass unrotated. Each
 * element is then written in out_type: F32 as is; F16 / BF16 rounded to
 * nearest even (overflow to infinity); any NaN of a float type as its
 * positive canonical quiet NaN (0x7FC00000 / 0x7E00 / 0x7FC0); INT8 / UINT8 as
 *   clamp(round_half_even(y / scale) + zero_point, code range),
 * NaN -> zero_point (saturated into the code range), with y / scale the
 * correctly rounded binary32 quotient; FP8_E4M3 (the OCP float8 E4M3 format,
 * "float8e4m3fn") as the code of y / scale rounded to nearest even, finite
 * values past 448 and infinities saturating to +-448, NaN as 0x7F.
 * The positions are absolute: past length + s on the windowed path,
 * write_indices[b] + s (before any circular wrap) on TensorScatter.
 * ---------------------------------------------------------------------------
 */
#define SWRT_XF_F32 1
#define SWRT_XF_F16 2
#define SWRT_XF_BF16 3
#define SWRT_XF_INT8 4
#define SWRT_XF_UINT8 5
#define SWRT_XF_FP8_E4M3 10  /* cache element type of the row transform only */

typedef struct swrt_row_transform {
  int in_type;             /* new rows: SWRT_XF_F32, _F16 or _BF16 */
  int out_type;            /* cache: any SWRT_XF_* type */
  const float *cos_table;  /* device binary32 [max_position, rotary_dim / 2],
                              or NULL: no rotation */
  const float *sin_table;  /* same shape; NULL exactly when cos_table is */
  int64_t max_position;    /* rows of the tables, >= 1 when rotating */
  int64_t rotary_dim;      /* even, 2 .. head_dim when rotating */
  int interleaved;         /* 0: pairs (j, j + rotary_dim/2); 1: (2j, 2j+1) */
  float scale[2];          /* K, V: positive, finite (INT8 / UINT8 / FP8 out_type) */
  int32_t zero_point[2];   /* K, V: inside the code range (INT8 / UINT8), 0 (FP8) */
  /* per-channel parameters, device [kv_heads, head_dim] (K, V), or NULL for
     the scalar: scales for INT8 / UINT8 / FP8 out_type, zero points for INT8 /
     UINT8; 4-byte aligned. Their values are data, not checked: the formulas
     apply as written (meaningful codes need positive finite scales and zero
     points inside the code range). kv_heads is the call's; for TensorScatter
     the cache's dimension 1 of rank 4 ([B, H, M, D]), 1 for rank 3, and no
     tables for a higher rank. */
  const float *channel_scale[2];
  const int32_t *channel_zero_point[2];
} swrt_row_transform;

/*
 * swrt_kv_window_append_xf -- swrt_kv_window_append_layers whose new rows
 * pass through *xf on their way into the caches (and staging): row s of
 * batch entry b sits at absolute position past_lens[b] + s. Caches and
 * staging hold out_type elements; new rows are in_type elements addressed by
 * new_strides (in elements). The shift moves cache rows unchanged.
 *
 * past_lens  device int64[batch]: the absolute past length P of
 *            swrt_kv_seq_lengths (or _drift) with the same S.
 * xf         host pointer, read during the call only. The tables must not
 *            overlap any written buffer.
 * d_flags    as for swrt_kv_window_append, and then SWRT_FLAG_ROPE_RANGE when
 *            rotating and P < 0 or P + S > max_position: that batch entry is
 *            left untouched, K and V, cache and staging (every phase checks).
 * Errors: SWRT_E_INVALID_ARG also for a transform outside the ranges above;
 * SWRT_E_UNSUPPORTED for S = 1 with head_dim > 4096.
 */
int swrt_kv_window_append_xf(int n_layers, void *const *k_caches,
                             void *const *v_caches, const void *const *k_news,
                             const void *const *v_news,
                             const int64_t *new_strides,
                             void *const *k_stagings, void *const *v_stagings,
                             const int32_t *cache_past_lens,
                             const int32_t *evict_counts,
                             const int64_t *past_lens, int batch, int kv_heads,
                             int capacity, int seq_len, int head_dim,
                             unsigned phase, const swrt_row_transform *xf,
                             uint32_t *d_flags, void *stream);

/*
 * swrt_kv_window_stage_step_xf -- swrt_kv_window_stage_step whose stage
 * phase is that of swrt_kv_window_append_xf: the new rows pass through *xf
 * at absolute positions P + s, P derived from seqlens_k like the lengths.
 * past_lens is then required too (the fused commit,
 * swrt_kv_window_append_xf with SWRT_PHASE_COMMIT, reads it); an entry whose
 * positions leave the rotary tables is flagged SWRT_FLAG_ROPE_RANGE and its
 * staging left untouched, as in the fused stage call. The caches and staging
 * buffers hold xf->out_type elements; other arguments as for
 * swrt_kv_window_stage_step and swrt_kv_window_append_xf.
 */
int swrt_kv_window_stage_step_xf(int n_layers, void *const *k_caches,
                                 void *const *v_caches, const void *const *k_news,
                                 const void *const *v_news,
                                 const int64_t *new_strides,
                                 void *const *k_stagings, void *const *v_stagings,
                                 const int32_t *seqlens_k, int capacity, int window,
                                 int64_t *total_lens, int64_t *past_lens,
                                 int32_t *cache_past_lens, int32_t *cache_total_lens,
                                 int32_t *evict_counts, int batch, int kv_heads,
                                 int seq_len, int head_dim,
                                 const swrt_row_transform *xf, uint32_t *d_flags,
                                 void *stream);

/*
 * swrt_tensor_scatter_xf -- swrt_tensor_scatter_batched with axis = rank - 2
 * (a row is the last dimension, head_dim) whose update rows (in_type) pass
 * through *xf: update row s of batch entry b at absolute position
 * write_indices[b] + s, before the circular wrap. present / past hold
 * out_type elements. tensors[i] is 0 for a K cache (rotated) and 1 for a V
 * cache; tensors is a host int[n_tensors]. rank 3 .. SWRT_MAX_RANK.
 * d_flags: SWRT_FLAG_LINEAR_OOB as for TensorScatter, and then
 * SWRT_FLAG_ROPE_RANGE (rotating, w_b < 0 or w_b + S > max_position): that
 * batch entry keeps past's rows in every tensor of the call.
 */
int swrt_tensor_scatter_xf(int n_tensors, void *const *presents,
                           const void *const *pasts, const void *const *updates,
                           const int *tensors, const int64_t *write_indices,
                           const int64_t *shape, int rank, int64_t seq_len,
                           int mode, const swrt_row_transform *xf,
                           uint32_t *d_flags, void *stream);

/*
 * swrt_kv_decode_step_xf -- swrt_kv_decode_step with the row transform fused
 * into every write: the same bytes as swrt_kv_seq_lengths(_drift), then
 * swrt_kv_window_append_xf with past_lens = P, then swrt_tensor_scatter_xf on
 * the full caches (K caches tensor 0, V caches tensor 1, linear mode), in one
 * launch. Full caches come as n_full_layers K and V pairs
 * (full_k_caches[i], full_v_caches[i]) with their new rows. Windowed caches
 * hold out_type elements; new rows are in_type. d_flags as for those calls.
 * n_full_layers: 0 .. SWRT_MAX_BATCHED / 2. SWRT_E_UNSUPPORTED for head_dim
 * above 4096 (above 512 when window < capacity).
 */
int swrt_kv_decode_step_xf(int n_window_layers, void *const *win_k_caches,
                           void *const *win_v_caches,
                           const void *const *win_k_new,
                           const void *const *win_v_new,
                           const int64_t *win_new_strides,
                           const int32_t *seqlens_k, int capacity, int window,
                           int64_t *total_lens, int64_t *past_lens,
                           int32_t *cache_past_lens, int32_t *cache_total_lens,
                           int32_t *evict_counts, int n_full_layers,
                           void *const *full_k_caches,
                           void *const *full_v_caches,
                           const void *const *full_k_new,
                           const void *const *full_v_new,
                           const int64_t *write_indices, int max_seq,
                           int batch, int kv_heads, int head_dim,
                           const swrt_row_transform *xf, uint32_t *d_flags,
                           void *stream);

/*
 * swrt_window_attention -- one-token decode attention over windowed caches
 * (onnx-light-cpu "Persistent KV Cache and Decode Performance Roadmap",
 * section "Phase 1: decode with contiguous KV cache": per KV block the
 * query/K dot products, the online-softmax update and the V accumulation,
 * without storing the score vector; query heads sharing a KV head read it
 * once; fp32 scores, softmax and accumulation. The window is that of the pull
 * request "GQA support sliding_window_cache": the query at absolute position
 * T - 1 sees the last W resident rows.) For every layer, batch entry b and
 * query head h, with L = cache_total_lens[b] and g = h / (q_heads / kv_heads):
 *   rows  r in [max(0, L - W), L)
 *   out[b, h, :] = sum_r softmax_r(scale * q[b, h, :] . k[b, g, r, :]) v[b, g, r, :]
 * An empty window (L = 0) writes zeros.
 *
 * n_layers          1 .. SWRT_MAX_LAYERS; q, k_caches, v_caches, out are host
 *                   arrays of n_layers device pointers (one launch for all).
 * q                 [batch, q_heads, head_dim] elem_type, 8-byte aligned.
 * k_caches, v_caches [batch, kv_heads, capacity, head_dim] elem_type, 8-byte
 *                   aligned (the windowed caches of swrt_kv_window_append).
 * out               [batch, q_heads, head_dim] out_type, aligned to its
 *                   element size; must not overlap any other buffer.
 * cache_total_lens  device int32[batch]: L of swrt_kv_seq_lengths (or _drift).
 * window            W >= 1 (W = capacity: every resident row; the ring-buffer
 *                   cache is this case).
 * scale             finite (usually 1 / sqrt(head_dim)).
 * elem_type         SWRT_XF_F32, _F16 or _BF16; out_type the same set.
 * d_flags           SWRT_FLAG_BAD_LENGTHS when L < 0 or L > capacity: that
 *                   entry's outputs are left as they were.
 * Supported shapes (else SWRT_E_UNSUPPORTED): 16-bit caches with q, k, v and
 * out all 16-byte aligned run on the matrix cores and take head_dim in
 * {32, 64, 96, 128, 192, 256} and any q_heads / kv_heads (a group of more
 * than 16 query heads runs as several waves per window, 16 heads each, which
 * all read the window's rows); fp32 caches, or 16-bit ones with an operand
 * only 8-byte aligned, run on the VALU and need head_dim * element size in
 * {64, 128, 256, 512} bytes, q_heads / kv_heads in {1, 2, 4, 8, 16} and
 * (q_heads / kv_heads) * head_dim * element size <= 2048 bytes.
 */
int swrt_window_attention(int n_layers, const void *const *q,
                          const void *const *k_caches, const void *const *v_caches,
                          void *const *out, const int32_t *cache_total_lens,
                          int window, int batch, int q_heads, int kv_heads,
                          int capacity, int head_dim, float scale, int elem_type,
                          int out_type, uint32_t *d_flags, void *stream);

/* ------------------------------------------------------------------------ */
/* Paged caches (onnx-light how-to "Persistent input/output feedback",        */
/* section "Optional heterogeneous paged KV": "Cache value declaration",      */
/* "Selected-block quantization", "Serialized cache values" and the kernel    */
/* description that follows them).                                            */
/* ------------------------------------------------------------------------ */

/* page formats beyond the row transform's: affine sub-byte codes */
#define SWRT_XF_INT4 6
#define SWRT_XF_UINT4 7
#define SWRT_XF_INT2 8
#define SWRT_XF_UINT2 9

/*
 * One page (block) of one stream (batch entry b, KV head g; stream
 * b * kv_heads + g): tokens [start, start + length) of the stream, capacity
 * physical rows of head_dim elements for K and for V at byte offsets of the
 * layer's arena. A payload is the block's logical [1, 1, capacity, head_dim]
 * tensor stored flat (row r, element e at r * head_dim + e). Dense formats
 * (SWRT_XF_F32 / _F16 / _BF16) hold values; affine formats (SWRT_XF_INT8,
 * _UINT8, _INT4, _UINT4, _INT2, _UINT2) hold codes c meaning
 * (c - zero_point) * scale, scale > 0 and finite, zero_point inside the code
 * range; sub-byte codes are packed from the least significant bits of each
 * byte (element 0 lowest), signed codes in two's complement. A stream's
 * pages, in token order, are contiguous from zero (each start is the previous
 * start + length) with 1 <= length <= capacity. 64 bytes, device memory.
 *
 * Library layout rule (not the pages'): the kernels read payloads in
 * aligned 16-byte blocks, so every payload offset is a multiple of 16; a page
 * whose offset is not is treated as invalid (SWRT_FLAG_BAD_PAGES).
 */
typedef struct swrt_page {
  int64_t start;
  int32_t length;
  int32_t capacity;
  int64_t k_offset;
  int64_t v_offset;
  int32_t k_format;
  int32_t v_format;
  float k_scale;
  float v_scale;
  int32_t k_zero_point;
  int32_t v_zero_point;
  int32_t reserved[2];
} swrt_page;

/*
 * One layer's paged cache plus its query and output, as the attention takes
 * them (host struct of device pointers):
 *   q          [batch, q_heads, head_dim] q_type, 16-byte aligned.
 *   out        [batch, q_heads, head_dim] out_type, 16-byte aligned; must not
 *              overlap any input.
 *   arena      device bytes holding every page payload, 16-byte aligned,
 *              arena_bytes long (a multiple of 16).
 *   pages      device swrt_page[n_pages].
 *   page_ids   device int32[n_ids]: indices into pages, the block table.
 *   The block table names each stream's pages in token order, in one of
 *   two forms:
 *   page_ptr   compressed rows (page_count NULL): device int32[batch *
 *              kv_heads + 1]; stream s owns page_ids[page_ptr[s] ..
 *              page_ptr[s + 1]).
 *   page_count slotted rows (non-NULL): device int32[batch * kv_heads];
 *              stream s owns the page_stride slots from s * page_stride and
 *              uses the first page_count[s] (0 .. page_stride) of them;
 *              page_ptr is then unused (may be NULL). The sealed append
 *              (swrt_paged_append) grows this form.
 * Layers may share pages and the block table (one table for every layer,
 * each with its own arena).
 */
typedef struct swrt_paged_layer {
  const void *q;
  void *out;
  const void *arena;
  int64_t arena_bytes;
  const swrt_page *pages;
  int64_t n_pages;
  const int32_t *page_ptr;
  const int32_t *page_ids;
  int64_t n_ids;
  int32_t *page_count;
  int64_t page_stride;
} swrt_paged_layer;

/*
 * swrt_paged_attention -- one-token decode attention over paged caches
 * (section "Optional heterogeneous paged KV": attention reads only valid,
 * visible tokens with online softmax, a left window bounds the preceding
 * tokens, grouped-query heads; onnx-light-cpu "Persistent KV Cache and Decode
 * Performance Roadmap", "Phase 1": fp32 scores, softmax and accumulation).
 * For every layer, batch entry b and query head h, with stream
 * s = b * kv_heads + h / (q_heads / kv_heads) holding T tokens (its last
 * page's start + length; 0 without pages):
 *   tokens  r in [max(0, T - 1 - left_window), T)   (left_window < 0: all T)
 *   out[b, h, :] = sum_r softmax_r(scale * q[b, h, :] . k_r) v_r
 * with k_r, v_r the decoded values of token r in its page's formats. Only the
 * pages the window reaches are read, and they are checked first (ids inside
 * [0, n_pages), contiguous, lengths, formats and parameters, payloads inside
 * the arena); a stream that fails raises SWRT_FLAG_BAD_PAGES and its query
 * heads' outputs are left as they were. An empty stream writes zeros.
 * n_layers 1 .. SWRT_MAX_LAYERS; q_heads a multiple of kv_heads (a group of
 * more than 16 query heads per KV head runs as several waves per stream, 16
 * heads each, which all read the stream's pages); head_dim in
 * {32, 64, 128, 256}; q_type, out_type SWRT_XF_F32 / _F16 / _BF16; scale
 * finite. Status codes for bad arguments; d_flags device uint32 or NULL.
 * page_formats: the page formats the caller's visible pages may have, bit
 * (1 << f) for each SWRT_XF_* format f (F32 .. UINT2), or 0 for any. A page
 * of a format outside a non-zero set fails its checks (SWRT_FLAG_BAD_PAGES
 * for its stream). A set without SWRT_XF_F32 and SWRT_XF_F16 runs a build of
 * the kernel without their tile paths: fewer registers, more waves per SIMD;
 * a set of SWRT_XF_BF16 and SWRT_XF_INT8 alone (either or both) a build for
 * those two formats only, the fastest. Other bits: SWRT_E_INVALID_ARG.
 */
int swrt_paged_attention(int n_layers, const swrt_paged_layer *layers, int64_t left_window,
                         int batch, int q_heads, int kv_heads, int head_dim, float scale,
                         int q_type, int out_type, uint32_t page_formats, uint32_t *d_flags,
                         void *stream);

/*
 * swrt_paged_quantize -- selected-block conversion ("Selected-block
 * quantization": QuantizePagedCache) inside one arena. Each page
 * pages_in[blocks[i]] is decoded (dense: its value; affine: (c - zero_point)
 * * scale rounded once to binary32) and its rows written in the target
 * formats at dst_offsets[2 i] (K) and dst_offsets[2 i + 1] (V): SWRT_XF_F32
 * as is, F16 / BF16 rounded to nearest even, NaN as the positive canonical
 * quiet NaN; affine targets saturate(round_half_even(y / scale) +
 * zero_point), NaN -> zero_point, packed. Rows [length, capacity) become
 * logical zeros of the target (0.0 or the zero point's code) without reading
 * the source. Then pages_out (may equal pages_in) receives every descriptor
 * of pages_in, the selected ones with the new formats, parameters (a dense
 * target: scale 1, zero point 0) and offsets.
 * Everything is checked on the device before anything is written: every
 * page of pages_in (valid, payloads inside the arena and outside the free
 * region [free_begin, free_end)); blocks strictly ascending inside
 * [0, n_pages); destinations in the order K0, V0, K1, V1, ... each at or
 * after the end of the one before, 16-byte aligned, inside the free region.
 * A failure raises SWRT_FLAG_BAD_PAGES and nothing is written. d_flags is
 * required and its SWRT_FLAG_BAD_PAGES bit must be clear on entry (a set bit
 * also stops the conversion). blocks, dst_offsets (int32[n_blocks],
 * int64[2 n_blocks]), pages_in and pages_out are device memory. Targets are
 * checked on the host (formats, scale > 0 and finite, zero points in range).
 */
int swrt_paged_quantize(void *arena, int64_t arena_bytes, const swrt_page *pages_in,
                        int64_t n_pages, const int32_t *blocks, int64_t n_blocks,
                        const int64_t *dst_offsets, int64_t free_begin, int64_t free_end,
                        swrt_page *pages_out, int k_format, float k_scale,
                        int32_t k_zero_point, int v_format, float v_scale,
                        int32_t v_zero_point, int head_dim, uint32_t *d_flags, void *stream);

/*
 * swrt_paged_append -- append with sealed blocks (section "Optional
 * heterogeneous paged KV": partial blocks are sealed, so an append adds new
 * blocks and never rewrites an earlier, partly filled one; the selected
 * format is stored in every new block; affine appends use scalar
 * parameters). Every stream s < n_streams of every layer appends seq_len
 * tokens as ONE new block:
 *   descriptor  pages[first_id + s], written whole: start = T (the stream's
 *               last block's start + length; 0 for a stream without
 *               blocks), length = capacity = seq_len, the call's formats and
 *               parameters (a dense format: scale 1, zero point 0)
 *   payload     K at free_begin + s * (kb + vb), V at that + kb, where kb, vb
 *               are the bytes of seq_len rows of head_dim elements in
 *               k_format / v_format; rows encoded from k_new / v_new
 *               ([n_streams, seq_len, head_dim] of new_type F32 / F16 / BF16,
 *               16-byte aligned) as swrt_paged_quantize encodes
 *   block table page_ids[s * page_stride + page_count[s]] = first_id + s,
 *               then page_count[s] + 1 (slotted rows: page_count required)
 * Only the last block's descriptor is read; no earlier payload, descriptor
 * or slot is written. A stream whose page_count is out of [0, page_stride],
 * or whose last block fails its checks (id in [0, n_pages) and not among the
 * ids this call hands out, a valid page), raises SWRT_FLAG_BAD_PAGES; one
 * with all page_stride slots in use, SWRT_FLAG_PAGE_FULL; either is skipped
 * and its id and payload room stay untouched. The caller keeps the free
 * region clear of live payload (not checked: it would cost a pass over every
 * page) and first_id .. first_id + n_streams - 1 clear of live descriptors.
 *
 * n_layers 1 .. SWRT_MAX_LAYERS: each layer's arena gets its own payloads
 * (at the same offsets); layers either share all of pages, page_count and
 * page_ids (the descriptors and the table then grow once, and their arenas
 * must be equally long) or share none of them. d_flags may be NULL.
 * SWRT_E_INVALID_ARG (nothing launched): a bad format or parameter, seq_len
 * < 1, first_id outside [0, n_pages - n_streams], a free region outside the
 * arena or too small for n_streams payloads, n_streams * page_stride > n_ids.
 * SWRT_E_UNSUPPORTED (library layout rule): head_dim not a multiple of 16 in
 * [16, 4096], free_begin, kb or vb not a multiple of 16.
 */
int swrt_paged_append(int n_layers, const swrt_paged_layer *layers, const void *const *k_new,
                      const void *const *v_new, int new_type, int n_streams, int seq_len,
                      int head_dim, int64_t first_id, int64_t free_begin, int64_t free_end,
                      int k_format, float k_scale, int32_t k_zero_point, int v_format,
                      float v_scale, int32_t v_zero_point, uint32_t *d_flags, void *stream);

/*
 * swrt_paged_append_open -- open-page append, an extension beside the pages'
 * sealed rule (it rewrites the last block, which a sealed cache never does):
 * stream s writes k_new[s, :] and v_new[s, :] (new_type F32 / F16 / BF16,
 * [n_streams, head_dim], 16-byte aligned) as row `length` of its last page,
 * encoded in that page's formats as swrt_paged_quantize encodes, and that
 * page's length grows by one (on the device). A stream without pages or
 * whose last page fails its checks raises SWRT_FLAG_BAD_PAGES, one whose
 * last page is full SWRT_FLAG_PAGE_FULL; either is skipped. n_layers 1 ..
 * SWRT_MAX_LAYERS, each with its own arena and either block-table form;
 * layers either share all of pages, page_ptr / page_count and page_ids (the
 * lengths grow once) or none. head_dim a multiple of 16 in [16, 4096].
 */
int swrt_paged_append_open(int n_layers, const swrt_paged_layer *layers, const void *const *k_new,
                           const void *const *v_new, int new_type, int n_streams, int head_dim,
                           uint32_t *d_flags, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *swrt_status_string(int status);

/* SWRT_ABI_VERSION of the built library. */
int swrt_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWRT_H */
