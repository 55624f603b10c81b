/*
 * swrt_oracle.h -- plain CPU oracle for the sliding-window KV-cache update path.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the package smoke check and the
 * benchmark's CPU-baseline leg are the only users of this library. The GPU
 * product path never includes this header, links this library or calls it, and
 * this code includes nothing from the GPU path: the two share no header, helper,
 * constant or table. The status and flag values below are written out here on
 * their own; the tests compare them with the product library's values.
 *
 * Sources (pages, by title and section):
 *   [TS]  ONNX operator "TensorScatter" (domain ai.onnx, since version 24):
 *         description, pseudocode, Inputs, Outputs, Attributes, Type Constraints.
 *   [RB]  Core AI model zoo, "Stateful decode & KV cache", section
 *         "Sliding-window ring buffer (long-context memory)".
 *   [GQA] onnxruntime pull request "GQA support sliding_window_cache" (#29904):
 *         section "Design" (the invariant and the append formulas, and the two
 *         details that follow them), and the follow-up commit that widens the
 *         end-pointer arithmetic to 64 bits and clamps the past length at zero.
 *   [GQA-CPU] the same pull request's CPU follow-up description, section "Key
 *         design decisions": the drifting layout (gap, end pointer, one
 *         compaction per gap decode steps).
 *   [GQA-ROPE] the same pull request's "Summary of Changes": the KV append
 *         writes at the cache-relative offset while RoPE keeps the absolute
 *         position, bounded by its own maximum position, not by the capacity.
 *   [ATT] onnx-light-cpu "Persistent KV Cache and Decode Performance
 *         Roadmap", section "Phase 1: decode with contiguous KV cache"
 *         (streaming decode attention, GQA head grouping), with [GQA] "Design"
 *         (the invariant and the local window) and [RB] (attention over the
 *         ring under a position mask; slot order does not change scores).
 *   [PF]  onnx-light how-to "Persistent input/output feedback", section
 *         "Optional heterogeneous paged KV" ("Selected-block quantization",
 *         "Serialized cache values"): affine INT8/UINT8 codes with FLOAT
 *         scales, scalar parameters on append, rounding ties to even and
 *         saturating to the code range.
 *   [PF-PAGED] the same section as a whole: pages with start, length and
 *         capacity, contiguous from zero; dense FLOAT/FLOAT16/BFLOAT16 or
 *         affine INT8/UINT8/INT4/UINT4/INT2/UINT2 payloads, independently for
 *         K and V and per page; QuantizePagedCache on selected blocks (valid
 *         prefix converted, unused rows logical zeros, all checks before
 *         anything is published); attention reading only visible tokens with
 *         a left window bounding the preceding tokens.
 *
 * Every function is a plain definition: scalar loops, one memcpy per row, no
 * blocking, no vector code, no threads.
 */
#ifndef SWRT_ORACLE_H
#define SWRT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* synchronous status codes */
#define ORC_OK 0
#define ORC_E_INVALID_ARG 1
#define ORC_E_UNSUPPORTED 2

/* per-call data flags (OR-ed into *flags) */
#define ORC_FLAG_LINEAR_OOB 1u  /* a linear write index left [0, M-S]; batch skipped */
#define ORC_FLAG_BAD_SEQLEN 2u  /* seqlens_k[b] < 0 or total length < S; clamped   */
#define ORC_FLAG_BAD_LENGTHS 4u /* (Lp, E) inconsistent with (C, S); batch skipped */
#define ORC_FLAG_ROPE_RANGE 8u  /* a rotary position outside [0, max); batch skipped */

/* TensorScatter "mode" attribute */
#define ORC_MODE_LINEAR 0
#define ORC_MODE_CIRCULAR 1

/* phases of a multi-token windowed step */
#define ORC_PHASE_STAGE 1u
#define ORC_PHASE_COMMIT 2u
#define ORC_PHASE_ALL 3u

#define ORC_MAX_RANK 8

/*
 * [TS] present = TensorScatter(past, update, write_indices; axis, mode).
 * shape: host array of `rank` dims of past (update has seq_len on `axis`).
 * write_indices: host int64[shape[0]] or NULL (all zeros).
 * present may equal past (in place); otherwise present first gets past's bytes.
 * elem_bits in {4, 8, 16, 32, 64, 128}; 4-bit needs an even row length.
 */
int orc_tensor_scatter(void *present, const void *past, const void *update,
                       const int64_t *write_indices, const int64_t *shape,
                       int rank, int axis, int64_t seq_len, int mode,
                       int elem_bits, uint32_t *flags);

/*
 * [GQA] lengths of one windowed step, for every batch entry.
 * T = seqlens_k + 1, P = max(0, T - S), Lp = min(P, C),
 * E = max(0, Lp + S - C), L = Lp + S - E  (all in 64-bit arithmetic).
 * total_lens, past_lens, cache_total_lens may be NULL.
 * work_offsets (int64[batch + 1], may be NULL): the exclusive prefix over the
 * batch of the rows each entry's step writes, r_b = (E_b > 0 ? Lp_b - E_b : 0)
 * + 1 for S = 1 (the shifted rows and the appended one) and Lp_b + S for
 * S > 1 (the staged rows); work_offsets[batch] is the total.
 */
int orc_kv_seq_lengths(const int32_t *seqlens_k, int64_t batch, int64_t seq_len,
                       int64_t capacity, int64_t *total_lens, int64_t *past_lens,
                       int32_t *cache_past_lens, int32_t *cache_total_lens,
                       int32_t *evict_counts, int64_t *work_offsets, uint32_t *flags);

/*
 * [GQA-CPU] lengths of one windowed step under the drifting layout of the
 * CPU follow-up ("Key design decisions", "Drifting layout"): with gap =
 * C - W + 1 the append point is end(x) = x while x <= C, else
 * x - gap * ceil((x - C) / gap). T = seqlens_k + 1, P = max(0, T - S),
 * Lp = end(P), L = end(T), E = Lp + S - L. W = C (gap 1) is the base method.
 * 1 <= window <= capacity. work_offsets as for orc_kv_seq_lengths.
 */
int orc_kv_seq_lengths_drift(const int32_t *seqlens_k, int64_t batch,
                             int64_t seq_len, int64_t capacity, int64_t window,
                             int64_t *total_lens, int64_t *past_lens,
                             int32_t *cache_past_lens, int32_t *cache_total_lens,
                             int32_t *evict_counts, int64_t *work_offsets, uint32_t *flags);

/*
 * [GQA] one windowed cache step for K and V.
 * caches [B, H, C, D]; new rows addressed by new_strides (elements) for b, h, s
 * with D contiguous; staging [B, H, C+S, D] (needed iff S > 1).
 * S == 1: in place, shift then append. S > 1: STAGE and/or COMMIT.
 * A batch entry whose (Lp, E) is not a step that fits (0 <= Lp <= C, E >= 0,
 * 1 <= Lp + S - E <= C) is flagged and left untouched.
 */
int orc_kv_window_append(void *k_cache, void *v_cache, const void *k_new,
                         const void *v_new, const int64_t *new_strides,
                         void *k_staging, void *v_staging,
                         const int32_t *cache_past_lens,
                         const int32_t *evict_counts, int64_t batch,
                         int64_t kv_heads, int64_t capacity, int64_t seq_len,
                         int64_t head_dim, int elem_bits, unsigned phase,
                         uint32_t *flags);

/* ------------------------------------------------------------------------ */
/* the row transform of a fused append: RoPE on K, then conversion or affine   */
/* quantization into the cache's element type                                  */
/* ------------------------------------------------------------------------ */
#define ORC_XF_F32 1
#define ORC_XF_F16 2
#define ORC_XF_BF16 3
#define ORC_XF_INT8 4
#define ORC_XF_UINT8 5
#define ORC_XF_FP8_E4M3 10 /* OCP float8 E4M3 (float8e4m3fn), scaled, saturating */

typedef struct {
    int in_type;            /* new rows: ORC_XF_F32, ORC_XF_F16 or ORC_XF_BF16 */
    int out_type;           /* cache rows: any ORC_XF_* type */
    const float *cos_table; /* [max_position, rotary_dim / 2]; NULL: no rotation */
    const float *sin_table; /* same shape; NULL exactly when cos_table is */
    int64_t max_position;   /* rows of the tables */
    int64_t rotary_dim;     /* even, 2 .. head_dim; later elements pass unrotated */
    int interleaved;        /* 0: pairs (j, j + rotary_dim/2); 1: pairs (2j, 2j+1) */
    float scale[2];         /* K, V scales: positive and finite (INT8 / UINT8 / FP8) */
    int32_t zero_point[2];  /* K, V zero points: inside the code range (0 for FP8) */
    /* per-channel parameters, shape [kv_heads, 1, head_dim] with the singleton
     * dimension dropped: element i of a row of KV head h takes entry
     * h * head_dim + i instead of the scalar. NULL: the scalar. Scales for
     * INT8 / UINT8 / FP8 targets, zero points for INT8 / UINT8 only. Table
     * entries are data (not checked): the formulas apply as written, a NaN
     * taking the zero point saturated into the code range. */
    const float *channel_scale[2];
    const int32_t *channel_zero_point[2];
} orc_row_xf;

/*
 * One row of head_dim elements of KV head `head`: read as float, rotate when
 * t == 0 (K) and tables are given, using table row `pos`; then write in
 * out_type. Every float operation is one IEEE binary32 operation, rounded to
 * nearest even:
 *   x0' = fl(fl(x0 * c) - fl(x1 * s)),  x1' = fl(fl(x1 * c) + fl(x0 * s)).
 * bf16 / f16 outputs round to nearest even (overflow -> infinity); every
 * float output stores NaN as the positive canonical quiet NaN of its type;
 * integer outputs are
 * saturate(round_half_even(fl(y / scale)) + zero_point), NaN -> zero_point;
 * FP8 outputs are E4M3(fl(y / scale)), nearest even, saturating at +-448.
 * scale and zero_point are element i's (per-channel tables) or the scalars.
 * Returns ORC_E_INVALID_ARG on a bad transform or a position outside the
 * tables.
 */
int orc_xf_row(const orc_row_xf *x, int t, int64_t head, int64_t pos, const void *in, void *out,
               int64_t head_dim);

/*
 * [GQA] + [GQA-ROPE] + [PF]: orc_kv_window_append whose new rows (in_type,
 * new_strides in elements) first pass through the transform, row s of batch
 * entry b at absolute position past_lens[b] + s; caches and staging hold
 * out_type rows. A batch entry whose lengths do not fit is flagged
 * BAD_LENGTHS and skipped; then one whose positions leave [0, max_position)
 * (rotation on) is flagged ROPE_RANGE and skipped.
 */
int orc_kv_window_append_xf(void *k_cache, void *v_cache, const void *k_new,
                            const void *v_new, const int64_t *new_strides,
                            void *k_staging, void *v_staging,
                            const int32_t *cache_past_lens,
                            const int32_t *evict_counts, const int64_t *past_lens,
                            int64_t batch, int64_t kv_heads, int64_t capacity,
                            int64_t seq_len, int64_t head_dim, unsigned phase,
                            const orc_row_xf *x, uint32_t *flags);

/*
 * [TS] + [GQA-ROPE] + [PF]: TensorScatter with axis = rank - 2 (a row is the
 * last dimension, head_dim) whose update rows (in_type) pass through the
 * transform first, update row s of batch entry b at absolute position
 * write_indices[b] + s (before any circular wrap). present / past hold
 * out_type rows. Per-channel tables, if any, are [shape[1], head_dim] for
 * rank 4 ([B, H, M, D]: prefix index 1 is the KV head) and [1, head_dim] for
 * rank 3; rank > 4 takes none. `t` selects K (0: rotated) or V (1). A linear entry out of
 * range is flagged LINEAR_OOB and skipped; then an entry whose positions leave
 * [0, max_position) (rotation on) is flagged ROPE_RANGE and skipped (keeping
 * past's rows).
 */
int orc_tensor_scatter_xf(void *present, const void *past, const void *update,
                          const int64_t *write_indices, const int64_t *shape,
                          int rank, int64_t seq_len, int mode, int t,
                          const orc_row_xf *x, uint32_t *flags);

/* ------------------------------------------------------------------------ */
/* windowed decode attention                                                 */
/* ------------------------------------------------------------------------ */

/*
 * [ATT] one-token decode attention over each batch entry's visible window of
 * a windowed cache, for every query head (the onnx-light-cpu roadmap, "Phase
 * 1: decode with contiguous KV cache": q.K dot products, softmax, weighted
 * V; GQA query heads share their KV head). In float64 from the decoded
 * elements:
 *   rows  r in [max(0, L_b - W), L_b)      (the last W resident tokens)
 *   kv    g = h / (Hq / Hkv)
 *   s_r   = scale * sum_d q[b,h,d] * k[b,g,r,d]
 *   o     = sum_r exp(s_r - max s) v[b,g,r,:] / sum_r exp(s_r - max s)
 * q [B, Hq, D], caches [B, Hkv, C, D] of elem_type (ORC_XF_F32 / F16 /
 * BF16), out [B, Hq, D] float64. An empty window (L_b = 0) gives zeros; an
 * entry with L_b < 0 or L_b > C is flagged BAD_LENGTHS and its outputs are
 * left as they were. Hq must be a multiple of Hkv; W >= 1.
 */
int orc_window_attention(const void *q, const void *k_cache, const void *v_cache,
                         double *out, const int32_t *cache_total_lens, int64_t window,
                         int64_t batch, int64_t q_heads, int64_t kv_heads,
                         int64_t capacity, int64_t head_dim, double scale, int elem_type,
                         uint32_t *flags);

/* ------------------------------------------------------------------------ */
/* paged caches with per-page formats                                         */
/* ------------------------------------------------------------------------ */

/* page formats beyond the row transform's: sub-byte affine codes */
#define ORC_XF_INT4 6
#define ORC_XF_UINT4 7
#define ORC_XF_INT2 8
#define ORC_XF_UINT2 9

#define ORC_FLAG_BAD_PAGES 16u /* a page table or page descriptor failed its checks */
#define ORC_FLAG_PAGE_FULL 32u /* an append found its page full; stream skipped      */

/*
 * [PF-PAGED] one page (block) of a paged cache: tokens [start, start + length)
 * of one stream (batch entry, KV head), capacity physical rows of K and of V
 * at byte offsets of an arena. Dense formats (ORC_XF_F32 / F16 / BF16) hold
 * values; affine formats (INT8, UINT8, INT4, UINT4, INT2, UINT2) hold codes c
 * with value (c - zero_point) * scale. A K (or V) payload is the block's
 * logical tensor [1, 1, capacity, head_size] stored flat: element e of row r
 * is element r * head_size + e; sub-byte codes pack from the least
 * significant bits of each byte (element 0 in the low bits), one after
 * another across row ends, the last byte padded; signed codes in two's
 * complement. The layout is the GPU library's page descriptor (64 bytes),
 * defined here on its own.
 */
typedef struct {
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
} orc_page;

/*
 * [PF-PAGED] the block table names each stream's pages in token order, as
 * ids into the descriptor array, in one of two forms:
 *   compressed rows  page_count NULL: stream s owns
 *                    page_ids[page_ptr[s] .. page_ptr[s + 1]);
 *   slotted rows     page_count given: stream s owns the page_stride slots
 *                    from s * page_stride and uses the first page_count[s]
 *                    (0 <= page_count[s] <= page_stride); page_ptr unused.
 */

/*
 * [PF-PAGED] + [ATT]: one-token decode attention over paged caches. Stream
 * s = b * kv_heads + g owns its pages through the block table; its length T
 * is the last page's start + length (0 without pages). Query head h of entry
 * b reads stream b * kv_heads + h / (Hq / Hkv) over tokens
 * [max(0, T - 1 - left_window), T) (left_window < 0: all T; the query is
 * token T - 1 and left_window bounds the tokens before it), in float64 from
 * the exactly decoded values:
 *   o = sum_r exp(s_r - max s) v_r / sum_r exp(s_r - max s),  s_r = scale q.k_r
 * q [B, Hq, D] of q_type (F32 / F16 / BF16); out [B, Hq, D] float64.
 * The pages the window reaches must be contiguous (each start the previous
 * start + length, the first page starting at 0), 1 <= length <= capacity, of
 * valid formats and parameters (scale > 0 and finite, zero point in the code
 * range) and inside the arena; page ids must be in [0, n_pages) and the
 * stream's range of the block table inside [0, n_ids). A stream that fails is
 * flagged BAD_PAGES and the outputs of its query heads are left as they were;
 * pages before the window are not read. An empty window gives zeros.
 */
int orc_paged_attention(const void *q, int q_type, const char *arena, int64_t arena_bytes,
                        const orc_page *pages, int64_t n_pages, const int32_t *page_ptr,
                        const int32_t *page_count, int64_t page_stride,
                        const int32_t *page_ids, int64_t n_ids, double *out,
                        int64_t left_window, int64_t batch, int64_t q_heads,
                        int64_t kv_heads, int64_t head_dim, double scale, uint32_t *flags);

/*
 * [PF-PAGED] selected-block conversion inside one arena: each page
 * pages_in[blocks[i]] is decoded (dense: its value; affine: fl((c -
 * zero_point) * scale) in binary32) and its rows written in the target
 * formats at dst_offsets[2 i] (K) and dst_offsets[2 i + 1] (V): F32 as is
 * (NaN canonical), F16 / BF16 rounded to nearest even (NaN canonical), affine
 * formats as saturate(round_half_even(fl(y / scale)) + zero_point) (NaN ->
 * zero point), packed (padding bits zero). Rows [length, capacity) are
 * written as logical zeros of the target (0.0, or the zero point's code)
 * without reading the source. pages_out (may be pages_in) is pages_in with
 * the selected descriptors' formats, parameters and offsets replaced; a
 * dense target's scale is 1 and zero point 0. Everything is checked first:
 * every page of pages_in (valid, its payloads outside the free region
 * [free_begin, free_end)); the indices strictly ascending in [0, n_pages);
 * the targets; the destinations in the order K0, V0, K1, V1, ... each at or
 * after the end of the one before, inside the free region. On any failure
 * nothing is written and the call returns ORC_E_INVALID_ARG.
 */
int orc_paged_quantize(char *arena, int64_t arena_bytes, const orc_page *pages_in,
                       int64_t n_pages, const int32_t *blocks, int64_t n_blocks,
                       const int64_t *dst_offsets, int64_t free_begin, int64_t free_end,
                       orc_page *pages_out, int k_format, float k_scale, int32_t k_zero_point,
                       int v_format, float v_scale, int32_t v_zero_point, int64_t head_dim);

/*
 * [PF-PAGED] append with sealed blocks ("Partial blocks are sealed": an append
 * adds new blocks and never rewrites an earlier, partly filled one). Every
 * stream s < n_streams appends seq_len tokens as ONE new block:
 *   id        first_id + s (descriptor pages[id] is written whole)
 *   start     T, the stream's length (its last block's start + length; 0 for
 *             a stream without blocks)
 *   length    = capacity = seq_len
 *   payload   K at free_begin + s * (kb + vb), V right after it, where kb and
 *             vb are the packed payload bytes of seq_len rows of k_head_dim /
 *             v_head_dim elements in k_format / v_format
 *   formats   the call's k_format / v_format with their scalar parameters (a
 *             dense format: scale 1, zero point 0), rows encoded from k_new /
 *             v_new ([n_streams, seq_len, head_dim] of new_type) as
 *             orc_paged_quantize encodes
 * and the block table's next slot of the stream, page_ids[s * page_stride +
 * page_count[s]], receives id, page_count[s] growing by one (slotted rows
 * only). No earlier block, descriptor or payload byte is read beyond the
 * last block's descriptor, and none is written. A stream whose slot count is
 * out of range, or whose last block fails its checks (id in [0, n_pages) and
 * not one this call hands out, a valid page), is flagged BAD_PAGES; one with
 * all page_stride slots in use, PAGE_FULL; either is skipped and its id and
 * payload room stay untouched. ORC_E_INVALID_ARG (nothing written) for bad
 * arguments: formats, ids past n_pages, a free region too small for
 * n_streams payloads or outside the arena, slots past n_ids.
 * *written_bytes (may be NULL) receives the payload bytes written.
 */
int orc_paged_append(char *arena, int64_t arena_bytes, orc_page *pages, int64_t n_pages,
                     int32_t *page_count, int64_t page_stride, int32_t *page_ids, int64_t n_ids,
                     const void *k_new, const void *v_new, int new_type, int64_t n_streams,
                     int64_t seq_len, int64_t k_head_dim, int64_t v_head_dim, int64_t first_id,
                     int64_t free_begin, int64_t free_end, int k_format, float k_scale,
                     int32_t k_zero_point, int v_format, float v_scale, int32_t v_zero_point,
                     uint32_t *flags, int64_t *written_bytes);

/*
 * Open-block append, an extension beside the pages' sealed rule: stream s
 * writes its new K and V rows (new_type F32 / F16 / BF16, [n_streams,
 * head_dim]) as row `length` of its last page, encoded in that page's
 * formats as orc_paged_quantize encodes, and the page's length grows by one.
 * A stream without pages, or whose last page is invalid, is flagged
 * BAD_PAGES; one whose last page is full, PAGE_FULL; either is skipped.
 * Either block-table form.
 */
int orc_paged_append_open(char *arena, int64_t arena_bytes, orc_page *pages, int64_t n_pages,
                          const int32_t *page_ptr, const int32_t *page_count, int64_t page_stride,
                          const int32_t *page_ids, int64_t n_ids, const void *k_new,
                          const void *v_new, int new_type, int64_t n_streams, int64_t head_dim,
                          uint32_t *flags);

#ifdef __cplusplus
}
#endif

#endif /* SWRT_ORACLE_H */
