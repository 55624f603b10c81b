/*
 * swrt_oracle.c -- plain CPU oracle for the sliding-window KV-cache update path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg, never by the product path. It shares
 * no code with the GPU library. Source pages and the tags [TS], [RB], [GQA]
 * are listed in swrt_oracle.h.
 *
 * Readings taken where the pages leave a point open (each is also listed with
 * the design notes of the repository):
 *   - [TS] applies np.mod to the whole cache index tuple; here the modulo is
 *     applied to the sequence index only, which is the same whenever every
 *     prefix index is below max_sequence_length and is what the description
 *     says ("the write index is modulo max_sequence_length").
 *   - [TS] linear mode "requires" write_indices + sequence_length <=
 *     max_sequence_length; an entry that breaks it (or is negative) is
 *     flagged and its batch entry keeps the past values.
 *   - [GQA] seqlens_k holds the total length minus one: T = seqlens_k + 1,
 *     the reading under which the follow-up's "seqlens_k[b] + 1" overflow note
 *     applies. The past length T - S is clamped at zero.
 *   - [GQA] rows at and beyond the new resident length L are left untouched,
 *     as are staging rows at and beyond Lp + S.
 *   - [GQA] an S = 1 step shifts first, then writes: when E = 1 the row the
 *     new token goes to is one of the shift's sources.
 *   - the append accepts any (Lp, E) that describes a step fitting the cache
 *     (0 <= Lp <= C, L = Lp + S - E with 1 <= L <= C, E >= 0): the base
 *     lengths evict only what does not fit, the drifting layout of the CPU
 *     follow-up evicts a whole gap of rows at once; both are such steps.
 */
#include "swrt_oracle.h"

#include <stdlib.h>
#include <string.h>

static int valid_elem_bits(int bits)
{
    return bits == 4 || bits == 8 || bits == 16 || bits == 32 || bits == 64 ||
           bits == 128;
}

/* np.mod with a positive modulus: the result lies in [0, m). */
static int64_t floor_mod(int64_t a, int64_t m)
{
    int64_t r = a % m;
    return r < 0 ? r + m : r;
}

static void set_flag(uint32_t *flags, uint32_t bit)
{
    if (flags)
        *flags |= bit;
}

/* ------------------------------------------------------------------------ */
/* [TS] TensorScatter                                                        */
/* ------------------------------------------------------------------------ */

int orc_tensor_scatter(void *present, const void *past, const void *update,
                       const int64_t *write_indices, const int64_t *shape,
                       int rank, int axis, int64_t seq_len, int mode,
                       int elem_bits, uint32_t *flags)
{
    int64_t idx[ORC_MAX_RANK];
    int64_t M, S = seq_len, n_prefix = 1, inner = 1, total = 1, row_bytes;
    int d;

    if (!shape || rank < 2 || rank > ORC_MAX_RANK)
        return ORC_E_INVALID_ARG;
    for (d = 0; d < rank; ++d)
        if (shape[d] < 0)
            return ORC_E_INVALID_ARG;
    /* [TS Attributes] axis counts from the end when negative and cannot be
     * 0, the batch dimension. */
    if (axis < 0)
        axis += rank;
    if (axis < 1 || axis >= rank)
        return ORC_E_INVALID_ARG;
    if (mode != ORC_MODE_LINEAR && mode != ORC_MODE_CIRCULAR)
        return ORC_E_INVALID_ARG;
    if (!valid_elem_bits(elem_bits))
        return ORC_E_INVALID_ARG;
    M = shape[axis];
    /* [TS description] sequence_length <= max_sequence_length */
    if (S < 0 || S > M)
        return ORC_E_INVALID_ARG;
    for (d = 0; d < axis; ++d)
        n_prefix *= shape[d];
    for (d = axis + 1; d < rank; ++d)
        inner *= shape[d];
    for (d = 0; d < rank; ++d)
        total *= shape[d];
    if ((inner * elem_bits) % 8 != 0)
        return ORC_E_UNSUPPORTED; /* a row that does not end on a byte */
    row_bytes = inner * elem_bits / 8;
    if (total > 0 && (!present || !past))
        return ORC_E_INVALID_ARG;
    if (n_prefix * S * inner > 0 && !update)
        return ORC_E_INVALID_ARG;

    /* [TS description] the op is functional: present starts as past. */
    if (present != past && total > 0)
        memcpy(present, past, (size_t)(total / inner * row_bytes));
    if (n_prefix == 0 || S == 0 || row_bytes == 0)
        return ORC_OK;

    /* [TS pseudocode] for prefix_idx in ndindex(shape[:axis]), row-major;
     * o is the flat position of prefix_idx. */
    for (d = 0; d < axis; ++d)
        idx[d] = 0;
    for (int64_t o = 0; o < n_prefix; ++o) {
        const int64_t batch_idx = idx[0];
        const int64_t w = write_indices ? write_indices[batch_idx] : 0;

        if (mode == ORC_MODE_LINEAR && (w < 0 || w > M - S)) {
            set_flag(flags, ORC_FLAG_LINEAR_OOB);
        } else {
            for (int64_t s = 0; s < S; ++s) {
                int64_t j;
                if (mode == ORC_MODE_CIRCULAR)
                    j = floor_mod(floor_mod(w, M) + s, M); /* (w + s) mod M */
                else
                    j = w + s;
                /* present[(*prefix_idx, j)] = update[(*prefix_idx, s)] */
                memcpy((char *)present + (o * M + j) * row_bytes,
                       (const char *)update + (o * S + s) * row_bytes,
                       (size_t)row_bytes);
            }
        }
        for (d = axis - 1; d >= 0; --d) { /* next prefix_idx */
            if (++idx[d] < shape[d])
                break;
            idx[d] = 0;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* [GQA] lengths of a windowed step                                         */
/* ------------------------------------------------------------------------ */

int orc_kv_seq_lengths(const int32_t *seqlens_k, int64_t batch, int64_t seq_len,
                       int64_t capacity, int64_t *total_lens, int64_t *past_lens,
                       int32_t *cache_past_lens, int32_t *cache_total_lens,
                       int32_t *evict_counts, uint32_t *flags)
{
    const int64_t S = seq_len, C = capacity;

    if (batch < 0 || S < 1 || C < 1 || S > INT32_MAX || C > INT32_MAX)
        return ORC_E_INVALID_ARG;
    if (batch > 0 && (!seqlens_k || !cache_past_lens || !evict_counts))
        return ORC_E_INVALID_ARG;

    for (int64_t b = 0; b < batch; ++b) {
        const int64_t T = (int64_t)seqlens_k[b] + 1; /* absolute total length */
        int64_t P, Lp, E, L;

        if (seqlens_k[b] < 0 || T < S)
            set_flag(flags, ORC_FLAG_BAD_SEQLEN);
        P = T - S; /* absolute past length, clamped at zero */
        if (P < 0)
            P = 0;
        Lp = P < C ? P : C;  /* tokens currently resident */
        E = Lp + S - C;      /* tokens evicted by this step */
        if (E < 0)
            E = 0;
        L = Lp + S - E;      /* resident after the step */

        if (total_lens)
            total_lens[b] = T;
        if (past_lens)
            past_lens[b] = P;
        cache_past_lens[b] = (int32_t)Lp;
        evict_counts[b] = (int32_t)E;
        if (cache_total_lens)
            cache_total_lens[b] = (int32_t)L;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* [GQA-CPU] drifting layout: lengths of a windowed step                     */
/* ------------------------------------------------------------------------ */

/* The append point of the drifting layout for an absolute length x: with
 * gap = C - W + 1 it is x while x <= C, afterwards x minus as many whole gaps
 * as it takes to come back to at most C (so W <= end <= C). */
static int64_t drift_end(int64_t x, int64_t C, int64_t gap)
{
    int64_t gaps;
    if (x <= C)
        return x;
    gaps = (x - C + gap - 1) / gap; /* ceil((x - C) / gap), 64-bit */
    return x - gap * gaps;
}

int orc_kv_seq_lengths_drift(const int32_t *seqlens_k, int64_t batch,
                             int64_t seq_len, int64_t capacity, int64_t window,
                             int64_t *total_lens, int64_t *past_lens,
                             int32_t *cache_past_lens, int32_t *cache_total_lens,
                             int32_t *evict_counts, uint32_t *flags)
{
    const int64_t S = seq_len, C = capacity, W = window;

    if (batch < 0 || S < 1 || C < 1 || S > INT32_MAX || C > INT32_MAX)
        return ORC_E_INVALID_ARG;
    if (W < 1 || W > C)
        return ORC_E_INVALID_ARG;
    if (batch > 0 && (!seqlens_k || !cache_past_lens || !evict_counts))
        return ORC_E_INVALID_ARG;

    for (int64_t b = 0; b < batch; ++b) {
        const int64_t gap = C - W + 1;
        const int64_t T = (int64_t)seqlens_k[b] + 1;
        int64_t P, Lp, L, E;

        if (seqlens_k[b] < 0 || T < S)
            set_flag(flags, ORC_FLAG_BAD_SEQLEN);
        P = T - S;
        if (P < 0)
            P = 0;
        Lp = drift_end(P, C, gap);     /* resident before the step */
        L = drift_end(P + S, C, gap);  /* resident after the step */
        E = Lp + S - L;                /* rows reclaimed by the step */

        if (total_lens)
            total_lens[b] = T;
        if (past_lens)
            past_lens[b] = P;
        cache_past_lens[b] = (int32_t)Lp;
        evict_counts[b] = (int32_t)E;
        if (cache_total_lens)
            cache_total_lens[b] = (int32_t)L;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* [GQA] windowed step: shift + append (S = 1), stage / commit (S > 1)       */
/* ------------------------------------------------------------------------ */

static void copy_row(char *dst, const char *src, int64_t row_bytes)
{
    memcpy(dst, src, (size_t)row_bytes);
}

int orc_kv_window_append(void *k_cache, void *v_cache, const void *k_new,
                         const void *v_new, const int64_t *new_strides,
                         void *k_staging, void *v_staging,
                         const int32_t *cache_past_lens,
                         const int32_t *evict_counts, int64_t batch,
                         int64_t kv_heads, int64_t capacity, int64_t seq_len,
                         int64_t head_dim, int elem_bits, unsigned phase,
                         uint32_t *flags)
{
    const int64_t B = batch, H = kv_heads, C = capacity, S = seq_len;
    int64_t row_bytes, nb_stride[3];
    char *caches[2], *stagings[2];
    const char *news[2];
    char *tmp;

    if (B < 0 || H < 0 || head_dim < 0 || C < 1 || S < 1)
        return ORC_E_INVALID_ARG;
    if (!valid_elem_bits(elem_bits))
        return ORC_E_INVALID_ARG;
    if (S > 1 && phase != ORC_PHASE_STAGE && phase != ORC_PHASE_COMMIT &&
        phase != ORC_PHASE_ALL)
        return ORC_E_INVALID_ARG;
    if ((head_dim * elem_bits) % 8 != 0)
        return ORC_E_UNSUPPORTED;
    row_bytes = head_dim * elem_bits / 8;
    if (B == 0 || H == 0 || row_bytes == 0)
        return ORC_OK;
    if (!k_cache || !v_cache || !k_new || !v_new || !new_strides ||
        !cache_past_lens || !evict_counts)
        return ORC_E_INVALID_ARG;
    if (S > 1 && (!k_staging || !v_staging))
        return ORC_E_INVALID_ARG;
    for (int i = 0; i < 3; ++i) {
        if ((new_strides[i] * elem_bits) % 8 != 0)
            return ORC_E_UNSUPPORTED;
        nb_stride[i] = new_strides[i] * elem_bits / 8; /* bytes */
    }

    caches[0] = (char *)k_cache;
    caches[1] = (char *)v_cache;
    news[0] = (const char *)k_new;
    news[1] = (const char *)v_new;
    stagings[0] = (char *)k_staging;
    stagings[1] = (char *)v_staging;
    tmp = (char *)malloc((size_t)(C * row_bytes));
    if (!tmp)
        return ORC_E_INVALID_ARG;

    for (int64_t b = 0; b < B; ++b) {
        const int64_t Lp = cache_past_lens[b];
        const int64_t E = evict_counts[b];
        const int64_t L = Lp + S - E;

        /* the step must fit: Lp resident rows, at least the rows that do not
         * fit the capacity evicted, and at least one row left */
        if (Lp < 0 || Lp > C || E < 0 || L > C || L < 1) {
            set_flag(flags, ORC_FLAG_BAD_LENGTHS);
            continue; /* this batch entry keeps every byte it had */
        }

        for (int t = 0; t < 2; ++t) { /* K, then V */
            for (int64_t h = 0; h < H; ++h) {
                char *cache = caches[t] + (b * H + h) * C * row_bytes;
                const char *nw = news[t] + b * nb_stride[0] + h * nb_stride[1];

                if (S == 1) {
                    /* shift: cache[E .. Lp) -> cache[0 .. Lp-E), through a
                     * snapshot so that the overlap cannot matter */
                    for (int64_t r = E; r < Lp; ++r)
                        copy_row(tmp + (r - E) * row_bytes, cache + r * row_bytes,
                                 row_bytes);
                    for (int64_t r = 0; r < Lp - E; ++r)
                        copy_row(cache + r * row_bytes, tmp + r * row_bytes,
                                 row_bytes);
                    /* write: new tokens -> cache[Lp-E .. Lp-E+S) */
                    for (int64_t s = 0; s < S; ++s)
                        copy_row(cache + (Lp - E + s) * row_bytes,
                                 nw + s * nb_stride[2], row_bytes);
                } else {
                    char *stage = stagings[t] + (b * H + h) * (C + S) * row_bytes;
                    if (phase & ORC_PHASE_STAGE) {
                        /* seed the C+S staging cache with the resident rows,
                         * then append the S new rows after them */
                        for (int64_t r = 0; r < Lp; ++r)
                            copy_row(stage + r * row_bytes, cache + r * row_bytes,
                                     row_bytes);
                        for (int64_t s = 0; s < S; ++s)
                            copy_row(stage + (Lp + s) * row_bytes,
                                     nw + s * nb_stride[2], row_bytes);
                    }
                    if (phase & ORC_PHASE_COMMIT) {
                        /* copy the surviving window back:
                         * cache[0 .. L) = staging[E .. E+L) */
                        for (int64_t r = 0; r < L; ++r)
                            copy_row(cache + r * row_bytes,
                                     stage + (E + r) * row_bytes, row_bytes);
                    }
                }
            }
        }
    }
    free(tmp);
    return ORC_OK;
}
