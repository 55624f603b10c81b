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
 *   - [GQA-ROPE] names RoPE at the absolute position but not its arithmetic:
 *     the rotation is the usual pairwise one, read from caller-given cosine
 *     and sine tables (one row per position), half-split or interleaved
 *     pairs, computed in binary32 one operation at a time (the precision the
 *     rounded value and the quantized code are decided in); only K turns.
 *     Row s of a windowed step sits at position P + s (P the absolute past
 *     length), row s of a TensorScatter at write_indices[b] + s before any
 *     wrap; an entry with a position outside the tables is flagged and
 *     skipped whole, K and V alike.
 *   - [ATT] the local window: the query at absolute position T - 1 sees the
 *     last W resident tokens, rows [max(0, L - W), L) (the drifting layout's
 *     "rows older than the window are masked"; C >= W is the minimum
 *     capacity). The ring-buffer cache is the case W = C with L = min(T, C).
 *     Scores are scaled dot products (the caller's scale, usually
 *     1/sqrt(head_dim)); an empty window gives zeros.
 *   - [PF] fixes rounding (ties to even) and saturation of affine codes but
 *     not NaN: NaN takes the zero point; float outputs (binary32 and the half
 *     types) store any NaN as the positive canonical quiet NaN, since the sign
 *     and payload a NaN carries out of float arithmetic differ between
 *     processors.
 */
#include "swrt_oracle.h"

#include <math.h>
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

/* Rows one batch entry's step writes: S = 1 shifts Lp - E rows when it
 * evicts (E > 0) and appends one; S > 1 fills Lp + S rows of staging. */
static int64_t work_rows(int64_t Lp, int64_t E, int64_t S)
{
    if (S == 1)
        return (E > 0 ? Lp - E : 0) + 1;
    return Lp + S;
}

/* work_offsets[0] = 0 and work_offsets[b + 1] = work_offsets[b] + the rows of
 * entry b: the exclusive prefix over the batch, its total last */
static void work_prefix(const int32_t *cache_past_lens, const int32_t *evict_counts,
                        int64_t batch, int64_t S, int64_t *work_offsets)
{
    if (!work_offsets)
        return;
    work_offsets[0] = 0;
    for (int64_t b = 0; b < batch; ++b)
        work_offsets[b + 1] = work_offsets[b] + work_rows(cache_past_lens[b], evict_counts[b], S);
}

int orc_kv_seq_lengths(const int32_t *seqlens_k, int64_t batch, int64_t seq_len,
                       int64_t capacity, int64_t *total_lens, int64_t *past_lens,
                       int32_t *cache_past_lens, int32_t *cache_total_lens,
                       int32_t *evict_counts, int64_t *work_offsets, uint32_t *flags)
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
    work_prefix(cache_past_lens, evict_counts, batch, S, work_offsets);
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
                             int32_t *evict_counts, int64_t *work_offsets, uint32_t *flags)
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
    work_prefix(cache_past_lens, evict_counts, batch, S, work_offsets);
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

/* ------------------------------------------------------------------------ */
/* [GQA-ROPE] + [PF] the row transform of a fused append                    */
/* ------------------------------------------------------------------------ */

static int xf_float_type(int type)
{
    return type == ORC_XF_F32 || type == ORC_XF_F16 || type == ORC_XF_BF16;
}

static int64_t xf_elem_bytes(int type)
{
    switch (type) {
    case ORC_XF_F32: return 4;
    case ORC_XF_F16:
    case ORC_XF_BF16: return 2;
    case ORC_XF_INT8:
    case ORC_XF_UINT8:
    case ORC_XF_FP8_E4M3: return 1;
    default: return 0;
    }
}

static int xf_code_range(int type, int32_t *lo, int32_t *hi)
{
    if (type == ORC_XF_INT8) {
        *lo = -128;
        *hi = 127;
        return 1;
    }
    if (type == ORC_XF_UINT8) {
        *lo = 0;
        *hi = 255;
        return 1;
    }
    return 0;
}

/* a transform the functions below accept, for rows of head_dim elements */
static int xf_valid(const orc_row_xf *x, int64_t head_dim)
{
    int32_t lo = 0, hi = 0;
    const int affine = xf_code_range(x ? x->out_type : 0, &lo, &hi);
    const int fp8 = x && x->out_type == ORC_XF_FP8_E4M3;
    if (!x || !xf_float_type(x->in_type) || xf_elem_bytes(x->out_type) == 0)
        return 0;
    if ((x->cos_table == NULL) != (x->sin_table == NULL))
        return 0;
    if (x->cos_table) {
        if (x->max_position < 1 || x->rotary_dim < 2 || x->rotary_dim % 2 != 0 ||
            x->rotary_dim > head_dim)
            return 0;
    }
    for (int t = 0; t < 2; ++t) {
        /* per-channel scales belong to the scaled targets, zero points to the
         * affine integer codes */
        if ((x->channel_scale[t] && !affine && !fp8) || (x->channel_zero_point[t] && !affine))
            return 0;
        if (affine || fp8) {
            if (!(x->scale[t] > 0.0f) || isinf(x->scale[t]))
                return 0;
            if (affine ? (x->zero_point[t] < lo || x->zero_point[t] > hi) : x->zero_point[t] != 0)
                return 0;
        }
    }
    return 1;
}

static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16; /* bf16 is the top half of a binary32 */
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
static float f16_bits_to_float(uint16_t h)
{
    const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

static uint16_t float_to_bf16_bits(float f)
{
    uint32_t u;
    if (isnan(f))
        return 0x7FC0; /* the positive canonical quiet NaN */
    memcpy(&u, &f, 4);
    /* round to nearest, ties to even, on the 16 bits that are dropped */
    const uint32_t dropped = u & 0xFFFF, kept = u >> 16;
    if (dropped > 0x8000 || (dropped == 0x8000 && (kept & 1)))
        return (uint16_t)(kept + 1); /* a carry into the exponent is exact */
    return (uint16_t)kept;
}

static uint16_t float_to_f16_bits(float f)
{
    uint16_t sign;
    double a;
    int e;
    if (isnan(f))
        return 0x7E00; /* the positive canonical quiet NaN */
    sign = signbit(f) ? 0x8000 : 0;
    a = fabs((double)f);
    if (a == 0.0)
        return sign;
    if (a >= 65520.0) /* half-way between 65504 and 2^16 rounds to the even 2^16 */
        return sign | 0x7C00;
    frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1: the leading bit is 2^(e-1) */
    if (e - 1 < -14) {
        /* subnormal range: count units of 2^-24; 1024 units is the smallest
         * normal, whose encoding is the same integer */
        const double q = nearbyint(ldexp(a, 24));
        return sign | (uint16_t)q;
    }
    {
        /* 11 significant bits: q in [1024, 2048] */
        double q = nearbyint(ldexp(a, 10 - (e - 1)));
        int ex = e - 1;
        if (q == 2048.0) {
            q = 1024.0;
            ex += 1;
        }
        if (ex > 15)
            return sign | 0x7C00;
        return sign | (uint16_t)((ex + 15) << 10) | (uint16_t)(q - 1024.0);
    }
}

static float xf_load(int type, const char *row, int64_t i)
{
    uint16_t h;
    float f;
    switch (type) {
    case ORC_XF_F32:
        memcpy(&f, row + 4 * i, 4);
        return f;
    case ORC_XF_F16:
        memcpy(&h, row + 2 * i, 2);
        return f16_bits_to_float(h);
    default: /* ORC_XF_BF16 */
        memcpy(&h, row + 2 * i, 2);
        return bf16_bits_to_float(h);
    }
}

/* [PF]: saturate(round_half_even(y / scale) + zero_point). A NaN quotient (a
 * NaN y, or a per-channel scale that makes y / scale NaN) takes the zero
 * point, itself saturated: a per-channel table is data, not checked. */
static int32_t xf_quantize(float y, float scale, int32_t zero_point, int32_t lo, int32_t hi)
{
    const float r = y / scale;
    float q;
    if (isnan(r))
        return zero_point < lo ? lo : (zero_point > hi ? hi : zero_point);
    q = nearbyintf(r) + (float)zero_point; /* default rounding: ties to even */
    if (q < (float)lo)
        return lo;
    if (q > (float)hi)
        return hi;
    return (int32_t)q;
}

/* The OCP 8-bit float E4M3 ("float8e4m3fn"): 1 sign bit, 4 exponent bits of
 * bias 7, 3 fraction bits, no infinities, S.1111.111 the only NaN, largest
 * finite 448 = 1.75 * 2^8, smallest normal 2^-6, subnormals m * 2^-9. A
 * binary32 value is rounded to nearest, ties to even; a finite value beyond
 * 448, or an infinity, saturates to +-448 (the saturating conversion); NaN
 * becomes the positive NaN 0x7F. */
static uint8_t float_to_e4m3_bits(float f)
{
    const uint8_t sign = signbit(f) ? 0x80 : 0;
    double a, q;
    int e;
    if (isnan(f))
        return 0x7F;
    a = fabs((double)f);
    if (a >= 448.0)
        return sign | 0x7E; /* +-448; beyond it saturates */
    if (a < ldexp(1.0, -6)) {
        /* zero or subnormal: count units of 2^-9; 8 units is the smallest normal,
         * whose encoding (exponent 1, fraction 0) is the same integer */
        q = nearbyint(ldexp(a, 9));
        return sign | (uint8_t)q;
    }
    frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1: the leading bit is 2^(e-1) */
    /* 4 significant bits: q in [8, 16] */
    q = nearbyint(ldexp(a, 3 - (e - 1)));
    if (q == 16.0) {
        q = 8.0;
        e += 1;
    }
    /* a < 448 rounds to at most 448 = exponent field 15, fraction 6 */
    return sign | (uint8_t)(((e - 1 + 7) << 3) | (int)(q - 8.0));
}

/* element i of a dense f32 / f16 / bf16 row */
static void store_dense(int type, char *row, int64_t i, float y)
{
    uint16_t h;
    switch (type) {
    case ORC_XF_F32:
        if (isnan(y)) {
            const uint32_t canonical = 0x7FC00000u; /* sign and payload are not fixed */
            memcpy(row + 4 * i, &canonical, 4);
        } else {
            memcpy(row + 4 * i, &y, 4);
        }
        break;
    case ORC_XF_F16:
        h = float_to_f16_bits(y);
        memcpy(row + 2 * i, &h, 2);
        break;
    default: /* ORC_XF_BF16 */
        h = float_to_bf16_bits(y);
        memcpy(row + 2 * i, &h, 2);
        break;
    }
}

/* element i of a row of KV head `head`: its scale and zero point, from the
 * per-channel tables [kv_heads, head_dim] when given, else the scalars */
static void xf_params(const orc_row_xf *x, int t, int64_t head, int64_t head_dim, int64_t i,
                      float *scale, int32_t *zero_point)
{
    *scale = x->channel_scale[t] ? x->channel_scale[t][head * head_dim + i] : x->scale[t];
    *zero_point = x->channel_zero_point[t] ? x->channel_zero_point[t][head * head_dim + i]
                                           : x->zero_point[t];
}

static void xf_store(const orc_row_xf *x, int t, int64_t head, int64_t head_dim, char *row,
                     int64_t i, float y)
{
    int32_t lo = 0, hi = 0, q, zp;
    float sc;
    switch (x->out_type) {
    case ORC_XF_F32:
    case ORC_XF_F16:
    case ORC_XF_BF16:
        store_dense(x->out_type, row, i, y);
        break;
    case ORC_XF_FP8_E4M3: {
        /* scaled like an affine code, y / scale rounded once to binary32 */
        uint8_t c;
        xf_params(x, t, head, head_dim, i, &sc, &zp);
        c = float_to_e4m3_bits(y / sc);
        memcpy(row + i, &c, 1);
        break;
    }
    default: /* ORC_XF_INT8, ORC_XF_UINT8 */
        xf_code_range(x->out_type, &lo, &hi);
        xf_params(x, t, head, head_dim, i, &sc, &zp);
        q = xf_quantize(y, sc, zp, lo, hi);
        if (x->out_type == ORC_XF_INT8) {
            const int8_t c = (int8_t)q;
            memcpy(row + i, &c, 1);
        } else {
            const uint8_t c = (uint8_t)q;
            memcpy(row + i, &c, 1);
        }
        break;
    }
}

int orc_xf_row(const orc_row_xf *x, int t, int64_t head, int64_t pos, const void *in, void *out,
               int64_t head_dim)
{
    float *v;
    if (head_dim < 0 || head < 0 || (t != 0 && t != 1) || !xf_valid(x, head_dim))
        return ORC_E_INVALID_ARG;
    if (head_dim == 0)
        return ORC_OK;
    if (!in || !out)
        return ORC_E_INVALID_ARG;
    if (t == 0 && x->cos_table && (pos < 0 || pos >= x->max_position))
        return ORC_E_INVALID_ARG;
    v = (float *)malloc((size_t)head_dim * sizeof(float));
    if (!v)
        return ORC_E_INVALID_ARG;
    for (int64_t i = 0; i < head_dim; ++i)
        v[i] = xf_load(x->in_type, (const char *)in, i);
    if (t == 0 && x->cos_table) {
        /* [GQA-ROPE] RoPE at the absolute position: each pair (x0, x1) turns
         * by the angle whose cosine and sine are table row pos, column j */
        const int64_t half = x->rotary_dim / 2;
        const float *c = x->cos_table + pos * half;
        const float *s = x->sin_table + pos * half;
        for (int64_t j = 0; j < half; ++j) {
            const int64_t i0 = x->interleaved ? 2 * j : j;
            const int64_t i1 = x->interleaved ? 2 * j + 1 : j + half;
            const float x0 = v[i0], x1 = v[i1];
            const float x0c = x0 * c[j], x1s = x1 * s[j];
            const float x1c = x1 * c[j], x0s = x0 * s[j];
            v[i0] = x0c - x1s;
            v[i1] = x1c + x0s;
        }
    }
    for (int64_t i = 0; i < head_dim; ++i)
        xf_store(x, t, head, head_dim, (char *)out, i, v[i]);
    free(v);
    return ORC_OK;
}

/* the positions [p0, p0 + n) all have table rows (or nothing rotates) */
static int xf_positions_ok(const orc_row_xf *x, int64_t p0, int64_t n)
{
    return !x->cos_table || (p0 >= 0 && p0 <= x->max_position - n);
}

int orc_kv_window_append_xf(void *k_cache, void *v_cache, const void *k_new,
                            const void *v_new, const int64_t *new_strides,
                            void *k_staging, void *v_staging,
                            const int32_t *cache_past_lens,
                            const int32_t *evict_counts, const int64_t *past_lens,
                            int64_t batch, int64_t kv_heads, int64_t capacity,
                            int64_t seq_len, int64_t head_dim, unsigned phase,
                            const orc_row_xf *x, uint32_t *flags)
{
    const int64_t B = batch, H = kv_heads, C = capacity, S = seq_len, D = head_dim;
    int64_t in_es, out_row, rows_strides[3];
    const char *news[2] = {(const char *)k_new, (const char *)v_new}; /* K, V */
    char *tmp[2];
    int status = ORC_OK;

    if (B < 0 || H < 0 || D < 0 || C < 1 || S < 1 || !xf_valid(x, D))
        return ORC_E_INVALID_ARG;
    in_es = xf_elem_bytes(x->in_type);
    out_row = D * xf_elem_bytes(x->out_type);
    if (B == 0 || H == 0 || D == 0)
        return ORC_OK;
    if (!k_new || !v_new || !new_strides || !past_lens || !cache_past_lens ||
        !evict_counts || !k_cache || !v_cache)
        return ORC_E_INVALID_ARG;
    /* the transformed rows of one batch entry, [1, H, S, D] in out_type */
    tmp[0] = (char *)malloc((size_t)(H * S * out_row));
    tmp[1] = (char *)malloc((size_t)(H * S * out_row));
    rows_strides[0] = H * S * D;
    rows_strides[1] = S * D;
    rows_strides[2] = D;
    if (!tmp[0] || !tmp[1]) {
        free(tmp[0]);
        free(tmp[1]);
        return ORC_E_INVALID_ARG;
    }
    for (int64_t b = 0; b < B && status == ORC_OK; ++b) {
        const int64_t Lp = cache_past_lens[b], E = evict_counts[b], L = Lp + S - E;
        if (L < 1 || L > C || E < 0 || Lp < 0 || Lp > C) {
            set_flag(flags, ORC_FLAG_BAD_LENGTHS); /* as orc_kv_window_append */
            continue;
        }
        if (!xf_positions_ok(x, past_lens[b], S)) {
            set_flag(flags, ORC_FLAG_ROPE_RANGE);
            continue; /* this batch entry keeps every byte it had */
        }
        for (int t = 0; t < 2 && status == ORC_OK; ++t)
            for (int64_t h = 0; h < H && status == ORC_OK; ++h)
                for (int64_t s = 0; s < S && status == ORC_OK; ++s)
                    status = orc_xf_row(x, t, h, past_lens[b] + s,
                                        news[t] + (b * new_strides[0] + h * new_strides[1] +
                                                   s * new_strides[2]) * in_es,
                                        tmp[t] + (h * S + s) * out_row, D);
        if (status != ORC_OK)
            break;
        /* then the plain step for this one batch entry, on out_type rows */
        status = orc_kv_window_append(
            (char *)k_cache + b * H * C * out_row, (char *)v_cache + b * H * C * out_row,
            tmp[0], tmp[1], rows_strides,
            S > 1 ? (char *)k_staging + b * H * (C + S) * out_row : NULL,
            S > 1 ? (char *)v_staging + b * H * (C + S) * out_row : NULL,
            cache_past_lens + b, evict_counts + b, 1, H, C, S, D,
            (int)(xf_elem_bytes(x->out_type) * 8), phase, flags);
    }
    free(tmp[0]);
    free(tmp[1]);
    return status;
}

int orc_tensor_scatter_xf(void *present, const void *past, const void *update,
                          const int64_t *write_indices, const int64_t *shape,
                          int rank, int64_t seq_len, int mode, int t,
                          const orc_row_xf *x, uint32_t *flags)
{
    int64_t D, M, O1 = 1, in_es, out_es, block, ushape[ORC_MAX_RANK];
    int64_t B;
    char *tmp;
    int status = ORC_OK;

    if (rank < 3 || rank > ORC_MAX_RANK || !shape || (t != 0 && t != 1))
        return ORC_E_INVALID_ARG;
    D = shape[rank - 1];
    M = shape[rank - 2];
    B = shape[0];
    if (!xf_valid(x, D) || seq_len < 0 || seq_len > M)
        return ORC_E_INVALID_ARG;
    /* per-channel tables: [shape[1], D] for rank 4 ([B, H, M, D]), [1, D] for rank 3 */
    if (rank > 4 && (x->channel_scale[0] || x->channel_scale[1] || x->channel_zero_point[0] ||
                     x->channel_zero_point[1]))
        return ORC_E_INVALID_ARG;
    for (int i = 0; i < rank; ++i)
        if (shape[i] < 0)
            return ORC_E_INVALID_ARG;
    for (int i = 1; i < rank - 2; ++i)
        O1 *= shape[i]; /* prefixes per batch entry */
    in_es = xf_elem_bytes(x->in_type);
    out_es = xf_elem_bytes(x->out_type);
    block = O1 * M * D * out_es; /* one batch entry of present / past */
    if (B == 0 || O1 == 0 || M == 0 || D == 0)
        return ORC_OK;
    if (!present || !past || (seq_len > 0 && !update))
        return ORC_E_INVALID_ARG;
    for (int i = 0; i < rank; ++i)
        ushape[i] = shape[i];
    ushape[0] = 1;
    tmp = (char *)malloc((size_t)(O1 * (seq_len ? seq_len : 1) * D * out_es));
    if (!tmp)
        return ORC_E_INVALID_ARG;
    for (int64_t b = 0; b < B && status == ORC_OK; ++b) {
        const int64_t w = write_indices ? write_indices[b] : 0;
        char *pres = (char *)present + b * block;
        const char *pst = (const char *)past + b * block;
        const int linear_ok = mode != ORC_MODE_LINEAR || (w >= 0 && w <= M - seq_len);
        if (linear_ok && !xf_positions_ok(x, w, seq_len)) {
            set_flag(flags, ORC_FLAG_ROPE_RANGE);
            if (pres != pst)
                memcpy(pres, pst, (size_t)block); /* the entry keeps past's rows */
            continue;
        }
        /* the entry's update rows, transformed at positions w + s */
        for (int64_t o = 0; o < O1 && linear_ok && status == ORC_OK; ++o)
            for (int64_t s = 0; s < seq_len && status == ORC_OK; ++s)
                status = orc_xf_row(x, t, rank == 4 ? o : 0, w + s,
                                    (const char *)update + ((b * O1 + o) * seq_len + s) * D * in_es,
                                    tmp + (o * seq_len + s) * D * out_es, D);
        if (status != ORC_OK)
            break;
        /* then plain TensorScatter of this one entry on out_type rows */
        status = orc_tensor_scatter(pres, pst, tmp, write_indices ? write_indices + b : NULL,
                                    ushape, rank, rank - 2, seq_len, mode,
                                    (int)(out_es * 8), flags);
    }
    free(tmp);
    return status;
}

/* ------------------------------------------------------------------------ */
/* [ATT] windowed decode attention                                          */
/* ------------------------------------------------------------------------ */

static double att_load(int type, const char *base, int64_t i)
{
    return (double)xf_load(type, base, i); /* every f32/f16/bf16 value is exact in float64 */
}

int orc_window_attention(const void *q, const void *k_cache, const void *v_cache,
                         double *out, const int32_t *cache_total_lens, int64_t window,
                         int64_t batch, int64_t q_heads, int64_t kv_heads,
                         int64_t capacity, int64_t head_dim, double scale, int elem_type,
                         uint32_t *flags)
{
    const int64_t B = batch, Hq = q_heads, Hkv = kv_heads, C = capacity, D = head_dim;
    int64_t es, group;
    double *s, *acc;

    if (B < 0 || Hq < 0 || Hkv < 1 || C < 1 || D < 0 || window < 1)
        return ORC_E_INVALID_ARG;
    if (!xf_float_type(elem_type) || Hq % Hkv != 0)
        return ORC_E_INVALID_ARG;
    if (B == 0 || Hq == 0 || D == 0)
        return ORC_OK;
    if (!q || !k_cache || !v_cache || !out || !cache_total_lens)
        return ORC_E_INVALID_ARG;
    es = xf_elem_bytes(elem_type);
    group = Hq / Hkv;
    s = (double *)malloc((size_t)C * sizeof(double));
    acc = (double *)malloc((size_t)D * sizeof(double));
    if (!s || !acc) {
        free(s);
        free(acc);
        return ORC_E_INVALID_ARG;
    }
    for (int64_t b = 0; b < B; ++b) {
        const int64_t L = cache_total_lens[b];
        const int64_t r0 = L > window ? L - window : 0; /* the last W resident rows */
        if (L < 0 || L > C) {
            set_flag(flags, ORC_FLAG_BAD_LENGTHS);
            continue;
        }
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t g = h / group; /* the KV head this query head reads */
            const char *qrow = (const char *)q + (b * Hq + h) * D * es;
            const char *kbase = (const char *)k_cache + (b * Hkv + g) * C * D * es;
            const char *vbase = (const char *)v_cache + (b * Hkv + g) * C * D * es;
            double m = -INFINITY, denom = 0.0;
            for (int64_t d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (int64_t r = r0; r < L; ++r) { /* scores */
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += att_load(elem_type, qrow, d) * att_load(elem_type, kbase, r * D + d);
                s[r] = scale * dot;
                if (s[r] > m)
                    m = s[r];
            }
            for (int64_t r = r0; r < L; ++r) { /* softmax weights and the weighted V */
                const double p = exp(s[r] - m);
                denom += p;
                for (int64_t d = 0; d < D; ++d)
                    acc[d] += p * att_load(elem_type, vbase, r * D + d);
            }
            for (int64_t d = 0; d < D; ++d)
                out[(b * Hq + h) * D + d] = L > r0 ? acc[d] / denom : 0.0;
        }
    }
    free(s);
    free(acc);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* [PF-PAGED] paged caches with per-page formats                              */
/* ------------------------------------------------------------------------ */

static int pg_bits(int fmt)
{
    switch (fmt) {
    case ORC_XF_F32: return 32;
    case ORC_XF_F16:
    case ORC_XF_BF16: return 16;
    case ORC_XF_INT8:
    case ORC_XF_UINT8: return 8;
    case ORC_XF_INT4:
    case ORC_XF_UINT4: return 4;
    case ORC_XF_INT2:
    case ORC_XF_UINT2: return 2;
    default: return 0;
    }
}

/* the code range of an affine format; 0 for a dense one */
static int pg_code_range(int fmt, int32_t *lo, int32_t *hi)
{
    switch (fmt) {
    case ORC_XF_INT8: *lo = -128; *hi = 127; return 1;
    case ORC_XF_UINT8: *lo = 0; *hi = 255; return 1;
    case ORC_XF_INT4: *lo = -8; *hi = 7; return 1;
    case ORC_XF_UINT4: *lo = 0; *hi = 15; return 1;
    case ORC_XF_INT2: *lo = -2; *hi = 1; return 1;
    case ORC_XF_UINT2: *lo = 0; *hi = 3; return 1;
    default: return 0;
    }
}

/* Bytes of a payload of n elements. A block's K (or V) payload is its logical
 * tensor [1, 1, capacity, head_size]: element e of row r sits at flat index
 * r * head_size + e, sub-byte codes follow one another with no gap at row
 * ends and only the last byte is padded. -1 for an unknown format. */
static int64_t pg_payload_bytes(int fmt, int64_t n)
{
    const int bits = pg_bits(fmt);
    if (bits == 0 || n < 0 || n > INT64_MAX / 32)
        return -1;
    return (n * bits + 7) / 8;
}

/* a format with its parameters: an affine one needs a positive finite scale and
 * a zero point inside its code range */
static int pg_format_ok(int fmt, float scale, int32_t zero_point)
{
    int32_t lo, hi;
    if (pg_bits(fmt) == 0)
        return 0;
    if (pg_code_range(fmt, &lo, &hi))
        return scale > 0.0f && !isinf(scale) && zero_point >= lo && zero_point <= hi;
    return 1;
}

/* [offset, offset + bytes) inside [0, arena_bytes) */
static int pg_inside(int64_t offset, int64_t bytes, int64_t arena_bytes)
{
    return offset >= 0 && bytes >= 0 && offset <= arena_bytes && bytes <= arena_bytes - offset;
}

/* a page whose K rows hold k_dim and V rows v_dim elements */
static int pg_page_ok(const orc_page *p, int64_t k_dim, int64_t v_dim, int64_t arena_bytes)
{
    if (p->start < 0 || p->capacity < 1 || p->length < 1 || p->length > p->capacity)
        return 0;
    if (!pg_format_ok(p->k_format, p->k_scale, p->k_zero_point) ||
        !pg_format_ok(p->v_format, p->v_scale, p->v_zero_point))
        return 0;
    if (p->start > INT64_MAX - p->length)
        return 0;
    return pg_inside(p->k_offset, pg_payload_bytes(p->k_format, p->capacity * k_dim), arena_bytes) &&
           pg_inside(p->v_offset, pg_payload_bytes(p->v_format, p->capacity * v_dim), arena_bytes);
}

/* The block table: stream s's pages, in token order, are page_ids[*p0 .. *p1).
 * Without page_count (compressed rows): *p0 = page_ptr[s], *p1 = page_ptr[s+1].
 * With page_count (slotted rows): the stream owns the page_stride slots from
 * *p0 = s * page_stride and uses the first page_count[s] of them. Returns 0
 * when the range does not lie inside page_ids. */
static int pg_stream(const int32_t *page_ptr, const int32_t *page_count, int64_t page_stride,
                     int64_t n_ids, int64_t s, int64_t *p0, int64_t *p1)
{
    if (page_count) {
        const int64_t n = page_count[s];
        *p0 = s * page_stride;
        *p1 = *p0 + n;
        return n >= 0 && n <= page_stride && page_stride <= n_ids - *p0;
    }
    *p0 = page_ptr[s];
    *p1 = page_ptr[s + 1];
    return *p0 >= 0 && *p1 >= *p0 && *p1 <= n_ids;
}

/* code i of an affine payload: bits i*b .. i*b + b - 1 counted from the least
 * significant bit of byte 0; signed formats in two's complement */
static int32_t pg_get_code(int fmt, const char *base, int64_t i)
{
    const int bits = pg_bits(fmt);
    const int64_t bit = i * bits;
    const unsigned byte = (unsigned char)base[bit / 8];
    const unsigned raw = (byte >> (bit % 8)) & ((1u << bits) - 1u);
    const int is_signed = fmt == ORC_XF_INT8 || fmt == ORC_XF_INT4 || fmt == ORC_XF_INT2;
    if (is_signed && (raw >> (bits - 1)))
        return (int32_t)raw - (int32_t)(1u << bits);
    return (int32_t)raw;
}

static void pg_put_code(int fmt, char *base, int64_t i, int32_t code)
{
    const int bits = pg_bits(fmt);
    const int64_t bit = i * bits;
    const unsigned mask = ((1u << bits) - 1u) << (bit % 8);
    unsigned byte = (unsigned char)base[bit / 8];
    byte = (byte & ~mask) | (((unsigned)code << (bit % 8)) & mask);
    base[bit / 8] = (char)byte;
}

/* element i of a payload as a float64 value (exact: a dense element, or
 * (c - zp) * scale with a small integer and a binary32 scale) */
static double pg_value64(int fmt, float scale, int32_t zero_point, const char *base, int64_t i)
{
    int32_t lo, hi;
    if (pg_code_range(fmt, &lo, &hi))
        return (double)(pg_get_code(fmt, base, i) - zero_point) * (double)scale;
    return (double)xf_load(fmt, base, i);
}

/* element i decoded in binary32: a dense element as is, an affine one as
 * fl((c - zp) * scale), one rounding */
static float pg_value32(int fmt, float scale, int32_t zero_point, const char *base, int64_t i)
{
    int32_t lo, hi;
    if (pg_code_range(fmt, &lo, &hi))
        return (float)(pg_get_code(fmt, base, i) - zero_point) * scale;
    return xf_load(fmt, base, i);
}

/* element i written in a target format */
static void pg_store(int fmt, float scale, int32_t zero_point, char *base, int64_t i, float y)
{
    int32_t lo, hi;
    if (pg_code_range(fmt, &lo, &hi))
        pg_put_code(fmt, base, i, xf_quantize(y, scale, zero_point, lo, hi));
    else
        store_dense(fmt, base, i, y);
}

int orc_paged_attention(const void *q, int q_type, const char *arena, int64_t arena_bytes,
                        const orc_page *pages, int64_t n_pages, const int32_t *page_ptr,
                        const int32_t *page_count, int64_t page_stride,
                        const int32_t *page_ids, int64_t n_ids, double *out,
                        int64_t left_window, int64_t batch, int64_t q_heads,
                        int64_t kv_heads, int64_t head_dim, double scale, uint32_t *flags)
{
    const int64_t B = batch, Hq = q_heads, Hkv = kv_heads, D = head_dim;
    int64_t group, qes;
    double *acc;
    int64_t *visit;

    if (B < 0 || Hq < 0 || Hkv < 1 || D < 0 || n_pages < 0 || n_ids < 0 || arena_bytes < 0)
        return ORC_E_INVALID_ARG;
    if (!xf_float_type(q_type) || Hq % Hkv != 0 || (page_count && page_stride < 1))
        return ORC_E_INVALID_ARG;
    if (B == 0 || Hq == 0 || D == 0)
        return ORC_OK;
    if (!q || !out || (!page_ptr && !page_count) || (n_pages > 0 && !pages) ||
        (n_ids > 0 && !page_ids) || (arena_bytes > 0 && !arena))
        return ORC_E_INVALID_ARG;
    qes = xf_elem_bytes(q_type);
    group = Hq / Hkv;
    acc = (double *)malloc((size_t)D * sizeof(double));
    visit = (int64_t *)malloc((size_t)(n_ids > 0 ? n_ids : 1) * sizeof(int64_t));
    if (!acc || !visit) {
        free(acc);
        free(visit);
        return ORC_E_INVALID_ARG;
    }
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t g = 0; g < Hkv; ++g) {
            const int64_t st = b * Hkv + g;
            int64_t p0, p1;
            int64_t T = 0, r0 = 0, nv = 0, ok = 1;
            /* the stream's pages the window reaches, walked back from the last:
             * each must be valid and end where the next one starts */
            if (!pg_stream(page_ptr, page_count, page_stride, n_ids, st, &p0, &p1))
                ok = 0;
            if (ok && p1 > p0) {
                int64_t end = -1;
                for (int64_t k = p1 - 1; k >= p0 && ok; --k) {
                    const int64_t id = page_ids[k];
                    const orc_page *p;
                    if (id < 0 || id >= n_pages || !pg_page_ok(&pages[id], D, D, arena_bytes)) {
                        ok = 0;
                        break;
                    }
                    p = &pages[id];
                    if (end < 0) { /* the last page fixes T and the window */
                        T = p->start + p->length;
                        r0 = left_window < 0 ? 0 : (T - 1 - left_window > 0 ? T - 1 - left_window : 0);
                    } else if (p->start + p->length != end) {
                        ok = 0;
                        break;
                    }
                    if (k == p0 && p->start != 0) { /* starts run from zero */
                        ok = 0;
                        break;
                    }
                    visit[nv++] = id;
                    end = p->start;
                    if (p->start <= r0)
                        break; /* earlier pages end before the window */
                }
            }
            if (!ok) {
                set_flag(flags, ORC_FLAG_BAD_PAGES);
                continue;
            }
            for (int64_t j = 0; j < group; ++j) {
                const int64_t h = g * group + j;
                const char *qrow = (const char *)q + (b * Hq + h) * D * qes;
                double m = -INFINITY, denom = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    acc[d] = 0.0;
                /* two passes over the visible tokens in order: the maximum score,
                 * then weights and the weighted values */
                for (int pass = 0; pass < 2; ++pass) {
                    for (int64_t v = nv - 1; v >= 0; --v) {
                        const orc_page *p = &pages[visit[v]];
                        const char *kbase = arena + p->k_offset, *vbase = arena + p->v_offset;
                        for (int64_t i = 0; i < p->length; ++i) {
                            double dot = 0.0, sc;
                            if (p->start + i < r0)
                                continue;
                            for (int64_t d = 0; d < D; ++d)
                                dot += (double)xf_load(q_type, qrow, d) *
                                       pg_value64(p->k_format, p->k_scale, p->k_zero_point, kbase,
                                                  i * D + d);
                            sc = scale * dot;
                            if (pass == 0) {
                                if (sc > m)
                                    m = sc;
                            } else {
                                const double w = exp(sc - m);
                                denom += w;
                                for (int64_t d = 0; d < D; ++d)
                                    acc[d] += w * pg_value64(p->v_format, p->v_scale,
                                                             p->v_zero_point, vbase, i * D + d);
                            }
                        }
                    }
                }
                for (int64_t d = 0; d < D; ++d)
                    out[(b * Hq + h) * D + d] = denom > 0.0 ? acc[d] / denom : 0.0;
            }
        }
    }
    free(acc);
    free(visit);
    return ORC_OK;
}

/* [a0, a0 + n0) and [a1, a1 + n1) share a byte */
static int pg_overlap(int64_t a0, int64_t n0, int64_t a1, int64_t n1)
{
    return n0 > 0 && n1 > 0 && a0 < a1 + n1 && a1 < a0 + n0;
}

int orc_paged_quantize(char *arena, int64_t arena_bytes, const orc_page *pages_in,
                       int64_t n_pages, const int32_t *blocks, int64_t n_blocks,
                       const int64_t *dst_offsets, int64_t free_begin, int64_t free_end,
                       orc_page *pages_out, int k_format, float k_scale, int32_t k_zero_point,
                       int v_format, float v_scale, int32_t v_zero_point, int64_t head_dim)
{
    const int64_t D = head_dim;
    const int fmt[2] = {k_format, v_format};
    int32_t lo, hi;
    float sc[2] = {k_scale, v_scale};
    int32_t zp[2] = {k_zero_point, v_zero_point};
    int64_t next = free_begin; /* where the next destination may start */

    /* every check before anything is written */
    if (n_pages < 0 || n_blocks < 0 || D < 1 || arena_bytes < 0)
        return ORC_E_INVALID_ARG;
    if ((n_pages > 0 && (!pages_in || !pages_out)) || (n_blocks > 0 && (!blocks || !dst_offsets)) ||
        (arena_bytes > 0 && !arena))
        return ORC_E_INVALID_ARG;
    if (free_begin < 0 || free_end < free_begin || free_end > arena_bytes)
        return ORC_E_INVALID_ARG;
    for (int t = 0; t < 2; ++t) {
        if (!pg_format_ok(fmt[t], sc[t], zp[t]))
            return ORC_E_INVALID_ARG;
        if (!pg_code_range(fmt[t], &lo, &hi)) { /* a dense target has no parameters */
            sc[t] = 1.0f;
            zp[t] = 0;
        }
    }
    for (int64_t i = 0; i < n_pages; ++i) {
        const orc_page *p = &pages_in[i];
        if (!pg_page_ok(p, D, D, arena_bytes))
            return ORC_E_INVALID_ARG;
        if (pg_overlap(free_begin, free_end - free_begin, p->k_offset,
                       pg_payload_bytes(p->k_format, p->capacity * D)) ||
            pg_overlap(free_begin, free_end - free_begin, p->v_offset,
                       pg_payload_bytes(p->v_format, p->capacity * D)))
            return ORC_E_INVALID_ARG; /* the free region holds no live payload */
    }
    for (int64_t i = 0; i < n_blocks; ++i) {
        const int64_t id = blocks[i];
        if (id < 0 || id >= n_pages || (i > 0 && id <= blocks[i - 1]))
            return ORC_E_INVALID_ARG;
        for (int t = 0; t < 2; ++t) {
            const int64_t bytes = pg_payload_bytes(fmt[t], pages_in[id].capacity * D);
            const int64_t dst = dst_offsets[2 * i + t];
            if (dst < next || bytes > free_end - dst)
                return ORC_E_INVALID_ARG;
            next = dst + bytes;
        }
    }
    /* convert the selected pages */
    for (int64_t i = 0; i < n_blocks; ++i) {
        const orc_page *p = &pages_in[blocks[i]];
        for (int t = 0; t < 2; ++t) {
            const int sfmt = t ? p->v_format : p->k_format;
            const float ss = t ? p->v_scale : p->k_scale;
            const int32_t sz = t ? p->v_zero_point : p->k_zero_point;
            const char *src = arena + (t ? p->v_offset : p->k_offset);
            char *dst = arena + dst_offsets[2 * i + t];
            /* a packed payload's padding bits in its last byte are zero */
            memset(dst, 0, (size_t)pg_payload_bytes(fmt[t], p->capacity * D));
            for (int64_t r = 0; r < p->capacity; ++r)
                for (int64_t e = 0; e < D; ++e) {
                    /* rows past the valid prefix are logical zeros, never read */
                    const float y = r < p->length ? pg_value32(sfmt, ss, sz, src, r * D + e) : 0.0f;
                    pg_store(fmt[t], sc[t], zp[t], dst, r * D + e, y);
                }
        }
    }
    /* publish: every descriptor, the selected ones with their new storage */
    for (int64_t i = 0; i < n_pages; ++i)
        if (pages_out != pages_in)
            pages_out[i] = pages_in[i];
    for (int64_t i = 0; i < n_blocks; ++i) {
        orc_page *p = &pages_out[blocks[i]];
        p->k_format = fmt[0];
        p->v_format = fmt[1];
        p->k_scale = sc[0];
        p->v_scale = sc[1];
        p->k_zero_point = zp[0];
        p->v_zero_point = zp[1];
        p->k_offset = dst_offsets[2 * i];
        p->v_offset = dst_offsets[2 * i + 1];
    }
    return ORC_OK;
}

int orc_paged_append(char *arena, int64_t arena_bytes, orc_page *pages, int64_t n_pages,
                     int32_t *page_count, int64_t page_stride, int32_t *page_ids, int64_t n_ids,
                     const void *k_new, const void *v_new, int new_type, int64_t n_streams,
                     int64_t seq_len, int64_t k_head_dim, int64_t v_head_dim, int64_t first_id,
                     int64_t free_begin, int64_t free_end, int k_format, float k_scale,
                     int32_t k_zero_point, int v_format, float v_scale, int32_t v_zero_point,
                     uint32_t *flags, int64_t *written_bytes)
{
    const int64_t S = seq_len, dim[2] = {k_head_dim, v_head_dim};
    const int fmt[2] = {k_format, v_format};
    const char *news[2] = {(const char *)k_new, (const char *)v_new};
    float sc[2] = {k_scale, v_scale};
    int32_t zp[2] = {k_zero_point, v_zero_point};
    int64_t bytes[2], stride, nes, written = 0;
    int32_t lo, hi;

    if (written_bytes)
        *written_bytes = 0;
    if (n_streams < 0 || S < 1 || k_head_dim < 1 || v_head_dim < 1 || n_pages < 0 || n_ids < 0 ||
        arena_bytes < 0 || !xf_float_type(new_type) || page_stride < 1)
        return ORC_E_INVALID_ARG;
    for (int t = 0; t < 2; ++t) {
        if (!pg_format_ok(fmt[t], sc[t], zp[t]) || dim[t] > INT64_MAX / 64 / S)
            return ORC_E_INVALID_ARG;
        if (!pg_code_range(fmt[t], &lo, &hi)) { /* a dense block has no parameters */
            sc[t] = 1.0f;
            zp[t] = 0;
        }
        bytes[t] = pg_payload_bytes(fmt[t], S * dim[t]);
    }
    stride = bytes[0] + bytes[1]; /* one stream's new payload: K, then V */
    /* the new descriptors take ids first_id .. first_id + n_streams - 1, the new
     * payloads the start of the free region, stream after stream */
    if (first_id < 0 || first_id > n_pages - n_streams)
        return ORC_E_INVALID_ARG;
    if (free_begin < 0 || free_end < free_begin || free_end > arena_bytes ||
        (n_streams > 0 && stride > (free_end - free_begin) / n_streams))
        return ORC_E_INVALID_ARG;
    if (n_streams > n_ids / page_stride)
        return ORC_E_INVALID_ARG; /* every stream's slots inside page_ids */
    if (n_streams == 0)
        return ORC_OK;
    if (!page_count || !page_ids || !k_new || !v_new || !pages || (arena_bytes > 0 && !arena))
        return ORC_E_INVALID_ARG;
    nes = xf_elem_bytes(new_type);
    for (int64_t s = 0; s < n_streams; ++s) {
        int64_t p0, p1, T = 0, id = first_id + s;
        char *dst[2];
        orc_page *np;
        if (!pg_stream(NULL, page_count, page_stride, n_ids, s, &p0, &p1)) {
            set_flag(flags, ORC_FLAG_BAD_PAGES);
            continue;
        }
        if (p1 == p0 + page_stride) { /* no free slot for the new block */
            set_flag(flags, ORC_FLAG_PAGE_FULL);
            continue;
        }
        if (p1 > p0) {
            /* the last block fixes where the new one starts; it is never written.
             * Its id may not be one of the ids this call hands out. */
            const int64_t last = page_ids[p1 - 1];
            if (last < 0 || last >= n_pages || (last >= first_id && last < first_id + n_streams) ||
                !pg_page_ok(&pages[last], k_head_dim, v_head_dim, arena_bytes) ||
                pages[last].start + pages[last].length > INT64_MAX - S) {
                set_flag(flags, ORC_FLAG_BAD_PAGES);
                continue;
            }
            T = pages[last].start + pages[last].length;
        }
        /* the new block: S tokens, capacity S, encoded in the call's formats */
        dst[0] = arena + free_begin + s * stride;
        dst[1] = dst[0] + bytes[0];
        for (int t = 0; t < 2; ++t) {
            memset(dst[t], 0, (size_t)bytes[t]); /* padding bits of a packed last byte */
            for (int64_t r = 0; r < S; ++r)
                for (int64_t e = 0; e < dim[t]; ++e)
                    pg_store(fmt[t], sc[t], zp[t], dst[t], r * dim[t] + e,
                             xf_load(new_type, news[t] + (s * S + r) * dim[t] * nes, e));
            written += bytes[t];
        }
        np = &pages[id];
        memset(np, 0, sizeof(*np));
        np->start = T;
        np->length = (int32_t)S;
        np->capacity = (int32_t)S;
        np->k_offset = free_begin + s * stride;
        np->v_offset = np->k_offset + bytes[0];
        np->k_format = fmt[0];
        np->v_format = fmt[1];
        np->k_scale = sc[0];
        np->v_scale = sc[1];
        np->k_zero_point = zp[0];
        np->v_zero_point = zp[1];
        /* the stream's next slot names the new block */
        page_ids[p1] = (int32_t)id;
        page_count[s] += 1;
    }
    if (written_bytes)
        *written_bytes = written;
    return ORC_OK;
}

int orc_paged_append_open(char *arena, int64_t arena_bytes, orc_page *pages, int64_t n_pages,
                          const int32_t *page_ptr, const int32_t *page_count, int64_t page_stride,
                          const int32_t *page_ids, int64_t n_ids, const void *k_new,
                          const void *v_new, int new_type, int64_t n_streams, int64_t head_dim,
                          uint32_t *flags)
{
    const int64_t D = head_dim;
    int64_t nes;
    if (n_streams < 0 || D < 1 || n_pages < 0 || n_ids < 0 || arena_bytes < 0 ||
        !xf_float_type(new_type) || (page_count && page_stride < 1))
        return ORC_E_INVALID_ARG;
    if (n_streams == 0)
        return ORC_OK;
    if ((!page_ptr && !page_count) || !k_new || !v_new || (n_pages > 0 && !pages) ||
        (n_ids > 0 && !page_ids) || (arena_bytes > 0 && !arena))
        return ORC_E_INVALID_ARG;
    nes = xf_elem_bytes(new_type);
    for (int64_t s = 0; s < n_streams; ++s) {
        int64_t p0, p1, id;
        orc_page *p;
        if (!pg_stream(page_ptr, page_count, page_stride, n_ids, s, &p0, &p1) || p1 == p0) {
            set_flag(flags, ORC_FLAG_BAD_PAGES);
            continue;
        }
        id = page_ids[p1 - 1]; /* the stream's last page takes the token */
        if (id < 0 || id >= n_pages || !pg_page_ok(&pages[id], D, D, arena_bytes)) {
            set_flag(flags, ORC_FLAG_BAD_PAGES);
            continue;
        }
        p = &pages[id];
        if (p->length == p->capacity) {
            set_flag(flags, ORC_FLAG_PAGE_FULL);
            continue;
        }
        for (int t = 0; t < 2; ++t) {
            const int fmt = t ? p->v_format : p->k_format;
            const float sc = t ? p->v_scale : p->k_scale;
            const int32_t zp = t ? p->v_zero_point : p->k_zero_point;
            const char *in = (const char *)(t ? v_new : k_new) + s * D * nes;
            char *base = arena + (t ? p->v_offset : p->k_offset);
            for (int64_t e = 0; e < D; ++e)
                pg_store(fmt, sc, zp, base, p->length * D + e, xf_load(new_type, in, e));
        }
        p->length += 1;
    }
    return ORC_OK;
}
