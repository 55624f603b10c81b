/*
 * Randomized calls of every oracle entry point, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_sanitizers.py). Each buffer is a
 * heap block of exactly the bytes the call may touch, so a read or write one
 * byte past it, or any undefined operation (signed overflow, an out-of-range
 * shift, a float-to-int conversion out of range), stops the run with a
 * report. Shapes are small and random, with the edge cases mixed in: empty
 * batches, single rows, ragged and wrapping write indices, bad lengths,
 * invalid descriptors and arguments. Results are not checked here (the pin
 * tests do that); status codes are counted so that the run shows it reached
 * the deep paths.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/swrt_oracle.h"

static uint64_t rng_state = 0x2545F4914F6CDD1Dull;
static uint64_t rnd(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}
static int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint64_t)(hi - lo + 1)); }
static size_t nz(int64_t n) { return n > 0 ? (size_t)n : 1; }  /* a block for n items, at least 1 */

/* exactly n bytes of random content (n may be 0: a unique 1-byte block that
 * the call must not touch is still returned, so NULL means "absent") */
static void *blob(size_t n) {
    unsigned char *p = malloc(n ? n : 1);
    for (size_t i = 0; i < n; ++i) p[i] = (unsigned char)rnd();
    return p;
}
/* n floats of moderate values (finite, some negative, a few zeros) */
static float *floats(size_t n) {
    float *p = malloc((n ? n : 1) * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = (float)((int64_t)(rnd() % 2001) - 1000) / 250.0f;
    return p;
}
/* new rows of a float type: random values written as that type */
static void *rows_of(int type, size_t n) {
    const size_t eb = type == ORC_XF_F32 ? 4 : 2;
    unsigned char *p = malloc(n ? n * eb : 1);
    for (size_t i = 0; i < n; ++i) {
        const float v = (float)((int64_t)(rnd() % 4001) - 2000) / 97.0f;
        uint32_t u;
        memcpy(&u, &v, 4);
        if (type == ORC_XF_F32) memcpy(p + 4 * i, &u, 4);
        else if (type == ORC_XF_BF16) { uint16_t h = (uint16_t)(u >> 16); memcpy(p + 2 * i, &h, 2); }
        else { uint16_t h = (uint16_t)(0x3C00u + (rnd() % 0x2000u)); memcpy(p + 2 * i, &h, 2); }
    }
    return p;
}

static long counts[8];
static void tally(int st) { counts[st >= 0 && st < 8 ? st : 7]++; }

static void fuzz_tensor_scatter(void) {
    const int rank = (int)pick(1, 5);
    int64_t shape[ORC_MAX_RANK];
    for (int d = 0; d < rank; ++d) shape[d] = pick(1, 5);
    const int axis = rank >= 2 ? (int)pick(1, rank - 1) : 0;
    const int bits_set[] = {4, 8, 16, 32, 64};
    int bits = bits_set[pick(0, 4)];
    if (bits == 4 && (shape[rank - 1] % 2)) shape[rank - 1] += 1;
    const int64_t M = shape[axis];
    const int64_t S = pick(0, M);
    int64_t n = 1;
    for (int d = 0; d < rank; ++d) n *= shape[d];
    const int64_t nu = n / M * S;
    const size_t pb = (size_t)(n * bits / 8), ub = (size_t)(nu * bits / 8);
    const int mode = (int)pick(0, 1);
    int64_t *wi = NULL;
    if (rnd() % 4) {
        wi = malloc((size_t)shape[0] * sizeof(int64_t));
        for (int64_t b = 0; b < shape[0]; ++b) wi[b] = pick(-2, M + 2);
    }
    void *past = blob(pb), *upd = blob(ub);
    uint32_t flags = 0;
    if (rnd() % 2) {
        tally(orc_tensor_scatter(past, past, upd, wi, shape, rank, axis, S, mode, bits, &flags));
    } else {
        void *present = blob(pb);
        tally(orc_tensor_scatter(present, past, upd, wi, shape, rank, axis, S, mode, bits, &flags));
        free(present);
    }
    /* invalid: axis out of range, odd 4-bit rows, rank past the maximum */
    tally(orc_tensor_scatter(past, past, upd, wi, shape, rank, rank, S, mode, bits, &flags));
    tally(orc_tensor_scatter(past, past, upd, wi, shape, 0, 0, S, mode, bits, &flags));
    free(past), free(upd), free(wi);
}

static void fuzz_lengths(void) {
    const int64_t B = pick(0, 6), C = pick(1, 40), S = pick(1, 6), W = pick(1, C);
    int32_t *sk = malloc((size_t)(B ? B : 1) * 4);
    for (int64_t b = 0; b < B; ++b) {
        const int64_t r = pick(0, 9);
        sk[b] = r == 0 ? -1 - (int32_t)pick(0, 3) : r == 1 ? INT32_MAX - (int32_t)pick(0, 2)
                                                           : (int32_t)pick(0, 4 * C);
    }
    int64_t *T = malloc((size_t)(B ? B : 1) * 8), *P = malloc((size_t)(B ? B : 1) * 8);
    int32_t *Lp = malloc((size_t)(B ? B : 1) * 4), *L = malloc((size_t)(B ? B : 1) * 4),
            *E = malloc((size_t)(B ? B : 1) * 4);
    int64_t *work = malloc((size_t)(B + 1) * 8);
    uint32_t flags = 0;
    tally(orc_kv_seq_lengths(sk, B, S, C, T, P, Lp, L, E, rnd() % 2 ? work : NULL, &flags));
    tally(orc_kv_seq_lengths_drift(sk, B, S, C, W, rnd() % 2 ? T : NULL, P, Lp, NULL, E, work,
                                   &flags));
    free(sk), free(T), free(P), free(Lp), free(L), free(E), free(work);
}

/* cache lengths for a windowed step: mostly from the lengths definition,
 * some made up (bad lengths) */
static void step_lengths(int64_t B, int64_t C, int64_t S, int32_t *Lp, int32_t *E, int64_t *P) {
    for (int64_t b = 0; b < B; ++b) {
        const int64_t past = pick(0, 3 * C);
        const int64_t lp = past < C ? past : C;
        const int64_t e = lp + S - C > 0 ? lp + S - C : 0;
        Lp[b] = (int32_t)lp, E[b] = (int32_t)e;
        if (P) P[b] = past;
        if (rnd() % 8 == 0) Lp[b] = (int32_t)pick(-1, C + 1), E[b] = (int32_t)pick(-1, C + S);
    }
}

static void fuzz_window(void) {
    const int64_t B = pick(0, 4), H = pick(1, 3), C = pick(1, 12), S = pick(1, 4), D = pick(1, 9);
    const int bits_set[] = {8, 16, 32};
    const int bits = bits_set[pick(0, 2)];
    const size_t eb = (size_t)bits / 8, cb = (size_t)(B * H * C * D) * eb,
                 nb = (size_t)(B * H * S * D) * eb, sb = (size_t)(B * H * (C + S) * D) * eb;
    void *kc = blob(cb), *vc = blob(cb), *kn = blob(nb), *vn = blob(nb);
    void *ks = S > 1 ? blob(sb) : NULL, *vs = S > 1 ? blob(sb) : NULL;
    int32_t *Lp = malloc((size_t)(B ? B : 1) * 4), *E = malloc((size_t)(B ? B : 1) * 4);
    step_lengths(B, C, S, Lp, E, NULL);
    const int64_t strides[3] = {H * S * D, S * D, D};
    uint32_t flags = 0;
    const unsigned phase = S > 1 ? (unsigned)pick(1, 3) : ORC_PHASE_ALL;
    tally(orc_kv_window_append(kc, vc, kn, vn, strides, ks, vs, Lp, E, B, H, C, S, D, bits, phase,
                               &flags));
    free(kc), free(vc), free(kn), free(vn), free(ks), free(vs), free(Lp), free(E);
}

/* a transform with exact-size tables; *tables receives what to free */
static orc_row_xf make_xf(int64_t heads, int64_t D, int64_t max_pos, void **tables) {
    orc_row_xf x;
    memset(&x, 0, sizeof(x));
    const int ins[] = {ORC_XF_F32, ORC_XF_F16, ORC_XF_BF16};
    const int outs[] = {ORC_XF_F32, ORC_XF_F16, ORC_XF_BF16, ORC_XF_INT8, ORC_XF_UINT8,
                        ORC_XF_FP8_E4M3};
    x.in_type = ins[pick(0, 2)];
    x.out_type = outs[pick(0, 5)];
    for (int i = 0; i < 6; ++i) tables[i] = NULL;
    if (D >= 2 && rnd() % 3) {
        x.rotary_dim = 2 * pick(1, D / 2);
        x.max_position = max_pos;
        const size_t n = (size_t)(max_pos * (x.rotary_dim / 2));
        tables[0] = floats(n), tables[1] = floats(n);
        x.cos_table = tables[0], x.sin_table = tables[1];
        x.interleaved = (int)pick(0, 1);
    }
    const int affine = x.out_type == ORC_XF_INT8 || x.out_type == ORC_XF_UINT8;
    const int byte_out = affine || x.out_type == ORC_XF_FP8_E4M3;
    for (int t = 0; t < 2; ++t) {
        x.scale[t] = byte_out ? 0.01f + (float)pick(0, 100) / 37.0f : 1.0f;
        x.zero_point[t] = !affine ? 0 : x.out_type == ORC_XF_INT8 ? (int32_t)pick(-128, 127)
                                                                  : (int32_t)pick(0, 255);
        if (byte_out && rnd() % 3 == 0) {
            float *cs = floats((size_t)(heads * D));
            for (int64_t i = 0; i < heads * D; ++i) cs[i] = fabsf(cs[i]) + 0.01f;
            if (rnd() % 5 == 0) cs[0] = NAN;
            tables[2 + t] = cs, x.channel_scale[t] = cs;
        }
        if (affine && rnd() % 3 == 0) {
            int32_t *cz = malloc((size_t)(heads * D) * 4);
            for (int64_t i = 0; i < heads * D; ++i) cz[i] = (int32_t)pick(-300, 300);
            tables[4 + t] = cz, x.channel_zero_point[t] = cz;
        }
    }
    return x;
}
static size_t xf_bytes(int type) {
    return type == ORC_XF_F32 ? 4 : type == ORC_XF_F16 || type == ORC_XF_BF16 ? 2 : 1;
}

static void fuzz_xf(void) {
    const int64_t B = pick(0, 4), H = pick(1, 3), C = pick(1, 10), S = pick(1, 3), D = pick(1, 8);
    const int64_t max_pos = pick(1, 40);
    void *tab[6];
    orc_row_xf x = make_xf(H, D, max_pos, tab);
    const size_t ib = xf_bytes(x.in_type), ob = xf_bytes(x.out_type);
    /* one row */
    void *in = rows_of(x.in_type, (size_t)D), *out = blob((size_t)D * ob);
    tally(orc_xf_row(&x, (int)pick(0, 1), pick(0, H - 1), pick(-1, max_pos), in, out, D));
    free(in), free(out);
    /* the windowed append */
    const size_t cb = (size_t)(B * H * C * D) * ob, sb = (size_t)(B * H * (C + S) * D) * ob;
    void *kc = blob(cb), *vc = blob(cb);
    void *kn = rows_of(x.in_type, (size_t)(B * H * S * D)), *vn = rows_of(x.in_type, (size_t)(B * H * S * D));
    void *ks = S > 1 ? blob(sb) : NULL, *vs = S > 1 ? blob(sb) : NULL;
    int32_t *Lp = malloc((size_t)(B ? B : 1) * 4), *E = malloc((size_t)(B ? B : 1) * 4);
    int64_t *P = malloc((size_t)(B ? B : 1) * 8);
    step_lengths(B, C, S, Lp, E, P);
    const int64_t strides[3] = {H * S * D, S * D, D};
    uint32_t flags = 0;
    tally(orc_kv_window_append_xf(kc, vc, kn, vn, strides, ks, vs, Lp, E, P, B, H, C, S, D,
                                  S > 1 ? (unsigned)pick(1, 3) : ORC_PHASE_ALL, &x, &flags));
    free(kc), free(vc), free(kn), free(vn), free(ks), free(vs), free(Lp), free(E), free(P);
    /* TensorScatter of transformed rows, rank 3 or 4 */
    const int rank = (int)pick(3, 4);
    const int64_t M = pick(1, 9), Su = pick(0, M), Bt = pick(1, 3);
    int64_t shape[4];
    if (rank == 4) shape[0] = Bt, shape[1] = H, shape[2] = M, shape[3] = D;
    else shape[0] = Bt, shape[1] = M, shape[2] = D;
    if (rank == 3) {  /* a rank-3 table has one row */
        for (int t = 0; t < 2; ++t) {
            if (x.channel_scale[t] && H != 1) x.channel_scale[t] = NULL;
            if (x.channel_zero_point[t] && H != 1) x.channel_zero_point[t] = NULL;
        }
    }
    const int64_t pre = rank == 4 ? Bt * H : Bt;
    void *past = blob((size_t)(pre * M * D) * ob);
    void *upd = rows_of(x.in_type, (size_t)(pre * Su * D));
    int64_t *wi = malloc((size_t)Bt * 8);
    for (int64_t b = 0; b < Bt; ++b) wi[b] = pick(-1, M + 1);
    tally(orc_tensor_scatter_xf(past, past, upd, wi, shape, rank, Su, (int)pick(0, 1),
                                (int)pick(0, 1), &x, &flags));
    (void)ib;
    free(past), free(upd), free(wi);
    for (int i = 0; i < 6; ++i) free(tab[i]);
}

static void fuzz_window_attention(void) {
    const int64_t B = pick(0, 3), Hkv = pick(1, 3), G = pick(1, 3), C = pick(1, 12), D = pick(1, 9);
    const int64_t Hq = Hkv * G, W = pick(1, C + 2);
    const int types[] = {ORC_XF_F32, ORC_XF_F16, ORC_XF_BF16};
    const int et = types[pick(0, 2)];
    void *q = rows_of(et, (size_t)(B * Hq * D));
    void *k = rows_of(et, (size_t)(B * Hkv * C * D)), *v = rows_of(et, (size_t)(B * Hkv * C * D));
    double *out = calloc(nz(B * Hq * D), sizeof(double));
    int32_t *L = malloc((size_t)(B ? B : 1) * 4);
    for (int64_t b = 0; b < B; ++b) L[b] = (int32_t)pick(-1, C + 1);
    uint32_t flags = 0;
    tally(orc_window_attention(q, k, v, out, L, W, B, Hq, Hkv, C, D, 0.125, et, &flags));
    free(q), free(k), free(v), free(out), free(L);
}

/* ------------------------------------------------------------------------ */
/* paged caches                                                               */
/* ------------------------------------------------------------------------ */
static const int kPageFormats[] = {ORC_XF_F32, ORC_XF_F16, ORC_XF_BF16, ORC_XF_INT8, ORC_XF_UINT8,
                                   ORC_XF_INT4, ORC_XF_UINT4, ORC_XF_INT2, ORC_XF_UINT2};
static int64_t fmt_bits(int f) {
    switch (f) {
        case ORC_XF_F32: return 32;
        case ORC_XF_F16: case ORC_XF_BF16: return 16;
        case ORC_XF_INT8: case ORC_XF_UINT8: return 8;
        case ORC_XF_INT4: case ORC_XF_UINT4: return 4;
        default: return 2;
    }
}
static int fmt_affine(int f) { return f >= ORC_XF_INT8 && f != ORC_XF_FP8_E4M3; }
static int32_t fmt_zero(int f) {
    switch (f) {
        case ORC_XF_INT8: return (int32_t)pick(-128, 127);
        case ORC_XF_UINT8: return (int32_t)pick(0, 255);
        case ORC_XF_INT4: return (int32_t)pick(-8, 7);
        case ORC_XF_UINT4: return (int32_t)pick(0, 15);
        case ORC_XF_INT2: return (int32_t)pick(-2, 1);
        case ORC_XF_UINT2: return (int32_t)pick(0, 3);
        default: return 0;
    }
}
static int64_t payload(int64_t rows, int64_t D, int f) { return (rows * D * fmt_bits(f) + 7) / 8; }

typedef struct {
    int64_t streams, n_pages, n_ids, stride, arena_bytes, layout_bytes, D;
    orc_page *pages;
    int32_t *ptr, *count, *ids;
    char *arena;
} paged_case;

/* streams with contiguous pages; CSR rows, or slotted rows with spare slots
 * and room after the layout for `spare` more bytes */
static paged_case make_paged(int64_t streams, int64_t D, int slotted, int64_t spare_pages,
                             int64_t spare_bytes) {
    paged_case c;
    memset(&c, 0, sizeof(c));
    c.streams = streams, c.D = D;
    int64_t *np = malloc((size_t)(streams ? streams : 1) * 8), total = 0, maxp = 0;
    for (int64_t s = 0; s < streams; ++s) {
        np[s] = pick(0, 4);
        total += np[s];
        if (np[s] > maxp) maxp = np[s];
    }
    c.n_pages = total + spare_pages;
    c.pages = calloc((size_t)(c.n_pages ? c.n_pages : 1), sizeof(orc_page));
    c.stride = slotted ? maxp + pick(0, 2) : 0;
    c.n_ids = slotted ? streams * c.stride : total;
    c.ids = malloc((size_t)(c.n_ids ? c.n_ids : 1) * 4);
    c.ptr = malloc((size_t)(streams + 1) * 4);
    c.count = slotted ? malloc((size_t)(streams ? streams : 1) * 4) : NULL;
    int64_t off = 0, id = 0, k = 0;
    for (int64_t s = 0; s < streams; ++s) {
        c.ptr[s] = (int32_t)k;
        if (slotted) c.count[s] = (int32_t)np[s], k = s * c.stride;
        int64_t start = 0;
        for (int64_t i = 0; i < np[s]; ++i, ++id) {
            orc_page *p = &c.pages[id];
            p->capacity = (int32_t)pick(1, 6);
            p->length = (int32_t)pick(1, p->capacity);
            p->start = start;
            start += p->length;
            p->k_format = kPageFormats[pick(0, 8)];
            p->v_format = kPageFormats[pick(0, 8)];
            p->k_scale = fmt_affine(p->k_format) ? 0.05f + (float)pick(0, 40) / 13.0f : 1.0f;
            p->v_scale = fmt_affine(p->v_format) ? 0.05f + (float)pick(0, 40) / 13.0f : 1.0f;
            p->k_zero_point = fmt_zero(p->k_format);
            p->v_zero_point = fmt_zero(p->v_format);
            p->k_offset = off, off += payload(p->capacity, D, p->k_format);
            p->v_offset = off, off += payload(p->capacity, D, p->v_format);
            c.ids[k++] = (int32_t)id;
        }
        if (slotted)
            for (int64_t i = np[s]; i < c.stride; ++i) c.ids[s * c.stride + i] = -1;
    }
    c.ptr[streams] = (int32_t)(slotted ? 0 : k);
    c.layout_bytes = off;
    c.arena_bytes = off + spare_bytes;
    c.arena = blob((size_t)c.arena_bytes);
    /* now and then a broken descriptor or id */
    if (total && rnd() % 4 == 0) {
        orc_page *p = &c.pages[pick(0, total - 1)];
        switch (pick(0, 4)) {
            case 0: p->length = p->capacity + 1; break;
            case 1: p->k_offset = c.arena_bytes; break;
            case 2: p->v_format = 42; break;
            case 3: p->k_scale = -1.0f; break;
            default: p->start += 1; break;
        }
    }
    if (c.n_ids && rnd() % 6 == 0) c.ids[pick(0, c.n_ids - 1)] = (int32_t)pick(-2, (int32_t)c.n_pages + 2);
    free(np);
    return c;
}
static void free_paged(paged_case *c) {
    free(c->pages), free(c->ids), free(c->ptr), free(c->count), free(c->arena);
}

static void fuzz_paged_attention(void) {
    const int64_t B = pick(0, 3), Hkv = pick(1, 2), G = pick(1, 3), D = pick(1, 8);
    const int slotted = (int)pick(0, 1);
    paged_case c = make_paged(B * Hkv, D, slotted, 0, 0);
    const int types[] = {ORC_XF_F32, ORC_XF_F16, ORC_XF_BF16};
    const int qt = types[pick(0, 2)];
    const int64_t Hq = Hkv * G;
    void *q = rows_of(qt, (size_t)(B * Hq * D));
    double *out = calloc(nz(B * Hq * D), sizeof(double));
    uint32_t flags = 0;
    tally(orc_paged_attention(q, qt, c.arena, c.arena_bytes, c.pages, c.n_pages,
                              slotted ? NULL : c.ptr, c.count, c.stride, c.ids, c.n_ids, out,
                              pick(-1, 12), B, Hq, Hkv, D, 0.3, &flags));
    free(q), free(out);
    free_paged(&c);
}

static void fuzz_paged_quantize(void) {
    const int64_t D = pick(1, 8);
    paged_case c = make_paged(pick(0, 4), D, 0, 0, 0);
    const int kf = kPageFormats[pick(0, 8)], vf = kPageFormats[pick(0, 8)];
    /* ascending blocks, destinations one after another in a free region */
    int64_t nb = c.n_pages ? pick(0, c.n_pages) : 0;
    int32_t *blocks = malloc((size_t)(nb ? nb : 1) * 4);
    int64_t *dst = malloc(nz(2 * nb) * 8), need = 0;
    int64_t id = -1;
    for (int64_t i = 0; i < nb; ++i) {
        id += 1 + pick(0, 1);
        if (id >= c.n_pages) { nb = i; break; }
        blocks[i] = (int32_t)id;
        need += payload(c.pages[id].capacity, D, kf) + payload(c.pages[id].capacity, D, vf);
    }
    if (nb && rnd() % 6 == 0) blocks[0] = blocks[nb - 1];  /* not ascending */
    const int64_t free_begin = c.layout_bytes, free_end = free_begin + need;
    char *arena = blob((size_t)free_end);
    memcpy(arena, c.arena, (size_t)c.layout_bytes);
    int64_t at = free_begin;
    for (int64_t i = 0; i < nb; ++i) {
        const orc_page *p = &c.pages[blocks[i]];
        dst[2 * i] = at, at += payload(p->capacity, D, kf);
        dst[2 * i + 1] = at, at += payload(p->capacity, D, vf);
    }
    orc_page *out = calloc((size_t)(c.n_pages ? c.n_pages : 1), sizeof(orc_page));
    tally(orc_paged_quantize(arena, free_end, c.pages, c.n_pages, blocks, nb, dst, free_begin,
                             free_end, out, kf, fmt_affine(kf) ? 0.3f : 1.0f, fmt_zero(kf), vf,
                             fmt_affine(vf) ? 0.7f : 1.0f, fmt_zero(vf), D));
    free(arena), free(out), free(blocks), free(dst);
    free_paged(&c);
}

static void fuzz_paged_append(void) {
    const int64_t D = pick(1, 8), Dv = rnd() % 3 ? D : pick(1, 8), S = pick(1, 3);
    const int64_t streams = pick(0, 4);
    const int kf = kPageFormats[pick(0, 8)], vf = kPageFormats[pick(0, 8)];
    const int64_t kb = payload(S, D, kf), vb = payload(S, Dv, vf);
    paged_case c = make_paged(streams, D, 1, streams, streams * (kb + vb));
    const int types[] = {ORC_XF_F32, ORC_XF_F16, ORC_XF_BF16};
    const int nt = types[pick(0, 2)];
    void *kn = rows_of(nt, (size_t)(streams * S * D)), *vn = rows_of(nt, (size_t)(streams * S * Dv));
    uint32_t flags = 0;
    int64_t written = 0;
    tally(orc_paged_append(c.arena, c.arena_bytes, c.pages, c.n_pages, c.count, c.stride, c.ids,
                           c.n_ids, kn, vn, nt, streams, S, D, Dv, c.n_pages - streams,
                           c.layout_bytes, c.arena_bytes, kf, fmt_affine(kf) ? 0.2f : 1.0f,
                           fmt_zero(kf), vf, fmt_affine(vf) ? 0.4f : 1.0f, fmt_zero(vf), &flags,
                           &written));
    free(kn), free(vn);
    free_paged(&c);
    /* the open-page extension, either table form */
    const int slotted = (int)pick(0, 1);
    paged_case o = make_paged(streams, D, slotted, 0, 0);
    void *kr = rows_of(nt, (size_t)(streams * D)), *vr = rows_of(nt, (size_t)(streams * D));
    tally(orc_paged_append_open(o.arena, o.arena_bytes, o.pages, o.n_pages, slotted ? NULL : o.ptr,
                                o.count, o.stride, o.ids, o.n_ids, kr, vr, nt, streams, D, &flags));
    free(kr), free(vr);
    free_paged(&o);
}

int main(int argc, char **argv) {
    if (argc > 1 && strcmp(argv[1], "--overrun") == 0) {
        /* the sanitizer's own check: one byte past a block must be reported */
        volatile char *p = malloc(16);
        p[16] = 1;
        free((void *)p);
        return 0;
    }
    const long rounds = argc > 1 ? atol(argv[1]) : 3000;
    for (long r = 0; r < rounds; ++r) {
        fuzz_tensor_scatter();
        fuzz_lengths();
        fuzz_window();
        fuzz_xf();
        fuzz_window_attention();
        fuzz_paged_attention();
        fuzz_paged_quantize();
        fuzz_paged_append();
    }
    printf("rounds %ld: ok %ld, invalid %ld, unsupported %ld\n", rounds, counts[ORC_OK],
           counts[ORC_E_INVALID_ARG], counts[ORC_E_UNSUPPORTED]);
    return 0;
}
