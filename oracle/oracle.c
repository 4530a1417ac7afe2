/*
 * CPU oracle for the ANS-resident 4D-STEM query path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library links, includes or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it. It is deliberately plain and slow: one value at a time,
 * no blocking, no fusion.
 *
 * What it follows:
 *  - the paired-resident page (quantem.gpu "Paired-count resident layout"),
 *    section "Contract": exact uint32 virtual images, uint64 when a full
 *    detector sum could pass 2^32; invalid pixels read as zero in patterns;
 *    a malformed stream yields an error and no result; 32 pair models with
 *    1024 states, a 2-byte stream header, sparse preferred unless the paired
 *    stream saves at least two bytes; section "Operation pipeline" item 2:
 *    empty/constant/sparse/raw fallbacks and grouped offsets (a 32-bit base
 *    plus 32 relative 16-bit offsets); 512-scan blocks; block stride.
 *  - the backend optimization matrix page, "Product Coverage" table: dense DF
 *    as the cached full-detector total minus the complement; CoM moments.
 *  - the scaled-uint16 page: per-region scale/offset in double precision,
 *    nearest ties-to-even codes, float32 reconstruction code*scale+offset.
 *  - the bit layout itself, which the pages leave open, from this
 *    repository's FORMAT.md (v1).
 *
 * Every product here is its plain definition on the dense counts; the codec is
 * implemented step by step from the format text.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG -1
#define ORC_ERR_MALFORMED -2
#define ORC_ERR_UNSUPPORTED -3
#define ORC_ERR_OOM -4

#define BLOCK 512
#define RANS_L 65536u
#define HDR_BYTES 256

typedef struct {
    uint32_t scan_rows, scan_cols, det_rows, det_cols;
    uint32_t dtype;  /* 1 = u8, 2 = u16 */
    uint32_t layout; /* 0 byte-rANS, 1 paired */
    uint32_t scaled; /* data is float32, stored as calibrated u16 codes */
} orc_geom;

/* ------------------------------------------------------------------ */
/* little helpers                                                      */
/* ------------------------------------------------------------------ */

typedef struct {
    uint8_t *p;
    uint64_t n, cap;
    int oom;
} buf;

static void put(buf *b, const void *src, uint64_t n) {
    if (b->oom) return;
    if (b->n + n > b->cap) {
        uint64_t c = b->cap ? b->cap : 4096;
        while (c < b->n + n) c *= 2;
        uint8_t *q = (uint8_t *)realloc(b->p, c);
        if (!q) {
            b->oom = 1;
            return;
        }
        b->p = q;
        b->cap = c;
    }
    memcpy(b->p + b->n, src, n);
    b->n += n;
}
static void put16(buf *b, uint16_t v) { put(b, &v, 2); }
static void put_zeros(buf *b, uint64_t n) {
    uint8_t z = 0;
    for (uint64_t i = 0; i < n; i++) put(b, &z, 1);
}
static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t rd32(const uint8_t *p) { return (uint32_t)rd16(p) | ((uint32_t)rd16(p + 2) << 16); }
static uint64_t rd64(const uint8_t *p) { return (uint64_t)rd32(p) | ((uint64_t)rd32(p + 4) << 32); }
static void wr32(uint8_t *p, uint32_t v) {
    for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void wr64(uint8_t *p, uint64_t v) {
    for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}

static uint32_t maxval(uint32_t dtype) { return dtype == 1 ? 255u : 65535u; }

/* value of scan s, pixel p from a dense (S x P) native array */
static uint32_t at(const void *counts, uint32_t dtype, uint64_t s, uint64_t P, uint64_t p) {
    if (dtype == 1) return ((const uint8_t *)counts)[s * P + p];
    return ((const uint16_t *)counts)[s * P + p];
}

/* ------------------------------------------------------------------ */
/* scaled uint16 calibration (scaled-uint16 page; FORMAT 1.5)          */
/* ------------------------------------------------------------------ */

/* nearest integer, ties to even, for a non-negative finite double */
static double round_half_even(double v) {
    double f = floor(v);
    double d = v - f;
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

int orc_calibrate(const float *x, uint64_t n, double *scale, double *offset, uint16_t *codes) {
    if (n == 0) return ORC_ERR_ARG;
    double lo = 0, hi = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (!isfinite(x[i])) return ORC_ERR_ARG;
        double v = (double)x[i];
        if (i == 0 || v < lo) lo = v;
        if (i == 0 || v > hi) hi = v;
    }
    if (hi == lo) {
        *scale = 1.0;
        *offset = lo;
        for (uint64_t i = 0; i < n; i++) codes[i] = 0;
        return ORC_OK;
    }
    double sc = (hi - lo) / 65535.0;
    *scale = sc;
    *offset = lo;
    for (uint64_t i = 0; i < n; i++) {
        double c = round_half_even(((double)x[i] - lo) / sc);
        if (c < 0) c = 0;
        if (c > 65535) c = 65535;
        codes[i] = (uint16_t)c;
    }
    return ORC_OK;
}

void orc_reconstruct(const uint16_t *codes, uint64_t n, double scale, double offset, float *out) {
    for (uint64_t i = 0; i < n; i++) {
        volatile double prod = (double)codes[i] * scale; /* rounded product, no fused add */
        volatile double sum = prod + offset;
        out[i] = (float)sum;
    }
}

/* ------------------------------------------------------------------ */
/* byte-rANS tables (FORMAT 2.2)                                       */
/* ------------------------------------------------------------------ */

static void quantize(const uint64_t h[256], uint16_t f[256]) {
    uint64_t N = 0;
    for (int s = 0; s < 256; s++) N += h[s];
    for (int s = 0; s < 256; s++) f[s] = 0;
    if (N == 0) return;
    uint64_t sum = 0;
    for (int s = 0; s < 256; s++) {
        if (h[s] == 0) continue;
        uint64_t v = h[s] * 4096 / N;
        f[s] = (uint16_t)(v < 1 ? 1 : v);
        sum += f[s];
    }
    while (sum > 4096) {
        int best = -1;
        for (int s = 0; s < 256; s++)
            if (f[s] > 1 && (best < 0 || f[s] > f[best])) best = s;
        f[best]--;
        sum--;
    }
    if (sum < 4096) {
        int best = 0;
        for (int s = 1; s < 256; s++)
            if (h[s] > h[best]) best = s;
        f[best] = (uint16_t)(f[best] + (4096 - sum));
    }
}

static int degenerate(const uint16_t f[256]) {
    for (int s = 0; s < 256; s++)
        if (f[s] == 4096) return 1;
    return 0;
}

static int table_empty(const uint16_t f[256]) {
    for (int s = 0; s < 256; s++)
        if (f[s]) return 0;
    return 1;
}

/* ------------------------------------------------------------------ */
/* byte-rANS stream encoding (FORMAT 2.3, 2.4)                         */
/* ------------------------------------------------------------------ */

static int all_equal(const uint32_t *v, int n) {
    for (int j = 1; j < n; j++)
        if (v[j] != v[0]) return 0;
    return 1;
}

/* rANS words of one stream, in stream order after the header; returns count */
static int rans_encode(const uint32_t *v, int n, uint32_t dtype, const uint16_t f[256], uint16_t *out) {
    uint32_t c[256];
    uint32_t acc = 0;
    for (int s = 0; s < 256; s++) {
        c[s] = acc;
        acc += f[s];
    }
    uint16_t *stack = (uint16_t *)malloc(sizeof(uint16_t) * (2 * n + 4));
    int top = 0;
    uint64_t x = RANS_L;
    for (int j = n - 1; j >= 0; j--) {
        uint32_t s = v[j];
        if (dtype == 2 && s >= 255) {
            stack[top++] = (uint16_t)v[j];
            s = 255;
        }
        uint64_t fs = f[s];
        if (x >= (fs << 20)) {
            stack[top++] = (uint16_t)(x & 0xFFFF);
            x >>= 16;
        }
        x = ((x / fs) << 12) + (x % fs) + c[s];
    }
    int k = 0;
    out[k++] = (uint16_t)(x & 0xFFFF);
    out[k++] = (uint16_t)(x >> 16);
    while (top > 0) out[k++] = stack[--top];
    free(stack);
    return k;
}

static void emit_raw(buf *b, const uint32_t *v, int n, uint32_t dtype) {
    if (dtype == 2) {
        for (int j = 0; j < n; j++) put16(b, (uint16_t)v[j]);
    } else {
        for (int j = 0; j < n; j++) {
            uint8_t byte = (uint8_t)v[j];
            put(b, &byte, 1);
        }
        if (n % 2) put_zeros(b, 1);
    }
}

static uint64_t raw_bytes(int n, uint32_t dtype) {
    return dtype == 2 ? 2 + 2 * (uint64_t)n : 2 + (uint64_t)n + (uint64_t)(n % 2);
}

/* ------------------------------------------------------------------ */
/* paired tANS models (FORMAT 3.1, 3.2)                                */
/* ------------------------------------------------------------------ */

#define TL 1024

typedef struct {
    uint16_t n[256];       /* normalized counts */
    uint32_t a0;           /* window base */
    uint32_t in_use;       /* bit k set: window symbol k < 15 is in use */
    uint16_t spread[TL];   /* state -> symbol */
    uint16_t occ[256][TL]; /* per symbol: states of its occurrences, spread order (first n[i] used) */
} pair_model;

static void model_counts(int m, uint16_t n_out[256], uint32_t *a0_out, uint32_t *in_use_out) {
    double lam = 0.01 * pow(2000.0, (double)m / 31.0);
    int a0 = (int)floor(lam) - 7;
    if (a0 < 0) a0 = 0;
    /* walk the Poisson pmf up to the end of the window */
    double pm[64];
    pm[0] = exp(-lam);
    for (int k = 1; k < a0 + 15; k++) pm[k] = (pm[k - 1] * lam) / (double)k;
    double q[16];
    uint32_t in_use = 0;
    double s = 0.0;
    for (int k = 0; k < 15; k++) {
        q[k] = pm[a0 + k];
        if (q[k] >= 1.0 / 1024.0) {
            in_use |= 1u << k;
            s += q[k];
        }
    }
    q[15] = 1.0 - s;
    if (q[15] < 0) q[15] = 0;
    /* support: both halves in use or escape */
    int support[256];
    double r[256];
    uint32_t total = 0;
    for (int i = 0; i < 256; i++) {
        int a = i >> 4, b = i & 15;
        support[i] = (a == 15 || ((in_use >> a) & 1)) && (b == 15 || ((in_use >> b) & 1));
        n_out[i] = 0;
        r[i] = 0;
        if (!support[i]) continue;
        double y = 1024.0 * (q[a] * q[b]);
        double fl = floor(y);
        r[i] = y - fl;
        n_out[i] = (uint16_t)(fl < 1.0 ? 1.0 : fl);
        total += n_out[i];
    }
    while (total > TL) {
        int best = -1;
        for (int i = 0; i < 256; i++)
            if (support[i] && (best < 0 || n_out[i] > n_out[best])) best = i;
        n_out[best]--;
        total--;
    }
    /* largest remainders, lowest index on ties, one unit each */
    int used[256] = {0};
    while (total < TL) {
        int best = -1;
        for (int i = 0; i < 256; i++)
            if (support[i] && !used[i] && (best < 0 || r[i] > r[best])) best = i;
        if (best < 0) { /* every support symbol had a unit: start another round */
            for (int i = 0; i < 256; i++) used[i] = 0;
            continue;
        }
        used[best] = 1;
        n_out[best]++;
        total++;
    }
    *a0_out = (uint32_t)a0;
    *in_use_out = in_use;
}

static void build_model(int m, pair_model *pm) {
    model_counts(m, pm->n, &pm->a0, &pm->in_use);
    int pos = 0;
    for (int i = 0; i < 256; i++)
        for (int k = 0; k < pm->n[i]; k++) {
            pm->spread[pos] = (uint16_t)i;
            pos = (pos + 643) % TL;
        }
    int seen[256] = {0};
    for (int X = 0; X < TL; X++) {
        int i = pm->spread[X];
        pm->occ[i][seen[i]++] = (uint16_t)X;
    }
}

static int floor_log2(uint32_t y) {
    int r = -1;
    while (y) {
        y >>= 1;
        r++;
    }
    return r;
}

/* decode entries of all states, states taken in increasing order (FORMAT 3.2) */
static void decode_entries(const uint16_t n[256], const uint16_t *spread, uint16_t *sym, uint8_t *nbits,
                           uint16_t *newX) {
    uint32_t next[256];
    for (int i = 0; i < 256; i++) next[i] = n[i];
    for (int X = 0; X < TL; X++) {
        int i = spread[X];
        uint32_t y = next[i]++;
        sym[X] = (uint16_t)i;
        nbits[X] = (uint8_t)(10 - floor_log2(y));
        newX[X] = (uint16_t)((y << nbits[X]) - TL);
    }
}

int orc_pair_models(uint16_t *out /* 32*256 */, uint32_t *a0 /* 32 */, uint32_t *in_use /* 32 */) {
    for (int m = 0; m < 32; m++) {
        uint32_t b, u;
        model_counts(m, out + 256 * m, &b, &u);
        if (a0) a0[m] = b;
        if (in_use) in_use[m] = u;
    }
    return ORC_OK;
}

/* bit writer, LSB first */
typedef struct {
    uint8_t *bytes;
    uint64_t nbits, cap;
} bitw;

static void bw_put(bitw *w, uint32_t val, int nb) {
    for (int i = 0; i < nb; i++) {
        uint64_t byte = w->nbits >> 3;
        if (byte >= w->cap) {
            w->cap = w->cap ? 2 * w->cap : 256;
            w->bytes = (uint8_t *)realloc(w->bytes, w->cap);
            memset(w->bytes + byte, 0, w->cap - byte);
        }
        if ((val >> i) & 1) w->bytes[byte] |= (uint8_t)(1u << (w->nbits & 7));
        w->nbits++;
    }
}

static int window_sym(uint32_t v, uint32_t a0, uint32_t in_use) {
    if (v >= a0 && v - a0 < 15 && ((in_use >> (v - a0)) & 1)) return (int)(v - a0);
    return 15;
}

/* static cost of coding v with model pm, in 1/256 bits (FORMAT 3.4) */
static int paired_cost(const pair_model *pm, const uint32_t *v, uint32_t dtype, uint64_t *cost) {
    uint64_t c = 0;
    int lit = dtype == 2 ? 16 : 8;
    for (int t = 0; t < 256; t++) {
        int a = window_sym(v[2 * t], pm->a0, pm->in_use), b = window_sym(v[2 * t + 1], pm->a0, pm->in_use);
        int i = 16 * a + b;
        if (pm->n[i] == 0) return 0;
        c += (uint64_t)ceil(256.0 * log2(1024.0 / (double)pm->n[i]));
        if (a == 15) c += 256 * (uint64_t)lit;
        if (b == 15) c += 256 * (uint64_t)lit;
    }
    *cost = c;
    return 1;
}

/* One encoder step of FORMAT 3.2: pair symbol i from encoder state x in
 * [1024, 2048). k = the fewest low bits of x whose removal leaves x >> k below
 * 2*n[i]; those bits are emitted; the new state is 1024 plus the state that
 * holds occurrence (x >> k) - n[i] of symbol i (occurrences counted in
 * increasing state order). */
static uint32_t encode_step(const pair_model *pm, int i, uint32_t x, uint32_t *bits, uint32_t *k_out) {
    uint32_t ni = pm->n[i];
    int k = 0;
    while ((x >> k) >= 2 * ni) k++;
    *bits = x & ((1u << k) - 1);
    *k_out = (uint32_t)k;
    uint32_t y = x >> k;
    return TL + pm->occ[i][y - ni];
}

/* PAIRED code section bytes (padded to 16 bits); returns byte count */
static uint64_t paired_encode(const pair_model *pm, const uint32_t *v, uint32_t dtype, uint8_t **out) {
    uint32_t chunk_val[256], chunk_nb[256];
    uint32_t x = TL;
    for (int t = 255; t >= 0; t--) {
        int a = window_sym(v[2 * t], pm->a0, pm->in_use), b = window_sym(v[2 * t + 1], pm->a0, pm->in_use);
        x = encode_step(pm, 16 * a + b, x, &chunk_val[t], &chunk_nb[t]);
    }
    bitw w = {0, 0, 0};
    int lit = dtype == 2 ? 16 : 8;
    bw_put(&w, x - TL, 10);
    for (int t = 0; t < 256; t++) {
        bw_put(&w, chunk_val[t], (int)chunk_nb[t]);
        if (window_sym(v[2 * t], pm->a0, pm->in_use) == 15) bw_put(&w, v[2 * t], lit);
        if (window_sym(v[2 * t + 1], pm->a0, pm->in_use) == 15) bw_put(&w, v[2 * t + 1], lit);
    }
    while (w.nbits % 16) bw_put(&w, 0, 1);
    *out = w.bytes;
    return w.nbits / 8;
}

/* Decode table of pair model m (FORMAT 3.2): for every state X, the pair
 * symbol, the code length and the next-state base. */
int orc_pair_decode_table(int m, uint16_t *sym, uint8_t *nbits, uint16_t *newX) {
    if (m < 0 || m > 31) return ORC_ERR_ARG;
    pair_model *pm = (pair_model *)malloc(sizeof(pair_model));
    if (!pm) return ORC_ERR_OOM;
    build_model(m, pm);
    decode_entries(pm->n, pm->spread, sym, nbits, newX);
    free(pm);
    return ORC_OK;
}

/* The encoder step of pair symbol i of model m from every state x in
 * [1024, 2048): emitted bit count, emitted bits and the new state (x - 1024
 * form, i.e. the decoder's state), index x - 1024. */
int orc_pair_encode_steps(int m, int i, uint32_t *k, uint32_t *bits, uint32_t *state) {
    if (m < 0 || m > 31 || i < 0 || i > 255) return ORC_ERR_ARG;
    pair_model *pm = (pair_model *)malloc(sizeof(pair_model));
    if (!pm) return ORC_ERR_OOM;
    build_model(m, pm);
    if (pm->n[i] == 0) {
        free(pm);
        return ORC_ERR_ARG;
    }
    for (uint32_t x = TL; x < 2 * TL; x++) state[x - TL] = encode_step(pm, i, x, &bits[x - TL], &k[x - TL]) - TL;
    free(pm);
    return ORC_OK;
}

/* Size of the PAIRED stream (header included) of 512 values with the model
 * the format's static cost picks (FORMAT 3.4), and that model. */
int orc_paired_size(const uint32_t *v, uint32_t dtype, int *model, uint64_t *bytes) {
    pair_model *models = (pair_model *)malloc(sizeof(pair_model) * 32);
    if (!models) return ORC_ERR_OOM;
    int best_m = -1;
    uint64_t best_cost = 0;
    for (int m = 0; m < 32; m++) {
        uint64_t cst;
        build_model(m, &models[m]);
        if (paired_cost(&models[m], v, dtype, &cst) && (best_m < 0 || cst < best_cost)) {
            best_m = m;
            best_cost = cst;
        }
    }
    uint8_t *code = NULL;
    *model = best_m;
    *bytes = 2 + paired_encode(&models[best_m], v, dtype, &code);
    free(code);
    free(models);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* container encoder                                                   */
/* ------------------------------------------------------------------ */

static void header_and_layout(const orc_geom *g, uint64_t nb, uint64_t *offs) {
    /* offs: dir, table, gbase, rel, payload */
    const uint64_t P = (uint64_t)g->det_rows * g->det_cols, G = (P + 31) / 32;
    uint64_t o = HDR_BYTES;
    offs[0] = o;
    o += 16 * nb;
    o = (o + 255) / 256 * 256;
    offs[1] = o;
    o += g->layout == 0 ? 512 * nb : 2 * 32 * 256;
    o = (o + 255) / 256 * 256;
    offs[2] = o;
    o += 4 * nb * G;
    o = (o + 255) / 256 * 256;
    offs[3] = o;
    o += 2 * 32 * nb * G;
    o = (o + 255) / 256 * 256;
    offs[4] = o;
}

/*
 * Encode dense data (S x P native values, or float32 when g->scaled) into a
 * freshly malloc'd blob. Returns the blob size, or a negative error.
 */
int64_t orc_encode(const orc_geom *g, const void *data, uint8_t **blob_out) {
    const uint64_t S = (uint64_t)g->scan_rows * g->scan_cols;
    const uint64_t P = (uint64_t)g->det_rows * g->det_cols, G = (P + 31) / 32;
    if (S == 0 || P == 0 || g->det_rows > 1024 || g->det_cols > 1024) return ORC_ERR_ARG;
    if (g->dtype != 1 && g->dtype != 2) return ORC_ERR_ARG;
    if (g->layout > 1) return ORC_ERR_ARG;
    if (g->layout == 1 && S % BLOCK) return ORC_ERR_ARG;
    if (g->scaled && (g->layout != 0 || g->dtype != 2)) return ORC_ERR_ARG;
    const uint64_t nb = (S + BLOCK - 1) / BLOCK;

    uint64_t offs[5];
    header_and_layout(g, nb, offs);
    uint8_t *dir = (uint8_t *)calloc(nb, 16);
    uint16_t *tables = (uint16_t *)calloc(g->layout == 0 ? 256 * nb : 32 * 256, 2);
    uint32_t *gbase = (uint32_t *)calloc(nb * G, 4);
    uint16_t *rel = (uint16_t *)calloc(nb * G * 32, 2);
    double *calib = g->scaled ? (double *)calloc(2 * nb, sizeof(double)) : NULL;
    buf pay = {0, 0, 0, 0};

    pair_model *models = NULL;
    if (g->layout == 1) {
        models = (pair_model *)malloc(sizeof(pair_model) * 32);
        for (int m = 0; m < 32; m++) {
            build_model(m, &models[m]);
            memcpy(tables + 256 * m, models[m].n, 512);
        }
    }

    uint32_t *v = (uint32_t *)malloc(sizeof(uint32_t) * BLOCK);
    uint16_t *words = (uint16_t *)malloc(sizeof(uint16_t) * (2 * BLOCK + 8));
    uint16_t *codes = NULL;

    for (uint64_t b = 0; b < nb; b++) {
        const uint64_t s0 = b * BLOCK;
        const int n = (int)((S - s0) < BLOCK ? (S - s0) : BLOCK);
        const void *src = data;
        uint64_t src_first = s0;
        if (g->scaled) {
            /* calibrate the block region, then code it as u16 */
            free(codes);
            codes = (uint16_t *)malloc(sizeof(uint16_t) * (uint64_t)n * P);
            double sc, off;
            if (orc_calibrate((const float *)data + s0 * P, (uint64_t)n * P, &sc, &off, codes) != ORC_OK) {
                free(codes);
                free(v); free(words); free(dir); free(tables); free(gbase); free(rel); free(calib); free(pay.p);
                free(models);
                return ORC_ERR_ARG;
            }
            calib[2 * b] = sc;
            calib[2 * b + 1] = off;
            src = codes;
            src_first = 0;
        }
        const uint64_t block_base = pay.n;
        uint16_t *f = tables + 256 * b;
        if (g->layout == 0) {
            uint64_t h[256] = {0};
            for (uint64_t p = 0; p < P; p++) {
                for (int j = 0; j < n; j++) v[j] = at(src, g->dtype, src_first + j, P, p);
                if (all_equal(v, n)) continue;
                for (int j = 0; j < n; j++) h[v[j] > 255 ? 255 : v[j]]++;
            }
            quantize(h, f);
        }
        for (uint64_t p = 0; p < P; p++) {
            const uint64_t start = pay.n - block_base;
            const uint64_t grp = p / 32, idx = p % 32;
            if (idx == 0) gbase[b * G + grp] = (uint32_t)start;
            rel[(b * G + grp) * 32 + idx] = (uint16_t)(start - gbase[b * G + grp]);
            for (int j = 0; j < n; j++) v[j] = at(src, g->dtype, src_first + j, P, p);
            if (g->layout == 0) {
                if (all_equal(v, n)) {
                    put16(&pay, 0);
                    put16(&pay, (uint16_t)v[0]);
                    continue;
                }
                int use_rans = 0, nw = 0;
                if (!degenerate(f)) {
                    nw = rans_encode(v, n, g->dtype, f, words);
                    use_rans = 2 + 2 * (uint64_t)nw < raw_bytes(n, g->dtype);
                }
                if (use_rans) {
                    put16(&pay, 1);
                    for (int k = 0; k < nw; k++) put16(&pay, words[k]);
                } else {
                    put16(&pay, 2);
                    emit_raw(&pay, v, n, g->dtype);
                }
            } else {
                int zero = 1;
                for (int j = 0; j < n; j++)
                    if (v[j]) zero = 0;
                if (zero) {
                    put16(&pay, 0);
                    continue;
                }
                if (all_equal(v, n)) {
                    put16(&pay, 1);
                    put16(&pay, (uint16_t)v[0]);
                    continue;
                }
                uint64_t nnz = 0;
                for (int j = 0; j < n; j++)
                    if (v[j]) nnz++;
                uint64_t sparse = 2 + 2 + 2 * nnz + (g->dtype == 2 ? 2 * nnz : nnz + (nnz % 2));
                int best_m = -1;
                uint64_t best_cost = 0;
                for (int m = 0; m < 32; m++) {
                    uint64_t cst;
                    if (paired_cost(&models[m], v, g->dtype, &cst) && (best_m < 0 || cst < best_cost)) {
                        best_m = m;
                        best_cost = cst;
                    }
                }
                uint8_t *code = NULL;
                uint64_t paired = 0;
                if (best_m >= 0) paired = 2 + paired_encode(&models[best_m], v, g->dtype, &code);
                /* 2 = SPARSE, 3 = PAIRED, 4 = RAW */
                int mode = 2;
                uint64_t size = sparse;
                if (best_m >= 0 && sparse >= paired + 2) {
                    mode = 3;
                    size = paired;
                }
                uint64_t raw = raw_bytes(n, g->dtype);
                if (raw < size) mode = 4;
                if (mode == 2) {
                    put16(&pay, 2);
                    put16(&pay, (uint16_t)nnz);
                    for (int j = 0; j < n; j++)
                        if (v[j]) put16(&pay, (uint16_t)j);
                    uint32_t nzv[BLOCK];
                    int k = 0;
                    for (int j = 0; j < n; j++)
                        if (v[j]) nzv[k++] = v[j];
                    emit_raw(&pay, nzv, k, g->dtype);
                } else if (mode == 3) {
                    put16(&pay, (uint16_t)(3 | (best_m << 3)));
                    put(&pay, code, paired - 2);
                } else {
                    put16(&pay, 4);
                    emit_raw(&pay, v, n, g->dtype);
                }
                free(code);
            }
        }
        /* unused entries of a final partial group point at the group end */
        const uint64_t last = (P - 1) / 32;
        for (uint64_t idx = P - last * 32; idx < 32; idx++)
            rel[(b * G + last) * 32 + idx] = (uint16_t)(pay.n - block_base - gbase[b * G + last]);
        wr64(dir + 16 * b, block_base);
        wr32(dir + 16 * b + 8, (uint32_t)n);
        wr32(dir + 16 * b + 12, (uint32_t)(pay.n - block_base));
    }
    free(v);
    free(words);
    free(codes);
    free(models);

    /* assemble */
    uint64_t payload_off = offs[4];
    uint64_t calib_off = 0;
    uint64_t total = payload_off + pay.n;
    if (g->scaled) {
        total = (total + 255) / 256 * 256;
        calib_off = total;
        total += 16 * nb;
    }
    uint8_t *blob = (uint8_t *)calloc(total, 1);
    if (!blob || pay.oom) {
        free(blob); free(dir); free(tables); free(gbase); free(rel); free(calib); free(pay.p);
        return ORC_ERR_OOM;
    }
    memcpy(blob, "QSCRES01", 8);
    strcpy((char *)blob + 8, g->layout == 0 ? "qsc-byte-rans-v1" : "qsc-paired-v1");
    uint32_t hv[10] = {1, g->layout, g->scan_rows, g->scan_cols, g->det_rows, g->det_cols, g->dtype, BLOCK,
                       (uint32_t)nb, g->scaled ? 1u : 0u};
    for (int i = 0; i < 10; i++) wr32(blob + 40 + 4 * i, hv[i]);
    wr64(blob + 80, offs[0]);
    wr64(blob + 88, offs[1]);
    wr64(blob + 96, offs[2]);
    wr64(blob + 104, offs[3]);
    wr64(blob + 112, payload_off);
    wr64(blob + 120, pay.n);
    wr64(blob + 128, calib_off);
    wr64(blob + 136, total);
    memcpy(blob + offs[0], dir, 16 * nb);
    for (uint64_t i = 0; i < (g->layout == 0 ? 256 * nb : 32 * 256); i++) {
        blob[offs[1] + 2 * i] = (uint8_t)tables[i];
        blob[offs[1] + 2 * i + 1] = (uint8_t)(tables[i] >> 8);
    }
    for (uint64_t i = 0; i < nb * G; i++) wr32(blob + offs[2] + 4 * i, gbase[i]);
    for (uint64_t i = 0; i < nb * G * 32; i++) {
        blob[offs[3] + 2 * i] = (uint8_t)rel[i];
        blob[offs[3] + 2 * i + 1] = (uint8_t)(rel[i] >> 8);
    }
    memcpy(blob + payload_off, pay.p, pay.n);
    if (g->scaled)
        for (uint64_t i = 0; i < 2 * nb; i++) memcpy(blob + calib_off + 8 * i, &calib[i], 8);
    free(dir); free(tables); free(gbase); free(rel); free(calib); free(pay.p);
    *blob_out = blob;
    return (int64_t)total;
}

void orc_free(void *p) { free(p); }

/* ------------------------------------------------------------------ */
/* container decoder                                                   */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint8_t *blob;
    uint64_t nbytes;
    orc_geom g;
    uint64_t S, P, G, nb;
    uint64_t dir, table, gbase, rel, payload, payload_bytes, calib;
} parsed;

static int parse(const uint8_t *blob, uint64_t nbytes, parsed *ps) {
    if (nbytes < HDR_BYTES || memcmp(blob, "QSCRES01", 8)) return ORC_ERR_MALFORMED;
    uint32_t layout = rd32(blob + 44);
    const char *want = layout == 0 ? "qsc-byte-rans-v1" : layout == 1 ? "qsc-paired-v1" : NULL;
    if (!want) return ORC_ERR_UNSUPPORTED;
    char tag[33];
    memcpy(tag, blob + 8, 32);
    tag[32] = 0;
    if (strcmp(tag, want) || rd32(blob + 40) != 1) return ORC_ERR_UNSUPPORTED;
    ps->blob = blob;
    ps->nbytes = nbytes;
    ps->g.layout = layout;
    ps->g.scan_rows = rd32(blob + 48);
    ps->g.scan_cols = rd32(blob + 52);
    ps->g.det_rows = rd32(blob + 56);
    ps->g.det_cols = rd32(blob + 60);
    ps->g.dtype = rd32(blob + 64);
    ps->g.scaled = rd32(blob + 76) & 1;
    ps->S = (uint64_t)ps->g.scan_rows * ps->g.scan_cols;
    ps->P = (uint64_t)ps->g.det_rows * ps->g.det_cols;
    ps->G = (ps->P + 31) / 32;
    ps->nb = rd32(blob + 72);
    if (rd32(blob + 68) != BLOCK || ps->nb != (ps->S + BLOCK - 1) / BLOCK) return ORC_ERR_MALFORMED;
    if (ps->g.dtype != 1 && ps->g.dtype != 2) return ORC_ERR_MALFORMED;
    if (rd32(blob + 76) & ~1u) return ORC_ERR_MALFORMED;
    ps->dir = rd64(blob + 80);
    ps->table = rd64(blob + 88);
    ps->gbase = rd64(blob + 96);
    ps->rel = rd64(blob + 104);
    ps->payload = rd64(blob + 112);
    ps->payload_bytes = rd64(blob + 120);
    ps->calib = rd64(blob + 128);
    if (rd64(blob + 136) != nbytes || ps->payload + ps->payload_bytes > nbytes) return ORC_ERR_MALFORMED;
    return ORC_OK;
}

/* extent [start, end) of stream (b, p) relative to the payload */
static int stream_extent(const parsed *ps, uint64_t b, uint64_t p, uint64_t *start, uint64_t *end) {
    const uint8_t *d = ps->blob + ps->dir + 16 * b;
    uint64_t base = rd64(d), nbytes = rd32(d + 12);
    uint64_t g = p / 32, i = p % 32;
    uint64_t gb = rd32(ps->blob + ps->gbase + 4 * (b * ps->G + g));
    *start = base + gb + rd16(ps->blob + ps->rel + 2 * ((b * ps->G + g) * 32 + i));
    if (p + 1 < ps->P) {
        uint64_t g2 = (p + 1) / 32, i2 = (p + 1) % 32;
        uint64_t gb2 = rd32(ps->blob + ps->gbase + 4 * (b * ps->G + g2));
        *end = base + gb2 + rd16(ps->blob + ps->rel + 2 * ((b * ps->G + g2) * 32 + i2));
    } else {
        *end = base + nbytes;
    }
    if (*end < *start || *end > ps->payload_bytes || *start % 2 || *end % 2) return ORC_ERR_MALFORMED;
    return ORC_OK;
}

/* reads u16 words of a stream, flags reads past the extent */
typedef struct {
    const uint8_t *p;
    uint64_t pos, end; /* byte positions within the stream */
    int overrun;
} wreader;

static uint32_t next_word(wreader *r) {
    if (r->pos + 2 > r->end) {
        r->overrun = 1;
        return 0;
    }
    uint32_t w = rd16(r->p + r->pos);
    r->pos += 2;
    return w;
}

static int decode_rans_stream(const uint8_t *st, uint64_t len, int n, uint32_t dtype, const uint16_t f[256],
                              uint32_t *v) {
    uint32_t hdr = rd16(st);
    uint32_t mode = hdr & 7;
    if (hdr >> 3) return ORC_ERR_MALFORMED;
    if (mode == 0) {
        if (len != 4) return ORC_ERR_MALFORMED;
        uint32_t c = rd16(st + 2);
        if (c > maxval(dtype)) return ORC_ERR_MALFORMED;
        for (int j = 0; j < n; j++) v[j] = c;
        return ORC_OK;
    }
    if (mode == 2) {
        if (len != raw_bytes(n, dtype)) return ORC_ERR_MALFORMED;
        for (int j = 0; j < n; j++) v[j] = dtype == 2 ? rd16(st + 2 + 2 * j) : st[2 + j];
        if (dtype == 1 && n % 2 && st[2 + n]) return ORC_ERR_MALFORMED;
        return ORC_OK;
    }
    if (mode != 1) return ORC_ERR_MALFORMED;
    if (table_empty(f) || degenerate(f)) return ORC_ERR_MALFORMED;
    wreader r = {st, 2, len, 0};
    uint32_t x = next_word(&r);
    x |= next_word(&r) << 16;
    for (int j = 0; j < n; j++) {
        uint32_t t = x & 4095;
        /* symbol whose cumulative range holds slot t */
        uint32_t c = 0;
        int s = 0;
        while (!(t < c + f[s])) {
            c += f[s];
            s++;
        }
        x = f[s] * (x >> 12) + t - c;
        if (x < RANS_L) x = (x << 16) | next_word(&r);
        if (dtype == 2 && s == 255) {
            uint32_t lit = next_word(&r);
            if (lit < 255) return ORC_ERR_MALFORMED;
            v[j] = lit;
        } else {
            v[j] = (uint32_t)s;
        }
    }
    if (r.overrun || r.pos != len || x != RANS_L) return ORC_ERR_MALFORMED;
    return ORC_OK;
}

/* bit reader, LSB first */
typedef struct {
    const uint8_t *p;
    uint64_t bit, nbits;
    int overrun;
} bitr;

static uint32_t br_get(bitr *r, int nb) {
    uint32_t v = 0;
    for (int i = 0; i < nb; i++) {
        if (r->bit >= r->nbits) {
            r->overrun = 1;
            return 0;
        }
        v |= (uint32_t)((r->p[r->bit >> 3] >> (r->bit & 7)) & 1) << i;
        r->bit++;
    }
    return v;
}

typedef struct {
    uint16_t sym[TL];
    uint8_t nbits[TL];
    uint16_t newX[TL];
} dec_table;

static int decode_paired_stream(const uint8_t *st, uint64_t len, uint32_t dtype, const dec_table *dt,
                                const uint32_t *a0s, const uint32_t *in_use, uint32_t *v) {
    uint32_t hdr = rd16(st);
    uint32_t mode = hdr & 7, model = (hdr >> 3) & 31;
    if (hdr >> 8) return ORC_ERR_MALFORMED;
    if (mode != 3 && model) return ORC_ERR_MALFORMED;
    const uint32_t mv = maxval(dtype);
    switch (mode) {
    case 0:
        if (len != 2) return ORC_ERR_MALFORMED;
        for (int j = 0; j < BLOCK; j++) v[j] = 0;
        return ORC_OK;
    case 1: {
        if (len != 4) return ORC_ERR_MALFORMED;
        uint32_t c = rd16(st + 2);
        if (c == 0 || c > mv) return ORC_ERR_MALFORMED;
        for (int j = 0; j < BLOCK; j++) v[j] = c;
        return ORC_OK;
    }
    case 2: {
        if (len < 4) return ORC_ERR_MALFORMED;
        uint32_t nnz = rd16(st + 2);
        if (nnz == 0 || nnz > BLOCK) return ORC_ERR_MALFORMED;
        uint64_t need = 2 + 2 + 2 * (uint64_t)nnz + (dtype == 2 ? 2 * (uint64_t)nnz : nnz + nnz % 2);
        if (len != need) return ORC_ERR_MALFORMED;
        for (int j = 0; j < BLOCK; j++) v[j] = 0;
        int prev = -1;
        for (uint32_t k = 0; k < nnz; k++) {
            int pos = rd16(st + 4 + 2 * k);
            if (pos <= prev || pos >= BLOCK) return ORC_ERR_MALFORMED;
            uint32_t val = dtype == 2 ? rd16(st + 4 + 2 * nnz + 2 * k) : st[4 + 2 * nnz + k];
            if (val == 0) return ORC_ERR_MALFORMED;
            v[pos] = val;
            prev = pos;
        }
        if (dtype == 1 && nnz % 2 && st[4 + 3 * nnz]) return ORC_ERR_MALFORMED;
        return ORC_OK;
    }
    case 3: {
        if (len < 4) return ORC_ERR_MALFORMED;
        const dec_table *T = &dt[model];
        const uint32_t a0 = a0s[model];
        const int lit = dtype == 2 ? 16 : 8;
        bitr r = {st + 2, 0, (len - 2) * 8, 0};
        int X = (int)br_get(&r, 10);
        for (int t = 0; t < 256; t++) {
            int sym = T->sym[X];
            X = T->newX[X] + (int)br_get(&r, T->nbits[X]);
            int ws[2] = {sym >> 4, sym & 15};
            for (int h = 0; h < 2; h++) {
                uint32_t val;
                if (ws[h] == 15) {
                    val = br_get(&r, lit);
                    if (window_sym(val, a0, in_use[model]) != 15) return ORC_ERR_MALFORMED;
                } else {
                    val = a0 + (uint32_t)ws[h];
                    if (val > mv) return ORC_ERR_MALFORMED;
                }
                v[2 * t + h] = val;
            }
        }
        if (r.overrun || X != 0) return ORC_ERR_MALFORMED;
        /* only zero padding, fewer than 16 bits, may remain */
        if (r.nbits - r.bit >= 16) return ORC_ERR_MALFORMED;
        while (r.bit < r.nbits)
            if (br_get(&r, 1)) return ORC_ERR_MALFORMED;
        return ORC_OK;
    }
    case 4:
        if (len != raw_bytes(BLOCK, dtype)) return ORC_ERR_MALFORMED;
        for (int j = 0; j < BLOCK; j++) v[j] = dtype == 2 ? rd16(st + 2 + 2 * j) : st[2 + j];
        return ORC_OK;
    default:
        return ORC_ERR_MALFORMED;
    }
}

/*
 * Decode every stream of the blob into dense native counts (S x P), or the
 * u16 codes of a scaled blob. On a malformed stream returns ORC_ERR_MALFORMED
 * and reports the first bad (block, pixel).
 */
int orc_decode(const uint8_t *blob, uint64_t nbytes, void *counts, int64_t *bad_block, int64_t *bad_pixel) {
    parsed ps;
    int rc = parse(blob, nbytes, &ps);
    if (rc) return rc;
    if (bad_block) *bad_block = -1;
    if (bad_pixel) *bad_pixel = -1;
    uint16_t *model_n = NULL;
    uint32_t a0s[32], in_use[32];
    dec_table *dt = NULL;
    uint16_t spread[TL];
    if (ps.g.layout == 1) {
        /* the stored model tables must be the ones the format defines */
        model_n = (uint16_t *)malloc(2 * 32 * 256);
        orc_pair_models(model_n, a0s, in_use);
        for (int i = 0; i < 32 * 256; i++)
            if (rd16(blob + ps.table + 2 * i) != model_n[i]) {
                free(model_n);
                return ORC_ERR_MALFORMED;
            }
        dt = (dec_table *)malloc(sizeof(dec_table) * 32);
        for (int m = 0; m < 32; m++) {
            int pos = 0;
            for (int i = 0; i < 256; i++)
                for (int k = 0; k < model_n[256 * m + i]; k++) {
                    spread[pos] = (uint16_t)i;
                    pos = (pos + 643) % TL;
                }
            decode_entries(model_n + 256 * m, spread, dt[m].sym, dt[m].nbits, dt[m].newX);
        }
    }
    uint32_t v[BLOCK];
    for (uint64_t b = 0; b < ps.nb; b++) {
        const uint8_t *d = blob + ps.dir + 16 * b;
        int n = (int)rd32(d + 8);
        uint64_t expect = ps.S - b * BLOCK < BLOCK ? ps.S - b * BLOCK : BLOCK;
        if ((uint64_t)n != expect) {
            free(model_n);
            free(dt);
            return ORC_ERR_MALFORMED;
        }
        uint16_t f[256];
        if (ps.g.layout == 0) {
            uint32_t sum = 0;
            for (int s = 0; s < 256; s++) {
                f[s] = rd16(blob + ps.table + 2 * (256 * b + s));
                sum += f[s];
            }
            if (sum != 0 && sum != 4096) {
                free(model_n);
                free(dt);
                return ORC_ERR_MALFORMED;
            }
        }
        for (uint64_t p = 0; p < ps.P; p++) {
            uint64_t st, en;
            rc = stream_extent(&ps, b, p, &st, &en);
            if (!rc && en - st < 2) rc = ORC_ERR_MALFORMED;
            if (!rc) {
                const uint8_t *sp = blob + ps.payload + st;
                rc = ps.g.layout == 0 ? decode_rans_stream(sp, en - st, n, ps.g.dtype, f, v)
                                      : decode_paired_stream(sp, en - st, ps.g.dtype, dt, a0s, in_use, v);
            }
            if (rc) {
                if (bad_block) *bad_block = (int64_t)b;
                if (bad_pixel) *bad_pixel = (int64_t)p;
                free(model_n);
                free(dt);
                return rc;
            }
            for (int j = 0; j < n; j++) {
                uint64_t s = b * BLOCK + j;
                if (ps.g.dtype == 1)
                    ((uint8_t *)counts)[s * ps.P + p] = (uint8_t)v[j];
                else
                    ((uint16_t *)counts)[s * ps.P + p] = (uint16_t)v[j];
            }
        }
    }
    free(model_n);
    free(dt);
    return ORC_OK;
}

/* per-block calibration of a scaled blob: out[2b] = scale, out[2b+1] = offset */
int orc_calibration(const uint8_t *blob, uint64_t nbytes, double *out) {
    parsed ps;
    int rc = parse(blob, nbytes, &ps);
    if (rc) return rc;
    if (!ps.g.scaled) return ORC_ERR_ARG;
    for (uint64_t i = 0; i < 2 * ps.nb; i++) memcpy(&out[i], blob + ps.calib + 8 * i, 8);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* products on dense counts (their plain definitions)                  */
/* ------------------------------------------------------------------ */

/* out[s] = sum over p with mask[p] && valid[p] of I[s,p]; 0 for skipped blocks */
int orc_masked_sum(const void *counts, uint32_t dtype, uint64_t S, uint64_t P, const uint8_t *mask,
                   const uint8_t *valid, uint32_t stride, uint64_t *out) {
    if (stride < 1) return ORC_ERR_ARG;
    for (uint64_t s = 0; s < S; s++) {
        uint64_t acc = 0;
        if ((s / BLOCK) % stride == 0)
            for (uint64_t p = 0; p < P; p++)
                if (mask[p] && (!valid || valid[p])) acc += at(counts, dtype, s, P, p);
        out[s] = acc;
    }
    return ORC_OK;
}

/* Sum and mean diffraction pattern: the dual of a virtual image, summing the
 * frames of the selected scans ("Scaled uint16 resident intensities", "MPS
 * implementation": mean diffraction queries accumulated straight from the
 * resident). Selected scans: scan_mask[s] != 0 (every scan when scan_mask is
 * NULL) in visited blocks ((s / 512) % stride == 0); n is their number.
 *   sum[p]  = sum of I[s,p] over the selected scans, for valid p (0 otherwise)
 *   mean[p] = (float)((double)sum[p] / n), 0 when n = 0
 * For scaled residents (calib = (scale, offset) per 512-scan region) the mean
 * is that of the reconstructed intensities code*scale + offset, accumulated
 * region by region in increasing order: acc += scale_b * C_b[p] + n_b * offset_b,
 * every product and sum rounded in float64, then acc / n rounded to float32. */
int orc_sum_dp(const void *counts, uint32_t dtype, uint64_t S, uint64_t P, const uint8_t *scan_mask,
               const uint8_t *valid, uint32_t stride, const double *calib, uint64_t *sum, float *mean) {
    if (stride < 1) return ORC_ERR_ARG;
    const uint64_t nb = (S + BLOCK - 1) / BLOCK;
    uint64_t n = 0;
    for (uint64_t s = 0; s < S; s++)
        if ((s / BLOCK) % stride == 0 && (!scan_mask || scan_mask[s])) n++;
    for (uint64_t p = 0; p < P; p++) {
        sum[p] = 0;
        mean[p] = 0.0f;
        if (valid && !valid[p]) continue;
        volatile double acc = 0.0;
        for (uint64_t b = 0; b < nb; b += stride) {
            uint64_t cb = 0, n_b = 0;
            for (uint64_t s = b * BLOCK; s < S && s < (b + 1) * BLOCK; s++) {
                if (scan_mask && !scan_mask[s]) continue;
                cb += at(counts, dtype, s, P, p);
                n_b++;
            }
            sum[p] += cb;
            if (calib) {
                volatile double t1 = calib[2 * b] * (double)cb;
                volatile double t2 = (double)n_b * calib[2 * b + 1];
                volatile double t = t1 + t2;
                acc = acc + t;
            }
        }
        if (n) mean[p] = calib ? (float)(acc / (double)n) : (float)((double)sum[p] / (double)n);
    }
    return ORC_OK;
}

/* exact moments, then one float64 division rounded to float32 (0 when M0 = 0) */
int orc_com(const void *counts, uint32_t dtype, uint64_t S, uint32_t det_rows, uint32_t det_cols,
            const uint8_t *mask, const uint8_t *valid, float *row, float *col, uint64_t *m0_out) {
    const uint64_t P = (uint64_t)det_rows * det_cols;
    for (uint64_t s = 0; s < S; s++) {
        uint64_t m0 = 0, mr = 0, mc = 0;
        for (uint64_t p = 0; p < P; p++) {
            if ((mask && !mask[p]) || (valid && !valid[p])) continue;
            uint64_t v = at(counts, dtype, s, P, p);
            m0 += v;
            mr += v * (p / det_cols);
            mc += v * (p % det_cols);
        }
        if (m0_out) m0_out[s] = m0;
        row[s] = m0 ? (float)((double)mr / (double)m0) : 0.0f;
        col[s] = m0 ? (float)((double)mc / (double)m0) : 0.0f;
    }
    return ORC_OK;
}
