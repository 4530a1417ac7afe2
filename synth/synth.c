/*
 * Seeded synthetic 4D-STEM detector counts.
 *
 * Input generation only: nothing in this file encodes, decodes or reduces.
 * Both the CPU oracle and the GPU library take their inputs from here, so the
 * two sides see identical counts.
 *
 * Counts are Poisson draws whose mean is lam_in inside a bright-field disk and
 * lam_out outside it. The disk is centred at (cr, cc) plus an integer shift per
 * scan: none, a jitter of -1/0/+1 per axis, or a smooth random field of up to
 * +-3 pixels. Optional sentinel pixels hold the dtype maximum in every frame.
 *
 * Randomness is counter based: u = (splitmix64(key) >> 11) * 2^-53 with
 * splitmix64 as published by Steele, Lea and Flood (2014), keyed by
 * (seed, scan, pixel), so any scan range can be generated independently and in
 * parallel. The Poisson draw is an inverse-CDF search in a float64 table.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define SALT_JITTER 0xA5A5A5A5F00DF00DULL
#define SALT_FIELD 0x3C3C3C3C12345678ULL
#define SALT_SENT 0x5EA7E1A15EA7E1A1ULL
#define SALT_NOISE 0x0123456789ABCDEFULL
#define KMAX 200

typedef struct {
    uint32_t scan_rows, scan_cols, det_rows, det_cols;
    uint32_t dtype;        /* 1 = uint8, 2 = uint16 */
    uint32_t shift_kind;   /* 0 none, 1 jitter +-1, 2 smooth field +-3 */
    uint32_t sentinel_pct; /* pixel is a sentinel iff hash % 100 < pct */
    uint32_t pad_;
    double lam_in, lam_out;
    double cr, cc, radius;
    uint64_t seed;
} synth_params;

static inline uint64_t splitmix64(uint64_t z) {
    z += GOLDEN;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline double unit(uint64_t salt_seed, uint64_t counter) {
    uint64_t h = splitmix64((salt_seed * GOLDEN) ^ counter);
    return (double)(h >> 11) * (1.0 / 9007199254740992.0);
}

/* cumulative Poisson table: cdf[k] = P(X <= k); returns the last index */
static int poisson_cdf(double lam, double *cdf) {
    double p = exp(-lam), c = p;
    int k = 0;
    cdf[0] = c;
    while (k < KMAX - 1 && c < 1.0 - 1e-17) {
        k++;
        p = p * lam / (double)k;
        c += p;
        cdf[k] = c;
    }
    return k;
}

static inline uint32_t draw(const double *cdf, int kmax, double u) {
    int k = 0;
    while (k < kmax && !(u < cdf[k])) k++;
    return (uint32_t)k;
}

/* smooth field parameters: 4 terms x (a, k, l, phi), two axes */
static void field_params(const synth_params *sp, double prm[2][4][4]) {
    uint64_t salt = sp->seed ^ SALT_FIELD;
    uint64_t ctr = 1;
    for (int ax = 0; ax < 2; ax++)
        for (int m = 0; m < 4; m++) {
            prm[ax][m][0] = 0.5 + 0.5 * unit(salt, ctr++);
            prm[ax][m][1] = (double)(1 + (int)(3.0 * unit(salt, ctr++)));
            prm[ax][m][2] = (double)(1 + (int)(3.0 * unit(salt, ctr++)));
            prm[ax][m][3] = 2.0 * M_PI * unit(salt, ctr++);
        }
}

/* integer disk shift of scan s */
void synth_shift(const synth_params *sp, uint64_t s, int32_t *dr, int32_t *dc) {
    *dr = 0;
    *dc = 0;
    if (sp->shift_kind == 1) {
        uint64_t h = splitmix64(((sp->seed ^ SALT_JITTER) * GOLDEN) ^ (s + 1));
        *dr = (int32_t)(h % 3) - 1;
        *dc = (int32_t)((h / 3) % 3) - 1;
    } else if (sp->shift_kind == 2) {
        double prm[2][4][4];
        field_params(sp, prm);
        double u = (double)(s / sp->scan_cols) / (double)sp->scan_rows;
        double v = (double)(s % sp->scan_cols) / (double)sp->scan_cols;
        int32_t out[2];
        for (int ax = 0; ax < 2; ax++) {
            double num = 0.0, den = 0.0;
            for (int m = 0; m < 4; m++) {
                num += prm[ax][m][0] *
                       sin(2.0 * M_PI * (prm[ax][m][1] * u + prm[ax][m][2] * v) + prm[ax][m][3]);
                den += prm[ax][m][0];
            }
            out[ax] = (int32_t)rint(3.0 * num / den);
        }
        *dr = out[0];
        *dc = out[1];
    }
}

int synth_is_sentinel(const synth_params *sp, uint32_t p) {
    if (sp->sentinel_pct == 0) return 0;
    uint64_t h = splitmix64(((sp->seed ^ SALT_SENT) * GOLDEN) ^ ((uint64_t)p + 1));
    return (h % 100) < sp->sentinel_pct;
}

typedef struct {
    const synth_params *sp;
    uint64_t s0, s1; /* scan range of this worker */
    uint64_t first;  /* first scan of the output buffer */
    void *out;
    float *fout; /* scaled variant */
    const double *cin, *cout;
    int kin, kout;
    const uint8_t *sent;
} job;

static void *worker(void *arg) {
    const job *j = (const job *)arg;
    const synth_params *sp = j->sp;
    const uint32_t R = sp->det_rows, C = sp->det_cols, P = R * C;
    const uint32_t maxv = sp->dtype == 1 ? 255u : 65535u;
    const double r2 = sp->radius * sp->radius;
    const uint64_t salt_noise = sp->seed ^ SALT_NOISE;
    const uint64_t key = sp->seed * GOLDEN, key_noise = salt_noise * GOLDEN;
    const double *cin = j->cin, *cout = j->cout;
    const int kin = j->kin, kout = j->kout;
    const uint8_t *sent = j->sent;
    float *fout = j->fout;
    uint8_t *o8 = sp->dtype == 1 ? (uint8_t *)j->out : NULL;
    uint16_t *o16 = sp->dtype == 2 ? (uint16_t *)j->out : NULL;
    for (uint64_t s = j->s0; s < j->s1; s++) {
        int32_t dr, dc;
        synth_shift(sp, s, &dr, &dc);
        const double cr = sp->cr + dr, cc = sp->cc + dc;
        const uint64_t row = (s - j->first) * (uint64_t)P;
        const uint64_t ctr0 = s * (uint64_t)P + 1;
        for (uint32_t kr = 0; kr < R; kr++) {
            const double dy2 = ((double)kr - cr) * ((double)kr - cr);
            for (uint32_t kc = 0; kc < C; kc++) {
                const uint32_t p = kr * C + kc;
                const double d2 = dy2 + ((double)kc - cc) * ((double)kc - cc);
                const uint64_t ctr = ctr0 + p;
                const double u = (double)(splitmix64(key ^ ctr) >> 11) * (1.0 / 9007199254740992.0);
                uint32_t v = d2 <= r2 ? draw(cin, kin, u) : draw(cout, kout, u);
                if (v > maxv) v = maxv;
                if (fout) {
                    const double n = (double)(splitmix64(key_noise ^ ctr) >> 11) * (1.0 / 9007199254740992.0);
                    fout[row + p] = (float)(0.731 * (double)v - 0.25 + 0.1 * (n - 0.5));
                    continue;
                }
                if (sent && sent[p]) v = maxv;
                if (o8)
                    o8[row + p] = (uint8_t)v;
                else
                    o16[row + p] = (uint16_t)v;
            }
        }
    }
    return NULL;
}

static int run(const synth_params *sp, uint64_t first, uint64_t n, void *out, float *fout,
               int threads) {
    if (!sp || (!out && !fout) || sp->det_rows == 0 || sp->det_cols == 0) return -1;
    if (sp->dtype != 1 && sp->dtype != 2) return -1;
    double cin[KMAX], cout[KMAX];
    int kin = poisson_cdf(sp->lam_in, cin), kout = poisson_cdf(sp->lam_out, cout);
    const uint32_t P = sp->det_rows * sp->det_cols;
    uint8_t *sent = NULL;
    if (sp->sentinel_pct && !fout) {
        sent = (uint8_t *)malloc(P);
        if (!sent) return -2;
        for (uint32_t p = 0; p < P; p++) sent[p] = (uint8_t)synth_is_sentinel(sp, p);
    }
    if (threads < 1) threads = 1;
    if ((uint64_t)threads > n) threads = n ? (int)n : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * threads);
    job *jobs = (job *)malloc(sizeof(job) * threads);
    for (int t = 0; t < threads; t++) {
        jobs[t] = (job){sp, first + n * t / threads, first + n * (t + 1) / threads, first, out, fout,
                        cin, cout, kin, kout, sent};
        pthread_create(&tid[t], NULL, worker, &jobs[t]);
    }
    for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
    free(tid);
    free(jobs);
    free(sent);
    return 0;
}

/* counts of scans [first, first+n) into out[(s-first)*P + p] (native dtype) */
int synth_counts(const synth_params *sp, uint64_t first, uint64_t n, void *out, int threads) {
    return run(sp, first, n, out, NULL, threads);
}

/* float32 intensities 0.731*count - 0.25 + 0.1*(u - 1/2) from sentinel-free counts */
int synth_scaled(const synth_params *sp, uint64_t first, uint64_t n, float *out, int threads) {
    return run(sp, first, n, NULL, out, threads);
}
