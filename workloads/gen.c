/*
 * Seeded synthetic input generator for the gradient-aggregation workloads.
 *
 * This module produces inputs only: gradient values, master weights and scale
 * draws.  It holds none of the aggregation arithmetic and is shared by the
 * CPU oracle side and the GPU side of every test and benchmark, so both see
 * byte-identical inputs.
 *
 * Definition (counter based, so any element can be produced independently):
 *   - SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): mix(z) with the published constants, and the
 *     n-th output of a generator seeded with s is mix(s + (n+1)*gamma).
 *   - Stream key = chained SplitMix64 outputs over (seed, kind, step, worker).
 *   - Element e of a stream belongs to pair p = e >> 1.  Output p gives two
 *     32-bit uniforms u1, u2 in (0,1); the Box-Muller transform (Box & Muller,
 *     Ann. Math. Stat. 1958) gives z = sqrt(-2 ln u1) * {cos,sin}(2 pi u2),
 *     cos for even e and sin for odd e (radius in binary64, angle in binary32,
 *     host libm).
 *   - value = (float)(z * (sigma * scale[segment(e)])).
 *   - fp16 outputs round that float to binary16, round-to-nearest-even.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm64_at(uint64_t state, uint64_t n) {
    return sm64_mix(state + (n + 1) * GAMMA);
}

uint64_t gagen_key(uint64_t seed, uint32_t kind, uint32_t step, uint32_t worker) {
    uint64_t k = sm64_at(seed, 0);
    k = sm64_at(k, kind);
    k = sm64_at(k, step);
    k = sm64_at(k, worker);
    return k;
}

uint64_t gagen_raw(uint64_t key, uint64_t n) { return sm64_at(key, n); }

/* Uniform double in (0,1) with 53 random bits. */
double gagen_uniform(uint64_t key, uint64_t n) {
    return ((double)(sm64_at(key, n) >> 11) + 0.5) * 0x1p-53;
}

/* The Box-Muller pair for pair index p: z0 = r cos t, z1 = r sin t with
 * r = sqrt(-2 ln u1) (binary64) and t = 2 pi u2 (binary32 sincosf). */
static inline void bm_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
    uint64_t x = sm64_at(key, p);
    double u1 = ((double)(x >> 32) + 0.5) * 0x1p-32;
    float u2 = (float)(((double)(x & 0xffffffffULL) + 0.5) * 0x1p-32);
    double r = sqrt(-2.0 * log(u1));
    float sn, cs;
    sincosf(6.2831853f * u2, &sn, &cs);
    *z0 = r * (double)cs;
    *z1 = r * (double)sn;
}

/* Standard normal for element e of the stream `key`. */
double gagen_normal(uint64_t key, uint64_t e) {
    double z0, z1;
    bm_pair(key, e >> 1, &z0, &z1);
    return (e & 1) ? z1 : z0;
}

/* binary32 -> binary16, round to nearest, ties to even (IEEE 754-2008). */
uint16_t gagen_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7fffffffu;
    if (ax >= 0x7f800000u) { /* inf or NaN */
        if (ax == 0x7f800000u) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | 0x7e00u | ((ax >> 13) & 0x3ffu));
    }
    uint32_t E = ax >> 23;              /* biased fp32 exponent */
    uint32_t full = (ax & 0x7fffffu) | (E ? 0x800000u : 0u);
    if (E < 113) {                      /* |f| < 2^-14: fp16 subnormal range */
        /* result m * 2^-24, m = full * 2^(E-126) (E==0 means 2^-149 units) */
        uint32_t shift = E ? (126u - E) : 125u;
        if (shift > 31) return (uint16_t)sign;
        uint32_t m = full >> shift;
        uint32_t rem = full & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1u);
        m += (uint32_t)(rem > half) | ((uint32_t)(rem == half) & m & 1u);
        return (uint16_t)(sign | m);    /* m == 1024 encodes 2^-14 exactly */
    }
    uint32_t h = ((E - 112u) << 10) | ((ax >> 13) & 0x3ffu);
    uint32_t rem = ax & 0x1fffu;
    h += (uint32_t)(rem > 0x1000u) | ((uint32_t)(rem == 0x1000u) & h & 1u);
    if (h >= 0x7c00u) h = 0x7c00u;      /* overflow rounds to infinity */
    return (uint16_t)(sign | h);
}

struct fill_job {
    uint64_t key;
    int64_t start, n;
    double sigma;
    int32_t n_seg;
    const int64_t* seg_end;
    const double* seg_scale;
    int32_t fp16;
    void* out;
    int64_t j0, j1;
};

static inline void put(const struct fill_job* J, int64_t j, double z, double scale) {
    float v = (float)(z * (J->sigma * scale));
    if (J->fp16)
        ((uint16_t*)J->out)[j] = gagen_f32_to_f16(v);
    else
        ((float*)J->out)[j] = v;
}

static inline double seg_scale_at(const struct fill_job* J, int32_t* s, int64_t e) {
    if (J->n_seg <= 0) return 1.0;
    while (*s < J->n_seg - 1 && J->seg_end[*s] <= e) (*s)++;
    return J->seg_scale[*s];
}

static void fill_range(const struct fill_job* J) {
    int32_t s = 0;
    int64_t j = J->j0;
    double z0, z1;
    if (j < J->j1 && ((J->start + j) & 1)) { /* odd first element: second half of a pair */
        int64_t e = J->start + j;
        bm_pair(J->key, (uint64_t)e >> 1, &z0, &z1);
        put(J, j, z1, seg_scale_at(J, &s, e));
        ++j;
    }
    for (; j + 1 < J->j1; j += 2) {
        int64_t e = J->start + j;
        bm_pair(J->key, (uint64_t)e >> 1, &z0, &z1);
        put(J, j, z0, seg_scale_at(J, &s, e));
        put(J, j + 1, z1, seg_scale_at(J, &s, e + 1));
    }
    if (j < J->j1) {
        int64_t e = J->start + j;
        bm_pair(J->key, (uint64_t)e >> 1, &z0, &z1);
        put(J, j, z0, seg_scale_at(J, &s, e));
    }
}

static void* fill_thread(void* p) {
    fill_range((const struct fill_job*)p);
    return 0;
}

/*
 * Fill out[0..n) with the values of stream elements start .. start+n-1.
 * Segment s covers stream elements [seg_end[s-1], seg_end[s]) (seg_end[-1]=0)
 * and scales its values by seg_scale[s]; n_seg == 0 means scale 1.
 * fp16 != 0 writes binary16 bit patterns, else binary32.
 */
int gagen_fill(uint64_t key, int64_t start, int64_t n, double sigma, int32_t n_seg,
               const int64_t* seg_end, const double* seg_scale, int32_t fp16, void* out,
               int32_t threads) {
    if (n < 0 || start < 0 || (n > 0 && !out)) return 1;
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if ((int64_t)threads > n / 65536 + 1) threads = (int32_t)(n / 65536 + 1);
    struct fill_job jobs[256];
    pthread_t tid[256];
    int started[256];
    for (int t = 0; t < threads; ++t) {
        struct fill_job J = {key, start, n, sigma, n_seg, seg_end, seg_scale, fp16, out,
                             n * t / threads, n * (t + 1) / threads};
        jobs[t] = J;
        started[t] = 0;
    }
    for (int t = 1; t < threads; ++t)
        started[t] = pthread_create(&tid[t], 0, fill_thread, &jobs[t]) == 0;
    fill_range(&jobs[0]);
    for (int t = 1; t < threads; ++t) {
        if (started[t])
            pthread_join(tid[t], 0);
        else
            fill_range(&jobs[t]);
    }
    return 0;
}
