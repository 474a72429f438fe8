/*
 * Oracle: a plain, slow, CPU-only statement of what the gradient-aggregation
 * hot path computes.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the benchmark's CPU-baseline leg call it; the product path never does.  It
 * shares no code, header or table with the GPU library.
 *
 * Sources (web pages, cited by title and section):
 *   [FC]  FireCaffe: near-linear acceleration of deep neural network training
 *         on compute clusters (paperlayer summary), sections 3, 4, 6 and the
 *         FAQ appendix.
 *   [GF]  Optimizing Network Performance for Distributed DNN Training on GPU
 *         Clusters: ImageNet/AlexNet Training in 1.5 Minutes (arXiv abstract).
 *
 * Compile with -O2 -ffp-contract=off -fno-fast-math: every float operation
 * below is one IEEE binary32 (or binary64) operation, rounded to nearest even.
 * Threads only split independent work (workers, or disjoint element ranges);
 * no arithmetic is reordered, so results do not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* A tiny parallel-for over items [0, n).                                    */
/* ------------------------------------------------------------------------ */
typedef void (*item_fn)(void* ctx, int64_t lo, int64_t hi);
struct pf_job { item_fn fn; void* ctx; int64_t lo, hi; };

static void* pf_thread(void* p) {
    struct pf_job* j = (struct pf_job*)p;
    j->fn(j->ctx, j->lo, j->hi);
    return 0;
}

static void parallel_for(int64_t n, int threads, item_fn fn, void* ctx) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if (threads > n) threads = (int)(n > 0 ? n : 1);
    struct pf_job jobs[256];
    pthread_t tid[256];
    int ok[256];
    for (int t = 0; t < threads; ++t) {
        jobs[t].fn = fn; jobs[t].ctx = ctx;
        jobs[t].lo = n * t / threads; jobs[t].hi = n * (t + 1) / threads;
        ok[t] = 0;
    }
    for (int t = 1; t < threads; ++t) ok[t] = pthread_create(&tid[t], 0, pf_thread, &jobs[t]) == 0;
    fn(ctx, jobs[0].lo, jobs[0].hi);
    for (int t = 1; t < threads; ++t) {
        if (ok[t]) pthread_join(tid[t], 0);
        else fn(ctx, jobs[t].lo, jobs[t].hi);
    }
}

/* ------------------------------------------------------------------------ */
/* binary16 decoding, from the IEEE 754 definition of the format:           */
/*   e == 0:  (-1)^s * m * 2^-24            (zero and subnormals)           */
/*   e == 31: infinity (m == 0) or NaN                                      */
/*   else:    (-1)^s * (1024 + m) * 2^(e-25)                                */
/* Mixed-precision transport [GF abstract]: gradients travel as binary16    */
/* and every sum is taken in binary32, so each leaf is this exact widening. */
/* ------------------------------------------------------------------------ */
float ora_f16_decode(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double mag;
    if (e == 0) mag = ldexp((double)m, -24);
    else if (e == 31) mag = m ? NAN : INFINITY;
    else mag = ldexp((double)(1024 + m), e - 25);
    return (float)(s ? -mag : mag);
}

static inline float leaf_value(const void* bucket, int fp16, int64_t ld, int w, int64_t i) {
    if (fp16) return ora_f16_decode(((const uint16_t*)bucket)[(int64_t)w * ld + i]);
    return ((const float*)bucket)[(int64_t)w * ld + i];
}

/* ------------------------------------------------------------------------ */
/* The binary reduction tree [FC sec. 6]: branching factor 2, depth         */
/* ceil(log2 W).  T(lo,1) = leaf lo;  T(lo,n) = T(lo,h) + T(lo+h,n-h) with  */
/* h the largest power of two below n, i.e. adjacent pairs are summed level */
/* by level and an odd last node is carried up.  Applied elementwise to the */
/* gradient vectors: allreduce is an elementwise sum of the workers'        */
/* vectors [FC sec. 6].                                                     */
/* ------------------------------------------------------------------------ */
typedef void (*leaf_fill)(const void* ctx, int w, int64_t i0, int64_t n, float* dst);

static void tree(leaf_fill leaf, const void* ctx, int lo, int cnt, int64_t i0, int64_t n,
                 float* out, float* scratch) {
    if (cnt == 1) { leaf(ctx, lo, i0, n, out); return; }
    int h = 1;
    while (2 * h < cnt) h *= 2;
    tree(leaf, ctx, lo, h, i0, n, out, scratch);
    float* right = scratch;
    tree(leaf, ctx, lo + h, cnt - h, i0, n, right, scratch + n);
    for (int64_t i = 0; i < n; ++i) out[i] = out[i] + right[i];
}

static int tree_depth(int W) { int d = 0; while ((1 << d) < W) ++d; return d; }

/* Mean over workers: each worker reports the mean gradient of its share of
 * the batch, so the mean of the W worker means reproduces the single-GPU
 * gradient [FC sec. 6].  Multiplying by the binary32 value of 1/W. */
static inline float inv_workers(int W) { return (float)(1.0 / (double)W); }

/* Momentum SGD on binary32 master weights, in the form Caffe uses (FireCaffe
 * runs Caffe models and matches Caffe's numbers [FC FAQ]):
 *   v <- mu*v + lr*g ;  w <- w - v     (three roundings, no fused multiply-add) */
static inline void sgd_one(float g, float lr, float mu, float* w, float* v) {
    float a = mu * *v;
    float b = lr * g;
    float vn = a + b;
    *v = vn;
    *w = *w - vn;
}

void ora_sgd(int64_t P, const float* gbar, float* w, float* v, float lr, float mu) {
    for (int64_t i = 0; i < P; ++i) sgd_one(gbar[i], lr, mu, &w[i], &v[i]);
}

/* Tree sum of W dense fp32 rows (leaves[w*n + i]), the building block alone. */
struct rows_ctx { const float* leaves; int64_t n; };
static void rows_leaf(const void* c, int w, int64_t i0, int64_t n, float* dst) {
    const struct rows_ctx* r = (const struct rows_ctx*)c;
    memcpy(dst, r->leaves + (int64_t)w * r->n + i0, (size_t)n * sizeof(float));
}

int ora_tree_sum(int32_t W, int64_t n, const float* leaves, float* out) {
    if (W < 1 || n < 0) return 1;
    if (n == 0) return 0;
    float* scratch = (float*)malloc(sizeof(float) * (size_t)n * (size_t)(tree_depth(W) + 1));
    if (!scratch) return 2;
    struct rows_ctx c = {leaves, n};
    tree(rows_leaf, &c, 0, W, 0, n, out, scratch);
    free(scratch);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dense step: tree over the decoded leaves, times 1/W, then momentum SGD.  */
/* ------------------------------------------------------------------------ */
struct dense_ctx {
    int W; int64_t P, ld; int fp16; const void* bucket;
    float lr, mu; float* w; float* v; float* gbar; int threads; int failed;
};

static void dense_leaf(const void* c, int wk, int64_t i0, int64_t n, float* dst) {
    const struct dense_ctx* d = (const struct dense_ctx*)c;
    for (int64_t j = 0; j < n; ++j) dst[j] = leaf_value(d->bucket, d->fp16, d->ld, wk, i0 + j);
}

static void dense_range(void* c, int64_t t0, int64_t t1) {
    struct dense_ctx* d = (struct dense_ctx*)c;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t i0 = d->P * t / d->threads, i1 = d->P * (t + 1) / d->threads, n = i1 - i0;
        if (n <= 0) continue;
        float* buf = (float*)malloc(sizeof(float) * (size_t)n * (size_t)(tree_depth(d->W) + 2));
        if (!buf) { d->failed = 1; continue; }
        float* S = buf;
        tree(dense_leaf, d, 0, d->W, i0, n, S, buf + n);
        float invW = inv_workers(d->W);
        for (int64_t j = 0; j < n; ++j) {
            float g = S[j] * invW;
            if (d->gbar) d->gbar[i0 + j] = g;
            if (d->w) sgd_one(g, d->lr, d->mu, &d->w[i0 + j], &d->v[i0 + j]);
        }
        free(buf);
    }
}

/* bucket: [W][ld] gradients (binary32, or binary16 bits when fp16 != 0).
 * w, v: [P] binary32 state updated in place (both NULL: no update).
 * gbar: [P] mean gradient out, or NULL. */
int ora_dense_step(int32_t W, int64_t P, int64_t ld, int32_t fp16, const void* bucket,
                   float lr, float mu, float* w, float* v, float* gbar, int32_t threads) {
    if (W < 1 || P < 0 || ld < P || !bucket || (!w) != (!v)) return 1;
    if (threads < 1) threads = 1;
    struct dense_ctx d = {W, P, ld, fp16, bucket, lr, mu, w, v, gbar, threads, 0};
    parallel_for(threads, threads, dense_range, &d);
    return d.failed ? 2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Coarse-grained sparse communication [GF abstract]: only important        */
/* gradient chunks are sent.  A chunk is a run of C consecutive elements of */
/* the fused flat gradient (the last one may be shorter).  Importance is    */
/* the chunk's L2 norm; we rank by its square, which orders identically.    */
/* ------------------------------------------------------------------------ */

/* Sum of squares of n binary32 values.  Each square is exact in binary64;
 * the sum is accumulated in long double with Neumaier's compensation so the
 * result is the real sum rounded (to within an ulp) to binary64. */
double ora_chunk_key(const float* a, int64_t n) {
    long double s = 0.0L, c = 0.0L;
    for (int64_t i = 0; i < n; ++i) {
        long double x = (long double)((double)a[i] * (double)a[i]);
        long double t = s + x;
        if (fabsl(s) >= fabsl(x)) c += (s - t) + x;
        else c += (x - t) + s;
        s = t;
    }
    if (!isfinite((double)s)) return (double)s;
    return (double)(s + c);
}

/* Number of chunks kept for keep ratio rho: the smallest count that is at
 * least rho of the chunks, clamped to [0, n_c]. */
int64_t ora_keep_count(int64_t n_chunks, double rho) {
    if (n_chunks <= 0) return 0;
    double k = ceil(rho * (double)n_chunks - 1e-9);
    if (k < 0) k = 0;
    if (k > (double)n_chunks) k = (double)n_chunks;
    return (int64_t)k;
}

struct kv { double key; int32_t idx; };

/* Importance order: larger key first, NaN above everything, equal keys by
 * lower chunk index. */
static int kv_cmp(const void* A, const void* B) {
    const struct kv* a = (const struct kv*)A;
    const struct kv* b = (const struct kv*)B;
    int an = isnan(a->key), bn = isnan(b->key);
    if (an != bn) return an ? -1 : 1;
    if (!an) {
        if (a->key > b->key) return -1;
        if (a->key < b->key) return 1;
    }
    return (a->idx > b->idx) - (a->idx < b->idx);
}

static int int_cmp(const void* A, const void* B) {
    int32_t a = *(const int32_t*)A, b = *(const int32_t*)B;
    return (a > b) - (a < b);
}

/* Select the k most important of n_c chunks.  idx_out gets their indices in
 * ascending order.  *margin (optional) gets (key_k - key_{k+1}) / key_k for
 * the last kept and first dropped keys (1 when k is 0 or n_c, 0 on a tie or
 * a zero/NaN boundary). */
int ora_topk(int64_t n_c, const double* keys, int32_t k, int32_t* idx_out, double* margin) {
    if (n_c < 0 || k < 0 || k > n_c) return 1;
    struct kv* e = (struct kv*)malloc(sizeof(struct kv) * (size_t)(n_c ? n_c : 1));
    if (!e) return 2;
    for (int64_t c = 0; c < n_c; ++c) { e[c].key = keys[c]; e[c].idx = (int32_t)c; }
    qsort(e, (size_t)n_c, sizeof(struct kv), kv_cmp);
    for (int32_t j = 0; j < k; ++j) idx_out[j] = e[j].idx;
    qsort(idx_out, (size_t)k, sizeof(int32_t), int_cmp);
    if (margin) {
        if (k == 0 || k == n_c) *margin = 1.0;
        else {
            double hi = e[k - 1].key, lo = e[k].key;
            if (isnan(hi) || isnan(lo) || !(hi > 0.0)) *margin = 0.0;
            else if (isinf(hi)) *margin = isinf(lo) ? 0.0 : 1.0;
            else *margin = (hi - lo) / hi;
        }
    }
    free(e);
    return 0;
}

struct sparse_ctx {
    int W; int64_t P, ld; int fp16; const void* bucket; int64_t C, n_c; int k; int mw;
    float* resid; double* keys; int32_t* sel_idx; uint32_t* sel_mask; double* margin;
    float lr, mu; float* w; float* v; float* gbar; int threads; int failed;
};

/* Per worker: a = leaf + r (the residual left over from earlier steps is
 * added before ranking), chunk keys on a, top-k, selection mask. */
static void sparse_select(void* c, int64_t w0, int64_t w1) {
    struct sparse_ctx* s = (struct sparse_ctx*)c;
    double* keys = (double*)malloc(sizeof(double) * (size_t)(s->n_c ? s->n_c : 1));
    if (!keys) { s->failed = 1; return; }
    for (int64_t wk = w0; wk < w1; ++wk) {
        float* a = s->resid + wk * s->ld;
        for (int64_t i = 0; i < s->P; ++i) a[i] = leaf_value(s->bucket, s->fp16, s->ld, (int)wk, i) + a[i];
        for (int64_t ch = 0; ch < s->n_c; ++ch) {
            int64_t i0 = ch * s->C, i1 = i0 + s->C < s->P ? i0 + s->C : s->P;
            keys[ch] = ora_chunk_key(a + i0, i1 - i0);
        }
        if (s->keys) memcpy(s->keys + wk * s->n_c, keys, sizeof(double) * (size_t)s->n_c);
        int32_t* idx = s->sel_idx + wk * s->k;
        double m = 1.0;
        if (ora_topk(s->n_c, keys, s->k, idx, &m)) s->failed = 1;
        if (s->margin) s->margin[wk] = m;
        uint32_t* mask = s->sel_mask + wk * s->mw;
        memset(mask, 0, sizeof(uint32_t) * (size_t)s->mw);
        for (int j = 0; j < s->k; ++j) mask[idx[j] >> 5] |= 1u << (idx[j] & 31);
    }
    free(keys);
}

static inline int chunk_selected(const struct sparse_ctx* s, int wk, int64_t i) {
    int64_t ch = i / s->C;
    return (s->sel_mask[(int64_t)wk * s->mw + (ch >> 5)] >> (ch & 31)) & 1u;
}

/* Transmitted value of worker wk at element i: a on its selected chunks,
 * +0 elsewhere; absent contributions stay in their place in the same tree. */
static void sparse_leaf(const void* c, int wk, int64_t i0, int64_t n, float* dst) {
    const struct sparse_ctx* s = (const struct sparse_ctx*)c;
    const float* a = s->resid + (int64_t)wk * s->ld;
    for (int64_t j = 0; j < n; ++j) dst[j] = chunk_selected(s, wk, i0 + j) ? a[i0 + j] : 0.0f;
}

static void sparse_reduce(void* c, int64_t t0, int64_t t1) {
    struct sparse_ctx* s = (struct sparse_ctx*)c;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t i0 = s->P * t / s->threads, i1 = s->P * (t + 1) / s->threads, n = i1 - i0;
        if (n <= 0) continue;
        float* buf = (float*)malloc(sizeof(float) * (size_t)n * (size_t)(tree_depth(s->W) + 2));
        if (!buf) { s->failed = 1; continue; }
        tree(sparse_leaf, s, 0, s->W, i0, n, buf, buf + n);
        float invW = inv_workers(s->W);
        for (int64_t j = 0; j < n; ++j) {
            float g = buf[j] * invW;
            if (s->gbar) s->gbar[i0 + j] = g;
            if (s->w) sgd_one(g, s->lr, s->mu, &s->w[i0 + j], &s->v[i0 + j]);
        }
        free(buf);
    }
}

/* What was sent leaves the residual; what was not stays for the next step. */
static void sparse_split(void* c, int64_t w0, int64_t w1) {
    struct sparse_ctx* s = (struct sparse_ctx*)c;
    for (int64_t wk = w0; wk < w1; ++wk) {
        float* r = s->resid + wk * s->ld;
        for (int64_t i = 0; i < s->P; ++i)
            if (chunk_selected(s, (int)wk, i)) r[i] = 0.0f;
    }
}

/* One sparse step.  resid: [W][ld] binary32, the residual carried in, and
 * the residual carried out (all-zero before the first step).  keys: [W][n_c]
 * or NULL.  sel_idx: [W][k] ascending chunk indices.  sel_mask: [W][mw]
 * bitmaps, mw = ceil(n_c/32).  margin: [W] or NULL. */
int ora_sparse_step(int32_t W, int64_t P, int64_t ld, int32_t fp16, const void* bucket,
                    int64_t C, int32_t k, float* resid, double* keys, int32_t* sel_idx,
                    uint32_t* sel_mask, double* margin, float lr, float mu, float* w, float* v,
                    float* gbar, int32_t threads) {
    if (W < 1 || P < 1 || ld < P || C < 1 || !bucket || !resid || (!w) != (!v)) return 1;
    int64_t n_c = (P + C - 1) / C;
    if (k < 0 || k > n_c || (k > 0 && !sel_idx) || !sel_mask) return 1;
    if (threads < 1) threads = 1;
    struct sparse_ctx s = {W, P, ld, fp16, bucket, C, n_c, k, (int)((n_c + 31) / 32),
                           resid, keys, sel_idx, sel_mask, margin, lr, mu, w, v, gbar, threads, 0};
    parallel_for(W, threads, sparse_select, &s);
    if (s.failed) return 2;
    parallel_for(threads, threads, sparse_reduce, &s);
    if (s.failed) return 2;
    parallel_for(W, threads, sparse_split, &s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Summation orders and wire precision of other aggregation schemes.        */
/*                                                                          */
/* Parameter server [FC sec. 6]: one server receives every worker's         */
/* gradient and sums them; read here as adding them in worker order,        */
/* ((x0 + x1) + x2) + ...                                                   */
/* Ring allreduce [GF abstract]: the vector is cut into W segments; segment */
/* s travels round the ring starting at worker s+1, each worker adding its  */
/* own gradient to the partial sum it receives, and worker s completes it.  */
/* Segment length Q = ceil(P/W) rounded up to 64 elements; segment s is     */
/* [s*Q, min((s+1)*Q, P)).                                                  */
/* Wire precision: with a binary16 wire (mixed-precision communication      */
/* [GF abstract]) every value sent between workers is rounded to binary16   */
/* and every add is binary32: in the tree the right operand of each add     */
/* (the subtree sum that was sent) and the final broadcast; at the server   */
/* the received gradients and the broadcast; on the ring each partial sum   */
/* passed on and the broadcast.                                             */
/* ------------------------------------------------------------------------ */

/* binary32 -> nearest binary16 value (ties to even), as a binary32: the     */
/* binary16 grid near |x| has spacing 2^(e-10) for 2^e <= |x| < 2^(e+1),    */
/* e >= -14, and 2^-24 below 2^-14; x/q is rounded to an integer with rint  */
/* (round-half-even) in binary64, where both the division by a power of two */
/* and the product are exact.  Beyond the largest finite value the result   */
/* is infinite (|x| >= 65520 rounds up).                                    */
float ora_round_f16(float x) {
    if (isnan(x) || isinf(x)) return x;
    double a = fabs((double)x);
    if (a >= 65520.0) return x > 0 ? INFINITY : -INFINITY;
    if (a == 0.0) return x;
    int e;
    frexp(a, &e);          /* a = f * 2^e, 0.5 <= f < 1, so 2^(e-1) <= a < 2^e */
    int ex = e - 1;
    if (ex < -14) ex = -14;
    double q = ldexp(1.0, ex - 10);
    double m = rint((double)x / q);
    return (float)(m * q);
}

static inline float wire(float x, int on) { return on ? ora_round_f16(x) : x; }

/* Tree with a wire: T(lo,n) = T(lo,h) + R(T(lo+h,n-h)); the left subtree's */
/* sum stays on the receiving worker, the right one was sent.               */
static float tree_wire(const float* leaf, int lo, int n, int on) {
    if (n == 1) return leaf[lo];
    int h = 1;
    while (2 * h < n) h *= 2;
    float left = tree_wire(leaf, lo, h, on);
    float right = tree_wire(leaf, lo + h, n - h, on);
    return left + wire(right, on);
}

int64_t ora_ring_segment(int32_t W, int64_t P) {
    int64_t q = (P + W - 1) / W;
    return (q + 63) / 64 * 64;
}

struct var_ctx {
    int W; int64_t P, ld; int fp16; const void* bucket; int order, wire; float lr, mu;
    float* w; float* v; float* gbar; int threads; int failed;
};

static void variant_range(void* c, int64_t t0, int64_t t1) {
    struct var_ctx* d = (struct var_ctx*)c;
    float* leaf = (float*)malloc(sizeof(float) * (size_t)d->W);
    if (!leaf) { d->failed = 1; return; }
    int64_t Q = ora_ring_segment(d->W, d->P);
    float invW = inv_workers(d->W);
    for (int64_t t = t0; t < t1; ++t) {
        int64_t i0 = d->P * t / d->threads, i1 = d->P * (t + 1) / d->threads;
        for (int64_t i = i0; i < i1; ++i) {
            for (int w = 0; w < d->W; ++w) leaf[w] = leaf_value(d->bucket, d->fp16, d->ld, w, i);
            float S;
            if (d->order == 0) {
                S = tree_wire(leaf, 0, d->W, d->wire);
            } else if (d->order == 1) {
                S = wire(leaf[0], d->wire);
                for (int w = 1; w < d->W; ++w) S = S + wire(leaf[w], d->wire);
            } else {
                int64_t seg = i / Q;
                int first = (int)((seg + 1) % d->W);
                S = leaf[first];
                for (int j = 1; j < d->W; ++j) {
                    int wk = (int)((seg + 1 + j) % d->W);
                    S = wire(S, d->wire) + leaf[wk];
                }
            }
            float g = wire(S, d->wire) * invW;
            if (d->gbar) d->gbar[i] = g;
            if (d->w) sgd_one(g, d->lr, d->mu, &d->w[i], &d->v[i]);
        }
    }
    free(leaf);
}

/* order: 0 binary tree, 1 parameter server (worker order), 2 ring.
 * wire16: nonzero for a binary16 wire.  Other arguments as ora_dense_step. */
int ora_reduce_variant(int32_t W, int64_t P, int64_t ld, int32_t fp16, const void* bucket, int32_t order,
                       int32_t wire16, float lr, float mu, float* w, float* v, float* gbar, int32_t threads) {
    if (W < 1 || P < 0 || ld < P || !bucket || (!w) != (!v) || order < 0 || order > 2) return 1;
    if (threads < 1) threads = 1;
    struct var_ctx d = {W, P, ld, fp16, bucket, order, wire16 != 0, lr, mu, w, v, gbar, threads, 0};
    parallel_for(threads, threads, variant_range, &d);
    return d.failed ? 2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Lazy allreduce [GF abstract]: many per-layer gradient tensors are fused  */
/* into one flat vector per worker so that one operation moves them all.    */
/* Layer l of worker w lands at offset sum_{m<l} numel_m of row w.          */
/* ------------------------------------------------------------------------ */
int ora_pack(int32_t W, int32_t L, const int64_t* numel, const void* const* layer_ptrs,
             int32_t elem_bytes, int64_t ld, void* bucket) {
    if (W < 1 || L < 1 || (elem_bytes != 2 && elem_bytes != 4)) return 1;
    int64_t P = 0;
    for (int l = 0; l < L; ++l) P += numel[l];
    if (P > ld) return 1;
    for (int w = 0; w < W; ++w) {
        int64_t off = 0;
        for (int l = 0; l < L; ++l) {
            memcpy((char*)bucket + ((int64_t)w * ld + off) * elem_bytes,
                   layer_ptrs[(int64_t)w * L + l], (size_t)(numel[l] * elem_bytes));
            off += numel[l];
        }
    }
    return 0;
}
