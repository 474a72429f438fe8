/*
 * gradagg.h - C ABI of the MI355X gradient-aggregation library (libgradagg.so).
 *
 * The library aggregates the weight gradients of W data-parallel workers that
 * are held as W buffers in one GPU's HBM, and applies the momentum-SGD update
 * to binary32 master weights.  Sources, cited by page title and section:
 *
 *   [FC] "FireCaffe: near-linear acceleration of deep neural network training
 *        on compute clusters" (paperlayer summary): sec. 4 (every worker holds
 *        the model and computes local weight gradients, which are aggregated),
 *        sec. 6 (allreduce = elementwise sum of the workers' |grad W|-long
 *        vectors; binary reduction tree, branching factor 2, depth log2 p;
 *        aggregation reproduces single-GPU numerics), FAQ (deterministic for a
 *        fixed seed and GPU count; Caffe compatibility).
 *   [GF] "Optimizing Network Performance for Distributed DNN Training on GPU
 *        Clusters: ImageNet/AlexNet Training in 1.5 Minutes" (arXiv abstract):
 *        lazy allreduce (fuse many communication operations into one),
 *        mixed-precision transport, coarse-grained sparse communication (send
 *        only important gradient chunks).
 *
 * Terms.  W = workers, L = layers, P = sum of the layers' element counts,
 * ld = row stride of a per-worker buffer in elements (P rounded up to 64),
 * C = chunk size in elements, n_c = ceil(P / C) chunks per worker (the last
 * one may be shorter; chunks run across layer boundaries), k = chunks kept per
 * worker, mw = ceil(n_c / 32) mask words per worker.
 *
 * Buffers.  A "bucket" is a [W][ld] row-major array of gradients, binary32 or
 * binary16 (GA_FP16), row w holding worker w's fused gradient in layer order
 * with no gap between layers; elements P..ld-1 of a row are padding, never
 * read into a result.  A "residual" is a [W][ld] binary32 array.  Gradient,
 * weight and velocity vectors are [P] binary32.
 *
 * Ownership.  The caller allocates and owns every buffer passed in; all
 * pointers named d_* are device pointers on the plan's device.  A plan owns
 * small device tables (layer offsets, the layer of each wavefront tile) and,
 * for a chunk longer than 2048 elements, a workspace of W * n_c * ceil(C/2048)
 * binary64 partial chunk sums, all allocated in ga_plan_create and freed in
 * ga_plan_destroy.  Every call is asynchronous on `stream`, allocates nothing
 * and does not synchronize.  A plan may be shared by threads and streams, with
 * one exception: the storing norm passes (ga_chunk_norm, ga_chunk_norm_topk,
 * ga_chunk_norm_layers, and ga_chunk_norm_deferred with store != 0) write the
 * plan's workspace when C > 2048, so two of them on one plan must not run at
 * the same time (issue them on one stream or order them with events).  Host
 * arrays are read before return.
 *
 * Errors.  Arguments are validated on the host before any launch: a bad size,
 * a NULL pointer or a keep ratio outside [0,1] gives GA_ERR_INVALID; a device
 * pointer that is not 16-byte aligned gives GA_ERR_ALIGN; a failed launch or
 * runtime call gives GA_ERR_DEVICE; a size beyond a kernel's limit gives
 * GA_ERR_UNSUPPORTED.  On error nothing is launched (except GA_ERR_DEVICE,
 * raised by the launch itself) and ga_last_error() describes it.  A fault
 * inside a kernel surfaces at the caller's next synchronization.  No C++
 * exception crosses this interface.
 *
 * Determinism.  Every result is a fixed function of the inputs: the summation
 * order is the fixed tree below, no floating-point value is accumulated by
 * atomics (the only atomics are integer increments of the top-k's histogram
 * counters in LDS, whose totals do not depend on their order), and repeated
 * calls give bitwise identical outputs [FC FAQ].
 */
#ifndef GRADAGG_H
#define GRADAGG_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GA_ABI_VERSION 4
#define GA_MAX_WORKERS 1024
#define GA_MAX_CHUNKS 65536
/* Most elements per worker (P) of a plan or an SGD call: every 1-D grid of
   4 or more elements per thread then stays within 2^31 work-items. */
#define GA_MAX_ELEMENTS ((int64_t)1 << 33)

typedef enum {
    GA_OK = 0,
    GA_ERR_INVALID = 1,
    GA_ERR_ALIGN = 2,
    GA_ERR_DEVICE = 3,
    GA_ERR_UNSUPPORTED = 4
} ga_status;

typedef enum { GA_FP32 = 0, GA_FP16 = 1 } ga_dtype;

/* Summation orders of ga_reduce_variant. */
typedef enum { GA_ORDER_TREE = 0, GA_ORDER_SERVER = 1, GA_ORDER_RING = 2 } ga_order;

/* Momentum SGD hyper-parameters (Caffe form, see ga_sgd_momentum_apply). */
typedef struct {
    float lr;
    float mu;
} ga_sgd;

typedef struct {
    int64_t P;          /* elements per worker */
    int64_t ld;         /* row stride of buckets and residuals, elements */
    int64_t chunk;      /* C, 0 for a dense-only plan */
    int64_t n_chunks;   /* n_c, 0 for a dense-only plan */
    int32_t W;
    int32_t n_layers;
    int32_t k;          /* chunks kept per worker */
    int32_t mask_words; /* mw */
    int32_t dtype;      /* ga_dtype of the gradients */
} ga_plan_info;

typedef struct ga_plan ga_plan;

/* Version of this interface (GA_ABI_VERSION). */
int32_t ga_abi_version(void);

/* Static name of a status code. */
const char* ga_status_str(ga_status s);

/* Message of the last failed call on this thread ("" if none). */
const char* ga_last_error(void);

/*
 * Plan arithmetic only (no device access): sizes for W workers and a layer
 * list (layer_numel[n_layers], host array, every entry >= 1).
 * chunk = 0 makes a dense-only plan; chunk >= 1 adds the sparse sizes with
 *   n_c = ceil(P / chunk) and k = min(n_c, ceil(keep_ratio * n_c - 1e-9)),
 *   i.e. the fewest chunks that are at least the keep ratio of all chunks.
 * Limits: 1 <= W <= GA_MAX_WORKERS, P <= GA_MAX_ELEMENTS, n_c <= GA_MAX_CHUNKS,
 * 0 <= keep_ratio <= 1; beyond them GA_ERR_UNSUPPORTED (sizes) or
 * GA_ERR_INVALID (W, keep_ratio).
 */
ga_status ga_plan_compute_info(int32_t W, int32_t n_layers, const int64_t* layer_numel,
                               ga_dtype grad_dtype, int64_t chunk, double keep_ratio,
                               ga_plan_info* out);

/* Create a plan on the current device (same arguments as above). */
ga_status ga_plan_create(int32_t W, int32_t n_layers, const int64_t* layer_numel,
                         ga_dtype grad_dtype, int64_t chunk, double keep_ratio, ga_plan** out);

/* Destroy a plan (NULL is ignored).  No call using it may still be queued. */
void ga_plan_destroy(ga_plan* plan);

ga_status ga_plan_get_info(const ga_plan* plan, ga_plan_info* out);

/*
 * Lazy allreduce fusion [GF]: copy every worker's per-layer gradient tensors
 * into one flat row of the bucket, in one launch.
 *   d_layer_ptrs: device array of W*n_layers device addresses, worker-major
 *                 (entry w*n_layers + l is worker w's layer l, a contiguous
 *                 tensor of layer_numel[l] elements of the plan's dtype).
 *                 Tensors need no particular alignment (16-byte aligned ones
 *                 are copied with 128-bit accesses).
 *   d_bucket:     [W][ld] output; the padding of each row is set to zero.
 * The copy is byte-exact: binary16 stays binary16.
 */
ga_status ga_bucket_pack(const ga_plan* plan, const uint64_t* d_layer_ptrs, void* d_bucket,
                         hipStream_t stream);

/*
 * Dense aggregation [FC sec. 6] with mixed-precision leaves [GF]:
 *   S[i] = T(0, W) over the workers' elements bucket[w][i], where
 *     T(lo, 1) = leaf_lo[i]   (binary16 leaves are widened exactly to binary32)
 *     T(lo, n) = T(lo, h) + T(lo + h, n - h),  h = largest power of two < n,
 *   i.e. a binary tree that adds adjacent nodes level by level and carries an
 *   odd last node up; every node is binary32.
 *   g[i] = S[i] * fl32(1/W)   (each worker reports the mean over its share of
 *   the batch, so the mean over workers is the single-GPU gradient).
 * d_grad: [P] output, or NULL not to store g.
 * sgd: NULL for no update; otherwise d_w and d_v ([P], in/out) receive the
 *   momentum-SGD update of ga_sgd_momentum_apply with g, fused in the same pass.
 * At least one of d_grad and sgd must be given.
 */
ga_status ga_tree_reduce(const ga_plan* plan, const void* d_bucket, float* d_grad,
                         const ga_sgd* sgd, float* d_w, float* d_v, hipStream_t stream);

/*
 * ga_tree_reduce with zero-copy fusion: the same result, with the leaves read
 * straight from every worker's per-layer tensors instead of a packed bucket
 * (lazy allreduce [GF] as one launch over all W*L tensors, no copy).
 *   d_layer_ptrs: as in ga_bucket_pack (W*n_layers device addresses,
 *                 worker-major).  16-byte aligned tensors are read with
 *                 128-bit loads, others element by element.
 */
ga_status ga_tree_reduce_layers(const ga_plan* plan, const uint64_t* d_layer_ptrs, float* d_grad,
                                const ga_sgd* sgd, float* d_w, float* d_v, hipStream_t stream);

/*
 * Dense aggregation under the other schemes of the pages, for comparison with
 * the tree (same bucket, mean and SGD as ga_tree_reduce):
 *   GA_ORDER_TREE    the tree of ga_tree_reduce [FC sec. 6];
 *   GA_ORDER_SERVER  a parameter server sums the gradients it receives, in
 *                    worker order: ((x0 + x1) + x2) + ... [FC sec. 6];
 *   GA_ORDER_RING    ring allreduce [GF]: the vector is cut into W segments of
 *                    Q = ceil(P/W) rounded up to 64 elements; segment s is
 *                    summed starting at worker s+1, each worker adding its
 *                    value to the partial sum it receives, worker s last.
 * wire_fp16 != 0: binary16 communication [GF] - every value sent between
 * workers is rounded to binary16 (nearest, ties to even), every add is
 * binary32: the right operand of each tree add, each ring partial sum passed
 * on, the gradients the server receives, and the broadcast sum, which is
 * rounded before the mean.  With GA_ORDER_TREE and wire_fp16 == 0 the result
 * equals ga_tree_reduce bit for bit.
 */
ga_status ga_reduce_variant(const ga_plan* plan, const void* d_bucket, ga_order order, int32_t wire_fp16,
                            float* d_grad, const ga_sgd* sgd, float* d_w, float* d_v, hipStream_t stream);

/*
 * Coarse-grained sparse communication [GF], part 1 (sparse plan required):
 * for every worker w and chunk c,
 *   a[w][i] = fl32(leaf(bucket[w][i]) + r[w][i])  for i in chunk c
 *   d_residual[w][i] <- a[w][i]
 *   d_keys[w*n_c + c] = sum over the chunk of (double)a^2   (binary64; each
 *                       square is exact; summation order is unspecified, so
 *                       keys agree with the exact sum to ~1e-15 relative)
 * r is d_residual, except that with d_prev_mask != NULL (lazy-zero mode) the
 * chunks whose bit is set in d_prev_mask[w][mw] are taken as zero and not read.
 * Pass the previous step's selection mask there after a gather with
 * zero_selected = 0.  d_residual must be all zero before the first step.
 */
ga_status ga_chunk_norm(const ga_plan* plan, const void* d_bucket, float* d_residual,
                        const uint32_t* d_prev_mask, double* d_keys, hipStream_t stream);

/*
 * ga_chunk_norm with zero-copy fusion: the gradient is read straight from the
 * workers' per-layer tensors (d_layer_ptrs as in ga_bucket_pack); a chunk that
 * spans several layers is assembled from each of them.  d_residual, the keys
 * and the lazy-zero mode are as in ga_chunk_norm.  Uses the plan's workspace
 * when C > 2048: not concurrently with another storing norm pass on the same
 * plan.
 */
ga_status ga_chunk_norm_layers(const ga_plan* plan, const uint64_t* d_layer_ptrs, float* d_residual,
                               const uint32_t* d_prev_mask, double* d_keys, hipStream_t stream);

/*
 * Part 2: per worker, select the k most important chunks by key (the squared
 * L2 norm orders chunks as the norm does): larger key first, a NaN key above
 * all others, equal keys by lower chunk index.
 *   d_sel_idx:  [W][k] selected chunk indices, ascending within each row
 *               (may be NULL when k == 0).
 *   d_sel_mask: [W][mw] bitmaps, bit (c & 31) of word c >> 5 set iff chosen;
 *               bits at or above n_c are zero.
 */
ga_status ga_chunk_topk(const ga_plan* plan, const double* d_keys, int32_t* d_sel_idx,
                        uint32_t* d_sel_mask, hipStream_t stream);

/* ga_chunk_norm followed by ga_chunk_topk on the same stream. */
ga_status ga_chunk_norm_topk(const ga_plan* plan, const void* d_bucket, float* d_residual,
                             const uint32_t* d_prev_mask, double* d_keys, int32_t* d_sel_idx,
                             uint32_t* d_sel_mask, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as ga_chunk_norm_topk, with its whole workspace in a fixed array
 * inside the library: the [W][n_c] binary64 keys (a caller buffer there) and,
 * for C > 2048, the W * n_c * ceil(C/2048) binary64 partial sums (the plan's
 * workspace there), so the plan's workspace is not used.  The array holds
 * GA_STATIC_KEYS binary64 values (32 MiB) on every device the library runs
 * on, until the process ends; its address on a device is looked up when a
 * plan is created there.  The call allocates nothing and calls no allocating
 * routine.  Every call on one device uses the same array, so calls that
 * overlap on one device (other streams, other threads) race; each call
 * overwrites every value it reads, so nothing needs clearing between calls.
 * Results equal ga_chunk_norm_topk's bit for bit.
 * Errors: those of ga_chunk_norm_topk (d_keys aside); GA_ERR_UNSUPPORTED when
 * W * n_c > GA_STATIC_KEYS, or, for C > 2048, W * n_c * (1 + ceil(C/2048)) >
 * GA_STATIC_KEYS; GA_ERR_DEVICE when the array's address could not be looked
 * up on the plan's device.
 */
#define GA_STATIC_KEYS ((int64_t)1 << 22)
ga_status ga_chunk_norm_topk_static(const ga_plan* plan, const void* d_bucket, float* d_residual,
                                    const uint32_t* d_prev_mask, int32_t* d_sel_idx, uint32_t* d_sel_mask,
                                    hipStream_t stream);

/*
 * Part 3: sum what the workers send.  Worker w sends t[w][i] = a[w][i] on its
 * selected chunks and nothing elsewhere; absent values enter the same fixed
 * tree as +0 (binary32 throughout, so residual + sent == a exactly):
 *   S[i] = T(0, W) over t[.][i];   g[i] = S[i] * fl32(1/W).
 * d_residual holds a (from ga_chunk_norm).  zero_selected != 0 sets the sent
 * chunks of d_residual to zero, leaving exactly the residual for the next
 * step; zero_selected == 0 leaves them (lazy-zero mode: pass d_sel_mask as
 * d_prev_mask of the next ga_chunk_norm; the residual is then d_residual with
 * the masked chunks read as zero).
 * d_grad, sgd, d_w, d_v: as in ga_tree_reduce.
 */
ga_status ga_sparse_gather_reduce(const ga_plan* plan, float* d_residual, const uint32_t* d_sel_mask,
                                  int32_t zero_selected, float* d_grad, const ga_sgd* sgd,
                                  float* d_w, float* d_v, hipStream_t stream);

/*
 * Coarse-grained sparse communication [GF] with a deferred residual, for
 * gradients held as per-layer tensors: the same step as ga_chunk_norm_layers
 * -> ga_chunk_topk -> ga_sparse_gather_reduce, moving fewer bytes.
 *
 * The residual recurrence is a_t = leaf_t + r_{t-1} (r_0 = 0), and r_t = +0 on
 * the chunks a worker sends at step t, a_t elsewhere.  d_residual (R, [W][ld]
 * binary32) is written only by a norm pass the caller marks as storing (it
 * writes a_t of every chunk) and by ga_residual_flush (it writes r_t).  Between
 * two writes the residual is re-formed from what the caller still holds,
 * described by a ga_history at step t:
 *   age            R was last written by step t-1-age's storing norm pass or
 *                  flush (0 <= age <= GA_MAX_AGE); a zero-filled R counts as
 *                  written at step 0;
 *   d_masks[j]     j = 0..age: the selection mask of step t-1-j ([W][mw], as
 *                  written by ga_chunk_topk), or NULL if no chunk counts as
 *                  sent then (steps before the first, or the step a flush ended);
 *   d_layer_ptrs[j] j = 0..age-1: the layer table of step t-1-j (as
 *                  d_layer_ptrs of ga_tree_reduce_layers); those tensors must
 *                  still hold that step's gradients.
 * For worker w and chunk c, let j be the smallest index whose mask has c set
 * for w: then r_{t-1} = g_{t-1} + (g_{t-2} + (... + (g_{t-j} + +0))), the j
 * gradients since that step added onto +0 (r_{t-1} = +0 for j = 0); if no mask
 * has it set, r_{t-1} = g_{t-1} + (... + (g_{t-age} + R)).  Every g is the
 * exact widening of the worker's gradient, and the adds are the recurrence's
 * own, in its order, so every value equals the plain recurrence bit for bit.
 *
 * One step t:
 *   ga_chunk_norm_deferred(g_t, hist, store)   keys; R <- a_t if store
 *   ga_chunk_topk(keys) -> m_t
 *   ga_sparse_gather_reduce_deferred(g_t, hist, store, m_t)
 * then the next step's history is {age 0, masks {m_t}} if this step stored,
 * else {age + 1, masks {m_t, the old masks}, tables {g_t, the old tables}}.
 * A caller that keeps D earlier gradient batches stores every D+1 steps (D = 0:
 * every step, which is the lazy-zero form; the mask buffers then rotate over
 * D+2 buffers).  A zero residual can be described without reading R: age 0
 * and d_masks[0] = a mask of all ones (every chunk "sent" before step 1).
 * Keys, selection, mean gradient, w and v equal the plain recurrence (and the
 * oracle) bit for bit.
 */
#define GA_MAX_AGE 2

typedef struct {
    int32_t age;
    const uint32_t* d_masks[GA_MAX_AGE + 1];
    const uint64_t* d_layer_ptrs[GA_MAX_AGE];
} ga_history;

/*
 * The norm pass of a deferred step: for every worker and chunk, a_t = g_t +
 * r_{t-1} (r_{t-1} re-formed as above), its key as in ga_chunk_norm, and with
 * store != 0, d_residual <- a_t on every chunk.  With store != 0 and C > 2048
 * it uses the plan's workspace: not concurrently with another storing norm
 * pass on the same plan.  d_layer_ptrs: this step's
 * layer table.  Errors: GA_ERR_INVALID (NULL argument, dense-only plan, age
 * outside [0, GA_MAX_AGE], a missing earlier table, an earlier table pointer
 * equal to this step's or to another earlier one: the tensors of different
 * steps must be different buffers), GA_ERR_ALIGN, GA_ERR_DEVICE.
 */
ga_status ga_chunk_norm_deferred(const ga_plan* plan, const uint64_t* d_layer_ptrs, const ga_history* hist,
                                 int32_t store, float* d_residual, double* d_keys, hipStream_t stream);

/*
 * The gather-reduce of a deferred step: worker w sends a_t on the chunks set
 * in d_sel_mask (read from d_residual if this step's norm pass stored, else
 * re-formed from the history as the norm pass formed it); absent values enter
 * the fixed tree as +0; g = S * fl32(1/W); d_grad, sgd, d_w, d_v as in
 * ga_tree_reduce.  d_residual is only read.  hist and stored: as given to
 * this step's norm pass.  d_sel_mask must differ from every history mask
 * (GA_ERR_INVALID); the chunk size must be a multiple of 256 elements
 * (GA_ERR_UNSUPPORTED).  Other errors as ga_chunk_norm_deferred.
 */
ga_status ga_sparse_gather_reduce_deferred(const ga_plan* plan, const uint64_t* d_layer_ptrs,
                                           const ga_history* hist, int32_t stored, const float* d_residual,
                                           const uint32_t* d_sel_mask, float* d_grad, const ga_sgd* sgd,
                                           float* d_w, float* d_v, hipStream_t stream);

/*
 * Write the residual after a deferred step into d_residual: r_t = +0 on the
 * chunks set in d_sel_mask, a_t elsewhere (already there if the step stored,
 * else re-formed from the history).  Arguments as given to the step's gather.
 * Afterwards d_residual is the whole residual (for a checkpoint, or before the
 * gradient tensors are reused), and the next step passes age 0 with
 * d_masks[0] = NULL: no earlier tensor or mask is needed to resume.  The
 * flush reads the buffer as R, so flush in place at most once per step's
 * history (a second call would add the history again on top of r_t); to keep
 * the live buffer, flush into a copy of it.
 * Errors as ga_sparse_gather_reduce_deferred (no chunk-size limit).
 */
ga_status ga_residual_flush(const ga_plan* plan, const uint64_t* d_layer_ptrs, const ga_history* hist,
                            int32_t stored, float* d_residual, const uint32_t* d_sel_mask, hipStream_t stream);

/*
 * Momentum SGD on binary32 master weights, Caffe form (FireCaffe runs Caffe
 * models and reproduces Caffe's numbers [FC FAQ]), per element:
 *   v <- fl(fl(mu * v) + fl(lr * g));   w <- fl(w - v)
 * three roundings, no fused multiply-add, no weight decay.
 * 0 <= P <= GA_MAX_ELEMENTS elements (GA_ERR_UNSUPPORTED above).
 */
ga_status ga_sgd_momentum_apply(int64_t P, const float* d_grad, float* d_w, float* d_v,
                                const ga_sgd* sgd, hipStream_t stream);

/*
 * The dense step split across G GPUs, as each GPU would run its part [FC
 * sec. 6: the reduction tree spans the nodes; its lower levels are local].
 * With W workers in G groups of m = W/G consecutive workers (m a power of
 * two), the W-worker tree T(0, W) is the G-leaf tree over the groups'
 * complete subtrees T(j*m, m), so
 *   1. every GPU sums its own m workers: ga_tree_partial;
 *   2. a reduce-scatter hands the owner of an element slice the G partial
 *      sums of that slice, one row per group in group order;
 *   3. the owner adds them in the tree's order, takes the mean over all W
 *      workers and applies SGD to its slice: ga_tree_combine;
 * and the result is bit for bit that of ga_tree_reduce over all W workers.
 *
 * ga_tree_partial: S[i] = T(0, W) over the plan's W rows of d_bucket (as in
 *   ga_tree_reduce), stored unscaled in d_sum ([P] binary32, 16-byte aligned).
 *   No mean, no SGD.
 */
ga_status ga_tree_partial(const ga_plan* plan, const void* d_bucket, float* d_sum, hipStream_t stream);

/*
 * ga_tree_combine: the owner's step.  plan: a binary32 plan with W = G rows
 * and the slice's length as its element count.  d_partials: [G][ld] binary32,
 * row j = group j's partial sums for the slice.  w_total: the number of
 * workers the partials stand for (>= 1); the mean is S * fl32(1/w_total).
 * d_grad, sgd, d_w, d_v: as in ga_tree_reduce, for the slice.
 * GA_ERR_INVALID for a binary16 plan or w_total < 1.
 */
ga_status ga_tree_combine(const ga_plan* plan, const float* d_partials, int32_t w_total, float* d_grad,
                          const ga_sgd* sgd, float* d_w, float* d_v, hipStream_t stream);

/*
 * Multi-bucket lazy allreduce [GF]: lazy allreduce fuses the layers' gradients
 * into buckets, and aggregation of a bucket overlaps with the computation of
 * the layers not yet produced.  A backward pass writes the last layer first,
 * so buckets are formed from the last layer towards the first.
 *
 * ga_bucket_boundaries (host only): cut n_layers layers of layer_numel[l]
 * elements of elem_bytes (2 or 4) bytes into buckets.  Walking from the last
 * layer down, a bucket is closed at the start of layer l once it holds at
 * least bucket_bytes per worker and that start offset (in elements of the
 * fused row) is a multiple of 8; layer 0 always closes the last bucket.
 * first_layer[b] (host array of n_layers entries) receives the first layer of
 * bucket b, bucket 0 being the one holding the last layer; bucket b spans
 * layers first_layer[b] .. first_layer[b-1]-1 (n_layers-1 for b = 0).
 * *n_buckets receives the count.  bucket_bytes >= 1; bucket_bytes = 1 makes
 * one bucket per aligned layer boundary, a huge value one bucket.
 */
ga_status ga_bucket_boundaries(int32_t n_layers, const int64_t* layer_numel, int32_t elem_bytes,
                               int64_t bucket_bytes, int32_t* first_layer, int32_t* n_buckets);

typedef struct ga_buckets ga_buckets;

/*
 * Bucket schedule of a plan (any plan; only its W, layers and dtype are used):
 * the buckets of ga_bucket_boundaries, each with a small device offset table of
 * its own (the only device memory it owns).  Created on the current device.
 */
ga_status ga_buckets_create(const ga_plan* plan, int64_t bucket_bytes, ga_buckets** out);

/* Destroy a schedule (NULL is ignored).  No call using it may still be queued. */
void ga_buckets_destroy(ga_buckets* buckets);

/* Number of buckets (0 for NULL). */
int32_t ga_buckets_count(const ga_buckets* buckets);

/*
 * Bucket b's layers (first_layer .. first_layer + n_layers - 1) and its slice
 * [elem_begin, elem_end) of the fused row, of w, v and g.  Output pointers may
 * be NULL.  GA_ERR_INVALID for b out of range.
 */
ga_status ga_bucket_range(const ga_buckets* buckets, int32_t b, int32_t* first_layer, int32_t* n_layers,
                          int64_t* elem_begin, int64_t* elem_end);

/*
 * Aggregate bucket b as ga_tree_reduce_layers does for the whole plan, on
 * elements [elem_begin, elem_end) only: same tree, mean and fused SGD, so that
 * reducing every bucket once gives bitwise the result of one
 * ga_tree_reduce_layers call.
 *   d_layer_ptrs: the whole plan's W*n_layers table (worker-major); only the
 *                 bucket's layers are read.
 *   ready:        NULL, or an event the stream waits for before the launch
 *                 (recorded by the producer once the bucket's layers are
 *                 written on every worker).
 *   d_grad, d_w, d_v: the whole [P] vectors (the bucket's slice is written).
 *   max_workgroups: 0 for the full grid (one workgroup of 256 threads per
 *                 2048 binary16 or 1024 binary32 elements); otherwise at most
 *                 this many workgroups, which stride over the elements, so
 *                 that a kernel running concurrently (the backward pass) keeps
 *                 the other compute units.  The result does not depend on it.
 */
ga_status ga_bucket_reduce_layers(const ga_buckets* buckets, int32_t b, const uint64_t* d_layer_ptrs,
                                  hipEvent_t ready, float* d_grad, const ga_sgd* sgd, float* d_w, float* d_v,
                                  int32_t max_workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GRADAGG_H */
