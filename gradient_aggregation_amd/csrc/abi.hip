// C ABI of libgradagg.so: plans, argument validation and launches.
// The operations are specified in include/gradagg.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "plan.h"

namespace {

thread_local char g_err[512];

ga_status fail(ga_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

ga_status ok() {
    g_err[0] = 0;
    return GA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

ga_status device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(GA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Fill a plan's sizes; shared by ga_plan_compute_info and ga_plan_create.
ga_status compute(int32_t W, int32_t L, const int64_t* numel, ga_dtype dt, int64_t chunk, double rho,
                  ga_plan_info* info) {
    if (!info) return fail(GA_ERR_INVALID, "info is NULL");
    if (W < 1 || W > GA_MAX_WORKERS) return fail(GA_ERR_INVALID, "W=%d outside [1,%d]", W, GA_MAX_WORKERS);
    if (L < 1) return fail(GA_ERR_INVALID, "n_layers=%d < 1", L);
    if (!numel) return fail(GA_ERR_INVALID, "layer_numel is NULL");
    if (dt != GA_FP32 && dt != GA_FP16) return fail(GA_ERR_INVALID, "unknown dtype %d", (int)dt);
    if (chunk < 0) return fail(GA_ERR_INVALID, "chunk=%lld < 0", (long long)chunk);
    if (!(rho >= 0.0 && rho <= 1.0)) return fail(GA_ERR_INVALID, "keep_ratio %g outside [0,1]", rho);
    int64_t P = 0;
    for (int32_t l = 0; l < L; ++l) {
        if (numel[l] < 1) return fail(GA_ERR_INVALID, "layer %d has %lld elements", l, (long long)numel[l]);
        if (numel[l] > ((int64_t)1 << 40) || P > ((int64_t)1 << 40))
            return fail(GA_ERR_UNSUPPORTED, "layer sizes too large");
        P += numel[l];
    }
    if (P > GA_MAX_ELEMENTS)
        return fail(GA_ERR_UNSUPPORTED, "P=%lld exceeds %lld elements", (long long)P, (long long)GA_MAX_ELEMENTS);
    memset(info, 0, sizeof *info);
    info->P = P;
    info->ld = (P + 63) / 64 * 64;
    info->W = W;
    info->n_layers = L;
    info->dtype = (int32_t)dt;
    if (chunk > 0) {
        if (chunk % 8 != 0)
            return fail(GA_ERR_UNSUPPORTED, "chunk=%lld is not a multiple of 8 elements", (long long)chunk);
        const int64_t n_c = (P + chunk - 1) / chunk;
        if (n_c > GA_MAX_CHUNKS)
            return fail(GA_ERR_UNSUPPORTED, "%lld chunks exceed %d", (long long)n_c, GA_MAX_CHUNKS);
        double k = ceil(rho * (double)n_c - 1e-9);
        if (k < 0) k = 0;
        if (k > (double)n_c) k = (double)n_c;
        info->chunk = chunk;
        info->n_chunks = n_c;
        info->k = (int32_t)k;
        info->mask_words = (int32_t)((n_c + 31) / 32);
    }
    return ok();
}

ga_plan_info info_of(const ga::Plan* p) {
    ga_plan_info i;
    memset(&i, 0, sizeof i);
    i.P = p->P;
    i.ld = p->ld;
    i.chunk = p->C;
    i.n_chunks = p->n_c;
    i.W = p->W;
    i.n_layers = p->L;
    i.k = p->k;
    i.mask_words = p->mw;
    i.dtype = p->dtype;
    return i;
}

const ga::Plan* as_plan(const ga_plan* p) { return reinterpret_cast<const ga::Plan*>(p); }

// The calling thread's current device must be the plan's.
ga_status check_device(const ga::Plan* p) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, "hipGetDevice");
    if (dev != p->device) return fail(GA_ERR_INVALID, "current device %d is not the plan's device %d", dev, p->device);
    return GA_OK;
}

}  // namespace

namespace ga {
// The fixed array of ga_chunk_norm_topk_static (noalloc.hip): look up its
// address on `device` (which must be current) once; then static_keys(device)
// returns it (nullptr before, or if the lookup failed).
hipError_t static_keys_setup(int device);
double* static_keys(int device);

// Record a failure message for ga_last_error (used by the other ABI sources).
ga_status api_fail(ga_status s, const char* msg) { return fail(s, "%s", msg); }
ga_status api_ok() { return ok(); }
}  // namespace ga

extern "C" {

int32_t ga_abi_version(void) { return GA_ABI_VERSION; }

const char* ga_status_str(ga_status s) {
    switch (s) {
        case GA_OK: return "GA_OK";
        case GA_ERR_INVALID: return "GA_ERR_INVALID";
        case GA_ERR_ALIGN: return "GA_ERR_ALIGN";
        case GA_ERR_DEVICE: return "GA_ERR_DEVICE";
        case GA_ERR_UNSUPPORTED: return "GA_ERR_UNSUPPORTED";
    }
    return "GA_ERR_UNKNOWN";
}

const char* ga_last_error(void) { return g_err; }

ga_status ga_plan_compute_info(int32_t W, int32_t n_layers, const int64_t* layer_numel, ga_dtype grad_dtype,
                               int64_t chunk, double keep_ratio, ga_plan_info* out) {
    return compute(W, n_layers, layer_numel, grad_dtype, chunk, keep_ratio, out);
}

ga_status ga_plan_create(int32_t W, int32_t n_layers, const int64_t* layer_numel, ga_dtype grad_dtype,
                         int64_t chunk, double keep_ratio, ga_plan** out) {
    if (!out) return fail(GA_ERR_INVALID, "out is NULL");
    *out = nullptr;
    ga_plan_info info;
    ga_status st = compute(W, n_layers, layer_numel, grad_dtype, chunk, keep_ratio, &info);
    if (st != GA_OK) return st;
    ga::Plan* p = new (std::nothrow) ga::Plan();
    if (!p) return fail(GA_ERR_DEVICE, "out of host memory");
    p->W = W;
    p->L = n_layers;
    p->dtype = (int32_t)grad_dtype;
    p->k = info.k;
    p->mw = info.mask_words;
    p->P = info.P;
    p->ld = info.ld;
    p->C = info.chunk;
    p->n_c = info.n_chunks;
    p->d_offsets = nullptr;
    p->h_offsets = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_layers + 1));
    if (!p->h_offsets) {
        delete p;
        return fail(GA_ERR_DEVICE, "out of host memory");
    }
    p->h_offsets[0] = 0;
    for (int32_t l = 0; l < n_layers; ++l) p->h_offsets[l + 1] = p->h_offsets[l] + layer_numel[l];
    // wavefront-tile -> layer table for the kernels that read the layer tensors
    const int64_t vec = grad_dtype == GA_FP16 ? 8 : 4;
    p->tile_elems = 64 * vec;
    const int64_t n_tiles = (info.P + p->tile_elems - 1) / p->tile_elems;
    p->n_tiles = n_tiles;
    uint32_t* h_tiles = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(2 * n_tiles));
    if (!h_tiles) {
        free(p->h_offsets);
        delete p;
        return fail(GA_ERR_DEVICE, "out of host memory");
    }
    {
        int32_t l = 0;
        for (int64_t t = 0; t < n_tiles; ++t) {
            const int64_t e0 = t * p->tile_elems;
            while (p->h_offsets[l + 1] <= e0) ++l;
            const bool whole = p->h_offsets[l + 1] >= e0 + p->tile_elems && p->h_offsets[l] % vec == 0;
            h_tiles[t] = (uint32_t)l | (whole ? 0x80000000u : 0u);
        }
        uint32_t* order = h_tiles + n_tiles;
        int64_t j = 0;
        for (int64_t t = 0; t < n_tiles; ++t)
            if (!(h_tiles[t] >> 31)) order[j++] = (uint32_t)t;
        for (int64_t t = 0; t < n_tiles; ++t)
            if (h_tiles[t] >> 31) order[j++] = (uint32_t)t;
    }
    p->d_tile_layer = nullptr;
    p->d_tile_order = nullptr;
    p->key_parts = p->C > ga::kNormPart ? (int32_t)((p->C + ga::kNormPart - 1) / ga::kNormPart) : 1;
    p->d_part_keys = nullptr;
    hipError_t e = hipGetDevice(&p->device);
    if (e == hipSuccess) e = hipMalloc((void**)&p->d_offsets, sizeof(int64_t) * (size_t)(n_layers + 1));
    if (e == hipSuccess)
        e = hipMemcpy(p->d_offsets, p->h_offsets, sizeof(int64_t) * (size_t)(n_layers + 1), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMalloc((void**)&p->d_tile_layer, sizeof(uint32_t) * (size_t)(2 * n_tiles));
    if (e == hipSuccess)
        e = hipMemcpy(p->d_tile_layer, h_tiles, sizeof(uint32_t) * (size_t)(2 * n_tiles), hipMemcpyHostToDevice);
    if (e == hipSuccess) p->d_tile_order = p->d_tile_layer + n_tiles;
    if (e == hipSuccess && p->key_parts > 1)
        e = hipMalloc((void**)&p->d_part_keys,
                      sizeof(double) * (size_t)W * (size_t)p->n_c * (size_t)p->key_parts);
    free(h_tiles);
    if (e != hipSuccess) {
        if (p->d_offsets) (void)hipFree(p->d_offsets);
        if (p->d_tile_layer) (void)hipFree(p->d_tile_layer);
        if (p->d_part_keys) (void)hipFree(p->d_part_keys);
        free(p->h_offsets);
        delete p;
        return device_status(e, "plan device table");
    }
    // the fixed array of ga_chunk_norm_topk_static: its address on this
    // device, looked up once per device (a failure shows as GA_ERR_DEVICE from
    // that call only)
    (void)ga::static_keys_setup(p->device);
    *out = reinterpret_cast<ga_plan*>(p);
    return ok();
}

void ga_plan_destroy(ga_plan* plan) {
    if (!plan) return;
    ga::Plan* p = reinterpret_cast<ga::Plan*>(plan);
    if (p->d_offsets) (void)hipFree(p->d_offsets);
    if (p->d_tile_layer) (void)hipFree(p->d_tile_layer);
    if (p->d_part_keys) (void)hipFree(p->d_part_keys);
    free(p->h_offsets);
    delete p;
}

ga_status ga_plan_get_info(const ga_plan* plan, ga_plan_info* out) {
    if (!plan || !out) return fail(GA_ERR_INVALID, "NULL argument");
    *out = info_of(as_plan(plan));
    return ok();
}

ga_status ga_bucket_pack(const ga_plan* plan, const uint64_t* d_layer_ptrs, void* d_bucket, hipStream_t stream) {
    if (!plan || !d_layer_ptrs || !d_bucket) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    if (!aligned16(d_bucket)) return fail(GA_ERR_ALIGN, "bucket not 16-byte aligned");
    if (((uintptr_t)d_layer_ptrs & 7u) != 0) return fail(GA_ERR_ALIGN, "layer pointer table not 8-byte aligned");
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_pack(*p, d_layer_ptrs, d_bucket, stream), "bucket_pack launch");
}

ga_status ga_tree_reduce(const ga_plan* plan, const void* d_bucket, float* d_grad, const ga_sgd* sgd, float* d_w,
                         float* d_v, hipStream_t stream) {
    if (!plan || !d_bucket) return fail(GA_ERR_INVALID, "NULL argument");
    if (!d_grad && !sgd) return fail(GA_ERR_INVALID, "neither a gradient output nor an SGD update requested");
    if (sgd && (!d_w || !d_v)) return fail(GA_ERR_INVALID, "SGD update needs w and v");
    if (!aligned16(d_bucket) || (d_grad && !aligned16(d_grad)) || (sgd && (!aligned16(d_w) || !aligned16(d_v))))
        return fail(GA_ERR_ALIGN, "device buffers must be 16-byte aligned");
    const ga::Plan* p = as_plan(plan);
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_tree(*p, d_bucket, d_grad, sgd, d_w, d_v, stream), "tree_reduce launch");
}

ga_status ga_tree_reduce_layers(const ga_plan* plan, const uint64_t* d_layer_ptrs, float* d_grad, const ga_sgd* sgd,
                                float* d_w, float* d_v, hipStream_t stream) {
    if (!plan || !d_layer_ptrs) return fail(GA_ERR_INVALID, "NULL argument");
    if (!d_grad && !sgd) return fail(GA_ERR_INVALID, "neither a gradient output nor an SGD update requested");
    if (sgd && (!d_w || !d_v)) return fail(GA_ERR_INVALID, "SGD update needs w and v");
    if (((uintptr_t)d_layer_ptrs & 7u) || (d_grad && !aligned16(d_grad)) ||
        (sgd && (!aligned16(d_w) || !aligned16(d_v))))
        return fail(GA_ERR_ALIGN, "misaligned device buffer");
    const ga::Plan* p = as_plan(plan);
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_tree_layers(*p, d_layer_ptrs, d_grad, sgd, d_w, d_v, stream),
                         "tree_reduce_layers launch");
}

ga_status ga_chunk_norm_layers(const ga_plan* plan, const uint64_t* d_layer_ptrs, float* d_residual,
                               const uint32_t* d_prev_mask, double* d_keys, hipStream_t stream) {
    if (!plan || !d_layer_ptrs || !d_residual || !d_keys) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    if (p->C == 0) return fail(GA_ERR_INVALID, "plan has no chunk size (dense-only plan)");
    if (((uintptr_t)d_layer_ptrs & 7u) || !aligned16(d_residual) || ((uintptr_t)d_keys & 7u) ||
        (d_prev_mask && ((uintptr_t)d_prev_mask & 3u)))
        return fail(GA_ERR_ALIGN, "misaligned device buffer");
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    // the lazy-zero norm pass is the deferred one at age 0, storing
    ga::HistArgs h;
    memset(&h, 0, sizeof h);
    h.layers[0] = d_layer_ptrs;
    h.masks[0] = d_prev_mask;
    return device_status(ga::launch_norm_hist(*p, h, true, d_residual, d_keys, stream), "chunk_norm_layers launch");
}

namespace {

// Validate a deferred step's history and turn it into kernel arguments.
ga_status history_args(const ga::Plan* p, const uint64_t* d_layer_ptrs, const ga_history* hist,
                       const uint32_t* d_sel_mask, ga::HistArgs* out) {
    if (!hist) return fail(GA_ERR_INVALID, "history is NULL");
    if (p->C == 0) return fail(GA_ERR_INVALID, "plan has no chunk size (dense-only plan)");
    if (hist->age < 0 || hist->age > GA_MAX_AGE)
        return fail(GA_ERR_INVALID, "age %d outside [0, %d]", hist->age, GA_MAX_AGE);
    memset(out, 0, sizeof *out);
    out->age = hist->age;
    out->layers[0] = d_layer_ptrs;
    if ((uintptr_t)d_layer_ptrs & 7u) return fail(GA_ERR_ALIGN, "misaligned layer table");
    for (int32_t j = 0; j < hist->age; ++j) {
        const uint64_t* t = hist->d_layer_ptrs[j];
        if (!t) return fail(GA_ERR_INVALID, "age %d needs the layer table of step t-%d", hist->age, j + 1);
        if ((uintptr_t)t & 7u) return fail(GA_ERR_ALIGN, "misaligned layer table of step t-%d", j + 1);
        if (t == d_layer_ptrs)
            return fail(GA_ERR_INVALID, "the layer table of step t-%d is this step's: every step's gradients "
                                        "must stay in their own tensors until they leave the history", j + 1);
        for (int32_t q = 0; q < j; ++q)
            if (t == hist->d_layer_ptrs[q])
                return fail(GA_ERR_INVALID, "steps t-%d and t-%d share a layer table", q + 1, j + 1);
        out->layers[j + 1] = t;
    }
    for (int32_t j = 0; j <= hist->age; ++j) {
        const uint32_t* m = hist->d_masks[j];
        if (m && ((uintptr_t)m & 3u)) return fail(GA_ERR_ALIGN, "misaligned mask of step t-%d", j + 1);
        if (m && d_sel_mask && m == d_sel_mask)
            return fail(GA_ERR_INVALID, "the mask of step t-%d is this step's selection buffer", j + 1);
        out->masks[j] = m;
    }
    return GA_OK;
}

}  // namespace

ga_status ga_chunk_norm_deferred(const ga_plan* plan, const uint64_t* d_layer_ptrs, const ga_history* hist,
                                 int32_t store, float* d_residual, double* d_keys, hipStream_t stream) {
    if (!plan || !d_layer_ptrs || !d_residual || !d_keys) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    ga::HistArgs h;
    ga_status st = history_args(p, d_layer_ptrs, hist, nullptr, &h);
    if (st != GA_OK) return st;
    if (!aligned16(d_residual) || ((uintptr_t)d_keys & 7u)) return fail(GA_ERR_ALIGN, "misaligned device buffer");
    st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_norm_hist(*p, h, store != 0, d_residual, d_keys, stream),
                         "chunk_norm_deferred launch");
}

ga_status ga_sparse_gather_reduce_deferred(const ga_plan* plan, const uint64_t* d_layer_ptrs,
                                           const ga_history* hist, int32_t stored, const float* d_residual,
                                           const uint32_t* d_sel_mask, float* d_grad, const ga_sgd* sgd,
                                           float* d_w, float* d_v, hipStream_t stream) {
    if (!plan || !d_layer_ptrs || !d_residual || !d_sel_mask) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    ga::HistArgs h;
    ga_status st = history_args(p, d_layer_ptrs, hist, d_sel_mask, &h);
    if (st != GA_OK) return st;
    if (p->C % 256 != 0) return fail(GA_ERR_UNSUPPORTED, "chunk=%lld is not a multiple of 256", (long long)p->C);
    if (!d_grad && !sgd) return fail(GA_ERR_INVALID, "neither a gradient output nor an SGD update requested");
    if (sgd && (!d_w || !d_v)) return fail(GA_ERR_INVALID, "SGD update needs w and v");
    if (!aligned16(d_residual) || ((uintptr_t)d_sel_mask & 3u) || (d_grad && !aligned16(d_grad)) ||
        (sgd && (!aligned16(d_w) || !aligned16(d_v))))
        return fail(GA_ERR_ALIGN, "misaligned device buffer");
    st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_gather_hist(*p, h, stored != 0, d_residual, d_sel_mask, d_grad, sgd, d_w, d_v,
                                                stream),
                         "sparse_gather_reduce_deferred launch");
}

ga_status ga_residual_flush(const ga_plan* plan, const uint64_t* d_layer_ptrs, const ga_history* hist,
                            int32_t stored, float* d_residual, const uint32_t* d_sel_mask, hipStream_t stream) {
    if (!plan || !d_layer_ptrs || !d_residual || !d_sel_mask) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    ga::HistArgs h;
    ga_status st = history_args(p, d_layer_ptrs, hist, d_sel_mask, &h);
    if (st != GA_OK) return st;
    if (!aligned16(d_residual) || ((uintptr_t)d_sel_mask & 3u)) return fail(GA_ERR_ALIGN, "misaligned device buffer");
    st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_flush_hist(*p, h, stored != 0, d_residual, d_sel_mask, stream),
                         "residual_flush launch");
}

ga_status ga_reduce_variant(const ga_plan* plan, const void* d_bucket, ga_order order, int32_t wire_fp16, float* d_grad,
                            const ga_sgd* sgd, float* d_w, float* d_v, hipStream_t stream) {
    if (!plan || !d_bucket) return fail(GA_ERR_INVALID, "NULL argument");
    if (order != GA_ORDER_TREE && order != GA_ORDER_SERVER && order != GA_ORDER_RING)
        return fail(GA_ERR_INVALID, "unknown order %d", (int)order);
    if (!d_grad && !sgd) return fail(GA_ERR_INVALID, "neither a gradient output nor an SGD update requested");
    if (sgd && (!d_w || !d_v)) return fail(GA_ERR_INVALID, "SGD update needs w and v");
    if (!aligned16(d_bucket) || (d_grad && !aligned16(d_grad)) || (sgd && (!aligned16(d_w) || !aligned16(d_v))))
        return fail(GA_ERR_ALIGN, "device buffers must be 16-byte aligned");
    const ga::Plan* p = as_plan(plan);
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_variant(*p, d_bucket, (int)order, wire_fp16 != 0, d_grad, sgd, d_w, d_v, stream),
                         "reduce_variant launch");
}

ga_status ga_chunk_norm(const ga_plan* plan, const void* d_bucket, float* d_residual, const uint32_t* d_prev_mask,
                        double* d_keys, hipStream_t stream) {
    if (!plan || !d_bucket || !d_residual || !d_keys) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    if (p->C == 0) return fail(GA_ERR_INVALID, "plan has no chunk size (dense-only plan)");
    if (!aligned16(d_bucket) || !aligned16(d_residual) || ((uintptr_t)d_keys & 7u) ||
        (d_prev_mask && ((uintptr_t)d_prev_mask & 3u)))
        return fail(GA_ERR_ALIGN, "misaligned device buffer");
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(
        ga::launch_chunk_norm(*p, d_bucket, d_residual, d_prev_mask, d_keys, p->d_part_keys, stream),
        "chunk_norm launch");
}

ga_status ga_chunk_topk(const ga_plan* plan, const double* d_keys, int32_t* d_sel_idx, uint32_t* d_sel_mask,
                        hipStream_t stream) {
    if (!plan || !d_keys || !d_sel_mask) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    if (p->C == 0) return fail(GA_ERR_INVALID, "plan has no chunk size (dense-only plan)");
    if (p->k > 0 && !d_sel_idx) return fail(GA_ERR_INVALID, "sel_idx is NULL with k > 0");
    if (((uintptr_t)d_keys & 7u) || ((uintptr_t)d_sel_mask & 3u) || (d_sel_idx && ((uintptr_t)d_sel_idx & 3u)))
        return fail(GA_ERR_ALIGN, "misaligned device buffer");
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_topk(*p, d_keys, d_sel_idx, d_sel_mask, stream), "chunk_topk launch");
}

ga_status ga_chunk_norm_topk(const ga_plan* plan, const void* d_bucket, float* d_residual,
                             const uint32_t* d_prev_mask, double* d_keys, int32_t* d_sel_idx, uint32_t* d_sel_mask,
                             hipStream_t stream) {
    if (!plan || !d_sel_mask || (as_plan(plan)->k > 0 && !d_sel_idx))
        return fail(GA_ERR_INVALID, "NULL argument");
    ga_status st = ga_chunk_norm(plan, d_bucket, d_residual, d_prev_mask, d_keys, stream);
    if (st != GA_OK) return st;
    return ga_chunk_topk(plan, d_keys, d_sel_idx, d_sel_mask, stream);
}

ga_status ga_chunk_norm_topk_static(const ga_plan* plan, const void* d_bucket, float* d_residual,
                                    const uint32_t* d_prev_mask, int32_t* d_sel_idx, uint32_t* d_sel_mask,
                                    hipStream_t stream) {
    if (!plan || !d_bucket || !d_residual || !d_sel_mask) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    if (p->C == 0) return fail(GA_ERR_INVALID, "plan has no chunk size (dense-only plan)");
    if (p->k > 0 && !d_sel_idx) return fail(GA_ERR_INVALID, "sel_idx is NULL with k > 0");
    // the keys, then (chunks longer than 2048 elements) the parts' partial sums
    const int64_t n_keys = (int64_t)p->W * p->n_c;
    const int64_t need = n_keys * (p->key_parts > 1 ? 1 + (int64_t)p->key_parts : 1);
    if (need > GA_STATIC_KEYS)
        return fail(GA_ERR_UNSUPPORTED, "%lld binary64 values (W * n_c = %lld keys, %d parts) exceed the %lld of "
                    "the fixed array", (long long)need, (long long)n_keys, (int)p->key_parts,
                    (long long)GA_STATIC_KEYS);
    if (!aligned16(d_bucket) || !aligned16(d_residual) || (d_prev_mask && ((uintptr_t)d_prev_mask & 3u)) ||
        ((uintptr_t)d_sel_mask & 3u) || (d_sel_idx && ((uintptr_t)d_sel_idx & 3u)))
        return fail(GA_ERR_ALIGN, "misaligned device buffer");
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    double* keys = ga::static_keys(p->device);
    if (!keys) return fail(GA_ERR_DEVICE, "the fixed array has no address on device %d", p->device);
    double* part_keys = p->key_parts > 1 ? keys + n_keys : nullptr;
    st = device_status(ga::launch_chunk_norm(*p, d_bucket, d_residual, d_prev_mask, keys, part_keys, stream),
                       "chunk_norm_topk_static launch");
    if (st != GA_OK) return st;
    return device_status(ga::launch_topk(*p, keys, d_sel_idx, d_sel_mask, stream), "chunk_norm_topk_static launch");
}

ga_status ga_sparse_gather_reduce(const ga_plan* plan, float* d_residual, const uint32_t* d_sel_mask,
                                  int32_t zero_selected, float* d_grad, const ga_sgd* sgd, float* d_w, float* d_v,
                                  hipStream_t stream) {
    if (!plan || !d_residual || !d_sel_mask) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    if (p->C == 0) return fail(GA_ERR_INVALID, "plan has no chunk size (dense-only plan)");
    if (!d_grad && !sgd && !zero_selected) return fail(GA_ERR_INVALID, "nothing to do");
    if (sgd && (!d_w || !d_v)) return fail(GA_ERR_INVALID, "SGD update needs w and v");
    if (!aligned16(d_residual) || ((uintptr_t)d_sel_mask & 3u) || (d_grad && !aligned16(d_grad)) ||
        (sgd && (!aligned16(d_w) || !aligned16(d_v))))
        return fail(GA_ERR_ALIGN, "misaligned device buffer");
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(
        ga::launch_sparse_gather(*p, d_residual, d_sel_mask, zero_selected, d_grad, sgd, d_w, d_v, stream),
        "sparse_gather_reduce launch");
}

ga_status ga_tree_partial(const ga_plan* plan, const void* d_bucket, float* d_sum, hipStream_t stream) {
    if (!plan || !d_bucket || !d_sum) return fail(GA_ERR_INVALID, "NULL argument");
    if (!aligned16(d_bucket) || !aligned16(d_sum)) return fail(GA_ERR_ALIGN, "device buffers must be 16-byte aligned");
    const ga::Plan* p = as_plan(plan);
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    // S * 1.0f is S, bit for bit
    return device_status(ga::launch_tree_scaled(*p, d_bucket, 1.0f, d_sum, nullptr, nullptr, nullptr, stream),
                         "tree_partial launch");
}

ga_status ga_tree_combine(const ga_plan* plan, const float* d_partials, int32_t w_total, float* d_grad,
                          const ga_sgd* sgd, float* d_w, float* d_v, hipStream_t stream) {
    if (!plan || !d_partials) return fail(GA_ERR_INVALID, "NULL argument");
    const ga::Plan* p = as_plan(plan);
    if (p->dtype != GA_FP32) return fail(GA_ERR_INVALID, "partial sums are binary32: the plan must be GA_FP32");
    if (w_total < 1) return fail(GA_ERR_INVALID, "w_total=%d < 1", w_total);
    if (!d_grad && !sgd) return fail(GA_ERR_INVALID, "neither a gradient output nor an SGD update requested");
    if (sgd && (!d_w || !d_v)) return fail(GA_ERR_INVALID, "SGD update needs w and v");
    if (!aligned16(d_partials) || (d_grad && !aligned16(d_grad)) || (sgd && (!aligned16(d_w) || !aligned16(d_v))))
        return fail(GA_ERR_ALIGN, "device buffers must be 16-byte aligned");
    ga_status st = check_device(p);
    if (st != GA_OK) return st;
    return device_status(ga::launch_tree_scaled(*p, d_partials, (float)(1.0 / (double)w_total), d_grad, sgd, d_w,
                                                d_v, stream),
                         "tree_combine launch");
}

ga_status ga_sgd_momentum_apply(int64_t P, const float* d_grad, float* d_w, float* d_v, const ga_sgd* sgd,
                                hipStream_t stream) {
    if (P < 0 || !sgd) return fail(GA_ERR_INVALID, "bad size or NULL sgd");
    if (P > GA_MAX_ELEMENTS)
        return fail(GA_ERR_UNSUPPORTED, "P=%lld exceeds %lld elements", (long long)P, (long long)GA_MAX_ELEMENTS);
    if (P == 0) return ok();
    if (!d_grad || !d_w || !d_v) return fail(GA_ERR_INVALID, "NULL argument");
    if (!aligned16(d_grad) || !aligned16(d_w) || !aligned16(d_v))
        return fail(GA_ERR_ALIGN, "device buffers must be 16-byte aligned");
    return device_status(ga::launch_sgd(P, d_grad, d_w, d_v, sgd, stream), "sgd launch");
}

}  // extern "C"
