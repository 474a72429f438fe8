// Multi-bucket lazy allreduce: the layer list is cut into buckets in the order
// a backward pass produces the gradients (last layer first), each bucket
// holding at least a byte threshold per worker, so that a bucket can be
// aggregated as soon as its layers are written while later layers are still
// being produced (GradientFlow, arXiv abstract: lazy allreduce fuses many
// operations; computation and communication overlap).  Each bucket is a plan
// over its sub-list of layers; its reduction waits on the caller's "layers
// ready" event on the caller's stream.
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "plan.h"

struct ga_buckets {
    int32_t W, L, dtype;
    std::vector<ga_plan*> plans;     // one per bucket
    std::vector<int32_t> first;      // first layer of each bucket (forward order)
    std::vector<int32_t> count;      // layers in each bucket
    std::vector<int64_t> begin, end; // element range of each bucket in the fused row
};

extern "C" {

ga_status ga_bucket_boundaries(int32_t n_layers, const int64_t* layer_numel, int32_t elem_bytes, int64_t bucket_bytes,
                               int32_t* first_layer, int32_t* n_buckets) {
    if (n_layers < 1 || !layer_numel || !first_layer || !n_buckets)
        return ga::api_fail(GA_ERR_INVALID, "NULL argument or n_layers < 1");
    if (bucket_bytes < 1) return ga::api_fail(GA_ERR_INVALID, "bucket_bytes < 1");
    if (elem_bytes != 2 && elem_bytes != 4) return ga::api_fail(GA_ERR_INVALID, "elem_bytes must be 2 or 4");
    std::vector<int64_t> off((size_t)n_layers + 1, 0);
    for (int32_t l = 0; l < n_layers; ++l) {
        if (layer_numel[l] < 1) return ga::api_fail(GA_ERR_INVALID, "a layer has no elements");
        off[l + 1] = off[l] + layer_numel[l];
    }
    // Walk backwards from the last layer; close a bucket at the start of layer
    // l once it holds >= bucket_bytes and that start is a multiple of 8
    // elements (so a bucket's slice of w, v and g stays 16-byte aligned).
    int32_t nb = 0;
    int64_t acc = 0;
    std::vector<int32_t> starts;
    for (int32_t l = n_layers - 1; l >= 0; --l) {
        acc += layer_numel[l] * elem_bytes;
        if (l == 0 || (acc >= bucket_bytes && off[l] % 8 == 0)) {
            starts.push_back(l);
            acc = 0;
        }
    }
    nb = (int32_t)starts.size();
    for (int32_t b = 0; b < nb; ++b) first_layer[b] = starts[b];  // bucket b in production order
    *n_buckets = nb;
    return ga::api_ok();
}

ga_status ga_buckets_create(const ga_plan* plan, int64_t bucket_bytes, ga_buckets** out) {
    if (!plan || !out) return ga::api_fail(GA_ERR_INVALID, "NULL argument");
    *out = nullptr;
    const ga::Plan* p = reinterpret_cast<const ga::Plan*>(plan);
    const int32_t esz = p->dtype == GA_FP16 ? 2 : 4;
    std::vector<int64_t> numel((size_t)p->L);
    for (int32_t l = 0; l < p->L; ++l) numel[l] = p->h_offsets[l + 1] - p->h_offsets[l];
    std::vector<int32_t> firsts((size_t)p->L);
    int32_t nb = 0;
    ga_status st = ga_bucket_boundaries(p->L, numel.data(), esz, bucket_bytes, firsts.data(), &nb);
    if (st != GA_OK) return st;
    ga_buckets* bk = new (std::nothrow) ga_buckets();
    if (!bk) return ga::api_fail(GA_ERR_DEVICE, "out of host memory");
    bk->W = p->W;
    bk->L = p->L;
    bk->dtype = p->dtype;
    int32_t stop = p->L;  // buckets come last-layer first
    for (int32_t b = 0; b < nb; ++b) {
        const int32_t f = firsts[b], n = stop - f;
        ga_plan* sub = nullptr;
        st = ga_plan_create(p->W, n, numel.data() + f, (ga_dtype)p->dtype, 0, 0.0, &sub);
        if (st != GA_OK) {
            for (ga_plan* q : bk->plans) ga_plan_destroy(q);
            delete bk;
            return st;
        }
        bk->plans.push_back(sub);
        bk->first.push_back(f);
        bk->count.push_back(n);
        bk->begin.push_back(p->h_offsets[f]);
        bk->end.push_back(p->h_offsets[stop]);
        stop = f;
    }
    *out = bk;
    return ga::api_ok();
}

void ga_buckets_destroy(ga_buckets* bk) {
    if (!bk) return;
    for (ga_plan* q : bk->plans) ga_plan_destroy(q);
    delete bk;
}

int32_t ga_buckets_count(const ga_buckets* bk) { return bk ? (int32_t)bk->plans.size() : 0; }

ga_status ga_bucket_range(const ga_buckets* bk, int32_t b, int32_t* first_layer, int32_t* n_layers,
                          int64_t* elem_begin, int64_t* elem_end) {
    if (!bk || b < 0 || b >= (int32_t)bk->plans.size()) return ga::api_fail(GA_ERR_INVALID, "bucket out of range");
    if (first_layer) *first_layer = bk->first[b];
    if (n_layers) *n_layers = bk->count[b];
    if (elem_begin) *elem_begin = bk->begin[b];
    if (elem_end) *elem_end = bk->end[b];
    return ga::api_ok();
}

ga_status ga_bucket_reduce_layers(const ga_buckets* bk, int32_t b, const uint64_t* d_layer_ptrs, hipEvent_t ready,
                                  float* d_grad, const ga_sgd* sgd, float* d_w, float* d_v, int32_t max_workgroups,
                                  hipStream_t stream) {
    if (!bk || !d_layer_ptrs) return ga::api_fail(GA_ERR_INVALID, "NULL argument");
    if (b < 0 || b >= (int32_t)bk->plans.size()) return ga::api_fail(GA_ERR_INVALID, "bucket out of range");
    if (!d_grad && !sgd)
        return ga::api_fail(GA_ERR_INVALID, "neither a gradient output nor an SGD update requested");
    if (sgd && (!d_w || !d_v)) return ga::api_fail(GA_ERR_INVALID, "SGD update needs w and v");
    if (((uintptr_t)d_layer_ptrs & 7u) || ((uintptr_t)d_grad & 15u) || ((uintptr_t)d_w & 15u) ||
        ((uintptr_t)d_v & 15u))
        return ga::api_fail(GA_ERR_ALIGN, "misaligned device buffer");
    if (max_workgroups < 0) return ga::api_fail(GA_ERR_INVALID, "max_workgroups < 0");
    const ga::Plan* sub = reinterpret_cast<const ga::Plan*>(bk->plans[b]);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != sub->device)
        return ga::api_fail(GA_ERR_INVALID, "current device is not the schedule's device");
    if (ready && hipStreamWaitEvent(stream, ready, 0) != hipSuccess)
        return ga::api_fail(GA_ERR_DEVICE, "hipStreamWaitEvent failed");
    const int64_t e0 = bk->begin[b];
    hipError_t e = ga::launch_tree_layers_sub(*sub, d_layer_ptrs, bk->L, bk->first[b], d_grad ? d_grad + e0 : nullptr,
                                              sgd, d_w ? d_w + e0 : nullptr, d_v ? d_v + e0 : nullptr,
                                              max_workgroups, stream);
    return e == hipSuccess ? ga::api_ok() : ga::api_fail(GA_ERR_DEVICE, hipGetErrorString(e));
}

}  // extern "C"
