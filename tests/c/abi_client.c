/*
 * A plain C client of libgradagg.so: no Python, no torch.  It drives the
 * dense step (fixed-tree reduce with fused momentum SGD) or the sparse step
 * (chunk norms + top-k, then gather-reduce with fused SGD) through the C ABI
 * of include/gradagg.h on device buffers it allocates itself, then the two
 * other calls of the path: the fusion of step 1's gradients, split into one
 * device tensor per (worker, layer) at odd offsets, into a bucket
 * (ga_bucket_pack), and one standalone momentum-SGD update of the final
 * weights and velocity with the final mean gradient (ga_sgd_momentum_apply),
 * so that a test can compare every result with the oracle.
 *
 * usage: abi_client <dir>
 *   <dir>/meta.txt   "W L fp16 chunk keep_ratio lr mu steps" then L layer sizes
 *   <dir>/bucket<s>.bin  step s's [W][ld] gradients (binary32, or binary16 bits)
 *   <dir>/w.bin      [P] binary32 initial weights (velocity starts at zero)
 * writes <dir>/gbar.bin, w_out.bin, v_out.bin (after the last step), pack.bin
 * (the fused bucket of step 1), w_sgd.bin, v_sgd.bin (w_out, v_out after one
 * more update with gbar) and, for a sparse plan, keys.bin, idx.bin,
 * mask.bin, resid.bin of the last step.
 * Exit status 0 on success; a failed call prints ga_last_error() and exits 1.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gradagg.h"

#define GA(call)                                                                      \
    do {                                                                              \
        ga_status st_ = (call);                                                       \
        if (st_ != GA_OK) {                                                           \
            fprintf(stderr, "%s failed: %s (%s)\n", #call, ga_status_str(st_),        \
                    ga_last_error());                                                 \
            exit(1);                                                                  \
        }                                                                             \
    } while (0)

#define HIP(call)                                                                     \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            exit(1);                                                                  \
        }                                                                             \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(1); }
    void* p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(1); }
    fclose(f);
    return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(1); }
    fclose(f);
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    HIP(hipMalloc(&p, bytes ? bytes : 16));
    HIP(hipMemset(p, 0, bytes ? bytes : 16));
    return p;
}

static void to_host(const char* dir, const char* name, const void* d, size_t bytes) {
    void* h = malloc(bytes ? bytes : 1);
    HIP(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
    write_file(dir, name, h, bytes);
    free(h);
}

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s <dir>\n", argv[0]); return 2; }
    const char* dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE* f = fopen(path, "r");
    if (!f) { fprintf(stderr, "cannot open %s\n", path); return 1; }
    int W, L, fp16, steps;
    long long chunk;
    double rho;
    float lr, mu;
    if (fscanf(f, "%d %d %d %lld %lf %f %f %d", &W, &L, &fp16, &chunk, &rho, &lr, &mu, &steps) != 8 || L < 1) {
        fprintf(stderr, "bad meta\n");
        return 1;
    }
    int64_t* numel = (int64_t*)malloc(sizeof(int64_t) * (size_t)L);
    for (int l = 0; l < L; ++l) {
        long long n;
        if (fscanf(f, "%lld", &n) != 1) { fprintf(stderr, "bad meta\n"); return 1; }
        numel[l] = n;
    }
    fclose(f);

    ga_plan* plan = NULL;
    GA(ga_plan_create(W, L, numel, fp16 ? GA_FP16 : GA_FP32, chunk, rho, &plan));
    ga_plan_info in;
    GA(ga_plan_get_info(plan, &in));
    const size_t esz = fp16 ? 2 : 4;
    const size_t bucket_bytes = (size_t)W * (size_t)in.ld * esz;
    const size_t vec_bytes = (size_t)in.P * 4;

    void* d_bucket = dev_alloc(bucket_bytes);
    float* d_grad = (float*)dev_alloc(vec_bytes);
    float* d_w = (float*)dev_alloc(vec_bytes);
    float* d_v = (float*)dev_alloc(vec_bytes);
    void* h_w = read_file(dir, "w.bin", vec_bytes);
    HIP(hipMemcpy(d_w, h_w, vec_bytes, hipMemcpyHostToDevice));
    free(h_w);

    float* d_resid = NULL;
    double* d_keys = NULL;
    int32_t* d_idx = NULL;
    uint32_t* d_mask = NULL;
    if (in.chunk > 0) {
        d_resid = (float*)dev_alloc((size_t)W * (size_t)in.ld * 4);
        d_keys = (double*)dev_alloc((size_t)W * (size_t)in.n_chunks * 8);
        d_idx = (int32_t*)dev_alloc((size_t)W * (size_t)(in.k > 0 ? in.k : 1) * 4);
        d_mask = (uint32_t*)dev_alloc((size_t)W * (size_t)in.mask_words * 4);
    }
    hipStream_t stream;
    HIP(hipStreamCreate(&stream));
    const ga_sgd sgd = {lr, mu};
    for (int s = 1; s <= steps; ++s) {
        char name[64];
        snprintf(name, sizeof name, "bucket%d.bin", s);
        void* h_b = read_file(dir, name, bucket_bytes);
        HIP(hipMemcpy(d_bucket, h_b, bucket_bytes, hipMemcpyHostToDevice));
        free(h_b);
        if (in.chunk == 0) {
            GA(ga_tree_reduce(plan, d_bucket, d_grad, &sgd, d_w, d_v, stream));
        } else {
            GA(ga_chunk_norm_topk(plan, d_bucket, d_resid, NULL, d_keys, d_idx, d_mask, stream));
            GA(ga_sparse_gather_reduce(plan, d_resid, d_mask, 1, d_grad, &sgd, d_w, d_v, stream));
        }
        HIP(hipStreamSynchronize(stream));
    }
    to_host(dir, "gbar.bin", d_grad, vec_bytes);
    to_host(dir, "w_out.bin", d_w, vec_bytes);
    to_host(dir, "v_out.bin", d_v, vec_bytes);

    /* ga_sgd_momentum_apply: one more update of the final state with gbar */
    GA(ga_sgd_momentum_apply(in.P, d_grad, d_w, d_v, &sgd, stream));
    HIP(hipStreamSynchronize(stream));
    to_host(dir, "w_sgd.bin", d_w, vec_bytes);
    to_host(dir, "v_sgd.bin", d_v, vec_bytes);

    /* ga_bucket_pack: step 1's gradients as W*L separate device tensors, each
       starting (w + l) % 3 elements past its allocation, fused into a bucket */
    {
        unsigned char* h_b = (unsigned char*)read_file(dir, "bucket1.bin", bucket_bytes);
        uint64_t* h_tab = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)W * (size_t)L);
        void** allocs = (void**)malloc(sizeof(void*) * (size_t)W * (size_t)L);
        for (int w = 0; w < W; ++w) {
            size_t off = 0;
            for (int l = 0; l < L; ++l) {
                const size_t skew = (size_t)((w + l) % 3) * esz;
                const size_t bytes = (size_t)numel[l] * esz;
                unsigned char* d = (unsigned char*)dev_alloc(bytes + 3 * esz);
                HIP(hipMemcpy(d + skew, h_b + ((size_t)w * (size_t)in.ld + off) * esz, bytes, hipMemcpyHostToDevice));
                allocs[w * L + l] = d;
                h_tab[w * L + l] = (uint64_t)(uintptr_t)(d + skew);
                off += (size_t)numel[l];
            }
        }
        uint64_t* d_tab = (uint64_t*)dev_alloc(sizeof(uint64_t) * (size_t)W * (size_t)L);
        HIP(hipMemcpy(d_tab, h_tab, sizeof(uint64_t) * (size_t)W * (size_t)L, hipMemcpyHostToDevice));
        void* d_packed = dev_alloc(bucket_bytes);
        HIP(hipMemset(d_packed, 0xff, bucket_bytes));   /* the pack writes every byte, padding included */
        GA(ga_bucket_pack(plan, d_tab, d_packed, stream));
        HIP(hipStreamSynchronize(stream));
        to_host(dir, "pack.bin", d_packed, bucket_bytes);
        for (int q = 0; q < W * L; ++q) HIP(hipFree(allocs[q]));
        HIP(hipFree(d_tab));
        HIP(hipFree(d_packed));
        free(allocs);
        free(h_tab);
        free(h_b);
    }
    if (in.chunk > 0) {
        to_host(dir, "keys.bin", d_keys, (size_t)W * (size_t)in.n_chunks * 8);
        to_host(dir, "idx.bin", d_idx, (size_t)W * (size_t)in.k * 4);
        to_host(dir, "mask.bin", d_mask, (size_t)W * (size_t)in.mask_words * 4);
        to_host(dir, "resid.bin", d_resid, (size_t)W * (size_t)in.ld * 4);
        HIP(hipFree(d_resid)); HIP(hipFree(d_keys)); HIP(hipFree(d_idx)); HIP(hipFree(d_mask));
    }
    HIP(hipStreamDestroy(stream));
    HIP(hipFree(d_bucket)); HIP(hipFree(d_grad)); HIP(hipFree(d_w)); HIP(hipFree(d_v));
    ga_plan_destroy(plan);
    free(numel);
    printf("abi_client: %d step(s) W=%d P=%lld %s ok\n", steps, W, (long long)in.P, in.chunk ? "sparse" : "dense");
    return 0;
}
