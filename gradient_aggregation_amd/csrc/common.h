// Internal declarations shared by the HIP sources of libgradagg.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gradagg.h"

namespace ga {

// 128-bit vector of binary32 and its binary16 counterpart.
struct alignas(16) f4 { float x, y, z, w; };

struct Plan {
    int32_t W, L, dtype, k, mw;
    int64_t P, ld, C, n_c;
    int device;
    int64_t* d_offsets;  // [L+1] layer start offsets in the fused row
    int64_t* h_offsets;  // host copy
    // Layer of each wavefront tile of the fused row (64 lanes x one 128-bit
    // vector: 512 binary16 or 256 binary32 elements): bits 0..30 the layer of
    // the tile's first element, bit 31 set when the whole tile lies in that
    // layer at a vector-aligned offset.
    uint32_t* d_tile_layer;
    int64_t tile_elems;
};

// ---- ABI error reporting (defined in abi.hip) ---------------------------
ga_status api_fail(ga_status s, const char* msg);
ga_status api_ok();

// ---- launchers (each returns hipSuccess or the launch error) -------------
hipError_t launch_tree(const Plan& p, const void* bucket, float* grad, const ga_sgd* sgd,
                       float* w, float* v, hipStream_t s);
hipError_t launch_chunk_norm(const Plan& p, const void* bucket, float* resid,
                             const uint32_t* prev_mask, double* keys, hipStream_t s);
hipError_t launch_chunk_norm_layers(const Plan& p, const uint64_t* layer_ptrs, float* resid,
                                    const uint32_t* prev_mask, double* keys, hipStream_t s);
hipError_t launch_tree_layers(const Plan& p, const uint64_t* layer_ptrs, float* grad, const ga_sgd* sgd,
                              float* w, float* v, hipStream_t s);
// launch_tree_layers over a sub-list of layers: worker w's layer l is entry
// w*tbl_stride + tbl_first + l of the layer table; max_blocks > 0 caps the
// grid (the workgroups then stride over the blocks of elements).
hipError_t launch_tree_layers_sub(const Plan& p, const uint64_t* layer_ptrs, int32_t tbl_stride, int32_t tbl_first,
                                  float* grad, const ga_sgd* sgd, float* w, float* v, int32_t max_blocks,
                                  hipStream_t s);
hipError_t launch_variant(const Plan& p, const void* bucket, int order, int wire16, float* grad, const ga_sgd* sgd,
                          float* w, float* v, hipStream_t s);
hipError_t launch_topk(const Plan& p, const double* keys, int32_t* sel_idx, uint32_t* sel_mask,
                       hipStream_t s);
hipError_t launch_sparse_gather(const Plan& p, float* resid, const uint32_t* sel_mask,
                                int zero_selected, float* grad, const ga_sgd* sgd, float* w,
                                float* v, hipStream_t s);
hipError_t launch_sgd(int64_t P, const float* g, float* w, float* v, const ga_sgd* sgd,
                      hipStream_t s);
hipError_t launch_pack(const Plan& p, const uint64_t* layer_ptrs, void* bucket, hipStream_t s);

// ---- device helpers ------------------------------------------------------

// Momentum SGD, Caffe form, three binary32 roundings (the library is built
// with -ffp-contract=off, so no multiply-add is fused).
__device__ __forceinline__ void sgd_update(float g, float lr, float mu, float& w, float& v) {
    float a = mu * v;
    float b = lr * g;
    v = a + b;
    w = w - v;
}

// A device address held as an integer (e.g. read from a layer table), typed as
// a global-memory pointer so that loads through it compile to global (not
// flat) instructions.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

template <typename T>
__device__ __forceinline__ gptr<T> as_global(uint64_t addr) {
    return reinterpret_cast<gptr<T>>(addr);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 128-bit loads through a global-memory pointer (16-byte aligned).
__device__ __forceinline__ uint4 load_u4(gptr<void> p) {
    const u32x4 x = *reinterpret_cast<gptr<u32x4>>(p);
    return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ float4 load_f4(gptr<void> p) {
    const f32x4 x = *reinterpret_cast<gptr<f32x4>>(p);
    return make_float4(x.x, x.y, x.z, x.w);
}

// binary16 -> binary32 widening (exact, subnormals included) of 8 packed values.
__device__ __forceinline__ void widen8(const uint4& r, float (&f)[8]) {
    const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[j] & 0xffffu));
        f[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[j] >> 16));
    }
}

__device__ __forceinline__ float widen1(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

}  // namespace ga
