// Internal host-side declarations shared by the HIP sources of libgradagg.so:
// the plan, the kernel launchers and ABI error reporting.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gradagg.h"

namespace ga {

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
    // The order in which the wavefronts take the tiles: tiles that straddle a
    // layer boundary (or start at an unaligned offset) first, then the rest
    // in ascending order, so that the slow ones do not form the kernel's tail.
    // Same allocation as d_tile_layer (its second half).
    uint32_t* d_tile_order;
    int64_t tile_elems, n_tiles;
};

// ---- ABI error reporting (defined in abi.hip) ---------------------------
ga_status api_fail(ga_status s, const char* msg);
ga_status api_ok();

// ---- launchers (each returns hipSuccess or the launch error) -------------
hipError_t launch_tree(const Plan& p, const void* bucket, float* grad, const ga_sgd* sgd,
                       float* w, float* v, hipStream_t s);
// launch_tree with g = S * scale instead of S * fl32(1/W).
hipError_t launch_tree_scaled(const Plan& p, const void* bucket, float scale, float* grad, const ga_sgd* sgd,
                              float* w, float* v, hipStream_t s);
hipError_t launch_chunk_norm(const Plan& p, const void* bucket, float* resid,
                             const uint32_t* prev_mask, double* keys, hipStream_t s);
hipError_t launch_chunk_norm_layers(const Plan& p, const uint64_t* layer_ptrs, float* resid,
                                    const uint32_t* prev_mask, double* keys, hipStream_t s);
// launch_chunk_norm_layers in deferred mode (prev_mask required): a chunk
// sent in the previous step does not store its a.
hipError_t launch_chunk_norm_layers_defer(const Plan& p, const uint64_t* layer_ptrs, float* resid,
                                          const uint32_t* prev_mask, double* keys, hipStream_t s);
// launch_chunk_norm_layers_defer, and a chunk set in prev2_mask but not in
// prev_mask takes the previous step's gradient (prev_layer_ptrs) + 0 as its
// residual.
hipError_t launch_chunk_norm_layers_pending(const Plan& p, const uint64_t* layer_ptrs,
                                            const uint64_t* prev_layer_ptrs, float* resid,
                                            const uint32_t* prev_mask, const uint32_t* prev2_mask, double* keys,
                                            hipStream_t s);
// Gather-reduce for deferred mode: a chunk sent now and in the previous step
// is read from the gradient tensors; with materialize, one sent before but not
// now gets its residual (the widened gradient) written.  C must be a multiple
// of 256.
hipError_t launch_sparse_gather_defer(const Plan& p, const uint64_t* layer_ptrs, float* resid,
                                      const uint32_t* prev_mask, const uint32_t* sel_mask, float* grad,
                                      const ga_sgd* sgd, float* w, float* v, bool materialize, hipStream_t s);
// The residual of every chunk set in prev_mask but not in sel_mask becomes
// the widened gradient (layer_ptrs) + 0; with prev2_mask (depth 2), that of
// every chunk set in prev2_mask and in neither later mask becomes g0 + (g1 +
// 0), g1 from prev_layer_ptrs.
hipError_t launch_residual_flush(const Plan& p, const uint64_t* layer_ptrs, float* resid, const uint32_t* prev_mask,
                                 const uint32_t* sel_mask, hipStream_t s, const uint64_t* prev_layer_ptrs = nullptr,
                                 const uint32_t* prev2_mask = nullptr);
// Depth-2 pending form of the norm pass: launch_chunk_norm_layers_pending,
// except that a chunk pending one step does not store its a, and a chunk set
// in prev3_mask and in neither later mask takes g1 + (g2 + 0) as its
// residual (prev_layer_ptrs, prev2_layer_ptrs).
hipError_t launch_chunk_norm_layers_pending2(const Plan& p, const uint64_t* layer_ptrs,
                                             const uint64_t* prev_layer_ptrs, const uint64_t* prev2_layer_ptrs,
                                             float* resid, const uint32_t* prev_mask, const uint32_t* prev2_mask,
                                             const uint32_t* prev3_mask, double* keys, hipStream_t s);
// Depth-2 pending gather: as launch_sparse_gather_defer without
// materialization, and a chunk sent now, set in prev2_mask and not in
// prev_mask has the leaf g0 + (g1 + 0), g1 from prev_layer_ptrs.
hipError_t launch_sparse_gather_pending2(const Plan& p, const uint64_t* layer_ptrs, const uint64_t* prev_layer_ptrs,
                                         float* resid, const uint32_t* prev_mask, const uint32_t* sel_mask,
                                         const uint32_t* prev2_mask, float* grad, const ga_sgd* sgd, float* w,
                                         float* v, hipStream_t s);
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

}  // namespace ga
