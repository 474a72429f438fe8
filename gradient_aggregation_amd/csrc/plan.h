// Internal host-side declarations shared by the HIP sources of libgradagg.so:
// the plan, the kernel launchers and ABI error reporting.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gradagg.h"

namespace ga {

// The storing layer-table chunk-norm pass splits a chunk longer than this
// many elements into parts of this size, one workgroup each, so that the
// resident workgroups stream one contiguous window of the residual instead of
// one sweep per chunk (measured faster for its mixed read/write traffic, and
// slower for read-only passes, which keep one workgroup per chunk); the
// parts' binary64 sums are added per chunk afterwards.
constexpr int64_t kNormPart = 2048;

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
    // Parts per chunk of the storing layer-table chunk-norm pass
    // (ceil(C / kNormPart), 1 for C <= kNormPart), and the plan's workspace of
    // their partial sums, [W][n_c][key_parts] binary64 (nullptr when
    // key_parts == 1).
    int32_t key_parts;
    double* d_part_keys;
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
// part_keys: [W][n_c][key_parts] binary64 partial sums when key_parts > 1
// (the plan's workspace, or the fixed array of the allocation-free call).
hipError_t launch_chunk_norm(const Plan& p, const void* bucket, float* resid,
                             const uint32_t* prev_mask, double* keys, double* part_keys, hipStream_t s);
// After a part-split storing norm pass: keys[w][c] = the chunk's key_parts
// partial sums in part_keys, added in part order.
hipError_t launch_key_parts(const Plan& p, const double* part_keys, double* keys, hipStream_t s);
// The deferred-residual form (history.hip).  layers[0] is this step's layer
// table and layers[j] that of step t-j (j <= age); masks[j] the selection of
// step t-1-j (j <= age), or nullptr.
struct HistArgs {
    const uint64_t* layers[GA_MAX_AGE + 1];
    const uint32_t* masks[GA_MAX_AGE + 1];
    int32_t age;
};
// Norm pass: keys of a_t; with store, a_t written into resid.
hipError_t launch_norm_hist(const Plan& p, const HistArgs& h, bool store, float* resid, double* keys,
                            hipStream_t s);
// Gather-reduce of the chunks set in sel (stored: this step's norm pass stored).
hipError_t launch_gather_hist(const Plan& p, const HistArgs& h, bool stored, const float* resid,
                              const uint32_t* sel, float* grad, const ga_sgd* sgd, float* w, float* v,
                              hipStream_t s);
// The residual after the step: +0 on the chunks set in sel, a_t elsewhere.
hipError_t launch_flush_hist(const Plan& p, const HistArgs& h, bool stored, float* resid, const uint32_t* sel,
                             hipStream_t s);
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
