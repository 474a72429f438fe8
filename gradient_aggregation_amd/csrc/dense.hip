// Dense aggregation: fixed-tree sum over W worker rows, mean, fused momentum SGD.
//
// Sources: FireCaffe (paperlayer summary) sec. 6 - allreduce is an elementwise
// sum of the workers' gradient vectors, taken here in a binary reduction tree;
// GradientFlow (arXiv abstract) - mixed-precision transport, i.e. binary16
// leaves summed in binary32.
//
// Layout and mapping.  The bucket is [W][ld]; a thread owns E consecutive
// elements (E*sizeof(T) = 16 bytes, so every leaf is one 128-bit load: 8
// binary16 or 4 binary32 values) and walks the W rows, so each gradient byte
// is read exactly once and the tree lives in registers.  Workers are loaded
// U at a time before they are merged, so U 128-bit loads per thread are in
// flight.  The mean and the SGD update are applied in the same pass: the
// kernel's HBM traffic is W*P*sizeof(T) + 16*P bytes (w, v read and written).
#include "device.h"
#include "plan.h"
#include "tree.h"

namespace ga {

namespace {

constexpr int kThreads = 256;
// Leaves in flight per thread (U): 16 in general; 4 for binary16 leaves with
// W >= 64, where 16 holds so many registers that only two wavefronts fit on a
// SIMD (4 is 2-4% faster at W = 128, 300 and 512; at W = 16, where a thread
// reads all its leaves in one round, 16 is 7% faster).
constexpr int kUnrollW = 16;
constexpr int kUnrollNarrow = 4;
constexpr int kNarrowMinW = 64;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Gradient leaves are read exactly once: non-temporal loads keep them from
// displacing reusable lines in the caches.
__device__ __forceinline__ uint4 load_leaf(const char* p) {
    const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ uint4 load_leaf_at(uint64_t addr) {
    const v4u x = __builtin_nontemporal_load(as_global<v4u>(addr));
    return make_uint4(x.x, x.y, x.z, x.w);
}

template <bool FP16>
struct LeafVec;

template <>
struct LeafVec<false> {
    static constexpr int E = 4;
    using raw = uint4;
    static __device__ __forceinline__ void widen(const raw& r, float (&f)[E]) {
        f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
};

template <>
struct LeafVec<true> {
    static constexpr int E = 8;
    using raw = uint4;
    static __device__ __forceinline__ void widen(const raw& r, float (&f)[E]) { widen8(r, f); }
};

// The thread's w and v, loaded before its leaves so that their latency
// overlaps the leaves' instead of following the tree (full vectors only; a
// ragged tail loads them in the epilogue).  PF = false (the 11-level trees,
// whose registers are needed for the tree) loads them in the epilogue.
template <int E, bool PF>
struct SgdState {
    float4 w[E / 4], v[E / 4];
};

template <int E, bool PF>
__device__ __forceinline__ void prefetch_state(int64_t i0, int64_t P, bool do_sgd, const float* __restrict__ w,
                                               const float* __restrict__ v, SgdState<E, PF>& st) {
    if (PF && do_sgd && i0 + E <= P) {
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            st.w[q] = *reinterpret_cast<const float4*>(w + i0 + 4 * q);
            st.v[q] = *reinterpret_cast<const float4*>(v + i0 + 4 * q);
        }
    }
}

template <int E, bool PF>
__device__ __forceinline__ void epilogue(const float (&s)[E], int64_t i0, int64_t P, float invW,
                                         float* __restrict__ grad, bool do_sgd, float lr, float mu,
                                         float* __restrict__ w, float* __restrict__ v, SgdState<E, PF>& st) {
    float g[E];
#pragma unroll
    for (int e = 0; e < E; ++e) g[e] = s[e] * invW;
    if (i0 + E <= P) {
        if (grad) {
#pragma unroll
            for (int e = 0; e < E; e += 4)
                *reinterpret_cast<float4*>(grad + i0 + e) = make_float4(g[e], g[e + 1], g[e + 2], g[e + 3]);
        }
        if (do_sgd) {
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                if (!PF) {
                    st.w[q] = *reinterpret_cast<const float4*>(w + i0 + 4 * q);
                    st.v[q] = *reinterpret_cast<const float4*>(v + i0 + 4 * q);
                }
                float4& wv = st.w[q];
                float4& vv = st.v[q];
                sgd_update(g[4 * q + 0], lr, mu, wv.x, vv.x);
                sgd_update(g[4 * q + 1], lr, mu, wv.y, vv.y);
                sgd_update(g[4 * q + 2], lr, mu, wv.z, vv.z);
                sgd_update(g[4 * q + 3], lr, mu, wv.w, vv.w);
                // streaming stores: w and v are not read again within the step
                __builtin_nontemporal_store(f32x4{wv.x, wv.y, wv.z, wv.w}, reinterpret_cast<f32x4*>(w + i0 + 4 * q));
                __builtin_nontemporal_store(f32x4{vv.x, vv.y, vv.z, vv.w}, reinterpret_cast<f32x4*>(v + i0 + 4 * q));
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (i0 + e < P) {
                if (grad) grad[i0 + e] = g[e];
                if (do_sgd) {
                    float wv = w[i0 + e], vv = v[i0 + e];
                    sgd_update(g[e], lr, mu, wv, vv);
                    w[i0 + e] = wv;
                    v[i0 + e] = vv;
                }
            }
        }
    }
}

template <int LEV, bool FP16, int U>
__global__ __launch_bounds__(kThreads) void k_tree(const void* __restrict__ bucket, int64_t ld,
                                                   int32_t W, int64_t P, float invW,
                                                   float* __restrict__ grad, int32_t do_sgd, float lr,
                                                   float mu, float* __restrict__ w,
                                                   float* __restrict__ v) {
    using LV = LeafVec<FP16>;
    constexpr int E = LV::E;
    using raw = typename LV::raw;
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * E;
    if (i0 >= P) return;
    const int64_t row_bytes = ld * (FP16 ? 2 : 4);
    const char* base = static_cast<const char*>(bucket) + i0 * (FP16 ? 2 : 4);
    SgdState<E, (LEV <= 8)> st;
    prefetch_state(i0, P, do_sgd != 0, w, v, st);

    TreeAcc<LEV, E> tree;
    uint32_t cnt = 0;
    for (int32_t w0 = 0; w0 < W; w0 += U) {
        raw x[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (w0 + u < W) x[u] = load_leaf(base + (int64_t)(w0 + u) * row_bytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (w0 + u < W) {
                float f[E];
                LV::widen(x[u], f);
                tree.push(f, cnt);
                ++cnt;
            }
        }
    }
    float s[E];
    tree.result((uint32_t)W, s);
    epilogue(s, i0, P, invW, grad, do_sgd != 0, lr, mu, w, v, st);
}

// Zero-copy lazy-allreduce fusion for the dense path: the leaves are read
// straight from every worker's per-layer tensors through the layer table.
// A wavefront whose 64*E elements lie in one layer (the common case) resolves
// the layer once and reads each worker's tensor with 128-bit loads (element
// loads when a tensor is not 16-byte aligned); a wavefront that straddles a
// layer boundary resolves the layer of every element.
template <int LEV, bool FP16, int U>
__device__ __forceinline__ void tree_layers_block(int64_t blk, const uint64_t* __restrict__ layer_ptrs,
                                                  const int64_t* __restrict__ offsets,
                                                  const uint32_t* __restrict__ tile_layer,
                                                  const uint32_t* __restrict__ tile_order, int64_t n_tiles,
                                                  int32_t L,
                                                  int32_t tbl_stride, int32_t tbl_first, int32_t W, int64_t P,
                                                  float invW, float* __restrict__ grad, int32_t do_sgd, float lr,
                                                  float mu, float* __restrict__ w, float* __restrict__ v) {
    using LV = LeafVec<FP16>;
    constexpr int E = LV::E;
    constexpr int kEsz = FP16 ? 2 : 4;
    using raw = typename LV::raw;
    const int lane = threadIdx.x & 63;
    // the wavefront's tile, in the plan's order (straddling tiles first)
    const int64_t gw = blk * (kThreads / 64) + (int64_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (gw >= n_tiles) return;
    const uint32_t tile = tile_order[gw];
    const int64_t wave_base = (int64_t)tile * (64 * E);
    const int64_t i0 = wave_base + (int64_t)lane * E;
    const bool valid = i0 < P;
    SgdState<E, (LEV <= 8)> st;
    prefetch_state(i0, P, do_sgd != 0, w, v, st);

    auto layer_of = [&](int64_t i) {
        int32_t lo = 0, hi = L;
        while (lo < hi) {
            const int32_t mid = (lo + hi) >> 1;
            if (offsets[mid + 1] <= i) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    };
    // The plan's tile table gives the wavefront's layer in one scalar load.
    const uint32_t tinfo = tile_layer[tile];
    const int32_t l0 = (int32_t)(tinfo & 0x7fffffffu);
    const int64_t off0 = offsets[l0];
    // Fast path: the wavefront's 64*E elements all exist, lie in layer l0 at an
    // E-aligned offset, and every worker's tensor of that layer is 16-byte
    // aligned (checked with one ballot per 64 workers).
    bool fast = (tinfo >> 31) != 0u;
    // For W < 256 the (at most four) 64-worker groups of addresses stay in
    // registers from the alignment check to the loads.
    constexpr int kGroups = LEV <= 8 ? 4 : 1;
    uint64_t gaddr[kGroups];
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) gaddr[gi] = 0ull;
    if (fast) {
        for (int32_t g0 = 0; g0 < W; g0 += 64) {
            const uint64_t a = g0 + lane < W ? layer_ptrs[(int64_t)(g0 + lane) * tbl_stride + tbl_first + l0] : 0ull;
            fast = fast && __ballot((a & 15ull) != 0ull) == 0ull;
            if (LEV <= 8) {
#pragma unroll
                for (int gi = 0; gi < kGroups; ++gi)
                    if (gi == (g0 >> 6)) gaddr[gi] = a;
            }
        }
    }

    TreeAcc<LEV, E> tree;
    uint32_t cnt = 0;
    if (fast) {
        for (int32_t g0 = 0; g0 < W; g0 += 64) {
            // lane l holds worker (g0 + l)'s tensor address; each worker's
            // address is then taken from its lane without a memory access
            uint64_t mine = 0ull;
            if (LEV <= 8) {
#pragma unroll
                for (int gi = 0; gi < kGroups; ++gi)
                    if (gi == (g0 >> 6)) mine = gaddr[gi];
            } else {
                mine = g0 + lane < W ? layer_ptrs[(int64_t)(g0 + lane) * tbl_stride + tbl_first + l0] : 0ull;
            }
            const uint32_t mine_lo = (uint32_t)mine, mine_hi = (uint32_t)(mine >> 32);
            const int32_t gn = W - g0 < 64 ? W - g0 : 64;
            const int64_t byte_off = (i0 - off0) * kEsz;
            for (int32_t u0 = 0; u0 < gn; u0 += U) {
                // All addresses first, then all loads with no branch between
                // them, so the U loads are in flight together (past the group
                // end the last worker is re-read and not pushed).
                uint64_t addr[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int ui = u0 + u < gn ? u0 + u : gn - 1;
                    addr[u] = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mine_hi, ui) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)mine_lo, ui);
                }
                raw x[U];
#pragma unroll
                for (int u = 0; u < U; ++u) x[u] = load_leaf_at(addr[u] + (uint64_t)byte_off);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (u0 + u < gn) {
                        float f[E];
                        LV::widen(x[u], f);
                        tree.push(f, cnt);
                        ++cnt;
                    }
                }
            }
        }
    } else {
        // General path (the wavefront straddles a layer boundary, holds the
        // tail, or meets an unaligned tensor): each lane resolves the layer of
        // its own first element and, when its E elements lie in that layer at
        // an E-aligned offset and the tensor is aligned, reads each worker
        // with one 128-bit load, otherwise element by element; up to 8
        // workers in flight.
        constexpr int kU = U < 8 ? U : 8;
        const int32_t la = valid ? layer_of(i0) : 0;
        const int64_t oa = offsets[la], ea = offsets[la + 1];
        const bool lane_vec = valid && i0 + E <= ea && (oa % E) == 0;
        for (int32_t w0 = 0; w0 < W; w0 += kU) {
            uint64_t ad[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                ad[u] = (w0 + u < W && valid) ? layer_ptrs[(int64_t)(w0 + u) * tbl_stride + tbl_first + la] : 0ull;
            raw x[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                x[u] = make_uint4(0u, 0u, 0u, 0u);
                if (w0 + u < W && valid) {
                    if (lane_vec && (ad[u] & 15) == 0) {
                        x[u] = load_leaf_at(ad[u] + (uint64_t)((i0 - oa) * kEsz));
                    } else {
                        uint32_t q[4] = {0u, 0u, 0u, 0u};
                        for (int e = 0; e < E; ++e) {
                            const int64_t i = i0 + e;
                            if (i < P) {
                                const int32_t l = i < ea ? la : layer_of(i);
                                const uint64_t a = l == la ? ad[u] : layer_ptrs[(int64_t)(w0 + u) * tbl_stride + tbl_first + l];
                                const int64_t j = i - offsets[l];
                                const uint32_t bits = FP16 ? (uint32_t)as_global<uint16_t>(a)[j]
                                                           : as_global<uint32_t>(a)[j];
                                if (FP16) q[e >> 1] |= bits << (16 * (e & 1));
                                else q[e] = bits;
                            }
                        }
                        x[u] = make_uint4(q[0], q[1], q[2], q[3]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (w0 + u < W) {
                    float f[E];
                    LV::widen(x[u], f);
                    tree.push(f, cnt);
                    ++cnt;
                }
            }
        }
    }
    float s[E];
    tree.result((uint32_t)W, s);
    if (valid) epilogue(s, i0, P, invW, grad, do_sgd != 0, lr, mu, w, v, st);
}

// One workgroup per block of 256 * E elements.
template <int LEV, bool FP16, int U>
__global__ __launch_bounds__(kThreads) void k_tree_layers(const uint64_t* __restrict__ layer_ptrs,
                                                          const int64_t* __restrict__ offsets,
                                                          const uint32_t* __restrict__ tile_layer,
                                                          const uint32_t* __restrict__ tile_order,
                                                          int64_t n_tiles, int32_t L, int32_t tbl_stride,
                                                          int32_t tbl_first, int32_t W, int64_t P, float invW,
                                                          float* __restrict__ grad, int32_t do_sgd, float lr,
                                                          float mu, float* __restrict__ w,
                                                          float* __restrict__ v) {
    tree_layers_block<LEV, FP16, U>(blockIdx.x, layer_ptrs, offsets, tile_layer, tile_order, n_tiles, L, tbl_stride,
                                 tbl_first, W, P, invW, grad, do_sgd, lr, mu, w, v);
}

// A capped grid (to leave compute units to a concurrent kernel): each
// workgroup strides over the blocks.
template <int LEV, bool FP16, int U>
__global__ __launch_bounds__(kThreads) void k_tree_layers_strided(const uint64_t* __restrict__ layer_ptrs,
                                                                  const int64_t* __restrict__ offsets,
                                                                  const uint32_t* __restrict__ tile_layer,
                                                                  const uint32_t* __restrict__ tile_order,
                                                                  int64_t n_tiles, int32_t L, int32_t tbl_stride,
                                                                  int32_t tbl_first, int32_t W, int64_t P,
                                                                  int64_t n_blocks, float invW,
                                                                  float* __restrict__ grad, int32_t do_sgd, float lr,
                                                                  float mu, float* __restrict__ w,
                                                                  float* __restrict__ v) {
    for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x)
        tree_layers_block<LEV, FP16, U>(blk, layer_ptrs, offsets, tile_layer, tile_order, n_tiles, L, tbl_stride,
                                     tbl_first, W, P, invW, grad, do_sgd, lr, mu, w, v);
}

__global__ __launch_bounds__(kThreads) void k_sgd(int64_t P, const float* __restrict__ g,
                                                  float* __restrict__ w, float* __restrict__ v,
                                                  float lr, float mu) {
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (i0 >= P) return;
    if (i0 + 4 <= P) {
        float4 gv = *reinterpret_cast<const float4*>(g + i0);
        float4 wv = *reinterpret_cast<const float4*>(w + i0);
        float4 vv = *reinterpret_cast<const float4*>(v + i0);
        sgd_update(gv.x, lr, mu, wv.x, vv.x);
        sgd_update(gv.y, lr, mu, wv.y, vv.y);
        sgd_update(gv.z, lr, mu, wv.z, vv.z);
        sgd_update(gv.w, lr, mu, wv.w, vv.w);
        *reinterpret_cast<float4*>(w + i0) = wv;
        *reinterpret_cast<float4*>(v + i0) = vv;
    } else {
        for (int64_t i = i0; i < P; ++i) {
            float wv = w[i], vv = v[i];
            sgd_update(g[i], lr, mu, wv, vv);
            w[i] = wv;
            v[i] = vv;
        }
    }
}

template <int LEV, bool FP16, int U>
hipError_t tree_launch(const Plan& p, const void* bucket, float invW, float* grad, const ga_sgd* sgd, float* w,
                       float* v, hipStream_t s) {
    constexpr int E = FP16 ? 8 : 4;
    const int64_t threads = (p.P + E - 1) / E;
    const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
    const float lr = sgd ? sgd->lr : 0.f, mu = sgd ? sgd->mu : 0.f;
    hipLaunchKernelGGL((k_tree<LEV, FP16, U>), dim3(blocks), dim3(kThreads), 0, s, bucket, p.ld, p.W, p.P, invW,
                       grad, sgd ? 1 : 0, lr, mu, w, v);
    return hipGetLastError();
}

template <int LEV>
hipError_t tree_dispatch(const Plan& p, const void* bucket, float invW, float* grad, const ga_sgd* sgd, float* w,
                         float* v, hipStream_t s) {
    // the 11-level tree serves W >= 256, so its binary16 form is always narrow
    if (p.dtype == GA_FP16 && (LEV > 8 || p.W >= kNarrowMinW))
        return tree_launch<LEV, true, kUnrollNarrow>(p, bucket, invW, grad, sgd, w, v, s);
    if constexpr (LEV == 8)
        if (p.dtype == GA_FP16) return tree_launch<LEV, true, kUnrollW>(p, bucket, invW, grad, sgd, w, v, s);
    return tree_launch<LEV, false, kUnrollW>(p, bucket, invW, grad, sgd, w, v, s);
}

template <int LEV, bool FP16, int U>
hipError_t tree_layers_launch(const Plan& p, const uint64_t* layer_ptrs, int32_t tbl_stride, int32_t tbl_first,
                              int64_t n_blocks, int32_t max_blocks, float invW, float* grad, int do_sgd, float lr,
                              float mu, float* w, float* v, hipStream_t s) {
    if (max_blocks > 0 && max_blocks < n_blocks)
        hipLaunchKernelGGL((k_tree_layers_strided<LEV, FP16, U>), dim3(max_blocks), dim3(kThreads), 0, s, layer_ptrs,
                           p.d_offsets, p.d_tile_layer, p.d_tile_order, p.n_tiles, p.L, tbl_stride, tbl_first, p.W,
                           p.P, n_blocks, invW, grad, do_sgd, lr, mu, w, v);
    else
        hipLaunchKernelGGL((k_tree_layers<LEV, FP16, U>), dim3((unsigned)n_blocks), dim3(kThreads), 0, s, layer_ptrs,
                           p.d_offsets, p.d_tile_layer, p.d_tile_order, p.n_tiles, p.L, tbl_stride, tbl_first, p.W,
                           p.P, invW, grad, do_sgd, lr, mu, w, v);
    return hipGetLastError();
}

template <int LEV>
hipError_t tree_layers_dispatch(const Plan& p, const uint64_t* layer_ptrs, int32_t tbl_stride, int32_t tbl_first,
                                float* grad, const ga_sgd* sgd, float* w, float* v, int32_t max_blocks,
                                hipStream_t s) {
    const int E = p.dtype == GA_FP16 ? 8 : 4;
    const int64_t threads = (p.P + E - 1) / E;
    const int64_t n_blocks = (threads + kThreads - 1) / kThreads;
    const float invW = (float)(1.0 / (double)p.W);
    const float lr = sgd ? sgd->lr : 0.f, mu = sgd ? sgd->mu : 0.f;
    const int do_sgd = sgd ? 1 : 0;
    if (p.dtype == GA_FP16 && (LEV > 8 || p.W >= kNarrowMinW))
        return tree_layers_launch<LEV, true, kUnrollNarrow>(p, layer_ptrs, tbl_stride, tbl_first, n_blocks,
                                                            max_blocks, invW, grad, do_sgd, lr, mu, w, v, s);
    if constexpr (LEV == 8)
        if (p.dtype == GA_FP16)
            return tree_layers_launch<LEV, true, kUnrollW>(p, layer_ptrs, tbl_stride, tbl_first, n_blocks,
                                                           max_blocks, invW, grad, do_sgd, lr, mu, w, v, s);
    return tree_layers_launch<LEV, false, kUnrollW>(p, layer_ptrs, tbl_stride, tbl_first, n_blocks, max_blocks,
                                                    invW, grad, do_sgd, lr, mu, w, v, s);
}

}  // namespace

hipError_t launch_tree(const Plan& p, const void* bucket, float* grad, const ga_sgd* sgd, float* w,
                       float* v, hipStream_t s) {
    return launch_tree_scaled(p, bucket, (float)(1.0 / (double)p.W), grad, sgd, w, v, s);
}

hipError_t launch_tree_scaled(const Plan& p, const void* bucket, float scale, float* grad, const ga_sgd* sgd,
                              float* w, float* v, hipStream_t s) {
    if (p.P == 0) return hipSuccess;
    // Eight levels for every W below 256: measured no slower than a shallower
    // tree for small W (fewer resident waves, same bytes in flight).
    if (p.W < (1 << 8)) return tree_dispatch<8>(p, bucket, scale, grad, sgd, w, v, s);
    return tree_dispatch<11>(p, bucket, scale, grad, sgd, w, v, s);
}

hipError_t launch_tree_layers(const Plan& p, const uint64_t* layer_ptrs, float* grad, const ga_sgd* sgd,
                              float* w, float* v, hipStream_t s) {
    return launch_tree_layers_sub(p, layer_ptrs, p.L, 0, grad, sgd, w, v, 0, s);
}

hipError_t launch_tree_layers_sub(const Plan& p, const uint64_t* layer_ptrs, int32_t tbl_stride, int32_t tbl_first,
                                  float* grad, const ga_sgd* sgd, float* w, float* v, int32_t max_blocks,
                                  hipStream_t s) {
    if (p.P == 0) return hipSuccess;
    if (p.W < (1 << 8))
        return tree_layers_dispatch<8>(p, layer_ptrs, tbl_stride, tbl_first, grad, sgd, w, v, max_blocks, s);
    return tree_layers_dispatch<11>(p, layer_ptrs, tbl_stride, tbl_first, grad, sgd, w, v, max_blocks, s);
}

hipError_t launch_sgd(int64_t P, const float* g, float* w, float* v, const ga_sgd* sgd,
                      hipStream_t s) {
    if (P == 0) return hipSuccess;
    const int64_t threads = (P + 3) / 4;
    const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(k_sgd, dim3(blocks), dim3(kThreads), 0, s, P, g, w, v, sgd->lr, sgd->mu);
    return hipGetLastError();
}

}  // namespace ga
