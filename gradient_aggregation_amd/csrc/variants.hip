// Other aggregation schemes of the pages, as summation orders over the same
// [W][ld] bucket, each optionally with a binary16 wire:
//
//   tree    the binary reduction tree (FireCaffe, paperlayer summary, sec. 6)
//   server  a parameter server receives every gradient and sums them, read as
//           worker order ((x0 + x1) + x2) + ... (same section)
//   ring    ring allreduce (GradientFlow, arXiv abstract): the vector is cut
//           into W segments of Q = ceil(P/W) rounded up to 64 elements; segment
//           s is summed starting at worker s+1, each worker adding its own value
//           to the partial sum it receives, worker s last
//
// Wire (GradientFlow's mixed-precision communication): every value sent
// between workers is binary16 and every add binary32 - the right operand of
// each tree add, each partial sum passed on the ring, the gradients the server
// receives, and the broadcast result.  The mean and momentum SGD follow as in
// the dense path.  A thread owns one 128-bit vector of every worker's row
// (8 binary16 or 4 binary32 elements); loads are issued 16 workers at a time.
#include "device.h"
#include "plan.h"
#include "tree.h"

namespace ga {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;
// The tree keeps 4 binary16 leaves in flight for W >= 64 (16 would leave room
// for only two wavefronts per SIMD), as the main tree kernel does.
constexpr int kUnrollNarrow = 4;
constexpr int kNarrowMinW = 64;

// One 128-bit vector of a worker's row: loaded raw (4 VGPRs) and widened to
// binary32 only when it is added.
template <bool FP16>
struct Vec;

template <>
struct Vec<false> {
    static constexpr int E = 4;
    static __device__ __forceinline__ void widen(const u32x4& r, float (&f)[4]) {
        f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
};

template <>
struct Vec<true> {
    static constexpr int E = 8;
    static __device__ __forceinline__ void widen(const u32x4& r, float (&f)[8]) {
        widen8(make_uint4(r.x, r.y, r.z, r.w), f);
    }
};

__device__ __forceinline__ u32x4 load_raw(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int E>
__device__ __forceinline__ void mean_sgd(float (&s)[E], bool wire, int64_t i0, int64_t P, float invW,
                                         float* __restrict__ grad, bool do_sgd, float lr, float mu,
                                         float* __restrict__ w, float* __restrict__ v) {
    float g[E];
#pragma unroll
    for (int e = 0; e < E; ++e) g[e] = (wire ? round_f16(s[e]) : s[e]) * invW;
    if (i0 + E <= P) {
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            if (grad) *reinterpret_cast<float4*>(grad + i0 + e) = make_float4(g[e], g[e + 1], g[e + 2], g[e + 3]);
            if (do_sgd) {
                float4 wv = *reinterpret_cast<const float4*>(w + i0 + e);
                float4 vv = *reinterpret_cast<const float4*>(v + i0 + e);
                sgd_update(g[e + 0], lr, mu, wv.x, vv.x);
                sgd_update(g[e + 1], lr, mu, wv.y, vv.y);
                sgd_update(g[e + 2], lr, mu, wv.z, vv.z);
                sgd_update(g[e + 3], lr, mu, wv.w, vv.w);
                *reinterpret_cast<float4*>(w + i0 + e) = wv;
                *reinterpret_cast<float4*>(v + i0 + e) = vv;
            }
        }
        return;
    }
    for (int e = 0; e < E; ++e) {
        const int64_t i = i0 + e;
        if (i >= P) break;
        if (grad) grad[i] = g[e];
        if (do_sgd) {
            float wv = w[i], vv = v[i];
            sgd_update(g[e], lr, mu, wv, vv);
            w[i] = wv;
            v[i] = vv;
        }
    }
}

template <int LEV, bool FP16, bool WIRE, int U>
__global__ __launch_bounds__(kThreads) void k_variant_tree(const void* __restrict__ bucket, int64_t ld, int32_t W,
                                                           int64_t P, float invW, float* __restrict__ grad,
                                                           int32_t do_sgd, float lr, float mu,
                                                           float* __restrict__ w, float* __restrict__ v) {
    using V = Vec<FP16>;
    constexpr int E = V::E;
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * E;
    if (i0 >= P) return;
    const int64_t esz = FP16 ? 2 : 4;
    const char* base = static_cast<const char*>(bucket);
    TreeAcc<LEV, E, WIRE> tree;
    uint32_t cnt = 0;
    for (int32_t w0 = 0; w0 < W; w0 += U) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (w0 + u < W) x[u] = load_raw(base + ((int64_t)(w0 + u) * ld + i0) * esz);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (w0 + u < W) {
                float f[E];
                V::widen(x[u], f);
                tree.push(f, cnt);
                ++cnt;
            }
        }
    }
    float s[E];
    tree.result((uint32_t)W, s);
    mean_sgd<E>(s, WIRE, i0, P, invW, grad, do_sgd != 0, lr, mu, w, v);
}

// Sequential orders.  RING: the lane's segment fixes the first worker.
template <bool FP16, bool WIRE, bool RING>
__global__ __launch_bounds__(kThreads) void k_variant_seq(const void* __restrict__ bucket, int64_t ld, int32_t W,
                                                          int64_t P, int64_t Q, float invW,
                                                          float* __restrict__ grad, int32_t do_sgd, float lr,
                                                          float mu, float* __restrict__ w, float* __restrict__ v) {
    using V = Vec<FP16>;
    constexpr int E = V::E;
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * E;
    if (i0 >= P) return;
    const int64_t esz = FP16 ? 2 : 4;
    const char* base = static_cast<const char*>(bucket);
    const int32_t first = RING ? (int32_t)((i0 / Q + 1) % W) : 0;
    float s[E];
    for (int32_t j0 = 0; j0 < W; j0 += kUnroll) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (j0 + u < W) {
                int32_t wk = first + j0 + u;
                if (wk >= W) wk -= W;
                x[u] = load_raw(base + ((int64_t)wk * ld + i0) * esz);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (j0 + u >= W) break;
            float f[E];
            V::widen(x[u], f);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (RING) {
                    // each worker adds its value to the partial sum it received
                    s[e] = (j0 + u == 0) ? f[e] : (WIRE ? round_f16(s[e]) : s[e]) + f[e];
                } else {
                    // the server adds the gradients it received, in worker order
                    const float r = WIRE ? round_f16(f[e]) : f[e];
                    s[e] = (j0 + u == 0) ? r : s[e] + r;
                }
            }
        }
    }
    mean_sgd<E>(s, WIRE, i0, P, invW, grad, do_sgd != 0, lr, mu, w, v);
}

template <bool FP16, bool WIRE>
hipError_t launch_variant_typed(const Plan& p, const void* bucket, int order, float* grad, const ga_sgd* sgd,
                                float* w, float* v, hipStream_t s) {
    constexpr int E = FP16 ? 8 : 4;
    const int64_t threads = (p.P + E - 1) / E;
    const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
    const float invW = (float)(1.0 / (double)p.W);
    const float lr = sgd ? sgd->lr : 0.f, mu = sgd ? sgd->mu : 0.f;
    const int do_sgd = sgd ? 1 : 0;
    const int64_t Q = ((p.P + p.W - 1) / p.W + 63) / 64 * 64;
    if (order == GA_ORDER_TREE) {
        constexpr int UW = FP16 ? kUnrollNarrow : kUnroll;  // leaves in flight for W >= 64
        if (p.W >= (1 << 8))
            hipLaunchKernelGGL((k_variant_tree<11, FP16, WIRE, UW>), dim3(blocks), dim3(kThreads), 0, s, bucket, p.ld,
                               p.W, p.P, invW, grad, do_sgd, lr, mu, w, v);
        else if (p.W >= kNarrowMinW)
            hipLaunchKernelGGL((k_variant_tree<8, FP16, WIRE, UW>), dim3(blocks), dim3(kThreads), 0, s, bucket, p.ld,
                               p.W, p.P, invW, grad, do_sgd, lr, mu, w, v);
        else
            hipLaunchKernelGGL((k_variant_tree<8, FP16, WIRE, kUnroll>), dim3(blocks), dim3(kThreads), 0, s, bucket,
                               p.ld, p.W, p.P, invW, grad, do_sgd, lr, mu, w, v);
    } else if (order == GA_ORDER_SERVER) {
        hipLaunchKernelGGL((k_variant_seq<FP16, WIRE, false>), dim3(blocks), dim3(kThreads), 0, s, bucket, p.ld,
                           p.W, p.P, Q, invW, grad, do_sgd, lr, mu, w, v);
    } else {
        hipLaunchKernelGGL((k_variant_seq<FP16, WIRE, true>), dim3(blocks), dim3(kThreads), 0, s, bucket, p.ld,
                           p.W, p.P, Q, invW, grad, do_sgd, lr, mu, w, v);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_variant(const Plan& p, const void* bucket, int order, int wire16, float* grad, const ga_sgd* sgd,
                          float* w, float* v, hipStream_t s) {
    if (p.P == 0) return hipSuccess;
    const bool f16 = p.dtype == GA_FP16;
    if (f16 && wire16) return launch_variant_typed<true, true>(p, bucket, order, grad, sgd, w, v, s);
    if (f16) return launch_variant_typed<true, false>(p, bucket, order, grad, sgd, w, v, s);
    if (wire16) return launch_variant_typed<false, true>(p, bucket, order, grad, sgd, w, v, s);
    return launch_variant_typed<false, false>(p, bucket, order, grad, sgd, w, v, s);
}

}  // namespace ga
