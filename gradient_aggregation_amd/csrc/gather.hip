// Coarse-grained sparse communication, part 3: gather-reduce of the chunks the
// workers send, in the fixed binary tree, with the mean and the fused
// momentum-SGD update.  A worker that did not select a chunk contributes +0
// without being read.
#include "device.h"
#include "plan.h"
#include "tree.h"

namespace ga {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 16;

typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// k_gather
// ---------------------------------------------------------------------------

// Mean, optional store of g and the fused SGD update for 4 elements at i0.
__device__ __forceinline__ void gather_epilogue(const float (&s)[4], int64_t i0, int64_t P, float invW,
                                                float* __restrict__ grad, bool do_sgd, float lr, float mu,
                                                float* __restrict__ w, float* __restrict__ v) {
    float g[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = s[e] * invW;
    if (i0 + 4 <= P) {
        if (grad) *reinterpret_cast<float4*>(grad + i0) = make_float4(g[0], g[1], g[2], g[3]);
        if (do_sgd) {
            float4 wv = *reinterpret_cast<const float4*>(w + i0);
            float4 vv = *reinterpret_cast<const float4*>(v + i0);
            sgd_update(g[0], lr, mu, wv.x, vv.x);
            sgd_update(g[1], lr, mu, wv.y, vv.y);
            sgd_update(g[2], lr, mu, wv.z, vv.z);
            sgd_update(g[3], lr, mu, wv.w, vv.w);
            *reinterpret_cast<float4*>(w + i0) = wv;
            *reinterpret_cast<float4*>(v + i0) = vv;
        }
    } else {
        for (int e = 0; e < 4; ++e) {
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

__device__ __forceinline__ void zero4(float* p, int64_t i0, int64_t P) {
    if (i0 + 4 <= P) {
        *reinterpret_cast<float4*>(p) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        for (int e = 0; e < 4; ++e)
            if (i0 + e < P) p[e] = 0.f;
    }
}

// Uniform-chunk form: C is a multiple of the 256 elements a wavefront covers
// (4 per lane), so the wavefront lies in one chunk.  Lane l reads worker
// (g0 + l)'s mask word for that chunk and a ballot turns the 64 bits into a
// wavefront-uniform bitmap: unselected workers cost no memory access, and a
// chunk that no worker selected skips the tree (its sum is +0).  For W < 256
// the (at most four) bitmaps stay in scalar registers; w and v are fetched
// before the tree so their latency overlaps the residual loads.
template <int LEV>
__global__ __launch_bounds__(kGatherThreads) void k_gather_wave(
    float* __restrict__ resid, int64_t ld, int32_t W, int64_t P, int64_t C,
    const uint32_t* __restrict__ sel_mask, int32_t mw, int32_t zero_sel, float invW,
    float* __restrict__ grad, int32_t do_sgd, float lr, float mu, float* __restrict__ w,
    float* __restrict__ v) {
    constexpr int E = 4;
    constexpr int kGroups = LEV <= 8 ? 4 : 0;  // cached 64-worker bitmaps (W < 256)
    const int lane = threadIdx.x & 63;
    const int64_t wave_base =
        ((int64_t)blockIdx.x * kGatherThreads + (int64_t)__builtin_amdgcn_readfirstlane(threadIdx.x & ~63u)) * E;
    if (wave_base >= P) return;  // whole wavefront past the end
    const int64_t i0 = wave_base + (int64_t)lane * E;
    const bool valid = i0 < P;
    const bool full = i0 + E <= P;
    const int32_t c = (int32_t)(wave_base / C);
    const int32_t cw = c >> 5;
    const uint32_t cb = 1u << (c & 31);

    float4 wv = make_float4(0.f, 0.f, 0.f, 0.f), vv = wv;
    if (do_sgd && full) {
        wv = *reinterpret_cast<const float4*>(w + i0);
        vv = *reinterpret_cast<const float4*>(v + i0);
    }

    auto bitmap = [&](int32_t g0) -> uint64_t {
        const bool bit = (g0 + lane < W) && (sel_mask[(int64_t)(g0 + lane) * mw + cw] & cb);
        return __ballot(bit);
    };
    uint64_t mb[kGroups > 0 ? kGroups : 1];
    bool any = false;
    if (kGroups > 0) {
        // every group's mask word is requested before the first ballot, so
        // the (at most four) loads are in flight together
        uint32_t word[kGroups > 0 ? kGroups : 1];
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
            const int32_t wk = gi * 64 + lane;
            word[gi] = wk < W ? sel_mask[(int64_t)wk * mw + cw] : 0u;
        }
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
            mb[gi] = __ballot((word[gi] & cb) != 0u);
            any |= mb[gi] != 0ull;
        }
    } else {
        for (int32_t g0 = 0; g0 < W; g0 += 64) any |= bitmap(g0) != 0ull;
    }

    float s[E] = {0.f, 0.f, 0.f, 0.f};
    if (any) {
        TreeAcc<LEV, E> tree;
        uint32_t cnt = 0;
        for (int32_t g0 = 0; g0 < W; g0 += 64) {
            uint64_t m;
            if (kGroups > 0) {
                const int gi = g0 >> 6;
                m = gi == 0 ? mb[0] : gi == 1 ? mb[kGroups > 1 ? 1 : 0] : gi == 2 ? mb[kGroups > 2 ? 2 : 0]
                                                                              : mb[kGroups > 3 ? 3 : 0];
            } else {
                m = bitmap(g0);
            }
            const int32_t gn = W - g0 < 64 ? W - g0 : 64;
            for (int32_t u0 = 0; u0 < gn; u0 += kGatherUnroll) {
                float4 x[kGatherUnroll];
#pragma unroll
                for (int u = 0; u < kGatherUnroll; ++u) {
                    x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (u0 + u < gn && ((m >> (u0 + u)) & 1ull) && valid) {
                        const v4f t = __builtin_nontemporal_load(
                            reinterpret_cast<const v4f*>(resid + (int64_t)(g0 + u0 + u) * ld + i0));
                        x[u] = make_float4(t.x, t.y, t.z, t.w);
                    }
                }
#pragma unroll
                for (int u = 0; u < kGatherUnroll; ++u) {
                    if (u0 + u < gn) {
                        float f[E] = {x[u].x, x[u].y, x[u].z, x[u].w};
                        tree.push(f, cnt);
                        ++cnt;
                        if (zero_sel && ((m >> (u0 + u)) & 1ull) && valid)
                            zero4(resid + (int64_t)(g0 + u0 + u) * ld + i0, i0, P);
                    }
                }
            }
        }
        tree.result((uint32_t)W, s);
    }
    if (!valid) return;
    if (full) {
        float g[E];
#pragma unroll
        for (int e = 0; e < E; ++e) g[e] = s[e] * invW;
        if (grad) *reinterpret_cast<float4*>(grad + i0) = make_float4(g[0], g[1], g[2], g[3]);
        if (do_sgd) {
            sgd_update(g[0], lr, mu, wv.x, vv.x);
            sgd_update(g[1], lr, mu, wv.y, vv.y);
            sgd_update(g[2], lr, mu, wv.z, vv.z);
            sgd_update(g[3], lr, mu, wv.w, vv.w);
            *reinterpret_cast<float4*>(w + i0) = wv;
            *reinterpret_cast<float4*>(v + i0) = vv;
        }
    } else {
        gather_epilogue(s, i0, P, invW, grad, do_sgd != 0, lr, mu, w, v);
    }
}

// General form: each lane finds its own chunk (C a multiple of 8, so the 4
// elements of a lane share a chunk) and tests every worker's bit itself.
template <int LEV>
__global__ __launch_bounds__(kGatherThreads) void k_gather_lane(
    float* __restrict__ resid, int64_t ld, int32_t W, int64_t P, int64_t C,
    const uint32_t* __restrict__ sel_mask, int32_t mw, int32_t zero_sel, float invW,
    float* __restrict__ grad, int32_t do_sgd, float lr, float mu, float* __restrict__ w,
    float* __restrict__ v) {
    constexpr int E = 4;
    const int64_t i0 = ((int64_t)blockIdx.x * kGatherThreads + threadIdx.x) * E;
    if (i0 >= P) return;
    const int32_t c = (int32_t)(i0 / C);
    const int32_t cw = c >> 5;
    const uint32_t cb = 1u << (c & 31);

    TreeAcc<LEV, E> tree;
    uint32_t cnt = 0;
    for (int32_t w0 = 0; w0 < W; w0 += kGatherUnroll) {
        float4 x[kGatherUnroll];
        bool on[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            on[u] = false;
            x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (w0 + u < W) {
                on[u] = (sel_mask[(int64_t)(w0 + u) * mw + cw] & cb) != 0;
                if (on[u]) x[u] = *reinterpret_cast<const float4*>(resid + (int64_t)(w0 + u) * ld + i0);
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            if (w0 + u < W) {
                float f[E] = {x[u].x, x[u].y, x[u].z, x[u].w};
                tree.push(f, cnt);
                ++cnt;
                if (zero_sel && on[u]) zero4(resid + (int64_t)(w0 + u) * ld + i0, i0, P);
            }
        }
    }
    float s[E];
    tree.result((uint32_t)W, s);
    gather_epilogue(s, i0, P, invW, grad, do_sgd != 0, lr, mu, w, v);
}

template <int LEV>
hipError_t gather_dispatch(const Plan& p, float* resid, const uint32_t* sel_mask, int zero_sel,
                           float* grad, const ga_sgd* sgd, float* w, float* v, hipStream_t s) {
    const int64_t threads = (p.P + 3) / 4;
    const unsigned blocks = (unsigned)((threads + kGatherThreads - 1) / kGatherThreads);
    const float invW = (float)(1.0 / (double)p.W);
    const float lr = sgd ? sgd->lr : 0.f, mu = sgd ? sgd->mu : 0.f;
    const bool uniform = (p.C % 256) == 0;
    if (uniform)
        hipLaunchKernelGGL((k_gather_wave<LEV>), dim3(blocks), dim3(kGatherThreads), 0, s, resid, p.ld,
                           p.W, p.P, p.C, sel_mask, p.mw, zero_sel, invW, grad, sgd ? 1 : 0, lr, mu, w, v);
    else
        hipLaunchKernelGGL((k_gather_lane<LEV>), dim3(blocks), dim3(kGatherThreads), 0, s, resid, p.ld,
                           p.W, p.P, p.C, sel_mask, p.mw, zero_sel, invW, grad, sgd ? 1 : 0, lr, mu, w, v);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_gather(const Plan& p, float* resid, const uint32_t* sel_mask, int zero_selected,
                                float* grad, const ga_sgd* sgd, float* w, float* v, hipStream_t s) {
    if (p.P == 0) return hipSuccess;
    if (p.W < (1 << 5)) return gather_dispatch<5>(p, resid, sel_mask, zero_selected, grad, sgd, w, v, s);
    if (p.W < (1 << 8)) return gather_dispatch<8>(p, resid, sel_mask, zero_selected, grad, sgd, w, v, s);
    return gather_dispatch<11>(p, resid, sel_mask, zero_selected, grad, sgd, w, v, s);
}

}  // namespace ga
