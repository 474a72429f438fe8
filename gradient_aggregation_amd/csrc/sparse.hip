// Coarse-grained sparse communication (GradientFlow, arXiv abstract: only the
// important gradient chunks are transmitted).  Three kernels:
//
//   k_chunk_norm  one workgroup per (worker, chunk): a = leaf + residual is
//                 written back over the residual and the chunk's key, the sum
//                 of a^2 in binary64 (each square exact), is reduced in
//                 registers, then across the wavefront with cross-lane moves,
//                 then across the 4 wavefronts through LDS.  Traffic per
//                 element: leaf read, residual read, residual write.
//   k_topk        one workgroup per worker: every chunk's rank under the order
//                 (key desc, index asc) is counted against all keys staged in
//                 LDS; rank < k selects.  Exact integer compares, no sort.
//   k_gather      the fixed tree over the workers' transmitted chunks, mean,
//                 and fused momentum SGD; a worker that did not select a chunk
//                 contributes +0 without being read.
#include "common.h"
#include "tree.h"

namespace ga {

namespace {

constexpr int kNormThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kTopkTile = 4096;
constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 8;

__device__ __forceinline__ void widen8(const uint4& r, float (&f)[8]) {
    const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[j] & 0xffffu));
        f[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[j] >> 16));
    }
}

__device__ __forceinline__ float widen1(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// ---------------------------------------------------------------------------
// k_chunk_norm
// ---------------------------------------------------------------------------
template <bool FP16, bool LAZY>
__global__ __launch_bounds__(kNormThreads) void k_chunk_norm(
    const void* __restrict__ bucket, float* __restrict__ resid, int64_t ld, int64_t P, int64_t C,
    int32_t n_c, const uint32_t* __restrict__ prev_mask, int32_t mw, double* __restrict__ keys) {
    const int64_t b = blockIdx.x;
    const int32_t w = (int32_t)(b / n_c);
    const int32_t c = (int32_t)(b - (int64_t)w * n_c);
    const int64_t s = (int64_t)c * C;
    const int64_t e = s + C < P ? s + C : P;
    bool rzero = false;
    if (LAZY) rzero = (prev_mask[(int64_t)w * mw + (c >> 5)] >> (c & 31)) & 1u;

    float* __restrict__ r = resid + (int64_t)w * ld;
    double acc0 = 0.0, acc1 = 0.0;

    // Body: 8-element vectors (chunk starts are multiples of 8).
    const int64_t nvec = (e - s) >> 3;
    constexpr int UN = 4;
    int64_t j = threadIdx.x;
    for (; j + (UN - 1) * kNormThreads < nvec; j += UN * kNormThreads) {
        float lf[UN][8];
        float4 r0[UN], r1[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t i = s + ((j + u * kNormThreads) << 3);
            if (FP16) {
                const uint4 gv = *reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(bucket) + (int64_t)w * ld + i);
                widen8(gv, lf[u]);
            } else {
                const float* gp = static_cast<const float*>(bucket) + (int64_t)w * ld + i;
                const float4 g0 = *reinterpret_cast<const float4*>(gp);
                const float4 g1 = *reinterpret_cast<const float4*>(gp + 4);
                lf[u][0] = g0.x; lf[u][1] = g0.y; lf[u][2] = g0.z; lf[u][3] = g0.w;
                lf[u][4] = g1.x; lf[u][5] = g1.y; lf[u][6] = g1.z; lf[u][7] = g1.w;
            }
            if (!rzero) {
                r0[u] = *reinterpret_cast<const float4*>(r + i);
                r1[u] = *reinterpret_cast<const float4*>(r + i + 4);
            } else {
                r0[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                r1[u] = r0[u];
            }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t i = s + ((j + u * kNormThreads) << 3);
            float4 a0, a1;
            a0.x = lf[u][0] + r0[u].x; a0.y = lf[u][1] + r0[u].y;
            a0.z = lf[u][2] + r0[u].z; a0.w = lf[u][3] + r0[u].w;
            a1.x = lf[u][4] + r1[u].x; a1.y = lf[u][5] + r1[u].y;
            a1.z = lf[u][6] + r1[u].z; a1.w = lf[u][7] + r1[u].w;
            *reinterpret_cast<float4*>(r + i) = a0;
            *reinterpret_cast<float4*>(r + i + 4) = a1;
            acc0 = fma((double)a0.x, (double)a0.x, acc0);
            acc1 = fma((double)a0.y, (double)a0.y, acc1);
            acc0 = fma((double)a0.z, (double)a0.z, acc0);
            acc1 = fma((double)a0.w, (double)a0.w, acc1);
            acc0 = fma((double)a1.x, (double)a1.x, acc0);
            acc1 = fma((double)a1.y, (double)a1.y, acc1);
            acc0 = fma((double)a1.z, (double)a1.z, acc0);
            acc1 = fma((double)a1.w, (double)a1.w, acc1);
        }
    }
    for (; j < nvec; j += kNormThreads) {
        const int64_t i = s + (j << 3);
        float lf[8];
        if (FP16) {
            widen8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(bucket) + (int64_t)w * ld + i), lf);
        } else {
            const float* gp = static_cast<const float*>(bucket) + (int64_t)w * ld + i;
#pragma unroll
            for (int q = 0; q < 8; ++q) lf[q] = gp[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float a = lf[q] + (rzero ? 0.f : r[i + q]);
            r[i + q] = a;
            acc0 = fma((double)a, (double)a, acc0);
        }
    }
    // Tail: fewer than 8 elements at the end of the last chunk.
    for (int64_t i = s + (nvec << 3) + threadIdx.x; i < e; i += kNormThreads) {
        float lf;
        if (FP16) lf = widen1(static_cast<const uint16_t*>(bucket)[(int64_t)w * ld + i]);
        else lf = static_cast<const float*>(bucket)[(int64_t)w * ld + i];
        const float a = lf + (rzero ? 0.f : r[i]);
        r[i] = a;
        acc0 = fma((double)a, (double)a, acc0);
    }

    double t = wave_sum(acc0 + acc1);
    __shared__ double part[kNormThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) part[wave] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        double k = part[0];
#pragma unroll
        for (int q = 1; q < kNormThreads / 64; ++q) k += part[q];
        keys[b] = k;
    }
}

// ---------------------------------------------------------------------------
// k_topk
// ---------------------------------------------------------------------------

// Order key of a chunk: binary64 keys are sums of squares, so non-negative;
// their bit patterns order as unsigned integers.  NaN ranks above everything.
__device__ __forceinline__ uint64_t order_key(double k) {
    if (k != k) return ~0ull;
    uint64_t u = __builtin_bit_cast(uint64_t, k);
    return u == 0x8000000000000000ull ? 0ull : u;
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(const double* __restrict__ keys, int32_t n_c,
                                                       int32_t k, int32_t mw,
                                                       int32_t* __restrict__ sel_idx,
                                                       uint32_t* __restrict__ sel_mask) {
    const int32_t w = blockIdx.x;
    const double* kw = keys + (int64_t)w * n_c;
    __shared__ uint64_t tile[kTopkTile];
    __shared__ uint32_t mask[GA_MAX_CHUNKS / 32];

    for (int32_t i = threadIdx.x; i < mw; i += kTopkThreads) mask[i] = 0;
    const bool one_tile = n_c <= kTopkTile;
    if (one_tile) {
        for (int32_t i = threadIdx.x; i < n_c; i += kTopkThreads) tile[i] = order_key(kw[i]);
    }
    __syncthreads();

    // Chunk c (owned by thread c mod 1024) is selected iff fewer than k chunks
    // precede it in the order.  The loop bounds are uniform, so every thread
    // reaches every barrier.
    for (int32_t c0 = 0; c0 < n_c; c0 += kTopkThreads) {
        const int32_t c = c0 + threadIdx.x;
        const uint64_t kc = c < n_c ? order_key(kw[c]) : 0;
        int32_t rank = 0;
        for (int32_t t0 = 0; t0 < n_c; t0 += kTopkTile) {
            const int32_t tn = n_c - t0 < kTopkTile ? n_c - t0 : kTopkTile;
            if (!one_tile) {
                __syncthreads();
                for (int32_t i = threadIdx.x; i < tn; i += kTopkThreads) tile[i] = order_key(kw[t0 + i]);
                __syncthreads();
            }
            if (c < n_c) {
                for (int32_t i = 0; i < tn; ++i) {
                    const uint64_t ko = tile[i];
                    rank += (ko > kc) || (ko == kc && t0 + i < c);
                }
            }
        }
        if (c < n_c && rank < k) atomicOr(&mask[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    for (int32_t i = threadIdx.x; i < mw; i += kTopkThreads) sel_mask[(int64_t)w * mw + i] = mask[i];
    // A selected chunk's place in the ascending list = selected chunks below it.
    for (int32_t c = threadIdx.x; c < n_c; c += kTopkThreads) {
        if ((mask[c >> 5] >> (c & 31)) & 1u) {
            int32_t pos = __popc(mask[c >> 5] & ((1u << (c & 31)) - 1u));
            for (int32_t m = 0; m < (c >> 5); ++m) pos += __popc(mask[m]);
            sel_idx[(int64_t)w * k + pos] = c;
        }
    }
}

// ---------------------------------------------------------------------------
// k_gather
// ---------------------------------------------------------------------------

// One thread owns 4 consecutive elements (one 128-bit residual load per
// worker).  With UNIFORM, C is a multiple of the 256 elements a wavefront
// covers, so the whole wavefront lies in one chunk and the selection bits are
// wavefront-uniform: unselected workers are skipped by a scalar branch.
template <int LEV, bool UNIFORM>
__global__ __launch_bounds__(kGatherThreads) void k_gather(
    float* __restrict__ resid, int64_t ld, int32_t W, int64_t P, int64_t C,
    const uint32_t* __restrict__ sel_mask, int32_t mw, int32_t zero_sel, float invW,
    float* __restrict__ grad, int32_t do_sgd, float lr, float mu, float* __restrict__ w,
    float* __restrict__ v) {
    constexpr int E = 4;
    const int64_t i0 = ((int64_t)blockIdx.x * kGatherThreads + threadIdx.x) * E;
    if (i0 >= P) return;
    int32_t c;
    if (UNIFORM) {
        const int64_t wave_base = ((int64_t)blockIdx.x * kGatherThreads +
                                   (int64_t)__builtin_amdgcn_readfirstlane(threadIdx.x & ~63u)) * E;
        c = (int32_t)(wave_base / C);
    } else {
        c = (int32_t)(i0 / C);
    }
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
                if (zero_sel && on[u]) {
                    float* rp = resid + (int64_t)(w0 + u) * ld + i0;
                    if (i0 + E <= P) {
                        *reinterpret_cast<float4*>(rp) = make_float4(0.f, 0.f, 0.f, 0.f);
                    } else {
                        for (int e = 0; e < E; ++e)
                            if (i0 + e < P) rp[e] = 0.f;
                    }
                }
            }
        }
    }
    float s[E];
    tree.result((uint32_t)W, s);
    float g[E];
#pragma unroll
    for (int e = 0; e < E; ++e) g[e] = s[e] * invW;
    if (i0 + E <= P) {
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

template <int LEV>
hipError_t gather_dispatch(const Plan& p, float* resid, const uint32_t* sel_mask, int zero_sel,
                           float* grad, const ga_sgd* sgd, float* w, float* v, hipStream_t s) {
    const int64_t threads = (p.P + 3) / 4;
    const unsigned blocks = (unsigned)((threads + kGatherThreads - 1) / kGatherThreads);
    const float invW = (float)(1.0 / (double)p.W);
    const float lr = sgd ? sgd->lr : 0.f, mu = sgd ? sgd->mu : 0.f;
    const bool uniform = (p.C % 256) == 0;
    if (uniform)
        hipLaunchKernelGGL((k_gather<LEV, true>), dim3(blocks), dim3(kGatherThreads), 0, s, resid, p.ld,
                           p.W, p.P, p.C, sel_mask, p.mw, zero_sel, invW, grad, sgd ? 1 : 0, lr, mu, w, v);
    else
        hipLaunchKernelGGL((k_gather<LEV, false>), dim3(blocks), dim3(kGatherThreads), 0, s, resid, p.ld,
                           p.W, p.P, p.C, sel_mask, p.mw, zero_sel, invW, grad, sgd ? 1 : 0, lr, mu, w, v);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_norm(const Plan& p, const void* bucket, float* resid, const uint32_t* prev_mask,
                             double* keys, hipStream_t s) {
    const int64_t blocks = (int64_t)p.W * p.n_c;
    if (blocks == 0) return hipSuccess;
    const bool f16 = p.dtype == GA_FP16;
    const int32_t n_c = (int32_t)p.n_c;
    if (f16 && prev_mask)
        hipLaunchKernelGGL((k_chunk_norm<true, true>), dim3((unsigned)blocks), dim3(kNormThreads), 0, s,
                           bucket, resid, p.ld, p.P, p.C, n_c, prev_mask, p.mw, keys);
    else if (f16)
        hipLaunchKernelGGL((k_chunk_norm<true, false>), dim3((unsigned)blocks), dim3(kNormThreads), 0, s,
                           bucket, resid, p.ld, p.P, p.C, n_c, prev_mask, p.mw, keys);
    else if (prev_mask)
        hipLaunchKernelGGL((k_chunk_norm<false, true>), dim3((unsigned)blocks), dim3(kNormThreads), 0, s,
                           bucket, resid, p.ld, p.P, p.C, n_c, prev_mask, p.mw, keys);
    else
        hipLaunchKernelGGL((k_chunk_norm<false, false>), dim3((unsigned)blocks), dim3(kNormThreads), 0, s,
                           bucket, resid, p.ld, p.P, p.C, n_c, prev_mask, p.mw, keys);
    return hipGetLastError();
}

hipError_t launch_topk(const Plan& p, const double* keys, int32_t* sel_idx, uint32_t* sel_mask,
                       hipStream_t s) {
    if (p.W == 0 || p.n_c == 0) return hipSuccess;
    hipLaunchKernelGGL(k_topk, dim3((unsigned)p.W), dim3(kTopkThreads), 0, s, keys, (int32_t)p.n_c, p.k,
                       p.mw, sel_idx, sel_mask);
    return hipGetLastError();
}

hipError_t launch_sparse_gather(const Plan& p, float* resid, const uint32_t* sel_mask, int zero_selected,
                                float* grad, const ga_sgd* sgd, float* w, float* v, hipStream_t s) {
    if (p.P == 0) return hipSuccess;
    if (p.W < (1 << 5)) return gather_dispatch<5>(p, resid, sel_mask, zero_selected, grad, sgd, w, v, s);
    if (p.W < (1 << 8)) return gather_dispatch<8>(p, resid, sel_mask, zero_selected, grad, sgd, w, v, s);
    return gather_dispatch<11>(p, resid, sel_mask, zero_selected, grad, sgd, w, v, s);
}

}  // namespace ga
