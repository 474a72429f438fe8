// Coarse-grained sparse communication (GradientFlow, arXiv abstract: only the
// important gradient chunks are transmitted).  Three kernels:
//
//   k_chunk_norm  one workgroup per (worker, chunk): a = leaf + residual is
//                 written back over the residual and the chunk's key, the sum
//                 of a^2 in binary64 (each square exact), is reduced in
//                 registers, then across the wavefront with cross-lane moves,
//                 then across the 4 wavefronts through LDS.  Traffic per
//                 element: leaf read, residual read, residual write.
//   k_topk        one workgroup per worker: radix select of the k-th largest
//                 key on the keys' bit patterns (exact integer compares), then
//                 masks and the ascending index list by prefix sums.
//   k_gather      the fixed tree over the workers' transmitted chunks, mean,
//                 and fused momentum SGD; a worker that did not select a chunk
//                 contributes +0 without being read.
#include "common.h"
#include "tree.h"

namespace ga {

namespace {

constexpr int kNormThreads = 256;
constexpr int kTopkThreads = 1024;
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

// Exclusive prefix sum of one value per thread, in thread order, over a
// workgroup of kTopkThreads threads.  *total receives the sum of all values.
// Every thread of the workgroup must call it.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* s_wave, int32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int32_t base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kTopkThreads / 64; ++i) {
        const int32_t t = s_wave[i];
        base += i < wave ? t : 0;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return base + x - v;
}

// One workgroup per worker.  The k-th largest order key T is found by a
// most-significant-digit radix select (8 passes of 8 bits, LDS histograms);
// the selection is then every key above T plus the lowest-index keys equal to
// T, as many as are still needed.  That is exactly the first k chunks of the
// order (key desc, index asc).  Masks and the ascending index list follow from
// two workgroup prefix sums in chunk order.
__global__ __launch_bounds__(kTopkThreads) void k_topk(const double* __restrict__ keys, int32_t n_c,
                                                       int32_t k, int32_t mw,
                                                       int32_t* __restrict__ sel_idx,
                                                       uint32_t* __restrict__ sel_mask) {
    const int32_t w = blockIdx.x;
    const int tid = threadIdx.x;
    const double* __restrict__ kw = keys + (int64_t)w * n_c;
    uint32_t* __restrict__ mrow = sel_mask + (int64_t)w * mw;
    __shared__ uint32_t hist[256];
    __shared__ uint64_t s_prefix;
    __shared__ int32_t s_kk;
    __shared__ int32_t s_wave[kTopkThreads / 64];

    if (k == 0) {  // uniform: nothing is sent
        for (int32_t i = tid; i < mw; i += kTopkThreads) mrow[i] = 0u;
        return;
    }
    int32_t* __restrict__ irow = sel_idx + (int64_t)w * k;

    uint64_t prefix = 0, pmask = 0;
    int32_t kk = k;  // rank of the wanted key among the keys that match prefix
    for (int shift = 56; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
        for (int32_t c = tid; c < n_c; c += kTopkThreads) {
            const uint64_t key = order_key(kw[c]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // Wavefront 0 finds the digit d holding the kk-th largest key:
            // lane l owns bins 4l..4l+3; a suffix sum over lanes gives the
            // count of keys in higher bins, and exactly one lane brackets kk.
            const int lane = tid;
            const int32_t h0 = (int32_t)hist[4 * lane], h1 = (int32_t)hist[4 * lane + 1];
            const int32_t h2 = (int32_t)hist[4 * lane + 2], h3 = (int32_t)hist[4 * lane + 3];
            const int32_t own = h0 + h1 + h2 + h3;
            int32_t x = own;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int32_t y = __shfl_down(x, off, 64);
                if (lane + off < 64) x += y;
            }
            const int32_t above = x - own;
            if (above < kk && kk <= x) {
                int32_t cum = above, d;
                if (cum + h3 >= kk) {
                    d = 4 * lane + 3;
                } else if ((cum += h3) + h2 >= kk) {
                    d = 4 * lane + 2;
                } else if ((cum += h2) + h1 >= kk) {
                    d = 4 * lane + 1;
                } else {
                    cum += h1;
                    d = 4 * lane;
                }
                s_prefix = prefix | ((uint64_t)d << shift);
                s_kk = kk - cum;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        kk = s_kk;
        pmask |= 0xFFull << shift;
    }
    const uint64_t T = prefix;  // k-th largest key; kk keys equal to T are taken

    // Each thread owns a run of q consecutive chunks, q a multiple of 32, so
    // every mask word has one writer.
    const int32_t q = 32 * ((n_c + 32 * kTopkThreads - 1) / (32 * kTopkThreads));
    const int32_t c0 = tid * q;
    const int32_t c1 = c0 + q < n_c ? c0 + q : n_c;
    int32_t neq = 0;
    for (int32_t c = c0; c < c1; ++c) neq += order_key(kw[c]) == T;
    int32_t total;
    const int32_t eq_base = block_exclusive_scan(neq, s_wave, &total);
    int32_t nsel = 0, e = eq_base;
    for (int32_t c = c0; c < c1; ++c) {
        const uint64_t key = order_key(kw[c]);
        nsel += (key > T) || (key == T && e < kk);
        e += key == T;
    }
    int32_t pos = block_exclusive_scan(nsel, s_wave, &total);
    e = eq_base;
    for (int32_t cw = c0; cw < c1; cw += 32) {
        uint32_t m = 0u;
        for (int32_t b = 0; b < 32 && cw + b < c1; ++b) {
            const int32_t c = cw + b;
            const uint64_t key = order_key(kw[c]);
            const bool sel = (key > T) || (key == T && e < kk);
            e += key == T;
            if (sel) {
                m |= 1u << b;
                irow[pos++] = c;
            }
        }
        mrow[cw >> 5] = m;
    }
}

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
// chunk that no worker selected skips the tree (its sum is +0).
template <int LEV>
__global__ __launch_bounds__(kGatherThreads) void k_gather_wave(
    float* __restrict__ resid, int64_t ld, int32_t W, int64_t P, int64_t C,
    const uint32_t* __restrict__ sel_mask, int32_t mw, int32_t zero_sel, float invW,
    float* __restrict__ grad, int32_t do_sgd, float lr, float mu, float* __restrict__ w,
    float* __restrict__ v) {
    constexpr int E = 4;
    const int lane = threadIdx.x & 63;
    const int64_t wave_base =
        ((int64_t)blockIdx.x * kGatherThreads + (int64_t)__builtin_amdgcn_readfirstlane(threadIdx.x & ~63u)) * E;
    if (wave_base >= P) return;  // whole wavefront past the end
    const int64_t i0 = wave_base + (int64_t)lane * E;
    const bool valid = i0 < P;
    const int32_t c = (int32_t)(wave_base / C);
    const int32_t cw = c >> 5;
    const uint32_t cb = 1u << (c & 31);

    bool any = false;
    for (int32_t g0 = 0; g0 < W; g0 += 64) {
        const bool bit = (g0 + lane < W) && (sel_mask[(int64_t)(g0 + lane) * mw + cw] & cb);
        any |= __ballot(bit) != 0ull;
    }
    float s[E] = {0.f, 0.f, 0.f, 0.f};
    if (any) {
        TreeAcc<LEV, E> tree;
        uint32_t cnt = 0;
        for (int32_t g0 = 0; g0 < W; g0 += 64) {
            const bool bit = (g0 + lane < W) && (sel_mask[(int64_t)(g0 + lane) * mw + cw] & cb);
            const uint64_t m = __ballot(bit);
            const int32_t gn = W - g0 < 64 ? W - g0 : 64;
            for (int32_t u0 = 0; u0 < gn; u0 += kGatherUnroll) {
                float4 x[kGatherUnroll];
#pragma unroll
                for (int u = 0; u < kGatherUnroll; ++u) {
                    x[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (u0 + u < gn && ((m >> (u0 + u)) & 1ull) && valid)
                        x[u] = *reinterpret_cast<const float4*>(resid + (int64_t)(g0 + u0 + u) * ld + i0);
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
    if (valid) gather_epilogue(s, i0, P, invW, grad, do_sgd != 0, lr, mu, w, v);
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
