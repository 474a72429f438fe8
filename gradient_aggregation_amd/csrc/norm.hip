// Coarse-grained sparse communication, part 1 (GradientFlow, arXiv abstract:
// only the important gradient chunks are transmitted): chunk norms.
//
// k_chunk_norm: one workgroup (256 threads) per (worker, chunk).  The
// gradient comes from the flat bucket, or (zero-copy lazy-allreduce fusion)
// straight from the workers' per-layer tensors through the layer table.  Each thread
// takes 8-element vectors (one 128-bit binary16 load of the gradient, two of
// the binary32 residual), 4 vectors in flight; a = leaf + residual is written
// back over the residual, and the chunk's key, the sum of a^2 in binary64
// (each square is exact), is reduced in registers, then across the wavefront
// with cross-lane moves, then across the 4 wavefronts through LDS.  Traffic
// per worker-element: 2 B (binary16 gradient) + 4 B (residual read) + 4 B
// (residual write); in lazy-zero mode the residual of a chunk sent in the
// previous step is taken as zero and not read.  In the pending form the residual of a
// chunk sent two steps ago but not in the previous step is still held as the
// previous step's gradient (it was that gradient plus +0) and is read from
// those tensors: 2 B per binary16 element instead of 4.  In the depth-2
// pending form such a chunk does not store its a either (the later passes
// recompute it from the two gradients), and a chunk sent three steps ago and
// not since reads its residual from the previous two steps' gradients.
#include "device.h"
#include "plan.h"

namespace ga {

namespace {

constexpr int kNormThreads = 256;

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// ---------------------------------------------------------------------------
// k_chunk_norm
// ---------------------------------------------------------------------------

// Gradient elements j .. j+7 (one 16-byte aligned vector), or element j, of
// the tensor src, widened to binary32.
template <bool FP16>
__device__ __forceinline__ void load8(gptr<void> src, int64_t j, float (&f)[8]) {
    if (FP16) {
        widen8(load_u4(static_cast<gptr<uint16_t>>(src) + j), f);
    } else {
        gptr<float> gp = static_cast<gptr<float>>(src) + j;
        const float4 g0 = load_f4(gp), g1 = load_f4(gp + 4);
        f[0] = g0.x; f[1] = g0.y; f[2] = g0.z; f[3] = g0.w;
        f[4] = g1.x; f[5] = g1.y; f[6] = g1.z; f[7] = g1.w;
    }
}

template <bool FP16>
__device__ __forceinline__ float load1(gptr<void> src, int64_t j) {
    return FP16 ? widen1(static_cast<gptr<uint16_t>>(src)[j]) : static_cast<gptr<float>>(src)[j];
}

// Flat elements [ss, se) of one worker: gradient element i is src[i - soff]
// (src typed by FP16), residual element i is r[i].  With vec_ok, ss is a
// multiple of 8 and src + (ss - soff) is 16-byte aligned, so the body runs on
// 8-element vectors; the rest goes element by element.
template <bool FP16, bool STORE = true>
__device__ __forceinline__ void norm_segment(gptr<void> __restrict__ src, int64_t soff, bool vec_ok,
                                             float* __restrict__ r, int64_t ss, int64_t se, bool rzero,
                                             double& acc0, double& acc1) {
    constexpr int UN = 4;
    const int64_t nvec = vec_ok ? (se - ss) >> 3 : 0;
    int64_t j = threadIdx.x;
    for (; j + (UN - 1) * kNormThreads < nvec; j += UN * kNormThreads) {
        float lf[UN][8];
        float4 r0[UN], r1[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t i = ss + ((j + u * kNormThreads) << 3);
            if (FP16) {
                widen8(load_u4(static_cast<gptr<uint16_t>>(src) + (i - soff)), lf[u]);
            } else {
                gptr<float> gp = static_cast<gptr<float>>(src) + (i - soff);
                const float4 g0 = load_f4(gp);
                const float4 g1 = load_f4(gp + 4);
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
            const int64_t i = ss + ((j + u * kNormThreads) << 3);
            float4 a0, a1;
            a0.x = lf[u][0] + r0[u].x; a0.y = lf[u][1] + r0[u].y;
            a0.z = lf[u][2] + r0[u].z; a0.w = lf[u][3] + r0[u].w;
            a1.x = lf[u][4] + r1[u].x; a1.y = lf[u][5] + r1[u].y;
            a1.z = lf[u][6] + r1[u].z; a1.w = lf[u][7] + r1[u].w;
            if (STORE) {
                *reinterpret_cast<float4*>(r + i) = a0;
                *reinterpret_cast<float4*>(r + i + 4) = a1;
            }
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
        const int64_t i = ss + (j << 3);
        float lf[8];
        if (FP16) {
            widen8(load_u4(static_cast<gptr<uint16_t>>(src) + (i - soff)), lf);
        } else {
            gptr<float> gp = static_cast<gptr<float>>(src) + (i - soff);
#pragma unroll
            for (int q = 0; q < 8; ++q) lf[q] = gp[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float a = lf[q] + (rzero ? 0.f : r[i + q]);
            if (STORE) r[i + q] = a;
            acc0 = fma((double)a, (double)a, acc0);
        }
    }
    for (int64_t i = ss + (nvec << 3) + threadIdx.x; i < se; i += kNormThreads) {
        const float lf = FP16 ? widen1(static_cast<gptr<uint16_t>>(src)[i - soff])
                              : static_cast<gptr<float>>(src)[i - soff];
        const float a = lf + (rzero ? 0.f : r[i]);
        if (STORE) r[i] = a;
        acc0 = fma((double)a, (double)a, acc0);
    }
}

// Flat elements [ss, se) of one worker whose residual is pending, that is,
// still held as the gradients of the steps since the chunk was last sent
// (its residual was zero then): with NP = 1 the previous step's gradient p1
// (residual = p1 + 0), with NP = 2 the previous two, p1 the later
// (residual = p1 + (p2 + 0)), read at the same offsets as the gradient src.
// a = leaf + residual is stored if STORE.  With vec_ok, all the tensors are
// 16-byte aligned at ss.
template <bool FP16, int NP, bool STORE>
__device__ __forceinline__ void norm_segment_pending(gptr<void> __restrict__ src, gptr<void> __restrict__ p1,
                                                     gptr<void> __restrict__ p2, int64_t soff, bool vec_ok,
                                                     float* __restrict__ r, int64_t ss, int64_t se, double& acc0,
                                                     double& acc1) {
    constexpr int UN = NP == 1 ? 4 : 2;
    const int64_t nvec = vec_ok ? (se - ss) >> 3 : 0;
    int64_t j = threadIdx.x;
    for (; j < nvec; j += UN * kNormThreads) {
        float lf[UN][8], rv[UN][8];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            if (j + u * kNormThreads >= nvec) continue;
            const int64_t i = ss + ((j + u * kNormThreads) << 3);
            float q1[8], q2[8];
            load8<FP16>(src, i - soff, lf[u]);
            load8<FP16>(p1, i - soff, q1);
            if (NP == 2) load8<FP16>(p2, i - soff, q2);
#pragma unroll
            for (int q = 0; q < 8; ++q) rv[u][q] = NP == 2 ? q1[q] + (q2[q] + 0.f) : q1[q] + 0.f;
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            if (j + u * kNormThreads >= nvec) continue;
            const int64_t i = ss + ((j + u * kNormThreads) << 3);
            float a[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                a[q] = lf[u][q] + rv[u][q];
                if (q & 1) acc1 = fma((double)a[q], (double)a[q], acc1);
                else acc0 = fma((double)a[q], (double)a[q], acc0);
            }
            if (STORE) {
                *reinterpret_cast<float4*>(r + i) = make_float4(a[0], a[1], a[2], a[3]);
                *reinterpret_cast<float4*>(r + i + 4) = make_float4(a[4], a[5], a[6], a[7]);
            }
        }
    }
    for (int64_t i = ss + (nvec << 3) + threadIdx.x; i < se; i += kNormThreads) {
        const float lf = load1<FP16>(src, i - soff);
        const float q1 = load1<FP16>(p1, i - soff);
        const float rv = NP == 2 ? q1 + (load1<FP16>(p2, i - soff) + 0.f) : q1 + 0.f;
        const float a = lf + rv;
        if (STORE) r[i] = a;
        acc0 = fma((double)a, (double)a, acc0);
    }
}

// One workgroup per (worker w = blockIdx.y, chunk c = blockIdx.x).  LAYERS: the gradient is read from
// the W*L per-layer tensors of the layer table (zero-copy fusion: the chunk's
// elements are gathered from the layers it overlaps); otherwise from the
// flat [W][ld] bucket.
// DEFER (lazy mode, layer tensors only): a chunk sent in the previous step
// computes its key but does not store a, which is the widened gradient; the
// deferred gather reads the gradient for it instead, and writes it as the
// residual if the chunk is not sent again.
// DEPTH >= 1 (with DEFER, the pending forms): a chunk set in prev2_mask
// (sent two steps ago) but not in prev_mask has the previous step's gradient
// + 0 as its residual, read from prev_layer_ptrs (the previous step's layer
// table) instead of resid; with DEPTH 1 its a is stored, with DEPTH 2 it is
// not.  DEPTH 2: a chunk set in prev3_mask (sent three steps ago) and in
// neither prev2_mask nor prev_mask has the residual g1 + (g2 + 0), g1 and g2
// read from prev_layer_ptrs and prev2_layer_ptrs (two steps back); its a is
// stored.
template <bool FP16, bool LAZY, bool LAYERS, bool DEFER = false, int DEPTH = 0>
__global__ __launch_bounds__(kNormThreads) void k_chunk_norm(
    const void* __restrict__ bucket, const uint64_t* __restrict__ layer_ptrs,
    const int64_t* __restrict__ offsets, int32_t L, float* __restrict__ resid, int64_t ld, int64_t P,
    int64_t C, int32_t n_c, const uint32_t* __restrict__ prev_mask, int32_t mw, double* __restrict__ keys,
    const uint64_t* __restrict__ prev_layer_ptrs, const uint32_t* __restrict__ prev2_mask,
    const uint64_t* __restrict__ prev2_layer_ptrs, const uint32_t* __restrict__ prev3_mask) {
    const int32_t w = (int32_t)blockIdx.y;
    const int32_t c = (int32_t)blockIdx.x;
    const int64_t b = (int64_t)w * n_c + c;
    const int64_t s = (int64_t)c * C;
    const int64_t e = s + C < P ? s + C : P;
    bool rzero = false;
    if (LAZY) rzero = (prev_mask[(int64_t)w * mw + (c >> 5)] >> (c & 31)) & 1u;
    bool pend = false, pend2 = false;
    if (DEPTH >= 1 && !rzero) pend = (prev2_mask[(int64_t)w * mw + (c >> 5)] >> (c & 31)) & 1u;
    if (DEPTH >= 2 && !rzero && !pend) pend2 = (prev3_mask[(int64_t)w * mw + (c >> 5)] >> (c & 31)) & 1u;

    float* __restrict__ r = resid + (int64_t)w * ld;
    double acc0 = 0.0, acc1 = 0.0;
    if (LAYERS) {
        // first layer ending after s (uniform binary search)
        int32_t lo = 0, hi = L;
        while (lo < hi) {
            const int32_t mid = (lo + hi) >> 1;
            if (offsets[mid + 1] <= s) lo = mid + 1;
            else hi = mid;
        }
        for (int32_t l = lo; l < L && offsets[l] < e; ++l) {
            const int64_t off = offsets[l], end = offsets[l + 1];
            const uint64_t addr = layer_ptrs[(int64_t)w * L + l];
            const bool vec_ok = (off & 7) == 0 && (addr & 15) == 0;
            if (DEFER && rzero) {
                norm_segment<FP16, false>(as_global<void>(addr), off, vec_ok, r, off > s ? off : s,
                                          end < e ? end : e, rzero, acc0, acc1);
            } else if (DEPTH >= 1 && pend) {
                const uint64_t a1 = prev_layer_ptrs[(int64_t)w * L + l];
                norm_segment_pending<FP16, 1, DEPTH == 1>(as_global<void>(addr), as_global<void>(a1),
                                                          as_global<void>(a1), off, vec_ok && (a1 & 15) == 0, r,
                                                          off > s ? off : s, end < e ? end : e, acc0, acc1);
            } else if (DEPTH >= 2 && pend2) {
                const uint64_t a1 = prev_layer_ptrs[(int64_t)w * L + l];
                const uint64_t a2 = prev2_layer_ptrs[(int64_t)w * L + l];
                norm_segment_pending<FP16, 2, true>(as_global<void>(addr), as_global<void>(a1),
                                                    as_global<void>(a2), off,
                                                    vec_ok && (a1 & 15) == 0 && (a2 & 15) == 0, r,
                                                    off > s ? off : s, end < e ? end : e, acc0, acc1);
            } else
                norm_segment<FP16>(as_global<void>(addr), off, vec_ok, r, off > s ? off : s, end < e ? end : e,
                                   rzero, acc0, acc1);
        }
    } else {
        const uint64_t row = reinterpret_cast<uint64_t>(bucket) + (uint64_t)(w * ld * (FP16 ? 2 : 4));
        norm_segment<FP16>(as_global<void>(row), 0, true, r, s, e, rzero, acc0, acc1);
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

template <bool LAYERS, bool DEFER = false, int DEPTH = 0>
hipError_t norm_dispatch(const Plan& p, const void* bucket, const uint64_t* layer_ptrs, float* resid,
                         const uint32_t* prev_mask, double* keys, hipStream_t s,
                         const uint64_t* prev_layer_ptrs = nullptr, const uint32_t* prev2_mask = nullptr,
                         const uint64_t* prev2_layer_ptrs = nullptr, const uint32_t* prev3_mask = nullptr) {
    // a 2-D grid: W * n_c workgroups would exceed the 32-bit work-item count
    // of a 1-D dispatch at the plan limits
    if (p.W == 0 || p.n_c == 0) return hipSuccess;
    const bool f16 = p.dtype == GA_FP16;
    const int32_t n_c = (int32_t)p.n_c;
#define GA_NORM_LAUNCH(F, Z)                                                                               \
    hipLaunchKernelGGL((k_chunk_norm<F, Z, LAYERS, DEFER && Z, Z ? DEPTH : 0>),                           \
                       dim3((unsigned)p.n_c, (unsigned)p.W), dim3(kNormThreads), 0, s, bucket, layer_ptrs,     \
                       p.d_offsets, p.L, resid, p.ld, p.P, p.C, n_c, prev_mask, p.mw, keys, prev_layer_ptrs,  \
                       prev2_mask, prev2_layer_ptrs, prev3_mask)
    if (f16 && prev_mask) GA_NORM_LAUNCH(true, true);
    else if (f16) GA_NORM_LAUNCH(true, false);
    else if (prev_mask) GA_NORM_LAUNCH(false, true);
    else GA_NORM_LAUNCH(false, false);
#undef GA_NORM_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_norm(const Plan& p, const void* bucket, float* resid, const uint32_t* prev_mask,
                             double* keys, hipStream_t s) {
    return norm_dispatch<false>(p, bucket, nullptr, resid, prev_mask, keys, s);
}

hipError_t launch_chunk_norm_layers(const Plan& p, const uint64_t* layer_ptrs, float* resid,
                                    const uint32_t* prev_mask, double* keys, hipStream_t s) {
    return norm_dispatch<true>(p, nullptr, layer_ptrs, resid, prev_mask, keys, s);
}

hipError_t launch_chunk_norm_layers_defer(const Plan& p, const uint64_t* layer_ptrs, float* resid,
                                          const uint32_t* prev_mask, double* keys, hipStream_t s) {
    return norm_dispatch<true, true>(p, nullptr, layer_ptrs, resid, prev_mask, keys, s);
}

hipError_t launch_chunk_norm_layers_pending(const Plan& p, const uint64_t* layer_ptrs,
                                            const uint64_t* prev_layer_ptrs, float* resid,
                                            const uint32_t* prev_mask, const uint32_t* prev2_mask, double* keys,
                                            hipStream_t s) {
    return norm_dispatch<true, true, 1>(p, nullptr, layer_ptrs, resid, prev_mask, keys, s, prev_layer_ptrs,
                                        prev2_mask);
}

hipError_t launch_chunk_norm_layers_pending2(const Plan& p, const uint64_t* layer_ptrs,
                                             const uint64_t* prev_layer_ptrs, const uint64_t* prev2_layer_ptrs,
                                             float* resid, const uint32_t* prev_mask, const uint32_t* prev2_mask,
                                             const uint32_t* prev3_mask, double* keys, hipStream_t s) {
    return norm_dispatch<true, true, 2>(p, nullptr, layer_ptrs, resid, prev_mask, keys, s, prev_layer_ptrs,
                                        prev2_mask, prev2_layer_ptrs, prev3_mask);
}

}  // namespace ga
