// Coarse-grained sparse communication, part 1 (GradientFlow, arXiv abstract:
// only the important gradient chunks are transmitted): chunk norms.
//
// k_chunk_norm: one workgroup (256 threads) per (worker, chunk).  Each thread
// takes 8-element vectors (one 128-bit binary16 load of the gradient, two of
// the binary32 residual), 4 vectors in flight; a = leaf + residual is written
// back over the residual, and the chunk's key, the sum of a^2 in binary64
// (each square is exact), is reduced in registers, then across the wavefront
// with cross-lane moves, then across the 4 wavefronts through LDS.  Traffic
// per worker-element: 2 B (binary16 gradient) + 4 B (residual read) + 4 B
// (residual write); in lazy-zero mode the residual of a chunk sent in the
// previous step is taken as zero and not read.
#include "common.h"

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

}  // namespace ga
