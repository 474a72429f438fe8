// Coarse-grained sparse communication, part 1 (GradientFlow, arXiv abstract:
// only the important gradient chunks are transmitted): chunk norms over a
// packed bucket.
//
// k_chunk_norm: one workgroup (256 threads) per (worker, chunk), or per
// (worker, 2048-element part) for chunks longer than 2048 elements (the
// resident workgroups then stream one contiguous window, measured faster for
// this mixed read/write pass; the parts' sums are added per chunk afterwards,
// in part order, by the key-sum kernel).  Each thread
// takes 8-element vectors (one 128-bit binary16 load of the gradient, two of
// the binary32 residual), 4 vectors in flight; a = leaf + residual is written
// back over the residual, and the chunk's key, the sum of a^2 in binary64
// (each square is exact), is reduced in registers, then across the wavefront
// with cross-lane moves, then across the 4 wavefronts through LDS.  Traffic
// per worker-element: 2 B (binary16 gradient) + 4 B (residual read) + 4 B
// (residual write); in lazy-zero mode the residual of a chunk sent in the
// previous step is taken as zero and not read.  The per-layer-tensor form of
// this pass is the history kernel at age 0 (history.hip).
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
    for (int64_t j = threadIdx.x; j < nvec; j += UN * kNormThreads) {
        float lf[UN][8];
        float4 r0[UN], r1[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t jj = j + u * kNormThreads;
            if (jj >= nvec) continue;
            const int64_t i = ss + (jj << 3);
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
            const int64_t jj = j + u * kNormThreads;
            if (jj >= nvec) continue;
            const int64_t i = ss + (jj << 3);
            float4 a0, a1;
            a0.x = lf[u][0] + r0[u].x; a0.y = lf[u][1] + r0[u].y;
            a0.z = lf[u][2] + r0[u].z; a0.w = lf[u][3] + r0[u].w;
            a1.x = lf[u][4] + r1[u].x; a1.y = lf[u][5] + r1[u].y;
            a1.z = lf[u][6] + r1[u].z; a1.w = lf[u][7] + r1[u].w;
            if (STORE && rzero) {
                // a residual taken as zero was not read: non-temporal stores
                __builtin_nontemporal_store(f32x4{a0.x, a0.y, a0.z, a0.w}, reinterpret_cast<f32x4*>(r + i));
                __builtin_nontemporal_store(f32x4{a1.x, a1.y, a1.z, a1.w}, reinterpret_cast<f32x4*>(r + i + 4));
            } else if (STORE) {
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
    for (int64_t i = ss + (nvec << 3) + threadIdx.x; i < se; i += kNormThreads) {
        const float lf = FP16 ? widen1(static_cast<gptr<uint16_t>>(src)[i - soff])
                              : static_cast<gptr<float>>(src)[i - soff];
        const float a = lf + (rzero ? 0.f : r[i]);
        if (STORE) r[i] = a;
        acc0 = fma((double)a, (double)a, acc0);
    }
}

// One workgroup per (worker w = blockIdx.y, part q of chunk c: blockIdx.x =
// c * S + q, the whole chunk when S == 1); the gradient is row w of the flat
// [W][ld] bucket.  The sum of squares goes to keys[w][c] (S == 1) or to
// part_keys[w][c][q].
template <bool FP16, bool LAZY>
__global__ __launch_bounds__(kNormThreads) void k_chunk_norm(const void* __restrict__ bucket,
                                                             float* __restrict__ resid, int64_t ld, int64_t P,
                                                             int64_t C, const uint32_t* __restrict__ prev_mask,
                                                             int32_t mw, int64_t n_c, int32_t S,
                                                             double* __restrict__ keys,
                                                             double* __restrict__ part_keys) {
    const int32_t w = (int32_t)blockIdx.y;
    const int32_t c = (int32_t)(blockIdx.x / (uint32_t)S);
    const int32_t q = (int32_t)(blockIdx.x - (uint32_t)c * (uint32_t)S);
    const int64_t cs = (int64_t)c * C;
    const int64_t ce = cs + C < P ? cs + C : P;
    const int64_t s = S == 1 ? cs : cs + (int64_t)q * kNormPart;
    const int64_t e = S == 1 ? ce : (s + kNormPart < ce ? s + kNormPart : ce);   // e <= s: an empty part
    const bool rzero = LAZY && ((prev_mask[(int64_t)w * mw + (c >> 5)] >> (c & 31)) & 1u);
    float* __restrict__ r = resid + (int64_t)w * ld;
    double acc0 = 0.0, acc1 = 0.0;
    const uint64_t row = reinterpret_cast<uint64_t>(bucket) + (uint64_t)(w * ld * (FP16 ? 2 : 4));
    if (s < e) norm_segment<FP16>(as_global<void>(row), 0, true, r, s, e, rzero, acc0, acc1);

    double t = wave_sum(acc0 + acc1);
    __shared__ double part[kNormThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) part[wave] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        double k = part[0];
#pragma unroll
        for (int j = 1; j < kNormThreads / 64; ++j) k += part[j];
        if (S == 1) keys[(int64_t)w * n_c + c] = k;
        else part_keys[((int64_t)w * n_c + c) * S + q] = k;
    }
}

}  // namespace

hipError_t launch_chunk_norm(const Plan& p, const void* bucket, float* resid, const uint32_t* prev_mask,
                             double* keys, double* part_keys, hipStream_t s) {
    // a 2-D grid: W * n_c workgroups would exceed the 32-bit work-item count
    // of a 1-D dispatch at the plan limits
    if (p.W == 0 || p.n_c == 0) return hipSuccess;
    const int32_t S = p.key_parts;
    const dim3 grid((unsigned)(p.n_c * S), (unsigned)p.W);
#define GA_NORM_LAUNCH(F, Z)                                                                                 \
    hipLaunchKernelGGL((k_chunk_norm<F, Z>), grid, dim3(kNormThreads), 0, s, bucket, resid, p.ld, p.P, p.C, \
                       prev_mask, p.mw, p.n_c, S, keys, part_keys)
    const bool f16 = p.dtype == GA_FP16;
    if (f16 && prev_mask) GA_NORM_LAUNCH(true, true);
    else if (f16) GA_NORM_LAUNCH(true, false);
    else if (prev_mask) GA_NORM_LAUNCH(false, true);
    else GA_NORM_LAUNCH(false, false);
#undef GA_NORM_LAUNCH
    if (S > 1) return launch_key_parts(p, part_keys, keys, s);
    return hipGetLastError();
}

}  // namespace ga
