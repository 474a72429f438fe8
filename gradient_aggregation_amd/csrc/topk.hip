// Coarse-grained sparse communication, part 2: top-k chunk selection.
//
// k_topk: one workgroup (1024 threads) per worker.  The k-th largest key is
// found by a most-significant-digit radix select on the keys' bit patterns
// (exact integer compares), then masks and the ascending index list follow
// from workgroup prefix sums in chunk order.
#include "device.h"
#include "plan.h"

namespace ga {

namespace {

constexpr int kTopkThreads = 1024;

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

}  // namespace

hipError_t launch_topk(const Plan& p, const double* keys, int32_t* sel_idx, uint32_t* sel_mask,
                       hipStream_t s) {
    if (p.W == 0 || p.n_c == 0) return hipSuccess;
    hipLaunchKernelGGL(k_topk, dim3((unsigned)p.W), dim3(kTopkThreads), 0, s, keys, (int32_t)p.n_c, p.k,
                       p.mw, sel_idx, sel_mask);
    return hipGetLastError();
}

}  // namespace ga
