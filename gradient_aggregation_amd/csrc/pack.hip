// Lazy-allreduce fusion (GradientFlow, arXiv abstract: many communication
// operations are fused into one): every worker's per-layer gradient tensors are
// copied into one flat row of the bucket, all W*L tensors in a single launch.
//
// Grid: x = tiles of a row (kTile elements), y = worker.  A workgroup finds the
// layers that overlap its tile in the offsets table (uniform binary search)
// and copies each overlap with 128-bit accesses when the layer tensor and its
// place in the row are both 16-byte aligned, element by element otherwise.
// Row padding (elements P..ld-1) is written with zeros.
#include "device.h"
#include "plan.h"

namespace ga {

namespace {

constexpr int kThreads = 256;
constexpr int kVecBytes = 16;
// 4 KiB per workgroup, one 128-bit vector per thread: the resident workgroups
// then copy one narrow window of the row (measured 6.1 TB/s on the AlexNet
// W=128 tensors, against 5.4-5.6 TB/s with 16 KiB tiles of four vectors per
// thread, or with 8 KiB)
constexpr int kTileBytes = kThreads * kVecBytes;

template <typename T>
__global__ __launch_bounds__(kThreads) void k_pack(const uint64_t* __restrict__ layer_ptrs,
                                                   const int64_t* __restrict__ offsets, int32_t L,
                                                   int64_t ld, T* __restrict__ bucket) {
    constexpr int V = kVecBytes / sizeof(T);
    constexpr int64_t kTile = kTileBytes / sizeof(T);
    const int32_t w = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * kTile;
    const int64_t e1 = e0 + kTile < ld ? e0 + kTile : ld;
    const int64_t P = offsets[L];
    T* __restrict__ row = bucket + (int64_t)w * ld;

    // First layer whose end is past e0.
    int32_t lo = 0, hi = L;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (offsets[mid + 1] <= e0) lo = mid + 1;
        else hi = mid;
    }
    for (int32_t l = lo; l < L && offsets[l] < e1; ++l) {
        const int64_t off = offsets[l];
        const int64_t s = off > e0 ? off : e0;
        const int64_t t = offsets[l + 1] < e1 ? offsets[l + 1] : e1;
        const uint64_t addr = layer_ptrs[(int64_t)w * L + l];
        gptr<T> __restrict__ src = as_global<T>(addr);  // element i of the row is src[i - off]
        const bool vec = (off % V) == 0 && (addr % kVecBytes) == 0;
        if (vec) {
            // s is a multiple of V here (e0 and off both are).
            const int64_t nv = (t - s) / V;
            for (int64_t j = threadIdx.x; j < nv; j += kThreads) {
                const int64_t i = s + j * V;
                *reinterpret_cast<uint4*>(row + i) = load_u4(src + (i - off));
            }
            for (int64_t i = s + nv * V + threadIdx.x; i < t; i += kThreads) row[i] = src[i - off];
        } else {
            for (int64_t i = s + threadIdx.x; i < t; i += kThreads) row[i] = src[i - off];
        }
    }
    for (int64_t i = (P > e0 ? P : e0) + threadIdx.x; i < e1; i += kThreads) row[i] = T(0);
}

}  // namespace

hipError_t launch_pack(const Plan& p, const uint64_t* layer_ptrs, void* bucket, hipStream_t s) {
    const int64_t elem = p.dtype == GA_FP16 ? 2 : 4;
    const int64_t tile = kTileBytes / elem;
    const unsigned gx = (unsigned)((p.ld + tile - 1) / tile);
    if (gx == 0) return hipSuccess;
    if (p.dtype == GA_FP16)
        hipLaunchKernelGGL(k_pack<uint16_t>, dim3(gx, (unsigned)p.W), dim3(kThreads), 0, s, layer_ptrs,
                           p.d_offsets, p.L, p.ld, static_cast<uint16_t*>(bucket));
    else
        hipLaunchKernelGGL(k_pack<uint32_t>, dim3(gx, (unsigned)p.W), dim3(kThreads), 0, s, layer_ptrs,
                           p.d_offsets, p.L, p.ld, static_cast<uint32_t*>(bucket));
    return hipGetLastError();
}

}  // namespace ga
