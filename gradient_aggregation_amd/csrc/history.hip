// Coarse-grained sparse communication with a deferred residual (GradientFlow,
// arXiv abstract: only the important gradient chunks are transmitted; the rest
// stay in each worker's residual and are added to its next gradient).
//
// The residual recurrence is a_t = leaf_t + r_{t-1}; r_t = 0 on the chunks a
// worker sends at step t and a_t elsewhere.  Writing r every step costs 4 bytes
// per worker-element on top of reading it, and HBM streams mixed reads and
// writes far slower than reads alone.  So the buffer R is written only on the
// steps the caller marks as storing (and by a flush).  Between two writes, the
// residual of each (worker, chunk) is re-formed from what the caller still
// holds: R (written `age` steps before the previous step), the selection
// masks of the steps since then, and their gradient tensors.  If the chunk was
// sent j steps before this one (the latest such step, j <= age), r_{t-1} is the
// j gradients since then added onto +0; otherwise it is the `age` gradients
// since R was written added onto R; newest outermost:
//   a_t = g_t + (g_{t-1} + (... + (g_{t-n} + base))),  base = +0 or R.
// These are the recurrence's own operations in its own order, so every a is
// the one the plain recurrence computes, bit for bit.
//
//   k_norm_hist    one workgroup per (worker, chunk): forms a, its key
//                  (binary64 sum of squares) and, on a storing step, writes a
//                  into R; as the flush, writes the residual itself (zero on
//                  the chunks sent this step).
//   k_gather_hist  one wavefront per 256 elements of one chunk: the fixed
//                  binary tree over the workers' sent values (absent workers
//                  are +0), the mean and the fused momentum-SGD update.  A sent
//                  value is read from R on a storing step, else re-formed as
//                  above.
//
// With age 0 and a store every step this is the lazy-zero form of the
// residual: the selection mask of the previous step stands for the zeroing.
#include "device.h"
#include "plan.h"
#include "tree.h"

namespace ga {

namespace {

constexpr int kNormThreads = 256;
constexpr int kGatherThreads = 256;

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// A 128-bit non-temporal load of four binary32 values (16-byte aligned).
__device__ __forceinline__ float4 load_f4_nt(const float* p) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ bool mask_bit(const uint32_t* __restrict__ m, int64_t w, int32_t mw, int32_t c) {
    return (m[w * mw + (c >> 5)] >> (c & 31)) & 1u;
}

// Eight gradient elements at element j of tensor src (16-byte aligned there), widened.
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

// a = x0 + (x1 + (x2 + base)) with the NP gradients after x0 (NP = 0: a = x0 + base).
template <int NP>
__device__ __forceinline__ float reform(float x0, float x1, float x2, float base) {
    float acc = base;
    if (NP >= 2) acc = x2 + acc;
    if (NP >= 1) acc = x1 + acc;
    return x0 + acc;
}

// ---------------------------------------------------------------------------
// k_norm_hist
// ---------------------------------------------------------------------------

// Elements [ss, se) of one worker, whose gradient element i is g0[i - soff]
// (this step), g1[i - soff] (one step back) and g2[i - soff] (two steps back),
// the tensors of one layer.  NP: how many earlier gradients the residual
// holds; BUF: its base is R (else +0); ST: a is written into R.  With vec_ok,
// ss is a multiple of 8 and every tensor used is 16-byte aligned at ss.
template <bool FP16, int NP, bool BUF, bool ST>
__device__ __forceinline__ void norm_seg(gptr<void> g0, gptr<void> g1, gptr<void> g2, int64_t soff, bool vec_ok,
                                         float* __restrict__ r, int64_t ss, int64_t se, double& acc0,
                                         double& acc1) {
    constexpr int UN = NP >= 2 ? 2 : 4;   // vectors in flight per thread
    const int64_t nvec = vec_ok ? (se - ss) >> 3 : 0;
    int64_t j = threadIdx.x;
    for (; j < nvec; j += UN * kNormThreads) {
        float x0[UN][8], x1[UN][8], x2[UN][8], rb[UN][8];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t jj = j + u * kNormThreads;
            if (jj >= nvec) continue;
            const int64_t i = ss + (jj << 3);
            load8<FP16>(g0, i - soff, x0[u]);
            if (NP >= 1) load8<FP16>(g1, i - soff, x1[u]);
            if (NP >= 2) load8<FP16>(g2, i - soff, x2[u]);
            if (BUF) {
                const float4 r0 = *reinterpret_cast<const float4*>(r + i);
                const float4 r1 = *reinterpret_cast<const float4*>(r + i + 4);
                rb[u][0] = r0.x; rb[u][1] = r0.y; rb[u][2] = r0.z; rb[u][3] = r0.w;
                rb[u][4] = r1.x; rb[u][5] = r1.y; rb[u][6] = r1.z; rb[u][7] = r1.w;
            }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t jj = j + u * kNormThreads;
            if (jj >= nvec) continue;
            const int64_t i = ss + (jj << 3);
            float a[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                a[q] = reform<NP>(x0[u][q], NP >= 1 ? x1[u][q] : 0.f, NP >= 2 ? x2[u][q] : 0.f,
                                  BUF ? rb[u][q] : 0.f);
                if (q & 1) acc1 = fma((double)a[q], (double)a[q], acc1);
                else acc0 = fma((double)a[q], (double)a[q], acc0);
            }
            if (ST) {
                *reinterpret_cast<float4*>(r + i) = make_float4(a[0], a[1], a[2], a[3]);
                *reinterpret_cast<float4*>(r + i + 4) = make_float4(a[4], a[5], a[6], a[7]);
            }
        }
    }
    for (int64_t i = ss + (nvec << 3) + threadIdx.x; i < se; i += kNormThreads) {
        const float a = reform<NP>(load1<FP16>(g0, i - soff), NP >= 1 ? load1<FP16>(g1, i - soff) : 0.f,
                                   NP >= 2 ? load1<FP16>(g2, i - soff) : 0.f, BUF ? r[i] : 0.f);
        if (ST) r[i] = a;
        acc0 = fma((double)a, (double)a, acc0);
    }
}

// Walk the layers that chunk [s, e) of worker w overlaps.
template <bool FP16, int NP, bool BUF, bool ST>
__device__ __forceinline__ void norm_walk(const HistArgs& h, const int64_t* __restrict__ offsets, int32_t L,
                                          int32_t w, float* __restrict__ r, int64_t s, int64_t e, double& acc0,
                                          double& acc1) {
    int32_t lo = 0, hi = L;   // first layer ending after s (uniform binary search)
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (offsets[mid + 1] <= s) lo = mid + 1;
        else hi = mid;
    }
    for (int32_t l = lo; l < L && offsets[l] < e; ++l) {
        const int64_t off = offsets[l], end = offsets[l + 1];
        const int64_t slot = (int64_t)w * L + l;
        const uint64_t a0 = h.layers[0][slot];
        const uint64_t a1 = NP >= 1 ? h.layers[1][slot] : 0ull;
        const uint64_t a2 = NP >= 2 ? h.layers[2][slot] : 0ull;
        const bool vec_ok = (off & 7) == 0 && ((a0 | a1 | a2) & 15) == 0;
        norm_seg<FP16, NP, BUF, ST>(as_global<void>(a0), as_global<void>(a1), as_global<void>(a2), off, vec_ok, r,
                                    off > s ? off : s, end < e ? end : e, acc0, acc1);
    }
}

// One workgroup per (worker w = blockIdx.y, chunk c = blockIdx.x).
// STORE: a storing step.  FLUSH: write the residual after this step instead
// of keys: zero on the chunks set in sel, and, unless this step stored (then
// R already holds a), a elsewhere.
template <bool FP16, int AGE, bool STORE, bool FLUSH>
__global__ __launch_bounds__(kNormThreads) void k_norm_hist(HistArgs h, const int64_t* __restrict__ offsets,
                                                            int32_t L, float* __restrict__ resid, int64_t ld,
                                                            int64_t P, int64_t C, int32_t mw,
                                                            double* __restrict__ keys,
                                                            const uint32_t* __restrict__ sel, int32_t stored) {
    const int32_t w = (int32_t)blockIdx.y;
    const int32_t c = (int32_t)blockIdx.x;
    const int64_t s = (int64_t)c * C;
    const int64_t e = s + C < P ? s + C : P;
    float* __restrict__ r = resid + (int64_t)w * ld;
    if (FLUSH) {
        if (mask_bit(sel, w, mw, c)) {
            for (int64_t i = s + threadIdx.x; i < e; i += kNormThreads) r[i] = 0.f;
            return;
        }
        if (stored) return;
    }
    // the residual's case: sent j steps back (n = j, base +0), else n = age on R
    int32_t n = h.age;
    bool zero = false;
#pragma unroll
    for (int j = 0; j <= AGE; ++j)
        if (!zero && j <= h.age && h.masks[j] != nullptr && mask_bit(h.masks[j], w, mw, c)) {
            n = j;
            zero = true;
        }
    constexpr bool ST = STORE || FLUSH;
    double acc0 = 0.0, acc1 = 0.0;
    if (zero) {
        if (n == 0) norm_walk<FP16, 0, false, ST>(h, offsets, L, w, r, s, e, acc0, acc1);
        if constexpr (AGE >= 1)
            if (n == 1) norm_walk<FP16, 1, false, ST>(h, offsets, L, w, r, s, e, acc0, acc1);
        if constexpr (AGE >= 2)
            if (n == 2) norm_walk<FP16, 2, false, ST>(h, offsets, L, w, r, s, e, acc0, acc1);
    } else {
        if (n == 0) norm_walk<FP16, 0, true, ST>(h, offsets, L, w, r, s, e, acc0, acc1);
        if constexpr (AGE >= 1)
            if (n == 1) norm_walk<FP16, 1, true, ST>(h, offsets, L, w, r, s, e, acc0, acc1);
        if constexpr (AGE >= 2)
            if (n == 2) norm_walk<FP16, 2, true, ST>(h, offsets, L, w, r, s, e, acc0, acc1);
    }
    if (FLUSH) return;
    const double t = wave_sum(acc0 + acc1);
    __shared__ double part[kNormThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) part[wave] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        double k = part[0];
#pragma unroll
        for (int q = 1; q < kNormThreads / 64; ++q) k += part[q];
        keys[(int64_t)w * gridDim.x + c] = k;
    }
}

template <bool FP16, int AGE>
hipError_t norm_launch(const Plan& p, const HistArgs& h, bool store, bool flush, float* resid, double* keys,
                       const uint32_t* sel, bool stored, hipStream_t s) {
    const dim3 grid((unsigned)p.n_c, (unsigned)p.W);
#define GA_NH(ST, FL)                                                                                      \
    hipLaunchKernelGGL((k_norm_hist<FP16, AGE, ST, FL>), grid, dim3(kNormThreads), 0, s, h, p.d_offsets, p.L, \
                       resid, p.ld, p.P, p.C, p.mw, keys, sel, stored ? 1 : 0)
    if (flush) GA_NH(false, true);
    else if (store) GA_NH(true, false);
    else GA_NH(false, false);
#undef GA_NH
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// k_gather_hist
// ---------------------------------------------------------------------------

// Four elements of worker wk's gradient at i0 (i0 % 4 == 0) through a layer
// table, element by element (zero past P): for tensors not aligned for a
// vector load, and for wavefronts that straddle layers (la: the lane's layer,
// ea: its end).
template <bool FP16>
__device__ __noinline__ float4 grad4_slow(const uint64_t* __restrict__ table, const int64_t* __restrict__ offsets,
                                          int32_t L, int32_t wk, int32_t la, int64_t ea, int64_t i0, int64_t P) {
    float f[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e;
        if (i < P) {
            int32_t l = la;
            if (i >= ea) {
                l = la + 1;
                while (offsets[l + 1] <= i) ++l;
            }
            const uint64_t a = table[(int64_t)wk * L + l];
            const int64_t j = i - offsets[l];
            f[e] = FP16 ? widen1(as_global<uint16_t>(a)[j]) : as_global<float>(a)[j];
        }
    }
    return make_float4(f[0], f[1], f[2], f[3]);
}

// Worker wk's four gradient elements at the lane's offset: a vector load from
// the address lane b of `mine` holds (vec), else element by element.
template <bool FP16>
__device__ __forceinline__ float4 grad4(bool vec, uint64_t mine, int b, int64_t byte_off,
                                        const uint64_t* __restrict__ table, const int64_t* __restrict__ offsets,
                                        int32_t L, int32_t wk, int32_t la, int64_t ea, int64_t i0, int64_t P) {
    if (vec) {
        const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(mine >> 32), b) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, b);
        const uint64_t addr = base + (uint64_t)byte_off;
        if (FP16) {
            typedef uint32_t v2u __attribute__((ext_vector_type(2)));
            const v2u x = *as_global<v2u>(addr);
            return make_float4(widen1((uint16_t)(x.x & 0xffffu)), widen1((uint16_t)(x.x >> 16)),
                               widen1((uint16_t)(x.y & 0xffffu)), widen1((uint16_t)(x.y >> 16)));
        }
        return load_f4(as_global<void>(addr));
    }
    return grad4_slow<FP16>(table, offsets, L, wk, la, ea, i0, P);
}

// The residual case of the worker at bit b of a group: sent j steps back
// (n = j, zero base) for the smallest such j, else n = age on R.
template <int AGE>
__device__ __forceinline__ void leaf_case(const uint64_t (&mh)[AGE + 1], int32_t age, int b, int32_t& n,
                                          bool& zero) {
    n = age;
    zero = false;
#pragma unroll
    for (int j = 0; j <= AGE; ++j)
        if (!zero && ((mh[j] >> b) & 1ull)) {
            n = j;
            zero = true;
        }
}

// STORED: this step's norm pass wrote a into R, so every sent value is read
// from R; otherwise each is re-formed from the gradients and R (age <= AGE).
template <int LEV, bool FP16, bool STORED, int AGE>
__global__ __launch_bounds__(kGatherThreads) void k_gather_hist(
    HistArgs h, const int64_t* __restrict__ offsets, const uint32_t* __restrict__ tile_layer, int64_t tile_elems,
    int32_t L, const float* __restrict__ resid, int64_t ld, int32_t W, int64_t P, int64_t C,
    const uint32_t* __restrict__ sel, int32_t mw, float invW, float* __restrict__ grad, int32_t do_sgd, float lr,
    float mu, float* __restrict__ w, float* __restrict__ v) {
    constexpr int E = 4;
    constexpr int UNR = STORED ? 16 : 8;   // leaves in flight
    constexpr int64_t kEsz = FP16 ? 2 : 4;
    constexpr uint64_t kAlignMask = FP16 ? 7ull : 15ull;
    const int lane = threadIdx.x & 63;
    const int64_t wave_base =
        ((int64_t)blockIdx.x * kGatherThreads + (int64_t)__builtin_amdgcn_readfirstlane(threadIdx.x & ~63u)) * E;
    if (wave_base >= P) return;
    const int64_t i0 = wave_base + (int64_t)lane * E;
    const bool valid = i0 < P;
    const bool full = i0 + E <= P;
    const int32_t c = (int32_t)(wave_base / C);
    const int32_t cw = c >> 5;
    const uint32_t cb = 1u << (c & 31);

    // did any worker send this chunk?
    bool any = false;
    for (int32_t g0 = 0; g0 < W; g0 += 64) {
        const int32_t wk = g0 + lane;
        const uint32_t sw = wk < W ? sel[(int64_t)wk * mw + cw] : 0u;
        any |= __ballot((sw & cb) != 0u) != 0ull;
    }

    float4 wv = make_float4(0.f, 0.f, 0.f, 0.f), vv = wv;
    if (do_sgd && full) {
        wv = *reinterpret_cast<const float4*>(w + i0);
        vv = *reinterpret_cast<const float4*>(v + i0);
    }

    float s[E] = {0.f, 0.f, 0.f, 0.f};
    if (any) {
        // the layer of the wavefront's tile; a tile that lies in one layer at a
        // vector-aligned offset is whole, otherwise each lane finds its layer
        const uint32_t tinfo = tile_layer[wave_base / tile_elems];
        const int32_t l0 = (int32_t)(tinfo & 0x7fffffffu);
        const bool whole = (tinfo >> 31) != 0u;
        const int64_t off0 = offsets[l0];
        int32_t la = l0;
        int64_t ea = offsets[l0 + 1];
        if (!STORED && !whole && valid) {
            int32_t lo = l0, hi = L;
            while (lo < hi) {
                const int32_t mid = (lo + hi) >> 1;
                if (offsets[mid + 1] <= i0) lo = mid + 1;
                else hi = mid;
            }
            la = lo;
            ea = offsets[lo + 1];
        }
        const int64_t byte_off = (i0 - off0) * kEsz;

        TreeAcc<LEV, E> tree;
        uint32_t cnt = 0;
        for (int32_t g0 = 0; g0 < W; g0 += 64) {
            const int32_t wk = g0 + lane;
            const bool in = wk < W;
            const uint64_t mc = __ballot(in && (sel[(int64_t)wk * mw + cw] & cb) != 0u);
            uint64_t mh[AGE + 1];
            uint64_t ad[AGE + 1];
            bool vec[AGE + 1];
#pragma unroll
            for (int j = 0; j <= AGE; ++j) {
                mh[j] = 0ull;
                ad[j] = 0ull;
                vec[j] = false;
            }
            if (!STORED && mc != 0ull) {
#pragma unroll
                for (int j = 0; j <= AGE; ++j)
                    if (j <= h.age && h.masks[j] != nullptr)
                        mh[j] = __ballot(in && (h.masks[j][(int64_t)wk * mw + cw] & cb) != 0u);
                // which gradient tables this group's sent leaves read: this
                // step's always, one step back when n >= 1, two when n >= 2
                if (whole) {
#pragma unroll
                    for (int j = 0; j <= AGE; ++j) {
                        if (j > h.age) continue;
                        ad[j] = in ? h.layers[j][(int64_t)wk * L + l0] : 0ull;
                        vec[j] = __ballot((ad[j] & kAlignMask) != 0ull) == 0ull;
                    }
                }
            }
            const int32_t gn = W - g0 < 64 ? W - g0 : 64;
            for (int32_t u0 = 0; u0 < gn; u0 += UNR) {
                float4 xr[UNR], x0[UNR], x1[UNR], x2[UNR];
                // every load of the batch first ...
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int32_t b = u0 + u;
                    if (b >= gn || !((mc >> b) & 1ull) || !valid) continue;
                    const float* rp = resid + (int64_t)(g0 + b) * ld + i0;
                    if (STORED) {
                        xr[u] = load_f4_nt(rp);
                    } else {
                        int32_t n;
                        bool zero;
                        leaf_case<AGE>(mh, h.age, b, n, zero);
                        x0[u] = grad4<FP16>(vec[0], ad[0], b, byte_off, h.layers[0], offsets, L, g0 + b, la, ea, i0,
                                            P);
                        if (!zero) xr[u] = load_f4_nt(rp);
                        if (AGE >= 1 && n >= 1)
                            x1[u] = grad4<FP16>(vec[AGE >= 1 ? 1 : 0], ad[AGE >= 1 ? 1 : 0], b, byte_off,
                                                h.layers[AGE >= 1 ? 1 : 0], offsets, L, g0 + b, la, ea, i0, P);
                        if (AGE >= 2 && n >= 2)
                            x2[u] = grad4<FP16>(vec[AGE >= 2 ? 2 : 0], ad[AGE >= 2 ? 2 : 0], b, byte_off,
                                                h.layers[AGE >= 2 ? 2 : 0], offsets, L, g0 + b, la, ea, i0, P);
                    }
                }
                // ... then the values, in worker order, into the tree
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int32_t b = u0 + u;
                    if (b >= gn) continue;
                    float f[E] = {0.f, 0.f, 0.f, 0.f};
                    if (((mc >> b) & 1ull) && valid) {
                        if (STORED) {
                            f[0] = xr[u].x; f[1] = xr[u].y; f[2] = xr[u].z; f[3] = xr[u].w;
                        } else {
                            int32_t n;
                            bool zero;
                            leaf_case<AGE>(mh, h.age, b, n, zero);
                            const float4 bs = zero ? make_float4(0.f, 0.f, 0.f, 0.f) : xr[u];
                            float4 acc = bs;
                            if (AGE >= 2 && n >= 2) {
                                acc.x = x2[u].x + acc.x; acc.y = x2[u].y + acc.y;
                                acc.z = x2[u].z + acc.z; acc.w = x2[u].w + acc.w;
                            }
                            if (AGE >= 1 && n >= 1) {
                                acc.x = x1[u].x + acc.x; acc.y = x1[u].y + acc.y;
                                acc.z = x1[u].z + acc.z; acc.w = x1[u].w + acc.w;
                            }
                            f[0] = x0[u].x + acc.x; f[1] = x0[u].y + acc.y;
                            f[2] = x0[u].z + acc.z; f[3] = x0[u].w + acc.w;
                        }
                    }
                    tree.push(f, cnt);
                    ++cnt;
                }
            }
        }
        tree.result((uint32_t)W, s);
    }

    if (!valid) return;
    float g[E];
#pragma unroll
    for (int e = 0; e < E; ++e) g[e] = s[e] * invW;
    if (full) {
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
        for (int e = 0; e < E; ++e) {
            if (i0 + e < P) {
                if (grad) grad[i0 + e] = g[e];
                if (do_sgd) {
                    float we = w[i0 + e], ve = v[i0 + e];
                    sgd_update(g[e], lr, mu, we, ve);
                    w[i0 + e] = we;
                    v[i0 + e] = ve;
                }
            }
        }
    }
}

template <int LEV>
hipError_t gather_launch(const Plan& p, const HistArgs& h, bool stored, const float* resid, const uint32_t* sel,
                         float* grad, const ga_sgd* sgd, float* w, float* v, hipStream_t s) {
    const int64_t threads = (p.P + 3) / 4;
    const unsigned blocks = (unsigned)((threads + kGatherThreads - 1) / kGatherThreads);
    const float invW = (float)(1.0 / (double)p.W);
    const float lr = sgd ? sgd->lr : 0.f, mu = sgd ? sgd->mu : 0.f;
#define GA_GH(F, ST, A)                                                                                            \
    hipLaunchKernelGGL((k_gather_hist<LEV, F, ST, A>), dim3(blocks), dim3(kGatherThreads), 0, s, h, p.d_offsets,     \
                       p.d_tile_layer, p.tile_elems, p.L, resid, p.ld, p.W, p.P, p.C, sel, p.mw, invW, grad,       \
                       sgd ? 1 : 0, lr, mu, w, v)
#define GA_GH_AGE(F)                            \
    do {                                        \
        if (stored) GA_GH(F, true, 0);          \
        else if (h.age == 0) GA_GH(F, false, 0); \
        else if (h.age == 1) GA_GH(F, false, 1); \
        else GA_GH(F, false, 2);                \
    } while (0)
    if (p.dtype == GA_FP16) GA_GH_AGE(true);
    else GA_GH_AGE(false);
#undef GA_GH_AGE
#undef GA_GH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_hist(const Plan& p, const HistArgs& h, bool store, float* resid, double* keys,
                            hipStream_t s) {
    if (p.W == 0 || p.n_c == 0) return hipSuccess;
    const bool f16 = p.dtype == GA_FP16;
    switch (h.age) {
        case 0: return f16 ? norm_launch<true, 0>(p, h, store, false, resid, keys, nullptr, false, s)
                           : norm_launch<false, 0>(p, h, store, false, resid, keys, nullptr, false, s);
        case 1: return f16 ? norm_launch<true, 1>(p, h, store, false, resid, keys, nullptr, false, s)
                           : norm_launch<false, 1>(p, h, store, false, resid, keys, nullptr, false, s);
        default: return f16 ? norm_launch<true, 2>(p, h, store, false, resid, keys, nullptr, false, s)
                            : norm_launch<false, 2>(p, h, store, false, resid, keys, nullptr, false, s);
    }
}

hipError_t launch_flush_hist(const Plan& p, const HistArgs& h, bool stored, float* resid, const uint32_t* sel,
                             hipStream_t s) {
    if (p.W == 0 || p.n_c == 0) return hipSuccess;
    const bool f16 = p.dtype == GA_FP16;
    switch (h.age) {
        case 0: return f16 ? norm_launch<true, 0>(p, h, true, true, resid, nullptr, sel, stored, s)
                           : norm_launch<false, 0>(p, h, true, true, resid, nullptr, sel, stored, s);
        case 1: return f16 ? norm_launch<true, 1>(p, h, true, true, resid, nullptr, sel, stored, s)
                           : norm_launch<false, 1>(p, h, true, true, resid, nullptr, sel, stored, s);
        default: return f16 ? norm_launch<true, 2>(p, h, true, true, resid, nullptr, sel, stored, s)
                            : norm_launch<false, 2>(p, h, true, true, resid, nullptr, sel, stored, s);
    }
}

hipError_t launch_gather_hist(const Plan& p, const HistArgs& h, bool stored, const float* resid,
                              const uint32_t* sel, float* grad, const ga_sgd* sgd, float* w, float* v,
                              hipStream_t s) {
    if (p.P == 0) return hipSuccess;
    if (p.W < (1 << 5)) return gather_launch<5>(p, h, stored, resid, sel, grad, sgd, w, v, s);
    if (p.W < (1 << 8)) return gather_launch<8>(p, h, stored, resid, sel, grad, sgd, w, v, s);
    return gather_launch<11>(p, h, stored, resid, sel, grad, sgd, w, v, s);
}

}  // namespace ga
