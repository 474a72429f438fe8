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
//   k_norm_hist    forms a, its key (binary64 sum of squares) and, on a
//                  storing step, writes a into R; as the flush, writes the
//                  residual itself (zero on the chunks sent this step).  One
//                  workgroup per (worker, chunk), except on storing steps
//                  with chunks longer than 2048 elements: one per (worker,
//                  2048-element part), the parts' sums then added per chunk
//                  in part order by k_key_parts.
//   k_gather_hist  one wavefront per 256 or 512 elements of one chunk: the fixed
//                  binary tree over the workers' sent values (absent workers
//                  are +0), the mean and the fused momentum-SGD update, on a
//                  step that did not store: every sent value is re-formed as
//                  above.  On a storing step the sent values are R itself, and
//                  the lazy-zero gather (k_gather_wave) reduces them.
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

// Eight gradient elements at element j of tensor src (16-byte aligned there),
// widened, by non-temporal loads (streamed once, not kept in the caches).
template <bool FP16>
__device__ __forceinline__ void load8_nt(gptr<void> src, int64_t j, float (&f)[8]) {
    if (FP16) {
        const u32x4 x =
            __builtin_nontemporal_load(reinterpret_cast<gptr<u32x4>>(static_cast<gptr<uint16_t>>(src) + j));
        widen8(make_uint4(x.x, x.y, x.z, x.w), f);
    } else {
        gptr<f32x4> gp = reinterpret_cast<gptr<f32x4>>(static_cast<gptr<float>>(src) + j);
        const f32x4 g0 = __builtin_nontemporal_load(gp), g1 = __builtin_nontemporal_load(gp + 1);
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
            // Gradients stream with non-temporal loads; so does R when it is
            // only read.  (Where R is also written here, non-temporal reads of
            // it measured slower.)
            load8_nt<FP16>(g0, i - soff, x0[u]);
            if (NP >= 1) load8_nt<FP16>(g1, i - soff, x1[u]);
            if (NP >= 2) load8_nt<FP16>(g2, i - soff, x2[u]);
            if (BUF) {
                const float4 r0 = ST ? *reinterpret_cast<const float4*>(r + i) : load_f4_nt(r + i);
                const float4 r1 = ST ? *reinterpret_cast<const float4*>(r + i + 4) : load_f4_nt(r + i + 4);
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
            // where R was not read (base +0) it is written with non-temporal
            // stores (the first store after a zero start: 15.3 -> 14.3 ms);
            // where it was just read, plain stores measured faster
            if (ST && !BUF) {
                __builtin_nontemporal_store(f32x4{a[0], a[1], a[2], a[3]}, reinterpret_cast<f32x4*>(r + i));
                __builtin_nontemporal_store(f32x4{a[4], a[5], a[6], a[7]}, reinterpret_cast<f32x4*>(r + i + 4));
            } else if (ST) {
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
                                          double& acc1, int32_t lo0) {
    int32_t lo = lo0;   // a layer at or before the one holding s
    while (offsets[lo + 1] <= s) ++lo;
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

// One workgroup per (worker w = blockIdx.y, part q of chunk c: blockIdx.x =
// c * S + q), the part being elements [c*C + q*kNormPart, +kNormPart) of the
// chunk (the whole chunk when S == 1).  With parts, consecutive workgroups
// take consecutive parts, so the resident ones stream one contiguous window
// of the residual and the gradients.  STORE: a storing step.  FLUSH: write the
// residual after this step instead of keys: zero on the chunks set in sel,
// and, unless this step stored (then R already holds a), a elsewhere.  The
// part's binary64 sum of squares goes to keys[w][c] (S == 1) or to
// part_keys[w][c][q], added per chunk by k_key_parts.
template <bool FP16, int AGE, bool STORE, bool FLUSH>
__global__ __launch_bounds__(kNormThreads) void k_norm_hist(HistArgs h, const int64_t* __restrict__ offsets,
                                                            int32_t L, float* __restrict__ resid, int64_t ld,
                                                            int64_t P, int64_t C, int32_t mw, int64_t n_c,
                                                            int32_t S, double* __restrict__ keys,
                                                            double* __restrict__ part_keys,
                                                            const uint32_t* __restrict__ sel, int32_t stored,
                                                            const uint32_t* __restrict__ tile_layer,
                                                            int64_t tile_elems) {
    const int32_t w = (int32_t)blockIdx.y;
    const int32_t c = (int32_t)(blockIdx.x / (uint32_t)S);
    const int32_t q = (int32_t)(blockIdx.x - (uint32_t)c * (uint32_t)S);
    const int64_t cs = (int64_t)c * C;
    const int64_t ce = cs + C < P ? cs + C : P;
    const int64_t s = S == 1 ? cs : cs + (int64_t)q * kNormPart;
    const int64_t e = S == 1 ? ce : (s + kNormPart < ce ? s + kNormPart : ce);   // e <= s: an empty part
    float* __restrict__ r = resid + (int64_t)w * ld;
    if (FLUSH) {
        if (mask_bit(sel, w, mw, c)) {
            for (int64_t i = s + threadIdx.x; i < e; i += kNormThreads) r[i] = 0.f;
            return;
        }
        if (stored) return;
    }
    // the residual's case: sent j steps back (n = j, base +0), else n = age on R;
    // the mask words and the tile's layer are requested together
    uint32_t mwd[AGE + 1];
#pragma unroll
    for (int j = 0; j <= AGE; ++j)
        mwd[j] = (j <= h.age && h.masks[j] != nullptr) ? h.masks[j][(int64_t)w * mw + (c >> 5)] : 0u;
    const int32_t lo0 = s < e ? (int32_t)(tile_layer[s / tile_elems] & 0x7fffffffu) : 0;
    int32_t n = h.age;
    bool zero = false;
#pragma unroll
    for (int j = 0; j <= AGE; ++j)
        if (!zero && ((mwd[j] >> (c & 31)) & 1u)) {
            n = j;
            zero = true;
        }
    constexpr bool ST = STORE || FLUSH;
    double acc0 = 0.0, acc1 = 0.0;
    if (s >= e) {
        // an empty part of the last chunk: it adds +0 to the chunk's key
    } else if (zero) {
        if (n == 0) norm_walk<FP16, 0, false, ST>(h, offsets, L, w, r, s, e, acc0, acc1, lo0);
        if constexpr (AGE >= 1)
            if (n == 1) norm_walk<FP16, 1, false, ST>(h, offsets, L, w, r, s, e, acc0, acc1, lo0);
        if constexpr (AGE >= 2)
            if (n == 2) norm_walk<FP16, 2, false, ST>(h, offsets, L, w, r, s, e, acc0, acc1, lo0);
    } else {
        if (n == 0) norm_walk<FP16, 0, true, ST>(h, offsets, L, w, r, s, e, acc0, acc1, lo0);
        if constexpr (AGE >= 1)
            if (n == 1) norm_walk<FP16, 1, true, ST>(h, offsets, L, w, r, s, e, acc0, acc1, lo0);
        if constexpr (AGE >= 2)
            if (n == 2) norm_walk<FP16, 2, true, ST>(h, offsets, L, w, r, s, e, acc0, acc1, lo0);
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
        for (int j = 1; j < kNormThreads / 64; ++j) k += part[j];
        if (S == 1) keys[(int64_t)w * n_c + c] = k;
        else part_keys[((int64_t)w * n_c + c) * S + q] = k;
    }
}

// keys[i] = the S partial sums of key i added in part order (binary64).
__global__ __launch_bounds__(256) void k_key_parts(const double* __restrict__ part_keys, int32_t S, int64_t n,
                                                   double* __restrict__ keys) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const double* pk = part_keys + i * S;
    double k = pk[0];
    for (int32_t j = 1; j < S; ++j) k += pk[j];
    keys[i] = k;
}

template <bool FP16, int AGE>
hipError_t norm_launch(const Plan& p, const HistArgs& h, bool store, bool flush, float* resid, double* keys,
                       const uint32_t* sel, bool stored, hipStream_t s) {
    // Storing passes run on 2048-element parts (their mixed read/write stream
    // measured faster as one contiguous window); read-only passes and the
    // flush sweep whole chunks, which measured faster for reads.
    const int32_t S = (store && !flush) ? p.key_parts : 1;
    const dim3 grid((unsigned)(p.n_c * S), (unsigned)p.W);
#define GA_NH(ST, FL)                                                                                      \
    hipLaunchKernelGGL((k_norm_hist<FP16, AGE, ST, FL>), grid, dim3(kNormThreads), 0, s, h, p.d_offsets, p.L, \
                       resid, p.ld, p.P, p.C, p.mw, p.n_c, S, keys, p.d_part_keys, sel, stored ? 1 : 0,        \
                       p.d_tile_layer, p.tile_elems)
    if (flush) GA_NH(false, true);
    else if (store) GA_NH(true, false);
    else GA_NH(false, false);
#undef GA_NH
    if (!flush && S > 1) return launch_key_parts(p, p.d_part_keys, keys, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// k_gather_hist
// ---------------------------------------------------------------------------

// A lane's E gradient elements of one worker as raw bits: binary16 two to a
// word (NW = E/2 words), binary32 one to a word (NW = E).
template <bool FP16, int E>
struct GradBits {
    static constexpr int NW = FP16 ? E / 2 : E;
    uint32_t w[NW];

    __device__ __forceinline__ float value(int e) const {
        if (FP16) return widen1((uint16_t)((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
        return __uint_as_float(w[e]);
    }
};

// Elements i0 .. i0+E-1 of worker wk's gradient through a layer table, element
// by element (zero past P): for tensors not aligned for a vector load, and for
// wavefronts that straddle layers (la: the lane's layer at i0, ea: its end).
template <bool FP16, int E>
__device__ __noinline__ GradBits<FP16, E> grad_slow(const uint64_t* __restrict__ table,
                                                    const int64_t* __restrict__ offsets, int32_t L, int32_t wk,
                                                    int32_t la, int64_t ea, int64_t i0, int64_t P) {
    GradBits<FP16, E> x;
#pragma unroll
    for (int q = 0; q < GradBits<FP16, E>::NW; ++q) x.w[q] = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t i = i0 + e;
        if (i < P) {
            int32_t l = la;
            if (i >= ea) {
                l = la + 1;
                while (offsets[l + 1] <= i) ++l;
            }
            const uint64_t a = table[(int64_t)wk * L + l];
            const int64_t j = i - offsets[l];
            if (FP16) x.w[e >> 1] |= (uint32_t)as_global<uint16_t>(a)[j] << ((e & 1) * 16);
            else x.w[e] = as_global<uint32_t>(a)[j];
        }
    }
    return x;
}

// Worker wk's gradient at the lane's elements: one vector load (E*b bytes,
// 8 or 16) from the address lane b of `mine` holds (vec), else element by
// element.
template <bool FP16, int E>
__device__ __forceinline__ GradBits<FP16, E> grad_bits(bool vec, uint64_t mine, int b, int64_t byte_off,
                                                       const uint64_t* __restrict__ table,
                                                       const int64_t* __restrict__ offsets, int32_t L, int32_t wk,
                                                       int32_t la, int64_t ea, int64_t i0, int64_t P) {
    constexpr int NW = GradBits<FP16, E>::NW;
    static_assert(NW == 2 || NW == 4, "8- or 16-byte loads");
    if (vec) {
        const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(mine >> 32), b) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, b);
        const uint64_t addr = base + (uint64_t)byte_off;
        GradBits<FP16, E> x;
        if (NW == 4) {
            const u32x4 t = *as_global<u32x4>(addr);
            x.w[0] = t.x; x.w[1] = t.y; x.w[NW > 2 ? 2 : 0] = t.z; x.w[NW > 3 ? 3 : 0] = t.w;
        } else {
            typedef uint32_t v2u __attribute__((ext_vector_type(2)));
            const v2u t = *as_global<v2u>(addr);
            x.w[0] = t.x; x.w[1] = t.y;
        }
        return x;
    }
    return grad_slow<FP16, E>(table, offsets, L, wk, la, ea, i0, P);
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

// What a wavefront needs of one 64-worker group: the bitmaps of the workers
// that send the chunk now (mc) and that sent it j+1 steps back (mh[j]), and,
// for a tile inside one layer, lane l's worker's tensor address of that layer
// in each step's table (ad[j]) with whether every address of the group allows
// a vector load (vec[j]).
template <int AGE>
struct Group {
    uint64_t mc;
    uint64_t mh[AGE + 1];
    uint64_t ad[AGE + 1];
    bool vec[AGE + 1];
};

// The raw words behind a Group, loaded first so that the loads of several
// groups are in flight together.
template <int AGE>
struct GroupWords {
    uint32_t hw[AGE + 1];
    uint64_t ad[AGE + 1];
};

template <int AGE>
__device__ __forceinline__ void group_issue(const HistArgs& h, int32_t W, int32_t mw, int32_t cw, int32_t L,
                                            int32_t l0, bool whole, int32_t wk, GroupWords<AGE>& gw) {
    const bool in = wk < W;
#pragma unroll
    for (int j = 0; j <= AGE; ++j) {
        gw.hw[j] = (in && j <= h.age && h.masks[j] != nullptr) ? h.masks[j][(int64_t)wk * mw + cw] : 0u;
        gw.ad[j] = (in && whole && j <= h.age) ? h.layers[j][(int64_t)wk * L + l0] : 0ull;
    }
}

// vec[j] holds only for a whole tile (otherwise no address was loaded and
// every lane finds its own layer) whose group's addresses are all aligned to
// the load width.
template <int AGE>
__device__ __forceinline__ void group_finish(const GroupWords<AGE>& gw, uint32_t cb, uint64_t mc, bool whole,
                                             uint64_t align_mask, Group<AGE>& g) {
    g.mc = mc;
#pragma unroll
    for (int j = 0; j <= AGE; ++j) {
        g.mh[j] = __ballot((gw.hw[j] & cb) != 0u);
        g.ad[j] = gw.ad[j];
        g.vec[j] = whole && __ballot((gw.ad[j] & align_mask) != 0ull) == 0ull;
    }
}

template <typename T>
__device__ __forceinline__ T pick4(int gi, const T (&a)[4]) {
    return gi == 0 ? a[0] : gi == 1 ? a[1] : gi == 2 ? a[2] : a[3];
}

// The (at most four) groups of W < 256 workers, field by field, so that every
// array index is a constant and the state stays in registers.
template <int AGE>
struct Groups4 {
    uint64_t mc[4];
    uint64_t mh[AGE + 1][4];
    uint64_t ad[AGE + 1][4];
    bool vec[AGE + 1][4];

    __device__ __forceinline__ void set(int gi, const Group<AGE>& g) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q == gi) {
                mc[q] = g.mc;
#pragma unroll
                for (int j = 0; j <= AGE; ++j) {
                    mh[j][q] = g.mh[j];
                    ad[j][q] = g.ad[j];
                    vec[j][q] = g.vec[j];
                }
            }
    }

    __device__ __forceinline__ void get(int gi, Group<AGE>& g) const {
        g.mc = pick4(gi, mc);
#pragma unroll
        for (int j = 0; j <= AGE; ++j) {
            g.mh[j] = pick4(gi, mh[j]);
            g.ad[j] = pick4(gi, ad[j]);
            g.vec[j] = pick4(gi, vec[j]);
        }
    }
};

// The gather-reduce of a step whose norm pass did not store: every sent value
// is re-formed, a = g_t + (g_{t-1} + (... + base)), from this step's gradient
// tensors, the n earlier ones its case needs and, unless its base is +0, R.
// (A storing step's values are R itself: that is the lazy-zero gather.)
// A wavefront covers 64*E elements of one chunk, E per lane (E = 8 for
// binary16 gradients when the chunk size allows it: 16-byte gradient loads).
// For W < 256 the (at most four) groups' bitmaps and addresses are loaded
// once, together, and kept in registers; w and v are requested first.
// Gradients stay raw bits until their leaf is formed.
template <int LEV, bool FP16, int AGE, int E>
__global__ __launch_bounds__(kGatherThreads) void k_gather_hist(
    HistArgs h, const int64_t* __restrict__ offsets, const uint32_t* __restrict__ tile_layer, int64_t tile_elems,
    int32_t L, const float* __restrict__ resid, int64_t ld, int32_t W, int64_t P, int64_t C,
    const uint32_t* __restrict__ sel, int32_t mw, float invW, float* __restrict__ grad, int32_t do_sgd, float lr,
    float mu, float* __restrict__ w, float* __restrict__ v) {
    static_assert(E == 4 || E == 8, "4 or 8 elements per lane");
    constexpr int UNR = E == 8 ? 4 : 8;   // leaves in flight
    constexpr int G = LEV <= 8 ? 4 : 1;   // groups kept in registers
    constexpr int64_t kEsz = FP16 ? 2 : 4;
    constexpr int E4 = E / 4;
    constexpr uint64_t kAlignMask = (uint64_t)(E * kEsz >= 16 ? 15 : 7);
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

    float4 wv[E4], vv[E4];
#pragma unroll
    for (int q = 0; q < E4; ++q) wv[q] = vv[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (do_sgd && full) {
#pragma unroll
        for (int q = 0; q < E4; ++q) {
            wv[q] = *reinterpret_cast<const float4*>(w + i0 + 4 * q);
            vv[q] = *reinterpret_cast<const float4*>(v + i0 + 4 * q);
        }
    }
    // this step's mask words of the first G groups, in flight together
    uint32_t sw[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        const int32_t wk = gi * 64 + lane;
        sw[gi] = wk < W ? sel[(int64_t)wk * mw + cw] : 0u;
    }
    uint64_t mc[G];
    bool any = false;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        mc[gi] = __ballot((sw[gi] & cb) != 0u);
        any |= mc[gi] != 0ull;
    }
    for (int32_t g0 = G * 64; g0 < W; g0 += 64) {
        const int32_t wk = g0 + lane;
        any |= __ballot(wk < W && (sel[(int64_t)wk * mw + cw] & cb) != 0u) != 0ull;
    }

    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = 0.f;
    if (any) {
        // the layer of the wavefront's tile; a tile that lies in one layer at a
        // vector-aligned offset is whole, otherwise each lane finds its layer
        const uint32_t tinfo = tile_layer[wave_base / tile_elems];
        const int32_t l0 = (int32_t)(tinfo & 0x7fffffffu);
        const bool whole = (tinfo >> 31) != 0u;
        const int64_t off0 = offsets[l0];
        int32_t la = l0;
        int64_t ea = offsets[l0 + 1];
        if (!whole && valid) {
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

        Groups4<AGE> gs;
        if (G == 4) {
            GroupWords<AGE> gw[4];
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) group_issue<AGE>(h, W, mw, cw, L, l0, whole, gi * 64 + lane, gw[gi]);
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                Group<AGE> g;
                group_finish<AGE>(gw[gi], cb, mc[gi < G ? gi : 0], whole, kAlignMask, g);
                gs.set(gi, g);
            }
        }

        TreeAcc<LEV, E> tree;
        uint32_t cnt = 0;
        for (int32_t g0 = 0; g0 < W; g0 += 64) {
            Group<AGE> g;
            if (G == 4) {
                gs.get(g0 >> 6, g);
            } else {
                const int32_t wk = g0 + lane;
                const uint32_t sw1 = wk < W ? sel[(int64_t)wk * mw + cw] : 0u;
                GroupWords<AGE> gw;
                group_issue<AGE>(h, W, mw, cw, L, l0, whole, wk, gw);
                group_finish<AGE>(gw, cb, __ballot((sw1 & cb) != 0u), whole, kAlignMask, g);
            }
            const int32_t gn = W - g0 < 64 ? W - g0 : 64;
            for (int32_t u0 = 0; u0 < gn; u0 += UNR) {
                float4 xr[UNR][E4];
                GradBits<FP16, E> x0[UNR], x1[UNR], x2[UNR];
                // every load of the batch first ...
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int32_t b = u0 + u;
                    if (b >= gn || !((g.mc >> b) & 1ull) || !valid) continue;
                    int32_t n;
                    bool zero;
                    leaf_case<AGE>(g.mh, h.age, b, n, zero);
                    x0[u] = grad_bits<FP16, E>(g.vec[0], g.ad[0], b, byte_off, h.layers[0], offsets, L, g0 + b, la,
                                               ea, i0, P);
                    if (!zero) {
                        const float* rp = resid + (int64_t)(g0 + b) * ld + i0;
#pragma unroll
                        for (int q = 0; q < E4; ++q) xr[u][q] = load_f4_nt(rp + 4 * q);
                    }
                    if (AGE >= 1 && n >= 1)
                        x1[u] = grad_bits<FP16, E>(g.vec[AGE >= 1 ? 1 : 0], g.ad[AGE >= 1 ? 1 : 0], b, byte_off,
                                                   h.layers[AGE >= 1 ? 1 : 0], offsets, L, g0 + b, la, ea, i0, P);
                    if (AGE >= 2 && n >= 2)
                        x2[u] = grad_bits<FP16, E>(g.vec[AGE >= 2 ? 2 : 0], g.ad[AGE >= 2 ? 2 : 0], b, byte_off,
                                                   h.layers[AGE >= 2 ? 2 : 0], offsets, L, g0 + b, la, ea, i0, P);
                }
                // ... then the values, in worker order, into the tree
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int32_t b = u0 + u;
                    if (b >= gn) continue;
                    float f[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) f[e] = 0.f;
                    if (((g.mc >> b) & 1ull) && valid) {
                        int32_t n;
                        bool zero;
                        leaf_case<AGE>(g.mh, h.age, b, n, zero);
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            const float4 r4 = xr[u][e >> 2];
                            const float rb = (e & 3) == 0 ? r4.x : (e & 3) == 1 ? r4.y : (e & 3) == 2 ? r4.z : r4.w;
                            float acc = zero ? 0.f : rb;
                            if (AGE >= 2 && n >= 2) acc = x2[u].value(e) + acc;
                            if (AGE >= 1 && n >= 1) acc = x1[u].value(e) + acc;
                            f[e] = x0[u].value(e) + acc;
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
#pragma unroll
        for (int q = 0; q < E4; ++q) {
            if (grad)
                *reinterpret_cast<float4*>(grad + i0 + 4 * q) =
                    make_float4(g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]);
            if (do_sgd) {
                sgd_update(g[4 * q], lr, mu, wv[q].x, vv[q].x);
                sgd_update(g[4 * q + 1], lr, mu, wv[q].y, vv[q].y);
                sgd_update(g[4 * q + 2], lr, mu, wv[q].z, vv[q].z);
                sgd_update(g[4 * q + 3], lr, mu, wv[q].w, vv[q].w);
                *reinterpret_cast<float4*>(w + i0 + 4 * q) = wv[q];
                *reinterpret_cast<float4*>(v + i0 + 4 * q) = vv[q];
            }
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

template <int LEV, int E>
hipError_t gather_launch(const Plan& p, const HistArgs& h, const float* resid, const uint32_t* sel, float* grad,
                         const ga_sgd* sgd, float* w, float* v, hipStream_t s) {
    const int64_t threads = (p.P + E - 1) / E;
    const unsigned blocks = (unsigned)((threads + kGatherThreads - 1) / kGatherThreads);
    const float invW = (float)(1.0 / (double)p.W);
    const float lr = sgd ? sgd->lr : 0.f, mu = sgd ? sgd->mu : 0.f;
#define GA_GH(F, A)                                                                                             \
    hipLaunchKernelGGL((k_gather_hist<LEV, F, A, E>), dim3(blocks), dim3(kGatherThreads), 0, s, h, p.d_offsets,  \
                       p.d_tile_layer, p.tile_elems, p.L, resid, p.ld, p.W, p.P, p.C, sel, p.mw, invW, grad,    \
                       sgd ? 1 : 0, lr, mu, w, v)
#define GA_GH_AGE(F)                       \
    do {                                   \
        if (h.age == 0) GA_GH(F, 0);       \
        else if (h.age == 1) GA_GH(F, 1);  \
        else GA_GH(F, 2);                  \
    } while (0)
    if constexpr (E == 8) {   // 8 elements per lane: binary16 only
        GA_GH_AGE(true);
    } else {
        if (p.dtype == GA_FP16) GA_GH_AGE(true);
        else GA_GH_AGE(false);
    }
#undef GA_GH_AGE
#undef GA_GH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_key_parts(const Plan& p, const double* part_keys, double* keys, hipStream_t s) {
    const int64_t n = (int64_t)p.W * p.n_c;
    hipLaunchKernelGGL(k_key_parts, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part_keys, p.key_parts,
                       n, keys);
    return hipGetLastError();
}

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
    // a storing step left every a in R: the lazy-zero gather, which does not write R
    if (stored) return launch_sparse_gather(p, const_cast<float*>(resid), sel, 0, grad, sgd, w, v, s);
    // 4 elements per lane: 8 (16-byte binary16 loads, 512 elements per
    // wavefront) measured slower at W = 128, its larger tree halving the
    // wavefronts per SIMD
    if (p.W < (1 << 5)) return gather_launch<5, 4>(p, h, resid, sel, grad, sgd, w, v, s);
    if (p.W < (1 << 8)) return gather_launch<8, 4>(p, h, resid, sel, grad, sgd, w, v, s);
    return gather_launch<11, 4>(p, h, resid, sel, grad, sgd, w, v, s);
}

}  // namespace ga
