// Coarse-grained sparse communication, part 3, deferred-residual form
// (GradientFlow, arXiv abstract: only the important chunks are sent; the rest
// stay in the worker's residual).
//
// In lazy-zero mode a chunk that a worker sent in the previous step has a zero
// residual, so its a is just the worker's widened gradient.  The deferred norm
// pass does not store that a.  This gather then
//   - takes the leaf of a chunk sent now and in the previous step from the
//     gradient tensors (2 bytes per binary16 element instead of 4),
//   - and otherwise reduces like k_gather_wave: every worker pushes its leaf or
//     +0 into the fixed tree, then the mean and the fused SGD update
//     (k_gather_defer; a wavefront covers 256 consecutive elements of one
//     chunk, C being a multiple of 256, so a worker's two mask bits are
//     wavefront-uniform);
//   - and writes the residual of a chunk sent in the previous step but not now
//     (the widened gradient), so that afterwards the residual buffer holds
//     exactly what the non-deferred lazy mode leaves (k_materialize).
// In the pending form the last part is left out: that residual stays held as
// the step's gradient, which the next step's norm pass reads in its place;
// launch_residual_flush writes it when the buffer itself is wanted.  In the
// depth-2 pending form (P2) the norm pass also left unstored the a of a chunk
// sent two steps back and not in the previous step; if that chunk is sent now,
// its leaf is recomputed here as g + (g' + 0) from this and the previous
// step's tensors (k_gather_defer<LEV, FP16, true>), and if not, the next norm pass or the
// flush (k_materialize<FP16, true>) forms it.
#include "device.h"
#include "plan.h"
#include "tree.h"

namespace ga {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Worker wk's 4 gradient elements at i0 (i0 % 4 == 0), element by element:
// for tensors that are not aligned for a vector load, or a wavefront that
// straddles layers (la: the lane's layer, ea: its end).  Widened, plus +0.
template <bool FP16>
__device__ __noinline__ float4 grad4_slow(const uint64_t* __restrict__ layer_ptrs,
                                          const int64_t* __restrict__ offsets, int32_t L, int32_t wk,
                                          int32_t la, int64_t ea, int64_t i0, int64_t P) {
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
            const uint64_t a = layer_ptrs[(int64_t)wk * L + l];
            const int64_t j = i - offsets[l];
            f[e] = FP16 ? widen1(as_global<uint16_t>(a)[j]) : as_global<float>(a)[j];
        }
    }
    return make_float4(f[0] + 0.f, f[1] + 0.f, f[2] + 0.f, f[3] + 0.f);
}

// Worker wk's 4 binary16 gradient elements at i0 as raw bits, two to a word
// (zero past P), element by element, for the same cases as grad4_slow.
__device__ __noinline__ v2u grad4_slow_raw16(const uint64_t* __restrict__ layer_ptrs,
                                             const int64_t* __restrict__ offsets, int32_t L, int32_t wk, int32_t la,
                                             int64_t ea, int64_t i0, int64_t P) {
    uint32_t h[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e;
        if (i < P) {
            int32_t l = la;
            if (i >= ea) {
                l = la + 1;
                while (offsets[l + 1] <= i) ++l;
            }
            h[e] = as_global<uint16_t>(layer_ptrs[(int64_t)wk * L + l])[i - offsets[l]];
        }
    }
    return v2u{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// A leaf as loaded: 4 binary32 residual values; or 4 gradient elements
// (binary16 in the first two words, or binary32) to widen and add +0 to (the
// residual of a chunk sent in the previous step is +0, and a = leaf + residual
// maps a -0 leaf to +0 exactly as the non-deferred pass does); or values the
// element-by-element path already produced.
enum LeafKind { kResid = 0, kGradVec = 1, kReady = 2 };

template <bool FP16>
__device__ __forceinline__ float4 decode_leaf(const v4u& x, int kind) {
    if (kind == kGradVec) {
        if (FP16)
            return make_float4(widen1((uint16_t)(x.x & 0xffffu)) + 0.f, widen1((uint16_t)(x.x >> 16)) + 0.f,
                               widen1((uint16_t)(x.y & 0xffffu)) + 0.f, widen1((uint16_t)(x.y >> 16)) + 0.f);
        return make_float4(__uint_as_float(x.x) + 0.f, __uint_as_float(x.y) + 0.f, __uint_as_float(x.z) + 0.f,
                           __uint_as_float(x.w) + 0.f);
    }
    return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
}

// Worker wk's gradient vector at the lane's elements: with a vector load from
// the address held by lane b of `mine` (vec), else element by element.
template <bool FP16>
__device__ __forceinline__ v4u load_grad(bool vec, uint64_t mine, int b, int64_t byte_off,
                                         const uint64_t* __restrict__ layer_ptrs,
                                         const int64_t* __restrict__ offsets, int32_t L, int32_t wk, int32_t la,
                                         int64_t ea, int64_t i0, int64_t P) {
    if (vec) {
        const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(mine >> 32), b) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, b);
        const uint64_t addr = base + (uint64_t)byte_off;
        if (FP16) {
            const v2u x = *as_global<v2u>(addr);
            return v4u{x.x, x.y, 0u, 0u};
        }
        return *as_global<v4u>(addr);
    }
    const float4 f = grad4_slow<FP16>(layer_ptrs, offsets, L, wk, la, ea, i0, P);
    return v4u{__float_as_uint(f.x), __float_as_uint(f.y), __float_as_uint(f.z), __float_as_uint(f.w)};
}

__device__ __forceinline__ uint64_t pick(int gi, uint64_t a0, uint64_t a1, uint64_t a2, uint64_t a3) {
    return gi == 0 ? a0 : gi == 1 ? a1 : gi == 2 ? a2 : a3;
}

// The bitmaps of the 64-worker group starting at g0 for chunk bit cb of mask
// word cw: sent now (mc), sent in the previous step (mp) and, with P2, sent
// two steps back (mq; else 0).
template <bool P2>
__device__ __forceinline__ void group_masks(const uint32_t* __restrict__ sel_mask,
                                            const uint32_t* __restrict__ prev_mask,
                                            const uint32_t* __restrict__ prev2_mask, int32_t W, int32_t mw,
                                            int32_t cw, uint32_t cb, int32_t g0, int lane, uint64_t& mc,
                                            uint64_t& mp, uint64_t& mq) {
    const int32_t wk = g0 + lane;
    const uint32_t sc = wk < W ? sel_mask[(int64_t)wk * mw + cw] : 0u;
    const uint32_t sp = wk < W ? prev_mask[(int64_t)wk * mw + cw] : 0u;
    const uint32_t sq = P2 && wk < W ? prev2_mask[(int64_t)wk * mw + cw] : 0u;
    mc = __ballot((sc & cb) != 0u);
    mp = __ballot((sp & cb) != 0u);
    mq = P2 ? __ballot((sq & cb) != 0u) : 0ull;
}

// P2 (the depth-2 pending form): a chunk sent now and two steps back but not
// in the previous step (its a was not stored) has the leaf g0 + (g1 + 0),
// read from this step's tensors and the previous step's (prev_layer_ptrs).
template <int LEV, bool FP16, bool P2 = false>
__global__ __launch_bounds__(kThreads) void k_gather_defer(
    const uint64_t* __restrict__ layer_ptrs, const int64_t* __restrict__ offsets,
    const uint32_t* __restrict__ tile_layer, int64_t tile_elems, int32_t L, float* __restrict__ resid,
    int64_t ld, int32_t W, int64_t P, int64_t C, const uint32_t* __restrict__ prev_mask,
    const uint32_t* __restrict__ sel_mask, int32_t mw, float invW, float* __restrict__ grad, int32_t do_sgd,
    float lr, float mu, float* __restrict__ w, float* __restrict__ v,
    const uint64_t* __restrict__ prev_layer_ptrs, const uint32_t* __restrict__ prev2_mask) {
    // W < 256 (LEV <= 8): the (at most four) groups' bitmaps and addresses
    // are read once and kept in registers; otherwise group by group.
    constexpr bool kCached = LEV <= 8;
    constexpr int UNR = kUnroll;   // leaves in flight
    constexpr int E = 4;
    constexpr int64_t kEsz = FP16 ? 2 : 4;
    constexpr uint64_t kAlignMask = FP16 ? 7ull : 15ull;
    const int lane = threadIdx.x & 63;
    const int64_t wave_base =
        ((int64_t)blockIdx.x * kThreads + (int64_t)__builtin_amdgcn_readfirstlane(threadIdx.x & ~63u)) * E;
    if (wave_base >= P) return;
    const int64_t i0 = wave_base + (int64_t)lane * E;
    const bool valid = i0 < P;
    const bool full = i0 + E <= P;
    const int32_t c = (int32_t)(wave_base / C);
    const int32_t cw = c >> 5;
    const uint32_t cb = 1u << (c & 31);

    // The layer of the wavefront's tile, its start and end (scalar loads, in
    // flight with the mask words below): the plan's tile table gives the
    // layer and whether the tile lies in it at an aligned offset (whole).
    const uint32_t tinfo = tile_layer[wave_base / tile_elems];
    const int32_t l0 = (int32_t)(tinfo & 0x7fffffffu);
    const bool whole = (tinfo >> 31) != 0u;
    const int64_t off0 = offsets[l0];
    const int64_t end0 = offsets[l0 + 1];

    // Both bitmaps of the (at most four) 64-worker groups, every mask word in
    // flight together: sent now (mc), sent in the previous step (mp).
    uint64_t mc0 = 0ull, mc1 = 0ull, mc2 = 0ull, mc3 = 0ull, mp0 = 0ull, mp1 = 0ull, mp2 = 0ull, mp3 = 0ull;
    uint64_t mq0 = 0ull, mq1 = 0ull, mq2 = 0ull, mq3 = 0ull;
    bool any_sent = false, any_resent = false, any_pend = false;
    if (kCached) {
        uint32_t sw[4], pw[4];
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int32_t wk = gi * 64 + lane;
            sw[gi] = wk < W ? sel_mask[(int64_t)wk * mw + cw] : 0u;
            pw[gi] = wk < W ? prev_mask[(int64_t)wk * mw + cw] : 0u;
        }
        mc0 = __ballot((sw[0] & cb) != 0u);
        mc1 = __ballot((sw[1] & cb) != 0u);
        mc2 = __ballot((sw[2] & cb) != 0u);
        mc3 = __ballot((sw[3] & cb) != 0u);
        mp0 = __ballot((pw[0] & cb) != 0u);
        mp1 = __ballot((pw[1] & cb) != 0u);
        mp2 = __ballot((pw[2] & cb) != 0u);
        mp3 = __ballot((pw[3] & cb) != 0u);
        any_sent = (mc0 | mc1 | mc2 | mc3) != 0ull;
        // some worker sent the chunk now and in the previous step: its leaf is
        // read from the gradient tensor
        any_resent = ((mc0 & mp0) | (mc1 & mp1) | (mc2 & mp2) | (mc3 & mp3)) != 0ull;
        if (P2 && any_sent) {
            // pending (sent two steps back, not in the previous step) and sent
            // now; the words of two steps back only where a leaf is sent
            uint32_t qw[4];
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const int32_t wk = gi * 64 + lane;
                qw[gi] = wk < W ? prev2_mask[(int64_t)wk * mw + cw] : 0u;
            }
            mq0 = __ballot((qw[0] & cb) != 0u) & mc0 & ~mp0;
            mq1 = __ballot((qw[1] & cb) != 0u) & mc1 & ~mp1;
            mq2 = __ballot((qw[2] & cb) != 0u) & mc2 & ~mp2;
            mq3 = __ballot((qw[3] & cb) != 0u) & mc3 & ~mp3;
            any_pend = (mq0 | mq1 | mq2 | mq3) != 0ull;
        }
    } else {
        for (int32_t g0 = 0; g0 < W; g0 += 64) {
            uint64_t mc, mp, mq;
            group_masks<P2>(sel_mask, prev_mask, prev2_mask, W, mw, cw, cb, g0, lane, mc, mp, mq);
            any_sent |= mc != 0ull;
            any_resent |= (mc & mp) != 0ull;
            any_pend |= (mq & mc & ~mp) != 0ull;
        }
    }

    float4 wv = make_float4(0.f, 0.f, 0.f, 0.f), vv = wv;
    if (do_sgd && full) {
        wv = *reinterpret_cast<const float4*>(w + i0);
        vv = *reinterpret_cast<const float4*>(v + i0);
    }

    // Where the gradient elements live: for a whole tile, lane l holds worker
    // (64 gi + l)'s tensor address for layer l0 and vN says every address of
    // group N allows the vector load; otherwise each lane finds its layer
    // (la, ending at ea).
    int32_t la = l0;
    int64_t ea = end0;
    uint64_t p0 = 0ull, p1 = 0ull, p2 = 0ull, p3 = 0ull;
    bool v0 = false, v1 = false, v2 = false, v3 = false;
    // and the previous step's tensor addresses (q, vq) for the pending leaves
    uint64_t q0 = 0ull, q1 = 0ull, q2 = 0ull, q3 = 0ull;
    bool vq0 = false, vq1 = false, vq2 = false, vq3 = false;
    if (any_resent || any_pend) {
        if (whole && kCached) {
            p0 = lane < W ? layer_ptrs[(int64_t)lane * L + l0] : 0ull;
            p1 = 64 + lane < W ? layer_ptrs[(int64_t)(64 + lane) * L + l0] : 0ull;
            p2 = 128 + lane < W ? layer_ptrs[(int64_t)(128 + lane) * L + l0] : 0ull;
            p3 = 192 + lane < W ? layer_ptrs[(int64_t)(192 + lane) * L + l0] : 0ull;
            v0 = __ballot((p0 & kAlignMask) != 0ull) == 0ull;
            v1 = __ballot((p1 & kAlignMask) != 0ull) == 0ull;
            v2 = __ballot((p2 & kAlignMask) != 0ull) == 0ull;
            v3 = __ballot((p3 & kAlignMask) != 0ull) == 0ull;
            if (P2 && any_pend) {
                q0 = lane < W ? prev_layer_ptrs[(int64_t)lane * L + l0] : 0ull;
                q1 = 64 + lane < W ? prev_layer_ptrs[(int64_t)(64 + lane) * L + l0] : 0ull;
                q2 = 128 + lane < W ? prev_layer_ptrs[(int64_t)(128 + lane) * L + l0] : 0ull;
                q3 = 192 + lane < W ? prev_layer_ptrs[(int64_t)(192 + lane) * L + l0] : 0ull;
                vq0 = __ballot((q0 & kAlignMask) != 0ull) == 0ull;
                vq1 = __ballot((q1 & kAlignMask) != 0ull) == 0ull;
                vq2 = __ballot((q2 & kAlignMask) != 0ull) == 0ull;
                vq3 = __ballot((q3 & kAlignMask) != 0ull) == 0ull;
            }
        } else if (!whole && valid) {
            int32_t lo = l0, hi = L;   // the lane's layer is l0 or a later one
            while (lo < hi) {
                const int32_t mid = (lo + hi) >> 1;
                if (offsets[mid + 1] <= i0) lo = mid + 1;
                else hi = mid;
            }
            la = lo;
            ea = offsets[lo + 1];
        }
    }
    const int64_t byte_off = (i0 - off0) * kEsz;

    float s[E] = {0.f, 0.f, 0.f, 0.f};
    if (any_sent) {
        TreeAcc<LEV, E> tree;
        uint32_t cnt = 0;
        for (int32_t g0 = 0; g0 < W; g0 += 64) {
            const int gi = g0 >> 6;
            uint64_t mc, mp, mq, mine, prv;
            bool vec, vecq;
            if (kCached) {
                mc = pick(gi, mc0, mc1, mc2, mc3);
                mp = pick(gi, mp0, mp1, mp2, mp3);
                mq = pick(gi, mq0, mq1, mq2, mq3);
                mine = pick(gi, p0, p1, p2, p3);
                prv = pick(gi, q0, q1, q2, q3);
                vec = gi == 0 ? v0 : gi == 1 ? v1 : gi == 2 ? v2 : v3;
                vecq = gi == 0 ? vq0 : gi == 1 ? vq1 : gi == 2 ? vq2 : vq3;
            } else {
                group_masks<P2>(sel_mask, prev_mask, prev2_mask, W, mw, cw, cb, g0, lane, mc, mp, mq);
                mq &= mc & ~mp;
                mine = prv = 0ull;
                vec = vecq = false;
                if (whole && ((mc & mp) | mq) != 0ull) {
                    mine = g0 + lane < W ? layer_ptrs[(int64_t)(g0 + lane) * L + l0] : 0ull;
                    vec = __ballot((mine & kAlignMask) != 0ull) == 0ull;
                }
                if (P2 && whole && mq != 0ull) {
                    prv = g0 + lane < W ? prev_layer_ptrs[(int64_t)(g0 + lane) * L + l0] : 0ull;
                    vecq = __ballot((prv & kAlignMask) != 0ull) == 0ull;
                }
            }
            const int32_t gn = W - g0 < 64 ? W - g0 : 64;
            for (int32_t u0 = 0; u0 < gn; u0 += UNR) {
                // A pending leaf (P2) needs the previous step's gradient too:
                // binary16 leaves hold both as raw bits, this step's in words
                // 0-1 of x and the previous step's in words 2-3; binary32
                // leaves keep the previous step's in y4.
                v4u x[UNR];
                v4u y4[P2 && !FP16 ? UNR : 1];
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    x[u] = v4u{0u, 0u, 0u, 0u};
                    if (P2 && !FP16) y4[u] = v4u{0u, 0u, 0u, 0u};
                    const int32_t b = u0 + u;
                    if (b < gn && ((mc >> b) & 1ull) && valid) {
                        const bool pend = P2 && ((mq >> b) & 1ull);
                        if (pend && FP16) {
                            v2u h0, h1;
                            if (vec) {
                                const v4u t = load_grad<FP16>(true, mine, b, byte_off, layer_ptrs, offsets, L, g0 + b,
                                                              la, ea, i0, P);
                                h0 = v2u{t.x, t.y};
                            } else {
                                h0 = grad4_slow_raw16(layer_ptrs, offsets, L, g0 + b, la, ea, i0, P);
                            }
                            if (vecq) {
                                const v4u t = load_grad<FP16>(true, prv, b, byte_off, prev_layer_ptrs, offsets, L,
                                                              g0 + b, la, ea, i0, P);
                                h1 = v2u{t.x, t.y};
                            } else {
                                h1 = grad4_slow_raw16(prev_layer_ptrs, offsets, L, g0 + b, la, ea, i0, P);
                            }
                            x[u] = v4u{h0.x, h0.y, h1.x, h1.y};
                        } else if (((mp >> b) & 1ull) || pend) {
                            x[u] = load_grad<FP16>(vec, mine, b, byte_off, layer_ptrs, offsets, L, g0 + b, la, ea,
                                                   i0, P);
                            if (pend)
                                y4[FP16 ? 0 : u] = load_grad<FP16>(vecq, prv, b, byte_off, prev_layer_ptrs, offsets,
                                                                   L, g0 + b, la, ea, i0, P);
                        } else {
                            x[u] = __builtin_nontemporal_load(
                                reinterpret_cast<const v4u*>(resid + (int64_t)(g0 + b) * ld + i0));
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int32_t b = u0 + u;
                    if (b < gn) {
                        const bool pend = P2 && ((mq >> b) & 1ull);
                        float4 a;
                        if (pend) {
                            // a = g0 + (g1 + 0): adding +0 to g0 as well changes
                            // nothing, since g1 + 0 is never -0
                            const float4 r1 = FP16 ? decode_leaf<FP16>(v4u{x[u].z, x[u].w, 0u, 0u}, kGradVec)
                                                   : decode_leaf<FP16>(y4[FP16 ? 0 : u], vecq ? kGradVec : kReady);
                            a = FP16 ? decode_leaf<FP16>(v4u{x[u].x, x[u].y, 0u, 0u}, kGradVec)
                                     : decode_leaf<FP16>(x[u], vec ? kGradVec : kReady);
                            a.x += r1.x; a.y += r1.y; a.z += r1.z; a.w += r1.w;
                        } else {
                            const int kind = (((mc & mp) >> b) & 1ull) ? (vec ? kGradVec : kReady) : kResid;
                            a = decode_leaf<FP16>(x[u], kind);
                        }
                        float f[E] = {a.x, a.y, a.z, a.w};
                        tree.push(f, cnt);
                        ++cnt;
                    }
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

// Residual = widened gradient (plus +0) on the elements [ss, se) of one
// worker, whose gradient element i is src[i - soff]; with vec_ok, ss is a
// multiple of 8 and src + (ss - soff) is 16-byte aligned.
template <bool FP16>
__device__ __forceinline__ void copy_segment(gptr<void> __restrict__ src, int64_t soff, bool vec_ok,
                                             float* __restrict__ r, int64_t ss, int64_t se) {
    constexpr int UN = 4;
    const int64_t nvec = vec_ok ? (se - ss) >> 3 : 0;
    int64_t j = threadIdx.x;
    for (; j + (UN - 1) * kThreads < nvec; j += UN * kThreads) {
        float f[UN][8];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t i = ss + ((j + u * kThreads) << 3);
            if (FP16) {
                widen8(load_u4(static_cast<gptr<uint16_t>>(src) + (i - soff)), f[u]);
            } else {
                gptr<float> gp = static_cast<gptr<float>>(src) + (i - soff);
                const float4 g0 = load_f4(gp), g1 = load_f4(gp + 4);
                f[u][0] = g0.x; f[u][1] = g0.y; f[u][2] = g0.z; f[u][3] = g0.w;
                f[u][4] = g1.x; f[u][5] = g1.y; f[u][6] = g1.z; f[u][7] = g1.w;
            }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t i = ss + ((j + u * kThreads) << 3);
            *reinterpret_cast<float4*>(r + i) =
                make_float4(f[u][0] + 0.f, f[u][1] + 0.f, f[u][2] + 0.f, f[u][3] + 0.f);
            *reinterpret_cast<float4*>(r + i + 4) =
                make_float4(f[u][4] + 0.f, f[u][5] + 0.f, f[u][6] + 0.f, f[u][7] + 0.f);
        }
    }
    for (; j < nvec; j += kThreads) {
        const int64_t i = ss + (j << 3);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            r[i + q] = (FP16 ? widen1(static_cast<gptr<uint16_t>>(src)[i + q - soff])
                             : static_cast<gptr<float>>(src)[i + q - soff]) + 0.f;
    }
    for (int64_t i = ss + (nvec << 3) + threadIdx.x; i < se; i += kThreads)
        r[i] = (FP16 ? widen1(static_cast<gptr<uint16_t>>(src)[i - soff]) : static_cast<gptr<float>>(src)[i - soff]) +
               0.f;
}

// Residual = g0 + (g1 + 0) on the elements [ss, se) of one worker, g0 from
// this step's tensor src and g1 from the previous step's psrc, at the same
// offsets; with vec_ok, both are 16-byte aligned at ss.
template <bool FP16>
__device__ __forceinline__ void copy2_segment(gptr<void> __restrict__ src, gptr<void> __restrict__ psrc,
                                              int64_t soff, bool vec_ok, float* __restrict__ r, int64_t ss,
                                              int64_t se) {
    const int64_t nvec = vec_ok ? (se - ss) >> 3 : 0;
    for (int64_t j = threadIdx.x; j < nvec; j += kThreads) {
        const int64_t i = ss + (j << 3);
        float f[8], q[8];
        if (FP16) {
            widen8(load_u4(static_cast<gptr<uint16_t>>(src) + (i - soff)), f);
            widen8(load_u4(static_cast<gptr<uint16_t>>(psrc) + (i - soff)), q);
        } else {
            gptr<float> gp = static_cast<gptr<float>>(src) + (i - soff);
            gptr<float> pp = static_cast<gptr<float>>(psrc) + (i - soff);
            const float4 g0 = load_f4(gp), g1 = load_f4(gp + 4), p0 = load_f4(pp), p1 = load_f4(pp + 4);
            f[0] = g0.x; f[1] = g0.y; f[2] = g0.z; f[3] = g0.w; f[4] = g1.x; f[5] = g1.y; f[6] = g1.z; f[7] = g1.w;
            q[0] = p0.x; q[1] = p0.y; q[2] = p0.z; q[3] = p0.w; q[4] = p1.x; q[5] = p1.y; q[6] = p1.z; q[7] = p1.w;
        }
        *reinterpret_cast<float4*>(r + i) =
            make_float4(f[0] + (q[0] + 0.f), f[1] + (q[1] + 0.f), f[2] + (q[2] + 0.f), f[3] + (q[3] + 0.f));
        *reinterpret_cast<float4*>(r + i + 4) =
            make_float4(f[4] + (q[4] + 0.f), f[5] + (q[5] + 0.f), f[6] + (q[6] + 0.f), f[7] + (q[7] + 0.f));
    }
    for (int64_t i = ss + (nvec << 3) + threadIdx.x; i < se; i += kThreads) {
        const float f = FP16 ? widen1(static_cast<gptr<uint16_t>>(src)[i - soff])
                             : static_cast<gptr<float>>(src)[i - soff];
        const float q = FP16 ? widen1(static_cast<gptr<uint16_t>>(psrc)[i - soff])
                             : static_cast<gptr<float>>(psrc)[i - soff];
        r[i] = f + (q + 0.f);
    }
}

// kMatParts workgroups per (worker, 32-chunk mask word): they write, each its
// share of every chunk, the chunks of that word the worker sent in the
// previous step but not now (their residual is the widened gradient) and,
// with P2, those sent two steps back and in neither later step (their
// residual is g0 + (g1 + 0), from this step's and the previous step's
// tensors).  Most words have none or one such chunk, so the grid stays far
// smaller than one workgroup per (worker, chunk).
constexpr int kMatParts = 4;
template <bool FP16, bool P2 = false>
__global__ __launch_bounds__(kThreads) void k_materialize(const uint64_t* __restrict__ layer_ptrs,
                                                          const int64_t* __restrict__ offsets,
                                                          const uint32_t* __restrict__ tile_layer, int64_t tile_elems,
                                                          int32_t L,
                                                          float* __restrict__ resid, int64_t ld, int64_t P, int64_t C,
                                                          int32_t n_c, const uint32_t* __restrict__ prev_mask,
                                                          const uint32_t* __restrict__ sel_mask, int32_t mw,
                                                          const uint64_t* __restrict__ prev_layer_ptrs,
                                                          const uint32_t* __restrict__ prev2_mask) {
    const int64_t b = blockIdx.x / kMatParts;
    const int32_t part = (int32_t)(blockIdx.x % kMatParts);
    const int32_t w = (int32_t)(b / mw);
    const int32_t q = (int32_t)(b - (int64_t)w * mw);
    const int64_t word = (int64_t)w * mw + q;
    const uint32_t bits1 = prev_mask[word] & ~sel_mask[word];
    uint32_t bits = bits1;
    if (P2) bits |= prev2_mask[word] & ~prev_mask[word] & ~sel_mask[word];
    float* __restrict__ r = resid + (int64_t)w * ld;
    // this workgroup's share of each chunk: a multiple of 8 elements
    const int64_t share = (C / kMatParts + 7) / 8 * 8;
    while (bits != 0u) {
        const int32_t cbit = __builtin_ctz(bits);
        const int32_t c = q * 32 + cbit;
        const bool two = P2 && !((bits1 >> cbit) & 1u);
        bits &= bits - 1u;
        if (c >= n_c) break;
        const int64_t c0 = (int64_t)c * C;
        const int64_t c1 = c0 + C < P ? c0 + C : P;
        const int64_t s = c0 + part * share < c1 ? c0 + part * share : c1;
        const int64_t e = s + share < c1 ? s + share : c1;
        if (s >= e) continue;
        // the layer of s: the tile table gives the layer of its tile's first
        // element, and s lies in that layer or a later one
        int32_t lo = (int32_t)(tile_layer[s / tile_elems] & 0x7fffffffu);
        while (offsets[lo + 1] <= s) ++lo;
        for (int32_t l = lo; l < L && offsets[l] < e; ++l) {
            const int64_t off = offsets[l], end = offsets[l + 1];
            const uint64_t addr = layer_ptrs[(int64_t)w * L + l];
            const bool vec_ok = (off & 7) == 0 && (addr & 15) == 0;
            if (P2 && two) {
                const uint64_t paddr = prev_layer_ptrs[(int64_t)w * L + l];
                copy2_segment<FP16>(as_global<void>(addr), as_global<void>(paddr), off, vec_ok && (paddr & 15) == 0,
                                    r, off > s ? off : s, end < e ? end : e);
            } else {
                copy_segment<FP16>(as_global<void>(addr), off, vec_ok, r, off > s ? off : s, end < e ? end : e);
            }
        }
    }
}

// k_materialize over every (worker, mask word): the residual of each chunk
// set in prev_mask but not in sel_mask becomes the widened gradient + 0; with
// prev2_mask (the depth-2 pending form), also that of each chunk set in
// prev2_mask and in neither later mask, g0 + (g1 + 0).
hipError_t materialize_dispatch(const Plan& p, const uint64_t* layer_ptrs, float* resid,
                                const uint32_t* prev_mask, const uint32_t* sel_mask, hipStream_t s,
                                const uint64_t* prev_layer_ptrs = nullptr, const uint32_t* prev2_mask = nullptr) {
    const int64_t words = (int64_t)p.W * p.mw * kMatParts;
    if (words == 0) return hipSuccess;
#define GA_MAT_LAUNCH(F, Q)                                                                                    \
    hipLaunchKernelGGL((k_materialize<F, Q>), dim3((unsigned)words), dim3(kThreads), 0, s, layer_ptrs, p.d_offsets, \
                       p.d_tile_layer, p.tile_elems, p.L, resid, p.ld, p.P, p.C, (int32_t)p.n_c, prev_mask,    \
                       sel_mask, p.mw, prev_layer_ptrs, prev2_mask)
    const bool two = prev2_mask != nullptr;
    if (p.dtype == GA_FP16) {
        if (two) GA_MAT_LAUNCH(true, true);
        else GA_MAT_LAUNCH(true, false);
    } else {
        if (two) GA_MAT_LAUNCH(false, true);
        else GA_MAT_LAUNCH(false, false);
    }
#undef GA_MAT_LAUNCH
    return hipGetLastError();
}

template <int LEV>
hipError_t defer_dispatch(const Plan& p, const uint64_t* layer_ptrs, float* resid, const uint32_t* prev_mask,
                          const uint32_t* sel_mask, float* grad, const ga_sgd* sgd, float* w, float* v,
                          bool materialize, hipStream_t s, const uint64_t* prev_layer_ptrs = nullptr,
                          const uint32_t* prev2_mask = nullptr) {
    const int64_t threads = (p.P + 3) / 4;
    const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
    const float invW = (float)(1.0 / (double)p.W);
    const float lr = sgd ? sgd->lr : 0.f, mu = sgd ? sgd->mu : 0.f;
#define GA_GATHER_LAUNCH(F, Q)                                                                                 \
    hipLaunchKernelGGL((k_gather_defer<LEV, F, Q>), dim3(blocks), dim3(kThreads), 0, s, layer_ptrs, p.d_offsets, \
                       p.d_tile_layer, p.tile_elems, p.L, resid, p.ld, p.W, p.P, p.C, prev_mask, sel_mask, p.mw, \
                       invW, grad, sgd ? 1 : 0, lr, mu, w, v, prev_layer_ptrs, prev2_mask)
    const bool two = prev2_mask != nullptr;
    if (p.dtype == GA_FP16) {
        if (two) GA_GATHER_LAUNCH(true, true);
        else GA_GATHER_LAUNCH(true, false);
    } else {
        if (two) GA_GATHER_LAUNCH(false, true);
        else GA_GATHER_LAUNCH(false, false);
    }
#undef GA_GATHER_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !materialize) return e;
    // the (worker, chunk) pairs written here are disjoint from those the
    // reduction reads, so the order of the two launches does not matter
    return materialize_dispatch(p, layer_ptrs, resid, prev_mask, sel_mask, s);
}

}  // namespace

hipError_t launch_sparse_gather_defer(const Plan& p, const uint64_t* layer_ptrs, float* resid,
                                      const uint32_t* prev_mask, const uint32_t* sel_mask, float* grad,
                                      const ga_sgd* sgd, float* w, float* v, bool materialize, hipStream_t s) {
    if (p.P == 0) return hipSuccess;
    if (p.W < (1 << 5))
        return defer_dispatch<5>(p, layer_ptrs, resid, prev_mask, sel_mask, grad, sgd, w, v, materialize, s);
    if (p.W < (1 << 8))
        return defer_dispatch<8>(p, layer_ptrs, resid, prev_mask, sel_mask, grad, sgd, w, v, materialize, s);
    return defer_dispatch<11>(p, layer_ptrs, resid, prev_mask, sel_mask, grad, sgd, w, v, materialize, s);
}

hipError_t launch_sparse_gather_pending2(const Plan& p, const uint64_t* layer_ptrs, const uint64_t* prev_layer_ptrs,
                                         float* resid, const uint32_t* prev_mask, const uint32_t* sel_mask,
                                         const uint32_t* prev2_mask, float* grad, const ga_sgd* sgd, float* w,
                                         float* v, hipStream_t s) {
    if (p.P == 0) return hipSuccess;
    if (p.W < (1 << 5))
        return defer_dispatch<5>(p, layer_ptrs, resid, prev_mask, sel_mask, grad, sgd, w, v, false, s,
                                 prev_layer_ptrs, prev2_mask);
    if (p.W < (1 << 8))
        return defer_dispatch<8>(p, layer_ptrs, resid, prev_mask, sel_mask, grad, sgd, w, v, false, s,
                                 prev_layer_ptrs, prev2_mask);
    return defer_dispatch<11>(p, layer_ptrs, resid, prev_mask, sel_mask, grad, sgd, w, v, false, s,
                              prev_layer_ptrs, prev2_mask);
}

hipError_t launch_residual_flush(const Plan& p, const uint64_t* layer_ptrs, float* resid, const uint32_t* prev_mask,
                                 const uint32_t* sel_mask, hipStream_t s, const uint64_t* prev_layer_ptrs,
                                 const uint32_t* prev2_mask) {
    if (p.P == 0) return hipSuccess;
    return materialize_dispatch(p, layer_ptrs, resid, prev_mask, sel_mask, s, prev_layer_ptrs, prev2_mask);
}

}  // namespace ga
