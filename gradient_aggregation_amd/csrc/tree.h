// The fixed binary reduction tree, evaluated in registers.
//
// FireCaffe (paperlayer summary, sec. 6) aggregates gradients with a binary
// tree: branching factor 2, depth log2(p).  The tree used here adds adjacent
// nodes level by level and carries an odd last node up, which is the same as
//   T(lo,1) = leaf lo,   T(lo,n) = T(lo,h) + T(lo+h,n-h),  h = 2^floor(log2(n-1)).
//
// Streaming form.  Leaves arrive in worker order.  acc[l] holds a finished
// subtree of 2^l leaves while bit l of the number of leaves pushed so far is
// set.  Pushing a leaf is a binary increment: the new leaf is merged with the
// pending subtrees of the low set bits (left operand = earlier subtree) until a
// clear bit is found, where the merged subtree is parked.  After all W leaves,
// the pending subtrees sit at the set bits of W, largest (leftmost workers) at
// the highest bit; folding them from the lowest level up gives T(0,W) exactly,
// because T splits off the largest power-of-two prefix at each level.
//
// Every branch depends only on the leaf count, which is uniform across a
// wavefront, so the merges compile to scalar branches and acc stays in VGPRs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

// Nearest binary16 value of a binary32 value (round to nearest even), as binary32.
__device__ __forceinline__ float round_f16(float x) { return (float)(_Float16)x; }

// WIRE: every subtree sum that travels to another worker is binary16 - the
// right operand of each add is rounded to binary16 first (the left operand is
// the receiving worker's own partial sum and stays binary32).
template <int LEV, int E, bool WIRE = false>
struct TreeAcc {
    float acc[LEV][E];

    // Push leaf number `cnt` (0-based).  x is consumed.  The levels are
    // expanded by template recursion so that every index is a constant and
    // acc stays in registers.
    __device__ __forceinline__ void push(float (&x)[E], uint32_t cnt) { push_from<0>(x, cnt); }

    // T(0, W) after W pushes (1 <= W < 2^LEV).
    __device__ __forceinline__ void result(uint32_t W, float (&out)[E]) const {
        fold_from<0>(W, out, false);
    }

   private:
    template <int L>
    __device__ __forceinline__ void push_from(float (&x)[E], uint32_t cnt) {
        if constexpr (L < LEV) {
            if (cnt & (1u << L)) {
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = acc[L][e] + (WIRE ? round_f16(x[e]) : x[e]);
                push_from<L + 1>(x, cnt);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) acc[L][e] = x[e];
            }
        }
    }

    template <int L>
    __device__ __forceinline__ void fold_from(uint32_t W, float (&out)[E], bool have) const {
        if constexpr (L < LEV) {
            if (W & (1u << L)) {
                if (!have) {
#pragma unroll
                    for (int e = 0; e < E; ++e) out[e] = acc[L][e];
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) out[e] = acc[L][e] + (WIRE ? round_f16(out[e]) : out[e]);
                }
                have = true;
            }
            fold_from<L + 1>(W, out, have);
        }
    }
};

// Levels needed for W workers: W < 2^LEV.
__host__ __device__ constexpr int tree_levels_for(int W) {
    int l = 1;
    while ((1 << l) <= W) ++l;
    return l;
}

}  // namespace ga
