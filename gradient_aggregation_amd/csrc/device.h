// Device helpers shared by the kernels of libgradagg.so: the SGD update,
// global-memory pointer typing, 128-bit loads and binary16 widening.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

// Momentum SGD, Caffe form, three binary32 roundings (the library is built
// with -ffp-contract=off, so no multiply-add is fused).
__device__ __forceinline__ void sgd_update(float g, float lr, float mu, float& w, float& v) {
    float a = mu * v;
    float b = lr * g;
    v = a + b;
    w = w - v;
}

// A device address held as an integer (e.g. read from a layer table), typed as
// a global-memory pointer so that loads through it compile to global (not
// flat) instructions.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

template <typename T>
__device__ __forceinline__ gptr<T> as_global(uint64_t addr) {
    return reinterpret_cast<gptr<T>>(addr);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 128-bit loads through a global-memory pointer (16-byte aligned).
__device__ __forceinline__ uint4 load_u4(gptr<void> p) {
    const u32x4 x = *reinterpret_cast<gptr<u32x4>>(p);
    return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ float4 load_f4(gptr<void> p) {
    const f32x4 x = *reinterpret_cast<gptr<f32x4>>(p);
    return make_float4(x.x, x.y, x.z, x.w);
}

// binary16 -> binary32 widening (exact, subnormals included) of 8 packed values.
__device__ __forceinline__ void widen8(const uint4& r, float (&f)[8]) {
    const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[j] & 0xffffu));
        f[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[j] >> 16));
    }
}

__device__ __forceinline__ float widen1(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

}  // namespace ga
