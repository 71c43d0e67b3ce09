// Small device helpers shared by the HIP kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte vector of T: 8 bf16 or 4 fp32.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
    static constexpr int n = 8;
    typedef bf16x8 type;
};
template <> struct Vec16<float> {
    static constexpr int n = 4;
    typedef f32x4 type;
};

template <typename T>
__device__ __forceinline__ void load16_f32(const T* p, float* out) {
    typedef typename Vec16<T>::type V;
    V v = *reinterpret_cast<const V*>(p);
#pragma unroll
    for (int i = 0; i < Vec16<T>::n; ++i) out[i] = static_cast<float>(v[i]);
}

template <typename T>
__device__ __forceinline__ void store16_f32(T* p, const float* in) {
    typedef typename Vec16<T>::type V;
    V v;
#pragma unroll
    for (int i = 0; i < Vec16<T>::n; ++i) v[i] = static_cast<T>(in[i]);  // RNE for bf16
    *reinterpret_cast<V*>(p) = v;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace ssd
