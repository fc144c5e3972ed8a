// Device helpers: storage types, per-lane vector loads/stores, lane reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cgtp {

// bfloat16 storage; arithmetic is done in fp32.
struct bf16 {
  uint16_t bits;
};

template <typename T>
struct AccOf {
  using type = float;
};
template <>
struct AccOf<double> {
  using type = double;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round to nearest, ties to even (gfx950 converts in hardware: two values per
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

template <typename A>
__device__ __forceinline__ A to_acc(float v) { return A(v); }
template <typename A>
__device__ __forceinline__ A to_acc(double v) { return A(v); }
template <typename A>
__device__ __forceinline__ A to_acc(bf16 v) { return A(bf16_to_f32(v.bits)); }

__device__ __forceinline__ void from_acc(float& d, float v) { d = v; }
__device__ __forceinline__ void from_acc(double& d, double v) { d = v; }
__device__ __forceinline__ void from_acc(bf16& d, float v) { d.bits = f32_to_bf16(v); }

// VEC consecutive elements per lane; pointer aligned to VEC * sizeof(T).
template <typename T, int VEC>
struct VecIO;

template <int VEC>
struct VecIO<float, VEC> {
  typedef float V __attribute__((ext_vector_type(VEC)));
  __device__ static __forceinline__ void load(const float* p, float (&o)[VEC]) {
    const V v = *reinterpret_cast<const V*>(p);
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = v[i];
  }
  __device__ static __forceinline__ void store(float* p, const float (&o)[VEC]) {
    V v;
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = o[i];
    *reinterpret_cast<V*>(p) = v;
  }
  __device__ static __forceinline__ void store_nt(float* p, const float (&o)[VEC]) {
    V v;
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = o[i];
    __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  }
};
template <>
struct VecIO<float, 1> {
  __device__ static __forceinline__ void load(const float* p, float (&o)[1]) { o[0] = *p; }
  __device__ static __forceinline__ void store(float* p, const float (&o)[1]) { *p = o[0]; }
  __device__ static __forceinline__ void store_nt(float* p, const float (&o)[1]) {
    __builtin_nontemporal_store(o[0], p);
  }
};

template <int VEC>
struct VecIO<double, VEC> {
  typedef double V __attribute__((ext_vector_type(VEC)));
  __device__ static __forceinline__ void load(const double* p, double (&o)[VEC]) {
    const V v = *reinterpret_cast<const V*>(p);
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = v[i];
  }
  __device__ static __forceinline__ void store(double* p, const double (&o)[VEC]) {
    V v;
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = o[i];
    *reinterpret_cast<V*>(p) = v;
  }
  __device__ static __forceinline__ void store_nt(double* p, const double (&o)[VEC]) {
    V v;
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = o[i];
    __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  }
};
template <>
struct VecIO<double, 1> {
  __device__ static __forceinline__ void load(const double* p, double (&o)[1]) { o[0] = *p; }
  __device__ static __forceinline__ void store(double* p, const double (&o)[1]) { *p = o[0]; }
  __device__ static __forceinline__ void store_nt(double* p, const double (&o)[1]) {
    __builtin_nontemporal_store(o[0], p);
  }
};

template <int VEC>
struct VecIO<bf16, VEC> {
  typedef uint16_t V __attribute__((ext_vector_type(VEC)));
  __device__ static __forceinline__ void load(const bf16* p, float (&o)[VEC]) {
    const V v = *reinterpret_cast<const V*>(p);
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = bf16_to_f32(v[i]);
  }
  __device__ static __forceinline__ void store(bf16* p, const float (&o)[VEC]) {
    V v;
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = f32_to_bf16(o[i]);
    *reinterpret_cast<V*>(p) = v;
  }
  __device__ static __forceinline__ void store_nt(bf16* p, const float (&o)[VEC]) {
    V v;
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = f32_to_bf16(o[i]);
    __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
  }
};
template <>
struct VecIO<bf16, 1> {
  __device__ static __forceinline__ void load(const bf16* p, float (&o)[1]) { o[0] = bf16_to_f32(p->bits); }
  __device__ static __forceinline__ void store(bf16* p, const float (&o)[1]) { p->bits = f32_to_bf16(o[0]); }
  __device__ static __forceinline__ void store_nt(bf16* p, const float (&o)[1]) {
    __builtin_nontemporal_store(f32_to_bf16(o[0]), &p->bits);
  }
};

// Read-only plan data (CG coefficients, path and slot tables) through the
// constant address space: the same address in every lane becomes one scalar
// load into SGPRs instead of one vector load per lane.
template <typename T>
__device__ __forceinline__ T ldc(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "ldc reads whole 32-bit words");
  constexpr int n = int(sizeof(T) / 4);
  const __attribute__((address_space(4))) uint32_t* q = (const __attribute__((address_space(4))) uint32_t*)(p);
  uint32_t w[n];
#pragma unroll
  for (int i = 0; i < n; ++i) w[i] = q[i];
  T r;
  __builtin_memcpy(&r, w, sizeof(T));
  return r;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64);
// every lane of a group receives the group's total.
template <typename A>
__device__ __forceinline__ A group_sum(A v, int width) {
  for (int off = 1; off < width; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace cgtp
