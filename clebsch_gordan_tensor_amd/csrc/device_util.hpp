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

// Value of v in lane (this lane ^ off) of the wave, for a precomputed byte
// address (lane ^ off) * 4; the source lane must be active.
__device__ __forceinline__ float lane_fetch(float v, int addr) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}
__device__ __forceinline__ double lane_fetch(double v, int addr) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_ds_bpermute(addr, int(b & 0xffffffffll));
  const int hi = __builtin_amdgcn_ds_bpermute(addr, int(b >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// Butterfly sums of N values over lane strides off_begin, 2*off_begin, ...
// < off_end (powers of two <= 64): with [1, G) every aligned group of G lanes
// ends with its total in all its lanes. The N exchanges of a step are issued
// together, so a step costs one exchange latency, not N.
template <int N, typename A>
__device__ __forceinline__ void xor_sum_n(A (&v)[N], int off_begin, int off_end) {
  const int lane = int(threadIdx.x & 63);
  for (int off = off_begin; off < off_end; off <<= 1) {
    const int addr = (lane ^ off) << 2;
    A t[N];
#pragma unroll
    for (int k = 0; k < N; ++k) t[k] = lane_fetch(v[k], addr);
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += t[k];
  }
}

}  // namespace cgtp
