// Real spherical harmonics of edge vectors and their vector-Jacobian product.
//
// The harmonic embedding of a direction (MolSSI e3nn course, lesson 02b),
// component-normalised as in e3nn_mlx "Modular v2106 point models"; the
// e^{i m phi} / (x + iy)^m structure of "E3J: An Efficient and Open-Source
// Backend for Euclidean Equivariant Operations on GPU and TPU", appendix G.1.
// For a unit vector (x, y, z):
//   Y_lm = sqrt(2l+1) sqrt((l-|m|)!/(l+|m|)!) Q_l^{|m|}(z) T_m
// with Q_l^k the k-th derivative of the Legendre polynomial, built by the
// three-term recurrence in l, and T_m = sqrt2 Re/Im (x+iy)^|m| (m >0 / <0),
// T_0 = 1, built by complex multiplication. One thread per vector; degrees
// are unrolled at compile time (lmax <= CGTP_LMAX).
#include "device_util.hpp"
#include "graph.hpp"

namespace cgtp {

namespace {

constexpr int kShThreads = 256;

constexpr double c_fact(int n) { return n <= 1 ? 1.0 : n * c_fact(n - 1); }
constexpr double c_sqrt(double x) {
  double r = x > 1 ? x : 1.0;
  for (int i = 0; i < 100; ++i) r = 0.5 * (r + x / r);
  return r;
}
// sqrt(2l+1) sqrt((l-k)!/(l+k)!), times sqrt2 for k > 0
constexpr double norm_lk(int l, int k) {
  return c_sqrt(2.0 * l + 1.0) * c_sqrt(c_fact(l - k) / c_fact(l + k)) * (k > 0 ? c_sqrt(2.0) : 1.0);
}

// Q[l][k] = d^k P_l / dz^k at z, 0 <= k <= l <= L (and 0 for k > l).
template <int L, typename A>
__device__ __forceinline__ void legendre_derivs(A z, A (&Q)[L + 2][L + 2]) {
#pragma unroll
  for (int l = 0; l < L + 2; ++l)
#pragma unroll
    for (int k = 0; k < L + 2; ++k) Q[l][k] = A(0);
  // Q_k^k = (2k-1)!!, Q_{k+1}^k = (2k+1) z Q_k^k,
  // (l-k) Q_l^k = (2l-1) z Q_{l-1}^k - (l+k-1) Q_{l-2}^k
#pragma unroll
  for (int k = 0; k <= L + 1; ++k) {
    A dd = A(1);
#pragma unroll
    for (int j = 1; j <= 2 * k - 1; j += 2) dd *= A(j);
    if (k <= L + 1) Q[k][k] = dd;
    if (k + 1 <= L + 1) Q[k + 1][k] = A(2 * k + 1) * z * dd;
#pragma unroll
    for (int l = k + 2; l <= L + 1; ++l)
      Q[l][k] = (A(2 * l - 1) * z * Q[l - 1][k] - A(l + k - 1) * Q[l - 2][k]) / A(l - k);
  }
}

template <typename T, typename A, int L>
__global__ __launch_bounds__(kShThreads) void sh_fwd_kernel(const T* __restrict__ vec, T* __restrict__ out,
                                                            int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * kShThreads + threadIdx.x;
  if (i >= n) return;
  constexpr int D = (L + 1) * (L + 1);
  A x = to_acc<A>(vec[3 * i]), y = to_acc<A>(vec[3 * i + 1]), z = to_acc<A>(vec[3 * i + 2]);
  const A r2 = x * x + y * y + z * z;
  T* o = out + i * D;
  if (r2 == A(0)) {
    from_acc(o[0], A(1));
#pragma unroll
    for (int k = 1; k < D; ++k) from_acc(o[k], A(0));
    return;
  }
  const A inv = A(1) / sqrt(r2);
  x *= inv;
  y *= inv;
  z *= inv;
  A Q[L + 2][L + 2];
  legendre_derivs<L, A>(z, Q);
  A c[L + 1], s[L + 1];  // Re, Im of (x + iy)^m
  c[0] = A(1);
  s[0] = A(0);
#pragma unroll
  for (int m = 1; m <= L; ++m) {
    c[m] = c[m - 1] * x - s[m - 1] * y;
    s[m] = c[m - 1] * y + s[m - 1] * x;
  }
#pragma unroll
  for (int l = 0; l <= L; ++l) {
#pragma unroll
    for (int m = -l; m <= l; ++m) {
      const int k = m < 0 ? -m : m;
      const A t = m > 0 ? c[k] : (m < 0 ? s[k] : A(1));
      from_acc(o[l * l + l + m], A(norm_lk(l, k)) * Q[l][k] * t);
    }
  }
}

template <typename T, typename A, int L>
__global__ __launch_bounds__(kShThreads) void sh_bwd_kernel(const T* __restrict__ vec, const T* __restrict__ gsh,
                                                            T* __restrict__ gvec, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * kShThreads + threadIdx.x;
  if (i >= n) return;
  constexpr int D = (L + 1) * (L + 1);
  A x = to_acc<A>(vec[3 * i]), y = to_acc<A>(vec[3 * i + 1]), z = to_acc<A>(vec[3 * i + 2]);
  const A r2 = x * x + y * y + z * z;
  T* go = gvec + 3 * i;
  if (r2 == A(0)) {
    from_acc(go[0], A(0));
    from_acc(go[1], A(0));
    from_acc(go[2], A(0));
    return;
  }
  const A rinv = A(1) / sqrt(r2);
  x *= rinv;
  y *= rinv;
  z *= rinv;
  A Q[L + 2][L + 2];
  legendre_derivs<L, A>(z, Q);
  A c[L + 1], s[L + 1];
  c[0] = A(1);
  s[0] = A(0);
#pragma unroll
  for (int m = 1; m <= L; ++m) {
    c[m] = c[m - 1] * x - s[m - 1] * y;
    s[m] = c[m - 1] * y + s[m - 1] * x;
  }
  // gradient of the polynomial P(x, y, z) at the unit vector
  A gx = A(0), gy = A(0), gz = A(0);
  const T* g = gsh + i * D;
#pragma unroll
  for (int l = 0; l <= L; ++l) {
#pragma unroll
    for (int m = -l; m <= l; ++m) {
      const int k = m < 0 ? -m : m;
      const A gv = to_acc<A>(g[l * l + l + m]) * A(norm_lk(l, k));
      A t, tx, ty;
      if (m == 0) {
        t = A(1);
        tx = A(0);
        ty = A(0);
      } else if (m > 0) {  // d Re(w^k)/dx = k Re(w^{k-1}), d/dy = -k Im(w^{k-1})
        t = c[k];
        tx = A(k) * c[k - 1];
        ty = -A(k) * s[k - 1];
      } else {  // d Im(w^k)/dx = k Im(w^{k-1}), d/dy = k Re(w^{k-1})
        t = s[k];
        tx = A(k) * s[k - 1];
        ty = A(k) * c[k - 1];
      }
      gx += gv * Q[l][k] * tx;
      gy += gv * Q[l][k] * ty;
      gz += gv * Q[l][k + 1] * t;
    }
  }
  // d/dvec of a function of vec/|vec|: tangential part divided by |vec|
  const A rad = x * gx + y * gy + z * gz;
  from_acc(go[0], (gx - x * rad) * rinv);
  from_acc(go[1], (gy - y * rad) * rinv);
  from_acc(go[2], (gz - z * rad) * rinv);
}

template <typename T>
void sh_fwd_typed(int lmax, int64_t n, const void* vec, void* sh, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const dim3 grid(unsigned((n + kShThreads - 1) / kShThreads));
  const T* v = static_cast<const T*>(vec);
  T* o = static_cast<T*>(sh);
  switch (lmax) {
    case 0: hipLaunchKernelGGL((sh_fwd_kernel<T, A, 0>), grid, dim3(kShThreads), 0, s, v, o, n); break;
    case 1: hipLaunchKernelGGL((sh_fwd_kernel<T, A, 1>), grid, dim3(kShThreads), 0, s, v, o, n); break;
    case 2: hipLaunchKernelGGL((sh_fwd_kernel<T, A, 2>), grid, dim3(kShThreads), 0, s, v, o, n); break;
    case 3: hipLaunchKernelGGL((sh_fwd_kernel<T, A, 3>), grid, dim3(kShThreads), 0, s, v, o, n); break;
    default: hipLaunchKernelGGL((sh_fwd_kernel<T, A, 4>), grid, dim3(kShThreads), 0, s, v, o, n); break;
  }
  CGTP_CHECK_HIP(hipGetLastError());
}

template <typename T>
void sh_bwd_typed(int lmax, int64_t n, const void* vec, const void* gsh, void* gvec, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const dim3 grid(unsigned((n + kShThreads - 1) / kShThreads));
  const T* v = static_cast<const T*>(vec);
  const T* g = static_cast<const T*>(gsh);
  T* o = static_cast<T*>(gvec);
  switch (lmax) {
    case 0: hipLaunchKernelGGL((sh_bwd_kernel<T, A, 0>), grid, dim3(kShThreads), 0, s, v, g, o, n); break;
    case 1: hipLaunchKernelGGL((sh_bwd_kernel<T, A, 1>), grid, dim3(kShThreads), 0, s, v, g, o, n); break;
    case 2: hipLaunchKernelGGL((sh_bwd_kernel<T, A, 2>), grid, dim3(kShThreads), 0, s, v, g, o, n); break;
    case 3: hipLaunchKernelGGL((sh_bwd_kernel<T, A, 3>), grid, dim3(kShThreads), 0, s, v, g, o, n); break;
    default: hipLaunchKernelGGL((sh_bwd_kernel<T, A, 4>), grid, dim3(kShThreads), 0, s, v, g, o, n); break;
  }
  CGTP_CHECK_HIP(hipGetLastError());
}

}  // namespace

void sh_forward_launch(int lmax, cgtp_dtype dtype, int64_t n, const void* vec, void* sh, hipStream_t s) {
  switch (dtype) {
    case CGTP_F32: sh_fwd_typed<float>(lmax, n, vec, sh, s); break;
    case CGTP_F64: sh_fwd_typed<double>(lmax, n, vec, sh, s); break;
    case CGTP_BF16: sh_fwd_typed<bf16>(lmax, n, vec, sh, s); break;
  }
}

void sh_backward_launch(int lmax, cgtp_dtype dtype, int64_t n, const void* vec, const void* grad_sh,
                        void* grad_vec, hipStream_t s) {
  switch (dtype) {
    case CGTP_F32: sh_bwd_typed<float>(lmax, n, vec, grad_sh, grad_vec, s); break;
    case CGTP_F64: sh_bwd_typed<double>(lmax, n, vec, grad_sh, grad_vec, s); break;
    case CGTP_BF16: sh_bwd_typed<bf16>(lmax, n, vec, grad_sh, grad_vec, s); break;
  }
}

}  // namespace cgtp
