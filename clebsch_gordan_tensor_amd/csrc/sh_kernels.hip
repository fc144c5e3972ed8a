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
// T_0 = 1, built by complex multiplication.
//
// One thread per vector, every degree unrolled at compile time. Rows of the
// [n][(L+1)^2] outputs (and grad inputs) go through LDS so that global memory
// is touched with consecutive lanes on consecutive words.
#include "cg_pattern.h"
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
constexpr double dfact(int k) {  // (2k-1)!!
  double r = 1.0;
  for (int j = 1; j <= 2 * k - 1; j += 2) r *= j;
  return r;
}

// Q[l][k] = d^k P_l / dz^k at z for 0 <= k <= l <= N-1 (zero for k > l).
// Q_k^k = (2k-1)!!, Q_{k+1}^k = (2k+1) z Q_k^k,
// (l-k) Q_l^k = (2l-1) z Q_{l-1}^k - (l+k-1) Q_{l-2}^k.
template <int N, typename A>
__device__ __forceinline__ void legendre_derivs(A z, A (&Q)[N][N]) {
  static_for<0, N>([&](auto Kc) {
    constexpr int k = decltype(Kc)::value;
    static_for<0, N>([&](auto Lc) {
      constexpr int l = decltype(Lc)::value;
      if constexpr (l < k) {
        Q[l][k] = A(0);
      } else if constexpr (l == k) {
        constexpr double d = dfact(k);
        Q[l][k] = A(d);
      } else if constexpr (l == k + 1) {
        constexpr double d = (2 * k + 1) * dfact(k);
        Q[l][k] = A(d) * z;
      } else {
        constexpr double a = double(2 * l - 1) / double(l - k), b = double(l + k - 1) / double(l - k);
        Q[l][k] = A(a) * z * Q[l - 1][k] - A(b) * Q[l - 2][k];
      }
    });
  });
}

template <int L, typename A>
__device__ __forceinline__ void powers(A x, A y, A (&c)[L + 1], A (&s)[L + 1]) {
  c[0] = A(1);
  s[0] = A(0);
  static_for<1, L + 1>([&](auto Mc) {
    constexpr int m = decltype(Mc)::value;
    c[m] = c[m - 1] * x - s[m - 1] * y;
    s[m] = c[m - 1] * y + s[m - 1] * x;
  });
}

template <typename T, typename A, int L>
__global__ __launch_bounds__(kShThreads) void sh_fwd_kernel(const T* __restrict__ vec, T* __restrict__ out,
                                                            int64_t n) {
  constexpr int D = (L + 1) * (L + 1);
  constexpr int P = D | 1;  // odd LDS row pitch: conflict-free per-thread rows
  __shared__ A tile[kShThreads * P];
  const int64_t base = int64_t(blockIdx.x) * kShThreads;
  const int64_t i = base + threadIdx.x;
  A* row = tile + threadIdx.x * P;
  if (i < n) {
    A x = to_acc<A>(vec[3 * i]), y = to_acc<A>(vec[3 * i + 1]), z = to_acc<A>(vec[3 * i + 2]);
    const A r2 = x * x + y * y + z * z;
    if (r2 == A(0)) {
      row[0] = A(1);
      static_for<1, D>([&](auto K) { row[decltype(K)::value] = A(0); });
    } else {
      const A inv = A(1) / sqrt(r2);
      x *= inv;
      y *= inv;
      z *= inv;
      A Q[L + 1][L + 1];
      legendre_derivs<L + 1, A>(z, Q);
      A c[L + 1], s[L + 1];
      powers<L, A>(x, y, c, s);
      static_for<0, L + 1>([&](auto Lc) {
        constexpr int l = decltype(Lc)::value;
        static_for<0, 2 * l + 1>([&](auto Mi) {
          constexpr int m = int(decltype(Mi)::value) - l;
          constexpr int k = m < 0 ? -m : m;
          constexpr double nrm = norm_lk(l, k);
          const A t = m > 0 ? c[k] : (m < 0 ? s[k] : A(1));
          row[l * l + l + m] = A(nrm) * Q[l][k] * t;
        });
      });
    }
  }
  __syncthreads();
  const int64_t rows = n - base < kShThreads ? n - base : kShThreads;
  T* o = out + base * D;
  for (int k = threadIdx.x; k < rows * D; k += kShThreads) from_acc(o[k], tile[(k / D) * P + (k % D)]);
}

template <typename T, typename A, int L>
__global__ __launch_bounds__(kShThreads) void sh_bwd_kernel(const T* __restrict__ vec, const T* __restrict__ gsh,
                                                            T* __restrict__ gvec, int64_t n) {
  constexpr int D = (L + 1) * (L + 1);
  constexpr int P = D | 1;
  __shared__ A tile[kShThreads * P];
  const int64_t base = int64_t(blockIdx.x) * kShThreads;
  const int64_t rows = n - base < kShThreads ? n - base : kShThreads;
  const T* g = gsh + base * D;
  for (int k = threadIdx.x; k < rows * D; k += kShThreads) tile[(k / D) * P + (k % D)] = to_acc<A>(g[k]);
  __syncthreads();
  const int64_t i = base + threadIdx.x;
  if (i >= n) return;
  const A* grow = tile + threadIdx.x * P;
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
  legendre_derivs<L + 2, A>(z, Q);
  A c[L + 1], s[L + 1];
  powers<L, A>(x, y, c, s);
  // gradient of the Cartesian polynomial at the unit vector
  A gx = A(0), gy = A(0), gz = A(0);
  static_for<0, L + 1>([&](auto Lc) {
    constexpr int l = decltype(Lc)::value;
    static_for<0, 2 * l + 1>([&](auto Mi) {
      constexpr int m = int(decltype(Mi)::value) - l;
      constexpr int k = m < 0 ? -m : m;
      constexpr double nrm = norm_lk(l, k);
      const A gv = grow[l * l + l + m] * A(nrm);
      if constexpr (m == 0) {
        gz += gv * Q[l][1];
      } else if constexpr (m > 0) {  // d Re(w^k)/dx = k Re(w^{k-1}), d/dy = -k Im(w^{k-1})
        gx += gv * Q[l][k] * A(k) * c[k - 1];
        gy -= gv * Q[l][k] * A(k) * s[k - 1];
        gz += gv * Q[l][k + 1] * c[k];
      } else {  // d Im(w^k)/dx = k Im(w^{k-1}), d/dy = k Re(w^{k-1})
        gx += gv * Q[l][k] * A(k) * s[k - 1];
        gy += gv * Q[l][k] * A(k) * c[k - 1];
        gz += gv * Q[l][k + 1] * s[k];
      }
    });
  });
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
  static_for<0, kLmax + 1>([&](auto Lc) {
    constexpr int L = decltype(Lc)::value;
    if (lmax == L) hipLaunchKernelGGL((sh_fwd_kernel<T, A, L>), grid, dim3(kShThreads), 0, s, v, o, n);
  });
  CGTP_CHECK_HIP(hipGetLastError());
}

template <typename T>
void sh_bwd_typed(int lmax, int64_t n, const void* vec, const void* gsh, void* gvec, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const dim3 grid(unsigned((n + kShThreads - 1) / kShThreads));
  const T* v = static_cast<const T*>(vec);
  const T* g = static_cast<const T*>(gsh);
  T* o = static_cast<T*>(gvec);
  static_for<0, kLmax + 1>([&](auto Lc) {
    constexpr int L = decltype(Lc)::value;
    if (lmax == L) hipLaunchKernelGGL((sh_bwd_kernel<T, A, L>), grid, dim3(kShThreads), 0, s, v, g, o, n);
  });
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
