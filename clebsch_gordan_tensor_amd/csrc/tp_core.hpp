// Per-path tensor-product core shared by the row kernels and the convolution.
//
// For one path (l1, l2, l3) and VEC channels of one lane:
//   o[m3][v] = sum over the pattern's (m1, m3) pairs of
//              (sum_m2 C[m1, m2, m3] y[m2]) * x[m1][v]
// with the pairs and coefficient offsets fixed at compile time (cg_pattern.h)
// and the coefficient values read from the plan's packed table.
#pragma once

#include "cg_pattern.h"
#include "device_util.hpp"

namespace cgtp {

template <int L1, int L2, int L3, int VEC, typename A>
__device__ __forceinline__ void fwd_core(const A (&xb)[2 * L1 + 1][VEC], const A (&yb)[2 * L2 + 1],
                                         const A* __restrict__ cf, A (&o)[2 * L3 + 1][VEC]) {
  using P = Pattern<L1, L2, L3>;
#pragma unroll
  for (int m = 0; m < 2 * L3 + 1; ++m)
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[m][v] = A(0);
  static_for<0, P::NP>([&](auto I) {
    constexpr PairT pr = P::arr.p[decltype(I)::value];
    A a = ldc(cf + pr.coef) * yb[pr.m2a + L2];
    if constexpr (pr.n == 2) a = fma(ldc(cf + pr.coef + 1), yb[pr.m2b + L2], a);
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[pr.m3 + L3][v] = fma(a, xb[pr.m1 + L1][v], o[pr.m3 + L3][v]);
  });
}

}  // namespace cgtp
