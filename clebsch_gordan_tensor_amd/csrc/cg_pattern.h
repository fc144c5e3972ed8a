// Compile-time sparsity pattern of a real-basis Clebsch-Gordan block.
//
// In the real harmonic basis (cos-type for m >= 0, sin-type for m < 0) the
// product of degree-l1 and degree-l2 components only feeds |m3| in
// { |m1|+|m2|, ||m1|-|m2|| }, and the trig type obeys
//   type(m2) = type(m1) xor type(m3) xor ((l1+l2+l3) odd)
// (an odd path couples like a cross product, which swaps cos and sin). So for
// each (m1, m3) at most two m2 survive. The planner packs coefficient values
// in exactly this order and the kernels unroll exactly this order, so a
// coefficient is read once per (path, m1, m3, term) from a dense table with
// no index arrays. Zero entries allowed by the rule are kept (as 0.0).
//
// Shared between the host planner and the device kernels; it holds no values.
#pragma once

#include <utility>

#if defined(__HIPCC__)
#define CGTP_HD __host__ __device__
#else
#define CGTP_HD
#endif

namespace cgtp {

struct PairT {
  int m1, m3;  // -l..l
  int n;       // terms: 1 or 2
  int m2a, m2b;
  int coef;    // offset of the first coefficient of this pair
};

constexpr int iabs_c(int a) { return a < 0 ? -a : a; }
constexpr int sin_type(int m) { return m < 0 ? 1 : 0; }

// Candidates of m2 for (m1, m3) under the rule above; returns their count.
constexpr int m2_candidates(int l1, int l2, int l3, int m1, int m3, int* out) {
  const int t = sin_type(m1) ^ sin_type(m3) ^ ((l1 + l2 + l3) & 1);
  const int s = iabs_c(m1) + iabs_c(m3);
  const int d = iabs_c(iabs_c(m1) - iabs_c(m3));
  int n = 0;
  // ascending magnitude: d first, then s (when distinct)
  const int mags[2] = {d, s};
  const int nm = (d == s) ? 1 : 2;
  for (int k = 0; k < nm; ++k) {
    const int a = mags[k];
    if (a > l2) continue;
    if (a == 0) {
      if (t == 0) out[n++] = 0;
    } else {
      out[n++] = t ? -a : a;
    }
  }
  return n;
}

constexpr int pattern_pairs(int l1, int l2, int l3) {
  int n = 0;
  for (int m1 = -l1; m1 <= l1; ++m1)
    for (int m3 = -l3; m3 <= l3; ++m3) {
      int c[2] = {0, 0};
      if (m2_candidates(l1, l2, l3, m1, m3, c) > 0) ++n;
    }
  return n;
}

constexpr int pattern_coefs(int l1, int l2, int l3) {
  int n = 0;
  for (int m1 = -l1; m1 <= l1; ++m1)
    for (int m3 = -l3; m3 <= l3; ++m3) {
      int c[2] = {0, 0};
      n += m2_candidates(l1, l2, l3, m1, m3, c);
    }
  return n;
}

// Largest coefficient count of one pattern with every degree <= lmax.
constexpr int max_pattern_coefs(int lmax) {
  int m = 0;
  for (int l1 = 0; l1 <= lmax; ++l1)
    for (int l2 = 0; l2 <= lmax; ++l2)
      for (int l3 = iabs_c(l1 - l2); l3 <= l1 + l2 && l3 <= lmax; ++l3) {
        const int n = pattern_coefs(l1, l2, l3);
        m = n > m ? n : m;
      }
  return m;
}

template <int L1, int L2, int L3>
struct Pattern {
  static constexpr int NP = pattern_pairs(L1, L2, L3);
  static constexpr int NC = pattern_coefs(L1, L2, L3);
  struct Arr {
    PairT p[NP > 0 ? NP : 1];
  };
  static constexpr Arr build() {
    Arr a{};
    int k = 0, coef = 0;
    for (int m1 = -L1; m1 <= L1; ++m1)
      for (int m3 = -L3; m3 <= L3; ++m3) {
        int c[2] = {0, 0};
        const int n = m2_candidates(L1, L2, L3, m1, m3, c);
        if (n == 0) continue;
        a.p[k] = PairT{m1, m3, n, c[0], n > 1 ? c[1] : c[0], coef};
        coef += n;
        ++k;
      }
    return a;
  }
  static constexpr Arr arr = build();
};

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
CGTP_HD inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(static_cast<F&&>(f));
  }
}

}  // namespace cgtp
