// Planner: irreps parsing, path enumeration, Clebsch-Gordan tables.
//
// Irreps strings and the parity rule: MolSSI e3nn course, lessons 02a and 03a.
// CG values: the construction of "E3J: An Efficient and Open-Source Backend
// for Euclidean Equivariant Operations on GPU and TPU", appendix G.2 - the
// top-weight vector of each coupled degree solves the raising-operator
// condition (a triangular, here bidiagonal, system) and every lower weight
// follows by applying the lowering operator and normalising. The complex
// (Condon-Shortley) result is then taken to the real harmonic basis.
#include <algorithm>
#include <cctype>
#include <cmath>
#include <complex>
#include <cstring>
#include <map>
#include <memory>
#include <set>
#include <utility>

#include "cg_pattern.h"
#include "common.hpp"
#include "linear.hpp"

namespace cgtp {

namespace {

Error parse_error(const std::string& s, const std::string& why) {
  return Error{CGTP_ERR_PARSE, "irreps '" + s + "': " + why};
}

std::vector<Irrep> parse_irreps(const char* cstr) {
  std::string s;
  for (const char* c = cstr; *c; ++c)
    if (!std::isspace(static_cast<unsigned char>(*c))) s.push_back(*c);
  std::vector<Irrep> out;
  if (s.empty()) return out;
  size_t pos = 0;
  while (true) {
    size_t end = s.find('+', pos);
    std::string t = s.substr(pos, end == std::string::npos ? std::string::npos : end - pos);
    if (t.empty()) throw parse_error(cstr, "empty term");
    long mul = 1;
    size_t i = 0;
    size_t xpos = t.find('x');
    if (xpos != std::string::npos) {
      if (xpos == 0) throw parse_error(cstr, "missing multiplicity before 'x'");
      for (size_t k = 0; k < xpos; ++k)
        if (!std::isdigit(static_cast<unsigned char>(t[k]))) throw parse_error(cstr, "bad multiplicity");
      if (xpos > 9) throw parse_error(cstr, "multiplicity too large");
      mul = std::stol(t.substr(0, xpos));
      i = xpos + 1;
    }
    size_t j = i;
    while (j < t.size() && std::isdigit(static_cast<unsigned char>(t[j]))) ++j;
    if (j == i || j > i + 4) throw parse_error(cstr, "bad degree in '" + t + "'");
    if (j + 1 != t.size() || (t[j] != 'e' && t[j] != 'o'))
      throw parse_error(cstr, "term '" + t + "' must end in e or o");
    if (mul < 1) throw parse_error(cstr, "multiplicity must be >= 1");
    out.push_back(Irrep{static_cast<int>(mul), std::stoi(t.substr(i, j - i)), t[j] == 'e' ? 1 : -1});
    if (end == std::string::npos) break;
    pos = end + 1;
  }
  return out;
}

// ladder coefficients: J+|j m> = up(j,m)|j m+1>, J-|j m> = dn(j,m)|j m-1>
double up(int j, int m) { return std::sqrt(double(j) * (j + 1) - double(m) * (m + 1)); }
double dn(int j, int m) { return std::sqrt(double(j) * (j + 1) - double(m) * (m - 1)); }

// Complex CG block <j1 m1 j2 m2 | J M> as dense [2j1+1][2j2+1][2J+1].
std::vector<double> complex_cg_ladder(int j1, int j2, int J) {
  const int n1 = 2 * j1 + 1, n2 = 2 * j2 + 1, n3 = 2 * J + 1;
  std::vector<double> C(size_t(n1) * n2 * n3, 0.0);
  auto at = [&](int m1, int m2, int M) -> double& {
    return C[(size_t(m1 + j1) * n2 + (m2 + j2)) * n3 + (M + J)];
  };
  // Top weight |J J> = sum_m1 a[m1] |m1>|J-m1>. The raising condition
  // (J1+ + J2+)|J J> = 0 couples neighbours only: for every k,
  //   a[k-1] up(j1, k-1) + a[k] up(j2, J-k) = 0,
  // solved upward from the lowest allowed m1.
  const int lo = std::max(-j1, J - j2), hi = std::min(j1, J + j2);
  std::vector<double> a(size_t(hi - lo + 1), 0.0);
  a[0] = 1.0;
  for (int k = lo + 1; k <= hi; ++k)
    a[size_t(k - lo)] = -a[size_t(k - 1 - lo)] * up(j1, k - 1) / up(j2, J - k);
  double nrm = 0.0;
  for (double v : a) nrm += v * v;
  nrm = std::sqrt(nrm);
  // Condon-Shortley: <j1 j1 j2 J-j1 | J J> > 0 (hi == j1 always holds here)
  const double sgn = a.back() > 0 ? 1.0 : -1.0;
  for (int k = lo; k <= hi; ++k) at(k, J - k, J) = sgn * a[size_t(k - lo)] / nrm;
  // Lowering: |J M-1> = (J1- + J2-)|J M> / dn(J, M).
  for (int M = J; M > -J; --M) {
    const double inv = 1.0 / dn(J, M);
    for (int m1 = -j1; m1 <= j1; ++m1) {
      const int m2 = M - 1 - m1;
      if (m2 < -j2 || m2 > j2) continue;
      double v = 0.0;
      if (m1 + 1 <= j1) v += at(m1 + 1, m2, M) * dn(j1, m1 + 1);  // J1- from m1+1
      if (m2 + 1 <= j2) v += at(m1, m2 + 1, M) * dn(j2, m2 + 1);  // J2- from m2+1
      at(m1, m2, M - 1) = v * inv;
    }
  }
  return C;
}

// Real harmonics from complex ones: row = real m, column = complex M.
//  m > 0: (Y^{-m} + (-1)^m Y^m)/sqrt2;  m = 0: Y^0;  m < 0: i (Y^m - (-1)^m Y^{-m})/sqrt2.
std::complex<double> U(int l, int m, int M) {
  const double r = 1.0 / std::sqrt(2.0);
  const double s = (m % 2 == 0) ? 1.0 : -1.0;
  if (m > 0) {
    if (M == -m) return {r, 0.0};
    if (M == m) return {s * r, 0.0};
  } else if (m == 0) {
    if (M == 0) return {1.0, 0.0};
  } else {
    if (M == m) return {0.0, r};
    if (M == -m) return {0.0, -s * r};
  }
  (void)l;
  return {0.0, 0.0};
}

}  // namespace

std::vector<Irrep> irreps_from_string(const char* s) {
  if (!s) throw Error{CGTP_ERR_INVALID_ARG, "null irreps"};
  return parse_irreps(s);
}

std::vector<double> real_cg_ladder(int l1, int l2, int l3) {
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
  const std::vector<double> Cc = complex_cg_ladder(l1, l2, l3);
  std::vector<std::complex<double>> X(size_t(n1) * n2 * n3);
  for (int m1 = -l1; m1 <= l1; ++m1)
    for (int m2 = -l2; m2 <= l2; ++m2)
      for (int m3 = -l3; m3 <= l3; ++m3) {
        // U(l, m, M) is nonzero only for M = +-m: visit each distinct M once
        const int nM1 = m1 == 0 ? 1 : 2, nM2 = m2 == 0 ? 1 : 2, nM3 = m3 == 0 ? 1 : 2;
        std::complex<double> acc = 0.0;
        for (int a = 0; a < nM1; ++a)
          for (int b = 0; b < nM2; ++b)
            for (int d = 0; d < nM3; ++d) {
              const int M1 = a ? -m1 : m1, M2 = b ? -m2 : m2, M3 = d ? -m3 : m3;
              if (M1 + M2 != M3) continue;
              const double c = Cc[(size_t(M1 + l1) * n2 + (M2 + l2)) * n3 + (M3 + l3)];
              if (c == 0.0) continue;
              acc += std::conj(U(l1, m1, M1)) * std::conj(U(l2, m2, M2)) * U(l3, m3, M3) * c;
            }
        X[(size_t(m1 + l1) * n2 + (m2 + l2)) * n3 + (m3 + l3)] = acc;
      }
  double re = 0.0, im = 0.0;
  for (auto& v : X) {
    re = std::max(re, std::abs(v.real()));
    im = std::max(im, std::abs(v.imag()));
  }
  std::vector<double> C(X.size());
  const bool take_re = re >= im;
  for (size_t i = 0; i < X.size(); ++i) {
    double v = take_re ? X[i].real() : X[i].imag();
    C[i] = std::abs(v) < 1e-15 ? 0.0 : v;
  }
  // Sign rule: even paths C[0,0,0] > 0; odd paths first nonzero positive.
  double ref = 0.0;
  if ((l1 + l2 + l3) % 2 == 0) {
    ref = C[(size_t(l1) * n2 + l2) * n3 + l3];
  } else {
    for (double v : C)
      if (std::abs(v) > 1e-9) {
        ref = v;
        break;
      }
  }
  if (ref < 0)
    for (double& v : C) v = -v;
  return C;
}

namespace {

std::vector<double> real_cg_checked(int l1, int l2, int l3) {
  std::vector<double> C = real_cg_ladder(l1, l2, l3);
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
  for (int a = 0; a < n3; ++a)
    for (int b = 0; b < n3; ++b) {
      double g = 0.0;
      for (int i = 0; i < n1 * n2; ++i) g += C[size_t(i) * n3 + a] * C[size_t(i) * n3 + b];
      if (std::abs(g - (a == b ? 1.0 : 0.0)) > 1e-12)
        throw Error{CGTP_ERR_UNSUPPORTED, "internal: CG block not orthonormal"};
    }
  return C;
}

// Pack one path's coefficients in the kernels' compile-time order.
template <int L1, int L2, int L3>
void pack_one(const std::vector<double>& C, std::vector<double>& out) {
  using P = Pattern<L1, L2, L3>;
  const int n2 = 2 * L2 + 1, n3 = 2 * L3 + 1;
  std::vector<char> covered(C.size(), 0);
  for (int k = 0; k < P::NP; ++k) {
    const PairT& pr = P::arr.p[k];
    for (int t = 0; t < pr.n; ++t) {
      const int m2 = t == 0 ? pr.m2a : pr.m2b;
      const size_t idx = (size_t(pr.m1 + L1) * n2 + (m2 + L2)) * n3 + (pr.m3 + L3);
      out.push_back(C[idx]);
      covered[idx] = 1;
    }
  }
  for (size_t i = 0; i < C.size(); ++i)
    if (!covered[i] && std::abs(C[i]) > 1e-12)
      throw Error{CGTP_ERR_UNSUPPORTED, "internal: CG entry outside the sparsity pattern"};
}

void pack_path(int l1, int l2, int l3, const std::vector<double>& C, std::vector<double>& out) {
  bool done = false;
  static_for<0, kLmax + 1>([&](auto A) {
    static_for<0, kLmax + 1>([&](auto B) {
      static_for<0, kLmax + 1>([&](auto D) {
        constexpr int a = decltype(A)::value, b = decltype(B)::value, d = decltype(D)::value;
        if constexpr (d >= (a > b ? a - b : b - a) && d <= a + b) {
          if (!done && l1 == a && l2 == b && l3 == d) {
            pack_one<a, b, d>(C, out);
            done = true;
          }
        }
      });
    });
  });
  if (!done) throw Error{CGTP_ERR_UNSUPPORTED, "degree above CGTP_LMAX"};
}

}  // namespace

cgtp_plan_s* build_plan(const char* ix, const char* iy, const char* io, const char* mode,
                        cgtp_dtype dtype, cgtp_wkind wkind, cgtp_paths select, bool collapse) {
  if (!ix || !iy || !io || !mode) throw Error{CGTP_ERR_INVALID_ARG, "null irreps or mode"};
  int md = -1;
  if (std::strcmp(mode, "uvu") == 0) md = 0;
  if (std::strcmp(mode, "uvw") == 0) md = 1;
  if (md < 0) throw Error{CGTP_ERR_UNSUPPORTED, std::string("mode '") + mode + "' (uvu or uvw)"};
  if (dtype != CGTP_F32 && dtype != CGTP_F64 && dtype != CGTP_BF16)
    throw Error{CGTP_ERR_INVALID_ARG, "bad dtype"};
  if (wkind != CGTP_W_SHARED && wkind != CGTP_W_PER_ROW)
    throw Error{CGTP_ERR_INVALID_ARG, "bad weight kind"};
  if (select != CGTP_PATHS_ALL && select != CGTP_PATHS_SYMMETRIC && select != CGTP_PATHS_SKEW)
    throw Error{CGTP_ERR_INVALID_ARG, "bad path selection"};
  auto plan = std::unique_ptr<cgtp_plan_s, void (*)(cgtp_plan_s*)>(new cgtp_plan_s, destroy_plan);
  plan->mode = md;
  plan->select = select;
  plan->collapse = collapse;
  plan->X = parse_irreps(ix);
  plan->Y = parse_irreps(iy);
  plan->O = parse_irreps(io);
  plan->dtype = dtype;
  plan->wkind = wkind;
  for (auto* v : {&plan->X, &plan->Y, &plan->O})
    for (const Irrep& r : *v)
      if (r.l > kLmax) throw Error{CGTP_ERR_UNSUPPORTED, "degree " + std::to_string(r.l) + " > CGTP_LMAX"};
  for (const Irrep& r : plan->Y) plan->max_ymul = std::max(plan->max_ymul, r.mul);
  if (md == 1) {
    // the fully connected product runs on the matrix cores with y of
    // multiplicity 1, shared weights, fp32 or bf16 storage, channel counts in
    // multiples of 4
    if (plan->max_ymul != 1) throw Error{CGTP_ERR_UNSUPPORTED, "uvw needs multiplicity 1 on the second operand"};
    if (wkind != CGTP_W_SHARED) throw Error{CGTP_ERR_UNSUPPORTED, "uvw takes shared weights (CGTP_W_SHARED)"};
    if (dtype == CGTP_F64) throw Error{CGTP_ERR_UNSUPPORTED, "uvw: fp64 is not supported (fp32, bf16)"};
    for (const auto* v : {&plan->X, &plan->O})
      for (const Irrep& r : *v)
        if (r.mul % 4 != 0) throw Error{CGTP_ERR_UNSUPPORTED, "uvw: multiplicities must be multiples of 4"};
  }
  if (md == 0 && plan->max_ymul > 1 && collapse)
    throw Error{CGTP_ERR_UNSUPPORTED, "uvu with y multiplicity > 1: collapsed outputs are not supported"};
  std::set<std::pair<int, int>> allowed;
  std::map<std::pair<int, int>, int> first_mul;  // (l, p) -> multiplicity of its first irreps_out entry
  for (const Irrep& r : plan->O) {
    allowed.insert({r.l, r.p});
    first_mul.insert({{r.l, r.p}, r.mul});
  }

  std::vector<int> xoff, yoff;
  int64_t o = 0;
  for (const Irrep& r : plan->X) {
    xoff.push_back(int(o));
    o += int64_t(r.mul) * (2 * r.l + 1);
    plan->max_mul = std::max(plan->max_mul, r.mul);
  }
  plan->dim_x = o;
  o = 0;
  for (const Irrep& r : plan->Y) {
    yoff.push_back(int(o));
    o += int64_t(r.mul) * (2 * r.l + 1);
  }
  plan->dim_y = o;

  int64_t out_off = 0, w_off = 0;
  std::vector<double> coef;
  for (int i1 = 0; i1 < int(plan->X.size()); ++i1) {
    const Irrep& a = plan->X[i1];
    BlockInfo blk{a.l, a.mul, xoff[i1], int(plan->paths.size()), 0};
    for (int i2 = 0; i2 < int(plan->Y.size()); ++i2) {
      const Irrep& b = plan->Y[i2];
      const int run_begin = int(plan->paths.size());
      for (int l3 = std::abs(a.l - b.l); l3 <= a.l + b.l; ++l3) {
        const int p3 = a.p * b.p;
        if (!allowed.count({l3, p3})) continue;
        // parity class of the path: symmetric when l1 + l2 + l3 is even
        const bool sym = (a.l + b.l + l3) % 2 == 0;
        if ((select == CGTP_PATHS_SYMMETRIC && !sym) || (select == CGTP_PATHS_SKEW && sym)) continue;
        PathInfo p{};
        p.i1 = i1; p.i2 = i2; p.l1 = a.l; p.l2 = b.l; p.l3 = l3; p.p3 = p3; p.mul = a.mul;
        p.v = b.mul;
        p.out_mul = md == 0 ? a.mul : first_mul.at({l3, p3});
        p.w_len = md == 0 ? a.mul * b.mul : a.mul * b.mul * p.out_mul;
        p.x_off = xoff[i1];
        p.y_off = yoff[i2];
        p.out_off = int(out_off);
        p.w_off = int(w_off);
        p.coef_off = int(coef.size());
        std::vector<double> C = real_cg_checked(a.l, b.l, l3);
        pack_path(a.l, b.l, l3, C, coef);
        plan->cg_dense.push_back(std::move(C));
        out_off += int64_t(p.out_mul) * (2 * l3 + 1);
        w_off += p.w_len;
        plan->paths.push_back(p);
      }
      for (int k = run_begin; k < int(plan->paths.size()); ++k) plan->paths[k].i2_end = int(plan->paths.size());
    }
    blk.path_end = int(plan->paths.size());
    if (blk.path_end > blk.path_begin)
      plan->blocks.push_back(blk);
    else
      plan->x_unread.push_back({xoff[i1], a.mul * (2 * a.l + 1)});
  }
  if (plan->paths.empty()) throw Error{CGTP_ERR_UNSUPPORTED, "no path connects the irreps"};
  if (!collapse) {
    for (const PathInfo& p : plan->paths) plan->outputs.push_back(OutBlock{p.l3, p.p3, p.out_mul, p.out_off});
  } else {
    // one block per (l3, p3) that a path reaches, in irreps_out order (first
    // occurrence); the paths feeding it must share their multiplicity
    out_off = 0;
    std::set<std::pair<int, int>> seen;
    for (const Irrep& r : plan->O) {
      if (!seen.insert({r.l, r.p}).second) continue;
      int mul = -1;
      for (const PathInfo& p : plan->paths)
        if (p.l3 == r.l && p.p3 == r.p) {
          if (mul >= 0 && p.out_mul != mul)
            throw Error{CGTP_ERR_UNSUPPORTED, "collapsed output " + std::to_string(r.l) + (r.p > 0 ? "e" : "o") +
                                                  " is fed by x blocks of different multiplicities"};
          mul = p.out_mul;
        }
      if (mul < 0) continue;
      for (PathInfo& p : plan->paths)
        if (p.l3 == r.l && p.p3 == r.p) p.out_off = int(out_off);
      plan->outputs.push_back(OutBlock{r.l, r.p, mul, int(out_off)});
      out_off += int64_t(mul) * (2 * r.l + 1);
    }
  }
  if (out_off > INT32_MAX || w_off > INT32_MAX || plan->dim_x > INT32_MAX || plan->dim_y > INT32_MAX)
    throw Error{CGTP_ERR_UNSUPPORTED, "row too large for 32-bit offsets"};
  plan->dim_out = out_off;
  plan->w_numel = w_off;
  plan->coef64 = coef;
  plan->coef32.assign(coef.begin(), coef.end());

  // Channels per lane: 16-byte vectors when every multiplicity allows it.
  const int vmax = dtype == CGTP_F64 ? 2 : 4;
  bool ok = true;
  for (const Irrep& r : plan->X) ok = ok && (r.mul % vmax == 0);
  plan->vec = ok ? vmax : 1;

  if (md == 1) {
    // the path outputs T: the unit-weight uvu product over the same paths
    plan->unit = build_plan(ix, iy, io, "uvu", dtype, CGTP_W_SHARED, select, false);
    plan->unit->with_ones = true;
    // channel mixing T -> out: path p's T block (u, l3, p3) into its output
    // block with W_p [u][1][w] = [u][w] (the linear map's [mu][mv] layout)
    auto mix = std::make_unique<cgtp_linear_s>();
    mix->dtype = dtype;
    for (size_t k = 0; k < plan->paths.size(); ++k) {
      const PathInfo& p = plan->paths[k];
      mix->I.push_back(Irrep{p.mul, p.l3, p.p3});
      mix->in_off.push_back(plan->unit->paths[k].out_off);
    }
    for (const OutBlock& ob : plan->outputs) {
      mix->O.push_back(Irrep{ob.mul, ob.l3, ob.p3});
      mix->out_off.push_back(ob.out_off);
    }
    for (size_t k = 0; k < plan->paths.size(); ++k) {
      const PathInfo& p = plan->paths[k];
      int o = -1;
      for (size_t j = 0; j < plan->outputs.size(); ++j)
        if (plan->outputs[j].out_off == p.out_off) o = int(j);
      mix->paths.push_back(cgtp_linear_s::Path{int(k), o, p.l3, p.mul, p.out_mul, int64_t(p.w_off)});
    }
    mix->dim_in = plan->unit->dim_out;
    mix->dim_out = plan->dim_out;
    mix->w_numel = plan->w_numel;
    plan->mix = mix.release();
  }

  // Fused-convolution slot tables (uvu with y of multiplicity 1).
  int ly = 0, lo = 0;
  bool distinct = md == 0 && plan->max_ymul == 1;
  for (int i2 = 0; i2 < int(plan->Y.size()); ++i2) {
    const int l = plan->Y[i2].l;
    if (plan->yoff_by_l[l] >= 0) distinct = false;
    plan->yoff_by_l[l] = yoff[i2];
    ly = std::max(ly, l);
  }
  for (const PathInfo& p : plan->paths) lo = std::max(lo, p.l3);
  plan->conv_fused = distinct;
  // The collapsed fused forward groups the slots of one x block by
  // (l2 mod 2, l3), which equals grouping by output type only when every y
  // block has parity s (-1)^l2 for one common sign s (harmonics: s = +1).
  // Otherwise two output types could share an accumulator, so such plans
  // take the general kernel.
  {
    int s = 0;
    bool same = true;
    for (const Irrep& r : plan->Y) {
      const int t = r.p * ((r.l % 2) ? -1 : 1);
      if (s == 0) s = t;
      same = same && t == s;
    }
    plan->conv_col_fused = distinct && same;
  }
  plan->conv_L = std::max(ly, lo);
  plan->lm = plan->conv_L;
  if (distinct) {
    const int L = plan->conv_L;
    for (const BlockInfo& b : plan->blocks) {
      plan->slot_off.push_back(int32_t(plan->slot_paths.size()));
      for (int l2 = 0; l2 <= L; ++l2)
        for (int l3 = std::abs(b.l1 - l2); l3 <= std::min(b.l1 + l2, L); ++l3) {
          int32_t found = -1;
          for (int q = b.path_begin; q < b.path_end; ++q)
            if (plan->paths[q].l2 == l2 && plan->paths[q].l3 == l3) found = q;
          plan->slot_paths.push_back(found);
        }
    }
    plan->slot_off.push_back(int32_t(plan->slot_paths.size()));
  }
  return plan.release();
}

void destroy_plan(cgtp_plan_s* plan) {
  if (!plan) return;
  free_plan_tables(plan);
  free_uvw_tables(plan);
  free_uvuv_tables(plan);
  free_radial_maps(plan);
  if (plan->mix) {
    free_linear_tables(plan->mix);
    delete plan->mix;
  }
  destroy_plan(plan->unit);
  delete plan;
}

namespace {
struct SideSet {
  hipStream_t st[kSideStreams] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kSideStreams] = {};
};
std::mutex g_side_mu;
std::map<int, SideSet> g_side;  // per HIP device id; kept until the process ends

SideSet& side_set_locked(int dev) {
  auto it = g_side.find(dev);
  if (it != g_side.end()) return it->second;
  SideSet ss;
  for (int i = 0; i < kSideStreams; ++i) {
    CGTP_CHECK_HIP(hipStreamCreateWithFlags(&ss.st[i], hipStreamNonBlocking));
    CGTP_CHECK_HIP(hipEventCreateWithFlags(&ss.join[i], hipEventDisableTiming));
  }
  CGTP_CHECK_HIP(hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming));
  return g_side.emplace(dev, ss).first->second;
}
}  // namespace

void side_streams_init() {
  int dev = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_side_mu);
  side_set_locked(dev);
}

#ifndef CGTP_SIDE_STREAMS
#define CGTP_SIDE_STREAMS 1  // 0: the launches of side_run stay on s, in order (for timing)
#endif

void side_run(hipStream_t s, int n, const std::function<void(int, hipStream_t)>& f, bool fork) {
  if (n <= 1 || !fork || CGTP_SIDE_STREAMS == 0) {
    for (int i = 0; i < n; ++i) f(i, s);
    return;
  }
  int dev = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  // one call's fork and join are queued under the lock, so calls from several
  // host threads do not interleave their event records
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideSet& ss = side_set_locked(dev);
  const int used = std::min(n - 1, kSideStreams);
  CGTP_CHECK_HIP(hipEventRecord(ss.fork, s));
  for (int j = 0; j < used; ++j) CGTP_CHECK_HIP(hipStreamWaitEvent(ss.st[j], ss.fork, 0));
  for (int i = 0; i < n; ++i) f(i, i == 0 ? s : ss.st[(i - 1) % kSideStreams]);
  for (int j = 0; j < used; ++j) {
    CGTP_CHECK_HIP(hipEventRecord(ss.join[j], ss.st[j]));
    CGTP_CHECK_HIP(hipStreamWaitEvent(s, ss.join[j], 0));
  }
}

const DevTables& plan_tables(cgtp_plan_s* plan) {
  int dev = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  side_streams_init();  // before any capture, like the tables
  std::lock_guard<std::mutex> lock(plan->mu);
  auto it = plan->dev.find(dev);
  if (it != plan->dev.end()) return it->second;
  std::vector<PathDev> pd;
  for (const PathInfo& p : plan->paths)
    pd.push_back(PathDev{p.l2, p.l3, p.y_off, p.out_off, p.w_off, p.coef_off, p.i2_end, p.mul,
                         p.l1, p.x_off, p.p3, p.v});
  std::vector<BlockDev> bd;
  for (const BlockInfo& b : plan->blocks)
    bd.push_back(BlockDev{b.l1, b.mul, b.x_off, b.path_begin, b.path_end, 0, 0, 0});
  DevTables t;
  const bool f64 = plan->dtype == CGTP_F64;
  // The device table is followed by one whole pattern of the largest degrees
  // in zeros: a kernel may run a pattern from offset 0 for a slot the plan
  // does not have (its results discarded) or from that zero run (its results
  // added as zeros).
  const size_t ncoef = plan->coef64.size() + size_t(max_pattern_coefs(kLmax));
  std::vector<double> c64(plan->coef64);
  std::vector<float> c32(plan->coef32);
  c64.resize(ncoef, 0.0);
  c32.resize(ncoef, 0.0f);
  const size_t cbytes = f64 ? ncoef * 8 : ncoef * 4;
  try {
    CGTP_CHECK_HIP(hipMalloc(&t.paths, pd.size() * sizeof(PathDev)));
    CGTP_CHECK_HIP(hipMalloc(&t.blocks, bd.size() * sizeof(BlockDev)));
    CGTP_CHECK_HIP(hipMalloc(&t.coef, cbytes));
    CGTP_CHECK_HIP(hipMemcpy(t.paths, pd.data(), pd.size() * sizeof(PathDev), hipMemcpyHostToDevice));
    CGTP_CHECK_HIP(hipMemcpy(t.blocks, bd.data(), bd.size() * sizeof(BlockDev), hipMemcpyHostToDevice));
    CGTP_CHECK_HIP(hipMemcpy(t.coef, f64 ? static_cast<const void*>(c64.data()) : static_cast<const void*>(c32.data()),
                             cbytes, hipMemcpyHostToDevice));
    if (plan->with_ones) {
      const size_t es = dtype_size(plan->dtype), n = size_t(plan->w_numel);
      std::vector<unsigned char> ones(n * es);
      for (size_t i = 0; i < n; ++i) {
        if (es == 8) {
          const double one = 1.0;
          std::memcpy(&ones[i * 8], &one, 8);
        } else if (es == 4) {
          const float one = 1.0f;
          std::memcpy(&ones[i * 4], &one, 4);
        } else {
          const uint16_t one = 0x3f80;  // bf16 1.0
          std::memcpy(&ones[i * 2], &one, 2);
        }
      }
      CGTP_CHECK_HIP(hipMalloc(&t.ones, ones.size()));
      CGTP_CHECK_HIP(hipMemcpy(t.ones, ones.data(), ones.size(), hipMemcpyHostToDevice));
    }
    if (plan->conv_fused) {
      CGTP_CHECK_HIP(hipMalloc(&t.slot_paths, plan->slot_paths.size() * 4 + 4));
      CGTP_CHECK_HIP(hipMalloc(&t.slot_off, plan->slot_off.size() * 4));
      CGTP_CHECK_HIP(hipMemcpy(t.slot_paths, plan->slot_paths.data(), plan->slot_paths.size() * 4,
                               hipMemcpyHostToDevice));
      CGTP_CHECK_HIP(hipMemcpy(t.slot_off, plan->slot_off.data(), plan->slot_off.size() * 4,
                               hipMemcpyHostToDevice));
    }
  } catch (...) {
    (void)hipFree(t.paths);
    (void)hipFree(t.blocks);
    (void)hipFree(t.coef);
    (void)hipFree(t.ones);
    (void)hipFree(t.slot_paths);
    (void)hipFree(t.slot_off);
    throw;
  }
  return plan->dev.emplace(dev, t).first->second;
}

void free_plan_tables(cgtp_plan_s* plan) {
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : plan->dev) {
    if (hipSetDevice(kv.first) == hipSuccess) {
      (void)hipFree(kv.second.paths);
      (void)hipFree(kv.second.blocks);
      (void)hipFree(kv.second.coef);
      (void)hipFree(kv.second.ones);
      (void)hipFree(kv.second.slot_paths);
      (void)hipFree(kv.second.slot_off);
    }
  }
  if (have) (void)hipSetDevice(cur);
  plan->dev.clear();
}

}  // namespace cgtp
