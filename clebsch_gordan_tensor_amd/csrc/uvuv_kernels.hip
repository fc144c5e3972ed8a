// Channel-wise ("uvu") tensor product with a second operand of multiplicity
// v > 1: the generic kernels.
//
// What is computed (MolSSI e3nn course, lesson 03b: instructions in the uvu
// connection mode; reverse rules by transposition as in "E3J: An Efficient and
// Open-Source Backend for Euclidean Equivariant Operations on GPU and TPU",
// E.1). For a path p = (i1, i2, l3), x block i1 of multiplicity u, y block i2
// of multiplicity v and weights w_p [u][v] (row-major; shared or per row):
//   out[z, p, m3, a] = sum_b w_p[a, b] sum_{m1,m2} C_p[m1,m2,m3] x[z,i1,m1,a] y[z,i2,m2,b]
//                    = sum_{m1,m2} C_p x[z,i1,m1,a] yt[m2, a],
//   yt[m2, a] = sum_b w_p[a, b] y[z,i2,m2,b]   (a per-channel mix of y).
// One lane per (row, channel a): it forms yt for each path and runs the
// path's compile-time coefficient pattern on it. Backward, with g the output
// cotangent and dyt[m2] = sum C x[m1] g[m3] per path:
//   dx[m1, a]       = sum_p sum C yt[m2] g[m3]            (lane (z, a), paths of one x block in turn)
//   dw_p[(z,) a, b] = sum_m2 dyt[m2] y[m2, b]             (lane (z, a); shared: per-row partials, then a
//                                                         fixed-order sum over rows)
//   dy[z, i2, m2, b] = sum_p sum_a w_p[a, b] dyt_p[m2, a] (lane (z, y component), channels in order,
//                                                         from the dyt rows the first kernel left in the
//                                                         workspace)
// Every sum has a fixed order; no atomics.
#include <map>
#include <mutex>
#include <vector>

#include "cg_pattern.h"
#include "common.hpp"
#include "device_util.hpp"
#include "tp_core.hpp"
#include "tp_impl.hpp"

namespace cgtp {

namespace {

struct UvuvArgs {
  const PathDev* paths;
  const BlockDev* blocks;
  const void* coef;
  const int32_t* ypaths;  // per y block: the paths that read it, [begin, end) into ypath_idx
  const int32_t* ypath_idx;
  const int32_t* yblk;    // per y block: y_off, l2, v (3 ints)
  const void* x;
  const void* y;
  const void* w;
  const void* g;
  void* out;
  void* dx;
  void* dy;
  void* dw;     // per-row grad_w (storage type) or per-row partials (accumulation type)
  void* dyt;    // per row, per path: dyt_p [2 l2 + 1][u] (accumulation type), at dyt_off[p]
  const int32_t* dyt_off;
  int dim_dyt;
  int64_t B;
  int64_t w_stride;  // elements between weight rows, 0 for shared
  int dim_x, dim_y, dim_out, W;
  int nblocks, nyblocks, cmax;
  int dw_acc;   // dw holds accumulation-type partials
};

// PathDev.pad1 carries the y multiplicity v of the path.
template <typename T, typename A, int L1, int L2, int L3>
__device__ __forceinline__ void uvuv_fwd_path(const UvuvArgs& a, const PathDev& pd, const A (&xb)[2 * L1 + 1][1],
                                              const T* yr, const T* wr, T* outr, int c) {
  const int v = pd.pad1;
  A yt[2 * L2 + 1];
  const T* __restrict__ wc = wr + pd.w_off + int64_t(c) * v;
#pragma unroll
  for (int m = 0; m < 2 * L2 + 1; ++m) {
    A s = A(0);
    for (int b = 0; b < v; ++b) s = fma(to_acc<A>(wc[b]), to_acc<A>(yr[pd.y_off + m * v + b]), s);
    yt[m] = s;
  }
  A o[2 * L3 + 1][1];
  fwd_core<L1, L2, L3, 1, A>(xb, yt, static_cast<const A*>(a.coef) + pd.coef_off, o);
#pragma unroll
  for (int m = 0; m < 2 * L3 + 1; ++m) from_acc(outr[pd.out_off + m * pd.mul + c], o[m][0]);
}

template <typename T, typename A>
__global__ __launch_bounds__(kBlock) void uvuv_fwd_kernel(UvuvArgs a) {
  const int64_t gid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t z = gid / a.cmax;
  const int c = int(gid - z * a.cmax);
  if (z >= a.B) return;
  const T* xr = static_cast<const T*>(a.x) + z * a.dim_x;
  const T* yr = static_cast<const T*>(a.y) + z * a.dim_y;
  const T* wr = static_cast<const T*>(a.w) + z * a.w_stride;
  T* outr = static_cast<T*>(a.out) + z * a.dim_out;
  for (int bi = 0; bi < a.nblocks; ++bi) {
    const BlockDev blk = ldc(a.blocks + bi);
    if (c >= blk.mul) continue;
    static_for<0, kLmax + 1>([&](auto L1c) {
      constexpr int L1 = decltype(L1c)::value;
      if (blk.l1 != L1) return;
      A xb[2 * L1 + 1][1];
#pragma unroll
      for (int m = 0; m < 2 * L1 + 1; ++m) xb[m][0] = to_acc<A>(xr[blk.x_off + m * blk.mul + c]);
      for (int p = blk.path_begin; p < blk.path_end; ++p) {
        const PathDev pd = ldc(a.paths + p);
        static_for<0, kLmax + 1>([&](auto L2c) {
          constexpr int L2 = decltype(L2c)::value;
          static_for<0, kLmax + 1>([&](auto L3c) {
            constexpr int L3 = decltype(L3c)::value;
            if constexpr (L3 >= (L1 > L2 ? L1 - L2 : L2 - L1) && L3 <= L1 + L2) {
              if (pd.l2 == L2 && pd.l3 == L3) uvuv_fwd_path<T, A, L1, L2, L3>(a, pd, xb, yr, wr, outr, c);
            }
          });
        });
      }
    });
  }
}

// Lane (z, c): grad_x of every x block and grad_w of every path.
template <typename T, typename A, int L1, int L2, int L3>
__device__ __forceinline__ void uvuv_bwd_path(const UvuvArgs& a, const PathDev& pd, int pidx,
                                              const A (&xb)[2 * L1 + 1], const T* yr, const T* wr, const T* gr,
                                              int64_t z, int c, A (&dxb)[2 * L1 + 1]) {
  using P = Pattern<L1, L2, L3>;
  const int v = pd.pad1;
  const T* __restrict__ wc = wr + pd.w_off + int64_t(c) * v;
  A yt[2 * L2 + 1], dyt[2 * L2 + 1], gb[2 * L3 + 1];
#pragma unroll
  for (int m = 0; m < 2 * L2 + 1; ++m) {
    A s = A(0);
    for (int b = 0; b < v; ++b) s = fma(to_acc<A>(wc[b]), to_acc<A>(yr[pd.y_off + m * v + b]), s);
    yt[m] = s;
    dyt[m] = A(0);
  }
#pragma unroll
  for (int m = 0; m < 2 * L3 + 1; ++m) gb[m] = to_acc<A>(gr[pd.out_off + m * pd.mul + c]);
  const A* __restrict__ cf = static_cast<const A*>(a.coef) + pd.coef_off;
  static_for<0, P::NP>([&](auto I) {
    constexpr PairT pr = P::arr.p[decltype(I)::value];
    const A ca = ldc(cf + pr.coef);
    A av = ca * yt[pr.m2a + L2];
    A cb = A(0);
    if constexpr (pr.n == 2) {
      cb = ldc(cf + pr.coef + 1);
      av = fma(cb, yt[pr.m2b + L2], av);
    }
    dxb[pr.m1 + L1] = fma(av, gb[pr.m3 + L3], dxb[pr.m1 + L1]);
    const A xg = xb[pr.m1 + L1] * gb[pr.m3 + L3];
    dyt[pr.m2a + L2] = fma(ca, xg, dyt[pr.m2a + L2]);
    if constexpr (pr.n == 2) dyt[pr.m2b + L2] = fma(cb, xg, dyt[pr.m2b + L2]);
  });
  if (a.dyt) {
    A* __restrict__ dr = static_cast<A*>(a.dyt) + z * a.dim_dyt + ldc(a.dyt_off + pidx);
#pragma unroll
    for (int m = 0; m < 2 * L2 + 1; ++m) dr[m * pd.mul + c] = dyt[m];
  }
  // grad_w[a = c][b] = sum_m2 dyt[m2] y[m2, b]
  for (int b = 0; b < v; ++b) {
    A s = A(0);
#pragma unroll
    for (int m = 0; m < 2 * L2 + 1; ++m) s = fma(dyt[m], to_acc<A>(yr[pd.y_off + m * v + b]), s);
    const int64_t k = pd.w_off + int64_t(c) * v + b;
    if (a.dw_acc)
      static_cast<A*>(a.dw)[z * a.W + k] = s;
    else if (a.dw)
      from_acc(static_cast<T*>(a.dw)[z * a.W + k], s);
  }
}

template <typename T, typename A>
__global__ __launch_bounds__(kBlock) void uvuv_bwd_xw_kernel(UvuvArgs a) {
  const int64_t gid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t z = gid / a.cmax;
  const int c = int(gid - z * a.cmax);
  if (z >= a.B) return;
  const T* xr = static_cast<const T*>(a.x) + z * a.dim_x;
  const T* yr = static_cast<const T*>(a.y) + z * a.dim_y;
  const T* wr = static_cast<const T*>(a.w) + z * a.w_stride;
  const T* gr = static_cast<const T*>(a.g) + z * a.dim_out;
  for (int bi = 0; bi < a.nblocks; ++bi) {
    const BlockDev blk = ldc(a.blocks + bi);
    if (c >= blk.mul) continue;
    static_for<0, kLmax + 1>([&](auto L1c) {
      constexpr int L1 = decltype(L1c)::value;
      if (blk.l1 != L1) return;
      A xb[2 * L1 + 1], dxb[2 * L1 + 1];
#pragma unroll
      for (int m = 0; m < 2 * L1 + 1; ++m) {
        xb[m] = to_acc<A>(xr[blk.x_off + m * blk.mul + c]);
        dxb[m] = A(0);
      }
      for (int p = blk.path_begin; p < blk.path_end; ++p) {
        const PathDev pd = ldc(a.paths + p);
        static_for<0, kLmax + 1>([&](auto L2c) {
          constexpr int L2 = decltype(L2c)::value;
          static_for<0, kLmax + 1>([&](auto L3c) {
            constexpr int L3 = decltype(L3c)::value;
            if constexpr (L3 >= (L1 > L2 ? L1 - L2 : L2 - L1) && L3 <= L1 + L2) {
              if (pd.l2 == L2 && pd.l3 == L3) uvuv_bwd_path<T, A, L1, L2, L3>(a, pd, p, xb, yr, wr, gr, z, c, dxb);
            }
          });
        });
      }
      if (a.dx) {
#pragma unroll
        for (int m = 0; m < 2 * L1 + 1; ++m) from_acc(static_cast<T*>(a.dx)[z * a.dim_x + blk.x_off + m * blk.mul + c], dxb[m]);
      }
    });
  }
}

// Lane (z, j): grad_y component j = (y block i2, m2, b) of row z, summed over
// the paths reading block i2 and their channels in order, from the dyt rows.
template <typename T, typename A>
__global__ __launch_bounds__(kBlock) void uvuv_bwd_y_kernel(UvuvArgs a) {
  const int64_t gid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t z = gid / a.dim_y;
  const int j = int(gid - z * a.dim_y);
  if (z >= a.B) return;
  int i2 = 0;
  for (int k = 0; k < a.nyblocks; ++k)
    if (j >= ldc(a.yblk + 3 * k)) i2 = k;
  const int y_off = ldc(a.yblk + 3 * i2), v = ldc(a.yblk + 3 * i2 + 2);
  const int m2 = (j - y_off) / v, b = (j - y_off) - m2 * v;
  const T* __restrict__ wr = static_cast<const T*>(a.w) + z * a.w_stride;
  const A* __restrict__ dr = static_cast<const A*>(a.dyt) + z * a.dim_dyt;
  A s = A(0);
  for (int q = ldc(a.ypaths + i2); q < ldc(a.ypaths + i2 + 1); ++q) {
    const int p = ldc(a.ypath_idx + q);
    const PathDev pd = ldc(a.paths + p);
    const A* __restrict__ dp = dr + ldc(a.dyt_off + p) + m2 * pd.mul;
    const T* __restrict__ wp = wr + pd.w_off + b;
    for (int c = 0; c < pd.mul; ++c) s = fma(to_acc<A>(wp[int64_t(c) * v]), dp[c], s);
  }
  from_acc(static_cast<T*>(a.dy)[z * a.dim_y + j], s);
}

struct UvuvTables {
  int32_t* ypaths = nullptr;
  int32_t* ypath_idx = nullptr;
  int32_t* yblk = nullptr;
  int32_t* dyt_off = nullptr;
};

// offset of each path's dyt block [2 l2 + 1][u] in a dyt row, and the row length
std::vector<int32_t> dyt_offsets(const cgtp_plan_s* plan, int64_t* total) {
  std::vector<int32_t> off;
  int64_t o = 0;
  for (const PathInfo& p : plan->paths) {
    off.push_back(int32_t(o));
    o += int64_t(2 * p.l2 + 1) * p.mul;
  }
  *total = o;
  return off;
}

std::mutex g_uvuv_mu;
std::map<std::pair<const cgtp_plan_s*, int>, UvuvTables> g_uvuv_tables;

const UvuvTables& uvuv_tables(const cgtp_plan_s* plan) {
  int dev = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_uvuv_mu);
  auto it = g_uvuv_tables.find({plan, dev});
  if (it != g_uvuv_tables.end()) return it->second;
  std::vector<int32_t> yp{0}, yi, yb;
  int64_t off = 0;
  for (size_t i2 = 0; i2 < plan->Y.size(); ++i2) {
    for (size_t k = 0; k < plan->paths.size(); ++k)
      if (plan->paths[k].i2 == int(i2)) yi.push_back(int32_t(k));
    yp.push_back(int32_t(yi.size()));
    yb.push_back(int32_t(off));
    yb.push_back(plan->Y[i2].l);
    yb.push_back(plan->Y[i2].mul);
    off += int64_t(plan->Y[i2].mul) * (2 * plan->Y[i2].l + 1);
  }
  UvuvTables t;
  auto up = [](const std::vector<int32_t>& v, int32_t** p) {
    CGTP_CHECK_HIP(hipMalloc(p, std::max<size_t>(v.size(), 1) * 4));
    if (!v.empty()) CGTP_CHECK_HIP(hipMemcpy(*p, v.data(), v.size() * 4, hipMemcpyHostToDevice));
  };
  int64_t total = 0;
  const std::vector<int32_t> doff = dyt_offsets(plan, &total);
  try {
    up(yp, &t.ypaths);
    up(yi, &t.ypath_idx);
    up(yb, &t.yblk);
    up(doff, &t.dyt_off);
  } catch (...) {
    (void)hipFree(t.ypaths);
    (void)hipFree(t.ypath_idx);
    (void)hipFree(t.yblk);
    (void)hipFree(t.dyt_off);
    throw;
  }
  return g_uvuv_tables.emplace(std::make_pair(plan, dev), t).first->second;
}

UvuvArgs make_uvuv_args(cgtp_plan_s* plan, int64_t B) {
  const DevTables& t = plan_tables(plan);
  const UvuvTables& u = uvuv_tables(plan);
  UvuvArgs a{};
  a.paths = t.paths;
  a.blocks = t.blocks;
  a.coef = t.coef;
  a.ypaths = u.ypaths;
  a.ypath_idx = u.ypath_idx;
  a.yblk = u.yblk;
  a.dyt_off = u.dyt_off;
  int64_t total = 0;
  (void)dyt_offsets(plan, &total);
  a.dim_dyt = int(total);
  a.B = B;
  a.w_stride = plan->wkind == CGTP_W_PER_ROW ? plan->w_numel : 0;
  a.dim_x = int(plan->dim_x);
  a.dim_y = int(plan->dim_y);
  a.dim_out = int(plan->dim_out);
  a.W = int(plan->w_numel);
  a.nblocks = int(plan->blocks.size());
  a.nyblocks = int(plan->Y.size());
  a.cmax = plan->max_mul;
  return a;
}

unsigned grid_of(int64_t n) { return unsigned((n + kBlock - 1) / kBlock); }

template <typename T>
void fwd_typed(const UvuvArgs& a, hipStream_t s) {
  using A = typename AccOf<T>::type;
  hipLaunchKernelGGL((uvuv_fwd_kernel<T, A>), dim3(grid_of(a.B * a.cmax)), dim3(kBlock), 0, s, a);
  CGTP_CHECK_HIP(hipGetLastError());
}

template <typename T>
void bwd_typed(const UvuvArgs& a, bool xw, bool yk, hipStream_t s) {
  using A = typename AccOf<T>::type;
  if (xw) hipLaunchKernelGGL((uvuv_bwd_xw_kernel<T, A>), dim3(grid_of(a.B * a.cmax)), dim3(kBlock), 0, s, a);
  CGTP_CHECK_HIP(hipGetLastError());
  if (yk) hipLaunchKernelGGL((uvuv_bwd_y_kernel<T, A>), dim3(grid_of(a.B * a.dim_y)), dim3(kBlock), 0, s, a);
  CGTP_CHECK_HIP(hipGetLastError());
}

}  // namespace

void free_uvuv_tables(const cgtp_plan_s* plan) {
  std::lock_guard<std::mutex> lock(g_uvuv_mu);
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto it = g_uvuv_tables.begin(); it != g_uvuv_tables.end();) {
    if (it->first.first == plan) {
      if (hipSetDevice(it->first.second) == hipSuccess) {
        (void)hipFree(it->second.ypaths);
        (void)hipFree(it->second.ypath_idx);
        (void)hipFree(it->second.yblk);
        (void)hipFree(it->second.dyt_off);
      }
      it = g_uvuv_tables.erase(it);
    } else {
      ++it;
    }
  }
  if (have) (void)hipSetDevice(cur);
}

void uvuv_forward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w, void* out,
                         hipStream_t s) {
  if (B == 0) return;
  UvuvArgs a = make_uvuv_args(plan, B);
  a.x = x;
  a.y = y;
  a.w = w;
  a.out = out;
  switch (plan->dtype) {
    case CGTP_F32: fwd_typed<float>(a, s); break;
    case CGTP_F64: fwd_typed<double>(a, s); break;
    case CGTP_BF16: fwd_typed<bf16>(a, s); break;
  }
  // output blocks of x blocks that no path reads do not exist; every output
  // element is written by its path's lane
}

// workspace: dyt rows [B][dim_dyt], then (shared weights) per-row grad_w
// partials [B][W] and chunk sums, all in the accumulation type
size_t uvuv_dyt_bytes(const cgtp_plan_s* plan, int64_t B) {
  int64_t total = 0;
  (void)dyt_offsets(plan, &total);
  return (size_t(B) * size_t(total) * acc_size(plan->dtype) + 255) / 256 * 256;
}

size_t uvuv_backward_ws_bytes(const cgtp_plan_s* plan, int64_t B) {
  if (B == 0) return 0;
  size_t n = uvuv_dyt_bytes(plan, B);
  if (plan->wkind == CGTP_W_SHARED) {
    const int64_t nchunks = (B + kRowsPerChunk - 1) / kRowsPerChunk;
    n += size_t(B + nchunks) * size_t(plan->w_numel) * acc_size(plan->dtype);
  }
  return n;
}

void uvuv_backward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w, const void* g,
                          void* dx, void* dy, void* dw, void* ws, size_t ws_bytes, hipStream_t s) {
  const bool shared = plan->wkind == CGTP_W_SHARED;
  if (B == 0) {
    if (dw && shared) zero_rows(dw, plan->w_numel, dtype_size(plan->dtype), s);
    return;
  }
  const size_t need = uvuv_backward_ws_bytes(plan, B);  // grad_y and shared grad_w go through it
  if ((dy || (shared && dw)) && (!ws || ws_bytes < need))
    throw Error{CGTP_ERR_WORKSPACE, "tp_backward needs " + std::to_string(need) + " workspace bytes"};
  char* wsw = ws ? static_cast<char*>(ws) + uvuv_dyt_bytes(plan, B) : nullptr;  // shared grad_w partials
  UvuvArgs a = make_uvuv_args(plan, B);
  a.x = x;
  a.y = y;
  a.w = w;
  a.g = g;
  a.dx = dx;
  a.dy = dy;
  a.dyt = dy ? ws : nullptr;
  a.dw = shared ? (dw ? static_cast<void*>(wsw) : nullptr) : dw;
  a.dw_acc = shared && dw ? 1 : 0;
  switch (plan->dtype) {
    case CGTP_F32: bwd_typed<float>(a, true, dy != nullptr, s); break;
    case CGTP_F64: bwd_typed<double>(a, true, dy != nullptr, s); break;
    case CGTP_BF16: bwd_typed<bf16>(a, true, dy != nullptr, s); break;
  }
  zero_unread_x(plan, dx, B, dtype_size(plan->dtype), s);
  if (shared && dw) {
    char* part = wsw + size_t(B) * plan->w_numel * acc_size(plan->dtype);
    const int nchunks = int((B + kRowsPerChunk - 1) / kRowsPerChunk);
    const unsigned gx = unsigned((plan->w_numel + kBlock - 1) / kBlock);
    auto run = [&](auto tag) {
      using T = decltype(tag);
      using A = typename AccOf<T>::type;
      hipLaunchKernelGGL((colsum_stage1<A>), dim3(gx, unsigned(nchunks)), dim3(kBlock), 0, s,
                         reinterpret_cast<const A*>(wsw), reinterpret_cast<A*>(part), B, int(plan->w_numel));
      hipLaunchKernelGGL((colsum_stage2<T, A>), dim3(gx), dim3(kBlock), 0, s, reinterpret_cast<const A*>(part),
                         static_cast<T*>(dw), nchunks, int(plan->w_numel));
    };
    switch (plan->dtype) {
      case CGTP_F32: run(float{}); break;
      case CGTP_F64: run(double{}); break;
      case CGTP_BF16: run(bf16{}); break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
  }
}

}  // namespace cgtp
