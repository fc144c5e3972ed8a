// Fully connected ("uvw") tensor product: the Clebsch-Gordan path outputs
// mixed over channels on the matrix cores, never written to memory.
//
// What is computed (MolSSI e3nn course, lesson 03b: instructions in the uvw
// connection mode; "E3J: An Efficient and Open-Source Backend for Euclidean
// Equivariant Operations on GPU and TPU", A.3 and B.2: channel mixing around
// the tensor product). For a path p = (i1, i2, l3) with x block i1 of
// multiplicity u, y of multiplicity 1 and output multiplicity w:
//   T_p[z, m3, a]   = sum_{m1,m2} C_p[m1,m2,m3] x[z,i1,m1,a] y[z,i2,m2]
//   out[z, o, m3, k] = sum over paths p into block o of sum_a W_p[a, k] T_p[z, m3, a]
// with W_p = [u][1][w] = [u][w] (shared weights). Collapsed outputs put every
// path of one (l3, p3) into one block o (the fully connected product).
//
// Forward, one kernel: a workgroup owns 16 rows and walks every output block
// and every path into it. Per path (and chunk of 128 x channels) the 256
// lanes first form T_p for the 16 rows in LDS on the vector ALUs (lane =
// (row, 4 channels), the coefficient sparsity pattern fixed at compile time,
// as in the channel-wise product), then the four waves run
// v_mfma_f32_16x16x4_f32 on D[k][z] += sum_a W_p[a][k] T_p[z, m3, a] for
// every m3: wave w owns output channels [32w, 32w + 32) of a 128-channel
// column tile (two 16-row A tiles, W read from L2, the next K step requested
// before the current one's products), all 2 l3 + 1 N tiles (16 rows each).
// D stays in the accumulators over all paths of the block; each lane then
// stores 4 consecutive output channels of one (row, m3). bf16 storage is
// widened exactly to fp32, so both storage types run the same fp32 products.
//
// Backward, composed from the library's kernels through the workspace:
//   T  = unit-weight uvu forward (the path outputs)
//   dW = sum over rows of T^T g, G' = g W^T    (the linear map's backward)
//   dx, dy = uvu backward with unit weights and cotangent G'
// so every sum keeps a fixed order and results are deterministic.
#include <algorithm>
#include <map>
#include <mutex>
#include <vector>

#include "cg_pattern.h"
#include "common.hpp"
#include "device_util.hpp"
#include "linear.hpp"
#include "tp_core.hpp"

namespace cgtp {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

struct alignas(16) UvwPathDev {
  int32_t l1, l2, u, x_off;
  int32_t y_off, coef_off, w_off, pad0;
};
struct alignas(16) UvwGroupDev {
  int32_t l3, out_off, w_out, p0;
  int32_t p1, pad0, pad1, pad2;
};

struct UvwArgs {
  const UvwPathDev* paths;  // in the order of gpaths
  const UvwGroupDev* groups;
  const float* coef;
  const void* x;
  const void* y;
  const void* w;
  void* out;
  int64_t B;
  int dim_x, dim_y, dim_out, ngroups;
};

constexpr int kUvwThreads = 256;
constexpr int kUvwRows = 16;         // rows per workgroup: the MFMA's N tile
constexpr int kUvwK = 128;           // x channels of one T chunk
constexpr int kUvwTP = kUvwK + 4;    // padded LDS row of T (floats)
constexpr int kUvwCols = 128;        // output channels per column tile (4 waves x 32)

size_t uvw_lds_bytes(int max_l3) { return size_t(2 * max_l3 + 1) * kUvwRows * kUvwTP * sizeof(float); }

// T_p for rows z0..z0+15 and x channels k0..k0+127 into LDS [m3][row][channel]
// (zeros past u). Lane (zt, rt) takes row zt and channel quads 4 rt, 4 rt + 64.
template <typename T, int L1, int L2, int L3>
__device__ __forceinline__ void uvw_t_chunk(const UvwArgs& a, const UvwPathDev& pd, const T* __restrict__ xr,
                                            const T* __restrict__ yr, int k0, int zt, int rt, float* tl) {
  float yb[2 * L2 + 1];
#pragma unroll
  for (int m = 0; m < 2 * L2 + 1; ++m) yb[m] = to_acc<float>(yr[pd.y_off + m]);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int al = 4 * rt + 64 * q, ag = k0 + al;
    const bool ok = ag < pd.u;  // u is a multiple of 4: a quad is wholly inside or past it
    float xb[2 * L1 + 1][4];
#pragma unroll
    for (int m = 0; m < 2 * L1 + 1; ++m) VecIO<T, 4>::load(xr + pd.x_off + m * pd.u + (ok ? ag : 0), xb[m]);
    float o[2 * L3 + 1][4];
    fwd_core<L1, L2, L3, 4, float>(xb, yb, a.coef + pd.coef_off, o);
#pragma unroll
    for (int m = 0; m < 2 * L3 + 1; ++m) {
      const v4f v = ok ? v4f{o[m][0], o[m][1], o[m][2], o[m][3]} : v4f{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<v4f*>(tl + (m * kUvwRows + zt) * kUvwTP + al) = v;
    }
  }
}

// W_p[a][k] for this lane's 4 contraction slots of K step kc (a = k0 + 16 kc
// + 4 lk + j) and its two output channels; clamped in-bounds addresses, zeros
// past u or w_out.
template <typename T>
__device__ __forceinline__ void uvw_load_w(const T* __restrict__ W, int u, int w_out, int k0, int kc, int lk,
                                           const int (&kout)[2], const bool (&kok)[2], float (&av)[2][4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ka = k0 + 16 * kc + 4 * lk + j;
    const bool aok = ka < u;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float v = to_acc<float>(W[int64_t(aok ? ka : 0) * w_out + (kok[s] ? kout[s] : 0)]);
      av[s][j] = aok && kok[s] ? v : 0.f;
    }
  }
}

template <typename T, int L3>
__device__ __forceinline__ void uvw_mix_chunk(const UvwArgs& a, const UvwPathDev& pd, int w_out, int k0, int c0,
                                              const float* tl, v4f (&acc)[2][2 * L3 + 1], int wave, int li, int lk) {
  const T* __restrict__ W = static_cast<const T*>(a.w) + pd.w_off;
  int kout[2];
  bool kok[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    kout[s] = c0 + 32 * wave + 16 * s + li;
    kok[s] = kout[s] < w_out;
  }
  const int kn = pd.u - k0 < kUvwK ? pd.u - k0 : kUvwK;
  const int nk = (kn + 15) / 16;
  float av[2][4], an[2][4];
  uvw_load_w<T>(W, pd.u, w_out, k0, 0, lk, kout, kok, av);
  for (int kc = 0; kc < nk; ++kc) {
    uvw_load_w<T>(W, pd.u, w_out, k0, kc + 1, lk, kout, kok, an);  // next step's operands (zeros past u)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nt = 0; nt < 2 * L3 + 1; ++nt) {
      const v4f b = *reinterpret_cast<const v4f*>(tl + (nt * kUvwRows + li) * kUvwTP + 16 * kc + 4 * lk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) acc[s][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s][j], b[j], acc[s][nt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) av[s][j] = an[s][j];
  }
}

template <typename T>
__global__ __launch_bounds__(kUvwThreads) void uvw_fwd_kernel(UvwArgs a) {
  extern __shared__ __attribute__((aligned(16))) float tl[];  // [2 l3 + 1][16 rows][kUvwTP]
  const int tid = int(threadIdx.x), lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
  const int64_t z0 = int64_t(blockIdx.x) * kUvwRows;
  const int zt = tid >> 4, rt = tid & 15;
  // rows past B compute from the last row; their results are not stored
  const int64_t rowt = z0 + zt < a.B ? z0 + zt : a.B - 1;
  const T* __restrict__ xr = static_cast<const T*>(a.x) + rowt * a.dim_x;
  const T* __restrict__ yr = static_cast<const T*>(a.y) + rowt * a.dim_y;
  const int64_t row_out = z0 + li;
  T* __restrict__ orow = static_cast<T*>(a.out) + (row_out < a.B ? row_out : int64_t(0)) * a.dim_out;
  for (int gi = 0; gi < a.ngroups; ++gi) {
    const UvwGroupDev gd = ldc(a.groups + gi);
    static_for<0, kLmax + 1>([&](auto L3c) {
      constexpr int L3 = decltype(L3c)::value;
      if (gd.l3 != L3) return;
      for (int c0 = 0; c0 < gd.w_out; c0 += kUvwCols) {
        v4f acc[2][2 * L3 + 1];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int nt = 0; nt < 2 * L3 + 1; ++nt) acc[s][nt] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int pi = gd.p0; pi < gd.p1; ++pi) {
          const UvwPathDev pd = ldc(a.paths + pi);
          for (int k0 = 0; k0 < pd.u; k0 += kUvwK) {
            __syncthreads();  // the previous chunk's T has been read
            static_for<0, kLmax + 1>([&](auto L1c) {
              constexpr int L1 = decltype(L1c)::value;
              static_for<0, kLmax + 1>([&](auto L2c) {
                constexpr int L2 = decltype(L2c)::value;
                if constexpr (L3 >= (L1 > L2 ? L1 - L2 : L2 - L1) && L3 <= L1 + L2) {
                  if (pd.l1 == L1 && pd.l2 == L2) uvw_t_chunk<T, L1, L2, L3>(a, pd, xr, yr, k0, zt, rt, tl);
                }
              });
            });
            __syncthreads();
            uvw_mix_chunk<T, L3>(a, pd, gd.w_out, k0, c0, tl, acc, wave, li, lk);
          }
        }
        // lane: output channels c0 + 32 wave + 16 s + 4 lk + r of row z0 + li, component nt
        if (row_out < a.B) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int kb = c0 + 32 * wave + 16 * s + 4 * lk;
            if (kb < gd.w_out) {
#pragma unroll
              for (int nt = 0; nt < 2 * L3 + 1; ++nt) {
                const float o[4] = {acc[s][nt][0], acc[s][nt][1], acc[s][nt][2], acc[s][nt][3]};
                VecIO<T, 4>::store(orow + gd.out_off + nt * gd.w_out + kb, o);
              }
            }
          }
        }
      }
    });
  }
}

struct UvwTables {
  UvwPathDev* paths = nullptr;
  UvwGroupDev* groups = nullptr;
  int ngroups = 0, max_l3 = 0;
};

std::mutex g_uvw_mu;
std::map<std::pair<const cgtp_plan_s*, int>, UvwTables> g_uvw_tables;

const UvwTables& uvw_tables(const cgtp_plan_s* plan) {
  int dev = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_uvw_mu);
  auto it = g_uvw_tables.find({plan, dev});
  if (it != g_uvw_tables.end()) return it->second;
  // output blocks in output order, each with its paths in path order
  std::vector<UvwPathDev> pd;
  std::vector<UvwGroupDev> gd;
  UvwTables t;
  for (const OutBlock& ob : plan->outputs) {
    UvwGroupDev g{ob.l3, ob.out_off, ob.mul, int32_t(pd.size()), 0, 0, 0, 0};
    for (const PathInfo& p : plan->paths)
      if (p.out_off == ob.out_off)
        pd.push_back(UvwPathDev{p.l1, p.l2, p.mul, p.x_off, p.y_off, p.coef_off, p.w_off, 0});
    g.p1 = int32_t(pd.size());
    gd.push_back(g);
    t.max_l3 = std::max(t.max_l3, ob.l3);
  }
  CGTP_CHECK_HIP(hipMalloc(&t.paths, std::max<size_t>(pd.size(), 1) * sizeof(UvwPathDev)));
  if (hipMalloc(&t.groups, std::max<size_t>(gd.size(), 1) * sizeof(UvwGroupDev)) != hipSuccess) {
    (void)hipFree(t.paths);
    throw Error{CGTP_ERR_ALLOC, "uvw: device tables"};
  }
  CGTP_CHECK_HIP(hipMemcpy(t.paths, pd.data(), pd.size() * sizeof(UvwPathDev), hipMemcpyHostToDevice));
  CGTP_CHECK_HIP(hipMemcpy(t.groups, gd.data(), gd.size() * sizeof(UvwGroupDev), hipMemcpyHostToDevice));
  t.ngroups = int(gd.size());
  return g_uvw_tables.emplace(std::make_pair(plan, dev), t).first->second;
}

bool aligned_ptr(const void* p, size_t bytes) { return reinterpret_cast<uintptr_t>(p) % bytes == 0; }

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

void free_uvw_tables(const cgtp_plan_s* plan) {
  std::lock_guard<std::mutex> lock(g_uvw_mu);
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto it = g_uvw_tables.begin(); it != g_uvw_tables.end();) {
    if (it->first.first == plan) {
      if (hipSetDevice(it->first.second) == hipSuccess) {
        (void)hipFree(it->second.paths);
        (void)hipFree(it->second.groups);
      }
      it = g_uvw_tables.erase(it);
    } else {
      ++it;
    }
  }
  if (have) (void)hipSetDevice(cur);
}

void uvw_forward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w, void* out,
                        hipStream_t s) {
  if (B == 0) return;
  const size_t es = dtype_size(plan->dtype);
  if (!aligned_ptr(x, 4 * es) || !aligned_ptr(out, 4 * es))
    throw Error{CGTP_ERR_INVALID_ARG, "uvw: x and out must be aligned to 4 elements"};
  const DevTables& dt = plan_tables(plan);
  const UvwTables& t = uvw_tables(plan);
  UvwArgs a{};
  a.paths = t.paths;
  a.groups = t.groups;
  a.coef = static_cast<const float*>(dt.coef);
  a.x = x;
  a.y = y;
  a.w = w;
  a.out = out;
  a.B = B;
  a.dim_x = int(plan->dim_x);
  a.dim_y = int(plan->dim_y);
  a.dim_out = int(plan->dim_out);
  a.ngroups = t.ngroups;
  const dim3 grid(unsigned((B + kUvwRows - 1) / kUvwRows));
  const size_t lds = uvw_lds_bytes(t.max_l3);
  if (plan->dtype == CGTP_BF16)
    hipLaunchKernelGGL((uvw_fwd_kernel<bf16>), grid, dim3(kUvwThreads), lds, s, a);
  else
    hipLaunchKernelGGL((uvw_fwd_kernel<float>), grid, dim3(kUvwThreads), lds, s, a);
  CGTP_CHECK_HIP(hipGetLastError());
}

size_t uvw_backward_ws_bytes(const cgtp_plan_s* plan, int64_t B) {
  const size_t rows = align256(size_t(B) * size_t(plan->unit->dim_out) * dtype_size(plan->dtype));
  return 2 * rows + linear_backward_ws_bytes(plan->mix, B);
}

void uvw_backward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w, const void* g,
                         void* dx, void* dy, void* dw, void* ws, size_t ws_bytes, hipStream_t s) {
  if (B == 0) {
    if (dw) zero_rows(dw, plan->w_numel, dtype_size(plan->dtype), s);
    return;
  }
  const size_t need = uvw_backward_ws_bytes(plan, B);
  if (!ws || ws_bytes < need)
    throw Error{CGTP_ERR_WORKSPACE, "uvw tp_backward needs " + std::to_string(need) + " workspace bytes"};
  const size_t rows = align256(size_t(B) * size_t(plan->unit->dim_out) * dtype_size(plan->dtype));
  char* T = static_cast<char*>(ws);     // path outputs [B][dim_T]
  char* Gp = T + rows;                  // their cotangent g W^T [B][dim_T]
  char* lin_ws = Gp + rows;             // grad_W partials
  const void* ones = plan_tables(plan->unit).ones;
  if (dw) tp_forward_launch(plan->unit, B, x, y, ones, T, s);
  const bool need_g = dx || dy;
  if (dw || need_g)
    linear_backward_launch(plan->mix, B, T, w, g, need_g ? Gp : nullptr, dw, lin_ws,
                           ws_bytes - size_t(lin_ws - static_cast<char*>(ws)), s);
  if (need_g) tp_backward_launch(plan->unit, B, x, y, ones, Gp, dx, dy, nullptr, nullptr, 0, s);
}

}  // namespace cgtp
