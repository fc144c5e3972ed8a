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
// Forward, one kernel: a workgroup owns 32 rows and walks every output block
// and every path into it. Per path (and chunk of 128 x channels) each lane
// first requests its W operands for the whole chunk (from L2), then the 512
// lanes form T_p for the 32 rows in LDS on the vector ALUs (lane = (row, 4
// channels), the coefficient sparsity pattern fixed at compile time, as in
// the channel-wise product), then the eight waves run the matrix cores on
// D[k][z] += sum_a W_p[a][k] T_p[z, m3, a] for every m3: wave w owns output
// channels [16w, 16w + 16) of a 128-channel column tile (one 16-row A tile),
// all 2 l3 + 1 components of both 16-row N tiles. D stays in the accumulators
// over all paths of the block; each lane then stores 4 consecutive output
// channels of one (row, m3). fp32 storage: v_mfma_f32_16x16x4_f32 on fp32 T;
// bf16 storage: v_mfma_f32_16x16x32_bf16 on T rounded to bf16 in LDS.
//
// Backward, composed from the library's kernels through the workspace:
//   T  = unit-weight uvu forward (the path outputs)
//   dW = sum over rows of T^T g, G' = g W^T    (the linear map's backward)
//   dx, dy = uvu backward with unit weights and cotangent G'
// so every sum keeps a fixed order and results are deterministic.
#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>
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

constexpr int kUvwThreads = 512;
// Rows per workgroup: RT MFMA N tiles of 16 rows (2 for plans up to degree 3,
// 1 at degree 4, where two tiles' accumulators would spill).
template <int LM>
constexpr int uvw_row_tiles() { return LM >= 4 ? 1 : 2; }
constexpr int kUvwK = 128;     // x channels of one T chunk
constexpr int kUvwCols = 128;  // output channels per column tile (8 waves x 16)

// How T and W meet on the matrix cores. fp32 storage: T as fp32 in LDS,
// v_mfma_f32_16x16x4_f32, lane slot lk of step j takes contraction index
// 16 kc + 4 lk + j (8 steps of 16 per chunk). bf16 storage: T rounded to bf16
// in LDS (as a bf16 store of the path outputs would round it) and
// v_mfma_f32_16x16x32_bf16, lane slot lk takes 32 kc + 8 lk + j, j < 8 (4 steps
// of 32); bf16 x bf16 products are exact in fp32 and sum in fp32.
template <typename T>
struct UvwMma {
  static constexpr int KS = 16;               // contraction per step
  static constexpr int NK = kUvwK / KS;       // steps per chunk
  static constexpr int TP = kUvwK + 4;        // padded LDS row of T, in elements
  using TL = float;                           // LDS element of T
  using AW = float __attribute__((ext_vector_type(4)));  // one step's W operand of one A tile
};
template <>
struct UvwMma<bf16> {
  static constexpr int KS = 32;
  static constexpr int NK = kUvwK / KS;
  static constexpr int TP = kUvwK + 8;
  using TL = uint16_t;
  using AW = uint16_t __attribute__((ext_vector_type(8)));
};
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <typename T>
size_t uvw_lds_bytes(int max_l3, int rows) {
  using M = UvwMma<T>;
  return size_t(2 * max_l3 + 1) * size_t(rows) * M::TP * sizeof(typename M::TL);
}

// T_p for one row of the workgroup and x channels k0..k0+127 into LDS [m3][row][channel]
// (zeros past u). The lane takes row zt and the channel quad 4 rt.
template <typename T, int L1, int L2, int L3, int ROWS>
__device__ __forceinline__ void uvw_t_chunk(const UvwArgs& a, const UvwPathDev& pd, const T* __restrict__ xr,
                                            const T* __restrict__ yr, int k0, int zt, int rt,
                                            typename UvwMma<T>::TL* tl) {
  using M = UvwMma<T>;
  float yb[2 * L2 + 1];
#pragma unroll
  for (int m = 0; m < 2 * L2 + 1; ++m) yb[m] = to_acc<float>(yr[pd.y_off + m]);
  {
    const int al = 4 * rt, ag = k0 + al;
    const bool ok = ag < pd.u;  // u is a multiple of 4: a quad is wholly inside or past it
    float xb[2 * L1 + 1][4];
#pragma unroll
    for (int m = 0; m < 2 * L1 + 1; ++m) VecIO<T, 4>::load(xr + pd.x_off + m * pd.u + (ok ? ag : 0), xb[m]);
    float o[2 * L3 + 1][4];
    fwd_core<L1, L2, L3, 4, float>(xb, yb, a.coef + pd.coef_off, o);
#pragma unroll
    for (int m = 0; m < 2 * L3 + 1; ++m) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ok ? o[m][i] : 0.f;
      VecIO<T, 4>::store(reinterpret_cast<T*>(tl + (m * ROWS + zt) * M::TP + al), v);
    }
  }
}

// This lane's W operands of a whole chunk: W_p[a][k] for its contraction
// slots of every step and its output channel, requested at once (before the
// T phase, so their latency hides behind it); zeros past u or w_out.
template <typename T>
__device__ __forceinline__ void uvw_load_w(const T* __restrict__ W, int u, int w_out, int k0, int lk, int kout,
                                           bool kok, typename UvwMma<T>::AW (&aw)[UvwMma<T>::NK]) {
  using M = UvwMma<T>;
  constexpr int J = M::KS / 4;  // contraction values per lane and step
#pragma unroll
  for (int kc = 0; kc < M::NK; ++kc)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int ka = k0 + M::KS * kc + J * lk + j;
      const bool aok = ka < u;
      const T v = W[int64_t(aok ? ka : 0) * w_out + (kok ? kout : 0)];
      if constexpr (std::is_same<T, bf16>::value)
        aw[kc][j] = aok && kok ? v.bits : uint16_t(0);
      else
        aw[kc][j] = aok && kok ? v : 0.f;
    }
}

template <typename T, int L3, int RT>
__device__ __forceinline__ void uvw_mix_chunk(int kn, const typename UvwMma<T>::TL* tl,
                                              const typename UvwMma<T>::AW (&aw)[UvwMma<T>::NK],
                                              v4f (&acc)[RT][2 * L3 + 1], int li, int lk) {
  using M = UvwMma<T>;
#pragma unroll
  for (int kc = 0; kc < M::NK; ++kc) {
    if (kc * M::KS >= kn) break;  // uniform: past the chunk's channels
#pragma unroll
    for (int nt = 0; nt < 2 * L3 + 1; ++nt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int row = nt * 16 * RT + 16 * rt + li;
        if constexpr (std::is_same<T, bf16>::value) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(tl + row * M::TP + M::KS * kc + 8 * lk));
          acc[rt][nt] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aw[kc]), b, acc[rt][nt], 0, 0, 0);
        } else {
          const v4f b = *reinterpret_cast<const v4f*>(tl + row * M::TP + M::KS * kc + 4 * lk);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[kc][j], b[j], acc[rt][nt], 0, 0, 0);
        }
      }
  }
}

// LM: the plan's largest degree (x, y and outputs), so that only the
// coefficient patterns a plan can take are compiled into the kernel.
template <typename T, int LM>
__global__ __launch_bounds__(kUvwThreads) void uvw_fwd_kernel(UvwArgs a) {
  using M = UvwMma<T>;
  constexpr int RT = uvw_row_tiles<LM>(), ROWS = 16 * RT;
  extern __shared__ __attribute__((aligned(16))) unsigned char uvw_smem[];
  typename M::TL* tl = reinterpret_cast<typename M::TL*>(uvw_smem);  // [2 l3 + 1][16 rows][M::TP]
  const int tid = int(threadIdx.x), lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
  const int64_t z0 = int64_t(blockIdx.x) * ROWS;
  const int zt = tid >> 5, rt = tid & 31;  // T phase: rows zt + 16 r of the workgroup, channel quad rt
  // rows past B compute from the last row; their results are not stored
  const T* __restrict__ xr[RT];
  const T* __restrict__ yr[RT];
  T* __restrict__ orow[RT];
  bool out_ok[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int64_t rowt = z0 + zt + 16 * r < a.B ? z0 + zt + 16 * r : a.B - 1;
    xr[r] = static_cast<const T*>(a.x) + rowt * a.dim_x;
    yr[r] = static_cast<const T*>(a.y) + rowt * a.dim_y;
    const int64_t row_out = z0 + 16 * r + li;
    out_ok[r] = row_out < a.B;
    orow[r] = static_cast<T*>(a.out) + (out_ok[r] ? row_out : int64_t(0)) * a.dim_out;
  }
  for (int gi = 0; gi < a.ngroups; ++gi) {
    const UvwGroupDev gd = ldc(a.groups + gi);
    static_for<0, LM + 1>([&](auto L3c) {
      constexpr int L3 = decltype(L3c)::value;
      if (gd.l3 != L3) return;
      for (int c0 = 0; c0 < gd.w_out; c0 += kUvwCols) {
        const int kout = c0 + 16 * wave + li;
        const bool kok = kout < gd.w_out;
        v4f acc[RT][2 * L3 + 1];
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int nt = 0; nt < 2 * L3 + 1; ++nt) acc[r][nt] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int pi = gd.p0; pi < gd.p1; ++pi) {
          const UvwPathDev pd = ldc(a.paths + pi);
          const T* __restrict__ W = static_cast<const T*>(a.w) + pd.w_off;
          for (int k0 = 0; k0 < pd.u; k0 += kUvwK) {
            typename M::AW aw[M::NK];
            uvw_load_w<T>(W, pd.u, gd.w_out, k0, lk, kout, kok, aw);
            __syncthreads();  // the previous chunk's T has been read
            static_for<0, LM + 1>([&](auto L1c) {
              constexpr int L1 = decltype(L1c)::value;
              static_for<0, LM + 1>([&](auto L2c) {
                constexpr int L2 = decltype(L2c)::value;
                if constexpr (L3 >= (L1 > L2 ? L1 - L2 : L2 - L1) && L3 <= L1 + L2) {
                  if (pd.l1 == L1 && pd.l2 == L2) {
#pragma unroll
                    for (int r = 0; r < RT; ++r)
                      uvw_t_chunk<T, L1, L2, L3, ROWS>(a, pd, xr[r], yr[r], k0, zt + 16 * r, rt, tl);
                  }
                }
              });
            });
            __syncthreads();
            uvw_mix_chunk<T, L3, RT>(pd.u - k0, tl, aw, acc, li, lk);
          }
        }
        // lane: output channels c0 + 16 wave + 4 lk + r of rows z0 + 16 rt + li, component nt
        const int kb = c0 + 16 * wave + 4 * lk;
        if (kb < gd.w_out) {
#pragma unroll
          for (int r = 0; r < RT; ++r)
            if (out_ok[r]) {
#pragma unroll
              for (int nt = 0; nt < 2 * L3 + 1; ++nt) {
                const float o[4] = {acc[r][nt][0], acc[r][nt][1], acc[r][nt][2], acc[r][nt][3]};
                VecIO<T, 4>::store(orow[r] + gd.out_off + nt * gd.w_out + kb, o);
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
  int lm = plan->lm;
  for (const BlockInfo& b : plan->blocks) lm = std::max(lm, b.l1);
  const bool h = plan->dtype == CGTP_BF16;
  auto go = [&](auto LMc) {
    constexpr int LM = decltype(LMc)::value;
    constexpr int ROWS = 16 * uvw_row_tiles<LM>();
    const dim3 grid(unsigned((B + ROWS - 1) / ROWS));
    const size_t lds = h ? uvw_lds_bytes<bf16>(t.max_l3, ROWS) : uvw_lds_bytes<float>(t.max_l3, ROWS);
    if (h)
      hipLaunchKernelGGL((uvw_fwd_kernel<bf16, LM>), grid, dim3(kUvwThreads), lds, s, a);
    else
      hipLaunchKernelGGL((uvw_fwd_kernel<float, LM>), grid, dim3(kUvwThreads), lds, s, a);
  };
  if (lm <= 2)
    go(std::integral_constant<int, 2>());
  else if (lm == 3)
    go(std::integral_constant<int, 3>());
  else
    go(std::integral_constant<int, kLmax>());
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
