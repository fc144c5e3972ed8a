// Message-passing convolution over CSR-by-destination edges.
//
// What is computed: the tensor-field-network convolution of the MolSSI e3nn
// course, lesson 06a, m_ij = (R(|r_ij|) Y(rhat_ij)) (x)_w h_j summed at the
// receiver i, with the radial factor given as per-edge, per-path, per-channel
// weights and a constant scale (the sqrt(num_neighbors) normalisation of
// e3nn_mlx "Modular v2106 point models"):
//   out[n] = scale * sum_{e: dst(e)=n} TP(x[src(e)], sh[e], w[e]).
// "E3J: An Efficient and Open-Source Backend for Euclidean Equivariant
// Operations on GPU and TPU", 3.1.2 / E.2.2 / E.3 / E.4: stream the edges of a
// receiver, aggregate in CSR order without atomics, never write edge messages
// to memory (complex layers that materialise edge-wise intermediates pay for
// it in traffic, as the Sobek card page notes).
//
// Forward, fused form (each degree occurs at most once in y): one wave owns
// (receiver n, x block b, 64-channel chunk); lanes are channels. For every
// edge of n it gathers x[src] for block b (one coalesced 256-byte run per m1),
// reads sh[e] with uniform loads, streams the block's weights w[e, p, :], and
// accumulates every path of the block in registers - the register layout of
// the accumulators is fixed at compile time by (l1 of the block, L), so the
// paths live at constant register offsets. One store per output element.
// Forward, general form (any y): one wave per (receiver, path, chunk).
//
// Backward: the row-parallel tensor-product backward runs over edges with x
// gathered by src and grad_out gathered by dst (times scale): it writes
// grad_sh[e] and grad_w[e] directly and a per-edge grad_x partial; the partials
// are then summed per source node over the transpose, in CSR-position order.
#pragma once

#include <type_traits>

#include "cg_pattern.h"
#include "common.hpp"
#include "device_util.hpp"
#include "graph.hpp"
#include "tp_core.hpp"

namespace cgtp {

// ------------------------------------------------- compile-time slot layout
struct SlotT {
  int l2, l3, acc;  // acc: first accumulator register of the slot
  int src;          // index of the slot in the plan's (l2, l3) slot table
};

constexpr int imin(int a, int b) { return a < b ? a : b; }
constexpr int idiff(int a, int b) { return a > b ? a - b : b - a; }

constexpr int slot_count(int L1, int L) {
  int n = 0;
  for (int l2 = 0; l2 <= L; ++l2)
    for (int l3 = idiff(L1, l2); l3 <= imin(L1 + l2, L); ++l3) ++n;
  return n;
}
constexpr int slot_regs(int L1, int L) {
  int n = 0;
  for (int l2 = 0; l2 <= L; ++l2)
    for (int l3 = idiff(L1, l2); l3 <= imin(L1 + l2, L); ++l3) n += 2 * l3 + 1;
  return n;
}

template <int L1, int L>
struct Slots {
  static constexpr int NS = slot_count(L1, L);
  static constexpr int NACC = slot_regs(L1, L);
  struct Arr {
    SlotT p[NS > 0 ? NS : 1];
  };
  static constexpr Arr build() {
    Arr a{};
    int k = 0, acc = 0;
    for (int l2 = 0; l2 <= L; ++l2)
      for (int l3 = idiff(L1, l2); l3 <= imin(L1 + l2, L); ++l3) {
        a.p[k] = SlotT{l2, l3, acc, k};
        ++k;
        acc += 2 * l3 + 1;
      }
    return a;
  }
  static constexpr Arr arr = build();
};

// Slots of a plan with outputs collapsed by (l3, p3). Within one x block the
// output parity of a slot is fixed by the parity of l2 when every y block has
// parity s (-1)^l2 for one sign s (harmonics: s = +1; the planner sends other
// plans to the general kernel), so the slots of one output type are those
// with equal (l2 mod 2, l3): they are listed together and share one
// accumulator.
constexpr int slot_regs_collapsed(int L1, int L) {
  int n = 0;
  for (int par = 0; par < 2; ++par)
    for (int l3 = 0; l3 <= L; ++l3) {
      bool any = false;
      for (int l2 = par; l2 <= L; l2 += 2) any = any || (l3 >= idiff(L1, l2) && l3 <= imin(L1 + l2, L));
      if (any) n += 2 * l3 + 1;
    }
  return n;
}

template <int L1, int L>
struct SlotsC {
  static constexpr int NS = slot_count(L1, L);
  static constexpr int NACC = slot_regs_collapsed(L1, L);
  struct Arr {
    SlotT p[NS > 0 ? NS : 1];
  };
  static constexpr Arr build() {
    Arr a{};
    int k = 0, acc = 0;
    for (int par = 0; par < 2; ++par)
      for (int l3 = 0; l3 <= L; ++l3) {
        bool any = false;
        for (int l2 = par; l2 <= L; l2 += 2)
          if (l3 >= idiff(L1, l2) && l3 <= imin(L1 + l2, L)) {
            // index of (l2, l3) in the (l2, l3)-ordered table
            int src = 0;
            for (int q2 = 0; q2 < l2; ++q2) src += imin(L1 + q2, L) - idiff(L1, q2) + 1;
            src += l3 - idiff(L1, l2);
            a.p[k++] = SlotT{l2, l3, acc, src};
            any = true;
          }
        if (any) acc += 2 * l3 + 1;
      }
    return a;
  }
  static constexpr Arr arr = build();
};

struct ConvArgs {
  const PathDev* paths;
  const BlockDev* blocks;
  const void* coef;
  const int32_t* slot_paths;
  const int32_t* slot_off;
  const int32_t* row_ptr;
  const int32_t* src;
  const int32_t* order;  // receiver schedule (a locality order of the nodes)
  const void* x;
  const void* sh;
  const void* w;
  void* out;
  int64_t N;
  int dim_x, dim_y, dim_out, W;
  int nblocks, nchunks, npaths, L;
  int block;    // x block of a degree-specialised launch
  int lg_log2;  // lanes per edge group (fused forward)
  int collapse; // outputs collapsed by (l3, p3): add into the (zeroed) output instead of storing
  void* acc;    // collapsed outputs: running sum [N][dim_out] in the accumulation type that the
                // x blocks add into instead of the output (NULL: the output itself)
  int coef_zero;  // offset of a run of zero coefficients (one whole pattern) in the table
  int pad;        // padding node (its incoming edges are skipped) or -1
  int yoff[kLmax + 1];
  double scale;
};

constexpr int kWaves = kBlock / 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

__device__ __forceinline__ int conv_wave_id() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6); }

// Workgroups are handed to the XCDs round-robin (workgroup w runs on XCD
// w mod 8). Renumber them so that each XCD takes one contiguous range of the
// receiver schedule: receivers that are close in the schedule share source
// rows, and those reads then meet in the same L2.
__device__ __forceinline__ int64_t xcd_block() {
  const int64_t P = gridDim.x, w = blockIdx.x;
  const int64_t q = P / kXcds, r = P % kXcds, x = w % kXcds, i = w / kXcds;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// ------------------------------------------------------------ fused forward
// Slot chunks: consecutive slots whose accumulators fit a register budget of
// `budget` entries per channel; the chunks of one block run as separate waves
// of the same workgroup (they share the gathered rows through the caches).
// Slots that share an accumulator (collapsed outputs) stay in one chunk.
template <typename S, int budget>
struct Chunks {
  static constexpr bool opens(int i) { return i == 0 || S::arr.p[i].acc != S::arr.p[i - 1].acc; }
  static constexpr int count() {
    int n = 0, acc = budget;
    for (int i = 0; i < S::NS; ++i) {
      if (!opens(i)) continue;
      const int sz = 2 * S::arr.p[i].l3 + 1;
      if (acc + sz > budget) {
        ++n;
        acc = 0;
      }
      acc += sz;
    }
    return n;
  }
  static constexpr int NCH = count();
  struct Arr {
    int begin[NCH + 1];
  };
  static constexpr Arr build() {
    Arr a{};
    int n = 0, acc = budget;
    for (int i = 0; i < S::NS; ++i) {
      if (!opens(i)) continue;
      const int sz = 2 * S::arr.p[i].l3 + 1;
      if (acc + sz > budget) {
        a.begin[n++] = i;
        acc = 0;
      }
      acc += sz;
    }
    a.begin[n] = S::NS;
    return a;
  }
  static constexpr Arr arr = build();
};

template <int L1, int L, bool COL>
using SlotsOf = typename std::conditional<COL, SlotsC<L1, L>, Slots<L1, L>>::type;

#ifndef CGTP_CONV_ACC_REGS
#define CGTP_CONV_ACC_REGS 64
#endif
// accumulator entries per channel that fit CGTP_CONV_ACC_REGS registers
template <typename A, int VEC>
constexpr int conv_budget() {
  return CGTP_CONV_ACC_REGS / (VEC * int(sizeof(A) / 4)) > 9 ? CGTP_CONV_ACC_REGS / (VEC * int(sizeof(A) / 4))
                                                              : 9;
}

// One wave = (receiver n, one slot chunk of x block b, one channel chunk).
// Lanes form G = 64 / LG groups of LG lanes; group g takes edges e0+g,
// e0+g+G, ... and lane k of a group owns channels c .. c+VEC-1.
//
// The edge loop body has no branches on the plan: a slot the plan does not
// have still runs, from valid addresses (weights at offset 0 of the edge's row,
// coefficients from the zero-padded start of the table, harmonics of a missing
// degree from the table as well) into accumulators that are never stored. So
// all loads of an edge are independent once its source index is known, and
// the source indices of up to 64 edges are fetched with one load and handed
// out with lane shuffles.
template <typename T, typename A, int VEC, int L1, int L, bool COL, int CH>
__device__ __forceinline__ void fwd_fused_chunk(const ConvArgs& a, int64_t n, const BlockDev& blk,
                                                int c, bool valid, int g, int G) {
  using S = SlotsOf<L1, L, COL>;
  using CK = Chunks<S, conv_budget<A, VEC>()>;
  constexpr int s0 = CK::arr.begin[CH], s1 = CK::arr.begin[CH + 1];
  constexpr int acc0 = S::arr.p[s0].acc;
  constexpr int NACC = (s1 < S::NS ? S::arr.p[s1].acc : S::NACC) - acc0;
  A acc[NACC][VEC];
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[i][v] = A(0);
  int pid[s1 - s0], woff[s1 - s0], coff[s1 - s0];
  const int so = ldc(a.slot_off + a.block);
#pragma unroll
  for (int s = 0; s < s1 - s0; ++s) {
    pid[s] = ldc(a.slot_paths + so + S::arr.p[s0 + s].src);
    woff[s] = pid[s] >= 0 ? ldc(&a.paths[pid[s]].w_off) : 0;
    // an absent slot runs on zero coefficients when its accumulator is
    // shared (collapsed outputs); otherwise on any in-bounds ones (discarded)
    coff[s] = pid[s] >= 0 ? ldc(&a.paths[pid[s]].coef_off) : (COL ? a.coef_zero : 0);
  }
  const A* __restrict__ cf = static_cast<const A*>(a.coef);
  const T* __restrict__ X = static_cast<const T*>(a.x);
  const int lane = int(threadIdx.x & 63);
  const int32_t e0 = a.row_ptr[n], e1 = n == a.pad ? e0 : a.row_ptr[n + 1];  // padding edges skipped
  for (int32_t base = e0; base < e1; base += 64) {
    const int nb = e1 - base < 64 ? e1 - base : 64;  // uniform over the wave
    const int32_t srcv = lane < nb ? a.src[base + lane] : 0;
    for (int k0 = 0; k0 < nb; k0 += G) {
      const int k = k0 + g;
      const int64_t j = __shfl(srcv, k < nb ? k : 0, 64);
      if (!valid || k >= nb) continue;
      const int64_t e = base + k;
      A xb[2 * L1 + 1][VEC];
#pragma unroll
      for (int m = 0; m < 2 * L1 + 1; ++m) VecIO<T, VEC>::load(X + j * a.dim_x + blk.x_off + m * blk.mul + c, xb[m]);
      const T* __restrict__ Ye = static_cast<const T*>(a.sh) + e * a.dim_y;
      const T* __restrict__ we = static_cast<const T*>(a.w) + e * a.W;
      // harmonics of the edge: per l2 run of slots, or (collapsed order, where
      // l2 alternates) every degree the chunk uses, once per edge
      A ycur[2 * L + 1];
      A yall[COL ? (L + 1) * (L + 1) : 1];
      if constexpr (COL) {
        static_for<0, L + 1>([&](auto D2) {
          constexpr int l2 = decltype(D2)::value;
          constexpr bool used = [] {
            for (int i = s0; i < s1; ++i)
              if (S::arr.p[i].l2 == l2) return true;
            return false;
          }();
          if constexpr (used) {
            const int yo = a.yoff[l2];
            const T* __restrict__ yp = yo >= 0 ? Ye + yo : static_cast<const T*>(a.coef);
#pragma unroll
            for (int m = 0; m < 2 * l2 + 1; ++m) yall[l2 * l2 + m] = to_acc<A>(yp[m]);
          }
        });
      }
      static_for<s0, s1>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr SlotT st = S::arr.p[i];
        constexpr bool first_of_l2 = (i == s0) || (S::arr.p[i > 0 ? i - 1 : 0].l2 != st.l2);
        if constexpr (!COL && first_of_l2) {
          const int yo = a.yoff[st.l2];
          const T* __restrict__ yp = yo >= 0 ? Ye + yo : static_cast<const T*>(a.coef);
#pragma unroll
          for (int m = 0; m < 2 * st.l2 + 1; ++m) ycur[m] = to_acc<A>(yp[m]);
        }
        A wv[VEC];
        VecIO<T, VEC>::load(we + woff[i - s0] + c, wv);
        A yb[2 * st.l2 + 1];
#pragma unroll
        for (int m = 0; m < 2 * st.l2 + 1; ++m) yb[m] = COL ? yall[st.l2 * st.l2 + m] : ycur[m];
        A t[2 * st.l3 + 1][VEC];
        fwd_core<L1, st.l2, st.l3, VEC, A>(xb, yb, cf + coff[i - s0], t);
        // an absent slot (zero coefficients) adds zero to a shared accumulator
        // for finite inputs
#pragma unroll
        for (int m = 0; m < 2 * st.l3 + 1; ++m)
#pragma unroll
          for (int v = 0; v < VEC; ++v)
            acc[st.acc - acc0 + m][v] = fma(wv[v], t[m][v], acc[st.acc - acc0 + m][v]);
      });
    }
  }
  // sum the groups' partial sums (every lane takes part), then group 0 stores
  xor_sum_n<NACC * VEC>(reinterpret_cast<A (&)[NACC * VEC]>(acc), 64 / G, 64);
  if (!valid || g != 0) return;
  T* __restrict__ outn = static_cast<T*>(a.out) + n * a.dim_out;
  const A sc = A(a.scale);
  static_for<s0, s1>([&](auto I) {
    constexpr int i = decltype(I)::value;
    constexpr SlotT st = S::arr.p[i];
    if constexpr (!COL) {
      if (pid[i - s0] >= 0) {
        const PathDev pd = ldc(a.paths + pid[i - s0]);
#pragma unroll
        for (int m = 0; m < 2 * st.l3 + 1; ++m) {
          A o[VEC];
#pragma unroll
          for (int v = 0; v < VEC; ++v) o[v] = sc * acc[st.acc - acc0 + m][v];
          VecIO<T, VEC>::store(outn + pd.out_off + m * pd.mul + c, o);
        }
      }
    } else if constexpr (i == s0 || S::arr.p[i > 0 ? i - 1 : 0].acc != st.acc) {
      // first slot of an output type: the block of any of its present slots;
      // x blocks of one output type add into it in launch order
      int path = -1;
      static_for<i, s1>([&](auto J) {
        constexpr int jj = decltype(J)::value;
        if constexpr (S::arr.p[jj].acc == st.acc) {
          if (path < 0) path = pid[jj - s0];
        }
      });
      if (path >= 0) {
        const PathDev pd = ldc(a.paths + path);
        A* __restrict__ accn = a.acc ? static_cast<A*>(a.acc) + n * a.dim_out : nullptr;
#pragma unroll
        for (int m = 0; m < 2 * st.l3 + 1; ++m) {
          A o[VEC], prev[VEC];
          const int off = pd.out_off + m * pd.mul + c;
          if (accn)
            VecIO<A, VEC>::load(accn + off, prev);
          else
            VecIO<T, VEC>::load(outn + off, prev);
#pragma unroll
          for (int v = 0; v < VEC; ++v) o[v] = prev[v] + sc * acc[st.acc - acc0 + m][v];
          if (accn)
            VecIO<A, VEC>::store(accn + off, o);
          else
            VecIO<T, VEC>::store(outn + off, o);
        }
      }
    }
  });
}

// Work items: (receiver, slot chunk, channel chunk), slot chunks innermost so
// one workgroup's waves read the same rows. With collapsed outputs (COL) the
// chunks hold whole output types, so no two waves of a launch add into the
// same block.
#ifndef CGTP_CONV_FWD_WAVES
#define CGTP_CONV_FWD_WAVES 0
#endif
// waves per SIMD a forward kernel is compiled for (0 in the macro: per
// kernel). The fp64 kernels of x blocks of degree 2-4 at L = 4 take 173-175
// VGPRs (2 waves) when left alone and fit under the 3-wave line (168) without
// spilling: 12 % faster on the 100k-point workload. Kernels already under the
// line are left alone: the hint made the compiler squeeze the degree-1 one
// (167 -> 149 VGPRs at the same occupancy) and it ran 35 % slower; the
// collapsed-output kernels would spill.
template <typename T, int L1, int L, bool COL>
struct ConvFwdWaves {
  static constexpr int value = CGTP_CONV_FWD_WAVES != 0 ? CGTP_CONV_FWD_WAVES
                               : (std::is_same<T, double>::value && !COL && L == 4 && L1 >= 2) ? 3
                                                                                              : 1;
};

template <typename T, typename A, int VEC, int L1, int L, bool COL>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(ConvFwdWaves<T, L1, L, COL>::value)))
void conv_fwd_fused_kernel(ConvArgs a) {
  using CK = Chunks<SlotsOf<L1, L, COL>, conv_budget<A, VEC>()>;
  const int64_t item = xcd_block() * kWaves + conv_wave_id();
  const int64_t per_node = int64_t(CK::NCH) * a.nchunks;
  const int64_t pos = item / per_node;
  if (pos >= a.N) return;
  const int rem = int(item - pos * per_node);
  const int64_t n = a.order[pos];
  const int cc = rem / CK::NCH;
  const int ch = rem - cc * CK::NCH;
  const BlockDev blk = ldc(a.blocks + a.block);
  const int lane = int(threadIdx.x & 63);
  const int LG = 1 << a.lg_log2;
  const int G = 64 >> a.lg_log2;
  const int g = lane >> a.lg_log2;
  const int c = (cc * LG + (lane & (LG - 1))) * VEC;
  const bool valid = c < blk.mul;
  static_for<0, CK::NCH>([&](auto C) {
    constexpr int CH = decltype(C)::value;
    if (ch == CH) fwd_fused_chunk<T, A, VEC, L1, L, COL, CH>(a, n, blk, c, valid, g, G);
  });
}

// ----------------------------------------------------------- general forward
template <typename T, typename A, int L1, int L2, int L3>
__device__ __forceinline__ void fwd_general_path(const ConvArgs& a, int64_t n, const PathDev& pd, int c) {
  A acc[2 * L3 + 1];
#pragma unroll
  for (int m = 0; m < 2 * L3 + 1; ++m) acc[m] = A(0);
  const A* __restrict__ cf = static_cast<const A*>(a.coef) + pd.coef_off;
  const T* __restrict__ X = static_cast<const T*>(a.x);
  const int32_t e0 = a.row_ptr[n], e1 = n == a.pad ? e0 : a.row_ptr[n + 1];  // padding edges skipped
  for (int32_t e = e0; e < e1; ++e) {
    const int64_t j = a.src[e];
    A xb[2 * L1 + 1][1];
#pragma unroll
    for (int m = 0; m < 2 * L1 + 1; ++m) xb[m][0] = to_acc<A>(X[j * a.dim_x + pd.x_off + m * pd.mul + c]);
    const T* __restrict__ Ye = static_cast<const T*>(a.sh) + int64_t(e) * a.dim_y;
    A yb[2 * L2 + 1];
#pragma unroll
    for (int m = 0; m < 2 * L2 + 1; ++m) yb[m] = to_acc<A>(Ye[pd.y_off + m]);
    const A wv = to_acc<A>(static_cast<const T*>(a.w)[int64_t(e) * a.W + pd.w_off + c]);
    A t[2 * L3 + 1][1];
    fwd_core<L1, L2, L3, 1, A>(xb, yb, cf, t);
#pragma unroll
    for (int m = 0; m < 2 * L3 + 1; ++m) acc[m] = fma(wv, t[m][0], acc[m]);
  }
  T* __restrict__ outn = static_cast<T*>(a.out) + n * a.dim_out;
  A* __restrict__ accn = a.acc ? static_cast<A*>(a.acc) + n * a.dim_out : nullptr;
  const A sc = A(a.scale);
#pragma unroll
  for (int m = 0; m < 2 * L3 + 1; ++m) {
    const int off = pd.out_off + m * pd.mul + c;
    A o = sc * acc[m];
    if (accn) {
      accn[off] += o;
    } else {
      if (a.collapse) o += to_acc<A>(outn[off]);
      from_acc(outn[off], o);
    }
  }
}

template <typename T, typename A>
__global__ __launch_bounds__(kBlock) void conv_fwd_general_kernel(ConvArgs a) {
  const int64_t item = xcd_block() * kWaves + conv_wave_id();
  // collapsed outputs: one wave takes every path of its receiver in turn
  const int np = a.collapse ? 1 : a.npaths;
  const int64_t per_node = int64_t(np) * a.nchunks;
  const int64_t pos = item / per_node;
  if (pos >= a.N) return;
  const int rem = int(item - pos * per_node);
  const int64_t n = a.order[pos];
  const int p0 = rem / a.nchunks;
  const int chunk = rem - p0 * a.nchunks;
  const int p1 = a.collapse ? a.npaths : p0 + 1;
  for (int p = p0; p < p1; ++p) {
    const PathDev pd = ldc(a.paths + p);
    const int c = chunk * 64 + int(threadIdx.x & 63);
    if (c >= pd.mul) continue;
    static_for<0, kLmax + 1>([&](auto A1) {
      constexpr int L1 = decltype(A1)::value;
      if (pd.l1 == L1) {
        static_for<0, kLmax + 1>([&](auto A2) {
          constexpr int L2 = decltype(A2)::value;
          if (pd.l2 == L2) {
            static_for<0, kLmax + 1>([&](auto A3) {
              constexpr int L3 = decltype(A3)::value;
              if constexpr (L3 >= idiff(L1, L2) && L3 <= L1 + L2) {
                if (pd.l3 == L3) fwd_general_path<T, A, L1, L2, L3>(a, n, pd, c);
              }
            });
          }
        });
      }
    });
  }
}

// ------------------------------------------------------------ fused backward
#ifndef CGTP_CONV_BWD_VEC
#define CGTP_CONV_BWD_VEC 4
#endif

// Extra arguments of the fused backward.
struct ConvBwdArgs {
  const void* g;  // grad_out [N][dim_out]
  void* dsh;      // grad_sh [E][dim_y] (accumulated over x blocks in stream order)
  void* dw;       // grad_w [E][W]
  void* dxp;      // grad_x partials [E][dim_x], accumulation type
  int dy_accum;
  int dsh_acc;    // dsh is this x block's own [E][dim_y] in the accumulation type
};

// One workgroup = (receiver n, x block b, channel chunk). The block's slice
// of scale * grad_out[n] is staged in LDS ([slot accumulator row][channel]);
// lane groups of LG lanes sweep the receiver's edges; per edge they form the
// transposed products of every path of the block:
//   q[m1]   = sum_m3 A[m1,m3] g[m3]                      (A = C y)
//   grad_w  = sum_m1 x[m1] q[m1]                          -> stored per edge
//   dx_e   += w q[m1]                                     -> per-edge partial
//   dy[m2] += C sum_u w x[m1] g[m3]                       -> reduced over the group
#ifndef CGTP_CONV_BWD_WAVES
#define CGTP_CONV_BWD_WAVES 0
#endif
// waves per SIMD the backward is compiled for (0 in the macro: per kernel).
// The fp32 (l1, L) = (2, 4) kernel needs two registers more than the 3-wave
// line when left alone and fits under it without spilling; the larger ones
// would spill.
template <typename T, int L1, int L>
struct ConvBwdWaves {
  static constexpr int value = CGTP_CONV_BWD_WAVES != 0                                      ? CGTP_CONV_BWD_WAVES
                               : (std::is_same<T, float>::value && L1 == 2 && L == 4) ? 3
                                                                                          : 1;
};

template <typename T, typename A, int VEC, int L1, int L>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(ConvBwdWaves<T, L1, L>::value)))
void conv_bwd_fused_kernel(ConvArgs a, ConvBwdArgs bw) {
  using S = Slots<L1, L>;
  constexpr int NS = S::NS;
  constexpr int NY = (L + 1) * (L + 1);
  extern __shared__ unsigned char smem_raw[];
  const int LG = 1 << a.lg_log2;
  const int CW = LG * VEC;  // channels per chunk
  A* gl = reinterpret_cast<A*>(smem_raw);  // [S::NACC][CW]
  A* dsl = gl + S::NACC * CW;              // [64][dim_y]
  const int64_t wg = xcd_block();
  const int64_t pos = wg / a.nchunks;
  const int cc = int(wg - pos * a.nchunks);
  const int64_t n = a.order[pos];
  const BlockDev blk = ldc(a.blocks + a.block);
  const int U = blk.mul;
  int pid[NS], woff[NS], coff[NS];
  const int so = ldc(a.slot_off + a.block);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    pid[s] = ldc(a.slot_paths + so + s);
    woff[s] = pid[s] >= 0 ? ldc(&a.paths[pid[s]].w_off) : 0;
    coff[s] = pid[s] >= 0 ? ldc(&a.paths[pid[s]].coef_off) : 0;
  }
  // stage scale * grad_out[n] for this block and channel chunk
  const T* __restrict__ gn = static_cast<const T*>(bw.g) + n * a.dim_out;
  const A sc = A(a.scale);
  static_for<0, NS>([&](auto I) {
    constexpr int i = decltype(I)::value;
    constexpr SlotT st = S::arr.p[i];
    if (pid[i] >= 0) {
      const int oo = ldc(&a.paths[pid[i]].out_off);
      for (int k = threadIdx.x; k < (2 * st.l3 + 1) * CW; k += kBlock) {
        const int m = k / CW, cl = k - m * CW, c = cc * CW + cl;
        gl[(st.acc + m) * CW + cl] = c < U ? sc * to_acc<A>(gn[oo + m * U + c]) : A(0);
      }
    }
  });
  __syncthreads();
  const int NG = kBlock / LG;
  const int gi = int(threadIdx.x) / LG, li = int(threadIdx.x) - gi * LG;
  const int c = cc * CW + li * VEC;
  const bool valid = c < U;
  const A* __restrict__ cf = static_cast<const A*>(a.coef);
  const T* __restrict__ X = static_cast<const T*>(a.x);
  const int32_t e0 = a.row_ptr[n], e1 = n == a.pad ? e0 : a.row_ptr[n + 1];  // padding edges skipped
  const int lane = int(threadIdx.x & 63);
  const int cl = valid ? c : 0;  // lanes past the channels load channel 0 and use zeros
  // Source indices of up to 64 edges come with one load and are handed out by
  // lane shuffles. The trip counts are uniform over the workgroup and a
  // group's lanes share their edge (grad_sh is reduced within the group).
  // Loads of an edge do not wait on the plan's branches: x and sh at the top,
  // the weights of slot i+1 issued before slot i is computed.
  for (int32_t base = e0; base < e1; base += 64) {
    const int nb = e1 - base < 64 ? e1 - base : 64;
    const int32_t srcv = lane < nb ? a.src[base + lane] : 0;
    // grad_sh of the batch's edges: [nb][dim_y] in LDS, starting from what the
    // previous x block's launch wrote (stream order) or from zero
    if (bw.dsh) {
      const T* __restrict__ dsb = static_cast<const T*>(bw.dsh) + int64_t(base) * a.dim_y;
      for (int t = threadIdx.x; t < nb * a.dim_y; t += kBlock) dsl[t] = bw.dy_accum ? to_acc<A>(dsb[t]) : A(0);
    }
    __syncthreads();
    for (int k0 = 0; k0 < nb; k0 += NG) {
      const int kk = k0 + gi;
      const int64_t j = __shfl(srcv, kk < nb ? kk : 0, 64);
      if (kk >= nb) continue;
      const int64_t e = base + kk;
      A xb[2 * L1 + 1][VEC], dxe[2 * L1 + 1][VEC];
#pragma unroll
      for (int m = 0; m < 2 * L1 + 1; ++m) {
        VecIO<T, VEC>::load(X + j * a.dim_x + blk.x_off + m * U + cl, xb[m]);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          xb[m][v] = valid ? xb[m][v] : A(0);
          dxe[m][v] = A(0);
        }
      }
      const T* __restrict__ Ye = static_cast<const T*>(a.sh) + e * a.dim_y;
      T* __restrict__ dwe = static_cast<T*>(bw.dw) + e * a.W;
      const T* __restrict__ we = static_cast<const T*>(a.w) + e * a.W;
      A dyl[NY];
#pragma unroll
      for (int k = 0; k < NY; ++k) dyl[k] = A(0);
      A ycur[2 * L + 1];
      A wnx[VEC];
      VecIO<T, VEC>::load(we + woff[0] + cl, wnx);
      static_for<0, NS>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr SlotT st = S::arr.p[i];
        constexpr int L2 = st.l2, L3 = st.l3;
        constexpr bool first_of_l2 = (i == 0) || (S::arr.p[i > 0 ? i - 1 : 0].l2 != L2);
        if constexpr (first_of_l2) {
          const int yo = a.yoff[L2];
          const T* __restrict__ yp = yo >= 0 ? Ye + yo : static_cast<const T*>(a.coef);
#pragma unroll
          for (int m = 0; m < 2 * L2 + 1; ++m) ycur[m] = to_acc<A>(yp[m]);
        }
        A wv[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) wv[v] = valid ? wnx[v] : A(0);
        if constexpr (i + 1 < NS) VecIO<T, VEC>::load(we + woff[i + 1] + cl, wnx);
        if (pid[i] >= 0) {
          using P = Pattern<L1, L2, L3>;
          const A* __restrict__ cp = cf + coff[i];
          A gb[2 * L3 + 1][VEC];
#pragma unroll
          for (int m = 0; m < 2 * L3 + 1; ++m) VecIO<A, VEC>::load(gl + (st.acc + m) * CW + li * VEC, gb[m]);  // one VEC-wide LDS read
          // pairs are m1-major: q[m1] = sum_m3 A[m1,m3] g[m3] is folded into
          // grad_w and the grad_x partial after the last pair of its m1
          A d[VEC], q[VEC], xw[VEC];
#pragma unroll
          for (int v = 0; v < VEC; ++v) d[v] = A(0);
          static_for<0, P::NP>([&](auto K) {
            constexpr int kp = decltype(K)::value;
            constexpr PairT pr = P::arr.p[kp];
            constexpr bool first = kp == 0 || P::arr.p[kp > 0 ? kp - 1 : 0].m1 != pr.m1;
            constexpr bool last = kp == P::NP - 1 || P::arr.p[kp + 1 < P::NP ? kp + 1 : kp].m1 != pr.m1;
            if constexpr (first) {
#pragma unroll
              for (int v = 0; v < VEC; ++v) {
                xw[v] = xb[pr.m1 + L1][v] * wv[v];
                q[v] = A(0);
              }
            }
            const A ca = ldc(cp + pr.coef);
            A av = ca * ycur[pr.m2a + L2];
            A cb = A(0);
            if constexpr (pr.n == 2) {
              cb = ldc(cp + pr.coef + 1);
              av = fma(cb, ycur[pr.m2b + L2], av);
            }
            A sdot = A(0);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              q[v] = fma(av, gb[pr.m3 + L3][v], q[v]);
              sdot = fma(xw[v], gb[pr.m3 + L3][v], sdot);
            }
            dyl[L2 * L2 + L2 + pr.m2a] = fma(ca, sdot, dyl[L2 * L2 + L2 + pr.m2a]);
            if constexpr (pr.n == 2) dyl[L2 * L2 + L2 + pr.m2b] = fma(cb, sdot, dyl[L2 * L2 + L2 + pr.m2b]);
            if constexpr (last) {
#pragma unroll
              for (int v = 0; v < VEC; ++v) {
                d[v] = fma(xb[pr.m1 + L1][v], q[v], d[v]);
                dxe[pr.m1 + L1][v] = fma(wv[v], q[v], dxe[pr.m1 + L1][v]);
              }
            }
          });
          if (valid && bw.dw) VecIO<T, VEC>::store(dwe + woff[i] + c, d);
        }
      });
      if (valid && bw.dxp) {
        A* __restrict__ dxr = static_cast<A*>(bw.dxp) + e * a.dim_x + blk.x_off;
#pragma unroll
        for (int m = 0; m < 2 * L1 + 1; ++m) VecIO<A, VEC>::store(dxr + m * U + c, dxe[m]);
      }
      // grad_sh: sum over the group's channels into the batch tile
      if (!bw.dsh) continue;
      xor_sum_n<NY>(dyl, 1, LG);
      if (li == 0) {
        static_for<0, L + 1>([&](auto L2c) {
          constexpr int L2 = decltype(L2c)::value;
          const int yo = a.yoff[L2];
          if (yo >= 0) {
#pragma unroll
            for (int m = 0; m < 2 * L2 + 1; ++m) dsl[kk * a.dim_y + yo + m] += dyl[L2 * L2 + m];
          }
        });
      }
    }
    // the batch's grad_sh rows leave in one coalesced pass
    __syncthreads();
    if (bw.dsh && bw.dsh_acc) {
      A* __restrict__ dsb = static_cast<A*>(bw.dsh) + int64_t(base) * a.dim_y;
      for (int t = threadIdx.x; t < nb * a.dim_y; t += kBlock) dsb[t] = dsl[t];
    } else if (bw.dsh) {
      T* __restrict__ dsb = static_cast<T*>(bw.dsh) + int64_t(base) * a.dim_y;
      for (int t = threadIdx.x; t < nb * a.dim_y; t += kBlock) from_acc(dsb[t], dsl[t]);
    }
    __syncthreads();  // the tile is refilled by the next batch
  }
}

template <typename T>
size_t conv_bwd_fused_lds(int l1, int L, int cw) {
  using A = typename AccOf<T>::type;
  size_t r = 0;
  static_for<0, kLmax + 1>([&](auto I) {
    static_for<0, kLmax + 1>([&](auto J) {
      constexpr int D = decltype(I)::value, M = decltype(J)::value;
      if constexpr (Slots<D, M>::NS > 0) {
        if (l1 == D && L == M) r = size_t(Slots<D, M>::NACC) * size_t(cw) * sizeof(A);
      }
    });
  });
  return r;
}

template <typename T>
void conv_bwd_fused_typed(const ConvArgs& a, const ConvBwdArgs& b, int l1, int L, dim3 grid, size_t lds,
                          hipStream_t s) {
  using A = typename AccOf<T>::type;
  constexpr int VEC = std::is_same<T, double>::value ? 2 : CGTP_CONV_BWD_VEC;
  static_for<0, kLmax + 1>([&](auto I) {
    static_for<0, kLmax + 1>([&](auto J) {
      constexpr int D = decltype(I)::value, M = decltype(J)::value;
      if constexpr (Slots<D, M>::NS > 0) {
        if (l1 == D && L == M)
          hipLaunchKernelGGL((conv_bwd_fused_kernel<T, A, VEC, D, M>), grid, dim3(kBlock), lds, s, a, b);
      }
    });
  });
}

// ------------------------------------------------------------ typed launchers
// One translation unit per (kind, storage type): inst/conv_*.hip.
constexpr int conv_vec(cgtp_dtype d) { return d == CGTP_F64 ? 2 : 4; }

// Waves per receiver for the fused forward of x degree l1 and largest degree L.
template <typename T>
int conv_fused_chunks(int l1, int L, bool col) {
  using A = typename AccOf<T>::type;
  constexpr int VEC = std::is_same<T, double>::value ? 2 : 4;
  int n = 0;
  static_for<0, kLmax + 1>([&](auto I) {
    static_for<0, kLmax + 1>([&](auto J) {
      constexpr int D = decltype(I)::value, M = decltype(J)::value;
      if constexpr (Slots<D, M>::NS > 0) {
        if (l1 == D && L == M)
          n = col ? Chunks<SlotsC<D, M>, conv_budget<A, VEC>()>::NCH : Chunks<Slots<D, M>, conv_budget<A, VEC>()>::NCH;
      }
    });
  });
  return n;
}

template <typename T>
void conv_fwd_fused_typed(const ConvArgs& a, int l1, int L, dim3 grid, hipStream_t s) {
  using A = typename AccOf<T>::type;
  constexpr int VEC = std::is_same<T, double>::value ? 2 : 4;
  static_for<0, kLmax + 1>([&](auto I) {
    static_for<0, kLmax + 1>([&](auto J) {
      constexpr int D = decltype(I)::value, M = decltype(J)::value;
      if constexpr (Slots<D, M>::NS > 0) {
        if (l1 == D && L == M) {
          if (a.collapse)
            hipLaunchKernelGGL((conv_fwd_fused_kernel<T, A, VEC, D, M, true>), grid, dim3(kBlock), 0, s, a);
          else
            hipLaunchKernelGGL((conv_fwd_fused_kernel<T, A, VEC, D, M, false>), grid, dim3(kBlock), 0, s, a);
        }
      }
    });
  });
}
template <typename T>
void conv_fwd_general_typed(const ConvArgs& a, dim3 grid, hipStream_t s) {
  using A = typename AccOf<T>::type;
  hipLaunchKernelGGL((conv_fwd_general_kernel<T, A>), grid, dim3(kBlock), 0, s, a);
}

#define CGTP_CONV_EXTERN(T)                                                                   \
  extern template void conv_fwd_fused_typed<T>(const ConvArgs&, int, int, dim3, hipStream_t); \
  extern template void conv_fwd_general_typed<T>(const ConvArgs&, dim3, hipStream_t);         \
  extern template int conv_fused_chunks<T>(int, int, bool);                                  \
  extern template void conv_bwd_fused_typed<T>(const ConvArgs&, const ConvBwdArgs&, int, int, dim3, size_t, \
                                               hipStream_t);                                   \
  extern template size_t conv_bwd_fused_lds<T>(int, int, int);

}  // namespace cgtp
