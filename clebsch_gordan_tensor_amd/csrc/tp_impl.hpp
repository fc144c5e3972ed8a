// Row-parallel uvu Clebsch-Gordan tensor product, forward and backward.
//
// What is computed: the full CG tensor product x (x)_w y of "E3J: An Efficient
// and Open-Source Backend for Euclidean Equivariant Operations on GPU and TPU",
// section 3.1.1 (memory-bound; not a compute bottleneck for L <= 3), with the
// uvu connection mode of the MolSSI e3nn course, lesson 03b, and the reverse
// rules of E3J appendix E.1 (transposition of the bilinear map).
//
// Mapping on gfx950 (64-wide waves): a row is owned by a power-of-two group of
// lanes; each lane owns VEC consecutive channels (16-byte loads/stores), so
// every load/store instruction of a row moves one contiguous channel run.
// The CG tables follow a compile-time sparsity pattern per (l1, l2, l3) and
// are read with uniform (scalar) loads; per path the lane first forms
// A[m1, m3] = sum_m2 C y[m2] for its row, then applies A to its channels
// (the channel-parallel, feature-sequential order of E3J E.2.1, with the
// coefficient cost amortised over VEC channels). Nothing is reduced across
// lanes in the forward pass; the backward pass reduces grad_y across the
// row's lanes with shuffles, and grad_w of shared weights in a fixed
// two-stage order (no atomics anywhere).
#pragma once

#include "cg_pattern.h"
#include "common.hpp"
#include "device_util.hpp"
#include "tp_core.hpp"

// Tuning knobs (compile-time): minimum waves per SIMD requested from the
// register allocator, and non-temporal stores for the streamed outputs.
#ifndef CGTP_TP_FWD_WAVES
#define CGTP_TP_FWD_WAVES 0
#endif
#ifndef CGTP_TP_BWD_WAVES
#define CGTP_TP_BWD_WAVES 3
#endif
#ifndef CGTP_NT_STORE
#define CGTP_NT_STORE 0
#endif
// Backward grad_x accumulators of the degree-specialised kernels in the
// lane's own LDS slots (1) instead of registers (0). With them out of the
// register file, the degree-specialised kernels with 4- and 2-byte storage
// and largest degree <= 3 ask the allocator for CGTP_TP_BWD_WAVES waves per
// SIMD (tp_large fp32 backward 27.7 -> 25.6 ms, bf16 23.2 -> 20.0 ms against
// registers and no request); the others make no request.
// The one-launch backward with 2-byte storage asks for 3 waves per SIMD when
// its x degrees are bounded by the largest y/output degree (code for x
// degree 4 left out at LM = 3: 224 -> 194 VGPRs at 2 waves, 168 with 26
// spilled at 3 waves; tp_large bf16 17.8 -> 15.9 ms); compiled for every x
// degree it keeps 2 waves (3 waves spilled 47 VGPRs and were no faster).
#ifndef CGTP_TP_BWD_WAVES_BF16_ALL
#define CGTP_TP_BWD_WAVES_BF16_ALL 3
#endif
#ifndef CGTP_TP_BWD_DX_LDS
#define CGTP_TP_BWD_DX_LDS 1
#endif
#if CGTP_TP_FWD_WAVES > 0
#define CGTP_FWD_OCC __attribute__((amdgpu_waves_per_eu(CGTP_TP_FWD_WAVES)))
#else
#define CGTP_FWD_OCC
#endif


namespace cgtp {

struct TPArgs {
  const PathDev* paths;
  const BlockDev* blocks;
  const void* coef;
  const void* x;
  const void* y;
  const void* w;
  const void* g;
  void* out;
  void* dx;
  void* dy;
  void* dw;     // per-row grad_w, storage type (PER_ROW plans)
  void* dw_ws;  // per-row grad_w partials, accumulation type (SHARED plans)
  void* dx_ws;  // per-row grad_x in the accumulation type (edge partials of the convolution)
  const int32_t* x_idx;  // optional: x row of each row (gather)
  const int32_t* g_idx;  // optional: grad_out row of each row (gather)
  double g_scale;        // grad_out multiplier (1 for the plain tensor product)
  int64_t B;
  int64_t w_stride;  // elements between weight rows; 0 for shared weights
  int dim_x, dim_y, dim_out, W;
  int nblocks;
  int lpr_log2;  // lanes per row = 1 << lpr_log2
  int ngroups;   // channel groups per row = ceil(max_mul / VEC)
  int block;     // x block of a degree-specialised launch
  int max_l1;    // largest x degree of the plan (LDS rows of the all-blocks backward)
  int dy_accum;  // add grad_y to what an earlier launch on the stream wrote
  // collapsed outputs: the output parity this launch writes and, per parity
  // (index 0: even, 1: odd) and degree l3, the block offset (-1 if absent)
  // and multiplicity
  int par;
  int32_t goff[2][kLmax + 1];
  int32_t gmul[2][kLmax + 1];
};

// LM: largest l2 and l3 compiled into a kernel (the plan's largest y or
// output degree); L1 is fixed per kernel, so each kernel only holds the paths
// one x block can take, which keeps registers and code size small.
template <typename T, typename A, int VEC, int LM>
struct TPFwd {
  template <int L1, int L2, int L3>
  __device__ static __forceinline__ void path(const TPArgs& a, const PathDev& pd,
                                              const A (&xb)[2 * L1 + 1][VEC],
                                              const A (&yb)[2 * L2 + 1], const T* wr, T* outr,
                                              int c) {
    A o[2 * L3 + 1][VEC];
    fwd_core<L1, L2, L3, VEC, A>(xb, yb, static_cast<const A*>(a.coef) + pd.coef_off, o);
    A wv[VEC];
    VecIO<T, VEC>::load(wr + pd.w_off + c, wv);
#pragma unroll
    for (int m = 0; m < 2 * L3 + 1; ++m) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[m][v] *= wv[v];
      if constexpr (CGTP_NT_STORE != 0)
        VecIO<T, VEC>::store_nt(outr + pd.out_off + m * pd.mul + c, o[m]);
      else
        VecIO<T, VEC>::store(outr + pd.out_off + m * pd.mul + c, o[m]);
    }
  }

  template <int L1, int L2>
  __device__ static __forceinline__ void run(const TPArgs& a, int p, int pend,
                                             const A (&xb)[2 * L1 + 1][VEC], const T* yr,
                                             const T* wr, T* outr, int c) {
    A yb[2 * L2 + 1];
    const int yoff = ldc(&a.paths[p].y_off);
#pragma unroll
    for (int m = 0; m < 2 * L2 + 1; ++m) yb[m] = to_acc<A>(yr[yoff + m]);
    for (int q = p; q < pend; ++q) {
      const PathDev pd = ldc(a.paths + q);
      static_for<0, LM + 1>([&](auto L3c) {
        constexpr int L3 = decltype(L3c)::value;
        if constexpr (L3 >= (L1 > L2 ? L1 - L2 : L2 - L1) && L3 <= L1 + L2) {
          if (pd.l3 == L3) path<L1, L2, L3>(a, pd, xb, yb, wr, outr, c);
        }
      });
    }
  }

  template <int L1>
  __device__ static __forceinline__ void block(const TPArgs& a, const BlockDev& blk, const T* xr,
                                               const T* yr, const T* wr, T* outr, int c) {
    A xb[2 * L1 + 1][VEC];
#pragma unroll
    for (int m = 0; m < 2 * L1 + 1; ++m) VecIO<T, VEC>::load(xr + blk.x_off + m * blk.mul + c, xb[m]);
    int p = blk.path_begin;
    while (p < blk.path_end) {
      const int l2 = ldc(&a.paths[p].l2);
      const int pend = ldc(&a.paths[p].i2_end);
      static_for<0, LM + 1>([&](auto L2c) {
        constexpr int L2 = decltype(L2c)::value;
        if (l2 == L2) run<L1, L2>(a, p, pend, xb, yr, wr, outr, c);
      });
      p = pend;
    }
  }
};

// L1 >= 0: one x block (a.block) of degree L1; L1 < 0: every block, degree
// dispatched at run time (L1 = -1: the general kernel, LM = CGTP_LMAX;
// L1 = -2: code for x degrees up to LM only, for calls too small for the
// degree-specialised launches to pay for their launch overhead).
template <typename T, typename A, int VEC, int L1, int LM>
__global__ __launch_bounds__(kBlock) CGTP_FWD_OCC void tp_fwd_kernel(TPArgs a) {
  const int64_t gt = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t row = gt >> a.lpr_log2;
  const int lpr = 1 << a.lpr_log2;
  const int lr = int(gt & (lpr - 1));
  if (row >= a.B) return;
  const T* xr = static_cast<const T*>(a.x) + row * a.dim_x;
  const T* yr = static_cast<const T*>(a.y) + row * a.dim_y;
  const T* wr = static_cast<const T*>(a.w) + row * a.w_stride;
  T* outr = static_cast<T*>(a.out) + row * a.dim_out;
  for (int grp = lr; grp < a.ngroups; grp += lpr) {
    const int c = grp * VEC;
    if constexpr (L1 >= 0) {
      const BlockDev blk = ldc(a.blocks + a.block);
      if (c < blk.mul) TPFwd<T, A, VEC, LM>::template block<L1>(a, blk, xr, yr, wr, outr, c);
    } else {
      for (int b = 0; b < a.nblocks; ++b) {
        const BlockDev blk = ldc(a.blocks + b);
        if (c >= blk.mul) continue;
        static_for<0, (L1 == -2 ? LM : kLmax) + 1>([&](auto L1c) {
          constexpr int D = decltype(L1c)::value;
          if (blk.l1 == D) TPFwd<T, A, VEC, LM>::template block<D>(a, blk, xr, yr, wr, outr, c);
        });
      }
    }
  }
}

// ------------------------------------------------------- collapsed forward
// Outputs collapsed by (l3, p3): every path of one output type adds into one
// block, so a lane accumulates all of them in registers (acc[l3^2 + m]) over
// every x block of its row and writes each block once. A launch covers one
// output parity (the parity of a path is fixed by its (i1, i2) run), which
// halves the accumulators; x and y are read once per parity.
template <typename T, typename A, int VEC, int LM>
struct TPFwdCol {
  static constexpr int NACC = (LM + 1) * (LM + 1);

  template <int L1, int L2>
  __device__ static __forceinline__ void run(const TPArgs& a, int p, int pend, const A (&xb)[2 * L1 + 1][VEC],
                                             const T* yr, const T* wr, int c, A (&acc)[NACC][VEC]) {
    A yb[2 * L2 + 1];
    const int yoff = ldc(&a.paths[p].y_off);
#pragma unroll
    for (int m = 0; m < 2 * L2 + 1; ++m) yb[m] = to_acc<A>(yr[yoff + m]);
    // the run's paths are in ascending l3: walk the possible degrees once
    int q = p;
    static_for<0, LM + 1>([&](auto L3c) {
      constexpr int L3 = decltype(L3c)::value;
      if constexpr (L3 >= (L1 > L2 ? L1 - L2 : L2 - L1) && L3 <= L1 + L2) {
        if (q < pend && ldc(&a.paths[q].l3) == L3) {
          const int coff = ldc(&a.paths[q].coef_off), woff = ldc(&a.paths[q].w_off);
          ++q;
          A o[2 * L3 + 1][VEC];
          fwd_core<L1, L2, L3, VEC, A>(xb, yb, static_cast<const A*>(a.coef) + coff, o);
          A wv[VEC];
          VecIO<T, VEC>::load(wr + woff + c, wv);
#pragma unroll
          for (int m = 0; m < 2 * L3 + 1; ++m)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[L3 * L3 + m][v] = fma(wv[v], o[m][v], acc[L3 * L3 + m][v]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    });
  }

  template <int L1>
  __device__ static __forceinline__ void block(const TPArgs& a, const BlockDev& blk, const T* xr, const T* yr,
                                               const T* wr, int c, A (&acc)[NACC][VEC]) {
    A xb[2 * L1 + 1][VEC];
#pragma unroll
    for (int m = 0; m < 2 * L1 + 1; ++m) VecIO<T, VEC>::load(xr + blk.x_off + m * blk.mul + c, xb[m]);
    int p = blk.path_begin;
    while (p < blk.path_end) {
      const int l2 = ldc(&a.paths[p].l2);
      const int pend = ldc(&a.paths[p].i2_end);
      if (ldc(&a.paths[p].p3) == a.par) {  // one parity per (i1, i2) run
        static_for<0, LM + 1>([&](auto L2c) {
          constexpr int L2 = decltype(L2c)::value;
          if (l2 == L2) run<L1, L2>(a, p, pend, xb, yr, wr, c, acc);
        });
      }
      p = pend;
    }
  }
};

template <typename T, typename A, int VEC, int LM>
__global__ __launch_bounds__(kBlock) void tp_fwd_collapsed_kernel(TPArgs a) {
  using F = TPFwdCol<T, A, VEC, LM>;
  const int64_t gt = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t row = gt >> a.lpr_log2;
  const int lpr = 1 << a.lpr_log2;
  const int lr = int(gt & (lpr - 1));
  if (row >= a.B) return;
  const T* xr = static_cast<const T*>(a.x) + row * a.dim_x;
  const T* yr = static_cast<const T*>(a.y) + row * a.dim_y;
  const T* wr = static_cast<const T*>(a.w) + row * a.w_stride;
  T* outr = static_cast<T*>(a.out) + row * a.dim_out;
  const int pi = a.par > 0 ? 0 : 1;
  for (int grp = lr; grp < a.ngroups; grp += lpr) {
    const int c = grp * VEC;
    A acc[F::NACC][VEC];
#pragma unroll
    for (int i = 0; i < F::NACC; ++i)
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[i][v] = A(0);
    for (int b = 0; b < a.nblocks; ++b) {
      const BlockDev blk = ldc(a.blocks + b);
      if (c >= blk.mul) continue;
      static_for<0, kLmax + 1>([&](auto L1c) {
        constexpr int D = decltype(L1c)::value;
        if (blk.l1 == D) F::template block<D>(a, blk, xr, yr, wr, c, acc);
      });
    }
    // addresses formed here, after the accumulation (kept out of the loop
    // so they do not hold registers through it)
    T* ob = outr + c;
    asm volatile("" : "+v"(ob));
    static_for<0, LM + 1>([&](auto L3c) {
      constexpr int L3 = decltype(L3c)::value;
      const int off = a.goff[pi][L3], mul = a.gmul[pi][L3];
      if (off >= 0 && c < mul) {
#pragma unroll
        for (int m = 0; m < 2 * L3 + 1; ++m) VecIO<T, VEC>::store(ob + off + m * mul, acc[L3 * L3 + m]);
      }
    });
  }
}

// ------------------------------------------------------------------ backward

// N rows of VEC accumulators owned by one lane: in registers, or in the
// lane's private LDS slots (layout [row][thread][VEC], no sharing, no sync).
template <typename A, int VEC, int N, bool IN_LDS>
struct RowAcc {
  A r[N][VEC];
  __device__ __forceinline__ explicit RowAcc(A*) {
#pragma unroll
    for (int m = 0; m < N; ++m)
#pragma unroll
      for (int v = 0; v < VEC; ++v) r[m][v] = A(0);
  }
  __device__ __forceinline__ void fma_row(int m, const A (&w)[VEC], const A (&q)[VEC]) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) r[m][v] = fma(w[v], q[v], r[m][v]);
  }
  __device__ __forceinline__ void get(int m, A (&o)[VEC]) const {
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[v] = r[m][v];
  }
};
template <typename A, int VEC, int N>
struct RowAcc<A, VEC, N, true> {
  A* p;  // this lane's row 0 (16-byte aligned: the rows start at a multiple of kBlock * VEC elements)
  __device__ __forceinline__ explicit RowAcc(A* base) : p(base + threadIdx.x * VEC) {
    A z[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) z[v] = A(0);
#pragma unroll
    for (int m = 0; m < N; ++m) VecIO<A, VEC>::store(p + m * kBlock * VEC, z);
  }
  // one VEC-wide LDS access per row (lanes at consecutive VEC-element slots,
  // so a wave's access has no bank conflict)
  __device__ __forceinline__ void fma_row(int m, const A (&w)[VEC], const A (&q)[VEC]) {
    A t[VEC];
    get(m, t);
#pragma unroll
    for (int v = 0; v < VEC; ++v) t[v] = fma(w[v], q[v], t[v]);
    VecIO<A, VEC>::store(p + m * kBlock * VEC, t);
  }
  __device__ __forceinline__ void get(int m, A (&o)[VEC]) const { VecIO<A, VEC>::load(p + m * kBlock * VEC, o); }
};

template <typename T, typename A, int VEC, int LM>
struct TPBwd {
  template <int L1, int L2, int L3, typename DX>
  __device__ static __forceinline__ void path(const TPArgs& a, const PathDev& pd,
                                              const A (&xb)[2 * L1 + 1][VEC],
                                              const A (&yb)[2 * L2 + 1], const T* gr,
                                              const T* wr, T* dwr, A* dwa, int c,
                                              DX& dxb, A (&dyb)[2 * L2 + 1]) {
    using P = Pattern<L1, L2, L3>;
    const A* __restrict__ cf = static_cast<const A*>(a.coef) + pd.coef_off;
    const A gs = A(a.g_scale);
    A gb[2 * L3 + 1][VEC];
#pragma unroll
    for (int m = 0; m < 2 * L3 + 1; ++m) {
      VecIO<T, VEC>::load(gr + pd.out_off + m * pd.mul + c, gb[m]);
#pragma unroll
      for (int v = 0; v < VEC; ++v) gb[m][v] *= gs;
    }
    A wv[VEC];
    VecIO<T, VEC>::load(wr + pd.w_off + c, wv);
    // Pairs come m1-major, so q[m1] = sum_m3 A[m1,m3] g[m3] (A = C y) is
    // complete after the last pair of its m1: it is folded into dw and dx
    // there, and only one m1's q and x*w are live at a time.
    //   dy[m2] += C sum_u w x[m1] g[m3];  dw = sum_m1 x[m1] q[m1];  dx[m1] += w q[m1]
    A d[VEC], q[VEC], xw[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) d[v] = A(0);
    static_for<0, P::NP>([&](auto I) {
      constexpr int i = decltype(I)::value;
      constexpr PairT pr = P::arr.p[i];
      constexpr bool first = i == 0 || P::arr.p[i > 0 ? i - 1 : 0].m1 != pr.m1;
      constexpr bool last = i == P::NP - 1 || P::arr.p[i + 1 < P::NP ? i + 1 : i].m1 != pr.m1;
      if constexpr (first) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          xw[v] = xb[pr.m1 + L1][v] * wv[v];
          q[v] = A(0);
        }
      }
      const A ca = ldc(cf + pr.coef);
      A av = ca * yb[pr.m2a + L2];
      A cb = A(0);
      if constexpr (pr.n == 2) {
        cb = ldc(cf + pr.coef + 1);
        av = fma(cb, yb[pr.m2b + L2], av);
      }
      A s = A(0);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        q[v] = fma(av, gb[pr.m3 + L3][v], q[v]);
        s = fma(xw[v], gb[pr.m3 + L3][v], s);
      }
      dyb[pr.m2a + L2] = fma(ca, s, dyb[pr.m2a + L2]);
      if constexpr (pr.n == 2) dyb[pr.m2b + L2] = fma(cb, s, dyb[pr.m2b + L2]);
      if constexpr (last) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) d[v] = fma(xb[pr.m1 + L1][v], q[v], d[v]);
        dxb.fma_row(pr.m1 + L1, wv, q);
      }
    });
    if (dwr) VecIO<T, VEC>::store(dwr + pd.w_off + c, d);
    if (dwa) VecIO<A, VEC>::store(dwa + pd.w_off + c, d);
  }

  template <int L1, int L2, typename DX>
  __device__ static __forceinline__ void run(const TPArgs& a, int p, int pend,
                                             const A (&xb)[2 * L1 + 1][VEC], const T* yr,
                                             const T* gr, const T* wr, T* dwr, A* dwa, int c,
                                             DX& dxb, A* lds) {
    A yb[2 * L2 + 1], dyb[2 * L2 + 1];
    const int yoff = ldc(&a.paths[p].y_off);
#pragma unroll
    for (int m = 0; m < 2 * L2 + 1; ++m) {
      yb[m] = to_acc<A>(yr[yoff + m]);
      dyb[m] = A(0);
    }
    for (int q = p; q < pend; ++q) {
      const PathDev pd = ldc(a.paths + q);
      static_for<0, LM + 1>([&](auto L3c) {
        constexpr int L3 = decltype(L3c)::value;
        if constexpr (L3 >= (L1 > L2 ? L1 - L2 : L2 - L1) && L3 <= L1 + L2) {
          if (pd.l3 == L3) path<L1, L2, L3>(a, pd, xb, yb, gr, wr, dwr, dwa, c, dxb, dyb);
        }
      });
    }
    // this lane's grad_y partial lives in its own LDS column (no sharing)
#pragma unroll
    for (int m = 0; m < 2 * L2 + 1; ++m) lds[(yoff + m) * kBlock + threadIdx.x] += dyb[m];
  }

  // dx_lds: grad_x rows in this lane's LDS slots after the grad_y columns
  template <int L1, bool DX_LDS>
  __device__ static __forceinline__ void block(const TPArgs& a, const BlockDev& blk, const T* xr,
                                               const T* yr, const T* gr, const T* wr, T* dxr,
                                               A* dxa, T* dwr, A* dwa, int c, A* lds) {
    A xb[2 * L1 + 1][VEC];
#pragma unroll
    for (int m = 0; m < 2 * L1 + 1; ++m) VecIO<T, VEC>::load(xr + blk.x_off + m * blk.mul + c, xb[m]);
    RowAcc<A, VEC, 2 * L1 + 1, DX_LDS> dxb(lds + a.dim_y * kBlock);
    int p = blk.path_begin;
    while (p < blk.path_end) {
      const int l2 = ldc(&a.paths[p].l2);
      const int pend = ldc(&a.paths[p].i2_end);
      static_for<0, LM + 1>([&](auto L2c) {
        constexpr int L2 = decltype(L2c)::value;
        if (l2 == L2) run<L1, L2>(a, p, pend, xb, yr, gr, wr, dwr, dwa, c, dxb, lds);
      });
      p = pend;
    }
#pragma unroll
    for (int m = 0; m < 2 * L1 + 1; ++m) {
      A o[VEC];
      dxb.get(m, o);
      if (dxr) VecIO<T, VEC>::store(dxr + blk.x_off + m * blk.mul + c, o);
      if (dxa) VecIO<A, VEC>::store(dxa + blk.x_off + m * blk.mul + c, o);
    }
  }
};

// (requested only where the spill it costs stays small: largest degree <= 3)
template <typename T, int L1, int LM, int MX>
struct BwdWaves {
  static constexpr int waves =
      sizeof(T) == 2 && L1 == -2 ? (MX <= LM ? CGTP_TP_BWD_WAVES_BF16_ALL : 2) : CGTP_TP_BWD_WAVES;
  static constexpr int value = ((L1 >= 0 || L1 == -2) && LM <= 3 && sizeof(T) <= 4 && waves > 1) ? waves : 1;
};

// MX: largest x degree the one-launch kernels (L1 < 0) hold code for.
template <typename T, typename A, int VEC, int L1, int LM, int MX = kLmax>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(BwdWaves<T, L1, LM, MX>::value)))
void tp_bwd_kernel(TPArgs a) {
  extern __shared__ unsigned char smem_raw[];
  A* lds = reinterpret_cast<A*>(smem_raw);  // [dim_y][kBlock], one column per lane
  const int64_t gt = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t row = gt >> a.lpr_log2;
  const int lpr = 1 << a.lpr_log2;
  const int lr = int(gt & (lpr - 1));
  const bool active = row < a.B;
  for (int k = 0; k < a.dim_y; ++k) lds[k * kBlock + threadIdx.x] = A(0);
  if (active) {
    const int64_t xrow = a.x_idx ? int64_t(a.x_idx[row]) : row;
    const int64_t grow = a.g_idx ? int64_t(a.g_idx[row]) : row;
    const T* xr = static_cast<const T*>(a.x) + xrow * a.dim_x;
    const T* yr = static_cast<const T*>(a.y) + row * a.dim_y;
    const T* gr = static_cast<const T*>(a.g) + grow * a.dim_out;
    const T* wr = static_cast<const T*>(a.w) + row * a.w_stride;
    T* dxr = a.dx ? static_cast<T*>(a.dx) + row * a.dim_x : nullptr;
    A* dxa = a.dx_ws ? static_cast<A*>(a.dx_ws) + row * a.dim_x : nullptr;
    T* dwr = a.dw ? static_cast<T*>(a.dw) + row * a.W : nullptr;
    A* dwa = a.dw_ws ? static_cast<A*>(a.dw_ws) + row * a.W : nullptr;
    for (int grp = lr; grp < a.ngroups; grp += lpr) {
      const int c = grp * VEC;
      if constexpr (L1 >= 0) {
        const BlockDev blk = ldc(a.blocks + a.block);
        if (c < blk.mul)
          TPBwd<T, A, VEC, LM>::template block<L1, CGTP_TP_BWD_DX_LDS != 0>(a, blk, xr, yr, gr, wr, dxr, dxa,
                                                                           dwr, dwa, c, lds);
      } else {
        // every x block in one launch (L1 = -1: grad_x rows in registers;
        // L1 = -2: in LDS, for collapsed outputs, whose x blocks share their
        // cotangent blocks and so read them while they are still in cache)
        for (int b = 0; b < a.nblocks; ++b) {
          const BlockDev blk = ldc(a.blocks + b);
          if (c >= blk.mul) continue;
          static_for<0, MX + 1>([&](auto L1c) {
            constexpr int D = decltype(L1c)::value;
            if (blk.l1 == D)
              TPBwd<T, A, VEC, LM>::template block<D, L1 == -2 && CGTP_TP_BWD_DX_LDS != 0>(
                  a, blk, xr, yr, gr, wr, dxr, dxa, dwr, dwa, c, lds);
          });
        }
      }
    }
  }
  // grad_y: sum the row's lanes; lane k % lpr writes component k (adding to
  // what the previous x block's launch wrote, in stream order)
  T* dyr = (a.dy && active) ? static_cast<T*>(a.dy) + row * a.dim_y : nullptr;
  constexpr int NYB = 8;  // components reduced together
  for (int k0 = 0; k0 < a.dim_y; k0 += NYB) {
    A v[NYB];
#pragma unroll
    for (int k = 0; k < NYB; ++k) v[k] = k0 + k < a.dim_y ? lds[(k0 + k) * kBlock + threadIdx.x] : A(0);
    xor_sum_n<NYB>(v, 1, lpr);
#pragma unroll
    for (int k = 0; k < NYB; ++k) {
      const int kk = k0 + k;
      if (kk < a.dim_y && dyr && lr == (kk & (lpr - 1))) {
        A o = v[k];
        if (a.dy_accum) o += to_acc<A>(dyr[kk]);
        from_acc(dyr[kk], o);
      }
    }
  }
}

// Shared weights: grad_w[j] = sum over rows of the per-row partials, in a
// fixed order: contiguous chunks of kRowsPerChunk rows, then over chunks.
constexpr int kRowsPerChunk = 256;

template <typename A>
__global__ __launch_bounds__(kBlock) void colsum_stage1(const A* __restrict__ in, A* __restrict__ part,
                                                        int64_t rows, int W) {
  const int col = blockIdx.x * kBlock + threadIdx.x;
  const int64_t r0 = int64_t(blockIdx.y) * kRowsPerChunk;
  if (col >= W) return;
  const int64_t r1 = r0 + kRowsPerChunk < rows ? r0 + kRowsPerChunk : rows;
  A s = A(0);
  for (int64_t r = r0; r < r1; ++r) s += in[r * W + col];
  part[int64_t(blockIdx.y) * W + col] = s;
}

template <typename T, typename A>
__global__ __launch_bounds__(kBlock) void colsum_stage2(const A* __restrict__ part, T* __restrict__ out,
                                                        int nchunks, int W) {
  const int col = blockIdx.x * kBlock + threadIdx.x;
  if (col >= W) return;
  A s = A(0);
  for (int k = 0; k < nchunks; ++k) s += part[int64_t(k) * W + col];
  from_acc(out[col], s);
}

// ------------------------------------------------------------ typed launchers
// Each (storage type, VEC) pair is instantiated in its own translation unit
// (inst/*.hip) so the large unrolled kernels compile in parallel.

inline dim3 grid_for(int64_t B, int lpr_log2) {
  const int64_t rows_per_block = kBlock >> lpr_log2;
  return dim3(unsigned((B + rows_per_block - 1) / rows_per_block));
}

// l1 < 0 (and every VEC = 1 build): the general kernel over all x blocks;
// otherwise the kernel specialised for x degree l1 and largest degree lm.
template <typename T, int VEC>
void tp_fwd_typed(const TPArgs& a, int l1, int lm, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const dim3 grid = grid_for(a.B, a.lpr_log2);
  if constexpr (VEC == 1) {
    (void)l1;
    (void)lm;
    hipLaunchKernelGGL((tp_fwd_kernel<T, A, VEC, -1, kLmax>), grid, dim3(kBlock), 0, s, a);
  } else {
    if (l1 == -2) {
      static_for<0, kLmax + 1>([&](auto J) {
        constexpr int M = decltype(J)::value;
        if (lm == M) hipLaunchKernelGGL((tp_fwd_kernel<T, A, VEC, -2, M>), grid, dim3(kBlock), 0, s, a);
      });
      return;
    }
    if (l1 < 0) {
      hipLaunchKernelGGL((tp_fwd_kernel<T, A, VEC, -1, kLmax>), grid, dim3(kBlock), 0, s, a);
      return;
    }
    static_for<0, kLmax + 1>([&](auto I) {
      static_for<0, kLmax + 1>([&](auto J) {
        constexpr int D = decltype(I)::value, M = decltype(J)::value;
        if (l1 == D && lm == M)
          hipLaunchKernelGGL((tp_fwd_kernel<T, A, VEC, D, M>), grid, dim3(kBlock), 0, s, a);
      });
    });
  }
}

// Dynamic LDS of tp_bwd_kernel: grad_y columns [dim_y][kBlock] and, for the
// degree-specialised (l1 >= 0) and all-blocks (l1 = -2) kernels with grad_x in
// LDS, 2 l1 + 1 (all blocks: 2 max_l1 + 1) rows of VEC accumulators per lane.
inline size_t tp_bwd_lds_bytes(int dim_y, int l1, int max_l1, int vec, size_t acc) {
  const size_t dx_rows =
      !CGTP_TP_BWD_DX_LDS || vec == 1 ? 0 : (l1 >= 0 ? 2 * l1 + 1 : l1 == -2 ? 2 * max_l1 + 1 : 0);
  return size_t(dim_y) * kBlock * acc + dx_rows * kBlock * size_t(vec) * acc;
}

template <typename T, int VEC>
void tp_bwd_typed(const TPArgs& a, int l1, int lm, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const dim3 grid = grid_for(a.B, a.lpr_log2);
  const size_t lds = tp_bwd_lds_bytes(a.dim_y, l1, a.max_l1, VEC, sizeof(A));
  if constexpr (VEC == 1) {
    (void)l1;
    (void)lm;
    hipLaunchKernelGGL((tp_bwd_kernel<T, A, VEC, -1, kLmax>), grid, dim3(kBlock), lds, s, a);
  } else {
    if (l1 == -1) {
      hipLaunchKernelGGL((tp_bwd_kernel<T, A, VEC, -1, kLmax>), grid, dim3(kBlock), lds, s, a);
      return;
    }
    if (l1 == -2) {
      // code for x degrees up to lm only, when no x block goes beyond it
      static_for<0, kLmax + 1>([&](auto J) {
        constexpr int M = decltype(J)::value;
        if (lm == M) {
          if (a.max_l1 <= M)
            hipLaunchKernelGGL((tp_bwd_kernel<T, A, VEC, -2, M, M>), grid, dim3(kBlock), lds, s, a);
          else
            hipLaunchKernelGGL((tp_bwd_kernel<T, A, VEC, -2, M, kLmax>), grid, dim3(kBlock), lds, s, a);
        }
      });
      return;
    }
    static_for<0, kLmax + 1>([&](auto I) {
      static_for<0, kLmax + 1>([&](auto J) {
        constexpr int D = decltype(I)::value, M = decltype(J)::value;
        if (l1 == D && lm == M)
          hipLaunchKernelGGL((tp_bwd_kernel<T, A, VEC, D, M>), grid, dim3(kBlock), lds, s, a);
      });
    });
  }
}

template <typename T, int VEC>
void tp_fwd_collapsed_typed(const TPArgs& a, int lm, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const dim3 grid = grid_for(a.B, a.lpr_log2);
  static_for<0, kLmax + 1>([&](auto J) {
    constexpr int M = decltype(J)::value;
    if (lm == M) hipLaunchKernelGGL((tp_fwd_collapsed_kernel<T, A, VEC, M>), grid, dim3(kBlock), 0, s, a);
  });
}

#define CGTP_TP_EXTERN_FWD(T, V) extern template void tp_fwd_typed<T, V>(const TPArgs&, int, int, hipStream_t);
#define CGTP_TP_EXTERN_FWDC(T, V) extern template void tp_fwd_collapsed_typed<T, V>(const TPArgs&, int, hipStream_t);
#define CGTP_TP_EXTERN_BWD(T, V) extern template void tp_bwd_typed<T, V>(const TPArgs&, int, int, hipStream_t);

}  // namespace cgtp
