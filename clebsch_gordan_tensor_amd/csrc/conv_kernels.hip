// Launchers of the message-passing convolution (kernels in conv_impl.hpp).
#include <algorithm>
#include <vector>

#include "conv_impl.hpp"

namespace cgtp {

CGTP_CONV_EXTERN(float)
CGTP_CONV_EXTERN(double)
CGTP_CONV_EXTERN(bf16)

namespace {

// ------------------------------------------------------- backward helpers
// grad_x[n] = sum of the per-edge partials of n's outgoing edges, in
// CSR-position order (the transpose). One wave = (node, run of 64*V
// channels), V channels per lane; the partial rows of eight edges are loaded
// before they are added, still in that order.
template <typename T, typename A, int V>
__global__ __launch_bounds__(kBlock) void dx_gather_kernel(const int32_t* __restrict__ col_ptr,
                                                           const int32_t* __restrict__ eid,
                                                           const A* __restrict__ part, T* __restrict__ dx,
                                                           int64_t N, int dim_x, int nchunk) {
  const int64_t item = int64_t(blockIdx.x) * kWaves + conv_wave_id();
  const int64_t n = item / nchunk;
  if (n >= N) return;
  const int k = (int(item - n * nchunk) * 64 + int(threadIdx.x & 63)) * V;
  if (k >= dim_x) return;
  const int32_t t0 = col_ptr[n], t1 = col_ptr[n + 1];
  A s[V];
#pragma unroll
  for (int v = 0; v < V; ++v) s[v] = A(0);
  constexpr int U = 8;
  int32_t t = t0;
  for (; t + U <= t1; t += U) {
    A r[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) VecIO<A, V>::load(part + int64_t(eid[t + u]) * dim_x + k, r[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v) s[v] += r[u][v];
  }
  for (; t < t1; ++t) {
    A r[V];
    VecIO<A, V>::load(part + int64_t(eid[t]) * dim_x + k, r);
#pragma unroll
    for (int v = 0; v < V; ++v) s[v] += r[v];
  }
  VecIO<T, V>::store(dx + n * dim_x + k, s);
}

// grad_sh[i] = sum over x blocks k = 0, 1, ... of part[k][i], added in that
// order (the order in which the x-block launches would accumulate it in place).
template <typename T, typename A>
__global__ __launch_bounds__(kBlock) void dsh_sum_kernel(const A* __restrict__ part, T* __restrict__ dsh, int64_t n,
                                                         int nb) {
  const int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= n) return;
  A v = part[i];
  for (int k = 1; k < nb; ++k) v += part[int64_t(k) * n + i];
  from_acc(dsh[i], v);
}

template <typename T>
void dsh_sum(const void* part, void* dsh, int64_t n, int nb, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const unsigned grid = unsigned((n + kBlock - 1) / kBlock);
  hipLaunchKernelGGL((dsh_sum_kernel<T, A>), dim3(grid), dim3(kBlock), 0, s, static_cast<const A*>(part),
                     static_cast<T*>(dsh), n, nb);
  CGTP_CHECK_HIP(hipGetLastError());
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

ConvArgs make_conv_args(cgtp_plan_s* plan, const DevTables& t, const cgtp_graph_s* g) {
  ConvArgs a{};
  a.paths = t.paths;
  a.blocks = t.blocks;
  a.coef = t.coef;
  a.slot_paths = t.slot_paths;
  a.slot_off = t.slot_off;
  a.row_ptr = g->row_ptr;
  a.src = g->src;
  a.order = g->order;
  a.N = g->N;
  a.dim_x = int(plan->dim_x);
  a.dim_y = int(plan->dim_y);
  a.dim_out = int(plan->dim_out);
  a.W = int(plan->w_numel);
  a.nblocks = int(plan->blocks.size());
  a.npaths = int(plan->paths.size());
  a.nchunks = (plan->max_mul + 63) / 64;
  a.L = plan->conv_L;
  a.coef_zero = int(plan->coef64.size());
  a.pad = g->pad;
  for (int l = 0; l <= kLmax; ++l) a.yoff[l] = plan->yoff_by_l[l];
  return a;
}

bool aligned_to(const void* p, size_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

// out[i] = acc[i] rounded to the storage type (one rounding of the running sum).
template <typename T, typename A>
__global__ __launch_bounds__(kBlock) void acc_store_kernel(const A* __restrict__ acc, T* __restrict__ out, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (i < n) from_acc(out[i], acc[i]);
}

template <typename T>
void fwd_launches(cgtp_plan_s* plan, ConvArgs a, bool big, hipStream_t s);

// Edge-tensor bytes of one call (weights and harmonics): calls below
// kSideMinBytes keep their x-block launches on the caller's stream.
double conv_edge_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g) {
  return double(g->E) * double(plan->w_numel + plan->dim_y) * double(dtype_size(plan->dtype));
}

template <typename T>
void fwd_typed(cgtp_plan_s* plan, ConvArgs a, void* acc_ws, bool big, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const int64_t nout = a.N * int64_t(a.dim_out);
  if (plan->collapse) {  // the kernels add into the output, or into an accumulation-type running sum
    a.collapse = 1;
    a.acc = acc_ws;
    if (a.acc)
      zero_rows(a.acc, nout, sizeof(A), s);
    else
      zero_rows(a.out, nout, dtype_size(plan->dtype), s);
  }
  fwd_launches<T>(plan, a, big, s);
  if (a.acc && nout > 0) {  // the running sum leaves rounded once, after every x block added into it
    hipLaunchKernelGGL((acc_store_kernel<T, A>), dim3(unsigned((nout + kBlock - 1) / kBlock)), dim3(kBlock), 0, s,
                       static_cast<const A*>(a.acc), static_cast<T*>(a.out), nout);
    CGTP_CHECK_HIP(hipGetLastError());
  }
}

template <typename T>
void fwd_launches(cgtp_plan_s* plan, ConvArgs a, bool big, hipStream_t s) {
  const size_t vb = size_t(conv_vec(plan->dtype)) * dtype_size(plan->dtype);
  const bool fused = plan->conv_fused && (!plan->collapse || plan->conv_col_fused) &&
                     plan->vec == conv_vec(plan->dtype) && aligned_to(a.x, vb) && aligned_to(a.w, vb) &&
                     aligned_to(a.out, vb);
  if (!fused) {
    const int64_t items = a.N * int64_t(a.collapse ? 1 : a.npaths) * a.nchunks;
    conv_fwd_general_typed<T>(a, dim3(unsigned((items + kWaves - 1) / kWaves)), s);
    CGTP_CHECK_HIP(hipGetLastError());
    return;
  }
  // One launch per x block, specialised for its degree and the plan's largest
  // degree. Without collapse the blocks write disjoint output columns, so
  // their launches run side by side (the memory-bound small degrees beside the
  // ALU-bound large ones), the largest degree first; collapsed blocks add into
  // shared output blocks in block order on s.
  const int VEC = conv_vec(plan->dtype);
  const int nb = int(plan->blocks.size());
  std::vector<int> order(nb);
  for (int b = 0; b < nb; ++b) order[b] = b;
  if (!a.collapse)
    std::stable_sort(order.begin(), order.end(),
                     [&](int i, int j) { return plan->blocks[i].l1 > plan->blocks[j].l1; });
  auto launch = [&](int i, hipStream_t st) {
    const int b = order[i];
    const BlockInfo& blk = plan->blocks[b];
    const int lanes = (blk.mul + VEC - 1) / VEC;
    int lg = 0;
    while ((1 << lg) < lanes && lg < 6) ++lg;
    ConvArgs ab = a;
    ab.block = b;
    ab.lg_log2 = lg;
    ab.nchunks = (lanes + (1 << lg) - 1) >> lg;
    const int nch = conv_fused_chunks<T>(blk.l1, plan->conv_L, ab.collapse != 0);
    const int64_t items = ab.N * int64_t(nch) * ab.nchunks;
    conv_fwd_fused_typed<T>(ab, blk.l1, plan->conv_L, dim3(unsigned((items + kWaves - 1) / kWaves)), st);
    CGTP_CHECK_HIP(hipGetLastError());
  };
  if (a.collapse)
    for (int i = 0; i < nb; ++i) launch(i, s);
  else
    side_run(s, nb, launch, big);
}

template <typename T>
void dx_gather(const cgtp_graph_s* g, const void* part, void* dx, int dim_x, hipStream_t s) {
  using A = typename AccOf<T>::type;
  constexpr int V = sizeof(A) == 8 ? 2 : 4;  // 16-byte partial loads
  const bool vec = dim_x % V == 0 && aligned_to(part, V * sizeof(A)) && aligned_to(dx, V * sizeof(T));
  const int width = vec ? V : 1;
  const int nchunk = (dim_x + 64 * width - 1) / (64 * width);
  const unsigned grid = unsigned((g->N * nchunk + kWaves - 1) / kWaves);
  const A* p = static_cast<const A*>(part);
  T* o = static_cast<T*>(dx);
  if (vec)
    hipLaunchKernelGGL((dx_gather_kernel<T, A, V>), dim3(grid), dim3(kBlock), 0, s, g->col_ptr, g->eid, p, o, g->N,
                       dim_x, nchunk);
  else
    hipLaunchKernelGGL((dx_gather_kernel<T, A, 1>), dim3(grid), dim3(kBlock), 0, s, g->col_ptr, g->eid, p, o, g->N,
                       dim_x, nchunk);
  CGTP_CHECK_HIP(hipGetLastError());
}

template <typename T>
void bwd_fused_typed(const ConvArgs& a, const ConvBwdArgs& b, int l1, int L, dim3 grid, size_t lds, hipStream_t s) {
  conv_bwd_fused_typed<T>(a, b, l1, L, grid, lds, s);
}

// Receiver-ordered backward; returns false when the plan or the pointers do
// not fit it (then the row-parallel backward over gathered rows is used).
bool conv_backward_fused(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh,
                         const void* w, double scale, const void* grad_out, void* grad_x, void* grad_sh,
                         void* grad_w, void* ws, size_t ws_bytes, hipStream_t s) {
  const int VEC = plan->dtype == CGTP_F64 ? 2 : CGTP_CONV_BWD_VEC;
  const size_t vb = size_t(VEC) * dtype_size(plan->dtype);
  if (!plan->conv_fused || plan->vec % VEC != 0) return false;
  for (const void* p : {x, w, grad_out, static_cast<const void*>(grad_w)})
    if (p && !aligned_to(p, vb)) return false;
  if (grad_x && !aligned_to(ws, size_t(VEC) * acc_size(plan->dtype))) return false;
  std::vector<int> lgs;
  std::vector<size_t> ldss;
  for (const BlockInfo& blk : plan->blocks) {
    const int lanes = (blk.mul + VEC - 1) / VEC;
    if (lanes > 64) return false;  // one channel chunk per receiver keeps grad_sh race-free
    int lg = 0;
    while ((1 << lg) < lanes) ++lg;
    size_t lds = 0;
    switch (plan->dtype) {
      case CGTP_F32: lds = conv_bwd_fused_lds<float>(blk.l1, plan->conv_L, (1 << lg) * VEC); break;
      case CGTP_F64: lds = conv_bwd_fused_lds<double>(blk.l1, plan->conv_L, (1 << lg) * VEC); break;
      case CGTP_BF16: lds = conv_bwd_fused_lds<bf16>(blk.l1, plan->conv_L, (1 << lg) * VEC); break;
    }
    if (lds == 0) return false;
    lds += size_t(64) * size_t(plan->dim_y) * acc_size(plan->dtype);  // grad_sh tile of 64 edges
    if (lds > 64 * 1024) return false;
    lgs.push_back(lg);
    ldss.push_back(lds);
  }
  const DevTables& t = plan_tables(plan);
  ConvArgs a = make_conv_args(plan, t, g);
  a.x = x;
  a.sh = sh;
  a.w = w;
  a.scale = scale;
  a.nchunks = 1;
  ConvBwdArgs b{};
  b.g = grad_out;
  b.dsh = grad_sh;
  b.dw = grad_w;
  b.dxp = grad_x ? ws : nullptr;
  // The x blocks write disjoint columns of grad_w and of the grad_x partials.
  // grad_sh sums over blocks: with room in the workspace each block writes its
  // own accumulation-type copy and the launches run side by side (largest
  // degree first), then one kernel adds the copies in block order; otherwise
  // the launches accumulate into grad_sh in block order on s.
  const int nb = int(plan->blocks.size());
  const size_t dy_off = grad_x ? align256(conv_backward_partials_bytes(plan, g)) : 0;
  const size_t dy_one = size_t(g->E) * size_t(plan->dim_y) * acc_size(plan->dtype);
  const bool side = nb > 1 && (!grad_sh || (ws && ws_bytes >= dy_off + size_t(nb) * dy_one));
  std::vector<int> order(nb);
  for (int k = 0; k < nb; ++k) order[k] = k;
  if (side)
    std::stable_sort(order.begin(), order.end(),
                     [&](int i, int j) { return plan->blocks[i].l1 > plan->blocks[j].l1; });
  auto launch = [&](int i, hipStream_t st) {
    const int k = order[i];
    ConvArgs ak = a;
    ConvBwdArgs bk = b;
    ak.block = k;
    ak.lg_log2 = lgs[k];
    if (side && grad_sh) {
      bk.dsh = static_cast<char*>(ws) + dy_off + size_t(k) * dy_one;
      bk.dsh_acc = 1;
    } else {
      bk.dy_accum = k > 0 ? 1 : 0;
    }
    const dim3 grid(unsigned(g->N));
    switch (plan->dtype) {
      case CGTP_F32: bwd_fused_typed<float>(ak, bk, plan->blocks[k].l1, plan->conv_L, grid, ldss[k], st); break;
      case CGTP_F64: bwd_fused_typed<double>(ak, bk, plan->blocks[k].l1, plan->conv_L, grid, ldss[k], st); break;
      case CGTP_BF16: bwd_fused_typed<bf16>(ak, bk, plan->blocks[k].l1, plan->conv_L, grid, ldss[k], st); break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
  };
  if (side) {
    side_run(s, nb, launch, conv_edge_bytes(plan, g) >= kSideMinBytes);
    if (grad_sh) {
      const char* part = static_cast<const char*>(ws) + dy_off;
      const int64_t n = g->E * plan->dim_y;
      switch (plan->dtype) {
        case CGTP_F32: dsh_sum<float>(part, grad_sh, n, nb, s); break;
        case CGTP_F64: dsh_sum<double>(part, grad_sh, n, nb, s); break;
        case CGTP_BF16: dsh_sum<bf16>(part, grad_sh, n, nb, s); break;
      }
    }
  } else {
    for (int i = 0; i < nb; ++i) launch(i, s);
  }
  if (grad_x) {
    switch (plan->dtype) {
      case CGTP_F32: dx_gather<float>(g, ws, grad_x, int(plan->dim_x), s); break;
      case CGTP_F64: dx_gather<double>(g, ws, grad_x, int(plan->dim_x), s); break;
      case CGTP_BF16: dx_gather<bf16>(g, ws, grad_x, int(plan->dim_x), s); break;
    }
  }
  return true;
}

}  // namespace

size_t conv_forward_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g) {
  if (!plan->collapse || acc_size(plan->dtype) == dtype_size(plan->dtype)) return 0;
  return size_t(g->N) * size_t(plan->dim_out) * acc_size(plan->dtype);
}

void conv_forward_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh,
                         const void* w, double scale, void* out, hipStream_t s, void* ws, size_t ws_bytes) {
  if (g->E == 0) {
    zero_rows(out, g->N * plan->dim_out, dtype_size(plan->dtype), s);
    return;
  }
  const DevTables& t = plan_tables(plan);
  ConvArgs a = make_conv_args(plan, t, g);
  a.x = x;
  a.sh = sh;
  a.w = w;
  a.out = out;
  a.scale = scale;
  const size_t nacc = conv_forward_ws_bytes(plan, g);
  void* acc_ws = nacc > 0 && ws && ws_bytes >= nacc && aligned_to(ws, 16) ? ws : nullptr;
  const bool big = conv_edge_bytes(plan, g) >= kSideMinBytes;
  switch (plan->dtype) {
    case CGTP_F32: fwd_typed<float>(plan, a, acc_ws, big, s); break;
    case CGTP_F64: fwd_typed<double>(plan, a, acc_ws, big, s); break;
    case CGTP_BF16: fwd_typed<bf16>(plan, a, acc_ws, big, s); break;
  }
}

size_t conv_backward_partials_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g) {
  return size_t(g->E) * size_t(plan->dim_x) * acc_size(plan->dtype);
}

// The grad_x partials, then (fused plans with several x blocks) one grad_sh
// copy per x block so that the blocks' launches can run side by side.
size_t conv_backward_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g) {
  size_t n = align256(conv_backward_partials_bytes(plan, g));
  if (plan->conv_fused && plan->blocks.size() > 1)
    n += plan->blocks.size() * size_t(g->E) * size_t(plan->dim_y) * acc_size(plan->dtype);
  return n;
}

void conv_backward_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh,
                          const void* w, double scale, const void* grad_out, void* grad_x,
                          void* grad_sh, void* grad_w, void* ws, size_t ws_bytes, hipStream_t s) {
  if (g->E == 0) {
    if (grad_x && g->N > 0)
      zero_rows(grad_x, g->N * plan->dim_x, dtype_size(plan->dtype), s);
    return;
  }
  if (grad_x) {
    const size_t need = conv_backward_partials_bytes(plan, g);
    if (!ws || ws_bytes < need)
      throw Error{CGTP_ERR_WORKSPACE, "conv_backward needs " + std::to_string(need) + " workspace bytes"};
  }
  if (!grad_x && !grad_sh && !grad_w) return;
  const size_t es = dtype_size(plan->dtype), as = acc_size(plan->dtype);
  // padding edges: their gradients are zero (their partials of grad_x are
  // not in the transpose, so dx_gather never reads them)
  auto zero_padding = [&] {
    const int64_t np = g->pad_e1 - g->pad_e0;
    if (np == 0) return;
    if (grad_sh) zero_rows(static_cast<char*>(grad_sh) + g->pad_e0 * plan->dim_y * es, np * plan->dim_y, es, s);
    if (grad_w) zero_rows(static_cast<char*>(grad_w) + g->pad_e0 * plan->w_numel * es, np * plan->w_numel, es, s);
  };
  if (conv_backward_fused(plan, g, x, sh, w, scale, grad_out, grad_x, grad_sh, grad_w, ws, ws_bytes, s)) {
    zero_unread_x(plan, grad_x, g->N, es, s);
    zero_padding();
    return;
  }
  // general kernel over edge rows, the padding range left out
  auto rows = [&](int64_t e0, int64_t e1) {
    if (e1 <= e0) return;
    auto off = [&](const void* p, int64_t per, size_t sz) -> const void* {
      return p ? static_cast<const char*>(p) + e0 * per * int64_t(sz) : nullptr;
    };
    TPBackwardRows r;
    r.rows = e1 - e0;
    r.x = x;
    r.x_idx = g->src + e0;
    r.y = off(sh, plan->dim_y, es);
    r.w = off(w, plan->w_numel, es);
    r.w_stride = plan->w_numel;
    r.g = grad_out;
    r.g_idx = g->dst + e0;
    r.g_scale = scale;
    r.dx_ws = grad_x ? const_cast<void*>(off(ws, plan->dim_x, as)) : nullptr;
    r.dy = const_cast<void*>(off(grad_sh, plan->dim_y, es));
    r.dw = const_cast<void*>(off(grad_w, plan->w_numel, es));
    tp_backward_rows(plan, r, s);
  };
  rows(0, g->pad_e0 < g->pad_e1 ? g->pad_e0 : g->E);
  if (g->pad_e0 < g->pad_e1) rows(g->pad_e1, g->E);
  zero_padding();
  if (grad_x) {
    switch (plan->dtype) {
      case CGTP_F32: dx_gather<float>(g, ws, grad_x, int(plan->dim_x), s); break;
      case CGTP_F64: dx_gather<double>(g, ws, grad_x, int(plan->dim_x), s); break;
      case CGTP_BF16: dx_gather<bf16>(g, ws, grad_x, int(plan->dim_x), s); break;
    }
    zero_unread_x(plan, grad_x, g->N, dtype_size(plan->dtype), s);
  }
}

}  // namespace cgtp
