// Launchers of the message-passing convolution (kernels in conv_impl.hpp).
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

template <typename T>
void fwd_typed(cgtp_plan_s* plan, ConvArgs a, hipStream_t s) {
  const size_t vb = size_t(conv_vec(plan->dtype)) * dtype_size(plan->dtype);
  const bool fused = plan->conv_fused && (!plan->collapse || plan->conv_col_fused) &&
                     plan->vec == conv_vec(plan->dtype) && aligned_to(a.x, vb) && aligned_to(a.w, vb) &&
                     aligned_to(a.out, vb);
  if (plan->collapse) {  // the kernels add into the output
    zero_rows(a.out, a.N * int64_t(a.dim_out), dtype_size(plan->dtype), s);
    a.collapse = 1;
  }
  if (!fused) {
    const int64_t items = a.N * int64_t(a.collapse ? 1 : a.npaths) * a.nchunks;
    conv_fwd_general_typed<T>(a, dim3(unsigned((items + kWaves - 1) / kWaves)), s);
    CGTP_CHECK_HIP(hipGetLastError());
    return;
  }
  // one launch per x block, specialised for its degree and the plan's largest degree
  const int VEC = conv_vec(plan->dtype);
  for (size_t b = 0; b < plan->blocks.size(); ++b) {
    const BlockInfo& blk = plan->blocks[b];
    const int lanes = (blk.mul + VEC - 1) / VEC;
    int lg = 0;
    while ((1 << lg) < lanes && lg < 6) ++lg;
    a.block = int(b);
    a.lg_log2 = lg;
    a.nchunks = (lanes + (1 << lg) - 1) >> lg;
    const int nch = conv_fused_chunks<T>(blk.l1, plan->conv_L, a.collapse != 0);
    const int64_t items = a.N * int64_t(nch) * a.nchunks;
    conv_fwd_fused_typed<T>(a, blk.l1, plan->conv_L, dim3(unsigned((items + kWaves - 1) / kWaves)), s);
    CGTP_CHECK_HIP(hipGetLastError());
  }
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
                         void* grad_w, void* ws, hipStream_t s) {
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
  for (size_t k = 0; k < plan->blocks.size(); ++k) {
    a.block = int(k);
    a.lg_log2 = lgs[k];
    b.dy_accum = k > 0 ? 1 : 0;
    const dim3 grid(unsigned(g->N));
    switch (plan->dtype) {
      case CGTP_F32: bwd_fused_typed<float>(a, b, plan->blocks[k].l1, plan->conv_L, grid, ldss[k], s); break;
      case CGTP_F64: bwd_fused_typed<double>(a, b, plan->blocks[k].l1, plan->conv_L, grid, ldss[k], s); break;
      case CGTP_BF16: bwd_fused_typed<bf16>(a, b, plan->blocks[k].l1, plan->conv_L, grid, ldss[k], s); break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
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

void conv_forward_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh,
                         const void* w, double scale, void* out, hipStream_t s) {
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
  switch (plan->dtype) {
    case CGTP_F32: fwd_typed<float>(plan, a, s); break;
    case CGTP_F64: fwd_typed<double>(plan, a, s); break;
    case CGTP_BF16: fwd_typed<bf16>(plan, a, s); break;
  }
}

size_t conv_backward_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g) {
  return size_t(g->E) * size_t(plan->dim_x) * acc_size(plan->dtype);
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
    const size_t need = conv_backward_ws_bytes(plan, g);
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
  if (conv_backward_fused(plan, g, x, sh, w, scale, grad_out, grad_x, grad_sh, grad_w, ws, s)) {
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
