// Launchers of the row-parallel tensor product (kernels in tp_impl.hpp).
#include "tp_impl.hpp"

namespace cgtp {

CGTP_TP_EXTERN_FWD(float, 1)
CGTP_TP_EXTERN_FWD(float, 4)
CGTP_TP_EXTERN_FWD(bf16, 1)
CGTP_TP_EXTERN_FWD(bf16, 4)
CGTP_TP_EXTERN_FWD(double, 1)
CGTP_TP_EXTERN_FWD(double, 2)
CGTP_TP_EXTERN_FWDC(float, 1)
CGTP_TP_EXTERN_FWDC(float, 2)
CGTP_TP_EXTERN_FWDC(float, 4)
CGTP_TP_EXTERN_FWDC(bf16, 1)
CGTP_TP_EXTERN_FWDC(bf16, 2)
CGTP_TP_EXTERN_FWDC(bf16, 4)
CGTP_TP_EXTERN_FWDC(double, 1)
CGTP_TP_EXTERN_FWDC(double, 2)
CGTP_TP_EXTERN_BWD(float, 1)
CGTP_TP_EXTERN_BWD(float, 2)
CGTP_TP_EXTERN_BWD(float, 4)
CGTP_TP_EXTERN_BWD(bf16, 1)
CGTP_TP_EXTERN_BWD(bf16, 2)
CGTP_TP_EXTERN_BWD(bf16, 4)
CGTP_TP_EXTERN_BWD(double, 1)
CGTP_TP_EXTERN_BWD(double, 2)

// Channels per lane of the backward kernel for 4-byte and 2-byte storage
// (the backward keeps more per-channel state than the forward).
#ifndef CGTP_TP_BWD_VEC
#define CGTP_TP_BWD_VEC 4
#endif
#ifndef CGTP_TP_BWD_VEC_BF16
#define CGTP_TP_BWD_VEC_BF16 4
#endif
// Channels per lane of the collapsed-output forward with 4- and 2-byte
// storage: its accumulators for every output degree stay in registers, and
// 2 channels keep the kernel at 3-4 waves per SIMD where 4 channels drop
// it to 1-2.
#ifndef CGTP_TP_BWDC_ALL_BLOCKS
#define CGTP_TP_BWDC_ALL_BLOCKS 1
#endif
#ifndef CGTP_TP_BWD_ALL_BLOCKS
#define CGTP_TP_BWD_ALL_BLOCKS 1
#endif
#ifndef CGTP_TP_FWDC_VEC
#define CGTP_TP_FWDC_VEC 2
#endif

// ----------------------------------------------------------------- launchers

namespace {

int ilog2_ceil(int v) {
  int k = 0;
  while ((1 << k) < v) ++k;
  return k;
}

bool aligned(const void* p, size_t bytes) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

// Dynamic LDS a workgroup may take on the current device.
size_t device_lds_limit() {
  int dev = 0, v = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  CGTP_CHECK_HIP(hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
  return size_t(v);
}

TPArgs make_args(cgtp_plan_s* plan, const DevTables& t, int64_t B, int vec) {
  TPArgs a{};
  a.g_scale = 1.0;
  a.paths = t.paths;
  a.blocks = t.blocks;
  a.coef = t.coef;
  a.B = B;
  a.w_stride = plan->wkind == CGTP_W_PER_ROW ? plan->w_numel : 0;
  a.dim_x = int(plan->dim_x);
  a.dim_y = int(plan->dim_y);
  a.dim_out = int(plan->dim_out);
  a.W = int(plan->w_numel);
  a.nblocks = int(plan->blocks.size());
  a.max_l1 = 0;
  for (const BlockInfo& b : plan->blocks) a.max_l1 = b.l1 > a.max_l1 ? b.l1 : a.max_l1;
  a.ngroups = (plan->max_mul + vec - 1) / vec;
  a.lpr_log2 = ilog2_ceil(a.ngroups < 64 ? a.ngroups : 64);
  return a;
}

template <typename T>
void colsum(const void* in, void* part, void* out, int64_t rows, int W, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const int nchunks = int((rows + kRowsPerChunk - 1) / kRowsPerChunk);
  const unsigned gx = unsigned((W + kBlock - 1) / kBlock);
  hipLaunchKernelGGL((colsum_stage1<A>), dim3(gx, unsigned(nchunks)), dim3(kBlock), 0, s,
                     static_cast<const A*>(in), static_cast<A*>(part), rows, W);
  hipLaunchKernelGGL((colsum_stage2<T, A>), dim3(gx), dim3(kBlock), 0, s, static_cast<const A*>(part),
                     static_cast<T*>(out), nchunks, W);
}

}  // namespace

void tp_forward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w,
                       void* out, hipStream_t stream) {
  const DevTables& t = plan_tables(plan);
  const size_t es = dtype_size(plan->dtype);
  int vec = plan->vec;
  if (!aligned(x, vec * es) || !aligned(w, vec * es) || !aligned(out, vec * es)) vec = 1;
  TPArgs a = make_args(plan, t, B, vec);
  a.x = x;
  a.y = y;
  a.w = w;
  a.out = out;
  if (plan->collapse) {
    // one launch per output parity that has blocks, all x blocks in each
    if (plan->dtype != CGTP_F64 && vec > CGTP_TP_FWDC_VEC) {
      vec = CGTP_TP_FWDC_VEC;
      a = make_args(plan, t, B, vec);
      a.x = x;
      a.y = y;
      a.w = w;
      a.out = out;
    }
    bool any[2] = {false, false};
    for (int pi = 0; pi < 2; ++pi)
      for (int l = 0; l <= kLmax; ++l) a.goff[pi][l] = -1, a.gmul[pi][l] = 0;
    for (const OutBlock& o : plan->outputs) {
      const int pi = o.p3 > 0 ? 0 : 1;
      a.goff[pi][o.l3] = o.out_off;
      a.gmul[pi][o.l3] = o.mul;
      any[pi] = true;
    }
    for (int pi = 0; pi < 2; ++pi) {
      if (!any[pi]) continue;
      a.par = pi == 0 ? 1 : -1;
      switch (plan->dtype) {
        case CGTP_F32:
          vec == 1   ? tp_fwd_collapsed_typed<float, 1>(a, plan->lm, stream)
          : vec == 2 ? tp_fwd_collapsed_typed<float, 2>(a, plan->lm, stream)
                     : tp_fwd_collapsed_typed<float, 4>(a, plan->lm, stream);
          break;
        case CGTP_BF16:
          vec == 1   ? tp_fwd_collapsed_typed<bf16, 1>(a, plan->lm, stream)
          : vec == 2 ? tp_fwd_collapsed_typed<bf16, 2>(a, plan->lm, stream)
                     : tp_fwd_collapsed_typed<bf16, 4>(a, plan->lm, stream);
          break;
        case CGTP_F64:
          vec == 1 ? tp_fwd_collapsed_typed<double, 1>(a, plan->lm, stream)
                   : tp_fwd_collapsed_typed<double, 2>(a, plan->lm, stream);
          break;
      }
      CGTP_CHECK_HIP(hipGetLastError());
    }
    return;
  }
  // one launch per x block with the kernel specialised for its degree (the
  // general kernel in one launch when channels are not vectorised)
  const int nb = vec == 1 ? 1 : int(plan->blocks.size());
  for (int b = 0; b < nb; ++b) {
    a.block = b;
    const int l1 = vec == 1 ? -1 : plan->blocks[size_t(b)].l1;
    switch (plan->dtype) {
      case CGTP_F32:
        vec == 1 ? tp_fwd_typed<float, 1>(a, l1, plan->lm, stream) : tp_fwd_typed<float, 4>(a, l1, plan->lm, stream);
        break;
      case CGTP_BF16:
        vec == 1 ? tp_fwd_typed<bf16, 1>(a, l1, plan->lm, stream) : tp_fwd_typed<bf16, 4>(a, l1, plan->lm, stream);
        break;
      case CGTP_F64:
        vec == 1 ? tp_fwd_typed<double, 1>(a, l1, plan->lm, stream)
                 : tp_fwd_typed<double, 2>(a, l1, plan->lm, stream);
        break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
  }
}

namespace {

// p[r * ld + off + j] = 0 for j < n (one element per thread)
template <typename E>
__global__ __launch_bounds__(kBlock) void zero_cols_kernel(E* __restrict__ p, int64_t rows, int64_t ld, int off, int n) {
  const int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= rows * n) return;
  const int64_t r = i / n;
  p[r * ld + off + (i - r * n)] = E(0);
}

}  // namespace

void zero_rows(void* p, int64_t n, size_t es, hipStream_t stream) {
  if (!p || n == 0) return;
  const dim3 grid(unsigned((n + kBlock - 1) / kBlock));
  if (es == 2)
    hipLaunchKernelGGL((zero_cols_kernel<uint16_t>), grid, dim3(kBlock), 0, stream, static_cast<uint16_t*>(p), n,
                       int64_t(1), 0, 1);
  else if (es == 4)
    hipLaunchKernelGGL((zero_cols_kernel<uint32_t>), grid, dim3(kBlock), 0, stream, static_cast<uint32_t*>(p), n,
                       int64_t(1), 0, 1);
  else
    hipLaunchKernelGGL((zero_cols_kernel<uint64_t>), grid, dim3(kBlock), 0, stream, static_cast<uint64_t*>(p), n,
                       int64_t(1), 0, 1);
  CGTP_CHECK_HIP(hipGetLastError());
}

void zero_unread_x(const cgtp_plan_s* plan, void* p, int64_t rows, size_t es, hipStream_t stream) {
  if (!p || rows == 0) return;
  for (const auto& blk : plan->x_unread) {
    const dim3 grid(unsigned((rows * blk.second + kBlock - 1) / kBlock));
    if (es == 2)
      hipLaunchKernelGGL((zero_cols_kernel<uint16_t>), grid, dim3(kBlock), 0, stream, static_cast<uint16_t*>(p), rows,
                         plan->dim_x, blk.first, blk.second);
    else if (es == 4)
      hipLaunchKernelGGL((zero_cols_kernel<uint32_t>), grid, dim3(kBlock), 0, stream, static_cast<uint32_t*>(p), rows,
                         plan->dim_x, blk.first, blk.second);
    else
      hipLaunchKernelGGL((zero_cols_kernel<uint64_t>), grid, dim3(kBlock), 0, stream, static_cast<uint64_t*>(p), rows,
                         plan->dim_x, blk.first, blk.second);
    CGTP_CHECK_HIP(hipGetLastError());
  }
}

size_t tp_backward_ws_bytes(const cgtp_plan_s* plan, int64_t B) {
  if (plan->wkind != CGTP_W_SHARED || B == 0) return 0;
  const int64_t nchunks = (B + kRowsPerChunk - 1) / kRowsPerChunk;
  return size_t(B + nchunks) * size_t(plan->w_numel) * acc_size(plan->dtype);
}

void tp_backward_rows(cgtp_plan_s* plan, const TPBackwardRows& r, hipStream_t stream) {
  const DevTables& t = plan_tables(plan);
  const size_t es = dtype_size(plan->dtype), as = acc_size(plan->dtype);
  int vec = plan->vec;
  const int max_vec = plan->dtype == CGTP_BF16 ? CGTP_TP_BWD_VEC_BF16 : CGTP_TP_BWD_VEC;
  if (plan->dtype != CGTP_F64 && vec > max_vec) vec = max_vec;
  if (!aligned(r.x, vec * es) || !aligned(r.w, vec * es) || !aligned(r.g, vec * es) ||
      !aligned(r.dx, vec * es) || !aligned(r.dw, vec * es) || !aligned(r.dx_ws, vec * as) ||
      !aligned(r.dw_ws, vec * as))
    vec = 1;
  // LDS: the vectorised kernels hold grad_y columns and grad_x rows of up to
  // the largest x degree; when that exceeds the device limit the one-channel
  // kernel (grad_y columns only) runs, and a plan whose grad_y columns alone
  // do not fit (many repeated y blocks) is refused
  int max_l1 = 0;
  for (const BlockInfo& b : plan->blocks) max_l1 = b.l1 > max_l1 ? b.l1 : max_l1;
  const size_t lds_max = device_lds_limit();
  if (vec > 1 && tp_bwd_lds_bytes(int(plan->dim_y), max_l1, max_l1, vec, as) > lds_max) vec = 1;
  if (tp_bwd_lds_bytes(int(plan->dim_y), -1, max_l1, vec, as) > lds_max)
    throw Error{CGTP_ERR_UNSUPPORTED, "tp_backward: per-lane grad_y columns of " + std::to_string(plan->dim_y) +
                                          " harmonic components do not fit the device's LDS"};
  TPArgs a = make_args(plan, t, r.rows, vec);
  a.w_stride = r.w_stride;
  a.x = r.x;
  a.y = r.y;
  a.w = r.w;
  a.g = r.g;
  a.dx = r.dx;
  a.dy = r.dy;
  a.dw = r.dw;
  a.dw_ws = r.dw_ws;
  a.dx_ws = r.dx_ws;
  a.x_idx = r.x_idx;
  a.g_idx = r.g_idx;
  a.g_scale = r.g_scale;
  // One launch over every x block (grad_x rows in LDS, the block's degree
  // dispatched per block), or one launch per x block (degree-specialised;
  // grad_y then accumulates across the launches in stream order). Either way
  // the summation order is fixed. With collapsed outputs the x blocks share
  // cotangent blocks, which one launch reads once from memory; without, the
  // single launch saves the per-launch tails and grad_y round trips
  // (tp_large fp32: 26.4 -> 25.0 ms).
  const bool all_blocks = vec > 1 && (plan->collapse ? CGTP_TP_BWDC_ALL_BLOCKS : CGTP_TP_BWD_ALL_BLOCKS);
  const int nb = vec == 1 || all_blocks ? 1 : int(plan->blocks.size());
  const int lm = plan->lm;
  for (int b = 0; b < nb; ++b) {
    a.block = b;
    a.dy_accum = b > 0 ? 1 : 0;
    const int l1 = vec == 1 ? -1 : all_blocks ? -2 : plan->blocks[size_t(b)].l1;
    switch (plan->dtype) {
      case CGTP_F32:
        vec == 1 ? tp_bwd_typed<float, 1>(a, l1, lm, stream)
                 : (vec == 2 ? tp_bwd_typed<float, 2>(a, l1, lm, stream) : tp_bwd_typed<float, 4>(a, l1, lm, stream));
        break;
      case CGTP_BF16:
        vec == 1 ? tp_bwd_typed<bf16, 1>(a, l1, lm, stream)
                 : (vec == 2 ? tp_bwd_typed<bf16, 2>(a, l1, lm, stream) : tp_bwd_typed<bf16, 4>(a, l1, lm, stream));
        break;
      case CGTP_F64:
        vec == 1 ? tp_bwd_typed<double, 1>(a, l1, lm, stream) : tp_bwd_typed<double, 2>(a, l1, lm, stream);
        break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
  }
}

void tp_backward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y,
                        const void* w, const void* g, void* dx, void* dy, void* dw, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  const bool shared = plan->wkind == CGTP_W_SHARED;
  if (shared && dw) {
    const size_t need = tp_backward_ws_bytes(plan, B);
    if (!ws || ws_bytes < need)
      throw Error{CGTP_ERR_WORKSPACE, "tp_backward needs " + std::to_string(need) + " workspace bytes"};
  }
  TPBackwardRows r;
  r.rows = B;
  r.x = x;
  r.y = y;
  r.w = w;
  r.w_stride = shared ? 0 : plan->w_numel;
  r.g = g;
  r.dx = dx;
  r.dy = dy;
  r.dw = shared ? nullptr : dw;
  r.dw_ws = (shared && dw) ? ws : nullptr;
  tp_backward_rows(plan, r, stream);
  zero_unread_x(plan, dx, B, dtype_size(plan->dtype), stream);
  if (shared && dw) {
    char* part = static_cast<char*>(ws) + size_t(B) * plan->w_numel * acc_size(plan->dtype);
    switch (plan->dtype) {
      case CGTP_F32: colsum<float>(ws, part, dw, B, int(plan->w_numel), stream); break;
      case CGTP_BF16: colsum<bf16>(ws, part, dw, B, int(plan->w_numel), stream); break;
      case CGTP_F64: colsum<double>(ws, part, dw, B, int(plan->w_numel), stream); break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
  }
}

}  // namespace cgtp
