// Launchers of the row-parallel tensor product (kernels in tp_impl.hpp).
#include <algorithm>
#include <map>
#include <mutex>

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
// One backward launch over every x block, for collapsed and uncollapsed
// outputs (1), or one launch per x block (0).
#ifndef CGTP_TP_BWDC_ALL_BLOCKS
#define CGTP_TP_BWDC_ALL_BLOCKS 1
#endif
#ifndef CGTP_TP_BWD_ALL_BLOCKS
#define CGTP_TP_BWD_ALL_BLOCKS 1
#endif
// Channels per lane of the collapsed-output forward with 4- and 2-byte
// storage: its accumulators for every output degree stay in registers, and
// 2 channels keep the kernel at 3-4 waves per SIMD where 4 channels drop
// it to 1-2.
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
    // the two parities write disjoint output blocks: their launches run side by side
    std::vector<int> pars;
    for (int pi = 0; pi < 2; ++pi)
      if (any[pi]) pars.push_back(pi);
    const bool big = double(B) * double(plan->dim_out + plan->dim_x) * double(es) >= kSideMinBytes;
    side_run(stream, int(pars.size()), [&](int i, hipStream_t st) {
      TPArgs ap = a;
      ap.par = pars[size_t(i)] == 0 ? 1 : -1;
      switch (plan->dtype) {
        case CGTP_F32:
          vec == 1   ? tp_fwd_collapsed_typed<float, 1>(ap, plan->lm, st)
          : vec == 2 ? tp_fwd_collapsed_typed<float, 2>(ap, plan->lm, st)
                     : tp_fwd_collapsed_typed<float, 4>(ap, plan->lm, st);
          break;
        case CGTP_BF16:
          vec == 1   ? tp_fwd_collapsed_typed<bf16, 1>(ap, plan->lm, st)
          : vec == 2 ? tp_fwd_collapsed_typed<bf16, 2>(ap, plan->lm, st)
                     : tp_fwd_collapsed_typed<bf16, 4>(ap, plan->lm, st);
          break;
        case CGTP_F64:
          vec == 1 ? tp_fwd_collapsed_typed<double, 1>(ap, plan->lm, st)
                   : tp_fwd_collapsed_typed<double, 2>(ap, plan->lm, st);
          break;
      }
      CGTP_CHECK_HIP(hipGetLastError());
    }, big);
    return;
  }
  const bool big = double(B) * double(plan->dim_out + plan->dim_x) * double(es) >= kSideMinBytes;
  // Small calls are bound by launch overhead: one launch over every x block
  // (x degrees up to the plan's largest y/output degree).
  if (!big && vec != 1 && plan->blocks.size() > 1 && a.max_l1 <= plan->lm) {
    switch (plan->dtype) {
      case CGTP_F32: tp_fwd_typed<float, 4>(a, -2, plan->lm, stream); break;
      case CGTP_BF16: tp_fwd_typed<bf16, 4>(a, -2, plan->lm, stream); break;
      case CGTP_F64: tp_fwd_typed<double, 2>(a, -2, plan->lm, stream); break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
    return;
  }
  // Otherwise one launch per x block with the kernel specialised for its
  // degree (the general kernel in one launch when channels are not
  // vectorised). The blocks write disjoint output columns, so their launches
  // run side by side, the largest degree first (measured against one launch
  // over every block at 2^20 rows: 19.8-20.0 against 20.9 ms).
  const int nb = vec == 1 ? 1 : int(plan->blocks.size());
  std::vector<int> order(nb);
  for (int b = 0; b < nb; ++b) order[b] = b;
  if (vec != 1)
    std::stable_sort(order.begin(), order.end(),
                     [&](int i, int j) { return plan->blocks[size_t(i)].l1 > plan->blocks[size_t(j)].l1; });
  side_run(stream, nb, [&](int i, hipStream_t st) {
    TPArgs ab = a;
    ab.block = order[size_t(i)];
    const int l1 = vec == 1 ? -1 : plan->blocks[size_t(ab.block)].l1;
    switch (plan->dtype) {
      case CGTP_F32:
        vec == 1 ? tp_fwd_typed<float, 1>(ab, l1, plan->lm, st) : tp_fwd_typed<float, 4>(ab, l1, plan->lm, st);
        break;
      case CGTP_BF16:
        vec == 1 ? tp_fwd_typed<bf16, 1>(ab, l1, plan->lm, st) : tp_fwd_typed<bf16, 4>(ab, l1, plan->lm, st);
        break;
      case CGTP_F64:
        vec == 1 ? tp_fwd_typed<double, 1>(ab, l1, plan->lm, st) : tp_fwd_typed<double, 2>(ab, l1, plan->lm, st);
        break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
  }, big);
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


// ---------------------------------------------- backward without allocation
// For callers that cannot allocate (work under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc): the shared-weight backward with its
// per-row grad_w partials and per-chunk sums in a file-scope device array
// instead of a caller workspace. Rows run in passes of a multiple of
// kRowsPerChunk rows, so the chunks and their order are those of
// tp_backward_launch and the results are bitwise the same. Every call on one
// device uses that device's one copy of the array: calls that overlap on a
// device race (the caller serialises them, e.g. on one stream).
namespace {

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;  // device id -> that device's copy of scratch

// Device address of scratch on the current device, looked up once per device
// (in host code the array's name is a host-side stand-in, not the address).
char* scratch_address() {
  int dev = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_addr.find(dev);
  if (it != g_scratch_addr.end()) return static_cast<char*>(it->second);
  void* p = nullptr;
  CGTP_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
  g_scratch_addr[dev] = p;
  return static_cast<char*>(p);
}

template <typename T>
void colsum_rows_into(const void* in, void* part, int64_t rows, int W, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const int nchunks = int((rows + kRowsPerChunk - 1) / kRowsPerChunk);
  const unsigned gx = unsigned((W + kBlock - 1) / kBlock);
  hipLaunchKernelGGL((colsum_stage1<A>), dim3(gx, unsigned(nchunks)), dim3(kBlock), 0, s,
                     static_cast<const A*>(in), static_cast<A*>(part), rows, W);
}

template <typename T>
void colsum_chunks(const void* part, void* out, int64_t nchunks, int W, hipStream_t s) {
  using A = typename AccOf<T>::type;
  const unsigned gx = unsigned((W + kBlock - 1) / kBlock);
  hipLaunchKernelGGL((colsum_stage2<T, A>), dim3(gx), dim3(kBlock), 0, s, static_cast<const A*>(part),
                     static_cast<T*>(out), int(nchunks), W);
}

}  // namespace

void tp_backward_noalloc_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w,
                                const void* g, void* dx, void* dy, void* dw, hipStream_t stream) {
  if (plan->wkind != CGTP_W_SHARED || !dw) {  // no partials needed
    tp_backward_launch(plan, B, x, y, w, g, dx, dy, dw, nullptr, 0, stream);
    return;
  }
  const size_t es = dtype_size(plan->dtype);
  const size_t wb = size_t(plan->w_numel) * acc_size(plan->dtype);  // one row of partials
  const int64_t nchunks = (B + kRowsPerChunk - 1) / kRowsPerChunk;
  const size_t part_bytes = (size_t(nchunks) * wb + 255) / 256 * 256;
  const int64_t rows_fit = part_bytes < kNoallocScratchBytes ? int64_t((kNoallocScratchBytes - part_bytes) / wb) : 0;
  const int64_t pass = B <= rows_fit ? B : rows_fit / kRowsPerChunk * kRowsPerChunk;
  if (pass == 0)
    throw Error{CGTP_ERR_WORKSPACE,
                "tp_backward_noalloc: " + std::to_string(B) + " rows of " + std::to_string(plan->w_numel) +
                    " shared weights need " + std::to_string(part_bytes + size_t(std::min<int64_t>(B, kRowsPerChunk)) * wb) +
                    " bytes of scratch; the library's scratch holds " + std::to_string(kNoallocScratchBytes)};
  char* base = scratch_address();
  char* part = base;               // [nchunks][W] chunk sums
  char* rows_ws = base + part_bytes;  // [pass][W] per-row partials
  for (int64_t r0 = 0; r0 < B; r0 += pass) {
    const int64_t n = std::min(pass, B - r0);
    auto at = [&](const void* p, int64_t per) -> const void* {
      return p ? static_cast<const char*>(p) + size_t(r0) * size_t(per) * es : nullptr;
    };
    TPBackwardRows r;
    r.rows = n;
    r.x = at(x, plan->dim_x);
    r.y = at(y, plan->dim_y);
    r.w = w;
    r.w_stride = 0;
    r.g = at(g, plan->dim_out);
    r.dx = const_cast<void*>(at(dx, plan->dim_x));
    r.dy = const_cast<void*>(at(dy, plan->dim_y));
    r.dw_ws = rows_ws;
    tp_backward_rows(plan, r, stream);
    char* pdst = part + size_t(r0 / kRowsPerChunk) * wb;
    switch (plan->dtype) {
      case CGTP_F32: colsum_rows_into<float>(rows_ws, pdst, n, int(plan->w_numel), stream); break;
      case CGTP_BF16: colsum_rows_into<bf16>(rows_ws, pdst, n, int(plan->w_numel), stream); break;
      case CGTP_F64: colsum_rows_into<double>(rows_ws, pdst, n, int(plan->w_numel), stream); break;
    }
    CGTP_CHECK_HIP(hipGetLastError());
  }
  zero_unread_x(plan, dx, B, es, stream);
  switch (plan->dtype) {
    case CGTP_F32: colsum_chunks<float>(part, dw, nchunks, int(plan->w_numel), stream); break;
    case CGTP_BF16: colsum_chunks<bf16>(part, dw, nchunks, int(plan->w_numel), stream); break;
    case CGTP_F64: colsum_chunks<double>(part, dw, nchunks, int(plan->w_numel), stream); break;
  }
  CGTP_CHECK_HIP(hipGetLastError());
}

}  // namespace cgtp
