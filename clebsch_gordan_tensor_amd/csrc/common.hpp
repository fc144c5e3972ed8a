// Internal types shared by the planner, the launchers and the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "cgtp.h"

namespace cgtp {

constexpr int kLmax = CGTP_LMAX;
constexpr int kBlock = 256;  // threads per workgroup for the row kernels

// ---------------------------------------------------------------- errors
void set_error(const std::string& msg);
struct Error {
  cgtp_status code;
  std::string msg;
};
#define CGTP_CHECK_HIP(expr)                                                              \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      throw ::cgtp::Error{CGTP_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)}; \
  } while (0)

// ------------------------------------------------------------ plan types
struct Irrep {
  int mul, l, p;
};

// One path in path order. Offsets are element offsets inside a row.
struct PathInfo {
  int i1, i2, l1, l2, l3, p3, mul;  // mul: x multiplicity u
  int x_off, y_off, out_off, w_off, coef_off;
  int i2_end;  // one past the last path of the run with the same (i1, i2)
  int v;        // y multiplicity
  int out_mul;  // output multiplicity (uvu: u; uvw: from irreps_out)
  int w_len;    // weights of the path (uvu: u v; uvw: u v w)
};

// One x block with the contiguous range of paths that read it.
struct BlockInfo {
  int l1, mul, x_off, path_begin, path_end;
};

// One output block: a path's own block, or with collapsed outputs the block
// that every path of one (l3, p3) adds into.
struct OutBlock {
  int l3, p3, mul, out_off;
};

// Device copies (plain 32-bit fields).
struct alignas(16) PathDev {
  int32_t l2, l3, y_off, out_off;
  int32_t w_off, coef_off, i2_end, mul;
  int32_t l1, x_off, p3, pad1;  // pad1: y multiplicity v of the path
};
struct alignas(16) BlockDev {
  int32_t l1, mul, x_off, path_begin;
  int32_t path_end, pad0, pad1, pad2;
};

struct DevTables {
  PathDev* paths = nullptr;
  BlockDev* blocks = nullptr;
  void* coef = nullptr;          // float (f32/bf16 plans) or double (f64 plans)
  void* ones = nullptr;          // unit shared weights [w_numel] in the storage type (uvw sub-plans)
  int32_t* slot_paths = nullptr;  // fused convolution: path index per (block, slot), -1 = none
  int32_t* slot_off = nullptr;    // first slot of each block
};

}  // namespace cgtp

struct cgtp_linear_s;

struct cgtp_plan_s {
  // connection mode: 0 = uvu (channel-wise), 1 = uvw (fully connected)
  int mode = 0;
  int max_ymul = 1;  // largest y multiplicity (uvu with > 1: the generic kernels)
  // uvw: the unit-weight uvu product over the same paths (its output rows are
  // the path outputs T) and the channel mixing T -> out as a linear map
  cgtp_plan_s* unit = nullptr;
  cgtp_linear_s* mix = nullptr;
  bool with_ones = false;  // upload unit weights with the device tables
  std::vector<cgtp::Irrep> X, Y, O;
  std::vector<cgtp::PathInfo> paths;
  std::vector<cgtp::BlockInfo> blocks;
  std::vector<cgtp::OutBlock> outputs;
  // x blocks that no path reads, as (offset, elements) within an x row: their
  // gradient is zero and is written as such
  std::vector<std::pair<int, int>> x_unread;
  cgtp_paths select = CGTP_PATHS_ALL;
  bool collapse = false;
  std::vector<std::vector<double>> cg_dense;  // per path, [2l1+1][2l2+1][2l3+1]
  std::vector<double> coef64;                 // packed in kernel pattern order
  std::vector<float> coef32;
  int64_t dim_x = 0, dim_y = 0, dim_out = 0, w_numel = 0;
  int max_mul = 0;
  int vec = 1;  // channels per lane of the vectorised kernels
  // Fused convolution (edge loop outside, all paths of one x block in
  // registers): possible when each degree occurs at most once in y. Slots of
  // block b are every (l2, l3) with l2, l3 <= conv_L and |l1-l2| <= l3 <= l1+l2,
  // ordered by l2 then l3; slot_paths maps them to path indices (-1 = absent).
  bool conv_fused = false;
  // collapsed outputs may use the fused forward (y parities are s (-1)^l)
  bool conv_col_fused = false;
  int conv_L = 0;
  int lm = 0;  // largest degree among y blocks and output paths (kernel specialisation)
  int yoff_by_l[CGTP_LMAX + 1] = {-1, -1, -1, -1, -1};
  std::vector<int32_t> slot_paths, slot_off;
  cgtp_dtype dtype = CGTP_F32;
  cgtp_wkind wkind = CGTP_W_SHARED;
  std::mutex mu;
  std::map<int, cgtp::DevTables> dev;  // per HIP device id
};

namespace cgtp {

// Planner (plan.cpp).
// "MxLp + ..." -> blocks, order kept (CGTP_ERR_PARSE on malformed strings).
std::vector<Irrep> irreps_from_string(const char* s);
cgtp_plan_s* build_plan(const char* ix, const char* iy, const char* io, const char* mode,
                        cgtp_dtype dtype, cgtp_wkind wkind, cgtp_paths select = CGTP_PATHS_ALL,
                        bool collapse = false);
// Release a plan and what it owns (device tables, uvw sub-plan and mixing map).
void destroy_plan(cgtp_plan_s* plan);
// Real CG block by the ladder construction, [2l1+1][2l2+1][2l3+1], fp64.
std::vector<double> real_cg_ladder(int l1, int l2, int l3);
// Device tables of a plan on the current device (uploaded on first use).
const DevTables& plan_tables(cgtp_plan_s* plan);
void free_plan_tables(cgtp_plan_s* plan);

// Launches of one call that write disjoint memory, run side by side: f(i, st)
// is called for i in [0, n) with st = s for i = 0 and a library-owned stream
// of the current device (default priority) for the others; those streams
// first wait for the work queued on s before the call, and s waits for them
// afterwards, so the call stays ordered on s (and capturable: the fork and
// join are event waits). The side streams are created with a plan's first
// device tables on a device. fork = false runs every f(i, s) on s in order:
// the fork and join cost about 10-20 us, more than small calls gain. The
// fork, the launches and the join are queued under one lock (so calls from
// several host threads do not interleave their event records): f must only
// launch, never call side_run or plan_tables itself. Concurrent calls share
// the side streams, so their forked launches run one call after another.
constexpr int kSideStreams = 3;
constexpr double kSideMinBytes = 256.0 * (1 << 20);  // calls that move less stay on s
void side_run(hipStream_t s, int n, const std::function<void(int, hipStream_t)>& f, bool fork = true);
void side_streams_init();

inline size_t dtype_size(cgtp_dtype d) { return d == CGTP_F64 ? 8 : (d == CGTP_BF16 ? 2 : 4); }
inline size_t acc_size(cgtp_dtype d) { return d == CGTP_F64 ? 8 : 4; }

// Launchers (tp_kernels.hip).
void tp_forward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w,
                       void* out, hipStream_t stream);
void tp_backward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y,
                        const void* w, const void* g, void* dx, void* dy, void* dw, void* ws,
                        size_t ws_bytes, hipStream_t stream);
size_t tp_backward_ws_bytes(const cgtp_plan_s* plan, int64_t B);
// The same backward with the shared-weight partials in the library's
// file-scope device scratch (CGTP_NOALLOC_SCRATCH_BYTES per device).
constexpr size_t kNoallocScratchBytes = CGTP_NOALLOC_SCRATCH_BYTES;
void tp_backward_noalloc_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w,
                                const void* g, void* dx, void* dy, void* dw, hipStream_t stream);
// Double backward (double_backward.hip).
size_t tp_double_backward_ws_bytes(const cgtp_plan_s* plan, int64_t B);
void tp_double_backward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w,
                               const void* g, const void* gx, const void* gy, const void* gw, void* ddx,
                               void* ddy, void* ddw, void* ddg, void* ws, size_t ws_bytes, hipStream_t s);

// Fully connected (uvw) product (uvw_kernels.hip): fused forward on the matrix
// cores; backward composed through the workspace.
void uvw_forward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w, void* out,
                        hipStream_t s);
size_t uvw_backward_ws_bytes(const cgtp_plan_s* plan, int64_t B);
void uvw_backward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w, const void* g,
                         void* dx, void* dy, void* dw, void* ws, size_t ws_bytes, hipStream_t s);
void free_uvw_tables(const cgtp_plan_s* plan);
// uvu with y multiplicity > 1 (uvuv_kernels.hip): generic kernels.
void uvuv_forward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w, void* out,
                         hipStream_t s);
size_t uvuv_backward_ws_bytes(const cgtp_plan_s* plan, int64_t B);
void uvuv_backward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w, const void* g,
                          void* dx, void* dy, void* dw, void* ws, size_t ws_bytes, hipStream_t s);
void free_uvuv_tables(const cgtp_plan_s* plan);
// Last-layer maps of the radial convolution (radial_kernels.hip).
void free_radial_maps(const cgtp_plan_s* plan);

// Backward over generic rows: row r reads x row x_idx[r] (or r), grad_out row
// g_idx[r] (or r) times g_scale, y/w row r; writes grad_x row r either in the
// storage type (dx) or the accumulation type (dx_ws), grad_y row r, and grad_w
// row r (dw, storage type) or its accumulation-type partial (dw_ws).
struct TPBackwardRows {
  int64_t rows = 0;
  const void* x = nullptr;
  const int32_t* x_idx = nullptr;
  const void* y = nullptr;
  const void* w = nullptr;
  int64_t w_stride = 0;
  const void* g = nullptr;
  const int32_t* g_idx = nullptr;
  double g_scale = 1.0;
  void* dx = nullptr;
  void* dx_ws = nullptr;
  void* dy = nullptr;
  void* dw = nullptr;
  void* dw_ws = nullptr;
};
void tp_backward_rows(cgtp_plan_s* plan, const TPBackwardRows& r, hipStream_t stream);

// Zero the x blocks no path reads in rows [rows][dim_x] of element size es
// (the gradient of x there is zero).
void zero_unread_x(const cgtp_plan_s* plan, void* p, int64_t rows, size_t es, hipStream_t stream);
// Zero n elements of size es (a fill kernel, so the call may sit in a captured graph).
void zero_rows(void* p, int64_t n, size_t es, hipStream_t stream);

}  // namespace cgtp
