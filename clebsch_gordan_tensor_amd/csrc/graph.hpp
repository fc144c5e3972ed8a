// Graph handle, convolution and harmonics launchers.
#pragma once

#include "common.hpp"

struct cgtp_graph_s {
  int64_t N = 0, E = 0;
  const int32_t* row_ptr = nullptr;  // caller-owned CSR by destination
  const int32_t* src = nullptr;
  int32_t* col_ptr = nullptr;  // owned: transpose (edges grouped by source)
  int32_t* eid = nullptr;      // CSR position of each source-ordered edge
  int32_t* dst = nullptr;      // owned: destination of each CSR edge
  int32_t* order = nullptr;    // owned: receiver schedule, a permutation of [0, N)
  int device = 0;
  // padding: edges whose destination is the padding node (the CSR range
  // [pad_e0, pad_e1)) contribute nothing and are left out of the transpose
  int32_t pad = -1;
  int64_t pad_e0 = 0, pad_e1 = 0;
  int64_t E_t() const { return E - (pad_e1 - pad_e0); }  // edges in the transpose
};

namespace cgtp {

void csr_from_coo_launch(int64_t N, int64_t E, const int32_t* src, const int32_t* dst,
                         int32_t* row_ptr, int32_t* src_sorted, int32_t* perm, hipStream_t s);
cgtp_graph_s* graph_create(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src,
                           hipStream_t s, int32_t pad = -1);
void graph_destroy(cgtp_graph_s* g);
void graph_transpose_copy(const cgtp_graph_s* g, int32_t* col_ptr, int32_t* eid, hipStream_t s);

// ws (nullable, conv_forward_ws_bytes): with collapsed outputs in a storage
// type narrower than the accumulation type, the x blocks add into a running
// sum there, rounded to the output once at the end.
void conv_forward_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh,
                         const void* w, double scale, void* out, hipStream_t s, void* ws = nullptr,
                         size_t ws_bytes = 0);
size_t conv_forward_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g);
void conv_backward_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh,
                          const void* w, double scale, const void* grad_out, void* grad_x,
                          void* grad_sh, void* grad_w, void* ws, size_t ws_bytes, hipStream_t s);
size_t conv_backward_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g);
// The part of it that grad_x needs (per-edge partials); the rest lets the
// x blocks' launches run side by side.
size_t conv_backward_partials_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g);
size_t conv_double_backward_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g);
void conv_double_backward_launch(cgtp_plan_s* plan, const cgtp_graph_s* gr, const void* x, const void* sh,
                                 const void* w, double scale, const void* g, const void* gx, const void* gsh,
                                 const void* gw, void* ddx, void* ddsh, void* ddw, void* ddg, void* ws,
                                 size_t ws_bytes, hipStream_t s);

// Convolution with the radial network's last layer joined (radial_kernels.hip):
// w = h W2 formed on the matrix cores inside the forward; the backward is
// composed through the workspace.
void conv_forward_radial_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh, const void* h,
                                int64_t H, const void* W2, double scale, void* out, hipStream_t s);
size_t conv_backward_radial_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g, int64_t H);
void conv_backward_radial_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh,
                                 const void* h, int64_t H, const void* W2, double scale, const void* grad_out,
                                 void* grad_x, void* grad_sh, void* grad_h, void* grad_W2, void* ws, size_t ws_bytes,
                                 hipStream_t s);

void sh_forward_launch(int lmax, cgtp_dtype dtype, int64_t n, const void* vec, void* sh, hipStream_t s);
void sh_backward_launch(int lmax, cgtp_dtype dtype, int64_t n, const void* vec, const void* grad_sh,
                        void* grad_vec, hipStream_t s);

// Exclusive prefix sum of counts[0..n) into out[0..n] (out[n] = total), int32.
void exclusive_scan_i32(const int32_t* counts, int32_t* out, int64_t n, hipStream_t s);

}  // namespace cgtp
