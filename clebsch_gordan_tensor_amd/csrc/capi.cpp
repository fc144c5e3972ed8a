// C ABI of libcgtp: argument checks, error translation, dispatch to launchers.
// Nothing here computes; every step of the path runs in the HIP kernels.
#include <cstring>
#include <exception>
#include <new>
#include <string>

#include "common.hpp"
#include "graph.hpp"
#include "linear.hpp"

namespace cgtp {

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }

template <typename F>
cgtp_status guarded(F&& f) {
  try {
    g_last_error.clear();
    f();
    return CGTP_OK;
  } catch (const Error& e) {
    g_last_error = e.msg;
    return e.code;
  } catch (const std::bad_alloc&) {
    g_last_error = "host allocation failed";
    return CGTP_ERR_ALLOC;
  } catch (const std::exception& e) {
    g_last_error = e.what();
    return CGTP_ERR_INVALID_ARG;
  } catch (...) {
    g_last_error = "unknown error";
    return CGTP_ERR_INVALID_ARG;
  }
}

inline void need(bool ok, const char* what) {
  if (!ok) throw Error{CGTP_ERR_INVALID_ARG, what};
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// uvw plans and uvu plans with y multiplicity > 1 run the tensor product's
// forward and backward only (their own kernels).
inline void need_plain_uvu(const cgtp_plan_s* plan, const char* what) {
  if (plan->mode != 0 || plan->max_ymul > 1)
    throw Error{CGTP_ERR_UNSUPPORTED, std::string(what) + ": only for uvu plans with y multiplicity 1"};
}

}  // namespace cgtp

using namespace cgtp;

extern "C" {

const char* cgtp_status_string(cgtp_status s) {
  switch (s) {
    case CGTP_OK: return "ok";
    case CGTP_ERR_INVALID_ARG: return "invalid argument";
    case CGTP_ERR_PARSE: return "irreps parse error";
    case CGTP_ERR_UNSUPPORTED: return "unsupported";
    case CGTP_ERR_INDEX: return "index out of range";
    case CGTP_ERR_WORKSPACE: return "workspace too small";
    case CGTP_ERR_HIP: return "HIP error";
    case CGTP_ERR_ALLOC: return "allocation failed";
  }
  return "unknown status";
}

const char* cgtp_last_error(void) { return g_last_error.c_str(); }

cgtp_status cgtp_plan_create(const char* irreps_x, const char* irreps_y, const char* irreps_out,
                             const char* mode, cgtp_dtype dtype, cgtp_wkind wkind, cgtp_plan* out) {
  return guarded([&] {
    need(out != nullptr, "out handle is NULL");
    *out = nullptr;
    *out = build_plan(irreps_x, irreps_y, irreps_out, mode, dtype, wkind);
  });
}

cgtp_status cgtp_plan_create_ex(const char* irreps_x, const char* irreps_y, const char* irreps_out,
                                const char* mode, cgtp_dtype dtype, cgtp_wkind wkind, cgtp_paths select,
                                int collapse, cgtp_plan* out) {
  return guarded([&] {
    need(out != nullptr, "out handle is NULL");
    *out = nullptr;
    *out = build_plan(irreps_x, irreps_y, irreps_out, mode, dtype, wkind, select, collapse != 0);
  });
}

cgtp_status cgtp_plan_outputs(cgtp_plan plan, int64_t* num_outputs, int32_t* host_table) {
  return guarded([&] {
    need(plan != nullptr, "NULL plan");
    if (num_outputs) *num_outputs = int64_t(plan->outputs.size());
    if (!host_table) return;
    for (size_t k = 0; k < plan->outputs.size(); ++k) {
      const OutBlock& o = plan->outputs[k];
      host_table[4 * k + 0] = o.l3;
      host_table[4 * k + 1] = o.p3;
      host_table[4 * k + 2] = o.mul;
      host_table[4 * k + 3] = o.out_off;
    }
  });
}

cgtp_status cgtp_plan_destroy(cgtp_plan plan) {
  return guarded([&] { destroy_plan(plan); });
}

cgtp_status cgtp_plan_query(cgtp_plan plan, int64_t* dim_x, int64_t* dim_y, int64_t* dim_out,
                            int64_t* num_paths, int64_t* w_numel) {
  return guarded([&] {
    need(plan != nullptr, "plan is NULL");
    if (dim_x) *dim_x = plan->dim_x;
    if (dim_y) *dim_y = plan->dim_y;
    if (dim_out) *dim_out = plan->dim_out;
    if (num_paths) *num_paths = int64_t(plan->paths.size());
    if (w_numel) *w_numel = plan->w_numel;
  });
}

cgtp_status cgtp_plan_paths(cgtp_plan plan, int32_t* t) {
  return guarded([&] {
    need(plan != nullptr && t != nullptr, "NULL argument");
    for (size_t i = 0; i < plan->paths.size(); ++i) {
      const PathInfo& p = plan->paths[i];
      const int32_t row[6] = {p.i1, p.i2, p.l1, p.l2, p.l3, p.p3};
      std::memcpy(t + 6 * i, row, sizeof(row));
    }
  });
}

cgtp_status cgtp_plan_cg(cgtp_plan plan, int32_t path, double* host_dense) {
  return guarded([&] {
    need(plan != nullptr && host_dense != nullptr, "NULL argument");
    need(path >= 0 && size_t(path) < plan->paths.size(), "path index out of range");
    const auto& C = plan->cg_dense[size_t(path)];
    std::memcpy(host_dense, C.data(), C.size() * sizeof(double));
  });
}

cgtp_status cgtp_tp_forward(cgtp_plan plan, int64_t B, const void* x, const void* y, const void* w,
                            void* out, void* stream) {
  return guarded([&] {
    need(plan != nullptr, "plan is NULL");
    need(B >= 0, "B < 0");
    if (B == 0) return;
    need(x && y && w && out, "NULL tensor with B > 0");
    if (plan->mode == 1)
      uvw_forward_launch(plan, B, x, y, w, out, as_stream(stream));
    else if (plan->max_ymul > 1)
      uvuv_forward_launch(plan, B, x, y, w, out, as_stream(stream));
    else
      tp_forward_launch(plan, B, x, y, w, out, as_stream(stream));
  });
}

cgtp_status cgtp_tp_backward(cgtp_plan plan, int64_t B, const void* x, const void* y, const void* w,
                             const void* grad_out, void* grad_x, void* grad_y, void* grad_w,
                             void* ws, size_t ws_bytes, void* stream) {
  return guarded([&] {
    need(plan != nullptr, "plan is NULL");
    need(B >= 0, "B < 0");
    if (B == 0) {
      // an empty batch still defines a (zero) gradient for shared weights
      if (grad_w && plan->wkind == CGTP_W_SHARED)
        zero_rows(grad_w, plan->w_numel, dtype_size(plan->dtype), as_stream(stream));
      return;
    }
    need(x && y && w && grad_out, "NULL input tensor with B > 0");
    if (!grad_x && !grad_y && !grad_w) return;
    if (plan->mode == 1)
      uvw_backward_launch(plan, B, x, y, w, grad_out, grad_x, grad_y, grad_w, ws, ws_bytes, as_stream(stream));
    else if (plan->max_ymul > 1)
      uvuv_backward_launch(plan, B, x, y, w, grad_out, grad_x, grad_y, grad_w, ws, ws_bytes, as_stream(stream));
    else
      tp_backward_launch(plan, B, x, y, w, grad_out, grad_x, grad_y, grad_w, ws, ws_bytes,
                         as_stream(stream));
  });
}

cgtp_status cgtp_tp_backward_noalloc(cgtp_plan plan, int64_t B, const void* x, const void* y, const void* w,
                                     const void* grad_out, void* grad_x, void* grad_y, void* grad_w,
                                     void* stream) {
  return guarded([&] {
    need(plan != nullptr, "plan is NULL");
    need(B >= 0, "B < 0");
    if (B == 0) {
      if (grad_w && plan->wkind == CGTP_W_SHARED)
        zero_rows(grad_w, plan->w_numel, dtype_size(plan->dtype), as_stream(stream));
      return;
    }
    need(x && y && w && grad_out, "NULL input tensor with B > 0");
    if (!grad_x && !grad_y && !grad_w) return;
    need_plain_uvu(plan, "tp_backward_noalloc");
    tp_backward_noalloc_launch(plan, B, x, y, w, grad_out, grad_x, grad_y, grad_w, as_stream(stream));
  });
}

cgtp_status cgtp_tp_double_backward(cgtp_plan plan, int64_t B, const void* x, const void* y, const void* w,
                                    const void* grad_out, const void* gg_x, const void* gg_y, const void* gg_w,
                                    void* out_x, void* out_y, void* out_w, void* out_grad_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  return guarded([&] {
    need(plan != nullptr, "NULL plan");
    need_plain_uvu(plan, "tp_double_backward");
    need(B >= 0, "B < 0");
    if (B == 0) {
      // shared weights still get their (zero) cotangent from an empty batch
      if (out_w && plan->wkind == CGTP_W_SHARED)
        zero_rows(out_w, plan->w_numel, dtype_size(plan->dtype), as_stream(stream));
      return;
    }
    need(x && y && w && grad_out, "NULL input tensor");
    tp_double_backward_launch(plan, B, x, y, w, grad_out, gg_x, gg_y, gg_w, out_x, out_y, out_w, out_grad_out, ws,
                              ws_bytes, as_stream(stream));
  });
}

cgtp_status cgtp_conv_double_backward(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                                      const void* w, double scale, const void* grad_out, const void* gg_x,
                                      const void* gg_sh, const void* gg_w, void* out_x, void* out_sh, void* out_w,
                                      void* out_grad_out, void* ws, size_t ws_bytes, void* stream) {
  return guarded([&] {
    need(plan != nullptr && graph != nullptr, "NULL plan or graph");
    need_plain_uvu(plan, "the convolution");
    if (plan->wkind != CGTP_W_PER_ROW)
      throw Error{CGTP_ERR_UNSUPPORTED, "the convolution needs per-edge weights (CGTP_W_PER_ROW)"};
    if (graph->N == 0) return;
    need(x && grad_out && (graph->E == 0 || (sh && w)), "NULL input tensor");
    conv_double_backward_launch(plan, graph, x, sh, w, scale, grad_out, gg_x, gg_sh, gg_w, out_x, out_sh, out_w,
                                out_grad_out, ws, ws_bytes, as_stream(stream));
  });
}

cgtp_status cgtp_workspace_size(cgtp_plan plan, cgtp_graph graph, int64_t B, int op, size_t* bytes) {
  return guarded([&] {
    need(plan != nullptr && bytes != nullptr, "NULL argument");
    if (op == CGTP_OP_TP_BACKWARD) {
      need(B >= 0, "B < 0");
      *bytes = plan->mode == 1       ? uvw_backward_ws_bytes(plan, B)
               : plan->max_ymul > 1 ? uvuv_backward_ws_bytes(plan, B)
                                    : tp_backward_ws_bytes(plan, B);
    } else if (op == CGTP_OP_CONV_FORWARD) {
      need(graph != nullptr, "graph is NULL");
      need_plain_uvu(plan, "the convolution");
      *bytes = conv_forward_ws_bytes(plan, graph);
    } else if (op == CGTP_OP_CONV_BACKWARD) {
      need(graph != nullptr, "graph is NULL");
      need_plain_uvu(plan, "the convolution");
      *bytes = conv_backward_ws_bytes(plan, graph);
    } else if (op == CGTP_OP_TP_DOUBLE_BACKWARD) {
      need(B >= 0, "B < 0");
      need_plain_uvu(plan, "tp_double_backward");
      *bytes = tp_double_backward_ws_bytes(plan, B);
    } else if (op == CGTP_OP_CONV_DOUBLE_BACKWARD) {
      need(graph != nullptr, "graph is NULL");
      need_plain_uvu(plan, "the convolution");
      *bytes = conv_double_backward_ws_bytes(plan, graph);
    } else {
      throw Error{CGTP_ERR_INVALID_ARG, "unknown op"};
    }
  });
}

cgtp_status cgtp_csr_from_coo(int64_t N, int64_t E, const int32_t* src, const int32_t* dst,
                              int32_t* row_ptr, int32_t* src_sorted, int32_t* perm, void* stream) {
  return guarded([&] {
    need(N >= 0 && E >= 0, "negative size");
    need(N < INT32_MAX && E < INT32_MAX, "graph too large for int32 indices");
    need(row_ptr != nullptr, "row_ptr is NULL");
    need(E == 0 || (src && dst && src_sorted && perm), "NULL edge array");
    csr_from_coo_launch(N, E, src, dst, row_ptr, src_sorted, perm, as_stream(stream));
  });
}

cgtp_status cgtp_graph_create(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src,
                              void* stream, cgtp_graph* out) {
  return guarded([&] {
    need(out != nullptr, "out handle is NULL");
    *out = nullptr;
    need(N >= 0 && E >= 0, "negative size");
    need(N < INT32_MAX && E < INT32_MAX, "graph too large for int32 indices");
    need(row_ptr != nullptr, "row_ptr is NULL");
    need(E == 0 || src != nullptr, "src is NULL");
    *out = graph_create(N, E, row_ptr, src, as_stream(stream));
  });
}

cgtp_status cgtp_graph_create_ex(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src,
                                 int32_t pad_node, void* stream, cgtp_graph* out) {
  return guarded([&] {
    need(out != nullptr, "out handle is NULL");
    *out = nullptr;
    need(N >= 0 && E >= 0, "negative size");
    need(N < INT32_MAX && E < INT32_MAX, "graph too large for int32 indices");
    need(row_ptr != nullptr, "row_ptr is NULL");
    need(E == 0 || src != nullptr, "src is NULL");
    *out = graph_create(N, E, row_ptr, src, as_stream(stream), pad_node);
  });
}

cgtp_status cgtp_graph_destroy(cgtp_graph graph) {
  return guarded([&] {
    if (graph) graph_destroy(graph);
  });
}

cgtp_status cgtp_graph_transpose(cgtp_graph graph, int32_t* col_ptr, int32_t* eid, void* stream) {
  return guarded([&] {
    need(graph != nullptr && col_ptr != nullptr, "NULL argument");
    need(graph->E == 0 || eid != nullptr, "eid is NULL");
    graph_transpose_copy(graph, col_ptr, eid, as_stream(stream));
  });
}

cgtp_status cgtp_conv_forward(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                              const void* w, double scale, void* out, void* stream) {
  return cgtp_conv_forward_ws(plan, graph, x, sh, w, scale, out, nullptr, 0, stream);
}

cgtp_status cgtp_conv_forward_ws(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                                 const void* w, double scale, void* out, void* ws, size_t ws_bytes,
                                 void* stream) {
  return guarded([&] {
    need(plan != nullptr && graph != nullptr, "NULL plan or graph");
    need_plain_uvu(plan, "the convolution");
    if (plan->wkind != CGTP_W_PER_ROW)
      throw Error{CGTP_ERR_UNSUPPORTED, "the convolution needs per-edge weights (CGTP_W_PER_ROW)"};
    if (graph->N == 0) return;
    need(out != nullptr, "out is NULL");
    need(graph->E == 0 || (x && sh && w), "NULL input tensor");
    if (ws) {
      const size_t nws = conv_forward_ws_bytes(plan, graph);
      if (ws_bytes < nws)
        throw Error{CGTP_ERR_WORKSPACE, "conv_forward needs " + std::to_string(nws) + " workspace bytes"};
      if (reinterpret_cast<uintptr_t>(ws) % 16 != 0)
        throw Error{CGTP_ERR_INVALID_ARG, "the workspace must be 16-byte aligned"};
    }
    conv_forward_launch(plan, graph, x, sh, w, scale, out, as_stream(stream), ws, ws_bytes);
  });
}

cgtp_status cgtp_conv_backward(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                               const void* w, double scale, const void* grad_out, void* grad_x,
                               void* grad_sh, void* grad_w, void* ws, size_t ws_bytes, void* stream) {
  return guarded([&] {
    need(plan != nullptr && graph != nullptr, "NULL plan or graph");
    need_plain_uvu(plan, "the convolution");
    if (plan->wkind != CGTP_W_PER_ROW)
      throw Error{CGTP_ERR_UNSUPPORTED, "the convolution needs per-edge weights (CGTP_W_PER_ROW)"};
    need(graph->E == 0 || (x && sh && w && grad_out), "NULL input tensor");
    conv_backward_launch(plan, graph, x, sh, w, scale, grad_out, grad_x, grad_sh, grad_w, ws,
                         ws_bytes, as_stream(stream));
  });
}

cgtp_status cgtp_conv_forward_radial(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                                     const void* h, int64_t hidden, const void* W2, double scale, void* out,
                                     void* stream) {
  return guarded([&] {
    need(plan != nullptr && graph != nullptr, "NULL plan or graph");
    need_plain_uvu(plan, "the convolution");
    if (plan->wkind != CGTP_W_PER_ROW)
      throw Error{CGTP_ERR_UNSUPPORTED, "the convolution needs per-edge weights (CGTP_W_PER_ROW)"};
    if (graph->N == 0) return;
    need(out != nullptr && W2 != nullptr, "NULL out or W2");
    need(graph->E == 0 || (x && sh && h), "NULL input tensor");
    conv_forward_radial_launch(plan, graph, x, sh, h, hidden, W2, scale, out, as_stream(stream));
  });
}

cgtp_status cgtp_conv_backward_radial(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                                      const void* h, int64_t hidden, const void* W2, double scale,
                                      const void* grad_out, void* grad_x, void* grad_sh, void* grad_h,
                                      void* grad_W2, void* ws, size_t ws_bytes, void* stream) {
  return guarded([&] {
    need(plan != nullptr && graph != nullptr, "NULL plan or graph");
    need_plain_uvu(plan, "the convolution");
    if (plan->wkind != CGTP_W_PER_ROW)
      throw Error{CGTP_ERR_UNSUPPORTED, "the convolution needs per-edge weights (CGTP_W_PER_ROW)"};
    need(W2 != nullptr && grad_out != nullptr, "NULL W2 or grad_out");
    need(graph->E == 0 || (x && sh && h), "NULL input tensor");
    conv_backward_radial_launch(plan, graph, x, sh, h, hidden, W2, scale, grad_out, grad_x, grad_sh, grad_h, grad_W2,
                                ws, ws_bytes, as_stream(stream));
  });
}

cgtp_status cgtp_conv_radial_workspace_size(cgtp_plan plan, cgtp_graph graph, int64_t hidden, size_t* bytes) {
  return guarded([&] {
    need(plan != nullptr && graph != nullptr && bytes != nullptr, "NULL argument");
    need(hidden > 0, "hidden <= 0");
    *bytes = conv_backward_radial_ws_bytes(plan, graph, hidden);
  });
}

cgtp_status cgtp_sh_forward(int lmax, cgtp_dtype dtype, int64_t n, const void* vec, void* sh,
                            void* stream) {
  return guarded([&] {
    need(n >= 0, "n < 0");
    if (lmax < 0 || lmax > kLmax) throw Error{CGTP_ERR_UNSUPPORTED, "lmax outside 0..CGTP_LMAX"};
    need(dtype == CGTP_F32 || dtype == CGTP_F64 || dtype == CGTP_BF16, "bad dtype");
    if (n == 0) return;
    need(vec && sh, "NULL tensor");
    sh_forward_launch(lmax, dtype, n, vec, sh, as_stream(stream));
  });
}

cgtp_status cgtp_sh_backward(int lmax, cgtp_dtype dtype, int64_t n, const void* vec,
                             const void* grad_sh, void* grad_vec, void* stream) {
  return guarded([&] {
    need(n >= 0, "n < 0");
    if (lmax < 0 || lmax > kLmax) throw Error{CGTP_ERR_UNSUPPORTED, "lmax outside 0..CGTP_LMAX"};
    need(dtype == CGTP_F32 || dtype == CGTP_F64 || dtype == CGTP_BF16, "bad dtype");
    if (n == 0) return;
    need(vec && grad_sh && grad_vec, "NULL tensor");
    sh_backward_launch(lmax, dtype, n, vec, grad_sh, grad_vec, as_stream(stream));
  });
}

cgtp_status cgtp_linear_create(const char* irreps_in, const char* irreps_out, cgtp_dtype dtype,
                               cgtp_linear* out) {
  return guarded([&] {
    need(out != nullptr, "NULL out");
    *out = nullptr;
    *out = build_linear(irreps_in, irreps_out, dtype);
  });
}

cgtp_status cgtp_linear_destroy(cgtp_linear lin) {
  return guarded([&] {
    if (!lin) return;
    free_linear_tables(lin);
    delete lin;
  });
}

cgtp_status cgtp_linear_query(cgtp_linear lin, int64_t* dim_in, int64_t* dim_out, int64_t* num_paths,
                              int64_t* w_numel) {
  return guarded([&] {
    need(lin != nullptr, "NULL linear");
    if (dim_in) *dim_in = lin->dim_in;
    if (dim_out) *dim_out = lin->dim_out;
    if (num_paths) *num_paths = int64_t(lin->paths.size());
    if (w_numel) *w_numel = lin->w_numel;
  });
}

cgtp_status cgtp_linear_paths(cgtp_linear lin, int32_t* t) {
  return guarded([&] {
    need(lin != nullptr && t != nullptr, "NULL argument");
    for (size_t k = 0; k < lin->paths.size(); ++k) {
      const auto& p = lin->paths[k];
      const int32_t row[5] = {p.i, p.o, p.l, p.mu, p.mv};
      std::memcpy(t + 5 * k, row, sizeof(row));
    }
  });
}

cgtp_status cgtp_linear_forward(cgtp_linear lin, int64_t B, const void* x, const void* w, void* out,
                                void* stream) {
  return guarded([&] {
    need(lin != nullptr, "NULL linear");
    need(B >= 0, "B < 0");
    if (B == 0 || lin->dim_out == 0) return;
    need(out && (lin->dim_in == 0 || x) && (lin->w_numel == 0 || w), "NULL tensor");
    linear_forward_launch(lin, B, x, w, out, as_stream(stream));
  });
}

cgtp_status cgtp_linear_backward(cgtp_linear lin, int64_t B, const void* x, const void* w,
                                 const void* grad_out, void* grad_x, void* grad_w, void* ws, size_t ws_bytes,
                                 void* stream) {
  return guarded([&] {
    need(lin != nullptr, "NULL linear");
    need(B >= 0, "B < 0");
    if (grad_x && (B == 0 || lin->dim_in == 0)) grad_x = nullptr;
    if (!grad_x && !grad_w) return;
    need(B == 0 || lin->dim_out == 0 || grad_out, "NULL grad_out");
    need(!grad_x || w, "NULL w");
    need(!grad_w || B == 0 || x, "NULL x");
    if (grad_w && linear_backward_ws_bytes(lin, B) > 0) need(ws != nullptr, "NULL workspace");
    linear_backward_launch(lin, B, x, w, grad_out, grad_x, grad_w, ws, ws_bytes, as_stream(stream));
  });
}

cgtp_status cgtp_linear_workspace_size(cgtp_linear lin, int64_t B, size_t* bytes) {
  return guarded([&] {
    need(lin != nullptr && bytes != nullptr, "NULL argument");
    need(B >= 0, "B < 0");
    *bytes = linear_backward_ws_bytes(lin, B);
  });
}

}  // extern "C"
