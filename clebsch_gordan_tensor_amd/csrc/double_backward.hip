// Double backward (the reverse mode of the backward) of the tensor product and
// the convolution, by composition of the forward and backward launches.
//
// The backward's outputs (the transposed maps of "E3J: An Efficient and
// Open-Source Backend for Euclidean Equivariant Operations on GPU and TPU",
// appendix E.1) are each linear in the other three tensors: with output
// cotangents (gx, gy, gw),
//   S = <gx, dx> + <gy, dy> + <gw, dw>
//     = <TP(gx, y, w) + TP(x, gy, w) + TP(x, y, gw), g>,
// so the cotangent of g is a sum of three forwards, and those of x, y, w are
// the backward of TP with one input replaced by its cotangent:
//   ddx = back(x, gy, w, g).dx + back(x, y, gw, g).dx
//   ddy = back(gx, y, w, g).dy + back(x, y, gw, g).dy
//   ddw = back(gx, y, w, g).dw + back(x, gy, w, g).dw.
// The convolution's backward is the same on gathered rows, so the same sums
// hold with the convolution's forward and backward. Partial results go to the
// workspace and are added in the fixed order of the sums above.
#include <algorithm>

#include "common.hpp"
#include "device_util.hpp"
#include "graph.hpp"

namespace cgtp {

namespace {

template <typename T>
__global__ __launch_bounds__(kBlock) void add_kernel(T* __restrict__ d, const T* __restrict__ s, int64_t n) {
  using A = typename AccOf<T>::type;
  const int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (i < n) from_acc(d[i], to_acc<A>(d[i]) + to_acc<A>(s[i]));
}

void add_into(void* d, const void* s, int64_t n, cgtp_dtype dt, hipStream_t st) {
  if (n == 0) return;
  const dim3 grid(unsigned((n + kBlock - 1) / kBlock));
  switch (dt) {
    case CGTP_F32:
      hipLaunchKernelGGL((add_kernel<float>), grid, dim3(kBlock), 0, st, static_cast<float*>(d),
                         static_cast<const float*>(s), n);
      break;
    case CGTP_BF16:
      hipLaunchKernelGGL((add_kernel<bf16>), grid, dim3(kBlock), 0, st, static_cast<bf16*>(d),
                         static_cast<const bf16*>(s), n);
      break;
    case CGTP_F64:
      hipLaunchKernelGGL((add_kernel<double>), grid, dim3(kBlock), 0, st, static_cast<double*>(d),
                         static_cast<const double*>(s), n);
      break;
  }
  CGTP_CHECK_HIP(hipGetLastError());
}

size_t up256(size_t b) { return (b + 255) / 256 * 256; }

// One output of the double backward: the first contribution is written in
// place, later ones go to a scratch buffer and are added.
struct Target {
  void* out;
  void* tmp;
  int64_t n;
  bool written = false;
  void* dest() const { return out ? (written ? tmp : out) : nullptr; }
  void done(cgtp_dtype dt, hipStream_t s) {
    if (!out) return;
    if (written) add_into(out, tmp, n, dt, s);
    written = true;
  }
  void finish(size_t es, hipStream_t s) {  // no contribution: the cotangent is zero
    if (out && !written) zero_rows(out, n, es, s);
  }
};

struct Sizes {
  size_t out, dx, dy, dw, inner;
  size_t total() const { return up256(out) + up256(dx) + up256(dy) + up256(dw) + inner; }
};

Sizes tp_sizes(const cgtp_plan_s* plan, int64_t B) {
  const size_t es = dtype_size(plan->dtype);
  const int64_t wrows = plan->wkind == CGTP_W_SHARED ? 1 : B;
  return Sizes{size_t(B) * plan->dim_out * es, size_t(B) * plan->dim_x * es, size_t(B) * plan->dim_y * es,
               size_t(wrows) * plan->w_numel * es, tp_backward_ws_bytes(plan, B)};
}

Sizes conv_sizes(const cgtp_plan_s* plan, const cgtp_graph_s* g) {
  const size_t es = dtype_size(plan->dtype);
  return Sizes{size_t(g->N) * plan->dim_out * es, size_t(g->N) * plan->dim_x * es, size_t(g->E) * plan->dim_y * es,
               size_t(g->E) * plan->w_numel * es, conv_backward_ws_bytes(plan, g)};
}

struct Carve {
  char *out, *dx, *dy, *dw, *inner;
};

Carve carve(void* ws, const Sizes& z) {
  char* p = static_cast<char*>(ws);
  Carve c{};
  c.out = p;
  p += up256(z.out);
  c.dx = p;
  p += up256(z.dx);
  c.dy = p;
  p += up256(z.dy);
  c.dw = p;
  p += up256(z.dw);
  c.inner = p;
  return c;
}

// The composition shared by both operations: fwd(a, b, c, out) and
// bwd(a, b, c, dx, dy, dw) are the forward and backward with the given inputs.
template <typename Fwd, typename Bwd>
void compose(const void* x, const void* y, const void* w, const void* gx, const void* gy, const void* gw,
             Target& tx, Target& ty, Target& tw, Target& tg, cgtp_dtype dt, hipStream_t s, Fwd fwd, Bwd bwd) {
  // cotangent of g: forwards with one input replaced by its cotangent
  if (tg.out) {
    if (gx) {
      fwd(gx, y, w, tg.dest());
      tg.done(dt, s);
    }
    if (gy) {
      fwd(x, gy, w, tg.dest());
      tg.done(dt, s);
    }
    if (gw) {
      fwd(x, y, gw, tg.dest());
      tg.done(dt, s);
    }
  }
  // back(gx, y, w, g): y and w parts
  if (gx && (ty.out || tw.out)) {
    bwd(gx, y, w, nullptr, ty.dest(), tw.dest());
    ty.done(dt, s);
    tw.done(dt, s);
  }
  // back(x, gy, w, g): x and w parts
  if (gy && (tx.out || tw.out)) {
    bwd(x, gy, w, tx.dest(), nullptr, tw.dest());
    tx.done(dt, s);
    tw.done(dt, s);
  }
  // back(x, y, gw, g): x and y parts
  if (gw && (tx.out || ty.out)) {
    bwd(x, y, gw, tx.dest(), ty.dest(), nullptr);
    tx.done(dt, s);
    ty.done(dt, s);
  }
  for (Target* t : {&tx, &ty, &tw, &tg}) t->finish(dtype_size(dt), s);
}

}  // namespace

size_t tp_double_backward_ws_bytes(const cgtp_plan_s* plan, int64_t B) { return tp_sizes(plan, B).total(); }

size_t conv_double_backward_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g) {
  return conv_sizes(plan, g).total();
}

void tp_double_backward_launch(cgtp_plan_s* plan, int64_t B, const void* x, const void* y, const void* w,
                               const void* g, const void* gx, const void* gy, const void* gw, void* ddx,
                               void* ddy, void* ddw, void* ddg, void* ws, size_t ws_bytes, hipStream_t s) {
  const Sizes z = tp_sizes(plan, B);
  if (!ws || ws_bytes < z.total())
    throw Error{CGTP_ERR_WORKSPACE, "tp_double_backward needs " + std::to_string(z.total()) + " workspace bytes"};
  const Carve c = carve(ws, z);
  const int64_t wrows = plan->wkind == CGTP_W_SHARED ? 1 : B;
  Target tx{ddx, c.dx, B * plan->dim_x}, ty{ddy, c.dy, B * plan->dim_y}, tw{ddw, c.dw, wrows * plan->w_numel},
      tg{ddg, c.out, B * plan->dim_out};
  compose(
      x, y, w, gx, gy, gw, tx, ty, tw, tg, plan->dtype, s,
      [&](const void* a, const void* b, const void* cw, void* out) { tp_forward_launch(plan, B, a, b, cw, out, s); },
      [&](const void* a, const void* b, const void* cw, void* dx, void* dy, void* dw) {
        tp_backward_launch(plan, B, a, b, cw, g, dx, dy, dw, c.inner, z.inner, s);
      });
}

void conv_double_backward_launch(cgtp_plan_s* plan, const cgtp_graph_s* gr, const void* x, const void* sh,
                                 const void* w, double scale, const void* g, const void* gx, const void* gsh,
                                 const void* gw, void* ddx, void* ddsh, void* ddw, void* ddg, void* ws,
                                 size_t ws_bytes, hipStream_t s) {
  const Sizes z = conv_sizes(plan, gr);
  if (!ws || ws_bytes < z.total())
    throw Error{CGTP_ERR_WORKSPACE, "conv_double_backward needs " + std::to_string(z.total()) + " workspace bytes"};
  const Carve c = carve(ws, z);
  Target tx{ddx, c.dx, gr->N * plan->dim_x}, ty{ddsh, c.dy, gr->E * plan->dim_y},
      tw{ddw, c.dw, gr->E * plan->w_numel}, tg{ddg, c.out, gr->N * plan->dim_out};
  compose(
      x, sh, w, gx, gsh, gw, tx, ty, tw, tg, plan->dtype, s,
      [&](const void* a, const void* b, const void* cw, void* out) {
        conv_forward_launch(plan, gr, a, b, cw, scale, out, s);
      },
      [&](const void* a, const void* b, const void* cw, void* dx, void* dy, void* dw) {
        conv_backward_launch(plan, gr, a, b, cw, scale, g, dx, dy, dw, c.inner, z.inner, s);
      });
}

}  // namespace cgtp
