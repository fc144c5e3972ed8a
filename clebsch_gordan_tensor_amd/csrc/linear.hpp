// Equivariant linear map (channel mixing within irrep types): plan and launchers.
#pragma once

#include "common.hpp"

struct cgtp_linear_s {
  struct Path {
    int i, o, l, mu, mv;
    int64_t w_off;
  };
  std::vector<cgtp::Irrep> I, O;
  std::vector<int64_t> in_off, out_off;
  std::vector<Path> paths;  // input-major: every (i, o) with equal (l, parity)
  int64_t dim_in = 0, dim_out = 0, w_numel = 0;
  cgtp_dtype dtype = CGTP_F32;
};

namespace cgtp {

cgtp_linear_s* build_linear(const char* irreps_in, const char* irreps_out, cgtp_dtype dtype);
void linear_forward_launch(const cgtp_linear_s* lin, int64_t B, const void* x, const void* w, void* out,
                           hipStream_t s);
void linear_backward_launch(const cgtp_linear_s* lin, int64_t B, const void* x, const void* w, const void* g,
                            void* dx, void* dw, void* ws, size_t ws_bytes, hipStream_t s);
size_t linear_backward_ws_bytes(const cgtp_linear_s* lin, int64_t B);
void free_linear_tables(const cgtp_linear_s* lin);

}  // namespace cgtp
