// Instantiation of the fused convolution backward kernels for storage type double.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_bwd_fused_typed<double>(const ConvArgs&, const ConvBwdArgs&, int, int, dim3, size_t, hipStream_t);
template size_t conv_bwd_fused_lds<double>(int, int, int);
}  // namespace cgtp
