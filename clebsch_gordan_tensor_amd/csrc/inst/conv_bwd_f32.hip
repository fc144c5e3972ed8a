// Instantiation of the fused convolution backward kernels for storage type float.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_bwd_fused_typed<float>(const ConvArgs&, const ConvBwdArgs&, int, int, dim3, size_t, hipStream_t);
template size_t conv_bwd_fused_lds<float>(int, int, int);
}  // namespace cgtp
