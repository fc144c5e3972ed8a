// Instantiation of the fused convolution backward kernels for storage type bf16.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_bwd_fused_typed<bf16>(const ConvArgs&, const ConvBwdArgs&, int, int, dim3, size_t, hipStream_t);
template size_t conv_bwd_fused_lds<bf16>(int, int, int);
}  // namespace cgtp
