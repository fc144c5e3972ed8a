// Instantiation of the fused convolution forward kernel for storage type bf16.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_fwd_fused_typed<bf16>(const ConvArgs&, dim3, hipStream_t);
}  // namespace cgtp
