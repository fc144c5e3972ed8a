// Instantiation of the fused convolution forward kernel for storage type double.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_fwd_fused_typed<double>(const ConvArgs&, dim3, hipStream_t);
}  // namespace cgtp
