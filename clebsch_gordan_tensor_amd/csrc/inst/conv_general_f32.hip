// Instantiation of the general convolution forward kernel for storage type float.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_fwd_general_typed<float>(const ConvArgs&, dim3, hipStream_t);
}  // namespace cgtp
