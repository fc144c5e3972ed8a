// Instantiation of the general convolution forward kernel for storage type bf16.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_fwd_general_typed<bf16>(const ConvArgs&, dim3, hipStream_t);
}  // namespace cgtp
