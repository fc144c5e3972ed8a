// Instantiation of the fused convolution forward kernels for storage type float.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_fwd_fused_typed<float>(const ConvArgs&, int, int, dim3, hipStream_t);
template int conv_fused_chunks<float>(int, int, bool);
}  // namespace cgtp
