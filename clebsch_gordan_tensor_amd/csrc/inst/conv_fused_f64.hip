// Instantiation of the fused convolution forward kernels for storage type double.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_fwd_fused_typed<double>(const ConvArgs&, int, int, dim3, hipStream_t);
template int conv_fused_chunks<double>(int, int, bool);
}  // namespace cgtp
