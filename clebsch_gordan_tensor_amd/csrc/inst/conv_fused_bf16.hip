// Instantiation of the fused convolution forward kernels for storage type bf16.
#include "../conv_impl.hpp"

namespace cgtp {
template void conv_fwd_fused_typed<bf16>(const ConvArgs&, int, int, dim3, hipStream_t);
template int conv_fused_chunks<bf16>(int, int, bool);
}  // namespace cgtp
