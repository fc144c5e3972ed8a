// Instantiation of the fwd tensor-product kernel for storage type float, 1 channel(s) per lane.
#include "../tp_impl.hpp"

namespace cgtp {
template void tp_fwd_typed<float, 1>(const TPArgs&, int, int, hipStream_t);
}  // namespace cgtp
