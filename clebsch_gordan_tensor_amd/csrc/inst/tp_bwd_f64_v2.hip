// Instantiation of the bwd tensor-product kernel for storage type double, 2 channel(s) per lane.
#include "../tp_impl.hpp"

namespace cgtp {
template void tp_bwd_typed<double, 2>(const TPArgs&, int, int, hipStream_t);
}  // namespace cgtp
