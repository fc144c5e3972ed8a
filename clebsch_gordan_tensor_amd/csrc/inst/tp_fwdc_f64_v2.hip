// Instantiation of the collapsed-output forward tensor-product kernel for storage type double, 2 channel(s) per lane.
#include "../tp_impl.hpp"

namespace cgtp {
template void tp_fwd_collapsed_typed<double, 2>(const TPArgs&, int, hipStream_t);
}  // namespace cgtp
