// Instantiation of the collapsed-output forward tensor-product kernel for storage type bf16, 2 channel(s) per lane.
#include "../tp_impl.hpp"

namespace cgtp {
template void tp_fwd_collapsed_typed<bf16, 2>(const TPArgs&, int, hipStream_t);
}  // namespace cgtp
