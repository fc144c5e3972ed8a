// Instantiation of the bwd tensor-product kernel for storage type bf16, 1 channel(s) per lane.
#include "../tp_impl.hpp"

namespace cgtp {
template void tp_bwd_typed<bf16, 1>(const TPArgs&, int, int, hipStream_t);
}  // namespace cgtp
