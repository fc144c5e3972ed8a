// Instantiation of the fwd tensor-product kernel for storage type bf16, 4 channel(s) per lane.
#include "../tp_impl.hpp"

namespace cgtp {
template void tp_fwd_typed<bf16, 4>(const TPArgs&, int, int, hipStream_t);
}  // namespace cgtp
