// dyt_launch_fwd_bf16.hip - the forward kernel instances for bf16_t activations.
#include "dyt_launch_impl.hpp"

namespace dyt {
namespace host {
template bool launch_forward<bf16_t>(int, bool, bool, const Plan&, const Geo&, const FwdPtrs&, hipStream_t);
template bool launch_forward_flat<bf16_t>(int, bool, const Plan&, const FlatGeo&, const FwdPtrs&, hipStream_t);
}  // namespace host
}  // namespace dyt
