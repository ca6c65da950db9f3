// dyt_launch_fwd_f16.hip - the forward kernel instances for f16_t activations.
#include "dyt_launch_impl.hpp"

namespace dyt {
namespace host {
template bool launch_forward<f16_t>(int, bool, bool, const Plan&, const Geo&, const FwdPtrs&, hipStream_t);
template bool launch_forward_flat<f16_t>(int, bool, const Plan&, const FlatGeo&, const FwdPtrs&, hipStream_t);
}  // namespace host
}  // namespace dyt
