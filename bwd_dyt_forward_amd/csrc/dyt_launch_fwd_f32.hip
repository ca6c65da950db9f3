// dyt_launch_fwd_f32.hip - the forward kernel instances for float activations.
#include "dyt_launch_impl.hpp"

namespace dyt {
namespace host {
template bool launch_forward<float>(int, bool, bool, const Plan&, const Geo&, const FwdPtrs&, hipStream_t);
template bool launch_forward_flat<float>(int, bool, const Plan&, const FlatGeo&, const FwdPtrs&, hipStream_t);
}  // namespace host
}  // namespace dyt
