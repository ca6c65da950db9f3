// dyt_launch_bwd_f32.hip - the backward pass-1 kernel instances for float activations.
#include "dyt_launch_impl.hpp"

namespace dyt {
namespace host {
template bool launch_backward<float>(int, bool, bool, const Plan&, const Geo&, const BwdPtrs&, hipStream_t);
}  // namespace host
}  // namespace dyt
