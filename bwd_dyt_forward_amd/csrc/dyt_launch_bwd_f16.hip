// dyt_launch_bwd_f16.hip - the backward pass-1 kernel instances for f16_t activations.
#include "dyt_launch_impl.hpp"

namespace dyt {
namespace host {
template bool launch_backward<f16_t>(int, bool, bool, const Plan&, const Geo&, const BwdPtrs&, hipStream_t);
}  // namespace host
}  // namespace dyt
