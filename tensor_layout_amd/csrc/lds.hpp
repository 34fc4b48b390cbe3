// lds.hpp -- the tiled transpose's launcher for one element width (defined
// in kernels_lds_impl.hpp, instantiated in kernels_lds_w*.hip).
#pragma once

#include "device.hpp"

namespace tpl {

template <int W, int NB, bool BIG>
hipError_t launch_lds_width(const Plan& p, const LdsArgs& a, hipStream_t st);

}  // namespace tpl
