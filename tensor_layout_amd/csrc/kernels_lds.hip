// kernels_lds.hip -- the tiled transpose through LDS: dispatch on the element
// width (the kernels are compiled in kernels_lds_w*.hip).
#include "lds.hpp"

namespace tpl {

template <int NB, bool BIG>
hipError_t launch_lds(const Plan& p, const uint8_t* src, uint8_t* dst, hipStream_t st) {
    LdsArgs a = p.lds;
    a.src = src;
    a.dst = dst;
    switch (p.w) {
    case 1: return launch_lds_width<1, NB, BIG>(p, a, st);
    case 2: return launch_lds_width<2, NB, BIG>(p, a, st);
    case 4: return launch_lds_width<4, NB, BIG>(p, a, st);
    case 8: return launch_lds_width<8, NB, BIG>(p, a, st);
    default: return launch_lds_width<16, NB, BIG>(p, a, st);
    }
}

TPL_LAUNCHER_INSTANCES(launch_lds)

}  // namespace tpl
