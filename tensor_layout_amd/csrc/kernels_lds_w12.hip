// kernels_lds_w12.hip -- tiled-transpose kernels for 1 and 2-byte elements.
#include "kernels_lds_impl.hpp"

TPL_LDS_WIDTH_INSTANCES(1)
TPL_LDS_WIDTH_INSTANCES(2)
