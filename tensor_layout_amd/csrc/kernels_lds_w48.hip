// kernels_lds_w48.hip -- tiled-transpose kernels for 4 and 8-byte elements.
#include "kernels_lds_impl.hpp"

TPL_LDS_WIDTH_INSTANCES(4)
TPL_LDS_WIDTH_INSTANCES(8)
