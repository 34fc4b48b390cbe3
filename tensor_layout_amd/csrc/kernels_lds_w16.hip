// kernels_lds_w16.hip -- tiled-transpose kernels for 16-byte elements.
#include "kernels_lds_impl.hpp"

TPL_LDS_WIDTH_INSTANCES(16)
