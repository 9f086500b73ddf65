// inst_8192.hip -- the twelve kernels of the 8192-element tile (see kernels.hpp).
#include "kernels.hpp"

DETK_EACH_KERNEL_OF_TILE(DETK_INSTANTIATE_KERNEL, 8192)
DETK_WIDE_KERNELS_OF_TILE(DETK_INSTANTIATE_KERNEL, 8192)
