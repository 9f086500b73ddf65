// inst_16384.hip -- the twelve kernels of the 16384-element tile (see kernels.hpp).
#include "kernels.hpp"

DETK_EACH_KERNEL_OF_TILE(DETK_INSTANTIATE_KERNEL, 16384)
DETK_WIDE_KERNELS_OF_TILE(DETK_INSTANTIATE_KERNEL, 16384)
