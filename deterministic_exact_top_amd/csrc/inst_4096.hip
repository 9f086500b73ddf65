// inst_4096.hip -- the twelve kernels of the 4096-element tile (see kernels.hpp).
#include "kernels.hpp"

DETK_EACH_KERNEL_OF_TILE(DETK_INSTANTIATE_KERNEL, 4096)
DETK_WIDE_KERNELS_OF_TILE(DETK_INSTANTIATE_KERNEL, 4096)
