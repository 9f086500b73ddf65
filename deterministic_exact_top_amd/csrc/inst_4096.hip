// inst_4096.hip -- the eight kernels of the 4096-element tile (see kernels.hpp).
#include "kernels.hpp"

DETK_EACH_KERNEL_OF_TILE(DETK_INSTANTIATE_KERNEL, 4096)
