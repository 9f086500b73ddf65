// inst_32768.hip -- the eight kernels of the 32768-element tile (see kernels.hpp).
#include "kernels.hpp"

DETK_EACH_KERNEL_OF_TILE(DETK_INSTANTIATE_KERNEL, 32768)
