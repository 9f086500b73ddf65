// kernels.hpp -- the kernel instantiations the library launches: the tile shapes, and an
// explicit instantiation declaration for each (tile, k capacity, launch kind, score width).
// Each inst_<tile>.hip instantiates one tile size's eight kernels, so the translation
// units compile in parallel; the host code (detk_api.hip) launches them through these
// declarations.
#pragma once

#include "topk_device.hpp"

namespace detk {

// Workgroup tile shapes (elements = threads x elements per lane).  Tiles keep the row in
// VGPRs; MINW is the waves per SIMD their register allocation must allow.
//   one workgroup per row (rows up to 32768): 4096 = 256 x 16, 8192 = 512 x 16,
//     16384 = 512 x 32 (four rows per CU), 32768 = 1024 x 32
//   rows split over workgroups: 4096 = 256 x 16, 8192 = 1024 x 8, 16384 = 1024 x 16
//     (default), 32768 = 1024 x 32; 1024 threads wherever the tile allows, for the
//     last arriving workgroup, which orders the whole row's candidates
//   one workgroup per row in a small batch (WIDE: no more rows than CUs, so no CU runs a
//     second row and nothing is gained from packing several per CU): 1024 threads for
//     every tile -- 4096 = 1024 x 4, 8192 = 1024 x 8, 16384 = 1024 x 16, 32768 as above --
//     so each of the row's serial phases is a quarter or half as long
constexpr int kSingleMaxLen = 32768;
constexpr int kSplitTile = 16384;

template <int TILE, bool MULTI, bool WIDE = false> struct Shape;
template <> struct Shape<4096, false> { static constexpr int NT = 256, EPT = 16, MINW = 2; };
template <> struct Shape<8192, false> { static constexpr int NT = 512, EPT = 16, MINW = 4; };
template <> struct Shape<16384, false> { static constexpr int NT = 512, EPT = 32, MINW = 8; };
template <> struct Shape<32768, false> { static constexpr int NT = 1024, EPT = 32, MINW = 4; };
template <> struct Shape<4096, true> { static constexpr int NT = 256, EPT = 16, MINW = 2; };
template <> struct Shape<8192, true> { static constexpr int NT = 1024, EPT = 8, MINW = 4; };
template <> struct Shape<16384, true> { static constexpr int NT = 1024, EPT = 16, MINW = 4; };
template <> struct Shape<32768, true> { static constexpr int NT = 1024, EPT = 32, MINW = 4; };
template <> struct Shape<4096, false, true> { static constexpr int NT = 1024, EPT = 4, MINW = 4; };
template <> struct Shape<8192, false, true> { static constexpr int NT = 1024, EPT = 8, MINW = 4; };
template <> struct Shape<16384, false, true> { static constexpr int NT = 1024, EPT = 16, MINW = 4; };
template <> struct Shape<32768, false, true> : Shape<32768, false> {};

// Waves per SIMD a kernel's registers must allow: the shape's, except where the LDS of the
// k <= 4096 layouts already limits a CU to two 512-thread workgroups (4 waves per SIMD), so a
// tighter register cap would only spill.
template <int TILE, int KMAX, bool MULTI, bool WIDE = false>
constexpr int min_waves() {
    return (!MULTI && !WIDE && TILE == 16384 && KMAX == 4096) ? 4 : Shape<TILE, MULTI, WIDE>::MINW;
}


}  // namespace detk

// One kernel: (tile, k capacity, rows split over workgroups, small-batch shape, bytes per
// score).
#define DETK_KERNEL(TILE, KMAX, MULTI, WIDE, VB)                                                              \
    detk::topk_ragged_kernel<detk::Shape<TILE, MULTI, WIDE>::NT, detk::Shape<TILE, MULTI, WIDE>::EPT, KMAX,    \
                             MULTI, detk::min_waves<TILE, KMAX, MULTI, WIDE>(), VB>
#define DETK_EACH_KERNEL_OF_TILE(X, TILE)                                                                     \
    X(TILE, 2048, false, false, 4) X(TILE, 4096, false, false, 4) X(TILE, 2048, true, false, 4)               \
    X(TILE, 4096, true, false, 4) X(TILE, 2048, false, false, 2) X(TILE, 4096, false, false, 2)               \
    X(TILE, 2048, true, false, 2) X(TILE, 4096, true, false, 2)
// (the 32768-element tile's small-batch shape is its usual one)
#define DETK_WIDE_KERNELS_OF_TILE(X, TILE)                                                                    \
    X(TILE, 2048, false, true, 4) X(TILE, 4096, false, true, 4) X(TILE, 2048, false, true, 2)                 \
    X(TILE, 4096, false, true, 2)
#define DETK_EXTERN_KERNEL(TILE, KMAX, MULTI, WIDE, VB)                                                       \
    extern template __global__ void DETK_KERNEL(TILE, KMAX, MULTI, WIDE, VB)(detk::Params);
#define DETK_INSTANTIATE_KERNEL(TILE, KMAX, MULTI, WIDE, VB)                                                  \
    template __global__ void DETK_KERNEL(TILE, KMAX, MULTI, WIDE, VB)(detk::Params);

DETK_EACH_KERNEL_OF_TILE(DETK_EXTERN_KERNEL, 4096)
DETK_EACH_KERNEL_OF_TILE(DETK_EXTERN_KERNEL, 8192)
DETK_EACH_KERNEL_OF_TILE(DETK_EXTERN_KERNEL, 16384)
DETK_EACH_KERNEL_OF_TILE(DETK_EXTERN_KERNEL, 32768)
DETK_WIDE_KERNELS_OF_TILE(DETK_EXTERN_KERNEL, 4096)
DETK_WIDE_KERNELS_OF_TILE(DETK_EXTERN_KERNEL, 8192)
DETK_WIDE_KERNELS_OF_TILE(DETK_EXTERN_KERNEL, 16384)
