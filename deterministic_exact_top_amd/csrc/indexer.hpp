// indexer.hpp -- the lightning-indexer score producer's launch interface (indexer.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detk_ix {

constexpr int kHeads = 16;     // indexer heads per query
constexpr int kHeadDim = 128;  // head dimension
constexpr int kChunk = 2048;   // keys per workgroup chunk

struct IxParams {
    const uint16_t* q;        // bfloat16 bits, [B][kHeads][kHeadDim]
    const float* w;           // [B][kHeads]
    const uint16_t* keys;     // bfloat16 bits, [n_keys][kHeadDim]
    const int32_t* lengths;   // nullable: every window max_len keys
    int32_t B;
    int32_t max_len;          // <= n_keys
    int32_t n_keys;
    int32_t chunks;           // ceil(max_len / kChunk)
    float* out;               // [B][max_len]; row b's first n_b entries written
};

hipError_t launch_indexer(const IxParams& p, hipStream_t stream);

}  // namespace detk_ix
