// indexer.hpp -- the lightning-indexer score producer's launch interface (indexer.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detk_ix {

constexpr int kHeads = 16;     // indexer heads per query
constexpr int kHeadDim = 128;  // head dimension
constexpr int kMinChunk = 1024;   // keys per workgroup chunk: a power of two in [kMinChunk,
constexpr int kMaxChunk = 16384;  //   kMaxChunk], chosen on the host (launch_indexer)

struct IxParams {
    const uint16_t* q;        // bfloat16 bits, [B][kHeads][kHeadDim]
    const float* w;           // [B][kHeads]
    const uint16_t* keys;     // bfloat16 bits, [n_keys][kHeadDim]
    const int32_t* lengths;   // nullable: every window max_len keys
    int32_t B;
    int32_t max_len;          // <= n_keys
    int32_t n_keys;
    int32_t chunk;            // keys per workgroup chunk
    int32_t chunks;           // ceil(max_len / chunk)
    float* out;               // [B][max_len]; row b's first n_b entries written
};

// Chooses p.chunk / p.chunks (the largest chunk that still gives at least 2 workgroups per
// CU, so long rows of big batches pay a workgroup's q-fragment loads once per 16K keys and
// small batches still spread over the GPU), then launches.
hipError_t launch_indexer(IxParams p, int cus, hipStream_t stream);

}  // namespace detk_ix
