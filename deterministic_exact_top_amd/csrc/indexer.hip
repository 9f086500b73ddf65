// indexer.hip -- the lightning-indexer score producer on the matrix cores (gfx950).
//
// SGLang PR #31115, review thread: the DSA lightning-indexer score of a query against a
// key is a sum over the indexer heads of ReLU-ed per-head dot products, weighted per head:
//     score[b, t] = sum_h w[b, h] * max(0, q[b, h, :] . k[t, :]),   t < n_b,
// which puts every key whose heads all score non-positive on exactly 0.0 -- the plateau
// the top-k selector is built to resolve.  Per query this is a [H x D] x [D x n] product
// followed by a weighted ReLU reduction over H, so it runs on the MFMA units
// (v_mfma_f32_16x16x32_bf16: bfloat16 operands, float32 accumulation) with the ReLU and the
// head reduction fused into the epilogue: the per-head logits never leave registers, and
// only the [B, max_len] float32 scores are written.
//
// Work split: a 512-thread workgroup (8 waves) takes 16 query rows (2 per wave) and one
// chunk of keys (1024 .. 16384, chosen per launch), walked in blocks of kKeyBlock keys.  A
// block's keys are staged in LDS (padded rows, double-buffered; the loads run two blocks
// ahead, in registers, so each block's HBM/L2 latency hides behind two blocks of MFMAs)
// and shared by the 16 queries; each wave keeps its queries' q fragments in registers for
// the whole chunk.  Per block and wave: 2 queries x 4 key groups of 16 x D / 32 steps
// MFMAs.  (Two queries per wave leave 126 VGPRs, four waves per SIMD; four per wave needed
// 244, two waves per SIMD, and ran 2-3 % slower.)  MFMA operand layout (16x16x32): lane l
// holds A[l % 16][8 (l / 16) + j] and B[8 (l / 16) + j][l % 16] (j < 8), and
// C[4 (l / 16) + i][l % 16] (i < 4); here A = the query's heads x head dims, B = head dims
// x 16 keys, so C holds four heads of one key per lane.  The epilogue sums a lane's four
// heads (w_h * max(0, c_h)) for each of its query's four key groups, then reduces over the
// four 16-lane rows and transposes at once with three row swaps (v_permlane16_swap,
// v_permlane32_swap: no LDS traffic), leaving in row r the totals of key group r -- the 64
// consecutive keys of the block, one per lane, in a fixed order of additions, so the bits
// do not depend on the schedule.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "indexer.hpp"

namespace detk_ix {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = kHeadDim;               // head dimension (contraction length)
constexpr int kH = kHeads;                 // heads (the MFMA's 16 rows)
constexpr int kSteps = kD / 32;            // MFMA steps over the head dimension
constexpr int kQPerWave = 2;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQPerGroup = kQPerWave * kWaves;  // query rows per workgroup
constexpr int kKeyBlock = 64;              // keys per staged block (4 groups of 16)
constexpr int kGroups = kKeyBlock / 16;
// LDS bytes per staged key row: 32 bytes of padding keep the B-fragment reads free of bank
// conflicts (16 bytes left one 4-cycle conflict per read; none measured with 32)
constexpr int kRowBytes = kD * 2 + 32;
constexpr int kChunksPerThread = kKeyBlock * kD * 2 / 16 / kThreads;  // 16-byte loads per thread per block
static_assert(kH == 16, "one 16-row MFMA tile of heads");
static_assert(kD % 32 == 0 && kChunksPerThread * kThreads * 16 == kKeyBlock * kD * 2, "whole 16-byte loads");

constexpr int32_t kBufferWord3 = 0x00020000;  // raw buffer resource, gfx9-family data format

// max(0, x) on the bits: negative patterns become +0.0 (finite inputs assumed: a NaN logit
// has no defined place in the score).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

__device__ __forceinline__ int32_t row_len(const IxParams& p, int64_t b) {
    if (b >= p.B) return 0;
    const int32_t len = p.lengths ? p.lengths[b] : p.max_len;
    return min(max(len, 0), p.max_len);
}

__global__ __launch_bounds__(kThreads, 2) void indexer_kernel(IxParams p) {
    __shared__ __align__(16) unsigned char stage[2][kKeyBlock * kRowBytes];
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t group = (int64_t)blockIdx.x / p.chunks;
    const int chunk = (int)((int64_t)blockIdx.x % p.chunks);
    const int64_t q0 = group * kQPerGroup;

    // The workgroup's key range: its chunk, cut at the longest window of its rows.
    int32_t nmax = 0;
    for (int j = 0; j < kQPerGroup; ++j) nmax = max(nmax, row_len(p, q0 + j));
    const int32_t k_begin = chunk * p.chunk;
    const int32_t k_end = min(k_begin + p.chunk, nmax);
    if (k_begin >= k_end) return;  // uniform: no row of the group reaches this chunk

    // This wave's rows: q fragments (rows past the batch are zero) and head weights.
    int32_t nq[kQPerWave];
    int64_t qi[kQPerWave];
    bf16x8 a[kQPerWave][kSteps];
    f32x4 wv[kQPerWave];
#pragma unroll
    for (int j = 0; j < kQPerWave; ++j) {
        qi[j] = q0 + wave * kQPerWave + j;
        nq[j] = row_len(p, qi[j]);
        const bool live = qi[j] < p.B;
        const uint16_t* const qrow = p.q + (qi[j] * kH + (lane & 15)) * kD + 8 * (lane >> 4);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const uint4 v = live ? *reinterpret_cast<const uint4*>(qrow + 32 * s) : make_uint4(0, 0, 0, 0);
            a[j][s] = __builtin_bit_cast(bf16x8, v);
        }
        wv[j] = live ? *reinterpret_cast<const f32x4*>(p.w + qi[j] * kH + 4 * (lane >> 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Key blocks: 16-byte loads through a buffer resource over the key rows (rows past
    // n_keys read as zero, so a block never reads outside the keys).
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.keys), (short)0, p.n_keys * kD * 2, kBufferWord3);  // (host: < 2^31 bytes)
    auto load_block = [&](int32_t kb, uint4 (&dst)[kChunksPerThread]) {
#pragma unroll
        for (int i = 0; i < kChunksPerThread; ++i) {
            const int c = tid + kThreads * i;  // 16-byte chunk: row c / (kD / 8), column c % (kD / 8)
            const int row = c / (kD / 8), col = c % (kD / 8);
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(krs, (row * kD + col * 8) * 2, kb * kD * 2, 0);
            dst[i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    auto stage_block = [&](int buf, const uint4 (&src)[kChunksPerThread]) {
#pragma unroll
        for (int i = 0; i < kChunksPerThread; ++i) {
            const int c = tid + kThreads * i;
            const int row = c / (kD / 8), col = c % (kD / 8);
            *reinterpret_cast<uint4*>(stage[buf] + row * kRowBytes + col * 16) = src[i];
        }
    };

    // One block: MFMAs over the staged keys of `buf`, the epilogue, then the next block's
    // keys (in `next`, loaded a block earlier) staged into the other buffer.  `ahead`
    // receives the keys of the block after that, loaded while this block computes.
    auto block = [&](int32_t kb, int buf, uint4 (&next)[kChunksPerThread], uint4 (&ahead)[kChunksPerThread]) {
        const bool more = kb + kKeyBlock < k_end;        // uniform
        const bool more2 = kb + 2 * kKeyBlock < k_end;   // uniform
        if (more2) load_block(kb + 2 * kKeyBlock, ahead);  // (in flight during two blocks)

        f32x4 acc[kQPerWave][kGroups];
#pragma unroll
        for (int j = 0; j < kQPerWave; ++j)
#pragma unroll
            for (int g = 0; g < kGroups; ++g) acc[j][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                const bf16x8 bk = *reinterpret_cast<const bf16x8*>(stage[buf] + (16 * g + (lane & 15)) * kRowBytes +
                                                                   (4 * s + (lane >> 4)) * 16);
#pragma unroll
                for (int j = 0; j < kQPerWave; ++j)
                    acc[j][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j][s], bk, acc[j][g], 0, 0, 0);
            }
        }

        // Epilogue: lane l holds heads 4 (l / 16) .. + 3 of key 16 g + l % 16; each quarter of
        // 64 keys (groups 4 h .. 4 h + 3) is reduced and stored on its own.
#pragma unroll
        for (int j = 0; j < kQPerWave; ++j)
#pragma unroll
        for (int h = 0; h < kGroups / 4; ++h) {
            uint32_t part[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float x = wv[j][0] * relu(acc[j][4 * h + g][0]);
                x += wv[j][1] * relu(acc[j][4 * h + g][1]);
                x += wv[j][2] * relu(acc[j][4 * h + g][2]);
                x += wv[j][3] * relu(acc[j][4 * h + g][3]);
                part[g] = as_u(x);
            }
            // rows (0, 1) and (2, 3) exchange: even rows sum groups 0 and 2 over the pair,
            // odd rows groups 1 and 3; then rows (0, 1) and (2, 3) exchange halves: row r
            // holds the total of group r.
            const auto x01 = __builtin_amdgcn_permlane16_swap(part[0], part[1], false, false);
            const auto x23 = __builtin_amdgcn_permlane16_swap(part[2], part[3], false, false);
            const float s01 = as_f(x01[0]) + as_f(x01[1]);
            const float s23 = as_f(x23[0]) + as_f(x23[1]);
            const auto y = __builtin_amdgcn_permlane32_swap(as_u(s01), as_u(s23), false, false);
            const float v = as_f(y[0]) + as_f(y[1]);
            // lane l stores key kb + 64 h + l: group l / 16, column l % 16 (one 256-byte store)
            const int32_t t = kb + 64 * h + lane;
            if (t < nq[j]) p.out[qi[j] * p.max_len + t] = v;
        }
        if (more) stage_block(buf ^ 1, next);  // (nobody reads that buffer until the barrier)
        __syncthreads();
    };

    uint4 kA[kChunksPerThread], kB[kChunksPerThread];
    load_block(k_begin, kA);
    stage_block(0, kA);
    if (k_begin + kKeyBlock < k_end) load_block(k_begin + kKeyBlock, kA);
    __syncthreads();
    // (two blocks per turn, so the two register sets keep fixed names)
    for (int32_t kb = k_begin; kb < k_end; kb += 2 * kKeyBlock) {
        block(kb, 0, kA, kB);
        if (kb + kKeyBlock < k_end) block(kb + kKeyBlock, 1, kB, kA);
    }
}

hipError_t launch_indexer(IxParams p, int cus, hipStream_t stream) {
    const int64_t groups = ((int64_t)p.B + kQPerGroup - 1) / kQPerGroup;
    // Larger chunks measured faster on the 8192 x 16384 prefill shape (1024: 467 us, 2048:
    // 436, 4096: 423-439, 8192: 423-430, 16384: 410-414), as long as the grid fills the GPU.
    int32_t chunk = kMaxChunk;
    while (chunk > kMinChunk && groups * (((int64_t)p.max_len + chunk - 1) / chunk) < 2 * (int64_t)cus) chunk >>= 1;
    p.chunk = chunk;
    p.chunks = (int32_t)(((int64_t)p.max_len + chunk - 1) / chunk);
    const int64_t grid = groups * p.chunks;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(indexer_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace detk_ix
