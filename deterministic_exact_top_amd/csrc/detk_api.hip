// detk_api.hip -- host side of the C ABI declared in include/detk.h.
//
// Validates arguments on the host (nothing is launched on an error), picks the
// launch shape from host-known sizes only (B, k, max_len, device properties) and
// enqueues the kernels on the caller's stream.  No allocation, no synchronisation,
// no device readback: a call can be captured into a HIP graph.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string.h>

#include "../../include/detk.h"
#include "topk_device.hpp"

namespace {

using detk::Params;
using detk::SmemAll;

// Workgroup tile shapes (elements = threads x elements per lane).  Tiles keep the row in
// VGPRs; MINW is the waves per SIMD their register allocation must allow.
//   one workgroup per row: 4096 = 256 x 16, 8192 = 512 x 16, 16384 = 512 x 32,
//                          32768 = 1024 x 32
//   several per row:       4096 = 256 x 16, 8192 = 512 x 16, 16384 = 512 x 32,
//                          32768 = 1024 x 32
constexpr int kSingleMaxLen = 32768;

template <int TILE> struct Shape;
template <> struct Shape<4096> { static constexpr int NT = 256, EPT = 16, MINW = 2, MINW_MULTI = 2; };
template <> struct Shape<8192> { static constexpr int NT = 512, EPT = 16, MINW = 4, MINW_MULTI = 4; };
template <> struct Shape<16384> { static constexpr int NT = 512, EPT = 32, MINW = 8, MINW_MULTI = 4; };
template <> struct Shape<32768> { static constexpr int NT = 1024, EPT = 32, MINW = 4, MINW_MULTI = 4; };

template <int TILE, bool MULTI>
constexpr int min_waves() { return MULTI ? Shape<TILE>::MINW_MULTI : Shape<TILE>::MINW; }

template <int TILE, int KMAX, bool MULTI>
const void* kernel_ptr() {
    using S = Shape<TILE>;
    return reinterpret_cast<const void*>(&detk::topk_ragged_kernel<S::NT, S::EPT, KMAX, MULTI, min_waves<TILE, MULTI>()>);
}

template <int TILE, int KMAX, bool MULTI>
constexpr size_t smem_bytes() {
    return sizeof(SmemAll<Shape<TILE>::NT, Shape<TILE>::EPT, KMAX, MULTI>);
}

struct DeviceInfo {
    bool init = false;
    bool gfx950 = false;
    int cus = 0;
    size_t max_lds = 0;
    int multi_occ[4][2] = {};   // [tile index][kmax index] co-resident workgroups per CU
};

std::mutex g_mu;
DeviceInfo g_dev[64];
int g_force_path = 0;       // 0 auto, 1 single, 2 multi
int g_stage_cap = -1;       // -1 default
int g_multi_tile = 0;       // 0 default
int g_fast = 1;             // 0 off, 1 on, 2 on with a pivot that always misses

template <int TILE, int KMAX, bool MULTI>
hipError_t prepare_kernel() {
    return hipFuncSetAttribute(kernel_ptr<TILE, KMAX, MULTI>(), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)smem_bytes<TILE, KMAX, MULTI>());
}

template <int TILE, int KMAX, bool MULTI>
int occupancy() {
    if (prepare_kernel<TILE, KMAX, MULTI>() != hipSuccess) return 0;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel_ptr<TILE, KMAX, MULTI>(), Shape<TILE>::NT,
                                                     smem_bytes<TILE, KMAX, MULTI>()) != hipSuccess)
        return 0;
    return blocks;
}
template <int TILE, int KMAX>
int multi_occupancy() { return occupancy<TILE, KMAX, true>(); }

template <int TILE>
void prepare_both(hipError_t* e) {
    hipError_t r;
    if ((r = prepare_kernel<TILE, 2048, false>()) != hipSuccess) *e = r;
    if ((r = prepare_kernel<TILE, 4096, false>()) != hipSuccess) *e = r;
}

int device_info(int device, DeviceInfo* out) {
    if (device < 0 || device >= 64) return DETK_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo& d = g_dev[device];
    if (!d.init) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return DETK_ERR_HIP;
        if (cur != device && hipSetDevice(device) != hipSuccess) return DETK_ERR_HIP;
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, device);
        if (e == hipSuccess) {
            d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            d.cus = prop.multiProcessorCount;
            d.max_lds = prop.sharedMemPerBlock;
            d.multi_occ[0][0] = multi_occupancy<4096, 2048>();
            d.multi_occ[0][1] = multi_occupancy<4096, 4096>();
            d.multi_occ[1][0] = multi_occupancy<8192, 2048>();
            d.multi_occ[1][1] = multi_occupancy<8192, 4096>();
            d.multi_occ[2][0] = multi_occupancy<16384, 2048>();
            d.multi_occ[2][1] = multi_occupancy<16384, 4096>();
            d.multi_occ[3][0] = multi_occupancy<32768, 2048>();
            d.multi_occ[3][1] = multi_occupancy<32768, 4096>();
            prepare_both<4096>(&e);
            prepare_both<8192>(&e);
            prepare_both<16384>(&e);
            prepare_both<32768>(&e);
        }
        if (cur != device) (void)hipSetDevice(cur);
        if (e != hipSuccess) return DETK_ERR_HIP;
        d.init = true;
    }
    *out = d;
    return DETK_OK;
}

struct Plan {
    bool multi = false;
    int tile = 0;         // elements per workgroup tile
    int kmax = 2048;
    int tiles_per_row = 1;
    int grid = 0;
    size_t lds = 0;
    size_t ws_bytes = 0;
    // workspace layout (bytes from the start)
    size_t off_zero = 0, n_zero_words = 0, off_ecnt = 0, off_stage = 0, off_cand = 0;
};

template <bool MULTI>
size_t lds_bytes_t(int tile, int kmax) {
    const bool k2 = kmax == 2048;
    switch (tile) {
    case 4096: return k2 ? smem_bytes<4096, 2048, MULTI>() : smem_bytes<4096, 4096, MULTI>();
    case 8192: return k2 ? smem_bytes<8192, 2048, MULTI>() : smem_bytes<8192, 4096, MULTI>();
    case 16384: return k2 ? smem_bytes<16384, 2048, MULTI>() : smem_bytes<16384, 4096, MULTI>();
    default: return k2 ? smem_bytes<32768, 2048, MULTI>() : smem_bytes<32768, 4096, MULTI>();
    }
}
size_t lds_bytes(int tile, int kmax, bool multi) { return multi ? lds_bytes_t<true>(tile, kmax) : lds_bytes_t<false>(tile, kmax); }

int tile_index(int tile) { return tile == 4096 ? 0 : tile == 8192 ? 1 : tile == 16384 ? 2 : 3; }

// Decide the launch shape from host-known sizes only.
int make_plan(const DeviceInfo& dev, int B, int k, int32_t max_len, Plan* pl) {
    if (B < 0 || k < 1 || max_len < 0) return DETK_ERR_INVALID_ARG;
    if (k > DETK_MAX_K) return DETK_ERR_UNSUPPORTED;
    if (!dev.gfx950) return DETK_ERR_UNSUPPORTED;
    pl->kmax = k <= 2048 ? 2048 : 4096;
    const int ki = pl->kmax == 2048 ? 0 : 1;

    bool multi;
    if (g_force_path == 1) {
        if (max_len > kSingleMaxLen) return DETK_ERR_UNSUPPORTED;
        multi = false;
    } else if (g_force_path == 2) {
        multi = true;
    } else {
        // One workgroup per row whenever the row fits one tile (splitting a row costs row
        // barriers, which outweigh the extra parallelism even for small batches).
        multi = max_len > kSingleMaxLen;
    }
    pl->multi = multi;
    if (!multi) {
        pl->tile = max_len <= 4096 ? 4096 : max_len <= 8192 ? 8192 : max_len <= 16384 ? 16384 : 32768;
        pl->tiles_per_row = 1;
        pl->grid = B;  // one workgroup per row: the dispatcher balances rows of unequal length
        pl->ws_bytes = 0;
    } else {
        pl->tile = g_multi_tile ? g_multi_tile : 32768;  // fewest tiles per row: fewest barrier arrivals
        const int64_t tpr = max_len == 0 ? 1 : ((int64_t)max_len + pl->tile - 1) / pl->tile;
        const int occ = dev.multi_occ[tile_index(pl->tile)][ki];
        const int64_t capacity = (int64_t)occ * dev.cus;
        if (occ <= 0 || tpr > capacity) return DETK_ERR_UNSUPPORTED;
        pl->tiles_per_row = (int)tpr;
        const int64_t items = (int64_t)B * tpr;
        const int64_t rows_resident = capacity / tpr;
        int64_t grid = rows_resident * tpr;
        if (grid > items) grid = items;
        pl->grid = (int)grid;
        pl->n_zero_words = 1 + (size_t)B * detk::kRowZeroWords;
        pl->off_zero = 0;
        size_t off = pl->n_zero_words * 4;
        off = (off + 255) & ~(size_t)255;
        pl->off_ecnt = off;
        off += (size_t)B * (size_t)tpr * 4;
        off = (off + 255) & ~(size_t)255;
        pl->off_stage = off;
        off += (size_t)B * (size_t)k * 8;
        off = (off + 255) & ~(size_t)255;
        pl->off_cand = off;
        off += (size_t)B * (size_t)(pl->kmax == 2048 ? detk::cand_cap<2048>() : detk::cand_cap<4096>()) * 8;
        pl->ws_bytes = off;
    }
    pl->lds = lds_bytes(pl->tile, pl->kmax, pl->multi);
    if (pl->lds > dev.max_lds) return DETK_ERR_UNSUPPORTED;
    // int32 offsets: every window must be addressable with int32 row_starts + length.
    if ((int64_t)B * k >= ((int64_t)1 << 31)) return DETK_ERR_UNSUPPORTED;
    return DETK_OK;
}

template <int TILE, int KMAX, bool MULTI>
hipError_t launch(const Params& p, int grid, size_t lds, hipStream_t stream) {
    using S = Shape<TILE>;
    hipLaunchKernelGGL((detk::topk_ragged_kernel<S::NT, S::EPT, KMAX, MULTI, min_waves<TILE, MULTI>()>), dim3(grid), dim3(S::NT), lds,
                       stream, p);
    return hipGetLastError();
}

hipError_t dispatch(const Plan& pl, const Params& p, hipStream_t stream) {
    const bool k2 = pl.kmax == 2048;
    if (!pl.multi) {
        switch (pl.tile) {
        case 4096: return k2 ? launch<4096, 2048, false>(p, pl.grid, pl.lds, stream)
                             : launch<4096, 4096, false>(p, pl.grid, pl.lds, stream);
        case 8192: return k2 ? launch<8192, 2048, false>(p, pl.grid, pl.lds, stream)
                             : launch<8192, 4096, false>(p, pl.grid, pl.lds, stream);
        case 16384: return k2 ? launch<16384, 2048, false>(p, pl.grid, pl.lds, stream)
                              : launch<16384, 4096, false>(p, pl.grid, pl.lds, stream);
        default: return k2 ? launch<32768, 2048, false>(p, pl.grid, pl.lds, stream)
                           : launch<32768, 4096, false>(p, pl.grid, pl.lds, stream);
        }
    }
    switch (pl.tile) {
    case 4096: return k2 ? launch<4096, 2048, true>(p, pl.grid, pl.lds, stream)
                         : launch<4096, 4096, true>(p, pl.grid, pl.lds, stream);
    case 8192: return k2 ? launch<8192, 2048, true>(p, pl.grid, pl.lds, stream)
                         : launch<8192, 4096, true>(p, pl.grid, pl.lds, stream);
    case 16384: return k2 ? launch<16384, 2048, true>(p, pl.grid, pl.lds, stream)
                          : launch<16384, 4096, true>(p, pl.grid, pl.lds, stream);
    default: return k2 ? launch<32768, 2048, true>(p, pl.grid, pl.lds, stream)
                       : launch<32768, 4096, true>(p, pl.grid, pl.lds, stream);
    }
}

}  // namespace

// A plain streaming read (measurement only): every 16-byte chunk once, eight loads in
// flight per thread, XOR-reduced so the loads cannot be dropped.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16, uint32_t* out) {
    constexpr int U = 8;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = p[i + j * stride];
#pragma unroll
        for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0) atomicXor(out, acc);
}

extern "C" {

int detk_can_implement(int device, int k, int32_t max_len) {
    DeviceInfo dev;
    int st = device_info(device, &dev);
    if (st != DETK_OK) return st;
    Plan pl;
    return make_plan(dev, 1, k, max_len, &pl);
}

size_t detk_workspace_size(int device, int B, int k, int32_t max_len) {
    DeviceInfo dev;
    if (device_info(device, &dev) != DETK_OK) return 0;
    Plan pl;
    if (make_plan(dev, B, k, max_len, &pl) != DETK_OK) return 0;
    return B == 0 ? 0 : pl.ws_bytes;
}

int detk_topk_ragged(const float* scores, const int32_t* row_starts, const int32_t* lengths, int B,
                     int32_t max_len, int k, int32_t* out_idx, float* out_val, void* workspace,
                     size_t workspace_bytes, void* stream_ptr) {
    if (B < 0 || k < 1 || max_len < 0) return DETK_ERR_INVALID_ARG;
    if (B > 0 && (!scores || !out_idx)) return DETK_ERR_INVALID_ARG;
    if (k > DETK_MAX_K) return DETK_ERR_UNSUPPORTED;
    if (B == 0) return DETK_OK;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return DETK_ERR_HIP;
    DeviceInfo dev;
    int st = device_info(device, &dev);
    if (st != DETK_OK) return st;
    Plan pl;
    st = make_plan(dev, B, k, max_len, &pl);
    if (st != DETK_OK) return st;
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return DETK_ERR_WORKSPACE;

    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    Params p;
    p.scores = reinterpret_cast<const uint32_t*>(scores);
    p.row_starts = row_starts;
    p.lengths = lengths;
    p.B = B;
    p.max_len = max_len;
    p.k = k;
    p.tiles_per_row = pl.tiles_per_row;
    p.stage_cap = g_stage_cap < 0 ? detk::kStageCap : (g_stage_cap > detk::kStageCap ? detk::kStageCap : g_stage_cap);
    p.fast = g_fast;
    p.out_idx = out_idx;
    p.out_val = reinterpret_cast<uint32_t*>(out_val);
    p.ws_zero = nullptr;
    p.ws_ecnt = nullptr;
    p.ws_stage = nullptr;
    p.ws_cand = nullptr;
    if (pl.multi) {
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        p.ws_zero = reinterpret_cast<uint32_t*>(ws + pl.off_zero);
        p.ws_ecnt = reinterpret_cast<uint32_t*>(ws + pl.off_ecnt);
        p.ws_stage = reinterpret_cast<uint64_t*>(ws + pl.off_stage);
        p.ws_cand = reinterpret_cast<uint2*>(ws + pl.off_cand);
        const int64_t nz = (int64_t)pl.n_zero_words;
        int zgrid = (int)((nz + 255) / 256);
        if (zgrid > 1024) zgrid = 1024;
        hipLaunchKernelGGL(detk::zero_words_kernel, dim3(zgrid), dim3(256), 0, stream, p.ws_zero, nz);
        if (hipGetLastError() != hipSuccess) return DETK_ERR_HIP;
    }
    if (dispatch(pl, p, stream) != hipSuccess) return DETK_ERR_HIP;
    return DETK_OK;
}

const char* detk_status_string(int status) {
    switch (status) {
    case DETK_OK: return "DETK_OK";
    case DETK_ERR_INVALID_ARG: return "DETK_ERR_INVALID_ARG: null pointer, B < 0, k < 1 or max_len < 0";
    case DETK_ERR_UNSUPPORTED:
        return "DETK_ERR_UNSUPPORTED: k > 4096, device is not gfx950, or the row is too long for the "
               "co-resident multi-workgroup path";
    case DETK_ERR_WORKSPACE: return "DETK_ERR_WORKSPACE: workspace missing or smaller than detk_workspace_size()";
    case DETK_ERR_HIP: return "DETK_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown detk status";
    }
}

int detk_workspace_error(const void* workspace, size_t workspace_bytes, void* stream_ptr) {
    if (!workspace || workspace_bytes < 4) return 0;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    if (hipStreamSynchronize(stream) != hipSuccess) return -1;
    uint32_t word = 0;
    if (hipMemcpy(&word, workspace, 4, hipMemcpyDeviceToHost) != hipSuccess) return -1;
    return (int)word;
}

int detk_read_probe(const void* data, size_t bytes, uint32_t* out, void* stream_ptr) {
    if (bytes == 0) return DETK_OK;
    if (!data || !out || (bytes & 15u) != 0 || (reinterpret_cast<uintptr_t>(data) & 15u) != 0)
        return DETK_ERR_INVALID_ARG;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return DETK_ERR_HIP;
    DeviceInfo dev;
    const int st = device_info(device, &dev);
    if (st != DETK_OK) return st;
    const size_t n16 = bytes / 16;
    const int64_t want = (int64_t)dev.cus * 8;  // 8 workgroups of 4 waves per CU: 32 waves
    const int64_t need = (int64_t)((n16 + 255) / 256);
    const int grid = (int)(need < want ? need : want);
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream_ptr),
                       reinterpret_cast<const uint4*>(data), n16, out);
    return hipGetLastError() == hipSuccess ? DETK_OK : DETK_ERR_HIP;
}

int detk_debug_set(int what, int value) {
    switch (what) {
    case DETK_DEBUG_PATH:
        if (value < 0 || value > 2) return DETK_ERR_INVALID_ARG;
        g_force_path = value;
        return DETK_OK;
    case DETK_DEBUG_STAGING_CAP:
        if (value < -1) return DETK_ERR_INVALID_ARG;
        g_stage_cap = value;
        return DETK_OK;
    case DETK_DEBUG_MULTI_TILE:
        if (value != 0 && value != 4096 && value != 8192 && value != 16384 && value != 32768)
            return DETK_ERR_INVALID_ARG;
        g_multi_tile = value;
        return DETK_OK;
    case DETK_DEBUG_FAST:
        if (value < 0 || value > 2) return DETK_ERR_INVALID_ARG;
        g_fast = value;
        return DETK_OK;
    default: return DETK_ERR_INVALID_ARG;
    }
}

}  // extern "C"
