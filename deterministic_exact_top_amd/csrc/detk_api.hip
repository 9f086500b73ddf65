// detk_api.hip -- host side of the C ABI declared in include/detk.h.
//
// Validates arguments on the host (nothing is launched on an error), picks the
// launch shape from host-known sizes only (B, k, max_len, device properties) and
// enqueues the kernels on the caller's stream.  No allocation, no synchronisation,
// no device readback: a call can be captured into a HIP graph.
#include <hip/hip_runtime.h>
#include <cmath>

#include <mutex>
#include <string.h>

#include "../../include/detk.h"
#include "indexer.hpp"
#include "kernels.hpp"

// Workspace of detk_topk_ragged_noalloc: one array per GPU the library runs on, held until
// the process ends.  Zero when the code object loads; every call leaves the words that
// must start at zero (the per-row counters) at zero again, so it is always ready.  In
// host code the name is a stand-in, never a device address: kernels get the address
// hipGetSymbolAddress returned for the current device (DeviceInfo::scratch).
static __device__ __align__(256) unsigned char scratch[DETK_SCRATCH_BYTES];

namespace {

using detk::Params;
using detk::SmemAll;
using detk::Shape;
using detk::min_waves;
using detk::kSingleMaxLen;
using detk::kSplitTile;

template <int TILE, int KMAX, bool MULTI, int VB = 4, bool WIDE = false>
const void* kernel_ptr() {
    using S = Shape<TILE, MULTI, WIDE>;
    return reinterpret_cast<const void*>(
        &detk::topk_ragged_kernel<S::NT, S::EPT, KMAX, MULTI, min_waves<TILE, KMAX, MULTI, WIDE>(), VB>);
}

template <int TILE, int KMAX, bool MULTI, bool WIDE = false>
constexpr size_t smem_bytes() {
    using S = Shape<TILE, MULTI, WIDE>;
    return sizeof(SmemAll<S::NT, S::EPT, KMAX, MULTI>);
}

struct DeviceInfo {
    bool init = false;
    bool gfx950 = false;
    int cus = 0;
    size_t max_lds = 0;
    int split_occ[2] = {};   // workgroups per CU of the 16K-element split tile, k <= 2048 / k <= 4096
    void* scratch = nullptr; // this device's copy of `scratch` (device address)
};

std::mutex g_mu;
DeviceInfo g_dev[64];
int g_force_path = 0;       // 0 auto, 1 single, 2 multi
int g_stage_cap = -1;       // -1 default
int g_multi_tile = 0;       // 0 default
int g_fast = 1;             // 0 off, 1 on, 2 on with a pivot that always misses
int g_small = 0;            // 0 by batch size, 1 never the small-batch shapes, 2 always
int g_split_samples = 0;    // split rows: 0 by the candidate list's room, 1 always 8192, 2 always 4096

template <int TILE, int KMAX, bool MULTI, int VB, bool WIDE = false>
hipError_t prepare_kernel() {
    return hipFuncSetAttribute(kernel_ptr<TILE, KMAX, MULTI, VB, WIDE>(), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)smem_bytes<TILE, KMAX, MULTI, WIDE>());
}

template <int TILE, int VB>
void prepare_all(hipError_t* e) {
    hipError_t r;
    if ((r = prepare_kernel<TILE, 2048, false, VB>()) != hipSuccess) *e = r;
    if ((r = prepare_kernel<TILE, 4096, false, VB>()) != hipSuccess) *e = r;
    if ((r = prepare_kernel<TILE, 2048, true, VB>()) != hipSuccess) *e = r;
    if ((r = prepare_kernel<TILE, 4096, true, VB>()) != hipSuccess) *e = r;
    if constexpr (TILE < 32768) {
        if ((r = prepare_kernel<TILE, 2048, false, VB, true>()) != hipSuccess) *e = r;
        if ((r = prepare_kernel<TILE, 4096, false, VB, true>()) != hipSuccess) *e = r;
    }
}

template <int TILE, int KMAX>
int split_occupancy() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel_ptr<TILE, KMAX, true>(), Shape<TILE, true>::NT,
                                                     smem_bytes<TILE, KMAX, true>()) != hipSuccess)
        return 0;
    return blocks;
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
            prepare_all<4096, 4>(&e);
            prepare_all<8192, 4>(&e);
            prepare_all<16384, 4>(&e);
            prepare_all<32768, 4>(&e);
            prepare_all<4096, 2>(&e);
            prepare_all<8192, 2>(&e);
            prepare_all<16384, 2>(&e);
            prepare_all<32768, 2>(&e);
            d.split_occ[0] = split_occupancy<kSplitTile, 2048>();
            d.split_occ[1] = split_occupancy<kSplitTile, 4096>();
            // (with this device current: each GPU holds its own copy at its own address)
            if (e == hipSuccess) e = hipGetSymbolAddress(&d.scratch, HIP_SYMBOL(scratch));
            if (e == hipSuccess && d.scratch == nullptr) e = hipErrorInvalidSymbol;
        }
        if (cur != device) (void)hipSetDevice(cur);
        if (e != hipSuccess) return DETK_ERR_HIP;
        d.init = true;
    }
    *out = d;
    return DETK_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    bool multi = false;
    int tile = 0;         // elements per workgroup tile
    int kmax = 2048;
    int tiles_per_row = 1;
    bool wide = false;    // one workgroup per row, small-batch (1024-thread) shape
    bool small = false;   // no more workgroups than CUs: every wave selects pivot digits
    bool half = false;    // split rows: half the row samples
    int grid = 0;
    size_t lds = 0;
    size_t ws_bytes = 0;
    // workspace layout: data regions, in bytes from the start of the data area
    size_t data_bytes = 0, off_ecnt = 0, off_cand = 0, off_tie = 0;
};

// Workspace layout.  The per-row control words (which must be zero when a call starts,
// and which every call leaves at zero) sit at the start, row b at byte b * kCtlRowBytes,
// in a control area of the first 1/64 of the workspace; every data region comes after
// it.  The area's size depends on the workspace's size alone, so calls of any shape on
// one buffer (passed with the same size) never write data over another call's control
// words, and a buffer zero-filled once stays ready.  A split row needs at least 32 KB of
// data, so the area always holds every row's words.
constexpr size_t kCtlRowBytes = detk::kRowCtlWords * 4;
size_t data_offset(size_t workspace_bytes) { return align256(workspace_bytes / 64); }

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
size_t lds_bytes_wide(int tile, int kmax) {
    const bool k2 = kmax == 2048;
    switch (tile) {
    case 4096: return k2 ? smem_bytes<4096, 2048, false, true>() : smem_bytes<4096, 4096, false, true>();
    case 8192: return k2 ? smem_bytes<8192, 2048, false, true>() : smem_bytes<8192, 4096, false, true>();
    case 16384: return k2 ? smem_bytes<16384, 2048, false, true>() : smem_bytes<16384, 4096, false, true>();
    default: return k2 ? smem_bytes<32768, 2048, false, true>() : smem_bytes<32768, 4096, false, true>();
    }
}
size_t lds_bytes(int tile, int kmax, bool multi, bool wide) {
    if (wide) return lds_bytes_wide(tile, kmax);
    return multi ? lds_bytes_t<true>(tile, kmax) : lds_bytes_t<false>(tile, kmax);
}

// Most workgroups launched for the split-row kernel; more items are taken by a grid-stride
// loop (the items never wait for one another, so any number may be resident).
constexpr int64_t kMaxSplitGrid = 65536;

// Decide the launch shape from host-known sizes only.
int make_plan(const DeviceInfo& dev, int B, int k, int32_t max_len, Plan* pl) {
    if (B < 0 || k < 1 || max_len < 0) return DETK_ERR_INVALID_ARG;
    if (k > DETK_MAX_K || max_len > DETK_MAX_LEN) return DETK_ERR_UNSUPPORTED;
    if (!dev.gfx950) return DETK_ERR_UNSUPPORTED;
    // int32 output offsets: b * k + t must be addressable.
    if ((int64_t)B * k >= ((int64_t)1 << 31)) return DETK_ERR_UNSUPPORTED;
    pl->kmax = k <= 2048 ? 2048 : 4096;

    bool multi;
    if (g_force_path == 1) {
        if (max_len > kSingleMaxLen) return DETK_ERR_UNSUPPORTED;
        multi = false;
    } else if (g_force_path == 2) {
        multi = true;
    } else {
        // One workgroup per row whenever the row fits one tile.
        multi = max_len > kSingleMaxLen;
    }
    pl->multi = multi;
    if (!multi) {
        pl->tile = max_len <= 4096 ? 4096 : max_len <= 8192 ? 8192 : max_len <= 16384 ? 16384 : 32768;
        pl->tiles_per_row = 1;
        pl->grid = B;  // one workgroup per row: the dispatcher balances rows of unequal length
        pl->ws_bytes = 0;
        // A batch with no more rows than CUs gives every row a CU of its own: then 1024
        // threads per row shorten the row's serial phases (the latency of a decode step).
        pl->wide = g_small == 2 || (g_small == 0 && (int64_t)B <= dev.cus);
    } else {
        // 16K-element tiles spread a row over more CUs; when a batch has more of them than
        // the GPU holds at once, 32K-element tiles (half as many workgroups, each ordering
        // nothing more) finish in fewer rounds.
        const int64_t tpr16 = ((int64_t)max_len + kSplitTile - 1) / kSplitTile;
        const int64_t resident = (int64_t)dev.cus * dev.split_occ[pl->kmax == 2048 ? 0 : 1];
        pl->tile = g_multi_tile ? g_multi_tile : ((int64_t)B * tpr16 <= resident ? kSplitTile : 2 * kSplitTile);
        const int64_t tpr = max_len == 0 ? 1 : ((int64_t)max_len + pl->tile - 1) / pl->tile;
        pl->tiles_per_row = (int)tpr;
        const int64_t items = (int64_t)B * tpr;
        pl->grid = (int)(items < kMaxSplitGrid ? items : kMaxSplitGrid);
        // Data regions, from the start of the data area (see data_offset()).
        const size_t cap = pl->kmax == 2048 ? detk::cand_cap<2048>() : detk::cand_cap<4096>();
        // Half the row samples when, even with them, the longest row's candidates stay
        // within the list by four standard deviations: the pivot passes cost half as much.
        // (Pivot at the r-th largest of s samples, r = e + 3.5 sqrt(e) + 4, e = s m / n:
        // about r n / s keys above it, give or take n sqrt(r) / s.)
        {
            const double s = detk::kSplitSamples / 2, n = (double)max_len, m = (double)(k < max_len ? k : max_len);
            const double e = s * m / n, r = e + 3.5 * std::sqrt(e) + 4.0;
            pl->half = g_split_samples == 2 ||
                       (g_split_samples == 0 && r * n / s + 4.0 * n * std::sqrt(r) / s <= (double)cap);
        }
        size_t off = 0;
        pl->off_ecnt = off;
        off = align256(off + (size_t)B * (size_t)tpr * 4);
        pl->off_cand = off;
        off = align256(off + (size_t)B * cap * 8);
        pl->off_tie = off;
        off = align256(off + (size_t)B * (size_t)tpr * (size_t)(pl->tile / 32) * 4);
        pl->data_bytes = off;
        // The smallest workspace whose control area and data area both fit.
        size_t w = align256(off + off / 63 + 512);
        while (data_offset(w) + off > w || (size_t)B * kCtlRowBytes > data_offset(w)) w += 256;
        pl->ws_bytes = w;
    }
    // Every wave selects the pivot digits itself when no more workgroups are launched than
    // CUs: one barrier fewer per pivot pass, where issue slots are not what limits the call.
    pl->small = g_small == 2 || (g_small == 0 && (int64_t)pl->grid <= dev.cus);
    pl->lds = lds_bytes(pl->tile, pl->kmax, pl->multi, pl->wide);
    if (pl->lds > dev.max_lds) return DETK_ERR_UNSUPPORTED;
    return DETK_OK;
}

template <int TILE, int KMAX, bool MULTI, int VB, bool WIDE = false>
hipError_t launch(const Params& p, int grid, size_t lds, hipStream_t stream) {
    using S = Shape<TILE, MULTI, WIDE>;
    hipLaunchKernelGGL((detk::topk_ragged_kernel<S::NT, S::EPT, KMAX, MULTI, min_waves<TILE, KMAX, MULTI, WIDE>(), VB>),
                       dim3(grid), dim3(S::NT), lds, stream, p);
    return hipGetLastError();
}

template <int VB>
hipError_t dispatch_vb(const Plan& pl, const Params& p, hipStream_t stream) {
    const bool k2 = pl.kmax == 2048;
    if (!pl.multi && pl.wide) {
        switch (pl.tile) {
        case 4096: return k2 ? launch<4096, 2048, false, VB, true>(p, pl.grid, pl.lds, stream)
                             : launch<4096, 4096, false, VB, true>(p, pl.grid, pl.lds, stream);
        case 8192: return k2 ? launch<8192, 2048, false, VB, true>(p, pl.grid, pl.lds, stream)
                             : launch<8192, 4096, false, VB, true>(p, pl.grid, pl.lds, stream);
        case 16384: return k2 ? launch<16384, 2048, false, VB, true>(p, pl.grid, pl.lds, stream)
                              : launch<16384, 4096, false, VB, true>(p, pl.grid, pl.lds, stream);
        default: break;  // the 32768-element tile has 1024 threads already
        }
    }
    if (!pl.multi) {
        switch (pl.tile) {
        case 4096: return k2 ? launch<4096, 2048, false, VB>(p, pl.grid, pl.lds, stream)
                             : launch<4096, 4096, false, VB>(p, pl.grid, pl.lds, stream);
        case 8192: return k2 ? launch<8192, 2048, false, VB>(p, pl.grid, pl.lds, stream)
                             : launch<8192, 4096, false, VB>(p, pl.grid, pl.lds, stream);
        case 16384: return k2 ? launch<16384, 2048, false, VB>(p, pl.grid, pl.lds, stream)
                              : launch<16384, 4096, false, VB>(p, pl.grid, pl.lds, stream);
        default: return k2 ? launch<32768, 2048, false, VB>(p, pl.grid, pl.lds, stream)
                           : launch<32768, 4096, false, VB>(p, pl.grid, pl.lds, stream);
        }
    }
    switch (pl.tile) {
    case 4096: return k2 ? launch<4096, 2048, true, VB>(p, pl.grid, pl.lds, stream)
                         : launch<4096, 4096, true, VB>(p, pl.grid, pl.lds, stream);
    case 8192: return k2 ? launch<8192, 2048, true, VB>(p, pl.grid, pl.lds, stream)
                         : launch<8192, 4096, true, VB>(p, pl.grid, pl.lds, stream);
    case 16384: return k2 ? launch<16384, 2048, true, VB>(p, pl.grid, pl.lds, stream)
                          : launch<16384, 4096, true, VB>(p, pl.grid, pl.lds, stream);
    default: return k2 ? launch<32768, 2048, true, VB>(p, pl.grid, pl.lds, stream)
                       : launch<32768, 4096, true, VB>(p, pl.grid, pl.lds, stream);
    }
}

hipError_t dispatch(const Plan& pl, const Params& p, int vb, hipStream_t stream) {
    return vb == 2 ? dispatch_vb<2>(pl, p, stream) : dispatch_vb<4>(pl, p, stream);
}

// The operation, on the caller's workspace or (use_scratch) on the device's scratch array.
// Allocates nothing in either case.
// dtype: DETK_DTYPE_F32, DETK_DTYPE_F16 or DETK_DTYPE_BF16 (checked by the caller).
int run(const void* scores, int dtype, const int32_t* row_starts, const int32_t* lengths, int B, int32_t max_len,
        int k, const detk_index_transform* xf, int32_t* out_idx, void* out_val, void* workspace,
        size_t workspace_bytes, bool use_scratch, void* stream_ptr) {
    if (B < 0 || k < 1 || max_len < 0) return DETK_ERR_INVALID_ARG;
    if (B > 0 && (!scores || !out_idx)) return DETK_ERR_INVALID_ARG;
    if (k > DETK_MAX_K || max_len > DETK_MAX_LEN) return DETK_ERR_UNSUPPORTED;
    int32_t xf_shift = -1;
    if (xf) {
        if (xf->mode < DETK_INDEX_LOCAL || xf->mode > DETK_INDEX_PAGE_TABLE) return DETK_ERR_INVALID_ARG;
        if (xf->mode == DETK_INDEX_OFFSET && B > 0 && !xf->offsets) return DETK_ERR_INVALID_ARG;
        if (xf->mode == DETK_INDEX_PAGE_TABLE) {
            if ((B > 0 && !xf->page_table) || xf->page_size < 1) return DETK_ERR_INVALID_ARG;
            // every page any window can touch must be in the row's part of the table (stride 0:
            // every row reads the same table)
            if (xf->page_table_stride < 0 ||
                (xf->page_table_stride != 0 &&
                 xf->page_table_stride < ((int64_t)max_len + xf->page_size - 1) / xf->page_size))
                return DETK_ERR_INVALID_ARG;
            if ((xf->page_size & (xf->page_size - 1)) == 0) xf_shift = __builtin_ctz((unsigned)xf->page_size);
        }
    }
    if (B == 0) return DETK_OK;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return DETK_ERR_HIP;
    DeviceInfo dev;
    int st = device_info(device, &dev);
    if (st != DETK_OK) return st;
    Plan pl;
    st = make_plan(dev, B, k, max_len, &pl);
    if (st != DETK_OK) return st;
    if (use_scratch) {
        workspace = dev.scratch;
        workspace_bytes = DETK_SCRATCH_BYTES;
    }
    size_t data_off = 0;
    if (pl.multi) {
        data_off = data_offset(workspace_bytes);
        if (!workspace || workspace_bytes < pl.ws_bytes || data_off + pl.data_bytes > workspace_bytes ||
            (size_t)B * kCtlRowBytes > data_off)
            return DETK_ERR_WORKSPACE;
    }

    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    Params p;
    p.scores = scores;
    p.row_starts = row_starts;
    p.lengths = lengths;
    p.B = B;
    p.max_len = max_len;
    p.k = k;
    p.tiles_per_row = pl.tiles_per_row;
    p.stage_cap = g_stage_cap < 0 ? detk::kStageCap : (g_stage_cap > detk::kStageCap ? detk::kStageCap : g_stage_cap);
    p.fast = g_fast;
    p.small_batch = pl.small ? 1 : 0;
    p.split_half = pl.half ? 1 : 0;
    p.out_idx = out_idx;
    p.out_val = out_val;
    p.val_pad = dtype == DETK_DTYPE_F16 ? 0xFC00u : dtype == DETK_DTYPE_BF16 ? 0xFF80u : detk::kNegInfBits;
    p.xf_mode = xf ? xf->mode : DETK_INDEX_LOCAL;
    p.xf_page = xf && xf->mode == DETK_INDEX_PAGE_TABLE ? xf->page_size : 1;
    p.xf_shift = xf_shift;
    p.xf_offsets = xf && xf->mode == DETK_INDEX_OFFSET ? xf->offsets : nullptr;
    p.xf_table = xf && xf->mode == DETK_INDEX_PAGE_TABLE ? xf->page_table : nullptr;
    p.xf_stride = xf && xf->mode == DETK_INDEX_PAGE_TABLE ? xf->page_table_stride : 0;
    p.ws_ctl = nullptr;
    p.ws_ecnt = nullptr;
    p.ws_cand = nullptr;
    p.ws_tie = nullptr;
    if (pl.multi) {
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        p.ws_ctl = reinterpret_cast<uint32_t*>(ws);
        p.ws_ecnt = reinterpret_cast<uint32_t*>(ws + data_off + pl.off_ecnt);
        p.ws_cand = reinterpret_cast<uint2*>(ws + data_off + pl.off_cand);
        p.ws_tie = reinterpret_cast<uint32_t*>(ws + data_off + pl.off_tie);
    }
    if (dispatch(pl, p, dtype == DETK_DTYPE_F32 ? 4 : 2, stream) != hipSuccess) return DETK_ERR_HIP;
    return DETK_OK;
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
    if (device_info(device, &dev) != DETK_OK) return DETK_WORKSPACE_UNSUPPORTED;
    Plan pl;
    if (make_plan(dev, B, k, max_len, &pl) != DETK_OK) return DETK_WORKSPACE_UNSUPPORTED;
    return B == 0 ? 0 : pl.ws_bytes;
}

int detk_topk_ragged(const float* scores, const int32_t* row_starts, const int32_t* lengths, int B,
                     int32_t max_len, int k, int32_t* out_idx, float* out_val, void* workspace,
                     size_t workspace_bytes, void* stream_ptr) {
    return run(scores, DETK_DTYPE_F32, row_starts, lengths, B, max_len, k, nullptr, out_idx, out_val, workspace,
               workspace_bytes, false, stream_ptr);
}

int detk_topk_ragged_16bit(const void* scores, int dtype, const int32_t* row_starts, const int32_t* lengths, int B,
                           int32_t max_len, int k, const detk_index_transform* transform, int32_t* out_idx,
                           void* out_val, void* workspace, size_t workspace_bytes, void* stream_ptr) {
    if (dtype != DETK_DTYPE_F16 && dtype != DETK_DTYPE_BF16) return DETK_ERR_INVALID_ARG;
    return run(scores, dtype, row_starts, lengths, B, max_len, k, transform, out_idx, out_val, workspace,
               workspace_bytes, false, stream_ptr);
}

int detk_topk_ragged_transform(const float* scores, const int32_t* row_starts, const int32_t* lengths, int B,
                               int32_t max_len, int k, const detk_index_transform* transform, int32_t* out_idx,
                               float* out_val, void* workspace, size_t workspace_bytes, void* stream_ptr) {
    return run(scores, DETK_DTYPE_F32, row_starts, lengths, B, max_len, k, transform, out_idx, out_val, workspace,
               workspace_bytes, false, stream_ptr);
}

int detk_topk_ragged_noalloc(const float* scores, const int32_t* row_starts, const int32_t* lengths, int B,
                             int32_t max_len, int k, int32_t* out_idx, float* out_val, void* stream_ptr) {
    return run(scores, DETK_DTYPE_F32, row_starts, lengths, B, max_len, k, nullptr, out_idx, out_val, nullptr, 0,
               true, stream_ptr);
}

const char* detk_status_string(int status) {
    switch (status) {
    case DETK_OK: return "DETK_OK";
    case DETK_ERR_INVALID_ARG:
        return "DETK_ERR_INVALID_ARG: a required pointer is NULL, or B < 0, k < 1 or max_len < 0";
    case DETK_ERR_UNSUPPORTED:
        return "DETK_ERR_UNSUPPORTED: k > 4096, max_len > 2^30, B * k >= 2^31, or the device is not gfx950";
    case DETK_ERR_WORKSPACE:
        return "DETK_ERR_WORKSPACE: workspace missing or smaller than detk_workspace_size() (it must also be "
               "zero-filled before its first use)";
    case DETK_ERR_HIP: return "DETK_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown detk status";
    }
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

int detk_indexer_scores(const void* q, const float* w, const void* keys, int32_t n_keys, const int32_t* lengths,
                        int B, int heads, int head_dim, int32_t max_len, float* out, void* stream) {
    if (B < 0 || max_len < 0 || n_keys < 0) return DETK_ERR_INVALID_ARG;
    if (heads != detk_ix::kHeads || head_dim != detk_ix::kHeadDim) return DETK_ERR_UNSUPPORTED;
    if (max_len > n_keys) return DETK_ERR_INVALID_ARG;  // every window lies inside the keys
    // the key rows are read through one buffer resource: at most 2^31 - 1 bytes of keys
    if ((int64_t)n_keys * detk_ix::kHeadDim * 2 > 0x7FFFFFFF) return DETK_ERR_UNSUPPORTED;
    if (B == 0 || max_len == 0) return DETK_OK;
    if (!q || !w || !keys || !out) return DETK_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(keys)) & 15u)
        return DETK_ERR_INVALID_ARG;  // 16-byte loads
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return DETK_ERR_HIP;
    DeviceInfo dev;
    const int st = device_info(device, &dev);
    if (st != DETK_OK) return st;
    if (!dev.gfx950) return DETK_ERR_UNSUPPORTED;
    detk_ix::IxParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.w = w;
    p.keys = static_cast<const uint16_t*>(keys);
    p.lengths = lengths;
    p.B = B;
    p.max_len = max_len;
    p.n_keys = n_keys;
    p.chunk = 0;   // (chosen by launch_indexer)
    p.chunks = 0;
    p.out = out;
    const hipError_t e = detk_ix::launch_indexer(p, dev.cus, reinterpret_cast<hipStream_t>(stream));
    if (e == hipErrorInvalidValue) return DETK_ERR_UNSUPPORTED;  // grid beyond 2^31 - 1 workgroups
    return e == hipSuccess ? DETK_OK : DETK_ERR_HIP;
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
    case DETK_DEBUG_SMALL_BATCH:
        if (value < 0 || value > 2) return DETK_ERR_INVALID_ARG;
        g_small = value;
        return DETK_OK;
    case DETK_DEBUG_SPLIT_SAMPLES:
        if (value < 0 || value > 2) return DETK_ERR_INVALID_ARG;
        g_split_samples = value;
        return DETK_OK;
    default: return DETK_ERR_INVALID_ARG;
    }
}

}  // extern "C"
