// topk_device.hpp -- gfx950 device code for exact, bitwise-deterministic ragged top-k.
//
// Method (SGLang PR #31115, "Modifications"): a coarse 8-bit radix histogram pass,
// MSB-first refinement to the exact threshold key, smallest-index resolution of the
// boundary tie set, and a sort of the unique (score, index) composites into the
// canonical order (score descending under the bitwise total order, index ascending).
// Threshold-bin overflow never drops a candidate: refinement rescans the row
// (same PR, summary and hardening commit).
//
// MI355X layout of the work:
//   * A workgroup owns a tile of up to NT*EPT consecutive elements of one row and keeps
//     it in VGPRs for its whole life (EPT 32-bit keys per lane).  HBM is read once.
//   * Histograms are per-wave LDS arrays of 256 u32 bins, merged by the workgroup;
//     lanes that share the first active lane's bin are merged with one ballot and a
//     single LDS add, which keeps 0.0-plateau rows from serialising on one bank.
//   * After the first pass the threshold bin's candidates are compacted into LDS when
//     they fit (`stage_cap`); otherwise every later pass rescans the registers.
//   * Boundary ties (key == T) are ranked in index order with an LDS bitmap over the
//     tile's positions plus a prefix over words; the first `need` are kept.
//   * Selected elements above T are sorted in LDS as u64 composites
//     (key << 32 | ~index), which are unique, so the order is total.
//   * Rows longer than one tile are split over several co-resident workgroups that
//     add their integer histograms into the workspace with atomics (order-independent,
//     hence deterministic) and meet at per-row counters between passes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detk {

constexpr int kRadix = 256;
constexpr int kStageCap = 4096;          // LDS threshold-bin staging capacity (entries)
constexpr uint32_t kNegInfBits = 0xFF800000u;
constexpr int kRowZeroWords = 4 * kRadix + 4;   // per-row words zeroed before a multi launch
constexpr uint32_t kSpinLimit = 1u << 21;       // bounded wait (polls, ~1 us each) at row barriers

struct Params {
    const uint32_t* scores;
    const int32_t* row_starts;  // nullable
    const int32_t* lengths;     // nullable
    int32_t B;
    int32_t max_len;
    int32_t k;
    int32_t tiles_per_row;      // multi path only
    int32_t stage_cap;          // <= kStageCap
    int32_t* out_idx;
    uint32_t* out_val;          // nullable
    uint32_t* ws_zero;          // [0] error word, then B * kRowZeroWords (zeroed per call)
    uint32_t* ws_ecnt;          // B * tiles_per_row
    uint64_t* ws_stage;         // B * k
};

// ----------------------------------------------------------------------------- bits

// Unsigned key whose order is IEEE totalOrder on the float bits.
__device__ __forceinline__ uint32_t key_of(uint32_t u) {
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
// Inverse of key_of (bit move only).
__device__ __forceinline__ uint32_t bits_of(uint32_t key) {
    return key ^ ((uint32_t)((int32_t)~key >> 31) | 0x80000000u);
}

// ----------------------------------------------------------------------------- wave helpers

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Count one per active lane into h[d]; lanes sharing the first active lane's bin are
// merged into one add.  Must be called from the lanes to count (divergence allowed).
__device__ __forceinline__ void hist_add(uint32_t* h, uint32_t d) {
    const uint32_t lead = __builtin_amdgcn_readfirstlane(d);
    const uint64_t same = __ballot(d == lead);
    if (d == lead) {
        if (lanes_below(same) == 0) lds_add(&h[lead], (uint32_t)__popcll(same));
    } else {
        lds_add(&h[d], 1u);
    }
}

// Wave-aggregated slot claim on an LDS counter: returns a unique slot for each lane
// with pred set (value meaningless otherwise).  Call with the whole wave converged.
__device__ __forceinline__ uint32_t claim_slot(bool pred, uint32_t* counter) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return 0;
    const int leader = __ffsll((unsigned long long)m) - 1;
    uint32_t base = 0;
    if ((int)(threadIdx.x & 63) == leader)
        base = __hip_atomic_fetch_add(counter, (uint32_t)__popcll(m), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
    base = __builtin_amdgcn_readlane(base, leader);
    return base + lanes_below(m);
}

// ----------------------------------------------------------------------------- shared memory

template <int NT, int EPT, int KMAX>
struct Smem {
    static constexpr int NW = NT / 64;
    static constexpr int TILE = NT * EPT;
    static constexpr int BWORDS = TILE / 32;
    uint32_t whist[NW][kRadix];   // per-wave histograms
    uint32_t hist[kRadix];        // merged histogram of the current pass (row-global)
    uint32_t lhist[kRadix];       // this tile's own merged histogram
    uint32_t wsum[32];            // per-wave partials for block scans
    uint32_t sel[4];              // digit select: digit, count above, bin count
    uint32_t ctr[8];              // [0] staged, [1] A fill, [2] bcast, [3] bcast
    uint32_t bitmap[BWORDS];      // tie positions of this tile
    uint32_t wpre[BWORDS];        // exclusive prefix of popcounts over bitmap words
    uint32_t skey[kStageCap];     // staged candidate keys
    uint32_t sidx[kStageCap];     // staged candidate row indices
    uint64_t A[KMAX];             // composites of selected elements above T
};

// ----------------------------------------------------------------------------- block helpers

template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum, uint32_t* total) {
    const int tid = threadIdx.x;
    const uint32_t incl = wave_incl_scan(x);
    if ((tid & 63) == 63) wsum[tid >> 6] = incl;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t v = wsum[w];
        off += (w < (tid >> 6)) ? v : 0u;
        tot += v;
    }
    *total = tot;
    __syncthreads();
    return off + incl - x;
}

// Pick the bin holding the k_rem-th largest key: scan bins 255..0; writes sel[] =
// {digit, count strictly above the digit, count of the digit}.  All threads call.
template <int NT>
__device__ __forceinline__ void select_digit(const uint32_t* hist, uint32_t k_rem, uint32_t* wsum,
                                             uint32_t* sel) {
    const int tid = threadIdx.x;
    if (tid == 0) {  // safe result should the counts ever be inconsistent
        sel[0] = 0;
        sel[1] = 0;
        sel[2] = 0;
    }
    uint32_t c = 0, incl = 0;
    if (tid < kRadix) {
        c = hist[kRadix - 1 - tid];
        incl = wave_incl_scan(c);
        if ((tid & 63) == 63) wsum[tid >> 6] = incl;
    }
    __syncthreads();
    if (tid < kRadix) {
        uint32_t off = 0;
#pragma unroll
        for (int w = 0; w < kRadix / 64; ++w) off += (w < (tid >> 6)) ? wsum[w] : 0u;
        incl += off;
        const uint32_t excl = incl - c;
        if (excl < k_rem && incl >= k_rem) {
            sel[0] = (uint32_t)(kRadix - 1 - tid);
            sel[1] = excl;
            sel[2] = c;
        }
    }
    __syncthreads();
}

// Descending bitonic sort of A[0..count) (count <= KMAX, KMAX a power of two).
template <int NT>
__device__ __forceinline__ void bitonic_desc(uint64_t* A, int count) {
    const int tid = threadIdx.x;
    int P = 1;
    while (P < count) P <<= 1;
    for (int i = count + tid; i < P; i += NT) A[i] = 0;  // 0 is never a real composite
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (P >> 1); i += NT) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const uint64_t a = A[lo], b = A[hi];
                const bool desc = (lo & size) == 0;
                if ((a < b) == desc) {
                    A[lo] = b;
                    A[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

// ----------------------------------------------------------------------------- row barrier

__device__ __forceinline__ void row_barrier(uint32_t* ctr, uint32_t target, uint32_t* err) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t spins = 0;
        while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > kSpinLimit) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
    __threadfence();
}

// ----------------------------------------------------------------------------- the tile

template <int NT, int EPT, int KMAX, bool MULTI>
__device__ __forceinline__ void process_tile(const Params& p, Smem<NT, EPT, KMAX>& s, int b, int tile) {
    constexpr int TILE = NT * EPT;
    constexpr int G4 = EPT / 4;  // float4 groups per lane
    constexpr int BW = Smem<NT, EPT, KMAX>::BWORDS;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;

    const int32_t len = p.lengths ? p.lengths[b] : p.max_len;
    const int32_t n = min(max(len, 0), p.max_len);
    const int64_t base = p.row_starts ? (int64_t)p.row_starts[b] : (int64_t)b * p.max_len;
    const int32_t k = p.k;
    const int32_t m = min(k, n);
    const int ntiles = MULTI ? max(1, (n + TILE - 1) / TILE) : 1;
    if (tile >= ntiles) return;
    const bool multi = MULTI && ntiles > 1;
    int32_t* oidx = p.out_idx + (int64_t)b * k;
    uint32_t* oval = p.out_val ? p.out_val + (int64_t)b * k : nullptr;

    __syncthreads();  // previous item of a persistent workgroup is done with LDS

    if (m == 0) {  // empty window: every slot is padding (single tile by construction)
        for (int q = tid; q < k; q += NT) {
            oidx[q] = -1;
            if (oval) oval[q] = kNegInfBits;
        }
        return;
    }

    uint32_t* rw = multi ? p.ws_zero + 1 + (int64_t)b * kRowZeroWords : nullptr;  // row words
    uint32_t* err = p.ws_zero;
    uint32_t bar_target = 0;

    const int32_t j0 = tile * TILE;
    const int32_t nt = min(TILE, n - j0);  // >= 1

    // ---------------------------------------------------------------- load (HBM, once)
    uint32_t key[EPT];
    {
        const uint32_t* src = p.scores + base + j0;
        const bool aligned = (((uintptr_t)src) & 15u) == 0;
#pragma unroll
        for (int v = 0; v < G4; ++v) {
            const int jl = (v * NT + tid) * 4;
            uint32_t u0 = 0, u1 = 0, u2 = 0, u3 = 0;
            if (jl < nt) {
                if (aligned) {
                    const uint4 q = *reinterpret_cast<const uint4*>(src + jl);
                    u0 = q.x; u1 = q.y; u2 = q.z; u3 = q.w;
                } else {
                    u0 = src[jl];
                    if (jl + 1 < nt) u1 = src[jl + 1];
                    if (jl + 2 < nt) u2 = src[jl + 2];
                    if (jl + 3 < nt) u3 = src[jl + 3];
                }
            }
            key[4 * v + 0] = key_of(u0);
            key[4 * v + 1] = key_of(u1);
            key[4 * v + 2] = key_of(u2);
            key[4 * v + 3] = key_of(u3);
        }
    }

    // Visit every valid register element: f(key, local index).
    auto for_each = [&](auto&& f) {
#pragma unroll
        for (int v = 0; v < G4; ++v) {
            const int lim = nt - v * NT * 4;
            if (lim <= 0) break;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int jl = (v * NT + tid) * 4 + c;
                if (tid * 4 + c < lim) f(key[4 * v + c], jl);
            }
        }
    };
    // Same, but every lane of the wave calls f (valid flag passed) -- for ballots.
    auto for_each_conv = [&](auto&& f) {
#pragma unroll
        for (int v = 0; v < G4; ++v) {
            const int lim = nt - v * NT * 4;
            if (lim <= 0) break;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int jl = (v * NT + tid) * 4 + c;
                f(key[4 * v + c], jl, tid * 4 + c < lim);
            }
        }
    };

    auto zero_whist = [&]() {
        uint32_t* w = &s.whist[0][0];
        for (int i = tid; i < Smem<NT, EPT, KMAX>::NW * kRadix; i += NT) w[i] = 0;
    };

    // Merge per-wave histograms; in multi mode also add into the row's global histogram
    // for `pass` and read the merged result back after the row barrier.
    auto merge_hist = [&](int pass) {
        __syncthreads();
        if (tid < kRadix) {
            uint32_t h = 0;
#pragma unroll
            for (int w = 0; w < Smem<NT, EPT, KMAX>::NW; ++w) h += s.whist[w][tid];
            s.lhist[tid] = h;
            s.hist[tid] = h;
            if (multi && h) atomicAdd(&rw[pass * kRadix + tid], h);
        }
        if (multi) {
            bar_target += (uint32_t)ntiles;
            row_barrier(&rw[4 * kRadix], bar_target, err);
            if (tid < kRadix)
                s.hist[tid] = __hip_atomic_load(&rw[pass * kRadix + tid], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    };

    // ---------------------------------------------------------------- pass 0: top digit
    if (tid < 8) s.ctr[tid] = 0;
    zero_whist();
    __syncthreads();
    for_each([&](uint32_t kk, int) { hist_add(s.whist[wave], kk >> 24); });
    merge_hist(0);
    select_digit<NT>(s.hist, (uint32_t)m, s.wsum, s.sel);
    uint32_t prefix = s.sel[0];
    uint32_t k_rem = (uint32_t)m - s.sel[1];
    const uint32_t d0 = prefix;
    const bool staged = s.lhist[d0] <= (uint32_t)p.stage_cap;
    __syncthreads();

    // Collect: digit > d0 are selected outright (into A); digit == d0 are candidates
    // (staged in LDS when they fit).
    for_each_conv([&](uint32_t kk, int jl, bool ok) {
        const uint32_t d = kk >> 24;
        const bool g = ok && d > d0;
        const uint32_t sa = claim_slot(g, &s.ctr[1]);
        if (g && sa < (uint32_t)KMAX) s.A[sa] = ((uint64_t)kk << 32) | (uint32_t)~(uint32_t)(j0 + jl);
        if (staged) {
            const bool cnd = ok && d == d0;
            const uint32_t sc = claim_slot(cnd, &s.ctr[0]);
            if (cnd && sc < (uint32_t)kStageCap) {
                s.skey[sc] = kk;
                s.sidx[sc] = (uint32_t)(j0 + jl);
            }
        }
    });
    __syncthreads();
    const uint32_t nstaged = staged ? min(s.ctr[0], (uint32_t)kStageCap) : 0u;

    // ---------------------------------------------------------------- passes 1..3: refine
#pragma unroll 1
    for (int pass = 1; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        zero_whist();
        __syncthreads();
        if (staged) {
            for (uint32_t i = tid; i < nstaged; i += NT) {
                const uint32_t kk = s.skey[i];
                if ((kk >> (shift + 8)) == prefix) hist_add(s.whist[wave], (kk >> shift) & 0xFFu);
            }
        } else {
            for_each([&](uint32_t kk, int) {
                if ((kk >> (shift + 8)) == prefix) hist_add(s.whist[wave], (kk >> shift) & 0xFFu);
            });
        }
        merge_hist(pass);
        select_digit<NT>(s.hist, k_rem, s.wsum, s.sel);
        prefix = (prefix << 8) | s.sel[0];
        k_rem -= s.sel[1];
        __syncthreads();
    }
    const uint32_t T = prefix;                    // exact threshold key
    const uint32_t need = min(k_rem, (uint32_t)m); // ties at T to keep (>= 1)
    const uint32_t cnt_gt = (uint32_t)m - need;   // selected elements strictly above T
    const uint32_t vT = bits_of(T);

    // ---------------------------------------------------------------- the rest of G
    if (staged) {
        for (uint32_t i0 = 0; i0 < nstaged; i0 += NT) {
            const uint32_t i = i0 + tid;
            const uint32_t kk = i < nstaged ? s.skey[i] : 0u;
            const bool g = i < nstaged && kk > T;
            const uint32_t sa = claim_slot(g, &s.ctr[1]);
            if (g && sa < (uint32_t)KMAX) s.A[sa] = ((uint64_t)kk << 32) | (uint32_t)~s.sidx[i];
        }
    } else {
        for_each_conv([&](uint32_t kk, int jl, bool ok) {
            const bool g = ok && (kk >> 24) == d0 && kk > T;
            const uint32_t sa = claim_slot(g, &s.ctr[1]);
            if (g && sa < (uint32_t)KMAX) s.A[sa] = ((uint64_t)kk << 32) | (uint32_t)~(uint32_t)(j0 + jl);
        });
    }

    // ---------------------------------------------------------------- boundary ties
    // Rank the tile's elements with key == T by index (bitmap over local positions),
    // offset by the ties of earlier tiles, keep ranks < need at slots cnt_gt + rank.
    for (int i = tid; i < BW; i += NT) s.bitmap[i] = 0;
    __syncthreads();
    auto mark = [&](uint32_t jl) {
        __hip_atomic_fetch_or(&s.bitmap[jl >> 5], 1u << (jl & 31u), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    if (staged) {
        for (uint32_t i = tid; i < nstaged; i += NT)
            if (s.skey[i] == T) mark(s.sidx[i] - (uint32_t)j0);
    } else {
        for_each([&](uint32_t kk, int jl) {
            if (kk == T) mark((uint32_t)jl);
        });
    }
    __syncthreads();
    {
        constexpr int WPT = (BW + NT - 1) / NT;
        uint32_t cnt = 0;
#pragma unroll
        for (int q = 0; q < WPT; ++q) {
            const int w = tid * WPT + q;
            if (w < BW) cnt += (uint32_t)__popc(s.bitmap[w]);
        }
        uint32_t total;
        uint32_t run = block_excl_scan<NT>(cnt, s.wsum, &total);
#pragma unroll
        for (int q = 0; q < WPT; ++q) {
            const int w = tid * WPT + q;
            if (w < BW) {
                s.wpre[w] = run;
                run += (uint32_t)__popc(s.bitmap[w]);
            }
        }
        if (tid == 0) s.ctr[2] = total;
    }
    __syncthreads();
    uint32_t tie_off = 0;
    if (multi) {
        if (tid == 0) p.ws_ecnt[(int64_t)b * p.tiles_per_row + tile] = s.ctr[2];
        bar_target += (uint32_t)ntiles;
        row_barrier(&rw[4 * kRadix], bar_target, err);
        if (tid == 0) {
            uint32_t o = 0;
            for (int t = 0; t < tile; ++t)
                o += __hip_atomic_load(&p.ws_ecnt[(int64_t)b * p.tiles_per_row + t], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            s.ctr[3] = o;
        }
        __syncthreads();
        tie_off = s.ctr[3];
    }
    if (tie_off < need) {
        for (int w = tid; w < BW; w += NT) {
            uint32_t word = s.bitmap[w];
            uint32_t r = tie_off + s.wpre[w];
            while (word && r < need) {
                const int bit = __ffs(word) - 1;
                word &= word - 1;
                const int32_t j = j0 + w * 32 + bit;
                oidx[cnt_gt + r] = j;
                if (oval) oval[cnt_gt + r] = vT;
                ++r;
            }
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- sort G and store
    const uint32_t nA = min(s.ctr[1], cnt_gt);
    if (!multi) {
        bitonic_desc<NT>(s.A, (int)nA);
        for (uint32_t q = tid; q < nA; q += NT) {
            const uint64_t c = s.A[q];
            oidx[q] = (int32_t)~(uint32_t)c;
            if (oval) oval[q] = bits_of((uint32_t)(c >> 32));
        }
        for (int q = m + tid; q < k; q += NT) {
            oidx[q] = -1;
            if (oval) oval[q] = kNegInfBits;
        }
        return;
    }

    // multi: publish this tile's G composites, last tile to arrive sorts the row.
    if (tid == 0) s.ctr[2] = nA ? atomicAdd(&rw[4 * kRadix + 2], nA) : 0u;
    __syncthreads();
    {
        uint64_t* st = p.ws_stage + (int64_t)b * k;
        const uint32_t gb = s.ctr[2];
        for (uint32_t q = tid; q < nA; q += NT)
            if (gb + q < cnt_gt) st[gb + q] = s.A[q];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&rw[4 * kRadix + 1], 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        s.ctr[3] = (old == (uint32_t)ntiles - 1u) ? 1u : 0u;
    }
    __syncthreads();
    if (s.ctr[3] == 0) return;
    __threadfence();
    {
        const uint64_t* st = p.ws_stage + (int64_t)b * k;
        for (uint32_t q = tid; q < cnt_gt; q += NT)
            s.A[q] = __hip_atomic_load(&st[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    bitonic_desc<NT>(s.A, (int)cnt_gt);
    for (uint32_t q = tid; q < cnt_gt; q += NT) {
        const uint64_t c = s.A[q];
        oidx[q] = (int32_t)~(uint32_t)c;
        if (oval) oval[q] = bits_of((uint32_t)(c >> 32));
    }
    for (int q = m + tid; q < k; q += NT) {
        oidx[q] = -1;
        if (oval) oval[q] = kNegInfBits;
    }
}

template <int NT, int EPT, int KMAX, bool MULTI>
__global__ __launch_bounds__(NT) void topk_ragged_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    auto& s = *reinterpret_cast<Smem<NT, EPT, KMAX>*>(smem_raw);
    const int64_t items = MULTI ? (int64_t)p.B * p.tiles_per_row : (int64_t)p.B;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int b = MULTI ? (int)(it / p.tiles_per_row) : (int)it;
        const int tile = MULTI ? (int)(it % p.tiles_per_row) : 0;
        process_tile<NT, EPT, KMAX, MULTI>(p, s, b, tile);
    }
}

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

}  // namespace detk
