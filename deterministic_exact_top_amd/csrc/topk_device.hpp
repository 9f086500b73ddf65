// topk_device.hpp -- gfx950 device code for exact, bitwise-deterministic ragged top-k.
//
// Result (SGLang PR #31115, PR summary and "Modifications"): per row, the k largest
// scores in canonical order -- score descending under the bitwise total order of the
// float bits, index ascending among bitwise-equal scores -- so the k-th boundary keeps
// the smallest indices of its tie set.  The pages' method: a coarse 8-bit radix
// histogram pass, MSB-first refinement to the exact threshold key, an index pass that
// picks the smallest-index tie subset, a sort of unique (score, index) composites; a
// threshold bin that overflows staging falls back to rescans, never dropping a
// candidate (same PR, summary and hardening commit).
//
// MI355X layout of the work:
//   * A workgroup owns a tile of up to NT*EPT consecutive elements of one row and keeps
//     it in VGPRs for its whole life: HBM is read once, with every buffer load of the
//     tile in flight together (out-of-range lanes read 0 from the buffer unit).
//   * Fast path (rows that fit one tile): a pivot P is taken from a 1024-element
//     sample (its r-th largest key, r set a few standard deviations above the expected
//     share of the top k).  One register pass sends keys > P to per-wave LDS candidate
//     regions and marks keys == P in an LDS bitmap of positions.  If at least min(k, n)
//     keys are >= P, the top k lie among them: candidates are bucketed by key (a
//     linear bucket index over [min candidate, max sample]), buckets get exclusive
//     offsets from an integer suffix scan, and each candidate's slot is its bucket
//     offset plus the number of bucket members with a larger (key, ~index) composite.
//     That one step both selects (slots >= k are dropped) and sorts.  Ties at P, when
//     needed, take the smallest positions from the bitmap.
//   * Exact path (pivot miss, oversized bucket, and rows split over several
//     workgroups): 8-bit MSD radix passes with per-wave LDS histograms merged into one
//     (lanes sharing the first active lane's bin are merged with one ballot and one
//     LDS add); threshold-bin candidates are staged in LDS when they fit, otherwise each
//     pass rescans the registers; boundary ties are ranked in index order with the
//     position bitmap; elements above the threshold are sorted as composites in LDS.
//   * Rows longer than one tile are split over co-resident workgroups that add their
//     integer histograms into the workspace with atomics (order-independent, hence
//     deterministic) and meet at per-row counters between passes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace detk {

constexpr int kRadix = 256;
constexpr int kStageCap = 4096;                 // exact path: LDS threshold-bin staging (entries)
constexpr int kBuckets = 4096;                  // fast path: buckets over the candidate key range
constexpr int kBucketBits = 12;
constexpr int kBucketLimit = 128;               // fast path: largest bucket ranked by comparisons
constexpr int kBucketLimitRow = 512;            // the same, ordering a split row's candidates
constexpr int kKeptSlack = 96;                  // fast path: kept candidates past KMAX that fit S
constexpr int kRankUnroll = 3;                  // composites compared per turn of the ranking loop
// Zero composites past the kept ones: a ranking loop running past a bucket's end reads
// lower buckets' composites or these, all smaller than its own, so it needs no bound.
template <bool LIMITED>
constexpr int rank_pad() { return (LIMITED ? kBucketLimit : kBucketLimitRow) + kRankUnroll; }
static_assert(kBuckets / 2 >= 5 * 256, "the packed bucket array doubles as the sample histograms");
constexpr uint32_t pow2_floor(uint32_t x) { return x < 2 ? x : 2 * pow2_floor(x / 2); }
// Fast path: pivot samples per lane.  Two, except where a lane holds no more than 8
// elements (the 1024-thread shapes of 4K and 8K rows): there two per lane would sample a
// half or a quarter of the row, and one keeps the candidates' excess small (3.5 sqrt(m n /
// s) + 4 n / s for s samples) at half the histogram work.  (A 4096-row decode batch: 9.8 ->
// 9.2 us.  One per lane on the 16K prefill tile overflows the candidate list.)
template <int EPT>
constexpr int samples_per_lane() { return EPT <= 8 ? 1 : 2; }
constexpr uint32_t kNegInfBits = 0xFF800000u;
// Per-row control words of the split-row path (a row spread over several workgroups).
// They are zero when a call starts, and the row's last arriving workgroup sets them back
// to zero, so a workspace zero-filled once stays ready for every later call.
constexpr int kRowCgt = 0;                      // candidates claimed (keys above P)
constexpr int kRowEq = 1;                       // keys equal to P
constexpr int kRowArrive = 2;                   // tiles done: the last to arrive orders the row
constexpr int kRowCtlWords = 4;                 // 16 bytes per row
constexpr int kSplitSamples = 8192;             // split rows: samples per row (4 per 16-byte load)
constexpr int kBufferWord3 = 0x00020000;        // raw buffer resource, gfx9-family data format

struct Params {
    const void* scores;         // float32 bits (VB 4) or 16-bit float bits (VB 2)
    const int32_t* row_starts;  // nullable
    const int32_t* lengths;     // nullable
    int32_t B;
    int32_t max_len;
    int32_t k;
    int32_t tiles_per_row;      // split-row kernel only
    int32_t stage_cap;          // <= kStageCap
    int32_t fast;               // 1: try the pivot fast path first
    int32_t small_batch;        // nonzero: no more workgroups than CUs (latency over issue
                                // slots: every wave selects the pivot digits itself)
    int32_t split_half;         // split-row kernel: nonzero, half the row samples (kSplitSamples / 2)
    int32_t* out_idx;
    void* out_val;              // nullable: VB-byte values
    uint32_t val_pad;           // the value written in padded slots (-inf of the format)
    uint32_t* ws_ctl;           // B * kRowCtlWords, zero on entry and on exit
    uint32_t* ws_ecnt;          // B * tiles_per_row: keys equal to P per tile
    uint2* ws_cand;             // B * cand_cap(KMAX): candidates (bits, position in the row)
    uint32_t* ws_tie;           // B * tiles_per_row * TILE / 32: per-tile bitmaps of keys == P
    // index written for a selected local index j (0 local, 1 offset, 2 page table)
    int32_t xf_mode;
    int32_t xf_page;            // page table: tokens per page
    int32_t xf_shift;           // page table: log2(tokens per page), or -1
    const int32_t* xf_offsets;  // offset: int32[B]
    const int32_t* xf_table;    // page table: row b's pages at xf_table[b * xf_stride ...]
    int64_t xf_stride;
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

// A list of (key, position) pairs kept as two separate LDS arrays: a pair is never one
// 64-bit store, which would make the register allocator pair every register-resident key
// with a spare register.  pos passes through an empty asm so it is formed only where the
// store happens.
struct PairList {
    uint32_t* key;
    uint32_t* pos;
    __device__ __forceinline__ void put(uint32_t i, uint32_t k, uint32_t p) const {
        asm volatile("" : "+v"(p));
        key[i] = k;
        pos[i] = p;
    }
    // Composite (key << 32) | ~pos: unique, and its descending order is the canonical order.
    __device__ __forceinline__ uint64_t composite(uint32_t i) const {
        return ((uint64_t)key[i] << 32) | (uint32_t)~pos[i];
    }
    __device__ __forceinline__ void set_composite(uint32_t i, uint64_t c) const {
        key[i] = (uint32_t)(c >> 32);
        pos[i] = ~(uint32_t)c;
    }
};

// threadIdx.x behind an empty asm: values derived from it are recomputed where they are
// used instead of being hoisted out of the persistent item loop into (spilled) registers.
__device__ __forceinline__ int opaque_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
// base + the number of lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below_plus(uint64_t m, uint32_t base) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, base));
}

// DPP lane moves (gfx9 encodings): row_shr:n shifts within 16-lane rows, row_bcast:15 /
// row_bcast:31 carry the last lane of a row / of the lower half into the next rows.
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes (Hillis-Steele within rows, then row carries).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp<kRowShr1, 0xF, true>(0, x);
    x += dpp<kRowShr2, 0xF, true>(0, x);
    x += dpp<kRowShr4, 0xF, true>(0, x);
    x += dpp<kRowShr8, 0xF, true>(0, x);
    x += dpp<kRowBcast15, 0xA, false>(0, x);
    x += dpp<kRowBcast31, 0xC, false>(0, x);
    return x;
}

// Wave-wide max / min, returned to every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    x = max(x, dpp<kRowShr1, 0xF, true>(0, x));
    x = max(x, dpp<kRowShr2, 0xF, true>(0, x));
    x = max(x, dpp<kRowShr4, 0xF, true>(0, x));
    x = max(x, dpp<kRowShr8, 0xF, true>(0, x));
    x = max(x, dpp<kRowBcast15, 0xA, false>(0, x));
    x = max(x, dpp<kRowBcast31, 0xC, false>(0, x));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
    const uint32_t y = ~x;  // min(x) = ~max(~x); zero-filled lanes stay neutral
    return ~wave_max(y);
}

__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Count one per active lane into h[d]; lanes sharing the first active lane's bin are
// merged into one add.  Must be called from the lanes to count (divergence allowed).
// (A second merge round, for the first lane outside that bin, measured slower: the extra
// instructions cost more than the same-address atomics they save.)
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
    if ((opaque_tid() & 63) == leader)
        base = __hip_atomic_fetch_add(counter, (uint32_t)__popcll(m), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
    base = __builtin_amdgcn_readlane(base, leader);
    return base + lanes_below(m);
}

// ----------------------------------------------------------------------------- loads

// Load one tile's raw bits: slot (v, c) of lane t holds window position
// (v * NT + t) * 4 + c.  The buffer resource covers exactly the tile's valid bytes, so
// slots past the window read 0 (callers mask them by position).  VB = 4: float32 bits,
// with 16-byte loads for a 16-byte aligned tile (a partially valid one never leaves the
// 16-byte chunk holding valid data), else 4-byte loads.  VB = 2: 16-bit float bits, each
// widened to (bits << 16) -- that 32-bit pattern keeps the 16-bit value's place in the
// total order and its ties (the key map's low half is fixed by the sign) -- with 8-byte
// loads for an 8-byte aligned tile, else 2-byte loads.  PART 0 loads the groups holding
// the pivot samples, PART 1 the others, PART 2 all of them (sample groups issued first).
template <int NT, int EPT>
constexpr bool sample_group(int v) {
    constexpr int SPL = samples_per_lane<EPT>();
    return v % (EPT / 4 >= SPL ? EPT / 4 / SPL : 1) == 0;
}

template <int NT, int EPT, int PART, int VB>
__device__ __forceinline__ void load_tile_part(uint32_t (&u)[EPT], const void* src, int nt) {
    static_assert(VB == 4 || VB == 2, "float32 or 16-bit scores");
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, nt * VB, kBufferWord3);
    const int tid = opaque_tid();
    constexpr int G4 = EPT / 4;
    // (one branch around all the loads: with a branch per load the compiler's wait counts
    // turn conservative, and the samples would wait for the whole tile)
    if ((((uintptr_t)src) & (4u * VB - 1u)) == 0) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if ((PART == 0 && pass == 1) || (PART == 1 && pass == 0)) continue;
#pragma unroll
            for (int v = 0; v < G4; ++v) {
                if (sample_group<NT, EPT>(v) != (pass == 0)) continue;
                // (the per-group offset rides in the scalar offset: one address VGPR for all)
                if constexpr (VB == 4) {
                    const auto q = __builtin_amdgcn_raw_buffer_load_b128(rsrc, tid * 16, v * NT * 16, 0);
                    u[4 * v + 0] = q[0];
                    u[4 * v + 1] = q[1];
                    u[4 * v + 2] = q[2];
                    u[4 * v + 3] = q[3];
                } else {
                    const auto q = __builtin_amdgcn_raw_buffer_load_b64(rsrc, tid * 8, v * NT * 8, 0);
                    u[4 * v + 0] = q[0] << 16;
                    u[4 * v + 1] = q[0] & 0xFFFF0000u;
                    u[4 * v + 2] = q[1] << 16;
                    u[4 * v + 3] = q[1] & 0xFFFF0000u;
                }
            }
        }
        if constexpr (VB == 2) {
            // With an odd element count the last element shares its 4-byte word with the two
            // bytes past the window; the range check zeroes such a word whole, so the lane
            // holding that element reloads it alone (never reading past the window).
            static_assert(VB == 4 || PART == 2, "16-bit tiles load whole");
            if (nt & 1) {  // uniform
                const int pl = nt - 1;
                const int slot = (pl / (NT * 4)) * 4 + (pl & 3);  // uniform register slot
                if (tid == (pl >> 2) % NT) {
                    const uint32_t x = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsrc, pl * 2, 0, 0) << 16;
#pragma unroll
                    for (int i = 0; i < EPT; ++i)
                        if (i == slot) u[i] = x;
                }
            }
        }
    } else {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if ((PART == 0 && pass == 1) || (PART == 1 && pass == 0)) continue;
#pragma unroll
            for (int v = 0; v < G4; ++v) {
                if (sample_group<NT, EPT>(v) != (pass == 0)) continue;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if constexpr (VB == 4)
                        u[4 * v + c] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, tid * 16 + c * 4, v * NT * 16, 0);
                    else
                        u[4 * v + c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsrc, tid * 8 + c * 2, v * NT * 8, 0)
                                       << 16;
                }
            }
        }
    }
}

template <int NT, int EPT, int VB>
__device__ __forceinline__ void load_tile(uint32_t (&u)[EPT], const void* src, int nt) {
    load_tile_part<NT, EPT, 2, VB>(u, src, nt);
}

// ----------------------------------------------------------------------------- shared memory

template <int NT, int EPT, int KMAX, int STAGE>
struct ExactSmem {
    static constexpr int NW = NT / 64;
    static constexpr int TILE = NT * EPT;
    static constexpr int BWORDS = TILE / 32;
    static constexpr int STAGE_CAP = STAGE;
    uint32_t whist[NW][kRadix];   // per-wave histograms
    uint32_t hist[kRadix];        // merged histogram of the current pass (row-global)
    uint32_t lhist[kRadix];       // this tile's own merged histogram
    uint32_t wsum[32];            // per-wave partials for block scans
    uint32_t sel[4];              // digit select: digit, count above, bin count
    uint32_t ctr[8];              // [0] staged, [1] A fill, [2] bcast, [3] bcast
    uint32_t bitmap[BWORDS];      // tie positions of this tile
    uint32_t wpre[BWORDS];        // exclusive prefix of popcounts over bitmap words
    uint32_t skey[STAGE];         // staged candidate keys
    uint32_t sidx[STAGE];         // staged candidate row indices
    uint32_t akey[KMAX];          // selected elements above T: keys
    uint32_t apos[KMAX];          //   and positions
};

// Candidate capacity (keys above the pivot) of the pivot path: 1.75 KMAX in LDS when one
// workgroup holds the row (the list still fits under the exact path's footprint, so four
// 16K-element rows share a CU; the pivot from two samples per lane overshoots by a few
// hundred keys); 2 KMAX in the workspace when several workgroups share a row.
template <int KMAX>
constexpr int cand_cap_single() { return 7 * KMAX / 4; }
template <int KMAX>
constexpr int cand_cap() { return 2 * KMAX; }

template <int NT, int EPT, int KMAX>
struct FastSmem {
    static constexpr int NW = NT / 64;
    static constexpr int TILE = NT * EPT;
    static constexpr int BWORDS = TILE / 32;
    static constexpr int CCAP = cand_cap_single<KMAX>();
    static constexpr int SCAP = KMAX + kKeptSlack;
    // (first, at LDS offset 0: the two candidate arrays sit at multiples of 256 bytes, so
    // one two-address LDS store writes a candidate with no offset arithmetic)
    union {
        struct {
            uint32_t bits[CCAP];  // candidates: raw bits (per-wave regions, then the shared
            uint32_t pos[CCAP];   //   overflow pool) and positions
        } cand;
        uint64_t S[SCAP + rank_pad<true>()];  // kept candidates as composites, grouped by
                                              // bucket, then zeros (written once every
                                              // candidate has been read into registers);
                                              // while choosing P, its first 2 KiB hold two
                                              // sample-digit histograms
        struct {
            uint64_t past_S[SCAP + rank_pad<true>()];
            uint64_t other[kBucketLimit];  // a plateau bucket's composites of other keys
            uint32_t bits[BWORDS];         //   and the positions holding its key
        } plateau;
    };
    static constexpr int CTL_WORDS = 24;
    uint32_t ctl[CTL_WORDS];      // control words, kCtl* below
    uint32_t wsum[32];
    uint32_t bitmap[BWORDS];      // positions with key == P
    uint32_t bucket[kBuckets / 2 + 2];  // 16-bit bucket counters, cursors and ends, two per
                                        // word; then a zero (the end above the top bucket)
    static_assert((CCAP * 4) % 256 == 0, "candidate arrays on 256-byte boundaries");
    static_assert(sizeof(plateau) <= sizeof(cand), "the plateau arrays fit past S");
    static_assert(sizeof(uint64_t) * SCAP >= sizeof(uint32_t) * 2 * kRadix, "S holds the sample histograms");
};

// A row split over several workgroups (one tile each): candidates live in the workspace,
// so LDS holds only the tile's tie bitmap, the buckets (which first hold the sample-digit
// histograms) and, in the row's last arriving workgroup, the kept composites it ranks.
template <int NT, int EPT, int KMAX>
struct SplitSmem {
    static constexpr int TILE = NT * EPT;
    static constexpr int BWORDS = TILE / 32;
    static constexpr int SCAP = cand_cap<KMAX>();
    uint32_t ctl[16];
    uint32_t wsum[32];
    uint32_t bitmap[BWORDS];
    uint32_t bucket[kBuckets / 2 + 2];
    uint64_t S[SCAP + rank_pad<false>()];
};

// Exact radix select over a whole row read from global memory in chunks, by one
// workgroup: the split row's fallback (its last arriving workgroup runs it alone).
template <int NT, int KMAX, int STAGE>
struct RowExactSmem {
    static constexpr int NW = NT / 64;
    static constexpr int STAGE_CAP = STAGE;
    uint32_t whist[NW][kRadix];   // per-wave histograms
    uint32_t hist[kRadix];        // merged histogram of the current pass
    uint32_t wsum[32];
    uint32_t sel[4];
    uint32_t ctr[8];              // [0] staged, [1] A fill
    uint32_t skey[STAGE];         // staged threshold-bin keys
    uint32_t sidx[STAGE];         //   and their row positions
    uint32_t akey[KMAX];          // selected elements above T: keys
    uint32_t apos[KMAX];          //   and positions
};

struct NoSmem {};

// Exact-path staging: smaller in one-workgroup-per-row kernels so that the LDS footprint
// lets three rows share a CU, and four for the 16K-element tile (1,248 entries keep its
// exact path at 40,880 bytes, the most that leaves room for four workgroups; more
// survivors than that only fall back to a rescan).
template <int NT, int EPT>
constexpr int stage_entries() { return (NT == 512 && EPT == 32) ? 1248 : 2560; }
constexpr int kRowStageEntries = 3072;  // the whole-row exact fallback's staging

// LDS of one workgroup.  Both kernels hold the one-tile path (pivot path, exact fallback);
// the split-row kernel also holds the split tile's and the whole-row fallback's layouts.
template <int NT, int EPT, int KMAX, bool MULTI>
union SmemAll {
    ExactSmem<NT, EPT, KMAX, stage_entries<NT, EPT>()> exact;
    FastSmem<NT, EPT, KMAX> fast;
    typename std::conditional<MULTI, SplitSmem<NT, EPT, KMAX>, NoSmem>::type split;
    typename std::conditional<MULTI, RowExactSmem<NT, KMAX, kRowStageEntries>, NoSmem>::type rexact;
};

// ----------------------------------------------------------------------------- block helpers

// Zero N words of LDS with the whole workgroup (trip count fixed at compile time).
template <int NT, int N>
__device__ __forceinline__ void block_zero(uint32_t* p) {
    const int tid = opaque_tid();
    if constexpr (N % 4 == 0 && N / 4 >= NT) {
        // (a zero made here: a zero vector hoisted out of the row loop gets spilled, and its
        // reload from scratch would wait for every outstanding tile load)
        uint32_t z = 0;
        asm volatile("" : "+v"(z));
#pragma unroll
        for (int i = 0; i < (N / 4 + NT - 1) / NT; ++i) {
            const int q = tid + i * NT;
            if ((N / 4) % NT == 0 || q < N / 4) reinterpret_cast<uint4*>(p)[q] = make_uint4(z, z, z, z);
        }
    } else {
#pragma unroll
        for (int i = 0; i < (N + NT - 1) / NT; ++i) {
            const int q = tid + i * NT;
            if (N % NT == 0 || q < N) p[q] = 0u;
        }
    }
}


// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.  One
// barrier: `wsum` must not be written again before the caller's next barrier.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum, uint32_t* total) {
    const int tid = opaque_tid();
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
    return off + incl - x;
}

// Pick the bin holding the k_rem-th largest key: scan bins 255..0; writes sel[] =
// {digit, count strictly above the digit, count of the digit}.  All threads call.
template <int NT>
__device__ __forceinline__ void select_digit(const uint32_t* hist, uint32_t k_rem, uint32_t* wsum,
                                             uint32_t* sel) {
    const int tid = opaque_tid();
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

// The same selection done by one wave alone, with no barrier, on a complete 256-bin
// histogram (every wave that calls it gets the same, wave-uniform answer).  Lane l owns
// bins 255 - 4l .. 252 - 4l.  Returns the digit; *above = count in higher bins, *count =
// the digit's count (all zero should the counts ever be inconsistent).
__device__ __forceinline__ uint32_t wave_select_digit(const uint32_t* hist, uint32_t r, uint32_t* above,
                                                      uint32_t* count) {
    const int lane = (opaque_tid() & 63);
    const uint4 q = *reinterpret_cast<const uint4*>(hist + 252 - 4 * lane);
    const uint32_t c0 = q.w, c1 = q.z, c2 = q.y, c3 = q.x;  // bins 255 - 4l, 254 - 4l, 253 - 4l, 252 - 4l
    const uint32_t t3 = c0 + c1 + c2 + c3;
    const uint32_t incl = wave_incl_scan(t3);
    const uint32_t e0 = incl - t3;       // keys in bins above this lane's
    const uint32_t e1 = e0 + c0, e2 = e1 + c1, e3 = e2 + c2;
    const uint64_t hit = __ballot(e0 < r && incl >= r);
    const uint32_t i = e1 >= r ? 0u : e2 >= r ? 1u : e3 >= r ? 2u : 3u;
    const uint32_t d = 255u - 4u * (uint32_t)lane - i;
    const uint32_t ab = i == 0 ? e0 : i == 1 ? e1 : i == 2 ? e2 : e3;
    const uint32_t ct = i == 0 ? c0 : i == 1 ? c1 : i == 2 ? c2 : c3;
    if (hit == 0) {
        *above = 0;
        *count = 0;
        return 0;
    }
    const int src = __ffsll((unsigned long long)hit) - 1;
    *above = __builtin_amdgcn_readlane(ab, src);
    *count = __builtin_amdgcn_readlane(ct, src);
    return __builtin_amdgcn_readlane(d, src);
}

// A plain LDS array of composites, with PairList's accessors.
struct U64List {
    uint64_t* a;
    __device__ __forceinline__ uint64_t composite(uint32_t i) const { return a[i]; }
    __device__ __forceinline__ void set_composite(uint32_t i, uint64_t c) const { a[i] = c; }
};

// x of lane ^ S: S = 1, 2, 8 one DPP move (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_ror:8), S = 4 two (row_half_mirror gives lane ^ 7, then quad_perm [3,2,1,0] lane ^ 3),
// S = 16, 32 a row swap (v_permlane16_swap / v_permlane32_swap of x with itself: each lane's
// partner value lands in one of the two results).  No LDS traffic.
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
    if constexpr (S == 1) return dpp<0xB1, 0xF, false>(x, x);
    else if constexpr (S == 2) return dpp<0x4E, 0xF, false>(x, x);
    else if constexpr (S == 4) {
        const uint32_t m = dpp<0x141, 0xF, false>(x, x);
        return dpp<0x1B, 0xF, false>(m, m);
    } else if constexpr (S == 8) return dpp<0x128, 0xF, false>(x, x);
    else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        static_assert(S == 32, "strides within a wave");
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}
template <int S>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t x, int lane) {
    return ((uint64_t)lane_xor<S>((uint32_t)(x >> 32), lane) << 32) | lane_xor<S>((uint32_t)x, lane);
}

// Bitonic compare-exchange stages on registers: a wave holds an aligned block of 128
// elements, lane l elements e0 = block + l (v0) and e0 + 64 (v1).  A pair (lo, lo + s) of
// merge `size` keeps the larger composite at lo when lo & size == 0 (descending), else the
// smaller.  Stride 64 pairs a lane's own two elements; smaller strides pair lanes l, l ^ s.
template <int S>
__device__ __forceinline__ void reg_stage(uint64_t& v0, uint64_t& v1, int e0, int lane, int size) {
    const uint64_t p0 = lane_xor64<S>(v0, lane), p1 = lane_xor64<S>(v1, lane);
    const bool lo = (lane & S) == 0;
    const bool m0 = ((e0 & size) == 0) == lo;  // this lane keeps the larger of the pair
    const bool m1 = (((e0 + 64) & size) == 0) == lo;
    // (one compare each: composites are unique, and equal pairs are padding zeros)
    v0 = (v0 > p0) == m0 ? v0 : p0;
    v1 = (v1 > p1) == m1 ? v1 : p1;
}
__device__ __forceinline__ void reg_merge(uint64_t& v0, uint64_t& v1, int e0, int lane, int size) {
    if (size > 64) {  // stride 64: within the lane
        const bool m = (e0 & size) == 0;
        const uint64_t hi = max(v0, v1), lo = min(v0, v1);
        v0 = m ? hi : lo;
        v1 = m ? lo : hi;
    }
    if (size > 32) reg_stage<32>(v0, v1, e0, lane, size);
    if (size > 16) reg_stage<16>(v0, v1, e0, lane, size);
    if (size > 8) reg_stage<8>(v0, v1, e0, lane, size);
    if (size > 4) reg_stage<4>(v0, v1, e0, lane, size);
    if (size > 2) reg_stage<2>(v0, v1, e0, lane, size);
    reg_stage<1>(v0, v1, e0, lane, size);
}

// Descending bitonic sort of the composites of A[0..count) (count <= KMAX), padded to a
// power of two P with composite 0, which no real element has (~pos != 0).
// Every stage of stride <= 64 runs in registers (reg_merge): each wave takes aligned
// 128-element blocks, and the merges of sizes 2 .. 128 run in one pass over a block (loaded
// and stored once).  A merge of size >= 256 first takes its stages of stride >= 128 through
// LDS (thread i takes the pair starting at 2i - (i mod stride), a workgroup barrier after
// each), then one register pass for strides 64 .. 1.  For 2048 entries: 10 LDS stages
// instead of 66.  Elements past P are never paired with ones below it (merges stay within
// aligned blocks of their size <= P), so a block's lanes past P only hold zeros.
template <int NT, class List>
__device__ __forceinline__ void bitonic_desc(const List& A, int count) {
    static_assert(NT % 64 == 0 && NT >= 128, "whole waves");
    const int tid = opaque_tid();
    const int lane = tid & 63, wave = tid >> 6;
    int P = 1;
    while (P < count) P <<= 1;
    for (int i = count + tid; i < P; i += NT) A.set_composite(i, 0);
    __syncthreads();
    auto reg_pass = [&](int size_lo, int size_hi) {
        for (int blk = wave; blk * 128 < P; blk += NT / 64) {
            const int e0 = blk * 128 + lane;
            uint64_t v0 = e0 < P ? A.composite(e0) : 0ull;
            uint64_t v1 = e0 + 64 < P ? A.composite(e0 + 64) : 0ull;
            for (int size = size_lo; size <= size_hi; size <<= 1) reg_merge(v0, v1, e0, lane, size);
            if (e0 < P) A.set_composite(e0, v0);
            if (e0 + 64 < P) A.set_composite(e0 + 64, v1);
        }
    };
    auto stage = [&](int size, int stride) {
        for (int i = tid; i < (P >> 1); i += NT) {
            const int lo = 2 * i - (i & (stride - 1));
            const int hi = lo + stride;
            const uint64_t a = A.composite(lo), b = A.composite(hi);
            const bool desc = (lo & size) == 0;
            if ((a < b) == desc) {
                A.set_composite(lo, b);
                A.set_composite(hi, a);
            }
        }
    };
    reg_pass(2, P < 128 ? P : 128);
    for (int size = 256; size <= P; size <<= 1) {
        __syncthreads();
        for (int stride = size >> 1; stride >= 128; stride >>= 1) {
            stage(size, stride);
            __syncthreads();
        }
        reg_pass(size, size);
    }
    __syncthreads();
}

// The same on a plain array of composites.
template <int NT>
__device__ __forceinline__ void bitonic_desc_u64(uint64_t* A, int count) {
    bitonic_desc<NT>(U64List{A}, count);
}

// base[i] = v, addressed as a 32-bit byte offset from the (wave-uniform) row base, which
// the store takes as its scalar base: no 64-bit address arithmetic per element.
template <class T>
__device__ __forceinline__ void store_at(T* base, uint32_t i, T v) {
    *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + i * (uint32_t)sizeof(T)) = v;
}

// A row's output values: put(slot, bits) writes a selected score from its 32-bit register
// pattern (16-bit scores sit in the top half of theirs), pad(slot) the padding value.
// Uniform across the launch.
struct ValOut {
    void* base;     // nullptr: the caller wants no values
    uint32_t padv;  // the padding pattern (the format's -inf)
    bool half;      // 16-bit values
    __device__ __forceinline__ explicit operator bool() const { return base != nullptr; }
    __device__ __forceinline__ void put(uint32_t slot, uint32_t bits32) const {
        if (half) store_at(static_cast<uint16_t*>(base), slot, (uint16_t)(bits32 >> 16));
        else store_at(static_cast<uint32_t*>(base), slot, bits32);
    }
    __device__ __forceinline__ void pad(uint32_t slot) const {
        if (half) store_at(static_cast<uint16_t*>(base), slot, (uint16_t)padv);
        else store_at(static_cast<uint32_t*>(base), slot, padv);
    }
};

// Write the padding slots [m, k) of one output row.
template <int NT>
__device__ __forceinline__ void write_padding(int32_t* oidx, const ValOut& ov, int m, int k) {
    for (int q = m + opaque_tid(); q < k; q += NT) {
        store_at(oidx, (uint32_t)q, -1);
        if (ov) ov.pad((uint32_t)q);
    }
}

// ----------------------------------------------------------------------------- row arrival

// Wait until this wave's outstanding global stores and atomics have completed (reached
// the L2, or memory for device-scope atomics), so that a release issued afterwards by
// another wave of the workgroup covers them.  A workgroup barrier alone does not wait
// for them.
__device__ __forceinline__ void wait_global_writes() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One tile of a split row is done: count it on the row's ticket counter and return, in
// every thread, whether this workgroup was the last of the row's `ntiles` to arrive.
// Every wave first waits for its own global writes; then one thread adds one with
// release semantics at device scope (the XCD's L2 is written back, so the workgroup's
// writes reach the other XCDs) and acquire semantics (the last arriver then sees every
// other tile's writes).  Nothing ever waits for another workgroup, so the launch needs
// no co-residency and cannot stall.  flag: one LDS word.
__device__ __forceinline__ bool arrive_last(uint32_t* ctr, uint32_t ntiles, uint32_t* flag) {
    wait_global_writes();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        *flag = old == ntiles - 1u ? 1u : 0u;
    }
    __syncthreads();
    return *flag != 0u;
}

// ----------------------------------------------------------------------------- row context

// The index a row writes for its selected local index j: j itself, an offset plus j (an
// index into a packed buffer), or the physical slot of the row's j-th token through its
// page table (pages of `ps` tokens).  The mode is uniform across the launch.
struct IndexOut {
    int32_t mode;
    int32_t off;
    int32_t ps;
    int32_t shift;
    const int32_t* pt;
    __device__ __forceinline__ int32_t operator()(uint32_t j) const {
        if (mode == 0) return (int32_t)j;
        if (mode == 1) return off + (int32_t)j;
        const uint32_t page = shift >= 0 ? j >> shift : j / (uint32_t)ps;
        const uint32_t within = j - page * (uint32_t)ps;
        return pt[page] * ps + (int32_t)within;
    }
};

struct RowCtx {
    int b, tile, ntiles;
    int32_t n, m, k, nt, j0;
    int64_t base;
    int32_t* oidx;
    ValOut ov;
    IndexOut xo;
    bool wave_select;  // every wave selects the pivot digits itself (no publishing barrier)
};

// ----------------------------------------------------------------------------- fast path

constexpr uint32_t kRefineAbove = 24;         // pivot: resolve one more sample digit past this bin count
constexpr uint32_t kKeyPosInf = 0xFF800000u;  // key of +inf; keys at or above it are +inf and +NaN

// Fast-path LDS control words.
enum : int {
    kCtlSmaxAll = 1,    // largest sample key
    kCtlLo = 2,         // least sample key above P (all ones when there is none)
    kCtlBt = 3,         // threshold bucket
    kCtlKept = 4,       // kept candidates
    kCtlMaxBucket = 5,  // set when some bucket is longer than the ranking limit
    kCtlSel = 6,        // [6..8] sample digit select: digit, count above, bin count
    kCtlEq = 9,         // keys equal to P
    kCtlSmaxFin = 10,   // largest sample key below key(+inf)
    kCtlBase = 11,      // several workgroups: this tile's first candidate slot in the row
    kCtlLast = 12,      // several workgroups: this tile arrived last
    kCtlRowCgt = 13,    // several workgroups: the row's candidates (last arriver)
    kCtlPool = 15,      // one workgroup: slots claimed in the candidate pool
    kCtlBinNotMin = 0,  // pivot: max of ~key over the samples in the selected 16-bit bin
    kCtlBinMax = 14,    // pivot: max of key over the same samples
    // one workgroup (FastSmem only): a plateau bucket
    kCtlPFirst = 16,    // [16..17] as one 64-bit word: max of (~position << 32 | key) over the
                        //   long bucket, i.e. its first element in position order and that key
    kCtlLongN = 18,     // buckets longer than the ranking limit
    kCtlPOther = 19,    // the bucket's composites of other keys
    kCtlPCount = 20,    // (its keys above the plateau key) << 16 | (those equal to it)
};

// Real samples among a tile's nt elements (uniform): slot i * EPT / SPL of each lane
// (SPL = samples_per_lane), for the lanes whose slot lies inside the tile.
template <int NT, int EPT>
__device__ __forceinline__ int tile_samples(int32_t nt) {
    constexpr int SPL = samples_per_lane<EPT>();
    int ns = 0;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int slot = i * (EPT / SPL);
        const int lim = nt - (slot / 4) * NT * 4 - slot % 4;
        ns += min(max((lim + 3) / 4, 0), NT);
    }
    return ns;
}

// This lane's samples: register slots i * EPT / SPL (the groups load_tile issues first).
// Slots past the tile give key 0, the least key, which never outranks a real sample at
// the ranks asked for.
template <int NT, int EPT>
__device__ __forceinline__ void take_samples(const uint32_t (&u)[EPT], int32_t nt,
                                             uint32_t (&sk)[samples_per_lane<EPT>()]) {
    constexpr int SPL = samples_per_lane<EPT>();
    const int t4 = opaque_tid() * 4;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        const int slot = i * (EPT / SPL);
        sk[i] = t4 + ((slot / 4) * NT * 4 + slot % 4) < nt ? key_of(u[slot]) : 0u;
    }
}

// Sample rank whose key bounds the m-th largest of n keys from below with high
// probability: the expected rank of that key among nsamp samples plus 3.5 standard
// deviations plus 4.
// (Only the path a row takes depends on it, never the result, so the hardware's
// reciprocal and square-root approximations serve: a few instructions instead of the
// correctly rounded sequences.)
__device__ __forceinline__ uint32_t pivot_rank(int nsamp, int32_t m, int32_t n) {
    const float expct = (float)nsamp * (float)m * __builtin_amdgcn_rcpf((float)n);
    return (uint32_t)ceilf(expct + 3.5f * __builtin_amdgcn_sqrtf(expct) + 4.0f);
}

// P = the key prefix of the rr-th largest sample, MSB first, one 8-bit digit per pass;
// a pass runs past the second only while the selected bin still holds more than
// kRefineAbove samples, so after four passes P is that sample's key itself.  When the
// bin selected by the second pass holds more than kRefineAbove samples that all have one
// key (a plateau of equal scores), that key is P at once, as four passes would make it
// (ctl[kCtlBinNotMin] and ctl[kCtlBinMax], zero on entry, collect the bin's extremes
// behind one barrier instead of the two passes' four).  Pass p
// counts into hist + 256 (p % NH), NH regions zeroed beforehand with a barrier behind
// (with NH < 4 a region is zeroed again, behind one more barrier, before its reuse); no
// pass waits for the previous one's histogram to be cleared, and every wave then
// selects the digit on its own.  merge(pass, h) turns this workgroup's histogram into
// the one the select reads (nothing to do for a single workgroup, a device-wide sum
// over the row's tiles otherwise).  Every wave, and every workgroup of a row, takes the
// same decisions.  With sel (three LDS words), wave 0 alone selects each digit and
// publishes it behind one more barrier, instead of every wave repeating the selection.
// FLOOR: the first pass counts only the samples at or above `floor`, a bin boundary
// known to lie at or below the rr-th largest sample (the ranks from the top, and so the
// pivot, are those of all the samples).
// spl (uniform): the samples that count are sk[0 .. spl); the rest hold key 0 and are
// skipped by the histograms.
template <int NT, int NH, bool FLOOR = false, int SPL, class Merge>
__device__ __forceinline__ uint32_t pivot_passes(const uint32_t (&sk)[SPL], uint32_t rr, uint32_t* hist,
                                                 Merge&& merge, uint32_t* ctl, int* passes = nullptr,
                                                 uint32_t* sel = nullptr, uint32_t floor = 0, int spl = SPL) {
    const int tid = opaque_tid();
    uint32_t prefix = 0, r_rem = rr, P = 0, cnt = 0xFFFFFFFFu;
    int pass = 0;
#pragma unroll 1
    for (; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (pass >= 2 && cnt <= kRefineAbove) break;  // uniform: bin resolved
        if (pass == 2) {  // uniform: a crowded 16-bit bin; one key only?
            uint32_t nmn = 0, mx = 0;
#pragma unroll
            for (int i = 0; i < SPL; ++i) {
                const bool in = (sk[i] >> 16) == prefix;
                nmn = in ? max(nmn, ~sk[i]) : nmn;
                mx = in ? max(mx, sk[i]) : mx;
            }
            nmn = wave_max(nmn);
            mx = wave_max(mx);
            if ((tid & 63) == 0) {
                __hip_atomic_fetch_max(&ctl[kCtlBinNotMin], nmn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_max(&ctl[kCtlBinMax], mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            __syncthreads();
            const uint32_t lo = ~__builtin_amdgcn_readfirstlane(ctl[kCtlBinNotMin]);
            if (lo == __builtin_amdgcn_readfirstlane(ctl[kCtlBinMax])) {  // uniform
                P = lo;
                pass = 4;
                break;
            }
        }
        uint32_t* h = hist + (pass % NH) * kRadix;
        if (pass >= NH) {  // every wave has selected from this region's previous pass
            if (tid < kRadix) h[tid] = 0;
            __syncthreads();
        }
        // (lanes sharing a bin merge into one atomic: scores concentrate on few digits,
        // and same-address LDS atomics serialise)
#pragma unroll
        for (int i = 0; i < SPL; ++i)
            if (i < spl && (pass == 0 ? (!FLOOR || sk[i] >= floor) : (sk[i] >> (shift + 8)) == prefix))
                hist_add(h, (sk[i] >> shift) & 0xFFu);
        __syncthreads();
        merge(pass, h);
        uint32_t above, d;
        if (sel) {
            if (tid < 64) {
                d = wave_select_digit(h, r_rem, &above, &cnt);
                if (tid == 0) {
                    sel[0] = d;
                    sel[1] = above;
                    sel[2] = cnt;
                }
            }
            __syncthreads();
            d = __builtin_amdgcn_readfirstlane(sel[0]);  // (uniform: kept scalar)
            above = __builtin_amdgcn_readfirstlane(sel[1]);
            cnt = __builtin_amdgcn_readfirstlane(sel[2]);
        } else {
            d = wave_select_digit(h, r_rem, &above, &cnt);
        }
        prefix = (prefix << 8) | d;
        r_rem -= above;
        P = prefix << shift;
    }
    if (passes) *passes = pass;
    return P;
}

// Visit the tile's register slots: f(x, slot constant c, group v, valid, 4 * thread).
// Full groups skip the per-lane bound check.
template <int NT, int EPT, class F>
__device__ __forceinline__ void visit_slots(const uint32_t (&u)[EPT], int32_t nt, F&& f) {
    const int t4 = opaque_tid() * 4;
#pragma unroll
    for (int v = 0; v < EPT / 4; ++v) {
        const int lim = nt - v * NT * 4;
        if (lim <= 0) break;
        if (lim >= NT * 4) {
#pragma unroll
            for (int c = 0; c < 4; ++c) f(u[4 * v + c], c, v, true, t4);
        } else {
            const int llim = lim - t4;
#pragma unroll
            for (int c = 0; c < 4; ++c) f(u[4 * v + c], c, v, c < llim, t4);
        }
    }
}

// The least key of a tile's nt elements, exact (the same value in every thread).  word:
// an LDS word that is zero, with a barrier behind, on entry (it collects the maximum of
// ~key).  Contains a barrier.
template <int NT, int EPT>
__device__ __forceinline__ uint32_t tile_min_key(const uint32_t (&u)[EPT], int32_t nt, uint32_t* word) {
    uint32_t nk = 0;
    visit_slots<NT, EPT>(u, nt, [&](uint32_t x, int, int, bool ok, int) { nk = ok ? max(nk, ~key_of(x)) : nk; });
    nk = wave_max(nk);
    if ((opaque_tid() & 63) == 0) __hip_atomic_fetch_max(word, nk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    return ~__builtin_amdgcn_readfirstlane(*word);
}

// Keys above P, compared on the raw bits when P >= key(+0.0) (then only non-negative
// patterns qualify and their signed order is the key order).
struct AboveP {
    uint32_t P;
    int32_t pr;  // P's float bits when P >= key(+0.0)
    __device__ explicit AboveP(uint32_t p) : P(p), pr((int32_t)(p & 0x7FFFFFFFu)) {}
    template <bool POS>
    __device__ __forceinline__ bool gt(uint32_t x) const { return POS ? (int32_t)x > pr : key_of(x) > P; }
    template <bool POS>
    __device__ __forceinline__ bool eq(uint32_t x) const { return POS ? x == (uint32_t)pr : key_of(x) == P; }
};

// Bucket of a key: linear in the key over [L, U] (keys below L share bucket 0, keys
// above U the top bucket); monotone, so bucket order never contradicts key order.
// TOP (rows split over workgroups): keys of +inf and NaNs get the top kTopBuckets buckets
// of their own -- +inf one, NaN payloads linear over the rest -- so a cluster of them
// (equal bits are ranked against their whole bucket) is not one long bucket; the finite
// keys share the others.
constexpr int kTopBuckets = 64;
template <bool TOP>
struct BucketMapT {
    static constexpr uint32_t NB = TOP ? kBuckets - kTopBuckets : kBuckets;  // buckets of finite keys
    uint32_t L;
    int sh;
    __device__ BucketMapT(uint32_t lo, uint32_t hi) : L(lo), sh(max(0, (32 - __clz(hi - lo)) - kBucketBits)) {}
    __device__ __forceinline__ uint32_t operator()(uint32_t kx) const {
        const uint32_t f = min((max(kx, L) - L) >> sh, NB - 1u);
        if constexpr (!TOP) {
            return f;
        } else {
            const uint32_t t =
                NB + (kx == kKeyPosInf ? 0u : 1u + min((kx - kKeyPosInf - 1u) >> 17, (uint32_t)kTopBuckets - 2u));
            return kx >= kKeyPosInf ? t : f;
        }
    }
};
using BucketMap = BucketMapT<false>;
// Count one key into the 16-bit bucket counters (bucket b lives in word b / 2, bits
// 16 * (b % 2) and up).
__device__ __forceinline__ void bucket_count(uint32_t* bucket, uint32_t bk) {
    lds_add(&bucket[bk >> 1], 1u << ((bk & 1u) << 4));
}

// Order the candidates: the m largest of the c_gt candidates (all of them when
// c_gt <= m) go to slots [0, min(m, c_gt)) in canonical order through
// emit(slot, xo(position), bits).  Each thread owns up to CPT candidates: valid(i) says
// whether its i-th exists, src(i) gives it as (raw bits, position), and live(i)
// (wave-uniform) whether some lane of the wave has an i-th candidate.
// The bucket (BucketMap) holding the m-th largest is the threshold; kept candidates
// (buckets at or above it) go to S grouped by bucket as composites
// (key << 32 | ~position), which are unique and whose descending order is the canonical
// order; a kept candidate's slot is its bucket's start plus the number of larger
// composites in its bucket.
// COUNTED: the caller has already counted every candidate into the bucket array (a
// barrier behind); otherwise the bucket array is zero (a barrier behind) and counted here.
// Every candidate is read into registers before the first barrier in here, so S may
// overlay the memory src reads.
// ctl[kCtlBt..kCtlMaxBucket] are zero on entry (kCtlMaxBucket becomes one more than the
// highest bucket longer than the limit, 0 when there is none); so are ctl[kCtlPFirst..
// kCtlPCount] when PBW > 0.  Only kept buckets (at or above the threshold) count as long.
// scattered() runs once the kept composites are in S, past the last point of returning
// false.
// LIMITED: returns false, having emitted nothing, when more than SCAP candidates are
// kept or a bucket holds more than kBucketLimit.  Otherwise c_gt <= SCAP (a power of
// two) is the caller's, and when a bucket holds more than kBucketLimitRow the kept
// composites are ordered by a bitonic sort of S instead (ranking compares each element
// with its whole bucket).
// bucket has kBuckets / 2 + 1 words (the last one is cleared here) and S has
// SCAP + rank_pad<LIMITED>() entries (those past the kept ones are cleared here).
// sort_long (LIMITED only): when a bucket is too long but at most SORT_MAX candidates are
// kept, sort them instead of returning false (a row output whole keeps at most KMAX).
// PBW > 0 (LIMITED only; positions are a tile's, below 32 PBW): a plateau bucket.  When
// exactly one kept bucket is longer than the limit, its key X is that of its first element
// in position order, and at most kBucketLimit of its elements have another key, those go
// to pl->other and are ranked among themselves (an element below X also passes all of
// X's); the elements of key X are not ranked: they take slots pl->base .. in position
// order, the caller emitting them from the bitmap pl->bits (PBW words) with pl->need of
// them inside the output.  Every key gives the same output; X a majority key makes the
// bucket cheap.  pl->on says whether this happened.
struct PlateauBucket {
    uint64_t* other;  // kBucketLimit composites
    uint32_t* bits;   // position bitmap
    bool on;
    uint32_t key, base, need;
};
template <int NT, int SCAP, int CPT, bool LIMITED, bool COUNTED, int PBW, class Src, class Valid, class Live,
          class Map, class Emit, class Scattered>
__device__ __forceinline__ bool bucket_rank(uint32_t* bucket, uint64_t* S, uint32_t* wsum, uint32_t* ctl, Src&& src,
                                            Valid&& valid, Live&& live, uint32_t c_gt, uint32_t m, bool ties,
                                            const Map& bucket_of, const IndexOut& xo, Emit&& emit,
                                            Scattered&& scattered, bool sort_long = false,
                                            PlateauBucket* pl = nullptr) {
    static_assert(PBW == 0 || LIMITED, "plateau buckets only where positions are a tile's");
    if constexpr (PBW > 0) pl->on = false;
    constexpr int BPT = kBuckets / NT;  // buckets per thread in the scan
    static_assert(BPT % 2 == 0, "threads own whole words of bucket counters");
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const uint32_t mlim = min(m, c_gt);  // slots the candidates fill
    if (tid == 0) bucket[kBuckets / 2] = 0;  // the end above the top bucket (read past a barrier)

    // ---- this thread's candidates, into registers as (key, position), with their buckets
    // (computed once for the count and the scatter; only for entries some lane of the
    // wave holds)
    // (keys and buckets stay in registers only for a few candidates per thread; with
    // more, the count and the scatter each derive them from the raw bits rather than spill)
    constexpr bool KEEP = CPT <= 8;
    uint2 cv[CPT];
    uint32_t bk[KEEP ? CPT : 1];
#pragma unroll
    for (int i = 0; i < CPT; ++i) cv[i] = valid(i) ? src(i) : make_uint2(0u, 0u);
    if constexpr (KEEP) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            bk[i] = 0;
            if (live(i)) {  // uniform
                cv[i].x = key_of(cv[i].x);
                bk[i] = bucket_of(cv[i].x);
            }
        }
    }
    auto key_at = [&](int i) -> uint32_t {
        if constexpr (KEEP) return cv[i].x;
        else return key_of(cv[i].x);
    };
    auto bucket_at = [&](int i) -> uint32_t {
        if constexpr (KEEP) return bk[i];
        else return bucket_of(key_of(cv[i].x));
    };

    // ---- counts
    if (!COUNTED) {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if (valid(i)) bucket_count(bucket, bucket_at(i));
        __syncthreads();
    }

    // ---- suffix scan: bucket starts.  Thread t owns buckets [kBuckets - (t + 1) * BPT,
    // kBuckets - t * BPT), i.e. counter words W - (t + 1) * WPT .. W - t * WPT - 1, scanned
    // from the top (high half first), so slot offsets grow with t.
    constexpr int WPT = BPT / 2;  // counter words per thread
    const int w0 = kBuckets / 2 - (tid + 1) * WPT;
    uint32_t cw[WPT];
    uint32_t packed = 0;  // both halves summed at once: no carry, counts stay below 2^16
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        cw[i] = bucket[w0 + i];
        packed += cw[i];
    }
    const uint32_t tsum = (packed >> 16) + (packed & 0xFFFFu);
    {  // does any bucket (kept or not) hold more than the limit?  Adding 0x7FFF - limit to
       // each 16-bit count sets its bit 15 exactly when it exceeds the limit; counts stay
       // below 2^15, so neither half carries into the other.
        constexpr uint32_t LIM = LIMITED ? kBucketLimit : kBucketLimitRow;
        constexpr uint32_t BIAS = (0x7FFFu - LIM) * 0x10001u;
        static_assert(CPT * NT + (0x7FFF - LIM) < 0x10000, "bucket counts (at most c_gt) stay below 2^15");
        uint32_t ov = 0;
#pragma unroll
        for (int i = 0; i < WPT; ++i) ov |= cw[i] + BIAS;
        if (ov & 0x80008000u) {  // rare: which buckets (word w0 + i: bit 15 bucket 2 (w0 + i), bit 31 the next)
            uint32_t top = 0, nlong = 0;
#pragma unroll
            for (int i = 0; i < WPT; ++i) {
                const uint32_t x = cw[i] + BIAS;
                if (x & 0x8000u) top = max(top, 2u * (uint32_t)(w0 + i) + 1u), ++nlong;
                if (x & 0x80000000u) top = max(top, 2u * (uint32_t)(w0 + i) + 2u), ++nlong;
            }
            __hip_atomic_fetch_max(&ctl[kCtlMaxBucket], top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if constexpr (PBW > 0) lds_add(&ctl[kCtlLongN], nlong);
        }
    }
    uint32_t total;
    const uint32_t run0 = block_excl_scan<NT>(tsum, wsum + 16, &total);
    {
        uint32_t run = run0;
#pragma unroll
        for (int i = WPT - 1; i >= 0; --i) {  // word w0 + i holds buckets 2 (w0 + i) + 1 (high), 2 (w0 + i)
            const uint32_t hi = cw[i] >> 16, lo = cw[i] & 0xFFFFu;
            bucket[w0 + i] = (run << 16) | (run + hi);  // cursors start at first slots
            run += hi + lo;
        }
    }
    if (!ties && run0 < m && run0 + tsum >= m) {  // this thread owns the threshold bucket
        uint32_t run = run0;
#pragma unroll
        for (int i = WPT - 1; i >= 0; --i) {
#pragma unroll
            for (int h = 1; h >= 0; --h) {
                const uint32_t c = h ? cw[i] >> 16 : cw[i] & 0xFFFFu;
                if (run < m && run + c >= m) {
                    ctl[kCtlBt] = (uint32_t)(2 * (w0 + i) + h);  // threshold bucket
                    ctl[kCtlKept] = run + c;                     // kept: slots of buckets >= b_t
                }
                run += c;
            }
        }
    }
    __syncthreads();
    const uint32_t bt = ties ? 0u : ctl[kCtlBt];
    const uint32_t kept = ties ? c_gt : ctl[kCtlKept];
    const uint32_t long_top = ctl[kCtlMaxBucket];  // highest long bucket + 1
    const bool too_long = long_top > bt;            // some kept bucket is long
    // A plateau bucket (see above) is looked at once the composites are in S: exactly one
    // long kept bucket.
    bool plateau = false;  // uniform
    if constexpr (PBW > 0) plateau = too_long && ctl[kCtlLongN] == 1u;
    // (the bitonic sort pads to a power of two, which must fit S)
    constexpr uint32_t SORT_MAX = pow2_floor((uint32_t)(SCAP + rank_pad<LIMITED>()));
    bool sort_all = too_long && !plateau && (!LIMITED || (sort_long && kept <= SORT_MAX));  // uniform
    if (LIMITED && (kept > (uint32_t)SCAP || (too_long && !plateau && !sort_all))) return false;  // uniform

    // ---- scatter kept candidates by bucket, two per lane at a time (claim both, then write).
    // A candidate that is not kept claims nothing: its claim word stays all ones, whose
    // 16-bit half (65535) is past SCAP, so it is not stored.
    static_assert(SCAP < 0xFFFF, "an unclaimed slot reads as past the end of S");
    constexpr int SUNR = 2;
#pragma unroll
    for (int i0 = 0; i0 < CPT; i0 += SUNR) {
        if (!live(i0) && !(i0 + 1 < CPT && live(i0 + 1))) continue;  // uniform
        uint32_t old[SUNR], sh[SUNR];
        uint64_t comp[SUNR];
#pragma unroll
        for (int d = 0; d < SUNR; ++d) {
            const int i = i0 + d < CPT ? i0 + d : CPT - 1;
            const uint32_t b = bucket_at(i);
            comp[d] = ((uint64_t)key_at(i) << 32) | (uint32_t)~cv[i].y;
            sh[d] = (b & 1u) << 4;
            old[d] = 0xFFFFFFFFu;
            if (i0 + d < CPT && valid(i0 + d) && b >= bt)
                old[d] = __hip_atomic_fetch_add(&bucket[b >> 1], 1u << sh[d], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        // (the claimed slots are read only once every claim of this turn is issued)
#pragma unroll
        for (int d = 0; d < SUNR; ++d) {
            const uint32_t pos = (old[d] >> sh[d]) & 0xFFFFu;
            if (pos < (uint32_t)SCAP) S[pos] = comp[d];
        }
    }
    for (int i = tid; i < rank_pad<LIMITED>(); i += NT) S[kept + i] = 0;  // kept <= SCAP here
    __syncthreads();
    const uint16_t* const b16 = reinterpret_cast<const uint16_t*>(bucket);
    if constexpr (PBW > 0) {
        if (plateau) {  // uniform: the long bucket's key X and its other composites
            const uint32_t pb = long_top - 1u;
            const uint32_t q0 = b16[pb + 1], q1 = b16[pb];  // its slots in S
            for (int w = tid; w < PBW; w += NT) pl->bits[w] = 0u;  // (S's tail: the candidates are in S)
            uint64_t f = 0;  // (one atomic per wave: same-address LDS atomics serialise)
            for (uint32_t q = q0 + tid; q < q1; q += NT) {
                const uint64_t c = S[q];
                f = max(f, (c << 32) | (c >> 32));
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) f = max(f, (uint64_t)__shfl_xor((unsigned long long)f, o));
            if (lane == 0 && f)
                __hip_atomic_fetch_max(reinterpret_cast<uint64_t*>(&ctl[kCtlPFirst]), f, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            __syncthreads();
            const uint32_t px = __builtin_amdgcn_readfirstlane(ctl[kCtlPFirst]);  // (the low word: the key)
            uint32_t cnt = 0;  // (above X) << 16 | (equal to X), this thread's
            for (uint32_t q = q0 + tid; q < q1; q += NT) {
                const uint64_t c = S[q];
                const uint32_t kx = (uint32_t)(c >> 32), pos = ~(uint32_t)c;
                if (kx == px) {
                    __hip_atomic_fetch_or(&pl->bits[pos >> 5], 1u << (pos & 31u), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WORKGROUP);
                    cnt += 1u;
                } else {
                    const uint32_t o = __hip_atomic_fetch_add(&ctl[kCtlPOther], 1u, __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_WORKGROUP);
                    if (o < (uint32_t)kBucketLimit) pl->other[o] = c;
                    if (kx > px) cnt += 1u << 16;
                }
            }
            cnt = wave_incl_scan(cnt);  // (both halves stay below 2^16: at most SCAP in the bucket)
            if (lane == 63 && cnt) lds_add(&ctl[kCtlPCount], cnt);
            __syncthreads();
            if (ctl[kCtlPOther] > (uint32_t)kBucketLimit) {  // uniform: X is not the bucket's one key
                plateau = false;
                sort_all = sort_long && kept <= SORT_MAX;
                if (!sort_all) return false;  // (nothing emitted yet)
            }
        }
    }
    scattered();  // past the point of falling back: the caller may reuse its registers

    if (sort_all) {  // uniform
        static_assert(LIMITED || (SCAP & (SCAP - 1)) == 0, "the sort pads S to a power of two");
        bitonic_desc_u64<NT>(S, (int)kept);
        for (uint32_t q = tid; q < mlim; q += NT) emit(q, xo(~(uint32_t)S[q]), bits_of((uint32_t)(S[q] >> 32)));
        return true;
    }

    // ---- rank inside buckets -> final slot.  Bucket b's 16-bit counter now holds its end;
    // its start is the end of bucket b + 1 (zero above the top bucket).  Each lane ranks
    // RUNR elements at once: it counts the larger composites among the lmax entries from
    // its bucket's start, lmax being the wave's longest bucket; entries past its bucket's
    // end belong to lower buckets or the zero padding, so every lane compares them all.
    constexpr int RUNR = 2;
    const uint32_t wbase = __builtin_amdgcn_readfirstlane((uint32_t)(tid & ~63));  // (scalar: a uniform loop exit)
    // SKIP: the plateau bucket's elements are placed apart (not ranked here)
    auto rank_kept = [&](auto skip_tag) {
        constexpr bool SKIP = decltype(skip_tag)::value;
        const uint32_t pb = SKIP ? long_top - 1u : 0u;
        for (uint32_t q0 = 0; q0 < kept; q0 += RUNR * NT) {
            if (q0 + wbase >= kept) break;  // nothing left for this wave
            uint64_t cc[RUNR];
            uint32_t st[RUNR], rank[RUNR];
            int32_t ox[RUNR];  // the index written for the element (a page-table load is issued here,
                               // so its latency hides behind the comparisons)
            bool in[RUNR];
            uint32_t lmax = 0;
#pragma unroll
            for (int i = 0; i < RUNR; ++i) {
                const uint32_t q = q0 + i * NT + tid;
                cc[i] = S[min(q, kept)];  // S[kept] is zero: no branch around the read
                const uint32_t bk = bucket_of((uint32_t)(cc[i] >> 32));
                in[i] = q < kept && (!SKIP || bk != pb);
                ox[i] = in[i] ? xo(~(uint32_t)cc[i]) : 0;
                const uint32_t en = min((uint32_t)b16[bk], kept);
                const uint32_t s0 = b16[bk + 1];
                st[i] = in[i] ? s0 : 0u;
                lmax = max(lmax, in[i] && en > s0 ? en - s0 : 0u);
                rank[i] = 0;
            }
            lmax = wave_max(lmax);
            for (uint32_t f = 0; f < lmax; f += kRankUnroll) {
#pragma unroll
                for (int i = 0; i < RUNR; ++i) {
                    const uint64_t* const o = S + st[i] + f;
#pragma unroll
                    for (int u = 0; u < kRankUnroll; ++u) rank[i] += o[u] > cc[i] ? 1u : 0u;
                }
            }
#pragma unroll
            for (int i = 0; i < RUNR; ++i) {
                const uint32_t slot = st[i] + rank[i];
                if (in[i] && slot < mlim) emit(slot, ox[i], bits_of((uint32_t)(cc[i] >> 32)));
            }
        }
    };
    if constexpr (PBW > 0) {
        if (plateau) {  // uniform
            rank_kept(std::true_type{});
            // the bucket's other keys, ranked among themselves; those below X also pass X's
            const uint32_t base = b16[long_top];  // the bucket's first slot (end of the one above)
            const uint32_t px = ctl[kCtlPFirst], pcount = ctl[kCtlPCount], pother = ctl[kCtlPOther];
            const uint32_t n_eq = pcount & 0xFFFFu, n_gt = pcount >> 16;
            for (uint32_t t = tid; t < pother; t += NT) {
                const uint64_t y = pl->other[t];
                uint32_t rk = (uint32_t)(y >> 32) < px ? n_eq : 0u;
                for (uint32_t j = 0; j < pother; ++j) rk += pl->other[j] > y ? 1u : 0u;
                const uint32_t slot = base + rk;
                if (slot < mlim) emit(slot, xo(~(uint32_t)y), bits_of((uint32_t)(y >> 32)));
            }
            const uint32_t b0 = base + n_gt;  // X's first slot
            pl->on = true;
            pl->key = px;
            pl->base = b0;
            pl->need = b0 < mlim ? min(n_eq, mlim - b0) : 0u;
            return true;
        }
    }
    rank_kept(std::false_type{});
    return true;
}

// Ties at P from one tile's position bitmap, spread over every thread in position order:
// thread t owns the tile's positions [t EPT, (t + 1) EPT), a field of one bitmap word
// (word_at(w) reads word w).  The set bits, counted from `first` (ties in earlier tiles),
// go to slots c_gt + i while i < need, as the index of tile position p0 + bit.  Returns
// the tile's set bits.  The positions are first listed in LDS (`stage`, at least need
// words, free from the first barrier in here to the caller's next one), so that the
// output stores run over consecutive slots: written straight from the bitmap fields,
// neighbouring lanes would store a field's length apart.  Contains barriers (a block
// scan over wsum, then the list).
template <int NT, int EPT, class WordAt>
__device__ __forceinline__ uint32_t emit_ties(WordAt&& word_at, int32_t p0, uint32_t first, uint32_t need,
                                              uint32_t c_gt, uint32_t vP, const RowCtx& r, uint32_t* wsum,
                                              uint32_t* stage) {
    static_assert(EPT <= 32 && 32 % EPT == 0, "a thread's positions lie in one bitmap word");
    const int tid = opaque_tid();
    uint32_t bits = word_at((tid * EPT) >> 5);
    if constexpr (EPT < 32) bits = (bits >> ((tid * EPT) & 31)) & ((1u << EPT) - 1u);
    uint32_t tot;
    uint32_t rr = first + block_excl_scan<NT>((uint32_t)__popc(bits), wsum, &tot);
    const int32_t pt = p0 + tid * EPT;
    while (bits && rr < need) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        stage[rr - first] = (uint32_t)(pt + bit);
        ++rr;
    }
    const uint32_t cnt = first < need ? min(tot, need - first) : 0u;  // (uniform)
    __syncthreads();
    for (uint32_t i = tid; i < cnt; i += NT) {
        const uint32_t slot = c_gt + first + i;
        r.oidx[slot] = r.xo(stage[i]);
        if (r.ov) r.ov.put(slot, vP);
    }
    return tot;
}

// Bucket range [L, U]: L is the least sample above P, U the largest sample below
// key(+inf) (the largest sample when P itself is +inf or +NaN), so neither a pivot on a
// plateau of equal scores far below the kept keys nor a few +inf / NaN scores stretch
// the range away from where the kept keys are.
__device__ __forceinline__ void bucket_range(uint32_t P, uint32_t lo, uint32_t smax_all, uint32_t smax_fin, uint32_t* L,
                                             uint32_t* U) {
    *U = max(P, P >= kKeyPosInf ? smax_all : smax_fin);
    *L = min(lo, *U);
}

// Pivot path of a row that fits one workgroup (raw bits in u[], dead after the write pass).
// Returns false, with LDS left dirty, when the row needs the exact path.  scattered() runs
// once the row can no longer fall back.
// PLATEAU: a long kept bucket of one key is placed by position (bucket_rank's plateau
// bucket) instead of sending the row to the sort or the exact path.
template <int NT, int EPT, int KMAX, bool PLATEAU, class Scattered>
__device__ __forceinline__ bool fast_tile(const RowCtx& r, FastSmem<NT, EPT, KMAX>& s, const uint32_t (&u)[EPT],
                                          int fast_mode, Scattered&& scattered) {
    using FS = FastSmem<NT, EPT, KMAX>;
    constexpr int BW = FS::BWORDS;
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int32_t nt = r.nt;
    const int32_t m = r.m;

    // ------------------------------------------------ clear LDS state
    block_zero<NT, BW>(s.bitmap);
    uint32_t* const shist = reinterpret_cast<uint32_t*>(s.S);  // sample histograms (the list's LDS is free until the write pass)
    block_zero<NT, 2 * kRadix>(shist);
    block_zero<NT, kBuckets / 2>(s.bucket);
    if (tid < FS::CTL_WORDS) s.ctl[tid] = tid == kCtlLo ? 0xFFFFFFFFu : 0u;

    // ------------------------------------------------ sample -> pivot
    constexpr int SPL = samples_per_lane<EPT>();
    uint32_t sk[SPL];
    take_samples<NT, EPT>(u, nt, sk);
    const int nsamp = tile_samples<NT, EPT>(nt);
    {
        uint32_t sf = 0;  // largest sample below key(+inf)
#pragma unroll
        for (int i = 0; i < SPL; ++i) sf = sk[i] < kKeyPosInf ? max(sf, sk[i]) : sf;
        sf = wave_max(sf);
        __syncthreads();
        if (lane == 0) __hip_atomic_fetch_max(&s.ctl[kCtlSmaxFin], sf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    uint32_t P = 0;
    int passes = 0;
    {
        // (fast_mode == 2, a test setting, takes the largest sample: the pivot misses.)
        const uint32_t rr = fast_mode == 2 ? 1u : pivot_rank(nsamp, m, nt);
        if (m < nt && rr < (uint32_t)nsamp) {
            P = pivot_passes<NT, 2>(sk, rr, shist, [](int, uint32_t*) {}, s.ctl, &passes,
                                    r.wave_select ? nullptr : s.ctl + kCtlSel);
        } else if (m == nt && fast_mode != 2) {
            // The whole row is output: pivot on its least key, taken exactly.  No key lies
            // below it, so the keys equal to it are the tail, in index order from the
            // bitmap; a plateau at the bottom of a short row then costs a bitmap scan
            // instead of a sort of one long bucket.  (Least key 0: no pivot.)
            P = tile_min_key<NT, EPT>(u, nt, s.ctl + kCtlSel);
            passes = P ? 4 : 0;
        }
    }
    // The least sample above P starts the bucket range when P may sit far below the kept
    // keys: P = 0 (no pivot) or P exactly a sample's key (a plateau of equal scores, four
    // passes); otherwise P, the low end of a bin holding samples, is as good.
    const bool need_lo = P == 0 || passes == 4;  // uniform
    if (need_lo) {
        uint32_t lo = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < SPL; ++i) lo = sk[i] > P ? min(lo, sk[i]) : lo;
        lo = wave_min(lo);
        if (lane == 0) __hip_atomic_fetch_min(&s.ctl[kCtlLo], lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const AboveP ap(P);

    // ------------------------------------------------ one pass: candidates (bits, position)
    // into per-wave regions of R slots, keys == P into the position bitmap when P is a
    // plateau value (then the tail may need them).  The running count is scalar and
    // checked once per group of four slots: a slot that no longer fits its wave's region
    // claims slots in the shared pool after the regions instead (one LDS atomic per wave
    // and slot); only an exhausted pool sends the row to the exact path.  (Past the
    // pivot's last barrier no wave reads the sample histograms, so the regions may
    // overwrite them.)
    constexpr uint32_t NW = NT / 64;
    constexpr uint32_t R = ((uint32_t)FS::CCAP * 7 / 8 / NW) / 64 * 64;  // region slots per wave
    constexpr uint32_t POOL = (uint32_t)FS::CCAP - NW * R;                 // shared overflow slots
    static_assert(R > 0 && POOL > 0, "regions and pool both have room");
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t base = (uint32_t)wave * R, limit = base + R;
    const bool mark_eq = passes == 4;  // uniform: P is a sample's key exactly
    uint32_t o = base, neq = 0;
    auto one_pass = [&](auto pos_tag, auto eq_tag) {
        constexpr bool POS = decltype(pos_tag)::value;
        constexpr bool EQ = decltype(eq_tag)::value;
        const int t4 = tid * 4;
        // One group of four slots (v): the four masks and counts first, so a group that
        // fits the region takes one check; a group that does not goes slot by slot,
        // region first, then the pool.  FULL: every lane's four slots are in the tile.
        auto group = [&](int v, auto full_tag, int llim) {
            constexpr bool FULL = decltype(full_tag)::value;
            const int p0 = t4 + v * NT * 4;
            bool g[4];
            uint64_t mk[4];
            uint32_t tot = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                g[c] = ap.gt<POS>(u[4 * v + c]) && (FULL || c < llim);
                mk[c] = __ballot(g[c]);
                tot += (uint32_t)__popcll(mk[c]);
            }
            if (o + tot <= limit) {  // uniform
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    uint32_t* const cb = s.cand.bits + o;  // (scalar base: one address op per lane)
                    if (g[c]) {
                        const uint32_t q = lanes_below(mk[c]);
                        cb[q] = u[4 * v + c];
                        cb[q + (uint32_t)FS::CCAP] = (uint32_t)(p0 + c);
                    }
                    o += (uint32_t)__popcll(mk[c]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t cnt = (uint32_t)__popcll(mk[c]);
                    if (o + cnt <= limit) {  // uniform
                        if (g[c]) {
                            const uint32_t q = lanes_below_plus(mk[c], o);
                            s.cand.bits[q] = u[4 * v + c];
                            s.cand.pos[q] = (uint32_t)(p0 + c);
                        }
                        o += cnt;
                    } else {  // the pool (rare)
                        const uint32_t q = claim_slot(g[c], &s.ctl[kCtlPool]);
                        if (g[c] && q < POOL) {
                            s.cand.bits[NW * R + q] = u[4 * v + c];
                            s.cand.pos[NW * R + q] = (uint32_t)(p0 + c);
                        }
                    }
                }
            }
            if (EQ) {
                uint32_t nib = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) nib |= (ap.eq<POS>(u[4 * v + c]) && (FULL || c < llim) ? 1u : 0u) << c;
                if (nib) {
                    __hip_atomic_fetch_or(&s.bitmap[p0 >> 5], nib << (p0 & 31), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WORKGROUP);
                    neq += (uint32_t)__popc(nib);
                }
            }
        };
#pragma unroll
        for (int v = 0; v < EPT / 4; ++v) {
            const int lim = nt - v * NT * 4;
            if (lim <= 0) break;
            if (lim >= NT * 4) group(v, std::true_type{}, 0);
            else group(v, std::false_type{}, lim - t4);
        }
    };
    if (P >= 0x80000000u) {
        if (mark_eq) one_pass(std::true_type{}, std::true_type{});
        else one_pass(std::true_type{}, std::false_type{});
    } else {
        if (mark_eq) one_pass(std::false_type{}, std::true_type{});
        else one_pass(std::false_type{}, std::false_type{});
    }
    if (mark_eq) {
        neq = wave_incl_scan(neq);
        if (lane == 63) lds_add(&s.ctl[kCtlEq], neq);
    }
    if (lane == 0) s.wsum[wave] = o - base;
    __syncthreads();
    // (past this barrier every wave has published its count, its sample extremes and its
    // keys equal to P)
    const uint32_t pooled = __builtin_amdgcn_readfirstlane(s.ctl[kCtlPool]);
    if (pooled > POOL) return false;  // uniform: the pool overflowed
    uint32_t c_gt = pooled;
#pragma unroll
    for (int w = 0; w < (int)NW; ++w) c_gt += s.wsum[w];
    c_gt = __builtin_amdgcn_readfirstlane(c_gt);
    const bool ties = c_gt < (uint32_t)m;  // uniform: keys == P fill the tail
    if (ties && (!mark_eq || c_gt + s.ctl[kCtlEq] < (uint32_t)m)) return false;  // uniform: pivot missed
    const uint32_t U = max(P, s.ctl[kCtlSmaxFin]);
    const uint32_t L = need_lo ? min(s.ctl[kCtlLo], U) : P;
    const BucketMap bucket_of(L, U);

    // ------------------------------------------------ order the candidates, straight to
    // the output row (S is in bucket order, so a wave's slots are nearly contiguous)
    // (a thread owns RC entries of its wave's region, lane + 64 i, then PC pool entries,
    // tid + NT i)
    constexpr int RC = (int)(R / 64), PC = (int)((POOL + NT - 1) / NT);
    const uint32_t c_w = o - base;  // this wave's region entries (scalar)
    PlateauBucket pl{s.plateau.other, s.plateau.bits};
    if (!bucket_rank<NT, FS::SCAP, RC + PC, true, false, PLATEAU ? FS::BWORDS : 0>(
            s.bucket, s.S, s.wsum, s.ctl,
            [&](int i) {
                const uint32_t q = i < RC ? base + (uint32_t)(lane + 64 * i) : NW * R + (uint32_t)(tid + (i - RC) * NT);
                return make_uint2(s.cand.bits[q], s.cand.pos[q]);
            },
            [&](int i) {
                return i < RC ? (uint32_t)(lane + 64 * i) < c_w : (uint32_t)(tid + (i - RC) * NT) < pooled;
            },
            [&](int i) { return i < RC ? (uint32_t)(64 * i) < c_w : (uint32_t)((i - RC) * NT) < pooled; },
            c_gt, (uint32_t)m, ties, bucket_of,
            r.xo,
            [&](uint32_t slot, int32_t idx, uint32_t bits) {
                store_at(r.oidx, slot, idx);
                if (r.ov) r.ov.put(slot, bits);
            },
            scattered, m == nt, &pl))
        return false;
    if (pl.on) {  // uniform: a plateau bucket's key, in position order
        emit_ties<NT, EPT>([&](int w) { return s.plateau.bits[w]; }, 0, 0u, pl.need, pl.base, bits_of(pl.key), r,
                           s.wsum, reinterpret_cast<uint32_t*>(s.S));
        __syncthreads();  // (wsum is scanned through again below)
    }

    // ------------------------------------------------ ties at P: smallest positions
    if (ties)
        emit_ties<NT, EPT>([&](int w) { return s.bitmap[w]; }, 0, 0u, (uint32_t)m - c_gt, c_gt, bits_of(P), r, s.wsum,
                           reinterpret_cast<uint32_t*>(s.S));
    write_padding<NT>(r.oidx, r.ov, m, r.k);
    return true;
}

// Samples of a split row, the same in every tile of the row: groups of 4 elements
// (16 bytes of float32, 8 of 16-bit floats, widened as the tile loads widen them), evenly
// spread over the window.  The groups start at the window's first group-size boundary
// (a0 = 0..3 elements in), so every load is an aligned buffer load and there is no
// alignment branch: the compiler counts the loads exactly, and the
// pivot waits for them alone, not for the tile loads issued after them.  Lane t's g-th
// group is group floor(q * G / (SL * NT)), q = g * NT + t, of the G = (n - a0) / 4 whole
// groups (a row shorter than 4 * SL * NT elements repeats some, which only weakens the
// pivot estimate).
// sl (<= SL, uniform): groups per lane actually sampled; the others hold the least key.
template <int NT, int SL, int VB>
__device__ __forceinline__ void load_row_samples(uint32_t (&sk)[4 * SL], const char* row, int32_t n, int sl) {
    // a0: elements before the first (4 * VB)-byte boundary (rows start VB-byte aligned)
    const uint32_t a0 = ((4u * VB - (uint32_t)((uintptr_t)row & (4u * VB - 1u))) & (4u * VB - 1u)) / VB;
    const char* base = row + (size_t)a0 * VB;
    const uint64_t groups = (uint64_t)((uint32_t)(n - (int32_t)a0) >> 2);
    // (2^30 float32 elements make 2^32 bytes: the range is clamped to 32 bits, and a sample
    // group past it reads zeros, which only nudges the pivot estimate)
    const uint64_t bytes = groups * 4u * VB;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), (short)0, (int)(uint32_t)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull),
        kBufferWord3);
    const uint32_t tid = (uint32_t)opaque_tid();
#pragma unroll
    for (int g = 0; g < SL; ++g) {
        if (g >= sl) {  // uniform: bits whose key is 0, below every sample (they rank last)
            sk[4 * g + 0] = sk[4 * g + 1] = sk[4 * g + 2] = sk[4 * g + 3] = VB == 4 ? 0xFFFFFFFFu : 0xFFFF0000u;
            continue;
        }
        const uint32_t q = (uint32_t)g * NT + tid;
        const uint32_t grp = (uint32_t)(((uint64_t)q * groups) / ((uint64_t)sl * NT));
        if constexpr (VB == 4) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, grp * 16u, 0, 0);
            sk[4 * g + 0] = v[0];
            sk[4 * g + 1] = v[1];
            sk[4 * g + 2] = v[2];
            sk[4 * g + 3] = v[3];
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, grp * 8u, 0, 0);
            sk[4 * g + 0] = v[0] << 16;
            sk[4 * g + 1] = v[0] & 0xFFFF0000u;
            sk[4 * g + 2] = v[1] << 16;
            sk[4 * g + 3] = v[1] & 0xFFFF0000u;
        }
    }
}

template <int NT, int KMAX, int STAGE, int VB>
__device__ void exact_row(const char* row, int32_t n, int32_t m, int32_t k, int32_t* oidx, ValOut ov, IndexOut xo,
                          RowExactSmem<NT, KMAX, STAGE>& s, int stage_cap);

// One tile of a row split over several workgroups.  No workgroup ever waits for another:
//   - every tile reads the same evenly spaced samples of the whole row and derives the
//     same pivot P from them, as a one-tile row does from its own registers;
//   - it counts its keys above and equal to P, claims room for its candidates in the
//     row's workspace list with one atomic add and writes them there (raw bits, row
//     position); when it holds keys equal to P it also stores its bitmap of their
//     positions and their count;
//   - it arrives at the row's ticket counter.  The last tile to arrive owns the row: it
//     sets the row's counters back to zero, then orders the candidates when the list held
//     them all and at least min(k, n) keys are >= P (keys equal to P fill the tail in
//     index order, tile by tile), and otherwise selects the row exactly on its own.
template <int NT, int EPT, int KMAX, int VB>
__device__ __forceinline__ void split_tile(const Params& p, const RowCtx& r, SmemAll<NT, EPT, KMAX, true>& sa) {
    using SS = SplitSmem<NT, EPT, KMAX>;
    SS& s = sa.split;
    constexpr int BW = SS::BWORDS;
    constexpr int TILE = SS::TILE;
    constexpr uint32_t CAP = (uint32_t)SS::SCAP;
    constexpr int SL = kSplitSamples / (4 * NT);  // 16-byte sample loads per lane
    static_assert(SL >= 1 && 4 * SL * NT == kSplitSamples, "whole sample groups per lane");
    const int tid = opaque_tid();
    const int lane = tid & 63;
    const int b = r.b, tile = r.tile, ntiles = r.ntiles;
    const int32_t nt = r.nt, m = r.m, n = r.n, j0 = r.j0;
    const char* const row = static_cast<const char*>(p.scores) + r.base * VB;
    uint32_t* const rw = p.ws_ctl + (int64_t)b * kRowCtlWords;
    uint32_t* const ecnt = p.ws_ecnt + (int64_t)b * p.tiles_per_row;
    uint32_t P = 0;

    if (p.fast) {
        uint32_t sk[4 * SL];
        const int sl = p.split_half ? SL / 2 : SL;  // (uniform)
        static_assert(SL % 2 == 0, "the samples halve");
        load_row_samples<NT, SL, VB>(sk, row, n, sl);
        // A 32K-element tile's loads go out with the samples: that tile serves batches that
        // fill the GPU, where the HBM stream matters more than one tile's latency (the pivot
        // then waits for all of them, see below).
        uint32_t u_early[EPT];
        if constexpr (EPT >= 32) load_tile<NT, EPT, VB>(u_early, row + (size_t)j0 * VB, nt);

        // ------------------------------------------------ pivot from the row's samples
        block_zero<NT, 5 * kRadix>(s.bucket);  // the sample-digit histograms, and the lane maxima's
        if (tid < 16) s.ctl[tid] = tid == kCtlLo ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int i = 0; i < 4 * SL; ++i) sk[i] = key_of(sk[i]);
        {
            uint32_t sx = 0, sf = 0;
#pragma unroll
            for (int i = 0; i < 4 * SL; ++i) {
                sx = max(sx, sk[i]);
                sf = sk[i] < kKeyPosInf ? max(sf, sk[i]) : sf;
            }
            sx = wave_max(sx);
            sf = wave_max(sf);
            __syncthreads();
            if (lane == 0) {
                __hip_atomic_fetch_max(&s.ctl[kCtlSmaxAll], sx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_max(&s.ctl[kCtlSmaxFin], sf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        // Smaller tiles issue their loads only past that barrier (which they cannot cross), so
        // the wait before it is for the samples alone -- the tile load takes one of two code
        // paths, and past that branch the compiler would wait for every load outstanding --
        // and they complete behind the pivot passes.
        uint32_t u[EPT];
        if constexpr (EPT < 32) load_tile<NT, EPT, VB>(u, row + (size_t)j0 * VB, nt);
        else {
#pragma unroll
            for (int i = 0; i < EPT; ++i) u[i] = u_early[i];
        }
        const int nsamp = 4 * sl * NT;
        // (fast == 2, a test setting, aims at the largest sample: the pivot misses.)
        const uint32_t rr = p.fast == 2 ? 1u : pivot_rank(nsamp, m, n);
        if (rr < (uint32_t)nsamp) {
            // The rr-th largest lane maximum is at most the rr-th largest sample (were it
            // larger, rr lanes would each hold a larger sample), so no sample below its
            // first-digit bin decides the pivot.  One count of the lane maxima (one atomic
            // per lane instead of one per sample) lets the first pass skip those samples:
            // for a long row with a small k, nearly all of them.  (With rr past a quarter of
            // the lanes the floor would filter little and cost a pass.)
            uint32_t floor = 0;
            if (rr <= (uint32_t)NT / 4) {
                uint32_t lm = 0;
#pragma unroll
                for (int i = 0; i < 4 * SL; ++i) lm = max(lm, sk[i]);
                uint32_t* const hm = s.bucket + 4 * kRadix;
                hist_add(hm, lm >> 24);
                __syncthreads();
                uint32_t above, cnt;
                floor = wave_select_digit(hm, rr, &above, &cnt) << 24;
            }
            P = pivot_passes<NT, 4, true>(sk, rr, s.bucket, [](int, uint32_t*) {}, s.ctl, nullptr,
                                          r.wave_select ? nullptr : s.ctl + kCtlSel, floor, 4 * sl);
        }
        {
            uint32_t lo = 0xFFFFFFFFu;
#pragma unroll
            for (int i = 0; i < 4 * SL; ++i) lo = sk[i] > P ? min(lo, sk[i]) : lo;
            lo = wave_min(lo);
            if (lane == 0) __hip_atomic_fetch_min(&s.ctl[kCtlLo], lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        const AboveP ap(P);

        // ------------------------------------------------ count, claim
        uint32_t cgt = 0, ceq = 0;
        if (P >= 0x80000000u)
            visit_slots<NT, EPT>(u, nt, [&](uint32_t x, int, int, bool ok, int) {
                cgt += (ap.gt<true>(x) && ok) ? 1u : 0u;
                ceq += (ap.eq<true>(x) && ok) ? 1u : 0u;
            });
        else
            visit_slots<NT, EPT>(u, nt, [&](uint32_t x, int, int, bool ok, int) {
                cgt += (ap.gt<false>(x) && ok) ? 1u : 0u;
                ceq += (ap.eq<false>(x) && ok) ? 1u : 0u;
            });
        // (one scan for both counts: per-thread counts <= EPT and tile totals <= TILE < 2^16,
        // so the two 16-bit halves never carry into each other)
        uint32_t both;
        uint32_t o = block_excl_scan<NT>(cgt | (ceq << 16), s.wsum, &both) & 0xFFFFu;
        const uint32_t c_tile = both & 0xFFFFu, e_tile = both >> 16;
        if (tid == 0) {
            s.ctl[kCtlBase] = c_tile ? atomicAdd(&rw[kRowCgt], c_tile) : 0u;
            if (e_tile) atomicAdd(&rw[kRowEq], e_tile);
            ecnt[tile] = e_tile;
        }
        const bool mark = e_tile != 0;  // uniform
        if (mark) block_zero<NT, BW>(s.bitmap);
        __syncthreads();
        const uint32_t base = s.ctl[kCtlBase];
        const bool fits = base + c_tile <= CAP;  // uniform; otherwise the row falls back

        // ------------------------------------------------ write candidates (+ tie bitmap)
        uint2* const gc = p.ws_cand + (int64_t)b * CAP + base;
        auto write_pass = [&](auto pos_tag, auto eq_tag, auto cand_tag) {
            constexpr bool POS = decltype(pos_tag)::value;
            constexpr bool EQ = decltype(eq_tag)::value;
            constexpr bool CAND = decltype(cand_tag)::value;
            uint32_t nib = 0;
            visit_slots<NT, EPT>(u, nt, [&](uint32_t x, int c, int v, bool ok, int t4) {
                if (CAND && ap.gt<POS>(x) && ok) {
                    gc[o] = make_uint2(x, (uint32_t)(j0 + t4 + (v * NT * 4 + c)));
                    ++o;
                }
                if (EQ) {
                    nib |= (ap.eq<POS>(x) && ok ? 1u : 0u) << c;
                    if (c == 3) {
                        if (nib) {
                            const int p0 = t4 + v * NT * 4;
                            __hip_atomic_fetch_or(&s.bitmap[p0 >> 5], nib << (p0 & 31), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_WORKGROUP);
                        }
                        nib = 0;
                    }
                }
            });
        };
        auto by_cand = [&](auto pos_tag, auto eq_tag) {
            if (fits) write_pass(pos_tag, eq_tag, std::true_type{});
            else if (decltype(eq_tag)::value) write_pass(pos_tag, eq_tag, std::false_type{});
        };
        if (P >= 0x80000000u) {
            if (mark) by_cand(std::true_type{}, std::true_type{});
            else by_cand(std::true_type{}, std::false_type{});
        } else {
            if (mark) by_cand(std::false_type{}, std::true_type{});
            else by_cand(std::false_type{}, std::false_type{});
        }
        if (mark) {  // this tile's bitmap of keys == P, for the last arriver
            __syncthreads();
            uint32_t* const gt = p.ws_tie + ((int64_t)b * p.tiles_per_row + tile) * BW;
            for (int w = tid; w < BW; w += NT) gt[w] = s.bitmap[w];
        }
    }

    // ------------------------------------------------ arrive; the last tile owns the row
    if (!arrive_last(&rw[kRowArrive], (uint32_t)ntiles, &s.ctl[kCtlLast])) return;
    if (tid == 0) {
        s.ctl[kCtlRowCgt] = __hip_atomic_load(&rw[kRowCgt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.ctl[kCtlEq] = __hip_atomic_load(&rw[kRowEq], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // Every other tile has counted and arrived: the row's words are free for the next call.
        __hip_atomic_store(&rw[kRowCgt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&rw[kRowEq], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&rw[kRowArrive], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t c_gt = s.ctl[kCtlRowCgt];
    const uint32_t n_eq = s.ctl[kCtlEq];
    if (!p.fast || c_gt > CAP || c_gt + n_eq < (uint32_t)m) {  // uniform
        __syncthreads();  // (the fallback's LDS overlays the words just read)
        exact_row<NT, KMAX, kRowStageEntries, VB>(row, n, m, r.k, r.oidx, r.ov, r.xo, sa.rexact, p.stage_cap);
        return;
    }
    const bool ties = c_gt < (uint32_t)m;
    block_zero<NT, kBuckets / 2>(s.bucket);
    if (tid >= kCtlBt && tid <= kCtlMaxBucket) s.ctl[tid] = 0;
    __syncthreads();
    uint32_t L, U;
    bucket_range(P, s.ctl[kCtlLo], s.ctl[kCtlSmaxAll], s.ctl[kCtlSmaxFin], &L, &U);
    const uint2* const gc = p.ws_cand + (int64_t)b * CAP;
    bucket_rank<NT, SS::SCAP, (SS::SCAP + NT - 1) / NT, false, false, 0>(
        s.bucket, s.S, s.wsum, s.ctl, [&](int i) { return gc[tid + i * NT]; },
        [&](int i) { return (uint32_t)(tid + i * NT) < c_gt; }, [&](int i) { return (uint32_t)(i * NT) < c_gt; },
        c_gt, (uint32_t)m, ties, BucketMapT<true>(L, U), r.xo,
        [&](uint32_t slot, int32_t idx, uint32_t bits) {
            r.oidx[slot] = idx;
            if (r.ov) r.ov.put(slot, bits);
        },
        [] {});

    // ------------------------------------------------ ties at P: smallest positions, tile by tile
    if (ties) {
        const uint32_t need = (uint32_t)m - c_gt;
        const uint32_t vP = bits_of(P);
        uint32_t off = 0;  // ties in earlier tiles (uniform)
#pragma unroll 1
        for (int t = 0; t < ntiles && off < need; ++t) {
            const uint32_t e = ecnt[t];
            if (e == 0) continue;  // uniform: that tile stored no bitmap
            const uint32_t* const gt = p.ws_tie + ((int64_t)b * p.tiles_per_row + t) * BW;
            emit_ties<NT, EPT>([&](int w) { return gt[w]; }, t * TILE, off, need, c_gt, vP, r, s.wsum,
                               reinterpret_cast<uint32_t*>(s.S));
            off += e;
            __syncthreads();  // (wsum is scanned again next turn)
        }
    }
    write_padding<NT>(r.oidx, r.ov, m, r.k);
}

// Exact selection of one whole row by one workgroup, reading the row from global memory
// in chunks of NT * 16 elements (the next chunk's loads in flight while one is counted):
// MSB-first 8-bit radix passes to the exact threshold key T -- threshold-bin survivors
// staged in LDS when they fit, otherwise every later pass reads the row again, so no
// candidate is ever dropped -- then the elements above T sorted as composites, then the
// boundary ties at T taken in index order by an ordered scan of the row.
template <int NT, int KMAX, int STAGE, int VB>
__device__ void exact_row(const char* row, int32_t n, int32_t m, int32_t k, int32_t* oidx, ValOut ov, IndexOut xo,
                          RowExactSmem<NT, KMAX, STAGE>& s, int stage_cap) {
    constexpr int EC = 16;
    constexpr int CH = NT * EC;
    constexpr int NW = NT / 64;
    const int tid = opaque_tid();
    const int wave = tid >> 6;
    const PairList A{s.akey, s.apos};

    // f(key, row position, valid) for every element of the row, in every lane.
    auto sweep = [&](auto&& f) {
        auto visit = [&](const uint32_t (&u)[EC], int32_t c0, int32_t nt) {
            const int t4 = opaque_tid() * 4;
#pragma unroll
            for (int v = 0; v < EC / 4; ++v)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int32_t jl = v * NT * 4 + t4 + c;
                    f(key_of(u[4 * v + c]), c0 + jl, jl < nt);
                }
        };
        uint32_t ua[EC], ub[EC];
        load_tile<NT, EC, VB>(ua, row, min(CH, n));
#pragma unroll 1
        for (int32_t c0 = 0; c0 < n; c0 += 2 * CH) {
            const int32_t c1 = c0 + CH;
            if (c1 < n) load_tile<NT, EC, VB>(ub, row + (size_t)c1 * VB, min(CH, n - c1));
            visit(ua, c0, min(CH, n - c0));
            if (c1 >= n) break;
            const int32_t c2 = c1 + CH;
            if (c2 < n) load_tile<NT, EC, VB>(ua, row + (size_t)c2 * VB, min(CH, n - c2));
            visit(ub, c1, min(CH, n - c1));
        }
    };
    auto zero_whist = [&]() {
        uint32_t* w = &s.whist[0][0];
        for (int i = tid; i < NW * kRadix; i += NT) w[i] = 0;
    };
    auto merge = [&]() {
        __syncthreads();
        if (tid < kRadix) {
            uint32_t h = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) h += s.whist[w][tid];
            s.hist[tid] = h;
        }
        __syncthreads();
    };

    // ---------------------------------------------------------------- pass 0: top digit
    if (tid < 8) s.ctr[tid] = 0;
    zero_whist();
    __syncthreads();
    sweep([&](uint32_t kk, int32_t, bool ok) {
        if (ok) hist_add(s.whist[wave], kk >> 24);
    });
    merge();
    select_digit<NT>(s.hist, (uint32_t)m, s.wsum, s.sel);
    uint32_t prefix = s.sel[0];
    uint32_t k_rem = (uint32_t)m - s.sel[1];
    const uint32_t d0 = prefix;
    const uint32_t cap = (uint32_t)min(stage_cap, STAGE);
    const bool staged = s.hist[d0] <= cap;
    __syncthreads();

    // Collect: digit > d0 selected outright (into A), digit == d0 staged when they fit.
    sweep([&](uint32_t kk, int32_t j, bool ok) {
        const uint32_t d = kk >> 24;
        const bool g = ok && d > d0;
        const uint32_t sa = claim_slot(g, &s.ctr[1]);
        if (g && sa < (uint32_t)KMAX) A.put(sa, kk, (uint32_t)j);
        if (staged) {
            const bool cnd = ok && d == d0;
            const uint32_t sc = claim_slot(cnd, &s.ctr[0]);
            if (cnd && sc < cap) {
                s.skey[sc] = kk;
                s.sidx[sc] = (uint32_t)j;
            }
        }
    });
    __syncthreads();
    const uint32_t nstaged = staged ? min(s.ctr[0], cap) : 0u;

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
            sweep([&](uint32_t kk, int32_t, bool ok) {
                if (ok && (kk >> (shift + 8)) == prefix) hist_add(s.whist[wave], (kk >> shift) & 0xFFu);
            });
        }
        merge();
        select_digit<NT>(s.hist, k_rem, s.wsum, s.sel);
        prefix = (prefix << 8) | s.sel[0];
        k_rem -= s.sel[1];
        __syncthreads();
    }
    const uint32_t T = prefix;                      // exact threshold key
    const uint32_t need = min(k_rem, (uint32_t)m);  // ties at T to keep (>= 1)
    const uint32_t cnt_gt = (uint32_t)m - need;     // selected elements strictly above T
    const uint32_t vT = bits_of(T);

    // ---------------------------------------------------------------- the rest above T
    if (staged) {
        for (uint32_t i0 = 0; i0 < nstaged; i0 += NT) {
            const uint32_t i = i0 + tid;
            const uint32_t kk = i < nstaged ? s.skey[i] : 0u;
            const bool g = i < nstaged && kk > T;
            const uint32_t sa = claim_slot(g, &s.ctr[1]);
            if (g && sa < (uint32_t)KMAX) A.put(sa, kk, s.sidx[i]);
        }
    } else {
        sweep([&](uint32_t kk, int32_t j, bool ok) {
            const bool g = ok && (kk >> 24) == d0 && kk > T;
            const uint32_t sa = claim_slot(g, &s.ctr[1]);
            if (g && sa < (uint32_t)KMAX) A.put(sa, kk, (uint32_t)j);
        });
    }
    __syncthreads();
    const uint32_t nA = min(s.ctr[1], cnt_gt);
    bitonic_desc<NT>(A, (int)nA);
    for (uint32_t q = tid; q < nA; q += NT) {
        oidx[q] = xo(s.apos[q]);
        if (ov) ov.put(q, bits_of(s.akey[q]));
    }

    // ---------------------------------------------------------------- boundary ties, in index order
    {
        constexpr int CT = NT * 4;
        uint32_t got = 0;  // ties emitted so far (uniform)
#pragma unroll 1
        for (int32_t c0 = 0; c0 < n && got < need; c0 += CT) {
            const int32_t nt = min(CT, n - c0);
            uint32_t u4[4];
            load_tile<NT, 4, VB>(u4, row + (size_t)c0 * VB, nt);
            const int t4 = opaque_tid() * 4;
            uint32_t mk = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) mk |= (t4 + c < nt && key_of(u4[c]) == T ? 1u : 0u) << c;
            uint32_t tot;
            uint32_t rr = got + block_excl_scan<NT>((uint32_t)__popc(mk), s.wsum, &tot);
            while (mk && rr < need) {
                const int c = __ffs(mk) - 1;
                mk &= mk - 1;
                oidx[cnt_gt + rr] = xo((uint32_t)(c0 + t4 + c));
                if (ov) ov.put(cnt_gt + rr, vT);
                ++rr;
            }
            got += tot;
            __syncthreads();  // (wsum is scanned again next turn)
        }
    }
    write_padding<NT>(oidx, ov, m, k);
}

// ----------------------------------------------------------------------------- exact path

// Exact path of a row held whole by one workgroup (keys in key[]).
template <int NT, int EPT, int KMAX, typename ES>
__device__ __forceinline__ void exact_tile(const Params& p, const RowCtx& r, ES& s, const uint32_t (&key)[EPT]) {
    constexpr int G4 = EPT / 4;
    constexpr int BW = ES::BWORDS;
    constexpr int NW = ES::NW;
    constexpr int SCAPX = ES::STAGE_CAP;
    const int tid = opaque_tid();
    const int wave = tid >> 6;
    const int32_t m = r.m, k = r.k, nt = r.nt, j0 = r.j0;
    int32_t* oidx = r.oidx;
    const ValOut& ov = r.ov;

    const PairList A{s.akey, s.apos};

    // Visit every valid register element: f(key, local index).
    // (Each visit re-reads the thread index so per-slot positions are not kept live
    // across passes.)
    auto for_each = [&](auto&& f) {
        const int t4 = opaque_tid() * 4;
#pragma unroll
        for (int v = 0; v < G4; ++v) {
            const int lim = nt - v * NT * 4;
            if (lim <= 0) break;
            const int llim = lim - t4;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (c < llim) f(key[4 * v + c], t4 + (v * NT * 4 + c));
        }
    };
    // Same, but every lane of the wave calls f (valid flag passed) -- for ballots.
    auto for_each_conv = [&](auto&& f) {
        const int t4 = opaque_tid() * 4;
#pragma unroll
        for (int v = 0; v < G4; ++v) {
            const int lim = nt - v * NT * 4;
            if (lim <= 0) break;
            const int llim = lim - t4;
#pragma unroll
            for (int c = 0; c < 4; ++c) f(key[4 * v + c], t4 + (v * NT * 4 + c), c < llim);
        }
    };

    auto zero_whist = [&]() {
        uint32_t* w = &s.whist[0][0];
        for (int i = tid; i < NW * kRadix; i += NT) w[i] = 0;
    };

    // Merge the per-wave histograms.
    auto merge_hist = [&](int) {
        __syncthreads();
        if (tid < kRadix) {
            uint32_t h = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) h += s.whist[w][tid];
            s.lhist[tid] = h;
            s.hist[tid] = h;
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
    const bool staged = s.lhist[d0] <= (uint32_t)min(p.stage_cap, SCAPX);
    __syncthreads();

    // Collect: digit > d0 are selected outright (into A); digit == d0 are candidates
    // (staged in LDS when they fit).
    for_each_conv([&](uint32_t kk, int jl, bool ok) {
        const uint32_t d = kk >> 24;
        const bool g = ok && d > d0;
        const uint32_t sa = claim_slot(g, &s.ctr[1]);
        if (g && sa < (uint32_t)KMAX) A.put(sa, kk, (uint32_t)(j0 + jl));
        if (staged) {
            const bool cnd = ok && d == d0;
            const uint32_t sc = claim_slot(cnd, &s.ctr[0]);
            if (cnd && sc < (uint32_t)SCAPX) {
                uint32_t j = (uint32_t)(j0 + jl);
                asm volatile("" : "+v"(j));
                s.skey[sc] = kk;
                s.sidx[sc] = j;
            }
        }
    });
    __syncthreads();
    const uint32_t nstaged = staged ? min(s.ctr[0], (uint32_t)SCAPX) : 0u;

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
    const uint32_t T = prefix;                      // exact threshold key
    const uint32_t need = min(k_rem, (uint32_t)m);  // ties at T to keep (>= 1)
    const uint32_t cnt_gt = (uint32_t)m - need;     // selected elements strictly above T
    const uint32_t vT = bits_of(T);

    // ---------------------------------------------------------------- the rest of G
    if (staged) {
        for (uint32_t i0 = 0; i0 < nstaged; i0 += NT) {
            const uint32_t i = i0 + tid;
            const uint32_t kk = i < nstaged ? s.skey[i] : 0u;
            const bool g = i < nstaged && kk > T;
            const uint32_t sa = claim_slot(g, &s.ctr[1]);
            if (g && sa < (uint32_t)KMAX) A.put(sa, kk, s.sidx[i]);
        }
    } else {
        for_each_conv([&](uint32_t kk, int jl, bool ok) {
            const bool g = ok && (kk >> 24) == d0 && kk > T;
            const uint32_t sa = claim_slot(g, &s.ctr[1]);
            if (g && sa < (uint32_t)KMAX) A.put(sa, kk, (uint32_t)(j0 + jl));
        });
    }

    // ---------------------------------------------------------------- boundary ties
    // Rank the row's elements with key == T by index (bitmap over positions, popcount
    // prefix over its words), keep ranks < need at slots cnt_gt + rank.
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
    }
    __syncthreads();
    for (int w = tid; w < BW; w += NT) {
        uint32_t word = s.bitmap[w];
        uint32_t rr = s.wpre[w];
        while (word && rr < need) {
            const int bit = __ffs(word) - 1;
            word &= word - 1;
            const int32_t j = j0 + w * 32 + bit;
            oidx[cnt_gt + rr] = r.xo((uint32_t)j);
            if (ov) ov.put(cnt_gt + rr, vT);
            ++rr;
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- sort G and store
    const uint32_t nA = min(s.ctr[1], cnt_gt);
    bitonic_desc<NT>(A, (int)nA);
    for (uint32_t q = tid; q < nA; q += NT) {
        oidx[q] = r.xo(s.apos[q]);
        if (ov) ov.put(q, bits_of(s.akey[q]));
    }
    write_padding<NT>(oidx, ov, m, k);
}

// ----------------------------------------------------------------------------- rows

// Row setup: window (clamped length, start), output rows, and the tile of it this
// workgroup item covers (nt <= 0 when the row has no such tile).
template <int TILE, bool MULTI, int VB>
__device__ __forceinline__ RowCtx row_setup(const Params& p, int b, int tile) {
    RowCtx r;
    const int32_t len = p.lengths ? p.lengths[b] : p.max_len;
    r.b = b;
    r.tile = tile;
    r.n = min(max(len, 0), p.max_len);
    r.base = p.row_starts ? (int64_t)p.row_starts[b] : (int64_t)b * p.max_len;
    r.k = p.k;
    r.m = min(r.k, r.n);
    r.ntiles = MULTI ? max(1, (r.n + TILE - 1) / TILE) : 1;
    r.oidx = p.out_idx + (int64_t)b * r.k;
    r.ov.half = VB == 2;
    r.ov.padv = p.val_pad;
    r.ov.base = p.out_val ? static_cast<char*>(p.out_val) + (int64_t)b * r.k * VB : nullptr;
    r.j0 = tile * TILE;
    r.nt = min(TILE, r.n - r.j0);
    r.xo.mode = p.xf_mode;
    r.xo.off = p.xf_mode == 1 ? p.xf_offsets[b] : 0;
    r.xo.ps = p.xf_page;
    r.xo.shift = p.xf_shift;
    r.xo.pt = p.xf_mode == 2 ? p.xf_table + (int64_t)b * p.xf_stride : nullptr;
    r.wave_select = p.small_batch != 0;
    return r;
}

// A row that fits one tile, held whole by this workgroup: the pivot path, and the exact
// path when it misses.
template <int NT, int EPT, int KMAX, bool MULTI, int VB>
__device__ __forceinline__ void whole_tile_row(const Params& p, SmemAll<NT, EPT, KMAX, MULTI>& s, const RowCtx& r) {
    if (r.m == 0) {  // empty window: every slot is padding
        write_padding<NT>(r.oidx, r.ov, 0, r.k);
        return;
    }
    const char* const row = static_cast<const char*>(p.scores) + r.base * VB;
    uint32_t u[EPT];
    load_tile<NT, EPT, VB>(u, row, r.nt);
    // (The plateau bucket is compiled into the kernels of 1024-thread workgroups -- small
    // batches, 32K-element rows -- and of split rows, where one slow row sets the time of
    // the call.  The many-row kernels leave it out: among thousands of rows a plateau row
    // costs only its own workgroup, while the extra code measured 1.2 % slower on the
    // prefill batch.)
    constexpr bool PLATEAU = MULTI || NT == 1024;
    if (p.fast && fast_tile<NT, EPT, KMAX, PLATEAU>(r, s.fast, u, p.fast, [] {})) return;
    if (p.fast) {
        __syncthreads();  // fall back to the exact path
        // (reloaded: kept in registers through the pivot path, the tile would crowd out its
        // later phases)
        load_tile<NT, EPT, VB>(u, row, r.nt);
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) u[i] = key_of(u[i]);
    exact_tile<NT, EPT, KMAX>(p, r, s.exact, u);
}

// MINW: waves per SIMD the register allocation must allow (the LDS footprint fixes
// how many workgroups share a CU, so more registers per wave would buy nothing).
// One workgroup per row (MULTI false, grid = B: no row loop, so nothing row-invariant is
// hoisted into registers that would stay live across rows), or one workgroup per
// (row, tile) item (MULTI true; a grid-stride loop over the items, in any order: no item
// waits for another).
// VB: bytes per score (4: float32, 2: binary16 or bfloat16, widened in registers).
template <int NT, int EPT, int KMAX, bool MULTI, int MINW, int VB>
__global__ __launch_bounds__(NT, MINW) void topk_ragged_kernel(Params p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    auto& s = *reinterpret_cast<SmemAll<NT, EPT, KMAX, MULTI>*>(smem_raw);
    if constexpr (!MULTI) {
        whole_tile_row<NT, EPT, KMAX, false, VB>(p, s, row_setup<NT * EPT, false, VB>(p, (int)blockIdx.x, 0));
    } else {
        const int64_t items = (int64_t)p.B * p.tiles_per_row;
        for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
            const RowCtx r =
                row_setup<NT * EPT, true, VB>(p, (int)(it / p.tiles_per_row), (int)(it % p.tiles_per_row));
            if (r.tile >= r.ntiles) continue;  // (uniform) the row is shorter than this tile
            __syncthreads();                   // the previous item is done with LDS
            if (r.ntiles == 1) whole_tile_row<NT, EPT, KMAX, true, VB>(p, s, r);
            else split_tile<NT, EPT, KMAX, VB>(p, r, s);
        }
    }
}

}  // namespace detk
