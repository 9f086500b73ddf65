/*
 * detk.h -- exact, bitwise-deterministic ragged top-k on AMD Instinct MI355X (gfx950).
 *
 * The operation (SGLang PR #31115 "opt-in deterministic CuTe-DSL DSA top-k backend":
 * PR summary, "Modifications" and the hardening commit; docai.hu blog
 * "Non-deterministic Qwen3.8-Flash-Next...", section "The price of the fix"):
 *
 *   For each row b of a ragged batch of float32 scores, return the k highest
 *   entries of the row's window in one canonical order: score descending under
 *   the bitwise total order of the float bits (IEEE 754 totalOrder: +NaN above
 *   +inf, -0.0 below +0.0, -NaN below -inf; NaNs placed by their bits), then index
 *   ascending among bitwise-equal scores.  At the k-th boundary the tie set
 *   therefore contributes its smallest indices.  Indices are local to the window
 *   (0 <= j < n_b), front-packed; slots past min(k, n_b) hold -1.  The result is a
 *   pure function of the row's bits and k: identical across runs, streams, batch
 *   compositions and graph replays.
 *
 * All entry points are plain C.  Pointers named "device" are HIP device pointers
 * owned by the caller; the library never frees or retains them.
 */
#ifndef DETK_H
#define DETK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point.  The pages' backend replaces asserts with
 * actionable errors and makes out-of-envelope calls fail loudly (SGLang PR #31115,
 * hardening commit); every code below is found on the host, before any launch. */
typedef enum {
    DETK_OK = 0,
    DETK_ERR_INVALID_ARG = 1, /* NULL required pointer, B < 0, k < 1, max_len < 0         */
    DETK_ERR_UNSUPPORTED = 2, /* k > DETK_MAX_K, max_len > DETK_MAX_LEN, B * k >= 2^31,    */
                              /* device not gfx950                                         */
    DETK_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than detk_workspace_size()       */
    DETK_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed                 */
} detk_status;

/* Largest k supported.  The pages' deterministic backend envelope is topk <= 4096
 * (SGLang PR #31115, "Modifications" and hardening commit). */
#define DETK_MAX_K 4096

/* Longest row window supported: 2^30 elements.  The pages' backend takes rows shorter
 * than 2^24 (its composite keeps 24 index bits; SGLang PR #31115, hardening commit);
 * here a composite keeps the full 32-bit index, and the bound comes from int32 window
 * offsets (row_starts[b] + n_b < 2^31) with room for the per-row workspace.  Rows of any
 * length up to this bound run on any number of free CUs: no part of a call waits for
 * another workgroup. */
#define DETK_MAX_LEN (1 << 30)

/* What detk_workspace_size returns for a configuration detk_topk_ragged would refuse. */
#define DETK_WORKSPACE_UNSUPPORTED ((size_t)-1)

/*
 * detk_can_implement -- host-only capability query, no launch.
 * Returns DETK_OK when a call with this k and max_len can run on `device`, else the
 * status such a call would return (DETK_ERR_INVALID_ARG, DETK_ERR_UNSUPPORTED, or
 * DETK_ERR_HIP if the device cannot be queried).  Meant for construction time, so an
 * unsupported configuration is found before the first batch: vLLM PR #55872, GB10
 * failure trace, shows the alternative, a shared-memory check that fired only inside
 * the engine's warmup.
 */
int detk_can_implement(int device, int k, int32_t max_len);

/*
 * detk_workspace_size -- bytes of device workspace a call with these arguments needs:
 * 0 when every row fits one workgroup (max_len <= 32768) or B == 0, and
 * DETK_WORKSPACE_UNSUPPORTED (SIZE_MAX) when detk_can_implement would refuse the
 * configuration, so "needs none" and "cannot run" are told apart.  The same value for
 * the same (device, B, k, max_len) in one process.  Sizing the workspace on the host
 * ahead of time keeps the call free of allocation, so it can be captured into a graph
 * (SGLang PR #31115, hardening commit: no first-touch allocation under graph capture).
 */
size_t detk_workspace_size(int device, int B, int k, int32_t max_len);

/*
 * detk_topk_ragged -- the operation above, enqueued on `stream`.
 *
 *   scores      device, float32.  Row b's window is
 *               scores[s_b .. s_b + n_b) with s_b = row_starts[b] (or b * max_len
 *               when row_starts is NULL, i.e. a dense (B, max_len) matrix) and
 *               n_b = clamp(lengths[b], 0, max_len) (max_len when lengths is NULL).
 *               Metadata is trusted, as in the pages' backend (SGLang PR #31115,
 *               hardening commit): the windows must lie inside the allocation and
 *               s_b + n_b < 2^31; the library does not check them.
 *   row_starts  device int32[B] absolute element offsets, or NULL.
 *   lengths     device int32[B], or NULL.
 *   B           rows (0 returns DETK_OK without launching anything).
 *   max_len     host-known upper bound of every n_b, <= DETK_MAX_LEN; fixes the launch
 *               shape so the call never reads device metadata on the host.
 *   k           1 <= k <= DETK_MAX_K.
 *   out_idx     device int32[B * k], row-major: local indices, -1 after min(k, n_b).
 *   out_val     device float32[B * k] or NULL: the selected scores' exact bits
 *               (NaN payloads and -0.0 preserved; no floating-point op touches them),
 *               -inf in padded slots.
 *   workspace   device, at least detk_workspace_size() bytes (may be NULL when that
 *               is 0), workspace_bytes its size.  Owned by the caller.  It must be
 *               zero-filled before its first use (any fill; once, at allocation).  The
 *               words that must start at zero are the per-row counters at its start,
 *               in a control area whose extent depends on workspace_bytes alone; every
 *               call sets them back to zero, and no call writes anything else there.
 *               So a buffer passed with the same workspace_bytes every time is reused
 *               by calls of any shape without clearing (passed with another size, it
 *               is zero-filled again first).  Calls that share one workspace must be
 *               ordered (same stream, or synchronised); overlapping calls race.
 *   stream      hipStream_t (NULL = default stream).
 *
 * The call allocates nothing, never synchronises and reads no device memory on the
 * host, so it can be captured into a HIP graph (SGLang PR #31115, "Modifications":
 * graph replay bitwise equal to eager).  Argument errors are detected on the host before
 * any launch and leave every output untouched.  Once launched, the call cannot fail or
 * stall on the device: no workgroup waits for another, so it needs no co-residency and
 * completes beside any other work on the GPU.
 */
int detk_topk_ragged(const float* scores, const int32_t* row_starts, const int32_t* lengths, int B,
                     int32_t max_len, int k, int32_t* out_idx, float* out_val, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Index transform fused into the stores of a call (detk_topk_ragged_transform): the
 * serving stacks turn a row's selected local indices into buffer positions right after
 * selection -- SGLang PR #31115, "Modifications" (the fused page-table transforms that
 * follow the selection step) and vLLM PR #55872, GB10 failure trace (FlashInfer's
 * top_k_ragged_transform).  For a selected local index j of row b the call writes
 *   DETK_INDEX_LOCAL       j
 *   DETK_INDEX_OFFSET      offsets[b] + j   (an index into a packed buffer of all rows)
 *   DETK_INDEX_PAGE_TABLE  page_table[b * page_table_stride + j / page_size] * page_size
 *                          + j % page_size  (the physical slot of the row's j-th token)
 * in place of j; -1 padding and out_val are unchanged, and so is the order.
 */
#define DETK_INDEX_LOCAL 0
#define DETK_INDEX_OFFSET 1
#define DETK_INDEX_PAGE_TABLE 2
typedef struct detk_index_transform {
    int32_t mode;              /* DETK_INDEX_LOCAL, DETK_INDEX_OFFSET or DETK_INDEX_PAGE_TABLE        */
    int32_t page_size;         /* DETK_INDEX_PAGE_TABLE: tokens per page, >= 1 (powers of two shift) */
    const int32_t* offsets;    /* DETK_INDEX_OFFSET: device int32[B]                                 */
    const int32_t* page_table; /* DETK_INDEX_PAGE_TABLE: device int32, row b's pages at
                                  page_table[b * page_table_stride ...]                              */
    int64_t page_table_stride; /* entries per row, >= ceil(max_len / page_size); 0: every row reads
                                  the same table (the query rows of one sequence)                    */
} detk_index_transform;

/*
 * detk_topk_ragged_transform -- detk_topk_ragged with the index transform above applied in
 * the kernels' own stores (one pass: no second kernel rewrites out_idx).  `transform` is a
 * host pointer read during the call (NULL = DETK_INDEX_LOCAL); the offsets and page table
 * it names are device arrays owned by the caller and trusted like the row metadata (every
 * entry a window reaches must exist, and the written index must fit int32).  Errors are
 * those of detk_topk_ragged, plus DETK_ERR_INVALID_ARG for an unknown mode, a NULL array
 * the mode needs, page_size < 1, or a page_table_stride that is negative or neither 0 nor
 * >= ceil(max_len / page_size), all found on the host before any launch.
 */
int detk_topk_ragged_transform(const float* scores, const int32_t* row_starts, const int32_t* lengths, int B,
                               int32_t max_len, int k, const detk_index_transform* transform, int32_t* out_idx,
                               float* out_val, void* workspace, size_t workspace_bytes, void* stream);

/*
 * 16-bit float scores (detk_topk_ragged_16bit): the same operation on binary16 or bfloat16
 * bit patterns, ordered by IEEE totalOrder on their 16 bits (NaNs by their bits, -0 below
 * +0), ties by index; half the score bytes of float32 per element.  The pages list a
 * 16-bit (fp16) coarse first pass among the deterministic backend's follow-up levers
 * (SGLang PR #31115, "Speed Tests and Profiling").
 */
#define DETK_DTYPE_F32 0
#define DETK_DTYPE_F16 1
#define DETK_DTYPE_BF16 2

/*
 * detk_topk_ragged_16bit -- detk_topk_ragged_transform on 16-bit scores.
 *   scores   device, B rows of `dtype` (DETK_DTYPE_F16 or DETK_DTYPE_BF16) bit patterns,
 *            addressed in elements exactly as the float32 entry points address theirs.
 *   out_val  device uint16[B * k] or NULL: the selected scores' exact 16 bits; padded
 *            slots hold the format's -inf (0xFC00 binary16, 0xFF80 bfloat16).
 *   transform, out_idx, workspace, stream: as for detk_topk_ragged_transform (transform
 *            may be NULL).  detk_workspace_size() gives the same workspace need.
 * Errors are those of detk_topk_ragged_transform, plus DETK_ERR_INVALID_ARG for another
 * dtype, found on the host before any launch.
 */
int detk_topk_ragged_16bit(const void* scores, int dtype, const int32_t* row_starts, const int32_t* lengths, int B,
                           int32_t max_len, int k, const detk_index_transform* transform, int32_t* out_idx,
                           void* out_val, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the per-GPU scratch array behind detk_topk_ragged_noalloc (16 MiB). */
#define DETK_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * detk_topk_ragged_noalloc -- detk_topk_ragged without a workspace argument, for callers
 * that cannot allocate device memory at all (code under graph capture, tight serving
 * loops, harnesses that forbid allocation).  It computes the same result with the same
 * kernels; rows longer than one workgroup tile use a scratch array of
 * DETK_SCRATCH_BYTES that the library holds on each GPU it runs on until the process
 * ends (its address is taken once per device at the library's first call there).  No
 * call allocates or frees anything, and the call is enqueued on `stream` like
 * detk_topk_ragged.
 *   Arguments, outputs and errors are those of detk_topk_ragged, except:
 *   DETK_ERR_WORKSPACE  the call would need more workspace than DETK_SCRATCH_BYTES
 *                       (detk_workspace_size() > DETK_SCRATCH_BYTES), found on the host
 *                       before any launch; every output is left untouched.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two
 *   streams, or two host threads, without ordering between them) race and give
 *   undefined results.  Each call leaves the array ready for the next one.
 */
int detk_topk_ragged_noalloc(const float* scores, const int32_t* row_starts, const int32_t* lengths, int B,
                             int32_t max_len, int k, int32_t* out_idx, float* out_val, void* stream);

/*
 * detk_indexer_scores -- the score producer upstream of the selection: the DSA
 * lightning-indexer score (SGLang PR #31115, review thread: a sum over the indexer heads
 * of ReLU-ed per-head dot products, weighted per head, which is why keys whose heads all
 * score non-positive sit on exactly 0.0), for B query rows over one key sequence:
 *     out[b * max_len + t] = sum_h w[b * heads + h] *
 *                            max(0, sum_d q[(b * heads + h) * head_dim + d] * keys[t * head_dim + d])
 * for t < n_b = clamp(lengths[b], 0, max_len) (lengths NULL: n_b = max_len): row b's window
 * is keys[0, n_b), as in chunked causal prefill.  Entries t >= n_b of a row are not written.
 *   q     device, bfloat16 bit patterns, [B][heads][head_dim], 16-byte aligned
 *   w     device, float32, [B][heads], 16-byte aligned
 *   keys  device, bfloat16 bit patterns, [n_keys][head_dim], 16-byte aligned
 *   out   device, float32, [B][max_len] -- the layout detk_topk_ragged reads with
 *         row_starts NULL (row b at b * max_len), so the two calls chain on one stream
 * Products are exact (bfloat16 x bfloat16 fits float32) and sums are float32 on the matrix
 * cores, in a fixed order: the same inputs give the same bits on every call.  The sums'
 * order is not the oracle's, so results agree with the exact value within the float32
 * forward error bound (D + H + 8) 2^-24 sum_h |w_h| sum_d |q_hd k_td|.
 * q, w and keys must be finite (a NaN or infinite operand leaves the scores it reaches
 * unspecified).  Supported shape: heads = 16, head_dim = 128, and at most 8,388,607 key
 * rows (2^31 - 1 bytes of keys) (else DETK_ERR_UNSUPPORTED).  max_len must
 * not exceed n_keys (DETK_ERR_INVALID_ARG), pointers must be non-NULL and aligned when
 * B > 0 and max_len > 0.  Allocates nothing, never synchronizes; ordered on `stream`.
 */
int detk_indexer_scores(const void* q, const float* w, const void* keys, int32_t n_keys, const int32_t* lengths,
                        int B, int heads, int head_dim, int32_t max_len, float* out, void* stream);

/*
 * detk_status_string -- human-readable text for a status code, naming the condition
 * that produced it (static storage; "unknown detk status" for other values).  The pages'
 * backend replaces bare asserts with actionable errors (SGLang PR #31115, hardening
 * commit).
 */
const char* detk_status_string(int status);

/*
 * detk_read_probe -- MEASUREMENT, not part of the top-k path.  Reads the `bytes` bytes at
 * `data` (device memory) exactly once with 16-byte loads, a grid-stride loop spread over
 * every CU, and XORs them into *out (one device word the caller zeroed).  Its bandwidth is
 * what a plain streaming read attains on the GPU: the ceiling for the score scan.
 * `data` must be 16-byte aligned and `bytes` a multiple of 16 (else DETK_ERR_INVALID_ARG);
 * bytes == 0 returns DETK_OK with no launch.  Ordered on `stream`; allocates nothing.
 */
int detk_read_probe(const void* data, size_t bytes, uint32_t* out, void* stream);

/*
 * detk_debug_set -- TEST-ONLY process-wide overrides (not thread-safe; set them before
 * issuing calls).  Every override changes only how the result is computed, never the
 * result, so tests can drive every fallback the pages require to exist (threshold-bin
 * overflow falls back to rescans and never drops a candidate: SGLang PR #31115, PR
 * summary).
 *   what = DETK_DEBUG_PATH:        0 automatic, 1 one workgroup per row, 2 rows split
 *                                  over several workgroups (one tile each).
 *   what = DETK_DEBUG_STAGING_CAP: -1 default; else the largest threshold-bin
 *                                  candidate count staged in LDS (0 forces every
 *                                  refinement pass to rescan the row).
 *   what = DETK_DEBUG_MULTI_TILE:  0 default; else elements per workgroup tile of the
 *                                  split-row path (4096, 8192, 16384 or 32768).
 *   what = DETK_DEBUG_FAST:        1 default (sampled-pivot path, exact radix path when
 *                                  it misses); 0 exact radix path only; 2 pivot forced
 *                                  to miss, so every row starts on the pivot path and
 *                                  falls back.
 *   what = DETK_DEBUG_SMALL_BATCH: 0 default (a batch with no more workgroups than CUs
 *                                  takes the small-batch shapes: 1024 threads per
 *                                  one-workgroup row, pivot digits selected by every
 *                                  wave); 1 never; 2 always.
 *   what = DETK_DEBUG_SPLIT_SAMPLES: 0 default (rows split over workgroups take 4096
 *                                  samples when the candidate list has room for the
 *                                  longest row, else 8192); 1 always 8192; 2 always 4096.
 * Returns DETK_OK or DETK_ERR_INVALID_ARG.
 */
#define DETK_DEBUG_PATH 1
#define DETK_DEBUG_STAGING_CAP 2
#define DETK_DEBUG_MULTI_TILE 3
#define DETK_DEBUG_FAST 4
#define DETK_DEBUG_SMALL_BATCH 5
#define DETK_DEBUG_SPLIT_SAMPLES 6
int detk_debug_set(int what, int value);

#ifdef __cplusplus
}
#endif

#endif /* DETK_H */
