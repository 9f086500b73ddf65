/*
 * detk_oracle.c -- plain CPU oracle for exact, bitwise-deterministic ragged top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path never
 * calls it and shares no source, header or table with it.
 *
 * What it computes (the plain definition, written out):
 *   SGLang PR #31115 "opt-in deterministic CuTe-DSL DSA top-k backend", PR summary
 *   and "Modifications": the result is the canonical order -- score descending,
 *   index ascending among bitwise-equal scores -- so the k-th boundary keeps the
 *   smallest-index subset of its tie set; output is (B, topk) int32 local
 *   indices, front-packed, padded with -1.
 *   The same PR's hardening commit: the order is a bitwise total order on the
 *   float bits (NaN is placed by its bits, not torch.topk's NaN-maximal rule),
 *   and window clamps trust the row metadata.
 *   docai.hu blog "Non-deterministic Qwen3.8-Flash-Next...", section "The price
 *   of the fix": the exact result equals a full sort followed by truncation to k
 *   and -1 padding when the row is shorter than k.
 *
 * Per row b:
 *   n   = clamp(lengths[b], 0, max_len)        (lengths NULL: n = max_len)
 *   s   = row_starts[b]                         (row_starts NULL: s = b * max_len)
 *   key = the float's 32 bits mapped so that unsigned order is IEEE 754
 *         totalOrder: a negative pattern (sign bit set) is complemented, a
 *         positive pattern gets its sign bit set.
 *   Sort positions 0..n-1 by (key descending, position ascending) with qsort --
 *   sorting on that pair is exactly a stable sort on the key -- keep the first
 *   m = min(k, n), write -1 / -inf after them.
 *
 * No floating-point operation ever touches a score: values are copied as bits.
 * 16-bit rows (binary16 or bfloat16) are ordered the same way on their 16 bits.
 * Rows are split over POSIX threads in contiguous blocks; each row is
 * independent, so the thread count does not change the result.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    uint32_t key;
    int32_t pos;
} oracle_item;

/* IEEE 754 totalOrder as an unsigned key (see header). */
static uint32_t oracle_total_order_key(uint32_t bits)
{
    if (bits & 0x80000000u)
        return ~bits;
    return bits | 0x80000000u;
}

/* (key descending, position ascending). */
static int oracle_cmp(const void* pa, const void* pb)
{
    const oracle_item* a = (const oracle_item*)pa;
    const oracle_item* b = (const oracle_item*)pb;
    if (a->key != b->key)
        return a->key > b->key ? -1 : 1;
    if (a->pos != b->pos)
        return a->pos < b->pos ? -1 : 1;
    return 0;
}

/* The same order for 16-bit floats (binary16 or bfloat16; both keep the sign in the top
 * bit): a negative pattern is complemented, a positive one gets its sign bit set, so
 * unsigned order is IEEE totalOrder on the 16-bit patterns. */
static uint32_t oracle_total_order_key16(uint16_t bits)
{
    if (bits & 0x8000u)
        return (uint16_t)~bits;
    return bits | 0x8000u;
}

typedef struct {
    const uint32_t* scores;
    const uint16_t* scores16;   /* 16-bit rows instead of scores (then out_val16, pad16) */
    const int32_t* row_starts;
    const int32_t* lengths;
    int32_t max_len;
    int k;
    int32_t* out_idx;
    uint32_t* out_val;
    uint16_t* out_val16;
    uint16_t pad16;
    int row_begin;
    int row_end;
    int status;
} oracle_job;

static void oracle_row(const oracle_job* job, int b, oracle_item* items)
{
    int64_t len = job->lengths ? job->lengths[b] : job->max_len;
    if (len < 0)
        len = 0;
    if (len > job->max_len)
        len = job->max_len;
    int32_t n = (int32_t)len;
    int64_t start = job->row_starts ? (int64_t)job->row_starts[b] : (int64_t)b * job->max_len;
    if (job->scores16) {
        const uint16_t* row16 = job->scores16 + start;
        for (int32_t j = 0; j < n; ++j) {
            items[j].key = oracle_total_order_key16(row16[j]);
            items[j].pos = j;
        }
        qsort(items, (size_t)n, sizeof(oracle_item), oracle_cmp);
        int32_t m = n < job->k ? n : job->k;
        int32_t* oi = job->out_idx + (int64_t)b * job->k;
        uint16_t* ov = job->out_val16 ? job->out_val16 + (int64_t)b * job->k : NULL;
        for (int t = 0; t < job->k; ++t) {
            oi[t] = t < m ? items[t].pos : -1;
            if (ov)
                ov[t] = t < m ? row16[items[t].pos] : job->pad16;
        }
        return;
    }
    const uint32_t* row = job->scores + start;

    for (int32_t j = 0; j < n; ++j) {
        items[j].key = oracle_total_order_key(row[j]);
        items[j].pos = j;
    }
    qsort(items, (size_t)n, sizeof(oracle_item), oracle_cmp);

    int32_t m = n < job->k ? n : job->k;
    int32_t* oi = job->out_idx + (int64_t)b * job->k;
    uint32_t* ov = job->out_val ? job->out_val + (int64_t)b * job->k : NULL;
    for (int t = 0; t < job->k; ++t) {
        if (t < m) {
            oi[t] = items[t].pos;
            if (ov)
                ov[t] = row[items[t].pos];
        } else {
            oi[t] = -1;
            if (ov)
                ov[t] = 0xFF800000u; /* -inf in padded slots */
        }
    }
}

static void* oracle_worker(void* arg)
{
    oracle_job* job = (oracle_job*)arg;
    if (job->row_begin >= job->row_end)
        return NULL;
    oracle_item* items = (oracle_item*)malloc(sizeof(oracle_item) * (size_t)(job->max_len > 0 ? job->max_len : 1));
    if (!items) {
        job->status = 1;
        return NULL;
    }
    for (int b = job->row_begin; b < job->row_end; ++b)
        oracle_row(job, b, items);
    free(items);
    return NULL;
}

/* Both entry points: 32-bit rows (scores, out_val) or 16-bit rows (scores16, out_val16). */
static int oracle_run(const uint32_t* scores, const uint16_t* scores16, const int32_t* row_starts,
                      const int32_t* lengths, int B, int32_t max_len, int k, int32_t* out_idx,
                      uint32_t* out_val, uint16_t* out_val16, uint16_t pad16, int nthreads)
{
    if (B < 0 || k < 1 || max_len < 0 || !out_idx || (B > 0 && !scores && !scores16))
        return 1;
    if (B == 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > B)
        nthreads = B;

    oracle_job* jobs = (oracle_job*)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return 1;
    }
    int per = B / nthreads, extra = B % nthreads, row = 0;
    for (int t = 0; t < nthreads; ++t) {
        oracle_job* j = &jobs[t];
        j->scores = scores;
        j->scores16 = scores16;
        j->out_val16 = out_val16;
        j->pad16 = pad16;
        j->row_starts = row_starts;
        j->lengths = lengths;
        j->max_len = max_len;
        j->k = k;
        j->out_idx = out_idx;
        j->out_val = out_val;
        j->row_begin = row;
        row += per + (t < extra ? 1 : 0);
        j->row_end = row;
        j->status = 0;
    }
    int status = 0;
    char* joined = (char*)calloc((size_t)nthreads, 1);
    for (int t = 1; t < nthreads; ++t) {
        if (joined && pthread_create(&tids[t], NULL, oracle_worker, &jobs[t]) == 0)
            joined[t] = 1;
        else
            oracle_worker(&jobs[t]); /* could not start a thread: run the block here */
    }
    oracle_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (joined && joined[t])
            pthread_join(tids[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        status |= jobs[t].status;
    free(joined);
    free(jobs);
    free(tids);
    return status;
}

/*
 * Host pointers only.  scores: float32 bit patterns; out_val may be NULL.
 * Returns 0 on success, 1 on bad arguments or allocation failure.
 */
int detk_oracle_topk_ragged(const uint32_t* scores, const int32_t* row_starts, const int32_t* lengths,
                            int B, int32_t max_len, int k, int32_t* out_idx, uint32_t* out_val,
                            int nthreads)
{
    return oracle_run(scores, NULL, row_starts, lengths, B, max_len, k, out_idx, out_val, NULL, 0, nthreads);
}

/*
 * The same for 16-bit floats (binary16 or bfloat16 bit patterns): the order is IEEE
 * totalOrder on the 16 bits, values are copied as 16 bits, and padded value slots get
 * pad16 (the format's -inf: 0xFC00 for binary16, 0xFF80 for bfloat16).
 */
int detk_oracle_topk_ragged16(const uint16_t* scores, const int32_t* row_starts, const int32_t* lengths,
                              int B, int32_t max_len, int k, int32_t* out_idx, uint16_t* out_val,
                              uint16_t pad16, int nthreads)
{
    return oracle_run(NULL, scores, row_starts, lengths, B, max_len, k, out_idx, NULL, out_val, pad16, nthreads);
}

/* The key of one bit pattern, exported so tests can pin the mapping itself. */
uint32_t detk_oracle_key(uint32_t bits) { return oracle_total_order_key(bits); }
uint32_t detk_oracle_key16(uint16_t bits) { return oracle_total_order_key16(bits); }

/*
 * Index transform of a selection -- the serving stacks' step right after top-k selection
 * (SGLang PR #31115, "Modifications": the deterministic backend returns local indices and
 * leaves the fused page-table transforms to a separate step; vLLM PR #55872, GB10 failure
 * trace: FlashInfer's ragged top-k with its transform, top_k_ragged_transform).  Written
 * out slot by slot, for a slot of row b holding a local index j >= 0:
 *   mode 1 (offset):     offsets[b] + j                      (an index into a packed buffer)
 *   mode 2 (page table): page_table[b * stride + j / page_size] * page_size + j % page_size
 *                        (the physical slot of the row's j-th logical token, pages of
 *                        page_size tokens)
 *   mode 0:              j
 * A slot holding -1 (padding) stays -1.
 * Returns 0, or 1 on bad arguments.
 */
int detk_oracle_index_transform(const int32_t* local_idx, int B, int k, int mode, const int32_t* offsets,
                                const int32_t* page_table, int64_t stride, int32_t page_size, int32_t* out)
{
    if (B < 0 || k < 1 || !local_idx || !out || mode < 0 || mode > 2)
        return 1;
    if (mode == 1 && !offsets)
        return 1;
    if (mode == 2 && (!page_table || page_size < 1 || stride < 0))
        return 1;
    for (int b = 0; b < B; ++b) {
        for (int t = 0; t < k; ++t) {
            int32_t j = local_idx[(int64_t)b * k + t];
            int32_t v = j;
            if (j >= 0 && mode == 1)
                v = offsets[b] + j;
            if (j >= 0 && mode == 2) {
                int32_t page = j / page_size;
                int32_t within = j % page_size;
                v = page_table[(int64_t)b * stride + page] * page_size + within;
            }
            out[(int64_t)b * k + t] = v;
        }
    }
    return 0;
}
