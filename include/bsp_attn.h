/*
 * bsp_attn.h -- C ABI of the MI355X (gfx950) causal block-sparse prefill
 * attention library, libbsp_attn.so.
 *
 * The operation is the dynamic sparse attention kernel of the page
 * "长上下文推理加速方案部署实战：基于动态稀疏注意力机制的推理服务优化指南" (a deployment
 * guide for a dynamic sparse attention kernel):
 *   - section 3.2: inside the online softmax the kernel keeps the running
 *     maximum of the scores; it takes key blocks in order, forms each block's
 *     local maximum, and when the running maximum exceeds the local maximum by
 *     more than lambda the block is negligible: its softmax exponentials, the
 *     load of its V block and its product with V are all skipped. The decision
 *     uses only intermediates the kernel already has.
 *   - section 3.3 / 9.3: lambda is set at run time, per call.
 *   - section 3.5: each call reports the skipped blocks (bitmap) and counts.
 *   - section 5, step 3: the block size is a kernel parameter aligned with the
 *     KV cache's page; section 5, step 4: paged KV cache and GQA.
 *
 * Semantics of one call (readings of what the page leaves open):
 *   - causal attention per sequence, query i sees key j iff j <= i, with
 *     score = <q, k> * s_q * s_k / sqrt(head_dim) (s_* = per-head fp8 scales,
 *     1 for bf16/fp32).
 *   - queries of a sequence are cut into tiles of block_q rows and keys into
 *     blocks of block_k; tile t visits blocks 0 .. floor((last row)/block_k)
 *     in ascending order. Block j is skipped for tile t of head h iff, for
 *     EVERY valid row of the tile, (running max before block j) minus (the
 *     row's max score inside block j) is strictly greater than lambda. Rows
 *     with no visible key in the block never hold a skip back. Block 0 is never
 *     skipped. lambda is in natural-log units of the scaled score; +inf gives
 *     dense attention. Skipped keys leave numerator and denominator.
 *   - o = sum_kept p v / sum_kept p (times s_v for fp8), lse = m + ln(l) over
 *     the kept keys (natural log).
 *
 * Ownership: every pointer is caller-owned device memory (descriptors are
 * host structs). The library allocates and frees nothing. A call only
 * enqueues work on `stream` (a hipStream_t; NULL = the default stream) and
 * returns without synchronising; results are valid once the stream reaches
 * that point. Calls on different streams may run concurrently when their
 * outputs do not overlap.
 *
 * Errors: return codes only; nothing throws across the ABI. All argument
 * checks happen on the host before any HIP call, so a rejected call has no
 * effect on the device. bsp_last_error_detail() describes the last non-OK
 * status of the calling thread. Bad *device* data (cu_seqlens not
 * non-decreasing, page ids out of range) is not checked on the normal path
 * and can fault. Debug mode: with the environment variable
 * BSP_DEBUG_VALIDATE set (to anything but "" or "0") every call first copies
 * cu_seqlens (and cu_seqlens_k, the block table, lambda_per_seq) to the
 * host on its stream, waits for the copy, and checks them with
 * bsp_validate_host() below, together with the extent of the device
 * allocations holding q, k, v and o (every row the call addresses must lie
 * inside the allocation; for a paged cache this bounds the page ids). A bad
 * descriptor returns BSP_ERR_INVALID_ARG with a detail string and launches
 * nothing. The mode synchronises the stream on every call: it is for
 * debugging, not for timing.
 */
#ifndef BSP_ATTN_H
#define BSP_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSP_OK = 0,
    BSP_ERR_INVALID_ARG = 1,   /* NULL / misaligned pointer, inconsistent sizes, lambda NaN or < 0 */
    BSP_ERR_UNSUPPORTED = 2,   /* (dtype, head_dim, block_q, block_k) without a compiled kernel */
    BSP_ERR_HIP = 3,           /* a HIP launch error */
    BSP_ERR_DEVICE = 4         /* no usable device, or the current device is not gfx950 */
} bsp_status_t;

typedef enum {
    BSP_F32 = 0,
    BSP_BF16 = 1,
    BSP_FP8_E4M3 = 2           /* OCP e4m3 (max 448), per-head float scale */
} bsp_dtype_t;

/* A [tokens, heads, head_dim] tensor; head_dim is contiguous. Strides are in
 * elements and the data pointer and both strides must give 16-byte aligned
 * rows. For a paged K/V cache the "token" index is the slot index
 * page * page_size + offset. */
typedef struct {
    void *data;                /* device pointer */
    int32_t dtype;             /* bsp_dtype_t */
    int64_t stride_token;      /* elements between consecutive tokens (slots) */
    int64_t stride_head;       /* elements between consecutive heads */
    const float *scale;        /* fp8 only: device float[heads] dequantisation scale; else NULL */
} bsp_tensor_t;

/* Packed variable-length batch (section 5 step 4: dynamic batching). */
typedef struct {
    const int32_t *cu_seqlens; /* device int32[n_seqs + 1]; cu[0] = 0, non-decreasing */
    int32_t n_seqs;            /* host: number of sequences (>= 0) */
    int32_t max_seqlen;        /* host: an upper bound of every sequence length */
    int64_t total_tokens;      /* host: cu[n_seqs]; rows of q, o and the lse row length */
} bsp_seqs_t;

/* Paged K/V cache (section 5 step 4). NULL descriptor => K/V are packed like q. */
typedef struct {
    const int32_t *table;      /* device int32[n_seqs][max_pages_per_seq]: physical page of
                                  logical page p of sequence s; only entries p < ceil(len/page) are read */
    int32_t max_pages_per_seq;
    int32_t page_size;         /* tokens per page: a power of two; block_k % page_size == 0
                                  or page_size % block_k == 0 */
} bsp_block_table_t;

/* Per-call skip observability (section 3.5). */
typedef struct {
    uint32_t *bitmap;          /* device, may be NULL. Bit j of row ((h*n_seqs + s)*T_max + t),
                                  where T_max = ceil(max_seqlen/block_q); each row is
                                  W = ceil(ceil(max_seqlen/block_k)/32) uint32 words, LSB first.
                                  1 = pair (tile t, block j) was visited and skipped. The whole
                                  bitmap is rewritten by each call. */
    int64_t bitmap_words;      /* capacity in words; >= bsp_skip_bitmap_words(...) when bitmap != NULL */
    unsigned long long *skip_count;    /* device uint64[n_heads_q] or NULL: skipped pairs per head */
    unsigned long long *visited_count; /* device uint64[n_heads_q] or NULL: visited pairs per head */
} bsp_skip_out_t;

/*
 * bsp_attn_fwd -- causal block-sparse prefill attention forward.
 *
 * q   : [total_tokens, n_heads_q, head_dim]           dtype F32, BF16 or FP8_E4M3
 * k, v: [total_tokens, n_heads_kv, head_dim] packed, or a paged cache
 *       [n_pages * page_size, n_heads_kv, head_dim] when block_table != NULL;
 *       same dtype as q.
 * o   : [total_tokens, n_heads_q, head_dim]; F32 for F32 inputs, BF16 otherwise.
 * lse : device float[n_heads_q][total_tokens] or NULL.
 * cu_seqlens : sequence descriptor (required).
 * block_table: paged-cache descriptor or NULL.
 * n_heads_q % n_heads_kv == 0; query head h reads KV head h / (n_heads_q / n_heads_kv).
 * head_dim in {64, 128}; (block_q, block_k) in {(64,64), (128,64), (128,128)}.
 *   FP8_E4M3 inputs: head_dim 128 only (other head_dim: BSP_ERR_UNSUPPORTED);
 *   the q, k and v descriptors must all carry scales (positive, finite), read
 *   on the device as float[n_heads_q] for q and float[n_heads_kv] for k and v.
 *   QK^T runs on fp8 MFMA; P and V (widened exactly) enter PV as bf16.
 * lambda >= 0 or +inf (NaN and negative values are rejected).
 * skip_mask_out: observability outputs or NULL.
 * stream: hipStream_t (as void*), NULL for the default stream.
 */
bsp_status_t bsp_attn_fwd(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v,
                          bsp_tensor_t *o, float *lse,
                          const bsp_seqs_t *cu_seqlens, const bsp_block_table_t *block_table,
                          int n_heads_q, int n_heads_kv, int head_dim, int block_q, int block_k,
                          float lambda, bsp_skip_out_t *skip_mask_out, void *stream);

/* Number of uint32 words the skip bitmap needs (0 for invalid arguments). */
int64_t bsp_skip_bitmap_words(int n_heads_q, int n_seqs, int max_seqlen, int block_q, int block_k);

/*
 * Options of bsp_attn_fwd_ex. Zero-initialise the struct and set what is
 * needed; a NULL options pointer (or an all-zero struct) is bsp_attn_fwd.
 *
 *   - chunked prefill against a cached prefix (the FlowPrefill page, "FlowPrefill：
 *     突破LLM推理瓶颈…", sections 2.1 and 4.5.2: a long prompt is prefilled in
 *     fixed-size chunks, 8K combining best with its scheduler): with cu_seqlens_k set, sequence s has
 *     Lq = cu_seqlens[s+1]-cu_seqlens[s] query rows (rows of q and o) and
 *     Lk = cu_seqlens_k[s+1]-cu_seqlens_k[s] >= Lq keys/values (rows of k and
 *     v, or positions of its block-table pages). The queries are the last Lq
 *     positions: query row r sees keys 0 .. (Lk - Lq) + r (bottom-right causal
 *     alignment). Lq = 1 is one decoding step. Lk < Lq is a caller error with
 *     undefined results (the bounds live in device memory and are not read
 *     on the host).
 *   - a lambda per sequence (the guide's per-request threshold, sections 3.3
 *     and 9.3): lambda_per_seq[s] >= 0 or +inf replaces the scalar lambda for
 *     sequence s (negative or NaN values: undefined results). Calls with
 *     lambda_per_seq always run the skip-deciding kernel.
 *   - per-sequence counts (section 3.5: per-request sparsity): skip and
 *     visited (tile, block) pairs summed over the query heads, uint64[n_seqs].
 *   - ablation switches (the guide's skip_value_load / skip_softmax_exp
 *     settings, section 5, step 3): BSP_FLAG_LOAD_SKIPPED_V copies V also for
 *     blocks that every query head of the workgroup skips; BSP_FLAG_EXP_SKIPPED
 *     computes (and discards) the exponentials of skipped blocks. Results are
 *     unchanged; only the work done changes. Without the first switch a V
 *     block is read from memory only when some query head of the workgroup
 *     keeps it (with an even GQA group the workgroup holds two query heads of
 *     one KV head).
 *   Sparse calls with an even GQA group (bf16, and fp8 with packed K/V)
 *   run on 128-row tiles and 128-key blocks whatever block_q and
 *   block_k are. Each 64-row half of a tile and each 64-key half of a block is
 *   then decided on its own, in key order, so the decisions, the bitmap and
 *   the counts are those of the caller's blocks. When one 64-key half of a
 *   128-key block is kept and the other skipped, the kernel still spends the
 *   whole block's PV and exponentials; the skipped half adds zero.
 */
#define BSP_FLAG_LOAD_SKIPPED_V 1u
#define BSP_FLAG_EXP_SKIPPED 2u

typedef struct {
    const int32_t *cu_seqlens_k;   /* device int32[n_seqs+1] or NULL (= cu_seqlens) */
    int32_t max_seqlen_k;          /* host: max Lk; required when cu_seqlens_k != NULL */
    const float *lambda_per_seq;   /* device float[n_seqs] or NULL */
    unsigned long long *skip_count_per_seq;     /* device uint64[n_seqs] or NULL */
    unsigned long long *visited_count_per_seq;  /* device uint64[n_seqs] or NULL */
    uint32_t flags;                /* BSP_FLAG_* */
} bsp_fwd_options_t;

/*
 * bsp_attn_fwd_ex -- bsp_attn_fwd with the options above. Arguments as for
 * bsp_attn_fwd; with cu_seqlens_k set, the bitmap rows are
 * bsp_skip_bitmap_words_kv(...) long (one bit per key block up to
 * max_seqlen_k) and paged caches need max_pages_per_seq * page_size >=
 * max_seqlen_k. Unknown flag bits: BSP_ERR_INVALID_ARG.
 */
bsp_status_t bsp_attn_fwd_ex(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v,
                             bsp_tensor_t *o, float *lse,
                             const bsp_seqs_t *cu_seqlens, const bsp_block_table_t *block_table,
                             int n_heads_q, int n_heads_kv, int head_dim, int block_q, int block_k,
                             float lambda, bsp_skip_out_t *skip_mask_out, void *stream,
                             const bsp_fwd_options_t *options);

/* Bitmap words for a call with max_seqlen_k keys per sequence (0 for invalid arguments). */
int64_t bsp_skip_bitmap_words_kv(int n_heads_q, int n_seqs, int max_seqlen_q, int max_seqlen_k, int block_q,
                                 int block_k);

/*
 * Decoding step (the guide, section 6.1: a smaller threshold in the decoding
 * phase; section 7.2: per-token decoding latency is a validation metric): each sequence appends one query row, which sees
 * all of its Lk keys. The same skip rule applies with the row as its own
 * tile: key block j is skipped when max over earlier blocks of the block
 * maximum score minus block j's maximum exceeds lambda (strict); block 0 is
 * never skipped. The result equals bsp_attn_fwd_ex with one query row per
 * sequence (cu_seqlens = 0,1,...,n_seqs; cu_seqlens_k = seqs_k->cu_seqlens),
 * up to rounding.
 *
 * Arguments:
 *   q        [n_seqs, n_heads_q, head_dim]: row s is sequence s's new query
 *            (stride_token = distance between sequences). bf16, or fp8 e4m3
 *            with per-head scales as in bsp_attn_fwd.
 *   k, v     packed [total_tokens, n_heads_kv, head_dim] rows addressed by
 *            seqs_k->cu_seqlens, or paged through block_table (any
 *            power-of-two page size; block_k and page_size are independent).
 *   o        [n_seqs, n_heads_q, head_dim] bf16.  lse: [n_heads_q, n_seqs]
 *            fp32 natural log, or NULL.
 *   seqs_k   cu_seqlens (device int32[n_seqs+1]) of the keys including the
 *            new token, n_seqs, max_seqlen = max Lk, total_tokens =
 *            cu_seqlens[n_seqs] (rows of the score workspace).
 *   block_k  decision granularity in keys (any positive value).
 *   skip_mask_out  bitmap of bsp_skip_bitmap_words_kv(n_heads_q, n_seqs, 1,
 *            max_seqlen, 1, block_k) words: row h * n_seqs + s, bit j set iff
 *            block j was skipped; counts per query head as in bsp_attn_fwd.
 *   options  lambda per sequence, counts per sequence, ablation flags (same
 *            meaning as in bsp_fwd_options_t), or NULL.
 *   workspace  caller-owned device memory, 256-byte aligned, of at least
 *            bsp_decode_workspace_bytes(...) bytes (scores, block maxima and
 *            partial sums); its contents need no initialisation and are
 *            overwritten. Concurrent calls need separate workspaces.
 * Supported: bf16 head_dim 64 or 128, fp8 e4m3 head_dim 128, up to 8 query
 * heads per KV head (else BSP_ERR_UNSUPPORTED). A sequence with Lk = 0 gets no
 * output. The call is asynchronous on `stream` (three kernels) and
 * allocates nothing.
 */
typedef struct {
    const float *lambda_per_seq;                /* device float[n_seqs] or NULL */
    unsigned long long *skip_count_per_seq;     /* device uint64[n_seqs] or NULL */
    unsigned long long *visited_count_per_seq;  /* device uint64[n_seqs] or NULL */
    uint32_t flags;                             /* BSP_FLAG_* */
} bsp_decode_options_t;

/* Workspace bytes for bsp_attn_decode (-1 for invalid arguments). */
int64_t bsp_decode_workspace_bytes(int n_heads_q, int n_heads_kv, int n_seqs, int64_t total_k, int max_seqlen_k,
                                   int head_dim, int block_k);

bsp_status_t bsp_attn_decode(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v,
                             bsp_tensor_t *o, float *lse, const bsp_seqs_t *seqs_k,
                             const bsp_block_table_t *block_table, int n_heads_q, int n_heads_kv, int head_dim,
                             int block_k, float lambda, bsp_skip_out_t *skip_mask_out, void *stream,
                             const bsp_decode_options_t *options, void *workspace, int64_t workspace_bytes);

/*
 * bsp_attn_decode_noalloc -- bsp_attn_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Arguments, results
 * and errors are those of bsp_attn_decode; the workspace is instead a static
 * device array of BSP_DECODE_SCRATCH_BYTES bytes inside the library, one per
 * GPU, held from the first use on that GPU until the process ends. The call
 * allocates and frees nothing (the array's device address is looked up once
 * per device, on the first call there). Limit: calls whose
 * bsp_decode_workspace_bytes(...) exceeds BSP_DECODE_SCRATCH_BYTES return
 * BSP_ERR_INVALID_ARG before touching the device; 96 MiB holds e.g. 16
 * contexts of 32K keys or 4 of 128K keys at 8 KV heads with 4 query heads
 * each. All calls on one GPU share its array: calls that overlap in time on
 * one GPU (other streams, other host threads) race and give wrong results;
 * serialise them, or give each its own workspace through bsp_attn_decode.
 * The array needs no initialisation (every call overwrites what it reads).
 * The array used is that of the current device; a non-NULL stream of another
 * device returns BSP_ERR_INVALID_ARG.
 */
#define BSP_DECODE_SCRATCH_BYTES (96LL << 20)

bsp_status_t bsp_attn_decode_noalloc(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v,
                                     bsp_tensor_t *o, float *lse, const bsp_seqs_t *seqs_k,
                                     const bsp_block_table_t *block_table, int n_heads_q, int n_heads_kv,
                                     int head_dim, int block_k, float lambda, bsp_skip_out_t *skip_mask_out,
                                     void *stream, const bsp_decode_options_t *options);

/*
 * Host-side check of sequence and page descriptors (host arrays), as the
 * BSP_DEBUG_VALIDATE mode applies it to the copies of a call's device
 * descriptors (the guide's section 5, step 4: packed dynamic batches and a
 * paged KV cache). Returns BSP_OK, or BSP_ERR_INVALID_ARG with a detail
 * string for the first problem found:
 *   cu_seqlens_q   int32[n_seqs+1]: cu[0] = 0, non-decreasing, every length
 *                  <= max_seqlen_q, cu[n_seqs] == total_q (total_q < 0: not checked).
 *   cu_seqlens_k   int32[n_seqs+1] or NULL (keys = queries): the same with
 *                  max_seqlen_k and total_k, and every sequence's key count >=
 *                  its query count (chunked prefill).
 *   block_table    int32[n_seqs][max_pages_per_seq] or NULL: the
 *                  ceil(keys / page_size) pages each sequence reads must fit
 *                  its row and hold ids in [0, n_pages) (n_pages <= 0: only
 *                  ids >= 0 are checked).
 * Touches no device and needs no GPU.
 */
bsp_status_t bsp_validate_host(const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t n_seqs,
                               int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t total_q, int64_t total_k,
                               const int32_t *block_table, int32_t max_pages_per_seq, int32_t page_size,
                               int64_t n_pages);

/* Static text for a status code. */
const char *bsp_status_string(int status);

/* Thread-local description of the calling thread's last non-OK status. */
const char *bsp_last_error_detail(void);

/* Library version, major*10000 + minor*100 + patch. */
int bsp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSP_ATTN_H */
