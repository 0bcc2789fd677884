/*
 * fd.h -- C ABI of the split-KV ("FlashDecoding") attention library for
 * AMD MI355X (gfx950).
 *
 * The operation.  For every sequence b, query head h and query position t,
 *
 *     out[b,h,t,:] = softmax_j( scale * <q[b,h,t,:], k[b,g,j,:]> ) . v[b,g,j,:]
 *     lse[b,h,t]   = ln sum_j exp( scale * <q[b,h,t,:], k[b,g,j,:]> )
 *
 * over the keys j the row may see, with g = h / (Hq / Hkv) (consecutive query
 * heads share one KV head; page "FlashDecoding算法原理与多GPU并行解码实战",
 * engineering details item 3).  For decode (q_len = 1) the row sees keys
 * 0 .. L_b-1, L_b = cache_lens[b] (the length mask of that page's multi-GPU
 * section).  For a chunk of q_len > 1 new tokens whose K/V are already the
 * last q_len entries of the cache, position t sees keys 0 .. L_b-q_len+t
 * (page "ChunkedPrefill与FlashDecoding技术解析" §2.1: causal within the chunk,
 * full view of the cached prefix).  A row with no visible key gets out = 0
 * and lse = -inf.
 *
 * The method.  The keys of each sequence are cut along the sequence axis into
 * tiles ("splits"); each tile yields a normalised partial output o_s, its row
 * max m_s and its log-sum-exp lse_s (page "ChunkedPrefill与FlashDecoding技术
 * 解析" §3.1, tiles of typically 256-1024 tokens); a second pass merges the
 * partials by rescaling with the global maximum (same page §3.1 and §3.2; the
 * merge of page "FlashDecoding算法原理..." multi-GPU step 3):
 *     LSE = ln sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) o_s.
 *
 * Conventions shared by every call:
 *   - Tensors are dense, row-major, in device memory owned by the caller.
 *     The library never allocates, frees or synchronises: work is enqueued
 *     on `stream` (a hipStream_t; NULL = the default stream) and the call
 *     returns at once.
 *   - q, out   [B, Hq, q_len, D]     dtype of fd_dims.dtype
 *     k_cache, v_cache [B, Hkv, Lmax, D]   same dtype
 *     cache_lens [B] int32 on the device, each in [0, Lmax] (values outside
 *     are clamped into that range on the device; they are never read past)
 *     lse [B, Hq, q_len] fp32, natural log, may be NULL
 *   - q, k_cache, v_cache, out, o_part must be 16-byte aligned.
 *   - Every call validates its arguments first.  On any error it returns a
 *     negative fd_status, records a message for fd_last_error(), and enqueues
 *     nothing.  A device-side launch failure returns FD_ERR_DEVICE.
 *   - Supported: dtype FD_F32 or FD_BF16; D = 64 or 128; any Hq/Hkv ratio;
 *     any q_len >= 1.  One tile's keys of one KV head must span fewer than
 *     2^31 bytes of a cache (for bf16 at D = 128, fewer than 8,388,608 keys):
 *     a call whose split rule allows a larger tile (few splits over a very
 *     long max_cache_len) returns FD_ERR_UNSUPPORTED; more splits fix it.
 *     Under balanced spans (fd_plan.spans > 0) a piece can hold a whole
 *     (sequence, KV head) pair, so max_cache_len itself must stay below
 *     that bound; the planner asks for spans only then.  Arithmetic is fp32 throughout (scores, softmax,
 *     accumulation); out is rounded to its dtype with round-to-nearest-even.
 *     Caches of one-byte codes (FP8 E4M3, INT8) with bf16 q and out have
 *     calls of their own (fd_decode_attention_fp8, fd_decode_attention_int8),
 *     and paged caches take a block table (fd_decode_attention_paged and the
 *     pages argument of the one-byte calls).
 */
#ifndef FD_H
#define FD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fd_status {
    FD_OK = 0,
    FD_ERR_INVALID = -1,     /* malformed arguments */
    FD_ERR_UNSUPPORTED = -2, /* well-formed but not implemented (dtype, D) */
    FD_ERR_WORKSPACE = -3,   /* workspace missing or too small */
    FD_ERR_DEVICE = -4       /* HIP runtime error */
} fd_status;

typedef enum fd_dtype {
    FD_F32 = 0,
    FD_BF16 = 1,
    FD_FP8_E4M3 = 2, /* K/V caches only */
    FD_INT8 = 3      /* K/V caches only */
} fd_dtype;

/* Most partial slots a row may have. */
#define FD_MAX_SPLITS 256

typedef struct fd_dims {
    int32_t batch;         /* B >= 0 (0: nothing to do) */
    int32_t num_q_heads;   /* Hq >= 1 */
    int32_t num_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t head_dim;      /* D: 64 or 128 */
    int32_t q_len;         /* query rows per sequence, >= 1 (1 = decode) */
    int32_t max_cache_len; /* Lmax >= 0: capacity (row stride) of the caches */
    int32_t dtype;         /* fd_dtype of q, k_cache, v_cache, out */
} fd_dims;

/* A split plan.  Sequence b is cut into tiles of `tile_len` keys,
 * S_b = min(ceil(L_b / tile_len), max_splits) of them; when the ceiling
 * exceeds max_splits the last tile also takes the remaining keys.
 *
 * With spans > 0 (and max_splits >= 2) the matrix-core decode kernel
 * (bf16 queries, up to 32 query rows per KV head, any cache format or
 * layout) balances the batch instead.  A launch uses n = min(spans, the
 * workgroups of the kernel that runs resident at once on the device) spans,
 * one workgroup each.  The 16-key blocks of all (sequence, KV head) pairs
 * with keys are laid on one line, sequence by sequence and head by head,
 * each pair's blocks preceded by 16 positions that stand for the fixed cost
 * of a piece; the line is cut into n equal contiguous spans of
 * max(ceil(line length / n), ceil(longest sequence's blocks / (max_splits -
 * 1))) positions, and the blocks of a pair inside one span are one split.  The pieces of a pair fill its slots 0, 1, ... in key order
 * (slot = span index - index of the span holding the pair's first block)
 * and its remaining slots are empty (m_part = lse_part = -inf, o_part
 * untouched), as are all slots of a sequence without keys.  The merged
 * result is the same attention; which keys share a split differs from the
 * tile rule.  Other kernels (fp32 queries, longer query chunks) keep the
 * tile rule.
 *
 * Callers may fill a plan by hand (tile_len >= 1, 1 <= max_splits <=
 * FD_MAX_SPLITS, 0 <= spans <= 2^20; zero-initialise it) or get one from
 * fd_plan_splits. */
typedef struct fd_plan {
    int32_t tile_len;         /* keys per tile */
    int32_t max_splits;       /* partial slots per row */
    uint64_t workspace_bytes; /* bytes fd_decode_attention needs (0 if max_splits == 1) */
    int32_t work_units;       /* (sequence, KV head, row block, tile) units holding keys */
    int32_t spans;            /* > 0: this many balanced spans on the matrix-core decode kernel, 0: tiles */
} fd_plan;

/* fd_plan_splits -- choose tile length and split counts from host lengths.
 *
 * Host-only and pure: reads `cache_lens_host` [B] (host memory), writes
 * `*plan` and, if non-NULL, `splits_per_seq` [B] (host memory, S_b per
 * sequence).  With `num_splits` > 0 the count is forced: sequence b uses
 * tiles of ceil(L_b / num_splits) keys (the chunk size of the algorithm
 * section of page "FlashDecoding算法原理..."), which may give fewer than
 * num_splits tiles; plan->tile_len is then 0 and plan->max_splits =
 * num_splits (<= FD_MAX_SPLITS).  With num_splits == 0 the planner picks one
 * tile length for the batch: the batch's (sequence, KV head, row block) key
 * rows spread over one work unit per compute unit when all lengths are equal
 * and four per compute unit otherwise, at least 256 keys (below
 * about 256 keys per chunk launch overhead eats the gain, page
 * "FlashDecoding算法原理..." benchmark section), at most the longest sequence,
 * raised if needed so no sequence needs more than FD_MAX_SPLITS.  When the
 * lengths differ, the batch has at most 256 sequences, the call goes to the
 * matrix-core decode kernel and the tiles outnumber two per compute unit,
 * the plan also asks for two spans per compute unit (spans of at least 256
 * keys) and raises max_splits to what they need
 * (equal shares of the batch's keys, as page "FlashDecoding算法原理..."
 * variable-length section allots them to devices).  splits_per_seq reports the tile rule's counts.
 * `num_cus` is the compute-unit count to plan for; 0 queries the current
 * HIP device (the only device call this function may make).
 * Errors: FD_ERR_INVALID for bad dims, negative lengths, lengths above
 * max_cache_len, num_splits outside [0, FD_MAX_SPLITS] or num_cus < 0. */
fd_status fd_plan_splits(const fd_dims* dims, const int32_t* cache_lens_host, int32_t num_splits,
                         int32_t num_cus, fd_plan* plan, int32_t* splits_per_seq);

/* fd_workspace_bytes -- bytes of workspace fd_decode_attention needs for
 * `max_splits` partial slots per row (0 when max_splits <= 1 or dims are
 * invalid).  The workspace holds o_part, m_part and lse_part as laid out for
 * fd_decode_partials, each starting on a 256-byte boundary. */
uint64_t fd_workspace_bytes(const fd_dims* dims, int32_t max_splits);

/* fd_decode_partials -- the first pass only: per-tile partials.
 *
 * Slots per row S = num_splits if num_splits > 0, else plan->max_splits
 * (plan must then be non-NULL).  Writes, for every row (b,h,t) and slot s:
 *   o_part  [B, Hq, q_len, S, D] fp32  tile output normalised by its own sum
 *   m_part  [B, Hq, q_len, S]    fp32  tile max of the scaled scores
 *   lse_part[B, Hq, q_len, S]    fp32  tile log-sum-exp (natural log)
 * A slot whose tile holds no key visible to the row gets m = lse = -inf and
 * its o_part entry is left unwritten.  This is the "local O and S" step of
 * page "ChunkedPrefill与FlashDecoding技术解析" §3.2; the partials of several
 * devices can be merged with fd_combine_splits.
 * Errors as listed under the conventions; FD_ERR_INVALID if o_part, m_part
 * or lse_part is NULL. */
fd_status fd_decode_partials(const fd_dims* dims, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* cache_lens, float scale,
                             int32_t num_splits, const fd_plan* plan, float* o_part,
                             float* m_part, float* lse_part, void* stream);

/* fd_combine_splits -- the second pass only: merge partials.
 *
 * rows = batch * num_heads * q_len; o_part [rows, max_splits, head_dim] and
 * lse_part [rows, max_splits] fp32 in device memory.  Row r belongs to
 * sequence b = r / (num_heads * q_len).  `splits_per_seq` (device [batch]
 * int32, or NULL) gives the slots S_b that sequence b holds: its rows merge
 * slots 0 .. S_b - 1 and never read the others (values are clamped into
 * [0, max_splits]; S_b = 0 gives out = 0, lse = -inf).  NULL means every
 * sequence holds max_splits slots.  This is the merge of page
 * "FlashDecoding算法原理与多GPU并行解码实战", multi-GPU section step 3, and of
 * the per-device local results of page "ChunkedPrefill与FlashDecoding技术解析"
 * §3.2, where sequences may carry different numbers of partials.  Slots with
 * lse = -inf are empty: their o_part entries do not affect the result and
 * may hold anything, NaN included.  Writes out [rows, head_dim] in out_dtype
 * (FD_F32 or FD_BF16, RNE) and, if non-NULL, lse [rows] fp32.  A row without
 * a finite slot gets out = 0 and lse = -inf.  Errors: FD_ERR_INVALID for
 * negative sizes, max_splits outside [1, FD_MAX_SPLITS], NULL or misaligned
 * buffers; FD_ERR_UNSUPPORTED for other head_dim or out_dtype values. */
fd_status fd_combine_splits(int32_t batch, int32_t num_heads, int32_t q_len, int32_t head_dim,
                            int32_t max_splits, const float* o_part, const float* lse_part,
                            const int32_t* splits_per_seq, int32_t out_dtype, void* out, float* lse,
                            void* stream);

/* fd_decode_attention -- the whole operation: partials, then merge.
 *
 * Split choice: num_splits > 0 forces that many tiles per sequence (as in
 * fd_plan_splits); else `plan` (may be NULL: one tile per sequence).  With a
 * single slot the partial kernel writes out and lse directly and no
 * workspace is needed (`workspace` may be NULL).  Otherwise `workspace`
 * (device memory, 256-byte aligned, caller-owned, contents irrelevant on
 * entry and clobbered on return) must hold at least
 * fd_workspace_bytes(dims, slots) bytes, else FD_ERR_WORKSPACE.  Calls that
 * share a workspace must not run concurrently. */
fd_status fd_decode_attention(const fd_dims* dims, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* cache_lens, float scale,
                              int32_t num_splits, const fd_plan* plan, void* workspace,
                              uint64_t workspace_bytes, void* out, float* lse, void* stream);

/* fd_decode_attention_noalloc -- fd_decode_attention for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.
 *
 * Same operation, arguments and errors as fd_decode_attention, without the
 * workspace arguments: the partials live in a statically allocated scratch
 * area of FD_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from
 * the library's load until the process ends.  A call whose workspace
 * (fd_workspace_bytes of its dims and slots) exceeds that returns
 * FD_ERR_WORKSPACE and enqueues nothing.  The call allocates nothing and
 * calls no allocating routine; the first call on a device looks up that
 * device's scratch address once.  Every call on one GPU uses the same scratch
 * and leaves its contents to the next: calls that may overlap on one GPU
 * (two streams, two threads) race and must be serialised by the caller.
 * Single-slot calls (one tile per sequence) use no scratch at all. */
#define FD_NOALLOC_SCRATCH_BYTES (32ull << 20)
fd_status fd_decode_attention_noalloc(const fd_dims* dims, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* cache_lens, float scale,
                                      int32_t num_splits, const fd_plan* plan, void* out, float* lse,
                                      void* stream);

/* Paged K/V caches.
 *
 * Page "FlashDecoding算法原理与多GPU并行解码实战" (deployment engineering
 * details, item 1) names the PagedAttention cache layout, pages of page_size
 * keys by num_kv_heads by head_dim, and notes that a split-KV kernel needing
 * contiguous sequences pays for a page-to-contiguous copy before attention;
 * the same page's section on combining methods pairs paged caches with the
 * split-KV method.  The paged entry point below reads the pages in place:
 * no copy.
 *
 * k_pages and v_pages hold num_pages pages of page_size keys each, laid out
 *   FD_PAGES_NHD: [num_pages, page_size, Hkv, D]  (the page's layout)
 *   FD_PAGES_HND: [num_pages, Hkv, page_size, D]
 * block_table [B, max_pages_per_seq] int32 (device memory): key j of
 * sequence b lives in page block_table[b][j / page_size], row
 * j mod page_size.  Only the entries for keys below cache_lens[b] are read.
 * An entry outside [0, num_pages) is never dereferenced: its keys read as
 * zero vectors (score 0, value 0) -- callers must not rely on that, it only
 * keeps a bad table from reading outside the pool.
 * page_size is a power of two, at least 16. */
typedef enum fd_page_layout { FD_PAGES_NHD = 0, FD_PAGES_HND = 1 } fd_page_layout;

typedef struct fd_kv_pages {
    const int32_t* block_table;  /* device [B, max_pages_per_seq] */
    int32_t max_pages_per_seq;   /* >= 1 */
    int32_t page_size;           /* keys per page: power of two, >= 16 */
    int32_t num_pages;           /* pages in k_pages and v_pages, >= 1 */
    int32_t layout;              /* fd_page_layout */
} fd_kv_pages;

/* fd_decode_attention_paged -- fd_decode_attention over a paged cache.
 *
 * Same operation, arguments and conventions as fd_decode_attention, with
 * k_pages / v_pages / pages in place of k_cache / v_cache.
 * dims->max_cache_len must equal max_pages_per_seq * page_size (the
 * capacity of a sequence; cache_lens are clamped into [0, capacity] on the
 * device).  Tiles start at multiples of 16 keys: a plan's tile_len must be a
 * multiple of 16 (fd_plan_splits gives multiples of 64), and with a forced
 * num_splits the tile is ceil(L_b / num_splits) rounded up to a multiple of
 * 16, which may give fewer tiles.  Plans and workspace sizes are those of
 * fd_plan_splits / fd_workspace_bytes for the same dims.
 * Errors: as fd_decode_attention; FD_ERR_INVALID for a NULL pages or
 * block_table, bad page counts or sizes, or max_cache_len mismatch;
 * FD_ERR_UNSUPPORTED for page sizes that are not powers of two >= 16 or an
 * unknown layout. */
fd_status fd_decode_attention_paged(const fd_dims* dims, const void* q, const void* k_pages,
                                    const void* v_pages, const fd_kv_pages* pages,
                                    const int32_t* cache_lens, float scale, int32_t num_splits,
                                    const fd_plan* plan, void* workspace, uint64_t workspace_bytes,
                                    void* out, float* lse, void* stream);

/* fd_decode_partials_paged -- fd_decode_partials over a paged cache: the
 * first pass alone, with the page arguments and rules of
 * fd_decode_attention_paged and the outputs of fd_decode_partials. */
fd_status fd_decode_partials_paged(const fd_dims* dims, const void* q, const void* k_pages,
                                   const void* v_pages, const fd_kv_pages* pages,
                                   const int32_t* cache_lens, float scale, int32_t num_splits,
                                   const fd_plan* plan, float* o_part, float* m_part, float* lse_part,
                                   void* stream);

/* FP8 K/V caches.
 *
 * Page "FlashDecoding算法原理与多GPU并行解码实战" (section on combining
 * methods) pairs the split-KV method with INT8/FP8 caches to save memory and
 * bandwidth, and advises dequantising to bf16 for the score computation.
 * Here k_cache and v_cache hold one-byte OCP FP8 E4M3 codes (the
 * "e4m3fn" format: bias 7, no infinities, 0x7F/0xFF are NaN, largest finite
 * 448) with one scale per tensor: the key is code * k_scale and the value is
 * code * v_scale.  q and out stay bf16 (dims->dtype must be FD_BF16).  Every
 * E4M3 value is exact in bf16, so the kernels dequantise each block to bf16
 * and run the bf16 products; k_scale is folded into the score scale and
 * v_scale into the output, so the arithmetic is that of the bf16 path.
 *
 * Layouts as for bf16 caches with one byte per element: contiguous
 * [B, Hkv, Lmax, D] when pages is NULL, else the paged layouts of
 * fd_kv_pages.  Every q_len is served (decode, verification chunks and long
 * prefill chunks).
 * Errors: as the bf16 calls; FD_ERR_UNSUPPORTED if dims->dtype is not
 * FD_BF16; FD_ERR_INVALID for non-finite scales. */
fd_status fd_decode_attention_fp8(const fd_dims* dims, const void* q, const void* k_cache,
                                  const void* v_cache, const fd_kv_pages* pages, float k_scale,
                                  float v_scale, const int32_t* cache_lens, float scale,
                                  int32_t num_splits, const fd_plan* plan, void* workspace,
                                  uint64_t workspace_bytes, void* out, float* lse, void* stream);

/* fd_decode_partials_fp8 -- the first pass alone over fp8 caches (outputs as
 * fd_decode_partials; o_part already carries v_scale). */
fd_status fd_decode_partials_fp8(const fd_dims* dims, const void* q, const void* k_cache,
                                 const void* v_cache, const fd_kv_pages* pages, float k_scale,
                                 float v_scale, const int32_t* cache_lens, float scale,
                                 int32_t num_splits, const fd_plan* plan, float* o_part,
                                 float* m_part, float* lse_part, void* stream);

/* INT8 K/V caches.
 *
 * The other cache format that the same section of page "FlashDecoding算法原理
 * 与多GPU并行解码实战" names (and page 3's memory section: INT8-quantised
 * cache data).  k_cache and v_cache hold one-byte two's-complement codes in
 * [-128, 127] with one scale per tensor, symmetric: the key is code * k_scale
 * and the value is code * v_scale.  Every such integer is exact in bf16, so
 * the arithmetic, layouts, arguments and errors are those of the FP8 calls
 * above (bf16 q and out, k_scale folded into the score scale, v_scale into
 * the output, every q_len served, contiguous or paged caches). */
fd_status fd_decode_attention_int8(const fd_dims* dims, const void* q, const void* k_cache,
                                   const void* v_cache, const fd_kv_pages* pages, float k_scale,
                                   float v_scale, const int32_t* cache_lens, float scale,
                                   int32_t num_splits, const fd_plan* plan, void* workspace,
                                   uint64_t workspace_bytes, void* out, float* lse, void* stream);

/* fd_decode_partials_int8 -- the first pass alone over int8 caches (outputs
 * as fd_decode_partials; o_part already carries v_scale). */
fd_status fd_decode_partials_int8(const fd_dims* dims, const void* q, const void* k_cache,
                                  const void* v_cache, const fd_kv_pages* pages, float k_scale,
                                  float v_scale, const int32_t* cache_lens, float scale,
                                  int32_t num_splits, const fd_plan* plan, float* o_part,
                                  float* m_part, float* lse_part, void* stream);

/* Diagnostics.  fd_status_string returns a static name for a status.
 * fd_last_error returns the message of the last failed call on this thread
 * ("" if none); the pointer stays valid until the next call on the thread. */
const char* fd_status_string(int32_t status);
const char* fd_last_error(void);

/* fd_stream_read -- a measurement aid, not part of the operation: reads
 * `bytes` bytes of device memory from `buf` once, in 16-byte pieces spread
 * over `workgroups` workgroups of 256 threads (0: eight per compute unit),
 * either strided over the whole grid (`pattern` 0: consecutive threads read
 * consecutive pieces) or one contiguous range per workgroup (`pattern` 1, as
 * the partial kernels read their tiles), and folds them into one word that
 * reaches `*sink` (device memory, 4 bytes) only if it equals a value no real
 * data is expected to give, so the reads cannot be optimised away.  Its time over the K/V bytes of a step gives the
 * bandwidth a plain streaming read reaches on the device, the ceiling against
 * which the partial kernel's rate is read (page "ChunkedPrefill与FlashDecoding
 * 技术解析" §4.2 item 2: find where the kernel's time goes before tuning it).
 * `buf` and `bytes` must be multiples of 16.  Errors: FD_ERR_INVALID for a
 * NULL or misaligned buffer, a size not a multiple of 16, workgroups < 0 or
 * a pattern other than 0 and 1. */
fd_status fd_stream_read(const void* buf, uint64_t bytes, int32_t workgroups, int32_t pattern, uint32_t* sink,
                         void* stream);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t fd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_H */
