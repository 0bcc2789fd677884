// fd_internal.h -- launch interface between the C-ABI layer (fd_api.cpp) and
// the HIP kernels (fd_decode.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdk {

// How the keys [0, L_b) of sequence b are cut into tiles.
//   tile_len > 0 : tiles of tile_len keys;
//   tile_len == 0: num_splits tiles of ceil(L_b / num_splits) keys, rounded
//                  up to a multiple of `granule` (1 for contiguous caches;
//                  16 for paged ones, so a 16-key block never straddles a
//                  page).
// At most `slots` tiles; if more would be needed the last tile takes the rest.
struct SplitRule {
    int32_t tile_len;
    int32_t num_splits;
    int32_t slots;
    int32_t granule;
    int32_t spans;  // > 0: the decode kernel cuts the batch's key blocks into this many equal spans (slots >= 2)
};

// Where the K/V rows of a paged cache live.  Key j of sequence b, KV head g
// is row (j mod page_size) of page table[b * max_pages + j / page_size], at
// element offset page * page_stride + (j mod page_size) * row_stride +
// g * head_stride of k (and v).  page_size is a power of two >= 16.  A table
// entry outside [0, num_pages) is never dereferenced: its keys read as zero
// rows.
struct PagedKV {
    const int32_t* table;  // [B, max_pages] device; nullptr: contiguous caches
    int32_t max_pages;
    int32_t num_pages;
    int32_t page_shift;    // log2(page_size)
    int32_t row_stride;    // elements
    int64_t page_stride;   // elements
    int64_t head_stride;   // elements
};

// Element formats of the K/V caches: the query's dtype, or one-byte codes
// with per-tensor scales (value = code value * scale), dequantised to bf16
// inside the matrix-core kernels.
enum KvFormat : int32_t {
    kKvBf16 = 0,  // same dtype as q (bf16 or fp32)
    kKvE4M3 = 1,  // OCP FP8 E4M3 ("e4m3fn") codes
    kKvInt8 = 2,  // two's-complement INT8 codes
};

struct PartialArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* cache_lens;
    float* o_part;   // [rows_total, slots, D]      (partials mode)
    float* m_part;   // [rows_total, slots]
    float* lse_part; // [rows_total, slots]
    void* out;       // [rows_total, D]             (direct mode)
    float* lse;      // [rows_total] or nullptr
    int32_t batch, Hq, Hkv, q_len, Lmax, n_rep;
    int32_t rows;       // query rows per (sequence, KV head): n_rep * q_len
    int32_t row_blocks; // workgroups per (sequence, KV head, tile) along rows
    SplitRule rule;
    float qk_scale;     // scale * log2(e): scores are kept in base 2
    int32_t direct;     // 1: single slot, write out/lse instead of partials
    PagedKV pages;      // pages.table == nullptr: k/v are [B, Hkv, Lmax, D]
    int32_t kv_codes;   // kKvBf16, or the one-byte code format of k/v (bf16 q/out); k_scale is in qk_scale
    float v_scale;      // codes: value of V = code * v_scale (applied to the output)
};

// Packed query rows per workgroup of the matrix-core chunk kernel (row
// groups of more than 32 rows per KV head).
constexpr int kChunkTileRows = 128;

// Kernel selection (fd_select.cpp, host code only).
//
// Query rows one workgroup of the partial pass serves, for calls with `rows`
// = n_rep * q_len rows per (sequence, KV head).  The grid has
// ceil(rows / partial_block_rows) row blocks per (sequence, KV head, tile).
int partial_block_rows(int dtype, int head_dim, int rows);

// The partial pass: picks a matrix-core kernel (bf16) or the vector kernel
// (fp32) and launches it on `stream`.
hipError_t launch_partials(int dtype, int head_dim, int batch, const PartialArgs& a,
                           hipStream_t stream);

// Matrix-core partial kernels: their applicability and the rows of a
// workgroup (all of a group of up to 32 rows; else a chunk tile); the rows
// of a vector-kernel workgroup.
bool mfma_partials_supported(int dtype, int head_dim, int rows);
int mfma_block_rows(int rows);
int vector_block_rows(int rows);
// Whether the partial pass of a (dtype, head_dim, rows) call runs on the
// matrix cores: where supported, unless the environment variable
// FD_DECODE_KERNEL=vector forces the vector kernel (an ablation switch for
// bf16 caches; read once per process).
bool use_mfma_partials(int dtype, int head_dim, int rows);
bool vector_kernel_forced();

// Matrix-core launches: row groups of up to 32 rows (fd_mfma.hip), which
// hands larger ones to the chunk kernel (fd_chunk.hip).
hipError_t launch_partials_mfma(int head_dim, int batch, const PartialArgs& a, hipStream_t stream);
hipError_t launch_chunk_mfma(int head_dim, int batch, const PartialArgs& a, hipStream_t stream);

// Merge pass over rows [rows] of `slots` partial slots each.  With
// `splits_per_seq` (device [rows / rows_per_seq] int32), row r merges only
// the first splits_per_seq[r / rows_per_seq] slots (clamped to [0, slots]);
// nullptr: every row merges all `slots`.
hipError_t launch_combine(int head_dim, int out_dtype, int64_t rows, int slots,
                          const float* o_part, const float* lse_part, const int32_t* splits_per_seq,
                          int64_t rows_per_seq, void* out, float* lse, hipStream_t stream);

// The statically allocated workspace of fd_decode_attention_noalloc
// (fd_scratch.hip): kNoallocScratchBytes per device, held until the process
// ends.  noalloc_scratch returns the current device's copy, looking its
// address up on the first call on that device.
constexpr uint64_t kNoallocScratchBytes = 32ull << 20;
hipError_t noalloc_scratch(void** ptr);

// Streaming read of [buf, buf + bytes) (bytes a multiple of 16) over
// `workgroups` workgroups, strided over the grid (pattern 0) or one
// contiguous range per workgroup (1), folded into *sink only on an
// improbable value.
hipError_t launch_stream_read(const void* buf, uint64_t bytes, int workgroups, int pattern, uint32_t* sink,
                              hipStream_t stream);

}  // namespace fdk
