// fd_select.cpp -- host-side choice of the partial-pass kernel and its row
// blocking, shared by the ABI layer (validation, planner, launch arguments)
// and the launch code.  No device code.
#include <cstdlib>
#include <cstring>

#include "fd_internal.h"

namespace fdk {

// The matrix-core kernels read bf16 caches (or one-byte FP8/INT8 codes) at
// head_dim 64 or 128.
bool mfma_partials_supported(int dtype, int head_dim, int rows) {
    return dtype == 1 && (head_dim == 64 || head_dim == 128) && rows >= 1;
}

// Decode kernel: the whole group of up to 32 rows; chunk kernel: tiles of
// kChunkTileRows packed rows.
int mfma_block_rows(int rows) { return rows <= 32 ? rows : kChunkTileRows; }

// Rows per workgroup of the vector kernel.
int vector_block_rows(int rows) {
    if (rows <= 1) return 1;
    if (rows <= 2) return 2;
    if (rows <= 4) return 4;
    return 8;
}

bool vector_kernel_forced() {
    static const bool forced = [] {
        const char* e = std::getenv("FD_DECODE_KERNEL");
        return e != nullptr && std::strcmp(e, "vector") == 0;
    }();
    return forced;
}

bool use_mfma_partials(int dtype, int head_dim, int rows) {
    return mfma_partials_supported(dtype, head_dim, rows) && !vector_kernel_forced();
}

int partial_block_rows(int dtype, int head_dim, int rows) {
    return use_mfma_partials(dtype, head_dim, rows) ? mfma_block_rows(rows) : vector_block_rows(rows);
}

}  // namespace fdk
