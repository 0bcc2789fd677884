// fd_api.cpp -- the C ABI declared in include/fd.h: argument validation, the
// split planner, workspace layout and kernel dispatch.  No device memory is
// allocated here and nothing is synchronised; kernels are enqueued on the
// caller's stream.
#include "fd.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fd_internal.h"

static_assert(fdk::kNoallocScratchBytes == FD_NOALLOC_SCRATCH_BYTES, "scratch size in fd.h and the library");

namespace {

thread_local char g_last_error[512] = "";

fd_status fail(fd_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_last_error[0] = '\0'; }

constexpr int64_t kAlign = 256;
constexpr float kLog2e = 1.44269504088896340736f;

// Planner constants.  The pages cut the cache into tiles of typically
// 256..1024 keys (page "ChunkedPrefill与FlashDecoding技术解析" §3.1) and find
// that fewer than about 256 keys per chunk loses to launch and merge overhead
// (page "FlashDecoding算法原理与多GPU并行解码实战", benchmark section); 256 is
// kept as the floor.  Above it, the tile length spreads the batch's key rows
// over a fixed number of work units per compute unit.  Measured on MI355X:
// with equal lengths one unit per CU is fastest (one long tile per CU
// streams at up to 88% of peak HBM bandwidth at 128k context, where
// 1024-key tiles reach 81%, and every extra split adds merge work); with
// unequal lengths (the variable-length section of the second page) units of
// unequal size leave CUs idle at the end, worst when the tile length is
// close to the even share of one or two units per CU.  Four units per CU
// keep every unit small against a CU's share: on a 32-sequence batch with
// lengths U[512, 8192] they take 9% less time than one unit per CU, within
// 5% of the best tile length found by a sweep.  Tiles are multiples of 64
// keys.
constexpr int kMinTile = 256;
constexpr int kTileGranule = 64;
constexpr int kUnitsPerCUEqual = 1;
constexpr int kUnitsPerCUMixed = 4;
// Mixed lengths on the matrix-core decode kernel (up to 32 rows per KV head):
// the plan asks for balanced spans (fdk::SplitRule::spans), sized for up to
// kSpanWGsPerCU workgroups per compute unit.  Every span workgroup scans the
// batch's lengths, so batches above kSpanMaxBatch keep tiles.
constexpr int kSpanWGsPerCU = 2;
constexpr int kSpanMaxBatch = 256;
constexpr int kSpanBlockKeys = 16;
constexpr int kSpanMax = 1 << 20;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

fd_status check_dims(const fd_dims* d) {
    if (!d) return fail(FD_ERR_INVALID, "dims is NULL");
    if (d->batch < 0) return fail(FD_ERR_INVALID, "batch %d < 0", d->batch);
    if (d->num_q_heads < 1 || d->num_kv_heads < 1)
        return fail(FD_ERR_INVALID, "head counts must be >= 1 (Hq=%d, Hkv=%d)", d->num_q_heads,
                    d->num_kv_heads);
    if (d->num_q_heads % d->num_kv_heads != 0)
        return fail(FD_ERR_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    d->num_q_heads, d->num_kv_heads);
    if (d->q_len < 1) return fail(FD_ERR_INVALID, "q_len %d < 1", d->q_len);
    if (d->max_cache_len < 0) return fail(FD_ERR_INVALID, "max_cache_len %d < 0", d->max_cache_len);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(FD_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
    if (d->dtype != FD_F32 && d->dtype != FD_BF16)
        return fail(FD_ERR_UNSUPPORTED, "dtype %d not supported (FD_F32 or FD_BF16)", d->dtype);
    if (d->batch > 65535) return fail(FD_ERR_UNSUPPORTED, "batch %d above 65535", d->batch);
    const int64_t rows = (int64_t)d->num_q_heads / d->num_kv_heads * d->q_len;
    if (rows > INT32_MAX) return fail(FD_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads x q_len too large");
    const int64_t blocks = ceil_div(rows, fdk::partial_block_rows(d->dtype, d->head_dim, (int)rows));
    if (blocks * d->num_kv_heads > 65535)
        return fail(FD_ERR_UNSUPPORTED, "num_kv_heads x row blocks (%lld) above 65535",
                    (long long)(blocks * d->num_kv_heads));
    const int64_t total_rows = (int64_t)d->batch * d->num_q_heads * d->q_len;
    if (total_rows > INT32_MAX) return fail(FD_ERR_UNSUPPORTED, "batch x heads x q_len too large");
    return FD_OK;
}

int64_t total_rows(const fd_dims* d) { return (int64_t)d->batch * d->num_q_heads * d->q_len; }

struct Layout {
    int64_t o_off, m_off, lse_off, bytes;
};

Layout workspace_layout(const fd_dims* d, int slots) {
    const int64_t rows = total_rows(d);
    Layout l;
    l.o_off = 0;
    l.m_off = align_up(rows * slots * d->head_dim * 4, kAlign);
    l.lse_off = l.m_off + align_up(rows * slots * 4, kAlign);
    l.bytes = l.lse_off + align_up(rows * slots * 4, kAlign);
    return l;
}

// Resolve the split rule of a call.  Returns FD_OK and fills *rule.
fd_status resolve_rule(int32_t num_splits, const fd_plan* plan, fdk::SplitRule* rule) {
    if (num_splits < 0 || num_splits > FD_MAX_SPLITS)
        return fail(FD_ERR_INVALID, "num_splits %d outside [0, %d]", num_splits, FD_MAX_SPLITS);
    if (num_splits > 0) {
        *rule = {0, num_splits, num_splits, 1};
        return FD_OK;
    }
    if (!plan) {
        *rule = {0, 1, 1, 1};  // one tile holding every key
        return FD_OK;
    }
    if (plan->max_splits < 1 || plan->max_splits > FD_MAX_SPLITS)
        return fail(FD_ERR_INVALID, "plan max_splits %d outside [1, %d]", plan->max_splits, FD_MAX_SPLITS);
    if (plan->tile_len < 1)
        return fail(FD_ERR_INVALID, "plan tile_len %d < 1 (a forced-count plan needs num_splits)",
                    plan->tile_len);
    if (plan->spans < 0 || plan->spans > kSpanMax)
        return fail(FD_ERR_INVALID, "plan spans %d outside [0, %d]", plan->spans, kSpanMax);
    *rule = {plan->tile_len, 1, plan->max_splits, 1, plan->max_splits >= 2 ? plan->spans : 0};
    return FD_OK;
}

// Bytes of one stored key row of one KV head: bf16 or fp32 elements, or
// one-byte codes.
int64_t row_bytes(const fd_dims* d, bool codes) {
    return (int64_t)d->head_dim * (codes ? 1 : (d->dtype == FD_BF16 ? 2 : 4));
}

// The most keys one tile of `rule` can hold for a sequence of at most Lmax
// keys (the tile rule of fdk::tile_of: the last tile takes the rest when the
// count reaches the slots).  Under balanced spans a piece is bounded only by
// its (sequence, KV head) pair, since few resident workgroups make long
// spans: all Lmax keys.
int64_t max_tile_keys(const fdk::SplitRule& r, int64_t Lmax) {
    if (Lmax <= 0) return 0;
    if (r.spans > 0) return Lmax;
    if (r.tile_len > 0) {
        const int64_t T = r.tile_len;
        const int64_t S = std::min<int64_t>(ceil_div(Lmax, T), r.slots);
        return std::max(std::min(T, Lmax), Lmax - (S - 1) * T);
    }
    const int64_t T = align_up(ceil_div(Lmax, r.num_splits), r.granule);
    return std::min(T, Lmax);
}

// The kernels address a tile's rows with 32-bit byte offsets and buffer
// ranges; reject a rule under which one tile of one KV head reaches 2^31
// bytes.
fd_status check_tile_bytes(const fd_dims* d, const fdk::SplitRule& r, bool codes) {
    const int64_t keys = max_tile_keys(r, d->max_cache_len);
    const int64_t bytes = keys * row_bytes(d, codes);
    if (bytes >= ((int64_t)1 << 31))
        return fail(FD_ERR_UNSUPPORTED,
                    "a tile of up to %lld keys spans %lld bytes of one KV head; tiles must stay below 2^31 bytes "
                    "(use more splits)",
                    (long long)keys, (long long)bytes);
    return FD_OK;
}

fd_status check_tensors(const fd_dims* d, const void* q, const void* k, const void* v,
                        const int32_t* lens) {
    if (!q || !k || !v || !lens) return fail(FD_ERR_INVALID, "q, k_cache, v_cache and cache_lens must be non-NULL");
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16))
        return fail(FD_ERR_INVALID, "q, k_cache and v_cache must be 16-byte aligned");
    if (misaligned(lens, 4)) return fail(FD_ERR_INVALID, "cache_lens must be 4-byte aligned");
    (void)d;
    return FD_OK;
}

fdk::PartialArgs make_args(const fd_dims* d, const void* q, const void* k, const void* v,
                           const int32_t* lens, float scale, const fdk::SplitRule& rule) {
    fdk::PartialArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cache_lens = lens;
    a.batch = d->batch;
    a.Hq = d->num_q_heads;
    a.Hkv = d->num_kv_heads;
    a.q_len = d->q_len;
    a.Lmax = d->max_cache_len;
    a.n_rep = d->num_q_heads / d->num_kv_heads;
    a.rows = a.n_rep * d->q_len;
    a.row_blocks = (int32_t)ceil_div(a.rows, fdk::partial_block_rows(d->dtype, d->head_dim, a.rows));
    a.rule = rule;
    a.qk_scale = scale * kLog2e;
    return a;
}

// FD_TRACE=1 in the environment prints each launch's plan and grid on
// stderr (read once per process).
bool trace_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("FD_TRACE");
        return e != nullptr && e[0] != '\0' && e[0] != '0';
    }();
    return on;
}

void trace_launch(const char* entry, const fd_dims* d, const fdk::PartialArgs& a) {
    if (!trace_enabled()) return;
    const bool mfma = a.kv_codes != fdk::kKvBf16 || fdk::use_mfma_partials(d->dtype, d->head_dim, a.rows);
    const char* kernel = !mfma ? "fd_partial_kernel (vector)"
                         : a.rows > 32 ? "fd_mfma_chunk_kernel" : "fd_mfma_partial_kernel";
    std::fprintf(stderr,
                 "[fd] %s: B=%d Hq=%d Hkv=%d D=%d q_len=%d Lmax=%d dtype=%d%s%s | tile_len=%d num_splits=%d "
                 "slots=%d granule=%d spans=%d | rows/KV head=%d row_blocks=%d | %s, %s\n",
                 entry, d->batch, d->num_q_heads, d->num_kv_heads, d->head_dim, d->q_len, d->max_cache_len,
                 d->dtype, a.pages.table ? " paged" : "",
                 a.kv_codes == fdk::kKvE4M3 ? " fp8-kv" : a.kv_codes == fdk::kKvInt8 ? " int8-kv" : "",
                 a.rule.tile_len,
                 a.rule.num_splits, a.rule.slots, a.rule.granule, a.rule.spans, a.rows, a.row_blocks, kernel,
                 a.rule.slots > 1 && !a.direct ? "partials + merge" : "direct output");
}

fd_status device_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FD_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return FD_OK;
}

}  // namespace

extern "C" {

const char* fd_status_string(int32_t status) {
    switch (status) {
        case FD_OK: return "FD_OK";
        case FD_ERR_INVALID: return "FD_ERR_INVALID";
        case FD_ERR_UNSUPPORTED: return "FD_ERR_UNSUPPORTED";
        case FD_ERR_WORKSPACE: return "FD_ERR_WORKSPACE";
        case FD_ERR_DEVICE: return "FD_ERR_DEVICE";
        default: return "FD_STATUS_UNKNOWN";
    }
}

const char* fd_last_error(void) { return g_last_error; }

int32_t fd_version(void) { return 500; }

uint64_t fd_workspace_bytes(const fd_dims* dims, int32_t max_splits) {
    if (max_splits <= 1 || max_splits > FD_MAX_SPLITS) return 0;
    char saved[sizeof g_last_error];
    std::memcpy(saved, g_last_error, sizeof saved);
    const bool ok = check_dims(dims) == FD_OK;
    std::memcpy(g_last_error, saved, sizeof saved);
    if (!ok) return 0;
    return (uint64_t)workspace_layout(dims, max_splits).bytes;
}

fd_status fd_plan_splits(const fd_dims* dims, const int32_t* cache_lens_host, int32_t num_splits,
                         int32_t num_cus, fd_plan* plan, int32_t* splits_per_seq) {
    clear_error();
    fd_status st = check_dims(dims);
    if (st != FD_OK) return st;
    if (!plan) return fail(FD_ERR_INVALID, "plan is NULL");
    if (dims->batch > 0 && !cache_lens_host) return fail(FD_ERR_INVALID, "cache_lens_host is NULL");
    if (num_splits < 0 || num_splits > FD_MAX_SPLITS)
        return fail(FD_ERR_INVALID, "num_splits %d outside [0, %d]", num_splits, FD_MAX_SPLITS);
    if (num_cus < 0) return fail(FD_ERR_INVALID, "num_cus %d < 0", num_cus);
    int64_t sum_len = 0;
    int32_t max_len = 0, min_len = INT32_MAX;
    for (int b = 0; b < dims->batch; ++b) {
        const int32_t L = cache_lens_host[b];
        if (L < 0 || L > dims->max_cache_len)
            return fail(FD_ERR_INVALID, "cache_lens[%d] = %d outside [0, %d]", b, L, dims->max_cache_len);
        sum_len += L;
        max_len = std::max(max_len, L);
        min_len = std::min(min_len, L);
    }
    const int rows = dims->num_q_heads / dims->num_kv_heads * dims->q_len;
    const int64_t row_blocks = ceil_div(rows, fdk::partial_block_rows(dims->dtype, dims->head_dim, rows));
    const int64_t lanes = (int64_t)dims->num_kv_heads * row_blocks;  // units per tile position

    fd_plan p{};
    if (num_splits > 0) {
        p.tile_len = 0;
        p.max_splits = num_splits;
        int64_t units = 0;
        for (int b = 0; b < dims->batch; ++b) {
            const int32_t L = cache_lens_host[b];
            const int64_t T = std::max<int64_t>(1, ceil_div(L, num_splits));
            const int64_t S = ceil_div(L, T);
            units += S * lanes;
            if (splits_per_seq) splits_per_seq[b] = (int32_t)S;
        }
        p.work_units = (int32_t)std::min<int64_t>(units, INT32_MAX);
    } else {
        if (num_cus == 0) {
            int dev = 0;
            hipDeviceProp_t prop;
            if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
                return fail(FD_ERR_DEVICE, "cannot query the compute-unit count; pass num_cus");
            num_cus = prop.multiProcessorCount;
        }
        // Spread the batch's key rows over a few units per CU.
        const int64_t key_rows = sum_len * lanes;
        const int units_per_cu = min_len == max_len ? kUnitsPerCUEqual : kUnitsPerCUMixed;
        int64_t T = ceil_div(std::max<int64_t>(key_rows, 1), (int64_t)num_cus * units_per_cu);
        T = align_up(T, kTileGranule);
        T = std::max<int64_t>(T, kMinTile);
        T = std::min<int64_t>(T, align_up(std::max<int64_t>(max_len, 1), kTileGranule));
        if (ceil_div(max_len, T) > FD_MAX_SPLITS) T = align_up(ceil_div(max_len, FD_MAX_SPLITS), kTileGranule);
        int64_t smax = 1, units = 0;
        for (int b = 0; b < dims->batch; ++b) {
            const int64_t S = ceil_div(cache_lens_host[b], T);
            smax = std::max(smax, S);
            units += S * lanes;
            if (splits_per_seq) splits_per_seq[b] = (int32_t)S;
        }
        p.tile_len = (int32_t)T;
        p.max_splits = (int32_t)smax;
        p.work_units = (int32_t)std::min<int64_t>(units, INT32_MAX);
        // Spans only where a whole pair of bf16 rows stays below 2^31 bytes
        // (the bound the launch checks a span rule against).
        const bool span_bytes_ok = (int64_t)dims->max_cache_len * dims->head_dim * 2 < ((int64_t)1 << 31);
        if (min_len != max_len && rows <= 32 && fdk::use_mfma_partials(dims->dtype, dims->head_dim, rows) &&
            dims->batch <= kSpanMaxBatch && units > (int64_t)num_cus * kSpanWGsPerCU && span_bytes_ok) {
            // More tiles than one round of workgroups: equal spans instead,
            // two per CU, none shorter than kMinTile keys, and enough slots
            // that a pair of the longest sequence spans ceil(blocks / span) + 1
            // of them.
            int64_t blocks = 0;
            for (int b = 0; b < dims->batch; ++b) blocks += ceil_div(cache_lens_host[b], kSpanBlockKeys);
            const int64_t nspans = std::min<int64_t>(
                {(int64_t)num_cus * kSpanWGsPerCU, ceil_div(blocks * dims->num_kv_heads, kMinTile / kSpanBlockKeys),
                 (int64_t)kSpanMax});
            const int64_t span = std::max<int64_t>(1, ceil_div(blocks * dims->num_kv_heads, nspans));
            const int64_t need = ceil_div(ceil_div(max_len, kSpanBlockKeys), span) + 1;
            p.max_splits = (int32_t)std::min<int64_t>(FD_MAX_SPLITS, std::max<int64_t>(smax, need));
            p.spans = p.max_splits >= 2 ? (int32_t)nspans : 0;
        }
    }
    p.workspace_bytes = p.max_splits > 1 ? (uint64_t)workspace_layout(dims, p.max_splits).bytes : 0;
    *plan = p;
    return FD_OK;
}

}  // extern "C"

namespace {

fd_status resolve_pages(const fd_dims* d, const fd_kv_pages* pages, fdk::SplitRule* rule, fdk::PagedKV* pk);

// Format and per-tensor dequantisation scales of a call with caches of
// one-byte codes (FP8 E4M3 or INT8).
struct CodeScales {
    int32_t format;  // fdk::kKvE4M3 or fdk::kKvInt8
    float k_scale, v_scale;
};

// Checks of a call over one-byte codes: bf16 queries, finite scales.
fd_status check_codes(const fd_dims* d, const CodeScales* cs) {
    const char* name = cs->format == fdk::kKvInt8 ? "int8" : "fp8";
    if (d->dtype != FD_BF16) return fail(FD_ERR_UNSUPPORTED, "%s caches need bf16 q and out (dims->dtype)", name);
    if (!std::isfinite(cs->k_scale) || !std::isfinite(cs->v_scale))
        return fail(FD_ERR_INVALID, "k_scale and v_scale must be finite");
    return FD_OK;
}

void apply_codes(fdk::PartialArgs* a, const CodeScales* cs, float scale) {
    a->v_scale = 1.f;
    a->kv_codes = fdk::kKvBf16;
    if (!cs) return;
    a->kv_codes = cs->format;
    a->v_scale = cs->v_scale;
    a->qk_scale = (float)((double)scale * cs->k_scale * kLog2e);
}

fd_status run_partials(const fd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                       const fd_kv_pages* pages, const CodeScales* cs, const int32_t* cache_lens, float scale,
                       int32_t num_splits, const fd_plan* plan, float* o_part, float* m_part, float* lse_part,
                       void* stream) {
    clear_error();
    fd_status st = check_dims(dims);
    if (st != FD_OK) return st;
    if (cs && (st = check_codes(dims, cs)) != FD_OK) return st;
    if (num_splits == 0 && !plan)
        return fail(FD_ERR_INVALID, "the partial pass needs num_splits > 0 or a plan");
    fdk::SplitRule rule;
    if ((st = resolve_rule(num_splits, plan, &rule)) != FD_OK) return st;
    fdk::PagedKV pk{};
    if (pages && (st = resolve_pages(dims, pages, &rule, &pk)) != FD_OK) return st;
    if ((st = check_tile_bytes(dims, rule, cs != nullptr)) != FD_OK) return st;
    if (dims->batch == 0) return FD_OK;
    if ((st = check_tensors(dims, q, k_cache, v_cache, cache_lens)) != FD_OK) return st;
    if (!o_part || !m_part || !lse_part)
        return fail(FD_ERR_INVALID, "o_part, m_part and lse_part must be non-NULL");
    if (misaligned(o_part, 16) || misaligned(m_part, 4) || misaligned(lse_part, 4))
        return fail(FD_ERR_INVALID, "o_part must be 16-byte aligned, m_part and lse_part 4-byte aligned");
    fdk::PartialArgs a = make_args(dims, q, k_cache, v_cache, cache_lens, scale, rule);
    a.pages = pk;
    apply_codes(&a, cs, scale);
    a.o_part = o_part;
    a.m_part = m_part;
    a.lse_part = lse_part;
    a.direct = 0;
    trace_launch("partials", dims, a);
    return device_status(fdk::launch_partials(dims->dtype, dims->head_dim, dims->batch, a,
                                              static_cast<hipStream_t>(stream)),
                         "partial kernel launch");
}

}  // namespace

extern "C" {

fd_status fd_decode_partials(const fd_dims* dims, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* cache_lens, float scale,
                             int32_t num_splits, const fd_plan* plan, float* o_part,
                             float* m_part, float* lse_part, void* stream) {
    return run_partials(dims, q, k_cache, v_cache, nullptr, nullptr, cache_lens, scale, num_splits, plan, o_part,
                        m_part, lse_part, stream);
}

fd_status fd_decode_partials_paged(const fd_dims* dims, const void* q, const void* k_pages,
                                   const void* v_pages, const fd_kv_pages* pages,
                                   const int32_t* cache_lens, float scale, int32_t num_splits,
                                   const fd_plan* plan, float* o_part, float* m_part, float* lse_part,
                                   void* stream) {
    if (!pages) {
        clear_error();
        return fail(FD_ERR_INVALID, "pages is NULL");
    }
    return run_partials(dims, q, k_pages, v_pages, pages, nullptr, cache_lens, scale, num_splits, plan, o_part,
                        m_part, lse_part, stream);
}

fd_status fd_decode_partials_fp8(const fd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                                 const fd_kv_pages* pages, float k_scale, float v_scale,
                                 const int32_t* cache_lens, float scale, int32_t num_splits, const fd_plan* plan,
                                 float* o_part, float* m_part, float* lse_part, void* stream) {
    const CodeScales cs{fdk::kKvE4M3, k_scale, v_scale};
    return run_partials(dims, q, k_cache, v_cache, pages, &cs, cache_lens, scale, num_splits, plan, o_part, m_part,
                        lse_part, stream);
}

fd_status fd_decode_partials_int8(const fd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                                  const fd_kv_pages* pages, float k_scale, float v_scale,
                                  const int32_t* cache_lens, float scale, int32_t num_splits, const fd_plan* plan,
                                  float* o_part, float* m_part, float* lse_part, void* stream) {
    const CodeScales cs{fdk::kKvInt8, k_scale, v_scale};
    return run_partials(dims, q, k_cache, v_cache, pages, &cs, cache_lens, scale, num_splits, plan, o_part, m_part,
                        lse_part, stream);
}

fd_status fd_combine_splits(int32_t batch, int32_t num_heads, int32_t q_len, int32_t head_dim,
                            int32_t max_splits, const float* o_part, const float* lse_part,
                            const int32_t* splits_per_seq, int32_t out_dtype, void* out, float* lse,
                            void* stream) {
    clear_error();
    if (batch < 0 || num_heads < 1 || q_len < 1)
        return fail(FD_ERR_INVALID, "bad sizes (batch=%d, num_heads=%d, q_len=%d)", batch, num_heads, q_len);
    if (max_splits < 1 || max_splits > FD_MAX_SPLITS)
        return fail(FD_ERR_INVALID, "max_splits %d outside [1, %d]", max_splits, FD_MAX_SPLITS);
    if (head_dim != 64 && head_dim != 128)
        return fail(FD_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
    if (out_dtype != FD_F32 && out_dtype != FD_BF16)
        return fail(FD_ERR_UNSUPPORTED, "out_dtype %d not supported", out_dtype);
    const int64_t rows = (int64_t)batch * num_heads * q_len;
    if (rows > INT32_MAX) return fail(FD_ERR_UNSUPPORTED, "too many rows");
    if (rows == 0) return FD_OK;
    if (!o_part || !lse_part || !out) return fail(FD_ERR_INVALID, "o_part, lse_part and out must be non-NULL");
    if (misaligned(o_part, 16) || misaligned(out, out_dtype == FD_BF16 ? 8 : 16) || misaligned(lse_part, 4) ||
        (lse && misaligned(lse, 4)) || (splits_per_seq && misaligned(splits_per_seq, 4)))
        return fail(FD_ERR_INVALID,
                    "misaligned buffer (o_part and out need 16 bytes, bf16 out 8, lse and splits_per_seq 4)");
    return device_status(fdk::launch_combine(head_dim, out_dtype, rows, max_splits, o_part, lse_part,
                                             splits_per_seq, (int64_t)num_heads * q_len, out, lse,
                                             static_cast<hipStream_t>(stream)),
                         "combine kernel launch");
}

fd_status fd_stream_read(const void* buf, uint64_t bytes, int32_t workgroups, int32_t pattern, uint32_t* sink,
                         void* stream) {
    clear_error();
    if (workgroups < 0) return fail(FD_ERR_INVALID, "workgroups %d < 0", workgroups);
    if (pattern != 0 && pattern != 1) return fail(FD_ERR_INVALID, "pattern %d is neither 0 nor 1", pattern);
    if (bytes % 16 != 0) return fail(FD_ERR_INVALID, "bytes %llu is not a multiple of 16", (unsigned long long)bytes);
    if (bytes == 0) return FD_OK;
    if (!buf || !sink) return fail(FD_ERR_INVALID, "buf and sink must be non-NULL");
    if (misaligned(buf, 16) || misaligned(sink, 4))
        return fail(FD_ERR_INVALID, "buf must be 16-byte aligned and sink 4-byte aligned");
    if (workgroups == 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(FD_ERR_DEVICE, "cannot query the compute-unit count; pass workgroups");
        workgroups = 8 * prop.multiProcessorCount;
    }
    return device_status(fdk::launch_stream_read(buf, bytes, workgroups, pattern, sink,
                                                 static_cast<hipStream_t>(stream)),
                         "stream read kernel launch");
}

}  // extern "C"

namespace {

// Check a paged-cache description against dims; on success fill *pk and
// make *rule cut tiles at multiples of 16 keys.
fd_status resolve_pages(const fd_dims* d, const fd_kv_pages* pages, fdk::SplitRule* rule, fdk::PagedKV* pk) {
    if (!pages) return fail(FD_ERR_INVALID, "pages is NULL");
    if (!pages->block_table) return fail(FD_ERR_INVALID, "block_table is NULL");
    if (misaligned(pages->block_table, 4)) return fail(FD_ERR_INVALID, "block_table must be 4-byte aligned");
    if (pages->max_pages_per_seq < 1 || pages->num_pages < 1)
        return fail(FD_ERR_INVALID, "max_pages_per_seq %d and num_pages %d must be >= 1", pages->max_pages_per_seq,
                    pages->num_pages);
    const int32_t P = pages->page_size;
    if (P < 16 || (P & (P - 1)) != 0)
        return fail(FD_ERR_UNSUPPORTED, "page_size %d is not a power of two >= 16", P);
    if (pages->layout != FD_PAGES_NHD && pages->layout != FD_PAGES_HND)
        return fail(FD_ERR_UNSUPPORTED, "page layout %d unknown", pages->layout);
    if ((int64_t)pages->max_pages_per_seq * P != d->max_cache_len)
        return fail(FD_ERR_INVALID, "max_cache_len %d != max_pages_per_seq %d x page_size %d", d->max_cache_len,
                    pages->max_pages_per_seq, P);
    if (rule->tile_len > 0 && rule->tile_len % 16 != 0)
        return fail(FD_ERR_INVALID, "plan tile_len %d is not a multiple of 16 (paged caches)", rule->tile_len);
    const int64_t D = d->head_dim, H = d->num_kv_heads;
    const int64_t page_elems = (int64_t)P * H * D;
    if ((int64_t)pages->num_pages * page_elems > ((int64_t)1 << 46))
        return fail(FD_ERR_UNSUPPORTED, "page pool too large");
    rule->granule = 16;
    pk->table = pages->block_table;
    pk->max_pages = pages->max_pages_per_seq;
    pk->num_pages = pages->num_pages;
    int shift = 0;
    while ((1 << shift) < P) ++shift;
    pk->page_shift = shift;
    pk->page_stride = page_elems;
    if (pages->layout == FD_PAGES_NHD) {
        pk->row_stride = (int32_t)(H * D);
        pk->head_stride = D;
    } else {
        pk->row_stride = (int32_t)D;
        pk->head_stride = (int64_t)P * D;
    }
    return FD_OK;
}

// The two passes of the operation over contiguous (pk == nullptr) or paged
// caches.
// With noalloc, the workspace is the library's static scratch of the
// current device (workspace and workspace_bytes are ignored): calls needing
// more than it holds fail with FD_ERR_WORKSPACE.
fd_status run_attention(const fd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                        const fd_kv_pages* pages, const CodeScales* cs, const int32_t* cache_lens, float scale,
                        int32_t num_splits, const fd_plan* plan, void* workspace, uint64_t workspace_bytes,
                        void* out, float* lse, void* stream, bool noalloc = false) {
    clear_error();
    fd_status st = check_dims(dims);
    if (st != FD_OK) return st;
    if (cs && (st = check_codes(dims, cs)) != FD_OK) return st;
    fdk::SplitRule rule;
    if ((st = resolve_rule(num_splits, plan, &rule)) != FD_OK) return st;
    fdk::PagedKV pk{};
    if (pages && (st = resolve_pages(dims, pages, &rule, &pk)) != FD_OK) return st;
    if ((st = check_tile_bytes(dims, rule, cs != nullptr)) != FD_OK) return st;
    if (dims->batch == 0) return FD_OK;
    if ((st = check_tensors(dims, q, k_cache, v_cache, cache_lens)) != FD_OK) return st;
    if (!out) return fail(FD_ERR_INVALID, "out is NULL");
    if (misaligned(out, 16)) return fail(FD_ERR_INVALID, "out must be 16-byte aligned");
    if (lse && misaligned(lse, 4)) return fail(FD_ERR_INVALID, "lse must be 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    fdk::PartialArgs a = make_args(dims, q, k_cache, v_cache, cache_lens, scale, rule);
    a.pages = pk;
    apply_codes(&a, cs, scale);
    if (rule.slots == 1) {
        a.out = out;
        a.lse = lse;
        a.direct = 1;
        trace_launch("attention", dims, a);
        return device_status(fdk::launch_partials(dims->dtype, dims->head_dim, dims->batch, a, s),
                             "partial kernel launch");
    }
    const Layout lay = workspace_layout(dims, rule.slots);
    if (noalloc) {
        if ((uint64_t)lay.bytes > fdk::kNoallocScratchBytes)
            return fail(FD_ERR_WORKSPACE,
                        "this call needs %llu bytes of workspace; the static scratch of the no-allocation entry "
                        "point holds %llu (use fd_decode_attention with a workspace, or fewer splits)",
                        (unsigned long long)lay.bytes, (unsigned long long)fdk::kNoallocScratchBytes);
        if ((st = device_status(fdk::noalloc_scratch(&workspace), "static scratch lookup")) != FD_OK) return st;
        workspace_bytes = fdk::kNoallocScratchBytes;
    }
    if (!workspace || workspace_bytes < (uint64_t)lay.bytes)
        return fail(FD_ERR_WORKSPACE, "workspace of %llu bytes needed, %llu given%s",
                    (unsigned long long)lay.bytes, (unsigned long long)workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (misaligned(workspace, kAlign)) return fail(FD_ERR_INVALID, "workspace must be 256-byte aligned");
    char* ws = static_cast<char*>(workspace);
    a.o_part = reinterpret_cast<float*>(ws + lay.o_off);
    a.m_part = reinterpret_cast<float*>(ws + lay.m_off);
    a.lse_part = reinterpret_cast<float*>(ws + lay.lse_off);
    a.direct = 0;
    trace_launch("attention", dims, a);
    if ((st = device_status(fdk::launch_partials(dims->dtype, dims->head_dim, dims->batch, a, s),
                            "partial kernel launch")) != FD_OK)
        return st;
    return device_status(fdk::launch_combine(dims->head_dim, dims->dtype, total_rows(dims), rule.slots,
                                             a.o_part, a.lse_part, nullptr, 0, out, lse, s),
                         "combine kernel launch");
}

}  // namespace

extern "C" {

fd_status fd_decode_attention(const fd_dims* dims, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* cache_lens, float scale,
                              int32_t num_splits, const fd_plan* plan, void* workspace,
                              uint64_t workspace_bytes, void* out, float* lse, void* stream) {
    return run_attention(dims, q, k_cache, v_cache, nullptr, nullptr, cache_lens, scale, num_splits, plan,
                         workspace, workspace_bytes, out, lse, stream);
}

fd_status fd_decode_attention_noalloc(const fd_dims* dims, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* cache_lens, float scale,
                                      int32_t num_splits, const fd_plan* plan, void* out, float* lse,
                                      void* stream) {
    return run_attention(dims, q, k_cache, v_cache, nullptr, nullptr, cache_lens, scale, num_splits, plan, nullptr,
                         0, out, lse, stream, true);
}

fd_status fd_decode_attention_paged(const fd_dims* dims, const void* q, const void* k_pages,
                                    const void* v_pages, const fd_kv_pages* pages,
                                    const int32_t* cache_lens, float scale, int32_t num_splits,
                                    const fd_plan* plan, void* workspace, uint64_t workspace_bytes,
                                    void* out, float* lse, void* stream) {
    if (!pages) {
        clear_error();
        return fail(FD_ERR_INVALID, "pages is NULL");
    }
    return run_attention(dims, q, k_pages, v_pages, pages, nullptr, cache_lens, scale, num_splits, plan,
                         workspace, workspace_bytes, out, lse, stream);
}

fd_status fd_decode_attention_fp8(const fd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                                  const fd_kv_pages* pages, float k_scale, float v_scale,
                                  const int32_t* cache_lens, float scale, int32_t num_splits, const fd_plan* plan,
                                  void* workspace, uint64_t workspace_bytes, void* out, float* lse, void* stream) {
    const CodeScales cs{fdk::kKvE4M3, k_scale, v_scale};
    return run_attention(dims, q, k_cache, v_cache, pages, &cs, cache_lens, scale, num_splits, plan, workspace,
                         workspace_bytes, out, lse, stream);
}

fd_status fd_decode_attention_int8(const fd_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                                   const fd_kv_pages* pages, float k_scale, float v_scale,
                                   const int32_t* cache_lens, float scale, int32_t num_splits, const fd_plan* plan,
                                   void* workspace, uint64_t workspace_bytes, void* out, float* lse, void* stream) {
    const CodeScales cs{fdk::kKvInt8, k_scale, v_scale};
    return run_attention(dims, q, k_cache, v_cache, pages, &cs, cache_lens, scale, num_splits, plan, workspace,
                         workspace_bytes, out, lse, stream);
}

}  // extern "C"
