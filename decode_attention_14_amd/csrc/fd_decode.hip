// fd_decode.hip -- split-KV decode attention kernels for gfx950 (CDNA4).
//
// Two kernels implement the two passes of the split-KV method (page
// "ChunkedPrefill与FlashDecoding技术解析" §3.1; page "FlashDecoding算法原理与
// 多GPU并行解码实战", algorithm section and multi-GPU step 3):
//
//   fd_partial_kernel  one workgroup per (tile s, KV head g, row block,
//                      sequence b).  It streams the tile's K and V rows from
//                      HBM once, with 16-byte loads, and uses each loaded row
//                      for every query row of the GQA group (engineering
//                      details item 3 of the second page: group by KV head so
//                      K/V are read once).  Scores, softmax and the P.V
//                      accumulation are fp32 on the vector ALUs; the dot
//                      product over D is spread over the lanes that loaded
//                      the key row and finished with DPP row reductions.
//                      Output: per-tile (o_s, m_s, lse_s), or out/lse
//                      directly when there is a single tile.
//   fd_combine_kernel  one wave per query row (four per row when a row has
//                      many tiles; fd_combine_narrow_kernel, one thread per
//                      float4 column of four rows, when it has at most four).
//                      It merges the row's tiles:
//                      LSE = ln sum_s exp(lse_s), out = sum_s
//                      exp(lse_s - LSE) o_s.
//
// Decode is matrix-vector work (about 4 flop per byte of K/V at a GQA ratio
// of 4), so it is bound by HBM bandwidth, not by the matrix cores; the
// partial kernel is built to keep many 16-byte loads in flight per CU and to
// keep the ALU work per byte small.
//
// Lane layout of the partial kernel (bf16, D = 128): a key row is 256 bytes,
// i.e. 16 lanes x 16 bytes; one wave load instruction covers 4 consecutive
// key rows (1 KiB contiguous).  Each lane keeps, for every query row, an
// online-softmax state (running max m, running sum l, and the 8 output
// columns it owns); lanes of the same 16-lane group see the same keys, so m
// and l are uniform within a group.  At the end the group states of a wave
// are merged with cross-lane shuffles and the 4 wave states through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_device.h"
#include "fd_internal.h"

namespace fdk {
namespace {

// Tuning constants of the partial kernel: 16-byte load instructions per
// tensor per step for row blocks of up to 4 rows and of 8 rows, and an
// optional occupancy target (waves per SIMD; 0 lets the compiler choose).
#ifndef FD_STEP_LOADS_R4
#define FD_STEP_LOADS_R4 4
#endif
#ifndef FD_STEP_LOADS_R8
#define FD_STEP_LOADS_R8 2
#endif
#ifndef FD_WAVES_PER_SIMD
#define FD_WAVES_PER_SIMD 0
#endif
// Cache-policy bits of the K/V buffer loads (2: non-temporal, the data is
// read once and should not displace anything).
#ifndef FD_LOAD_AUX
#define FD_LOAD_AUX 2
#endif
#if FD_WAVES_PER_SIMD > 0
#define FD_OCCUPANCY __attribute__((amdgpu_waves_per_eu(FD_WAVES_PER_SIMD)))
#else
#define FD_OCCUPANCY
#endif

#ifndef FD_PARTIAL_THREADS
#define FD_PARTIAL_THREADS 256
#endif

constexpr int kPThreads = FD_PARTIAL_THREADS;     // partial kernel
constexpr int kPWaves = kPThreads / 64;

// One 16-byte slice of a row: E elements.
template <bool BF16> struct Slice;
template <> struct Slice<true> {
    static constexpr int E = 8;
    uint32_t w[4];
};
template <> struct Slice<false> {
    static constexpr int E = 4;
    float w[4];
};

template <bool BF16>
__device__ __forceinline__ void load_slice(Slice<BF16>& s, const void* p) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    if constexpr (BF16) {
        s.w[0] = x.x; s.w[1] = x.y; s.w[2] = x.z; s.w[3] = x.w;
    } else {
        s.w[0] = __uint_as_float(x.x); s.w[1] = __uint_as_float(x.y);
        s.w[2] = __uint_as_float(x.z); s.w[3] = __uint_as_float(x.w);
    }
}

template <bool BF16>
__device__ __forceinline__ void to_float(const Slice<BF16>& s, float (&f)[Slice<BF16>::E]) {
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_lo(s.w[i]);
            f[2 * i + 1] = bf16_hi(s.w[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = s.w[i];
    }
}

// Partial dot product of this lane's slices.  bf16: the raw q bits with the
// bf16 dot2 instruction (products of bf16 values are exact in fp32), the
// score scale applied afterwards.  fp32: q was pre-scaled at load time.
template <bool BF16>
__device__ __forceinline__ float slice_dot(const Slice<BF16>& q, const Slice<BF16>& k) {
    if constexpr (BF16) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w[i]),
                                                  __builtin_bit_cast(bf16x2_t, k.w[i]), acc, false);
        return acc;
    } else {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(q.w[i], k.w[i], acc);
        return acc;
    }
}

template <bool BF16>
__device__ __forceinline__ void buffer_slice(Slice<BF16>& s, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, FD_LOAD_AUX);
    if constexpr (BF16) {
        s.w[0] = x[0]; s.w[1] = x[1]; s.w[2] = x[2]; s.w[3] = x[3];
    } else {
        s.w[0] = __uint_as_float(x[0]); s.w[1] = __uint_as_float(x[1]);
        s.w[2] = __uint_as_float(x[2]); s.w[3] = __uint_as_float(x[3]);
    }
}

template <bool BF16, int U>
struct StepBuf {
    Slice<BF16> k[U];
    Slice<BF16> v[U];
};

template <bool BF16, int D, int ROWS, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kPThreads) FD_OCCUPANCY void fd_partial_kernel(PartialArgs a) {
    using S16 = Slice<BF16>;
    constexpr int E = S16::E;             // elements per lane per row slice
    constexpr int LPR = D / E;            // lanes per key row
    constexpr int KPI = 64 / LPR;         // key rows per wave load instruction
    constexpr int U = ROWS >= 8 ? FD_STEP_LOADS_R8 : FD_STEP_LOADS_R4;  // loads per tensor per step
    constexpr int WKEYS = U * KPI;        // keys per wave per step
    constexpr int KSTEP = kPWaves * WKEYS; // keys per workgroup step
    constexpr int ROWB = D * (BF16 ? 2 : 4);  // bytes per key row
    constexpr uint32_t UBYTES = KPI * ROWB;   // bytes per wave load instruction
    constexpr uint32_t SBYTES = KSTEP * ROWB; // bytes per workgroup step
    static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "lane layout");

    __shared__ float sm_m[kPWaves][ROWS];
    __shared__ float sm_l[kPWaves][ROWS];
    __shared__ float sm_acc[kPWaves][ROWS][D];

    const int s = blockIdx.x;
    const int g = blockIdx.y / a.row_blocks;
    const int rb = blockIdx.y - g * a.row_blocks;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int grp = lane / LPR;
    const int pos = lane - grp * LPR;

    int L = a.cache_lens[b];
    L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
    int lo, hi, S;
    tile_of(a.rule, L, s, lo, hi, S);

    const int r0 = rb * ROWS;
    const int nrows = min(ROWS, a.rows - r0);
    // Global index (into [B*Hq*q_len]) of local row 0: rows of one (b, g) are
    // the n_rep heads of the group, each with q_len positions, contiguous.
    const int64_t row0 = ((int64_t)b * a.Hq + (int64_t)g * a.n_rep) * a.q_len + r0;
    const int slots = a.rule.slots;

    if (s >= S) {
        // No keys in this slot.  Mark it empty for the merge (or, with a
        // single slot and an empty sequence, write the empty-row result).
        if (a.direct) {
            for (int idx = tid; idx < nrows * D; idx += kPThreads) {
                if constexpr (BF16)
                    reinterpret_cast<uint16_t*>(a.out)[row0 * D + idx] = 0;
                else
                    reinterpret_cast<float*>(a.out)[row0 * D + idx] = 0.f;
            }
            if (a.lse && tid < nrows) a.lse[row0 + tid] = -INFINITY;
            return;
        }
        if (tid < nrows) {
            a.m_part[(row0 + tid) * slots + s] = -INFINITY;
            a.lse_part[(row0 + tid) * slots + s] = -INFINITY;
        }
        return;
    }

    // Visible-key end of each row inside this tile.  Position t of a chunk
    // of q_len rows sees keys < L - q_len + t + 1; decode rows see < L.
    // Keys at or past mask_from need per-row masking; below it all are live.
    int rend[ROWS];
    int mask_from = hi;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        rend[r] = hi;
        if constexpr (CAUSAL) {
            const int t = (r0 + r) % a.q_len;
            const int nv = L - a.q_len + t + 1;
            if (r < nrows) rend[r] = max(lo, min(hi, nv));
            mask_from = min(mask_from, rend[r]);
        }
    }

    // This lane's slice of every query row (inactive rows are zero).
    S16 qs[ROWS];
    const size_t elem = BF16 ? 2 : 4;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        if (r < nrows) {
            load_slice<BF16>(qs[r], static_cast<const char*>(a.q) + ((row0 + r) * D + pos * E) * elem);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) qs[r].w[i] = 0;
        }
    }
    const float c = a.qk_scale;  // scale * log2(e): scores live in base 2

    float m[ROWS], l[ROWS], acc[ROWS][E];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][e] = 0.f;
    }

    // Each step reads through a buffer resource covering the rest of the
    // tile from that step on: the base and range are scalars, the lane
    // offset is fixed, and the per-instruction offsets are immediates.  A
    // paged cache takes one resource per load instruction instead, over the
    // KPI rows it reads from their page.
    constexpr int ESZ = BF16 ? 2 : 4;
    const char* kt;
    const char* vt;
    const int32_t* tbl = nullptr;
    int rsb = ROWB;  // bytes from one key row of the head to the next
    if constexpr (PAGED) {
        kt = uniform(static_cast<const char*>(a.k) + g * a.pages.head_stride * ESZ);
        vt = uniform(static_cast<const char*>(a.v) + g * a.pages.head_stride * ESZ);
        tbl = a.pages.table + (int64_t)b * a.pages.max_pages;
        rsb = a.pages.row_stride * ESZ;
    } else {
        const int64_t tile_row = ((int64_t)b * a.Hkv + g) * a.Lmax + lo;
        kt = uniform(static_cast<const char*>(a.k) + tile_row * ROWB);
        vt = uniform(static_cast<const char*>(a.v) + tile_row * ROWB);
    }
    const uint32_t tile_bytes = uniform((uint32_t)(hi - lo) * (uint32_t)ROWB);
    const uint32_t lane_off = PAGED ? (uint32_t)(grp * rsb + pos * 16)
                                    : (uint32_t)((w * WKEYS + grp) * ROWB + pos * 16);
    const int lane_key = lo + w * WKEYS + grp;  // key of (step 0, u 0) for this lane
    const int nsteps = (hi - lo + KSTEP - 1) / KSTEP;

    using Buf = StepBuf<BF16, U>;
    auto load = [&](Buf& x, int step) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (PAGED) {
                const int key0 = (int)uniform((uint32_t)(lo + step * KSTEP + w * WKEYS + u * KPI));
                int64_t off;
                const uint32_t n = paged_rows(a.pages, tbl, key0, KPI, hi, rsb, ROWB, &off);
                buffer_slice<BF16>(x.k[u], tile_rsrc(kt + off * ESZ, n), lane_off);
                buffer_slice<BF16>(x.v[u], tile_rsrc(vt + off * ESZ, n), lane_off);
            } else {
                // Scalar arithmetic only (tile_bytes < 2^31): bytes of the
                // tile left from this instruction's first row on, or 0 past
                // its end.
                const int done = (int)uniform((uint32_t)step) * (int)SBYTES + u * (int)UBYTES;
                const int left = max((int)tile_bytes - done, 0);
                buffer_slice<BF16>(x.k[u], tile_rsrc(kt + done, (uint32_t)left), lane_off);
                buffer_slice<BF16>(x.v[u], tile_rsrc(vt + done, (uint32_t)left), lane_off);
            }
        }
    };

    auto compute = [&](const Buf& x, int step) {
        float sc[U][ROWS];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < ROWS; ++r) sc[u][r] = group_sum<LPR>(slice_dot<BF16>(qs[r], x.k[u])) * c;
        // Only a step reaching mask_from has dead keys (tile tail, causal
        // limit); the test is uniform over the workgroup.
        if (lo + (step + 1) * KSTEP > mask_from) {
            const int j0 = lane_key + step * KSTEP;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    if (j0 + u * KPI >= rend[r]) sc[u][r] = -INFINITY;
        }
        // Running max; rescale the state only when some max moved.
        float mx[ROWS];
        bool moved = false;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            mx[r] = m[r];
#pragma unroll
            for (int u = 0; u < U; ++u) mx[r] = fmaxf(mx[r], sc[u][r]);
            moved |= mx[r] > m[r];
        }
        if (__any(moved)) {
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const float mref = mx[r] == -INFINITY ? 0.f : mx[r];
                const float alpha = fast_exp2(m[r] - mref);
                l[r] *= alpha;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[r][e] *= alpha;
                m[r] = mx[r];
            }
        }
        float p[U][ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const float mref = m[r] == -INFINITY ? 0.f : m[r];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                p[u][r] = fast_exp2(sc[u][r] - mref);
                l[r] += p[u][r];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[E];
            to_float<BF16>(x.v[u], vf);
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[r][e] = fmaf(p[u][r], vf[e], acc[r][e]);
        }
    };

    // Two register buffers in turn: the loads of step i+1 are in flight while
    // step i is computed.  The load past the last step falls outside the
    // tile's buffer range and reads nothing.
    Buf A, B;
    load(A, 0);
    for (int step = 0;;) {
        load(B, step + 1);
        compute(A, step);
        if (++step >= nsteps) break;
        load(A, step + 1);
        compute(B, step);
        if (++step >= nsteps) break;
    }

    // Merge the KPI key groups of this wave (lanes with equal pos).
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const float m2 = __shfl_xor(m[r], off);
            const float l2 = __shfl_xor(l[r], off);
            const float M = fmaxf(m[r], m2);
            const float Mr = M == -INFINITY ? 0.f : M;
            const float a1 = fast_exp2(m[r] - Mr);
            const float a2 = fast_exp2(m2 - Mr);
            l[r] = l[r] * a1 + l2 * a2;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[r][e] = acc[r][e] * a1 + __shfl_xor(acc[r][e], off) * a2;
            m[r] = M;
        }
    }

    if (grp == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
#pragma unroll
            for (int e = 0; e < E; ++e) sm_acc[w][r][pos * E + e] = acc[r][e];
            if (pos == 0) {
                sm_m[w][r] = m[r];
                sm_l[w][r] = l[r];
            }
        }
    }
    __syncthreads();

    // Merge the wave states; thread idx handles output (r, d).
    for (int idx = tid; idx < nrows * D; idx += kPThreads) {
        const int r = idx / D;
        const int d = idx - r * D;
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < kPWaves; ++x) M = fmaxf(M, sm_m[x][r]);
        const float Mr = M == -INFINITY ? 0.f : M;
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int x = 0; x < kPWaves; ++x) {
            const float f = fast_exp2(sm_m[x][r] - Mr);
            num = fmaf(f, sm_acc[x][r][d], num);
            den = fmaf(f, sm_l[x][r], den);
        }
        const bool empty = M == -INFINITY;
        const float o = empty ? 0.f : num / den;
        const float lse_v = empty ? -INFINITY : (M + log2f(den)) * kLn2;
        const int64_t row = row0 + r;
        if (a.direct) {
            if constexpr (BF16)
                reinterpret_cast<uint16_t*>(a.out)[row * D + d] = f32_to_bf16(o);
            else
                reinterpret_cast<float*>(a.out)[row * D + d] = o;
            if (d == 0 && a.lse) a.lse[row] = lse_v;
        } else {
            if (!empty) a.o_part[(row * slots + s) * D + d] = o;
            if (d == 0) {
                a.m_part[row * slots + s] = empty ? -INFINITY : M * kLn2;
                a.lse_part[row * slots + s] = lse_v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Merge pass.  WPR waves per query row: up to 32 slots one wave per row (four
// rows per workgroup); with more, four waves split the row's slots (wave w
// takes slots w, w + 4, ...) and wave 0 merges their states through LDS.
// At most four slots go to fd_combine_narrow_kernel below.  Rows hold
// `slots` slots each; with a per-sequence count (spl, [rows / rps]) a row
// merges only the first spl[row / rps] of them.

constexpr int kCThreads = 256;
constexpr int kCWaves = kCThreads / 64;
constexpr int kCombineWideSlots = 32;  // above this, four waves per row

// Slots that row `row` merges: all `slots`, or its sequence's count.
static __device__ __forceinline__ int row_slots(const int32_t* spl, int64_t rps, int64_t row, int slots) {
    if (!spl) return slots;
    const int n = spl[row / rps];
    return n < 0 ? 0 : (n > slots ? slots : n);
}

template <int D, bool OUT_BF16, int WPR>
__global__ __launch_bounds__(kCThreads) void fd_combine_kernel(const float* __restrict__ o_part,
                                                               const float* __restrict__ lse_part, int slots,
                                                               const int32_t* __restrict__ spl, int64_t rps,
                                                               int64_t rows, void* out, float* lse) {
    constexpr int C4 = D / 4;
    constexpr int RPB = kCWaves / WPR;  // rows per workgroup
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * RPB + w / WPR;
    const int64_t r = row < rows ? row : rows - 1;  // spare waves read a valid row, write nothing
    const int n = row_slots(spl, rps, r, slots);
    MergeState st = merge_slots_wave<D>(o_part + r * slots * D, lse_part + r * slots, n, w % WPR, WPR, lane);
    if constexpr (WPR > 1) {
        __shared__ float sm_m[kCWaves], sm_z[kCWaves];
        __shared__ float4 sm_acc[kCWaves][C4];
        if (lane < C4) {
            sm_acc[w][lane] = st.acc;
            if (lane == 0) {
                sm_m[w] = st.m;
                sm_z[w] = st.z;
            }
        }
        __syncthreads();
        if (w != 0) return;
        if (lane < C4) {
            st = MergeState{sm_m[0], sm_z[0], sm_acc[0][lane]};
#pragma unroll
            for (int x = 1; x < WPR; ++x) merge_into(st, MergeState{sm_m[x], sm_z[x], sm_acc[x][lane]});
        }
    }
    if (row < rows && lane < C4) {
        void* orow = OUT_BF16 ? (void*)(reinterpret_cast<uint16_t*>(out) + row * D)
                              : (void*)(reinterpret_cast<float*>(out) + row * D);
        write_merged<OUT_BF16>(st, orow, lane, lse ? lse + row : nullptr);
    }
}

// Few slots (a long prefill chunk cut into 2-4 tiles): one thread per (row,
// float4 column), kCombineRowsPerThread rows per thread whose loads are all
// issued before any arithmetic, so each thread keeps several 16-byte loads
// in flight instead of one per wave-row.
constexpr int kCombineNarrowSlots = 4;
constexpr int kCombineRowsPerThread = 4;

template <int D, bool OUT_BF16, int S>
__global__ __launch_bounds__(kCThreads) void fd_combine_narrow_kernel(const float* __restrict__ o_part,
                                                                      const float* __restrict__ lse_part,
                                                                      const int32_t* __restrict__ spl, int64_t rps,
                                                                      int64_t rows, void* out, float* lse) {
    constexpr int C4 = D / 4;                  // float4 columns
    constexpr int RPB = kCThreads / C4;        // rows of the workgroup per round
    constexpr int RPT = kCombineRowsPerThread;
    const int c4 = threadIdx.x % C4;
    const int64_t row0 = (int64_t)blockIdx.x * RPB * RPT + threadIdx.x / C4;
    float lv[RPT][S];
    float4 ov[RPT][S];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int64_t row = row0 + (int64_t)i * RPB;
        const int64_t r = row < rows ? row : rows - 1;  // spare rows read a valid row, write nothing
        const int n = row_slots(spl, rps, r, S);
#pragma unroll
        for (int sl = 0; sl < S; ++sl) {
            lv[i][sl] = sl < n ? lse_part[r * S + sl] : -INFINITY;
            ov[i][sl] = sl < n ? reinterpret_cast<const float4*>(o_part)[(r * S + sl) * C4 + c4]
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int64_t row = row0 + (int64_t)i * RPB;
        if (row >= rows) continue;
        MergeState st{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll
        for (int sl = 0; sl < S; ++sl) st.m = fmaxf(st.m, lv[i][sl]);
        if (st.m != -INFINITY) {
#pragma unroll
            for (int sl = 0; sl < S; ++sl) {
                if (lv[i][sl] == -INFINITY) continue;  // empty slot: its o entry never enters
                const float wgt = __expf(lv[i][sl] - st.m);
                st.z += wgt;
                st.acc.x = fmaf(wgt, ov[i][sl].x, st.acc.x);
                st.acc.y = fmaf(wgt, ov[i][sl].y, st.acc.y);
                st.acc.z = fmaf(wgt, ov[i][sl].z, st.acc.z);
                st.acc.w = fmaf(wgt, ov[i][sl].w, st.acc.w);
            }
        }
        void* orow = OUT_BF16 ? (void*)(reinterpret_cast<uint16_t*>(out) + row * D)
                              : (void*)(reinterpret_cast<float*>(out) + row * D);
        write_merged<OUT_BF16>(st, orow, c4, lse ? lse + row : nullptr);
    }
}

template <int D, bool OUT_BF16, int S>
void launch_combine_narrow(int64_t rows, const float* o_part, const float* lse_part, const int32_t* spl,
                           int64_t rps, void* out, float* lse, hipStream_t stream) {
    constexpr int rows_per_block = kCThreads / (D / 4) * kCombineRowsPerThread;
    hipLaunchKernelGGL((fd_combine_narrow_kernel<D, OUT_BF16, S>),
                       dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)), dim3(kCThreads), 0, stream,
                       o_part, lse_part, spl, rps, rows, out, lse);
}

template <int D, bool OUT_BF16>
void launch_combine_d(int64_t rows, int slots, const float* o_part, const float* lse_part, const int32_t* spl,
                      int64_t rps, void* out, float* lse, hipStream_t stream) {
    dim3 block(kCThreads);
    if (slots <= kCombineNarrowSlots) {
        switch (slots) {
            case 1: launch_combine_narrow<D, OUT_BF16, 1>(rows, o_part, lse_part, spl, rps, out, lse, stream); return;
            case 2: launch_combine_narrow<D, OUT_BF16, 2>(rows, o_part, lse_part, spl, rps, out, lse, stream); return;
            case 3: launch_combine_narrow<D, OUT_BF16, 3>(rows, o_part, lse_part, spl, rps, out, lse, stream); return;
            default: launch_combine_narrow<D, OUT_BF16, 4>(rows, o_part, lse_part, spl, rps, out, lse, stream); return;
        }
    }
    if (slots > kCombineWideSlots)
        hipLaunchKernelGGL((fd_combine_kernel<D, OUT_BF16, kCWaves>), dim3((unsigned)rows), block, 0, stream,
                           o_part, lse_part, slots, spl, rps, rows, out, lse);
    else
        hipLaunchKernelGGL((fd_combine_kernel<D, OUT_BF16, 1>), dim3((unsigned)((rows + kCWaves - 1) / kCWaves)),
                           block, 0, stream, o_part, lse_part, slots, spl, rps, rows, out, lse);
}

// ---------------------------------------------------------------------------
// Streaming read (a measurement aid): each thread reads 16-byte pieces
// kStreamUnroll at a time, all issued before any is used, and folds them by
// XOR.  Two patterns: strided over the whole grid (consecutive threads read
// consecutive pieces, the grid sweeps the buffer together), or one
// contiguous range per workgroup (as the partial kernels read their tiles).
// A thread's fold reaches *sink only if it equals kStreamMagic, which the
// compiler cannot rule out, so no load can be removed.

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;
constexpr uint32_t kStreamMagic = 0x6a09e667u;

typedef __attribute__((ext_vector_type(4))) uint32_t stream_u32x4;

__global__ __launch_bounds__(kStreamThreads) void fd_stream_read_kernel(const stream_u32x4* __restrict__ buf,
                                                                        uint64_t n16, uint32_t* sink) {
    const uint64_t nthreads = (uint64_t)gridDim.x * kStreamThreads;
    uint64_t i = (uint64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kStreamUnroll - 1) * nthreads < n16; i += kStreamUnroll * nthreads) {
        stream_u32x4 x[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) x[u] = __builtin_nontemporal_load(buf + i + u * nthreads);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    for (; i < n16; i += nthreads) {
        const stream_u32x4 x = __builtin_nontemporal_load(buf + i);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    if (acc == kStreamMagic) *sink = acc;
}

// Workgroup w reads pieces [w * per, (w + 1) * per) (per a multiple of
// kStreamThreads), kStreamUnroll rows of kStreamThreads pieces at a time.
__global__ __launch_bounds__(kStreamThreads) void fd_stream_read_chunk_kernel(const stream_u32x4* __restrict__ buf,
                                                                              uint64_t n16, uint64_t per,
                                                                              uint32_t* sink) {
    const uint64_t beg = (uint64_t)blockIdx.x * per;
    const uint64_t end = beg + per < n16 ? beg + per : n16;
    uint64_t i = beg + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kStreamUnroll - 1) * kStreamThreads < end; i += kStreamUnroll * kStreamThreads) {
        stream_u32x4 x[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) x[u] = __builtin_nontemporal_load(buf + i + u * kStreamThreads);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
    for (; i < end; i += kStreamThreads) {
        const stream_u32x4 x = __builtin_nontemporal_load(buf + i);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    if (acc == kStreamMagic) *sink = acc;
}

template <bool BF16, int D, bool CAUSAL, bool PAGED>
void launch_partials_c(int batch, const PartialArgs& a, hipStream_t stream) {
    const int rpb = vector_block_rows(a.rows);
    dim3 grid(a.rule.slots, a.Hkv * a.row_blocks, batch);
    dim3 block(kPThreads);
    switch (rpb) {
        case 1: hipLaunchKernelGGL((fd_partial_kernel<BF16, D, 1, CAUSAL, PAGED>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((fd_partial_kernel<BF16, D, 2, CAUSAL, PAGED>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((fd_partial_kernel<BF16, D, 4, CAUSAL, PAGED>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((fd_partial_kernel<BF16, D, 8, CAUSAL, PAGED>), grid, block, 0, stream, a); break;
    }
}

// bf16 caches go to the matrix-core kernels whenever those apply (every
// supported head_dim), so the paged variants exist for fp32 only.
template <bool BF16, int D>
hipError_t launch_partials_d(int batch, const PartialArgs& a, hipStream_t stream) {
    const bool paged = a.pages.table != nullptr;
    if (paged && BF16) return hipErrorNotSupported;
    if (a.q_len > 1) {
        if (paged) launch_partials_c<BF16, D, true, !BF16>(batch, a, stream);
        else launch_partials_c<BF16, D, true, false>(batch, a, stream);
    } else {
        if (paged) launch_partials_c<BF16, D, false, !BF16>(batch, a, stream);
        else launch_partials_c<BF16, D, false, false>(batch, a, stream);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partials(int dtype, int head_dim, int batch, const PartialArgs& a,
                           hipStream_t stream) {
    // Caches of one-byte codes are read by the matrix-core kernels only.
    if (a.kv_codes != kKvBf16 || use_mfma_partials(dtype, head_dim, a.rows))
        return launch_partials_mfma(head_dim, batch, a, stream);
    const bool bf16 = dtype == 1;
    if (bf16) {
        return head_dim == 64 ? launch_partials_d<true, 64>(batch, a, stream)
                              : launch_partials_d<true, 128>(batch, a, stream);
    }
    return head_dim == 64 ? launch_partials_d<false, 64>(batch, a, stream)
                          : launch_partials_d<false, 128>(batch, a, stream);
}

hipError_t launch_combine(int head_dim, int out_dtype, int64_t rows, int slots,
                          const float* o_part, const float* lse_part, const int32_t* splits_per_seq,
                          int64_t rows_per_seq, void* out, float* lse, hipStream_t stream) {
    const bool bf16 = out_dtype == 1;
    const int32_t* spl = splits_per_seq;
    const int64_t rps = rows_per_seq > 0 ? rows_per_seq : 1;
    if (head_dim == 64) {
        if (bf16) launch_combine_d<64, true>(rows, slots, o_part, lse_part, spl, rps, out, lse, stream);
        else launch_combine_d<64, false>(rows, slots, o_part, lse_part, spl, rps, out, lse, stream);
    } else {
        if (bf16) launch_combine_d<128, true>(rows, slots, o_part, lse_part, spl, rps, out, lse, stream);
        else launch_combine_d<128, false>(rows, slots, o_part, lse_part, spl, rps, out, lse, stream);
    }
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, uint64_t bytes, int workgroups, int pattern, uint32_t* sink,
                              hipStream_t stream) {
    const uint64_t n16 = bytes / 16;
    if (pattern == 0) {
        hipLaunchKernelGGL(fd_stream_read_kernel, dim3((unsigned)workgroups), dim3(kStreamThreads), 0, stream,
                           static_cast<const stream_u32x4*>(buf), n16, sink);
    } else {
        uint64_t per = (n16 + (uint64_t)workgroups - 1) / (uint64_t)workgroups;
        per = (per + kStreamThreads - 1) / kStreamThreads * kStreamThreads;
        hipLaunchKernelGGL(fd_stream_read_chunk_kernel, dim3((unsigned)workgroups), dim3(kStreamThreads), 0, stream,
                           static_cast<const stream_u32x4*>(buf), n16, per, sink);
    }
    return hipGetLastError();
}

}  // namespace fdk
