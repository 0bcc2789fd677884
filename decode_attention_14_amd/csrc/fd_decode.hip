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
//   fd_combine_kernel  one workgroup per query row.  It merges the row's
//                      tiles: LSE = ln sum_s exp(lse_s), out = sum_s
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
#if FD_WAVES_PER_SIMD > 0
#define FD_OCCUPANCY __attribute__((amdgpu_waves_per_eu(FD_WAVES_PER_SIMD)))
#else
#define FD_OCCUPANCY
#endif

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
#define FD_COMBINE_MAX_SLOTS 256
static_assert(FD_COMBINE_MAX_SLOTS == kThreads, "one lse slot per combine thread");

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane moves inside 16-lane rows (bound_ctrl: no lane reads outside).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;           // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;           // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within 16

// Sum over aligned groups of N lanes; every lane of the group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "N");
    if constexpr (N >= 2) x += dpp<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ void tile_of(const SplitRule& r, int L, int s, int& lo, int& hi, int& S) {
    int T = r.tile_len > 0 ? r.tile_len : (L + r.num_splits - 1) / r.num_splits;
    if (T < 1) T = 1;
    S = (L + T - 1) / T;
    if (S > r.slots) S = r.slots;
    lo = s * T;
    hi = (s == S - 1) ? L : min(L, lo + T);
}

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

// Wave-uniform copies (scalar registers) of values the compiler cannot prove
// uniform by itself.
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const char* uniform(const char* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = uniform((uint32_t)u), hi = uniform((uint32_t)(u >> 32));
    return reinterpret_cast<const char*>(lo | (hi << 32));
}

// Buffer resource over [base, base + bytes): loads at or past `bytes` return 0
// and touch no memory, so tail lanes need no address clamping.  Base and
// range must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(uniform(base)), (short)0,
                                             (int)uniform(bytes), 0x00020000);
}

template <bool BF16>
__device__ __forceinline__ void buffer_slice(Slice<BF16>& s, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
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

template <bool BF16, int D, int ROWS, bool CAUSAL>
__global__ __launch_bounds__(kThreads) FD_OCCUPANCY void fd_partial_kernel(PartialArgs a) {
    using S16 = Slice<BF16>;
    constexpr int E = S16::E;             // elements per lane per row slice
    constexpr int LPR = D / E;            // lanes per key row
    constexpr int KPI = 64 / LPR;         // key rows per wave load instruction
    constexpr int U = ROWS >= 8 ? FD_STEP_LOADS_R8 : FD_STEP_LOADS_R4;  // loads per tensor per step
    constexpr int WKEYS = U * KPI;        // keys per wave per step
    constexpr int KSTEP = kWaves * WKEYS; // keys per workgroup step
    constexpr int ROWB = D * (BF16 ? 2 : 4);  // bytes per key row
    constexpr uint32_t UBYTES = KPI * ROWB;   // bytes per wave load instruction
    constexpr uint32_t SBYTES = KSTEP * ROWB; // bytes per workgroup step
    static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "lane layout");

    __shared__ float sm_m[kWaves][ROWS];
    __shared__ float sm_l[kWaves][ROWS];
    __shared__ float sm_acc[kWaves][ROWS][D];

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
            for (int idx = tid; idx < nrows * D; idx += kThreads) {
                if constexpr (BF16)
                    reinterpret_cast<uint16_t*>(a.out)[row0 * D + idx] = 0;
                else
                    reinterpret_cast<float*>(a.out)[row0 * D + idx] = 0.f;
            }
            if (a.lse && tid < nrows) a.lse[row0 + tid] = -INFINITY;
        } else if (tid < nrows) {
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
    // offset is fixed, and the per-instruction offsets are immediates.
    const int64_t tile_row = ((int64_t)b * a.Hkv + g) * a.Lmax + lo;
    const char* kt = uniform(static_cast<const char*>(a.k) + tile_row * ROWB);
    const char* vt = uniform(static_cast<const char*>(a.v) + tile_row * ROWB);
    const uint32_t tile_bytes = uniform((uint32_t)(hi - lo) * (uint32_t)ROWB);
    const uint32_t lane_off = (uint32_t)((w * WKEYS + grp) * ROWB + pos * 16);
    const int lane_key = lo + w * WKEYS + grp;  // key of (step 0, u 0) for this lane
    const int nsteps = (hi - lo + KSTEP - 1) / KSTEP;

    using Buf = StepBuf<BF16, U>;
    auto load = [&](Buf& x, int step) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // Scalar arithmetic only (tile_bytes < 2^31): bytes of the tile
            // left from this instruction's first row on, or 0 past its end.
            const int done = (int)uniform((uint32_t)step) * (int)SBYTES + u * (int)UBYTES;
            const int left = max((int)tile_bytes - done, 0);
            buffer_slice<BF16>(x.k[u], tile_rsrc(kt + done, (uint32_t)left), lane_off);
            buffer_slice<BF16>(x.v[u], tile_rsrc(vt + done, (uint32_t)left), lane_off);
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
    for (int idx = tid; idx < nrows * D; idx += kThreads) {
        const int r = idx / D;
        const int d = idx - r * D;
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) M = fmaxf(M, sm_m[x][r]);
        const float Mr = M == -INFINITY ? 0.f : M;
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) {
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
// Merge pass.

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// One workgroup per row.  Thread (sp, c) owns float4 column c of the slots
// sp, sp + NSP, ...; all of its o_part loads are issued before the lse
// reductions so that a single memory round trip covers the row.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void fd_combine_kernel(const float* __restrict__ o_part,
                                                              const float* __restrict__ lse_part,
                                                              int slots, void* out, float* lse) {
    constexpr int TPS = D / 4;           // threads per slot, one float4 each
    constexpr int NSP = kThreads / TPS;  // slots read in parallel
    constexpr int CH = 16;               // slots per thread per batch of loads
    __shared__ float red[kWaves];
    __shared__ float sm_lse[FD_COMBINE_MAX_SLOTS];
    __shared__ float4 sm_acc[NSP][TPS];

    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int sp = tid / TPS;
    const int c = tid - sp * TPS;
    const float* lp = lse_part + row * slots;
    const float4* op = reinterpret_cast<const float4*>(o_part + row * slots * D) + c;

    float4 ov[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int s = sp + i * NSP;
        ov[i] = s < slots ? op[(int64_t)s * TPS] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float x = tid < slots ? lp[tid] : -INFINITY;
    sm_lse[tid] = x;

    float mx = wave_max(x);
    if (lane == 0) red[w] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const bool empty = mx == -INFINITY;
    float z = (empty || x == -INFINITY) ? 0.f : __expf(x - mx);
    z = wave_sum(z);
    if (lane == 0) red[w] = z;
    __syncthreads();
    z = (red[0] + red[1]) + (red[2] + red[3]);
    const float LSE = empty ? -INFINITY : mx + __logf(z);

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!empty) {
        for (int base = 0; base < slots; base += CH * NSP) {
            if (base > 0) {
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int s = base + sp + i * NSP;
                    ov[i] = s < slots ? op[(int64_t)s * TPS] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int s = base + sp + i * NSP;
                const float xs = s < slots ? sm_lse[s] : -INFINITY;
                const bool live = xs != -INFINITY;
                const float wgt = live ? __expf(xs - LSE) : 0.f;
                acc.x = live ? fmaf(wgt, ov[i].x, acc.x) : acc.x;
                acc.y = live ? fmaf(wgt, ov[i].y, acc.y) : acc.y;
                acc.z = live ? fmaf(wgt, ov[i].z, acc.z) : acc.z;
                acc.w = live ? fmaf(wgt, ov[i].w, acc.w) : acc.w;
            }
        }
    }
    sm_acc[sp][c] = acc;
    __syncthreads();
    if (tid < TPS) {
        float4 t = sm_acc[0][tid];
#pragma unroll
        for (int i = 1; i < NSP; ++i) {
            const float4 y = sm_acc[i][tid];
            t.x += y.x; t.y += y.y; t.z += y.z; t.w += y.w;
        }
        if constexpr (OUT_BF16) {
            uint16_t* o = reinterpret_cast<uint16_t*>(out) + row * D + tid * 4;
            uint2 packed;
            packed.x = (uint32_t)f32_to_bf16(t.x) | ((uint32_t)f32_to_bf16(t.y) << 16);
            packed.y = (uint32_t)f32_to_bf16(t.z) | ((uint32_t)f32_to_bf16(t.w) << 16);
            *reinterpret_cast<uint2*>(o) = packed;
        } else {
            reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * D)[tid] = t;
        }
        if (tid == 0 && lse) lse[row] = LSE;
    }
}

template <bool BF16, int D, bool CAUSAL>
void launch_partials_c(int batch, const PartialArgs& a, hipStream_t stream) {
    const int rpb = partial_rows_per_block(a.rows);
    dim3 grid(a.rule.slots, a.Hkv * a.row_blocks, batch);
    dim3 block(kThreads);
    switch (rpb) {
        case 1: hipLaunchKernelGGL((fd_partial_kernel<BF16, D, 1, CAUSAL>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((fd_partial_kernel<BF16, D, 2, CAUSAL>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((fd_partial_kernel<BF16, D, 4, CAUSAL>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((fd_partial_kernel<BF16, D, 8, CAUSAL>), grid, block, 0, stream, a); break;
    }
}

template <bool BF16, int D>
hipError_t launch_partials_d(int batch, const PartialArgs& a, hipStream_t stream) {
    if (a.q_len > 1)
        launch_partials_c<BF16, D, true>(batch, a, stream);
    else
        launch_partials_c<BF16, D, false>(batch, a, stream);
    return hipGetLastError();
}

}  // namespace

int partial_rows_per_block(int rows) {
    if (rows <= 1) return 1;
    if (rows <= 2) return 2;
    if (rows <= 4) return 4;
    return 8;
}

hipError_t launch_partials(int dtype, int head_dim, int batch, const PartialArgs& a,
                           hipStream_t stream) {
    const bool bf16 = dtype == 1;
    if (bf16) {
        return head_dim == 64 ? launch_partials_d<true, 64>(batch, a, stream)
                              : launch_partials_d<true, 128>(batch, a, stream);
    }
    return head_dim == 64 ? launch_partials_d<false, 64>(batch, a, stream)
                          : launch_partials_d<false, 128>(batch, a, stream);
}

hipError_t launch_combine(int head_dim, int out_dtype, int64_t rows, int slots,
                          const float* o_part, const float* lse_part, void* out, float* lse,
                          hipStream_t stream) {
    dim3 grid((unsigned)rows), block(kThreads);
    const bool bf16 = out_dtype == 1;
    if (head_dim == 64) {
        if (bf16)
            hipLaunchKernelGGL((fd_combine_kernel<64, true>), grid, block, 0, stream, o_part, lse_part, slots, out, lse);
        else
            hipLaunchKernelGGL((fd_combine_kernel<64, false>), grid, block, 0, stream, o_part, lse_part, slots, out, lse);
    } else {
        if (bf16)
            hipLaunchKernelGGL((fd_combine_kernel<128, true>), grid, block, 0, stream, o_part, lse_part, slots, out, lse);
        else
            hipLaunchKernelGGL((fd_combine_kernel<128, false>), grid, block, 0, stream, o_part, lse_part, slots, out, lse);
    }
    return hipGetLastError();
}

}  // namespace fdk
