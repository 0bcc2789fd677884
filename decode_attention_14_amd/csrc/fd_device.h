// fd_device.h -- device helpers shared by the HIP kernels of the library
// (fd_decode.hip, fd_mfma.hip, fd_chunk.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fdk {

constexpr float kLn2 = 0.69314718055994530942f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

static __device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
static __device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even; NaN stays a quiet NaN.
static __device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static __device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane moves inside 16-lane rows (bound_ctrl: no lane reads outside).
template <int CTRL>
static __device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
static constexpr int kDppXor1 = 0xB1;           // quad_perm [1,0,3,2]
static constexpr int kDppXor2 = 0x4E;           // quad_perm [2,3,0,1]
static constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
static constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within 16

// Sum over aligned groups of N lanes; every lane of the group gets the sum.
template <int N>
static __device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "N");
    if constexpr (N >= 2) x += dpp<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

static __device__ __forceinline__ void tile_of(const SplitRule& r, int L, int s, int& lo, int& hi, int& S) {
    int T = r.tile_len;
    if (T <= 0) {
        T = (L + r.num_splits - 1) / r.num_splits;
        T = (T + r.granule - 1) / r.granule * r.granule;
    }
    if (T < 1) T = 1;
    S = (L + T - 1) / T;
    if (S > r.slots) S = r.slots;
    lo = s * T;
    hi = (s == S - 1) ? L : min(L, lo + T);
}

// Entry i of a block table row, read through the scalar cache: the table
// does not change during a kernel, and a vector load here would make the
// compiler wait for every load in flight (vmcnt counts in order) before the
// page's own loads can issue.  i must be wave-uniform.
static __device__ __forceinline__ int page_id(const int32_t* tbl, int i) {
    typedef const __attribute__((address_space(4))) int32_t* const_ptr;
    return ((const_ptr)(reinterpret_cast<uintptr_t>(tbl)))[i];
}

// Page id of the rows from key0 on (a wave-uniform key), or -1 if key0 is
// at or past hi: then nothing is read, not even the table entry.
static __device__ __forceinline__ int page_at(const PagedKV& pk, const int32_t* tbl, int key0, int hi) {
    return key0 < hi ? page_id(tbl, key0 >> pk.page_shift) : -1;
}

// Rows [key0, key0 + nkeys) of one KV head of a paged cache held by page
// `page`, cut at `hi`: sets *off to the element offset of row key0 from the
// head's base and returns the byte range that covers the rows below hi
// ((rows - 1) * rsb + rowb), or 0 when there are none or the page id lies
// outside the pool (then every row reads as zeros).  The rows must lie in
// one page: nkeys divides the page size and key0 is a multiple of nkeys.
static __device__ __forceinline__ uint32_t paged_rows_in(const PagedKV& pk, int page, int key0, int nkeys, int hi,
                                                         int rsb, int rowb, int64_t* off) {
    *off = 0;
    const int nrow = min(nkeys, hi - key0);
    if (nrow <= 0 || (uint32_t)page >= (uint32_t)pk.num_pages) return 0u;
    *off = (int64_t)page * pk.page_stride + (int64_t)(key0 & ((1 << pk.page_shift) - 1)) * pk.row_stride;
    return (uint32_t)((nrow - 1) * rsb + rowb);
}

// The same, looking the page up in the table row tbl.
static __device__ __forceinline__ uint32_t paged_rows(const PagedKV& pk, const int32_t* tbl, int key0, int nkeys,
                                                      int hi, int rsb, int rowb, int64_t* off) {
    return paged_rows_in(pk, page_at(pk, tbl, key0, hi), key0, nkeys, hi, rsb, rowb, off);
}

// Wave-uniform copies (scalar registers) of values the compiler cannot prove
// uniform by itself.
static __device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
static __device__ __forceinline__ const char* uniform(const char* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = uniform((uint32_t)u), hi = uniform((uint32_t)(u >> 32));
    return reinterpret_cast<const char*>(lo | (hi << 32));
}

// Buffer resource over [base, base + bytes): loads at or past `bytes` return 0
// and touch no memory, so tail lanes need no address clamping.  Base and
// range must be wave-uniform.
static __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(uniform(base)), (short)0,
                                             (int)uniform(bytes), 0x00020000);
}

// ---------------------------------------------------------------------------
// Merge of per-tile partials (page "FlashDecoding算法原理与多GPU并行解码实战",
// multi-GPU step 3, with each tile's weight read as its softmax denominator):
//   LSE = ln sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) o_s.
// Slots with lse = -inf are empty; their o entries never enter the arithmetic
// (they may hold anything, NaN included).  No finite slot: out = 0,
// lse = -inf.

// Running merge state of a set of slots, with reference max m: z = sum
// exp(lse_s - m), acc = sum exp(lse_s - m) o_s (one float4 column).
struct MergeState {
    float m, z;
    float4 acc;
};

static __device__ __forceinline__ void merge_into(MergeState& a, const MergeState& b) {
    const float M = fmaxf(a.m, b.m);
    const float f1 = a.m == -INFINITY ? 0.f : __expf(a.m - M);
    const float f2 = b.m == -INFINITY ? 0.f : __expf(b.m - M);
    a.z = a.z * f1 + b.z * f2;
    a.acc.x = a.acc.x * f1 + b.acc.x * f2;
    a.acc.y = a.acc.y * f1 + b.acc.y * f2;
    a.acc.z = a.acc.z * f1 + b.acc.z * f2;
    a.acc.w = a.acc.w * f1 + b.acc.w * f2;
    a.m = M;
}

// One wave accumulates the slots first, first + stride, first + 2 stride, ...
// (< slots) of one row: o_row [slots][D], lse_row [slots] fp32.  Lane (slot
// group sg, float4 column c4) takes every SG-th of those slots, 32 slots of
// the wave per batch of loads; the slot groups are merged with shuffles, so
// lanes c4 < D/4 return the wave's state for column c4.
template <int D>
static __device__ __forceinline__ MergeState merge_slots_wave(const float* o_row, const float* lse_row, int slots,
                                                             int first, int stride, int lane) {
    constexpr int C4 = D / 4;     // float4 columns
    constexpr int SG = 64 / C4;   // slot groups (2 for D = 128, 4 for D = 64)
    constexpr int CH = 32 / SG;   // slots per lane per batch
    const int sg = lane / C4;
    const int c4 = lane - sg * C4;
    const float4* op = reinterpret_cast<const float4*>(o_row) + c4;
    MergeState st{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
    for (int base = first + sg * stride; base < slots; base += SG * CH * stride) {
        float lv[CH];
        float4 ov[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int s = base + k * SG * stride;
            lv[k] = s < slots ? lse_row[s] : -INFINITY;
            ov[k] = s < slots ? op[(int64_t)s * C4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float bm = st.m;
#pragma unroll
        for (int k = 0; k < CH; ++k) bm = fmaxf(bm, lv[k]);
        if (bm != -INFINITY) {
            const float sc = st.m == -INFINITY ? 0.f : __expf(st.m - bm);
            st.z *= sc;
            st.acc.x *= sc; st.acc.y *= sc; st.acc.z *= sc; st.acc.w *= sc;
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if (lv[k] != -INFINITY) {
                    const float wgt = __expf(lv[k] - bm);
                    st.z += wgt;
                    st.acc.x = fmaf(wgt, ov[k].x, st.acc.x);
                    st.acc.y = fmaf(wgt, ov[k].y, st.acc.y);
                    st.acc.z = fmaf(wgt, ov[k].z, st.acc.z);
                    st.acc.w = fmaf(wgt, ov[k].w, st.acc.w);
                }
            }
            st.m = bm;
        }
    }
#pragma unroll
    for (int off = C4; off < 64; off <<= 1) {
        MergeState o;
        o.m = __shfl_xor(st.m, off);
        o.z = __shfl_xor(st.z, off);
        o.acc.x = __shfl_xor(st.acc.x, off); o.acc.y = __shfl_xor(st.acc.y, off);
        o.acc.z = __shfl_xor(st.acc.z, off); o.acc.w = __shfl_xor(st.acc.w, off);
        merge_into(st, o);
    }
    return st;
}

// Final output of a merged row for column c4: out (bf16 or fp32) and lse.
template <bool OUT_BF16>
static __device__ __forceinline__ void write_merged(const MergeState& st, void* out_row, int c4, float* lse_out) {
    const bool empty = st.m == -INFINITY;
    const float inv = empty ? 0.f : 1.f / st.z;
    const float4 o = make_float4(st.acc.x * inv, st.acc.y * inv, st.acc.z * inv, st.acc.w * inv);
    if constexpr (OUT_BF16) {
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16(o.x) | ((uint32_t)f32_to_bf16(o.y) << 16);
        packed.y = (uint32_t)f32_to_bf16(o.z) | ((uint32_t)f32_to_bf16(o.w) << 16);
        reinterpret_cast<uint2*>(out_row)[c4] = packed;
    } else {
        reinterpret_cast<float4*>(out_row)[c4] = o;
    }
    if (c4 == 0 && lse_out) *lse_out = empty ? -INFINITY : st.m + __logf(st.z);
}

}  // namespace fdk
