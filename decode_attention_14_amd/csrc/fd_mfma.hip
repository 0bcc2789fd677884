// fd_mfma.hip -- split-KV partial kernel on the matrix cores, for bf16 caches
// on gfx950 (CDNA4).
//
// Same operation as the vector kernel in fd_decode.hip: one workgroup per
// (tile s, KV head g, sequence b) turns the tile's keys into a partial output
// with its max and log-sum-exp (page "ChunkedPrefill与FlashDecoding技术解析"
// §3.1: tile-local attention, then the online-softmax merge), with each K/V
// row read once for all query rows of the GQA group (page "FlashDecoding算法
// 原理与多GPU并行解码实战", engineering details item 3).  It serves row
// groups of up to 32 query rows: the n_rep heads of a decode step, or the
// rows of a short causal chunk.
//
// Why matrix cores for decode.  The method does 4 flop per byte of K/V at a
// GQA ratio of 4, so the work is bound by HBM; on the vector ALUs, though,
// the dot products, cross-lane sums and P.V FMAs cost about half of the
// issue slots that streaming at full HBM speed leaves, and the waves then
// stall on their own arithmetic instead of keeping loads in flight.  On the
// matrix cores the same work takes a few percent of the SIMD, so each wave
// mostly issues loads and waits on memory.
//
// Data path.  The tile is cut into blocks of 16 keys.  Wave w takes blocks
// w, w + 4, w + 8, ... (the four waves stream adjacent memory) and keeps a
// private ring of FD_MFMA_STAGES block buffers in LDS, filled by direct
// buffer-to-LDS loads, so the loads in flight cost no registers.  Each row's
// 16-byte chunks are stored XOR-swizzled by the row, which keeps both LDS
// read patterns below free of bank conflicts.
//
//   S^T = K Q^T  v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims of K (one
//                ds_read_b128 per lane), B = the query rows, held in
//                registers for the whole tile.  Lane (group G, column q)
//                receives the scores of keys 4G..4G+3 for query row q.
//   P V          v_mfma_f32_16x16x16bf16_1k per 16 output dims: A = V^T
//                (ds_read_b64_tr_b16 turns row-major V into the transposed
//                operand), B = P^T, which is exactly the score layout above,
//                so P never moves between lanes.  P is split into a bf16
//                high part and a bf16 remainder, two products, so the
//                weights keep about 16 significant bits.
//   softmax      per lane in base 2 with a lazily moved reference max: the
//                state is rescaled only when a score exceeds the reference
//                by more than 2^8 (an exact identity; p <= 256 stays
//                representable), so most blocks need no cross-lane traffic.
//                The exact tile max is tracked separately for m_part.
//
// The four waves' states are merged through LDS at the end, as in the vector
// kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_device.h"
#include "fd_internal.h"

namespace fdk {
namespace {

#ifndef FD_MFMA_STAGES
#define FD_MFMA_STAGES 2
#endif
#ifndef FD_LOAD_AUX
#define FD_LOAD_AUX 2
#endif

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

#ifndef FD_MFMA_THREADS
#define FD_MFMA_THREADS 256
#endif
constexpr int kMT = FD_MFMA_THREADS;  // threads per workgroup (bf16 caches)
constexpr int kMW = kMT / 64;     // waves per workgroup
#ifndef FD_FP8_WAVES
#define FD_FP8_WAVES 8
#endif
constexpr int kMW8 = FD_FP8_WAVES;  // waves per workgroup over fp8 caches
constexpr int kKB = 16;           // keys per block
constexpr int kNS = FD_MFMA_STAGES;
constexpr float kTau = 8.f;       // lazy rescale threshold, log2 units

template <int D>
struct Geo {
    static constexpr int ROWB = 2 * D;          // bytes per key row
    static constexpr int CH = ROWB / 16;        // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;         // rows per 1 KiB LDS-load instruction
    static constexpr int IPB = kKB / RPI;       // instructions per block per tensor
    static constexpr int BLKB = kKB * ROWB;     // bytes per block per tensor
    static constexpr int STAGEB = 2 * BLKB;     // K then V
    static constexpr int WAVEB = kNS * STAGEB;  // ring bytes per wave
    static constexpr int KS = D / 32;           // k-steps of the score product
    static constexpr int DB = D / 16;           // output blocks of the P.V product
    static_assert(CH == 8 || CH == 16, "D = 64 or 128");
};

// Stored-row geometry of the decode kernel's LDS ring: bf16 caches keep
// 2D-byte rows (the operand layout itself); fp8 caches keep D-byte rows,
// dequantised per block into a bf16 block of the operand layout.  An fp8
// block carries half the bytes, so the ring keeps twice the blocks in flight.
#ifndef FD_FP8_STAGES
#define FD_FP8_STAGES 2
#endif
template <int D, bool FP8>
struct LGeo {
    static constexpr int ROWB = FP8 ? D : 2 * D;    // bytes per stored key row
    static constexpr int CH = ROWB / 16;            // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;             // rows per 1 KiB LDS-load instruction
    static constexpr int IPB = kKB / RPI;           // instructions per block per tensor
    static constexpr int BLKB = kKB * ROWB;         // bytes per block per tensor
    static constexpr int STAGEB = 2 * BLKB;         // K then V
    static constexpr int NS = FP8 ? FD_FP8_STAGES : kNS;
    static constexpr int CONVB = FP8 ? 2 * Geo<D>::BLKB : 0;  // bf16 K and V block
    static constexpr int WAVEB = NS * STAGEB + CONVB;
    static_assert(IPB >= 1, "whole load instructions per block");
};

// XOR swizzle of the 16-byte chunks of row r (CH chunks per row).  Two read
// patterns must be free of LDS bank conflicts: 16 consecutive rows at one
// chunk (K operands), and 4 aligned consecutive rows at an even/odd chunk
// pair (transposed V reads).  For CH = 16 the map sends row bits (1:0) to
// chunk bits (2:1), row bit 2 to bit 3 and row bit 3 to bit 0: a bijection on
// 16 rows that keeps bit 0 fixed within an aligned group of 4.  For CH = 8,
// two 128-byte rows share a bank cycle, so the same construction applies to
// the row pair index r >> 1.
template <int CH>
__device__ __forceinline__ int swf(int r) {
    if constexpr (CH == 16) return ((r & 3) << 1) | (((r >> 2) & 1) << 3) | ((r >> 3) & 1);
    const int u = (r >> 1) & 7;
    return ((u & 1) << 1) | (((u >> 1) & 1) << 2) | ((u >> 2) & 1);
}

// Byte offset inside a block of global chunk c of row r.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
    return r * Geo<D>::ROWB + ((c ^ swf<Geo<D>::CH>(r)) << 4);
}

// s_waitcnt with only the vector-memory counter constrained: wait until at
// most N vector loads of this wave are outstanding (gfx9 encoding: vmcnt in
// bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// LDS address (byte offset in the workgroup's LDS) of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// Transposing LDS read, ds_read_b64_tr_b16: in each 16-lane group, lane
// 4j + q names 4 consecutive bf16 of a row; lane i receives element i % 4 of
// lane 4j + i / 4 for j = 0..3.  Issued as inline assembly because the
// compiler treats the builtin as possibly aliasing the LDS loads in flight and
// would wait for all of them; the result is only valid after lds_settle().
__device__ __forceinline__ bf16x4_t tr_read(const char* p) {
    const auto p3 = (const __attribute__((address_space(3))) char*)p;
    const uint32_t addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p3));
    bf16x4_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
    return r;
}

// Wait for every LDS read of this wave, then make the transposed reads'
// registers visible to the compiler as defined here.
template <int N>
__device__ __forceinline__ void lds_settle(bf16x4_t (&v)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// Start the loads of one block (16 rows of K and of V, `left` bytes of the
// tile from kp/vp on; none if left <= 0) into LDS at dst: K rows first, then
// V rows.  Lane l of load instruction i reads its row's global chunk
// dma_off[i]; the data lands at dst + i * 1024 + 16 * l.  Rows past `left`
// read as zeros and cost no memory traffic.
template <int D, bool FP8>
__device__ __forceinline__ void load_block(const char* kp, const char* vp, int left, char* dst,
                                           const uint32_t* dma_off) {
    using L = LGeo<D, FP8>;
    const uint32_t n = left > 0 ? (uint32_t)left : 0u;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kp, n);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vp, n);
#pragma unroll
    for (int i = 0; i < L::IPB; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(dst + i * 1024), 16, dma_off[i], 0, 0,
                                                 FD_LOAD_AUX);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(dst + L::BLKB + i * 1024), 16, dma_off[i], 0, 0,
                                                 FD_LOAD_AUX);
    }
}

// Start the loads of the wave's block `blk` of the tile [lo, hi) into dst:
// contiguous caches address the tile directly (kt/vt: its first row);
// paged caches read the block from page `page` (kt/vt: the KV head's base).
// ESZ: bytes per stored element.
template <int D, bool FP8, bool PAGED>
__device__ __forceinline__ void load_block_at(const PagedKV& pk, int page, const char* kt, const char* vt, int lo,
                                              int hi, int blk, int rsb, char* dst, const uint32_t* dma_off) {
    using L = LGeo<D, FP8>;
    constexpr int ESZ = FP8 ? 1 : 2;
    if constexpr (PAGED) {
        int64_t off;
        const uint32_t n = paged_rows_in(pk, page, lo + blk * kKB, kKB, hi, rsb, L::ROWB, &off);
        load_block<D, FP8>(kt + off * ESZ, vt + off * ESZ, (int)n, dst, dma_off);
    } else {
        const int off = blk * L::BLKB;
        load_block<D, FP8>(kt + off, vt + off, (hi - lo) * L::ROWB - off, dst, dma_off);
    }
}

// Dequantise one landed fp8 block (K at src, V at src + LGeo::BLKB, rows of
// D one-byte OCP E4M3 codes) into bf16 blocks of the operand layout (K at
// dst, V at dst + Geo::BLKB, swizzled as swz).  Every E4M3 value is exact in
// bf16; the per-tensor scales are applied outside (k_scale in the score
// scale, v_scale to the output).  Lane l converts 16-byte chunks l, l + 64,
// ... of each tensor: consecutive lanes read consecutive LDS bytes.
//
// The LDS accesses are inline assembly: as plain loads and stores the
// compiler would treat them as possibly aliasing the buffer-to-LDS loads in
// flight and wait for all of those first, which serialises the ring.  The
// block at src has landed (the caller waited for it), and dst is this
// wave's own area, read only by its own later reads; LDS executes one wave's
// accesses in order.
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__device__ __forceinline__ u32x4_t lds_read_b128(const char* p) {
    u32x4_t r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return r;
}

__device__ __forceinline__ void lds_write_b128(char* p, u32x4_t x) {
    asm volatile("ds_write_b128 %0, %1" : : "v"(lds_addr(p)), "v"(x) : "memory");
}

template <int D>
__device__ __forceinline__ void dequant_block(const char* src, char* dst, int lane) {
    using L = LGeo<D, true>;
    using G = Geo<D>;
    constexpr int NQ = L::BLKB / 16 / 64;  // 16-byte chunks per lane per tensor
    u32x4_t x[2][NQ];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int n = 0; n < NQ; ++n) x[t][n] = lds_read_b128(src + t * L::BLKB + (n * 64 + lane) * 16);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int n = 0; n < NQ; ++n) asm volatile("" : "+v"(x[t][n]));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int q = n * 64 + lane;
            const int r = q / L::CH;
            const int c = q % L::CH;  // 16 codes = dims 16c .. 16c + 15
            const uint32_t w[4] = {x[t][n][0], x[t][n][1], x[t][n][2], x[t][n][3]};
            uint32_t b[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                b[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.f, false));
                b[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.f, true));
            }
            char* o = dst + t * G::BLKB;
            lds_write_b128(o + swz<D>(r, 2 * c), u32x4_t{b[0], b[1], b[2], b[3]});
            lds_write_b128(o + swz<D>(r, 2 * c + 1), u32x4_t{b[4], b[5], b[6], b[7]});
        }
    }
}

// The math of one 16-key block for NB blocks of 16 query rows, given the
// block's K fragments (A operand of S^T = K Q^T) and transposed V fragments
// (A operand of O^T = V^T P^T) in registers.  Lane (group grp, column q)
// holds, per row block nb: the running reference max m (equal in the four
// groups), its share l of the running sum, the exact running max mx of its
// own scores, and acc[nb][db] = O^T rows 16 db + 4 grp .. +3 of column q.
// Keys at or past rend[nb] are masked when `edge` (the block reaches a row's
// end); c = scale * log2(e).
template <int D, int NB>
__device__ __forceinline__ void block_math(const bf16x8_t (&kf)[Geo<D>::KS], const bf16x4_t (&vf)[Geo<D>::DB],
                                           const bf16x8_t (&qf)[NB][Geo<D>::KS], f32x4_t (&acc)[NB][Geo<D>::DB],
                                           float (&m)[NB], float (&l)[NB], float (&mx)[NB], int key0, bool edge,
                                           const int (&rend)[NB], float c, int grp) {
    using G = Geo<D>;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        f32x4_t st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks)
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[nb][ks], st, 0, 0, 0);
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = st[i] * c;
        if (edge) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key0 + 4 * grp + i >= rend[nb]) x[i] = -INFINITY;
        }
        const float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx[nb] = fmaxf(mx[nb], bm);
        if (__any(bm > m[nb] + kTau)) {
            float bw = fmaxf(bm, __shfl_xor(bm, 16));
            bw = fmaxf(bw, __shfl_xor(bw, 32));
            const float mn = fmaxf(m[nb], bw);
            const float alpha = m[nb] == -INFINITY ? 0.f : fast_exp2(m[nb] - mn);
            l[nb] *= alpha;
#pragma unroll
            for (int db = 0; db < G::DB; ++db) acc[nb][db] *= alpha;
            m[nb] = mn;
        }
        const float mref = m[nb] == -INFINITY ? 0.f : m[nb];
        float p[4];
        bf16x4_t ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(x[i] - mref);
            ph[i] = (__bf16)p[i];
            pl[i] = (__bf16)(p[i] - (float)ph[i]);
        }
        l[nb] += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
        for (int db = 0; db < G::DB; ++db) {
            acc[nb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(s16x4_t, vf[db]), __builtin_bit_cast(s16x4_t, ph), acc[nb][db], 0, 0, 0);
            acc[nb][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(s16x4_t, vf[db]), __builtin_bit_cast(s16x4_t, pl), acc[nb][db], 0, 0, 0);
        }
    }
}

// Operand fragments of one 16-key block stored (swizzled) at kb / vb in LDS:
// K rows as the A operand of the score product, V^T through transposed reads.
template <int D>
__device__ __forceinline__ void load_fragments(const char* kb, const char* vb, bf16x8_t (&kf)[Geo<D>::KS],
                                               bf16x4_t (&vf)[Geo<D>::DB], int grp, int col) {
    using G = Geo<D>;
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks)
        kf[ks] = *reinterpret_cast<const bf16x8_t*>(kb + swz<D>(col, grp + 4 * ks));
    const int r = 4 * grp + (col >> 2);
    const int q4 = col & 3;
#pragma unroll
    for (int db = 0; db < G::DB; ++db) vf[db] = tr_read(vb + swz<D>(r, 2 * db + (q4 >> 1)) + 8 * (q4 & 1));
    lds_settle(vf);
}

template <int D, int NB, bool CAUSAL, bool PAGED, bool FP8>
__global__ __launch_bounds__(FP8 ? 64 * kMW8 : kMT) void fd_mfma_partial_kernel(PartialArgs a) {
    using G = Geo<D>;
    using LG = LGeo<D, FP8>;
    constexpr int MW = FP8 ? kMW8 : kMW;  // waves per workgroup
    constexpr int MT = 64 * MW;
    constexpr int NS = LG::NS;
    constexpr int ESZ = FP8 ? 1 : 2;  // bytes per stored K/V element
    constexpr int NR = 16 * NB;  // query rows per workgroup
    constexpr int RS = D + 4;    // padded row stride of the merge area (floats)
    constexpr int MERGEB = MW * (NR * RS + 3 * NR) * 4;
    constexpr int SMEMB = MW * LG::WAVEB > MERGEB ? MW * LG::WAVEB : MERGEB;
    __shared__ __attribute__((aligned(16))) char smem[SMEMB];

    // KV head fastest: workgroups are dealt to the eight XCDs round-robin in
    // launch order, so consecutive ids take the heads of one (tile, sequence)
    // and every XCD gets the same mix of tiles (all heads of a sequence have
    // the same length).  With the tile fastest instead, a tile index would
    // pin to a subset of XCDs and short sequences would leave some idle.
    const int g = blockIdx.x;
    const int s = blockIdx.y;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = (int)uniform((uint32_t)(tid >> 6));
    const int grp = lane >> 4;
    const int col = lane & 15;

    int L = a.cache_lens[b];
    L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
    int lo, hi, S;
    tile_of(a.rule, L, s, lo, hi, S);
    lo = (int)uniform((uint32_t)lo);
    hi = (int)uniform((uint32_t)hi);

    const int nrows = a.rows;
    const int64_t row0 = ((int64_t)b * a.Hq + (int64_t)g * a.n_rep) * a.q_len;
    const int slots = a.rule.slots;

    if (s >= S) {
        if (a.direct) {
            for (int idx = tid; idx < nrows * D; idx += MT)
                reinterpret_cast<uint16_t*>(a.out)[row0 * D + idx] = 0;
            if (a.lse && tid < nrows) a.lse[row0 + tid] = -INFINITY;
            return;
        }
        if (tid < nrows) {
            a.m_part[(row0 + tid) * slots + s] = -INFINITY;
            a.lse_part[(row0 + tid) * slots + s] = -INFINITY;
        }
        return;
    }

    // Visible-key end of this lane's query row in each N block.  Causal rows
    // t of a chunk see keys < L - q_len + t + 1; the smallest end (t = 0)
    // bounds the keys every row sees.
    int rend[NB];
    int mask_from = hi;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        rend[nb] = hi;
        const int r = nb * 16 + col;
        if constexpr (CAUSAL) {
            if (r < nrows) rend[nb] = max(lo, min(hi, L - a.q_len + (r % a.q_len) + 1));
        }
    }
    if constexpr (CAUSAL) mask_from = max(lo, min(hi, L - a.q_len + 1));

    // Query rows: B operand of S^T = K Q^T (column = row, 8 dims per lane).
    bf16x8_t qf[NB][G::KS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 16 + col;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            if (r < nrows) {
                const uint4 x = *reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(a.q) + (row0 + r) * D + 8 * grp + 32 * ks);
                qf[nb][ks] = __builtin_bit_cast(bf16x8_t, x);
            } else {
                qf[nb][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
            }
        }
    }
    const float c = a.qk_scale;  // scale * log2(e)

    f32x4_t acc[NB][G::DB];
    float m[NB], l[NB], mx[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m[nb] = -INFINITY;
        l[nb] = 0.f;
        mx[nb] = -INFINITY;
#pragma unroll
        for (int db = 0; db < G::DB; ++db) acc[nb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    char* ring = smem + w * LG::WAVEB;
    char* conv = ring + NS * LG::STAGEB;  // fp8: this wave's dequantised block
    const char* kt;
    const char* vt;
    int rsb;  // bytes from one stored key row of the head to the next
    const int32_t* tbl = nullptr;
    if constexpr (PAGED) {
        kt = static_cast<const char*>(a.k) + g * a.pages.head_stride * ESZ;
        vt = static_cast<const char*>(a.v) + g * a.pages.head_stride * ESZ;
        rsb = a.pages.row_stride * ESZ;
        tbl = a.pages.table + (int64_t)b * a.pages.max_pages;
    } else {
        const int64_t tile_row = ((int64_t)b * a.Hkv + g) * a.Lmax + lo;
        kt = static_cast<const char*>(a.k) + tile_row * LG::ROWB;
        vt = static_cast<const char*>(a.v) + tile_row * LG::ROWB;
        rsb = LG::ROWB;
    }
    const int nblk = (hi - lo + kKB - 1) / kKB;
    const int nw = w < nblk ? (nblk - w + MW - 1) / MW : 0;

    // Lane l of load instruction i fills LDS slot (row i*RPI + l/CH, chunk
    // l%CH) of the block: bf16 rows with the row's global chunk (l%CH) ^
    // row (the operand swizzle), fp8 rows in their stored order.
    uint32_t dma_off[LG::IPB];
#pragma unroll
    for (int i = 0; i < LG::IPB; ++i) {
        const int r = i * LG::RPI + lane / LG::CH;
        const int cg = FP8 ? lane % LG::CH : (lane % LG::CH) ^ swf<LG::CH>(r);
        dma_off[i] = (uint32_t)(r * rsb + cg * 16);
    }

    // Wave block j is tile block w + 4j and goes to ring slot j % NS.  A
    // paged cache's page ids are read one block ahead of their loads, so the
    // scalar table reads overlap the work of the previous block.
    auto page_of = [&](int blk) { return PAGED ? page_at(a.pages, tbl, lo + blk * kKB, hi) : 0; };
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
        load_block_at<D, FP8, PAGED>(a.pages, page_of(w + j * MW), kt, vt, lo, hi, w + j * MW, rsb,
                                     ring + j * LG::STAGEB, dma_off);
    int page_next = page_of(w + (NS - 1) * MW);

    for (int j = 0; j < nw; ++j) {
        {
            const int jn = j + NS - 1;
            const int page = page_next;
            page_next = page_of(w + (jn + 1) * MW);
            load_block_at<D, FP8, PAGED>(a.pages, page, kt, vt, lo, hi, w + jn * MW, rsb,
                                         ring + (jn % NS) * LG::STAGEB, dma_off);
        }
        wait_vmcnt_le<(NS - 1) * 2 * LG::IPB>();  // block j has landed
        const char* kb = ring + (j % NS) * LG::STAGEB;
        const char* vb = kb + LG::BLKB;
        if constexpr (FP8) {
            dequant_block<D>(kb, conv, lane);
            kb = conv;
            vb = conv + G::BLKB;
        }

        bf16x8_t kf[G::KS];
        bf16x4_t vf[G::DB];
        load_fragments<D>(kb, vb, kf, vf, grp, col);

        const int key0 = lo + (w + j * MW) * kKB;  // first key of the block
        block_math<D, NB>(kf, vf, qf, acc, m, l, mx, key0, key0 + kKB > mask_from, rend, c, grp);
    }

    // Merge: the four lane groups of a column, then the four waves via LDS.
    wait_vmcnt_le<0>();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        l[nb] += __shfl_xor(l[nb], 16);
        l[nb] += __shfl_xor(l[nb], 32);
        mx[nb] = fmaxf(mx[nb], __shfl_xor(mx[nb], 16));
        mx[nb] = fmaxf(mx[nb], __shfl_xor(mx[nb], 32));
    }
    __syncthreads();  // every wave is done with its ring
    float* sm_acc = reinterpret_cast<float*>(smem);  // [MW][NR][RS]
    float* sm_m = sm_acc + MW * NR * RS;            // [MW][NR]
    float* sm_l = sm_m + MW * NR;
    float* sm_x = sm_l + MW * NR;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 16 + col;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
            *reinterpret_cast<f32x4_t*>(sm_acc + (w * NR + r) * RS + 16 * db + 4 * grp) = acc[nb][db];
        if (grp == 0) {
            sm_m[w * NR + r] = m[nb];
            sm_l[w * NR + r] = l[nb];
            sm_x[w * NR + r] = mx[nb];
        }
    }
    __syncthreads();

    for (int idx = tid; idx < nrows * D; idx += MT) {
        const int r = idx / D;
        const int d = idx - r * D;
        float M = -INFINITY, X = -INFINITY;
#pragma unroll
        for (int x = 0; x < MW; ++x) {
            M = fmaxf(M, sm_m[x * NR + r]);
            X = fmaxf(X, sm_x[x * NR + r]);
        }
        float num = 0.f, den = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int x = 0; x < MW; ++x) {
                const float mw = sm_m[x * NR + r];
                const float f = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
                num = fmaf(f, sm_acc[(x * NR + r) * RS + d], num);
                den = fmaf(f, sm_l[x * NR + r], den);
            }
        }
        const bool empty = M == -INFINITY;
        float o = empty ? 0.f : num / den;
        if constexpr (FP8) o *= a.v_scale;  // V was dequantised without its scale
        const float lse_v = empty ? -INFINITY : (M + log2f(den)) * kLn2;
        const int64_t row = row0 + r;
        if (a.direct) {
            reinterpret_cast<uint16_t*>(a.out)[row * D + d] = f32_to_bf16(o);
            if (d == 0 && a.lse) a.lse[row] = lse_v;
        } else {
            if (!empty) a.o_part[(row * slots + s) * D + d] = o;
            if (d == 0) {
                a.m_part[row * slots + s] = empty ? -INFINITY : X * kLn2;
                a.lse_part[row * slots + s] = lse_v;
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Chunked prefill: row groups of more than 32 query rows (page
// "ChunkedPrefill与FlashDecoding技术解析" §2.1: a chunk of q_len new tokens,
// causal inside the chunk, full view of the cached prefix).  Here the work is
// a dense contraction, run on the 32x32x16 matrix instructions (twice the
// rate of the 16x16 shapes on gfx950).
//
// A workgroup takes kChunkRows packed rows; packed row p = t * n_rep + i is
// position t of query head i of the GQA group, so a tile's rows span few
// positions and share one causal limit.  Its eight waves form four row groups
// of 32 rows times two key halves: in every 64-key stage, wave (rg, kh) takes
// the 32-key block kh for the rows of group rg, and the two halves of a group
// are merged through LDS at the end.  Two waves per SIMD hide each other's
// LDS and softmax latency.  Stages stream through one LDS ring of
// FD_CHUNK_STAGES stages, loaded cooperatively with buffer-to-LDS loads, one
// barrier per stage.  Keys that no row of the tile can see are never loaded.
//
//   S^T = K Q^T  (32 keys x 32 rows, k = 16 dims per instruction)
//   O^T = V^T P^T (32 dims x 32 rows, k = 16 keys per instruction): lane
//                (half G, column q) holds the scores of keys 8a + 4G + b of
//                the block (a, b = 0..3), which are exactly its B operand
//                for the two 16-key steps, so P stays in place; V^T comes
//                from transposed LDS reads.  P enters as bf16, plus its
//                bf16 remainder while single keys still carry a visible
//                share of a row's weight (see chunk_softmax).

#ifndef FD_CHUNK_STAGES
#define FD_CHUNK_STAGES 2
#endif
// Vector instructions the scheduler places after each P.V instruction of
// the previous block (the rest of the softmax follows them).
#ifndef FD_CHUNK_VALU_PER_MFMA
#define FD_CHUNK_VALU_PER_MFMA 8
#endif
constexpr int kCT = 512;                // threads per workgroup
constexpr int kCW = kCT / 64;           // waves
constexpr int kCRG = 4;                 // row groups of 32 rows
constexpr int kCKW = kCW / kCRG;        // waves per row group: key halves
constexpr int kChunkRows = 32 * kCRG;   // rows per workgroup
static_assert(kChunkRows == kChunkTileRows, "row tile of the chunk kernel");
constexpr int kCBK = 32;                // keys per block
constexpr int kCNS = FD_CHUNK_STAGES;

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

template <int D>
struct CGeo {
    static constexpr int ROWB = 2 * D;
    static constexpr int CH = ROWB / 16;            // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;             // rows per 1 KiB load instruction
    static constexpr int IPB = kCBK / RPI;          // instructions per block per tensor
    static constexpr int BLKB = kCBK * ROWB;        // bytes per block per tensor
    static constexpr int SKB = kCKW;                // blocks per stage
    static constexpr int SKEYS = SKB * kCBK;        // keys per stage
    static constexpr int STGB = 2 * SKB * BLKB;     // K blocks, then V blocks
    static constexpr int NDMA = SKB * IPB;          // instructions per tensor per stage
    static constexpr int DPW = NDMA / kCW;          // per wave, per tensor
    static constexpr int KS = D / 16;               // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;               // 32-dim blocks of O^T
    static_assert(NDMA % kCW == 0 && DPW >= 1, "stage loads split evenly over the waves");
};

// XOR swizzle of the chunk kernel's 16-byte chunks (CH chunks per row).
// Its read patterns: 16 consecutive rows at one chunk (K operands), and an
// aligned group of 4 rows at 4 consecutive chunks 4d .. 4d + 3 (transposed
// V reads of 32 lanes, 256 bytes per LDS cycle).  For CH = 16 (256-byte
// rows, one bank cycle each) row bits 1:0 go to chunk bits 3:2 and row bits
// 3:2 to bits 1:0: a bijection on 16 rows, and within a 4-row group it
// moves only bits 3:2, which the 4 consecutive chunks leave apart.  For
// CH = 8 two 128-byte rows share a bank cycle, so the rows of one parity
// must differ: the row pair index u = r >> 1 gives bit 2 from u bit 0 and
// bits 1:0 from u bits 2:1.
template <int CH>
__device__ __forceinline__ int cswf(int r) {
    if constexpr (CH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    const int u = (r >> 1) & 7;
    return ((u & 1) << 2) | (u >> 1);
}

// Byte offset inside a 32-row block of global chunk c of row r (the swizzle
// of cswf repeats every 16 rows).
template <int D>
__device__ __forceinline__ int cswz(int r, int c) {
    return r * CGeo<D>::ROWB + ((c ^ cswf<CGeo<D>::CH>(r)) << 4);
}

// Start this wave's share of one stage's loads: bytes [off, off + stage) of
// the K and V tiles, `left` bytes of the tile remaining from off (none if
// left <= 0; rows past it read as zeros), into the stage buffer at dst.
template <int D>
__device__ __forceinline__ void chunk_load_stage(const char* kt, const char* vt, int left, int off, char* dst,
                                                 const uint32_t* dma_off, const int* lds_off) {
    using G = CGeo<D>;
    const uint32_t n = left > 0 ? (uint32_t)left : 0u;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kt + off, n);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vt + off, n);
#pragma unroll
    for (int k = 0; k < G::DPW; ++k) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(dst + lds_off[k]), 16, dma_off[k], 0, 0,
                                                 FD_LOAD_AUX);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(dst + G::SKB * G::BLKB + lds_off[k]), 16,
                                                 dma_off[k], 0, 0, FD_LOAD_AUX);
    }
}

// Stage j of the tile [lo, kend) into dst.  Contiguous caches: kt/vt point
// at the tile's first row and one buffer range covers the stage.  Paged
// caches: kt/vt point at the KV head's base and each load instruction looks
// up the page of its RPI rows (koff[k]: the instruction's first key within
// the stage).
template <int D, bool PAGED>
__device__ __forceinline__ void chunk_stage_at(const PagedKV& pk, const int32_t* tbl, const char* kt, const char* vt,
                                               int lo, int kend, int j, int rsb, char* dst, const uint32_t* dma_off,
                                               const int* lds_off, const int* koff) {
    using G = CGeo<D>;
    if constexpr (PAGED) {
#pragma unroll
        for (int k = 0; k < G::DPW; ++k) {
            int64_t off;
            const uint32_t n = paged_rows(pk, tbl, lo + j * G::SKEYS + koff[k], G::RPI, kend, rsb, G::ROWB, &off);
            const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kt + off * 2, n);
            const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vt + off * 2, n);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(dst + lds_off[k]), 16, dma_off[k], 0, 0,
                                                     FD_LOAD_AUX);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(dst + G::SKB * G::BLKB + lds_off[k]), 16,
                                                     dma_off[k], 0, 0, FD_LOAD_AUX);
        }
    } else {
        const int off = j * G::SKEYS * G::ROWB;
        chunk_load_stage<D>(kt, vt, (kend - lo) * G::ROWB - off, off, dst, dma_off, lds_off);
    }
}

// FP8 caches in the chunk kernel: each stage's E4M3 rows (D bytes, stored
// order) stream into a second two-stage ring, and the workgroup dequantises
// stage j + 1 into the bf16 ring while it computes on stage j, so the
// products run unchanged on bf16 operands.
template <int D>
struct CGeo8 {
    static constexpr int ROWB = D;                    // bytes per stored key row
    static constexpr int CH = ROWB / 16;              // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;               // rows per 1 KiB load instruction
    static constexpr int NDMA = CGeo<D>::SKEYS / RPI; // instructions per tensor per stage
    static constexpr int PW = 2 * NDMA / kCW;         // instructions per wave per stage (K and V)
    static constexpr int TENB = CGeo<D>::SKEYS * ROWB;
    static constexpr int STGB = 2 * TENB;             // K rows, then V rows
    static constexpr int NQ = STGB / 16 / kCT;        // 16-byte chunks each thread dequantises
    static_assert((2 * NDMA) % kCW == 0 && PW >= 1 && STGB % (16 * kCT) == 0, "even split");
};

// Start this wave's loads of fp8 stage j into dst (see chunk_stage_at).
// Instruction k covers RPI rows of K (isv 0) or V (isv 1) from key koff[k]
// of the stage.
template <int D, bool PAGED>
__device__ __forceinline__ void chunk_stage8_at(const PagedKV& pk, const int32_t* tbl, const char* kt,
                                                const char* vt, int lo, int kend, int j, int rsb, char* dst,
                                                const uint32_t* dma_off, const int* lds_off, const int* koff,
                                                const int* isv) {
    using G8 = CGeo8<D>;
    constexpr int SKEYS = CGeo<D>::SKEYS;
#pragma unroll
    for (int k = 0; k < G8::PW; ++k) {
        const char* base = isv[k] ? vt : kt;
        __amdgpu_buffer_rsrc_t r;
        if constexpr (PAGED) {
            int64_t off;
            const uint32_t n = paged_rows(pk, tbl, lo + j * SKEYS + koff[k], G8::RPI, kend, rsb, G8::ROWB, &off);
            r = tile_rsrc(base + off, n);
        } else {
            const int soff = j * SKEYS * G8::ROWB;
            const int left = (kend - lo) * G8::ROWB - soff;
            r = tile_rsrc(base + soff, left > 0 ? (uint32_t)left : 0u);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dst + lds_off[k]), 16, dma_off[k], 0, 0,
                                                 FD_LOAD_AUX);
    }
}

// Dequantise a landed fp8 stage (src) into the bf16 stage layout (dst):
// thread t converts 16-byte chunks t, t + kCT, ... (inline-assembly LDS
// accesses, as in dequant_block).
template <int D>
__device__ __forceinline__ void chunk_dequant_stage(const char* src, char* dst, int tid) {
    using G = CGeo<D>;
    using G8 = CGeo8<D>;
    constexpr int QPT = G8::TENB / 16;  // chunks per tensor
    u32x4_t x[G8::NQ];
#pragma unroll
    for (int n = 0; n < G8::NQ; ++n) x[n] = lds_read_b128(src + (n * kCT + tid) * 16);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int n = 0; n < G8::NQ; ++n) asm volatile("" : "+v"(x[n]));
#pragma unroll
    for (int n = 0; n < G8::NQ; ++n) {
        const int q = n * kCT + tid;
        const int tsr = q / QPT;  // 0: K, 1: V
        const int rem = q - tsr * QPT;
        const int r = rem / G8::CH;
        const int c8 = rem - r * G8::CH;  // codes of dims 16 c8 .. 16 c8 + 15
        uint32_t bw[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bw[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[n][i], 1.f, false));
            bw[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[n][i], 1.f, true));
        }
        char* o = dst + tsr * G::SKB * G::BLKB + (r / kCBK) * G::BLKB;
        lds_write_b128(o + cswz<D>(r % kCBK, 2 * c8), u32x4_t{bw[0], bw[1], bw[2], bw[3]});
        lds_write_b128(o + cswz<D>(r % kCBK, 2 * c8 + 1), u32x4_t{bw[4], bw[5], bw[6], bw[7]});
    }
}

template <int N>
__device__ __forceinline__ void lds_settle8(bf16x8_t (&v)[N]) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}


// 16-byte LDS load at a lane address plus a compile-time offset (folded into
// the instruction's offset field).
template <int OFF>
__device__ __forceinline__ bf16x8_t lds_b128(uint32_t addr) {
    return *(const __attribute__((address_space(3))) bf16x8_t*)(uintptr_t)(addr + OFF);
}

// Transposed read (see tr_read) at a lane address plus a compile-time offset.
template <int OFF>
__device__ __forceinline__ bf16x4_t tr_read_at(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    bf16x4_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// The chunk kernel's work on one 32-key block is spread over two steps so
// that a wave keeps its matrix core fed while it runs the softmax: step j
// issues the score product of block j and the head part of block j - 1's
// P.V product back to back, runs block j's softmax on the vector units while
// they execute, and ends with the (rare) rescale and, where needed, the
// remainder part of block j's P.V product.

// K operands of a block (stage buffer at compile-time offset OFF) and S^T.
template <int D, int OFF>
__device__ __forceinline__ void chunk_scores(const uint32_t (&ka)[CGeo<D>::KS], const bf16x8_t (&qf)[CGeo<D>::KS],
                                             f32x16_t& st) {
    using G = CGeo<D>;
    bf16x8_t kf[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) kf[ks] = lds_b128<OFF>(ka[ks]);
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], st, 0, 0, 0);
    // All K reads first, so the products wait on LDS once.
    __builtin_amdgcn_sched_group_barrier(0x100, G::KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, G::KS, 0);
}

// Start the transposed reads of a block's V operands; valid after lds_settle8.
template <int D, int OFF>
__device__ __forceinline__ void chunk_v_reads(const uint32_t (&va)[CGeo<D>::DB][2], bf16x8_t (&vf)[CGeo<D>::DB * 2]) {
    using G = CGeo<D>;
    constexpr int K2 = 16 * G::ROWB;  // 16 rows further down the block
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
        const bf16x4_t a0 = tr_read_at<OFF>(va[db][0]);
        const bf16x4_t a1 = tr_read_at<OFF>(va[db][1]);
        const bf16x4_t b0 = tr_read_at<OFF + K2>(va[db][0]);
        const bf16x4_t b1 = tr_read_at<OFF + K2>(va[db][1]);
        vf[db * 2] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        vf[db * 2 + 1] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// O^T += V^T P^T for one block and one bf16 part of P.  The 16-key halves
// are the outer loop so that consecutive instructions use different
// accumulators.
template <int D>
__device__ __forceinline__ void chunk_pv(const bf16x8_t (&vf)[CGeo<D>::DB * 2], const bf16x8_t (&pp)[2],
                                         f32x16_t (&acc)[CGeo<D>::DB]) {
    using G = CGeo<D>;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db * 2 + k2], pp[k2], acc[db], 0, 0, 0);
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;

__device__ __forceinline__ bf16x8_t pack8(bf16x2_t a, bf16x2_t b, bf16x2_t c, bf16x2_t d) {
    const bf16x4_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4_t cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Online-softmax statistics and weights of one block (no access to the
// accumulators, so it can overlap the matrix work of the previous block):
// tracks the exact max mx, moves the lazy reference m when the block's max
// passes it by more than kTau (alpha is then the factor that the
// accumulators still owe, else 1), and writes P as bf16 head ph and, if lo,
// remainder pl.
//
// The running sum l adds the weights that the products actually use: the
// bf16 heads, plus the remainders where they are used.  With weights rounded
// to bf16 (relative error at most 2^-9), a row's output is then still a
// convex combination of the V rows, off by sum_i w_i d_i (v_i - o) with
// centred errors d_i; a block that holds a key with more than 1/16 of the
// row's running sum takes the remainder product as well, which bounds that
// sum's spread by 2^-9 * sqrt(1/16 / 3) * rms(v - o) = 2.8e-4 rms(v - o), and
// keeps few dominant keys (short rows, peaked scores) exact to 2^-17.  c > 0.
__device__ __forceinline__ void chunk_softmax(const f32x16_t& st, float c, float& m, float& l, float& mx, float& alpha,
                                              bool& moved, bf16x8_t (&ph)[2], bf16x8_t (&pl)[2], bool& lo) {
    // IEEE maximum (v_maximum3_f32): unlike fmaxf it needs no quieting of
    // the matrix results first; a NaN score propagates either way.
    float sm = st[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) sm = __builtin_elementwise_maximum(sm, st[r]);
    const float bm = sm == -INFINITY ? -INFINITY : sm * c;
    mx = fmaxf(mx, bm);
    moved = __any(bm > m + kTau);
    const float bw = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = moved ? fmaxf(m, bw) : m;
    alpha = m == -INFINITY ? 0.f : fast_exp2(m - mn);
    m = mn;
    l *= alpha;
    const float mref = m == -INFINITY ? 0.f : m;
    lo = __any(fast_exp2(bm - mref) * 16.f > l);
    // P rounded to bf16 two values per instruction; the block's share of
    // the running sum accumulates the rounded values with bf16 dot products
    // against ones (exact products, fp32 sums).
    float pr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(fmaf(st[r], c, -mref));
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
    bf16x2_t h2[8];
    float bs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h2[i] = __builtin_convertvector(f32x2_t{pr[2 * i], pr[2 * i + 1]}, bf16x2_t);
        bs = __builtin_amdgcn_fdot2_f32_bf16(h2[i], ones, bs, false);
    }
    ph[0] = pack8(h2[0], h2[1], h2[2], h2[3]);
    ph[1] = pack8(h2[4], h2[5], h2[6], h2[7]);
    if (lo) {
        bf16x2_t l2[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f32x2_t d = {pr[2 * i] - (float)h2[i][0], pr[2 * i + 1] - (float)h2[i][1]};
            l2[i] = __builtin_convertvector(d, bf16x2_t);
            bs = __builtin_amdgcn_fdot2_f32_bf16(l2[i], ones, bs, false);
        }
        pl[0] = pack8(l2[0], l2[1], l2[2], l2[3]);
        pl[1] = pack8(l2[4], l2[5], l2[6], l2[7]);
    }
    l += bs;
}

// One step of the chunk kernel at stage buffer offset OFF (see above).  On
// entry vf/ph hold block j - 1's V operands and P head (zeros before the
// first block); on exit, block j's.  Keys of an edge block at or past rend
// are masked (a block past the tile's last key is masked whole; its stage
// area reads as zeros).
template <int D, int OFF>
__device__ __forceinline__ void chunk_step(bool edge, const uint32_t (&ka)[CGeo<D>::KS],
                                           const uint32_t (&va)[CGeo<D>::DB][2], const bf16x8_t (&qf)[CGeo<D>::KS],
                                           f32x16_t (&acc)[CGeo<D>::DB], bf16x8_t (&vf)[CGeo<D>::DB * 2],
                                           bf16x8_t (&ph)[2], float& m, float& l, float& mx, int key0, int rend,
                                           float c, int hl) {
    using G = CGeo<D>;
    f32x16_t st;
    chunk_scores<D, OFF>(ka, qf, st);
    if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (key0 + 8 * (r >> 2) + 4 * hl + (r & 3) >= rend) st[r] = -INFINITY;
    }
    chunk_pv<D>(vf, ph, acc);
    float alpha;
    bool moved, lo;
    bf16x8_t pl[2];
    chunk_softmax(st, c, m, l, mx, alpha, moved, ph, pl, lo);
    chunk_v_reads<D, OFF>(va, vf);
    // P.V products of the previous block with the softmax's vector work
    // between them.
#pragma unroll
    for (int i = 0; i < 2 * G::DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, FD_CHUNK_VALU_PER_MFMA, 0);
    }
    lds_settle8(vf);
    if (moved) {
#pragma unroll
        for (int db = 0; db < G::DB; ++db) acc[db] *= alpha;
    }
    if (lo) chunk_pv<D>(vf, pl, acc);
}

template <int D, bool PAGED, bool FP8>
__global__ __launch_bounds__(kCT) void fd_mfma_chunk_kernel(PartialArgs a) {
    using G = CGeo<D>;
    using G8 = CGeo8<D>;
    static_assert(!FP8 || kCNS == 2, "the fp8 pipeline keeps two stages in each ring");
    constexpr int ESZ = FP8 ? 1 : 2;  // bytes per stored K/V element
    constexpr int RS = D + 4;  // padded row stride of the merge area (floats)
    constexpr int MERGEB = kCRG * (32 * RS + 3 * 32) * 4;
    constexpr int RINGB = kCNS * G::STGB + (FP8 ? 2 * G8::STGB : 0);
    constexpr int SMEMB = RINGB > MERGEB ? RINGB : MERGEB;
    __shared__ __attribute__((aligned(16))) char smem[SMEMB];

    const int s = blockIdx.x;
    const int g = blockIdx.y / a.row_blocks;
    const int rt = blockIdx.y - g * a.row_blocks;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = (int)uniform((uint32_t)(tid >> 6));
    const int rg = w % kCRG;   // row group
    const int kh = w / kCRG;   // key half
    const int hl = lane >> 5;  // lane half: G of the 32x32 layouts
    const int col = lane & 31;

    int L = a.cache_lens[b];
    L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
    int lo, hi, S;
    tile_of(a.rule, L, s, lo, hi, S);
    lo = (int)uniform((uint32_t)lo);
    hi = (int)uniform((uint32_t)hi);

    const int R = a.rows;
    const int n_rep = a.n_rep;
    const int q_len = a.q_len;
    const int p0 = rt * kChunkRows;
    const int64_t rowbase = ((int64_t)b * a.Hq + (int64_t)g * n_rep) * q_len;
    const int slots = a.rule.slots;
    const int nrows = min(kChunkRows, R - p0);

    if (s >= S) {
        for (int idx = tid; idx < nrows; idx += kCT) {
            const int p = p0 + idx;
            const int64_t row = rowbase + (int64_t)(p % n_rep) * q_len + p / n_rep;
            if (a.direct) {
                uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + row * D);
                for (int k = 0; k < D / 8; ++k) o[k] = make_uint4(0, 0, 0, 0);
                if (a.lse) a.lse[row] = -INFINITY;
            } else {
                a.m_part[row * slots + s] = -INFINITY;
                a.lse_part[row * slots + s] = -INFINITY;
            }
        }
        return;
    }

    // Keys the tile's rows can see inside [lo, hi): the last row's limit
    // bounds them all; masking starts at the first row's limit.
    const int t_first = p0 / n_rep;
    const int t_last = (p0 + nrows - 1) / n_rep;
    const int kend = max(lo, min(hi, L - q_len + t_last + 1));
    const int mask_from = max(lo, min(hi, L - q_len + t_first + 1));

    // This lane's query row (column of the 32x32 layouts).
    const int p = p0 + rg * 32 + col;
    const bool valid = p < R;
    const int t = p / n_rep;
    const int64_t mrow = rowbase + (int64_t)(p % n_rep) * q_len + t;
    const int rend = valid ? max(lo, min(hi, L - q_len + t + 1)) : lo;
    // Scores are scaled inside the exponent's FMA, which needs c > 0: a
    // negative scale moves into q (exact sign flips of bf16) and a zero scale
    // becomes a tiny positive one (all weights then equal to within 1e-26).
    const bool neg = a.qk_scale < 0.f;
    const float c = fmaxf(fabsf(a.qk_scale), 1e-30f);
    const uint32_t flip = neg ? 0x80008000u : 0u;
    bf16x8_t qf[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (valid)
            x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + mrow * D + 16 * ks + 8 * hl);
        x.x ^= flip; x.y ^= flip; x.z ^= flip; x.w ^= flip;
        qf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }

    f32x16_t acc[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m = -INFINITY, l = 0.f, mx = -INFINITY;

    const char* kt;
    const char* vt;
    int rsb;  // bytes from one key row of the head to the next
    const int32_t* tbl = nullptr;
    if constexpr (PAGED) {
        kt = static_cast<const char*>(a.k) + g * a.pages.head_stride * ESZ;
        vt = static_cast<const char*>(a.v) + g * a.pages.head_stride * ESZ;
        rsb = a.pages.row_stride * ESZ;
        tbl = a.pages.table + (int64_t)b * a.pages.max_pages;
    } else {
        const int64_t tile_row = ((int64_t)b * a.Hkv + g) * a.Lmax + lo;
        kt = static_cast<const char*>(a.k) + tile_row * (D * ESZ);
        vt = static_cast<const char*>(a.v) + tile_row * (D * ESZ);
        rsb = D * ESZ;
    }
    const int nst = (kend - lo + G::SKEYS - 1) / G::SKEYS;

    // fp8 loads: instruction n = w + k * kCW of a stage covers RPI rows of K
    // (n < NDMA) or V, in stored order.
    uint32_t dma8[FP8 ? G8::PW : 1];
    int lds8[FP8 ? G8::PW : 1], koff8[FP8 ? G8::PW : 1], isv8[FP8 ? G8::PW : 1];
    if constexpr (FP8) {
#pragma unroll
        for (int k = 0; k < G8::PW; ++k) {
            const int n = w + k * kCW;
            isv8[k] = n / G8::NDMA;
            const int i = n - isv8[k] * G8::NDMA;
            koff8[k] = i * G8::RPI;
            lds8[k] = isv8[k] * G8::TENB + i * 1024;
            dma8[k] = (uint32_t)((PAGED ? lane / G8::CH : koff8[k] + lane / G8::CH) * rsb + (lane % G8::CH) * 16);
        }
    }

    // Load instruction k of this wave fills RPI rows of block bb of a stage;
    // lane l takes row l / CH, global chunk (l % CH) ^ swizzle.
    uint32_t dma_off[G::DPW];
    int lds_off[G::DPW];
    int koff[G::DPW];
#pragma unroll
    for (int k = 0; k < G::DPW; ++k) {
        const int n = w + k * kCW;
        const int bb = n / G::IPB;
        const int i = n - bb * G::IPB;
        const int r = i * G::RPI + lane / G::CH;
        const int cg = (lane % G::CH) ^ cswf<G::CH>(r);
        koff[k] = bb * kCBK + i * G::RPI;
        dma_off[k] = (uint32_t)((PAGED ? lane / G::CH : koff[k] + lane / G::CH) * rsb + cg * 16);
        lds_off[k] = bb * G::BLKB + i * 1024;
    }

    // Lane-constant LDS addresses of this wave's operands in stage 0; other
    // stages and the second 16-key step add compile-time offsets.
    uint32_t ka[G::KS];
    uint32_t va[G::DB][2];
    {
        const uint32_t base = lds_addr(smem) + kh * G::BLKB;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) ka[ks] = base + cswz<D>(col, 2 * ks + hl);
        const int g16 = lane >> 4;
        const int i16 = lane & 15;
        const int q4 = i16 & 3;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                va[db][t] = base + G::SKB * G::BLKB +
                            cswz<D>(8 * t + 4 * hl + (i16 >> 2), (32 * db + 16 * (g16 & 1)) / 8 + (q4 >> 1)) +
                            8 * (q4 & 1);
    }

    char* ring8 = smem + kCNS * G::STGB;  // fp8: the stored-row ring
    if constexpr (FP8) {
        // fp8 stages 0 and 1 in flight; stage 0 dequantised into bf16 slot 0.
        chunk_stage8_at<D, PAGED>(a.pages, tbl, kt, vt, lo, kend, 0, rsb, ring8, dma8, lds8, koff8, isv8);
        chunk_stage8_at<D, PAGED>(a.pages, tbl, kt, vt, lo, kend, 1, rsb, ring8 + G8::STGB, dma8, lds8, koff8,
                                  isv8);
        wait_vmcnt_le<G8::PW>();
        __syncthreads();
        chunk_dequant_stage<D>(ring8, smem, tid);
    } else {
#pragma unroll
        for (int j = 0; j < kCNS - 1; ++j)
            chunk_stage_at<D, PAGED>(a.pages, tbl, kt, vt, lo, kend, j, rsb, smem + j * G::STGB, dma_off, lds_off,
                                     koff);
    }

    // Stage j lives in ring slot j % kCNS; unrolling by kCNS makes the slot,
    // and so every LDS offset, a compile-time constant.  A wave whose block
    // lies past kend masks it whole (its stage area reads as zeros).
    bf16x8_t vf[G::DB * 2], ph[2];
#pragma unroll
    for (int i = 0; i < G::DB * 2; ++i) vf[i] = bf16x8_t{};
    ph[0] = ph[1] = bf16x8_t{};
    for (int j0 = 0; j0 < nst; j0 += kCNS) {
#pragma unroll
        for (int u = 0; u < kCNS; ++u) {
            const int j = j0 + u;
            if (j >= nst) break;
            if constexpr (FP8) {
                // Own loads of fp8 stage j + 1 landed; after the barrier
                // everyone's have, bf16 slot u holds stage j, slot 1 - u and
                // fp8 slot u are free.
                wait_vmcnt_le<0>();
                __syncthreads();
                chunk_stage8_at<D, PAGED>(a.pages, tbl, kt, vt, lo, kend, j + 2, rsb, ring8 + u * G8::STGB, dma8,
                                          lds8, koff8, isv8);
                if (j + 1 < nst)
                    chunk_dequant_stage<D>(ring8 + (1 - u) * G8::STGB, smem + (1 - u) * G::STGB, tid);
            } else {
                wait_vmcnt_le<(kCNS - 1) * 2 * G::DPW>();  // this wave's loads of stage j
                __syncthreads();                           // everyone's; stage j - 1 is free
                chunk_stage_at<D, PAGED>(a.pages, tbl, kt, vt, lo, kend, j + kCNS - 1, rsb,
                                         smem + ((u + kCNS - 1) % kCNS) * G::STGB, dma_off, lds_off, koff);
            }
            const int key0 = lo + j * G::SKEYS + kh * kCBK;
            const bool edge = key0 + kCBK > mask_from;
            if (u == 0) chunk_step<D, 0>(edge, ka, va, qf, acc, vf, ph, m, l, mx, key0, rend, c, hl);
            if (u == 1) chunk_step<D, G::STGB>(edge, ka, va, qf, acc, vf, ph, m, l, mx, key0, rend, c, hl);
            if constexpr (kCNS > 2)
                if (u == 2) chunk_step<D, 2 * G::STGB>(edge, ka, va, qf, acc, vf, ph, m, l, mx, key0, rend, c, hl);
        }
    }
    chunk_pv<D>(vf, ph, acc);
    wait_vmcnt_le<0>();

    // Per-row totals over the two lane halves; then merge the key halves.
    l += __shfl_xor(l, 32);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    __syncthreads();  // the ring is free
    float* sm_acc = reinterpret_cast<float*>(smem);  // [kCRG][32][RS]
    float* sm_m = sm_acc + kCRG * 32 * RS;           // [kCRG][32]
    float* sm_l = sm_m + kCRG * 32;
    float* sm_x = sm_l + kCRG * 32;
    if (kh == 1) {
        float* o = sm_acc + (rg * 32 + col) * RS;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4)
                *reinterpret_cast<f32x4_t*>(o + 32 * db + 8 * a4 + 4 * hl) =
                    f32x4_t{acc[db][4 * a4], acc[db][4 * a4 + 1], acc[db][4 * a4 + 2], acc[db][4 * a4 + 3]};
        if (hl == 0) {
            sm_m[rg * 32 + col] = m;
            sm_l[rg * 32 + col] = l;
            sm_x[rg * 32 + col] = mx;
        }
    }
    __syncthreads();
    if (kh == 1 || !valid) return;
    const float m2 = sm_m[rg * 32 + col];
    const float M = fmaxf(m, m2);
    const float f1 = m == -INFINITY ? 0.f : fast_exp2(m - M);
    const float f2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - M);
    const float den = l * f1 + sm_l[rg * 32 + col] * f2;
    const float X = fmaxf(mx, sm_x[rg * 32 + col]);
    const bool empty = M == -INFINITY;
    // fp8: V was dequantised without its scale
    const float inv = empty ? 0.f : (FP8 ? a.v_scale : 1.f) / den;
    const float lse_v = empty ? -INFINITY : (M + log2f(den)) * kLn2;
    const float* o2 = sm_acc + (rg * 32 + col) * RS;
    if (a.direct) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + mrow * D;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d = 32 * db + 8 * a4 + 4 * hl;
                const f32x4_t y = *reinterpret_cast<const f32x4_t*>(o2 + d);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (acc[db][4 * a4 + e] * f1 + y[e] * f2) * inv;
                uint2 packed;
                packed.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                packed.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                *reinterpret_cast<uint2*>(o + d) = packed;
            }
        if (hl == 0 && a.lse) a.lse[mrow] = lse_v;
    } else {
        if (!empty) {
            float* o = a.o_part + (mrow * slots + s) * D;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d = 32 * db + 8 * a4 + 4 * hl;
                    const f32x4_t y = *reinterpret_cast<const f32x4_t*>(o2 + d);
                    f32x4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (acc[db][4 * a4 + e] * f1 + y[e] * f2) * inv;
                    *reinterpret_cast<f32x4_t*>(o + d) = v;
                }
        }
        if (hl == 0) {
            a.m_part[mrow * slots + s] = empty ? -INFINITY : X * kLn2;
            a.lse_part[mrow * slots + s] = lse_v;
        }
    }
}

template <int D, bool PAGED>
void launch_chunk_p(int batch, const PartialArgs& a, hipStream_t stream) {
    dim3 grid(a.rule.slots, a.Hkv * a.row_blocks, batch), block(kCT);
    if (a.kv_fp8)
        hipLaunchKernelGGL((fd_mfma_chunk_kernel<D, PAGED, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((fd_mfma_chunk_kernel<D, PAGED, false>), grid, block, 0, stream, a);
}

template <int D>
void launch_chunk(int batch, const PartialArgs& a, hipStream_t stream) {
    if (a.pages.table != nullptr)
        launch_chunk_p<D, true>(batch, a, stream);
    else
        launch_chunk_p<D, false>(batch, a, stream);
}

template <int D, int NB, bool FP8>
void launch_nb_kv(int batch, const PartialArgs& a, hipStream_t stream) {
    dim3 grid(a.Hkv, a.rule.slots, batch), block(FP8 ? 64 * kMW8 : kMT);
    const bool paged = a.pages.table != nullptr;
    if (a.q_len > 1) {
        if (paged)
            hipLaunchKernelGGL((fd_mfma_partial_kernel<D, NB, true, true, FP8>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((fd_mfma_partial_kernel<D, NB, true, false, FP8>), grid, block, 0, stream, a);
    } else {
        if (paged)
            hipLaunchKernelGGL((fd_mfma_partial_kernel<D, NB, false, true, FP8>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((fd_mfma_partial_kernel<D, NB, false, false, FP8>), grid, block, 0, stream, a);
    }
}

template <int D, int NB>
void launch_nb(int batch, const PartialArgs& a, hipStream_t stream) {
    if (a.kv_fp8)
        launch_nb_kv<D, NB, true>(batch, a, stream);
    else
        launch_nb_kv<D, NB, false>(batch, a, stream);
}

}  // namespace

hipError_t launch_partials_mfma(int head_dim, int batch, const PartialArgs& a, hipStream_t stream) {
    if (a.rows > 32) {
        if (head_dim == 64)
            launch_chunk<64>(batch, a, stream);
        else
            launch_chunk<128>(batch, a, stream);
        return hipGetLastError();
    }
    const bool two = a.rows > 16;
    if (head_dim == 64) {
        if (two) launch_nb<64, 2>(batch, a, stream);
        else launch_nb<64, 1>(batch, a, stream);
    } else {
        if (two) launch_nb<128, 2>(batch, a, stream);
        else launch_nb<128, 1>(batch, a, stream);
    }
    return hipGetLastError();
}

}  // namespace fdk
