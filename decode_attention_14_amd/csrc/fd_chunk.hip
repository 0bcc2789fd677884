// fd_chunk.hip -- split-KV partial kernel on the matrix cores for chunked
// prefill on gfx950 (CDNA4): bf16 queries over bf16, FP8 E4M3 or INT8 caches,
// contiguous or paged.
//
// It serves row groups of more than 32 query rows per KV head (page
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
//                share of a row's weight (see pipe_needs_remainder).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fd_device.h"
#include "fd_internal.h"
#include "fd_mfma_common.h"

#ifndef FD_WG_TIMELINE
#define FD_WG_TIMELINE 0
#endif

// Workgroup timeline of fd_mfma_chunk_kernel (a diagnostic build only,
// FD_WG_TIMELINE=1, laid out as the decode kernel's): workgroup i of the last
// launch (dispatch order, i < 4096) leaves at [i * 16] its start, the landing
// of its first stage, each wave's exit from the stage loop (8 waves), its end
// and its XCD, in the 100 MHz s_memrealtime clock, and at [12], [13] the
// shader clock (s_memtime) at the first stage and at wave 0's loop exit.
#if FD_WG_TIMELINE
__device__ uint64_t fd_chunk_timeline[4096 * 16];
extern "C" int fd_debug_chunk_timeline(void* host_dst, uint64_t bytes) {
    if (bytes > sizeof(fd_chunk_timeline)) bytes = sizeof(fd_chunk_timeline);
    return (int)hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(fd_chunk_timeline), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

namespace fdk {
namespace {

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
template <class G>
__device__ __forceinline__ void chunk_load_stage(const char* kt, const char* vt, int left, int off, char* dst,
                                                 const uint32_t* dma_off, const int* lds_off) {
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
template <class G, bool PAGED>
__device__ __forceinline__ void chunk_stage_at(const PagedKV& pk, const int32_t* tbl, const char* kt, const char* vt,
                                               int lo, int kend, int j, int rsb, char* dst, const uint32_t* dma_off,
                                               const int* lds_off, const int* koff) {
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
        chunk_load_stage<G>(kt, vt, (kend - lo) * G::ROWB - off, off, dst, dma_off, lds_off);
    }
}

// Caches of one-byte codes (FP8 E4M3 or INT8) in the chunk kernel: each
// stage's rows of codes (D bytes, stored order) stream into a second
// two-stage ring, and the workgroup dequantises
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
    static_assert((2 * NDMA) % kCW == 0 && PW >= 1 && STGB % (8 * kCT) == 0, "even split");
};

// Start this wave's loads of code stage j into dst (see chunk_stage_at).
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

// Dequantise a landed code stage (src, format KV) into the bf16 stage layout
// (dst), exactly (see codes_to_bf16): thread t converts the 8-byte code units
// t, t + kCT, ... (8 codes each, one 16-byte bf16 chunk) through lds_load_b64
// / lds_write_b128, so the stage loads still in flight are not waited for.
// The 8 lanes of a write cycle (8 lanes over 128 bytes of banks) convert 8
// consecutive units of one code row, one aligned group of 8 bf16 chunks, which
// cswz keeps on 8 distinct chunks modulo 8.
template <int D, int KV>
__device__ __forceinline__ void chunk_dequant_stage(const char* src, char* dst, int tid) {
    using G = CGeo<D>;
    using G8 = CGeo8<D>;
    constexpr int NU = G8::STGB / 8 / kCT;  // units per thread
    constexpr int UPT = G8::TENB / 8;       // units per tensor
    constexpr int UPR = G8::ROWB / 8;       // units per code row
    u32x2_t x[NU];
#pragma unroll
    for (int n = 0; n < NU; ++n) x[n] = lds_load_b64(lds_addr(src + (n * kCT + tid) * 8));
#pragma unroll
    for (int n = 0; n < NU; ++n) {
        const int q = n * kCT + tid;
        const int tsr = q / UPT;  // 0: K, 1: V
        const int rem = q - tsr * UPT;
        const int r = rem / UPR;
        const int c = rem - r * UPR;  // codes of dims 8 c .. 8 c + 7
        uint32_t bw[4];
        codes_to_bf16<KV>(x[n][0], bw[0], bw[1]);
        codes_to_bf16<KV>(x[n][1], bw[2], bw[3]);
        char* o = dst + tsr * G::SKB * G::BLKB + (r / kCBK) * G::BLKB;
        lds_write_b128(o + cswz<D>(r % kCBK, c), u32x4_t{bw[0], bw[1], bw[2], bw[3]});
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
// The instruction's offset field holds 16 bits: a larger offset (later
// stages of a deep ring) moves its high part into the address.
template <int OFF>
__device__ __forceinline__ bf16x4_t tr_read_at(uint32_t addr) {
    static_assert(OFF >= 0, "ds offset");
    constexpr int HI = OFF & ~0x7fff;
    bf16x4_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr + HI), "i"(OFF - HI));
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

// A block's V operands (stage buffer at offset OFF from the lane addresses
// va) through transposed reads, waited for.
template <int D, int OFF>
__device__ __forceinline__ void chunk_v_reads_wait(const uint32_t (&va)[CGeo<D>::DB][2],
                                                   bf16x8_t (&vf)[CGeo<D>::DB * 2]) {
    using G = CGeo<D>;
    constexpr int K2 = 16 * G::ROWB;  // 16 rows further down the block
    uint32_t a[2 * G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
        a[2 * db] = va[db][0];
        a[2 * db + 1] = va[db][1];
    }
    bf16x4_t x[2 * G::DB], y[2 * G::DB];
    tr_read_wait<OFF>(a, x);
    tr_read_wait<OFF + K2>(a, y);
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
        vf[db * 2] = __builtin_shufflevector(x[2 * db], x[2 * db + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        vf[db * 2 + 1] = __builtin_shufflevector(y[2 * db], y[2 * db + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
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


__device__ __forceinline__ bf16x8_t pack8(bf16x2_t a, bf16x2_t b, bf16x2_t c, bf16x2_t d) {
    const bf16x4_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4_t cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Online softmax of a block, in base 2 with a lazily moved reference max m
// (moved when a key passes it by more than kTau, so the accumulators are
// rescaled rarely), the exact running max tracked apart for the partial's m.
//
// The running sum l adds the weights that the products actually use: the
// bf16 heads, plus the remainders where they are used.  With weights rounded
// to bf16 (relative error at most 2^-9), a row's output is then still a
// convex combination of the V rows, off by sum_i w_i d_i (v_i - o) with
// centred errors d_i; a block that holds a key with more than 1/16 of the
// row's running sum takes the remainder product as well, which bounds that
// sum's spread by 2^-9 * sqrt(1/16 / 3) * rms(v - o) = 2.8e-4 rms(v - o), and
// keeps few dominant keys (short rows, peaked scores) exact to 2^-17.  c > 0.

// max and sum of x over lanes i and i ^ 32 (the two halves of a 32x32 tile
// hold the same rows); the swap hands every lane the pair (x of the low
// lane, x of the high lane), so both lanes get the same bits.
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Running statistics of one lane's query row in the pipelined kernel: the
// reference max m (scaled scores, log2 units; -inf before the row's first
// visible key), the exponent offset mref (m, or 0 while m is -inf), thr, the
// raw score above which a key moves the reference (m + kTau in raw units,
// -inf while m is -inf), the running sum l of the weights the products use
// (this lane's keys), and the running max xr of this lane's raw scores.
struct RowStat {
    float m, mref, thr, l, xr;
};

// Weights of a block against the offset mref, in place: the scores st become
// 2^(c s - mref); their bf16 heads ph, and l = l0 plus the heads (bf16 dot
// products against ones: exact products, fp32 sums).
__device__ __forceinline__ void pipe_weights(f32x16_t& st, float c, float mref, float l0, bf16x8_t (&ph)[2],
                                             float& l) {
    f32x16_t& pr = st;
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(fmaf(st[r], c, -mref));
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
    bf16x2_t h2[8];
    float bs = l0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h2[i] = __builtin_convertvector(f32x2_t{pr[2 * i], pr[2 * i + 1]}, bf16x2_t);
        bs = __builtin_amdgcn_fdot2_f32_bf16(h2[i], ones, bs, false);
    }
    ph[0] = pack8(h2[0], h2[1], h2[2], h2[3]);
    ph[1] = pack8(h2[4], h2[5], h2[6], h2[7]);
    l = bs;
}

// Whether the block also needs its remainder (pipe_remainder): whether some
// row's largest weight in the block, 2^(c sm - mref), passes 1/16 of the
// row's running sum, this block's heads included (both lane halves).
__device__ __forceinline__ bool pipe_needs_remainder(float sm, float c, const RowStat& rs) {
    const float pm = fast_exp2(fmaf(sm, c, -rs.mref));
    return __any(pm * 16.f > xor32_sum(rs.l));
}

// The common path of one block's online softmax comes in two halves without
// branches, so that the scheduler can place each between matrix
// instructions: the first beside the previous block's P.V product, the
// second beside the next block's score product.
//
// First half, in place on the block's (masked) scores st: the block's raw
// max sm (also folded into xr), whether it moves the reference (some row's
// max passes thr), the exponents c s - mref, and the weights of the first
// eight of them.
__device__ __forceinline__ void pipe_softmax1(f32x16_t& st, float c, RowStat& rs, float& sm, bool& moved) {
    // IEEE maximum (v_maximum3_f32): no quieting of the matrix results.
    sm = st[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) sm = __builtin_elementwise_maximum(sm, st[r]);
    rs.xr = __builtin_elementwise_maximum(rs.xr, sm);
    moved = __any(sm > rs.thr);
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = fmaf(st[r], c, -rs.mref);
#pragma unroll
    for (int r = 0; r < 8; ++r) st[r] = fast_exp2(st[r]);
}

// Second half: the other eight weights (st then holds all sixteen), their
// bf16 heads ph, the running sum (l0 keeps it from before the block, for a
// reference move) and the remainder test.  When the reference moves, the
// caller recomputes the weights (pipe_move).
__device__ __forceinline__ void pipe_softmax2(f32x16_t& st, float c, RowStat& rs, float sm, float& l0,
                                              bf16x8_t (&ph)[2], bool& lo) {
#pragma unroll
    for (int r = 8; r < 16; ++r) st[r] = fast_exp2(st[r]);
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
    bf16x2_t h2[8];
    l0 = rs.l;
    float bs = l0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h2[i] = __builtin_convertvector(f32x2_t{st[2 * i], st[2 * i + 1]}, bf16x2_t);
        bs = __builtin_amdgcn_fdot2_f32_bf16(h2[i], ones, bs, false);
    }
    ph[0] = pack8(h2[0], h2[1], h2[2], h2[3]);
    ph[1] = pack8(h2[4], h2[5], h2[6], h2[7]);
    rs.l = bs;
    lo = pipe_needs_remainder(sm, c, rs);
}

// The rare path of a block whose max moved the reference: the new reference
// is the larger of the old one and the row's block max (both lane halves);
// alpha is the factor the sum and the accumulators owe (0 after -inf).  The
// weights, the sum and the remainder test are redone against it from the
// block's scores st, in place (recomputed by the caller: the common path's
// weights may have overflowed, and keeping the scores alive would cost
// registers).
__device__ __forceinline__ float pipe_move(f32x16_t& st, float c, float cinv, float sm, float l0, RowStat& rs,
                                           bf16x8_t (&ph)[2], bool& lo) {
    const float bw = xor32_max(sm * c);
    const float mn = fmaxf(rs.m, bw);
    const float alpha = rs.m == -INFINITY ? 0.f : fast_exp2(rs.m - mn);
    rs.m = mn;
    rs.mref = mn == -INFINITY ? 0.f : mn;
    rs.thr = mn == -INFINITY ? -INFINITY : (mn + kTau) * cinv;
    pipe_weights(st, c, rs.mref, l0 * alpha, ph, rs.l);
    lo = pipe_needs_remainder(sm, c, rs);
    return alpha;
}

// The bf16 remainder pl = pr - ph of a block's weights, and its share of the
// running sum (taken when pipe_needs_remainder says so).
__device__ __forceinline__ void pipe_remainder(const f32x16_t& pr, const bf16x8_t (&ph)[2], bf16x8_t (&pl)[2],
                                               float& l) {
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
    bf16x2_t l2[8];
    float bs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bf16x8_t& h = ph[i / 4];
        const f32x2_t d = {pr[2 * i] - (float)h[2 * (i % 4)], pr[2 * i + 1] - (float)h[2 * (i % 4) + 1]};
        l2[i] = __builtin_convertvector(d, bf16x2_t);
        bs = __builtin_amdgcn_fdot2_f32_bf16(l2[i], ones, bs, false);
    }
    pl[0] = pack8(l2[0], l2[1], l2[2], l2[3]);
    pl[1] = pack8(l2[4], l2[5], l2[6], l2[7]);
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
                                           bf16x8_t (&ph)[2], RowStat& rs, int key0, int rend, float c, float cinv,
                                           int hl) {
    using G = CGeo<D>;
    f32x16_t st;
    chunk_scores<D, OFF>(ka, qf, st);
    if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (key0 + 8 * (r >> 2) + 4 * hl + (r & 3) >= rend) st[r] = -INFINITY;
    }
    chunk_pv<D>(vf, ph, acc);
    // The common path of this block's softmax (as the pipelined kernel's:
    // the block max, the move test, the weights against the current
    // reference, the sum and the remainder test); the scores stay for a
    // reference move.  IEEE maximum (v_maximum3_f32): no quieting of the
    // matrix results.
    float sm = st[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) sm = __builtin_elementwise_maximum(sm, st[r]);
    rs.xr = __builtin_elementwise_maximum(rs.xr, sm);
    const bool moved = __any(sm > rs.thr);
    f32x16_t pr = st;
    const float l0 = rs.l;
    pipe_weights(pr, c, rs.mref, l0, ph, rs.l);
    bool lo = pipe_needs_remainder(sm, c, rs);
    // P.V products of the previous block with the softmax's vector work
    // between them.
#pragma unroll
    for (int i = 0; i < 2 * G::DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, FD_CHUNK_VALU_PER_MFMA, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // The rare paths read their inputs through register barriers inside the
    // branch, so the compiler cannot compute them on every block instead.
    if (moved) {
        f32x16_t sc = st;
        float smv = sm, l0v = l0;
        asm volatile("" : "+v"(sc), "+v"(smv), "+v"(l0v));
        const float al = pipe_move(sc, c, cinv, smv, l0v, rs, ph, lo);
        pr = sc;
#pragma unroll
        for (int db = 0; db < G::DB; ++db) acc[db] *= al;
    }
    bf16x8_t pl[2];
    if (lo) {
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(pr[r]));
        pipe_remainder(pr, ph, pl, rs.l);
    }
    // This block's V operands (the products above have taken the previous ones).
    chunk_v_reads_wait<D, OFF>(va, vf);
    if (lo) chunk_pv<D>(vf, pl, acc);
}

template <int D, bool PAGED, int KV>
__global__ __launch_bounds__(kCT) void fd_mfma_chunk8_kernel(PartialArgs a) {
    using G = CGeo<D>;
    using G8 = CGeo8<D>;
    constexpr bool C8 = KV != kKvBf16;  // one-byte codes
    static_assert(!C8 || kCNS == 2, "the code pipeline keeps two stages in each ring");
    constexpr int ESZ = C8 ? 1 : 2;  // bytes per stored K/V element
    constexpr int RS = D + 4;  // padded row stride of the merge area (floats)
    constexpr int MERGEB = kCRG * (32 * RS + 3 * 32) * 4;
    constexpr int RINGB = kCNS * G::STGB + (C8 ? 2 * G8::STGB : 0);
    constexpr int SMEMB = RINGB > MERGEB ? RINGB : MERGEB;
    __shared__ __attribute__((aligned(16))) char smem[SMEMB];

    // Workgroups are dispatched round-robin over the 8 XCDs in linear order
    // (x fastest).  Along x (one sequence: KV heads x tiles x row tiles) the
    // logical index puts the row tiles of one (KV head, tile) next to each
    // other and, when the row length is a multiple of 8, gives each XCD a
    // contiguous range of it, so row tiles that read the same K/V stages
    // share one L2.
    const uint32_t nx = gridDim.x;
    uint32_t li = blockIdx.x;
    if ((nx & 7u) == 0) li = (li & 7u) * (nx >> 3) + (li >> 3);
    const int rt = (int)(li % (uint32_t)a.row_blocks);
    li /= (uint32_t)a.row_blocks;
    const int s = (int)(li % (uint32_t)a.rule.slots);
    const int g = (int)(li / (uint32_t)a.rule.slots);
    const int b = blockIdx.y;
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
    RowStat rs = {-INFINITY, 0.f, -INFINITY, 0.f, -INFINITY};
    const float cinv = __uint_as_float(uniform(__float_as_uint(1.f / c)));

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

    // Code loads: instruction n = w + k * kCW of a stage covers RPI rows of K
    // (n < NDMA) or V, in stored order.
    uint32_t dma8[C8 ? G8::PW : 1];
    int lds8[C8 ? G8::PW : 1], koff8[C8 ? G8::PW : 1], isv8[C8 ? G8::PW : 1];
    if constexpr (C8) {
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

    char* ring8 = smem + kCNS * G::STGB;  // codes: the stored-row ring
    if constexpr (C8) {
        // Code stages 0 and 1 in flight; stage 0 dequantised into bf16 slot 0.
        chunk_stage8_at<D, PAGED>(a.pages, tbl, kt, vt, lo, kend, 0, rsb, ring8, dma8, lds8, koff8, isv8);
        chunk_stage8_at<D, PAGED>(a.pages, tbl, kt, vt, lo, kend, 1, rsb, ring8 + G8::STGB, dma8, lds8, koff8,
                                  isv8);
        wait_vmcnt_le<G8::PW>();
        __syncthreads();
        chunk_dequant_stage<D, KV>(ring8, smem, tid);
    } else {
#pragma unroll
        for (int j = 0; j < kCNS - 1; ++j)
            chunk_stage_at<G, PAGED>(a.pages, tbl, kt, vt, lo, kend, j, rsb, smem + j * G::STGB, dma_off, lds_off,
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
            if constexpr (C8) {
                // Own loads of code stage j + 1 landed; after the barrier
                // everyone's have, bf16 slot u holds stage j, slot 1 - u and
                // code slot u are free.
                wait_vmcnt_le<0>();
                __syncthreads();
                chunk_stage8_at<D, PAGED>(a.pages, tbl, kt, vt, lo, kend, j + 2, rsb, ring8 + u * G8::STGB, dma8,
                                          lds8, koff8, isv8);
                if (j + 1 < nst)
                    chunk_dequant_stage<D, KV>(ring8 + (1 - u) * G8::STGB, smem + (1 - u) * G::STGB, tid);
            } else {
                wait_vmcnt_le<(kCNS - 1) * 2 * G::DPW>();  // this wave's loads of stage j
                __syncthreads();                           // everyone's; stage j - 1 is free
                chunk_stage_at<G, PAGED>(a.pages, tbl, kt, vt, lo, kend, j + kCNS - 1, rsb,
                                         smem + ((u + kCNS - 1) % kCNS) * G::STGB, dma_off, lds_off, koff);
            }
            const int key0 = lo + j * G::SKEYS + kh * kCBK;
            const bool edge = key0 + kCBK > mask_from;
            if (u == 0) chunk_step<D, 0>(edge, ka, va, qf, acc, vf, ph, rs, key0, rend, c, cinv, hl);
            if (u == 1) chunk_step<D, G::STGB>(edge, ka, va, qf, acc, vf, ph, rs, key0, rend, c, cinv, hl);
            if constexpr (kCNS > 2)
                if (u == 2) chunk_step<D, 2 * G::STGB>(edge, ka, va, qf, acc, vf, ph, rs, key0, rend, c, cinv, hl);
        }
    }
    chunk_pv<D>(vf, ph, acc);
    wait_vmcnt_le<0>();

    // Per-row totals over the two lane halves; then merge the key halves.
    const float m = rs.m;
    const float l = xor32_sum(rs.l);
    const float mx = xor32_max(rs.xr) * c;
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
    // codes: V was dequantised without its scale
    const float inv = empty ? 0.f : (C8 ? a.v_scale : 1.f) / den;
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

// ---------------------------------------------------------------------------
// bf16 caches: the software-pipelined chunk kernel (fd_mfma_chunk_kernel).
//
// The same work split as fd_mfma_chunk8_kernel -- eight waves, four row
// groups of 32 rows times two key halves, 64-key stages of which wave (rg,
// kh) takes block kh, the halves merged through LDS at the end -- but inside
// a wave the work of consecutive blocks overlaps.  Step j of a wave issues
// block j + 1's score product beside the second half of block j's softmax,
// then block j's P.V product beside the first half of block j + 1's softmax,
// so that vector work sits between both groups of matrix instructions (two
// score tiles in flight).  K operands are read a step ahead of their
// product and V operands a step ahead of theirs; the ring has four stages,
// and after the barrier of step t, which shows stage t + 2 landed for every
// wave (each waits for its own loads before it) and every wave done with
// step t - 1, the loads of stage t + 3 start into the slot of stage t - 1.
// The barrier is a bare s_barrier between compiler memory barriers: a
// workgroup fence would also wait for every load in flight.  K stages share
// one LDS array, read with plain 16-byte loads; each V stage has an array of
// its own, read with the transposing-load builtin, so that the compiler
// sees which buffer-to-LDS loads a read depends on and waits for exactly
// those.

constexpr int kPT = 512;               // threads per workgroup
constexpr int kPW = kPT / 64;          // waves
constexpr int kPRG = 4;                // row groups of 32 rows
static_assert(kPRG * 32 == kChunkTileRows, "row tile of the chunk kernel");
constexpr int kPNS = 4;  // ring stages
// Vector instructions the scheduler places after each matrix instruction (a
// probe kernel hides about four 4-cycle vector instructions under each
// 32x32x16 matrix instruction of a SIMD).
#ifndef FD_PIPE_VALU_PER_MFMA
#define FD_PIPE_VALU_PER_MFMA 4
#endif

template <int D>
struct PGeo {
    static constexpr int ROWB = 2 * D;
    static constexpr int CH = ROWB / 16;            // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;             // rows per 1 KiB load instruction
    static constexpr int IPB = kCBK / RPI;          // load instructions per block per tensor
    static constexpr int BLKB = kCBK * ROWB;        // bytes per block per tensor
    static constexpr int SKB = 2;                   // blocks per stage (key halves)
    static constexpr int SKEYS = SKB * kCBK;        // keys per stage
    static constexpr int STGB = SKB * BLKB;         // bytes per stage per tensor
    static constexpr int NDMA = SKB * IPB;          // load instructions per tensor per stage
    static constexpr int DPW = NDMA / kPW;          // per wave, per tensor
    static constexpr int PER = 2 * DPW;             // loads per wave per stage
    static constexpr int KS = D / 16;               // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;               // 32-dim blocks of O^T
    static_assert(NDMA % kPW == 0 && DPW >= 1, "stage loads split evenly over the waves");
};

// Page ids of this wave's loads of stage j (wave-uniform scalar loads), or
// -1 past kend.  They are read at the end of the step before the stage's
// loads: a scalar load in flight makes the compiler wait for every LDS read
// at the next LDS wait, so it is issued after the step's K-operand waits and
// consumed after the next barrier, when nothing else is left in flight.
template <int D, bool PAGED>
__device__ __forceinline__ void pipe_pages(const PagedKV& pk, const int32_t* tbl, int lo, int kend, int j,
                                           const int* koff, int* pg) {
    if constexpr (PAGED) {
#pragma unroll
        for (int k = 0; k < PGeo<D>::DPW; ++k) pg[k] = page_at(pk, tbl, lo + j * PGeo<D>::SKEYS + koff[k], kend);
    }
}

// Start this wave's loads of stage j of the tile [lo, kend): K rows into dk,
// V rows into dv (the stage's slots of the two rings; see chunk_stage_at).
// A paged cache's page ids of this wave's loads come in pg (read a step
// ahead, pipe_pages).
template <int D, bool PAGED>
__device__ __forceinline__ void pipe_stage(const PagedKV& pk, const int* pg, const char* kt, const char* vt,
                                           int lo, int kend, int j, int rsb, char* dk, char* dv,
                                           const uint32_t* dma_off, const int* lds_off, const int* koff) {
    using G = PGeo<D>;
#pragma unroll
    for (int k = 0; k < G::DPW; ++k) {
        __amdgpu_buffer_rsrc_t rk, rv;
        uint32_t off_lane = dma_off[k];
        if constexpr (PAGED) {
            int64_t off;
            const uint32_t n = paged_rows_in(pk, pg[k], lo + j * G::SKEYS + koff[k], G::RPI, kend, rsb, G::ROWB,
                                             &off);
            rk = tile_rsrc(kt + off * 2, n);
            rv = tile_rsrc(vt + off * 2, n);
        } else {
            const int off = j * G::SKEYS * G::ROWB;
            const int left = (kend - lo) * G::ROWB - off;
            const uint32_t n = left > 0 ? (uint32_t)left : 0u;
            rk = tile_rsrc(kt + off, n);
            rv = tile_rsrc(vt + off, n);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(dk + lds_off[k]), 16, off_lane, 0, 0, FD_LOAD_AUX);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(dv + lds_off[k]), 16, off_lane, 0, 0, FD_LOAD_AUX);
    }
}

// Workgroup barrier without a memory fence: the compiler keeps memory
// accesses on their side of it; the waits for loads are the caller's.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most n (0 or 1, wave-uniform) stages' loads of this wave are
// in flight, PER loads each.
template <int PER>
__device__ __forceinline__ void wait_stages(int n) {
    if (n >= 1)
        wait_vmcnt_le<PER>();
    else
        wait_vmcnt_le<0>();
}


// Transposed LDS read (ds_read_b64_tr_b16, lane layout as tr_read_wait) at
// byte offset off of the V stage array sv.
__device__ __forceinline__ bf16x4_t v_tr_read(const char* sv, uint32_t off) {
    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(sv + off));
    return __builtin_bit_cast(bf16x4_t, r);
}

// A block's V operands from the V stage array sv (lane offsets va, which
// include the wave's block).
template <int D>
__device__ __forceinline__ void pipe_v_reads(const char* sv, const uint32_t (&va)[PGeo<D>::DB][2],
                                             bf16x8_t (&vf)[PGeo<D>::DB * 2]) {
    constexpr int K2 = 16 * PGeo<D>::ROWB;  // 16 rows further down the block
#pragma unroll
    for (int db = 0; db < PGeo<D>::DB; ++db) {
        const bf16x4_t a0 = v_tr_read(sv, va[db][0]);
        const bf16x4_t a1 = v_tr_read(sv, va[db][1]);
        const bf16x4_t b0 = v_tr_read(sv, va[db][0] + K2);
        const bf16x4_t b1 = v_tr_read(sv, va[db][1] + K2);
        vf[db * 2] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        vf[db * 2 + 1] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// K operands of a block at K-region offset OFF (LDS addresses ka).
template <int D, int OFF>
__device__ __forceinline__ void pipe_k_reads(const uint32_t (&ka)[PGeo<D>::KS], bf16x8_t (&kf)[PGeo<D>::KS]) {
#pragma unroll
    for (int ks = 0; ks < PGeo<D>::KS; ++ks) kf[ks] = lds_b128<OFF>(ka[ks]);
}

// Scores of a block, S^T = K Q^T, from K operands kf.
template <int D>
__device__ __forceinline__ void pipe_scores(const bf16x8_t (&kf)[PGeo<D>::KS], const bf16x8_t (&qf)[PGeo<D>::KS],
                                            f32x16_t& st) {
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < PGeo<D>::KS; ++ks) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], st, 0, 0, 0);
}

// Keys of a block at or past rend (this lane's row) get score -inf.
__device__ __forceinline__ void pipe_mask(f32x16_t& st, int key0, int rend, int hl) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
        if (key0 + 8 * (r >> 2) + 4 * hl + (r & 3) >= rend) st[r] = -INFINITY;
}

// Step j of this wave.  On entry stc holds block j's softmax after its
// first half (pipe_softmax1; sm, moved: its max and move test), kf block j +
// 1's K operands, vf block j's V operands.  Computes block j + 1's scores
// into stn beside the second half of block j's softmax (reading block j +
// 2's K operands at K-ring offset KNEXT into kf as the score instructions
// issue), takes the rare paths (a reference move recomputes block j's
// scores from its K stage at offset KOFF), then block j's P.V product
// beside the first half of block j + 1's softmax (its keys masked from
// rend when edge1), which leaves its max and move test in sm and moved.
template <int D, int KOFF, int KNEXT>
__device__ __forceinline__ void pipe_block(bool edge, bool edge1, f32x16_t& stc, f32x16_t& stn,
                                           const uint32_t (&ka)[PGeo<D>::KS], bf16x8_t (&kf)[PGeo<D>::KS],
                                           const bf16x8_t (&qf)[PGeo<D>::KS], bf16x8_t (&vf)[PGeo<D>::DB * 2],
                                           f32x16_t (&acc)[PGeo<D>::DB], RowStat& rs, float& sm, bool& moved,
                                           const char* svn, const uint32_t (&va)[PGeo<D>::DB][2], int key0,
                                           int rend, float c, float cinv, int hl) {
    using G = PGeo<D>;
    // Block j + 1's scores; each K operand is replaced by block j + 2's once
    // its instruction has issued.
#pragma unroll
    for (int r = 0; r < 16; ++r) stn[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        stn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], stn, 0, 0, 0);
        kf[ks] = lds_b128<KNEXT>(ka[ks]);
    }
    float l0;
    bool lo;
    bf16x8_t ph[2];
    pipe_softmax2(stc, c, rs, sm, l0, ph, lo);
#pragma unroll
    for (int i = 0; i < G::KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, FD_PIPE_VALU_PER_MFMA, 0);
    }
    // stc now holds block j's weights.  The rare paths read their inputs
    // through register barriers inside the branch, so the compiler cannot
    // compute them on every block instead.
    if (moved) {
        // The block's scores again, bit for bit (same operands: its K stage
        // stays in the ring through this step; same instructions), in place
        // of the weights.
#pragma unroll
        for (int r = 0; r < 16; ++r) stc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
            // one K operand at a time: block j + 2's are live here
            stc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128<KOFF>(ka[ks]), qf[ks], stc, 0, 0, 0);
            asm volatile("" ::: "memory");
        }
        if (edge) pipe_mask(stc, key0, rend, hl);
        float smv = sm, l0v = l0;
        asm volatile("" : "+v"(smv), "+v"(l0v));
        const float al = pipe_move(stc, c, cinv, smv, l0v, rs, ph, lo);
#pragma unroll
        for (int db = 0; db < G::DB; ++db) acc[db] *= al;
    }
    if (lo) {
        f32x16_t pr = stc;
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(pr[r]));
        bf16x8_t pl[2];
        pipe_remainder(pr, ph, pl, rs.l);
        chunk_pv<D>(vf, pl, acc);
    }
    // Block j's P.V product beside the first half of block j + 1's softmax,
    // then block j + 1's V operands (from the V stage array svn) into vf.
    if (edge1) pipe_mask(stn, key0 + G::SKEYS, rend, hl);
    chunk_pv<D>(vf, ph, acc);
    pipe_softmax1(stn, c, rs, sm, moved);
    pipe_v_reads<D>(svn, va, vf);
#pragma unroll
    for (int i = 0; i < G::KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, FD_PIPE_VALU_PER_MFMA, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * G::DB, 1);
    // computed here, not where they are used
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(stn[r]));
    asm volatile("" : "+v"(sm));
}



// f(integral_constant<int, 0>), f(.. 1), ..., f(.. N - 1) in order, stopping
// after the first call that returns false.
template <class F, int... Us>
__device__ __forceinline__ void unrolled_seq(F& f, std::integer_sequence<int, Us...>) {
    (void)(f(std::integral_constant<int, Us>{}) && ...);
}
template <int N, class F>
__device__ __forceinline__ void unrolled(F& f) {
    unrolled_seq(f, std::make_integer_sequence<int, N>{});
}

// Float offset of dims d .. d + 3 (d a multiple of 4) of row r in a row
// group's merge block [32][D]: 16-byte chunks XOR-swizzled by r & 15, so that
// 16 consecutive rows at one chunk fall in distinct banks.
template <int D>
__device__ __forceinline__ int merge_at(int r, int d) {
    return r * D + (((d >> 2) ^ (r & 15)) << 2);
}

template <int D, bool PAGED>
__global__ __launch_bounds__(kPT) void fd_mfma_chunk_kernel(PartialArgs a) {
#if FD_WG_TIMELINE
    const uint64_t tl_start = __builtin_amdgcn_s_memrealtime();
    uint64_t tl_first = 0;
    uint64_t* tl_row = nullptr;
    {
        const uint32_t i = blockIdx.y * gridDim.x + blockIdx.x;
        if (i < 4096u) tl_row = fd_chunk_timeline + (uint64_t)i * 16;
    }
#endif
    using G = PGeo<D>;
    constexpr int NS = kPNS;
    // One array per V stage (more strictly aligned, so that they come first
    // and the V reads' LDS addresses fit the instructions' offset field), then
    // the K ring.  The merge at the end reuses them: the statistics at the
    // start of the K ring, a row group's accumulators in V stage rg.
    __shared__ __attribute__((aligned(1024))) char sv0[G::STGB];
    __shared__ __attribute__((aligned(1024))) char sv1[G::STGB];
    __shared__ __attribute__((aligned(1024))) char sv2[G::STGB];
    __shared__ __attribute__((aligned(1024))) char sv3[G::STGB];
    __shared__ __attribute__((aligned(16))) char sk[NS * G::STGB];
    char* const svs[4] = {sv0, sv1, sv2, sv3};
    static_assert(32 * D * 4 == G::STGB, "a row group's merge block fills one V stage");
    static_assert(2048 <= NS * G::STGB, "the statistics fit the K ring");

    // Grid order as in fd_mfma_chunk8_kernel: the row tiles of one (KV head,
    // tile) next to each other, one contiguous range of them per XCD.
    const uint32_t nx = gridDim.x;
    uint32_t li = blockIdx.x;
    if ((nx & 7u) == 0) li = (li & 7u) * (nx >> 3) + (li >> 3);
    const int rt = (int)(li % (uint32_t)a.row_blocks);
    li /= (uint32_t)a.row_blocks;
    const int s = (int)(li % (uint32_t)a.rule.slots);
    const int g = (int)(li / (uint32_t)a.rule.slots);
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = (int)uniform((uint32_t)(tid >> 6));
    const int rg = w % kPRG;   // row group
    const int kh = w / kPRG;   // key half
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
        for (int idx = tid; idx < nrows; idx += kPT) {
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
    // Scores are scaled inside the exponent's FMA, which needs c > 0 (see
    // fd_mfma_chunk8_kernel).
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
    RowStat rs = {-INFINITY, 0.f, -INFINITY, 0.f, -INFINITY};
    const float cinv = __uint_as_float(uniform(__float_as_uint(1.f / c)));

    const char* kt;
    const char* vt;
    int rsb;  // bytes from one key row of the head to the next
    const int32_t* tbl = nullptr;
    if constexpr (PAGED) {
        kt = static_cast<const char*>(a.k) + g * a.pages.head_stride * 2;
        vt = static_cast<const char*>(a.v) + g * a.pages.head_stride * 2;
        rsb = a.pages.row_stride * 2;
        tbl = a.pages.table + (int64_t)b * a.pages.max_pages;
    } else {
        const int64_t tile_row = ((int64_t)b * a.Hkv + g) * a.Lmax + lo;
        kt = static_cast<const char*>(a.k) + tile_row * G::ROWB;
        vt = static_cast<const char*>(a.v) + tile_row * G::ROWB;
        rsb = G::ROWB;
    }
    kt = uniform(kt);  // scalar registers for the whole loop
    vt = uniform(vt);
    const int nst = (kend - lo + G::SKEYS - 1) / G::SKEYS;

    // Load instruction k of this wave fills RPI rows of block bb of a stage;
    // lane l takes row l / CH, global chunk (l % CH) ^ swizzle.
    uint32_t dma_off[G::DPW];
    int lds_off[G::DPW];
    int koff[G::DPW];
#pragma unroll
    for (int k = 0; k < G::DPW; ++k) {
        const int n = w + k * kPW;
        const int bb = n / G::IPB;
        const int i = n - bb * G::IPB;
        const int r = i * G::RPI + lane / G::CH;
        const int cg = (lane % G::CH) ^ cswf<G::CH>(r);
        koff[k] = bb * kCBK + i * G::RPI;
        dma_off[k] = (uint32_t)((PAGED ? lane / G::CH : koff[k] + lane / G::CH) * rsb + cg * 16);
        lds_off[k] = bb * G::BLKB + i * 1024;
    }
    // Page ids of the next stage to load (paged caches).
    int pg[G::DPW];
    auto pages = [&](int j) { pipe_pages<D, PAGED>(a.pages, tbl, lo, kend, j, koff, pg); };
    auto stage = [&](int j, auto SLOT) {
        constexpr int SL = decltype(SLOT)::value;
        pipe_stage<D, PAGED>(a.pages, pg, kt, vt, lo, kend, j, rsb, sk + SL * G::STGB, svs[SL], dma_off, lds_off,
                             koff);
    };

    // Lane addresses of this wave's operands (block kh): K absolute in ring
    // slot 0 (other slots add compile-time offsets), V relative to a V stage.
    uint32_t ka[G::KS];
    uint32_t va[G::DB][2];
    {
        const uint32_t kbase = lds_addr(sk) + kh * G::BLKB;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) ka[ks] = kbase + cswz<D>(col, 2 * ks + hl);
        const int g16 = lane >> 4;
        const int i16 = lane & 15;
        const int q4 = i16 & 3;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
                va[db][t2] = kh * G::BLKB +
                             cswz<D>(8 * t2 + 4 * hl + (i16 >> 2), (32 * db + 16 * (g16 & 1)) / 8 + (q4 >> 1)) +
                             8 * (q4 & 1);
    }

    // Stage t is at ring slot t % NS.  Step t uses block t's scores, block t +
    // 1's K operands and block t's V operands (all read in step t - 1), and
    // reads block t + 2's K operands and block t + 1's V operands; block t's
    // K stays readable through step t (the rare reference move recomputes
    // its scores).  So after the barrier of step t, which shows stage t + 2
    // landed for every wave (each waits for its own loads before it) and
    // every wave done with step t - 1, the loads of stage t + 3 start into
    // the slot of stage t - 1.  Stages past the last one are never loaded
    // (their slots are read but the results never used).
    {
        const auto issue = [&](auto UC) -> bool {
            if (decltype(UC)::value < nst) {
                pages(decltype(UC)::value);
                stage(decltype(UC)::value, UC);
            }
            return true;
        };
        unrolled<NS - 1>(issue);
    }
    pages(NS - 1);
    wait_stages<G::PER>(min(nst, NS - 1) - 2);  // stages 0 and 1
    bare_barrier();
#if FD_WG_TIMELINE
    tl_first = __builtin_amdgcn_s_memrealtime();
    const uint64_t tl_clk0 = __builtin_amdgcn_s_memtime();
#endif
    f32x16_t st[2];
    bf16x8_t kf[G::KS], vf[G::DB * 2];
    pipe_k_reads<D, 0>(ka, kf);
    pipe_scores<D>(kf, qf, st[0]);
    pipe_k_reads<D, G::STGB>(ka, kf);
    pipe_v_reads<D>(svs[0], va, vf);
    float sm;
    bool moved;
    {
        const int key00 = lo + kh * kCBK;
        if (key00 + kCBK > mask_from) pipe_mask(st[0], key00, rend, hl);
        pipe_softmax1(st[0], c, rs, sm, moved);
    }

    // Unrolled by NS stages, so that ring slots and the score buffer are
    // compile-time constants (U: the stage's place in the unrolled run).
    static_assert(NS % 2 == 0, "score buffers alternate within the unrolled run");
    for (int j0 = 0; j0 < nst; j0 += NS) {
        const auto step = [&](auto UC) -> bool {
            constexpr int U = decltype(UC)::value;
            const int j = j0 + U;
            if (j >= nst) return false;
            if (j + 2 < nst) {
                wait_vmcnt_le<0>();  // this wave's loads of stage j + 2
                bare_barrier();
                if (j + 3 < nst) stage(j + 3, std::integral_constant<int, (U + 3) % NS>{});
            }
            const int key0 = lo + j * G::SKEYS + kh * kCBK;
            const bool edge = key0 + kCBK > mask_from;
            const bool edge1 = key0 + G::SKEYS + kCBK > mask_from;
            pipe_block<D, (U % NS) * G::STGB, ((U + 2) % NS) * G::STGB>(edge, edge1, st[U % 2], st[1 - U % 2], ka, kf,
                                                                         qf, vf, acc, rs, sm, moved,
                                                                         svs[(U + 1) % NS], va, key0, rend, c, cinv,
                                                                         hl);
            if (j + NS < nst) pages(j + NS);
            return true;
        };
        unrolled<NS>(step);
    }
    wait_vmcnt_le<0>();
#if FD_WG_TIMELINE
    {
        const uint64_t t = __builtin_amdgcn_s_memrealtime();
        const uint64_t clk = __builtin_amdgcn_s_memtime();
        if (tl_row && lane == 0) tl_row[2 + w] = t;
        if (tl_row && tid == 0) {
            tl_row[12] = tl_clk0;
            tl_row[13] = clk;
        }
    }
#endif

    // This lane's row again, from an opaque lane id: recomputed here rather
    // than kept live (in registers the loop needs) through the loop.
    uint32_t lane_e;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
    const int col_e = (int)(lane_e & 31u);
    const int hl_e = (int)(lane_e >> 5);
    const int p_e = p0 + rg * 32 + col_e;
    const bool valid_e = p_e < R;
    const int64_t mrow_e = rowbase + (int64_t)(p_e % n_rep) * q_len + p_e / n_rep;

    // Per-row totals over the two lane halves; then merge the key halves.
    const float m = rs.m;
    const float l = xor32_sum(rs.l);
    const float mx = xor32_max(rs.xr) * c;
    __syncthreads();  // the rings are free
    float* sm_m = reinterpret_cast<float*>(sk);  // [kPRG][32]
    float* sm_l = sm_m + kPRG * 32;
    float* sm_x = sm_l + kPRG * 32;
    char* const mblk = rg == 0 ? sv0 : rg == 1 ? sv1 : rg == 2 ? sv2 : sv3;
    float* sm_acc = reinterpret_cast<float*>(mblk);  // [32][D], swizzled
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4)
                *reinterpret_cast<f32x4_t*>(sm_acc + merge_at<D>(col_e, 32 * db + 8 * a4 + 4 * hl_e)) =
                    f32x4_t{acc[db][4 * a4], acc[db][4 * a4 + 1], acc[db][4 * a4 + 2], acc[db][4 * a4 + 3]};
        if (hl_e == 0) {
            sm_m[rg * 32 + col_e] = m;
            sm_l[rg * 32 + col_e] = l;
            sm_x[rg * 32 + col_e] = mx;
        }
    }
    __syncthreads();
    if (kh == 1 || !valid_e) return;
    const float m2 = sm_m[rg * 32 + col_e];
    const float M = fmaxf(m, m2);
    const float f1 = m == -INFINITY ? 0.f : fast_exp2(m - M);
    const float f2 = m2 == -INFINITY ? 0.f : fast_exp2(m2 - M);
    const float den = l * f1 + sm_l[rg * 32 + col_e] * f2;
    const float X = fmaxf(mx, sm_x[rg * 32 + col_e]);
    const bool empty = M == -INFINITY;
    const float inv = empty ? 0.f : 1.f / den;
    const float lse_v = empty ? -INFINITY : (M + log2f(den)) * kLn2;
    if (a.direct) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + mrow_e * D;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d = 32 * db + 8 * a4 + 4 * hl_e;
                const f32x4_t y = *reinterpret_cast<const f32x4_t*>(sm_acc + merge_at<D>(col_e, d));
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (acc[db][4 * a4 + e] * f1 + y[e] * f2) * inv;
                uint2 packed;
                packed.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                packed.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                *reinterpret_cast<uint2*>(o + d) = packed;
            }
        if (hl_e == 0 && a.lse) a.lse[mrow_e] = lse_v;
    } else {
        if (!empty) {
            float* o = a.o_part + (mrow_e * slots + s) * D;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d = 32 * db + 8 * a4 + 4 * hl_e;
                    const f32x4_t y = *reinterpret_cast<const f32x4_t*>(sm_acc + merge_at<D>(col_e, d));
                    f32x4_t v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (acc[db][4 * a4 + e] * f1 + y[e] * f2) * inv;
                    *reinterpret_cast<f32x4_t*>(o + d) = v;
                }
        }
        if (hl_e == 0) {
            a.m_part[mrow_e * slots + s] = empty ? -INFINITY : X * kLn2;
            a.lse_part[mrow_e * slots + s] = lse_v;
        }
    }
#if FD_WG_TIMELINE
    if (tid == 0 && tl_row) {
        tl_row[0] = tl_start;
        tl_row[1] = tl_first;
        tl_row[10] = __builtin_amdgcn_s_memrealtime();
        tl_row[11] = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);  // HW_REG_XCC_ID bits 3:0
    }
#endif
}

template <int D, bool PAGED>
void launch_chunk_p(int batch, const PartialArgs& a, hipStream_t stream) {
    const uint32_t x = (uint32_t)a.rule.slots * a.Hkv * a.row_blocks;
    switch (a.kv_codes) {
        case kKvE4M3:
            hipLaunchKernelGGL((fd_mfma_chunk8_kernel<D, PAGED, kKvE4M3>), dim3(x, batch), dim3(kCT), 0, stream, a);
            break;
        case kKvInt8:
            hipLaunchKernelGGL((fd_mfma_chunk8_kernel<D, PAGED, kKvInt8>), dim3(x, batch), dim3(kCT), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL((fd_mfma_chunk_kernel<D, PAGED>), dim3(x, batch), dim3(kPT), 0, stream, a);
            break;
    }
}

template <int D>
void launch_chunk(int batch, const PartialArgs& a, hipStream_t stream) {
    if (a.pages.table != nullptr)
        launch_chunk_p<D, true>(batch, a, stream);
    else
        launch_chunk_p<D, false>(batch, a, stream);
}

}  // namespace

hipError_t launch_chunk_mfma(int head_dim, int batch, const PartialArgs& a, hipStream_t stream) {
    // x = KV heads x tiles x row tiles of one sequence: its threads must stay
    // within the 32-bit launch limit.
    if ((uint64_t)a.rule.slots * a.Hkv * a.row_blocks * kCT > 0xffffffffull) return hipErrorInvalidConfiguration;
    if (head_dim == 64)
        launch_chunk<64>(batch, a, stream);
    else
        launch_chunk<128>(batch, a, stream);
    return hipGetLastError();
}

}  // namespace fdk
