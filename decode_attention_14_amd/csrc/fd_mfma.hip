// fd_mfma.hip -- split-KV partial kernel on the matrix cores for decode-sized
// row groups on gfx950 (CDNA4): bf16 queries over bf16, FP8 E4M3 or INT8 caches,
// contiguous or paged.
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
// kernel.  Caches of one-byte codes run eight waves per workgroup over rows
// of D codes: the K codes are converted into the A operands of the score
// product in registers, the V codes into a bf16 block for the transposed
// reads (see codes_read / codes_settle).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <cstdlib>

#include "fd_device.h"
#include "fd_internal.h"
#include "fd_mfma_common.h"

#ifndef FD_WG_TIMELINE
#define FD_WG_TIMELINE 0
#endif

// Workgroup timeline (a diagnostic build only, FD_WG_TIMELINE=1; the
// library proper compiles none of it).  Workgroup i of the last launch (in
// dispatch order, i < kTimelineWGs) leaves at [i * kTimelineSlots]: its start,
// the landing of wave 0's first block, each wave's exit from its block loop
// (up to 8 waves), its end, all in the 100 MHz s_memrealtime clock, and the
// XCD it ran on.  fd_debug_timeline copies the array to host memory.
#if FD_WG_TIMELINE
namespace fdk {
constexpr int kTimelineWGs = 4096;
constexpr int kTimelineSlots = 16;
enum { kTlStart = 0, kTlFirst = 1, kTlLoop = 2, kTlEnd = 10, kTlXcc = 11 };
}  // namespace fdk
__device__ uint64_t fd_wg_timeline[fdk::kTimelineWGs * fdk::kTimelineSlots];
extern "C" int fd_debug_timeline(void* host_dst, uint64_t bytes) {
    if (bytes > sizeof(fd_wg_timeline)) bytes = sizeof(fd_wg_timeline);
    return (int)hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(fd_wg_timeline), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

namespace fdk {
namespace {

#if FD_WG_TIMELINE
__device__ __forceinline__ uint64_t* timeline_row() {
    const uint32_t i = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    return i < (uint32_t)kTimelineWGs ? fd_wg_timeline + (uint64_t)i * kTimelineSlots : nullptr;
}
#endif

#ifndef FD_MFMA_STAGES
#define FD_MFMA_STAGES 2
#endif

#ifndef FD_MFMA_THREADS
#define FD_MFMA_THREADS 256
#endif
constexpr int kMT = FD_MFMA_THREADS;  // threads per workgroup (bf16 caches)
constexpr int kMW = kMT / 64;     // waves per workgroup
#ifndef FD_CODE8_WAVES
#define FD_CODE8_WAVES 8
#endif
constexpr int kMW8 = FD_CODE8_WAVES;  // waves per workgroup over one-byte caches
#ifndef FD_CODE8_SPAN_WAVES
#define FD_CODE8_SPAN_WAVES 4
#endif
// ... in span mode: three four-wave workgroups fit a compute unit's LDS, and
// while one merges a piece or waits for a piece's first loads the others
// stream (FP8 caches, 32-sequence variable-length batch: 56.7-56.8 against
// 57.7 us with eight waves).
constexpr int kMW8S = FD_CODE8_SPAN_WAVES;

// Waves per workgroup of the decode kernel for a cache format and mode.
__host__ __device__ constexpr int decode_waves(int kv, bool spans) {
    return kv == kKvBf16 ? kMW : (spans ? kMW8S : kMW8);
}
constexpr int kKB = 16;           // keys per block
constexpr int kNS = FD_MFMA_STAGES;
// Span mode: line positions in front of each (sequence, KV head) pair, the
// fixed cost of one piece (its first loads and its merge) in 16-key blocks:
// a span holding more pieces gets fewer blocks.  Measured on the 32-sequence
// variable-length batch: FP8 caches 58.7 against 60.4 us at 16 (57.7-58.0 at
// 32), bf16 caches 101.9 against 102.0 us (103.1 at 32).
constexpr int kSpanPieceBlocks = 16;

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
// 2D-byte rows (the operand layout itself); caches of one-byte codes (C8:
// FP8 E4M3 or INT8) keep D-byte rows, whose K codes are converted into the
// score operands in registers and whose V codes are converted per block
// into a bf16 block of the operand layout (CONVB).
#ifndef FD_CODE8_STAGES
#define FD_CODE8_STAGES 2
#endif
template <int D, bool C8>
struct LGeo {
    static constexpr int ROWB = C8 ? D : 2 * D;     // bytes per stored key row
    static constexpr int CH = ROWB / 16;            // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;             // rows per 1 KiB LDS-load instruction
    static constexpr int IPB = kKB / RPI;           // instructions per block per tensor
    static constexpr int BLKB = kKB * ROWB;         // bytes per block per tensor
    static constexpr int STAGEB = 2 * BLKB;         // K then V
    static constexpr int NS = C8 ? FD_CODE8_STAGES : kNS;
    static constexpr int CONVB = C8 ? Geo<D>::BLKB : 0;  // bf16 V block (K is converted in registers)
    static constexpr int WAVEB = NS * STAGEB + CONVB;
    static_assert(IPB >= 1, "whole load instructions per block");
};

// XOR swizzle of the 16-byte chunks of row r (CH chunks per row).  Two read
// patterns must be free of LDS bank conflicts: 16 consecutive rows at one
// chunk (K operands, ds_read_b128), and 4 aligned consecutive rows at an
// even/odd chunk pair (transposed V reads).  For CH = 16 the map is the
// linear bijection r -> (r1 r0) in chunk bits 1:0, r2 ^ r3 in bit 2 and
// r0 ^ r3 in bit 3: the hardware's SQ_LDS_BANK_CONFLICT counter reads zero
// for both patterns with it, where a map sending row bits 1:0 to chunk bits
// 2:1 (conflict-free under a plain 64-bank model) cost 4 cycles on every K
// read.  For CH = 8, two 128-byte rows share a bank cycle, and the map acts
// on the row pair index r >> 1.
template <int CH>
__device__ __forceinline__ int swf(int r) {
    if constexpr (CH == 16) return (r & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 3);
    const int u = (r >> 1) & 7;
    return ((u & 1) << 1) | (((u >> 1) & 1) << 2) | ((u >> 2) & 1);
}

// Byte offset inside a block of global chunk c of row r.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
    return r * Geo<D>::ROWB + ((c ^ swf<Geo<D>::CH>(r)) << 4);
}

// Start the loads of one block (16 rows of K and of V, `left` bytes of the
// tile from kp/vp on; none if left <= 0) into LDS at dst: K rows first, then
// V rows.  Lane l of load instruction i reads its row's global chunk
// dma_off[i]; the data lands at dst + i * 1024 + 16 * l.  Rows past `left`
// read as zeros and cost no memory traffic.
template <int D, bool C8>
__device__ __forceinline__ void load_block(const char* kp, const char* vp, int left, char* dst,
                                           const uint32_t* dma_off) {
    using L = LGeo<D, C8>;
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
template <int D, bool C8, bool PAGED>
__device__ __forceinline__ void load_block_at(const PagedKV& pk, int page, const char* kt, const char* vt, int lo,
                                              int hi, int blk, int rsb, char* dst, const uint32_t* dma_off) {
    using L = LGeo<D, C8>;
    constexpr int ESZ = C8 ? 1 : 2;
    if constexpr (PAGED) {
        int64_t off;
        const uint32_t n = paged_rows_in(pk, page, lo + blk * kKB, kKB, hi, rsb, L::ROWB, &off);
        load_block<D, C8>(kt + off * ESZ, vt + off * ESZ, (int)n, dst, dma_off);
    } else {
        const int off = blk * L::BLKB;
        load_block<D, C8>(kt + off, vt + off, (hi - lo) * L::ROWB - off, dst, dma_off);
    }
}

// Caches of one-byte codes.  A landed block holds 16 rows of K codes, then
// 16 of V codes (D bytes a row).  Row r's 16-byte chunks are stored XOR-
// swizzled by cswz8(r): physical chunk p holds chunk p ^ cswz8(r).  The K
// operands are read straight from these rows and converted in registers
// (lane (grp, col) takes the D / 4 codes of row col for dims grp * D / 4 ..,
// read as D / 64 16-byte chunks): each 16-byte read covers 16 consecutive
// rows at one chunk.  For 128-byte code rows that is the pattern of the K
// operands of bf16 caches at D = 64, and swf<8> (measured free of bank
// conflicts for it) serves; 64-byte rows take the row pair r / 2, which of
// five maps measured left the fewest conflicts (a third fewer than r / 4;
// what remains at that row size comes from other accesses).  V goes through
// LDS: each wave converts its block's V codes into a bf16 block of the
// operand layout (swz) for the transposed reads.  Both conversions are exact
// (see codes_to_bf16).  The query rows of such a call are loaded in the same
// order of dims as the K operands (qf_dim), so each score is the same dot
// product.
template <int D>
__device__ __forceinline__ int cswz8(int r) {
    constexpr int CH8 = LGeo<D, true>::CH;  // 16-byte chunks per code row
    if constexpr (CH8 == 8) return swf<8>(r);
    return (r >> 1) & (CH8 - 1);
}

// First dim of query fragment ks of lane group grp: the order of the K
// operands (bf16 caches: 8 grp + 32 ks; codes: grp D / 4 + 8 ks).
template <int D, bool C8>
__device__ __forceinline__ int qf_dim(int grp, int ks) {
    return C8 ? grp * (D / 4) + 8 * ks : 8 * grp + 32 * ks;
}

template <int D>
struct DQ {
    static constexpr int NU = LGeo<D, true>::BLKB / 8 / 64;  // 8-byte V code units per lane
    static constexpr int KC = D / 64;                         // 16-byte K chunks per lane
};

// LDS reads of one landed code block (at src): the lane's V code units (xv:
// unit n * 64 + lane of the block, so each read covers consecutive bytes)
// and its K operand chunks (xk), as plain loads the compiler waits for.
template <int D>
__device__ __forceinline__ void codes_read(const char* src, int lane, int grp, int col,
                                           u32x2_t (&xv)[DQ<D>::NU], u32x4_t (&xk)[DQ<D>::KC]) {
    using L = LGeo<D, true>;
#pragma unroll
    for (int n = 0; n < DQ<D>::NU; ++n) xv[n] = lds_load_b64(lds_addr(src + L::BLKB + (n * 64 + lane) * 8));
#pragma unroll
    for (int k = 0; k < DQ<D>::KC; ++k) {
        const int c = grp * DQ<D>::KC + k;  // chunk of dims 16 c .. 16 c + 15
        xk[k] = lds_load_b128(lds_addr(src + col * L::ROWB + ((c ^ cswz8<D>(col)) << 4)));
    }
}

// Write the bf16 V block at dst from codes_read's V units and turn its K
// chunks into the score product's A operands.  A V unit (8 codes of row r,
// physical code chunk pu / 2, half pu % 2) becomes one 16-byte bf16 chunk.
// A 16-byte write serves 8 lanes per LDS cycle over 128 bytes of banks; the 8
// lanes of a group hold 8 consecutive units of one code row, whose bf16
// chunks form one aligned group of 8 (cswz8 XORs whole code chunks, bf16
// chunk pairs, so an aligned group stays one), and swz keeps them on 8
// distinct chunks modulo 8: the writes are conflict-free in lane order.
template <int D, int KV>
__device__ __forceinline__ void codes_settle(u32x2_t (&xv)[DQ<D>::NU], u32x4_t (&xk)[DQ<D>::KC], char* dst,
                                             int lane, bf16x8_t (&kf)[Geo<D>::KS]) {
    constexpr int UPR = LGeo<D, true>::ROWB / 8;  // 8-byte units per code row
#pragma unroll
    for (int n = 0; n < DQ<D>::NU; ++n) {
        const int u = n * 64 + lane;
        const int r = u / UPR, pu = u % UPR;
        const int c = (((pu >> 1) ^ cswz8<D>(r)) << 1) | (pu & 1);  // 8 codes of row r = dims 8c .. 8c + 7
        uint32_t b[4];
        codes_to_bf16<KV>(xv[n][0], b[0], b[1]);
        codes_to_bf16<KV>(xv[n][1], b[2], b[3]);
        lds_write_b128(dst + swz<D>(r, c), u32x4_t{b[0], b[1], b[2], b[3]});
    }
    // K: 16 codes per chunk, 8 per operand (ks = 2 k + half).
#pragma unroll
    for (int k = 0; k < DQ<D>::KC; ++k) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t b[4];
            codes_to_bf16<KV>(xk[k][2 * h], b[0], b[1]);
            codes_to_bf16<KV>(xk[k][2 * h + 1], b[2], b[3]);
            kf[2 * k + h] = __builtin_bit_cast(bf16x8_t, u32x4_t{b[0], b[1], b[2], b[3]});
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

// V^T operands of one 16-key block stored (swizzled) at vb in LDS, through
// transposed reads (waited for).
template <int D>
__device__ __forceinline__ void v_fragments(const char* vb, bf16x4_t (&vf)[Geo<D>::DB], int grp, int col) {
    using G = Geo<D>;
    const int r = 4 * grp + (col >> 2);
    const int q4 = col & 3;
    uint32_t a[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db) a[db] = lds_addr(vb + swz<D>(r, 2 * db + (q4 >> 1)) + 8 * (q4 & 1));
    tr_read_wait<0>(a, vf);
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
    v_fragments<D>(vb, vf, grp, col);
}

// Launch geometry and LDS bytes of the decode kernel.
template <int D, int NB, int KV, bool SPANS>
struct DecodeGeo {
    static constexpr bool C8 = KV != kKvBf16;  // one-byte codes
    static constexpr int MW = decode_waves(KV, SPANS);  // waves per workgroup
    static constexpr int MT = 64 * MW;
    static constexpr int NR = 16 * NB;          // query rows per workgroup
    static constexpr int RS = D + 4;            // padded row stride of the merge area (floats)
    static constexpr int MERGEB = MW * (NR * RS + 3 * NR) * 4;
    static constexpr int RINGB = MW * LGeo<D, C8>::WAVEB;
    static constexpr int SMEMB = RINGB > MERGEB ? RINGB : MERGEB;
};

// One work unit of the decode kernel: KV head g of sequence b (L visible
// keys), keys [lo, hi) (lo < hi), partial slot s.  Slots [pad_from, slots)
// of the unit's rows get the empty state (m_part = lse_part = -inf, o_part
// untouched); pad_from = slots pads nothing.  smem: the kernel's LDS block;
// on return every wave is past its last LDS access of the unit only after a
// barrier, which the caller places before reusing it.
template <int D, int NB, bool CAUSAL, bool PAGED, int KV, bool SPANS>
__device__ __forceinline__ void partial_unit(const PartialArgs& a, char* smem, int g, int b, int s, int L, int lo,
                                             int hi, int pad_from, uint64_t& tl_first) {
    using DG = DecodeGeo<D, NB, KV, SPANS>;
    constexpr bool C8 = DG::C8;
    using G = Geo<D>;
    using LG = LGeo<D, C8>;
    constexpr int MW = DG::MW;
    constexpr int MT = DG::MT;
    constexpr int NS = LG::NS;
    constexpr int ESZ = C8 ? 1 : 2;  // bytes per stored K/V element
    constexpr int NR = DG::NR;
    constexpr int RS = DG::RS;
    (void)tl_first;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = (int)uniform((uint32_t)(tid >> 6));
    const int grp = lane >> 4;
    const int col = lane & 15;

    const int nrows = a.rows;
    const int64_t row0 = ((int64_t)b * a.Hq + (int64_t)g * a.n_rep) * a.q_len;
    const int slots = a.rule.slots;

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
                    static_cast<const uint16_t*>(a.q) + (row0 + r) * D + qf_dim<D, C8>(grp, ks));
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
    char* conv = ring + NS * LG::STAGEB;  // codes: this wave's bf16 V block
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
    // row (the operand swizzle), rows of codes in their stored order.
    uint32_t dma_off[LG::IPB];
#pragma unroll
    for (int i = 0; i < LG::IPB; ++i) {
        const int r = i * LG::RPI + lane / LG::CH;
        const int cg = C8 ? (lane % LG::CH) ^ cswz8<D>(r) : (lane % LG::CH) ^ swf<LG::CH>(r);
        dma_off[i] = (uint32_t)(r * rsb + cg * 16);
    }

    // Wave block j is tile block w + 4j and goes to ring slot j % NS.  A
    // paged cache's page ids are read one block ahead of their loads, so the
    // scalar table reads overlap the work of the previous block.
    auto page_of = [&](int blk) { return PAGED ? page_at(a.pages, tbl, lo + blk * kKB, hi) : 0; };
    int page_next = page_of(w);
    // Start the loads of wave block jn (issued in order jn = 0, 1, ...) into
    // ring slot jn % NS.
    auto issue = [&](int jn) {
        const int page = page_next;
        page_next = page_of(w + (jn + 1) * MW);
        load_block_at<D, C8, PAGED>(a.pages, page, kt, vt, lo, hi, w + jn * MW, rsb, ring + (jn % NS) * LG::STAGEB,
                                    dma_off);
    };

#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(j);
    for (int j = 0; j < nw; ++j) {
        issue(j + NS - 1);
        wait_vmcnt_le<(NS - 1) * 2 * LG::IPB>();  // block j has landed
#if FD_WG_TIMELINE
        if (j == 0) tl_first = __builtin_amdgcn_s_memrealtime();
#endif
        const char* kb = ring + (j % NS) * LG::STAGEB;
        bf16x8_t kf[G::KS];
        bf16x4_t vf[G::DB];
        if constexpr (C8) {
            u32x2_t xv[DQ<D>::NU];
            u32x4_t xk[DQ<D>::KC];
            codes_read<D>(kb, lane, grp, col, xv, xk);
            codes_settle<D, KV>(xv, xk, conv, lane, kf);
            v_fragments<D>(conv, vf, grp, col);
        } else {
            load_fragments<D>(kb, kb + LG::BLKB, kf, vf, grp, col);
        }
        const int key0 = lo + (w + j * MW) * kKB;  // first key of the block
        block_math<D, NB>(kf, vf, qf, acc, m, l, mx, key0, key0 + kKB > mask_from, rend, c, grp);
    }

    // Merge: the four lane groups of a column, then the four waves via LDS.
    wait_vmcnt_le<0>();
#if FD_WG_TIMELINE
    {
        const uint64_t t = __builtin_amdgcn_s_memrealtime();
        uint64_t* row = timeline_row();
        if (row && lane == 0 && w < 8) row[kTlLoop + w] = t;
    }
#endif
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

    // Outputs, four columns per thread: the weighted sum of the waves' rows
    // with weights exp2(m_w - M) / sum.  Every thread derives its row's
    // weights from the wave states itself (the reads of one row's entries
    // are LDS broadcasts), so no further barrier is needed; the thread at
    // column 0 also writes the row's statistics.  A row with no visible key
    // gets zeros (direct) or no o_part entry.
    constexpr int C4 = D / 4;
    for (int idx = tid; idx < nrows * C4; idx += MT) {
        const int r = idx / C4;
        const int c4 = idx - r * C4;
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < MW; ++x) M = fmaxf(M, sm_m[x * NR + r]);
        const bool empty = M == -INFINITY;
        float f[MW];
        float den = 0.f;
#pragma unroll
        for (int x = 0; x < MW; ++x) {
            const float mw = sm_m[x * NR + r];
            f[x] = (empty || mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            den = fmaf(f[x], sm_l[x * NR + r], den);
        }
        const int64_t row = row0 + r;
        if (c4 == 0) {
            const float lse_v = empty ? -INFINITY : (M + log2f(den)) * kLn2;
            if (a.direct) {
                if (a.lse) a.lse[row] = lse_v;
            } else {
                float X = -INFINITY;
#pragma unroll
                for (int x = 0; x < MW; ++x) X = fmaxf(X, sm_x[x * NR + r]);
                a.m_part[row * slots + s] = empty ? -INFINITY : X * kLn2;
                a.lse_part[row * slots + s] = lse_v;
            }
        }
        if (!a.direct && empty) continue;
        // codes: V was dequantised without its scale
        const float inv = empty ? 0.f : (C8 ? a.v_scale : 1.f) * __builtin_amdgcn_rcpf(den);
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < MW; ++x)
            o += (f[x] * inv) * *reinterpret_cast<const f32x4_t*>(sm_acc + (x * NR + r) * RS + 4 * c4);
        if (a.direct) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
            pk.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + row * D + 4 * c4) = pk;
        } else {
            *reinterpret_cast<f32x4_t*>(a.o_part + (row * slots + s) * D + 4 * c4) = o;
        }
    }
    // Slots past this unit's (span mode: the last segment of its KV head).
    const int npad = slots - pad_from;
    if (npad > 0) {
        for (int idx = tid; idx < nrows * npad; idx += MT) {
            const int r = idx / npad;
            const int sl = pad_from + (idx - r * npad);
            a.m_part[(row0 + r) * slots + sl] = -INFINITY;
            a.lse_part[(row0 + r) * slots + sl] = -INFINITY;
        }
    }
}

// Span mode (equal shares of a ragged batch's keys per workgroup, as page
// "FlashDecoding算法原理与多GPU并行解码实战", variable-length section, fills
// equal token bins per device): the (sequence, KV head) pairs' 16-key blocks
// laid end to end (sequence-major, then KV head, each pair's blocks in key
// order, each pair preceded by kSpanPieceBlocks positions that stand for the
// fixed cost of a piece: its first loads and its merge), cut into
// rule.spans equal contiguous spans; workgroup w runs spans w, w + grid, ...
// (the launch makes grid = spans, so one each)
// A span runs one unit per pair it touches; the pair's units take slots 0,
// 1, ... in span order (slot = span - the span of the pair's first block),
// and the span holding a pair's last block pads the pair's remaining slots.
// The span length is at least ceil(line length / spans) and at least
// ceil(max blocks of a pair / (slots - 1)), so no pair needs more than
// `slots` units whatever the lengths are.  Sequences without keys are padded
// whole by workgroup b % grid.  Every workgroup computes the totals from
// cache_lens itself (wave-uniform scalar loop over the batch).
template <int D, int NB, bool CAUSAL, bool PAGED, int KV, bool SPANS>
__global__ __launch_bounds__(64 * decode_waves(KV, SPANS)) void fd_mfma_partial_kernel(PartialArgs a) {
    using DG = DecodeGeo<D, NB, KV, SPANS>;
    __shared__ __attribute__((aligned(16))) char smem[DG::SMEMB];
    uint64_t tl_first = 0;
#if FD_WG_TIMELINE
    const uint64_t tl_start = __builtin_amdgcn_s_memrealtime();
#endif
    const int slots = a.rule.slots;
    if constexpr (!SPANS) {
        // Tile mode.  KV head fastest: workgroups are dealt to the eight XCDs
        // round-robin in launch order, so consecutive ids take the heads of
        // one (tile, sequence) and every XCD gets the same mix of tiles (all
        // heads of a sequence have the same length).  With the tile fastest
        // instead, a tile index would pin to a subset of XCDs and short
        // sequences would leave some idle.
        const int g = blockIdx.x;
        const int s = blockIdx.y;
        const int b = blockIdx.z;
        int L = a.cache_lens[b];
        L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
        int lo, hi, S;
        tile_of(a.rule, L, s, lo, hi, S);
        lo = (int)uniform((uint32_t)lo);
        hi = (int)uniform((uint32_t)hi);
        if (s >= S) {
            const int tid = threadIdx.x;
            const int64_t row0 = ((int64_t)b * a.Hq + (int64_t)g * a.n_rep) * a.q_len;
            if (a.direct) {
                for (int idx = tid; idx < a.rows * D; idx += DG::MT)
                    reinterpret_cast<uint16_t*>(a.out)[row0 * D + idx] = 0;
                if (a.lse && tid < a.rows) a.lse[row0 + tid] = -INFINITY;
                return;
            }
            if (tid < a.rows) {
                a.m_part[(row0 + tid) * slots + s] = -INFINITY;
                a.lse_part[(row0 + tid) * slots + s] = -INFINITY;
            }
            return;
        }
        partial_unit<D, NB, CAUSAL, PAGED, KV, SPANS>(a, smem, g, b, s, L, lo, hi, slots, tl_first);
    } else {
        // Span state: span sp of nsp, [R0, R1) of per blocks; the current
        // pair (sb, sg) of sb's snb blocks and sL keys, sC the first block of
        // sequence sb's pairs.
        const int nsp = a.rule.spans;
        int sp = blockIdx.x;
        int sb = 0, sg = 0, snb = 0, sL = 0;
        int64_t sC = 0, per = 1, R0 = 0, R1 = 0, N = 0;
        bool more = false;
        auto clamp_len = [&](int b) {
            const int L = a.cache_lens[b];
            return L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
        };
        // Start span sp: more = it holds blocks; then (sb, sg) is the pair
        // holding block R0.
        auto begin_span = [&]() {
            R0 = (int64_t)sp * per;
            R1 = R0 + per < N ? R0 + per : N;
            more = R0 < R1;
            if (!more) return;
            sC = 0;
            for (sb = 0; sb < a.batch; ++sb) {
                sL = clamp_len(sb);
                snb = (sL + kKB - 1) / kKB;
                const int64_t wseq = snb > 0 ? (int64_t)a.Hkv * (kSpanPieceBlocks + snb) : 0;
                if (snb > 0 && sC + wseq > R0) break;
                sC += wseq;
            }
            sg = R0 > sC ? (int)((R0 - sC) / (kSpanPieceBlocks + snb)) : 0;
        };
        int nbmax = 0;
        for (int b = 0; b < a.batch; ++b) {
            const int nb = (clamp_len(b) + kKB - 1) / kKB;
            N += nb > 0 ? (int64_t)a.Hkv * (kSpanPieceBlocks + nb) : 0;
            nbmax = nb > nbmax ? nb : nbmax;
        }
        per = (N + nsp - 1) / nsp;
        const int64_t per_min = (nbmax + slots - 2) / (slots - 1);
        per = per > per_min ? per : per_min;
        per = per > 1 ? per : 1;
        // Sequences without keys: every slot of every row empty.
        for (int b = blockIdx.x; b < a.batch; b += gridDim.x) {
            if (clamp_len(b) > 0) continue;
            const int64_t r0 = (int64_t)b * a.Hq * a.q_len;
            const int64_t n = (int64_t)a.Hq * a.q_len * slots;
            for (int64_t idx = threadIdx.x; idx < n; idx += DG::MT) {
                a.m_part[r0 * slots + idx] = -INFINITY;
                a.lse_part[r0 * slots + idx] = -INFINITY;
            }
        }
        begin_span();
        for (int it = 0;; ++it) {
            // The next piece: in this span, else in this workgroup's next span.
            bool done = false;
            for (;;) {
                if (more && sC + (int64_t)sg * (kSpanPieceBlocks + snb) + kSpanPieceBlocks < R1) break;
                sp += gridDim.x;
                if (sp >= nsp) {
                    done = true;
                    break;
                }
                begin_span();
            }
            if (done) break;
            const int64_t st = sC + (int64_t)sg * (kSpanPieceBlocks + snb) + kSpanPieceBlocks;  // first block
            const int64_t en = st + snb;
            const int blo = (int)((R0 > st ? R0 : st) - st);
            const int bhi = (int)((R1 < en ? R1 : en) - st);
            const int g = sg, b = sb, L = sL;
            const int s = sp - (int)(st / per);
            const int lo = (int)uniform((uint32_t)(blo * kKB));
            const int hi = (int)uniform((uint32_t)(bhi * kKB < L ? bhi * kKB : L));
            const int pad_from = en <= R1 ? s + 1 : slots;
            // Next pair: the next KV head, else the next sequence with keys.
            if (++sg == a.Hkv) {
                sg = 0;
                sC += (int64_t)a.Hkv * (kSpanPieceBlocks + snb);
                snb = 0;
                while (snb == 0 && ++sb < a.batch) {
                    sL = clamp_len(sb);
                    snb = (sL + kKB - 1) / kKB;
                }
                more = sb < a.batch;
            }
            if (it > 0) __syncthreads();  // the previous unit's LDS reads are done
            partial_unit<D, NB, CAUSAL, PAGED, KV, SPANS>(a, smem, g, b, s, L, lo, hi, pad_from, tl_first);
        }
    }
#if FD_WG_TIMELINE
    if (threadIdx.x == 0) {
        const uint64_t t = __builtin_amdgcn_s_memrealtime();
        uint64_t* row = timeline_row();
        if (row) {
            row[kTlStart] = tl_start;
            row[kTlFirst] = tl_first;
            row[kTlEnd] = t;
            row[kTlXcc] = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);  // HW_REG_XCC_ID bits 3:0
        }
    }
#endif
}

// FD_TRACE=1 in the environment: print each span launch's grid on stderr.
bool span_trace() {
    static const bool on = [] {
        const char* e = std::getenv("FD_TRACE");
        return e != nullptr && e[0] != '\0' && e[0] != '0';
    }();
    return on;
}

// Workgroups of kernel K resident at once on the current device, as many per
// compute unit as its registers and LDS allow (cached per device).
template <auto K>
int span_workgroups(int threads) {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, K, threads, 0) != hipSuccess || occ < 1) occ = 1;
    const int n = cus * occ;
    if (dev >= 0 && dev < 64) cached[dev] = n;
    return n;
}

// A span-mode launch cuts the batch into min(plan spans, resident workgroups)
// spans, one workgroup each: more spans than can run at once would only add
// per-span fills and merges (measured: 512 spans on the 256 resident
// workgroups of the one-byte kernel took 64 against 60 us on the
// variable-length batch).
template <auto K>
void launch_decode(dim3 grid, dim3 block, const PartialArgs& a, hipStream_t stream) {
    if (a.rule.spans > 0) {
        const int n = span_workgroups<K>((int)block.x);
        PartialArgs as = a;
        as.rule.spans = a.rule.spans < n ? a.rule.spans : n;
        if (span_trace())
            std::fprintf(stderr, "[fd] span launch: %d spans asked, %d resident workgroups\n", a.rule.spans, n);
        hipLaunchKernelGGL(K, dim3((unsigned)as.rule.spans), block, 0, stream, as);
        return;
    }
    hipLaunchKernelGGL(K, grid, block, 0, stream, a);
}

template <int D, int NB, int KV, bool SPANS>
void launch_nb_kv_s(int batch, const PartialArgs& a, hipStream_t stream) {
    const dim3 grid(a.Hkv, a.rule.slots, batch), block(64 * decode_waves(KV, SPANS));
    const bool paged = a.pages.table != nullptr;
    if (a.q_len > 1) {
        if (paged)
            launch_decode<fd_mfma_partial_kernel<D, NB, true, true, KV, SPANS>>(grid, block, a, stream);
        else
            launch_decode<fd_mfma_partial_kernel<D, NB, true, false, KV, SPANS>>(grid, block, a, stream);
    } else {
        if (paged)
            launch_decode<fd_mfma_partial_kernel<D, NB, false, true, KV, SPANS>>(grid, block, a, stream);
        else
            launch_decode<fd_mfma_partial_kernel<D, NB, false, false, KV, SPANS>>(grid, block, a, stream);
    }
}

template <int D, int NB, int KV>
void launch_nb_kv(int batch, const PartialArgs& a, hipStream_t stream) {
    if (a.rule.spans > 0)
        launch_nb_kv_s<D, NB, KV, true>(batch, a, stream);
    else
        launch_nb_kv_s<D, NB, KV, false>(batch, a, stream);
}

template <int D, int NB>
void launch_nb(int batch, const PartialArgs& a, hipStream_t stream) {
    switch (a.kv_codes) {
        case kKvE4M3: launch_nb_kv<D, NB, kKvE4M3>(batch, a, stream); break;
        case kKvInt8: launch_nb_kv<D, NB, kKvInt8>(batch, a, stream); break;
        default: launch_nb_kv<D, NB, kKvBf16>(batch, a, stream); break;
    }
}

}  // namespace

hipError_t launch_partials_mfma(int head_dim, int batch, const PartialArgs& a, hipStream_t stream) {
    if (a.rows > 32) return launch_chunk_mfma(head_dim, batch, a, stream);
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
