// fd_mfma_common.h -- operand types and LDS access helpers shared by the
// matrix-core kernels (fd_mfma.hip: decode row groups; fd_chunk.hip: chunk
// tiles).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fdk {

// Cache policy bits of the buffer-to-LDS loads (the `aux` operand).
#ifndef FD_LOAD_AUX
#define FD_LOAD_AUX 2
#endif

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Lazy rescale threshold of the online softmax, in log2 units: a running
// state is moved to a new reference max only when a score passes the old
// one by more than this (weights up to 2^8 stay representable).
constexpr float kTau = 8.f;

// s_waitcnt with only the vector-memory counter constrained: wait until at
// most N vector loads of this wave are outstanding (gfx9 encoding: vmcnt in
// bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
template <int N>
static __device__ __forceinline__ void wait_vmcnt_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// LDS address (byte offset in the workgroup's LDS) of a shared-memory pointer.
static __device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// Transposing LDS read, ds_read_b64_tr_b16: in each 16-lane group, lane
// 4j + q names 4 consecutive bf16 of a row; lane i receives element i % 4 of
// lane 4j + i / 4 for j = 0..3.  Issued as inline assembly because the
// compiler treats the builtin as possibly aliasing the LDS loads in flight and
// would wait for all of them; the result is only valid after an explicit
// s_waitcnt lgkmcnt(0).
static __device__ __forceinline__ bf16x4_t tr_read(const char* p) {
    bf16x4_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return r;
}

// 16-byte LDS read and write as inline assembly.  As plain loads and stores
// the compiler would treat them as possibly aliasing the buffer-to-LDS loads
// in flight and wait for all of those first, which serialises a load ring.
// The caller makes sure that what it reads has landed and that what it
// writes is read only after its own later waits; LDS executes one wave's
// accesses in order.  A read's result is valid after s_waitcnt lgkmcnt(0).
static __device__ __forceinline__ u32x4_t lds_read_b128(const char* p) {
    u32x4_t r;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return r;
}

static __device__ __forceinline__ void lds_write_b128(char* p, u32x4_t x) {
    asm volatile("ds_write_b128 %0, %1" : : "v"(lds_addr(p)), "v"(x) : "memory");
}

// Four one-byte K/V codes (bytes 0..3 of w) as four bf16 values: lo holds
// codes 0 and 1, hi codes 2 and 3.  Exact: every E4M3 value and every
// integer in [-128, 127] is a bf16 value.  The per-tensor scales are applied
// outside (k_scale in the score scale, v_scale to the output).
template <int KV>
static __device__ __forceinline__ void codes_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
    if constexpr (KV == kKvE4M3) {
        lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false));
        hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true));
    } else {
        static_assert(KV == kKvInt8, "one-byte code format");
        float f[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) f[n] = (float)(int)(int8_t)(w >> (8 * n));  // sign-extended byte n
        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
        lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{f[0], f[1]}, bf16x2_v));
        hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{f[2], f[3]}, bf16x2_v));
    }
}

}  // namespace fdk
