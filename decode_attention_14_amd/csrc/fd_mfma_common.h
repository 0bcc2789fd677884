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
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
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

// LDS loads.  A load result must never be in flight outside the compiler's
// view: either the compiler issues the load and counts it (plain loads,
// builtins), or one inline-asm statement issues the loads and waits for them.
//
// 16-byte load as a plain load through the integer LDS address: the compiler
// counts it and waits for it before its first use, and with the pointer
// rebuilt from an integer it does not hold it back for the buffer-to-LDS
// loads in flight.  The caller makes sure the bytes have landed.
static __device__ __forceinline__ u32x4_t lds_load_b128(uint32_t addr) {
    return *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)addr;
}
// The same for 8 bytes (the compiler may pair two into one ds_read2_b64).
static __device__ __forceinline__ u32x2_t lds_load_b64(uint32_t addr) {
    return *(const __attribute__((address_space(3))) u32x2_t*)(uintptr_t)addr;
}

// N (4 or 8) transposing reads, ds_read_b64_tr_b16 (in each 16-lane group,
// lane 4j + q names 4 consecutive bf16 of a row; lane i receives element i % 4
// of lane 4j + i / 4 for j = 0..3), at lane addresses a[i] + OFF, and the wait
// for all of this wave's LDS accesses, in one asm statement.  The outputs are
// early-clobber, so no result lands on an address still to be read.  (The
// builtin would make the compiler wait for every buffer-to-LDS load in flight
// into the same LDS array.)
template <int OFF>
static __device__ __forceinline__ void tr_read_wait(const uint32_t (&a)[4], bf16x4_t (&v)[4]) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
        "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
        "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
        : "memory");
}
template <int OFF>
static __device__ __forceinline__ void tr_read_wait(const uint32_t (&a)[8], bf16x4_t (&v)[8]) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF)
        : "memory");
}

// 16-byte LDS write as inline assembly (no result register).  As a plain
// store the compiler would treat it as possibly aliasing the buffer-to-LDS
// loads in flight and wait for all of those first; the caller makes sure the
// bytes it overwrites are no longer read and that what it writes is read only
// after its own later waits (LDS executes one wave's accesses in order).
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
