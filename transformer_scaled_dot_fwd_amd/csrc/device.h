// device.h -- gfx950 (CDNA4) primitives shared by the attention and GEMM
// kernels: vector types, the bf16 MFMA, the LDS transpose read, and
// cross-half-wave exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// D = A B + C on a 32x32x16 bf16 tile, fp32 accumulate.
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. 8*(l/32)+7
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. 8*(l/32)+7
//   D (32 x 32): lane l holds column l%32, rows
//                (r%4) + 8*(r/4) + 4*(l/32) for register r = 0..15
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator that register r of this lane holds.
__device__ __forceinline__ constexpr int acc_row(int r, int half) {
    return (r & 3) + 8 * (r >> 2) + 4 * half;
}

// LDS transpose read (ds_read_b64_tr_b16).  Inside each group of 16 lanes,
// lane 4*r + c points at 4 consecutive bf16 of "row" r (columns 4c..4c+3 of
// a 4 x 16 block); lane j of the group receives column j of that block:
// the 4 elements (row 0..3, column j).
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// v_permlane32_swap(x, x) exchanges the upper half of the first operand with
// the lower half of the second: lane l < 32 gets (x[l], x[l+32]) and lane
// l >= 32 gets (x[l-32], x[l]).  A symmetric reduction of the pair therefore
// combines lanes l and l ^ 32 with identical bits in both.
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over [base, base + bytes): a buffer load whose bytes lie
// past `bytes` returns zeros instead of touching memory.  (gfx9 descriptor
// word 3: 32-bit data format, no swizzle.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Byte offset that is out of range of every resource made here: a load
// from it returns zeros without a memory access.
constexpr uint32_t OOB_OFFSET = 0x80000000u;

// 16-byte load at per-lane byte offset `off` (the range check applies to
// this offset).
__device__ __forceinline__ bf16x8 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Workgroup barrier for LDS hand-offs: each wave's LDS reads and writes
// complete before it arrives, while its in-flight global loads (register
// prefetches and direct-to-LDS loads) keep flying; callers wait for those
// explicitly where needed (__syncthreads() would also wait for every
// outstanding global load).  The wait and the barrier are builtins so the
// compiler's own wait bookkeeping sees every LDS read retired here; the
// empty asm statements with "memory" clobbers keep memory accesses on their
// side.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    // s_waitcnt lgkmcnt(0), vmcnt and expcnt unconstrained (gfx9 encoding)
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Direct global-to-LDS load of 16 bytes per lane: lane i writes LDS bytes
// lds_base + 16 i .. + 15 from byte offset voff of the buffer (zeros past
// its end).  Issued as inline asm so the compiler adds no waits of its own
// for it: the caller waits with s_waitcnt vmcnt before the data is read.
// M0 carries the LDS base; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base,
                                           uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_base),
                 "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// 32-bit LDS address of a __shared__ object.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(p);
}

// Unpadded LDS tiles of 128-byte rows (what a direct global-to-LDS load
// writes): the eight 16-byte chunks of row r are permuted so that both read
// patterns spread over the banks.
//   Row-read tiles (16-byte reads, one row per lane): chunk c at c ^ (r & 7).
//   Transpose-read tiles (ds_read_b64_tr_b16 over 8 rows x 64 bytes): chunk c
//   at c ^ 4((r >> 1) & 1).
__device__ __forceinline__ constexpr int k_swz(int r) { return r & 7; }
__device__ __forceinline__ constexpr int v_swz(int r) { return 4 * ((r >> 1) & 1); }

// s_waitcnt vmcnt(n) leaving the other counters unconstrained (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Output store that bypasses cache retention (nontemporal): results are
// written once and never read back by the kernel, and keeping them out of
// L2 spares the writeback of dirty lines when the kernel ends.
template <typename T>
__device__ __forceinline__ void store_stream(T* p, T v) {
    __builtin_nontemporal_store(v, p);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
}

__device__ __forceinline__ bf16x8 join(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace mha
