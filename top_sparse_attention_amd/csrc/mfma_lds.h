// Device helpers shared by the matrix-core attention kernels: operand types, wave-wide
// global-to-LDS loads with explicit vector-memory waits, the LDS transpose read, cross-lane
// reductions over the four 16-lane groups, and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tsa_internal.h"   // TSA_LOAD_POLICY

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((lds_u8*)(p)));
}

// Wave-wide global-to-LDS load: lane i's 16 bytes land at (uniform) lds + 16 * i.
__device__ __forceinline__ void load_lds16(const void* gsrc, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" TSA_LOAD_POLICY
                 :
                 : "v"(gsrc), "s"(lds)
                 : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset.
__device__ __forceinline__ void load_lds16_s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" TSA_LOAD_POLICY
                 :
                 : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}

// Wait until at most N vector-memory instructions of this wave are outstanding.  Emitted as a
// real s_waitcnt (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their
// maxima) so that the compiler's own wait tracking sees it too.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// max over lanes l, l^16, l^32, l^48 (the four 16-lane groups), with the cross-half swaps
__device__ __forceinline__ float max4groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// two floats rounded to nearest-even bf16, packed (first in the low half)
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    const bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
}

// LDS transpose load of 4 x 16-bit.  In each 16-lane group, lane i supplies the address of 4
// consecutive elements; lane j receives element j%4 of the data addressed by lanes
// j/4, 4 + j/4, 8 + j/4, 12 + j/4.
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
    lds_i16x4* lp = (lds_i16x4*)((lds_u8*)(p));
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}

}  // namespace
