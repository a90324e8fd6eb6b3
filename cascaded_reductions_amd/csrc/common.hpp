// Device-side helpers shared by the librf kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rf {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short bf16x8 __attribute__((ext_vector_type(8)));   // 8 bf16 values: one MFMA operand
typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));      // 32 fp8 values: one MFMA operand
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round to nearest even; inputs are finite.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two floats -> two bf16 (RNE) packed low/high in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane max / sum over the lanes that differ in the bits of `mask` (xor butterfly).
__device__ __forceinline__ float xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }
__device__ __forceinline__ float xor_sum(float v, int mask) { return v + __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = xor_max(v, m);
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = xor_sum(v, m);
    return v;
}

// Launch-size helper.
__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace rf

namespace rf {

// DPP lane move within a row of 16 lanes (dpp_ctrl is a compile-time constant).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes (row_ror 8, 4, 2, 1); every lane gets the total.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0x128>(v);
    v += dpp_mov<0x124>(v);
    v += dpp_mov<0x122>(v);
    v += dpp_mov<0x121>(v);
    return v;
}

// Sum over each aligned group of 8 lanes (quad_perm xor 1, xor 2, then half-row mirror).
__device__ __forceinline__ float row8_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    return v;
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane i writes LDS bytes [lds_base + 16 i, +16). lds_base must be wave-uniform.
// Issued through inline assembly so the compiler does not track the LDS write: it would
// otherwise wait for every such load before any LDS read it cannot prove disjoint,
// including loads of buffers that are only used later. The caller orders them with
// an explicit "s_waitcnt vmcnt(N)" and a barrier (vmcnt retires loads in issue order,
// so loads the compiler does not know of can only make its own waits stricter).
// The LDS base goes to M0 through the "{m0}" operand constraint, so the compiler sets M0
// itself and knows the value it holds. A global load to LDS needs one wait state after a
// scalar write of M0, which the compiler emits right before the assembly and does not
// check against it, so the wait state is part of it.
__device__ __forceinline__ void lds_dma16(const void* gptr, const void* lds_base) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds_base)));
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "{m0}"(base) : "memory");
}

// The same with a wave-uniform 64-bit global base (SGPR pair) and a per-lane 32-bit
// byte offset: the address costs no vector instruction. A vector-memory instruction that
// reads an SGPR written by a vector instruction (v_readfirstlane_b32, which the compiler
// uses when it forms the base in VGPRs) needs 5 wait states, and the compiler's hazard
// check does not see the operands of inline assembly, so the wait states (which also
// cover the one after the M0 write) are part of it.
__device__ __forceinline__ void lds_dma16_sb(const void* gbase, uint32_t voff_bytes, uint32_t lds_base) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff_bytes), "s"(gbase), "{m0}"(lds_base)
                 : "memory");
}

// A pointer the caller knows to be wave-uniform, moved to scalar registers (the direct-load
// helper above takes its global base in an SGPR pair).
template <class T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    return reinterpret_cast<const T*>((uint64_t(hi) << 32) | lo);
}

// LDS byte address of a __shared__ object (wave-uniform when the pointer is).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// Unpack a dword holding two bf16 values (low half first).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

}  // namespace rf
