// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}
// low / high halves of a packed pair
__device__ __forceinline__ float bf16lo_to_f32(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 round-to-nearest-even (NaN kept quiet): gfx950's v_cvt_pk_bf16_f32, which
// converts two values per instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}

// SiLU(z) = z / (1 + exp(-z)), the quotient taken with the hardware reciprocal (1 ulp;
// the result is rounded to bf16 afterwards).  For z << 0, exp(-z) overflows to +inf, its
// reciprocal is 0 and the product -0, the limit.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// ------------------------------------------------ direct-to-LDS operand loads (DMA)
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kOOB = 0x80000000u;          // an offset past every buffer: reads zeros

// A raw buffer resource over [base, base + bytes): loads past the end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Swizzle of LDS rows of 64 bytes (four 16-byte chunks, one K step of 32 bf16): chunk q of
// row m sits at slot q ^ swa4(m).  On gfx950 a ds_read_b128 serves 16 lanes per LDS cycle
// (64 banks), grouped by bit2^bit3^bit4 of the lane index (lanes 0-3, 12-15 and 20-27
// share a cycle; measured with the bank-conflict counter); an MFMA fragment read has lane
// l on row l & 15, chunk l >> 4.  With swa4(m) = (m >> 1) & 2 the 16 lanes of every cycle
// land on distinct bank quads.
__device__ __forceinline__ int swa4(int m) { return (m >> 1) & 2; }

}  // namespace moe
