// Device-side building blocks shared by the gfx950 kernels: vector types,
// bf16 packing, the bf16 MFMA, wave reductions and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_internal.h"

namespace ra {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));   // MFMA A/B operand (8 bf16)
typedef float f32x16_t __attribute__((ext_vector_type(16)));  // 32x32 MFMA accumulator
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// C[32x32] += A[32x16] * B[16x32], bf16 operands, fp32 accumulate.
// Lane l: A row (l % 32), B column (l % 32), k-group (l / 32) of 8 elements.
// C: lane l holds column (l % 32); register r holds row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Max and sum of a value over the lane pair (l, l ^ 32).  v_permlane32_swap trades the
// upper half of its first operand with the lower half of its second; with both operands
// holding x, every lane ends up with x of both lanes of its pair, in the same order in
// both halves (so the two lanes get bit-identical sums).
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The hardware hands consecutive workgroups of a launch to the 8 XCDs in
// round-robin order.  Remap the linear block id so that each XCD works on one
// contiguous range of the logical work list (which keeps the work items that
// share K/V, or Q/dO, in the same XCD's L2).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks) {
    constexpr uint32_t kXcd = 8;
    const uint32_t per = nblocks / kXcd, rem = nblocks % kXcd;
    const uint32_t xcd = bid % kXcd, slot = bid / kXcd;
    const uint32_t start = xcd * per + (xcd < rem ? xcd : rem);
    return start + slot;
}

}  // namespace ra
