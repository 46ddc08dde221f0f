// Device-side building blocks shared by the forward and backward kernels:
// CDNA4 (gfx950) MFMA wrappers, bf16 packing, cross-lane helpers and the
// LDS swizzles. Everything here is wave64-specific.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// D(32x32,f32) += A(32x16,bf16) * B(16x32,bf16).
// Operand layout used throughout: lane l supplies row (A) / column (B)
// l % 32 and eight consecutive-in-register values of the contraction index
// for lane group g = l / 32. A and B use the same (g, element) -> k mapping,
// so any consistent assignment of contraction indices to (g, element) is a
// valid product. Accumulator register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16_t mfma_32x32x16(const u32x4_t& a, const u32x4_t& b,
                                                  const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Same product with fp16 operands (same rate on gfx950, 3 more mantissa bits).
__device__ __forceinline__ f32x16_t mfma_32x32x16_f16(const u32x4_t& a, const u32x4_t& b,
                                                      const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two fp32 values -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2_t p = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// A packed bf16 pair times s (a power of two), as a packed fp16 pair.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, float s) {
    return pack_f16x2(__uint_as_float(w << 16) * s, __uint_as_float(w & 0xffff0000u) * s);
}

// A packed bf16 pair times s (a power of two), still bf16 (exact unless the
// result leaves the fp32 exponent range).
__device__ __forceinline__ uint32_t bf16x2_scale(uint32_t w, float s) {
    const uint32_t lo = __float_as_uint(__uint_as_float(w << 16) * s) >> 16;
    const uint32_t hi = __float_as_uint(__uint_as_float(w & 0xffff0000u) * s) & 0xffff0000u;
    return lo | hi;
}

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Value of x held by the lane 32 positions away (l ^ 32), via v_permlane32_swap.
__device__ __forceinline__ float partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    // r[0]: lanes 0-31 keep x, lanes 32-63 receive x of lanes 0-31;
    // r[1]: lanes 0-31 receive x of lanes 32-63, lanes 32-63 keep x.
    const int lane = __lane_id();
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ float max_with_partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-byte-chunk XOR swizzle for a row-major [rows][D] bf16 tile in LDS.
// D = 128: rows are 256 B (16 chunks); D = 64: rows are 128 B (8 chunks).
// Sixteen consecutive rows reading the same logical chunk land on distinct
// 16-byte bank groups (and so do eight).
template <int D>
__device__ __forceinline__ int row_chunk_swizzle(int row) {
    if constexpr (D == 128) return row & 15;
    else return (row ^ (row >> 3)) & 7;
}

template <int D>
__device__ __forceinline__ int row_chunk_offset(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ row_chunk_swizzle<D>(row)) << 4);
}

// Transposed tile layout ("[n][key]"), 64 keys per row = 128 B = 16 slots of
// 8 B. Within every group of 16 keys the order is permuted so that the eight
// keys one MFMA lane group needs are contiguous (key 16t + 8a + 4g + c is
// stored at position 16t + 8g + 4a + c), and the 8-byte slot is XORed with an
// even, row-dependent value so 16-byte reads stay aligned and consecutive rows
// spread over the banks.
__device__ __forceinline__ int tr_slot_swizzle(int n) { return ((n ^ (n >> 3)) & 7) << 1; }

__device__ __forceinline__ int tr_key_position(int key) {
    const int t = key >> 4, a = (key >> 3) & 1, g = (key >> 2) & 1, c = key & 3;
    return (t << 4) | (g << 3) | (a << 2) | c;
}

// Byte offset of the 8-byte slot that holds positions [4s, 4s+4) of row n.
__device__ __forceinline__ int tr_slot_offset(int n, int slot) {
    return n * 128 + ((slot ^ tr_slot_swizzle(n)) << 3);
}

}  // namespace fa
