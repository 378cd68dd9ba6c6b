// Device-side building blocks shared by the liblinformer kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, one wave of 64 lanes):
//   lane i, h = i / 32, l = i % 32
//   A operand (32 x 16): lane i holds 8 bf16 A[l][8h .. 8h+7]
//   B operand (16 x 32): lane i holds 8 bf16 B[8h .. 8h+7][l]
//   C/D (32 x 32 fp32) : lane i, element j (0..15) holds C[8*(j/4) + 4h + (j%4)][l]
// Only the row/column placement matters for correctness: the eight reduction indices a lane
// supplies are the same set for A and B, so any consistent relabelling of the reduction axis
// (used below to feed softmax weights straight from a C tile into a B operand) is exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf_launch.h"

namespace lf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 64;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 -> two bf16 (round to nearest even, hardware v_cvt_pk_bf16_f32), packed low-first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

// Eight fp32 -> bf16x8 operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
    u32x4 u = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5),
               pack_bf16x2(a6, a7)};
    return __builtin_bit_cast(bf16x8, u);
}

// ---- Kbar lo-plane encoding (layout in lf_launch.h)
// Byte of column d within a lo row.
__device__ __forceinline__ int lo_pos(int d) { return ((d >> 3) & 1) * 32 + (d >> 4) * 8 + (d & 7); }
// Block shift s for a block whose largest residual magnitude is m: 2^s m in [128, 256), clamped
// to the exponent range of the E8M0 scale byte 127 - s (m == 0 gives the smallest scale).
__device__ __forceinline__ int lo_shift(float m) {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xFF) - 127;   // floor(log2 m), m normal
    const int s = 7 - e;
    return s < -127 ? -127 : (s > 127 ? 127 : s);
}
// Four residuals -> four e4m3 bytes (round to nearest even) of lo * 2^s.
__device__ __forceinline__ uint32_t lo_bytes(float l0, float l1, float l2, float l3, int s) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(l0, s), ldexpf(l1, s), 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(l2, s), ldexpf(l3, s), w, true);
}
// bf16 hi of x and the fp32 residual x - hi.
__device__ __forceinline__ uint32_t hi_pair(float x0, float x1, float& r0, float& r1) {
    const uint32_t h = pack_bf16x2(x0, x1);
    r0 = x0 - __uint_as_float(h << 16);
    r1 = x1 - __uint_as_float(h & 0xFFFF0000u);
    return h;
}

__device__ __forceinline__ int clamp_len(const int32_t* lengths, int b, int n) {
    if (lengths == nullptr) return n;
    int L = lengths[b];
    return L < 0 ? 0 : (L > n ? n : L);
}

// Block-index remap so that logically consecutive blocks land on the same XCD.  The hardware
// hands workgroups to the 8 XCDs round-robin by dispatch order; each XCD has its own L2, so
// blocks that read the same operand (a projection chunk of E, or one head's Kbar/Vbar) should
// share an XCD.  Grid = 8 * per; returns -1 for the padding blocks.
__device__ __forceinline__ int xcd_remap(int bid, int nlogical) {
    const int per = (nlogical + 7) >> 3;
    const int lid = (bid & 7) * per + (bid >> 3);
    return lid < nlogical ? lid : -1;
}

}  // namespace lf
