// Split bf16 products with fp32 accumulation (the "bf16x3" scheme of Henry, Tang and Heinecke,
// "Leveraging the bfloat16 Artificial Intelligence Datatype For Higher-Precision Computations",
// ARITH 2019): v = hi + lo with hi = bf16(v), lo = bf16(v - hi) carries v to within 2^-16 |v|, and
// a b = ah bh + ah bl + al bh (the al bl term, below 2^-16 |a b|, dropped).  Building blocks of
// the fp32-accurate kernels on v_mfma_f32_16x16x32_bf16 (the backward's fused kernel and the fp32
// forward's attention): lane i of the MFMA holds A[i % 16][8 (i / 16) .. + 7], B[8 (i / 16) .. + 7]
// [i % 16], and C[4 (i / 16) + e][i % 16] for e < 4.
//
// Kbar / Vbar planes in LDS: [k][64] bf16 (hi and lo each), 16-byte chunks XOR-swizzled by
// (r ^ r >> 3) & 7.  Row reads (8 consecutive columns of one row) are 16-byte reads; column reads
// (8 rows of one column, the transposed operand) use ds_read_b64_tr_b16, whose lane i of a
// 16-lane group receives element i % 4 of source lanes 4 r + i / 4.
#pragma once

#include "lf_device.h"

namespace lf {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// byte offset of element (r, d) of a [k][64] bf16 plane (d % 4 == 0: 8 bytes in one chunk)
__device__ __forceinline__ int kv_off(int r, int d) {
    return r * 128 + (((d >> 3) ^ ((r ^ (r >> 3)) & 7)) << 4) + (d & 7) * 2;
}
// hi = bf16(v), lo = bf16(v - hi) of four values, as packed pairs
__device__ __forceinline__ void split4(f32x4 v, u32x2& hi, u32x2& lo) {
    uint16_t h[4], o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = f32_to_bf16(v[e]);
        o[e] = f32_to_bf16(v[e] - bf16_to_f32(h[e]));
    }
    hi = u32x2{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
    lo = u32x2{(uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
}
__device__ __forceinline__ bf16x8 pair8(u32x2 a, u32x2 b) {
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}
__device__ __forceinline__ bf16x8 lds16(const uint8_t* base, int off) {
    return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(
        (const __attribute__((address_space(3))) uint8_t*)(base + off));
}
__device__ __forceinline__ s16x4 lds_tr(const uint8_t* base, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(uintptr_t)(
            (__attribute__((address_space(3))) const uint8_t*)(base + off)));
}

// LDS loads at an absolute LDS byte address, and an address hidden from constant folding (so a
// loop-invariant per-lane base stays in one register and the constant parts of the offsets go
// into the instructions' offset fields)
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ bf16x8 lds16a(uint32_t addr) {
    return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)addr;
}
__device__ __forceinline__ s16x4 lds_tra(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
}

// Kbar and Vbar ([K][64] fp32 each, at kg and vg) into LDS as hi and lo bf16 planes at lds,
// lds + K 128, lds + 2 K 128, lds + 3 K 128 (bytes), by NT threads: every thread's loads are
// issued before the first is split, so the staging costs one load latency, not one per step
template <int K, int NT>
__device__ __forceinline__ void stage_kv(uint8_t* lds, const float* kg, const float* vg, int tid) {
    constexpr int PL = K * 128, NIT = K * 16 / NT;
    static_assert(K * 16 % NT == 0, "whole steps");
    f32x4 kx[NIT], vx[NIT];
#pragma unroll
    for (int i = 0; i < NIT; ++i) {   // 4 values (16 bytes) each
        kx[i] = *(const f32x4*)(kg + 4 * (tid + i * NT));
        vx[i] = *(const f32x4*)(vg + 4 * (tid + i * NT));
    }
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        const int e = tid + i * NT, r = e >> 4, d = 4 * (e & 15);
        const int off = kv_off(r, d);
        u32x2 hi, lo;
        split4(kx[i], hi, lo);
        *(u32x2*)(lds + off) = hi;
        *(u32x2*)(lds + PL + off) = lo;
        split4(vx[i], hi, lo);
        *(u32x2*)(lds + 2 * PL + off) = hi;
        *(u32x2*)(lds + 3 * PL + off) = lo;
    }
}

// Buffer descriptor over `rows` rows of 64 values of TQ from `base`: loads at or past them return
// zeros, so rows past a length need no branch around their loads.
template <typename TQ>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const TQ* base, int rows) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (uint32_t)rows * 64 * sizeof(TQ),
                                             0x00020000);
}

// The query row's slices d = 32 kc + 8 g .. + 7 (kc = 0, 1) of Q or dO, as loaded (rows past the
// descriptor's end: zeros), and as bf16 operands hi (and lo for fp32 inputs)
template <typename TQ>
struct RowOps {
    u32x4 raw[2][sizeof(TQ) / 2];   // 16 bytes (bf16) or 32 bytes (fp32) per slice
    __device__ void load(__amdgpu_buffer_rsrc_t rs, int row, int g) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int w = 0; w < (int)(sizeof(TQ) / 2); ++w)   // w > 0: fp32 only
                raw[kc][w] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, (uint32_t)(row * 64 + 32 * kc + 8 * g) * sizeof(TQ) + 16 * w, 0, 0);
    }
    __device__ void ops(int kc, bf16x8& hi, bf16x8& lo) const {
        if constexpr (sizeof(TQ) == 2) {
            hi = __builtin_bit_cast(bf16x8, raw[kc][0]);
        } else {
            u32x2 h0, l0, h1, l1;
            split4(__builtin_bit_cast(f32x4, raw[kc][0]), h0, l0);
            split4(__builtin_bit_cast(f32x4, raw[kc][1]), h1, l1);
            hi = pair8(h0, h1);
            lo = pair8(l0, l1);
        }
    }
};

}  // namespace lf
