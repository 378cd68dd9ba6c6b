// The attention's per-tile arithmetic, shared by the attention kernel (attend_bf16.hip) and the
// fused short-sequence kernel (fused_bf16.hip): the head's Kbar planes and Vbar resident in LDS in
// the layouts below, a 32-query tile of Q in registers, the scores (bf16 MFMA on the Kbar plane
// plus the scaled fp8 MFMA on its residual), the exact streaming softmax over the k slots and the
// weighted sum of Vbar (Linformer 요약 설명, section "Model": n x k scores, softmax over the k
// projected slots of each query, weighted sum of the projected values).
//
// LDS layout of one head (AttnLayout), bytes from its base:
//   Kbar hi : [k][64] bf16, 16-byte chunks XOR-swizzled by (r ^ r>>3) & 7 (conflict-free reads)
//   Vbar    : [k][64] bf16, 32-byte blocks XOR-swizzled by (r & 3), read with the transposing
//             ds_read_b64_tr_b16 so each lane gets 8 slots of one column
//   Kbar lo : [k][64] fp8, 16-byte chunks XOR-swizzled by (r >> 1) & 3, bytes of a row in the
//             order of the Kbar storage format (lf_launch.h)
//   scales  : [k][2] bytes, the residual's block scales
#pragma once

#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace attn {


constexpr int kTileQ = 32;
constexpr float kRaise = 32.0f;            // how far the softmax reference may lag a block max

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ int swz16(int r) { return (r ^ (r >> 3)) & 7; }

// LDS byte address of a shared-memory pointer, and loads at "opaque base + constant offset" (the
// base is hidden from constant folding so that every offset stays in the instruction's field).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}
template <class T>
__device__ __forceinline__ T lds_ld(uint32_t base, int off) {
    return *(const __attribute__((address_space(3))) T*)(uintptr_t)(base + off);
}
__device__ __forceinline__ s16x4 lds_tr16(uint32_t base, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(uintptr_t)(base + off));
}

// The value lane l ^ 32 holds (v_permlane32_swap exchanges the two 32-lane halves of the wave).
__device__ __forceinline__ float other_half(float x, bool upper) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(upper ? r[0] : r[1]);
}

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from `rsrc` at byte offset `voff` into LDS at lds_base + 16 * lane (inline asm
// so completion is tracked by the explicit waits below, not by conservative compiler waits).
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "memory");
}

// The value lane l ^ 32 holds, as raw bits.
__device__ __forceinline__ uint32_t other_half_u(uint32_t x, bool upper) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return upper ? r[0] : r[1];
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Q of this lane (32 values: columns 16 ks + 8 hh + j, j = 0..7, for ks = 0..3) as e4m3 bytes in
// the same order (byte 8 ks + j), round to nearest even: the B operand of the residual product.
// Each (query, 32-column block) gets its own power of two 2^s, chosen so that the block's largest
// |q| times 2^s lies in [128, 256): below e4m3's largest finite value (448; unscaled, elements of
// 464 and more would convert to NaN) and high enough that small queries keep their precision.
// Columns 0..31 are block 0 (bytes 0..15 of both lanes of the query), 32..63 block 1.  `qsc`
// receives 127 - s of block hh, the E8M0 scale byte the matrix core multiplies the products of
// that block back by (lane 32 b + q supplies block b of query q).
__device__ __forceinline__ i32x8 q_fp8(const bf16x8 (&qop)[4], bool upper, int& qsc) {
    // largest magnitude per block: bf16 magnitudes order like their bit patterns without the sign
    uint32_t mb[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const u32x4 w0 = __builtin_bit_cast(u32x4, qop[2 * blk]);
        const u32x4 w1 = __builtin_bit_cast(u32x4, qop[2 * blk + 1]);
        uint32_t m = w0[0] & 0x7FFF7FFFu;
#pragma unroll
        for (int i = 1; i < 4; ++i) m = max_u16x2(m, w0[i] & 0x7FFF7FFFu);
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max_u16x2(m, w1[i] & 0x7FFF7FFFu);
        mb[blk] = m;
    }
    // (block 0, block 1) maxima of this lane's 16-bit halves, then of the query's two lanes
    uint32_t m = max_u16x2(__builtin_amdgcn_perm(mb[1], mb[0], 0x05040100u),
                           __builtin_amdgcn_perm(mb[1], mb[0], 0x07060302u));
    m = max_u16x2(m, other_half_u(m, upper));
    // 127 - s = biased exponent of the block max - 7, kept in [1, 247] (zero blocks take s = 126)
    const int sb0 = min(max((int)((m >> 7) & 0xFF) - 7, 1), 247);
    const int sb1 = min(max((int)((m >> 23) & 0xFF) - 7, 1), 247);
    qsc = upper ? sb1 : sb0;
    // the conversion divides by its scale operand: 2^(127 - s - 127) = 2^-s
    const float dv[2] = {__uint_as_float((uint32_t)sb0 << 23), __uint_as_float((uint32_t)sb1 << 23)};
    // v_cvt_scalef32_pk_fp8_bf16 converts a bf16 pair straight into one 16-bit half of the
    // destination, keeping the other half (op_sel[2] picks the high half).  Inline asm with the
    // destination tied, so that both halves are written into the same register in order.
    i32x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4 w = __builtin_bit_cast(u32x4, qop[i >> 1]);
        const float d = dv[i >> 2];
        uint32_t v = 0;
        asm volatile("v_cvt_scalef32_pk_fp8_bf16 %0, %1, %2" : "+v"(v) : "v"(w[2 * (i & 1)]), "v"(d));
        asm volatile("v_cvt_scalef32_pk_fp8_bf16 %0, %1, %2 op_sel:[0,0,1]" : "+v"(v) : "v"(w[2 * (i & 1) + 1]), "v"(d));
        r[i] = (int)v;
    }
    return r;
}

// acc + (residual block of 32 slots) . (Q e4m3): the A operand's two 32-column blocks of row l32
// are scaled by 2^(byte - 127) with the byte taken from byte `SEL` of `scl` in lanes l32 (block 0)
// and l32 + 32 (block 1); the B operand's blocks of query l32 likewise by byte 0 of `qsc`.
template <int SEL>
__device__ __forceinline__ f32x16 mfma_lo_sel(i32x8 lo, i32x8 q8, f32x16 acc, int scl, int qsc) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lo, q8, acc, 0, 0, SEL, scl, 0, qsc);
}
__device__ __forceinline__ f32x16 mfma_lo(int sel, i32x8 lo, i32x8 q8, f32x16 acc, int scl,
                                          int qsc) {
    switch (sel) {   // sel is a compile-time constant after unrolling
        case 0: return mfma_lo_sel<0>(lo, q8, acc, scl, qsc);
        case 1: return mfma_lo_sel<1>(lo, q8, acc, scl, qsc);
        case 2: return mfma_lo_sel<2>(lo, q8, acc, scl, qsc);
        default: return mfma_lo_sel<3>(lo, q8, acc, scl, qsc);
    }
}


template <int KB>
struct AttnLayout {
    static constexpr int K = KB * 32;
    static constexpr int PLANE = K * 128;   // bytes of one k x 64 bf16 plane
    static constexpr int LOB = K * 64;      // bytes of the fp8 residual plane
    static constexpr int OFF_V = PLANE, OFF_L = 2 * PLANE, OFF_S = 2 * PLANE + LOB;
    static constexpr int BYTES = OFF_S + 1024;   // scales: K * 2 <= 512 B, padded
};

// Per-lane operand addresses into a head's planes at lds0: every LDS read is an opaque per-lane
// base plus a compile-time offset below 64 KB.
struct Lanes {
    uint32_t kaddr[4][2];   // Kbar hi row 32 rb + l32, chunk 2 ks + hh, by slot-block parity
    uint32_t vaddr[2];      // Vbar^T operand rows, by 32-column half
    uint32_t laddr[2];      // Kbar lo row 32 rb + l32, chunks 2 hh and 2 hh + 1
};

template <int KB>
__device__ __forceinline__ Lanes attn_lanes(uint32_t lds0, int lane) {
    using Ly = AttnLayout<KB>;
    const int l32 = lane & 31, hh = lane >> 5;
    Lanes ln;
    //   Kbar hi row r = 32 rb + l32: swizzle (r ^ r>>3) & 7 = bsw ^ 4 (rb & 1), bsw from l32 alone.
    const int bsw = (l32 ^ (l32 >> 3)) & 7;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int par = 0; par < 2; ++par)
            ln.kaddr[ks][par] = opaque(lds0 + l32 * 128 + (((2 * ks + hh) ^ bsw ^ (4 * par)) << 4));
    //   Vbar rows 32 rb + 16 al + 8 rd + trow: the 32-byte block swizzle only sees trow & 3.
    const int grp16 = lane >> 4, s16 = lane & 15;
    const int trow = 4 * (grp16 >> 1) + (s16 >> 2);
    const int tcb = grp16 & 1;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        ln.vaddr[mt] = opaque(lds0 + Ly::OFF_V + trow * 128 + (((2 * mt + tcb) ^ (trow & 3)) << 5) + (s16 & 3) * 8);
    //   Kbar lo row 32 rb + l32, this lane's half hh = chunks 2 hh, 2 hh + 1, swizzle (l32 >> 1) & 3
#pragma unroll
    for (int part = 0; part < 2; ++part)
        ln.laddr[part] = opaque(lds0 + Ly::OFF_L + l32 * 64 + (((2 * hh + part) ^ ((l32 >> 1) & 3)) << 4));
    return ln;
}

// Block scales of this lane's residual rows: byte rb & 3 of scl[rb >> 2] is the scale of row
// 32 rb + l32, block hh.
template <int KB>
__device__ __forceinline__ void attn_scales(const uint8_t* head, int lane, int (&scl)[2]) {
    using Ly = AttnLayout<KB>;
    const int l32 = lane & 31, hh = lane >> 5;
    scl[0] = scl[1] = 0;
#pragma unroll
    for (int rb = 0; rb < KB; ++rb)
        scl[rb >> 2] |= (int)head[Ly::OFF_S + (32 * rb + l32) * 2 + hh] << (8 * (rb & 3));
}

// One 32-query tile against the head in LDS.  qop: this lane's Q operand (columns
// 16 ks + 8 hh + (0..7) of query l32).  Returns the unnormalised output blocks o0, o1 (O^T,
// columns 0..31 and 32..63) and the weight sum z of the lane's query (both lanes summed).
// `bias` holds -mref, the score accumulators' start value (zero unless bias_dirty).  on_last()
// runs once the last block's score products are issued (the caller prefetches there).
//   1. S^T (k x 32) = Kbar . Q^T: per 32 slots four v_mfma_f32_32x32x16_bf16 for the hi plane
//      times Q, then one v_mfma_scale_f32_32x32x64_f8f6f4 for the residual (fp8 lo plane times Q
//      rounded to e4m3 with a power-of-two scale per query and 32-column block, both scaled back
//      by their block scales), so the scores carry Kbar to within 2^-12 of each row half's
//      largest value.  The accumulators start from -mref (see 2), so they hold s - mref.
//   2. Exact softmax per query in one streaming pass over blocks of 64 slots: the scores of a query
//      sit in lanes l and l + 32, so the block max is an in-register reduction plus one exchange
//      of the wave halves.  The reference mref starts at 0 and moves to the block max only when
//      that exceeds it by more than kRaise (or, in the first block, lies more than kRaise below
//      it); then the partial sums are rescaled.  Weights w = exp2(s - mref) stay in
//      [2^-32, 2^32] at the maximum, far inside fp32 and bf16 range, and numerator and
//      denominator share mref, so the normalisation is exact.
//   3. O^T (64 x 32) = Vbar^T . W^T with the unnormalised weights rounded to bf16 as the B operand
//      straight from the score accumulators: lane (l, h) holds, for slot block rb, the weights of
//      slots 32 rb + 8 (j/4) + 4 h + j%4, and the Vbar^T operand is read at exactly those slots
//      (no permutation in memory).  The row sum z adds the same rounded weights (v_dot2 with
//      (1, 1)).
//   The score MFMAs of block j+1 are issued before the softmax of block j so that matrix and
//   vector work interleave within the wave.
template <int KB, class OnLast>
__device__ __forceinline__ void tile_math(const Lanes& ln, const bf16x8 (&qop)[4],
                                          const int (&scl)[2], int hh, f32x16& bias,
                                          bool& bias_dirty, f32x16& o0, f32x16& o1, float& z,
                                          OnLast&& on_last) {
    if (bias_dirty) {
#pragma unroll
        for (int j = 0; j < 16; ++j) asm volatile("v_mov_b32 %0, 0" : "+v"(bias[j]));
        bias_dirty = false;
    }
    int qsc;
    const i32x8 q8 = q_fp8(qop, hh, qsc);

    constexpr int NBLK = (KB + 1) / 2;
    f32x16 sc[2][2];   // [buffer][rb within block]
    auto scores = [&](int blk, f32x16* dst) {
        const int nrb = min(2, KB - 2 * blk);
        // hi plane first (the first MFMA starts from the bias), the residual last
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                if (r2 < nrb) {
                    const int rb = 2 * blk + r2;
                    const bf16x8 kh = lds_ld<bf16x8>(ln.kaddr[ks][rb & 1], rb * 4096);
                    dst[r2] = mfma32(kh, qop[ks], ks == 0 ? bias : dst[r2]);
                }
            }
        }
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            if (r2 < nrb) {
                const int rb = 2 * blk + r2;
                const u32x4 l0 = lds_ld<u32x4>(ln.laddr[0], rb * 2048);
                const u32x4 l1 = lds_ld<u32x4>(ln.laddr[1], rb * 2048);
                const i32x8 lop = __builtin_bit_cast(
                    i32x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
                dst[r2] = mfma_lo(rb & 3, lop, q8, dst[r2], scl[rb >> 2], qsc);
            }
        }
    };

#pragma unroll
    for (int j = 0; j < 16; ++j) {
        o0[j] = 0.0f;
        o1[j] = 0.0f;
    }
    z = 0.0f;

    scores(0, sc[0]);
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
        const int cur = blk & 1;
        if (blk + 1 < NBLK) scores(blk + 1, sc[cur ^ 1]);
        else on_last();
        __builtin_amdgcn_sched_barrier(0);
        const int nrb = min(2, KB - 2 * blk);
        // block max of s - mref (both lanes of a query)
        float bm = sc[cur][0][0];
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
            if (r2 < nrb)
#pragma unroll
                for (int j = 0; j < 16; ++j) bm = fmaxf(bm, sc[cur][r2][j]);
        bm = fmaxf(bm, other_half(bm, hh));
        const bool move = bm > kRaise || (blk == 0 && bm < -kRaise);
        if (__builtin_amdgcn_ballot_w64(move)) {   // rare: move mref to the block max
            const float sh = move ? bm : 0.0f;
            if (blk > 0) {
                const float alpha = __builtin_amdgcn_exp2f(-sh);
                o0 *= alpha;
                o1 *= alpha;
                z *= alpha;
            }
            // in place (tied operands), so the common path needs no register copies
#pragma unroll
            for (int j = 0; j < 16; ++j) asm volatile("v_sub_f32 %0, %0, %1" : "+v"(bias[j]) : "v"(sh));
            bias_dirty = true;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                if (r2 < nrb) sc[cur][r2] -= sh;
                if (blk + 1 < NBLK && r2 < min(2, KB - 2 * (blk + 1))) sc[cur ^ 1][r2] -= sh;
            }
        }
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            if (r2 >= nrb) continue;
            const int rb = 2 * blk + r2;
            float wv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) wv[j] = __builtin_amdgcn_exp2f(sc[cur][r2][j]);
#pragma unroll
            for (int al = 0; al < 2; ++al) {
                const bf16x8 pw = pack_bf16x8(wv[8 * al], wv[8 * al + 1], wv[8 * al + 2],
                                              wv[8 * al + 3], wv[8 * al + 4],
                                              wv[8 * al + 5], wv[8 * al + 6],
                                              wv[8 * al + 7]);
                // row sum of the rounded weights the matrix cores use (two per v_dot2)
                z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pw, pw, 0, 1), kOnes2, z, false);
                z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pw, pw, 2, 3), kOnes2, z, false);
                z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pw, pw, 4, 5), kOnes2, z, false);
                z = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pw, pw, 6, 7), kOnes2, z, false);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    // Vbar^T operand: columns 32 mt + l32,
                    // slots 32 rb + 16 al + 4 h + {0..3, 8..11}
                    const int vo = rb * 4096 + al * 2048;
                    const s16x4 v0 = lds_tr16(ln.vaddr[mt], vo);
                    const s16x4 v1 = lds_tr16(ln.vaddr[mt], vo + 1024);
                    const bf16x8 vop = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                    if (mt == 0) o0 = mfma32(vop, pw, o0);
                    else o1 = mfma32(vop, pw, o1);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    z += other_half(z, hh);
}

// Per-lane offsets of the tile staging buffer: row 8 i + lane / 8, 16-byte chunk lane % 8,
// chunks swizzled by swz16(row).
__device__ __forceinline__ void stage_offsets(int lane, uint32_t (&coff)[4]) {
    const int crow = lane >> 3, ccol = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + crow;
        coff[i] = r * 128 + ((ccol ^ swz16(r)) << 4);
    }
}

// Raw Q rows (as loaded: row 8 i + lane / 8, chunk lane % 8) -> the wave's staging buffer -> the
// operand layout.  The LDS operations of a wave execute in issue order, so a read issued after a
// write sees it (no counter wait in between, only a compiler barrier against reordering), and
// the previous tile's output staging reads are done before these writes land.
__device__ __forceinline__ void stage_q(uint32_t stg, const uint32_t (&coff)[4],
                                       const u32x4 (&qraw)[4], int lane, bf16x8 (&qop)[4]) {
    const int l32 = lane & 31, hh = lane >> 5;
    const int sw_l = swz16(l32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(stg + coff[i]) = qraw[i];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        qop[ks] = lds_ld<bf16x8>(stg, l32 * 128 + (((2 * ks + hh) ^ sw_l) << 4));
}

// Normalises and stores one tile: lane holds O[q0 + l32][c] for c = 32 mt + 8 gq + 4 hh + (0..3),
// i.e. 8 bytes of chunk 4 mt + gq; staged, then written as whole rows with streaming stores
// (rows at or past L as zeros).  dst: row q0 of this head's O.
__device__ __forceinline__ void tile_store(uint32_t stg, const uint32_t (&coff)[4], int lane,
                                           const f32x16& o0, const f32x16& o1, float z,
                                           uint16_t* dst_rows, int q0, int L) {
    const int l32 = lane & 31, hh = lane >> 5, crow = lane >> 3;
    const int sw_l = swz16(l32);
    const float inv = 1.0f / z;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
        const u32x2 v0 = {pack_bf16x2(o0[4 * gq] * inv, o0[4 * gq + 1] * inv),
                          pack_bf16x2(o0[4 * gq + 2] * inv, o0[4 * gq + 3] * inv)};
        const u32x2 v1 = {pack_bf16x2(o1[4 * gq] * inv, o1[4 * gq + 1] * inv),
                          pack_bf16x2(o1[4 * gq + 2] * inv, o1[4 * gq + 3] * inv)};
        *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(
            stg + l32 * 128 + ((gq ^ sw_l) << 4) + 8 * hh) = v0;
        *(__attribute__((address_space(3))) u32x2*)(uintptr_t)(
            stg + l32 * 128 + (((4 + gq) ^ sw_l) << 4) + 8 * hh) = v1;
    }
    __builtin_amdgcn_wave_barrier();
    u32x4* dst = (u32x4*)dst_rows + lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u32x4 v = lds_ld<u32x4>(stg, coff[i]);
        if (q0 + 8 * i + crow >= L) v = u32x4{0u, 0u, 0u, 0u};
        __builtin_nontemporal_store(v, &dst[64 * i]);
    }
}

}  // namespace attn
}  // namespace lf
