// Compressed attention O = softmax(scale * Q . Kbar^T) . Vbar for bf16 inputs (Linformer 요약 설명,
// section "Model": n x k scores, softmax over the k projected slots of each query, weighted sum of
// Vbar; queries are not compressed, so there is one output row per position).
//
// Persistent kernel: one workgroup (8 waves) per compute unit.  The work is the list of valid
// 32-query tiles of every (b, h) (tiles wholly past a sequence's length hold no work), split into
// equal contiguous ranges, one per workgroup; consecutive workgroups go to the same XCD so the
// workgroups that share a head's Kbar/Vbar share an L2.  The lengths are read once into LDS
// tables (length and valid-tile prefix per batch item).  Rows past the lengths are zero-filled
// with streaming stores issued early in each workgroup's tile work, spread evenly over the
// workgroups.
//
// Kbar arrives pre-scaled by c = scale * log2(e) (so scores come out as base-2 logits) as a bf16
// plane plus an fp8 residual plane with per-block scales (format in lf_launch.h).  Per (b, h)
// segment of its range a workgroup copies the head's Kbar planes and Vbar into LDS with
// direct-to-LDS buffer loads (about 80 KB at k = 256) and keeps them resident:
//   Kbar hi : [k][64] bf16, 16-byte chunks XOR-swizzled by (r ^ r>>3) & 7 (conflict-free reads)
//   Vbar    : [k][64] bf16, 32-byte blocks XOR-swizzled by (r & 3), read with the transposing
//             ds_read_b64_tr_b16 so each lane gets 8 slots of one column
//   Kbar lo : [k][64] fp8, 16-byte chunks XOR-swizzled by (r >> 1) & 3; block scales [k][2]
// Per wave and tile of 32 queries:
//   1. S^T (k x 32) = Kbar . Q^T: per 32 slots four v_mfma_f32_32x32x16_bf16 for the hi plane
//      times Q, then one v_mfma_scale_f32_32x32x64_f8f6f4 for the residual (fp8 lo plane times Q
//      rounded to e4m3 with a power-of-two scale per query and 32-column block, both scaled back
//      by their block scales), so the scores carry Kbar to within
//      2^-12 of each row half's largest value.  The accumulators start from -mref (see 2), so
//      they hold s - mref directly.
//   2. Exact softmax per query in one streaming pass over blocks of 64 slots: the scores of a query
//      sit in lanes l and l + 32, so the block max is an in-register reduction plus one exchange
//      of the wave halves.  The reference mref starts at 0 and moves to the block max only when
//      that exceeds it by more than 32 (or, in the first block, lies more than 32 below it); then
//      the partial sums are rescaled.  Weights w = exp2(s - mref) stay in [2^-32, 2^32] at the
//      maximum, far inside fp32 and bf16 range, and numerator and denominator share mref, so the
//      normalisation is exact.
//   3. O^T (64 x 32) = Vbar^T . W^T with the unnormalised weights rounded to bf16 as the B operand
//      straight from the score accumulators: lane (l, h) holds, for slot block rb, the weights of
//      slots 32 rb + 8 (j/4) + 4 h + j%4, and the Vbar^T operand is read at exactly those slots
//      (no permutation in memory).  The row sum z adds the same rounded weights (v_dot2 with
//      (1, 1)), and each output column (one query) is divided by it.
//   The score MFMAs of block j+1 are issued before the softmax of block j so that matrix and
//   vector work interleave within the wave.
// Q and O move between HBM and the wave as whole rows: a 32-query tile is 4 KB of contiguous
// memory, loaded (and stored) by four 1 KB wave instructions and rearranged through a 4 KB
// per-wave LDS staging buffer into (out of) the operand layout, in which each lane holds 16 or 8
// bytes of every one of 32 rows.  O and the zero rows are written with streaming
// (non-temporal) stores: this kernel never reads them back, and lines that do not linger dirty in
// L2 leave less to write back when the kernel ends.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kThreads = kAttendThreads;   // 8 waves
constexpr int kTileQ = 32;
constexpr float kRaise = 32.0f;            // see step 2 above

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

// Tile index -> (b, h, j) for the valid-tile list: batch-major, then head, then tile.  cum[b] is
// the number of valid tiles (all heads) before batch item b; the lookup is a binary search for the
// last b with cum[b] <= t (that b has at least one tile, since t < cum[B]).
struct TilePos {
    int b, h, j, ntb;   // ntb = valid tiles per (b, h) of this batch item
};
__device__ __forceinline__ TilePos tile_pos(const int* cum, const int* len, int B, int t) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cum[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    TilePos p;
    p.b = lo;
    p.ntb = (len[lo] + kTileQ - 1) / kTileQ;
    const int rel = t - cum[lo];
    p.h = rel / p.ntb;
    p.j = rel - p.h * p.ntb;
    return p;
}

template <int KB>
__global__ __launch_bounds__(kThreads) void attend_bf16_kernel(AttendBf16Args a) {
    constexpr int K = KB * 32;
    constexpr int PLANE = K * 128;                 // bytes of one k x 64 bf16 plane
    constexpr int LOB = K * 64;                    // bytes of the fp8 residual plane
    constexpr int OFF_V = PLANE, OFF_L = 2 * PLANE, OFF_S = 2 * PLANE + LOB;
    __shared__ __attribute__((aligned(16))) uint8_t smem[OFF_S + 1024];   // scales: K*2 <= 512 B
    __shared__ int s_next;   // next tile of the current segment (relative to its start)
    __shared__ int s_len[kMaxAttendBatch];       // clamped length per batch item
    __shared__ int s_cum[kMaxAttendBatch + 1];   // valid tiles (all heads) before each batch item
    // per-wave staging of one 32-query tile (32 rows x 128 bytes, 16-byte chunks swizzled by
    // swz16(row)): Q on its way in and O on its way out, so that both move between HBM and the
    // wave as whole contiguous rows (each wave instruction covers 1 KB, eight full rows)
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[kThreads / 64][kTileQ * 128];
    const uint32_t lds0 = lds_addr(smem);

    const int G = gridDim.x;
    const int w = xcd_remap(blockIdx.x, G);   // G is a multiple of 8, so every block is mapped
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

    // ---- lengths -> LDS: clamped length per batch item and the valid-tile prefix over batch items
    // (one round of loads, then a scan), so no later step waits on global memory for them
    if (a.B <= 64) {
        // one wave: lane b holds batch item b, inclusive scan by shuffles
        if (wave == 0) {
            const int L = lane < a.B ? clamp_len(a.lengths, lane, a.n) : 0;
            const int ntb = (L + kTileQ - 1) / kTileQ;
            int inc = ntb;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(inc, off);
                if (lane >= off) inc += v;
            }
            if (lane < a.B) {
                s_len[lane] = L;
                s_cum[lane] = (inc - ntb) * a.H;
            }
            if (lane == a.B - 1) s_cum[a.B] = inc * a.H;
        }
        __syncthreads();
    } else {
        const int per = (a.B + kThreads - 1) / kThreads;
        const int b0 = min(a.B, tid * per), b1 = min(a.B, b0 + per);
        int run = 0;
        for (int b = b0; b < b1; ++b) {
            const int L = clamp_len(a.lengths, b, a.n);
            s_len[b] = L;
            run += (L + kTileQ - 1) / kTileQ;
        }
        int* scan = (int*)smem;   // the Kbar/Vbar planes are not loaded yet
        scan[tid] = run;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            const int v = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += v;
            __syncthreads();
        }
        int excl = scan[tid] - run;
        for (int b = b0; b < b1; ++b) {
            s_cum[b] = excl * a.H;
            excl += (s_len[b] + kTileQ - 1) / kTileQ;
        }
        if (tid == kThreads - 1) s_cum[a.B] = scan[tid] * a.H;
        __syncthreads();
    }
    const int T = s_cum[a.B];   // valid tiles in total

    // ---- this workgroup's valid tiles
    const int t_lo = (int)((long long)T * w / G), t_hi = (int)((long long)T * (w + 1) / G);

    // per-lane operand addressing: every LDS read is an opaque per-lane base plus a compile-time
    // offset below 64 KB.
    //   Kbar hi row r = 32 rb + l32: swizzle (r ^ r>>3) & 7 = bsw ^ 4 (rb & 1), bsw from l32 alone.
    const int bsw = (l32 ^ (l32 >> 3)) & 7;
    uint32_t kaddr[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int par = 0; par < 2; ++par)
            kaddr[ks][par] = opaque(lds0 + l32 * 128 + (((2 * ks + hh) ^ bsw ^ (4 * par)) << 4));
    //   Vbar rows 32 rb + 16 al + 8 rd + trow: the 32-byte block swizzle only sees trow & 3.
    const int grp16 = lane >> 4, s16 = lane & 15;
    const int trow = 4 * (grp16 >> 1) + (s16 >> 2);
    const int tcb = grp16 & 1;
    uint32_t vaddr[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        vaddr[mt] = opaque(lds0 + OFF_V + trow * 128 + (((2 * mt + tcb) ^ (trow & 3)) << 5) + (s16 & 3) * 8);
    //   Kbar lo row 32 rb + l32, this lane's half hh = chunks 2 hh, 2 hh + 1, swizzle (l32 >> 1) & 3
    uint32_t laddr[2];
#pragma unroll
    for (int part = 0; part < 2; ++part)
        laddr[part] = opaque(lds0 + OFF_L + l32 * 64 + (((2 * hh + part) ^ ((l32 >> 1) & 3)) << 4));

    // ---- zero the rows wholly past each length.  Each wave issues its share once its first
    // tile's Q is in registers, so the streaming stores drain under the tile work (the next wait
    // that counts them is for the Q prefetch, a whole tile later); the chunks are split by thread,
    // so waves may do this at different times.  Per (b, h) those rows are one contiguous
    // block of per_h 16-byte chunks; concatenated over (b, h) the blocks of batch item b start at
    // chunk zb(b) = 8 (b H n - 32 cum[b]), and each workgroup zeroes an equal share of the chunks.
    bool zeroed = false;
    auto zero_fill = [&]() {
        zeroed = true;
        const long long Z = 8LL * ((long long)a.B * a.H * a.n - 32LL * T);
        if (Z <= 0) return;
        const long long z0 = Z * w / G, z1 = Z * (w + 1) / G;
        auto zb = [&](int b) { return 8LL * ((long long)b * a.H * a.n - 32LL * s_cum[b]); };
        int b = 0, hi = a.B - 1;   // last batch item whose blocks start at or before z0
        while (b < hi) {
            const int mid = (b + hi + 1) >> 1;
            if (zb(mid) <= z0) b = mid;
            else hi = mid - 1;
        }
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (; b < a.B && zb(b) < z1; ++b) {
            const int r0 = ((s_len[b] + kTileQ - 1) / kTileQ) * kTileQ;
            const long long per_h = (long long)(a.n - r0) * 8;
            long long base = zb(b);
            for (int h = 0; h < a.H && base < z1; ++h, base += per_h) {
                const long long lo = max(z0, base), hi2 = min(z1, base + per_h);
                if (lo >= hi2) continue;
                u32x4* blk = (u32x4*)(a.O + ((size_t)(b * a.H + h) * a.n + r0) * kHeadDim);
                for (int c = (int)(lo - base) + tid; c < (int)(hi2 - base); c += kThreads)
                    __builtin_nontemporal_store(zero, &blk[c]);
            }
        }
    };

    int t = t_lo;
    while (t < t_hi) {
        const TilePos p0 = tile_pos(s_cum, s_len, a.B, t);
        const int seg_end = min(t_hi, t + (p0.ntb - p0.j));   // tiles of this (b, h) in range
        const int bh = p0.b * a.H + p0.h;
        const int L = s_len[p0.b];
        const size_t rowbase = (size_t)bh * a.n;

        // ---- fill LDS with this head's Kbar planes and Vbar
        __syncthreads();   // previous segment's readers are done with the LDS planes
        {
            const size_t off = (size_t)bh * K * kHeadDim;
            const i32x4 rh = make_rsrc(a.Khi + off, PLANE);
            const i32x4 rv = make_rsrc(a.Vb + off, PLANE);
            const i32x4 rl = make_rsrc(a.Klo + off, LOB);
            const i32x4 rs = make_rsrc(a.Ksc + (size_t)bh * K * 2, K * 2);
            const int lrow = lane >> 3, lpc = lane & 7;
            for (int I = wave; I < K / 8; I += 8) {   // 8 rows of 128 bytes per instruction
                const int r = I * 8 + lrow;
                const int lck = lpc ^ swz16(r);
                const int lcv = 2 * ((lpc >> 1) ^ (r & 3)) + (lpc & 1);
                dma16(rh, lds0 + I * 1024, (uint32_t)(r * 128 + lck * 16));
                dma16(rv, lds0 + OFF_V + I * 1024, (uint32_t)(r * 128 + lcv * 16));
            }
            for (int I = wave; I < K / 16; I += 8) {  // 16 rows of 64 bytes per instruction
                const int r = I * 16 + (lane >> 2), ch = lane & 3;
                dma16(rl, lds0 + OFF_L + I * 1024, (uint32_t)(r * 64 + ((ch ^ ((r >> 1) & 3)) << 4)));
            }
            if (wave == 0) dma16(rs, lds0 + OFF_S, (uint32_t)(lane * 16));   // past K*2: zeros
            __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));   // vmcnt(0)
            if (tid == 0) s_next = 8;   // tiles t .. t+7 are taken statically below
        }
        __syncthreads();
        // block scales of this lane's residual rows: byte rb & 3 of scl[rb >> 2] is the scale of
        // row 32 rb + l32, block hh
        int scl[2] = {0, 0};
#pragma unroll
        for (int rb = 0; rb < KB; ++rb)
            scl[rb >> 2] |= (int)smem[OFF_S + (32 * rb + l32) * 2 + hh] << (8 * (rb & 3));

        // ---- tiles of this segment, taken dynamically by the waves from an LDS counter (so waves
        // that finish early take more), Q of the next tile prefetched during the current one
        int tt = t + wave;
        bf16x8 qop[4];   // operand layout: columns 16 ks + 8 hh + (0..7) of query q0 + l32
        u32x4 qraw[4];   // the tile as loaded: row 8 i + lane / 8, chunk lane % 8, i = 0..3
        auto load_q = [&](int tile) {
            const int q0 = (p0.j + (tile - t)) * kTileQ;
            const u32x4* src = (const u32x4*)(a.Q + (rowbase + q0) * kHeadDim) + lane;
#pragma unroll
            for (int i = 0; i < 4; ++i) qraw[i] = src[64 * i];
        };
        // lane's chunk of the coalesced layout: row 8 i + crow, chunk ccol, at this LDS offset
        const int crow = lane >> 3, ccol = lane & 7;
        uint32_t coff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + crow;
            coff[i] = r * 128 + ((ccol ^ swz16(r)) << 4);
        }
        const uint32_t stg = lds_addr(&s_stage[wave][0]);
        const int sw_l = swz16(l32);
        // raw Q -> staging -> operand layout.  The LDS operations of a wave execute in issue
        // order, so a read issued after a write sees it (no counter wait in between, only a
        // compiler barrier against reordering), and the previous tile's output staging reads are
        // done before these writes land.
        auto stage_q = [&]() {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(__attribute__((address_space(3))) u32x4*)(uintptr_t)(stg + coff[i]) = qraw[i];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qop[ks] = lds_ld<bf16x8>(stg, l32 * 128 + (((2 * ks + hh) ^ sw_l) << 4));
        };
        // the counter's reply (lane 0) is read into a scalar only where the tile is first needed,
        // so the atomic's round trip overlaps the current tile's work
        auto grab_raw = [&]() {
            int v = 0;
            if (lane == 0) v = atomicAdd(&s_next, 1);
            return v;
        };
        f32x16 bias;   // -mref of this lane's query, the score accumulators' start value
#pragma unroll
        for (int j = 0; j < 16; ++j) bias[j] = 0.0f;
        bool bias_dirty = false;
        if (tt < seg_end) load_q(tt);
        int tnext = t + __builtin_amdgcn_readfirstlane(grab_raw());
        int gv = 0;              // reply of the grab for the tile after tt, if `pending`
        bool pending = false;
        for (; tt < seg_end; tt = tnext, pending = tnext < seg_end, gv = pending ? grab_raw() : 0) {
            const int q0 = (p0.j + (tt - t)) * kTileQ;
            stage_q();
            if (!zeroed) zero_fill();   // once, after the first tile's Q is in registers
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
                            const bf16x8 kh = lds_ld<bf16x8>(kaddr[ks][rb & 1], rb * 4096);
                            dst[r2] = mfma32(kh, qop[ks], ks == 0 ? bias : dst[r2]);
                        }
                    }
                }
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2) {
                    if (r2 < nrb) {
                        const int rb = 2 * blk + r2;
                        const u32x4 l0 = lds_ld<u32x4>(laddr[0], rb * 2048);
                        const u32x4 l1 = lds_ld<u32x4>(laddr[1], rb * 2048);
                        const i32x8 lop = __builtin_bit_cast(
                            i32x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
                        dst[r2] = mfma_lo(rb & 3, lop, q8, dst[r2], scl[rb >> 2], qsc);
                    }
                }
            };

            f32x16 o0, o1;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                o0[j] = 0.0f;
                o1[j] = 0.0f;
            }
            float z = 0.0f;
            float mref = 0.0f;

            scores(0, sc[0]);
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) {
                const int cur = blk & 1;
                if (blk + 1 < NBLK) scores(blk + 1, sc[cur ^ 1]);
                else {
                    if (pending) tnext = t + __builtin_amdgcn_readfirstlane(gv);
                    pending = false;
                    if (tnext < seg_end) load_q(tnext);
                }
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
                    mref += sh;
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
                            const s16x4 v0 = lds_tr16(vaddr[mt], vo);
                            const s16x4 v1 = lds_tr16(vaddr[mt], vo + 1024);
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
            const float inv = 1.0f / z;

            // ---- store: lane holds O[q0 + l32][c] for c = 32 mt + 8 gq + 4 hh + (0..3), i.e.
            // 8 bytes of chunk 4 mt + gq; staged, then written as whole rows (rows past the
            // length as zeros)
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
            u32x4* dst = (u32x4*)(a.O + (rowbase + q0) * kHeadDim) + lane;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 v = lds_ld<u32x4>(stg, coff[i]);
                if (q0 + 8 * i + crow >= L) v = u32x4{0u, 0u, 0u, 0u};
                __builtin_nontemporal_store(v, &dst[64 * i]);
            }
        }
        if (!zeroed) zero_fill();   // a wave that took no tile of the segment
        t = seg_end;
    }

    if (!zeroed) zero_fill();   // a workgroup without tiles

}

}  // namespace

hipError_t launch_attend_bf16(const AttendBf16Args& a, hipStream_t stream) {
    const int grid = ((a.nlogical + 7) / 8) * 8;
    switch (a.k / 32) {
        case 1: hipLaunchKernelGGL(attend_bf16_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, a); break;
        case 2: hipLaunchKernelGGL(attend_bf16_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, a); break;
        case 3: hipLaunchKernelGGL(attend_bf16_kernel<3>, dim3(grid), dim3(kThreads), 0, stream, a); break;
        case 4: hipLaunchKernelGGL(attend_bf16_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, a); break;
        case 5: hipLaunchKernelGGL(attend_bf16_kernel<5>, dim3(grid), dim3(kThreads), 0, stream, a); break;
        case 6: hipLaunchKernelGGL(attend_bf16_kernel<6>, dim3(grid), dim3(kThreads), 0, stream, a); break;
        case 7: hipLaunchKernelGGL(attend_bf16_kernel<7>, dim3(grid), dim3(kThreads), 0, stream, a); break;
        case 8: hipLaunchKernelGGL(attend_bf16_kernel<8>, dim3(grid), dim3(kThreads), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lf
