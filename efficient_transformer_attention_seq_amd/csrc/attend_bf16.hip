// Compressed attention O = softmax(scale * Q . Kbar^T) . Vbar for bf16 inputs (Linformer 요약 설명,
// section "Model": n x k scores, softmax over the k projected slots of each query, weighted sum of
// Vbar; queries are not compressed, so there is one output row per position).
//
// Persistent kernel: one workgroup (8 waves) per compute unit.  The work is the list of valid
// 32-query tiles of every (b, h) (tiles wholly past a sequence's length hold no work), split into
// equal contiguous ranges, one per workgroup; consecutive workgroups go to the same XCD so the
// workgroups that share a head's Kbar/Vbar share an L2.  Rows past the lengths are zero-filled
// with plain stores, spread evenly over the workgroups.
//
// Per (b, h) segment of its range a workgroup copies Kbar (hi and lo planes) and Vbar, k x 64
// bf16 each, into LDS with direct-to-LDS buffer loads (96 KB at k = 256) and keeps them resident:
//   Kbar planes: [k][64], 16-byte chunks XOR-swizzled by (r ^ r>>3) & 7 (conflict-free A reads)
//   Vbar       : [k][64], 32-byte blocks XOR-swizzled by (r & 3), read with the transposing
//                ds_read_b64_tr_b16 so each lane gets 8 slots of one column.
// Per wave and tile of 32 queries (v_mfma_f32_32x32x16_bf16):
//   1. S^T (k x 32) = Kbar . Q^T, two MFMAs per step (hi plane, lo plane) so the scores carry Kbar
//      to fp32 accuracy; Q is the B operand, its next tile loaded during this tile's softmax.
//   2. Exact softmax per query in one streaming pass over blocks of 64 slots: the scores of a query
//      sit in lanes l and l+32, so block max and sums are in-register reductions plus one
//      cross-lane exchange; w = exp2(s * c - mref) with c = scale * log2(e) in one FMA, against a
//      reference max that is raised (with a rescale of the partial sums) only when a block max
//      exceeds it by more than 2^8 -- numerator and denominator share it, so the result is exact.
//   3. O^T (64 x 32) = Vbar^T . W^T with the unnormalised weights rounded to bf16 as the B operand
//      straight from the score accumulators: lane (l, h) holds, for slot block rb, the weights of
//      slots 32 rb + 8 (j/4) + 4 h + j%4, and the Vbar^T operand is read at exactly those slots
//      (no permutation in memory).  Each output column (one query) is divided by its row sum.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kThreads = kAttendThreads;   // 8 waves
constexpr int kTileQ = 32;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz16(int r) { return (r ^ (r >> 3)) & 7; }

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

// Tile index -> (b, h, j) for the valid-tile list: batch-major, then head, then tile.
struct TilePos {
    int b, h, j, ntb;   // ntb = valid tiles per (b, h) of this batch item
};
__device__ __forceinline__ TilePos tile_pos(const AttendBf16Args& a, int t) {
    TilePos p{0, 0, 0, 0};
    for (int b = 0; b < a.B; ++b) {
        const int L = clamp_len(a.lengths, b, a.n);
        const int ntb = (L + kTileQ - 1) / kTileQ;
        const int tb = ntb * a.H;
        if (t < tb) {
            p.b = b;
            p.h = t / ntb;
            p.j = t % ntb;
            p.ntb = ntb;
            return p;
        }
        t -= tb;
    }
    return p;
}

template <int KB>
__global__ __launch_bounds__(kThreads) void attend_bf16_kernel(AttendBf16Args a) {
    constexpr int K = KB * 32;
    constexpr int PLANE = K * 128;            // bytes of one k x 64 bf16 plane
    __shared__ __attribute__((aligned(16))) uint8_t smem[3 * PLANE];
    __shared__ int s_next;   // next tile of the current segment (relative to its start)
    uint8_t* sKh = smem;
    uint8_t* sKl = smem + PLANE;
    uint8_t* sV = smem + 2 * PLANE;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;

    const int G = gridDim.x;
    const int w = xcd_remap(blockIdx.x, G);   // G is a multiple of 8, so every block is mapped
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;

    // ---- totals: valid tiles and zero-filled rows (rows from the first padded tile to n)
    int T = 0;
    long long Z = 0;   // 16-byte chunks to zero
    for (int b = 0; b < a.B; ++b) {
        const int L = clamp_len(a.lengths, b, a.n);
        const int ntb = (L + kTileQ - 1) / kTileQ;
        T += ntb * a.H;
        Z += (long long)(a.n - ntb * kTileQ) * a.H * 8;
    }

    // ---- zero rows wholly past each length.  Per (b, h) those rows are one contiguous block;
    // the workgroup takes an equal share of the concatenated blocks (16-byte stores).
    if (Z > 0) {
        const long long z0 = Z * w / G, z1 = Z * (w + 1) / G;   // in 16-byte chunks
        const u32x4 zero = {0u, 0u, 0u, 0u};
        long long base = 0;
        for (int b = 0; b < a.B && base < z1; ++b) {
            const int L = clamp_len(a.lengths, b, a.n);
            const int r0 = ((L + kTileQ - 1) / kTileQ) * kTileQ;
            const long long per_h = (long long)(a.n - r0) * 8;
            for (int h = 0; h < a.H && base < z1; ++h, base += per_h) {
                const long long lo = max(z0, base), hi = min(z1, base + per_h);
                if (lo >= hi) continue;
                u32x4* blk = (u32x4*)(a.O + ((size_t)(b * a.H + h) * a.n + r0) * kHeadDim);
                for (int c = (int)(lo - base) + tid; c < (int)(hi - base); c += kThreads)
                    blk[c] = zero;
            }
        }
    }

    // ---- this workgroup's valid tiles
    const int t_lo = (int)((long long)T * w / G), t_hi = (int)((long long)T * (w + 1) / G);
    const float c = a.c;
    const size_t plane_elems = (size_t)a.B * a.H * K * kHeadDim;

    // per-lane operand addressing: every LDS read is a per-lane base plus a compile-time offset.
    //   Kbar row r = 32 rb + l32: swizzle (r ^ r>>3) & 7 = bsw ^ 4 (rb & 1), bsw from l32 alone.
    const int bsw = (l32 ^ (l32 >> 3)) & 7;
    int kaddr[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int par = 0; par < 2; ++par)
            kaddr[ks][par] = l32 * 128 + (((2 * ks + hh) ^ bsw ^ (4 * par)) << 4);
    //   Vbar rows 32 rb + 16 al + 8 rd + trow: the 32-byte block swizzle only sees trow & 3.
    const int grp16 = lane >> 4, s16 = lane & 15;
    const int trow = 4 * (grp16 >> 1) + (s16 >> 2);
    const int tcb = grp16 & 1;
    int vaddr[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        vaddr[mt] = trow * 128 + (((2 * mt + tcb) ^ (trow & 3)) << 5) + (s16 & 3) * 8;

    int t = t_lo;
    while (t < t_hi) {
        const TilePos p0 = tile_pos(a, t);
        const int seg_end = min(t_hi, t + (p0.ntb - p0.j));   // tiles of this (b, h) in range
        const int bh = p0.b * a.H + p0.h;
        const int L = clamp_len(a.lengths, p0.b, a.n);
        const size_t rowbase = (size_t)bh * a.n;

        // ---- fill LDS with this head's Kbar hi/lo and Vbar (every wave issues 3K/64 loads)
        __syncthreads();   // previous segment's readers are done with the LDS planes
        {
            const size_t off = (size_t)bh * K * kHeadDim;
            const i32x4 rh = make_rsrc(a.Khi + off, PLANE);
            const i32x4 rl = make_rsrc(a.Khi + plane_elems + off, PLANE);
            const i32x4 rv = make_rsrc(a.Vb + off, PLANE);
            const int lrow = lane >> 3, lpc = lane & 7;
            for (int I = wave; I < K / 8; I += 8) {
                const int r = I * 8 + lrow;
                const int lck = lpc ^ swz16(r);
                const int lcv = 2 * ((lpc >> 1) ^ (r & 3)) + (lpc & 1);
                dma16(rh, lds0 + I * 1024, (uint32_t)(r * 128 + lck * 16));
                dma16(rl, lds0 + PLANE + I * 1024, (uint32_t)(r * 128 + lck * 16));
                dma16(rv, lds0 + 2 * PLANE + I * 1024, (uint32_t)(r * 128 + lcv * 16));
            }
            __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));   // vmcnt(0)
            if (tid == 0) s_next = 8;   // tiles t .. t+7 are taken statically below
        }
        __syncthreads();

        // ---- tiles of this segment, taken dynamically by the waves from an LDS counter (so waves
        // that finish early take more), Q of the next tile prefetched during the current one
        int tt = t + wave;
        bf16x8 qop[4];
        auto load_q = [&](int tile) {
            const int q0 = (p0.j + (tile - t)) * kTileQ;
            const uint16_t* qrow = a.Q + (rowbase + q0 + l32) * kHeadDim + hh * 8;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qop[ks] = *(const bf16x8*)(qrow + ks * 16);
        };
        auto grab = [&]() {
            int v = 0;
            if (lane == 0) v = atomicAdd(&s_next, 1);
            return t + __builtin_amdgcn_readfirstlane(v);
        };
        if (tt < seg_end) load_q(tt);
        int tnext = grab();
        for (; tt < seg_end; tt = tnext, tnext = (tnext < seg_end ? grab() : tnext)) {
            const int q0 = (p0.j + (tt - t)) * kTileQ;

            // ---- streaming exact softmax over blocks of 64 slots.  The score MFMAs of block j+1
            // are issued before the softmax of block j, so the matrix cores and the vector ALUs
            // work side by side within the wave.  Scores are taken in log2 units x = s * c; the
            // reference max mref only moves when a block max exceeds it by more than 8 (then O and
            // z are rescaled), so weights stay <= 2^8 and numerator and denominator always share
            // the same reference: the normalisation is exact.
            constexpr int NBLK = (KB + 1) / 2;
            f32x16 sc[2][2];   // [buffer][rb within block]
            auto scores = [&](int blk, f32x16* dst) {
                const int nrb = min(2, KB - 2 * blk);
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                    for (int j = 0; j < 16; ++j) dst[r2][j] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                    for (int r2 = 0; r2 < 2; ++r2) {
                        if (r2 < nrb) {
                            const int rb = 2 * blk + r2;
                            const uint8_t* pk = sKh + kaddr[ks][rb & 1] + rb * 4096;
                            dst[r2] = mfma32(*(const bf16x8*)pk, qop[ks], dst[r2]);
                            dst[r2] = mfma32(*(const bf16x8*)(pk + PLANE), qop[ks], dst[r2]);
                        }
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
            float mref = -INFINITY;

            scores(0, sc[0]);
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) {
                const int cur = blk & 1;
                if (blk + 1 < NBLK) scores(blk + 1, sc[cur ^ 1]);
                else if (tnext < seg_end) load_q(tnext);   // Q is dead: prefetch the next tile
                __builtin_amdgcn_sched_barrier(0);
                const int nrb = min(2, KB - 2 * blk);
                // block max (both lanes of a query), in log2 units
                float bm = sc[cur][0][0];
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2)
                    if (r2 < nrb)
#pragma unroll
                        for (int j = 0; j < 16; ++j) bm = fmaxf(bm, sc[cur][r2][j]);
                bm = fmaxf(bm, __shfl_xor(bm, 32)) * c;
                if (__builtin_amdgcn_ballot_w64(bm > mref + 8.0f)) {
                    const float nref = fmaxf(mref, bm);
                    const float alpha = __builtin_amdgcn_exp2f(mref - nref);   // 0 on the first block
                    o0 *= alpha;
                    o1 *= alpha;
                    z *= alpha;
                    mref = nref;
                }
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2) {
                    if (r2 >= nrb) continue;
                    const int rb = 2 * blk + r2;
                    float wv[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        wv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cur][r2][j], c, -mref));
                        z += wv[j];
                    }
#pragma unroll
                    for (int al = 0; al < 2; ++al) {
                        const bf16x8 pw = pack_bf16x8(wv[8 * al], wv[8 * al + 1], wv[8 * al + 2],
                                                      wv[8 * al + 3], wv[8 * al + 4],
                                                      wv[8 * al + 5], wv[8 * al + 6],
                                                      wv[8 * al + 7]);
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt) {
                            // Vbar^T operand: columns 32 mt + l32,
                            // slots 32 rb + 16 al + 4 h + {0..3, 8..11}
                            s16x4 v[2];
#pragma unroll
                            for (int rd = 0; rd < 2; ++rd) {
                                const uint8_t* pv =
                                    sV + vaddr[mt] + rb * 4096 + al * 2048 + rd * 1024;
                                v[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                    (__attribute__((address_space(3))) s16x4*)(uintptr_t)(
                                        (__attribute__((address_space(3))) const uint8_t*)pv));
                            }
                            const bf16x8 vop = __builtin_bit_cast(
                                bf16x8,
                                __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
                            if (mt == 0) o0 = mfma32(vop, pw, o0);
                            else o1 = mfma32(vop, pw, o1);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            z += __shfl_xor(z, 32);
            const float inv = 1.0f / z;

            // ---- store: lane holds O[q0 + l32][c] for c = 32 mt + 8 gq + 4 hh + (0..3)
            const int q = q0 + l32;
            uint16_t* orow = a.O + (rowbase + q) * kHeadDim + 4 * hh;
            const bool valid = q < L;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 v0 = {0u, 0u}, v1 = {0u, 0u};
                if (valid) {
                    v0[0] = pack_bf16x2(o0[4 * gq] * inv, o0[4 * gq + 1] * inv);
                    v0[1] = pack_bf16x2(o0[4 * gq + 2] * inv, o0[4 * gq + 3] * inv);
                    v1[0] = pack_bf16x2(o1[4 * gq] * inv, o1[4 * gq + 1] * inv);
                    v1[1] = pack_bf16x2(o1[4 * gq + 2] * inv, o1[4 * gq + 3] * inv);
                }
                *(u32x2*)(orow + 8 * gq) = v0;
                *(u32x2*)(orow + 32 + 8 * gq) = v1;
            }
        }
        t = seg_end;
    }
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
