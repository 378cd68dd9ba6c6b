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
#include "attend_core.h"

namespace lf {
namespace {

using namespace attn;
constexpr int kThreads = kAttendThreads;   // 8 waves

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
    using Ly = AttnLayout<KB>;
    constexpr int K = Ly::K, PLANE = Ly::PLANE, LOB = Ly::LOB;
    constexpr int OFF_V = Ly::OFF_V, OFF_L = Ly::OFF_L, OFF_S = Ly::OFF_S;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Ly::BYTES];
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
    const int lane = tid & 63, hh = lane >> 5;

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

    const Lanes ln = attn_lanes<KB>(lds0, lane);

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

        // this wave's first tile of the segment (tiles t .. t+7 are taken statically): its Q is
        // loaded before the head's planes, so the two loads' latencies overlap
        int tt = t + wave;
        u32x4 qraw[4];   // the tile as loaded: row 8 i + lane / 8, chunk lane % 8, i = 0..3
        auto load_q = [&](int tile) {
            const int q0 = (p0.j + (tile - t)) * kTileQ;
            const u32x4* src = (const u32x4*)(a.Q + (rowbase + q0) * kHeadDim) + lane;
#pragma unroll
            for (int i = 0; i < 4; ++i) qraw[i] = src[64 * i];
        };
        if (tt < seg_end) load_q(tt);

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
            __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));   // vmcnt(0): Q too
            if (tid == 0) s_next = 8;   // tiles t .. t+7 are taken statically
        }
        __syncthreads();
        int scl[2];
        attn_scales<KB>(smem, lane, scl);

        // ---- tiles of this segment, taken dynamically by the waves from an LDS counter (so waves
        // that finish early take more), Q of the next tile prefetched during the current one
        bf16x8 qop[4];   // operand layout: columns 16 ks + 8 hh + (0..7) of query q0 + l32
        uint32_t coff[4];
        stage_offsets(lane, coff);
        const uint32_t stg = lds_addr(&s_stage[wave][0]);
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
        int tnext = t + __builtin_amdgcn_readfirstlane(grab_raw());
        int gv = 0;              // reply of the grab for the tile after tt, if `pending`
        bool pending = false;
        for (; tt < seg_end; tt = tnext, pending = tnext < seg_end, gv = pending ? grab_raw() : 0) {
            const int q0 = (p0.j + (tt - t)) * kTileQ;
            stage_q(stg, coff, qraw, lane, qop);
            if (!zeroed) zero_fill();   // once, after the first tile's Q is in registers
            f32x16 o0, o1;
            float z;
            tile_math<KB>(ln, qop, scl, hh, bias, bias_dirty, o0, o1, z, [&]() {
                if (pending) tnext = t + __builtin_amdgcn_readfirstlane(gv);
                pending = false;
                if (tnext < seg_end) load_q(tnext);
            });
            tile_store(stg, coff, lane, o0, o1, z, a.O + (rowbase + q0) * kHeadDim, q0, L);
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
