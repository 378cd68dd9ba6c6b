// Dense projections of the encoder attention stack, Y = X . W^T in bf16 with fp32 accumulation
// (Linformer 요약 설명, section "Transformer and Self-Attention": each layer maps its input to
// every head's queries, keys and values, and maps the concatenated heads through an output
// projection).
//
// GEMM with M = output features (rows of W), N = tokens, reduction over the K input features.
// Workgroup tile 192 features x 256 tokens (8 waves as 2 features x 4 tokens) or x 128 tokens (4
// waves, 2 x 2, for grids too small to fill the chip); wave tile
// 96 x 64 = 3 x 2 blocks of v_mfma_f32_32x32x16_bf16 with W as the A operand and the activations
// as the B operand, so both operands are read K-contiguous, 8 bf16 per lane, from LDS and each
// accumulator lane ends with runs of 4 consecutive features of one token.
//
// K streams through LDS in 64-wide stages (one 128-byte row per feature and per token) with
// direct-to-LDS buffer loads, 1 KB per wave instruction, double-buffered: the loads of stage i + 1
// are issued, a quarter at a time, between the matrix sub-steps of stage i.  Within a row the
// eight 16-byte chunks are XOR-swizzled by (r ^ r >> 3) & 7, so the operand reads of consecutive
// rows hit distinct banks; the swizzle is realised by choosing which global chunk each lane
// fetches.  The operands of sub-step ks + 1 are read while the MFMAs of sub-step ks run.
//
// Activation layouts: row-major [T, K], or head-planar [B, H, n, 64] (the attention output, read
// as its head concatenation: a 64-wide K stage is one head).  T need not fill the last token
// tile: rows past T read as zero through the buffer descriptors and are not stored.  Output layouts: row-major
// [T, F], or the head-planar query | key | value planes [3][B, H, n, 64] (F = 3 d_model) that the
// attention reads.  The epilogue stages each wave's tile through LDS so that global stores are 16
// bytes per lane over whole row pieces.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kBF = kLinearTileF;                       // 192 features per tile
constexpr int kBK = 64;                                 // K per stage
constexpr int kNS = 2;                                  // stages (double buffer)
constexpr int kRowB = kBK * 2;                          // 128-byte LDS rows
constexpr int kTileW = kBF * kRowB;                     // 24 KB
constexpr int kStgRow = 96 * 2 + 16;                    // epilogue staging row (bytes)

// Token tile BT = 256 (8 waves, 2 x 4) or 128 (4 waves, 2 x 2); the wave tile is 96 x 64 either way.
template <int BT>
struct LinTile {
    static constexpr int kWaves = BT / 32;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kTileX = BT * kRowB;                 // 32 or 16 KB
    static constexpr int kStage = kTileW + kTileX;
    static constexpr int kDmaW = kTileW / 1024, kDmaX = kTileX / 1024;
    static constexpr int kPer = (kDmaW + kDmaX) / kWaves;     // 7 or 10 per wave
    static_assert((kDmaW + kDmaX) % kWaves == 0, "every wave issues the same number of loads");
    static_assert(kWaves * 64 * kStgRow <= kNS * kStage, "staging fits in the ring");
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
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

// 16 bytes per lane from `rsrc` at byte offset `voff` into LDS at lds_base + 16 * lane; inline asm
// so completion is tracked by the explicit vmcnt waits below rather than by compiler waits.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void vmcnt_le() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int BT>
__global__ __launch_bounds__(LinTile<BT>::kThreads) void linear_bf16_kernel(LinearBf16Args a) {
    using Tl = LinTile<BT>;
    constexpr int kWaves = Tl::kWaves, kStage = Tl::kStage;
    constexpr int kDmaW = Tl::kDmaW, kPer = Tl::kPer;
    constexpr int kBT = BT;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kNS * kStage];
    const int lid = xcd_remap(blockIdx.x, a.nlogical);
    if (lid < 0) return;
    // logical order: feature tiles fastest, so the workgroups that share a token tile (and read
    // the same activations) are consecutive and land on one XCD
    const int nft = a.F / kBF;
    const int f0 = (lid % nft) * kBF, t0 = (lid / nft) * kBT;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wf = wave & 1, wt = wave >> 1;
    const uint32_t lds0 = lds_addr(smem);
    const int nsteps = a.K / kBK;   // K % 64 == 0

    // ---- this wave's DMA instructions of a stage: I = wave + kWaves j (j < kPer); I < kDmaW
    // covers the W rows 8 I .. 8 I + 7, the others the token rows 8 (I - kDmaW) ..; lane -> row
    // lane / 8, LDS chunk lane % 8, which holds global chunk (lane % 8) ^ swz(row)
    const i32x4 rw = make_rsrc(a.W, (uint32_t)((size_t)a.F * a.K * 2));
    const i32x4 rx = make_rsrc(a.X, (uint32_t)((size_t)a.T * a.K * 2));
    uint32_t base_off[kPer];   // per instruction: byte offset of this lane's 16 bytes at k = 0
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int I = wave + kWaves * j;
        const int r = (I < kDmaW ? I : I - kDmaW) * 8 + (lane >> 3);
        const int gch = (lane & 7) ^ swz(r);
        uint32_t off;
        if (I < kDmaW) {
            off = (uint32_t)(((size_t)(f0 + r) * a.K) * 2);
        } else {
            const int t = t0 + r;
            if (a.act_mode == 0) {
                off = (uint32_t)(((size_t)t * a.K) * 2);
            } else {   // head-planar: token t = b n + i, column k = 64 h + c at ((b H + h) n + i) 64 + c
                const int b = t / a.n, i = t - b * a.n;
                off = (uint32_t)(((size_t)b * a.H * a.n + i) * 64 * 2);
            }
        }
        base_off[j] = off + (uint32_t)(gch * 16);
    }
    // part p (0..3) of stage `step`'s loads: instructions j with j % 4 == p
    auto issue_part = [&](int step, int slot, int part) {
        const int k0 = step * kBK;
        // byte offset of column k0 within a row: row-major adds k0; head-planar moves to head
        // k0 / 64, n rows of 64 further per head
        const uint32_t xk = a.act_mode == 0 ? (uint32_t)(k0 * 2)
                                            : (uint32_t)(((size_t)(k0 >> 6) * a.n) * 64 * 2);
        const uint32_t sb = lds0 + (uint32_t)slot * kStage;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (j % 4 != part) continue;
            const int I = wave + kWaves * j;
            if (I < kDmaW) dma16(rw, sb + I * 1024, base_off[j] + (uint32_t)(k0 * 2));
            else dma16(rx, sb + kTileW + (I - kDmaW) * 1024, base_off[j] + xk);
        }
    };

    f32x16 acc[3][2];
#pragma unroll
    for (int mf = 0; mf < 3; ++mf)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mf][mt][j] = 0.0f;

    // per-lane LDS read offsets of the operand rows: row * 128 and the row's swizzle
    int w_off[3], w_sw[3], x_off[2], x_sw[2];
#pragma unroll
    for (int mf = 0; mf < 3; ++mf) {
        const int r = wf * 96 + mf * 32 + l32;
        w_off[mf] = r * kRowB;
        w_sw[mf] = swz(r);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int r = wt * 64 + mt * 32 + l32;
        x_off[mt] = kTileW + r * kRowB;
        x_sw[mt] = swz(r);
    }

#pragma unroll
    for (int part = 0; part < 4; ++part) issue_part(0, 0, part);

    for (int i = 0; i < nsteps; ++i) {
        vmcnt_le<0>();     // this wave's loads of stage i (the only ones in flight)
        __syncthreads();   // everyone's; the other slot (stage i - 1) is free
        const bool more = i + 1 < nsteps;
        const uint8_t* st = smem + (size_t)(i & 1) * kStage;
        bf16x8 wv[2][3], xv[2][2];
        auto load_ops = [&](int ks, bf16x8 (&w)[3], bf16x8 (&x)[2]) {
            const int c = 2 * ks + hh;
#pragma unroll
            for (int mf = 0; mf < 3; ++mf)
                w[mf] = *(const bf16x8*)(st + w_off[mf] + ((c ^ w_sw[mf]) << 4));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                x[mt] = *(const bf16x8*)(st + x_off[mt] + ((c ^ x_sw[mt]) << 4));
        };
        load_ops(0, wv[0], xv[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) load_ops(ks + 1, wv[(ks + 1) & 1], xv[(ks + 1) & 1]);
            if (more) issue_part(i + 1, (i + 1) & 1, ks);
#pragma unroll
            for (int mf = 0; mf < 3; ++mf)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    acc[mf][mt] = mfma32(wv[ks & 1][mf], xv[ks & 1][mt], acc[mf][mt]);
        }
    }

    if (a.out_mode == 2) {
        // ---- projected keys and values straight from the accumulators: lane (l32, hh) holds,
        // for slot row 32 mt + l32 of the wave tile, features 32 mf + 8 g + 4 hh + (0..3); the 32
        // features of block mf are one row half of one head, shared with lane l32 + 32 (hh = 1)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int t = t0 + wt * 64 + mt * 32 + l32;
            const int b = t / a.n, r = t - b * a.n;
#pragma unroll
            for (int mf = 0; mf < 3; ++mf) {
                const int fb = f0 + wf * 96 + mf * 32;   // first feature of the block
                const f32x16& x = acc[mf][mt];
                if (fb >= a.dm) {   // values: bf16
                    if (t >= a.T) continue;   // (a last token tile past T)
                    const int fh = fb - a.dm;
                    uint16_t* dst = a.Yv + (((size_t)b * a.H + (fh >> 6)) * a.n + r) * 64 + (fh & 63);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const u32x2 v = {pack_bf16x2(x[4 * g], x[4 * g + 1]),
                                         pack_bf16x2(x[4 * g + 2], x[4 * g + 3])};
                        *(u32x2*)(dst + 8 * g + 4 * hh) = v;
                    }
                } else {            // keys: c Kbar as hi plane + fp8 residual with a block scale
                    float lo[16];
                    u32x2 hv[4];
                    float m = 0.0f;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        hv[g][0] = hi_pair(a.c * x[4 * g], a.c * x[4 * g + 1], lo[4 * g], lo[4 * g + 1]);
                        hv[g][1] = hi_pair(a.c * x[4 * g + 2], a.c * x[4 * g + 3], lo[4 * g + 2], lo[4 * g + 3]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(lo[4 * g + i]));
                    }
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
                    m = fmaxf(m, __uint_as_float(hh ? sw[0] : sw[1]));
                    const int sh = lo_shift(m);
                    const size_t row = ((size_t)b * a.H + (fb >> 6)) * a.n + r;
                    const int d0 = fb & 63;   // 0 or 32: the row half
                    if (t >= a.T) continue;   // after the exchange, which every lane joins
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int d = d0 + 8 * g + 4 * hh;
                        *(u32x2*)(a.Y + row * 64 + d) = hv[g];
                        *(uint32_t*)(a.Klo + row * 64 + lo_pos(d)) =
                            lo_bytes(lo[4 * g], lo[4 * g + 1], lo[4 * g + 2], lo[4 * g + 3], sh);
                    }
                    if (hh == 0) a.Ksc[row * 2 + (d0 >> 5)] = (uint8_t)(127 - sh);
                }
            }
        }
        return;
    }

    // ---- epilogue: lane (l32, hh) holds, for token 32 mt + l32 of the wave tile, features
    // 32 mf + 8 g + 4 hh + (0..3); stage as [64 tokens][96 features] bf16, then store rows
    __syncthreads();   // every wave is done with the ring
    uint8_t* stg = smem + (size_t)wave * 64 * kStgRow;
#pragma unroll
    for (int mf = 0; mf < 3; ++mf)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16& x = acc[mf][mt];
                const u32x2 v = {pack_bf16x2(x[4 * g], x[4 * g + 1]),
                                 pack_bf16x2(x[4 * g + 2], x[4 * g + 3])};
                *(u32x2*)(stg + (32 * mt + l32) * kStgRow + (32 * mf + 8 * g + 4 * hh) * 2) = v;
            }
    __syncthreads();
    const int dm = a.dm;   // (output mode 1 only)
#pragma unroll
    for (int j = 0; j < 12; ++j) {
        const int idx = j * 64 + lane;        // 64 tokens x 12 chunks of 8 features
        const int tr = idx / 12, q = idx - tr * 12;
        const u32x4 v = *(const u32x4*)(stg + tr * kStgRow + q * 16);
        const int t = t0 + wt * 64 + tr;
        if (t >= a.T) continue;   // (a last token tile past T)
        const int f = f0 + wf * 96 + q * 8;
        size_t dst;
        if (a.out_mode == 0) {
            dst = (size_t)t * a.F + f;
        } else {
            const int which = f / dm, fh = f - which * dm;
            const int h = fh >> 6, c = fh & 63;
            const int b = t / a.n, i = t - b * a.n;
            dst = (size_t)which * a.plane + (((size_t)b * a.H + h) * a.n + i) * 64 + c;
        }
        *(u32x4*)(a.Y + dst) = v;
    }
}

}  // namespace

hipError_t launch_linear_bf16(const LinearBf16Args& a, hipStream_t stream) {
    const int grid = ((a.nlogical + 7) / 8) * 8;
    if (a.tile_t == 128)
        hipLaunchKernelGGL(linear_bf16_kernel<128>, dim3(grid), dim3(LinTile<128>::kThreads), 0,
                           stream, a);
    else if (a.tile_t == 256)
        hipLaunchKernelGGL(linear_bf16_kernel<256>, dim3(grid), dim3(LinTile<256>::kThreads), 0,
                           stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace lf
