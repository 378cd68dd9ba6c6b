// Dense projections of the encoder attention stack, Y = X . W^T in bf16 with fp32 accumulation
// (Linformer 요약 설명, section "Transformer and Self-Attention": each layer maps its input to
// every head's queries, keys and values, and maps the concatenated heads through an output
// projection).
//
// GEMM with M = output features (rows of W), N = tokens, reduction over the K input features.
// Workgroup tile 192 features x 256 tokens; 8 waves as 2 (features) x 4 (tokens), wave tile
// 96 x 64 = 3 x 2 blocks of v_mfma_f32_32x32x16_bf16 with W as the A operand and the activations
// as the B operand, so both operands are read K-contiguous, 8 bf16 per lane, from LDS and each
// accumulator lane ends with runs of 4 consecutive features of one token.
//
// K streams through LDS in 32-wide stages (one 64-byte row per feature and per token) with
// direct-to-LDS buffer loads, 1 KB per wave instruction, in a ring of kNS stages so that kNS - 1
// stages are in flight while the matrix cores work on the oldest.  Within a row the four 16-byte
// chunks are XOR-swizzled by (r >> 1) & 3, which makes the operand reads of eight consecutive rows
// hit distinct banks; the swizzle is realised by choosing which global chunk each lane fetches.
//
// Activation layouts: row-major [T, K], or head-planar [B, H, n, 64] (the attention output, read
// as its head concatenation: a 32-wide K stage lies inside one head).  Output layouts: row-major
// [T, F], or the head-planar query | key | value planes [3][B, H, n, 64] (F = 3 d_model) that the
// attention reads.  The epilogue stages each wave's tile through LDS so that global stores are 16
// bytes per lane over whole row pieces.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kThreads = 512;
constexpr int kBF = kLinearTileF, kBT = kLinearTileT;   // 192 x 256
constexpr int kBK = 32;                                 // K per stage
constexpr int kNS = 4;                                  // ring depth
constexpr int kRowB = kBK * 2;                          // 64-byte LDS rows
constexpr int kTileW = kBF * kRowB;                     // 12 KB
constexpr int kTileX = kBT * kRowB;                     // 16 KB
constexpr int kStage = kTileW + kTileX;                 // 28 KB
constexpr int kDmaW = kTileW / 1024, kDmaX = kTileX / 1024;   // 12 + 16 instructions per stage
constexpr int kDma = kDmaW + kDmaX;
constexpr int kStgRow = 96 * 2 + 16;                    // epilogue staging row (bytes)
static_assert(8 * 64 * kStgRow <= kNS * kStage, "staging fits in the ring");

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

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
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
        case 0: vmcnt_le<0>(); break;
        case 3: vmcnt_le<3>(); break;
        case 4: vmcnt_le<4>(); break;
        case 6: vmcnt_le<6>(); break;
        case 8: vmcnt_le<8>(); break;
        default: vmcnt_le<0>(); break;   // (other counts do not occur; waiting for all is safe)
    }
}

__global__ __launch_bounds__(kThreads) void linear_bf16_kernel(LinearBf16Args a) {
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
    const int nsteps = a.K / kBK;

    // ---- this wave's DMA instructions of a stage: I = wave + 8 j < kDma; I < kDmaW covers the W
    // rows 16 I .. 16 I + 15, the others the token rows 16 (I - kDmaW) ..; lane -> row lane / 4,
    // LDS chunk lane % 4, which holds global chunk (lane % 4) ^ swz(row)
    const int my_count = (kDma - wave + 7) / 8;   // 4 for waves 0..3, 3 for waves 4..7
    const i32x4 rw = make_rsrc(a.W, (uint32_t)((size_t)a.F * a.K * 2));
    const i32x4 rx = make_rsrc(a.X, (uint32_t)((size_t)a.T * a.K * 2));
    uint32_t base_off[4];   // per instruction: byte offset of this lane's row at k = 0
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int I = wave + 8 * j;
        const int r = (I < kDmaW ? I : I - kDmaW) * 16 + (lane >> 2);
        const int gch = (lane & 3) ^ swz(r);
        uint32_t off = 0;
        if (I < kDmaW) {
            off = (uint32_t)(((size_t)(f0 + r) * a.K) * 2);
        } else if (I < kDma) {
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
    auto issue = [&](int step, int slot) {
        const int k0 = step * kBK;
        // byte offset of column k0 within a row: row-major adds k0; head-planar moves to head
        // k0 / 64 (n rows of 64 further per head) and column k0 % 64
        const uint32_t xk = a.act_mode == 0
                                ? (uint32_t)(k0 * 2)
                                : (uint32_t)((((size_t)(k0 >> 6) * a.n) * 64 + (k0 & 63)) * 2);
        const uint32_t sb = lds0 + (uint32_t)slot * kStage;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int I = wave + 8 * j;
            if (I < kDmaW) dma16(rw, sb + I * 1024, base_off[j] + (uint32_t)(k0 * 2));
            else if (I < kDma) dma16(rx, sb + kTileW + (I - kDmaW) * 1024, base_off[j] + xk);
        }
    };

    f32x16 acc[3][2];
#pragma unroll
    for (int mf = 0; mf < 3; ++mf)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[mf][mt][j] = 0.0f;

    // per-lane LDS read offsets (row part and swizzle) of the operand rows
    int w_row[3], x_row[2];
#pragma unroll
    for (int mf = 0; mf < 3; ++mf) w_row[mf] = wf * 96 + mf * 32 + l32;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) x_row[mt] = wt * 64 + mt * 32 + l32;

    const int npro = min(kNS - 1, nsteps);
    for (int s = 0; s < npro; ++s) issue(s, s);

    for (int i = 0; i < nsteps; ++i) {
        wait_vmcnt(min(kNS - 2, nsteps - 1 - i) * my_count);   // this wave's loads of stage i
        __syncthreads();                                        // everyone's; slot i-1 is free
        if (i + kNS - 1 < nsteps) issue(i + kNS - 1, (i + kNS - 1) % kNS);
        const uint8_t* st = smem + (size_t)(i % kNS) * kStage;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = 2 * ks + hh;
            bf16x8 wv[3], xv[2];
#pragma unroll
            for (int mf = 0; mf < 3; ++mf)
                wv[mf] = *(const bf16x8*)(st + w_row[mf] * kRowB + ((c ^ swz(w_row[mf])) << 4));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                xv[mt] = *(const bf16x8*)(st + kTileW + x_row[mt] * kRowB +
                                          ((c ^ swz(x_row[mt])) << 4));
#pragma unroll
            for (int mf = 0; mf < 3; ++mf)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) acc[mf][mt] = mfma32(wv[mf], xv[mt], acc[mf][mt]);
        }
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
    const int dm = a.F / 3;   // (output mode 1 only)
#pragma unroll
    for (int j = 0; j < 12; ++j) {
        const int idx = j * 64 + lane;        // 64 tokens x 12 chunks of 8 features
        const int tr = idx / 12, q = idx - tr * 12;
        const u32x4 v = *(const u32x4*)(stg + tr * kStgRow + q * 16);
        const int t = t0 + wt * 64 + tr;
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
    hipLaunchKernelGGL(linear_bf16_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lf
