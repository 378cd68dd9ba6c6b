// Sequence projection Kbar = E_h . K_{b,h}, Vbar = F_h . V_{b,h} in bf16 with fp32 accumulation
// (Linformer 요약 설명, section "Model": each row of E combines the n positions' keys into one
// projected key; positions past a sequence's length contribute nothing).
//
// As a GEMM per group of units sharing one projection matrix A (k x n):
//   M = k projected slots, N = 64 columns per unit, reduction over the n positions.
// Workgroup (512 threads, 8 waves) = all k slots x `upt` units x one split of the positions.
// Wave w computes slot block w % (k/32) (32 slots) for `upw` units.
//   * A rows (positions contiguous) are the MFMA A operand and go straight from global memory
//     to registers: each wave owns its 32 rows, nothing is shared.
//   * K/V rows arrive with the head dimension contiguous but the B operand needs the positions
//     contiguous, so each 64-position step of K/V is transposed on its way into LDS: a thread
//     loads two consecutive positions (16 B each), interleaves them into (t, t+1) pairs and
//     writes 8 dwords.  LDS tile per unit: [64 columns][64 positions], 128 B rows, 16-B chunks
//     XOR-swizzled by (c ^ c>>3) & 7 so both the pair writes and the 16-B MFMA reads spread over
//     all banks.  Double-buffered: the next step's global loads are in flight during the MFMAs.
// Splits (S > 1) write fp32 partial sums; a fixup kernel adds them in split order (so results are
// bitwise reproducible) and casts.  With S == 1 the cast happens here.
// Output cast: Kbar -> (hi = bf16(x), lo = bf16(x - hi)); Vbar -> bf16(x), round to nearest even.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kThreads = 512;
constexpr int kStep = 64;                 // positions per pipeline step
constexpr int kUnitTileBytes = 64 * kStep * 2;

__device__ __forceinline__ int swz(int c) { return (c ^ (c >> 3)) & 7; }

struct Unit {
    int which, b, h;
};

__device__ __forceinline__ Unit unit_of(const ProjGeom& g, int grp, int j) {
    Unit u;
    if (g.share == 0) {               // unshared: group = which * H + h, member = b
        u.which = grp / g.H;
        u.h = grp % g.H;
        u.b = j;
    } else if (g.share == 1) {        // headwise: group = which, member = (b, h)
        u.which = grp;
        u.b = j / g.H;
        u.h = j % g.H;
    } else {                          // key-value / layerwise: member = (which, b, h)
        const int bh = g.B * g.H;
        u.which = j / bh;
        const int r = j % bh;
        u.b = r / g.H;
        u.h = r % g.H;
    }
    return u;
}

__device__ __forceinline__ const uint16_t* group_matrix(const ProjBf16Args& a, int grp) {
    const ProjGeom& g = a.g;
    if (g.share == 0) {
        const int which = grp / g.H, h = grp % g.H;
        return (which ? a.F : a.E) + (size_t)h * g.k * g.n;
    }
    if (g.share == 1) return grp ? a.F : a.E;
    return a.E;
}

template <int UPT, int UPW>
__global__ __launch_bounds__(kThreads) void proj_bf16_kernel(ProjBf16Args a) {
    constexpr int WN = UPT / UPW;                  // wave groups along units
    constexpr int LPT = (UPT * 256 + kThreads - 1) / kThreads;  // pair-chunks per thread
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const ProjGeom& g = a.g;
    const int lid = xcd_remap(blockIdx.x, g.nlogical);
    if (lid < 0) return;
    const int tile = lid % g.tiles_per_group;
    const int rest = lid / g.tiles_per_group;
    const int s = rest % g.S;
    const int grp = rest / g.S;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int SB = g.k >> 5;
    const bool computes = wave < SB * WN;
    const int sb = wave % SB, wn = wave / SB;
    const int j0 = tile * UPT;

    const int t_begin = s * g.steps_per_split * kStep;
    const int t_end = min(g.n, t_begin + g.steps_per_split * kStep);
    const int nsteps = (t_end - t_begin) / kStep;

    // ---- loader assignment: pair-chunk pc -> (unit ut, positions 2tp, 2tp+1, columns 8cg..)
    const uint16_t* lsrc[LPT];
    int llen[LPT], lrow[LPT], lcg[LPT], lut[LPT];
    bool lon[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int pc = tid + i * kThreads;
        const int ut = pc >> 8, rem = pc & 255;
        lut[i] = ut;
        lrow[i] = (rem >> 3) * 2;
        lcg[i] = rem & 7;
        lon[i] = (pc < UPT * 256) && (j0 + ut < g.members);
        lsrc[i] = nullptr;
        llen[i] = 0;
        if (lon[i]) {
            const Unit u = unit_of(g, grp, j0 + ut);
            const uint16_t* X = u.which ? a.V : a.K;
            lsrc[i] = X + ((size_t)(u.b * g.H + u.h) * g.n) * kHeadDim + lcg[i] * 8;
            llen[i] = clamp_len(a.lengths, u.b, g.n);
        }
    }

    const uint16_t* arow = group_matrix(a, grp) + (size_t)(sb * 32 + l32) * g.n + hh * 8;

    f32x16 acc[UPW][2];
#pragma unroll
    for (int u = 0; u < UPW; ++u)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[u][nt][j] = 0.0f;

    u32x4 xr[LPT][2];
    bf16x8 ea[4], ean[4];

    auto load_x = [&](int t0) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            xr[i][0] = z;
            xr[i][1] = z;
            if (lon[i]) {
                const int t = t0 + lrow[i];
                if (t < llen[i]) xr[i][0] = *(const u32x4*)(lsrc[i] + (size_t)t * kHeadDim);
                if (t + 1 < llen[i])
                    xr[i][1] = *(const u32x4*)(lsrc[i] + (size_t)(t + 1) * kHeadDim);
            }
        }
    };
    auto load_a = [&](int t0, bf16x8* dst) {
        if (computes) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) dst[ks] = *(const bf16x8*)(arow + t0 + ks * 16);
        }
    };
    auto store_x = [&](int buf) {
        uint8_t* base = smem + buf * (UPT * kUnitTileBytes);
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            if (i * kThreads + tid >= UPT * 256) continue;
            const int t = lrow[i];
            const int q = t >> 3;
            uint8_t* ub = base + lut[i] * kUnitTileBytes + (t & 7) * 2;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w0 = xr[i][0][e >> 1], w1 = xr[i][1][e >> 1];
                const uint32_t v = (e & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u))
                                           : ((w0 & 0xFFFFu) | (w1 << 16));
                const int c = lcg[i] * 8 + e;
                *(uint32_t*)(ub + c * 128 + ((q ^ swz(c)) << 4)) = v;
            }
        }
    };

    if (nsteps > 0) {
        load_x(t_begin);
        load_a(t_begin, ea);
        store_x(0);
    }
    __syncthreads();

    for (int step = 0; step < nsteps; ++step) {
        const bool more = step + 1 < nsteps;
        if (more) {
            load_x(t_begin + (step + 1) * kStep);
            load_a(t_begin + (step + 1) * kStep, ean);
        }
        if (computes) {
            const uint8_t* base = smem + (step & 1) * (UPT * kUnitTileBytes);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int q = ks * 2 + hh;
#pragma unroll
                for (int u = 0; u < UPW; ++u) {
                    const uint8_t* ub = base + (wn * UPW + u) * kUnitTileBytes;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const int c = nt * 32 + l32;
                        const bf16x8 bop = *(const bf16x8*)(ub + c * 128 + ((q ^ swz(c)) << 4));
                        acc[u][nt] = mfma32(ea[ks], bop, acc[u][nt]);
                    }
                }
            }
        }
        if (more) {
            store_x((step + 1) & 1);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) ea[ks] = ean[ks];
        }
        __syncthreads();
    }

    if (!computes) return;
    const size_t bhk = (size_t)g.B * g.H * g.k;
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
        const int j = j0 + wn * UPW + u;
        if (j >= g.members) continue;
        const Unit un = unit_of(g, grp, j);
        const size_t ubase = ((size_t)(un.b * g.H + un.h) * g.k) * kHeadDim;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int c = nt * 32 + l32;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int r = sb * 32 + 8 * (jj >> 2) + 4 * hh + (jj & 3);
                const float x = acc[u][nt][jj];
                const size_t idx = ubase + (size_t)r * kHeadDim + c;
                if (g.S == 1) {
                    if (un.which == 0) {
                        const uint16_t hi = f32_to_bf16(x);
                        a.Khi[idx] = hi;
                        a.Klo[idx] = f32_to_bf16(x - bf16_to_f32(hi));
                    } else {
                        a.Vb[idx] = f32_to_bf16(x);
                    }
                } else {
                    a.part[((size_t)s * 2 + un.which) * bhk * kHeadDim + idx] = x;
                }
            }
        }
    }
}

// Adds the S fp32 partial sums of every Kbar/Vbar element in split order and casts.
__global__ __launch_bounds__(256) void proj_fixup_bf16_kernel(const float* part, int S,
                                                              size_t half, uint16_t* Khi,
                                                              uint16_t* Klo, uint16_t* Vb) {
    const size_t e4 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (e4 >= 2 * half) return;
    f32x4 acc = *(const f32x4*)(part + e4);
    for (int s = 1; s < S; ++s) acc += *(const f32x4*)(part + (size_t)s * 2 * half + e4);
    if (e4 < half) {
        const u32x2 hi = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        const float h0 = __uint_as_float(hi[0] << 16), h1 = __uint_as_float(hi[0] & 0xFFFF0000u);
        const float h2 = __uint_as_float(hi[1] << 16), h3 = __uint_as_float(hi[1] & 0xFFFF0000u);
        const u32x2 lo = {pack_bf16x2(acc[0] - h0, acc[1] - h1),
                          pack_bf16x2(acc[2] - h2, acc[3] - h3)};
        *(u32x2*)(Khi + e4) = hi;
        *(u32x2*)(Klo + e4) = lo;
    } else {
        const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *(u32x2*)(Vb + (e4 - half)) = v;
    }
}

}  // namespace

bool proj_geometry(int B, int H, int n, int k, int share, int split_override, int upt_override,
                   ProjGeom* out) {
    if (B < 1 || H < 1 || n < kStep || n % kStep || k < 32 || k > 256 || k % 32) return false;
    ProjGeom g{};
    g.B = B;
    g.H = H;
    g.n = n;
    g.k = k;
    g.share = share;
    if (share == 0) {
        g.groups = 2 * H;
        g.members = B;
    } else if (share == 1) {
        g.groups = 2;
        g.members = B * H;
    } else {
        g.groups = 1;
        g.members = 2 * B * H;
    }
    // units per tile: 2 when all 8 waves already cover the slots (k = 256 or k > 128),
    // 4 for k <= 128 so that 8 waves stay busy.
    int upt = (k > 128) ? 2 : 4;
    if (upt_override == 1 || upt_override == 2 || (upt_override == 4 && k <= 128)) upt = upt_override;
    g.upt = upt;
    g.tiles_per_group = (g.members + upt - 1) / upt;
    const int steps = n / kStep;
    const int tiles = g.groups * g.tiles_per_group;
    int S;
    if (split_override > 0) {
        S = split_override;
    } else {
        // aim for about two workgroups per compute unit (256 CUs) without splitting below
        // four steps (256 positions) per split.
        const int target = 512;
        S = (target + tiles - 1) / tiles;
        if (S > steps / 4) S = steps / 4;
        if (S < 1) S = 1;
    }
    if (S > steps) S = steps;
    g.steps_per_split = (steps + S - 1) / S;
    g.S = (steps + g.steps_per_split - 1) / g.steps_per_split;
    g.nlogical = g.groups * g.S * g.tiles_per_group;
    *out = g;
    return true;
}

hipError_t launch_proj_bf16(const ProjBf16Args& a, hipStream_t stream) {
    const ProjGeom& g = a.g;
    const int grid = ((g.nlogical + 7) / 8) * 8;
    const size_t lds = 2 * (size_t)g.upt * kUnitTileBytes;
    if (g.upt == 1)
        hipLaunchKernelGGL((proj_bf16_kernel<1, 1>), dim3(grid), dim3(kThreads), lds, stream, a);
    else if (g.upt == 2)
        hipLaunchKernelGGL((proj_bf16_kernel<2, 2>), dim3(grid), dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((proj_bf16_kernel<4, 2>), dim3(grid), dim3(kThreads), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.S == 1) return e;
    const size_t half = (size_t)g.B * g.H * g.k * kHeadDim;
    const size_t threads = (2 * half) / 4;
    const int blocks = (int)((threads + 255) / 256);
    hipLaunchKernelGGL(proj_fixup_bf16_kernel, dim3(blocks), dim3(256), 0, stream, a.part, g.S,
                       half, a.Khi, a.Klo, a.Vb);
    return hipGetLastError();
}

}  // namespace lf
