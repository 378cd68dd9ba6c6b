// Backward pass of one Linformer layer for learned projections, in fp32 arithmetic (Linformer
// card, 方法适配: E and F are learned, so training needs the gradients with respect to Q, K, V, E
// and F).  Per (b, h), with the keys, values and dO rows past the length zeroed beforehand (those
// positions contribute nothing, and rows of O past the length are fixed at zero):
//   Kbar = E K, Vbar = F V (recomputed),  P = softmax(s Q Kbar^T)
//   dP = dO Vbar^T,  dS = P o (dP - rowsum(P o dP)),  dQ = s dS Kbar        (bw_attend_kernel)
//   dVbar = P^T dO,  dKbar = s dS^T Q                                        (bw_gemm_kernel)
//   dE += dKbar K^T, dK = E^T dKbar, dF += dVbar V^T, dV = F^T dVbar         (bw_gemm_kernel)
// Every contraction runs on the fp32 matrix cores: one strided, batched GEMM (split along the
// reduction when its output is too small to fill the chip) and a fused kernel for P, the softmax
// Jacobian and dQ with Kbar and Vbar resident in LDS.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

// ---- inputs to fp32, eight elements per thread; with `mask`, rows ([B, H, n, 64]) at or past
// their item's length are written as zero
__global__ __launch_bounds__(256) void bw_convert_kernel(const void* src, int src_bf16, float* dst,
                                                        size_t count8, const int32_t* lengths,
                                                        int H, int n, int mask) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count8) return;
    f32x4 lo, hi;
    if (src_bf16) {
        const u32x4 u = ((const u32x4*)src)[i];
        lo = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
        hi = f32x4{__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xFFFF0000u),
                   __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xFFFF0000u)};
    } else {
        lo = ((const f32x4*)src)[2 * i];
        hi = ((const f32x4*)src)[2 * i + 1];
    }
    if (mask) {
        const uint32_t row = (uint32_t)(i >> 3);   // < 2^25 rows
        const int t = (int)(row % (uint32_t)n);
        const int b = (int)(row / ((uint32_t)n * (uint32_t)H));
        if (t >= clamp_len(lengths, b, n)) lo = hi = f32x4{};
    }
    ((f32x4*)dst)[2 * i] = lo;
    ((f32x4*)dst)[2 * i + 1] = hi;
}

// ---- C = alpha A B + beta C over a batch z, operands addressed through strides (BwGemm in
// lf_launch.h), on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).  Workgroup tile 128 x TN
// (TN = 64 NI), four waves in a 2 x 2 grid, each wave 64 x 32 NI as 2 x NI blocks of 32 x 32;
// 32-deep reduction steps staged through LDS, the next step's operands loaded into registers
// while the current one is multiplied.  Operand tiles are read with consecutive threads along
// the operand's contiguous direction (the reduction index when its stride is 1, else the row or
// column index), so global reads coalesce either way.
constexpr int kGM = 128, kGK = 32, kGPad = 1;

__device__ __forceinline__ f32x16 mfma_f32_32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int NI>
__global__ __launch_bounds__(256) void bw_gemm_kernel(BwGemm g) {
    constexpr int TN = 64 * NI;
    constexpr int AE = kGK * kGM / 256, BE = kGK * TN / 256;   // elements per thread and step
    __shared__ float As[kGK][kGM + kGPad];
    __shared__ float Bs[kGK][TN + kGPad];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l = lane & 31, h = lane >> 5;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * (TN / 2);
    const int i0 = blockIdx.y * kGM, j0 = blockIdx.x * TN;
    const int z = blockIdx.z / g.splits, sp = blockIdx.z % g.splits;
    const int kbeg = sp * g.kchunk, kend = min(g.K, kbeg + g.kchunk);
    const long long z1 = z / g.zdiv, z2 = z % g.zdiv;
    const float* A = g.A + z1 * g.a_z1 + z2 * g.a_z2;
    const float* Bm = g.B + z1 * g.b_z1 + z2 * g.b_z2;
    // element it of this thread: reduction index kk0 + it dkk, row / column x0 + it dx
    const bool akf = g.a_kc == 1, bkf = g.b_kc == 1;
    const int a_kk0 = akf ? tid % kGK : tid / kGM, a_dkk = akf ? 0 : 256 / kGM;
    const int a_x0 = akf ? tid / kGK : tid % kGM, a_dx = akf ? 256 / kGK : 0;
    const int b_kk0 = bkf ? tid % kGK : tid / TN, b_dkk = bkf ? 0 : 256 / TN;
    const int b_x0 = bkf ? tid / kGK : tid % TN, b_dx = bkf ? 256 / kGK : 0;
    const long long a_off = (long long)a_x0 * g.a_i + (long long)a_kk0 * g.a_kc;
    const long long b_off = (long long)b_x0 * g.b_j + (long long)b_kk0 * g.b_kc;
    const long long a_st = (long long)a_dx * g.a_i + (long long)a_dkk * g.a_kc;   // uniform
    const long long b_st = (long long)b_dx * g.b_j + (long long)b_dkk * g.b_kc;
    float ra[AE], rb[BE];
    auto fetch = [&](int k0) {
        const float* pa = A + (long long)(k0 / g.kblk) * g.a_kb + (long long)(k0 % g.kblk) * g.a_kc +
                          (long long)i0 * g.a_i + a_off;
        const float* pb = Bm + (long long)(k0 / g.kblk) * g.b_kb + (long long)(k0 % g.kblk) * g.b_kc +
                          (long long)j0 * g.b_j + b_off;
#pragma unroll
        for (int it = 0; it < AE; ++it) {
            const int kk = a_kk0 + it * a_dkk, x = a_x0 + it * a_dx;
            ra[it] = (k0 + kk < kend && i0 + x < g.M) ? pa[it * a_st] : 0.0f;
        }
#pragma unroll
        for (int it = 0; it < BE; ++it) {
            const int kk = b_kk0 + it * b_dkk, x = b_x0 + it * b_dx;
            rb[it] = (k0 + kk < kend && j0 + x < g.N) ? pb[it * b_st] : 0.0f;
        }
    };
    f32x16 acc[2][NI];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};
    if (kbeg < kend) fetch(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += kGK) {
#pragma unroll
        for (int it = 0; it < AE; ++it) As[a_kk0 + it * a_dkk][a_x0 + it * a_dx] = ra[it];
#pragma unroll
        for (int it = 0; it < BE; ++it) Bs[b_kk0 + it * b_dkk][b_x0 + it * b_dx] = rb[it];
        __syncthreads();
        if (k0 + kGK < kend) fetch(k0 + kGK);
#pragma unroll
        for (int kp = 0; kp < kGK; kp += 2) {
            float av[2], bv[NI];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) av[mi] = As[kp + h][wm + 32 * mi + l];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bv[ni] = Bs[kp + h][wn + 32 * ni + l];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma_f32_32(av[mi], bv[ni], acc[mi][ni]);
        }
        __syncthreads();
    }
    // C tile element j of lane (h, l): row 8 (j / 4) + 4 h + j % 4, column l
    float* C = g.C + z1 * g.c_z1 + z2 * g.c_z2;
    const int row_end = g.row_len ? clamp_len(g.row_len, (int)z1, g.M) : g.M;
    float* part = g.splits > 1 ? g.part + ((size_t)sp * g.Z + z) * g.M * g.N : nullptr;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int j = j0 + wn + 32 * ni + l;
            if (j >= g.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = i0 + wm + 32 * mi + 8 * (e >> 2) + 4 * h + (e & 3);
                if (i >= g.M) continue;
                if (part) {
                    part[(size_t)i * g.N + j] = acc[mi][ni][e];
                } else {
                    float* c = C + (long long)i * g.c_i + (long long)j * g.c_j;
                    const float v = g.alpha * acc[mi][ni][e] + (g.beta != 0.0f ? g.beta * *c : 0.0f);
                    *c = i < row_end ? v : 0.0f;
                }
            }
        }
}

// ---- sum of the split partials in chunk order, then alpha / beta into C
__global__ __launch_bounds__(256) void bw_gemm_reduce_kernel(BwGemm g) {
    const size_t mn = (size_t)g.M * g.N, total = mn * g.Z;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    float s = 0.0f;
    for (int sp = 0; sp < g.splits; ++sp) s += g.part[(size_t)sp * total + idx];
    const int z = (int)(idx / mn);
    const int i = (int)((idx % mn) / g.N), j = (int)(idx % g.N);
    const long long z1 = z / g.zdiv, z2 = z % g.zdiv;
    float* c = g.C + z1 * g.c_z1 + z2 * g.c_z2 + (long long)i * g.c_i + (long long)j * g.c_j;
    const float v = g.alpha * s + (g.beta != 0.0f ? g.beta * *c : 0.0f);
    *c = (!g.row_len || i < clamp_len(g.row_len, (int)z1, g.M)) ? v : 0.0f;
}

// ---- per (b, h) and 128 query rows: P and dS (stored transposed, [k, n]) and dQ, on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32).  Kbar and Vbar sit in LDS (row stride 68 floats).  Each
// wave owns 16 query rows q0 + l and works on transposed products, so that a lane (g, l) holds
// the values of query column l:
//   S^T = Kbar Q^T, dP^T = Vbar dO^T   (k x 16: lane holds rows r = 16 rb + 4 g + e, e < 4)
//   softmax and the Jacobian down each column (within the lane, then across the four lanes g)
//   dQ^T = Kbar^T dS^T                  (64 x 16), its B operand taken straight from the dS^T
//                                       accumulators by matching the reduction order
// In the first two products the reduction index c runs over 16 g + t for lane group g, so the
// lane's B operand is its own query row's slice Q[q][16 g .. 16 g + 15] held in registers.
constexpr int kKS = 68;   // LDS row stride of Kbar / Vbar (floats)
constexpr int kAttWaves = 8, kAttRows = 16 * kAttWaves;

template <int KB>   // KB = k / 16 row blocks
__global__ __launch_bounds__(64 * kAttWaves) void bw_attend_kernel(BwAttendArgs a) {
    constexpr int K = KB * 16;
    extern __shared__ float lds[];
    float* kb = lds;              // [K][68]
    float* vb = kb + K * kKS;     // [K][68]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l = lane & 15;
    const int bh = blockIdx.y;
    const int q0 = blockIdx.x * kAttRows + wave * 16;
    const float* kg = a.Kb + (size_t)bh * K * 64;
    const float* vg = a.Vb + (size_t)bh * K * 64;
    for (int e = tid; e < K * 16; e += 64 * kAttWaves) {   // 16-byte pieces
        const int r = e >> 4, c4 = e & 15;
        *(f32x4*)(kb + r * kKS + 4 * c4) = *(const f32x4*)(kg + 4 * e);
        *(f32x4*)(vb + r * kKS + 4 * c4) = *(const f32x4*)(vg + 4 * e);
    }
    __syncthreads();
    if (q0 >= a.n) return;   // no barrier follows
    const size_t head = (size_t)bh * a.n * 64;
    const int q = q0 + l;
    f32x4 qr[4], gr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        qr[u] = *(const f32x4*)(a.Q + head + (size_t)q * 64 + 16 * g + 4 * u);
        gr[u] = *(const f32x4*)(a.dO + head + (size_t)q * 64 + 16 * g + 4 * u);
    }
    f32x4 st[KB], dp[KB];
#pragma unroll
    for (int r = 0; r < KB; ++r) {
        st[r] = f32x4{};
        dp[r] = f32x4{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int r = 0; r < KB; r += 2) {
            const f32x4 k0 = *(const f32x4*)(kb + (16 * r + l) * kKS + 16 * g + 4 * u);
            const f32x4 k1 = *(const f32x4*)(kb + (16 * r + 16 + l) * kKS + 16 * g + 4 * u);
            const f32x4 v0 = *(const f32x4*)(vb + (16 * r + l) * kKS + 16 * g + 4 * u);
            const f32x4 v1 = *(const f32x4*)(vb + (16 * r + 16 + l) * kKS + 16 * g + 4 * u);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                st[r] = mfma_f32_16(k0[t], qr[u][t], st[r]);
                st[r + 1] = mfma_f32_16(k1[t], qr[u][t], st[r + 1]);
                dp[r] = mfma_f32_16(v0[t], gr[u][t], dp[r]);
                dp[r + 1] = mfma_f32_16(v1[t], gr[u][t], dp[r + 1]);
            }
        }
    }
    float mx = st[0][0];
#pragma unroll
    for (int r = 0; r < KB; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, st[r][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < KB; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            st[r][e] = expf(a.scale * (st[r][e] - mx));
            sum += st[r][e];
        }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    const float inv = 1.0f / sum;
    float dsum = 0.0f;
#pragma unroll
    for (int r = 0; r < KB; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            st[r][e] *= inv;   // P
            dsum = fmaf(st[r][e], dp[r][e], dsum);
        }
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    const size_t pcol = (size_t)bh * K * a.n + q;
#pragma unroll
    for (int r = 0; r < KB; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t at = pcol + (size_t)(16 * r + 4 * g + e) * a.n;
            dp[r][e] = st[r][e] * (dp[r][e] - dsum);   // dS
            a.P[at] = st[r][e];
            a.dS[at] = dp[r][e];
        }
    // dQ^T = Kbar^T dS^T: reduction step (r, e) takes row 16 r + 4 g + e in lane group g
    f32x4 dq[4] = {};
#pragma unroll
    for (int r = 0; r < KB; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float* krow = kb + (16 * r + 4 * g + e) * kKS + l;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) dq[cb] = mfma_f32_16(krow[16 * cb], dp[r][e], dq[cb]);
        }
    // dq[cb] element e of lane (g, l): dQ[q][16 cb + 4 g + e]
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
        *(f32x4*)(a.dQ + head + (size_t)q * 64 + 16 * cb + 4 * g) = dq[cb] * a.scale;
}

}  // namespace

hipError_t launch_bw_convert(const void* src, int src_bf16, float* dst, size_t count,
                             const int32_t* lengths, int H, int n, int mask, hipStream_t stream) {
    if (count % 8) return hipErrorInvalidValue;
    const size_t count8 = count / 8;
    const int grid = (int)((count8 + 255) / 256);
    hipLaunchKernelGGL(bw_convert_kernel, dim3(grid), dim3(256), 0, stream, src, src_bf16, dst,
                       count8, lengths, H, n, mask);
    return hipGetLastError();
}

void bw_gemm_plan(BwGemm& g) {
    const long long tiles = (long long)((g.M + kGM - 1) / kGM) *
                            ((g.N + (g.N <= 64 ? 63 : 127)) / (g.N <= 64 ? 64 : 128)) * g.Z;
    int s = 1;
    while (s < 8 && tiles * s < 512 && g.K / (2 * s) >= 256 && 2LL * s * g.Z <= 65535) s *= 2;
    g.kchunk = ((g.K + s - 1) / s + kGK - 1) / kGK * kGK;
    g.splits = (g.K + g.kchunk - 1) / g.kchunk;
    if (g.splits < 1) g.splits = 1;
}

size_t bw_gemm_part_bytes(int M, int N, int K, int Z) {
    BwGemm g{};
    g.M = M; g.N = N; g.K = K; g.Z = Z;
    bw_gemm_plan(g);
    return g.splits > 1 ? (size_t)g.splits * Z * M * N * sizeof(float) : 0;
}

hipError_t launch_bw_gemm(const BwGemm& g, hipStream_t stream) {
    if (g.kblk % kGK || g.splits < 1 || g.kchunk % kGK || (g.splits > 1 && !g.part) ||
        (long long)g.Z * g.splits > 65535 || (g.M + kGM - 1) / kGM > 65535)
        return hipErrorInvalidValue;
    const dim3 grid(g.N <= 64 ? (g.N + 63) / 64 : (g.N + 127) / 128, (g.M + kGM - 1) / kGM,
                    g.Z * g.splits);
    if (g.N <= 64)
        hipLaunchKernelGGL(bw_gemm_kernel<1>, grid, dim3(256), 0, stream, g);
    else
        hipLaunchKernelGGL(bw_gemm_kernel<2>, grid, dim3(256), 0, stream, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.splits == 1) return e;
    const size_t total = (size_t)g.Z * g.M * g.N;
    hipLaunchKernelGGL(bw_gemm_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, g);
    return hipGetLastError();
}

template <int KB>
static hipError_t launch_attend_kb(const BwAttendArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)2 * KB * 16 * kKS * sizeof(float);
    auto kern = bw_attend_kernel<KB>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((a.n + kAttRows - 1) / kAttRows, a.B * a.H),
                       dim3(64 * kAttWaves), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_bw_attend(const BwAttendArgs& a, hipStream_t stream) {
    if (a.n % 16 || a.B * a.H > 65535) return hipErrorInvalidValue;
    switch (a.k / 32) {   // k % 32 == 0, 32 .. 256
        case 1: return launch_attend_kb<2>(a, stream);
        case 2: return launch_attend_kb<4>(a, stream);
        case 3: return launch_attend_kb<6>(a, stream);
        case 4: return launch_attend_kb<8>(a, stream);
        case 5: return launch_attend_kb<10>(a, stream);
        case 6: return launch_attend_kb<12>(a, stream);
        case 7: return launch_attend_kb<14>(a, stream);
        case 8: return launch_attend_kb<16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lf
