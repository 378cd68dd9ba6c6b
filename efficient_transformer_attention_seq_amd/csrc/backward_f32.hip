// Backward pass of one Linformer layer for learned projections, in fp32 arithmetic (Linformer
// card, 方法适配: E and F are learned, so training needs the gradients with respect to Q, K, V, E
// and F).  Per (b, h), with the keys, values and dO rows past the length zeroed beforehand (those
// positions contribute nothing, and rows of O past the length are fixed at zero):
//   Kbar = E K, Vbar = F V (recomputed),  P = softmax(s Q Kbar^T)
//   dP = dO Vbar^T,  dS = P o (dP - rowsum(P o dP)),  dQ = s dS Kbar        (bw_attend_kernel)
//   dVbar = P^T dO,  dKbar = s dS^T Q                                        (bw_gemm_kernel)
//   dE += dKbar K^T, dK = E^T dKbar, dF += dVbar V^T, dV = F^T dVbar         (bw_gemm_kernel)
// The contractions run through one strided, batched fp32 GEMM on the vector units (64 x 64
// tiles, 16-deep K steps through LDS); the softmax Jacobian runs per query row with Kbar and
// Vbar resident in LDS.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

// ---- inputs to fp32, rows at or past each length set to zero ([B, H, n, 64]) or plain copies
__global__ __launch_bounds__(256) void bw_convert_kernel(const void* src, int src_bf16, float* dst,
                                                        size_t count, const int32_t* lengths,
                                                        int H, int n, int mask) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    float v = src_bf16 ? bf16_to_f32(((const uint16_t*)src)[i]) : ((const float*)src)[i];
    if (mask) {
        const size_t row = i / 64;
        const int t = (int)(row % n);
        const int b = (int)(row / ((size_t)n * H));
        if (t >= clamp_len(lengths, b, n)) v = 0.0f;
    }
    dst[i] = v;
}

__global__ __launch_bounds__(256) void bw_mask_rows_kernel(float* x, size_t count,
                                                          const int32_t* lengths, int H, int n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    const size_t row = i / 64;
    const int t = (int)(row % n);
    const int b = (int)(row / ((size_t)n * H));
    if (t >= clamp_len(lengths, b, n)) x[i] = 0.0f;
}

// ---- C = alpha A B + beta C over a batch z, every operand addressed through strides (see
// BwGemm in lf_launch.h); 64 x 64 output tile per workgroup, each thread 4 x 4 outputs.
constexpr int kGT = 64, kGK = 16;

__global__ __launch_bounds__(256) void bw_gemm_kernel(BwGemm g) {
    __shared__ float As[kGK][kGT + 1];
    __shared__ float Bs[kGK][kGT + 1];
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int i0 = blockIdx.y * kGT, j0 = blockIdx.x * kGT;
    const int z = blockIdx.z;
    const long long z1 = z / g.zdiv, z2 = z % g.zdiv;
    const float* A = g.A + z1 * g.a_z1 + z2 * g.a_z2;
    const float* Bm = g.B + z1 * g.b_z1 + z2 * g.b_z2;
    float* C = g.C + z1 * g.c_z1 + z2 * g.c_z2;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < g.K; k0 += kGK) {
        // each thread loads 4 elements of each 16 x 64 operand tile
        for (int e = threadIdx.x; e < kGK * kGT; e += 256) {
            const int kk = e / kGT, x = e % kGT;
            const int k = k0 + kk;
            float av = 0.0f, bv = 0.0f;
            if (k < g.K) {
                const long long kb = k / g.kblk, kc = k % g.kblk;
                if (i0 + x < g.M) av = A[(long long)(i0 + x) * g.a_i + kb * g.a_kb + kc * g.a_kc];
                if (j0 + x < g.N) bv = Bm[kb * g.b_kb + kc * g.b_kc + (long long)(j0 + x) * g.b_j];
            }
            As[kk][x] = av;
            Bs[kk][x] = bv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a[u] = As[kk][ty + 16 * u];
                b[u] = Bs[kk][tx + 16 * u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = i0 + ty + 16 * u;
        if (i >= g.M) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int j = j0 + tx + 16 * v;
            if (j >= g.N) continue;
            float* c = C + (long long)i * g.c_i + (long long)j * g.c_j;
            *c = g.alpha * acc[u][v] + (g.beta != 0.0f ? g.beta * *c : 0.0f);
        }
    }
}

// ---- per (b, h) and 16 query rows: P, dS (stored [n, k]) and dQ.  16 threads per row; thread g
// of a row owns slots r = g + 16 m.  Kbar and Vbar sit in LDS with a 65-float row stride (the 16
// threads of a row read 16 consecutive rows, so they hit distinct banks).
constexpr int kRows = 16;
constexpr int kKS = 65;   // LDS row stride of Kbar / Vbar (floats)

template <int KM>   // KM = k / 16 slots per thread
__global__ __launch_bounds__(256) void bw_attend_kernel(BwAttendArgs a) {
    constexpr int K = KM * 16;
    extern __shared__ float lds[];
    float* kb = lds;                      // [K][65]
    float* vb = kb + K * kKS;             // [K][65]
    float* qs = vb + K * kKS;             // [16][64]
    float* gs = qs + kRows * 64;          // [16][64] dO rows
    float* ds = gs + kRows * 64;          // [16][K]
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int bh = blockIdx.y;
    const int i = blockIdx.x * kRows + ty;
    const size_t head = (size_t)bh * a.n * 64;
    for (int e = tid; e < K * 64; e += 256) {
        const int r = e >> 6, c = e & 63;
        kb[r * kKS + c] = a.Kb[(size_t)bh * K * 64 + e];
        vb[r * kKS + c] = a.Vb[(size_t)bh * K * 64 + e];
    }
    for (int e = tid; e < kRows * 64; e += 256) {
        const int row = blockIdx.x * kRows + (e >> 6);
        qs[e] = a.Q[head + (size_t)row * 64 + (e & 63)];
        gs[e] = a.dO[head + (size_t)row * 64 + (e & 63)];
    }
    __syncthreads();
    const float* q = qs + ty * 64;
    const float* go = gs + ty * 64;
    float sc[KM], dp[KM];
#pragma unroll
    for (int m = 0; m < KM; ++m) {
        const float* kr = kb + (tx + 16 * m) * kKS;
        const float* vr = vb + (tx + 16 * m) * kKS;
        float s = 0.0f, p = 0.0f;
        for (int c = 0; c < 64; ++c) {
            s = fmaf(q[c], kr[c], s);
            p = fmaf(go[c], vr[c], p);
        }
        sc[m] = s * a.scale;
        dp[m] = p;
    }
    float mx = sc[0];
#pragma unroll
    for (int m = 1; m < KM; ++m) mx = fmaxf(mx, sc[m]);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float sum = 0.0f;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
        sc[m] = expf(sc[m] - mx);
        sum += sc[m];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off);
    const float inv = 1.0f / sum;
    float dsum = 0.0f;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
        sc[m] *= inv;   // P
        dsum = fmaf(sc[m], dp[m], dsum);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) dsum += __shfl_xor(dsum, off);
    const size_t prow = ((size_t)bh * a.n + i) * K;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
        const int r = tx + 16 * m;
        const float dsv = sc[m] * (dp[m] - dsum);
        a.P[prow + r] = sc[m];
        a.dS[prow + r] = dsv;
        ds[ty * K + r] = dsv;
    }
    __syncthreads();
    // dQ[i][c] = s sum_r dS[i][r] Kbar[r][c], thread tx owns columns tx + 16 j
    float dq[4] = {0.f, 0.f, 0.f, 0.f};
    const float* dr = ds + ty * K;
    for (int r = 0; r < K; ++r) {
        const float d = dr[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) dq[j] = fmaf(d, kb[r * kKS + tx + 16 * j], dq[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) a.dQ[head + (size_t)i * 64 + tx + 16 * j] = a.scale * dq[j];
}

}  // namespace

hipError_t launch_bw_convert(const void* src, int src_bf16, float* dst, size_t count,
                             const int32_t* lengths, int H, int n, int mask, hipStream_t stream) {
    const int grid = (int)((count + 255) / 256);
    hipLaunchKernelGGL(bw_convert_kernel, dim3(grid), dim3(256), 0, stream, src, src_bf16, dst,
                       count, lengths, H, n, mask);
    return hipGetLastError();
}

hipError_t launch_bw_mask_rows(float* x, size_t count, const int32_t* lengths, int H, int n,
                               hipStream_t stream) {
    const int grid = (int)((count + 255) / 256);
    hipLaunchKernelGGL(bw_mask_rows_kernel, dim3(grid), dim3(256), 0, stream, x, count, lengths,
                       H, n);
    return hipGetLastError();
}

hipError_t launch_bw_gemm(const BwGemm& g, hipStream_t stream) {
    const dim3 grid((g.N + kGT - 1) / kGT, (g.M + kGT - 1) / kGT, g.Z);
    hipLaunchKernelGGL(bw_gemm_kernel, grid, dim3(256), 0, stream, g);
    return hipGetLastError();
}

template <int KM>
static hipError_t launch_attend_km(const BwAttendArgs& a, hipStream_t stream) {
    constexpr int K = KM * 16;
    const size_t lds = (size_t)(2 * K * kKS + 2 * kRows * 64 + kRows * K) * sizeof(float);
    auto kern = bw_attend_kernel<KM>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.n / kRows, a.B * a.H), dim3(256), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_bw_attend(const BwAttendArgs& a, hipStream_t stream) {
    switch (a.k / 32) {   // k % 32 == 0, 32 .. 256
        case 1: return launch_attend_km<2>(a, stream);
        case 2: return launch_attend_km<4>(a, stream);
        case 3: return launch_attend_km<6>(a, stream);
        case 4: return launch_attend_km<8>(a, stream);
        case 5: return launch_attend_km<10>(a, stream);
        case 6: return launch_attend_km<12>(a, stream);
        case 7: return launch_attend_km<14>(a, stream);
        case 8: return launch_attend_km<16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lf
