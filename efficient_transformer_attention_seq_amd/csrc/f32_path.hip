// fp32 path: the same Linformer layer computed in fp32 with vector FMAs (Linformer 요약 설명,
// section "Model").  On MI355X fp32 matrix-core and fp32 vector peaks are the same
// (157.3 TFLOP/s), so this path uses plain vector code; it serves fp32 accuracy (single-head,
// short-sequence workloads), not throughput.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

__device__ __forceinline__ const float* f32_matrix(const F32Args& a, int which, int h) {
    if (a.share == 0) return (which ? a.F : a.E) + (size_t)h * a.k * a.n;
    if (a.share == 1) return which ? a.F : a.E;
    return a.E;
}

// Kbar[b,h][r][c] = sum_{t < L_b} E_h[r][t] K[b,h][t][c]  (and Vbar with F, V).
// Block: 4 slots x 64 columns; grid: (k / 4, 2 * B * H); ascending-t accumulation.
__global__ __launch_bounds__(256) void proj_f32_kernel(F32Args a) {
    const int c = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int BH = a.B * a.H;
    const int which = blockIdx.y / BH;
    const int bh = blockIdx.y % BH;
    const int b = bh / a.H, h = bh % a.H;
    const int L = clamp_len(a.lengths, b, a.n);
    const float* A = f32_matrix(a, which, h) + (size_t)r * a.n;
    const float* X = (which ? a.V : a.K) + (size_t)bh * a.n * kHeadDim + c;
    float acc = 0.0f;
    for (int t = 0; t < L; ++t) acc = __builtin_fmaf(A[t], X[(size_t)t * kHeadDim], acc);
    float* out = which ? a.Vbar : a.Kbar;
    out[((size_t)bh * a.k + r) * kHeadDim + c] = acc;
}

// One wave per query at a time; lane r-stripes the k slots for the scores and owns output column
// c = lane for the weighted sum.  Kbar and Vbar of the head are resident in LDS.
constexpr int kMaxK = 256;
__global__ __launch_bounds__(256) void attend_f32_kernel(F32Args a) {
    __shared__ float sK[kMaxK * 65];
    __shared__ float sV[kMaxK * 64];
    const int bh = blockIdx.y;
    const int b = bh / a.H;
    const int L = clamp_len(a.lengths, b, a.n);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const float* gK = a.Kbar + (size_t)bh * a.k * kHeadDim;
    const float* gV = a.Vbar + (size_t)bh * a.k * kHeadDim;
    for (int i = tid; i < a.k * kHeadDim; i += 256) {
        sK[(i >> 6) * 65 + (i & 63)] = gK[i];
        sV[i] = gV[i];
    }
    __syncthreads();
    const int kq = a.k >> 6;        // full 64-slot stripes
    const int krem = a.k & 63;      // slots in the last partial stripe
    const int q_begin = blockIdx.x * 64;
    for (int q = q_begin + wave; q < min(a.n, q_begin + 64); q += 4) {
        float* orow = a.O + ((size_t)bh * a.n + q) * kHeadDim;
        if (q >= L) {
            orow[lane] = 0.0f;
            continue;
        }
        const float qv = a.Q[((size_t)bh * a.n + q) * kHeadDim + lane];
        float sc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int cc = 0; cc < kHeadDim; ++cc) {
            const float qc = __shfl(qv, cc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = i * 64 + lane;
                if (r < a.k) sc[i] = __builtin_fmaf(qc, sK[r * 65 + cc], sc[i]);
            }
        }
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = i * 64 + lane;
            sc[i] *= a.scale;
            if (r < a.k) m = fmaxf(m, sc[i]);
        }
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        float w[4], z = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = i * 64 + lane;
            w[i] = (r < a.k) ? expf(sc[i] - m) : 0.0f;
            z += w[i];
        }
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cnt = (i < kq) ? 64 : (i == kq ? krem : 0);
            for (int j = 0; j < cnt; ++j)
                acc = __builtin_fmaf(__shfl(w[i], j), sV[(i * 64 + j) * 64 + lane], acc);
        }
        orow[lane] = acc / z;
    }
}

}  // namespace

hipError_t launch_proj_f32(const F32Args& a, hipStream_t stream) {
    hipLaunchKernelGGL(proj_f32_kernel, dim3(a.k / 4, 2 * a.B * a.H), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_attend_f32(const F32Args& a, hipStream_t stream) {
    hipLaunchKernelGGL(attend_f32_kernel, dim3((a.n + 63) / 64, a.B * a.H), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace lf
