// fp32 path: the same Linformer layer computed in fp32 with vector FMAs (Linformer 요약 설명,
// section "Model").  It serves fp32 accuracy on small workloads (the single-head n = 512 case is
// 34 MFLOP): what bounds it is latency and the number of workgroups, so both kernels spread the
// work over many short workgroups rather than feeding the matrix cores.
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
// Block (4 waves): 8 slots x 64 columns of one (which, b, h); lane = column, wave w sums the
// positions of the w-th contiguous quarter of [0, L) in ascending order (8 independent
// accumulators; the 8 E entries of a position are the same for the whole wave, so they come in
// through scalar loads), then wave 0 adds the four quarters in order.
constexpr int kProjSlots = 8;
__global__ __launch_bounds__(256) void proj_f32_kernel(F32Args a) {
    __shared__ float part[4][kProjSlots][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r0 = blockIdx.x * kProjSlots;
    const int BH = a.B * a.H;
    const int which = blockIdx.y / BH;
    const int bh = blockIdx.y % BH;
    const int b = bh / a.H, h = bh % a.H;
    const int L = clamp_len(a.lengths, b, a.n);
    const float* A = f32_matrix(a, which, h) + (size_t)r0 * a.n;
    const float* X = (which ? a.V : a.K) + (size_t)bh * a.n * kHeadDim + lane;
    const int t0 = (int)((long long)L * wave / 4), t1 = (int)((long long)L * (wave + 1) / 4);
    float acc[kProjSlots];
#pragma unroll
    for (int i = 0; i < kProjSlots; ++i) acc[i] = 0.0f;
#pragma unroll 4
    for (int t = t0; t < t1; ++t) {
        const float x = X[(size_t)t * kHeadDim];
#pragma unroll
        for (int i = 0; i < kProjSlots; ++i) acc[i] = __builtin_fmaf(A[(size_t)i * a.n + t], x, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < kProjSlots; ++i) part[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave != 0) return;
    float* out = (which ? a.Vbar : a.Kbar) + ((size_t)bh * a.k + r0) * kHeadDim + lane;
#pragma unroll
    for (int i = 0; i < kProjSlots; ++i)
        out[(size_t)i * kHeadDim] = ((part[0][i][lane] + part[1][i][lane]) + part[2][i][lane]) + part[3][i][lane];
}

// One query per wave (4 per block), the head's Kbar and Vbar resident in LDS.  Scores: lane = slot
// (k / 64 passes), the query's 64 values in every lane's registers; softmax over the k slots with
// wave reductions; weighted sum: lane = output column, the weights read back from LDS.
constexpr int kMaxK = 256;
__global__ __launch_bounds__(256) void attend_f32_kernel(F32Args a) {
    __shared__ float sK[kMaxK * 65];   // row stride 65: lane r reads row r conflict-free
    __shared__ float sV[kMaxK * 64];
    __shared__ float sw[4][kMaxK];
    const int bh = blockIdx.y;
    const int b = bh / a.H;
    const int L = clamp_len(a.lengths, b, a.n);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float* gK = a.Kbar + (size_t)bh * a.k * kHeadDim;
    const float* gV = a.Vbar + (size_t)bh * a.k * kHeadDim;
    for (int i = tid; i < a.k * kHeadDim; i += 256) {
        sK[(i >> 6) * 65 + (i & 63)] = gK[i];
        sV[i] = gV[i];
    }
    __syncthreads();
    const int q = blockIdx.x * 4 + wave;
    if (q >= a.n) return;
    float* orow = a.O + ((size_t)bh * a.n + q) * kHeadDim;
    if (q >= L) {
        orow[lane] = 0.0f;
        return;
    }
    float qv[64];
    const f32x4* qrow = (const f32x4*)(a.Q + ((size_t)bh * a.n + q) * kHeadDim);
#pragma unroll
    for (int c4 = 0; c4 < 16; ++c4) {
        const f32x4 v = qrow[c4];
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[4 * c4 + e] = v[e];
    }
    float sc[kMaxK / 64];
    float m = -INFINITY;
#pragma unroll
    for (int p = 0; p < kMaxK / 64; ++p) {
        const int r = 64 * p + lane;
        float s = 0.0f;
        if (r < a.k) {
#pragma unroll
            for (int c = 0; c < 64; ++c) s = __builtin_fmaf(qv[c], sK[r * 65 + c], s);
            s *= a.scale;
            m = fmaxf(m, s);
        }
        sc[p] = s;
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float z = 0.0f;
#pragma unroll
    for (int p = 0; p < kMaxK / 64; ++p) {
        const int r = 64 * p + lane;
        if (r < a.k) {
            const float w = expf(sc[p] - m);
            sw[wave][r] = w;
            z += w;
        }
    }
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's weights are in LDS
    __builtin_amdgcn_wave_barrier();
    float acc = 0.0f;
    for (int r = 0; r < a.k; ++r) acc = __builtin_fmaf(sw[wave][r], sV[r * 64 + lane], acc);
    orow[lane] = acc / z;
}

}  // namespace

hipError_t launch_proj_f32(const F32Args& a, hipStream_t stream) {
    hipLaunchKernelGGL(proj_f32_kernel, dim3(a.k / kProjSlots, 2 * a.B * a.H), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
}

hipError_t launch_attend_f32(const F32Args& a, hipStream_t stream) {
    hipLaunchKernelGGL(attend_f32_kernel, dim3((a.n + 3) / 4, a.B * a.H), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lf
