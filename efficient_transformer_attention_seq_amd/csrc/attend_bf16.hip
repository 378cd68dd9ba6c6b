// Compressed attention O = softmax(scale * Q . Kbar^T) . Vbar for bf16 inputs, one query tile of
// 32 rows per wave (Linformer 요약 설명, section "Model": n x k scores, softmax over the k
// projected slots of each query, weighted sum of Vbar; queries are not compressed).
//
// Workgroup = one (b, h) and `qtb` consecutive queries, 8 waves.  Kbar (hi and lo planes) and
// Vbar of that head stay resident in LDS for the whole workgroup:
//   Kbar planes: [k][72] bf16 (64 + 8 pad -> 16-B reads of 8 consecutive rows hit distinct banks)
//   Vbar^T     : [64][k + 8] bf16, slots permuted inside each group of 16 (bits 2 and 3 of the
//                slot index swapped) so a lane's eight softmax weights, taken straight from the
//                score accumulator, meet eight contiguous Vbar^T entries.
// Per wave and tile of 32 queries:
//   1. S^T (k x 32) = Kbar . Q^T with 32x32x16 bf16 MFMAs: two per step (hi plane, lo plane), so the
//      scores carry Kbar to fp32 accuracy; Q is the B operand straight from global memory.
//   2. Exact single-pass softmax per query: all k scores of a query sit in two lanes (l, l+32),
//      so the row max and row sum are in-register reductions plus one cross-lane exchange.
//      w = exp2(s * c - m * c) with c = scale * log2(e) folded into one FMA.
//   3. O^T (64 x 32) = Vbar^T . W^T with the unnormalised weights rounded to bf16 as the B
//      operand, then each output column (one query) is divided by its row sum.
// Rows at or past the sequence length are written as zeros.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kThreads = kAttendThreads;
constexpr int kKS = 72;  // Kbar plane row stride in bf16 elements

__device__ __forceinline__ int vperm(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ void zero_rows(uint16_t* O, size_t row0, int nrows, int lane) {
    // nrows x 64 bf16 = nrows * 128 B, 16 B per lane per store
    const u32x4 z = {0u, 0u, 0u, 0u};
    uint16_t* base = O + row0 * kHeadDim;
    for (int ch = lane; ch < nrows * 8; ch += 64) *(u32x4*)(base + ch * 8) = z;
}

template <int KB>
__global__ __launch_bounds__(kThreads) void attend_bf16_kernel(AttendBf16Args a) {
    constexpr int K = KB * 32;
    constexpr int VS = K + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sKh[K * kKS];
    __shared__ __attribute__((aligned(16))) uint16_t sKl[K * kKS];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[64 * VS];

    const int lid = xcd_remap(blockIdx.x, a.nlogical);
    if (lid < 0) return;
    const int qb = lid % a.QB;
    const int bh = lid / a.QB;
    const int b = bh / a.H;
    const int L = clamp_len(a.lengths, b, a.n);
    const int q_begin = qb * a.qtb;
    const int q_end = min(a.n, q_begin + a.qtb);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const size_t rowbase = (size_t)bh * a.n;

    if (q_begin >= L) {  // whole workgroup in the padding: zeros only
        for (int r0 = q_begin + wave * 32; r0 < q_end; r0 += 8 * 32)
            zero_rows(a.O, rowbase + r0, min(32, q_end - r0), lane);
        return;
    }

    {
        const uint16_t* gKh = a.Khi + (size_t)bh * K * kHeadDim;
        const uint16_t* gKl = a.Klo + (size_t)bh * K * kHeadDim;
        const uint16_t* gV = a.Vb + (size_t)bh * K * kHeadDim;
        for (int ch = tid; ch < K * 8; ch += kThreads) {
            const int r = ch >> 3, cc = ch & 7;
            const u32x4 kh = *(const u32x4*)(gKh + r * kHeadDim + cc * 8);
            const u32x4 kl = *(const u32x4*)(gKl + r * kHeadDim + cc * 8);
            const u32x4 v = *(const u32x4*)(gV + r * kHeadDim + cc * 8);
            *(u32x4*)(sKh + r * kKS + cc * 8) = kh;
            *(u32x4*)(sKl + r * kKS + cc * 8) = kl;
            const int p = vperm(r);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w = v[e >> 1];
                sVt[(cc * 8 + e) * VS + p] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
            }
        }
    }
    __syncthreads();

    const float c = a.c;
    for (int q0 = q_begin + wave * 32; q0 < q_end; q0 += 8 * 32) {
        if (q0 >= L) {
            zero_rows(a.O, rowbase + q0, min(32, q_end - q0), lane);
            continue;
        }
        // ---- Q tile as the B operand: lane holds Q[q0 + l32][16 ks + 8 hh .. +8]
        const uint16_t* qrow = a.Q + (rowbase + q0 + l32) * kHeadDim + hh * 8;
        bf16x8 qop[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qop[ks] = *(const bf16x8*)(qrow + ks * 16);

        // ---- scores S^T = Kbar . Q^T, Kbar = hi + lo
        f32x16 s[KB];
#pragma unroll
        for (int rb = 0; rb < KB; ++rb)
#pragma unroll
            for (int j = 0; j < 16; ++j) s[rb][j] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int rb = 0; rb < KB; ++rb) {
                const int off = (rb * 32 + l32) * kKS + ks * 16 + hh * 8;
                s[rb] = mfma32(*(const bf16x8*)(sKh + off), qop[ks], s[rb]);
                s[rb] = mfma32(*(const bf16x8*)(sKl + off), qop[ks], s[rb]);
            }
        }

        // ---- exact softmax over the k slots of query q0 + l32 (split over lanes l32, l32+32)
        float m = s[0][0];
#pragma unroll
        for (int rb = 0; rb < KB; ++rb)
#pragma unroll
            for (int j = 0; j < 16; ++j) m = fmaxf(m, s[rb][j]);
        m = fmaxf(m, __shfl_xor(m, 32));
        const float mc = m * c;

        f32x16 o0, o1;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            o0[j] = 0.0f;
            o1[j] = 0.0f;
        }
        float z = 0.0f;
#pragma unroll
        for (int rb = 0; rb < KB; ++rb) {
            float w[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                w[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][j], c, -mc));
                z += w[j];
            }
            const bf16x8 p0 = pack_bf16x8(w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]);
            const bf16x8 p1 = pack_bf16x8(w[8], w[9], w[10], w[11], w[12], w[13], w[14], w[15]);
            const int vo = l32 * VS + rb * 32 + hh * 8;
            o0 = mfma32(*(const bf16x8*)(sVt + vo), p0, o0);
            o0 = mfma32(*(const bf16x8*)(sVt + vo + 16), p1, o0);
            o1 = mfma32(*(const bf16x8*)(sVt + vo + 32 * VS), p0, o1);
            o1 = mfma32(*(const bf16x8*)(sVt + vo + 32 * VS + 16), p1, o1);
        }
        z += __shfl_xor(z, 32);
        const float inv = 1.0f / z;

        // ---- store: lane holds O[q0 + l32][c] for c = 32 mt + 8 gq + 4 hh + (0..3)
        const int q = q0 + l32;
        uint16_t* orow = a.O + (rowbase + q) * kHeadDim + 4 * hh;
        const bool valid = q < L;
        if (q < q_end) {
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
