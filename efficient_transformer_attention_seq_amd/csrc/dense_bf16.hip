// Standard O(n^2) softmax attention, O = softmax(scale * Q . K^T) . V per (b, h), bf16 in, fp32
// accumulation: the dense baseline Linformer is compared against (Linformer 요약 설명, section
// "Transformer and Self-Attention"; Linformer summary card, section 证据 "evidence").
//
// It never stores the n x n matrix: each wave keeps 32 queries and streams 64-key tiles of K and
// V through LDS, updating a running row max and row sum (the softmax is exact; only the order of
// the additions differs from the textbook).  Keys at or past the length are left out of the
// softmax; output rows at or past the length are zero.
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kThreads = 512;
constexpr int kQTB = kDenseQTB;  // queries per workgroup (8 waves x 32)
constexpr int kKT = 64;    // keys per tile
constexpr int kRS = 72;    // LDS row stride (bf16) for both tiles

__device__ __forceinline__ int vperm(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__global__ __launch_bounds__(kThreads) void dense_bf16_kernel(DenseBf16Args a) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKT * kRS];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[2][64 * kRS];

    const int lid = xcd_remap(blockIdx.x, a.nlogical);
    if (lid < 0) return;
    const int qb = lid % a.QB;
    const int bh = lid / a.QB;
    const int b = bh / a.H;
    const int L = clamp_len(a.lengths, b, a.n);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const size_t rowbase = (size_t)bh * a.n;
    const int q0 = qb * kQTB + wave * 32;
    const bool active = q0 < a.n && q0 < L;
    const float c = a.c;

    bf16x8 qop[4];
    if (active) {
        const uint16_t* qrow = a.Q + (rowbase + q0 + l32) * kHeadDim + hh * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qop[ks] = *(const bf16x8*)(qrow + ks * 16);
    }

    // loader: thread -> (key row kr, column chunk cc) of one 64 x 64 tile
    const int kr = tid >> 3, cc = tid & 7;
    const uint16_t* kbase = a.K + rowbase * kHeadDim + cc * 8;
    const uint16_t* vbase = a.V + rowbase * kHeadDim + cc * 8;
    const int ntiles = (L + kKT - 1) / kKT;
    u32x4 kreg = {0u, 0u, 0u, 0u}, vreg = {0u, 0u, 0u, 0u};
    auto load_tile = [&](int kt) {
        const int key = kt * kKT + kr;
        const u32x4 z = {0u, 0u, 0u, 0u};
        kreg = z;
        vreg = z;
        if (key < L) {
            kreg = *(const u32x4*)(kbase + (size_t)key * kHeadDim);
            vreg = *(const u32x4*)(vbase + (size_t)key * kHeadDim);
        }
    };
    auto store_tile = [&](int buf) {
        *(u32x4*)(&sK[buf][kr * kRS + cc * 8]) = kreg;
        const int p = vperm(kr);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = vreg[e >> 1];
            sVt[buf][(cc * 8 + e) * kRS + p] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
        }
    };

    f32x16 o0, o1;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        o0[j] = 0.0f;
        o1[j] = 0.0f;
    }
    float m = -INFINITY, lsum = 0.0f;

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const bool more = kt + 1 < ntiles;
        if (more) load_tile(kt + 1);
        if (active) {
            const uint16_t* tk = sK[kt & 1];
            const uint16_t* tv = sVt[kt & 1];
            f32x16 s[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int j = 0; j < 16; ++j) s[rb][j] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    s[rb] = mfma32(*(const bf16x8*)(tk + (rb * 32 + l32) * kRS + ks * 16 + hh * 8),
                                   qop[ks], s[rb]);
            float tmax = -INFINITY;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = kt * kKT + rb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
                    if (key >= L) s[rb][j] = -INFINITY;
                    tmax = fmaxf(tmax, s[rb][j]);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float mnew = fmaxf(m, tmax);
            const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c);
            const float mc = mnew * c;
            o0 *= alpha;
            o1 *= alpha;
            lsum *= alpha;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                float w[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    w[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][j], c, -mc));
                    lsum += w[j];
                }
                const bf16x8 p0 = pack_bf16x8(w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]);
                const bf16x8 p1 =
                    pack_bf16x8(w[8], w[9], w[10], w[11], w[12], w[13], w[14], w[15]);
                const int vo = l32 * kRS + rb * 32 + hh * 8;
                o0 = mfma32(*(const bf16x8*)(tv + vo), p0, o0);
                o0 = mfma32(*(const bf16x8*)(tv + vo + 16), p1, o0);
                o1 = mfma32(*(const bf16x8*)(tv + vo + 32 * kRS), p0, o1);
                o1 = mfma32(*(const bf16x8*)(tv + vo + 32 * kRS + 16), p1, o1);
            }
            m = mnew;
        }
        __syncthreads();
        if (more) store_tile((kt + 1) & 1);
        __syncthreads();
    }

    if (q0 >= a.n) return;
    const int q = q0 + l32;
    uint16_t* orow = a.O + (rowbase + q) * kHeadDim + 4 * hh;
    const float tot = lsum + __shfl_xor(lsum, 32);
    const bool valid = active && q < L;
    const float inv = valid ? 1.0f / tot : 0.0f;
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

}  // namespace

hipError_t launch_dense_bf16(const DenseBf16Args& a, hipStream_t stream) {
    const int grid = ((a.nlogical + 7) / 8) * 8;
    hipLaunchKernelGGL(dense_bf16_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lf
