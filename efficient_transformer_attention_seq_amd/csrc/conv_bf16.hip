// Convolution / pooling compression of the keys and values (Linformer 요약 설명, section
// "Additional Efficiency Techniques": the sequence may be compressed by pooling or a convolution
// instead of a learned dense projection).  With window s = n / k and stride s:
//     Kbar[r][c] = sum_{j < s} wE[j] K[r s + j][c],   Vbar[r][c] = sum_{j < s} wF[j] V[r s + j][c]
// over the valid positions (r s + j < length), i.e. the projection by the banded E with
// E[r][r s + j] = wE[j]; mean pooling is w = 1/s.  No E is read, so the step streams K and V once
// and is bound by HBM bandwidth: one thread per (unit, projected row, 8 columns), eight
// consecutive threads read one 128-byte row, fp32 accumulation, outputs in the same formats as
// the dense projection (Kbar scaled by c as a bf16 plane + fp8 residual plane + block scales,
// Vbar bf16; lf_launch.h).
#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void conv_proj_bf16_kernel(ConvBf16Args a) {
    const size_t g = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const size_t per_unit = (size_t)a.k * 8;
    const size_t bhn = (size_t)a.B * a.H;
    if (g >= 2 * bhn * per_unit) return;   // (whole 8-lane groups leave together)
    const int u = (int)(g / per_unit);
    const int rem = (int)(g - (size_t)u * per_unit);
    const int r = rem >> 3, cc = rem & 7;
    const int which = u >= (int)bhn ? 1 : 0;
    const int bh = u - which * (int)bhn;
    const int b = bh / a.H, h = bh - b * a.H;
    const int L = clamp_len(a.lengths, b, a.n);
    const uint16_t* w = (which ? a.wF : a.wE) + (size_t)(a.e_heads > 1 ? h : 0) * a.s;
    const uint16_t* X = (which ? a.V : a.K) + ((size_t)bh * a.n) * kHeadDim + cc * 8;

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int t0 = r * a.s;
    const int t1 = min(t0 + a.s, L);
    for (int t = t0; t < t1; ++t) {
        const float wj = bf16_to_f32(w[t - t0]);
        const u32x4 v = *(const u32x4*)(X + (size_t)t * kHeadDim);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += wj * __uint_as_float(v[i] << 16);
            acc[2 * i + 1] += wj * __uint_as_float(v[i] & 0xFFFF0000u);
        }
    }

    const size_t row = (size_t)bh * a.k + r;
    if (which == 1) {
        const u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
        *(u32x4*)(a.Vb + row * kHeadDim + cc * 8) = o;
        return;
    }
    // Kbar: x = c Kbar, hi = bf16(x), lo = x - hi; the four lanes cc = 4 hf .. 4 hf + 3 hold
    // row half hf (d < 32 or d >= 32) and agree on its scale through two shuffles
    float lo[8];
    u32x4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = hi_pair(a.c * acc[2 * i], a.c * acc[2 * i + 1], lo[2 * i], lo[2 * i + 1]);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(lo[i]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    const int sh = lo_shift(m);
    *(u32x4*)(a.Khi + row * kHeadDim + cc * 8) = hv;
    const u32x2 lb = {lo_bytes(lo[0], lo[1], lo[2], lo[3], sh), lo_bytes(lo[4], lo[5], lo[6], lo[7], sh)};
    *(u32x2*)(a.Klo + row * 64 + lo_pos(cc * 8)) = lb;   // columns 8 cc .. 8 cc + 7 are consecutive bytes
    if ((cc & 3) == 0) a.Ksc[row * 2 + (cc >> 2)] = (uint8_t)(127 - sh);
}

}  // namespace

hipError_t launch_conv_bf16(const ConvBf16Args& a, hipStream_t stream) {
    const size_t threads = 2 * (size_t)a.B * a.H * a.k * 8;
    const int grid = (int)((threads + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(conv_proj_bf16_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lf
