// fp32 path: the same Linformer layer to fp32 accuracy (Linformer 요약 설명, section "Model":
// n x k scores, softmax over the k projected slots of each query, weighted sum of Vbar).  The
// projection Kbar = E K, Vbar = F V runs on the strided batched GEMM of backward_f32.hip; the
// attention below.  Both multiply on the bf16 matrix cores as split bf16 pairs with fp32
// accumulation (split_bf16.h: every operand carried to within 2^-16), which holds the fp32 path's
// 1e-4 bar with room to spare (tested: 1e-5 on Kbar, 1e-4 on O).
//
// attend_f32_kernel: one 8-wave workgroup per (b, h) and range of 128-query blocks, Kbar and Vbar
// resident in LDS as hi and lo bf16 planes.  Each wave owns 16 query rows q0 + l of a block and
// works on transposed products so that lane (g, l) holds the values of query l (as the backward's
// fused kernel does):
//   S^T = Kbar Q^T   (k x 16: lane holds rows 16 rb + 4 g + e), Q split into hi and lo in
//                    registers (slices d = 32 kc + 8 g .. + 7), the planes' rows as A operands
//   the exact softmax down each column (within the lane, then across the four lanes g), in base 2
//   O^T = Vbar^T P^T (64 x 16): per 32 slots the B operand is the lane's unnormalised weights of
//                    rows 32 j + 4 g + e and 32 j + 16 + 4 g + e straight from the accumulators
//                    (split into hi and lo), the A operand Vbar^T read at exactly those slots
//                    with the transposing ds_read_b64_tr_b16; each column divided by its weight
//                    sum at the end
// Rows at or past the length are written as zeros.
#include "lf_device.h"
#include "lf_launch.h"
#include "split_bf16.h"

namespace lf {
namespace {

constexpr int kAttWaves = 8, kAttRows = 16 * kAttWaves;

template <int KB>   // KB = k / 16 row blocks (even)
__global__ __launch_bounds__(64 * kAttWaves) void attend_f32_kernel(F32Args a, int qb) {
    constexpr int K = KB * 16;
    constexpr int PL = K * 128;   // bytes of one [k][64] bf16 plane
    extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];
    const uint8_t* kh = lds8;
    const uint8_t* kl = lds8 + PL;
    const uint8_t* vh = lds8 + 2 * PL;
    const uint8_t* vl = lds8 + 3 * PL;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l = lane & 15;
    const int bh = blockIdx.y;
    const float* kg = a.Kbar + (size_t)bh * K * 64;
    const float* vg = a.Vbar + (size_t)bh * K * 64;
    stage_kv<K, 64 * kAttWaves>(lds8, kg, vg, tid);
    __syncthreads();   // the only barrier
    const int L = clamp_len(a.lengths, bh / a.H, a.n);
    const size_t head = (size_t)bh * a.n * 64;
    const __amdgpu_buffer_rsrc_t rsq = row_rsrc(a.Q + head, L);   // rows past the length: zeros
    const float c = a.scale * kLog2e;   // scores to base-2 exponents
    const int nblk = (a.n + kAttRows - 1) / kAttRows;
    const int blk0 = blockIdx.x * qb, blk1 = min(nblk, blk0 + qb);
    // per-lane LDS offsets of the transposed Vbar^T reads: source lane s = l of group g reads
    // columns 16 cb + 4 (l % 4) of rows 32 j + 4 g + l / 4 (+ 16)
    const int tr_row = 4 * g + (l >> 2), tr_col = 4 * (l & 3);
    RowOps<float> qr;
    bool loaded = false;
    for (int blk = blk0; blk < blk1; ++blk) {
        const int q0 = blk * kAttRows + wave * 16;
        if (q0 >= a.n) break;
        const int q = q0 + l;
        if (q0 >= L) {   // wholly past the length
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                *(f32x4*)(a.O + head + (size_t)q * 64 + 16 * cb + 4 * g) = f32x4{};
            continue;
        }
        if (!loaded) qr.load(rsq, q, g);
        f32x4 st[KB];
#pragma unroll
        for (int r = 0; r < KB; ++r) st[r] = f32x4{};
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            bf16x8 qh, ql;
            qr.ops(kc, qh, ql);
#pragma unroll
            for (int r = 0; r < KB; ++r) {
                const int off = kv_off(16 * r + l, 32 * kc + 8 * g);
                const bf16x8 k0 = lds16(kh, off), k1 = lds16(kl, off);
                st[r] = mfma16(k1, qh, st[r]);
                st[r] = mfma16(k0, ql, st[r]);
                st[r] = mfma16(k0, qh, st[r]);
            }
        }
        // next block's Q slices into the same registers; they arrive during the products below
        loaded = false;
        if (blk + 1 < blk1 && q0 + kAttRows < min(a.n, L)) {
            qr.load(rsq, q + kAttRows, g);
            loaded = true;
        }
        float mx = st[0][0];
#pragma unroll
        for (int r = 0; r < KB; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, st[r][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mc = mx * c;
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < KB; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                st[r][e] = __builtin_amdgcn_exp2f(fmaf(st[r][e], c, -mc));
                sum += st[r][e];
            }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        // O^T = Vbar^T W^T over 32 slots at a time, then divided by the weight sum
        f32x4 o[4] = {};
#pragma unroll
        for (int j = 0; j < KB / 2; ++j) {
            u32x2 h0, l0, h1, l1;
            split4(st[2 * j], h0, l0);
            split4(st[2 * j + 1], h1, l1);
            const bf16x8 bhi = pair8(h0, h1), blo = pair8(l0, l1);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int o0 = kv_off(32 * j + tr_row, 16 * cb + tr_col);
                const int o1 = kv_off(32 * j + 16 + tr_row, 16 * cb + tr_col);
                const bf16x8 ah = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lds_tr(vh, o0), lds_tr(vh, o1), 0, 1, 2, 3, 4, 5, 6, 7));
                const bf16x8 al = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lds_tr(vl, o0), lds_tr(vl, o1), 0, 1, 2, 3, 4, 5, 6, 7));
                o[cb] = mfma16(al, bhi, o[cb]);
                o[cb] = mfma16(ah, blo, o[cb]);
                o[cb] = mfma16(ah, bhi, o[cb]);
            }
        }
        // o[cb] element e of lane (g, l): O[q][16 cb + 4 g + e]
        const float inv = 1.0f / sum;
        const bool live = q < L;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            *(f32x4*)(a.O + head + (size_t)q * 64 + 16 * cb + 4 * g) = live ? o[cb] * inv : f32x4{};
    }
}

template <int KB>
hipError_t launch_kb(const F32Args& a, hipStream_t stream) {
    const size_t lds = (size_t)4 * KB * 16 * 128;   // Kbar, Vbar: hi and lo bf16 planes
    auto kern = attend_f32_kernel<KB>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // about three rounds of one workgroup per compute unit (MI355X: 256)
    const int nblk = (a.n + kAttRows - 1) / kAttRows;
    const int qb = max(1, min(nblk, nblk * a.B * a.H / 768));
    hipLaunchKernelGGL(kern, dim3((nblk + qb - 1) / qb, a.B * a.H), dim3(64 * kAttWaves), lds,
                       stream, a, qb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_f32(const F32Args& a, hipStream_t stream) {
    if (a.n % 16 || a.B * a.H > 65535) return hipErrorInvalidValue;
    switch (a.k / 32) {   // k % 32 == 0, 32 .. 256
        case 1: return launch_kb<2>(a, stream);
        case 2: return launch_kb<4>(a, stream);
        case 3: return launch_kb<6>(a, stream);
        case 4: return launch_kb<8>(a, stream);
        case 5: return launch_kb<10>(a, stream);
        case 6: return launch_kb<12>(a, stream);
        case 7: return launch_kb<14>(a, stream);
        case 8: return launch_kb<16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lf
