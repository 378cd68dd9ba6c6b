// Backward pass of one Linformer layer for learned projections, in fp32 arithmetic (Linformer
// card, 方法适配: E and F are learned, so training needs the gradients with respect to Q, K, V, E
// and F).  Per (b, h), with the keys, values and dO rows past the length taken as zero (those
// positions contribute nothing, and rows of O past the length are fixed at zero):
//   Kbar = E K, Vbar = F V (recomputed),  P = softmax(s Q Kbar^T)
//   dP = dO Vbar^T,  dS = P o (dP - rowsum(P o dP)),  dQ = s dS Kbar        (bw_attend_kernel)
//   dVbar = P^T dO,  dKbar = s dS^T Q   (P, dS recomputed per slot block)   (bw_kv_kernel)
//   dE += dKbar K^T, dK = E^T dKbar, dF += dVbar V^T, dV = F^T dVbar         (bw_gemm_kernel)
// Every contraction runs on the matrix cores with fp32 accumulation: one strided, batched GEMM
// (split along the reduction when its output is too small to fill the chip) and two fused kernels
// with Kbar and Vbar resident on chip, one per query block (P, the softmax Jacobian, dQ and the
// per-query softmax statistics) and one per slot block (P and dS again from those statistics, and
// the reductions over the queries), so no n x k matrix is ever stored, as in FlashAttention-2's
// backward.  All read the inputs in their own dtype and never read the masked rows.
//
// The GEMM multiplies fp32 operands as split bf16 pairs (the "bf16x3" scheme of Henry, Tang and
// Heinecke, "Leveraging the bfloat16 Artificial Intelligence Datatype For Higher-Precision
// Computations", ARITH 2019): v = hi + lo with hi = bf16(v), lo = bf16(v - hi), so hi + lo holds v
// to within 2^-16 |v|, and a b = ah bh + ah bl + al bh with the al bl term (below 2^-16 |a b|)
// dropped, three v_mfma_f32_32x32x16_bf16 in place of 8 v_mfma_f32_32x32x2_f32 per 16-deep step.
// A bf16 operand (Q, K, V, E, F, dO in bf16) is its own hi part, so its products take two.  The
// fused kernel multiplies the same way on v_mfma_f32_16x16x32_bf16.
#include <type_traits>

#include "lf_device.h"
#include "lf_launch.h"
#include "split_bf16.h"

namespace lf {
namespace {

// ---- C = alpha A B + beta C over a batch z, operands addressed through strides (BwGemm in
// lf_launch.h), as split bf16 products (above) on v_mfma_f32_32x32x16_bf16.  Workgroup tile
// 128 x TN (TN = 64 NI), four waves in a 2 x 2 grid, each wave 64 x 32 NI as 2 x NI blocks of
// 32 x 32; 32-deep reduction steps staged through LDS as bf16 hi (and, for fp32 operands, lo)
// planes, the next step's tiles loaded into registers while the current one is multiplied.
// Operand tiles are read with consecutive threads along the operand's contiguous direction (the
// reduction index when its stride is 1, else the row or column index), so global reads coalesce
// either way; the planes keep that direction contiguous ([x][kk] rows of 80 bytes, read 16 bytes
// per lane, or [kk][x] rows with 32-byte blocks XOR-swizzled by kk & 3, read with the transposing
// ds_read_b64_tr_b16), so staging is 8- or 16-byte writes either way.
constexpr int kGM = 128, kGK = 32;
// Strides and bases must keep every 16-byte vector aligned: launch_bw_gemm checks them.

__device__ __forceinline__ f32x4 mfma_f32_16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16 raw bytes (4 fp32 or 8 bf16) <-> fp32 values; the loads keep the raw bytes so that no
// conversion forces an early wait on them
__device__ __forceinline__ void unpack(const u32x4& w, float* v, float) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(w[e]);
}
__device__ __forceinline__ void unpack(const u32x4& w, float* v, uint16_t) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
}
// raw bits of element e of a vector
__device__ __forceinline__ void put_raw(u32x4& w, int e, const float* p) { w[e] = *(const uint32_t*)p; }
__device__ __forceinline__ void put_raw(u32x4& w, int e, const uint16_t* p) {
    w[e >> 1] |= (uint32_t)*p << (16 * (e & 1));
}

// One operand's 32 x TX tile (reduction index kk < 32, row / column x < TX) per step, read in
// 16-byte vectors along the operand's contiguous direction (kk when its stride is 1, else x) and
// staged into LDS as [kk][x].  Vector v of this thread starts at (kk0 + v dkk, x0 + v dx).
template <typename T, int TX, bool kf>   // kf: vectors along kk (its stride is 1), else along x
struct TileLoader {
    static constexpr int VEC = 16 / sizeof(T);
    static constexpr int NV = kGK * TX / (256 * VEC);
    int kk0, dkk, x0, dx;
    long long sx, sk, off, st;   // element strides along x and kk; this thread's offsets
    u32x4 raw[NV];
    __device__ void init(int tid, long long stride_x, long long stride_k) {
        sx = stride_x;
        sk = stride_k;
        if constexpr (kf) {
            constexpr int per = kGK / VEC;   // vectors along one row
            kk0 = (tid % per) * VEC; dkk = 0;
            x0 = tid / per; dx = 256 / per;
        } else {
            constexpr int per = TX / VEC;
            x0 = (tid % per) * VEC; dx = 0;
            kk0 = tid / per; dkk = 256 / per;
        }
        off = (long long)x0 * sx + (long long)kk0 * sk;
        st = (long long)dx * sx + (long long)dkk * sk;
    }
    // p: element (kk = 0, x = 0) of this step; elements with kk >= kn or x >= xn read as zero
    __device__ void fetch(const T* p, int kn, int xn) {
        if (kn >= kGK && xn >= TX) {   // the whole tile (uniform across the workgroup)
#pragma unroll
            for (int v = 0; v < NV; ++v) raw[v] = *(const u32x4*)(p + off + v * st);
            return;
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int kk = kk0 + v * dkk, x = x0 + v * dx;
            const T* q = p + off + v * st;
            constexpr bool k_vec = kf;
            const bool full = k_vec ? (x < xn && kk + VEC <= kn) : (kk < kn && x + VEC <= xn);
            if (full) {
                raw[v] = *(const u32x4*)q;
            } else {
                raw[v] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (k_vec ? (x < xn && kk + e < kn) : (kk < kn && x + e < xn)) put_raw(raw[v], e, q + e);
            }
        }
    }
    // byte offset of (kk, x) in a [kk][x] plane (TX bf16 per row, 32-byte blocks swizzled by kk & 3)
    __device__ static int tr_off(int kk, int x) {
        return kk * TX * 2 + ((((x >> 4) ^ (kk & 3))) << 5) + (x & 15) * 2;
    }
    // The tile as bf16 planes, [x][kk] (reduction index contiguous) when kf, else [kk][x]
    // (read back transposed): hi = bf16(v) and, for fp32
    // operands, lo = bf16(v - hi), so hi + lo carries v to within 2^-16 of |v|
    template <int LDK, bool LO>
    __device__ void stage_split(uint16_t (*Sh)[LDK], uint16_t (*Sl)[LDK]) const {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int kk = kk0 + v * dkk, x = x0 + v * dx;
            if constexpr (!LO) {   // bf16 operand: its bits are the hi plane
                if constexpr (kf) {
                    *(u32x4*)&Sh[x][kk] = raw[v];
                } else {   // [kk][x] rows, 32-byte blocks swizzled by kk & 3
                    *(u32x4*)((uint8_t*)Sh + tr_off(kk, x)) = raw[v];
                }
            } else {
                float d[VEC];
                unpack(raw[v], d, T{});
                uint16_t hv[VEC], lv[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    hv[e] = f32_to_bf16(d[e]);
                    lv[e] = f32_to_bf16(d[e] - bf16_to_f32(hv[e]));
                }
                if constexpr (kf) {
#pragma unroll
                    for (int e = 0; e < VEC; e += 2) {
                        *(uint32_t*)&Sh[x][kk + e] = (uint32_t)hv[e] | ((uint32_t)hv[e + 1] << 16);
                        *(uint32_t*)&Sl[x][kk + e] = (uint32_t)lv[e] | ((uint32_t)lv[e + 1] << 16);
                    }
                } else {   // [kk][x] rows: VEC (4) consecutive x, 8 bytes in one 32-byte block
                    *(u32x2*)((uint8_t*)Sh + tr_off(kk, x)) =
                        u32x2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
                    *(u32x2*)((uint8_t*)Sl + tr_off(kk, x)) =
                        u32x2{(uint32_t)lv[0] | ((uint32_t)lv[1] << 16), (uint32_t)lv[2] | ((uint32_t)lv[3] << 16)};
                }
            }
        }
    }
};

// TA, TB: float or uint16_t (bf16) operands; AKF, BKF: the operand's reduction stride is 1
template <int NI, typename TA, bool AKF, typename TB, bool BKF>
__global__ __launch_bounds__(256) void bw_gemm_kernel(BwGemm g) {
    constexpr int TN = 64 * NI;
    constexpr bool LOA = !std::is_same<TA, uint16_t>::value, LOB = !std::is_same<TB, uint16_t>::value;
    // kf operands: [x][kk] planes with 80-byte rows (the 16-byte operand reads of 8 rows cover
    // all banks); the others: [kk][x] planes (same bytes), read with ds_read_b64_tr_b16
    constexpr int LDK = kGK + 8;
    static_assert(kGK * kGM <= kGM * LDK && kGK * TN <= TN * LDK, "planes fit");
    __shared__ __attribute__((aligned(16))) uint16_t Ash[kGM][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Asl[LOA ? kGM : 1][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bsh[TN][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bsl[LOB ? TN : 1][LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l = lane & 31, h = lane >> 5;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * (TN / 2);
    // operand of columns c0 .. c0 + 31 (c0 % 32 == 0), reduction 16 ks + 8 h .. + 7, from a plane
    auto read_op = [&](const uint16_t (*S)[LDK], bool kfo, int TXo, int c0, int ks) {
        if (kfo) return *(const bf16x8*)&S[c0 + l][16 * ks + 8 * h];
        // transposed read: each 16-lane group takes a 4 x 16 block of [kk][x] (the operand order
        // of lane (l, h) = column c0 + l, reduction 16 ks + 8 h + (0..7))
        const int grp16 = lane >> 4, s16 = lane & 15;
        const int tq = 8 * (grp16 >> 1) + (s16 >> 2);
        const int cblk = 2 * (c0 >> 5) + (grp16 & 1);
        const int cin = (s16 & 3) * 8;
        s16x4 v[2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int t = 16 * ks + tq + 4 * rd;
            const uint8_t* p = (const uint8_t*)S + t * TXo * 2 + ((cblk ^ (t & 3)) << 5) + cin;
            v[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(uintptr_t)(
                    (__attribute__((address_space(3))) const uint8_t*)p));
        }
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };

    const int i0 = blockIdx.y * kGM, j0 = blockIdx.x * TN;
    const int z = blockIdx.z / g.splits, sp = blockIdx.z % g.splits;
    // second operand set for the upper half of the batch (zhalf > 0)
    const bool hi2 = g.zhalf > 0 && z >= g.zhalf;
    const int zo = hi2 ? z - g.zhalf : z;
    const long long z1 = zo / g.zdiv, z2 = zo % g.zdiv;
    const int row_end = g.row_len ? clamp_len(g.row_len, (int)z1, g.M) : g.M;
    const int kbeg = sp * g.kchunk;
    int kend = min(g.K, kbeg + g.kchunk);
    if (g.k_len) kend = min(kend, clamp_len(g.k_len, (int)z1, g.K));   // terms past it are zero
    if (i0 >= row_end) kend = kbeg;                                      // rows written as zero
    const TA* A = (const TA*)(hi2 ? g.A2 : g.A) + z1 * g.a_z1 + z2 * g.a_z2 + (long long)i0 * g.a_i;
    const TB* Bm = (const TB*)(hi2 ? g.B2 : g.B) + z1 * g.b_z1 + z2 * g.b_z2 + (long long)j0 * g.b_j;
    TileLoader<TA, kGM, AKF> la;
    TileLoader<TB, TN, BKF> lb;
    la.init(tid, g.a_i, g.a_kc);
    lb.init(tid, g.b_j, g.b_kc);
    auto fetch = [&](int k0) {
        const long long kb = k0 / g.kblk, kc = k0 % g.kblk;
        // columns of B at or past the length of the reduction block's item read as zero
        const int jend = g.bj_len ? clamp_len(g.bj_len, (int)(kb / g.bj_div), g.N) : g.N;
        la.fetch(A + kb * g.a_kb + kc * g.a_kc, kend - k0, g.M - i0);
        lb.fetch(Bm + kb * g.b_kb + kc * g.b_kc, kend - k0, jend - j0);
    };
    f32x16 acc[2][NI];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};
    if (kbeg < kend) fetch(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += kGK) {
        la.template stage_split<LDK, LOA>(Ash, Asl);
        lb.template stage_split<LDK, LOB>(Bsh, Bsl);
        __syncthreads();
        if (k0 + kGK < kend) fetch(k0 + kGK);
        // two 16-deep sub-steps: a b = ah bh + ah bl + al bh (the al bl term, below 2^-16 of |a b|,
        // is dropped), v_mfma_f32_32x32x16_bf16 with fp32 accumulation
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 ah[2], al[2], bh[NI], bl[NI];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                ah[mi] = read_op(Ash, AKF, kGM, wm + 32 * mi, ks);
                if constexpr (LOA) al[mi] = read_op(Asl, AKF, kGM, wm + 32 * mi, ks);
            }
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                bh[ni] = read_op(Bsh, BKF, TN, wn + 32 * ni, ks);
                if constexpr (LOB) bl[ni] = read_op(Bsl, BKF, TN, wn + 32 * ni, ks);
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    if constexpr (LOA) acc[mi][ni] = mfma32(al[mi], bh[ni], acc[mi][ni]);
                    if constexpr (LOB) acc[mi][ni] = mfma32(ah[mi], bl[ni], acc[mi][ni]);
                    acc[mi][ni] = mfma32(ah[mi], bh[ni], acc[mi][ni]);
                }
        }
        __syncthreads();
    }
    // C tile element j of lane (h, l): row 8 (j / 4) + 4 h + j % 4, column l
    float* C = (hi2 ? g.C2 : g.C) + z1 * g.c_z1 + z2 * g.c_z2;
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
template <int V>   // V consecutive columns per thread (4 when C's rows are contiguous, N % 4 == 0)
__global__ __launch_bounds__(256) void bw_gemm_reduce_kernel(BwGemm g) {
    const size_t mn = (size_t)g.M * g.N, total = mn * g.Z;
    const size_t idx = ((size_t)blockIdx.x * 256 + threadIdx.x) * V;
    if (idx >= total) return;
    float s[V] = {};
    auto add = [&](const float* q) {
        if constexpr (V == 4) {
            const f32x4 w = *(const f32x4*)q;
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] += w[e];
        } else {
            s[0] += *q;
        }
    };
    // eight splits' loads in flight at a time (the adds stay in split order)
    int sp = 0;
    for (; sp + 8 <= g.splits; sp += 8) {
        float w[8][V];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float* q = g.part + (size_t)(sp + u) * total + idx;
            if constexpr (V == 4) {
                const f32x4 x = *(const f32x4*)q;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[u][e] = x[e];
            } else {
                w[u][0] = *q;
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < V; ++e) s[e] += w[u][e];
    }
    for (; sp < g.splits; ++sp) add(g.part + (size_t)sp * total + idx);
    const int z = (int)(idx / mn);
    const int i = (int)((idx % mn) / g.N), j = (int)(idx % g.N);
    const bool hi2 = g.zhalf > 0 && z >= g.zhalf;
    const int zo = hi2 ? z - g.zhalf : z;
    const long long z1 = zo / g.zdiv, z2 = zo % g.zdiv;
    const bool keep = !g.row_len || i < clamp_len(g.row_len, (int)z1, g.M);
    float* c = (hi2 ? g.C2 : g.C) + z1 * g.c_z1 + z2 * g.c_z2 + (long long)i * g.c_i + (long long)j * g.c_j;
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const float v = g.alpha * s[e] + (g.beta != 0.0f ? g.beta * c[e] : 0.0f);
        c[e] = keep ? v : 0.0f;
    }
}

// ---- per (b, h) and a range of 128-query blocks: the softmax statistics and dQ, as split bf16
// products (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Kbar and Vbar sit in LDS for the whole
// range as bf16 hi and lo planes ([k][64], 16-byte chunks XOR-swizzled by (r ^ r >> 3) & 7).  Each
// wave owns 16 query rows q0 + l of a block and works on transposed products, so that lane (g, l)
// holds the values of query l:
//   S^T = Kbar Q^T, dP^T = Vbar dO^T   (k x 16: lane holds rows 16 rb + 4 g + e, e < 4), the
//        query's Q / dO slices at d = 32 kc + 8 g .. + 7 (kc = 0, 1) as the B operands, the
//        planes' rows 16 rb + l as the A operands (hi and lo: Kbar = hi + lo within 2^-16)
//   softmax and the Jacobian down each column (within the lane, then across the four lanes g)
//   dQ^T = Kbar^T dS^T                  (64 x 16): per 32 slots the B operand is the lane's dS^T
//        values of rows 32 j + 4 g + e and 32 j + 16 + 4 g + e straight from the accumulators
//        (split into hi and lo), and the A operand Kbar^T is read at exactly those slots with the
//        transposing ds_read_b64_tr_b16 (lane i of a 16-lane group receives element i % 4 of
//        source lanes 4 r + i / 4: source lane s reads the 4 columns 16 cb + 4 (s % 4) of row
//        32 j + 4 g + s / 4, so lane i gets column 16 cb + i of those rows)
// Per query it stores (c m, 1 / sum, D) (D = rowsum(P o dP)), from which bw_kv_kernel recomputes
// P and dS for the reductions over the queries, so neither [n, k] matrix reaches memory.  The next
// block's Q, dO slices are loaded into registers before this block's dQ products.  A wave whose 16
// rows all lie at or past the item's length only writes zero dQ rows (its statistics are left
// unwritten: bw_kv_kernel never uses queries past the length).
constexpr int kAttWaves = 8, kAttRows = 16 * kAttWaves;

template <int KB, typename TQ>   // KB = k / 16 row blocks (even); TQ: float or uint16_t (bf16) Q, dO
__global__ __launch_bounds__(64 * kAttWaves) void bw_attend_kernel(BwAttendArgs a) {
    constexpr int K = KB * 16;
    constexpr int PL = K * 128;   // bytes of one [k][64] bf16 plane
    constexpr bool QLO = sizeof(TQ) == 4;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l = lane & 15;
    const int bh = blockIdx.y;
    const float* kg = a.Kb + (size_t)bh * K * 64;
    const float* vg = a.Vb + (size_t)bh * K * 64;
    const int L = clamp_len(a.lengths, bh / a.H, a.n);
    const size_t head = (size_t)bh * a.n * 64;
    const float c = a.scale * 1.4426950408889634f;   // scores to base-2 exponents
    const int nblk = (a.n + kAttRows - 1) / kAttRows;
    const int blk0 = blockIdx.x * a.qb, blk1 = min(nblk, blk0 + a.qb);
    // Q and dO rows past the length read as zeros (their dQ rows come out zero)
    const __amdgpu_buffer_rsrc_t rsq = row_rsrc((const TQ*)a.Q + head, L);
    const __amdgpu_buffer_rsrc_t rsg = row_rsrc((const TQ*)a.dO + head, L);
    RowOps<TQ> qr, gr;
    auto load_rows = [&](int q) {
        qr.load(rsq, q, g);
        gr.load(rsg, q, g);
    };
    // the first block's rows are in flight while Kbar and Vbar are staged
    bool loaded = false;
    if (blk0 < blk1 && blk0 * kAttRows + wave * 16 < min(a.n, L)) {
        load_rows(blk0 * kAttRows + wave * 16 + l);
        loaded = true;
    }
    stage_kv<K, 64 * kAttWaves>(lds8, kg, vg, tid);
    __syncthreads();   // the only barrier
    // per-lane LDS bases.  Row reads of rows 16 r + l: the chunk swizzle repeats every 4 blocks
    // (it sees (2 r) mod 8), so block r reads base[kc][r % 4] + (r / 4) 8192 (+ PL for the lo
    // plane), the Vbar planes from their own bases.  Transposed reads of rows 32 j (+ 16) + tr_row:
    // the swizzle repeats every 2 blocks, so tb[j % 2][half][cb] + (j / 2) 8192.
    uint32_t kbase[2][4], vbase[2][4], tb[2][2][4];
    {
        const uint32_t l0 = lds_u32(lds8);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                kbase[kc][rr] = opaque_u32(l0 + kv_off(16 * rr + l, 32 * kc + 8 * g));
                vbase[kc][rr] = opaque_u32(l0 + 2 * PL + kv_off(16 * rr + l, 32 * kc + 8 * g));
            }
#pragma unroll
        for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    tb[par][hf][cb] = opaque_u32(
                        l0 + kv_off(32 * par + 16 * hf + 4 * g + (l >> 2), 16 * cb + 4 * (l & 3)));
    }
    for (int blk = blk0; blk < blk1; ++blk) {
        const int q0 = blk * kAttRows + wave * 16;
        if (q0 >= a.n) break;
        const int q = q0 + l;
        if (q0 >= L) {   // wholly past the length: zero dQ
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                *(f32x4*)(a.dQ + head + (size_t)q * 64 + 16 * cb + 4 * g) = f32x4{};
            continue;
        }
        if (!loaded) load_rows(q);
        f32x4 st[KB], dp[KB];
#pragma unroll
        for (int r = 0; r < KB; ++r) {
            st[r] = f32x4{};
            dp[r] = f32x4{};
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            bf16x8 qh, ql, gh, gl;
            qr.ops(kc, qh, ql);
            gr.ops(kc, gh, gl);
#pragma unroll
            for (int r = 0; r < KB; ++r) {
                const uint32_t ro = (r >> 2) * 8192;
                const bf16x8 k0 = lds16a(kbase[kc][r & 3] + ro), k1 = lds16a(kbase[kc][r & 3] + PL + ro);
                const bf16x8 v0 = lds16a(vbase[kc][r & 3] + ro), v1 = lds16a(vbase[kc][r & 3] + PL + ro);
                st[r] = mfma16(k1, qh, st[r]);
                dp[r] = mfma16(v1, gh, dp[r]);
                if constexpr (QLO) {
                    st[r] = mfma16(k0, ql, st[r]);
                    dp[r] = mfma16(v0, gl, dp[r]);
                }
                st[r] = mfma16(k0, qh, st[r]);
                dp[r] = mfma16(v0, gh, dp[r]);
            }
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
        // the query's statistics, from which bw_kv_kernel recomputes P and dS
        if (g == 0)
            *(f32x4*)(a.stats + ((size_t)bh * a.n + q) * 4) = f32x4{mc, inv, dsum, 0.0f};
#pragma unroll
        for (int r = 0; r < KB; ++r) dp[r] = st[r] * (dp[r] - dsum);   // dS
        // next block's rows into the same registers; they arrive during the dQ products
        loaded = false;
        if (blk + 1 < blk1 && q0 + kAttRows < min(a.n, L)) {
            load_rows(q + kAttRows);
            loaded = true;
        }
        // dQ^T = Kbar^T dS^T over 32 slots at a time
        f32x4 dq[4] = {};
#pragma unroll
        for (int j = 0; j < KB / 2; ++j) {
            u32x2 h0, l0, h1, l1;
            split4(dp[2 * j], h0, l0);
            split4(dp[2 * j + 1], h1, l1);
            const bf16x8 bhi = pair8(h0, h1), blo = pair8(l0, l1);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const uint32_t a0 = tb[j & 1][0][cb] + (j >> 1) * 8192;
                const uint32_t a1 = tb[j & 1][1][cb] + (j >> 1) * 8192;
                const bf16x8 ah = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lds_tra(a0), lds_tra(a1), 0, 1, 2, 3, 4, 5, 6, 7));
                const bf16x8 al = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lds_tra(a0 + PL), lds_tra(a1 + PL), 0, 1, 2, 3, 4, 5, 6, 7));
                dq[cb] = mfma16(al, bhi, dq[cb]);
                dq[cb] = mfma16(ah, blo, dq[cb]);
                dq[cb] = mfma16(ah, bhi, dq[cb]);
            }
        }
        // dq[cb] element e of lane (g, l): dQ[q][16 cb + 4 g + e]
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            *(f32x4*)(a.dQ + head + (size_t)q * 64 + 16 * cb + 4 * g) = dq[cb] * a.scale;
    }
}

// ---- dVbar = P^T dO and dKbar = scale dS^T Q per (b, h), block of 64 slots and half of the valid
// queries (or all of them), P and dS recomputed from bw_attend_kernel's per-query statistics (the
// reductions over the queries of FlashAttention-2's backward, with the projected slots in the role
// of its keys).  Four waves; wave w owns the 16 slots s0 = 64 blockIdx.x + 16 w: their Kbar and
// Vbar rows sit in registers as hi and lo bf16 operands.  The workgroup streams its queries
// through LDS in chunks of 32 (Q and dO as hi, and for fp32 inputs lo, planes [32][64] with the
// 16-byte chunk swizzle of split_bf16.h, and the chunk's statistics), double-buffered, the
// next-but-one chunk in registers.  Per chunk and wave, with lane (g, l) holding C[4 g + e][l] of a
// 16 x 16 block:
//   S = Q Kbar^T, dP = dO Vbar^T   (32 queries x 16 slots: query rows as A operands from LDS,
//                                   the slots' rows as B operands from registers)
//   P = exp2(c s - c m) / sum, dS = P o (dP - D)   (queries at or past the length: 0)
//   dVbar^T += dO^T P, dKbar^T += Q^T dS   (64 x 16: per 32 queries the B operand is the lane's
//        P / dS of queries 4 g + e and 16 + 4 g + e straight from the accumulators, split into hi
//        and lo, and the A operand dO^T / Q^T is read at exactly those queries with the
//        transposing ds_read_b64_tr_b16)
// and at the end each wave writes its 16 slots' rows of dKbar (times scale) and dVbar, after
// adding the other query half's sums when the queries are split (BwKvArgs).  Small workgroups
// and the query split fill the chip: three workgroups share a compute unit, and B H ceil(k / 64)
// tiles below two per compute unit are doubled by the split.
constexpr int kKvWaves = 4, kKvSlots = 16 * kKvWaves;

template <typename TQ>
__global__ __launch_bounds__(64 * kKvWaves) void bw_kv_kernel(BwKvArgs a) {
    constexpr bool QLO = sizeof(TQ) == 4;
    constexpr int CQ = 32;                  // queries per chunk
    constexpr int PLB = CQ * 128;           // bytes of one [32][64] bf16 plane
    constexpr int NPL = QLO ? 4 : 2;        // planes per chunk: Q hi (lo), dO hi (lo)
    constexpr int BUF = NPL * PLB + CQ * 16; // planes, then the statistics
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l = lane & 15;
    const int bh = blockIdx.z, qpart = blockIdx.y;
    const int s0 = kKvSlots * blockIdx.x + 16 * wave;
    const bool active = s0 < a.k;
    const int L = clamp_len(a.lengths, bh / a.H, a.n);
    const size_t head = (size_t)bh * a.n * 64;
    const float c = a.scale * kLog2e;
    // this wave's slots' rows as B operands: lane (g, l) holds row s0 + l, columns 32 kc + 8 g ..
    bf16x8 kbh[2], kbl[2], vbh[2], vbl[2];
    if (active) {
        const float* kr = a.Kb + ((size_t)bh * a.k + s0 + l) * 64;
        const float* vr = a.Vb + ((size_t)bh * a.k + s0 + l) * 64;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            u32x2 h0, l0, h1, l1;
            split4(*(const f32x4*)(kr + 32 * kc + 8 * g), h0, l0);
            split4(*(const f32x4*)(kr + 32 * kc + 8 * g + 4), h1, l1);
            kbh[kc] = pair8(h0, h1);
            kbl[kc] = pair8(l0, l1);
            split4(*(const f32x4*)(vr + 32 * kc + 8 * g), h0, l0);
            split4(*(const f32x4*)(vr + 32 * kc + 8 * g + 4), h1, l1);
            vbh[kc] = pair8(h0, h1);
            vbl[kc] = pair8(l0, l1);
        }
    }
    // chunk loads: thread t takes 8 values of Q and of dO (bf16: 16 bytes; fp32: 32 bytes, split)
    // at row t / 8, columns 8 (t % 8) .. + 7, and thread t < 32 the statistics of query t.
    // Buffer descriptors sized to the rows before the length return zeros past it, so the loads
    // need no branches (and none waits for another).
    const uint32_t rows = (uint32_t)L * 64 * sizeof(TQ);
    const __amdgpu_buffer_rsrc_t rsq =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const TQ*)a.Q + head), 0, rows, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsg =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const TQ*)a.dO + head), 0, rows, 0x00020000);
    const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.stats + (size_t)bh * a.n * 4), 0, (uint32_t)L * 16, 0x00020000);
    const int lr = tid >> 3, lc = 8 * (tid & 7);
    // two register sets: chunk ch + 2 is loaded into set ch % 2 while chunk ch is multiplied and
    // chunk ch + 1 (set (ch + 1) % 2) waits to be stored, so each load has two chunks' time to land
    constexpr int QW = sizeof(TQ) / 2;   // 16-byte pieces per thread and matrix
    u32x4 rq[2][QW], rg[2][QW];
    f32x4 rs[2];
    auto load_chunk = [&](auto set, int q0) {
        constexpr int S = decltype(set)::value;
        const uint32_t off = (uint32_t)((q0 + lr) * 64 + lc) * sizeof(TQ);
#pragma unroll
        for (int w = 0; w < QW; ++w) {
            rq[S][w] = __builtin_amdgcn_raw_buffer_load_b128(rsq, off + 16 * w, 0, 0);
            rg[S][w] = __builtin_amdgcn_raw_buffer_load_b128(rsg, off + 16 * w, 0, 0);
        }
        rs[S] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rss, (uint32_t)(q0 + (tid & (CQ - 1))) * 16, 0, 0));
    };
    auto store_chunk = [&](auto set) {
        constexpr int S = decltype(set)::value;
        uint8_t* buf = lds + S * BUF;
        const int off = kv_off(lr, lc);   // one whole 16-byte chunk of the row
        if constexpr (QLO) {
            u32x2 h0, o0, h1, o1;
            split4(__builtin_bit_cast(f32x4, rq[S][0]), h0, o0);
            split4(__builtin_bit_cast(f32x4, rq[S][1]), h1, o1);
            *(bf16x8*)(buf + off) = pair8(h0, h1);
            *(bf16x8*)(buf + PLB + off) = pair8(o0, o1);
            split4(__builtin_bit_cast(f32x4, rg[S][0]), h0, o0);
            split4(__builtin_bit_cast(f32x4, rg[S][1]), h1, o1);
            *(bf16x8*)(buf + 2 * PLB + off) = pair8(h0, h1);
            *(bf16x8*)(buf + 3 * PLB + off) = pair8(o0, o1);
        } else {
            *(u32x4*)(buf + off) = rq[S][0];
            *(u32x4*)(buf + PLB + off) = rg[S][0];
        }
        if (tid < CQ) *(f32x4*)(buf + NPL * PLB + tid * 16) = rs[S];
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    const int tr_row = 4 * g + (l >> 2), tr_col = 4 * (l & 3);
    f32x4 dk[4] = {}, dv[4] = {};
    // this workgroup's chunks: all of them, or one of two halves of the valid ones
    const int ntot = (L + CQ - 1) / CQ;
    const int cbeg = ntot * qpart / a.qparts, nchunk = ntot * (qpart + 1) / a.qparts - cbeg;
    const int qbase = cbeg * CQ;
    if (nchunk > 0) {
        load_chunk(I0{}, qbase);
        if (nchunk > 1) load_chunk(I1{}, qbase + CQ);
        store_chunk(I0{});
    }
    __syncthreads();
    // one chunk; the buffer parity is a compile-time constant, so every LDS read is a per-lane
    // offset (the same for both buffers) plus an immediate
    auto chunk = [&](auto parity, int ch) {
        constexpr int PAR = decltype(parity)::value;
        const uint8_t* buf = lds + PAR * BUF;
        if (ch + 2 < nchunk) load_chunk(parity, qbase + (ch + 2) * CQ);
        if (active) {
            const uint8_t* qh = buf;
            const uint8_t* ql = buf + PLB;
            const uint8_t* gh = buf + (QLO ? 2 : 1) * PLB;
            const uint8_t* gl = buf + 3 * PLB;
            const float* st = (const float*)(buf + NPL * PLB);
            f32x4 sc[2], dp[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                sc[qb] = f32x4{};
                dp[qb] = f32x4{};
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const int off = kv_off(16 * qb + l, 32 * kc + 8 * g);
                    const bf16x8 aq = lds16(qh, off), ag = lds16(gh, off);
                    sc[qb] = mfma16(aq, kbl[kc], sc[qb]);
                    dp[qb] = mfma16(ag, vbl[kc], dp[qb]);
                    if constexpr (QLO) {
                        sc[qb] = mfma16(lds16(ql, off), kbh[kc], sc[qb]);
                        dp[qb] = mfma16(lds16(gl, off), vbh[kc], dp[qb]);
                    }
                    sc[qb] = mfma16(aq, kbh[kc], sc[qb]);
                    dp[qb] = mfma16(ag, vbh[kc], dp[qb]);
                }
                // P and dS of queries 16 qb + 4 g + e.  Past the length Q, dO and the statistics
                // all read as zero, so P = exp2(0) * 0 and dS = 0 there without a test.
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f32x4 sq = *(const f32x4*)(st + 4 * (16 * qb + 4 * g + e));
                    const float P = __builtin_amdgcn_exp2f(fmaf(sc[qb][e], c, -sq[0])) * sq[1];
                    sc[qb][e] = P;
                    dp[qb][e] = P * (dp[qb][e] - sq[2]);
                }
            }
            u32x2 ph0, pl0, ph1, pl1, dh0, dl0, dh1, dl1;
            split4(sc[0], ph0, pl0);
            split4(sc[1], ph1, pl1);
            split4(dp[0], dh0, dl0);
            split4(dp[1], dh1, dl1);
            const bf16x8 bph = pair8(ph0, ph1), bpl = pair8(pl0, pl1);
            const bf16x8 bdh = pair8(dh0, dh1), bdl = pair8(dl0, dl1);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int o0 = kv_off(tr_row, 16 * cb + tr_col);
                const int o1 = kv_off(16 + tr_row, 16 * cb + tr_col);
                const bf16x8 agh = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lds_tr(gh, o0), lds_tr(gh, o1), 0, 1, 2, 3, 4, 5, 6, 7));
                const bf16x8 aqh = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lds_tr(qh, o0), lds_tr(qh, o1), 0, 1, 2, 3, 4, 5, 6, 7));
                dv[cb] = mfma16(agh, bpl, dv[cb]);
                dk[cb] = mfma16(aqh, bdl, dk[cb]);
                if constexpr (QLO) {
                    const bf16x8 agl = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lds_tr(gl, o0), lds_tr(gl, o1), 0, 1, 2, 3, 4, 5, 6, 7));
                    const bf16x8 aql = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lds_tr(ql, o0), lds_tr(ql, o1), 0, 1, 2, 3, 4, 5, 6, 7));
                    dv[cb] = mfma16(agl, bph, dv[cb]);
                    dk[cb] = mfma16(aql, bdh, dk[cb]);
                }
                dv[cb] = mfma16(agh, bph, dv[cb]);
                dk[cb] = mfma16(aqh, bdh, dk[cb]);
            }
        }
        if (ch + 1 < nchunk) store_chunk(std::integral_constant<int, 1 - PAR>{});
        __syncthreads();
    };
    for (int ch = 0; ch < nchunk; ch += 2) {
        chunk(I0{}, ch);
        if (ch + 1 < nchunk) chunk(I1{}, ch + 1);
    }
    if (a.qparts == 2) {
        // the two query halves of a tile: the first to get here leaves its sums (agent-coherent
        // stores, 1 KB of contiguous bytes per instruction) and exits, the other adds them
        const int tile = bh * gridDim.x + blockIdx.x;
        unsigned long long* ctr = a.pair_ctr + tile;
        const unsigned long long tag_in = a.pair_epoch << 1, tag_ready = tag_in | 1ull;
        __shared__ int s_role;   // 0: first, 1: second (sums not ready yet), 2: second (ready)
        if (tid == 0) {
            const unsigned long long prev =
                __hip_atomic_exchange(ctr, tag_in, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_role = prev == tag_ready ? 2 : (prev == tag_in ? 1 : 0);
        }
        __syncthreads();
        const int role = s_role;
        constexpr uint32_t kWaveBytes = 8 * 64 * 16;   // dk[4], dv[4] of every lane
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            a.part + ((size_t)tile * kKvWaves + wave) * (kWaveBytes / 4), 0, kWaveBytes, 0x00020000);
        constexpr int kSC0 = 1, kSC1 = 16;   // cache-policy bits: agent-coherent access
        if (role == 0) {
            if (active) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4, q < 4 ? dk[q] : dv[q - 4]), rp, (q * 64 + lane) * 16, 0, kSC1);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's sums are out
            __syncthreads();                      // everyone's
            if (tid == 0)
                __hip_atomic_store(ctr, tag_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (tid == 0) {
            // the first workgroup is past its exchange with only stores left, so this wait ends;
            // the bound only guards against a counter that held this call's tag before it
            for (int it = 0; role == 1 && it < (1 << 20) &&
                             __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag_ready;
                 ++it)
                __builtin_amdgcn_s_sleep(2);
            __hip_atomic_store(ctr, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const f32x4 v = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, (q * 64 + lane) * 16, 0, kSC0 | kSC1));
                if (q < 4) dk[q] += v;
                else dv[q - 4] += v;
            }
        }
    }
    if (!active) return;
    // dv[cb] element e of lane (g, l): dVbar[s0 + l][16 cb + 4 g + e]
    float* dkr = a.dKb + ((size_t)bh * a.k + s0 + l) * 64;
    float* dvr = a.dVb + ((size_t)bh * a.k + s0 + l) * 64;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        *(f32x4*)(dkr + 16 * cb + 4 * g) = dk[cb] * a.scale;
        *(f32x4*)(dvr + 16 * cb + 4 * g) = dv[cb];
    }
}

}  // namespace

// Every 16-byte vector the tile loaders read stays aligned: bases 16-byte aligned, every stride a
// multiple of the elements per vector.
static bool vec_aligned(const BwGemm& g) {
    auto ok = [](long long contiguous, long long other, long long z1, long long z2, long long kb,
                 long long vec) {
        return contiguous == 1 && other % vec == 0 && z1 % vec == 0 && z2 % vec == 0 &&
               kb % vec == 0;
    };
    const long long va = g.a_bf16 ? 8 : 4, vb = g.b_bf16 ? 8 : 4;
    const bool a = g.a_kc == 1 ? ok(g.a_kc, g.a_i, g.a_z1, g.a_z2, g.a_kb, va)
                               : ok(g.a_i, g.a_kc, g.a_z1, g.a_z2, g.a_kb, va);
    const bool b = g.b_kc == 1 ? ok(g.b_kc, g.b_j, g.b_z1, g.b_z2, g.b_kb, vb)
                               : ok(g.b_j, g.b_kc, g.b_z1, g.b_z2, g.b_kb, vb);
    return a && b && ((uintptr_t)g.A & 15) == 0 && ((uintptr_t)g.B & 15) == 0 &&
           (g.zhalf == 0 || (((uintptr_t)g.A2 & 15) == 0 && ((uintptr_t)g.B2 & 15) == 0));
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
        (g.bj_len && g.bj_div < 1) || !vec_aligned(g) ||
        (long long)g.Z * g.splits > 65535 || (g.M + kGM - 1) / kGM > 65535)
        return hipErrorInvalidValue;
    const dim3 grid(g.N <= 64 ? (g.N + 63) / 64 : (g.N + 127) / 128, (g.M + kGM - 1) / kGM,
                    g.Z * g.splits);
    const int v = (g.N <= 64 ? 0 : 16) + (g.a_bf16 ? 8 : 0) + (g.a_kc == 1 ? 4 : 0) +
                  (g.b_bf16 ? 2 : 0) + (g.b_kc == 1 ? 1 : 0);
    switch (v) {
#define LF_BW_GEMM(V, NI, TA, AKF, TB, BKF)                                                     \
    case V:                                                                                     \
        hipLaunchKernelGGL((bw_gemm_kernel<NI, TA, AKF, TB, BKF>), grid, dim3(256), 0, stream, g); \
        break;
#define LF_BW_GEMM_B(V, NI, TA, AKF)                 \
    LF_BW_GEMM(V + 0, NI, TA, AKF, float, false)     \
    LF_BW_GEMM(V + 1, NI, TA, AKF, float, true)      \
    LF_BW_GEMM(V + 2, NI, TA, AKF, uint16_t, false)  \
    LF_BW_GEMM(V + 3, NI, TA, AKF, uint16_t, true)
        LF_BW_GEMM_B(0, 1, float, false)
        LF_BW_GEMM_B(4, 1, float, true)
        LF_BW_GEMM_B(8, 1, uint16_t, false)
        LF_BW_GEMM_B(12, 1, uint16_t, true)
        LF_BW_GEMM_B(16, 2, float, false)
        LF_BW_GEMM_B(20, 2, float, true)
        LF_BW_GEMM_B(24, 2, uint16_t, false)
        LF_BW_GEMM_B(28, 2, uint16_t, true)
#undef LF_BW_GEMM_B
#undef LF_BW_GEMM
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.splits == 1) return e;
    const size_t total = (size_t)g.Z * g.M * g.N;
    if (g.c_j == 1 && g.N % 4 == 0)   // four contiguous columns per thread
        hipLaunchKernelGGL(bw_gemm_reduce_kernel<4>, dim3((unsigned)((total / 4 + 255) / 256)),
                           dim3(256), 0, stream, g);
    else
        hipLaunchKernelGGL(bw_gemm_reduce_kernel<1>, dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, stream, g);
    return hipGetLastError();
}

template <int KB, typename TQ>
static hipError_t launch_attend_kb(const BwAttendArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)4 * KB * 16 * 128;   // Kbar, Vbar: hi and lo bf16 planes
    auto kern = bw_attend_kernel<KB, TQ>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int nblk = (a.n + kAttRows - 1) / kAttRows;
    hipLaunchKernelGGL(kern, dim3((nblk + a.qb - 1) / a.qb, a.B * a.H), dim3(64 * kAttWaves), lds,
                       stream, a);
    return hipGetLastError();
}

template <typename TQ>
static hipError_t launch_attend_t(const BwAttendArgs& a, hipStream_t stream) {
    switch (a.k / 32) {   // k % 32 == 0, 32 .. 256
        case 1: return launch_attend_kb<2, TQ>(a, stream);
        case 2: return launch_attend_kb<4, TQ>(a, stream);
        case 3: return launch_attend_kb<6, TQ>(a, stream);
        case 4: return launch_attend_kb<8, TQ>(a, stream);
        case 5: return launch_attend_kb<10, TQ>(a, stream);
        case 6: return launch_attend_kb<12, TQ>(a, stream);
        case 7: return launch_attend_kb<14, TQ>(a, stream);
        case 8: return launch_attend_kb<16, TQ>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

int kv_qparts(int B, int H, int k) {
    // fewer than two tiles per compute unit (MI355X: 256): split each tile's queries in two
    const long long tiles = (long long)B * H * ((k + kKvSlots - 1) / kKvSlots);
    return tiles < 512 ? 2 : 1;
}

size_t kv_sums_bytes(int B, int H, int k) {
    return (size_t)B * H * ((k + kKvSlots - 1) / kKvSlots) * kKvWaves * 8 * 64 * 16;
}

size_t kv_part_bytes(int B, int H, int k) {   // the sums, then one counter per tile
    return kv_sums_bytes(B, H, k) + (size_t)B * H * ((k + kKvSlots - 1) / kKvSlots) * 8;
}

hipError_t launch_bw_kv(const BwKvArgs& a, hipStream_t stream) {
    if (a.k % 32 || a.k > 256 || a.B * a.H > 65535 || (a.qparts != 1 && a.qparts != 2) ||
        (a.qparts == 2 && (!a.part || !a.pair_ctr || a.pair_epoch == 0)))
        return hipErrorInvalidValue;
    const dim3 grid((a.k + kKvSlots - 1) / kKvSlots, a.qparts, a.B * a.H);
    if (a.in_bf16) hipLaunchKernelGGL(bw_kv_kernel<uint16_t>, grid, dim3(64 * kKvWaves), 0, stream, a);
    else hipLaunchKernelGGL(bw_kv_kernel<float>, grid, dim3(64 * kKvWaves), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bw_attend(const BwAttendArgs& a, hipStream_t stream) {
    if (a.n % 16 || a.B * a.H > 65535 || a.qb < 1) return hipErrorInvalidValue;
    return a.in_bf16 ? launch_attend_t<uint16_t>(a, stream) : launch_attend_t<float>(a, stream);
}

}  // namespace lf
