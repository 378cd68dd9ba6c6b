// Internal launcher interface between the C-ABI host layer (api.cpp) and the kernel translation
// units.  Every launcher assumes its arguments were validated by api.cpp and returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace lf {

// Projection work is organised in "units": one unit = one (which, b, h) output matrix, with
// which = 0 for Kbar = A.K and 1 for Vbar = A.V.  Units that multiply the same projection matrix A
// form a group; a group's units share every load of A.
//   unshared  : group g = which * H + h, members b            (A = E_h or F_h)
//   headwise  : group g = which,          members (b, h)       (A = E or F)
//   key-value / layerwise: one group,     members (which, b, h) (A = E)
//   single (kProjSingle, internal): one group, members (b, h), which = 1 only: Vbar = E . V with
//             bf16 output (used by the encoder stack to project its layer input once)
// Unit (which, b, h) reads rows t = 0 .. n-1 of K or V at element offset b xb + h xh + t xrow
// (64 contiguous elements per row): [B, H, n, 64] is xb = H n 64, xh = n 64, xrow = 64.
constexpr int kProjSingle = 4;
struct ProjGeom {
    int B, H, n, k, share;
    long long xb, xh;     // unit strides of K and V (elements)
    int xrow;             // row stride of K and V (elements, >= 64)
    int groups;           // number of distinct A matrices in use
    int members;          // units per group
    int cfg;              // tile configuration id
    int upt;              // units per workgroup tile
    int slot_tiles;       // workgroup tiles along the k slots
    int stages;           // LDS ring depth
    int threads;          // threads per workgroup
    int tiles_per_group;  // ceil(members / upt)
    int S;                // splits of the position axis
    int steps_per_split;  // 64-position steps in one split
    int nlogical;         // groups * S * tiles_per_group
};

// bf16 Kbar storage (the attention kernel's operand format).  With c = scale * log2(e) and
// x = c * Kbar[r][d] (fp32):
//   Khi [B, H, k, 64] bf16 : hi = bf16(x), round to nearest even
//   Klo [B, H, k, 64] byte : e4m3(lo * 2^s) with lo = x - hi, one power-of-two scale 2^s per row
//                            and per half d < 32 / d >= 32 ("block"), chosen so that the block's
//                            largest |lo| * 2^s lies in [128, 256); within a row, byte
//                            32 h + p holds d = 16 (p / 8) + 8 h + p % 8 (the order in which a
//                            lane of the 32x32x64 fp8 MFMA holds the 64 products)
//   Ksc [B, H, k, 2]  byte : 127 - s for blocks 0 and 1 (an E8M0 exponent: the MFMA scales the
//                            block's products by 2^-s)
// so x = hi + lo8 * 2^-s to within 2^-12 of the largest |x| of its block.
constexpr int kLoBlockHi = 128, kLoBlockTop = 256;

struct ProjBf16Args {
    const uint16_t* K;
    const uint16_t* V;
    const uint16_t* E;
    const uint16_t* F;      // never null here (= E when shared or when unshared F is omitted)
    const int32_t* lengths;
    uint16_t* Khi;          // [B, H, k, 64]
    uint8_t* Klo;           // [B, H, k, 64]
    uint8_t* Ksc;           // [B, H, k, 2]
    uint16_t* Vb;           // [B, H, k, 64]
    // fp32 outputs instead (the backward pass): when Kf is set, Kbar and Vbar are stored unscaled
    // in fp32 at Kf and Vf ([B, H, k, 64] each) and Khi, Klo, Ksc, Vb and c are not used
    float* Kf;
    float* Vf;
    float* part;            // [S, 2, B*H, k, 64] when S > 1 (paired: per tile, see below)
    float c;                // scale * log2(e), applied to Kbar before it is stored
    ProjGeom g;
    // Two splits paired in the kernel (S == 2 and pair_epoch != 0): of the two workgroups of a
    // tile, the one that finishes its half of the reduction first leaves its sums in `part` (per
    // tile, the workgroup's accumulators in register order: tile t's block starts at t * KS * UPT
    // * 64 floats) and marks the tile's counter ready; the other adds them to its own sums and
    // stores the result (no fixup launch).  pair_ctr[t] (one per tile) holds 0 or this call's tags
    // 2 pair_epoch (one arrived) and 2 pair_epoch + 1 (sums ready) and is left at 0; pair_epoch is
    // unique per call and below 2^62, so counters left over by an earlier call never match.
    unsigned long long* pair_ctr;
    unsigned long long pair_epoch;
};

struct AttendBf16Args {
    const uint16_t* Q;
    const uint16_t* Khi;
    const uint8_t* Klo;
    const uint8_t* Ksc;
    const uint16_t* Vb;
    const int32_t* lengths;
    uint16_t* O;
    int B, H, n, k;
    int nlogical;  // persistent grid size (multiple of 8)
};

// fp32 attention (f32_path.hip); the fp32 projection is a BwGemm (below)
struct F32Args {
    const float* Q;         // [B, H, n, 64]
    const int32_t* lengths;
    const float* Kbar;      // [B, H, k, 64], unscaled
    const float* Vbar;
    float* O;
    int B, H, n, k;
    float scale;
};

// Convolution / pooling compression (conv_bf16.hip): window weights instead of a dense E.
struct ConvBf16Args {
    const uint16_t* K;
    const uint16_t* V;
    const uint16_t* wE;     // [e_heads, s] window weights for the keys
    const uint16_t* wF;     // [e_heads, s] for the values (= wE when shared)
    const int32_t* lengths;
    uint16_t* Khi;          // Kbar planes as for the dense projection
    uint8_t* Klo;
    uint8_t* Ksc;
    uint16_t* Vb;
    int B, H, n, k, s;      // s = n / k
    int e_heads;            // H (per-head weights) or 1
    float c;                // scale * log2(e)
};

// Backward pass (backward_f32.hip).  Strided batched fp32 GEMM on the matrix cores:
//   C(z, i, j) = alpha sum_{kk < K} A(z, i, kk) B(z, kk, j) + beta C(z, i, j)
// with z1 = z / zdiv, z2 = z % zdiv, kb = kk / kblk, kc = kk % kblk and
//   A(z, i, kk) at A + z1 a_z1 + z2 a_z2 + i a_i + kb a_kb + kc a_kc
//   B(z, kk, j) at B + z1 b_z1 + z2 b_z2 + kb b_kb + kc b_kc + j b_j
//   C(z, i, j)  at C + z1 c_z1 + z2 c_z2 + i c_i + j c_j
// kblk must be a multiple of 32.  The reduction may be split into `splits` chunks of `kchunk`
// (set by bw_gemm_plan); each chunk then writes its partial sums to `part` ([splits][Z][M][N]
// fp32, bw_gemm_part_bytes) and a second kernel adds them in chunk order.
struct BwGemm {
    const void* A;     // fp32, or bf16 with a_bf16
    const void* B;     // fp32, or bf16 with b_bf16
    float* C;
    int M, N, K, Z, zdiv, kblk;
    long long a_z1, a_z2, a_i, a_kb, a_kc;   // strides in elements
    long long b_z1, b_z2, b_kb, b_kc, b_j;
    long long c_z1, c_z2, c_i, c_j;
    float alpha, beta;
    int splits, kchunk;
    float* part;
    const int32_t* row_len;   // optional: rows i >= row_len[z1] of C are written as zero
    const int32_t* k_len;     // optional: the reduction stops at kk < k_len[z1] (the terms past
                              // it are known to be zero, or their operands unwritten)
    const int32_t* bj_len;    // optional: B(z, kk, j) reads as zero for j >= bj_len[kb / bj_div]
    int bj_div;
    int a_bf16, b_bf16;
    // optional: batch entries z >= zhalf (> 0) use A2, B2, C2 with z - zhalf (two products of one
    // shape in one launch: Z = 2 zhalf)
    int zhalf;
    const void* A2;
    const void* B2;
    float* C2;
};

// Chooses splits / kchunk for g's shape (enough workgroups to cover the chip).
void bw_gemm_plan(BwGemm& g);
// Partial-sum bytes a GEMM of this shape needs after bw_gemm_plan (0 without a split).
size_t bw_gemm_part_bytes(int M, int N, int K, int Z);

struct BwAttendArgs {
    const void* Q;     // [B, H, n, 64], fp32 or (in_bf16) bf16
    const void* dO;    // [B, H, n, 64]; rows at or past the length read as zero
    const float* Kb;   // [B, H, k, 64]
    const float* Vb;
    const int32_t* lengths;   // optional per-item lengths
    float* stats;      // [B, H, n, 4]: per query (c m, 1 / sum, D, 0) with P = exp2(c s - c m) / sum
                       // (c = scale log2 e) and D = rowsum(P o dP); rows of 16-query groups wholly
                       // past the length unwritten
    float* dQ;         // [B, H, n, 64]
    int B, H, n, k;
    int qb;            // 128-query blocks per workgroup
    int in_bf16;
    float scale;
};

// dVbar = P^T dO and dKbar = scale dS^T Q (backward_f32.hip, bw_kv_kernel), P and dS recomputed
// from Q, dO, Kbar, Vbar and the fused kernel's per-query statistics
struct BwKvArgs {
    const void* Q;     // as BwAttendArgs
    const void* dO;
    const float* Kb;
    const float* Vb;
    const float* stats;
    const int32_t* lengths;
    float* dKb;        // [B, H, k, 64]
    float* dVb;
    int B, H, n, k;
    int in_bf16;
    float scale;
    // qparts = 2: the valid queries of each (b, h) are split in two halves, one workgroup each; of
    // the two, the one that finishes first leaves its partial sums in `part` (kv_part_bytes()
    // bytes, per 64-slot tile and wave 8 KB in register order) and marks the tile's counter
    // pair_ctr[tile] (B H ceil(k / 64) counters) with 2 pair_epoch + 1; the other adds them (a + b,
    // the same bits in either order) and stores.  Counters hold 0 or this call's tags and are left
    // at 0; pair_epoch is unique per call and below 2^62.
    int qparts;
    float* part;
    unsigned long long* pair_ctr;
    unsigned long long pair_epoch;
};
hipError_t launch_bw_kv(const BwKvArgs& a, hipStream_t stream);
// query halves per (b, h) the slot-block kernel uses; the bytes of its partial sums, and of the
// sums followed by the tiles' counters
int kv_qparts(int B, int H, int k);
size_t kv_sums_bytes(int B, int H, int k);
size_t kv_part_bytes(int B, int H, int k);

// Dense projection Y = X . W^T of the encoder attention stack (linear_bf16.hip).
struct LinearBf16Args {
    const uint16_t* W;   // [F, K] bf16, row f = output feature f
    const uint16_t* X;   // activations, per act_mode
    uint16_t* Y;         // output, per out_mode
    int T, F, K;         // tokens (a partial last tile reads zeros), features (multiple of
                         // kLinearTileF), K % 64 == 0
    int n, H;            // tokens per batch item and heads (head-planar layouts)
    int act_mode;        // 0: row-major [T, K]; 1: head-planar [B, H, n, 64] with K = 64 H
    int out_mode;        // 0: row-major [T, F]; 1: head-planar planes [F / dm][B, H, n, 64];
                         // 2: Kbar (features < dm, stored as the attention's Kbar planes, scaled
                         //    by c) then Vbar (features >= dm, bf16 [B, H, n, 64]); here the
                         //    "tokens" are projected slots, n = k
    int dm;              // plane width in features (64 H) for out_modes 1 and 2
    size_t plane;        // elements of one plane (out_mode 1)
    uint8_t* Klo;        // out_mode 2: Kbar residual plane and block scales; Y is the Kbar hi
    uint8_t* Ksc;        //   plane and Yv the Vbar plane
    uint16_t* Yv;
    float c;             // out_mode 2: scale * log2(e)
    int tile_t;          // token tile: 256 or 128
    int nlogical;        // (F / kLinearTileF) * ceil(T / tile_t)
};

struct DenseBf16Args {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    const int32_t* lengths;
    uint16_t* O;
    int B, H, n;
    int QB;
    int nlogical;
    float c;  // scale * log2(e)
};

// Fused path (fused_bf16.hip): projection into LDS and attention in one launch, one workgroup per
// (b, h).  Sequence form (dm = 0): Kbar = E_h K, Vbar = E_h V over the valid positions, one
// projection matrix for keys and values.  Stack form (dm = d_model): Kbar = Xbar_b W_K,h^T,
// Vbar = Xbar_b W_V,h^T over the d_model features, with E = Xbar ([B, H, k, 64], the layer input
// projected along the sequence) and K = W (the layer's rows of W_K then W_V, [2 dm, dm]).
struct FusedBf16Args {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    const uint16_t* E;      // [e_heads, k, n], projects both the keys and the values
    const int32_t* lengths;
    uint16_t* O;
    int B, H, n, k;
    int e_heads;            // H (per-head E_h) or 1
    float c;                // scale * log2(e)
    int dm;                 // 0, or d_model for the stack form
    // Work split, mode 0: workgroups 0 .. whole - 1 take (b, h) = their index, all of its query
    // tiles; the units after those are each taken by `parts` workgroups that all project the unit
    // and attend contiguous shares of its tiles (a last round of fewer units than compute units).
    // Mode 2 (grid < units <= 3 grid / 2, sequence form): `grid` workgroups each take unit w;
    // workgroup 2 j also projects the extra unit grid + j first and publishes its planes in
    // global memory (Khi, Klo, Ksc, Vb in the attention kernel's format, then an epoch-tagged
    // flag per unit), and workgroup 2 j + 1 attends all of it after its own unit.  A workgroup
    // only waits for a unit published by a workgroup of lower index.
    int whole;
    int parts;
    int mode;
    int grid;
    uint16_t* Khi;
    uint8_t* Klo;
    uint8_t* Ksc;
    uint16_t* Vb;
    unsigned long long* flags;   // one per unit
    unsigned long long epoch;    // this call's tag (nonzero)
};
bool fused_supported(int n, int k);
hipError_t launch_fused_bf16(const FusedBf16Args& a, hipStream_t stream);

// Projection geometry for a problem (deterministic; `split_override` > 0 forces S,
// `cfg_override` names a tile configuration).  Returns false if the shape is unsupported.
bool proj_geometry(int B, int H, int n, int k, int share, int split_override,
                   const char* cfg_override, ProjGeom* out);

hipError_t launch_proj_bf16(const ProjBf16Args& a, hipStream_t stream);
hipError_t launch_attend_bf16(const AttendBf16Args& a, hipStream_t stream);
hipError_t launch_attend_f32(const F32Args& a, hipStream_t stream);
hipError_t launch_dense_bf16(const DenseBf16Args& a, hipStream_t stream);
hipError_t launch_linear_bf16(const LinearBf16Args& a, hipStream_t stream);
hipError_t launch_conv_bf16(const ConvBf16Args& a, hipStream_t stream);
hipError_t launch_bw_gemm(const BwGemm& g, hipStream_t stream);
hipError_t launch_bw_attend(const BwAttendArgs& a, hipStream_t stream);

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kAttendThreads = 512;
constexpr int kMaxAttendBatch = 4096;   // batch items the bf16 attention kernel tables in LDS
constexpr int kDenseQTB = 256;  // queries per dense-attention workgroup
constexpr int kLinearTileF = 192;   // dense projection workgroup tile (features)

}  // namespace lf
