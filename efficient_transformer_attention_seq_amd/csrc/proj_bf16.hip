// Sequence projection Kbar = E_h . K_{b,h}, Vbar = F_h . V_{b,h} in bf16 with fp32 accumulation
// (Linformer 요약 설명, section "Model": each row of E combines the n positions' keys into one
// projected key; positions past a sequence's length contribute nothing).
//
// As a GEMM per group of units sharing one projection matrix A (k x n):
//   M = k projected slots, N = 64 columns per unit, reduction over the n positions.
// Workgroup (512 threads, 8 waves) = all k slots x `UPT` units x one split of the positions.
// Wave w computes a (32 WM) slot x 64 column tile of one unit.
//
// Data movement (HBM-bound, so this is what matters):
//   * Each 64-position step of the A rows and of the units' K/V rows is copied global -> LDS
//     by buffer loads that write LDS directly (no register staging), 1 KB per wave instruction,
//     every instruction covering whole 128-byte rows.  A ring of NS stages keeps NS-1 steps in
//     flight while the matrix cores work on the oldest one.
//   * K/V loads use a buffer descriptor whose size is the sequence's valid length, so positions
//     past the length read as zero in hardware: padding costs no branch and no bytes.
//   * LDS layouts: A tile [k rows][64 positions], 16-byte chunks XOR-swizzled by
//     (r ^ r>>3) & 7 so the A-operand reads of consecutive rows hit distinct banks.  K/V tile
//     [64 positions][64 columns], 32-byte blocks XOR-swizzled by (t & 3); the B operand (positions
//     contiguous per lane) is read with the transposing ds_read_b64_tr_b16 (each 16-lane group
//     gets a 4 x 16 block transposed), so no explicit transpose is done anywhere.
//   The swizzles are realised by choosing which global 16-byte chunk each lane fetches.
// Splits (S > 1) write fp32 partial sums; a fixup kernel adds them in split order (so results are
// bitwise reproducible) and casts.  With S == 1 the cast happens here.
// Output: Kbar scaled by c = scale * log2(e) and stored as a bf16 plane plus an fp8 residual plane
// with per-block power-of-two scales (format in lf_launch.h); Vbar -> bf16, round to nearest even.
// The backward pass takes both unscaled in fp32 instead (Kf, Vf).
// Unsplit Kbar / Vbar outputs are written with streaming (non-temporal) stores (RoBERTa-shaped
// forward 59.8 -> 57.9 us on two boxes, -0.3 us on a third); split partials and the stack's E.X output use ordinary stores
// (streaming measured flat for the former and 1.5% slower for the stack).
#include <cstring>

#include "lf_device.h"
#include "lf_launch.h"

namespace lf {
namespace {

constexpr int kStep = 64;               // positions per pipeline stage
constexpr int kUnitTile = 64 * kStep * 2;  // bytes of one unit's K/V stage tile
constexpr int kLdsBudget = 150 * 1024;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz_e(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ float other_half(float x, bool upper) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(upper ? r[0] : r[1]);
}

// Raw buffer descriptor: base, size in bytes (loads at or past it return zero).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from `rsrc` at byte offset `voff` into LDS at lds_base + 16 * lane.
// Issued as inline asm so the compiler does not add a conservative vmcnt(0) before every LDS
// read of the ring; completion is tracked explicitly with wait_vmcnt().
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    i32x4 rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs)
                 : "memory");
}

// dma16 with the streaming (non-temporal) cache policy, for the K/V rows: each is read by one
// pass only, so they need not displace E (re-read by every tile of its group) or the split sums
// from the caches (n = 65536 layerwise: projection 49.2-51.5 -> 45.6-46.6 us; bench shape -0.9 us).
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    i32x4 rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void vmcnt_le() {
    // s_waitcnt: vmcnt N, expcnt and lgkmcnt left at "no wait"
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
#define LF_W(i) case i: vmcnt_le<i>(); break;
        LF_W(0) LF_W(1) LF_W(2) LF_W(3) LF_W(4) LF_W(5) LF_W(6) LF_W(7) LF_W(8) LF_W(9)
        LF_W(10) LF_W(11) LF_W(12) LF_W(13) LF_W(14) LF_W(15) LF_W(16) LF_W(17) LF_W(18)
        LF_W(19) LF_W(20) LF_W(21) LF_W(22) LF_W(23) LF_W(24) LF_W(25) LF_W(26) LF_W(27)
        LF_W(28) LF_W(29) LF_W(30) LF_W(31)
#undef LF_W
        default: vmcnt_le<0>(); break;
    }
}

struct Unit {
    int which, b, h;
};

__device__ __forceinline__ Unit unit_of(const ProjGeom& g, int grp, int j) {
    Unit u;
    if (g.share == 0) {               // unshared: group = which * H + h, member = b
        u.which = grp / g.H;
        u.h = grp % g.H;
        u.b = j;
    } else if (g.share == 1) {        // headwise: group = which, member = (b, h)
        u.which = grp;
        u.b = j / g.H;
        u.h = j % g.H;
    } else if (g.share == kProjSingle) {   // one matrix, member = (b, h), values only
        u.which = 1;
        u.b = j / g.H;
        u.h = j % g.H;
    } else {                          // key-value / layerwise: member = (which, b, h)
        const int bh = g.B * g.H;
        u.which = j / bh;
        const int r = j % bh;
        u.b = r / g.H;
        u.h = r % g.H;
    }
    return u;
}

__device__ __forceinline__ const uint16_t* group_matrix(const ProjBf16Args& a, int grp) {
    const ProjGeom& g = a.g;
    if (g.share == 0) {
        const int which = grp / g.H, h = grp % g.H;
        return (which ? a.F : a.E) + (size_t)h * g.k * g.n;
    }
    if (g.share == 1) return grp ? a.F : a.E;
    return a.E;
}

// Workgroup geometry: NW = SG * UG waves; wave (sg, ug) computes 32*WM slots x WN units (64 columns
// each); the workgroup tile is KS = 32*WM*SG slots x UPT = WN*UG units.
template <int WM_, int WN_, int SG_, int UG_>
struct ProjCfg {
    static constexpr int WM = WM_, WN = WN_, SG = SG_, UG = UG_;
    static constexpr int NW = SG * UG;
    static constexpr int KS = 32 * WM * SG;
    static constexpr int UPT = WN * UG;
    static constexpr int XPW = 8 / NW;   // K/V row-block instructions per unit per wave
    // ring depth: as many 64-position stages as the LDS budget holds (2..5); the host geometry
    // uses the same rule
    static constexpr int STAGE = KS * 128 + UPT * kUnitTile;
    static constexpr int NS = kLdsBudget / STAGE > 5 ? 5 : (kLdsBudget / STAGE < 2 ? 2 : kLdsBudget / STAGE);
    // DMA instructions per wave per step, when every wave issues the same number
    static constexpr bool UNIFORM = (KS / 8) % NW == 0;
    static constexpr int MYC = (KS / 8) / NW + UPT * XPW;
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
};

template <class C>
__global__ __launch_bounds__(C::NW * 64) void proj_bf16_kernel(ProjBf16Args a) {
    constexpr int WM = C::WM, WN = C::WN, SG = C::SG, NW = C::NW, KS = C::KS, UPT = C::UPT;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const ProjGeom& g = a.g;
    const int lid = xcd_remap(blockIdx.x, g.nlogical);
    if (lid < 0) return;
    // logical order (fastest first): unit tile, slot tile, split, group -- consecutive blocks
    // share the same A chunk, then the same K/V chunk.
    const int utile = lid % g.tiles_per_group;
    int rest = lid / g.tiles_per_group;
    const int stile = rest % g.slot_tiles;
    rest /= g.slot_tiles;
    const int s = rest % g.S;
    const int grp = rest / g.S;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int sg = wave % SG, ug = wave / SG;
    const int j0 = utile * UPT;
    const int r0 = stile * KS;

    // lengths of the tile's units in one round of loads (lane u < UPT fetches unit u's), then
    // broadcast; steps past every unit's length are all zero and skipped
    int lane_len = 0;
    if (lane < UPT && j0 + lane < g.members)
        lane_len = clamp_len(a.lengths, unit_of(g, grp, j0 + lane).b, g.n);
    int ulen[UPT];
    int maxlen = 0;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        ulen[u] = __builtin_amdgcn_readlane(lane_len, u);
        maxlen = max(maxlen, ulen[u]);
    }
    const int t_begin = s * g.steps_per_split * kStep;
    const int t_end = min(min(g.n, t_begin + g.steps_per_split * kStep), maxlen);
    const int nsteps = t_end > t_begin ? (t_end - t_begin + kStep - 1) / kStep : 0;

    constexpr uint32_t stage_bytes = (uint32_t)KS * 128 + UPT * kUnitTile;
    constexpr int NS = C::NS;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;

    // ---- this wave's share of one stage's DMA instructions (1 KB each):
    //   A rows  : I = 0 .. KS/8-1 (rows 8I .. 8I+7 of the slot tile), wave I % NW issues I;
    //   K/V     : unit u, positions 8q .. 8q+7 for q = 0..7, wave w issues q = xq0 + NW*qi.
    constexpr int n_e = KS / 8;
    const int my_e = (wave < n_e) ? (n_e - wave + NW - 1) / NW : 0;
    const int my_count = my_e + UPT * C::XPW;
    const int xq0 = (wave - (n_e % NW) + NW) % NW;

    const uint16_t* A = group_matrix(a, grp);
    const i32x4 rsrc_a = make_rsrc(A, (uint32_t)g.k * g.n * 2);
    // per-unit K/V descriptors, bounded by the valid length (indexed only by unrolled loops, so
    // they stay in scalar registers)
    i32x4 rsrc_x[UPT];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const int j = j0 + u;
        if (j < g.members) {
            const Unit un = unit_of(g, grp, j);
            const uint16_t* X = (un.which ? a.V : a.K) + un.b * g.xb + un.h * g.xh;
            // rows past the length lie at or beyond the descriptor's size, so they read as zero
            rsrc_x[u] = make_rsrc(X, ulen[u] > 0 ? (uint32_t)(((size_t)(ulen[u] - 1) * g.xrow + kHeadDim) * 2) : 0u);
        } else {
            rsrc_x[u] = make_rsrc(a.K, 0u);
        }
    }
    const int lrow = lane >> 3, lpc = lane & 7;

    // One step's DMA share of this wave, in four parts so that it can be spread over the four
    // MFMA sub-steps of the step before (the TA queue then drains while the matrix cores work):
    // part 0 = the A rows, parts 1..3 = the units u with u % 3 == part - 1.  The per-step count
    // of instructions (my_count) and their order within a step are what the waits rely on.
    auto issue_part = [&](int step, int slot, int part) {
        const int t0 = t_begin + step * kStep;
        const uint32_t sb = lds0 + (uint32_t)slot * stage_bytes;
        if (part == 0) {
            for (int I = wave; I < n_e; I += NW) {
                const int r = I * 8 + lrow;                 // row within the slot tile
                const int lc = lpc ^ swz_e(r);
                dma16(rsrc_a, sb + I * 1024,
                      (uint32_t)((size_t)(r0 + r) * g.n + t0 + lc * 8) * 2);
            }
            return;
        }
#pragma unroll
        for (int qi = 0; qi < C::XPW; ++qi) {
            const int q = xq0 + NW * qi;
            const int tl = q * 8 + lrow;
            const int lc = 2 * ((lpc >> 1) ^ (tl & 3)) + (lpc & 1);
            const uint32_t xoff = (uint32_t)(((size_t)(t0 + tl) * g.xrow + lc * 8) * 2);
#pragma unroll
            for (int u = 0; u < UPT; ++u)
                if (u % 3 == part - 1)
                    dma16_nt(rsrc_x[u], sb + (uint32_t)KS * 128 + u * kUnitTile + q * 1024, xoff);
        }
    };
    auto issue = [&](int step, int slot) {
#pragma unroll
        for (int part = 0; part < 4; ++part) issue_part(step, slot, part);
    };

    // acc[wn][ct][mt]: rows = 32 columns (ct) of unit wn, columns = 32 slots (mt)
    f32x16 acc[WN][2][WM];
#pragma unroll
    for (int wn = 0; wn < WN; ++wn)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int mt = 0; mt < WM; ++mt)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[wn][ct][mt][j] = 0.0f;

    // ---- per-lane LDS offsets for the operand reads
    int a_off[WM];
    int a_sw[WM];
#pragma unroll
    for (int mt = 0; mt < WM; ++mt) {
        const int r = sg * 32 * WM + mt * 32 + l32;
        a_off[mt] = r * 128;
        a_sw[mt] = swz_e(r);
    }
    const int grp16 = lane >> 4, s16 = lane & 15;
    const int tq = 8 * (grp16 >> 1) + (s16 >> 2);          // + 16 ks + 4 rd
    const int cb = grp16 & 1;
    const int cin = (s16 & 3) * 8;                          // byte offset inside a 32-B block

    const int npro = min(NS - 1, nsteps);
    for (int i = 0; i < npro; ++i) issue(i, i);

    int cslot = 0;           // ring slot of step i
    int islot = NS - 1;      // ring slot of step i + NS - 1
    for (int i = 0; i < nsteps; ++i) {
        // stage i has landed once at most `later` younger stages are still in flight
        if constexpr (C::UNIFORM) {
            if (i + NS - 2 < nsteps) vmcnt_le<(NS - 2) * C::MYC>();
            else vmcnt_le<0>();   // the last stages: wait for everything
        } else {
            wait_vmcnt(min(NS - 2, nsteps - 1 - i) * my_count);
        }
        __syncthreads();
        const bool refill = i + NS - 1 < nsteps;   // the slot read at step i - 1 is free now
        const int fill_slot = islot;
        islot = (islot + 1 == NS) ? 0 : islot + 1;
        const int cur = cslot;
        cslot = (cslot + 1 == NS) ? 0 : cslot + 1;
        const uint8_t* st = smem + (size_t)cur * stage_bytes;
        // operands of sub-step ks (16 positions): E rows (B operand, 8 consecutive positions per
        // lane) and K/V columns (A operand, read transposed); two register sets, so the reads
        // of sub-step ks + 1 are in flight while the MFMAs of sub-step ks run
        bf16x8 ev[2][WM];
        bf16x8 xo[2][WN][2];
        auto load_ops = [&](int ks, bf16x8 (&e)[WM], bf16x8 (&x)[WN][2]) {
#pragma unroll
            for (int mt = 0; mt < WM; ++mt)
                e[mt] = *(const bf16x8*)(st + a_off[mt] + (((2 * ks + hh) ^ a_sw[mt]) << 4));
#pragma unroll
            for (int wn = 0; wn < WN; ++wn) {
                const uint8_t* xt = st + KS * 128 + (ug * WN + wn) * kUnitTile;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const int cblk = ct * 2 + cb;
                    s16x4 v[2];
#pragma unroll
                    for (int rd = 0; rd < 2; ++rd) {
                        const int t = ks * 16 + tq + 4 * rd;
                        const uint8_t* p = xt + t * 128 + ((cblk ^ (t & 3)) << 5) + cin;
                        v[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4*)(uintptr_t)(
                                (__attribute__((address_space(3))) const uint8_t*)p));
                    }
                    x[wn][ct] = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
            }
        };
        load_ops(0, ev[0], xo[0]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) load_ops(ks + 1, ev[(ks + 1) & 1], xo[(ks + 1) & 1]);
            if (refill) issue_part(i + NS - 1, fill_slot, ks);
#pragma unroll
            for (int wn = 0; wn < WN; ++wn)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int mt = 0; mt < WM; ++mt)
                        acc[wn][ct][mt] = mfma32(xo[ks & 1][wn][ct], ev[ks & 1][mt], acc[wn][ct][mt]);
        }
    }

    // ---- two splits paired in the kernel: the workgroup that gets here first leaves its sums
    // and exits, the other adds them to its own and goes on to the unsplit epilogue.  The sums
    // move with agent-coherent (sc1) stores and loads, so the pair need not share an L2; the
    // summation a + b is exact in either order, so the result does not depend on which is first.
    bool split_out = g.S > 1;
    if (a.pair_epoch != 0) {
        split_out = false;
        const int tile = (grp * g.slot_tiles + stile) * g.tiles_per_group + utile;
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
        // this wave's accumulators, 16-byte chunk c of accumulator q at ((q 4 + c) 64 + lane) 16
        // bytes from the wave's block (1 KB of contiguous bytes per instruction)
        constexpr int NACC = WN * 2 * WM;
        constexpr uint32_t kWaveBytes = NACC * 4 * 64 * 16;
        const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
            a.part + ((size_t)tile * NW + wave) * (kWaveBytes / 4), 0, kWaveBytes, 0x00020000);
        constexpr int kSC0 = 1, kSC1 = 16;   // cache-policy bits: agent-coherent access
        if (role == 0) {
#pragma unroll
            for (int wn = 0; wn < WN; ++wn)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4) {
                            const int q = (wn * 2 + ct) * WM + mt;
                            const f32x16& x = acc[wn][ct][mt];
                            const f32x4 v = {x[4 * c4], x[4 * c4 + 1], x[4 * c4 + 2], x[4 * c4 + 3]};
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp,
                                                                   ((q * 4 + c4) * 64 + lane) * 16, 0, kSC1);
                        }
            vmcnt_le<0>();     // this wave's sums have reached the coherence point
            __syncthreads();   // everyone's
            if (tid == 0)
                __hip_atomic_store(ctr, tag_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (tid == 0) {
            // the first workgroup is past its exchange and only has stores left, so this wait
            // ends; the bound only guards against a counter that held this call's tag before it
            for (int it = 0; role == 1 && it < (1 << 20) &&
                             __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag_ready;
                 ++it)
                __builtin_amdgcn_s_sleep(2);
            __hip_atomic_store(ctr, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
#pragma unroll
        for (int wn = 0; wn < WN; ++wn)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int mt = 0; mt < WM; ++mt)
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4) {
                        const int q = (wn * 2 + ct) * WM + mt;
                        const f32x4 v = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, ((q * 4 + c4) * 64 + lane) * 16, 0,
                                                                         kSC0 | kSC1));
                        f32x16& x = acc[wn][ct][mt];
                        x[4 * c4] += v[0];
                        x[4 * c4 + 1] += v[1];
                        x[4 * c4 + 2] += v[2];
                        x[4 * c4 + 3] += v[3];
                    }
    }

    // ---- epilogue: stage each wave's tile through LDS (the ring is free once every wave has
    // left the loop) so global stores are whole rows, 16 bytes per lane.
    //   lane (l32, hh) holds, for slot (32 mt + l32) of the wave, columns 32 ct + 8 q + 4 hh + (0..3)
    __syncthreads();
    constexpr int RW = 32 * WM;                      // slot rows per wave tile
    // per-wave staging region: RW rows x 64 columns, fp32 (row stride 272 B), or the bf16 plane
    // (row stride 136 B) followed by the fp8 lo plane (row stride 80 B); at most 17 KB per wave
    constexpr int kRowF = 64 * 4 + 16, kRowH = 64 * 2 + 8, kRowL = 80;
    uint8_t* stg = smem + (size_t)wave * (RW * kRowF);
    uint8_t* stg_lo = stg + RW * kRowH;
    const size_t bhk = (size_t)g.B * g.H * g.k;
    const float c = a.c;
    const bool f32_out = a.Kf != nullptr;
#pragma unroll
    for (int wn = 0; wn < WN; ++wn) {
        const int j = j0 + ug * WN + wn;
        const bool live = j < g.members;
        const Unit un = live ? unit_of(g, grp, j) : Unit{0, 0, 0};
        const int rbase = r0 + sg * RW;     // first slot row of this wave tile
        const size_t urow = (size_t)(un.b * g.H + un.h) * g.k + rbase;   // global Kbar row
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
            const int row = mt * 32 + l32;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                if (split_out || f32_out) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = ct * 32 + q * 8 + 4 * hh;
                        const f32x4 v = {acc[wn][ct][mt][4 * q], acc[wn][ct][mt][4 * q + 1],
                                         acc[wn][ct][mt][4 * q + 2], acc[wn][ct][mt][4 * q + 3]};
                        *(f32x4*)(stg + row * kRowF + col * 4) = v;
                    }
                } else if (un.which == 1) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = ct * 32 + q * 8 + 4 * hh;
                        const f32x16& x = acc[wn][ct][mt];
                        const u32x2 v = {pack_bf16x2(x[4 * q], x[4 * q + 1]),
                                         pack_bf16x2(x[4 * q + 2], x[4 * q + 3])};
                        *(u32x2*)(stg + row * kRowH + col * 2) = v;
                    }
                } else {
                    // Kbar: x = c * Kbar, hi = bf16(x), lo = x - hi; block ct of this row is
                    // split between this lane and lane l ^ 32
                    float lo[16];
                    float m = 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = ct * 32 + q * 8 + 4 * hh;
                        const f32x16& x = acc[wn][ct][mt];
                        const u32x2 hv = {hi_pair(c * x[4 * q], c * x[4 * q + 1], lo[4 * q], lo[4 * q + 1]),
                                          hi_pair(c * x[4 * q + 2], c * x[4 * q + 3], lo[4 * q + 2], lo[4 * q + 3])};
                        *(u32x2*)(stg + row * kRowH + col * 2) = hv;
#pragma unroll
                        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(lo[4 * q + i]));
                    }
                    m = fmaxf(m, other_half(m, hh));
                    const int sh = lo_shift(m);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = ct * 32 + q * 8 + 4 * hh;
                        *(uint32_t*)(stg_lo + row * kRowL + lo_pos(col)) =
                            lo_bytes(lo[4 * q], lo[4 * q + 1], lo[4 * q + 2], lo[4 * q + 3], sh);
                    }
                    if (live && hh == 0) a.Ksc[(urow + row) * 2 + ct] = (uint8_t)(127 - sh);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's staging writes are done
        __builtin_amdgcn_wave_barrier();
        if (live) {
            const size_t ubase = urow * kHeadDim;
            if (split_out || f32_out) {
                float* dst = split_out ? a.part + ((size_t)s * 2 + un.which) * bhk * kHeadDim + ubase
                                       : (un.which == 0 ? a.Kf : a.Vf) + ubase;
                // RW rows x 256 B: 16 lanes per row
#pragma unroll
                for (int it = 0; it < RW / 4; ++it) {
                    const int row = it * 4 + (lane >> 4), ch = lane & 15;
                    *(f32x4*)(dst + row * kHeadDim + ch * 4) = *(const f32x4*)(stg + row * kRowF + ch * 16);
                }
            } else {
                // streaming stores for a layer's Kbar / Vbar; the encoder stack's E.X output is read
                // by the next GEMM straight away and stays cached
                const bool stream_out = g.share != kProjSingle;
                uint16_t* dst_hi = (un.which == 0 ? a.Khi : a.Vb) + ubase;
#pragma unroll
                for (int it = 0; it < RW / 8; ++it) {
                    const int row = it * 8 + (lane >> 3), ch = lane & 7;
                    const u32x4 v = *(const u32x4*)(stg + row * kRowH + ch * 16);
                    u32x4* d = (u32x4*)(dst_hi + row * kHeadDim + ch * 8);
                    if (stream_out) __builtin_nontemporal_store(v, d);
                    else *d = v;
                }
                if (un.which == 0) {
                    uint8_t* dst_lo = a.Klo + ubase;   // 64 bytes per row
#pragma unroll
                    for (int it = 0; it < RW / 16; ++it) {
                        const int row = it * 16 + (lane >> 2), ch = lane & 3;
                        __builtin_nontemporal_store(*(const u32x4*)(stg_lo + row * kRowL + ch * 16), (u32x4*)(dst_lo + row * 64 + ch * 16));
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
    }
}

// Adds the S fp32 partial sums of every Kbar/Vbar element and stores them in the bf16 formats
// (Kbar: hi plane, fp8 lo plane and block scales, see lf_launch.h) or, given Kf, in fp32.  NG = 1: a thread adds all S
// splits of 4 consecutive columns in split order (loads issued 4 ahead).  NG = 4 (many splits): a
// block covers 64 such chunks and its 4 waves each add a contiguous quarter of the splits in
// order, then wave 0 adds the quarter sums in order.  Either way the summation order is fixed,
// so results are bitwise reproducible; the 8 lanes of a 32-column block are consecutive lanes
// of the finishing wave.
template <int NG>
__global__ __launch_bounds__(256) void proj_fixup_bf16_kernel(const float* part, int S,
                                                              size_t half, size_t e0, float c,
                                                              uint16_t* Khi, uint8_t* Klo,
                                                              uint8_t* Ksc, uint16_t* Vb,
                                                              float* Kf, float* Vf) {
    constexpr int CH = 256 / NG;   // four-column chunks per block
    __shared__ f32x4 quarter[NG > 1 ? NG : 1][CH];
    const int ci = threadIdx.x % CH, grp = threadIdx.x / CH;
    const size_t e4 = e0 + ((size_t)blockIdx.x * CH + ci) * 4;   // e0: first element (0 or half)
    const bool live = e4 < 2 * half;   // 2 * half is a multiple of 64: whole blocks leave together
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
        const int s0 = S * grp / NG, s1 = S * (grp + 1) / NG;
        int s = s0;
        for (; s + 4 <= s1; s += 4) {
            const f32x4 p0 = *(const f32x4*)(part + (size_t)s * 2 * half + e4);
            const f32x4 p1 = *(const f32x4*)(part + (size_t)(s + 1) * 2 * half + e4);
            const f32x4 p2 = *(const f32x4*)(part + (size_t)(s + 2) * 2 * half + e4);
            const f32x4 p3 = *(const f32x4*)(part + (size_t)(s + 3) * 2 * half + e4);
            acc += p0;
            acc += p1;
            acc += p2;
            acc += p3;
        }
        for (; s < s1; ++s) acc += *(const f32x4*)(part + (size_t)s * 2 * half + e4);
    }
    if constexpr (NG > 1) {
        quarter[grp][ci] = acc;
        __syncthreads();
        if (grp != 0) return;
        acc = quarter[0][ci];
#pragma unroll
        for (int q = 1; q < NG; ++q) acc += quarter[q][ci];
    }
    if (!live) return;
    if (Kf) {   // fp32 outputs
        *(f32x4*)(e4 < half ? Kf + e4 : Vf + (e4 - half)) = acc;
    } else if (e4 < half) {
        float r0, r1, r2, r3;
        const u32x2 hi = {hi_pair(c * acc[0], c * acc[1], r0, r1), hi_pair(c * acc[2], c * acc[3], r2, r3)};
        float m = fmaxf(fmaxf(fabsf(r0), fabsf(r1)), fmaxf(fabsf(r2), fabsf(r3)));
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        m = fmaxf(m, __shfl_xor(m, 4));
        const int sh = lo_shift(m);
        const size_t row = e4 / 64;
        const int d0 = (int)(e4 % 64);
        *(u32x2*)(Khi + e4) = hi;
        *(uint32_t*)(Klo + row * 64 + lo_pos(d0)) = lo_bytes(r0, r1, r2, r3, sh);
        if ((d0 & 31) == 0) Ksc[row * 2 + (d0 >> 5)] = (uint8_t)(127 - sh);
    } else {
        const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *(u32x2*)(Vb + (e4 - half)) = v;
    }
}

// Tile configurations (compile-time geometry).  The names are what LINFORMER_PROJ_CFG selects.
using Cfg256x128 = ProjCfg<2, 1, 4, 2>;   // 8 waves, 64x64 wave tiles
using Cfg256x256 = ProjCfg<2, 2, 4, 2>;   // 8 waves, 64x128 wave tiles
using Cfg128x256w4 = ProjCfg<2, 2, 2, 2>; // 4 waves, 64x128 wave tiles
using Cfg128x256 = ProjCfg<2, 1, 2, 4>;   // 8 waves, 64x64 wave tiles
using Cfg64x512 = ProjCfg<2, 1, 1, 8>;    // 8 waves, 64x64 wave tiles
using Cfg32x512 = ProjCfg<1, 1, 1, 8>;    // 8 waves, 32x64 wave tiles (any k % 32 == 0)
using Cfg128x128w4 = ProjCfg<2, 1, 2, 2>; // 4 waves, 64x64 wave tiles

struct CfgInfo {
    const char* name;
    int id, ks, upt, nw;
};
constexpr CfgInfo kCfgs[] = {
    {"256x128", 0, Cfg256x128::KS, Cfg256x128::UPT, Cfg256x128::NW},
    {"256x256", 1, Cfg256x256::KS, Cfg256x256::UPT, Cfg256x256::NW},
    {"128x256w4", 2, Cfg128x256w4::KS, Cfg128x256w4::UPT, Cfg128x256w4::NW},
    {"128x256", 3, Cfg128x256::KS, Cfg128x256::UPT, Cfg128x256::NW},
    {"64x512", 4, Cfg64x512::KS, Cfg64x512::UPT, Cfg64x512::NW},
    {"32x512", 5, Cfg32x512::KS, Cfg32x512::UPT, Cfg32x512::NW},
    {"128x128w4", 6, Cfg128x128w4::KS, Cfg128x128w4::UPT, Cfg128x128w4::NW},
};

}  // namespace

bool proj_geometry(int B, int H, int n, int k, int share, int split_override,
                   const char* cfg_override, ProjGeom* out) {
    if (B < 1 || H < 1 || n < kStep || n % kStep || k < 32 || k > 256 || k % 32) return false;
    ProjGeom g{};
    g.B = B;
    g.H = H;
    g.n = n;
    g.k = k;
    g.share = share;
    g.xb = (long long)H * n * kHeadDim;   // [B, H, n, 64] unless the caller sets other strides
    g.xh = (long long)n * kHeadDim;
    g.xrow = kHeadDim;
    if (share == 0) {
        g.groups = 2 * H;
        g.members = B;
    } else if (share == 1) {
        g.groups = 2;
        g.members = B * H;
    } else if (share == kProjSingle) {
        g.groups = 1;
        g.members = B * H;
    } else {
        g.groups = 1;
        g.members = 2 * B * H;
    }
    int cfg = -1;
    if (cfg_override && cfg_override[0]) {
        for (const CfgInfo& c : kCfgs)
            if (std::strcmp(c.name, cfg_override) == 0 && k % c.ks == 0) cfg = c.id;
    }
    const int steps = n / kStep;
    if (cfg < 0) {
        if (k % 128 == 0) cfg = 3;
        else if (k % 64 == 0) cfg = 4;
        else cfg = 5;
        // A short reduction (no split) over more 128-slot tiles than there are compute units
        // leaves a partial second round of workgroups; 256-slot tiles halve the count (one
        // round at n = 512, B32 H12 key-value: 36.3 -> 31.5 us) and read fewer LDS bytes per
        // product.
        if (k % 256 == 0 && steps <= 16) {
            const long long t128 = (long long)g.groups * (k / kCfgs[3].ks) *
                                   ((g.members + kCfgs[3].upt - 1) / kCfgs[3].upt);
            if (t128 > 256) cfg = 1;
        }
    }
    auto plan = [&](int c) {
        const CfgInfo& ci = kCfgs[c];
        g.cfg = c;
        g.upt = ci.upt;
        g.slot_tiles = k / ci.ks;
        g.tiles_per_group = (g.members + ci.upt - 1) / ci.upt;
        const int stage = ci.ks * 128 + ci.upt * kUnitTile;
        int ns = kLdsBudget / stage;
        if (ns > 5) ns = 5;
        if (ns < 2) ns = 2;
        g.stages = ns;
        g.threads = ci.nw * 64;
        const int tiles = g.groups * g.slot_tiles * g.tiles_per_group;
        int S;
        if (split_override > 0) {
            S = split_override;
        } else {
            // workgroups resident per compute unit (LDS-limited), 256 compute units: split the
            // positions so that all tiles x splits fit in one wave of workgroups, keeping at
            // least 4 steps (256 positions) per split.
            const int per_cu = (160 * 1024) / (ns * stage);
            const int slots = 256 * (per_cu > 0 ? per_cu : 1);
            S = slots / tiles;
            if (S > steps / 4) S = steps / 4;
            // a short reduction (<= 1024 positions) over tiles that already fill a quarter of
            // the slots gains less from splitting than the fixup pass costs
            if (steps <= 16 && 4 * tiles >= slots) S = 1;
            // at most 512 positions: the fixup launch costs more than a split saves
            // (B1 H12 n512 layerwise: 25.9 -> 23.7 us at k = 128, 28.6 -> 26.0 us at k = 256)
            if (steps <= 8) S = 1;
            if (S < 1) S = 1;
        }
        if (S > steps) S = steps;
        g.steps_per_split = (steps + S - 1) / S;
        g.S = (steps + g.steps_per_split - 1) / g.steps_per_split;
        return tiles;
    };
    const int tiles = plan(cfg);
    // An unsplit reduction over 128 x 256 tiles that occupy at most half of the compute units
    // (the stack's E . X: 96 tiles) runs on twice as many 128 x 128 tiles instead.
    if (!(cfg_override && cfg_override[0]) && cfg == 3 && g.S == 1 && 2 * tiles <= 256) plan(6);
    g.nlogical = g.groups * g.S * g.slot_tiles * g.tiles_per_group;
    *out = g;
    return true;
}

namespace {
template <class C>
hipError_t launch_cfg(const ProjBf16Args& a, hipStream_t stream) {
    const ProjGeom& g = a.g;
    const int grid = ((g.nlogical + 7) / 8) * 8;
    if (g.stages != C::NS) return hipErrorInvalidValue;   // host and kernel ring depths agree
    const size_t ring = (size_t)C::NS * C::STAGE;
    const size_t staging = (size_t)C::NW * (32 * C::WM) * (64 * 4 + 16);   // epilogue staging
    const size_t lds = ring > staging ? ring : staging;
    auto kern = proj_bf16_kernel<C>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NW * 64), lds, stream, a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_proj_bf16(const ProjBf16Args& a, hipStream_t stream) {
    const ProjGeom& g = a.g;
    hipError_t e;
    switch (g.cfg) {
        case 0: e = launch_cfg<Cfg256x128>(a, stream); break;
        case 1: e = launch_cfg<Cfg256x256>(a, stream); break;
        case 2: e = launch_cfg<Cfg128x256w4>(a, stream); break;
        case 3: e = launch_cfg<Cfg128x256>(a, stream); break;
        case 4: e = launch_cfg<Cfg64x512>(a, stream); break;
        case 6: e = launch_cfg<Cfg128x128w4>(a, stream); break;
        default: e = launch_cfg<Cfg32x512>(a, stream); break;
    }
    if (e != hipSuccess || g.S == 1 || a.pair_epoch != 0) return e;
    const size_t half = (size_t)g.B * g.H * g.k * kHeadDim;
    // the single-matrix mode has only the values half
    const size_t e0 = g.share == kProjSingle ? half : 0;
    const size_t chunks = (2 * half - e0) / 4;
    if (g.S >= 8) {   // many splits: spread each chunk's reduction over 4 waves
        hipLaunchKernelGGL(proj_fixup_bf16_kernel<4>, dim3((int)((chunks + 63) / 64)), dim3(256), 0,
                           stream, a.part, g.S, half, e0, a.c, a.Khi, a.Klo, a.Ksc, a.Vb, a.Kf, a.Vf);
    } else {
        hipLaunchKernelGGL(proj_fixup_bf16_kernel<1>, dim3((int)((chunks + 255) / 256)), dim3(256), 0,
                           stream, a.part, g.S, half, e0, a.c, a.Khi, a.Klo, a.Ksc, a.Vb, a.Kf, a.Vf);
    }
    return hipGetLastError();
}

}  // namespace lf
