// Linformer attention for short sequences in one launch (n <= 1024, bf16, one projection matrix
// for the keys and the values: key-value or layerwise sharing, or per-head E_h with F_h = E_h).
// One workgroup per (b, h): it projects that head's keys and values along the sequence,
// Kbar = E . K and Vbar = E . V over the valid positions (Linformer 요약 설명, section "Model"),
// straight into LDS in the attention's operand layouts (attend_core.h), then attends every query
// tile of the head there.  Kbar and Vbar never reach HBM, and nothing waits on a second launch:
// at n = 512 the separate projection and attention pass of them would add a quarter to the
// layer's HBM bytes (the regime of the n = 512 row of "Inference-time Efficiency Results").
//
// Projection (k slots x 128 columns: 64 of Kbar, 64 of Vbar, reduced over the positions): wave w
// computes the 32 WM slots from 32 WM (w % 4) of Kbar (w < 4) or Vbar (w >= 4) with
// v_mfma_f32_32x32x16_bf16, the K/V rows as the A operand (read transposed with
// ds_read_b64_tr_b16) and E as the B operand.  Each 64-position step of E's k rows and of the
// head's K and V rows is copied global -> LDS by direct-to-LDS buffer loads (1 KB per wave
// instruction, whole 128-byte rows) in a ring of 3 (k = 256) or 4 (k = 128) stages; K/V
// descriptors are sized to the valid
// length, so positions past it read as zero.  The epilogue writes x = c Kbar (c = scale log2 e)
// as the bf16 plane, its e4m3 residual with one power-of-two scale per row half, and Vbar in
// bf16, into the head's planes, which reuse the ring's LDS.
// Attention: the waves take the head's 32-query tiles in turn (tile_math / tile_store of
// attend_core.h), the first tile's Q loaded before the projection starts and each next tile's Q
// during the current one; the rows past the last valid tile are zero-filled with streaming
// stores issued at the start, so they drain under the projection.
// Work split: when the units do not fill whole rounds of workgroups, each unit of the last,
// partial round is taken by several workgroups that all project it and attend contiguous shares
// of its tiles, so that round fills the compute units (every output tile is still computed once,
// by the same arithmetic).  Hand-off (HANDOFF, between one and one and a half units per compute
// unit): one round of workgroups; workgroup 2 j first projects the extra unit grid + j and
// copies its planes, un-swizzled, to the workspace in the attention kernel's format with
// agent-coherent stores, then sets the unit's flag to the call's tag; workgroup 2 j + 1, after
// its own unit, waits for that flag (set by a workgroup of lower index, which is already
// running), loads the planes with agent-coherent loads, clears the flag (a replayed graph reuses
// the captured call's tag) and attends all of the unit's tiles.  The planes are the same bytes
// either way, so the output is bitwise that of the plain split.
#include "attend_core.h"

namespace lf {
namespace {

using namespace attn;
constexpr int kThreads = 512;   // 8 waves
constexpr int kStep = 64;       // positions per projection stage

__device__ __forceinline__ int swz_e(int r) { return (r ^ (r >> 3)) & 7; }

template <int KB>
struct FusedLayout {
    using Ly = AttnLayout<KB>;
    static constexpr int K = Ly::K;
    static constexpr int E_STAGE = K * 128;       // E: k rows x 64 positions, bf16
    static constexpr int X_TILE = kStep * 128;    // K or V: 64 positions x 64 columns, bf16
    static constexpr int STAGE = E_STAGE + 2 * X_TILE;
    static constexpr int NS = 144 * 1024 / STAGE > 4 ? 4 : 144 * 1024 / STAGE;   // ring depth
    static constexpr int RING = NS * STAGE;
    static constexpr int OFF_STG = Ly::BYTES;     // per-wave tile staging after the planes
    static constexpr int ATT = OFF_STG + 8 * 32 * 128;
    static constexpr int BYTES = RING > ATT ? RING : ATT;
    // direct-to-LDS instructions per stage (E rows, then K rows, then V rows), per wave
    static constexpr int NI = K / 8 + 16;
    static constexpr int PER_WAVE = NI / 8;
    static_assert(NI % 8 == 0, "whole instructions per wave");
};

template <int N>
__device__ __forceinline__ void vmcnt_le() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// dma16 with the descriptor read from lane 0 (so that it sits in scalar registers even where
// the compiler cannot prove it wave-uniform).
__device__ __forceinline__ void dma16u(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    i32x4 rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
    dma16(rs, lds_base, voff);
}

// dma16u with the streaming (non-temporal) cache policy, for the head's K/V rows, which only this
// workgroup reads, once (RoBERTa shape -0.3 to -0.9 us, stack-layer shape -0.3 us)
__device__ __forceinline__ void dma16u_nt(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    i32x4 rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs)
                 : "memory");
}

// dma16 with agent-coherent loads (sc0 sc1): data another workgroup stored with agent-coherent
// stores, possibly on another XCD, is read from the coherence point, not from a stale L2 line.
__device__ __forceinline__ void dma16_coherent(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
    i32x4 rs;
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen sc0 sc1 lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs)
                 : "memory");
}

template <int KB, bool STACK, bool HANDOFF>
__global__ __launch_bounds__(kThreads) void fused_bf16_kernel(FusedBf16Args a) {
    using FL = FusedLayout<KB>;
    using Ly = AttnLayout<KB>;
    constexpr int K = Ly::K;
    constexpr int WM = KB / 4;   // 32-slot blocks per wave: the k slots over 4 waves
    __shared__ __attribute__((aligned(16))) uint8_t smem[FL::BYTES];
    constexpr int kSC1 = 16;   // cache-policy bit: agent-coherent stores

    // One unit (b, h): its planes come from its own projection (publish: also copied to global
    // memory and flagged for another workgroup) or, `fill`, from the copy another workgroup
    // published; then the query tiles [ntiles lo / den, ntiles hi / den) of the unit.
    auto run_unit = [&](int bh, bool fill, bool publish, int lo, int hi,
                        int den) __attribute__((always_inline)) {
        // with several units per workgroup, the per-lane constants are derived inside each unit
        // (through an opaque copy of the thread index), so that the compiler does not share them
        // between the units and keep them live across the projection's register-heavy loop
        uint32_t tid_o = threadIdx.x;
        if constexpr (HANDOFF) asm volatile("" : "+v"(tid_o));
        const int tid = (int)tid_o;
        const uint32_t lds0 = HANDOFF ? opaque(lds_addr(smem)) : lds_addr(smem);
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
        const int b = bh / a.H, h = bh % a.H;
        const int L = clamp_len(a.lengths, b, a.n);
        const int ntiles = (L + kTileQ - 1) / kTileQ;
        const int t0 = ntiles * lo / den, t1 = ntiles * hi / den;
        const size_t rowbase = (size_t)bh * a.n;
        __syncthreads();   // the previous unit's readers are done with the LDS

        // ---- the first tile's Q, in flight during the projection
        u32x4 qraw[4];
        auto load_q = [&](int tile) {
            const u32x4* src = (const u32x4*)(a.Q + (rowbase + (size_t)tile * kTileQ) * kHeadDim) + lane;
#pragma unroll
            for (int i = 0; i < 4; ++i) qraw[i] = src[64 * i];
        };
        if (t0 + wave < t1) load_q(t0 + wave);

        // ---- zero the rows past the last valid tile (streaming stores, drained under the work)
        if (lo == 0 && hi > 0) {   // the workgroup that attends the unit's first tiles
            const u32x4 zero = {0u, 0u, 0u, 0u};
            u32x4* blk = (u32x4*)(a.O + (rowbase + (size_t)ntiles * kTileQ) * kHeadDim);
            const int nz = (a.n - ntiles * kTileQ) * 8;   // 16-byte chunks
            for (int c = tid; c < nz; c += kThreads) __builtin_nontemporal_store(zero, &blk[c]);
        }

        if (!fill) {
        // ---- projection.  Sequence form: the slot rows are E's (positions contiguous), the columns
        // the head's K, V rows (read transposed), 64 positions per stage, over the valid length.
        // Stack form: the slot rows are the head's batch item's projected input Xbar_b (features
        // contiguous; stage j is its head-planar block j, features 64 j .. 64 j + 63), the columns
        // the rows 64 h .. 64 h + 63 of W_K and of W_V (features contiguous), over all d_model features.
        const int lrow = lane >> 3, lpc = lane & 7;
        i32x4 rsrc_e, rsrc_k, rsrc_v;
        int nsteps;
        if constexpr (STACK) {
            rsrc_e = make_rsrc(a.E + (size_t)b * a.H * K * kHeadDim, (uint32_t)a.H * K * kHeadDim * 2);
            rsrc_k = make_rsrc(a.K, (uint32_t)((size_t)2 * a.dm * a.dm * 2));   // W_K then W_V
            rsrc_v = rsrc_k;
            nsteps = a.dm / kStep;
        } else {
            const uint16_t* Eh = a.E + (size_t)(a.e_heads > 1 ? h : 0) * K * a.n;
            rsrc_e = make_rsrc(Eh, (uint32_t)K * a.n * 2);
            const uint32_t xbytes = L > 0 ? (uint32_t)(((size_t)(L - 1) * kHeadDim + kHeadDim) * 2) : 0u;
            rsrc_k = make_rsrc(a.K + rowbase * kHeadDim, xbytes);
            rsrc_v = make_rsrc(a.V + rowbase * kHeadDim, xbytes);
            nsteps = (L + kStep - 1) / kStep;
        }
        auto issue = [&](int step, int slot) {
            const int t0 = step * kStep;
            const uint32_t sbase = lds0 + (uint32_t)slot * FL::STAGE;
#pragma unroll
            for (int p = 0; p < FL::PER_WAVE; ++p) {
                const int j = wave + 8 * p;   // instruction index, the same split in every stage
                if (j < K / 8) {              // slot rows 8 j .. 8 j + 7, chunks swizzled by swz_e(row)
                    const int r = j * 8 + lrow;
                    const int lc = lpc ^ swz_e(r);
                    const size_t e = STACK ? ((size_t)step * K + r) * kHeadDim + lc * 8
                                           : (size_t)r * a.n + t0 + lc * 8;
                    dma16u(rsrc_e, sbase + j * 1024, (uint32_t)(e * 2));
                } else if constexpr (STACK) {   // W rows: 64 of W_K then 64 of W_V, as slot rows are
                    const int wr = (j - K / 8) * 8 + lrow;
                    const int lc = lpc ^ swz_e(wr);
                    const size_t grow = (size_t)(wr >> 6) * a.dm + 64 * h + (wr & 63);
                    dma16u(rsrc_k, sbase + FL::E_STAGE + (j - K / 8) * 1024,
                          (uint32_t)((grow * a.dm + t0 + lc * 8) * 2));
                } else {                      // K (then V) positions 8 q .. 8 q + 7, 32-byte blocks
                    const int jj = j - K / 8;  // swizzled by the position's low bits
                    const int q = jj & 7;
                    const int tl = q * 8 + lrow;
                    const int lc = 2 * ((lpc >> 1) ^ (tl & 3)) + (lpc & 1);
                    const uint32_t off = (uint32_t)(((t0 + tl) * kHeadDim + lc * 8) * 2);
                    const uint32_t dst = sbase + FL::E_STAGE + (jj >> 3) * FL::X_TILE + q * 1024;
                    dma16u_nt((jj >> 3) ? rsrc_v : rsrc_k, dst, off);
                }
            }
        };
        const int which = wave >> 2, sb = wave & 3;
        f32x16 acc[2][WM];   // [ct][mt]: rows = 32 columns ct, columns = 32 slots mt
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int mt = 0; mt < WM; ++mt)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[ct][mt][j] = 0.0f;
        int e_off[WM], e_sw[WM];
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
            const int r = 32 * (sb * WM + mt) + l32;
            e_off[mt] = r * 128;
            e_sw[mt] = swz_e(r);
        }
        const int grp16 = lane >> 4, s16 = lane & 15;
        const int tq = 8 * (grp16 >> 1) + (s16 >> 2);
        const int cb = grp16 & 1;
        const int cin = (s16 & 3) * 8;
        constexpr int NS = FL::NS;
        for (int i = 0; i < NS - 1 && i < nsteps; ++i) issue(i, i);
        for (int i = 0; i < nsteps; ++i) {
            // this wave's share of stage i has landed once at most the younger stages are in flight
            if (i + NS - 2 < nsteps) vmcnt_le<(NS - 2) * FL::PER_WAVE>();
            else vmcnt_le<0>();
            __syncthreads();   // everyone's has, and step i - 1's reads of its slot are done
            if (i + NS - 1 < nsteps) issue(i + NS - 1, (i + NS - 1) % NS);
            const uint8_t* st = smem + (size_t)(i % NS) * FL::STAGE;
            const uint8_t* xt = st + FL::E_STAGE + which * FL::X_TILE;
            bf16x8 ev[2][WM], xo[2][2];
            auto load_ops = [&](int ks, bf16x8 (&e)[WM], bf16x8 (&x)[2]) {
#pragma unroll
                for (int mt = 0; mt < WM; ++mt)
                    e[mt] = *(const bf16x8*)(st + e_off[mt] + (((2 * ks + hh) ^ e_sw[mt]) << 4));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    if constexpr (STACK) {   // W rows 64 which + 32 ct + l32, features contiguous
                        const int wr = 64 * which + 32 * ct + l32;
                        x[ct] = *(const bf16x8*)(st + FL::E_STAGE + wr * 128 + (((2 * ks + hh) ^ swz_e(wr)) << 4));
                        continue;
                    }
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
                    x[ct] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
            };
            load_ops(0, ev[0], xo[0]);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks + 1 < 4) load_ops(ks + 1, ev[(ks + 1) & 1], xo[(ks + 1) & 1]);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int mt = 0; mt < WM; ++mt)
                        acc[ct][mt] = mfma32(xo[ks & 1][ct], ev[ks & 1][mt], acc[ct][mt]);
            }
        }
        __syncthreads();   // every wave is done with the ring: the head's planes take its place

        // ---- epilogue: lane (l32, hh) holds, for slot r = 32 (sb WM + mt) + l32, the columns
        // d = 32 ct + 8 q + 4 hh + (0..3)
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
            const int r = 32 * (sb * WM + mt) + l32;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const f32x16& x = acc[ct][mt];
                if (which == 1) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const u32x2 v = {pack_bf16x2(x[4 * q], x[4 * q + 1]), pack_bf16x2(x[4 * q + 2], x[4 * q + 3])};
                        *(u32x2*)(smem + Ly::OFF_V + r * 128 + (((2 * ct + (q >> 1)) ^ (r & 3)) << 5) +
                                  16 * (q & 1) + 8 * hh) = v;
                    }
                } else {
                    float lo[16];
                    float m = 0.0f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const u32x2 hv = {hi_pair(a.c * x[4 * q], a.c * x[4 * q + 1], lo[4 * q], lo[4 * q + 1]),
                                          hi_pair(a.c * x[4 * q + 2], a.c * x[4 * q + 3], lo[4 * q + 2], lo[4 * q + 3])};
                        *(u32x2*)(smem + r * 128 + (((4 * ct + q) ^ swz16(r)) << 4) + 8 * hh) = hv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(lo[4 * q + e]));
                    }
                    m = fmaxf(m, other_half(m, hh));   // the row half's 32 residuals
                    const int sh = lo_shift(m);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int pos = 32 * (q & 1) + 16 * ct + 8 * (q >> 1) + 4 * hh;   // lo_pos
                        *(uint32_t*)(smem + Ly::OFF_L + r * 64 + (((pos >> 4) ^ ((r >> 1) & 3)) << 4) +
                                     (pos & 15)) =
                            lo_bytes(lo[4 * q], lo[4 * q + 1], lo[4 * q + 2], lo[4 * q + 3], sh);
                    }
                    if (hh == 0) smem[Ly::OFF_S + r * 2 + ct] = (uint8_t)(127 - sh);
                }
            }
        }
        __syncthreads();

        if (publish) {
            // the planes, un-swizzled, to the unit's global copy (the attention kernel's format)
            // with agent-coherent stores; then the flag, once every wave's stores have completed
            const size_t off = (size_t)bh * K * kHeadDim;
            auto rsrc = [](void* p, int bytes) {
                return __builtin_amdgcn_make_buffer_rsrc(p, 0, bytes, 0x00020000);
            };
            const __amdgpu_buffer_rsrc_t gh = rsrc(a.Khi + off, Ly::PLANE);
            const __amdgpu_buffer_rsrc_t gv = rsrc(a.Vb + off, Ly::PLANE);
            const __amdgpu_buffer_rsrc_t gl = rsrc(a.Klo + off, Ly::LOB);
            const __amdgpu_buffer_rsrc_t gs = rsrc(a.Ksc + (size_t)bh * K * 2, K * 2);
            for (int c = tid; c < K * 8; c += kThreads) {   // 16-byte chunk c % 8 of row c / 8
                const int r = c >> 3, lc = c & 7;
                const u32x4 vh = *(const u32x4*)(smem + r * 128 + ((lc ^ swz16(r)) << 4));
                const u32x4 vv = *(const u32x4*)(smem + Ly::OFF_V + r * 128 +
                                                  ((2 * ((lc >> 1) ^ (r & 3)) + (lc & 1)) << 4));
                __builtin_amdgcn_raw_buffer_store_b128(vh, gh, c * 16, 0, kSC1);
                __builtin_amdgcn_raw_buffer_store_b128(vv, gv, c * 16, 0, kSC1);
            }
            for (int c = tid; c < K * 4; c += kThreads) {   // 16-byte chunk c % 4 of residual row c / 4
                const int r = c >> 2, ch = c & 3;
                const u32x4 vl = *(const u32x4*)(smem + Ly::OFF_L + r * 64 + ((ch ^ ((r >> 1) & 3)) << 4));
                __builtin_amdgcn_raw_buffer_store_b128(vl, gl, c * 16, 0, kSC1);
            }
            if (tid < K * 2 / 16)
                __builtin_amdgcn_raw_buffer_store_b128(*(const u32x4*)(smem + Ly::OFF_S + tid * 16), gs,
                                                       tid * 16, 0, kSC1);
            vmcnt_le<0>();     // this wave's stores have reached the coherence point
            __syncthreads();   // everyone's
            if (tid == 0)
                __hip_atomic_store(a.flags + bh, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        } else {
            // the unit's planes from the copy its projecting workgroup (of lower index, so already
            // running) publishes; the bound only guards against a flag that never arrives
            if (tid == 0) {
                for (int it = 0; it < (1 << 22) &&
                                 __hip_atomic_load(a.flags + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.epoch;
                     ++it)
                    __builtin_amdgcn_s_sleep(2);
            }
            __syncthreads();
            const size_t off = (size_t)bh * K * kHeadDim;
            const i32x4 rh = make_rsrc(a.Khi + off, Ly::PLANE);
            const i32x4 rv = make_rsrc(a.Vb + off, Ly::PLANE);
            const i32x4 rl = make_rsrc(a.Klo + off, Ly::LOB);
            const i32x4 rs = make_rsrc(a.Ksc + (size_t)bh * K * 2, K * 2);
            const int lrow = lane >> 3, lpc = lane & 7;
            for (int I = wave; I < K / 8; I += 8) {   // 8 rows of 128 bytes per instruction
                const int r = I * 8 + lrow;
                const int lck = lpc ^ swz16(r);
                const int lcv = 2 * ((lpc >> 1) ^ (r & 3)) + (lpc & 1);
                dma16_coherent(rh, lds0 + I * 1024, (uint32_t)(r * 128 + lck * 16));
                dma16_coherent(rv, lds0 + Ly::OFF_V + I * 1024, (uint32_t)(r * 128 + lcv * 16));
            }
            for (int I = wave; I < K / 16; I += 8) {  // 16 rows of 64 bytes per instruction
                const int r = I * 16 + (lane >> 2), ch = lane & 3;
                dma16_coherent(rl, lds0 + Ly::OFF_L + I * 1024, (uint32_t)(r * 64 + ((ch ^ ((r >> 1) & 3)) << 4)));
            }
            if (wave == 0) dma16_coherent(rs, lds0 + Ly::OFF_S, (uint32_t)(lane * 16));   // past K*2: zeros
            vmcnt_le<0>();
            __syncthreads();
            // consumed: clear the flag, so that a replay of this call (a captured graph reuses its
            // tag) waits for its own publication again
            if (tid == 0) __hip_atomic_store(a.flags + bh, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- attention over this workgroup's query tiles t0 .. t1 - 1, tile t0 + j to wave j % 8
        if (t0 + wave < t1) {
        const Lanes ln = attn_lanes<KB>(lds0, lane);
        int scl[2];
        attn_scales<KB>(smem, lane, scl);
        uint32_t coff[4];
        stage_offsets(lane, coff);
        const uint32_t stg = lds0 + FL::OFF_STG + wave * (kTileQ * 128);
        f32x16 bias;
#pragma unroll
        for (int j = 0; j < 16; ++j) bias[j] = 0.0f;
        bool bias_dirty = false;
        bf16x8 qop[4];
        for (int tile = t0 + wave; tile < t1; tile += 8) {
            stage_q(stg, coff, qraw, lane, qop);
            f32x16 o0, o1;
            float z;
            tile_math<KB>(ln, qop, scl, hh, bias, bias_dirty, o0, o1, z, [&]() {
                if (tile + 8 < t1) load_q(tile + 8);
            });
            tile_store(stg, coff, lane, o0, o1, z, a.O + (rowbase + (size_t)tile * kTileQ) * kHeadDim,
                       tile * kTileQ, L);
        }
        }
    };

    const int w = blockIdx.x;
    if constexpr (!HANDOFF) {
        int bh = w, lo = 0, den = 1;
        if (w >= a.whole) {
            const int r = w - a.whole;
            bh = a.whole + r / a.parts;
            lo = r % a.parts;
            den = a.parts;
        }
        run_unit(bh, false, false, lo, lo + 1, den);
    } else {
        // `grid` workgroups for grid + extra units: workgroup 2 j projects and publishes the extra
        // unit grid + j before its own unit; workgroup 2 j + 1 attends it after its own
        const int units = a.B * a.H;
        const bool paired = w < 2 * (units - a.grid);
        const int extra = a.grid + (w >> 1);
        if (paired && (w & 1) == 0) run_unit(extra, false, true, 0, 0, 1);
        run_unit(w, false, false, 0, 1, 1);
        if (paired && (w & 1) == 1) run_unit(extra, true, false, 0, 1, 1);
    }
}

}  // namespace

bool fused_supported(int n, int k) { return n <= 1024 && (k == 128 || k == 256); }

hipError_t launch_fused_bf16(const FusedBf16Args& a, hipStream_t stream) {
    const int units = a.B * a.H;
    int nwg;
    if (a.mode == 2) {
        if (a.grid >= units || 2 * (units - a.grid) > a.grid || !a.flags || !a.epoch || a.dm > 0)
            return hipErrorInvalidValue;
        nwg = a.grid;
    } else {
        if (a.mode != 0 || a.whole < 0 || a.whole > units || a.parts < 1) return hipErrorInvalidValue;
        nwg = a.whole + (units - a.whole) * a.parts;
    }
    const dim3 grid(nwg), block(kThreads);
    if (a.dm > 0 && (a.dm % kStep || a.dm != 64 * a.H)) return hipErrorInvalidValue;
    const bool stack = a.dm > 0;
    const bool ho = a.mode == 2;
    switch (a.k) {
        case 128:
            if (stack) hipLaunchKernelGGL((fused_bf16_kernel<4, true, false>), grid, block, 0, stream, a);
            else if (ho) hipLaunchKernelGGL((fused_bf16_kernel<4, false, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((fused_bf16_kernel<4, false, false>), grid, block, 0, stream, a);
            break;
        case 256:
            if (stack) hipLaunchKernelGGL((fused_bf16_kernel<8, true, false>), grid, block, 0, stream, a);
            else if (ho) hipLaunchKernelGGL((fused_bf16_kernel<8, false, true>), grid, block, 0, stream, a);
            else hipLaunchKernelGGL((fused_bf16_kernel<8, false, false>), grid, block, 0, stream, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lf
