// liblinformer C ABI: argument validation, workspace layout and kernel dispatch.
// The operations are declared (with their citations) in include/linformer.h.
#include "linformer.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "lf_launch.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

size_t elem_size(int dtype) { return dtype == LF_BF16 ? 2 : 4; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int env_int(const char* name) {
    const char* v = std::getenv(name);
    return v ? std::atoi(v) : 0;
}

// Tuning overrides (for measurement sweeps only; one code path): LINFORMER_PROJ_SPLIT forces
// the number of position splits, LINFORMER_PROJ_CFG names the projection tile configuration,
// LINFORMER_ATTEND_GRID the number of attention workgroups.
bool geometry(const lf_problem* p, lf::ProjGeom* g) {
    return lf::proj_geometry(p->batch, p->heads, p->n, p->k, p->share,
                             env_int("LINFORMER_PROJ_SPLIT"), std::getenv("LINFORMER_PROJ_CFG"), g);
}

int check_problem(const lf_problem* p) {
    if (!p) return LF_ERR_NULL;
    if (p->dtype != LF_F32 && p->dtype != LF_BF16) return LF_ERR_DTYPE;
    if (p->share < LF_SHARE_NONE || p->share > LF_SHARE_LAYERWISE) return LF_ERR_SHARE;
    if (p->batch < 1 || p->batch > lf::kMaxAttendBatch || p->heads < 1 || p->d != 64)
        return LF_ERR_SHAPE;
    if (p->n < 64 || p->n % 64) return LF_ERR_SHAPE;
    if (p->k < 32 || p->k > 256 || p->k % 32) return LF_ERR_SHAPE;
    if (!(p->scale >= 0.0f) || !std::isfinite(p->scale)) return LF_ERR_SHAPE;
    const long long qkv = (long long)p->batch * p->heads * p->n * p->d;
    const long long ef = (long long)p->heads * p->k * p->n;
    if (qkv >= (1LL << 31) || ef >= (1LL << 31)) return LF_ERR_SHAPE;
    return LF_OK;
}

float eff_scale(const lf_problem* p) {
    return p->scale > 0.0f ? p->scale : 1.0f / std::sqrt((float)p->d);
}

size_t qkv_bytes(const lf_problem* p) {
    return (size_t)p->batch * p->heads * p->n * p->d * elem_size(p->dtype);
}
size_t ef_bytes(const lf_problem* p) {
    const size_t he = p->share == LF_SHARE_NONE ? (size_t)p->heads : 1;
    return he * p->k * p->n * elem_size(p->dtype);
}
size_t kbar_bytes(const lf_problem* p) {
    // bf16: hi plane (2 B per element), fp8 lo plane (1 B), two scale bytes per row
    const size_t e = (size_t)p->batch * p->heads * p->k * p->d;
    const size_t rows = (size_t)p->batch * p->heads * p->k;
    return p->dtype == LF_BF16 ? 3 * e + 2 * rows : e * 4;
}
size_t vbar_bytes(const lf_problem* p) {
    return (size_t)p->batch * p->heads * p->k * p->d * elem_size(p->dtype);
}
// A two-way split is paired inside the projection kernel: per workgroup tile one block of
// fp32 sums (the tile's KS x UPT x 64 outputs) and one 8-byte counter.
size_t pair_tiles(const lf::ProjGeom& g) {
    return (size_t)g.groups * g.slot_tiles * g.tiles_per_group;
}
size_t pair_sums_bytes(const lf::ProjGeom& g) {
    return round_up(pair_tiles(g) * (size_t)(g.k / g.slot_tiles) * g.upt * 64 * 4, 256);
}
// fp32 projection (one BwGemm launch for Kbar and Vbar, z = (which, b, h)): the reduction over
// the positions is split into chunks of at least 32 until about 512 workgroups run, summed in
// chunk order by the GEMM's second kernel.
void f32_proj_plan(const lf_problem* p, int* splits, int* kchunk) {
    const long long tiles = 2LL * p->batch * p->heads * ((p->k + 127) / 128);
    long long s = 512 / std::max(1LL, tiles);
    s = std::max(1LL, std::min<long long>(s, std::min(p->n / 32, 64)));
    const int chunk = (int)((p->n + s - 1) / s + 31) / 32 * 32;
    *kchunk = chunk;
    *splits = (p->n + chunk - 1) / chunk;
}

size_t part_bytes(const lf_problem* p, const lf::ProjGeom& g) {
    if (p->dtype == LF_F32) {
        int s, c;
        f32_proj_plan(p, &s, &c);
        return s > 1 ? (size_t)s * 2 * p->batch * p->heads * p->k * 64 * 4 : 0;   // Kbar and Vbar
    }
    if (g.S <= 1) return 0;
    if (g.S == 2) return pair_sums_bytes(g) + pair_tiles(g) * 8;
    return (size_t)g.S * 2 * p->batch * p->heads * p->k * p->d * 4;
}

// Per-call tag of the paired split: unique within the process (and, salted by the start time,
// unlikely to repeat across processes), in [1, 2^62).
unsigned long long next_pair_epoch() {
    static std::atomic<unsigned long long> next{[] {
        unsigned long long x = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
        x ^= x >> 33;
        x *= 0xff51afd7ed558ccdull;
        x ^= x >> 33;
        return x;
    }()};
    for (;;) {
        const unsigned long long e = next.fetch_add(1) & ((1ull << 62) - 1);
        if (e != 0) return e;
    }
}

struct Range {
    const void* p;
    size_t n;
};
bool overlap(Range a, Range b) {
    if (!a.p || !b.p || !a.n || !b.n) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}
bool any_overlap(const Range* outs, int nout, const Range* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i], ins[j])) return true;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return true;
    }
    return false;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Resolves F per the sharing rule; returns LF_OK or LF_ERR_SHARE / LF_ERR_NULL.
int resolve_f(const lf_problem* p, const void* E, const void* F, const void** Fout) {
    if (p->share == LF_SHARE_HEADWISE) {
        if (!F) return LF_ERR_NULL;
        *Fout = F;
        return LF_OK;
    }
    if (p->share == LF_SHARE_KV || p->share == LF_SHARE_LAYERWISE) {
        if (F && F != E) return LF_ERR_SHARE;
        *Fout = E;
        return LF_OK;
    }
    *Fout = F ? F : E;
    return LF_OK;
}

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LF_ERR_NO_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return LF_ERR_ARCH;
    int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return LF_ERR_NO_DEVICE;
        }
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? LF_OK : LF_ERR_ARCH;
}

int launch_status(hipError_t e) { return e == hipSuccess ? LF_OK : LF_ERR_LAUNCH; }

std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (cached; 256 on MI355X).
int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        hipDeviceProp_t prop;
        c = (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
                ? prop.multiProcessorCount
                : 256;
        g_cu_count[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

// Validation shared by project_kv and forward (everything about K, V, E, F, lengths, ws).
int check_project_args(const lf_problem* p, const void* K, const void* V, const void* E,
                       const void* F, const int32_t* lengths, const lf::ProjGeom& g, void* ws,
                       size_t ws_bytes, size_t ws_needed, const void** Fres) {
    if (!K || !V || !E) return LF_ERR_NULL;
    int st = resolve_f(p, E, F, Fres);
    if (st) return st;
    if (!aligned16(K) || !aligned16(V) || !aligned16(E) || !aligned16(*Fres)) return LF_ERR_ALIGN;
    if (lengths && ((uintptr_t)lengths & 3u)) return LF_ERR_ALIGN;
    if (ws_needed > 0) {
        if (!ws || ws_bytes < ws_needed) return LF_ERR_WORKSPACE;
        if (!aligned16(ws)) return LF_ERR_ALIGN;
    }
    (void)g;
    return LF_OK;
}

// Kbar, Vbar in the attention kernels' formats, or (f32_out, the backward pass) unscaled fp32
int do_project(const lf_problem* p, const void* K, const void* V, const void* E, const void* F,
               const int32_t* lengths, void* Kbar, void* Vbar, void* part,
               const lf::ProjGeom& g, hipStream_t stream, bool f32_out = false) {
    if (p->dtype == LF_F32) {
        // Kbar = E_h K, Vbar = F_h V on the split-bf16 batched GEMM (backward_f32.hip), one
        // reduction per output tile: z = (b, h), M = k, N = 64, reduction over the positions
        // before the length
        const int B = p->batch, H = p->heads, n = p->n, k = p->k;
        const long long kn = (long long)k * n, hn64 = (long long)n * 64, hk64 = (long long)k * 64;
        // one launch for both: batch entries (b, h) then (b, h) again with F, V, Vbar
        lf::BwGemm g{};
        g.A = E; g.B = K; g.C = (float*)Kbar;
        g.A2 = F; g.B2 = V; g.C2 = (float*)Vbar;
        g.zhalf = B * H;
        g.alpha = 1.0f;
        g.M = k; g.N = 64; g.K = n; g.Z = 2 * B * H; g.zdiv = H; g.kblk = n;
        g.k_len = lengths;
        g.a_z2 = p->share == LF_SHARE_NONE ? kn : 0; g.a_i = n; g.a_kc = 1;
        g.b_z1 = H * hn64; g.b_z2 = hn64; g.b_kc = 64; g.b_j = 1;
        g.c_z1 = H * hk64; g.c_z2 = hk64; g.c_i = 64; g.c_j = 1;
        f32_proj_plan(p, &g.splits, &g.kchunk);
        g.part = (float*)part;
        return launch_status(lf::launch_bw_gemm(g, stream));
    }
    lf::ProjBf16Args a{};
    a.K = (const uint16_t*)K;
    a.V = (const uint16_t*)V;
    a.E = (const uint16_t*)E;
    a.F = (const uint16_t*)F;
    a.lengths = lengths;
    const size_t e = (size_t)p->batch * p->heads * p->k * p->d;
    a.Khi = (uint16_t*)Kbar;
    a.Klo = (uint8_t*)Kbar + 2 * e;
    a.Ksc = (uint8_t*)Kbar + 3 * e;
    a.Vb = (uint16_t*)Vbar;
    if (f32_out) {
        a.Khi = nullptr; a.Klo = nullptr; a.Ksc = nullptr; a.Vb = nullptr;
        a.Kf = (float*)Kbar;
        a.Vf = (float*)Vbar;
    }
    a.part = (float*)part;
    a.c = eff_scale(p) * lf::kLog2e;
    a.g = g;
    if (g.S == 2) {
        a.pair_ctr = (unsigned long long*)((uint8_t*)part + pair_sums_bytes(g));
        a.pair_epoch = next_pair_epoch();
    }
    return launch_status(lf::launch_proj_bf16(a, stream));
}

int do_attend(const lf_problem* p, const void* Q, const void* Kbar, const void* Vbar,
              const int32_t* lengths, void* O, hipStream_t stream) {
    if (p->dtype == LF_F32) {
        lf::F32Args a{};
        a.Q = (const float*)Q;
        a.Kbar = (const float*)Kbar;
        a.Vbar = (const float*)Vbar;
        a.O = (float*)O;
        a.lengths = lengths;
        a.B = p->batch;
        a.H = p->heads;
        a.n = p->n;
        a.k = p->k;
        a.scale = eff_scale(p);
        return launch_status(lf::launch_attend_f32(a, stream));
    }
    lf::AttendBf16Args a{};
    const size_t e = (size_t)p->batch * p->heads * p->k * p->d;
    a.Q = (const uint16_t*)Q;
    a.Khi = (const uint16_t*)Kbar;
    a.Klo = (const uint8_t*)Kbar + 2 * e;
    a.Ksc = (const uint8_t*)Kbar + 3 * e;
    a.Vb = (const uint16_t*)Vbar;
    a.lengths = lengths;
    a.O = (uint16_t*)O;
    a.B = p->batch;
    a.H = p->heads;
    a.n = p->n;
    a.k = p->k;
    // persistent grid: one workgroup per compute unit (LINFORMER_ATTEND_GRID overrides, for tests),
    // never more than the number of 32-query tiles, a multiple of 8 (one share per XCD)
    int grid = env_int("LINFORMER_ATTEND_GRID");
    if (grid <= 0) grid = cu_count();
    const long long max_tiles = (long long)p->batch * p->heads * (p->n / 32);
    if ((long long)grid > max_tiles) grid = (int)max_tiles;
    grid = (grid + 7) / 8 * 8;
    a.nlogical = grid;
    return launch_status(lf::launch_attend_bf16(a, stream));
}

// ---- convolution / pooling compression
int check_conv(const lf_problem* p, const void* K, const void* V, const void* wE, const void* wF,
               const int32_t* lengths, const void** wFres) {
    int st = check_problem(p);
    if (st) return st;
    if (p->dtype != LF_BF16) return LF_ERR_DTYPE;
    if (p->n % p->k) return LF_ERR_SHAPE;
    if (!K || !V || !wE) return LF_ERR_NULL;
    st = resolve_f(p, wE, wF, wFres);
    if (st) return st;
    if (!aligned16(K) || !aligned16(V)) return LF_ERR_ALIGN;
    if (((uintptr_t)wE & 1u) || ((uintptr_t)*wFres & 1u)) return LF_ERR_ALIGN;
    if (lengths && ((uintptr_t)lengths & 3u)) return LF_ERR_ALIGN;
    return LF_OK;
}

size_t conv_w_bytes(const lf_problem* p) {
    const size_t he = p->share == LF_SHARE_NONE ? (size_t)p->heads : 1;
    return he * (size_t)(p->n / p->k) * 2;
}

int do_conv(const lf_problem* p, const void* K, const void* V, const void* wE, const void* wF,
            const int32_t* lengths, void* Kbar, void* Vbar, hipStream_t stream) {
    lf::ConvBf16Args a{};
    a.K = (const uint16_t*)K;
    a.V = (const uint16_t*)V;
    a.wE = (const uint16_t*)wE;
    a.wF = (const uint16_t*)wF;
    a.lengths = lengths;
    const size_t e = (size_t)p->batch * p->heads * p->k * p->d;
    a.Khi = (uint16_t*)Kbar;
    a.Klo = (uint8_t*)Kbar + 2 * e;
    a.Ksc = (uint8_t*)Kbar + 3 * e;
    a.Vb = (uint16_t*)Vbar;
    a.B = p->batch;
    a.H = p->heads;
    a.n = p->n;
    a.k = p->k;
    a.s = p->n / p->k;
    a.e_heads = p->share == LF_SHARE_NONE ? p->heads : 1;
    a.c = eff_scale(p) * lf::kLog2e;
    return launch_status(lf::launch_conv_bf16(a, stream));
}

// ---- backward pass
struct BwWs {
    size_t kb, vb, stats, dkb, dvb, part, total;   // byte offsets
};

void bw_ws(const lf_problem* p, BwWs* w) {
    const size_t kv = (size_t)p->batch * p->heads * p->k * 64 * 4;
    const size_t st = (size_t)p->batch * p->heads * p->n * 4 * 4;   // 4 floats per query
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o += round_up(bytes, 256); return at; };
    w->kb = take(kv);
    w->vb = take(kv);
    w->stats = take(st);
    w->dkb = take(kv);
    w->dvb = take(kv);
    // split-reduction partial sums, the largest any of the backward's kernels asks for
    const int B = p->batch, H = p->heads, n = p->n, k = p->k;
    const bool unshared = p->share == LF_SHARE_NONE;
    size_t part = lf::bw_gemm_part_bytes(k, n, unshared ? B * 64 : B * H * 64,
                                         2 * (unshared ? H : 1));                   // dE (+ dF)
    part = std::max(part, lf::bw_gemm_part_bytes(n, 64, k, 2 * B * H));            // dK and dV
    lf::ProjGeom g;
    if (geometry(p, &g)) part = std::max(part, part_bytes(p, g));                  // Kbar, Vbar
    part = std::max(part, lf::kv_part_bytes(B, H, k));                              // dKbar, dVbar
    w->part = take(part);
    w->total = o;
}

bool bw_separate(const lf_problem* p, const void* E, const void* F) {
    return (p->share == LF_SHARE_NONE || p->share == LF_SHARE_HEADWISE) && F && F != E;
}

lf::BwGemm gemm0() {
    lf::BwGemm g{};
    g.Z = 1;
    g.zdiv = 1;
    g.alpha = 1.0f;
    return g;
}

// ---- encoder attention stack
int check_stack(const lf_stack* s) {
    if (!s) return LF_ERR_NULL;
    if (s->dtype != LF_BF16) return LF_ERR_DTYPE;
    if (s->layers < 1 || s->heads < 1 || s->d_model != 64 * s->heads) return LF_ERR_SHAPE;
    if (s->d_model % lf::kLinearTileF) return LF_ERR_SHAPE;
    if (s->batch < 1 || s->n < 64) return LF_ERR_SHAPE;
    if (3LL * s->batch * s->n * s->d_model >= (1LL << 30)) return LF_ERR_SHAPE;
    if (s->keep_layers != 0 && s->keep_layers != 1) return LF_ERR_SHAPE;
    return LF_OK;
}

lf_problem layer_problem(const lf_stack* s) {
    lf_problem p{};
    p.batch = s->batch;
    p.heads = s->heads;
    p.n = s->n;
    p.d = 64;
    p.k = s->k;
    p.dtype = LF_BF16;
    p.share = LF_SHARE_LAYERWISE;
    p.scale = s->scale;
    return p;
}

// Projection of a layer input X [B, n, d_model] (row-major) by the one E: unit (b, h) = columns
// 64 h .. 64 h + 63 of X_b, output Xbar = E . X_b as bf16 [B, H, k, 64].
bool stack_geometry(const lf_stack* s, lf::ProjGeom* g) {
    if (!lf::proj_geometry(s->batch, s->heads, s->n, s->k, lf::kProjSingle,
                           env_int("LINFORMER_PROJ_SPLIT"), std::getenv("LINFORMER_PROJ_CFG"), g))
        return false;
    g->xb = (long long)s->n * s->d_model;
    g->xh = 64;
    g->xrow = s->d_model;
    return true;
}

struct StackWs {
    size_t act;                                        // bytes of one [B, n, d_model] activation
    size_t q, o, xbar, kbar, vbar, part, ping, total;  // byte offsets
};

// Workspace: queries, attention output, Xbar, Kbar, Vbar, the projection's split partials, and
// two activation buffers (only when intermediate layer outputs are not kept in Y).
void stack_ws(const lf_stack* s, const lf_problem& p, const lf::ProjGeom& g, StackWs* w) {
    w->act = (size_t)s->batch * s->n * s->d_model * 2;
    const size_t xbar = (size_t)s->batch * s->k * s->d_model * 2;
    const size_t part = g.S > 1 ? (size_t)g.S * 2 * s->batch * s->heads * s->k * 64 * 4 : 0;
    w->q = 0;
    w->o = w->q + round_up(w->act, 256);
    w->xbar = w->o + round_up(w->act, 256);
    w->kbar = w->xbar + round_up(xbar, 256);
    w->vbar = w->kbar + round_up(kbar_bytes(&p), 256);
    w->part = w->vbar + round_up(vbar_bytes(&p), 256);
    w->ping = w->part + round_up(part, 256);
    const size_t nping = (s->keep_layers || s->layers == 1) ? 0 : (s->layers == 2 ? 1 : 2);
    w->total = w->ping + nping * round_up(w->act, 256);
}

int do_linear(const lf::LinearBf16Args& base, hipStream_t stream) {
    lf::LinearBf16Args a = base;
    const int ftiles = a.F / lf::kLinearTileF;
    // 256-token tiles unless that leaves compute units idle (MI355X: 256 CUs); the 128-token
    // tile runs four waves and two workgroups fit on a CU
    a.tile_t = ftiles * ((a.T + 255) / 256) < 256 ? 128 : 256;
    a.nlogical = ftiles * ((a.T + a.tile_t - 1) / a.tile_t);
    return launch_status(lf::launch_linear_bf16(a, stream));
}

// Workspace of one forward call: Kbar | Vbar | split partial sums, each 256-byte aligned.
// Flags of the fused kernel's hand-off (one 8-byte tag per (b, h)), after the partials; only
// shapes the fused kernel takes have them.
size_t flag_bytes(const lf_problem* p) {
    return p->dtype == LF_BF16 && lf::fused_supported(p->n, p->k)
               ? round_up((size_t)8 * p->batch * p->heads, 256) : 0;
}

size_t forward_ws_bytes(const lf_problem* p, const lf::ProjGeom& g) {
    return round_up(kbar_bytes(p), 256) + round_up(vbar_bytes(p), 256) +
           round_up(part_bytes(p, g), 256) + flag_bytes(p);
}

// The whole layer in one launch (fused_bf16.hip): bf16, short sequences, and one matrix
// projecting both the keys and the values (LINFORMER_FUSED=0 turns it off, for measurements).
bool use_fused(const lf_problem* p, const void* E, const void* F) {
    if (p->dtype != LF_BF16 || F != E || !lf::fused_supported(p->n, p->k)) return false;
    const char* v = std::getenv("LINFORMER_FUSED");
    return !(v && v[0] == '0');
}

// The stack layer's projected keys and values and its attention in one launch (fused_bf16.hip,
// stack form): k of 128 or 256, and enough (b, h) pairs to occupy a quarter of the compute units
// (LINFORMER_FUSED=0 turns it off, =force turns it on regardless of the pair count).
bool stack_fused(const lf_stack* s) {
    const char* v = std::getenv("LINFORMER_FUSED");
    if (v && v[0] == '0') return false;
    if (s->k != 128 && s->k != 256) return false;
    if (v && std::strcmp(v, "force") == 0) return true;
    return (long long)s->batch * s->heads >= 64;
}

// Validation of a forward call, everything but the device; `own_ws`: the workspace is the
// library's fixed scratch (not the caller's), so only its size is checked, by the caller.
struct FwdPlan {
    lf::ProjGeom g;
    size_t kb, vb, pb, need;
    const void* Fr;
};

int forward_validate(const lf_problem* p, const void* Q, const void* K, const void* V,
                     const void* E, const void* F, const int32_t* lengths, void* O, void* ws,
                     size_t ws_bytes, bool own_ws, FwdPlan* pl) {
    int st = check_problem(p);
    if (st) return st;
    if (!geometry(p, &pl->g)) return LF_ERR_SHAPE;
    pl->kb = round_up(kbar_bytes(p), 256);
    pl->vb = round_up(vbar_bytes(p), 256);
    pl->pb = part_bytes(p, pl->g);
    pl->need = forward_ws_bytes(p, pl->g);
    pl->Fr = nullptr;
    st = check_project_args(p, K, V, E, F, lengths, pl->g, ws, ws_bytes, own_ws ? 0 : pl->need,
                            &pl->Fr);
    if (st) return st;
    if (!Q || !O) return LF_ERR_NULL;
    if (!aligned16(Q) || !aligned16(O)) return LF_ERR_ALIGN;
    const Range ins[] = {{Q, qkv_bytes(p)}, {K, qkv_bytes(p)}, {V, qkv_bytes(p)},
                         {E, ef_bytes(p)},  {pl->Fr, ef_bytes(p)},
                         {lengths, lengths ? 4u * p->batch : 0u}};
    const Range outs[] = {{O, qkv_bytes(p)}, {own_ws ? nullptr : ws, pl->need}};
    if (any_overlap(outs, 2, ins, 6)) return LF_ERR_ALIAS;
    return LF_OK;
}

// Work split of the fused kernel (one workgroup per compute unit at a time; G compute units, U
// = B H units).  With G < U <= 3G/2 and a flag region (the forward's workspace), mode 2: G
// workgroups, each of the U - G extra units projected by one workgroup and attended by its
// neighbour after their own units.  Otherwise the (b, h) units of the last, partial round of
// workgroups are each taken by `parts` workgroups (all project the unit, each attends a
// contiguous share of its query tiles), as many as fill the compute units that round would leave
// idle, with at least eight query tiles (one per wave) per share at full length.
// LINFORMER_FUSED_SPLIT=0: no split at all; LINFORMER_FUSED_HANDOFF=0: no mode 2.
void fused_split(lf::FusedBf16Args& f, uint8_t* Kbar = nullptr, uint16_t* Vbar = nullptr,
                 unsigned long long* flags = nullptr) {
    const int units = f.B * f.H, G = cu_count();
    f.whole = units;
    f.parts = 1;
    f.mode = 0;
    f.grid = G;
    const char* e = std::getenv("LINFORMER_FUSED_SPLIT");
    if ((e && e[0] == '0') || G <= 0) return;
    const char* ho = std::getenv("LINFORMER_FUSED_HANDOFF");
    if (flags && f.dm == 0 && !(ho && ho[0] == '0') && units > G && 2 * (units - G) <= G) {
        const size_t el = (size_t)units * f.k * 64;
        f.mode = 2;
        f.Khi = (uint16_t*)Kbar;
        f.Klo = Kbar + 2 * el;
        f.Ksc = Kbar + 3 * el;
        f.Vb = Vbar;
        f.flags = flags;
        f.epoch = next_pair_epoch();
        return;
    }
    const int rest = units % G;
    if (rest == 0) return;
    const int parts = std::min(G / rest, std::max(1, f.n / 32 / 8));
    if (parts < 2) return;
    f.whole = units - rest;
    f.parts = parts;
}

// The projection into the workspace (Kbar | Vbar | partials), then the attention.
int forward_run(const lf_problem* p, const FwdPlan& pl, const void* Q, const void* K,
                const void* V, const void* E, const int32_t* lengths, void* O, void* ws,
                void* stream) {
    uint8_t* w = (uint8_t*)ws;
    void* Kbar = w;
    void* Vbar = w + pl.kb;
    void* part = pl.pb ? (void*)(w + pl.kb + pl.vb) : nullptr;
    hipStream_t s = (hipStream_t)stream;
    if (use_fused(p, E, pl.Fr)) {
        lf::FusedBf16Args f{};
        f.Q = (const uint16_t*)Q;
        f.K = (const uint16_t*)K;
        f.V = (const uint16_t*)V;
        f.E = (const uint16_t*)E;
        f.lengths = lengths;
        f.O = (uint16_t*)O;
        f.B = p->batch;
        f.H = p->heads;
        f.n = p->n;
        f.k = p->k;
        f.e_heads = p->share == LF_SHARE_NONE ? p->heads : 1;
        f.c = eff_scale(p) * lf::kLog2e;
        fused_split(f, (uint8_t*)Kbar, (uint16_t*)Vbar,
                    (unsigned long long*)(w + pl.kb + pl.vb + round_up(pl.pb, 256)));
        return launch_status(lf::launch_fused_bf16(f, s));
    }
    int st = do_project(p, K, V, E, pl.Fr, lengths, Kbar, Vbar, part, pl.g, s);
    if (st) return st;
    return do_attend(p, Q, Kbar, Vbar, lengths, O, s);
}

// ---- fixed scratch of the no-allocation forward.  Every GPU the library runs on holds its own
// copy of this array from the first use on that device until the process ends.  On the host,
// `scratch` names a host-side stand-in, not device memory: host code only ever uses the device
// address hipGetSymbolAddress returns for the current device, kept per device below.
constexpr size_t kScratchBytes = (size_t)LINFORMER_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_ptr(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LF_ERR_NO_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return LF_ERR_ARCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return LF_ERR_SCRATCH;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LF_OK;
}

}  // namespace

extern "C" {

const char* linformer_status_string(int status) {
    switch (status) {
        case LF_OK: return "LF_OK";
        case LF_ERR_NULL: return "LF_ERR_NULL: a required pointer is NULL";
        case LF_ERR_SHAPE: return "LF_ERR_SHAPE: a dimension or the scale is out of range";
        case LF_ERR_DTYPE: return "LF_ERR_DTYPE: unknown dtype";
        case LF_ERR_SHARE: return "LF_ERR_SHARE: bad sharing mode or F must alias E";
        case LF_ERR_WORKSPACE: return "LF_ERR_WORKSPACE: workspace missing or too small";
        case LF_ERR_ALIGN: return "LF_ERR_ALIGN: a pointer is not 16-byte aligned";
        case LF_ERR_ALIAS: return "LF_ERR_ALIAS: an output overlaps another buffer";
        case LF_ERR_NO_DEVICE: return "LF_ERR_NO_DEVICE: no HIP device available";
        case LF_ERR_ARCH: return "LF_ERR_ARCH: the current device is not gfx950";
        case LF_ERR_LAUNCH: return "LF_ERR_LAUNCH: kernel launch failed";
        case LF_ERR_SCRATCH:
            return "LF_ERR_SCRATCH: the problem needs more than the no-allocation scratch buffer "
                   "holds, or the buffer could not be located on this device";
        default: return "unknown liblinformer status";
    }
}

int linformer_kv_sizes(const lf_problem* p, size_t* kb, size_t* vb) {
    int st = check_problem(p);
    if (st) return st;
    if (!kb || !vb) return LF_ERR_NULL;
    *kb = kbar_bytes(p);
    *vb = vbar_bytes(p);
    return LF_OK;
}

int linformer_workspace_size(const lf_problem* p, size_t* bytes) {
    int st = check_problem(p);
    if (st) return st;
    if (!bytes) return LF_ERR_NULL;
    lf::ProjGeom g;
    if (!geometry(p, &g)) return LF_ERR_SHAPE;
    *bytes = forward_ws_bytes(p, g);
    return LF_OK;
}

int linformer_project_kv(const lf_problem* p, const void* K, const void* V, const void* E,
                         const void* F, const int32_t* lengths, void* Kbar, void* Vbar,
                         void* ws, size_t ws_bytes, void* stream) {
    int st = check_problem(p);
    if (st) return st;
    lf::ProjGeom g;
    if (!geometry(p, &g)) return LF_ERR_SHAPE;
    const size_t need = part_bytes(p, g);
    const void* Fr = nullptr;
    st = check_project_args(p, K, V, E, F, lengths, g, ws, ws_bytes, need, &Fr);
    if (st) return st;
    if (!Kbar || !Vbar) return LF_ERR_NULL;
    if (!aligned16(Kbar) || !aligned16(Vbar)) return LF_ERR_ALIGN;
    const Range ins[] = {{K, qkv_bytes(p)}, {V, qkv_bytes(p)}, {E, ef_bytes(p)},
                         {Fr, ef_bytes(p)}, {lengths, lengths ? 4u * p->batch : 0u}};
    const Range outs[] = {{Kbar, kbar_bytes(p)}, {Vbar, vbar_bytes(p)}, {ws, need}};
    if (any_overlap(outs, 3, ins, 5)) return LF_ERR_ALIAS;
    st = check_device();
    if (st) return st;
    return do_project(p, K, V, E, Fr, lengths, Kbar, Vbar, ws, g, (hipStream_t)stream);
}

int linformer_attend(const lf_problem* p, const void* Q, const void* Kbar, const void* Vbar,
                     const int32_t* lengths, void* O, void* stream) {
    int st = check_problem(p);
    if (st) return st;
    if (!Q || !Kbar || !Vbar || !O) return LF_ERR_NULL;
    if (!aligned16(Q) || !aligned16(Kbar) || !aligned16(Vbar) || !aligned16(O)) return LF_ERR_ALIGN;
    if (lengths && ((uintptr_t)lengths & 3u)) return LF_ERR_ALIGN;
    const Range ins[] = {{Q, qkv_bytes(p)}, {Kbar, kbar_bytes(p)}, {Vbar, vbar_bytes(p)},
                         {lengths, lengths ? 4u * p->batch : 0u}};
    const Range outs[] = {{O, qkv_bytes(p)}};
    if (any_overlap(outs, 1, ins, 4)) return LF_ERR_ALIAS;
    st = check_device();
    if (st) return st;
    return do_attend(p, Q, Kbar, Vbar, lengths, O, (hipStream_t)stream);
}

int linformer_forward(const lf_problem* p, const void* Q, const void* K, const void* V,
                      const void* E, const void* F, const int32_t* lengths, void* O, void* ws,
                      size_t ws_bytes, void* stream) {
    FwdPlan pl;
    int st = forward_validate(p, Q, K, V, E, F, lengths, O, ws, ws_bytes, false, &pl);
    if (st) return st;
    st = check_device();
    if (st) return st;
    return forward_run(p, pl, Q, K, V, E, lengths, O, ws, stream);
}

int linformer_forward_noalloc(const lf_problem* p, const void* Q, const void* K, const void* V,
                              const void* E, const void* F, const int32_t* lengths, void* O,
                              void* stream) {
    FwdPlan pl;
    int st = forward_validate(p, Q, K, V, E, F, lengths, O, nullptr, 0, true, &pl);
    if (st) return st;
    if (pl.need > kScratchBytes) return LF_ERR_SCRATCH;
    st = check_device();
    if (st) return st;
    void* ws = nullptr;
    st = scratch_ptr(&ws);   // first call on this device: locate its copy of the array
    if (st) return st;
    return forward_run(p, pl, Q, K, V, E, lengths, O, ws, stream);
}

int attention_dense_forward(const lf_problem* p, const void* Q, const void* K, const void* V,
                            const int32_t* lengths, void* O, void* stream) {
    if (!p) return LF_ERR_NULL;
    if (p->dtype != LF_BF16) return LF_ERR_DTYPE;
    if (p->batch < 1 || p->heads < 1 || p->d != 64 || p->n < 64 || p->n % 64)
        return LF_ERR_SHAPE;
    if (!(p->scale >= 0.0f) || !std::isfinite(p->scale)) return LF_ERR_SHAPE;
    if ((long long)p->batch * p->heads * p->n * p->d >= (1LL << 31)) return LF_ERR_SHAPE;
    if (!Q || !K || !V || !O) return LF_ERR_NULL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return LF_ERR_ALIGN;
    if (lengths && ((uintptr_t)lengths & 3u)) return LF_ERR_ALIGN;
    const Range ins[] = {{Q, qkv_bytes(p)}, {K, qkv_bytes(p)}, {V, qkv_bytes(p)},
                         {lengths, lengths ? 4u * p->batch : 0u}};
    const Range outs[] = {{O, qkv_bytes(p)}};
    if (any_overlap(outs, 1, ins, 4)) return LF_ERR_ALIAS;
    int st = check_device();
    if (st) return st;
    lf::DenseBf16Args a{};
    a.Q = (const uint16_t*)Q;
    a.K = (const uint16_t*)K;
    a.V = (const uint16_t*)V;
    a.lengths = lengths;
    a.O = (uint16_t*)O;
    a.B = p->batch;
    a.H = p->heads;
    a.n = p->n;
    a.QB = (p->n + lf::kDenseQTB - 1) / lf::kDenseQTB;
    a.nlogical = p->batch * p->heads * a.QB;
    a.c = eff_scale(p) * lf::kLog2e;
    return launch_status(lf::launch_dense_bf16(a, (hipStream_t)stream));
}

int linformer_stack_workspace_size(const lf_stack* s, size_t* bytes) {
    int st = check_stack(s);
    if (st) return st;
    if (!bytes) return LF_ERR_NULL;
    const lf_problem p = layer_problem(s);
    st = check_problem(&p);
    if (st) return st;
    lf::ProjGeom g;
    if (!stack_geometry(s, &g)) return LF_ERR_SHAPE;
    StackWs w;
    stack_ws(s, p, g, &w);
    *bytes = w.total;
    return LF_OK;
}

// Per layer, with one E for the keys and the values of every head (layerwise sharing), the
// projected keys are E . (X W_K^T) = (E . X) W_K^T, and likewise for the values: the layer
// projects its input once along the sequence (Xbar = E . X, k x d_model per batch item) and maps
// Xbar by W_K and W_V, so the n-long keys and values are never formed.  The queries are X W_Q^T.
int linformer_stack_forward(const lf_stack* s, const void* X, const void* Wqkv, const void* Wo,
                            const void* E, const int32_t* lengths, void* Y, void* ws,
                            size_t ws_bytes, void* stream) {
    int st = check_stack(s);
    if (st) return st;
    const lf_problem p = layer_problem(s);
    st = check_problem(&p);
    if (st) return st;
    lf::ProjGeom g;
    if (!stack_geometry(s, &g)) return LF_ERR_SHAPE;
    StackWs w;
    stack_ws(s, p, g, &w);
    if (!X || !Wqkv || !Wo || !E || !Y || !ws) return LF_ERR_NULL;
    if (ws_bytes < w.total) return LF_ERR_WORKSPACE;
    if (!aligned16(X) || !aligned16(Wqkv) || !aligned16(Wo) || !aligned16(E) || !aligned16(Y) ||
        !aligned16(ws))
        return LF_ERR_ALIGN;
    if (lengths && ((uintptr_t)lengths & 3u)) return LF_ERR_ALIGN;
    const size_t L = (size_t)s->layers, dm = (size_t)s->d_model;
    const size_t ybytes = (s->keep_layers ? L : 1) * w.act;
    const Range ins[] = {{X, w.act}, {Wqkv, L * 3 * dm * dm * 2}, {Wo, L * dm * dm * 2},
                         {E, ef_bytes(&p)}, {lengths, lengths ? 4u * s->batch : 0u}};
    const Range outs[] = {{Y, ybytes}, {ws, w.total}};
    if (any_overlap(outs, 2, ins, 5)) return LF_ERR_ALIAS;
    st = check_device();
    if (st) return st;

    hipStream_t strm = (hipStream_t)stream;
    uint8_t* base = (uint8_t*)ws;
    uint16_t* Qp = (uint16_t*)(base + w.q);
    uint16_t* O = (uint16_t*)(base + w.o);
    uint16_t* Xbar = (uint16_t*)(base + w.xbar);
    uint8_t* Kbar = base + w.kbar;
    uint16_t* Vbar = (uint16_t*)(base + w.vbar);
    const size_t e = (size_t)s->batch * s->heads * s->k * 64;
    const int T = s->batch * s->n, D = s->d_model;
    const float c = eff_scale(&p) * lf::kLog2e;
    const void* in = X;
    for (int l = 0; l < s->layers; ++l) {
        void* out;
        if (s->keep_layers) out = (uint8_t*)Y + (size_t)l * w.act;
        else if (l == s->layers - 1) out = Y;
        else out = base + w.ping + (size_t)(l & 1) * round_up(w.act, 256);
        const uint16_t* Wl = (const uint16_t*)Wqkv + (size_t)l * 3 * dm * dm;
        const uint16_t* Wol = (const uint16_t*)Wo + (size_t)l * dm * dm;
        // queries: X W_Q^T into the head-planar plane the attention reads
        lf::LinearBf16Args q{};
        q.W = Wl;
        q.X = (const uint16_t*)in;
        q.Y = Qp;
        q.T = T;
        q.F = D;
        q.K = D;
        q.n = s->n;
        q.H = s->heads;
        q.act_mode = 0;
        q.out_mode = 1;
        q.dm = D;
        q.plane = (size_t)T * D;
        st = do_linear(q, strm);
        if (st) return st;
        // Xbar = E . X over the valid positions
        lf::ProjBf16Args pa{};
        pa.K = (const uint16_t*)in;
        pa.V = (const uint16_t*)in;
        pa.E = (const uint16_t*)E;
        pa.F = (const uint16_t*)E;
        pa.lengths = lengths;
        pa.Vb = Xbar;
        pa.part = g.S > 1 ? (float*)(base + w.part) : nullptr;
        pa.c = 1.0f;
        pa.g = g;
        st = launch_status(lf::launch_proj_bf16(pa, strm));
        if (st) return st;
        if (stack_fused(s)) {
            // Kbar, Vbar = Xbar_b [W_K; W_V]_h^T per (b, h) into LDS, then the attention, in one
            // launch (fused_bf16.hip, stack form)
            lf::FusedBf16Args f{};
            f.Q = Qp;
            f.K = Wl + dm * dm;   // W_K rows, then W_V rows
            f.E = Xbar;
            f.lengths = lengths;
            f.O = O;
            f.B = s->batch;
            f.H = s->heads;
            f.n = s->n;
            f.k = s->k;
            f.e_heads = 1;
            f.c = c;
            f.dm = D;
            fused_split(f);
            st = launch_status(lf::launch_fused_bf16(f, strm));
            if (st) return st;
        } else {
        // Kbar | Vbar = Xbar [W_K; W_V]^T, Kbar straight into the attention's format
        lf::LinearBf16Args kv{};
        kv.W = Wl + dm * dm;
        kv.X = Xbar;
        kv.Y = (uint16_t*)Kbar;
        kv.Klo = Kbar + 2 * e;
        kv.Ksc = Kbar + 3 * e;
        kv.Yv = Vbar;
        kv.c = c;
        kv.T = s->batch * s->k;
        kv.F = 2 * D;
        kv.K = D;
        kv.n = s->k;
        kv.H = s->heads;
        kv.act_mode = 1;
        kv.out_mode = 2;
        kv.dm = D;
        st = do_linear(kv, strm);
        if (st) return st;
        st = do_attend(&p, Qp, Kbar, Vbar, lengths, O, strm);
        if (st) return st;
        }
        // output projection of the concatenated heads
        lf::LinearBf16Args o{};
        o.W = Wol;
        o.X = O;
        o.Y = (uint16_t*)out;
        o.T = T;
        o.F = D;
        o.K = D;
        o.n = s->n;
        o.H = s->heads;
        o.act_mode = 1;
        o.out_mode = 0;
        o.dm = D;
        st = do_linear(o, strm);
        if (st) return st;
        in = out;
    }
    return LF_OK;
}

int linformer_project_kv_conv(const lf_problem* p, const void* K, const void* V, const void* wE,
                              const void* wF, const int32_t* lengths, void* Kbar, void* Vbar,
                              void* stream) {
    const void* wFr = nullptr;
    int st = check_conv(p, K, V, wE, wF, lengths, &wFr);
    if (st) return st;
    if (!Kbar || !Vbar) return LF_ERR_NULL;
    if (!aligned16(Kbar) || !aligned16(Vbar)) return LF_ERR_ALIGN;
    const Range ins[] = {{K, qkv_bytes(p)}, {V, qkv_bytes(p)}, {wE, conv_w_bytes(p)},
                         {wFr, conv_w_bytes(p)}, {lengths, lengths ? 4u * p->batch : 0u}};
    const Range outs[] = {{Kbar, kbar_bytes(p)}, {Vbar, vbar_bytes(p)}};
    if (any_overlap(outs, 2, ins, 5)) return LF_ERR_ALIAS;
    st = check_device();
    if (st) return st;
    return do_conv(p, K, V, wE, wFr, lengths, Kbar, Vbar, (hipStream_t)stream);
}

int linformer_forward_conv(const lf_problem* p, const void* Q, const void* K, const void* V,
                           const void* wE, const void* wF, const int32_t* lengths, void* O,
                           void* ws, size_t ws_bytes, void* stream) {
    const void* wFr = nullptr;
    int st = check_conv(p, K, V, wE, wF, lengths, &wFr);
    if (st) return st;
    const size_t kb = round_up(kbar_bytes(p), 256), vb = round_up(vbar_bytes(p), 256);
    if (!Q || !O || !ws) return LF_ERR_NULL;
    if (ws_bytes < kb + vb) return LF_ERR_WORKSPACE;
    if (!aligned16(Q) || !aligned16(O) || !aligned16(ws)) return LF_ERR_ALIGN;
    const Range ins[] = {{Q, qkv_bytes(p)}, {K, qkv_bytes(p)}, {V, qkv_bytes(p)},
                         {wE, conv_w_bytes(p)}, {wFr, conv_w_bytes(p)},
                         {lengths, lengths ? 4u * p->batch : 0u}};
    const Range outs[] = {{O, qkv_bytes(p)}, {ws, kb + vb}};
    if (any_overlap(outs, 2, ins, 6)) return LF_ERR_ALIAS;
    st = check_device();
    if (st) return st;
    uint8_t* w = (uint8_t*)ws;
    hipStream_t strm = (hipStream_t)stream;
    st = do_conv(p, K, V, wE, wFr, lengths, w, w + kb, strm);
    if (st) return st;
    return do_attend(p, Q, w, w + kb, lengths, O, strm);
}

int linformer_backward_workspace_size(const lf_problem* p, size_t* bytes) {
    int st = check_problem(p);
    if (st) return st;
    if (!bytes) return LF_ERR_NULL;
    BwWs w;
    bw_ws(p, &w);
    *bytes = w.total;
    return LF_OK;
}

int linformer_backward(const lf_problem* p, const void* Q, const void* K, const void* V,
                       const void* E, const void* F, const int32_t* lengths, const void* dO,
                       float* dQ, float* dK, float* dV, float* dE, float* dF, void* ws,
                       size_t ws_bytes, void* stream) {
    int st = check_problem(p);
    if (st) return st;
    if (!Q || !K || !V || !E || !dO || !dQ || !dK || !dV || !dE || !ws) return LF_ERR_NULL;
    const void* Fr = nullptr;
    st = resolve_f(p, E, F, &Fr);
    if (st) return st;
    const bool separate = bw_separate(p, E, F);
    if (separate != (dF != nullptr)) return separate ? LF_ERR_NULL : LF_ERR_SHARE;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(E) || !aligned16(Fr) ||
        !aligned16(dO) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(dE) ||
        (dF && !aligned16(dF)) || !aligned16(ws))
        return LF_ERR_ALIGN;
    if (lengths && ((uintptr_t)lengths & 3u)) return LF_ERR_ALIGN;
    BwWs w;
    bw_ws(p, &w);
    size_t need = 0;
    linformer_backward_workspace_size(p, &need);
    if (ws_bytes < need) return LF_ERR_WORKSPACE;
    const size_t g4 = (size_t)p->batch * p->heads * p->n * 64 * 4;
    const size_t m4 = (size_t)(p->share == LF_SHARE_NONE ? p->heads : 1) * p->k * p->n * 4;
    const Range ins[] = {{Q, qkv_bytes(p)}, {K, qkv_bytes(p)}, {V, qkv_bytes(p)},
                         {E, ef_bytes(p)}, {Fr, ef_bytes(p)}, {dO, qkv_bytes(p)},
                         {lengths, lengths ? 4u * p->batch : 0u}};
    const Range outs[] = {{dQ, g4}, {dK, g4}, {dV, g4}, {dE, m4}, {dF, dF ? m4 : 0}, {ws, need}};
    if (any_overlap(outs, 6, ins, 7)) return LF_ERR_ALIAS;
    st = check_device();
    if (st) return st;

    hipStream_t strm = (hipStream_t)stream;
    uint8_t* b = (uint8_t*)ws;
    float *Kb = (float*)(b + w.kb), *Vb = (float*)(b + w.vb), *stats = (float*)(b + w.stats);
    float *dKb = (float*)(b + w.dkb), *dVb = (float*)(b + w.dvb);
    float* part = (float*)(b + w.part);
    auto run_gemm = [&](lf::BwGemm& g) {
        lf::bw_gemm_plan(g);
        g.part = part;
        return lf::launch_bw_gemm(g, strm);
    };
    // Q, K, V, E, F and dO are read in their own dtype; rows of K, V and dO at or past a length are
    // never read (the reductions over positions stop there, or read them as zero)
    const int bf = p->dtype == LF_BF16 ? 1 : 0;
    const int B = p->batch, H = p->heads, n = p->n, k = p->k;
    const float s = eff_scale(p);
    const bool unshared = p->share == LF_SHARE_NONE;
    hipError_t e = hipSuccess;
    const long long hn64 = (long long)n * 64, hk64 = (long long)k * 64, kn = (long long)k * n;
    // Kbar = E_h K, Vbar = F_h V in fp32, by the forward pass's projection (positions past the
    // length contribute nothing)
    {
        lf::ProjGeom g;
        if (!geometry(p, &g)) return LF_ERR_SHAPE;
        st = do_project(p, K, V, E, Fr, lengths, Kb, Vb, part, g, strm, true);
        if (st) return st;
    }
    lf::BwAttendArgs at{};
    at.Q = Q; at.dO = dO; at.in_bf16 = bf; at.Kb = Kb; at.Vb = Vb; at.stats = stats; at.dQ = dQ;
    at.B = B; at.H = H; at.n = n; at.k = k; at.scale = s; at.lengths = lengths;
    {   // about three rounds of one workgroup per compute unit (MI355X: 256)
        const int nblk = (n + 127) / 128;
        at.qb = std::max(1, std::min(nblk, nblk * B * H / 768));
    }
    if (lf::launch_bw_attend(at, strm) != hipSuccess) return LF_ERR_LAUNCH;
    // dVbar = P^T dO, dKbar = s dS^T Q, reductions over the queries before the length, P and dS
    // recomputed from the statistics the kernel above stored
    lf::BwKvArgs kv{};
    kv.Q = Q; kv.dO = dO; kv.in_bf16 = bf; kv.Kb = Kb; kv.Vb = Vb; kv.stats = stats;
    kv.lengths = lengths; kv.dKb = dKb; kv.dVb = dVb;
    kv.B = B; kv.H = H; kv.n = n; kv.k = k; kv.scale = s;
    kv.qparts = lf::kv_qparts(B, H, k);
    if (kv.qparts == 2) {
        kv.part = part;
        kv.pair_ctr = (unsigned long long*)((uint8_t*)part + lf::kv_sums_bytes(B, H, k));
        kv.pair_epoch = next_pair_epoch();
    }
    if (lf::launch_bw_kv(kv, strm) != hipSuccess) return LF_ERR_LAUNCH;
    // dE (+)= dXbar X^T: M = k, N = n, reduction over (b, c) (unshared: z = h) or over (b, h, c);
    // positions at or past item b's length read as zero
    // (dF given: dE and dF in one launch, batch entries z >= zhalf taking dVbar, V, dF)
    auto grad_mat = [&](const float* dXb, const void* X, float* out, float beta, bool both) {
        lf::BwGemm g = gemm0();
        g.A = dXb; g.B = X; g.C = out; g.beta = beta; g.b_bf16 = bf;
        g.M = k; g.N = n; g.kblk = 64;
        g.bj_len = lengths; g.bj_div = unshared ? 1 : H;
        if (unshared) {
            g.Z = H; g.K = B * 64;
            g.a_z1 = hk64; g.a_kb = H * hk64;
            g.b_z1 = hn64; g.b_kb = H * hn64;
            g.c_z1 = kn;
        } else {
            g.Z = 1; g.K = B * H * 64;
            g.a_kb = hk64;
            g.b_kb = hn64;
        }
        g.a_i = 64; g.a_kc = 1;
        g.b_kc = 1; g.b_j = 64;
        g.c_i = n; g.c_j = 1;
        if (both) {
            g.A2 = dVb; g.B2 = V; g.C2 = dF;
            g.zhalf = g.Z;
            g.Z *= 2;
        }
        return run_gemm(g);
    };
    if (separate) {
        e = grad_mat(dKb, K, dE, 0.0f, true);
    } else {   // one matrix: dE = dKbar K^T + dVbar V^T
        e = grad_mat(dKb, K, dE, 0.0f, false);
        if (e == hipSuccess) e = grad_mat(dVb, V, dE, 1.0f, false);
    }
    if (e != hipSuccess) return LF_ERR_LAUNCH;
    // dK = E_h^T dKbar, dV = F_h^T dVbar in one launch: z = (b, h) for dK, then again for dV
    // (batch entries z >= zhalf take F, dVbar, dV), M = n, N = 64, reduction over k
    {
        lf::BwGemm g = gemm0();
        g.A = E; g.B = dKb; g.C = dK; g.a_bf16 = bf;
        g.A2 = Fr; g.B2 = dVb; g.C2 = dV; g.zhalf = B * H;
        g.M = n; g.N = 64; g.K = k; g.Z = 2 * B * H; g.zdiv = H; g.kblk = k;
        g.a_z2 = unshared ? kn : 0; g.a_i = 1; g.a_kc = n;
        g.b_z1 = H * hk64; g.b_z2 = hk64; g.b_kc = 64; g.b_j = 1;
        g.c_z1 = H * hn64; g.c_z2 = hn64; g.c_i = 64; g.c_j = 1;
        g.row_len = lengths;   // positions past the length get zero gradients
        e = run_gemm(g);
    }
    return launch_status(e);
}

}  // extern "C"
