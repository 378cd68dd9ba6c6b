/*
 * liblinformer -- Linformer low-rank self-attention for one non-causal encoder layer,
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (Linformer 요약 설명, greeksharifa.github.io, section "Model"; Linformer summary
 * card, ai-papers.xuzou.cn, section 方法适配 "method"): for every batch item b and head h the keys
 * and values are projected along the sequence axis by E, F of shape k x n,
 *     Kbar = E . K,   Vbar = F . V               (k x d each)
 * and each query attends to the k projected slots,
 *     O = softmax(scale * Q . Kbar^T) . Vbar     (n x d, softmax over the k slots of a row).
 *
 * Tensor layouts (all row-major, contiguous, element type per lf_problem.dtype):
 *   Q, K, V, O : [batch, heads, n, d]
 *   E, F       : [H_E, k, n], H_E = heads for LF_SHARE_NONE, 1 for the shared modes
 *   lengths    : int32 [batch] in device memory, or NULL (every position valid)
 * n is the fixed, padded maximum length.  With lengths, positions t >= lengths[b] contribute
 * nothing to Kbar, Vbar (exactly what zero padding would give), the softmax still covers all k
 * slots, and output rows i >= lengths[b] are written as zero.  Lengths are clamped to [0, n] on
 * the device.  (Padding: Linformer 요약 설명, section "Model" -- the length-axis projection is
 * sized for a maximum length, so shorter inputs are padded.)
 *
 * Projection sharing (Linformer summary card, section 方法适配; Linformer 요약 설명, section
 * "Additional Efficiency Techniques"):
 *   LF_SHARE_NONE      per-head E_h and F_h (E, F hold `heads` matrices; F may equal E)
 *   LF_SHARE_HEADWISE  one E and one F for all heads of the layer
 *   LF_SHARE_KV        one matrix for all heads, E = F (F must be NULL or equal to E)
 *   LF_SHARE_LAYERWISE one matrix for all heads, E = F, and the caller passes the same E to
 *                      every layer (within one call it computes what LF_SHARE_KV computes)
 *
 * Precision:
 *   LF_F32  : fp32 in, fp32 arithmetic, fp32 out.
 *   LF_BF16 : bf16 Q, K, V, E, F, O; all sums accumulate in fp32; the softmax runs in fp32.
 *             Kbar is kept to within 2^-12 of the largest value of each row half, as a bf16
 *             plane plus an fp8 (e4m3) residual plane with power-of-two block scales (layout
 *             below); the residual's product with Q takes Q in e4m3 with its own power-of-two
 *             scale per query and 32-column block, so every finite bf16 Q is in range (e4m3
 *             alone ends at 448).  Vbar and the softmax weights are rounded once to bf16 (round
 *             to nearest even) for the matrix cores.
 *   Inputs must be finite; results for NaN or infinite inputs are not defined.
 *
 * Shape limits: d == 64; k % 32 == 0 and 32 <= k <= 256; n % 64 == 0 and n >= 64;
 * 1 <= batch <= 4096, heads >= 1; batch * heads * n * d < 2^31 elements.
 *
 * Ownership and threading: the caller owns every buffer (device memory) and keeps it alive until
 * the stream has finished the call.  The library allocates nothing and keeps no state between
 * calls except a per-device architecture check (and, for linformer_forward_noalloc(), the device
 * address of its fixed scratch buffer); calls are reentrant, except that overlapping
 * linformer_forward_noalloc() calls on one device share that buffer.  Work is enqueued on
 * `stream` (a hipStream_t; NULL means the default stream) and the calls return before it runs.
 *
 * Errors: every argument is validated on the host before anything is enqueued, so an error
 * return means no work was queued.  Faults during execution surface at the caller's next
 * synchronisation.  No C++ exception crosses this interface.
 */
#ifndef LINFORMER_H
#define LINFORMER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lf_status {
    LF_OK = 0,
    LF_ERR_NULL = 1,       /* a required pointer is NULL                                   */
    LF_ERR_SHAPE = 2,      /* a dimension is outside the limits above                       */
    LF_ERR_DTYPE = 3,      /* unknown dtype                                                 */
    LF_ERR_SHARE = 4,      /* unknown sharing mode, or F given where it must alias E        */
    LF_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than linformer_workspace_size()     */
    LF_ERR_ALIGN = 6,      /* a tensor pointer is not 16-byte aligned                       */
    LF_ERR_ALIAS = 7,      /* an output range overlaps an input or another output range     */
    LF_ERR_NO_DEVICE = 8,  /* no HIP device is available                                    */
    LF_ERR_ARCH = 9,       /* the current device is not gfx950                              */
    LF_ERR_LAUNCH = 10,    /* a kernel launch was rejected by the runtime                   */
    LF_ERR_SCRATCH = 11    /* linformer_forward_noalloc: the problem's workspace exceeds
                              LINFORMER_NOALLOC_SCRATCH_BYTES, or the fixed buffer could not
                              be located on the current device                              */
};

enum lf_dtype { LF_F32 = 0, LF_BF16 = 1 };

enum lf_share {
    LF_SHARE_NONE = 0,
    LF_SHARE_HEADWISE = 1,
    LF_SHARE_KV = 2,
    LF_SHARE_LAYERWISE = 3
};

/* Problem descriptor, passed by pointer; read only during the call. */
typedef struct lf_problem {
    int32_t batch;   /* B                                                    */
    int32_t heads;   /* H                                                    */
    int32_t n;       /* padded maximum sequence length                       */
    int32_t d;       /* head dimension (64)                                  */
    int32_t k;       /* projected length                                     */
    int32_t dtype;   /* enum lf_dtype                                        */
    int32_t share;   /* enum lf_share                                        */
    float scale;     /* score scale; 0 means 1/sqrt(d)                       */
} lf_problem;

/* Human-readable name of a status code (static string, never NULL). */
const char* linformer_status_string(int status);

/* Bytes of device workspace linformer_forward() and linformer_project_kv() need for `p`
 * (it covers Kbar/Vbar staging, the projection's split partial sums and, for shapes the
 * one-launch short-sequence path takes, one 8-byte hand-off flag per (b, h)).  Host only. */
int linformer_workspace_size(const lf_problem* p, size_t* bytes);

/* Bytes of the Kbar and Vbar buffers linformer_project_kv() writes and linformer_attend() reads.
 *   LF_F32 : Kbar fp32 [B, H, k, d]; Vbar fp32 [B, H, k, d].
 *   LF_BF16: Vbar bf16 [B, H, k, d].  Kbar holds x = c * Kbar with c = scale * log2(e) (the
 *            attention kernel works in base-2 logits), as three consecutive planes:
 *              hi  bf16 [B, H, k, 64]: bf16(x), round to nearest even;
 *              lo  byte [B, H, k, 64]: fp8 e4m3 of (x - hi) * 2^s, where each row has one s for
 *                  d < 32 and one for d >= 32 (the row's "blocks"), chosen so that the block's
 *                  largest |x - hi| * 2^s lies in [128, 256); within a row, byte 32 h + p holds
 *                  d = 16 (p / 8) + 8 h + p % 8 (p = 0..31, h = 0, 1);
 *              sc  byte [B, H, k, 2] : 127 - s of blocks 0 and 1.
 *            So x = hi + lo * 2^-s, and linformer_attend() must get the same scale as the
 *            linformer_project_kv() call that wrote Kbar.  Total 3 B H k d + 2 B H k bytes.
 *   Host only. */
int linformer_kv_sizes(const lf_problem* p, size_t* kbar_bytes, size_t* vbar_bytes);

/* Sequence projection, Kbar = E_h . K_{b,h} and Vbar = F_h . V_{b,h} over the valid positions
 * (Linformer 요약 설명, section "Model").  K, V, E, F and lengths are read; Kbar, Vbar are
 * written in the layouts of linformer_kv_sizes(); ws is scratch: its contents on entry do not
 * matter (the per-tile arrival counters of a two-way position split carry a tag unique to each
 * call and are left at zero), but calls that may run at the same time must not share one.
 * F: per the sharing mode above (NULL allowed for NONE, meaning F = E). */
int linformer_project_kv(const lf_problem* p, const void* K, const void* V, const void* E,
                         const void* F, const int32_t* lengths, void* Kbar, void* Vbar,
                         void* ws, size_t ws_bytes, void* stream);

/* Compressed attention, O = softmax(scale * Q . Kbar^T) . Vbar per (b, h), rows >= lengths[b]
 * zero (Linformer 요약 설명, sections "Model" and "Transformer and Self-Attention").  Q, Kbar,
 * Vbar, lengths are read; O is written. */
int linformer_attend(const lf_problem* p, const void* Q, const void* Kbar, const void* Vbar,
                     const int32_t* lengths, void* O, void* stream);

/* The whole layer: linformer_project_kv() into the workspace, then linformer_attend(). */
int linformer_forward(const lf_problem* p, const void* Q, const void* K, const void* V,
                      const void* E, const void* F, const int32_t* lengths, void* O, void* ws,
                      size_t ws_bytes, void* stream);

/* Bytes of the fixed scratch buffer linformer_forward_noalloc() uses (64 MiB per device). */
#define LINFORMER_NOALLOC_SCRATCH_BYTES (64u << 20)

/* linformer_forward() for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The workspace comes from a
 * buffer of LINFORMER_NOALLOC_SCRATCH_BYTES inside the library instead of an argument; every
 * device the library runs on holds its own copy from the first call on that device until the
 * process ends.  The caller still owns Q, K, V, E, F, lengths and O, with the layouts, sharing
 * rules and errors of linformer_forward(); the call allocates nothing (no hipMalloc, no library
 * allocation) and, like linformer_forward(), only enqueues kernels on `stream`.
 * Returns LF_ERR_SCRATCH, before anything is enqueued, when linformer_workspace_size(p) exceeds
 * the buffer (the pages' workloads need at most about 33 MiB).  The buffer's contents on entry do
 * not matter, and every call on one device shares it: calls that can overlap in time on the same
 * device (other streams, other host threads) race, and the caller must order them. */
int linformer_forward_noalloc(const lf_problem* p, const void* Q, const void* K, const void* V,
                              const void* E, const void* F, const int32_t* lengths, void* O,
                              void* stream);

/* Standard O(n^2) softmax attention of every (b, h) on the same device, the comparison
 * baseline for Linformer (Linformer 요약 설명, section "Transformer and Self-Attention"):
 * O = softmax(scale * Q . K^T) . V.  With lengths, keys at positions >= lengths[b] are left out
 * of the softmax and rows >= lengths[b] are zero.  p->k, p->share are ignored; bf16 only. */
int attention_dense_forward(const lf_problem* p, const void* Q, const void* K, const void* V,
                            const int32_t* lengths, void* O, void* stream);

/* ---- Convolution / pooling compression (Linformer 요약 설명, section "Additional Efficiency
 * Techniques": the sequence may be compressed by pooling or a convolution instead of a learned
 * dense projection).  With window s = n / k and stride s the projected rows are
 *     Kbar[r] = sum_{j < s} wE[j] K[r s + j],   Vbar[r] = sum_{j < s} wF[j] V[r s + j]
 * over the valid positions, which is the projection by the banded E with E[r][r s + j] = wE[j]
 * (mean pooling: w = 1/s).  wE, wF: bf16 [H_E, s] with H_E and the sharing rules of E and F
 * above.  Requires n % k == 0 and LF_BF16; Kbar and Vbar in the layouts of linformer_kv_sizes();
 * no workspace (ws may be NULL for the projection; linformer_forward_conv needs
 * linformer_workspace_size() bytes).  Attention is linformer_attend() unchanged. */
int linformer_project_kv_conv(const lf_problem* p, const void* K, const void* V, const void* wE,
                              const void* wF, const int32_t* lengths, void* Kbar, void* Vbar,
                              void* stream);

/* linformer_project_kv_conv() into the workspace, then linformer_attend(). */
int linformer_forward_conv(const lf_problem* p, const void* Q, const void* K, const void* V,
                           const void* wE, const void* wF, const int32_t* lengths, void* O,
                           void* ws, size_t ws_bytes, void* stream);

/* ---- Backward pass for learned projections (Linformer card, section 方法适配: E and F are
 * learned).  Given dO = dLoss/dO for the layer above, writes the gradients of the loss with
 * respect to Q, K, V, E and F, from the softmax Jacobian: with P = softmax(s Q Kbar^T),
 *   dVbar = P^T dO, dP = dO Vbar^T, dS = P o (dP - rowsum(P o dP)),
 *   dQ = s dS Kbar, dKbar = s dS^T Q, dE = dKbar K^T, dK = E^T dKbar, dF = dVbar V^T, dV = F^T dVbar
 * per (b, h); shared matrices collect every head that uses them.  Padding as in the forward:
 * rows of K, V and dO past the length are not read (they have no effect), and the gradients of
 * K, V rows and of the E, F columns past the length are zero.  Inputs in p->dtype and the forward layouts; gradients fp32:
 * dQ, dK, dV [B, H, n, d]; dE [H_E, k, n]; dF like dE when F is a separate matrix (headwise, or
 * unshared with F given and != E), else dF must be NULL and dE holds both projections' parts.
 * fp32 accumulation throughout (Kbar, Vbar recomputed in fp32); the GEMMs multiply fp32 operands
 * as split bf16 pairs (hi + lo, within 2^-16 of the value: the bf16x3 scheme), and the results
 * meet the 1e-4 relative bar of an fp32 computation (tested).  ws:
 * linformer_backward_workspace_size() bytes of scratch (16-byte aligned): fp32 Kbar, Vbar, dKbar,
 * dVbar, four floats of softmax statistics per query and split partial sums, O(B H (k d + n))
 * bytes; no n x k matrix is stored (P and dS are recomputed where they are reduced). */
int linformer_backward_workspace_size(const lf_problem* p, size_t* bytes);
int linformer_backward(const lf_problem* p, const void* Q, const void* K, const void* V,
                       const void* E, const void* F, const int32_t* lengths, const void* dO,
                       float* dQ, float* dK, float* dV, float* dE, float* dF, void* ws,
                       size_t ws_bytes, void* stream);

/* ---- Encoder attention stack.  Each of `layers` layers maps its input X [B, n, d_model] to
 * every head's queries, keys and values, runs Linformer attention (above) on every head with one
 * layerwise-shared E, concatenates the heads and applies the output projection; the result is the
 * next layer's input (Linformer 요약 설명, section "Transformer and Self-Attention": per-head
 * projections X W^Q, X W^K, X W^V of width d = d_model / heads, heads concatenated and mapped by
 * an output projection; Linformer summary card, section 方法适配: layerwise sharing, one
 * projection matrix for the whole model).  No other step (bias, residual, normalisation).
 *
 * Layouts (bf16, row-major, contiguous):
 *   X     [B, n, d_model]
 *   Wqkv  [layers, 3 d_model, d_model], applied as x . W^T: rows 0 .. d_model-1 give the queries,
 *         then the keys, then the values; feature f of each is column f % 64 of head f / 64
 *   Wo    [layers, d_model, d_model], applied as x . W^T to the concatenated heads (head h's
 *         column c is feature 64 h + c)
 *   E     [1, k, n], the one projection for every layer, head, key and value
 *   Y     [B, n, d_model] (keep_layers = 0) or [layers, B, n, d_model] (every layer's output)
 *   lengths as for the single layer: padded positions contribute nothing and output rows past
 *   the length are zero in every layer.
 * Shape limits: d_model = 64 heads, d_model % 192 == 0, the single layer's limits on n, k and
 * batch, and 3 batch n d_model < 2^30.  dtype must be LF_BF16.  Ownership, threading and errors
 * as above; Y must not overlap any input or the workspace.
 * With one E for the keys and the values, E . (X W_K^T) = (E . X) W_K^T: each layer projects its
 * input once along the sequence and maps the k projected rows by W_K and W_V (the same result up
 * to rounding, with the n-long keys and values never formed). */
typedef struct lf_stack {
    int32_t batch;        /* B                                                       */
    int32_t n;            /* padded maximum sequence length                          */
    int32_t d_model;      /* model width = 64 * heads                                */
    int32_t heads;        /* H                                                       */
    int32_t k;            /* projected length                                        */
    int32_t layers;       /* >= 1                                                    */
    int32_t dtype;        /* LF_BF16                                                 */
    int32_t keep_layers;  /* 1: Y holds every layer's output                         */
    float scale;          /* score scale; 0 means 1/sqrt(64)                         */
} lf_stack;

/* Bytes of device workspace linformer_stack_forward() needs (host only). */
int linformer_stack_workspace_size(const lf_stack* s, size_t* bytes);

/* The whole stack on `stream`; ws is scratch (its contents on entry do not matter). */
int linformer_stack_forward(const lf_stack* s, const void* X, const void* Wqkv, const void* Wo,
                            const void* E, const int32_t* lengths, void* Y, void* ws,
                            size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LINFORMER_H */
