/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts
 * feed-forward layer, forward pass.
 *
 * The layer (GLaM study note, "Sparse MoE Layer"; "Shared Expert" GLM-4.5
 * study note, "How it works"; GLM-5 "Shared expert" inspector page, "All 5
 * steps"):
 *
 *   l_t   = W_r x_t                                  router logits, fp32
 *   score = softmax(l_t)            (SOFTMAX scorer)  selection = gate = score
 *         = sigmoid(l_t)            (SIGMOID scorer)  selection = score + bias,
 *                                                     gate = score
 *   S_t   = the k experts with the largest selection score
 *   w_j   = alpha * g_j / (sum_{i in S_t} g_i + eps)  (renorm = 1)
 *         = alpha * g_j                               (renorm = 0)
 *   E_e(x) = W2[e] (SiLU(gate rows of W1[e] x) * (up rows of W1[e] x))  SWIGLU
 *          = W2[e] gelu(W1[e] x + b1[e]) + b2[e]                         GELU
 *   y_t   = sum_j w_j E_{e_j}(x_t) + E_sh(x_t)
 *
 * E_sh is a SwiGLU of width F_shared applied to every token's pre-routing
 * x_t (absent when F_shared == 0).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer to a dense, row-major, contiguous
 *   buffer that the caller allocated and owns, 16-byte aligned.  The library
 *   never allocates, frees or keeps a caller pointer past the call.
 * - `dtype` types x, the expert weights W1/b1/W2/b2 and the shared weights:
 *   fp32 (MOE_DTYPE_F32) or bf16 (MOE_DTYPE_BF16, stored as raw uint16 bit
 *   patterns).  `out_dtype` types y.  W_r, bias, w, the sorted expert
 *   outputs O and the shared-expert output Ysh are always fp32; indices are
 *   int32.
 * - `stream` / `aux_stream` are hipStream_t values passed as void*; NULL is
 *   the null stream.  All work is enqueued asynchronously; no call copies
 *   between host and device or synchronises the host, so results are valid
 *   once the stream(s) complete, and every call may be captured in a graph
 *   (moe_forward with its aux-stream fork and join included).
 * - Every buffer, the workspace included, must be ready on `stream` when the
 *   call is enqueued: work that produced it, or that still uses memory the
 *   allocator handed out again for it, must be ordered before `stream` (the
 *   same stream, an event wait, or a synchronisation).  The library orders
 *   `aux_stream` after `stream` itself.
 * - Validation happens before anything is enqueued: on any error nothing is
 *   launched and the outputs are untouched.  T == 0 is a valid no-op.
 * - Identical inputs on the same device give bitwise-identical outputs
 *   (no floating-point atomics anywhere).
 * - A handle is not thread-safe; use one handle per host thread.
 *
 * Return codes are moe_status values; moe_status_string() names them and
 * moe_last_error_detail() (per host thread) explains the last failure.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,      /* null pointer, bad enum, T < 0, k < 1, k > M, ... */
    MOE_ERR_UNSUPPORTED = 2,  /* k > 16, M > 1024, D/F/F_shared not multiples of 8,
                                 T*k or a buffer index beyond int32 */
    MOE_ERR_WORKSPACE = 3,    /* ws_bytes smaller than the call needs */
    MOE_ERR_HIP = 4           /* a HIP runtime call or launch failed */
} moe_status;

enum { MOE_SCORER_SOFTMAX = 0, MOE_SCORER_SIGMOID = 1 };
enum { MOE_ACT_SWIGLU = 0, MOE_ACT_GELU = 1 };
enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };
/* Layout of the weight matrices W1, W2, Wsh_gu, Wsh_dn (see moe_tile_weights). */
enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILED = 1 };
/* Weight matrices, for moe_tiled_weight_size / moe_tile_weights. */
enum { MOE_WEIGHT_W1 = 0, MOE_WEIGHT_W2 = 1, MOE_WEIGHT_SH_GU = 2, MOE_WEIGHT_SH_DN = 3 };

#define MOE_MAX_K 16
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_GROUPS 64

/* Layer descriptor (plain data).
 *   T        tokens (the flattened batch x positions, as the GLM-4.5 note's
 *            "Shapes" paragraph flattens (B,S,D) to (BS,D))
 *   D        hidden size;  M routed experts;  F routed expert width
 *   F_shared shared SwiGLU width (n_shared * expert width; 0 = none)
 *   k        experts per token (1..min(M,16))
 *   scorer   MOE_SCORER_*;  act MOE_ACT_*;  dtype MOE_DTYPE_* (inputs)
 *   out_dtype MOE_DTYPE_* of y (the reference layer returns y in the input
 *            dtype; fp32 keeps the fp32 accumulation unrounded)
 *   renorm   1: divide the selected gate values by their sum + eps
 *   alpha    routed scaling factor (multiplies every routed weight)
 *   eps      renormalisation epsilon (1e-20 in the GLM-4.5 note)
 *   weight_layout MOE_LAYOUT_ROWS (the row-major layouts below) or
 *            MOE_LAYOUT_TILED (W1, W2, Wsh_gu, Wsh_dn as moe_tile_weights
 *            writes them; bf16 only)
 *   n_group, topk_group  group-limited routing (the GLM-4.5 note's router
 *            "optionally masks by expert group"): with n_group > 1 the M
 *            experts form n_group groups of M/n_group consecutive experts,
 *            a group's score is the largest selection score among its
 *            experts, only the topk_group best groups (lower group index on
 *            an exact tie) stay candidates for the top-k.  Requires
 *            n_group | M, n_group <= 64 and k <= topk_group * M / n_group.
 *            n_group <= 1: no grouping.
 *
 * Launch tuning (zero everywhere = the library's own choice; outputs are
 * bitwise the same for every setting, only speed and the workspace size
 * change, so moe_workspace_size must see the same values as the call):
 *   tile_rows[4]  rows per workgroup tile of the bf16 GEMMs, in the order
 *                 routed up, routed down, shared up, shared down projection:
 *                 0 (choose), 64, 128, 160 or 256
 *   tile_order[4] workgroup order of the same four GEMMs over the 8 XCDs:
 *                 0 (choose), 1 whole tile groups dealt to the XCDs in turn,
 *                 2 hardware order, 3 one contiguous eighth per XCD
 *   group_m       m-tiles per group of the tile order: 0 (choose) or 1..16
 *   shared_mode   0 (choose), 1 the shared expert in launches of its own
 *                 (on aux_stream when given), 2 the shared expert as one
 *                 more group of the routed GEMM launches (needs F_shared ==
 *                 F, SwiGLU, bf16 and T <= 1024; otherwise as 1)
 * With rows_format 1 every tuning setting gives bitwise the same output; the
 * compact rows are used only where the shared expert is not merged, so with
 * them a merged and a separate shared expert differ by that rounding.
 *
 * Precision of one intermediate (a choice of rounding inside the layer's
 * stated tolerance, not tuning):
 *   rows_format   the gate-weighted expert rows that moe_forward hands from
 *                 the down projection to the combine: 0 (choose: compact
 *                 for bf16 layers), 1 fp32, 2 compact: fp16 values with one
 *                 power-of-two scale per 64 consecutive values of a row,
 *                 chosen so that the group's largest finite magnitude lands
 *                 in [2^14, 2^15) (scaling is exact, one round-to-nearest-
 *                 even to fp16: relative error <= 2^-11; half the bytes of
 *                 fp32).  bf16 layers only; a shared expert merged into the
 *                 routed GEMMs keeps fp32 rows.  The stage entry points
 *                 (moe_expert_ffn, moe_combine) always exchange fp32 rows. */
typedef struct moe_desc {
    int64_t T, D, M, F, F_shared;
    int32_t k;
    int32_t scorer;
    int32_t act;
    int32_t dtype;
    int32_t out_dtype;
    int32_t renorm;
    float alpha;
    float eps;
    int32_t weight_layout;
    int32_t n_group;
    int32_t topk_group;
    int32_t tile_rows[4];
    int32_t tile_order[4];
    int32_t group_m;
    int32_t shared_mode;
    int32_t rows_format;
} moe_desc;

/* Indices of moe_desc.tile_rows / tile_order. */
enum { MOE_GEMM_UP = 0, MOE_GEMM_DOWN = 1, MOE_GEMM_SHARED_UP = 2, MOE_GEMM_SHARED_DOWN = 3 };

typedef struct moe_handle moe_handle;

/* Create a handle bound to HIP device `device` (it becomes current during
 * calls).  Allocates only host state and two timing-free HIP events, and
 * looks up (once per device) the address of that device's fixed scratch
 * used by moe_forward_no_alloc. */
int moe_create(int device, moe_handle** out);
int moe_destroy(moe_handle* h);

/* Bytes of device workspace that moe_forward needs for `d`; the same size
 * also satisfies every stage call below.  Host-only computation. */
int moe_workspace_size(const moe_desc* d, size_t* bytes);

/* Tiled weight layout.  The expert and shared weights stream from HBM once
 * per tile of rows, which makes weight reads the layer's dominant traffic
 * when experts hold few rows (the GLaM-shaped and decode layers).  In the
 * row-major layouts each 64-element K stage of a 256-row weight tile is 256
 * separate 128-byte pieces; the tiled layout stores every such stage as one
 * contiguous 32 KB block, exactly as the GEMM keeps it in LDS, so it streams
 * at the full sequential rate.  A one-time copy, made when weights are
 * loaded.  For a matrix with B rows of K elements (per expert for W1, W2):
 *   W1 SWIGLU: B = 2F rows, output columns N = F; W1 GELU: B = N = F; K = D
 *   W2: B = N = D, K = F;  Wsh_gu: B = 2 F_shared, N = F_shared, K = D;
 *   Wsh_dn: B = N = D, K = F_shared
 * the tiled copy is, per expert, n_tiles = ceil(N / C) tiles (C = 128 for
 * the gate/up matrices of a SwiGLU, else 256) by n_k = ceil(K / 64) stages,
 * block (tile n, stage s) at element offset (n * n_k + s) * 16384 of the
 * expert's part, experts one after another.  A block holds 256 rows of 64
 * elements: row b is weight row R(n, b) (SwiGLU: within each group of 64
 * rows g = b / 64, rows b % 64 < 32 are gate rows n*128 + 32 g + b % 32 and
 * the others the matching up rows F + n*128 + 32 g + (b % 32); otherwise
 * n*256 + b), element c of the row (column s*64 + c of the weight) sits at
 * b*64 + 8*((c/8) ^ (b % 8)) + c % 8; rows past the matrix and columns past
 * K are zero. */

/* Bytes of the tiled copy of weight matrix `which` (MOE_WEIGHT_*, all M
 * experts for W1/W2) for `d` (bf16; F_shared > 0 for the shared ones).
 * Host-only computation. */
int moe_tiled_weight_size(const moe_desc* d, int which, size_t* bytes);

/* Write the tiled copy of weight matrix `which` from its row-major form
 * `src` (the layouts documented at moe_expert_ffn / moe_shared_expert) into
 * `dst` (moe_tiled_weight_size bytes; must not overlap src).  d's
 * weight_layout is ignored here.  Asynchronous on `stream`. */
int moe_tile_weights(moe_handle* h, const moe_desc* d, int which, const void* src, void* dst,
                     void* stream);

/* Router: logits, scores, top-k selection and weights [GLaM "Sparse MoE
 * Layer" router and TopK equations; GLM-4.5 "How it works" sigmoid router,
 * correction bias, renormalisation and scaling].
 *   x[T,D] (dtype), W_r[M,D] fp32, bias[M] fp32 (SIGMOID only; NULL = zero;
 *   ignored for SOFTMAX) -> idx[T,k] int32, w[T,k] fp32.
 * A token's k experts are distinct and stored in ascending expert order;
 * an exactly equal selection score goes to the lower expert index.  With
 * d->n_group > 1 only the kept groups' experts compete (see moe_desc).
 * Uses workspace (the split router weights and partial logits). */
int moe_route(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
              const float* bias, int32_t* idx, float* w, void* ws, size_t ws_bytes,
              void* stream);

/* Dispatch: group the T*k flat slots f = t*k + j by expert, stably
 * [GLaM "Capacity, Active Compute, and Reporting": dispatch / expert
 * batching].
 *   idx[T,k] -> counts[M], offsets[M+1] (exclusive prefix, offsets[M] =
 *   number of kept slots), sorted_slot[T*k] (flat slot of sorted row r),
 *   sorted_token[T*k] (= sorted_slot / k), slot_row[T*k] (row of slot f).
 * Rows of one expert are in ascending slot order.  An index equal to M (or
 * outside [0,M)) is a dropped slot, the extra one-hot class of the GLM-5
 * routed-experts excerpt: counted nowhere, slot_row = -1, and the unused
 * tail rows r >= offsets[M] of sorted_slot/sorted_token are -1.
 * Precondition: a token's kept entries are distinct experts (the router
 * guarantees it); repeated entries leave the order unspecified (no access
 * goes out of bounds).  Uses workspace. */
int moe_permute(moe_handle* h, const moe_desc* d, const int32_t* idx, int32_t* counts,
                int32_t* offsets, int32_t* sorted_token, int32_t* sorted_slot,
                int32_t* slot_row, void* ws, size_t ws_bytes, void* stream);

/* Routed experts over the dispatched rows [GLaM dense FFN equation; GLM-5
 * "All 5 steps"]: for every sorted row r of expert e, with t =
 * sorted_token[r] and f = sorted_slot[r],
 *   O[r,:] = w[f] * E_e(x[t,:])
 * W1[M,G*F,D] (SWIGLU: G = 2, gate rows 0..F-1 then up rows F..2F-1;
 * GELU: G = 1), b1[M,F] and b2[M,D] (GELU only, NULL = zero), W2[M,D,F],
 * w[T*k] fp32 indexed by flat slot, O[T*k,D] fp32 (rows >= offsets[M]
 * untouched).  The hidden activations (dtype) live in the workspace.
 * With d->weight_layout == MOE_LAYOUT_TILED, W1 and W2 are the tiled
 * copies (moe_tile_weights). */
int moe_expert_ffn(moe_handle* h, const moe_desc* d, const void* x,
                   const int32_t* sorted_token, const int32_t* sorted_slot,
                   const int32_t* offsets, const float* w, const void* W1,
                   const void* b1, const void* W2, const void* b2, float* O,
                   void* ws, size_t ws_bytes, void* stream);

/* Shared expert on every token's pre-routing x ["Shared Expert" GLM-4.5
 * note, shared-expert equation; GLM-5 "All 5 steps"]:
 *   Ysh[t,:] = Wsh_dn (SiLU(Wsh_gate x_t) * (Wsh_up x_t))
 * Wsh_gu[2*F_shared, D] (gate rows then up rows), Wsh_dn[D, F_shared],
 * Ysh[T,D] fp32.  Requires F_shared > 0.  Uses workspace.  With
 * d->weight_layout == MOE_LAYOUT_TILED both are the tiled copies. */
int moe_shared_expert(moe_handle* h, const moe_desc* d, const void* x,
                      const void* Wsh_gu, const void* Wsh_dn, float* Ysh, void* ws,
                      size_t ws_bytes, void* stream);

/* Combine [GLaM MoE output sum; GLM-4.5 "How it works" output equation]:
 *   y[t,:] = sum_{j<k} O[slot_row[t*k+j], :]  (+ Ysh[t,:] if Ysh != NULL)
 * summed in fp32 in fixed j order, then rounded once to out_dtype.  O[T*k,D]
 * fp32.  A slot with slot_row < 0 contributes nothing.  No atomics.  y must
 * not alias O or Ysh. */
int moe_combine(moe_handle* h, const moe_desc* d, const float* O, const int32_t* slot_row,
                const float* Ysh, void* y, void* stream);

/* Whole layer: route, permute, expert FFNs, shared expert, combine.
 * The shared expert runs on `aux_stream` (forked from and joined back into
 * `stream` with events) so it overlaps the routed path; aux_stream == NULL
 * runs it on `stream`, with bitwise-identical results.  y[T,D] (out_dtype)
 * must not alias x.  Shared weights may be NULL only when F_shared == 0. */
int moe_forward(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
                const float* bias, const void* W1, const void* b1, const void* W2,
                const void* b2, const void* Wsh_gu, const void* Wsh_dn, void* y,
                void* ws, size_t ws_bytes, void* stream, void* aux_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_forward, same arguments and results (bitwise), but the
 * workspace is a fixed scratch array compiled into the library, one per GPU,
 * MOE_NO_ALLOC_SCRATCH_BYTES (64 MiB) each, held until the process ends.
 * It allocates and frees nothing.  Layers whose moe_workspace_size exceeds
 * the scratch (prefill-sized batches; at the GLM-4.5 decode shape, batches
 * of more than about 250 tokens) return MOE_ERR_UNSUPPORTED before anything
 * is enqueued.  Every call on one GPU uses that GPU's one scratch: calls
 * that may overlap in time on one GPU (on different streams, or from
 * different host threads) race and must be ordered by the caller.  The
 * scratch keeps the last call's contents; nothing in it needs to start
 * zeroed. */
#define MOE_NO_ALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_no_alloc(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
                         const float* bias, const void* W1, const void* b1, const void* W2,
                         const void* b2, const void* Wsh_gu, const void* Wsh_dn, void* y,
                         void* stream, void* aux_stream);

/* Layer backward (training).  Gradient of moe_forward for the output
 * gradient dy[T,D] (bf16): the chain rule through each step of the forward
 * definition (GLaM study note, "Sparse MoE Layer": routed sum of gate-
 * weighted expert FFNs, trained under the causal LM objective; GLM-4.5 note,
 * "How it works": sigmoid scores, selection-only correction bias,
 * renormalisation with eps, alpha, shared expert).  The top-k selection and
 * the correction bias are piecewise constant and get no gradient; the
 * weights pass it through the renormalisation and the gate values (softmax
 * probabilities or sigmoid scores) to the router logits.  The routing is
 * recomputed from x.
 *
 * bf16 layers with row-major weights only (MOE_ERR_UNSUPPORTED otherwise).
 * Outputs, all fp32 and written whole: dx[T,D]; dW_r[M,D]; dW1, dW2, dWsh_gu,
 * dWsh_dn in their weights' layouts (shared ones only when F_shared > 0);
 * db1[M,F] and db2[M,D] for GELU experts when non-NULL (ignored for SwiGLU);
 * load_count[M] (int32 slots routed to each expert) and load_score[M] (sum
 * over tokens of each expert's gate value), the per-expert load statistics
 * of this batch.  Workspace: moe_backward_workspace_size() bytes.  T == 0
 * writes zero gradients.  Deterministic (no atomics). */
int moe_backward_workspace_size(const moe_desc* d, size_t* bytes);
int moe_backward(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
                 const float* bias, const void* W1, const void* b1, const void* W2,
                 const void* b2, const void* Wsh_gu, const void* Wsh_dn, const void* dy,
                 float* dx, float* dW_r, float* dW1, float* db1, float* dW2, float* db2,
                 float* dWsh_gu, float* dWsh_dn, int32_t* load_count, float* load_score,
                 void* ws, size_t ws_bytes, void* stream);

/* Per-kernel timing for measurement harnesses.  While enabled, every kernel
 * the handle launches whose label contains `filter` (NULL or "" = all) is
 * bracketed by a pair of HIP timing events on the stream it runs on, up to
 * `capacity` launches.  moe_profile_stop() waits for those events and folds
 * them into per-label totals readable with moe_profile_results().  Labels:
 * route, perm_count, perm_scan, perm_scatter, tile_table, ffn_up, ffn_down,
 * shared_up, shared_down, combine, and for the backward b_up, b_dh, b_dx,
 * b_wgrad, b_transpose, b_other. */
typedef struct moe_kernel_time {
    char label[32];
    int64_t launches;
    double total_ms;
} moe_kernel_time;

int moe_profile_start(moe_handle* h, int capacity, const char* filter);
int moe_profile_stop(moe_handle* h);
int moe_profile_results(moe_handle* h, moe_kernel_time* out, int max_entries, int* n_entries);

const char* moe_status_string(int status);
const char* moe_last_error_detail(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
