// Internal definitions shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;   // MOE_MAX_EXPERTS
constexpr int kMaxK = 16;           // MOE_MAX_K

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (gfx950's v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float floatx2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2_v{lo, hi}, bf16x2_v));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
// Four bf16 at p (8-byte aligned) to fp32, and back.
__device__ __forceinline__ void load_bf16x4(const bf16_t* p, float (&v)[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void store_bf16x4(bf16_t* p, float a, float b, float c, float d) {
    uint2 u;
    u.x = pack_bf16x2(a, b);
    u.y = pack_bf16x2(c, d);
    *reinterpret_cast<uint2*>(p) = u;
}

// Activations in fp32.
// SiLU(z) = z sigmoid(z); the hardware reciprocal (1 ulp) in place of a
// full-precision division.  z -> -inf gives -0.
__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
// GELU(z) = z Phi(z) with Phi(z) = erfc(-z / sqrt 2) / 2.  erfc(a), a >= 0,
// by Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7): t P(t) exp(-a^2) with
// t = 1 / (1 + p a) and a degree-5 polynomial P.  Branch-free, and for
// z << 0 it yields Phi(z) directly rather than the cancellation 1 + erf.
__device__ __forceinline__ float gelu_erf_f32(float z) {
    const float a = fabsf(z) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, a, 1.0f));
    float p = fmaf(1.061405429f, t, -1.453152027f);
    p = fmaf(p, t, 1.421413741f);
    p = fmaf(p, t, -0.284496736f);
    p = fmaf(p, t, 0.254829592f);
    const float lower = 0.5f * t * p * __expf(-a * a);   // Phi(-|z|)
    return z * (z >= 0.f ? 1.0f - lower : lower);
}

// Derivatives for the backward.  silu'(z) = s (1 + z (1 - s)), s = sigmoid(z).
__device__ __forceinline__ float silu_grad_f32(float z) {
    const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-z));
    return s * (1.0f + z * (1.0f - s));
}
// gelu'(z) = Phi(z) + z phi(z); Phi from the same erfc approximation as
// gelu_erf_f32, phi(z) = exp(-z^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_grad_f32(float z) {
    const float a = fabsf(z) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, a, 1.0f));
    float p = fmaf(1.061405429f, t, -1.453152027f);
    p = fmaf(p, t, 1.421413741f);
    p = fmaf(p, t, -0.284496736f);
    p = fmaf(p, t, 0.254829592f);
    const float e = __expf(-a * a);
    const float lower = 0.5f * t * p * e;   // Phi(-|z|)
    const float Phi = z >= 0.f ? 1.0f - lower : lower;
    return Phi + z * e * 0.3989422804014327f;   // exp(-z^2/2) = exp(-a^2)
}

// Kernel labels (indices into the profiling table).
enum Label : int {
    L_ROUTE = 0, L_PERM_COUNT, L_PERM_SCAN, L_PERM_SCATTER, L_TILE_TABLE,
    L_FFN_UP, L_FFN_DOWN, L_SHARED_UP, L_SHARED_DOWN, L_COMBINE,
    // backward
    L_B_UP, L_B_DH, L_B_DX, L_B_WGRAD, L_B_TRANSPOSE, L_B_OTHER, L_COUNT
};

// Epilogues of the expert GEMMs.
enum Epi : int {
    EPI_SWIGLU = 0,      // out[r, n] = silu(gate) * up            -> dtype
    EPI_GELU = 1,        // out[r, n] = gelu(acc + b1[e, n])       -> dtype
    EPI_DOWN_SCALED = 2, // out[r, n] = w[slot(r)] * (acc + b2[e, n]) -> fp32
    EPI_DOWN_F32 = 3,    // out[r, n] = acc                         -> fp32
    // backward (bf16 only):
    EPI_SWIGLU_SAVE = 4, // EPI_SWIGLU, and c2[r, n] = gate, c2[r, N + n] = up   (bf16)
    EPI_GELU_SAVE = 5,   // EPI_GELU, and c2[r, n] = acc + b1[e, n]             (bf16)
    EPI_DH_SWIGLU = 6,   // acc = dH_raw[r, n]; with dH = w * acc, gate / up from c2:
                         // out[r, n] = dH up silu'(gate), out[r, N + n] = dH silu(gate)
    EPI_DH_GELU = 7      // out[r, n] = w * acc * gelu'(z), z = c2[r, n]
    // EPI_DH_*: part[r][n-tile x waves] = sum over the wave's columns of
    // aux[r, n] * acc (aux = H), when part is non-null; w = row_w[r] or 1.
};

constexpr bool epi_pairs(int epi) { return epi == EPI_SWIGLU || epi == EPI_SWIGLU_SAVE; }

// One expert GEMM launch: C[rows, N] = epi(A[rows, K] . B[e]^T), where
// A rows come from `a` (through `gather` when non-null) and B[e] is the
// expert's [NB, K] row-major weight block.
struct GemmArgs {
    const void* a;            // [*, K] dtype
    const int32_t* gather;    // A row of sorted row r = gather[r]; NULL: r itself
    const void* b;            // [E, NB, K] dtype
    int64_t b_stride;         // elements between experts in b
    const void* bias;         // [E, N] dtype, nullable (GELU b1 or DOWN b2)
    const float* row_w;       // DOWN_SCALED: scale of sorted row r (its slot's weight); NULL: 1
    void* c;                  // [rows, N]
    const int32_t* tiles;     // grouped: per m-tile (expert, row0); NULL: dense
    const int32_t* offsets;   // grouped: expert row ranges [M+1]
    int64_t dense_rows;       // total rows (dense) / sorted rows (grouped)
    int64_t a_rows;           // rows of the matrix `a` points to (gathered loads)
    int b_rows;               // rows of one expert's weight block
    int K;                    // reduction length
    int N;                    // output columns
    int F_split;              // SWIGLU: row offset of the up block in B (= N)
    int k_split;              // dense DOWN_F32 only: K chunks, each writing its own
                              // [rows, N] partial at c + chunk * rows * N (0 = 1)
    int group_m;              // m-tiles per group of the tile order (0 = 4)
    int b_tiled;              // b holds tiled blocks (bf16): b_stride = one expert's blocks
    int b_kn;                 // b[e] is [K, N] row-major (b_stride = K * N); bf16, K = 64 stages
    int xcd_mode;             // workgroup order: 0 groups dealt to XCDs in turn, 1 plain,
                              // 2 contiguous slices per XCD
    const void* b_extra;      // grouped: weights of group extra_group, in place of
    int extra_group;          // b + extra_group * b_stride (NULL: none)
    // backward epilogues
    void* c2;                 // EPI_*_SAVE: pre-activations out; EPI_DH_*: in (bf16)
    const void* aux;          // EPI_DH_*: H (bf16, [rows, N]) for the weight-gradient dots
    float* part;              // EPI_DH_*: [rows][part_ld] partial dots (nullable)
    int part_ld;
    // K-grouped mode (koff non-null): group q multiplies A and B over the K
    // range [koff[q], koff[q+1]) (multiples of 64) and writes its own
    // [a_rows, N] output at c + q * c_group_stride; kgroups groups, dense
    // tiles over the A rows (dense_rows) and the N B rows.
    const int32_t* koff;
    int kgroups;
    int64_t c_group_stride;
    // EPI_DOWN_SCALED, compact rows (c16 non-null, c unused): c16[r, n] fp16
    // values with one scale exponent cexp[r, n / kRowGroup] per kRowGroup
    // columns, the value being c16 * 2^cexp
    void* c16;
    int8_t* cexp;
};

// Compact expert rows: fp16 values with one power-of-two scale per
// kRowGroup consecutive values of a row (the 64 columns one wave of the
// down projection holds of a row); [rows, N] fp16, then the exponents
// [rows, ceil(N / kRowGroup)] int8 at a 256-byte aligned offset.
constexpr int kRowGroup = 64;
inline int64_t compact_exp_offset(int64_t rows, int64_t N) {
    return ((rows * N * 2) + 255) & ~int64_t(255);
}
inline int64_t compact_row_bytes(int64_t rows, int64_t N) {
    return compact_exp_offset(rows, N) + rows * ((N + kRowGroup - 1) / kRowGroup);
}

// Weight tiles of the bf16 GEMM: 256 weight rows by K stages of 64.
constexpr int kTileRows = 256;
constexpr int kTileK = 64;
// Elements of one expert's tiled copy of a weight matrix with n_out output
// columns (SwiGLU: 128 per tile) and reduction length K.
inline int64_t tiled_elems(int64_t n_out, int64_t K, bool swiglu) {
    const int64_t per = swiglu ? kTileRows / 2 : kTileRows;
    return ((n_out + per - 1) / per) * ((K + kTileK - 1) / kTileK) * (int64_t)kTileRows * kTileK;
}
// Writes the tiled copy of E weight matrices (each b_rows x K row-major,
// n_out output columns; SwiGLU: gate rows then up rows at f_split).
hipError_t launch_tile_weights(hipStream_t s, const void* src, void* dst, int64_t E,
                               int64_t b_rows, int64_t n_out, int64_t K, bool swiglu);

// m-tiles per group of the tile order for a grouped GEMM: about the m-tiles
// one expert spans, so that the workgroups one XCD runs together share that
// expert's weight tiles and rows in its L2; one for a grouped down
// projection (`down`, groups > 1), whose groups are dealt to the XCDs.
// `request` (1..16) overrides the choice.
int gemm_group_m(int64_t rows, int64_t groups, int bm, int request = 0, bool down = false);
// Columns of the EPI_DH_* partial-dot buffer (part_ld) for a GEMM of N
// output columns on the tile height bm.
int gemm_part_cols(int bm, int64_t N);
// Workgroup order (GemmArgs::xcd_mode) of a grouped or dense up or down
// projection; one_group: a grouped GEMM whose rows all belong to one group.
// `request` (moe_desc.tile_order: 1..3) overrides the choice.
int gemm_xcd_mode(bool grouped, bool down, bool one_group = false, int request = 0);

}  // namespace moe

// Host-side launchers (defined in the .hip files, called by the ABI layer).
namespace moe {
hipError_t launch_route(hipStream_t s, int dtype, int scorer, const void* x, const float* W_r,
                        const float* bias, int32_t* idx, float* w, int64_t T, int64_t D,
                        int64_t M, int k, int renorm, float alpha, float eps, int n_group,
                        int topk_group, void* ws);
// Router workspace (bytes) and its K-split count; the bf16 router leaves
// the fp32 logits L[T][M] at route_logits_offset() bytes into it.
size_t route_workspace(int dtype, int64_t T, int64_t D, int64_t M);
size_t route_logits_offset(int dtype, int64_t T, int64_t D, int64_t M);
int route_ksplit(int64_t T, int64_t D, int64_t M);
hipError_t launch_perm_count(hipStream_t s, const int32_t* idx, int32_t* hist, int64_t T, int k,
                             int64_t M);
hipError_t launch_perm_scan(hipStream_t s, int32_t* hist, int64_t nblk, int64_t T, int k,
                            int64_t M, int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                            int32_t* sorted_slot);
hipError_t launch_perm_scatter(hipStream_t s, const int32_t* idx, const int32_t* hist,
                               const int32_t* offsets, int64_t T, int k, int64_t M,
                               int32_t* sorted_token, int32_t* sorted_slot, int32_t* slot_row);
// Up to two tile tables built by one launch (table y uses bm[y]).
struct TileTables {
    int bm[2];
    int max_tiles[2];
    int32_t* tiles[2];
};
// The tile tables, plus row_scale[r] = w[sorted_slot[r]] (0 for an unused
// row) for the S sorted rows, in one launch.  With extra > 0 the tables get
// one more group, index M, of `extra` rows starting at offsets[M] (= S):
// the kernel writes offsets[M + 1] = offsets[M] + extra, and for those rows
// row_scale = 1 and sorted_token[S + t] = t (every token once, in order).
hipError_t launch_tile_table(hipStream_t s, int32_t* offsets, int64_t M, const TileTables& tt,
                             int count, const int32_t* sorted_slot, const float* w, int64_t S,
                             float* row_scale, int64_t extra, int32_t* sorted_token);
// Count, scan and scatter in one workgroup for T <= kSmallT tokens; with
// ntables > 0 the same launch also does launch_tile_table's work (tables
// tt, row scales from w, `extra` rows of group M), saving that launch.
constexpr int64_t kSmallT = 1024;
hipError_t launch_perm_small(hipStream_t s, const int32_t* idx, int64_t T, int k, int64_t M,
                             int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                             int32_t* sorted_slot, int32_t* slot_row,
                             const TileTables* tt = nullptr, int ntables = 0,
                             const float* w = nullptr, float* row_scale = nullptr,
                             int64_t extra = 0);
hipError_t launch_wgrad(hipStream_t s, const GemmArgs& g);
hipError_t launch_gemm(hipStream_t s, int dtype, int bm, int epi, const GemmArgs& g,
                       int64_t m_tiles);
hipError_t launch_combine(hipStream_t s, int out_dtype, const float* O, const int32_t* slot_row,
                          const float* Ysh, void* y, int64_t T, int k, int64_t D);
// The combine over compact rows (fp16 values O16 with exponents Oexp, as the
// compact EPI_DOWN_SCALED epilogue writes them); same order and rounding of
// the fp32 sum as launch_combine.  The shared rows are fp32 (Ysh) or, with
// Ysh16 non-null, compact in the same format (values Ysh16, exponents
// YshExp, one row per token).
hipError_t launch_combine_compact(hipStream_t s, int out_dtype, const void* O16,
                                  const int8_t* Oexp, const int32_t* slot_row, const float* Ysh,
                                  const void* Ysh16, const int8_t* YshExp, void* y, int64_t T,
                                  int k, int64_t D);

// Backward (backward.hip).
hipError_t launch_transpose(hipStream_t s, const void* src, int64_t ld_src, int64_t src_rows,
                            int64_t src_bstride, const int32_t* idx1, const int32_t* idx2,
                            const float* scale, int64_t C, int64_t P, void* out, int64_t ld_out,
                            int64_t out_bstride, int batches);
hipError_t launch_pad_layout(hipStream_t s, const int32_t* offsets, int64_t M,
                             const int32_t* sorted_token, int64_t P, int32_t* poff,
                             int32_t* pad_row, int32_t* pad_tok);
hipError_t launch_router_backward(hipStream_t s, const float* L, const int32_t* idx,
                                  const float* w, const int32_t* slot_row, const float* part,
                                  int part_ld, const void* b2, const void* dy, int64_t D,
                                  int64_t T, int64_t M, int k, int scorer, int renorm,
                                  float alpha, float eps, float* dl, float* gate);
hipError_t launch_bwd_combine(hipStream_t s, const float* dXs, const int32_t* slot_row,
                              const float* dXsh, const float* dl, const int32_t* idx,
                              const float* W_r, int64_t T, int k, int64_t M, int64_t D,
                              int sparse_dl, float* dx);
hipError_t launch_split_transpose_dl(hipStream_t s, const float* dl, int64_t T, int64_t M,
                                     int64_t Tp, void* out);
hipError_t launch_sum3(hipStream_t s, const float* a, const float* b, const float* c, int64_t n,
                       float* out);
hipError_t launch_seg_colsum(hipStream_t s, const void* src, int64_t ld, const int32_t* offsets,
                             const int32_t* gather, const float* row_scale, int64_t M, int64_t C,
                             float* out);
// partial: ceil(T / 256) x M floats of scratch
hipError_t launch_load_stats(hipStream_t s, const float* gate, int64_t T, int64_t M,
                             const int32_t* counts, float* partial, int32_t* count_out,
                             float* score);
hipError_t launch_fill_zero(hipStream_t s, float* p, int64_t n);

// Rows per m-tile of a GEMM for a dtype, given its total rows, the number of
// groups (experts) sharing them, whether it is a down projection and the
// rows of its weight matrix (output columns, both halves for SwiGLU).
// `request` (64, 128, 160 or 256; moe_desc.tile_rows) overrides the choice.
int gemm_block_m(int dtype, int64_t rows, int64_t groups, bool down, int64_t b_rows,
                 int request = 0);
// Token block of the permute kernels.
constexpr int kPermBlock = 256;
}  // namespace moe
