// Layer backward: the kernels around the expert GEMMs (which run on the
// forward's grouped GEMM with the backward epilogues and its K-grouped mode).
//
// What is differentiated is the forward definition (GLaM study note,
// "Sparse MoE Layer", and the GLM-4.5 note's "How it works"): y = sum over
// the selected experts of w_j E_j(x) + E_sh(x), with w the renormalised,
// alpha-scaled gate values.  The selection and the correction bias are
// piecewise constant and pass no gradient; dy reaches the router logits
// through the weights only.  The training objective producing dy is the
// GLaM note's causal LM loss.
//
//  - pad layout: each expert's sorted rows padded to a multiple of 64 so
//    the weight-gradient GEMMs contract over whole K stages per expert;
//  - transpose: row-major [rows, C] -> [C, positions], optionally gathered,
//    scaled and zero-padded (the weight-gradient operands; the input-
//    gradient GEMMs read the weights in place, as [K, N] B operands);
//  - router backward: per token, the weights' gradient dw_j = dy . E_j(x)
//    (summed from the GEMM epilogue's per-tile dots) through the
//    renormalisation and the gate values to the logits;
//  - combine: dx = sum of the token's expert-row input gradients + the
//    shared expert's + the router's W_r^T dl;
//  - reductions: bias gradients, load statistics, split-plane sums.
#include "common.hpp"

#include <math.h>

namespace moe {
namespace {

// Transpose block tile: 64 positions x 256 columns, one wave per 64 x 64.
constexpr int kTP = 64, kTC = 256;

// out[b][c * ld_out + p] = scale(r1) * src[b][r2 * ld_src + c] for p < P,
// c < C, where r1 = idx1 ? idx1[p] : p, r2 = idx2 ? idx2[r1] : r1; a position
// whose r1 is negative or >= src_rows is zero.  Batch b = blockIdx.z with the
// given strides.  C and P multiples of 8, rows 16-byte aligned.  Each lane
// moves one 8 x 8 block through its registers: eight 16-byte loads (8
// positions, 8 consecutive columns each), the 16-bit halves regrouped, and
// eight 16-byte stores (8 columns, 8 consecutive positions each).  The 8
// lanes of a column block read 128 contiguous bytes of each source row; the
// 8 lanes of a position block write 128 contiguous bytes of each output row.
// The transposes of a layer move a read and a write stream at about 5 TB/s
// (GLM-4.5 prefill: 2.5 GB each way in 1.0 ms); a 64 x 64 LDS tile with
// 2-byte accesses ran 3-15% slower, and 256 positions x 64 columns per block
// (512-byte output runs) no faster.
__global__ __launch_bounds__(256) void transpose_bf16(
    const bf16_t* __restrict__ src, int64_t ld_src, int64_t src_rows, int64_t src_bstride,
    const int32_t* __restrict__ idx1, const int32_t* __restrict__ idx2,
    const float* __restrict__ scale, int64_t C, int64_t P, bf16_t* __restrict__ out,
    int64_t ld_out, int64_t out_bstride) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t p0 = (int64_t)blockIdx.x * kTP + (lane & 7) * 8;
    const int64_t c0 = (int64_t)blockIdx.y * kTC + wave * 64 + (lane >> 3) * 8;
    if (p0 >= P || c0 >= C) return;   // P, C multiples of 8: the block is wholly inside
    src += (int64_t)blockIdx.z * src_bstride;
    out += (int64_t)blockIdx.z * out_bstride;
    u32x4 r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t p = p0 + i;
        u32x4 v = {0u, 0u, 0u, 0u};
        const int64_t r1 = idx1 ? (int64_t)idx1[p] : p;
        if (r1 >= 0 && r1 < src_rows) {
            const int64_t r2 = idx2 ? (int64_t)idx2[r1] : r1;
            v = *reinterpret_cast<const u32x4*>(src + r2 * ld_src + c0);
            if (scale) {
                const float sc = scale[r1];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float lo = bf16_to_f32((bf16_t)(v[q] & 0xffffu)) * sc;
                    const float hi = bf16_to_f32((bf16_t)(v[q] >> 16)) * sc;
                    v[q] = pack_bf16x2(lo, hi);
                }
            }
        }
        r[i] = v;
    }
    // output column j: element j of rows 0..7 (row i holds element j in
    // word j / 2, low half for even j)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t a = r[2 * q][j >> 1], b = r[2 * q + 1][j >> 1];
            o[q] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        *reinterpret_cast<u32x4*>(out + (c0 + j) * ld_out + p0) = o;
    }
}

// poff[e] = sum over e' < e of round_up(count[e'], 64), poff[M] = total
// (one workgroup, M <= 1024).
__global__ __launch_bounds__(1024) void pad_offsets(const int32_t* __restrict__ offsets, int M,
                                                    int32_t* __restrict__ poff) {
    __shared__ int32_t s_warp[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t v = 0;
    if (tid < M) v = ((offsets[tid + 1] - offsets[tid] + 63) / 64) * 64;
    int32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_warp[wv] = incl;
    __syncthreads();
    int32_t base = 0;
    for (int i = 0; i < wv; ++i) base += s_warp[i];
    incl += base;
    if (tid < M) poff[tid] = incl - v;
    if (tid == M - 1) poff[M] = incl;
}

// pad_row[p] = the sorted row at padded position p, or -1 (padding and
// positions past poff[M]); pad_tok[p] = its token, or -1.
__global__ __launch_bounds__(256) void pad_rows(const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ poff, int M,
                                                const int32_t* __restrict__ sorted_token,
                                                int64_t P, int32_t* __restrict__ pad_row,
                                                int32_t* __restrict__ pad_tok) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= P) return;
    int32_t r = -1;
    if (p < poff[M]) {
        int lo = 0, hi = M;   // largest e with poff[e] <= p
        while (hi - lo > 1) {
            const int mid = (lo + hi) / 2;
            if (poff[mid] <= p) lo = mid;
            else hi = mid;
        }
        const int64_t rr = offsets[lo] + (p - poff[lo]);
        if (rr < offsets[lo + 1]) r = (int32_t)rr;
    }
    pad_row[p] = r;
    pad_tok[p] = r >= 0 ? sorted_token[r] : -1;
}

// One wave per token: dw_j = sum over the GEMM's partial dots of the slot's
// row (fixed order); dg over the selected experts through the
// renormalisation; dl through softmax or sigmoid (fp64); gate values out.
__global__ __launch_bounds__(256) void router_backward(
    const float* __restrict__ L, const int32_t* __restrict__ idx, const float* __restrict__ w,
    const int32_t* __restrict__ slot_row, const float* __restrict__ part, int part_ld,
    const bf16_t* __restrict__ b2, const bf16_t* __restrict__ dy, int D, int T, int M, int k,
    int scorer, int renorm, float alpha, float eps, float* __restrict__ dl,
    float* __restrict__ gate) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;   // whole wave
    const float* lt = L + (int64_t)t * M;
    double mx = -INFINITY;
    if (scorer == 0)
        for (int e = lane; e < M; e += 64) mx = fmax(mx, (double)lt[e]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
    double Z = 0.0;
    if (scorer == 0)
        for (int e = lane; e < M; e += 64) Z += exp((double)lt[e] - mx);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) Z += __shfl_xor(Z, off);
    // lane j < k: its slot's expert, gate value and dw
    int my_e = -1;
    double my_g = 0.0, my_dw = 0.0;
    if (lane < k) {
        my_e = idx[(int64_t)t * k + lane];
        if (my_e >= 0 && my_e < M) {
            const double l = (double)lt[my_e];
            my_g = scorer == 0 ? exp(l - mx) / Z : 1.0 / (1.0 + exp(-l));
            const int32_t r = slot_row[(int64_t)t * k + lane];
            double s = 0.0;
            if (r >= 0)
                for (int q = 0; q < part_ld; ++q) s += (double)part[(int64_t)r * part_ld + q];
            my_dw = s;
        } else {
            my_e = -1;
        }
    }
    // with output biases the expert output is W2 h + b2: dw_j gains dy . b2[e_j]
    if (b2) {
        for (int j = 0; j < k; ++j) {
            const int ej = __shfl(my_e, j);
            double s = 0.0;
            if (ej >= 0)
                for (int dd = lane; dd < D; dd += 64)
                    s += (double)bf16_to_f32(dy[(int64_t)t * D + dd]) *
                         (double)bf16_to_f32(b2[(int64_t)ej * D + dd]);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
            if (lane == j) my_dw += s;
        }
    }
    double Gs = my_g, S = my_dw * my_g;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        Gs += __shfl_xor(Gs, off);
        S += __shfl_xor(S, off);
    }
    double my_dg = 0.0;
    if (my_e >= 0) {
        if (renorm) {
            const double den = Gs + (double)eps;
            my_dg = (double)alpha * (my_dw / den - S / (den * den));
        } else {
            my_dg = (double)alpha * my_dw;
        }
    }
    // softmax: dl_m = g_m (dg_m - sum_i dg_i g_i); sigmoid: dg g (1 - g)
    double sdg = my_dg * my_g;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sdg += __shfl_xor(sdg, off);
    // every lane gets all slots' (expert, dg) while the whole wave is active
    int ej[kMaxK];
    double dgj[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        ej[j] = __shfl(my_e, j);
        dgj[j] = __shfl(my_dg, j);
    }
    for (int e = lane; e < M; e += 64) {
        const double l = (double)lt[e];
        const double ge = scorer == 0 ? exp(l - mx) / Z : 1.0 / (1.0 + exp(-l));
        double dge = 0.0;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k && ej[j] == e) dge = dgj[j];
        const double d = scorer == 0 ? ge * (dge - sdg) : dge * ge * (1.0 - ge);
        dl[(int64_t)t * M + e] = (float)d;
        gate[(int64_t)t * M + e] = (float)ge;
    }
}

// dx[t, d] = sum_j dXs[slot_row[t k + j], d] + dXsh[t, d] + sum_m dl[t, m]
// W_r[m, d] (over the selected experts only for the sigmoid router, whose dl
// is zero elsewhere).  One wave per (token, 256 columns), fp32, fixed order.
__global__ __launch_bounds__(256) void bwd_combine(
    const float* __restrict__ dXs, const int32_t* __restrict__ slot_row,
    const float* __restrict__ dXsh, const float* __restrict__ dl, const int32_t* __restrict__ idx,
    const float* __restrict__ W_r, int T, int k, int M, int D, int chunks, int sparse_dl,
    float* __restrict__ dx) {
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = (int)(wid / chunks);
    if (t >= T) return;
    const int d0 = (int)(wid % chunks) * 256 + lane * 4;
    if (d0 >= D) return;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int32_t r = slot_row[(int64_t)t * k + j];
        if (r < 0) continue;
        const float4 v = *reinterpret_cast<const float4*>(dXs + (int64_t)r * D + d0);
        acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
    }
    if (dXsh) {
        const float4 v = *reinterpret_cast<const float4*>(dXsh + (int64_t)t * D + d0);
        acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
    }
    const float* dlt = dl + (int64_t)t * M;
    const int n = sparse_dl ? k : M;
    for (int j = 0; j < n; ++j) {
        const int m = sparse_dl ? idx[(int64_t)t * k + j] : j;
        if (m < 0 || m >= M) continue;
        const float g = dlt[m];
        const float4 v = *reinterpret_cast<const float4*>(W_r + (int64_t)m * D + d0);
        acc[0] += g * v.x; acc[1] += g * v.y; acc[2] += g * v.z; acc[3] += g * v.w;
    }
    *reinterpret_cast<float4*>(dx + (int64_t)t * D + d0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// dlT3[p][t] for p < 3M: the three bf16 planes (hi, mid, lo by truncation)
// whose sum is dl[t][m] exactly, transposed, zero past T (t < Tp).
__global__ __launch_bounds__(256) void split_transpose_dl(const float* __restrict__ dl, int T,
                                                          int M, int64_t Tp,
                                                          bf16_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * Tp) return;
    const int m = (int)(i / Tp);
    const int64_t t = i % Tp;
    const float v = t < T ? dl[t * M + m] : 0.f;
    const uint32_t u = __float_as_uint(v), uh = u & 0xffff0000u;
    const float r1 = v - __uint_as_float(uh);
    const uint32_t um = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(um);
    out[(int64_t)m * Tp + t] = (bf16_t)(uh >> 16);
    out[((int64_t)M + m) * Tp + t] = (bf16_t)(um >> 16);
    out[((int64_t)2 * M + m) * Tp + t] = (bf16_t)(__float_as_uint(r2) >> 16);
}

// out[i] = a[i] + b[i] + c[i] (the three planes of the router's weight
// gradient, summed in fixed order).
__global__ __launch_bounds__(256) void sum3(const float* __restrict__ a,
                                            const float* __restrict__ b,
                                            const float* __restrict__ c, int64_t n,
                                            float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = a[i] + (b[i] + c[i]);
}

// Segmented column sums: out[e][c] = sum over rows r in [offsets[e],
// offsets[e+1]) of scale(r) * src[row(r)][c] (src bf16; row(r) = gather[r]
// or r; scale = row_scale[r] or 1), in row order.  Bias gradients.
__global__ __launch_bounds__(256) void seg_colsum(const bf16_t* __restrict__ src, int64_t ld,
                                                  const int32_t* __restrict__ offsets,
                                                  const int32_t* __restrict__ gather,
                                                  const float* __restrict__ row_scale, int M,
                                                  int64_t C, float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * C) return;
    const int e = (int)(i / C);
    const int64_t c = i % C;
    float acc = 0.f;
    for (int32_t r = offsets[e]; r < offsets[e + 1]; ++r) {
        const int64_t row = gather ? gather[r] : r;
        const float v = bf16_to_f32(src[row * ld + c]);
        acc += row_scale ? row_scale[r] * v : v;
    }
    out[i] = acc;
}

// Load statistics, deterministically in two passes: partial[c][e] = sum of
// gate[t][e] over token chunk c of 256 (four 64-token runs added in order),
// then score[e] = sum over chunks in order; count[e] copied from the
// dispatch counts.
__global__ __launch_bounds__(256) void load_partial(const float* __restrict__ gate, int T, int M,
                                                    float* __restrict__ partial) {
    __shared__ float s_p[4][64];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int e = blockIdx.y * 64 + tx;
    const int t0 = blockIdx.x * 256 + ty * 64;
    float acc = 0.f;
    if (e < M)
        for (int i = 0; i < 64 && t0 + i < T; ++i) acc += gate[(int64_t)(t0 + i) * M + e];
    s_p[ty][tx] = acc;
    __syncthreads();
    if (ty == 0 && e < M)
        partial[(int64_t)blockIdx.x * M + e] = ((s_p[0][tx] + s_p[1][tx]) + s_p[2][tx]) + s_p[3][tx];
}

__global__ __launch_bounds__(256) void load_stats(const float* __restrict__ partial, int chunks,
                                                  int M, const int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ count_out,
                                                  float* __restrict__ score) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= M) return;
    float acc = 0.f;
    for (int c = 0; c < chunks; ++c) acc += partial[(int64_t)c * M + e];
    score[e] = acc;
    count_out[e] = counts[e];
}

__global__ __launch_bounds__(256) void fill_zero(float* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t launch_fill_zero(hipStream_t s, float* p, int64_t n) {
    if (!p || n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_transpose(hipStream_t s, const void* src, int64_t ld_src, int64_t src_rows,
                            int64_t src_bstride, const int32_t* idx1, const int32_t* idx2,
                            const float* scale, int64_t C, int64_t P, void* out, int64_t ld_out,
                            int64_t out_bstride, int batches) {
    if (C <= 0 || P <= 0 || batches <= 0) return hipSuccess;
    if (C % 8 || P % 8 || ld_src % 8 || ld_out % 8) return hipErrorInvalidValue;
    dim3 grid((unsigned)((P + kTP - 1) / kTP), (unsigned)((C + kTC - 1) / kTC), (unsigned)batches);
    hipLaunchKernelGGL(transpose_bf16, grid, dim3(256), 0, s, static_cast<const bf16_t*>(src),
                       ld_src, src_rows, src_bstride, idx1, idx2, scale, C, P,
                       static_cast<bf16_t*>(out), ld_out, out_bstride);
    return hipGetLastError();
}

hipError_t launch_pad_layout(hipStream_t s, const int32_t* offsets, int64_t M,
                             const int32_t* sorted_token, int64_t P, int32_t* poff,
                             int32_t* pad_row, int32_t* pad_tok) {
    if (M > 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pad_offsets, dim3(1), dim3(1024), 0, s, offsets, (int)M, poff);
    hipLaunchKernelGGL(pad_rows, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, s, offsets, poff,
                       (int)M, sorted_token, P, pad_row, pad_tok);
    return hipGetLastError();
}

hipError_t launch_router_backward(hipStream_t s, const float* L, const int32_t* idx,
                                  const float* w, const int32_t* slot_row, const float* part,
                                  int part_ld, const void* b2, const void* dy, int64_t D,
                                  int64_t T, int64_t M, int k, int scorer, int renorm,
                                  float alpha, float eps, float* dl, float* gate) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(router_backward, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, L, idx, w,
                       slot_row, part, part_ld, static_cast<const bf16_t*>(b2),
                       static_cast<const bf16_t*>(dy), (int)D, (int)T, (int)M, k, scorer, renorm,
                       alpha, eps, dl, gate);
    return hipGetLastError();
}

hipError_t launch_bwd_combine(hipStream_t s, const float* dXs, const int32_t* slot_row,
                              const float* dXsh, const float* dl, const int32_t* idx,
                              const float* W_r, int64_t T, int k, int64_t M, int64_t D,
                              int sparse_dl, float* dx) {
    if (T == 0) return hipSuccess;
    if (D % 4) return hipErrorInvalidValue;
    const int chunks = (int)((D + 255) / 256);
    hipLaunchKernelGGL(bwd_combine, dim3((unsigned)((T * chunks + 3) / 4)), dim3(256), 0, s, dXs,
                       slot_row, dXsh, dl, idx, W_r, (int)T, k, (int)M, (int)D, chunks, sparse_dl,
                       dx);
    return hipGetLastError();
}

hipError_t launch_split_transpose_dl(hipStream_t s, const float* dl, int64_t T, int64_t M,
                                     int64_t Tp, void* out) {
    hipLaunchKernelGGL(split_transpose_dl, dim3((unsigned)((M * Tp + 255) / 256)), dim3(256), 0, s,
                       dl, (int)T, (int)M, Tp, static_cast<bf16_t*>(out));
    return hipGetLastError();
}

hipError_t launch_sum3(hipStream_t s, const float* a, const float* b, const float* c, int64_t n,
                       float* out) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(sum3, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, b, c, n, out);
    return hipGetLastError();
}

hipError_t launch_seg_colsum(hipStream_t s, const void* src, int64_t ld, const int32_t* offsets,
                             const int32_t* gather, const float* row_scale, int64_t M, int64_t C,
                             float* out) {
    hipLaunchKernelGGL(seg_colsum, dim3((unsigned)((M * C + 255) / 256)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(src), ld, offsets, gather, row_scale, (int)M, C,
                       out);
    return hipGetLastError();
}

hipError_t launch_load_stats(hipStream_t s, const float* gate, int64_t T, int64_t M,
                             const int32_t* counts, float* partial, int32_t* count_out,
                             float* score) {
    const int chunks = (int)((T + 255) / 256);
    hipLaunchKernelGGL(load_partial, dim3((unsigned)chunks, (unsigned)((M + 63) / 64)), dim3(256),
                       0, s, gate, (int)T, (int)M, partial);
    hipLaunchKernelGGL(load_stats, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, partial,
                       chunks, (int)M, counts, count_out, score);
    return hipGetLastError();
}

}  // namespace moe
