// Router: logits, scores, top-k selection and weights for every token.
//
// Definition (GLaM study note, "Sparse MoE Layer": r = softmax(W_r x),
// S = TopK(r, k), normalised gate weights; "Shared Expert" GLM-4.5 note,
// "How it works": sigmoid scores, correction bias that only enters the
// selection, renormalisation by the selected scores' sum plus eps, routed
// scaling factor alpha).
//
// bf16 x (prefill / decode layers): a block of 32 tokens x all experts is a
// small GEMM on bf16 MFMA.  W_r is fp32, so each weight is split exactly
// into three bf16 parts (w = hi + mid + lo, by truncation); x is already
// bf16, so every partial product is exact and the logits carry fp32
// accumulation error only, far below the 1e-6 selection-score gap that
// decides ties.  fp32 x (the tiny fp32 layer): one wave per token with fp64
// dot products.  Both paths leave fp32 logits in LDS and share one
// wavefront top-k epilogue.
#include "common.hpp"

#include <math.h>

namespace moe {
namespace {

constexpr int kRouteTB = 32;            // tokens per workgroup (MFMA path)
constexpr int kMaxLanesJ = 1024 / 64;   // expert registers per lane

// Split 8 fp32 values into three bf16x8 vectors whose sum is exact.
__device__ __forceinline__ void split3(const float* v, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t u = __float_as_uint(v[i]);
        uint32_t uh = u & 0xffff0000u;
        float r1 = v[i] - __uint_as_float(uh);
        uint32_t um = __float_as_uint(r1) & 0xffff0000u;
        float r2 = r1 - __uint_as_float(um);
        h[i] = uh >> 16;
        m[i] = um >> 16;
        l[i] = __float_as_uint(r2) >> 16;   // r2 has at most 8 significant bits
    }
    u32x4 ph, pm, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ph[i] = h[2 * i] | (h[2 * i + 1] << 16);
        pm[i] = m[2 * i] | (m[2 * i + 1] << 16);
        pl[i] = l[2 * i] | (l[2 * i + 1] << 16);
    }
    hi = __builtin_bit_cast(bf16x8, ph);
    mid = __builtin_bit_cast(bf16x8, pm);
    lo = __builtin_bit_cast(bf16x8, pl);
}

__device__ __forceinline__ bool better(double av, int ai, double bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

// One wave: top-k of one token from its fp32 logits `lrow[0..M)`.
// Writes k (expert, weight) pairs in ascending expert order.
__device__ void topk_epilogue(const float* lrow, int M, int k, int scorer, const float* bias,
                              int renorm, double alpha, double eps, int32_t* idx_t, float* w_t) {
    const int lane = threadIdx.x & 63;
    const int nj = (M + 63) >> 6;
    double sel[kMaxLanesJ];
    double mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxLanesJ; ++j) {
        const int e = lane + 64 * j;
        sel[j] = -INFINITY;
        if (j < nj && e < M) {
            const double l = (double)lrow[e];
            if (scorer == 0) {
                sel[j] = l;   // softmax is increasing in the logit
                mx = fmax(mx, l);
            } else {
                const double s = 1.0 / (1.0 + exp(-l));
                sel[j] = s + (bias ? (double)bias[e] : 0.0);
            }
            // a NaN score ranks last, so k valid experts are always chosen
            if (sel[j] != sel[j]) sel[j] = -INFINITY;
        }
    }
    double Z = 0.0;
    if (scorer == 0) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
#pragma unroll
        for (int j = 0; j < kMaxLanesJ; ++j) {
            const int e = lane + 64 * j;
            if (j < nj && e < M) Z += exp((double)lrow[e] - mx);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) Z += __shfl_xor(Z, off);
    }

    uint32_t taken = 0;
    int my_e = 0;
    for (int r = 0; r < k; ++r) {
        double bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < kMaxLanesJ; ++j) {
            const int e = lane + 64 * j;
            if (j < nj && e < M && !((taken >> j) & 1u) && better(sel[j], e, bv, bi)) {
                bv = sel[j];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const double ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (lane == r) my_e = bi;
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }

    // gate value of this lane's chosen expert
    double g = 0.0;
    if (lane < k) {
        const double l = (double)lrow[my_e];
        g = (scorer == 0) ? exp(l - mx) / Z : 1.0 / (1.0 + exp(-l));
    }
    double gsum = g;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) gsum += __shfl_xor(gsum, off);
    int rank = 0;
    for (int i = 0; i < k; ++i) {
        const int ei = __shfl(my_e, i);
        rank += (ei < my_e) ? 1 : 0;
    }
    if (lane < k) {
        const double wv = renorm ? alpha * g / (gsum + eps) : alpha * g;
        idx_t[rank] = my_e;
        w_t[rank] = (float)wv;
    }
}

// MFMA router for bf16 x.  Wave w owns expert fragments w, w+4, ... (16
// experts each) for both 16-token groups of the block.
template <int FPW>
__global__ __launch_bounds__(256) void route_bf16_mfma(
    const bf16_t* __restrict__ x, const float* __restrict__ W_r, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ w, int T, int D, int M, int k, int scorer,
    int renorm, float alpha, float eps) {
    extern __shared__ float s_logit[];   // [kRouteTB][ldl]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kRouteTB;
    const int NF = (M + 15) >> 4;
    const int ldl = NF * 16;
    const int r16 = lane & 15;
    const int kq = lane >> 4;

    floatx4 acc[2][FPW];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < FPW; ++i) acc[g][i] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int ta0 = t0 + r16, ta1 = t0 + 16 + r16;
    const bool va0 = ta0 < T, va1 = ta1 < T;
    const bf16_t* xa0 = x + (int64_t)(va0 ? ta0 : 0) * D;
    const bf16_t* xa1 = x + (int64_t)(va1 ? ta1 : 0) * D;

    for (int k0 = 0; k0 < D; k0 += 32) {
        const int kk = k0 + 8 * kq;
        const bool kv = kk < D;
        u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 a0u = (va0 && kv) ? *reinterpret_cast<const u32x4*>(xa0 + kk) : z;
        const u32x4 a1u = (va1 && kv) ? *reinterpret_cast<const u32x4*>(xa1 + kk) : z;
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, a0u);
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, a1u);
#pragma unroll
        for (int i = 0; i < FPW; ++i) {
            const int fr = wave + 4 * i;
            if (fr < NF) {
                const int e = fr * 16 + r16;
                float wv[8];
                if (e < M && kv) {
                    const float4* p = reinterpret_cast<const float4*>(W_r + (int64_t)e * D + kk);
                    const float4 p0 = p[0], p1 = p[1];
                    wv[0] = p0.x; wv[1] = p0.y; wv[2] = p0.z; wv[3] = p0.w;
                    wv[4] = p1.x; wv[5] = p1.y; wv[6] = p1.z; wv[7] = p1.w;
                } else {
#pragma unroll
                    for (int q = 0; q < 8; ++q) wv[q] = 0.f;
                }
                bf16x8 bh, bm, bl;
                split3(wv, bh, bm, bl);
                acc[0][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bl, acc[0][i], 0, 0, 0);
                acc[0][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bm, acc[0][i], 0, 0, 0);
                acc[0][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bh, acc[0][i], 0, 0, 0);
                acc[1][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bl, acc[1][i], 0, 0, 0);
                acc[1][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bm, acc[1][i], 0, 0, 0);
                acc[1][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bh, acc[1][i], 0, 0, 0);
            }
        }
    }
    // MFMA 16x16 result: lane holds column (expert) lane%16, rows (tokens)
    // 4*(lane/16) + q.
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < FPW; ++i) {
            const int fr = wave + 4 * i;
            if (fr < NF) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int tl = g * 16 + 4 * kq + q;
                    s_logit[tl * ldl + fr * 16 + r16] = acc[g][i][q];
                }
            }
        }
    __syncthreads();
    for (int tl = wave; tl < kRouteTB; tl += 4) {
        const int t = t0 + tl;
        if (t >= T) break;
        topk_epilogue(s_logit + tl * ldl, M, k, scorer, bias, renorm, (double)alpha, (double)eps,
                      idx + (int64_t)t * k, w + (int64_t)t * k);
    }
}

// Generic router: one wave per token, fp64 dot products (fp32 or bf16 x).
template <typename XT>
__global__ __launch_bounds__(256) void route_simple(
    const XT* __restrict__ x, const float* __restrict__ W_r, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ w, int T, int D, int M, int k, int scorer,
    int renorm, float alpha, float eps) {
    extern __shared__ float s_logit[];   // [4][M]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;   // whole wave leaves; no block barrier follows
    float* lrow = s_logit + wave * M;
    const XT* xr = x + (int64_t)t * D;
    for (int e = lane; e < M; e += 64) {
        const float* wr = W_r + (int64_t)e * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) {
            double xv;
            if constexpr (sizeof(XT) == 4) xv = (double)xr[d];
            else xv = (double)bf16_to_f32(xr[d]);
            acc += xv * (double)wr[d];
        }
        lrow[e] = (float)acc;
    }
    // the wave's own LDS row: make the writes visible across lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    topk_epilogue(lrow, M, k, scorer, bias, renorm, (double)alpha, (double)eps,
                  idx + (int64_t)t * k, w + (int64_t)t * k);
}

template <int FPW>
hipError_t launch_mfma(hipStream_t s, const void* x, const float* W_r, const float* bias,
                       int32_t* idx, float* w, int T, int D, int M, int k, int scorer, int renorm,
                       float alpha, float eps) {
    const int NF = (M + 15) / 16;
    const size_t lds = (size_t)kRouteTB * NF * 16 * sizeof(float);
    dim3 grid((T + kRouteTB - 1) / kRouteTB);
    hipLaunchKernelGGL(route_bf16_mfma<FPW>, grid, dim3(256), lds, s,
                       static_cast<const bf16_t*>(x), W_r, bias, idx, w, T, D, M, k, scorer,
                       renorm, alpha, eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(hipStream_t s, int dtype, int scorer, const void* x, const float* W_r,
                        const float* bias, int32_t* idx, float* w, int64_t T, int64_t D,
                        int64_t M, int k, int renorm, float alpha, float eps) {
    if (T == 0) return hipSuccess;
    const float* b = (scorer == 1) ? bias : nullptr;
    const int NF = (int)((M + 15) / 16);
    if (dtype == 1 && M <= 512) {
        const int fpw = (NF + 3) / 4;
        if (fpw <= 1) return launch_mfma<1>(s, x, W_r, b, idx, w, T, D, M, k, scorer, renorm, alpha, eps);
        if (fpw <= 2) return launch_mfma<2>(s, x, W_r, b, idx, w, T, D, M, k, scorer, renorm, alpha, eps);
        if (fpw <= 4) return launch_mfma<4>(s, x, W_r, b, idx, w, T, D, M, k, scorer, renorm, alpha, eps);
        return launch_mfma<8>(s, x, W_r, b, idx, w, T, D, M, k, scorer, renorm, alpha, eps);
    }
    dim3 grid((unsigned)((T + 3) / 4));
    const size_t lds = 4 * (size_t)M * sizeof(float);
    if (dtype == 0)
        hipLaunchKernelGGL(route_simple<float>, grid, dim3(256), lds, s,
                           static_cast<const float*>(x), W_r, b, idx, w, (int)T, (int)D, (int)M,
                           k, scorer, renorm, alpha, eps);
    else
        hipLaunchKernelGGL(route_simple<bf16_t>, grid, dim3(256), lds, s,
                           static_cast<const bf16_t*>(x), W_r, b, idx, w, (int)T, (int)D, (int)M,
                           k, scorer, renorm, alpha, eps);
    return hipGetLastError();
}

}  // namespace moe
