// Router: logits, scores, top-k selection and weights for every token.
//
// Definition (GLaM study note, "Sparse MoE Layer": r = softmax(W_r x),
// S = TopK(r, k), normalised gate weights; "Shared Expert" GLM-4.5 note,
// "How it works": sigmoid scores, correction bias that only enters the
// selection, renormalisation by the selected scores' sum plus eps, routed
// scaling factor alpha).
//
// bf16 x (prefill / decode layers): the logits are a GEMM x . W_r^T on bf16
// MFMA.  W_r is fp32, so a pre-pass splits it exactly into three bf16
// planes (w = hi + mid + lo, by truncation) stacked as a [3M, D] matrix; x is
// already bf16, so every partial product is exact and the logits carry fp32
// accumulation error only, far below the 1e-6 selection-score gap that
// decides ties.  The GEMM is the expert GEMM kernel in dense mode with
// split-K (so even 64 tokens fill the GPU); the top-k kernel sums the
// planes and K chunks in fixed order.  fp32 x (the tiny fp32 layer): one wave per
// token with fp64 dot products.  Both paths share one wavefront top-k
// epilogue.
#include "common.hpp"

#include <math.h>

#include <type_traits>

namespace moe {
namespace {

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

// Wave-wide reductions without LDS.  Step S pairs every lane with one
// partner: S = 0, 1 the lanes l ^ 1 and l ^ 2 (DPP quad permutations), S = 2
// the mirror lane inside each 8-lane half row, S = 3 inside each 16-lane row
// (DPP mirrors), S = 4 and 5 the lanes l ^ 16 and l ^ 32 (v_permlane16_swap,
// v_permlane32_swap).  After steps 0..5 in order every lane has met all 64
// values.  xpair returns {own, partner} or {partner, own}; the same order in
// every register of one step, so (value, index) pairs stay together.  Every
// reduction below is symmetric in the two values (a strict total order, a
// commutative sum), so both lanes of a pair hold the same bits afterwards.
// These moves run on the VALU; the shuffles they replace were routed through
// the LDS crossbar, where they queue behind any MFMA kernel sharing the CU.
struct Pair32 {
    uint32_t a, b;
};
template <int S>
__device__ __forceinline__ Pair32 xpair(uint32_t x) {
    if constexpr (S <= 3) {
        constexpr int ctrl = S == 0 ? 0xB1 : S == 1 ? 0x4E : S == 2 ? 0x141 : 0x140;
        return {x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, ctrl, 0xF, 0xF, false)};
    } else if constexpr (S == 4) {
        const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return {p[0], p[1]};
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return {p[0], p[1]};
    }
}
template <int S>
__device__ __forceinline__ void dpair(double x, double& a, double& b) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const Pair32 lo = xpair<S>((uint32_t)u), hi = xpair<S>((uint32_t)(u >> 32));
    a = __longlong_as_double((long long)(((uint64_t)hi.a << 32) | lo.a));
    b = __longlong_as_double((long long)(((uint64_t)hi.b << 32) | lo.b));
}
template <int S>
__device__ __forceinline__ void argmax_step(double& v, int& i) {
    double va, vb;
    dpair<S>(v, va, vb);
    const Pair32 ip = xpair<S>((uint32_t)i);
    const int ia = (int)ip.a, ib = (int)ip.b;
    const bool tb = better(vb, ib, va, ia);
    v = tb ? vb : va;
    i = tb ? ib : ia;
}
// (v, i) of the best lane by `better` (larger v, then smaller i), in every lane
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
    argmax_step<0>(v, i);
    argmax_step<1>(v, i);
    argmax_step<2>(v, i);
    argmax_step<3>(v, i);
    argmax_step<4>(v, i);
    argmax_step<5>(v, i);
}
template <int S>
__device__ __forceinline__ void max_step(double& v) {
    double a, b;
    dpair<S>(v, a, b);
    v = fmax(a, b);
}
__device__ __forceinline__ double wave_max(double v) {
    max_step<0>(v);
    max_step<1>(v);
    max_step<2>(v);
    max_step<3>(v);
    max_step<4>(v);
    max_step<5>(v);
    return v;
}
template <int S>
__device__ __forceinline__ void sum_step(double& v) {
    double a, b;
    dpair<S>(v, a, b);
    v = a + b;
}
__device__ __forceinline__ double wave_sum(double v) {
    sum_step<0>(v);
    sum_step<1>(v);
    sum_step<2>(v);
    sum_step<3>(v);
    sum_step<4>(v);
    sum_step<5>(v);
    return v;
}

// One wave: top-k of one token from its fp32 logits `lrow[0..M)` (LDS or
// global; read once into registers, expert e = lane + 64 j in register j).
// Writes k (expert, weight) pairs in ascending expert order.  With
// n_group > 1 the experts form n_group contiguous groups and only the
// topk_group groups with the largest best selection score compete (the
// GLM-4.5 note's optional masking by expert group).
template <int NJ>
__device__ __forceinline__ void topk_epilogue_nj(const float* lrow, int M, int k, int scorer,
                                              const float* bias, int renorm, double alpha,
                                              double eps, int n_group, int topk_group,
                                              int32_t* idx_t, float* w_t) {
    const int lane = threadIdx.x & 63;
    double sel[NJ];
    float lj[NJ];
    double mx = -INFINITY;
    // the logit and bias loads all go out before the first score is formed
    float bj[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        bj[j] = 0.f;
        lj[j] = lrow[min(lane + 64 * j, M - 1)];   // lanes past M re-read a valid entry
    }
    if (scorer != 0 && bias) {   // uniform
#pragma unroll
        for (int j = 0; j < NJ; ++j) bj[j] = bias[min(lane + 64 * j, M - 1)];
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + 64 * j;
        sel[j] = -INFINITY;
        if (e < M) {
            const double l = (double)lj[j];
            if (scorer == 0) {
                sel[j] = l;   // softmax is increasing in the logit
                mx = fmax(mx, l);
            } else {
                const double s = 1.0 / (1.0 + exp(-l));
                sel[j] = s + (double)bj[j];
            }
            // a NaN score ranks last, so k valid experts are always chosen
            if (sel[j] != sel[j]) sel[j] = -INFINITY;
        }
    }
    double Z = 0.0;
    if (scorer == 0) {
        mx = wave_max(mx);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int e = lane + 64 * j;
            if (e < M) Z += exp((double)lj[j] - mx);
        }
        Z = wave_sum(Z);
    }

    uint32_t taken = 0;
    if (n_group > 1) {
        // lane g holds group g's score: the largest selection score in it
        const int gs = M / n_group;
        double my_gs = -INFINITY;
        for (int gi = 0; gi < n_group; ++gi) {
            double v = -INFINITY;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int e = lane + 64 * j;
                if (e < M && e / gs == gi) v = fmax(v, sel[j]);
            }
            v = wave_max(v);
            if (lane == gi) my_gs = v;
        }
        // keep the topk_group best groups (the lower group index on a tie)
        uint64_t kept = 0;
        bool mine = false;
        for (int r = 0; r < topk_group; ++r) {
            const bool cand = lane < n_group && !mine;
            double bv = cand ? my_gs : -INFINITY;
            int bi = cand ? lane : 0x7fffffff;
            wave_argmax(bv, bi);
            bi = __builtin_amdgcn_readfirstlane(bi);
            if (lane == bi) mine = true;
            kept |= 1ull << bi;
        }
        // experts of the other groups leave the selection
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int e = lane + 64 * j;
            if (e < M && !((kept >> (e / gs)) & 1ull)) taken |= 1u << j;
        }
    }
    int my_e = 0;
    float my_l = 0.f;
    for (int r = 0; r < k; ++r) {
        double bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int e = lane + 64 * j;
            if (e < M && !((taken >> j) & 1u) && better(sel[j], e, bv, bi)) {
                bv = sel[j];
                bi = e;
            }
        }
        wave_argmax(bv, bi);
        bi = __builtin_amdgcn_readfirstlane(bi);   // the same in every lane
        // the winner's logit, from its owner lane's register
        const int jw = bi >> 6;
        float lw = lj[0];
#pragma unroll
        for (int j = 1; j < NJ; ++j)
            if (j == jw) lw = lj[j];
        lw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lw), bi & 63));
        if (lane == r) {
            my_e = bi;
            my_l = lw;
        }
        if ((bi & 63) == lane) taken |= 1u << jw;
    }

    // gate value of this lane's chosen expert
    double g = 0.0;
    if (lane < k) {
        const double l = (double)my_l;
        g = (scorer == 0) ? exp(l - mx) / Z : 1.0 / (1.0 + exp(-l));
    }
    const double gsum = wave_sum(g);
    int rank = 0;
    for (int i = 0; i < k; ++i) {
        const int ei = __builtin_amdgcn_readlane(my_e, i);
        rank += (ei < my_e) ? 1 : 0;
    }
    if (lane < k) {
        const double wv = renorm ? alpha * g / (gsum + eps) : alpha * g;
        idx_t[rank] = my_e;
        w_t[rank] = (float)wv;
    }
}

// Kernels carry NJ (expert registers per lane, M <= 64 NJ) as a template
// parameter: the loops unroll over exactly the registers the layer needs,
// and each instantiation allocates only its own registers (a kernel
// covering every NJ would hold the largest one's), so the common sizes stay
// small enough to share a CU with the expert GEMMs' waves.
template <typename F>
__host__ __forceinline__ hipError_t with_nj(int64_t M, F&& f) {
    const int64_t nj = (M + 63) >> 6;
    if (nj <= 1) return f(std::integral_constant<int, 1>{});
    if (nj == 2) return f(std::integral_constant<int, 2>{});
    if (nj == 3) return f(std::integral_constant<int, 3>{});
    if (nj == 4) return f(std::integral_constant<int, 4>{});
    if (nj <= 8) return f(std::integral_constant<int, 8>{});
    return f(std::integral_constant<int, kMaxLanesJ>{});
}

// ---- bf16 x: exact three-way split of W_r, MFMA partial logits, top-k ----

// W_r = hi + mid + lo exactly, each a bf16 plane of W3[3][M][D].
__global__ __launch_bounds__(256) void router_split(const float* __restrict__ W_r,
                                                    bf16_t* __restrict__ W3, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= n) return;
    float v[8];
    const float4 a = *reinterpret_cast<const float4*>(W_r + i);
    const float4 b = *reinterpret_cast<const float4*>(W_r + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    bf16x8 hi, mid, lo;
    split3(v, hi, mid, lo);
    *reinterpret_cast<bf16x8*>(W3 + i) = hi;
    *reinterpret_cast<bf16x8*>(W3 + n + i) = mid;
    *reinterpret_cast<bf16x8*>(W3 + 2 * n + i) = lo;
}

constexpr int64_t kSmallRouteT = 256;   // bf16 batches up to this many tokens: fp64 dot router

// Small batches (decode): L[t][e] = x_t . W_r[e] accumulated in fp64 (the
// bf16 x fp32 products are exact in fp64), rounded once to fp32; a cheaper
// route to the same logits than splitting W_r and running the GEMM, whose
// tile grid a few dozen tokens cannot fill.  A block of 256 threads covers
// 4 experts (one per wave) x 4 tokens: a wave reads its expert's W_r row
// once for the 4 tokens, lane q taking the groups of four k at 4 q + 256 i
// (1 KB of the row per wave and step), one fp64 chain per token; the lanes
// are then summed in a fixed order.  Latency bounds this kernel: 64 lanes
// per dot product take D / 256 steps (20 at D = 5120), and the loop has no
// branch, so loads of consecutive steps overlap.  GLM-4.5 decode (64 tokens,
// 160 experts): 13.4 us, against 19.4 us with 16 lanes per dot product, 40 us
// with a per-token branch in the loop and 28-30 us unrolled 8 or 16 deep.
// Requires D % 4 == 0.
__global__ __launch_bounds__(256) void route_logits_small(const bf16_t* __restrict__ x,
                                                          const float* __restrict__ W_r, int T,
                                                          int D, int M, float* __restrict__ L) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int e = blockIdx.x * 4 + wv, t0 = blockIdx.y * 4;
    const int nt = min(4, T - t0);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (e < M) {
        const float* wr = W_r + (int64_t)e * D;
        // rows past the batch re-read its last row (no branch in the loop);
        // their sums are never written
        const bf16_t* xr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[j] = x + (int64_t)(t0 + min(j, nt - 1)) * D;
#pragma unroll 2
        for (int k = 4 * lane; k < D; k += 256) {
            const float4 w4 = *reinterpret_cast<const float4*>(wr + k);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint2 xv = *reinterpret_cast<const uint2*>(xr[j] + k);
                double a = acc[j];
                a = fma((double)__uint_as_float(xv.x << 16), (double)w4.x, a);
                a = fma((double)__uint_as_float(xv.x & 0xffff0000u), (double)w4.y, a);
                a = fma((double)__uint_as_float(xv.y << 16), (double)w4.z, a);
                a = fma((double)__uint_as_float(xv.y & 0xffff0000u), (double)w4.w, a);
                acc[j] = a;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc[j] += __shfl_xor(acc[j], off);
    if (e < M && lane < nt) {
        const double v = lane == 0 ? acc[0] : lane == 1 ? acc[1] : lane == 2 ? acc[2] : acc[3];
        L[(int64_t)(t0 + lane) * M + e] = (float)v;
    }
}

// One wave per token straight from the GEMM's partial logits: the wave sums
// its token's P[z][t][p M + e] over the K chunks z in order for each plane
// p, adds the planes as hi + (mid + lo) (so the logits are bitwise those of
// a separate reduction pass), stores them in L[t][0..M) (the backward's
// recomputed routing reads them there), stages them in its own LDS row and
// runs the top-k epilogue on it.
template <int NJ>
__global__ __launch_bounds__(256) void route_topk_partials(
    const float* __restrict__ P, int nK, float* __restrict__ L, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ w, int T, int M, int k, int scorer,
    int renorm, float alpha, float eps, int n_group, int topk_group) {
    extern __shared__ float s_logit[];   // [4][M]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;   // whole wave leaves; no block barrier follows
    float* lrow = s_logit + wave * M;
    const int64_t ld = 3 * (int64_t)M;
    // Two experts per lane and two K chunks per round have all their loads
    // in flight before the first sum; each plane still sums its chunks in
    // chunk order, then the planes as h + (m + l).
    for (int e0 = lane; e0 < M; e0 += 128) {
        float h[2] = {0.f, 0.f}, m[2] = {0.f, 0.f}, l[2] = {0.f, 0.f};
        for (int z0 = 0; z0 < nK; z0 += 2) {
            float hv[2][2], mv[2][2], lv[2][2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const float* row = P + ((int64_t)min(z0 + q, nK - 1) * T + t) * ld;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int e = min(e0 + 64 * u, M - 1);
                    hv[q][u] = row[e];
                    mv[q][u] = row[M + e];
                    lv[q][u] = row[2 * M + e];
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (z0 + q >= nK) continue;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    h[u] += hv[q][u];
                    m[u] += mv[q][u];
                    l[u] += lv[q][u];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = e0 + 64 * u;
            if (e >= M) continue;
            const float v = h[u] + (m[u] + l[u]);
            lrow[e] = v;
            L[(int64_t)t * M + e] = v;
        }
    }
    // the wave's own LDS row: make the writes visible across lanes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    topk_epilogue_nj<NJ>(lrow, M, k, scorer, bias, renorm, (double)alpha, (double)eps, n_group,
                         topk_group, idx + (int64_t)t * k, w + (int64_t)t * k);
}

// One wave per token: the top-k epilogue on its logits L[t][0..M).
template <int NJ>
__global__ __launch_bounds__(256) void route_topk(const float* __restrict__ L,
                                                  const float* __restrict__ bias,
                                                  int32_t* __restrict__ idx, float* __restrict__ w,
                                                  int T, int M, int k, int scorer, int renorm,
                                                  float alpha, float eps, int n_group,
                                                  int topk_group) {
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;   // whole wave leaves; no block barrier follows
    topk_epilogue_nj<NJ>(L + (int64_t)t * M, M, k, scorer, bias, renorm, (double)alpha,
                         (double)eps, n_group, topk_group, idx + (int64_t)t * k,
                         w + (int64_t)t * k);
}

// Generic router: one wave per token, fp64 dot products (fp32 or bf16 x).
template <typename XT, int NJ>
__global__ __launch_bounds__(256) void route_simple(
    const XT* __restrict__ x, const float* __restrict__ W_r, const float* __restrict__ bias,
    int32_t* __restrict__ idx, float* __restrict__ w, int T, int D, int M, int k, int scorer,
    int renorm, float alpha, float eps, int n_group, int topk_group) {
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
    topk_epilogue_nj<NJ>(lrow, M, k, scorer, bias, renorm, (double)alpha, (double)eps, n_group,
                         topk_group, idx + (int64_t)t * k, w + (int64_t)t * k);
}

}  // namespace

int route_ksplit(int64_t T, int64_t D, int64_t M) {
    // The logits GEMM (T x 3M, K = D) runs in 128 x 256 tiles, one
    // workgroup per CU at a time (256 CUs).  K chunks multiply the
    // workgroups; each chunk is at least 512 long (256 when the tile grid is
    // tiny).  The count minimises rounds of workgroups x K stages per
    // workgroup, so that no round runs half empty (GLM-4.5 prefill: 128
    // tiles x 2 chunks = one full round of 40 stages, against 3 chunks = 1.5
    // rounds of 27); on a tie, fewer chunks (less partial-logit traffic).
    const int64_t base = ((T + 127) / 128) * ((3 * M + 255) / 256);
    if (base <= 0 || D <= 0) return 1;
    constexpr int64_t kCUs = 256;
    const int64_t stages = (D + 63) / 64;
    int64_t maxk = D / (base < 32 ? 256 : 512);
    if (maxk < 1) maxk = 1;
    int64_t best = 1, best_cost = -1;
    for (int64_t nk = 1; nk <= maxk; ++nk) {
        const int64_t cost = ((base * nk + kCUs - 1) / kCUs) * ((stages + nk - 1) / nk);
        if (best_cost < 0 || cost < best_cost) {
            best = nk;
            best_cost = cost;
        }
    }
    return (int)best;
}

// Workspace: the split router weights W3 [3][M][D] bf16, the partial logits
// P [nK][T][3M] fp32 and the logits L [T][M] fp32, each 256-byte aligned.
static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
size_t route_workspace(int dtype, int64_t T, int64_t D, int64_t M) {
    if (dtype != 1) return 0;
    return align256((size_t)3 * M * D * 2) +
           align256((size_t)route_ksplit(T, D, M) * T * 3 * M * 4) + (size_t)T * M * 4;
}

size_t route_logits_offset(int dtype, int64_t T, int64_t D, int64_t M) {
    if (dtype != 1) return 0;
    return align256((size_t)3 * M * D * 2) + align256((size_t)route_ksplit(T, D, M) * T * 3 * M * 4);
}

hipError_t launch_route(hipStream_t s, int dtype, int scorer, const void* x, const float* W_r,
                        const float* bias, int32_t* idx, float* w, int64_t T, int64_t D,
                        int64_t M, int k, int renorm, float alpha, float eps, int n_group,
                        int topk_group, void* ws) {
    if (T == 0) return hipSuccess;
    const float* b = (scorer == 1) ? bias : nullptr;
    if (dtype == 1) {
        const int nK = route_ksplit(T, D, M);
        bf16_t* W3 = static_cast<bf16_t*>(ws);
        char* base = static_cast<char*>(ws);
        float* P = reinterpret_cast<float*>(base + align256((size_t)3 * M * D * 2));
        float* L = reinterpret_cast<float*>(base + align256((size_t)3 * M * D * 2) +
                                            align256((size_t)nK * T * 3 * M * 4));
        if (T <= kSmallRouteT && D % 4 == 0) {
            hipLaunchKernelGGL(route_logits_small,
                               dim3((unsigned)((M + 3) / 4), (unsigned)((T + 3) / 4)), dim3(256),
                               0, s, static_cast<const bf16_t*>(x), W_r, (int)T, (int)D, (int)M, L);
            return with_nj(M, [&](auto nj) {
                hipLaunchKernelGGL(route_topk<decltype(nj)::value>, dim3((unsigned)((T + 3) / 4)),
                                   dim3(256), 0, s, L, b, idx, w, (int)T, (int)M, k, scorer,
                                   renorm, alpha, eps, n_group, topk_group);
                return hipGetLastError();
            });
        }
        const int64_t n = M * D;
        hipLaunchKernelGGL(router_split, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s,
                           W_r, W3, n);
        // partial logits P[z][T][3M] = x . W3^T over K chunk z, on the expert GEMM
        GemmArgs g{};
        g.a = x;
        g.b = W3;
        g.c = P;
        g.dense_rows = T;
        g.a_rows = T;
        g.b_rows = (int)(3 * M);
        g.K = (int)D;
        g.N = (int)(3 * M);
        g.k_split = nK;
        hipError_t e = launch_gemm(s, 1, 128, EPI_DOWN_F32, g, (T + 127) / 128);
        if (e != hipSuccess) return e;
        return with_nj(M, [&](auto nj) {
            hipLaunchKernelGGL(route_topk_partials<decltype(nj)::value>,
                               dim3((unsigned)((T + 3) / 4)), dim3(256),
                               4 * (size_t)M * sizeof(float), s, P, nK, L, b, idx, w, (int)T,
                               (int)M, k, scorer, renorm, alpha, eps, n_group, topk_group);
            return hipGetLastError();
        });
    }
    dim3 grid((unsigned)((T + 3) / 4));
    const size_t lds = 4 * (size_t)M * sizeof(float);
    return with_nj(M, [&](auto nj) {
        hipLaunchKernelGGL((route_simple<float, decltype(nj)::value>), grid, dim3(256), lds, s,
                           static_cast<const float*>(x), W_r, b, idx, w, (int)T, (int)D, (int)M,
                           k, scorer, renorm, alpha, eps, n_group, topk_group);
        return hipGetLastError();
    });
}

}  // namespace moe
