// Combine: y[t] = sum_j O[slot_row[t*k + j]] + Ysh[t]  (the GLaM study note's
// MoE output sum over the selected experts; the GLM-4.5 note's output
// equation adds the shared expert).  The sorted rows O (fp32) already carry
// their gate weights.  fp32 sum in fixed slot order, one rounding to the
// output dtype, 16-byte vector loads and stores, one wave per token and
// column chunk.  It is a gather, not a scatter: no atomics, so the result
// is deterministic.
#include "common.hpp"

namespace moe {
namespace {

template <int V>
__device__ __forceinline__ void load_f32(const float* p, float* v) {
#pragma unroll
    for (int i = 0; i < V; i += 4) {
        const float4 f = *reinterpret_cast<const float4*>(p + i);
        v[i] = f.x; v[i + 1] = f.y; v[i + 2] = f.z; v[i + 3] = f.w;
    }
}

template <typename TY>
struct Out;
template <>
struct Out<bf16_t> {
    static constexpr int V = 8;   // 8 outputs = one 16-byte store
    __device__ static void store(bf16_t* p, const float* v) {
        u32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        *reinterpret_cast<u32x4*>(p) = u;
    }
};
template <>
struct Out<float> {
    static constexpr int V = 4;
    __device__ static void store(float* p, const float* v) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

template <typename TY>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ O,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ Ysh,
                                                      TY* __restrict__ y, int Tn, int k, int D,
                                                      int chunks) {
    // one wave per (token, chunk of 64 x V columns): enough waves to keep
    // HBM busy even for a decode-sized batch
    constexpr int V = Out<TY>::V;
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = (int)(wid / chunks);
    if (t >= Tn) return;
    const int d0 = (int)(wid % chunks) * 64 * V + lane * V;
    if (d0 >= D) return;
    int rows[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) rows[j] = (j < k) ? slot_row[(int64_t)t * k + j] : -1;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (rows[j] < 0) continue;
        float v[V];
        load_f32<V>(O + (int64_t)rows[j] * D + d0, v);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += v[i];
    }
    if (Ysh) {
        float v[V];
        load_f32<V>(Ysh + (int64_t)t * D + d0, v);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += v[i];
    }
    Out<TY>::store(y + (int64_t)t * D + d0, acc);
}

// The same combine over compact rows: row j's value at column d is
// O16[j, d] * 2^Oexp[j, d / 16] (fp16 times a power of two, exact in fp32),
// so the fp32 sum runs over exactly the values the rows hold, in the same
// slot order, then the shared row, then one rounding.  A lane's V columns
// share one scale group (V divides kRowGroup and d0 is a multiple of V).
// The shared row is fp32 (Ysh) or compact as well (Ysh16 / YshExp, one row
// per token, the same format).
template <typename TY>
__global__ __launch_bounds__(256) void combine_compact_kernel(
    const uint16_t* __restrict__ O16, const int8_t* __restrict__ Oexp,
    const int32_t* __restrict__ slot_row, const float* __restrict__ Ysh,
    const uint16_t* __restrict__ Ysh16, const int8_t* __restrict__ YshExp, TY* __restrict__ y,
    int Tn, int k, int D, int chunks) {
    constexpr int V = Out<TY>::V;
    static_assert(kRowGroup % V == 0, "a lane's columns lie in one scale group");
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = (int)(wid / chunks);
    if (t >= Tn) return;
    const int d0 = (int)(wid % chunks) * 64 * V + lane * V;
    if (d0 >= D) return;
    const int G = (D + kRowGroup - 1) / kRowGroup;
    int rows[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) rows[j] = (j < k) ? slot_row[(int64_t)t * k + j] : -1;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    // acc += row `row` of a compact matrix (values v16, exponents ve)
    auto add_compact = [&](const uint16_t* v16, const int8_t* ve, int64_t row) {
        const uint16_t* p = v16 + row * D + d0;
        const int e = ve[row * G + d0 / kRowGroup];
        uint16_t h[V];
        if constexpr (V == 8) {
            const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[2 * i] = (uint16_t)(u[i] & 0xffffu);
                h[2 * i + 1] = (uint16_t)(u[i] >> 16);
            }
        } else {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            h[0] = (uint16_t)(u.x & 0xffffu); h[1] = (uint16_t)(u.x >> 16);
            h[2] = (uint16_t)(u.y & 0xffffu); h[3] = (uint16_t)(u.y >> 16);
        }
#pragma unroll
        for (int i = 0; i < V; ++i)
            acc[i] += ldexpf((float)__builtin_bit_cast(_Float16, h[i]), e);
    };
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (rows[j] < 0) continue;
        add_compact(O16, Oexp, rows[j]);
    }
    if (Ysh16) {
        add_compact(Ysh16, YshExp, t);
    } else if (Ysh) {
        float v[V];
        load_f32<V>(Ysh + (int64_t)t * D + d0, v);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += v[i];
    }
    Out<TY>::store(y + (int64_t)t * D + d0, acc);
}

}  // namespace

hipError_t launch_combine_compact(hipStream_t s, int out_dtype, const void* O16,
                                  const int8_t* Oexp, const int32_t* slot_row, const float* Ysh,
                                  const void* Ysh16, const int8_t* YshExp, void* y, int64_t T,
                                  int k, int64_t D) {
    if (T == 0) return hipSuccess;
    const int V = out_dtype == 1 ? Out<bf16_t>::V : Out<float>::V;
    const int chunks = (int)((D + 64 * V - 1) / (64 * V));
    dim3 grid((unsigned)((T * chunks + 3) / 4));
    const uint16_t* o = static_cast<const uint16_t*>(O16);
    if (out_dtype == 1)
        hipLaunchKernelGGL(combine_compact_kernel<bf16_t>, grid, dim3(256), 0, s, o, Oexp,
                           slot_row, Ysh, static_cast<const uint16_t*>(Ysh16), YshExp,
                           static_cast<bf16_t*>(y), (int)T, k, (int)D, chunks);
    else
        hipLaunchKernelGGL(combine_compact_kernel<float>, grid, dim3(256), 0, s, o, Oexp,
                           slot_row, Ysh, static_cast<const uint16_t*>(Ysh16), YshExp,
                           static_cast<float*>(y), (int)T, k, (int)D, chunks);
    return hipGetLastError();
}

hipError_t launch_combine(hipStream_t s, int out_dtype, const float* O, const int32_t* slot_row,
                          const float* Ysh, void* y, int64_t T, int k, int64_t D) {
    if (T == 0) return hipSuccess;
    const int V = out_dtype == 1 ? Out<bf16_t>::V : Out<float>::V;
    const int chunks = (int)((D + 64 * V - 1) / (64 * V));
    dim3 grid((unsigned)((T * chunks + 3) / 4));
    if (out_dtype == 1)
        hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, s, O, slot_row, Ysh,
                           static_cast<bf16_t*>(y), (int)T, k, (int)D, chunks);
    else
        hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, O, slot_row, Ysh,
                           static_cast<float*>(y), (int)T, k, (int)D, chunks);
    return hipGetLastError();
}

}  // namespace moe
