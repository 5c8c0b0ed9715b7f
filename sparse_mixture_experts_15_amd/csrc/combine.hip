// Combine: y[t] = sum_j O[slot_row[t*k + j]] + Ysh[t]  (the GLaM study note's
// MoE output sum over the selected experts; the GLM-4.5 note's output
// equation adds the shared expert).  The sorted rows O (fp32) already carry
// their gate weights.  fp32 sum in fixed slot order, one rounding to the
// output dtype, 16-byte vector loads and stores, one wave per token and
// column chunk.  It is a gather, not a scatter: no atomics, so the result
// is deterministic.
#include <type_traits>

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

// The token's slot rows for all k slots as wave-uniform values, read while
// every lane of the wave is active (lane j holds slot j, lanes past k hold
// -1).
__device__ __forceinline__ void token_rows(const int32_t* __restrict__ slot_row, int64_t t, int k,
                                           int lane, int (&r)[kMaxK]) {
    const int rl = lane < k ? slot_row[t * k + lane] : -1;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) r[j] = __builtin_amdgcn_readlane(rl, j);
}

// Rows are taken NB slots at a time: all NB loads are issued before the
// first is added, so a wave keeps NB + 1 rows (with the shared row) in
// flight instead of waiting on each in turn.  A dropped slot (row -1) or a
// slot past k in the last batch loads the token's own first slot row t k,
// which exists (the rows hold T k entries), and its value is not added, so
// the sum is the same, bit for bit, as one that skips it.
template <typename TY, int NB>
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
    if (t >= Tn) return;   // t is one value per wave
    int rows[kMaxK];
    token_rows(slot_row, t, k, lane, rows);
    const int d0 = (int)(wid % chunks) * 64 * V + lane * V;
    if (d0 >= D) return;
    const int64_t own = (int64_t)t * k;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    float sh[V];
    for (int j0 = 0; j0 < k; j0 += NB) {
        float v[NB][V];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            const int r = j0 + jj < kMaxK ? rows[j0 + jj] : -1;
            load_f32<V>(O + (r >= 0 ? (int64_t)r : own) * D + d0, v[jj]);
        }
        // the shared row is added last but fetched with the first batch
        if (j0 == 0 && Ysh) load_f32<V>(Ysh + (int64_t)t * D + d0, sh);
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            const bool use = j0 + jj < kMaxK && rows[j0 + jj] >= 0;
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = use ? acc[i] + v[jj][i] : acc[i];
        }
    }
    if (Ysh) {
        if (k <= 0) load_f32<V>(Ysh + (int64_t)t * D + d0, sh);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += sh[i];
    }
    Out<TY>::store(y + (int64_t)t * D + d0, acc);
}

// The same combine over compact rows: row j's value at column d is
// O16[j, d] * 2^Oexp[j, d / 64] (fp16 times a power of two, exact in fp32),
// so the fp32 sum runs over exactly the values the rows hold, in the same
// slot order, then the shared row, then one rounding.  A lane's V columns
// share one scale group (V divides kRowGroup and d0 is a multiple of V).
// The shared row is fp32 (Ysh) or compact as well (Ysh16 / YshExp, one row
// per token, the same format).
template <typename TY, int NB>
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
    if (t >= Tn) return;   // t is one value per wave
    int rows[kMaxK];
    token_rows(slot_row, t, k, lane, rows);
    const int d0 = (int)(wid % chunks) * 64 * V + lane * V;
    if (d0 >= D) return;
    const int64_t own = (int64_t)t * k;
    const int G = (D + kRowGroup - 1) / kRowGroup;
    const int grp = d0 / kRowGroup;
    // one row's V values at d0 and its scale exponent
    struct Piece { u32x4 u; int e; };
    auto load_row = [&](const uint16_t* v16, const int8_t* ve, int64_t row, Piece& pc) {
        const uint16_t* p = v16 + row * D + d0;
        if constexpr (V == 8) {
            pc.u = *reinterpret_cast<const u32x4*>(p);
        } else {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            pc.u = u32x4{u.x, u.y, 0u, 0u};
        }
        pc.e = ve[row * G + grp];
    };
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    auto add_piece = [&](const Piece& pc, bool use) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const uint32_t w = pc.u[i / 2];
            const uint16_t h = (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu));
            const float v = ldexpf((float)__builtin_bit_cast(_Float16, h), pc.e);
            acc[i] = use ? acc[i] + v : acc[i];
        }
    };
    Piece sh{};
    float shf[V];
    auto load_shared = [&] {
        if (Ysh16) load_row(Ysh16, YshExp, t, sh);
        else if (Ysh) load_f32<V>(Ysh + (int64_t)t * D + d0, shf);
    };
    for (int j0 = 0; j0 < k; j0 += NB) {
        Piece pc[NB];
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            const int r = j0 + jj < kMaxK ? rows[j0 + jj] : -1;
            load_row(O16, Oexp, r >= 0 ? (int64_t)r : own, pc[jj]);
        }
        // the shared row is added last but fetched with the first batch
        if (j0 == 0) load_shared();
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) add_piece(pc[jj], j0 + jj < kMaxK && rows[j0 + jj] >= 0);
    }
    if (k <= 0) load_shared();
    if (Ysh16) {
        add_piece(sh, true);
    } else if (Ysh) {
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += shf[i];
    }
    Out<TY>::store(y + (int64_t)t * D + d0, acc);
}

}  // namespace

// Slots per batch: the smallest power of two >= k, at most 8.
template <typename F>
hipError_t with_batch(int k, F&& f) {
    if (k <= 1) return f(std::integral_constant<int, 1>{});
    if (k <= 2) return f(std::integral_constant<int, 2>{});
    if (k <= 4) return f(std::integral_constant<int, 4>{});
    return f(std::integral_constant<int, 8>{});
}

hipError_t launch_combine_compact(hipStream_t s, int out_dtype, const void* O16,
                                  const int8_t* Oexp, const int32_t* slot_row, const float* Ysh,
                                  const void* Ysh16, const int8_t* YshExp, void* y, int64_t T,
                                  int k, int64_t D) {
    if (T == 0) return hipSuccess;
    if (k < 1 || k > kMaxK) return hipErrorInvalidValue;
    const int V = out_dtype == 1 ? Out<bf16_t>::V : Out<float>::V;
    const int chunks = (int)((D + 64 * V - 1) / (64 * V));
    dim3 grid((unsigned)((T * chunks + 3) / 4));
    const uint16_t* o = static_cast<const uint16_t*>(O16);
    const uint16_t* s16 = static_cast<const uint16_t*>(Ysh16);
    return with_batch(k, [&](auto nb) {
        constexpr int NB = decltype(nb)::value;
        if (out_dtype == 1)
            hipLaunchKernelGGL((combine_compact_kernel<bf16_t, NB>), grid, dim3(256), 0, s, o,
                               Oexp, slot_row, Ysh, s16, YshExp, static_cast<bf16_t*>(y), (int)T,
                               k, (int)D, chunks);
        else
            hipLaunchKernelGGL((combine_compact_kernel<float, NB>), grid, dim3(256), 0, s, o,
                               Oexp, slot_row, Ysh, s16, YshExp, static_cast<float*>(y), (int)T,
                               k, (int)D, chunks);
        return hipGetLastError();
    });
}

hipError_t launch_combine(hipStream_t s, int out_dtype, const float* O, const int32_t* slot_row,
                          const float* Ysh, void* y, int64_t T, int k, int64_t D) {
    if (T == 0) return hipSuccess;
    if (k < 1 || k > kMaxK) return hipErrorInvalidValue;
    const int V = out_dtype == 1 ? Out<bf16_t>::V : Out<float>::V;
    const int chunks = (int)((D + 64 * V - 1) / (64 * V));
    dim3 grid((unsigned)((T * chunks + 3) / 4));
    return with_batch(k, [&](auto nb) {
        constexpr int NB = decltype(nb)::value;
        if (out_dtype == 1)
            hipLaunchKernelGGL((combine_kernel<bf16_t, NB>), grid, dim3(256), 0, s, O, slot_row,
                               Ysh, static_cast<bf16_t*>(y), (int)T, k, (int)D, chunks);
        else
            hipLaunchKernelGGL((combine_kernel<float, NB>), grid, dim3(256), 0, s, O, slot_row,
                               Ysh, static_cast<float*>(y), (int)T, k, (int)D, chunks);
        return hipGetLastError();
    });
}

}  // namespace moe
