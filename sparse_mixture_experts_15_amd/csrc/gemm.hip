// Expert FFN GEMMs: a grouped GEMM over the experts' contiguous row ranges
// (or a dense GEMM for the shared expert), with the FFN nonlinearity and
// the gate weight fused into the epilogues.
//
// What is computed (GLM-5 "Shared expert" page, "All 5 steps": g = x W1,
// u = x W3, a = g sigma(g), h = a (.) u, y = h W2; GLaM study note dense FFN
// W2 s(W1 x + b1) + b2; the GLM-5 routed-experts excerpt scales each
// expert output row by its slot's top-k weight after the down projection):
//
//   up   (SWIGLU):  H[r, n] = silu(A[r] . Wg[e, n]) * (A[r] . Wu[e, n])
//   up   (GELU):    H[r, n] = gelu(A[r] . W1[e, n] + b1[e, n])
//   down (scaled):  O[r, n] = w[slot(r)] * (H[r] . W2[e, n] + b2[e, n])   (fp32)
//   down (fp32):    Y[r, n] = H[r] . W2[n]            (shared expert)
//
// bf16 path: 128 x 128 workgroup tile (128 A rows x 128 B rows), K step 64,
// four waves of 64 x 64, v_mfma_f32_16x16x32_bf16, operands staged through
// double-buffered LDS with rows padded to 144 bytes (conflict-free 16-byte
// fragment reads for 32 or 64 LDS banks).  A rows of the up projection are
// gathered on load through the sorted token list, so the permuted
// activations are never materialised.  For SwiGLU each wave's 64 B rows are
// 32 gate rows and the 32 matching up rows, so silu(gate) * up is formed in
// registers.  fp32 path: a plain SIMT tile kernel (64 x 64, K step 16).
#include "common.hpp"

namespace moe {
namespace {

// ------------------------------------------------------------------ tiles

struct Tile {
    int e;
    int64_t r0, rend;
};

// Tile of m-tile index `mt`; returns false when the index is past the end.
__device__ __forceinline__ bool tile_of(const GemmArgs& g, int mt, int bm, Tile& t) {
    if (g.tiles) {
        const int e = g.tiles[2 * mt];
        if (e < 0) return false;
        t.e = e;
        t.r0 = g.tiles[2 * mt + 1];
        t.rend = g.offsets[e + 1];
        return true;
    }
    t.e = 0;
    t.r0 = (int64_t)mt * bm;
    t.rend = g.dense_rows;
    return t.r0 < t.rend;
}

// Output column and B row of B-tile row b.  SWIGLU tiles hold `half`
// output columns: per 64-row wave block, 32 gate rows then their 32 up rows.
template <int EPI>
__device__ __forceinline__ void brow_map(int b, int n_base, int F_split, int& out_col,
                                         int& b_row) {
    if (EPI == EPI_SWIGLU) {
        const int wb = b >> 6, within = b & 63;
        out_col = n_base + 32 * wb + (within & 31);
        b_row = out_col + ((within >> 5) ? F_split : 0);
    } else {
        out_col = n_base + b;
        b_row = out_col;
    }
}

// ------------------------------------------------------------ bf16 / MFMA

constexpr int BM = 128;      // A rows per tile
constexpr int BNB = 128;     // B rows per tile
constexpr int BK = 64;       // K per stage
constexpr int LDR = BK + 8;  // padded LDS row (bf16 elements): 144 bytes
constexpr int NT = 256;

template <int EPI>
__global__ __launch_bounds__(NT, 2) void gemm_bf16(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDR];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][BNB * LDR];

    Tile tl;
    if (!tile_of(g, blockIdx.y, BM, tl)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int K = g.K, N = g.N;
    const int out_per_tile = (EPI == EPI_SWIGLU) ? BNB / 2 : BNB;
    const int n_base = blockIdx.x * out_per_tile;

    const bf16_t* __restrict__ A = static_cast<const bf16_t*>(g.a);
    const bf16_t* __restrict__ B = static_cast<const bf16_t*>(g.b) + (int64_t)tl.e * g.b_stride;

    // per-thread global sources: rows (tid >> 3) + 32 i, 16-byte chunk tid & 7
    const int lc = tid & 7;
    const bf16_t* asrc[4];
    const bf16_t* bsrc[4];
    bool aval[4], bval[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        const int64_t r = tl.r0 + row;
        aval[i] = r < tl.rend;
        int64_t src = 0;
        if (aval[i]) src = g.gather ? (int64_t)g.gather[r] : r;
        asrc[i] = A + src * K + lc * 8;
        int oc, br;
        brow_map<EPI>(row, n_base, g.F_split, oc, br);
        bval[i] = oc < N;
        bsrc[i] = B + (int64_t)(bval[i] ? br : 0) * K + lc * 8;
    }

    u32x4 ra[4], rb[4];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int k0) {
        const bool kv = k0 + lc * 8 < K;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = (aval[i] && kv) ? *reinterpret_cast<const u32x4*>(asrc[i] + k0) : zero;
            rb[i] = (bval[i] && kv) ? *reinterpret_cast<const u32x4*>(bsrc[i] + k0) : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (tid >> 3) + 32 * i;
            *reinterpret_cast<u32x4*>(&sA[buf][row * LDR + lc * 8]) = ra[i];
            *reinterpret_cast<u32x4*>(&sB[buf][row * LDR + lc * 8]) = rb[i];
        }
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 64 + 16 * i + fr;
                af[i] = *reinterpret_cast<const bf16x8*>(&sA[cur][row * LDR + kk + fk]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wn * 64 + 16 * j + fr;
                bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[cur][row * LDR + kk + fk]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  MFMA 16x16 layout: lane holds column lane%16 and rows
    // 4*(lane/16) + q of each 16x16 block.
    const int rq = 4 * (lane >> 4);
    if (EPI == EPI_SWIGLU) {
        bf16_t* C = static_cast<bf16_t*>(g.c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n_base + 32 * wn + 16 * j + fr;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t r = tl.r0 + wm * 64 + 16 * i + rq + q;
                    if (r < tl.rend && n < N)
                        C[r * N + n] = f32_to_bf16(silu_f32(acc[i][j][q]) * acc[i][j + 2][q]);
                }
            }
    } else {
        const bf16_t* bias = static_cast<const bf16_t*>(g.bias);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float wrow[4];
            int64_t rr[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                rr[q] = tl.r0 + wm * 64 + 16 * i + rq + q;
                wrow[q] = 1.f;
                if (EPI == EPI_DOWN_SCALED && rr[q] < tl.rend) wrow[q] = g.row_w[g.row_slot[rr[q]]];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n_base + 64 * wn + 16 * j + fr;
                if (n >= N) continue;
                const float bv = bias ? bf16_to_f32(bias[(int64_t)tl.e * N + n]) : 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (rr[q] >= tl.rend) continue;
                    const float v = acc[i][j][q];
                    if (EPI == EPI_GELU)
                        static_cast<bf16_t*>(g.c)[rr[q] * N + n] = f32_to_bf16(gelu_erf_f32(v + bv));
                    else if (EPI == EPI_DOWN_SCALED)
                        static_cast<float*>(g.c)[rr[q] * N + n] = wrow[q] * (v + bv);
                    else
                        static_cast<float*>(g.c)[rr[q] * N + n] = v;
                }
            }
        }
    }
}

// ------------------------------------------------------------ fp32 / SIMT

constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32(GemmArgs g) {
    __shared__ float sA[FBK][FBM + 4];
    __shared__ float sB[FBK][FBN + 4];
    Tile tl;
    if (!tile_of(g, blockIdx.y, FBM, tl)) return;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int K = g.K, N = g.N;
    const int out_per_tile = (EPI == EPI_SWIGLU) ? FBN / 2 : FBN;
    const int n_base = blockIdx.x * out_per_tile;
    const float* A = static_cast<const float*>(g.a);
    const float* B = static_cast<const float*>(g.b) + (int64_t)tl.e * g.b_stride;

    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += FBK) {
        for (int i = tid; i < FBM * FBK; i += 256) {
            const int m = i / FBK, kq = i % FBK;
            const int64_t r = tl.r0 + m;
            float v = 0.f;
            if (r < tl.rend && k0 + kq < K) {
                const int64_t src = g.gather ? (int64_t)g.gather[r] : r;
                v = A[src * K + k0 + kq];
            }
            sA[kq][m] = v;
        }
        for (int i = tid; i < FBN * FBK; i += 256) {
            const int b = i / FBK, kq = i % FBK;
            int oc, br;
            if (EPI == EPI_SWIGLU) {   // 32 gate rows then their 32 up rows
                oc = n_base + (b & 31);
                br = oc + ((b >> 5) ? g.F_split : 0);
            } else {
                oc = n_base + b;
                br = oc;
            }
            float v = 0.f;
            if (oc < N && k0 + kq < K) v = B[(int64_t)br * K + k0 + kq];
            sB[kq][b] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < FBK; ++kq) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[kq][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sB[kq][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
    }
    const float* bias = static_cast<const float*>(g.bias);
    float* C = static_cast<float*>(g.c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = tl.r0 + ty * 4 + i;
        if (r >= tl.rend) continue;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n_base + tx + 16 * j;
                if (n < N) C[r * N + n] = silu_f32(acc[i][j]) * acc[i][j + 2];
            }
        } else {
            const float wr = (EPI == EPI_DOWN_SCALED) ? g.row_w[g.row_slot[r]] : 1.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n_base + tx + 16 * j;
                if (n >= N) continue;
                const float bv = bias ? bias[(int64_t)tl.e * N + n] : 0.f;
                const float v = acc[i][j];
                if (EPI == EPI_GELU) C[r * N + n] = gelu_erf_f32(v + bv);
                else if (EPI == EPI_DOWN_SCALED) C[r * N + n] = wr * (v + bv);
                else C[r * N + n] = v;
            }
        }
    }
}

template <int EPI>
hipError_t launch_one(hipStream_t s, int dtype, const GemmArgs& g, int64_t m_tiles) {
    if (m_tiles <= 0) return hipSuccess;
    if (dtype == 1) {
        const int opt = (EPI == EPI_SWIGLU) ? BNB / 2 : BNB;
        dim3 grid((unsigned)((g.N + opt - 1) / opt), (unsigned)m_tiles);
        hipLaunchKernelGGL(gemm_bf16<EPI>, grid, dim3(NT), 0, s, g);
    } else {
        const int opt = (EPI == EPI_SWIGLU) ? FBN / 2 : FBN;
        dim3 grid((unsigned)((g.N + opt - 1) / opt), (unsigned)m_tiles);
        hipLaunchKernelGGL(gemm_f32<EPI>, grid, dim3(256), 0, s, g);
    }
    return hipGetLastError();
}

}  // namespace

int gemm_block_m(int dtype) { return dtype == 1 ? BM : FBM; }

hipError_t launch_gemm(hipStream_t s, int dtype, int epi, const GemmArgs& g, int64_t m_tiles) {
    switch (epi) {
        case EPI_SWIGLU: return launch_one<EPI_SWIGLU>(s, dtype, g, m_tiles);
        case EPI_GELU: return launch_one<EPI_GELU>(s, dtype, g, m_tiles);
        case EPI_DOWN_SCALED: return launch_one<EPI_DOWN_SCALED>(s, dtype, g, m_tiles);
        default: return launch_one<EPI_DOWN_F32>(s, dtype, g, m_tiles);
    }
}

}  // namespace moe
