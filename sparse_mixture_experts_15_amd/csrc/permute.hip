// Dispatch: group the T*k flat routing slots f = t*k + j by expert, stably
// (the "dispatch / expert batching" part of the routing overhead in the
// GLaM study note's "Capacity, Active Compute, and Reporting" table; the
// GLM-5 routed-experts excerpt gathers each expert's tokens the same way,
// with an extra one-hot class, index M, that is skipped).
//
// Three kernels, no global atomics:
//  1. count:   per block of 256 tokens, an LDS histogram over experts.
//  2. scan:    one workgroup turns the block histograms into per-block
//              bases (exclusive over blocks) and the expert counts into
//              offsets (exclusive over experts); marks unused tail rows.
//  3. scatter: per block, each wave sets bit `lane` of a 64-bit LDS mask
//              per expert its token picked; a slot's rank among earlier
//              slots of the same expert is the popcount of the lower lanes'
//              bits plus the masks of the lower waves.  A token picks an
//              expert at most once, so this is exactly the stable order.
#include "common.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(kPermBlock) void perm_count(const int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ hist, int T, int k,
                                                        int M) {
    extern __shared__ int32_t s_cnt[];   // [M]
    for (int e = threadIdx.x; e < M; e += kPermBlock) s_cnt[e] = 0;
    __syncthreads();
    const int t = blockIdx.x * kPermBlock + threadIdx.x;
    if (t < T) {
        // all of the token's indices are loaded before the first atomic
        int ev[kMaxK];
        const int32_t* it = idx + (int64_t)t * k;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) ev[j] = j < k ? it[j] : -1;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k) break;
            const int e = ev[j];
            if (e >= 0 && e < M) atomicAdd(&s_cnt[e], 1);
        }
    }
    __syncthreads();
    int32_t* h = hist + (int64_t)blockIdx.x * M;
    for (int e = threadIdx.x; e < M; e += kPermBlock) h[e] = s_cnt[e];
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void perm_scan(int32_t* __restrict__ hist, int nblk,
                                                         int T, int k, int M,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted_token,
                                                         int32_t* __restrict__ sorted_slot) {
    __shared__ int32_t s_tot[kMaxExperts];
    __shared__ int32_t s_warp[kScanThreads / 64];
    const int tid = threadIdx.x;
    // per expert: exclusive running sum over blocks, in block order
    for (int e = tid; e < M; e += kScanThreads) {
        int32_t run = 0;
        // eight blocks' counts are loaded before any is overwritten (the
        // clamped index re-reads the last block, not yet overwritten)
        for (int b0 = 0; b0 < nblk; b0 += 8) {
            int32_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = hist[(int64_t)min(b0 + q, nblk - 1) * M + e];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (b0 + q >= nblk) break;
                hist[(int64_t)(b0 + q) * M + e] = run;
                run += v[q];
            }
        }
        counts[e] = run;
        s_tot[e] = run;
    }
    __syncthreads();
    // exclusive scan of counts over experts (M <= 1024: one value per thread)
    const int32_t v = (tid < M) ? s_tot[tid] : 0;
    int32_t incl = v;
    const int lane = tid & 63, wv = tid >> 6;
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
    if (tid < M) offsets[tid] = incl - v;
    if (tid == M - 1) offsets[M] = incl;
    __syncthreads();
    // rows past the kept slots (dropped slots only) are marked -1
    int32_t total = 0;
    for (int i = 0; i < kScanThreads / 64; ++i) total += s_warp[i];
    const int64_t S = (int64_t)T * k;
    for (int64_t r = total + tid; r < S; r += kScanThreads) {
        sorted_token[r] = -1;
        sorted_slot[r] = -1;
    }
}

__global__ __launch_bounds__(kPermBlock) void perm_scatter(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ hist,
    const int32_t* __restrict__ offsets, int T, int k, int M, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_row) {
    extern __shared__ unsigned long long s_mask[];   // [4][M]
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int i = tid; i < 4 * M; i += kPermBlock) s_mask[i] = 0ull;
    __syncthreads();
    const int t = blockIdx.x * kPermBlock + tid;
    int e_of[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) e_of[j] = -1;
    if (t < T) {
        // all of the token's indices are loaded before the first atomic
        int ev[kMaxK];
        const int32_t* it = idx + (int64_t)t * k;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) ev[j] = j < k ? it[j] : -1;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k) break;
            const int e = ev[j];
            if (e >= 0 && e < M) {
                e_of[j] = e;
                atomicOr(&s_mask[wv * M + e], 1ull << lane);
            }
        }
    }
    __syncthreads();
    if (t >= T) return;
    const int32_t* hb = hist + (int64_t)blockIdx.x * M;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j >= k) break;
        const int64_t f = (int64_t)t * k + j;
        const int e = e_of[j];
        if (e < 0) {
            slot_row[f] = -1;
            continue;
        }
        int rank = __popcll(s_mask[wv * M + e] & below);
        for (int w2 = 0; w2 < wv; ++w2) rank += __popcll(s_mask[w2 * M + e]);
        const int32_t r = offsets[e] + hb[e] + rank;
        sorted_slot[r] = (int32_t)f;
        sorted_token[r] = t;
        slot_row[f] = r;
    }
}

// One tile table, built by a whole workgroup of kScanThreads threads from
// the expert offsets (offsets[0..M], written earlier and visible to it):
// one thread per expert writes its own tiles after a scan of the tile
// counts.  The extra group (index M) ends `extra` rows after the last
// expert's; with set_end its end goes to offsets[M + 1].  Begins with a
// barrier, so consecutive calls may share s_warp.
__device__ void build_tiles(int32_t* offsets, int M, int64_t extra, int bm, int max_tiles,
                            int32_t* __restrict__ tiles, bool set_end, int32_t* s_warp) {
    __syncthreads();
    const int Mg = extra > 0 ? M + 1 : M;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int32_t nt = 0, r0 = 0;
    if (tid < Mg) {
        r0 = offsets[tid];
        const int32_t end = tid == M ? r0 + (int32_t)extra : offsets[tid + 1];
        nt = (end - r0 + bm - 1) / bm;
        if (tid == M && set_end) offsets[M + 1] = end;
    }
    int32_t incl = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_warp[wv] = incl;
    __syncthreads();
    int32_t base = 0, total = 0;
    for (int i = 0; i < kScanThreads / 64; ++i) {
        if (i < wv) base += s_warp[i];
        total += s_warp[i];
    }
    const int32_t first = base + incl - nt;
    for (int i = 0; i < nt; ++i) {
        tiles[2 * (first + i)] = tid;
        tiles[2 * (first + i) + 1] = r0 + i * bm;
    }
    for (int i = total + tid; i < max_tiles; i += kScanThreads) {
        tiles[2 * i] = -1;
        tiles[2 * i + 1] = 0;
    }
    if (tid == 0) tiles[2 * max_tiles] = total;
}

// The whole dispatch in one workgroup when T <= kSmallT (one token per
// thread, decode-sized batches): the per-wave expert masks of the scatter
// give both the counts (their popcounts) and the stable ranks, so count,
// scan and scatter run back to back without a launch in between.  Same
// results as the three kernels above.
__global__ __launch_bounds__(kScanThreads) void perm_small(const int32_t* __restrict__ idx, int T,
                                                          int k, int M, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_token,
                                                          int32_t* __restrict__ sorted_slot,
                                                          int32_t* __restrict__ slot_row,
                                                          TileTables tt, int ntables,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ row_scale,
                                                          int64_t extra) {
    constexpr int NW = kScanThreads / 64;
    extern __shared__ unsigned long long s_mask[];   // [NW][M], then s_off[M]
    int32_t* s_off = reinterpret_cast<int32_t*>(s_mask + NW * M);
    __shared__ int32_t s_warp[NW];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int i = tid; i < NW * M; i += kScanThreads) s_mask[i] = 0ull;
    __syncthreads();
    const int t = tid;
    int e_of[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) e_of[j] = -1;
    if (t < T) {
        // all of the token's indices are loaded before the first atomic
        int ev[kMaxK];
        const int32_t* it = idx + (int64_t)t * k;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) ev[j] = j < k ? it[j] : -1;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k) break;
            const int e = ev[j];
            if (e >= 0 && e < M) {
                e_of[j] = e;
                atomicOr(&s_mask[wv * M + e], 1ull << lane);
            }
        }
    }
    __syncthreads();
    // counts and their exclusive scan over experts (one expert per thread)
    int32_t c = 0;
    if (tid < M)
        for (int w2 = 0; w2 < NW; ++w2) c += __popcll(s_mask[w2 * M + tid]);
    int32_t incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_warp[wv] = incl;
    __syncthreads();
    int32_t base = 0, total = 0;
    for (int i = 0; i < NW; ++i) {
        if (i < wv) base += s_warp[i];
        total += s_warp[i];
    }
    incl += base;
    if (tid < M) {
        counts[tid] = c;
        offsets[tid] = incl - c;
        s_off[tid] = incl - c;
    }
    if (tid == M - 1) offsets[M] = incl;
    __syncthreads();
    const int64_t S = (int64_t)T * k;
    const bool tables = ntables > 0;   // uniform
    for (int64_t r = total + tid; r < S; r += kScanThreads) {
        sorted_token[r] = -1;
        sorted_slot[r] = -1;
        if (tables) row_scale[r] = 0.f;
    }
    if (t < T) {
        const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k) break;
            const int64_t f = (int64_t)t * k + j;
            const int e = e_of[j];
            if (e < 0) {
                slot_row[f] = -1;
                continue;
            }
            int rank = __popcll(s_mask[wv * M + e] & below);
            for (int w2 = 0; w2 < wv; ++w2) rank += __popcll(s_mask[w2 * M + e]);
            const int32_t r = s_off[e] + rank;
            sorted_slot[r] = (int32_t)f;
            sorted_token[r] = t;
            slot_row[f] = r;
            if (tables) row_scale[r] = w[f];
        }
    }
    if (!tables) return;
    // the tile tables and the row scales of tile_table, without its launch:
    // the extra group's rows (every token once, scale 1), then the tables
    for (int64_t r = S + tid; r < S + extra; r += kScanThreads) {
        row_scale[r] = 1.f;
        sorted_token[r] = (int32_t)(r - S);
    }
    for (int y = 0; y < ntables; ++y)
        build_tiles(offsets, M, extra, tt.bm[y], tt.max_tiles[y], tt.tiles[y], y == 0, s_warp);
}

// Per m-tile of `bm` rows: (expert, first row).  Tiles are laid out expert
// after expert; entries past the last tile are (-1, 0), and the number of
// valid tiles is stored after the table, at tiles[2 * max_tiles].  One
// thread per expert writes its own tiles after a scan of the tile counts.
// Workgroup y builds table y (the up and down projections may use different
// tile heights).
__global__ __launch_bounds__(kScanThreads) void tile_table(int32_t* __restrict__ offsets, int M,
                                                          TileTables tt,
                                                          const int32_t* __restrict__ sorted_slot,
                                                          const float* __restrict__ w, int64_t S,
                                                          float* __restrict__ row_scale,
                                                          int64_t extra,
                                                          int32_t* __restrict__ sorted_token) {
    __shared__ int32_t s_warp[kScanThreads / 64];
    if (blockIdx.x > 0) {
        // blocks 1.. of row y = 0: the down projection's row scales,
        // row_scale[r] = w[sorted_slot[r]] (gate weight of each sorted row),
        // and the extra group's rows: every token once, scale 1
        if (blockIdx.y != 0) return;
        const int64_t r = (int64_t)(blockIdx.x - 1) * kScanThreads + threadIdx.x;
        if (r < S) {
            const int32_t f = sorted_slot[r];
            row_scale[r] = f >= 0 ? w[f] : 0.f;
        } else if (r < S + extra) {
            row_scale[r] = 1.f;
            sorted_token[r] = (int32_t)(r - S);
        }
        return;
    }
    build_tiles(offsets, M, extra, tt.bm[blockIdx.y], tt.max_tiles[blockIdx.y],
                tt.tiles[blockIdx.y], blockIdx.y == 0, s_warp);
}

}  // namespace

hipError_t launch_perm_count(hipStream_t s, const int32_t* idx, int32_t* hist, int64_t T, int k,
                             int64_t M) {
    const int nblk = (int)((T + kPermBlock - 1) / kPermBlock);
    hipLaunchKernelGGL(perm_count, dim3(nblk), dim3(kPermBlock), M * sizeof(int32_t), s, idx,
                       hist, (int)T, k, (int)M);
    return hipGetLastError();
}

hipError_t launch_perm_scan(hipStream_t s, int32_t* hist, int64_t nblk, int64_t T, int k,
                            int64_t M, int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                            int32_t* sorted_slot) {
    hipLaunchKernelGGL(perm_scan, dim3(1), dim3(kScanThreads), 0, s, hist, (int)nblk, (int)T, k,
                       (int)M, counts, offsets, sorted_token, sorted_slot);
    return hipGetLastError();
}

hipError_t launch_perm_scatter(hipStream_t s, const int32_t* idx, const int32_t* hist,
                               const int32_t* offsets, int64_t T, int k, int64_t M,
                               int32_t* sorted_token, int32_t* sorted_slot, int32_t* slot_row) {
    const int nblk = (int)((T + kPermBlock - 1) / kPermBlock);
    hipLaunchKernelGGL(perm_scatter, dim3(nblk), dim3(kPermBlock),
                       4 * M * sizeof(unsigned long long), s, idx, hist, offsets, (int)T, k,
                       (int)M, sorted_token, sorted_slot, slot_row);
    return hipGetLastError();
}

hipError_t launch_tile_table(hipStream_t s, int32_t* offsets, int64_t M, const TileTables& tt,
                             int count, const int32_t* sorted_slot, const float* w, int64_t S,
                             float* row_scale, int64_t extra, int32_t* sorted_token) {
    if (M + (extra > 0 ? 1 : 0) > kScanThreads) return hipErrorInvalidValue;
    const unsigned rs_blocks = (unsigned)((S + extra + kScanThreads - 1) / kScanThreads);
    hipLaunchKernelGGL(tile_table, dim3(1 + rs_blocks, count), dim3(kScanThreads), 0, s, offsets,
                       (int)M, tt, sorted_slot, w, S, row_scale, extra, sorted_token);
    return hipGetLastError();
}

size_t perm_small_lds(int64_t M) {
    return (size_t)(kScanThreads / 64) * M * sizeof(unsigned long long) + M * sizeof(int32_t);
}

hipError_t launch_perm_small(hipStream_t s, const int32_t* idx, int64_t T, int k, int64_t M,
                             int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                             int32_t* sorted_slot, int32_t* slot_row, const TileTables* tt,
                             int ntables, const float* w, float* row_scale, int64_t extra) {
    if (ntables > 0 && (!tt || ntables > 2 || M + (extra > 0 ? 1 : 0) > kScanThreads))
        return hipErrorInvalidValue;
    const TileTables none{};
    hipLaunchKernelGGL(perm_small, dim3(1), dim3(kScanThreads), perm_small_lds(M), s, idx, (int)T,
                       k, (int)M, counts, offsets, sorted_token, sorted_slot, slot_row,
                       ntables > 0 ? *tt : none, ntables, w, row_scale, extra);
    return hipGetLastError();
}

}  // namespace moe
