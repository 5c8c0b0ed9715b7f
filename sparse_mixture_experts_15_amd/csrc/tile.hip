// The tiled weight layout: every 256-row x 64-element stage of a weight tile
// stored as one contiguous block in the order the grouped GEMM holds it in
// LDS (row b of 64 elements, 16-byte chunk c at chunk c ^ (b % 8)), so the
// GEMM's weight loads are plain sequential 32 KB reads.  Row b of tile n is
// the weight row the GEMM's row map gives (SwiGLU: per 64 rows, 32 gate rows
// and the matching 32 up rows).  A one-time copy; rows past the matrix and
// columns past K are written as zeros.
#include "common.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void tile_weights(const uint16_t* __restrict__ src,
                                                    uint16_t* __restrict__ dst, int64_t b_rows,
                                                    int64_t n_out, int64_t K, int swiglu,
                                                    int n_tiles, int n_k) {
    // one workgroup per block (expert e, tile n, stage s); 2048 chunks of 16 bytes
    const int64_t blk = blockIdx.x;
    const int s = (int)(blk % n_k);
    const int n = (int)((blk / n_k) % n_tiles);
    const int64_t e = blk / ((int64_t)n_k * n_tiles);
    const uint16_t* W = src + e * b_rows * K;
    uint16_t* out = dst + blk * (int64_t)kTileRows * kTileK;
    const int per = swiglu ? kTileRows / 2 : kTileRows;   // output columns per tile
    for (int q = threadIdx.x; q < kTileRows * kTileK / 8; q += 256) {
        const int b = q / 8, pc = q % 8;          // row, stored chunk
        const int c = pc ^ (b & 7);               // logical chunk held there
        int64_t col, row;
        if (swiglu) {
            const int g = b / 64, w = b % 64;
            col = (int64_t)n * per + 32 * g + (w % 32);
            row = col + (w >= 32 ? n_out : 0);
        } else {
            col = (int64_t)n * per + b;
            row = col;
        }
        const int64_t k0 = (int64_t)s * kTileK + 8 * c;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (col < n_out && k0 < K) v = *reinterpret_cast<const uint4*>(W + row * K + k0);
        *reinterpret_cast<uint4*>(out + 8 * q) = v;
    }
}

}  // namespace

hipError_t launch_tile_weights(hipStream_t s, const void* src, void* dst, int64_t E,
                               int64_t b_rows, int64_t n_out, int64_t K, bool swiglu) {
    const int64_t per = swiglu ? kTileRows / 2 : kTileRows;
    const int64_t n_tiles = (n_out + per - 1) / per, n_k = (K + kTileK - 1) / kTileK;
    const int64_t blocks = E * n_tiles * n_k;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(tile_weights, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), b_rows,
                       n_out, K, swiglu ? 1 : 0, (int)n_tiles, (int)n_k);
    return hipGetLastError();
}

}  // namespace moe
