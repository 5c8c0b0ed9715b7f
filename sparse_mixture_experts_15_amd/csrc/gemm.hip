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
//   backward (bf16; the chain rule of the same steps):
//   up + save:      H as above, and the pre-activations Z (bf16)
//   dH (DH_*):      dZ[r] = act'(Z[r]) * w[slot(r)] * (dy[tok(r)] . W2[e])
//                   plus per-tile partial dots H . dH_raw for the gate gradient
//   dX (fp32):      dX[r] = dZ[r] . W1[e]                 (W2, W1 read as [K, N])
//   weight grads:   dW[e] = A_e^T B_e over expert e's rows (wgrad_bf16)
//
// bf16 path: workgroup tiles of BM A rows x 256 B rows (BM = 64, 128, 160
// or 256, chosen per GEMM from the rows per group), eight waves on
// v_mfma_f32_16x16x32_bf16, each wave 64 B rows x BM/2 A rows.  Operands
// stream through an LDS ring of K = 64 stages (2-5 deep, up to 160 KB)
// filled by buffer loads that write LDS directly, with explicit vmcnt waits
// and one barrier per stage; in 256-row tiles whose fragments all hold rows
// each wave reads the next fragment group from LDS among the current
// group's MFMAs, an order pinned with scheduling-group barriers.
// Out-of-range rows and the K tail read as zeros
// through the buffer bounds.  LDS rows carry an XOR chunk swizzle
// (conflict-free 16-byte fragment reads, measured).  A rows of the up
// projection are gathered on load through the sorted token list, so the
// permuted activations are never materialised.  For SwiGLU each wave's 64 B
// rows are 32 gate rows and the 32 matching up rows, so silu(gate) * up is
// formed in registers.  B may be row-major, tiled (one contiguous block per
// 256-row tile and stage) or [K, N] (the backward's weights, read in place
// through transposed LDS reads).  Tiles are taken in groups of a few m-tiles
// x all n-tiles, dealt to the XCDs in an order chosen per GEMM, so the
// workgroups resident on one XCD share operand K slabs in its L2.  fp32
// path: a plain SIMT tile kernel (64 x 64, K step 16).
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

// Output column and B row of B-tile row b.  SWIGLU tiles hold half as many
// output columns: per 64-row block (one wave's B rows), 32 gate rows then
// their 32 up rows.
template <int EPI>
__device__ __forceinline__ void brow_map(int b, int n_base, int F_split, int& out_col,
                                         int& b_row) {
    if (epi_pairs(EPI)) {
        const int wb = b >> 6, within = b & 63;
        out_col = n_base + 32 * wb + (within & 31);
        b_row = out_col + ((within >> 5) ? F_split : 0);
    } else {
        out_col = n_base + b;
        b_row = out_col;
    }
}

// ------------------------------------------------------------ bf16 / MFMA

constexpr int BK = 64;       // default K per pipeline stage: 128-byte row segments
constexpr int NT = 512;      // 8 waves: 2 (rows) x 4 (B rows)
constexpr uint32_t kOOB = 0x80000000u;   // byte offset past every buffer: loads zero

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t* lds_u32_ptr;

// Raw buffer load of 16 bytes per lane straight into LDS (lane l writes the
// 16 bytes at lds + 16 l); an offset at or past the buffer size reads zeros.
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(i32x4 rsrc, lds_u32_ptr lds, int size,
                                                           int voffset, int soffset, int offset,
                                                           int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;   // raw buffer, 32-bit data format
    return r;
}

// s_waitcnt vmcnt(n) leaving the other counters untouched (gfx9 encoding:
// vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14, expcnt bits 6:4,
// lgkmcnt bits 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Wait until at most `later` (0 .. STAGES-2) stages of L loads each are
// still in flight.
template <int L, int STAGES>
__device__ __forceinline__ void wait_stages(int later) {
    if constexpr (STAGES >= 5) {
        if (later >= 3) {
            wait_vmcnt<3 * L>();
            return;
        }
    }
    if constexpr (STAGES >= 4) {
        if (later >= 2) {
            wait_vmcnt<2 * L>();
            return;
        }
    }
    if constexpr (STAGES >= 3) {
        if (later >= 1) {
            wait_vmcnt<L>();
            return;
        }
    }
    wait_vmcnt<0>();
}

// LDS tile rows are KS bf16 (KS = 64: 128 bytes, 8 chunks of 16 bytes;
// KS = 32: 64 bytes, 4 chunks).  Chunk c of row r lives at chunk
// c ^ (r & 7) (128-byte rows) or c ^ ((r >> 1) & 3) (64-byte rows).
// Measured on gfx950 these make the 16-byte MFMA fragment reads (16 rows x
// 4 chunks per wave) conflict-free, as fast as contiguous reads; unswizzled
// or padded rows run at half rate.
template <int KS>
__device__ __forceinline__ int swz_chunk(int row) {
    return KS == 64 ? (row & 7) : ((row >> 1) & 3);
}
template <int KS>
__device__ __forceinline__ int swz(int row, int c) {
    return row * KS + ((c ^ swz_chunk<KS>(row)) << 3);
}

// Workgroup order.  Tiles are taken in groups of group_m m-tiles with all
// n-tiles inside a group, so the ~32 workgroups one XCD runs at a time
// cover a few m-tiles x several n-tiles and share both operands' K slabs in
// that XCD's L2.  Hardware hands consecutive workgroup ids to the eight
// XCDs in turn; mode 0 deals whole groups to the XCDs in turn as well (XCD
// x runs groups x, x + 8, ...), which keeps each group on one XCD and
// spreads the groups of a grouped GEMM, whose cost varies with the rows
// its experts received, evenly over the XCDs; with fewer than 64 groups
// (fewer than 8 per XCD, e.g. a decode batch's few dozen experts) whole
// groups cannot be spread evenly, and mode 0 falls back to the hardware
// order.  Mode 2 gives each XCD one contiguous eighth of the tiles, mode 1
// keeps the hardware order.  Ids past the valid tiles return false.
// `m_tiles` is the number of valid m-tiles; the grid holds grid_tiles() ids.
__device__ __forceinline__ bool tile_coords(int m_tiles, int n_tiles, int group_m, int p, int& mt,
                                            int& nt, int mode = 0) {
    const int G = m_tiles * n_tiles;
    const int gsz = group_m * n_tiles;
    int first, in;
    if (mode == 0 && (m_tiles + group_m - 1) / group_m < 64) mode = 1;
    if (mode == 0) {
        const int x = p & 7, i = p >> 3;
        const int grp = x + 8 * (i / gsz);
        first = grp * group_m;
        in = i - (i / gsz) * gsz;
        if (first >= m_tiles) return false;
    } else {
        if (p >= G) return false;
        const int per = G / 8;
        if (mode == 2 && p < per * 8) p = (p & 7) * per + (p >> 3);
        const int group = p / gsz;
        first = group * group_m;
        in = p - group * gsz;
    }
    const int gsize = min(m_tiles - first, group_m);
    if (in >= gsize * n_tiles) return false;
    mt = first + in % gsize;
    nt = in / gsize;
    return true;
}

// Packed halves of two output fragments (f0, f1) of a wave row -> one
// 16-byte piece per lane.  Lane l holds columns 4 c .. 4 c + 3 (c = l / 16)
// of each fragment; v_permlane16_swap trades the odd 16-lane rows of its
// first operand for the even rows of its second, so a lane with c even keeps
// its own f0 columns and receives the next four from lane l + 16, and a lane
// with c odd keeps its own f1 columns and receives the four before them from
// lane l - 16.  The piece starts at column 4 c (c even) or 16 + 4 (c - 1) (c
// odd) of the pair, so the four lanes of a row cover its 32 columns with
// 64 contiguous bytes (fp16 / bf16), half the store instructions.
__device__ __forceinline__ uint4 pair_to_piece(uint32_t x0, uint32_t y0, uint32_t x1,
                                               uint32_t y1) {
    const auto sx = __builtin_amdgcn_permlane16_swap(x0, x1, false, false);
    const auto sy = __builtin_amdgcn_permlane16_swap(y0, y1, false, false);
    return uint4{sx[0], sy[0], sx[1], sy[1]};
}
__device__ __forceinline__ int piece_col(int lane) {
    return 4 * (lane >> 4) + 12 * ((lane >> 4) & 1);
}

// Largest value over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes
// holding one fragment row).  Each swap hands every lane its partner's value
// beside its own, in VALU instructions rather than LDS-routed permutes.
__device__ __forceinline__ float row_max4(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the same four lanes, each pair added as x + (partner's x): the
// values and rounding of the two __shfl_xor steps it replaces.
__device__ __forceinline__ float row_sum4(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t w = __float_as_uint(x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Backward epilogue of the down projection's input gradient (EPI_DH_*): the
// accumulator is dH_raw = dy . W2[e] for sorted row r and output column n
// (an expert-width column).  With the row's gate weight w (row_w, or 1 for
// the shared expert) dH = w dH_raw passes through the activation's
// derivative at the saved pre-activations (c2) into the bf16 gradient of
// the up projection's output (c: SwiGLU [rows, 2N] gate then up, GELU
// [rows, N]).  The weight gradient's dot dw = H . dH_raw over the columns
// is summed per row over the wave's columns (lanes of a row meet by
// shuffles) and stored per (row, n-tile, wave) in part, without atomics.
template <int EPI, int TM, int TN, int WROWS, int WN>
__device__ __forceinline__ void dh_epilogue(const GemmArgs& g, const Tile& tl,
                                            const floatx4 (&acc)[TM][TN], int wlive, int wm,
                                            int wn, int n_base, int nt, int lane) {
    const int N = g.N;
    const int lr = lane & 15, lc = 4 * (lane >> 4);
    const bf16_t* zp = static_cast<const bf16_t*>(g.c2);
    const bf16_t* hp = static_cast<const bf16_t*>(g.aux);
    bf16_t* out = static_cast<bf16_t*>(g.c);
    const bool vec = (N % 4) == 0;   // 8-byte aligned 4-column groups
    const int nw = n_base + 64 * wn;
    if (TN == 4 && (N % 8) == 0 && nw + 64 <= N) {
        // The wave's whole 64-column segment on 16-byte aligned rows.  Each
        // row's weight, pre-activations and H are loaded before the previous
        // row's outputs are stored (its inputs are spent by then), so a load
        // never waits behind those stores (memory operations retire in
        // order); outputs go out as paired 16-byte pieces.  Same arithmetic
        // as the general path below.
        constexpr bool SW = EPI == EPI_DH_SWIGLU;
        const int64_t ldz = SW ? 2 * (int64_t)N : (int64_t)N;
        const int64_t rlast = (int64_t)tl.rend - 1;
        uint2 zg[TN], zu[TN], hh[TN];
        float wnext = 1.f;
        auto load_row = [&](int i) {   // rows past the tile re-read its last row
            const int64_t r = min(tl.r0 + wm * WROWS + 16 * i + lr, rlast);
            wnext = g.row_w ? g.row_w[r] : 1.f;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = nw + 16 * j + lc;
                zg[j] = *reinterpret_cast<const uint2*>(zp + r * ldz + n);
                if constexpr (SW) zu[j] = *reinterpret_cast<const uint2*>(zp + r * ldz + N + n);
                hh[j] = hp ? *reinterpret_cast<const uint2*>(hp + r * N + n) : uint2{0u, 0u};
            }
        };
        if (wlive > 0) load_row(0);
        const int pc = piece_col(lane);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= wlive) continue;   // wave-uniform
            const int64_t r = tl.r0 + wm * WROWS + 16 * i + lr;
            const bool rv = r < tl.rend;
            const float wr = wnext;
            float pw = 0.f;
            uint32_t ox[2][TN], oy[2][TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const float hv[4] = {__uint_as_float(hh[j].x << 16),
                                     __uint_as_float(hh[j].x & 0xffff0000u),
                                     __uint_as_float(hh[j].y << 16),
                                     __uint_as_float(hh[j].y & 0xffff0000u)};
                const float z0[4] = {__uint_as_float(zg[j].x << 16),
                                     __uint_as_float(zg[j].x & 0xffff0000u),
                                     __uint_as_float(zg[j].y << 16),
                                     __uint_as_float(zg[j].y & 0xffff0000u)};
                float o[2][4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float a = acc[i][j][q];
                    if (hp) pw += hv[q] * a;
                    if constexpr (SW) {
                        const float dh = wr * a;
                        const uint32_t uw = (q < 2) ? zu[j].x : zu[j].y;
                        const float up = __uint_as_float((q & 1) ? (uw & 0xffff0000u) : (uw << 16));
                        o[0][q] = dh * up * silu_grad_f32(z0[q]);
                        o[1][q] = dh * silu_f32(z0[q]);
                    } else {
                        o[0][q] = wr * a * gelu_grad_f32(z0[q]);
                    }
                }
#pragma unroll
                for (int h = 0; h < (SW ? 2 : 1); ++h) {
                    ox[h][j] = pack_bf16x2(o[h][0], o[h][1]);
                    oy[h][j] = pack_bf16x2(o[h][2], o[h][3]);
                }
            }
            if (i + 1 < wlive) load_row(i + 1);
#pragma unroll
            for (int h = 0; h < (SW ? 2 : 1); ++h) {
#pragma unroll
                for (int pp = 0; pp < TN / 2; ++pp) {
                    const uint4 piece = pair_to_piece(ox[h][2 * pp], oy[h][2 * pp],
                                                      ox[h][2 * pp + 1], oy[h][2 * pp + 1]);
                    if (rv)
                        *reinterpret_cast<uint4*>(out + r * ldz + h * N + nw + 32 * pp + pc) = piece;
                }
            }
            pw = row_sum4(pw);
            if (rv && g.part && lane < 16) g.part[r * g.part_ld + nt * WN + wn] = pw;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (i >= wlive) continue;   // wave-uniform
        const int64_t r = tl.r0 + wm * WROWS + 16 * i + lr;
        const bool rv = r < tl.rend;
        float pw = 0.f;
        if (rv) {
            const float wr = g.row_w ? g.row_w[r] : 1.f;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n_base + 64 * wn + 16 * j + lc;
                if (vec && n + 4 <= N) {
                    float hv[4] = {0.f, 0.f, 0.f, 0.f}, o[2][4];
                    if (hp) load_bf16x4(hp + r * N + n, hv);
                    if (EPI == EPI_DH_SWIGLU) {
                        float gt[4], up[4];
                        load_bf16x4(zp + r * 2 * N + n, gt);
                        load_bf16x4(zp + r * 2 * N + N + n, up);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float a = acc[i][j][q], dh = wr * a;
                            if (hp) pw += hv[q] * a;
                            o[0][q] = dh * up[q] * silu_grad_f32(gt[q]);
                            o[1][q] = dh * silu_f32(gt[q]);
                        }
                        store_bf16x4(out + r * 2 * N + n, o[0][0], o[0][1], o[0][2], o[0][3]);
                        store_bf16x4(out + r * 2 * N + N + n, o[1][0], o[1][1], o[1][2], o[1][3]);
                    } else {
                        float z[4];
                        load_bf16x4(zp + r * N + n, z);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float a = acc[i][j][q];
                            if (hp) pw += hv[q] * a;
                            o[0][q] = wr * a * gelu_grad_f32(z[q]);
                        }
                        store_bf16x4(out + r * N + n, o[0][0], o[0][1], o[0][2], o[0][3]);
                    }
                    continue;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (n + q >= N) continue;
                    const float a = acc[i][j][q];
                    if (hp) pw += bf16_to_f32(hp[r * N + n + q]) * a;
                    const float dh = wr * a;
                    if (EPI == EPI_DH_SWIGLU) {
                        const float gt = bf16_to_f32(zp[r * 2 * N + n + q]);
                        const float up = bf16_to_f32(zp[r * 2 * N + N + n + q]);
                        out[r * 2 * N + n + q] = f32_to_bf16(dh * up * silu_grad_f32(gt));
                        out[r * 2 * N + N + n + q] = f32_to_bf16(dh * silu_f32(gt));
                    } else {
                        const float z = bf16_to_f32(zp[r * N + n + q]);
                        out[r * N + n + q] = f32_to_bf16(dh * gelu_grad_f32(z));
                    }
                }
            }
        }
        pw += __shfl_xor(pw, 16);
        pw += __shfl_xor(pw, 32);
        if (rv && g.part && lane < 16) g.part[r * g.part_ld + nt * WN + wn] = pw;
    }
}

// Epilogue of the forward and save epilogues, straight from registers.  The
// MFMAs take the B fragment as their first operand, so for fragment (i, j)
// lane l holds tile row 16 i + l % 16 of its wave and the four consecutive
// fragment columns 4 (l / 16) .. +3: one 8-byte (bf16) or 16-byte (fp32)
// store each.  The four lanes of a row write 32 / 64 contiguous bytes, and a
// row's fragments fill whole cache lines in L2.  kg / kc_id: the K group or
// split-K chunk whose output block this tile writes.
template <int EPI, int TM, int TN, int WROWS>
__device__ __forceinline__ void out_epilogue(const GemmArgs& g, const Tile& tl,
                                             const floatx4 (&acc)[TM][TN], int wlive, int wm,
                                             int wn, int n_base, int kg, int kc_id, int lane,
                                             const float (&wpre)[TM]) {
    const int N = g.N;
    const int lr = lane & 15, lc = 4 * (lane >> 4);
    const bf16_t* bias = static_cast<const bf16_t*>(g.bias);
    constexpr bool SAVE = (EPI == EPI_SWIGLU_SAVE || EPI == EPI_GELU_SAVE);
    constexpr bool OUT_BF16 = (EPI == EPI_SWIGLU || EPI == EPI_GELU || SAVE);
    constexpr bool HAS_BIAS = (EPI == EPI_GELU || EPI == EPI_GELU_SAVE || EPI == EPI_DOWN_SCALED);
    constexpr int OUT_FR = epi_pairs(EPI) ? TN / 2 : TN;   // output fragments per row
    constexpr int OUT_W = epi_pairs(EPI) ? 32 : 64;        // output columns per wave
    const bool vec = (N % 4) == 0;                              // aligned 4-column groups
    const bool HAS_BIAS_RT = HAS_BIAS && bias != nullptr;
    float bv[OUT_FR][4];
#pragma unroll
    for (int j = 0; j < OUT_FR; ++j) {
        const int n = n_base + OUT_W * wn + 16 * j + lc;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bv[j][q] = (HAS_BIAS && bias && n + q < N)
                           ? bf16_to_f32(bias[(int64_t)tl.e * N + n + q]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        if (i >= wlive) continue;
        const int64_t r = tl.r0 + wm * WROWS + 16 * i + lr;
        if (r >= tl.rend) continue;
        float wr = 1.f;
        if (EPI == EPI_DOWN_SCALED) wr = wpre[i];
        if constexpr (EPI == EPI_DOWN_SCALED) {
            if (g.c16) {
                // compact rows: the four lanes holding this row's 64 columns
                // agree on a power-of-two scale that puts the group's largest
                // finite magnitude in [2^14, 2^15) (exponent read from its
                // bits), then each stores its values scaled (exactly) and
                // rounded once to fp16
                static_assert(OUT_W == kRowGroup, "one scale per wave row segment");
                const int G = (N + kRowGroup - 1) / kRowGroup;
                const int n0 = n_base + OUT_W * wn;
                // every column of this wave's segment exists (wave-uniform)
                const bool full = vec && n0 + OUT_W <= N;
                if (full && !HAS_BIAS_RT) {
                    // Whole segment, no bias: the largest |wr a| is |wr| times
                    // the largest |a| (rounding is monotonic), and wr a 2^-e
                    // rounds to (wr 2^-e) a exactly while wr 2^-e stays a
                    // normal float, so one scaled weight serves the segment
                    // with the general path's bits (except products below
                    // the fp32 normal range, rounded once here, twice there).
                    float ma = 0.f;
#pragma unroll
                    for (int j = 0; j < OUT_FR; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) ma = fmaxf(ma, fabsf(acc[i][j][q]));
                    ma = row_max4(ma);
                    const float mw = fabsf(wr) * ma;
                    const int bw = (int)((__float_as_uint(mw) >> 23) & 0xffu);
                    const int ew = min(max(bw - 127 - 14, -128), 113);
                    const float sw = ldexpf(wr, -ew);
                    const float asw = fabsf(sw);
                    // uniform over the four lanes: same row, same maximum
                    if (mw <= 3.402823466e38f &&
                        (sw == 0.f || (asw >= 1.175494351e-38f && asw <= 3.402823466e38f))) {
                        if ((N % 8) == 0) {   // 16-byte aligned rows: paired pieces
                            uint32_t px[OUT_FR], py[OUT_FR];
#pragma unroll
                            for (int j = 0; j < OUT_FR; ++j) {
                                px[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sw * acc[i][j][0])) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sw * acc[i][j][1])) << 16);
                                py[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sw * acc[i][j][2])) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sw * acc[i][j][3])) << 16);
                            }
                            const int pc = piece_col(lane);
#pragma unroll
                            for (int h = 0; h < OUT_FR / 2; ++h)
                                *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g.c16) + r * N + n0 +
                                                          32 * h + pc) =
                                    pair_to_piece(px[2 * h], py[2 * h], px[2 * h + 1], py[2 * h + 1]);
                            if (lc == 0) g.cexp[r * G + n0 / kRowGroup] = (int8_t)ew;
                            continue;
                        }
#pragma unroll
                        for (int j = 0; j < OUT_FR; ++j) {
                            const int n = n0 + 16 * j + lc;
                            uint2 pk;
                            pk.x = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sw * acc[i][j][0])) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sw * acc[i][j][1])) << 16);
                            pk.y = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sw * acc[i][j][2])) |
                                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(sw * acc[i][j][3])) << 16);
                            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c16) + r * N + n) = pk;
                        }
                        if (lc == 0) g.cexp[r * G + n0 / kRowGroup] = (int8_t)ew;
                        continue;
                    }
                }
                float v[OUT_FR][4];
                float m = 0.f;
                if (full && !HAS_BIAS_RT) {
#pragma unroll
                    for (int j = 0; j < OUT_FR; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            v[j][q] = wr * acc[i][j][q];
                            m = fmaxf(m, fabsf(v[j][q]));
                        }
                } else {
#pragma unroll
                    for (int j = 0; j < OUT_FR; ++j) {
                        const int n = n0 + 16 * j + lc;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            v[j][q] = n + q < N ? wr * (acc[i][j][q] + bv[j][q]) : 0.f;
                            m = fmaxf(m, fabsf(v[j][q]));
                        }
                    }
                }
                // fmaxf skips NaNs; an infinity would set the scale, so then
                // the maximum is taken again over the finite values only
                m = row_max4(m);
                if (!(m <= 3.402823466e38f)) {   // uniform over the four lanes
                    m = 0.f;
#pragma unroll
                    for (int j = 0; j < OUT_FR; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float a = fabsf(v[j][q]);
                            if (a <= 3.402823466e38f) m = fmaxf(m, a);
                        }
                    m = row_max4(m);
                }
                const int be = (int)((__float_as_uint(m) >> 23) & 0xffu);   // biased exponent
                const int e = min(max(be - 127 - 14, -128), 113);
#pragma unroll
                for (int j = 0; j < OUT_FR; ++j) {
                    const int n = n0 + 16 * j + lc;
                    if (!full && n >= N) continue;
                    uint16_t hv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        hv[q] = __builtin_bit_cast(uint16_t, (_Float16)ldexpf(v[j][q], -e));
                    uint16_t* dst = static_cast<uint16_t*>(g.c16) + r * N + n;
                    if (full || (vec && n + 4 <= N)) {
                        uint2 pk;
                        pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
                        pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
                        *reinterpret_cast<uint2*>(dst) = pk;
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (n + q < N) dst[q] = hv[q];
                    }
                }
                if (lc == 0 && n0 < N) g.cexp[r * G + n0 / kRowGroup] = (int8_t)e;
                continue;
            }
        }
        if constexpr (OUT_BF16 && !SAVE) {
            // whole bf16 segment on 16-byte aligned rows: paired pieces
            const int nw = n_base + OUT_W * wn;
            if ((N % 8) == 0 && nw + OUT_W <= N) {
                uint32_t px[OUT_FR], py[OUT_FR];
#pragma unroll
                for (int j = 0; j < OUT_FR; ++j) {
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (EPI == EPI_SWIGLU)
                            v[q] = silu_f32(acc[i][j][q]) * acc[i][j + 2][q];
                        else
                            v[q] = gelu_erf_f32(acc[i][j][q] + bv[j][q]);
                    }
                    px[j] = pack_bf16x2(v[0], v[1]);
                    py[j] = pack_bf16x2(v[2], v[3]);
                }
                const int pc = piece_col(lane);
#pragma unroll
                for (int h = 0; h < OUT_FR / 2; ++h)
                    *reinterpret_cast<uint4*>(static_cast<bf16_t*>(g.c) + r * N + nw + 32 * h + pc) =
                        pair_to_piece(px[2 * h], py[2 * h], px[2 * h + 1], py[2 * h + 1]);
                continue;
            }
        }
#pragma unroll
        for (int j = 0; j < OUT_FR; ++j) {
            const int n = n_base + OUT_W * wn + 16 * j + lc;
            if (n >= N) continue;
            float v[4];
            if constexpr (SAVE) {
                // pre-activations for the backward: gate and up (SwiGLU, row
                // stride 2N) or z = acc + b1 (GELU, row stride N), bf16
                bf16_t* zp = static_cast<bf16_t*>(g.c2);
                if (vec && n + 4 <= N) {
                    const floatx4 a0 = acc[i][j];
                    if (EPI == EPI_SWIGLU_SAVE) {
                        const floatx4 a1 = acc[i][j + 2];
                        store_bf16x4(zp + r * 2 * N + n, a0[0], a0[1], a0[2], a0[3]);
                        store_bf16x4(zp + r * 2 * N + N + n, a1[0], a1[1], a1[2], a1[3]);
                    } else {
                        store_bf16x4(zp + r * N + n, a0[0] + bv[j][0], a0[1] + bv[j][1],
                                     a0[2] + bv[j][2], a0[3] + bv[j][3]);
                    }
                } else
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (n + q >= N) continue;
                    if (EPI == EPI_SWIGLU_SAVE) {
                        zp[r * 2 * N + n + q] = f32_to_bf16(acc[i][j][q]);
                        zp[r * 2 * N + N + n + q] = f32_to_bf16(acc[i][j + 2][q]);
                    } else {
                        zp[r * N + n + q] = f32_to_bf16(acc[i][j][q] + bv[j][q]);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE)
                    v[q] = silu_f32(acc[i][j][q]) * acc[i][j + 2][q];
                else if (EPI == EPI_GELU || EPI == EPI_GELU_SAVE)
                    v[q] = gelu_erf_f32(acc[i][j][q] + bv[j][q]);
                else if (EPI == EPI_DOWN_SCALED) v[q] = wr * (acc[i][j][q] + bv[j][q]);
                else v[q] = acc[i][j][q];
            }
            if constexpr (OUT_BF16) {
                bf16_t* dst = static_cast<bf16_t*>(g.c) + r * N + n;
                if (vec && n + 4 <= N) {
                    uint2 pk;
                    pk.x = pack_bf16x2(v[0], v[1]);
                    pk.y = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2*>(dst) = pk;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (n + q < N) dst[q] = f32_to_bf16(v[q]);
                }
            } else {
                float* dst = static_cast<float*>(g.c) +
                             (g.koff ? (int64_t)kg * g.c_group_stride
                                     : (int64_t)kc_id * g.dense_rows * N) +
                             r * N + n;
                if (vec && n + 4 <= N) {
                    *reinterpret_cast<floatx4*>(dst) = floatx4{v[0], v[1], v[2], v[3]};
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (n + q < N) dst[q] = v[q];
                }
            }
        }
    }
}

// One tile configuration: BM A rows x BNB B rows per workgroup, STAGES LDS
// stages of K = KS (64 or 32); the eight waves form WM x WN with 64 B rows
// per wave.
// KN-layout B operand (BKN): B[e] is stored [K][N] row-major (the layout
// the backward finds the weights in: W2[e] = [D][F] against dy, W1[e] =
// [G F][D] against dZ), so no transposed copy is made.  A stage's B tile is
// 64 K-rows of BNB columns in LDS, 16-byte chunk c of row k stored at chunk
// c ^ kn_swz(k); the MFMA B fragments (8 consecutive k of one column per
// lane) come from pairs of ds_read_b64_tr_b16.  That instruction works on
// groups of 16 lanes: lane i of a group receives element i % 4 of the
// 8-byte pieces addressed by lanes 4 j + i / 4 (j = 0..3) of its group, so
// lane 4 j + q addressing columns n0 + 4 q .. +3 of k-row k0 + j hands lane
// i the four k values k0 .. k0 + 3 of column n0 + i (measured on gfx950).
template <int BNB>
__device__ __forceinline__ int kn_swz(int krow) {
    return (krow % (BNB / 16)) * 2;   // even: keeps a fragment's two chunks adjacent
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t* lds_s4_ptr;

template <int BNB>
__device__ __forceinline__ bf16x8 kn_fragment(const bf16_t* bt, int kbase, int n0, int lane) {
    const int grp = lane >> 4, L = lane & 15, q = L & 3, jr = L >> 2;
    const int n = n0 + 4 * q;
    const int c = n >> 3, half = (n >> 2) & 1;
    short4_t v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = kbase + 8 * grp + 4 * h + jr;
        const bf16_t* p = bt + k * BNB + ((c ^ kn_swz<BNB>(k)) << 3) + half * 4;
        v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)p);
    }
    typedef short short8_t __attribute__((ext_vector_type(8)));
    const short8_t r = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
    return __builtin_bit_cast(bf16x8, r);
}

// The multiply of one K = 64 stage of a 256 x 256 tile whose fragments all
// hold rows: eight waves, each 128 A rows (wave row wm) x 64 B rows (wave
// column wn), accumulators acc[8][4]; the A rows sit at the stage's start,
// the 256 B rows after them (row-major, or [K, N] when BKN).
struct NoIssue {
    __device__ void operator()() const {}
};
// `issue` enqueues the next stage's global loads; it runs after the first
// fragment reads, so their LDS latency overlaps the loads' issue instead of
// following it.
template <int BNB, int BKN, typename Issue = NoIssue>
__device__ __forceinline__ void mfma_stage_full256(const bf16_t* st, floatx4 (&acc)[8][4], int wm,
                                                   int wn, int lane, Issue&& issue = Issue{}) {
    constexpr int BM = 256, BK = 64, TN = 4, WROWS = 128;
    const int fr = lane & 15, fc = lane >> 4;
    // 256-row tiles, whole fragments: each K half's rows 0-3 then
    // 4-7, the next group's fragments read among the current
    // group's MFMAs (pinned with scheduling groups; 22 more VGPRs
    // than reading per K half, no spills).  Measured against the
    // general body on one device: GLM-5-shaped routed up projection
    // 7.56 -> 7.11 ms, GLM-4.5-shaped 2.29 -> 2.13 ms, its backward
    // 15.1 -> 14.7 ms; outputs bitwise equal.
    constexpr int RB = BKN ? 2 : 1;   // LDS reads per weight fragment
    bf16x8 b0[TN], b1[TN], a00[4], a01[4], a10[4], a11[4];
    auto rdB = [&](int kk, bf16x8(&bb)[TN]) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if constexpr (BKN)
                bb[j] = kn_fragment<BNB>(st + BM * BK, kk * 32, wn * 64 + 16 * j, lane);
            else
                bb[j] = *reinterpret_cast<const bf16x8*>(
                    st + BM * BK + swz<BK>(wn * 64 + 16 * j + fr, kk * 4 + fc));
        }
    };
    auto rdA = [&](int kk, int i0, bf16x8(&aa)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            aa[i] = *reinterpret_cast<const bf16x8*>(
                st + swz<BK>(wm * WROWS + 16 * (i0 + i) + fr, kk * 4 + fc));
    };
    auto mm = [&](int i0, const bf16x8(&aa)[4], const bf16x8(&bb)[TN]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i0 + i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    bb[j], aa[i], acc[i0 + i][j], 0, 0, 0);
    };
    rdB(0, b0);
    rdA(0, 0, a00);
    __builtin_amdgcn_sched_group_barrier(0x100, TN * RB + 4, 0);
    issue();
    rdA(0, 4, a01);
    mm(0, a00, b0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    rdB(1, b1);
    rdA(1, 0, a10);
    mm(4, a01, b0);
    if constexpr (BKN) {   // 12 reads among 16 MFMAs
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    } else {   // 8 reads among 16 MFMAs
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
    rdA(1, 4, a11);
    mm(0, a10, b1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    mm(4, a11, b1);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
}

template <int EPI, int BM, int BNB, int STAGES, int KS, int BKN = 0>
__global__ __launch_bounds__(NT, 1) void gemm_bf16(GemmArgs g, int m_tiles, int n_tiles) {
    static_assert(!BKN || (KS == 64 && !epi_pairs(EPI)), "KN-layout B: K = 64 stages, no pairing");
    constexpr int BK = KS;
    constexpr int CPR = BK / 8;                        // 16-byte chunks per row
    constexpr int ROWS_PER_LOAD = 1024 / (BK * 2);     // rows per 1 KB wave load
    constexpr int A_LOADS = BM / ROWS_PER_LOAD;
    constexpr int B_LOADS = BNB / ROWS_PER_LOAD;
    constexpr int LOADS = A_LOADS + B_LOADS;
    // load ins = wave + 8 q: the first B_LOADS fill B blocks, the rest A
    // blocks; when LOADS % 8 != 0 the first LOADS % 8 waves issue one more
    constexpr int LPW = (LOADS + 7) / 8;               // most loads of a wave per stage
    constexpr int LPW_LO = LOADS / 8;
    constexpr int QB = B_LOADS / 8;                    // loads q < QB are B loads
    constexpr int STAGE = (BM + BNB) * BK;             // bf16 elements per stage
    constexpr int WN = BNB / 64, WM = 8 / WN;          // wave grid
    constexpr int WROWS = BM / WM;                     // A rows per wave
    constexpr int TM = WROWS / 16;                     // 16-row fragments per wave
    constexpr int TN = 4;                              // 16-column fragments per wave
    static_assert(BM % 16 == 0 && B_LOADS % 8 == 0, "whole fragments; B loads split evenly");
    static_assert(WM * WN == 8 && TM >= 1 && WROWS % 16 == 0, "eight waves");
    static_assert(STAGES >= 2 && STAGES <= 5 && LPW * (STAGES - 2) < 64, "pipeline depth");
    static_assert(BK == 64 || BK == 32, "stage depth");
    __shared__ __attribute__((aligned(1024))) bf16_t sm[STAGES * STAGE];

    // grouped: the valid m-tile count follows the tile table
    const int m_valid = g.tiles ? min(m_tiles, g.tiles[2 * m_tiles]) : m_tiles;
    // split-K (dense fp32 output only): chunk kc of g.k_split covers a K range
    const int nsplit = g.k_split > 1 ? g.k_split : 1;
    int kc_id = 0, kg = 0, p = (int)blockIdx.x, mt, nt;
    if (g.koff) {       // K-grouped: group-major ids, plain order inside a group
        kg = p / max(m_valid * n_tiles, 1);
        if (kg >= g.kgroups) return;
        p -= kg * m_valid * n_tiles;
    } else if (nsplit > 1) {   // split-K: chunk-major ids, plain order inside a chunk
        kc_id = p / max(m_valid * n_tiles, 1);
        if (kc_id >= nsplit) return;
        p -= kc_id * m_valid * n_tiles;
    }
    if (!tile_coords(m_valid, n_tiles, g.group_m > 0 ? g.group_m : 4, p, mt, nt,
                     (nsplit > 1 || g.koff) ? 1 : g.xcd_mode))
        return;
    Tile tl;
    if (!tile_of(g, mt, BM, tl)) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN;
    const int K = g.K, N = g.N;
    const int out_per_tile = epi_pairs(EPI) ? BNB / 2 : BNB;
    const int n_base = nt * out_per_tile;

    // buffer descriptors: A rows (whole activation matrix), B = this expert
    const int64_t a_rows = g.gather ? g.a_rows : tl.rend;
    const i32x4 ra = make_rsrc(g.a, (uint32_t)(a_rows * K * 2));
    const bf16_t* Bp = (g.b_extra && tl.e == g.extra_group)
                           ? static_cast<const bf16_t*>(g.b_extra)
                           : static_cast<const bf16_t*>(g.b) + (int64_t)tl.e * g.b_stride;
    const i32x4 rb = make_rsrc(
        Bp, (uint32_t)((g.b_tiled || BKN ? g.b_stride : (int64_t)g.b_rows * K) * 2));
    // tiled weights: stage kt of a 256-row weight tile is one contiguous
    // block of 256 LDS-image rows; a 128-row n-tile takes half of one
    constexpr uint32_t TILE_STAGE = kTileRows * BK * 2;
    const uint32_t tile_base =
        (uint32_t)(nt * BNB / kTileRows) * (uint32_t)((K + BK - 1) / BK) * TILE_STAGE +
        (uint32_t)(nt * BNB % kTileRows) * (BK * 2);

    // Load q of wave w (ins = w + 8 q) fills ROWS_PER_LOAD rows: B rows of
    // block ins for q < QB, else A rows of block ins - B_LOADS; lane l -> row
    // l / CPR of the block, stored chunk l % CPR, which holds the logical
    // chunk given by the swizzle.  Invalid rows get offset kOOB.
    const int lrow = lane / CPR, pc = lane % CPR;
    // blocks start at multiples of 8 rows, so the swizzle depends on lrow only
    const int lchunk = pc ^ swz_chunk<BK>(lrow);
    uint32_t rowoff[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
        const int ins = wave + 8 * q;
        if (q >= QB) {
            const int64_t r = tl.r0 + ROWS_PER_LOAD * (ins - B_LOADS) + lrow;
            uint32_t off = kOOB;
            if (ins < LOADS && r < tl.rend)
                off = (uint32_t)((g.gather ? (int64_t)g.gather[r] : r) * K * 2);
            rowoff[q] = off;
        } else if (BKN) {
            // k-row kn_row(q) of the stage, stored chunk lane % CPRn holding
            // the logical chunk given by the swizzle; column base per lane
            constexpr int CPRn = BNB / 8, RPLn = 64 / CPRn;
            const int krow = RPLn * ins + lane / CPRn;
            const int col = n_base + ((lane % CPRn) ^ kn_swz<BNB>(krow)) * 8;
            rowoff[q] = col < N ? (uint32_t)krow * (uint32_t)N * 2u + (uint32_t)col * 2u : kOOB;
        } else if (g.b_tiled) {
            // tiled weights: this lane's 16 bytes of stage 0; stage kt is
            // TILE_STAGE bytes further (and past K reads zeros, as the A
            // rows there do)
            rowoff[q] = tile_base + (uint32_t)ins * 1024u + lane * 16u;
        } else {
            const int row = ROWS_PER_LOAD * ins + lrow;
            int oc, br;
            brow_map<EPI>(row, n_base, g.F_split, oc, br);
            rowoff[q] = oc < N ? (uint32_t)br * (uint32_t)K * 2u + (uint32_t)lchunk * 16u : kOOB;
        }
        if (q >= QB) rowoff[q] += (uint32_t)lchunk * 16u;   // stays >= kOOB when invalid
    }
    // bytes from one stage to the next: row-major operands move BK columns,
    // tiled weights one whole stage block (wave-uniform)
    const uint32_t bstep = g.b_tiled ? TILE_STAGE : (uint32_t)BK * 2u;
    // load q of this wave for stage kt: offset = rowoff + kt * step, no
    // branch per load
    auto issue_q = [&](int kt, int q) {
        bf16_t* st = sm + (kt % STAGES) * STAGE;
        const int kc = kt * BK + lchunk * 8;
        {
            const int ins = wave + 8 * q;
            // an invalid row stays >= kOOB (offsets are < 2^31); a K-tail chunk -> kOOB
            uint32_t off = rowoff[q] + (uint32_t)kt * (q < QB ? bstep : (uint32_t)BK * 2u);
            off = kc < K ? off : kOOB;
            if (BKN && q < QB) {   // KN-layout B: whole k-rows of the stage
                constexpr int CPRn = BNB / 8, RPLn = 64 / CPRn;
                const int krow = kt * BK + RPLn * ins + lane / CPRn;
                off = krow < K ? rowoff[q] + (uint32_t)(kt * BK) * (uint32_t)N * 2u : kOOB;
            }
            if (q < QB)
                llvm_amdgcn_raw_buffer_load_lds(rb, (lds_u32_ptr)(st + BM * BK + ins * 512), 16,
                                                (int)off, 0, 0, 0);
            else if (q < LPW_LO || ins < LOADS)   // wave-uniform
                llvm_amdgcn_raw_buffer_load_lds(ra, (lds_u32_ptr)(st + (ins - B_LOADS) * 512), 16,
                                                (int)off, 0, 0, 0);
        }
    };
    auto issue = [&](int kt) {
#pragma unroll
        for (int q = 0; q < LPW; ++q) issue_q(kt, q);
    };

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // 16-row fragments of this wave that hold valid rows: a group's last tile
    // is usually partial, and fragments past its end skip their LDS reads and
    // MFMAs (wave-uniform branches).
    const int valid_rows = (int)min<int64_t>(tl.rend - tl.r0, (int64_t)BM);
    const int wlive = min(TM, max(0, (valid_rows - wm * WROWS + 15) / 16));
    // the down projection's row weights, loaded before the K loop so that
    // their latency hides behind the first stage's
    float wpre[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t r = tl.r0 + wm * WROWS + 16 * i + (lane & 15);
        wpre[i] = (EPI == EPI_DOWN_SCALED && g.row_w && i < wlive && r < tl.rend) ? g.row_w[r]
                                                                                  : 1.f;
    }

    // STAGES-deep ring: stages kt+1 .. kt+STAGES-1 load while stage kt is
    // multiplied.  With split-K this workgroup runs stages [k_first, k_last).
    const int nk_all = (K + BK - 1) / BK;
    const int k_first = g.koff ? g.koff[kg] / BK : (int)((int64_t)nk_all * kc_id / nsplit);
    const int k_last = g.koff ? g.koff[kg + 1] / BK : (int)((int64_t)nk_all * (kc_id + 1) / nsplit);
    const int nk = k_last - k_first;
#pragma unroll
    for (int s0 = 0; s0 < STAGES - 1; ++s0)
        if (s0 < nk) issue(k_first + s0);
    const int fr = lane & 15, fc = lane >> 4;
    auto kloop = [&](auto&& body) {
        for (int kt = 0; kt < nk; ++kt) {
            // stage kt has landed once only later stages' loads are pending
            const int later = min(nk - 1, kt + STAGES - 2) - kt;
            if (LPW == LPW_LO || wave < LOADS % 8) wait_stages<LPW, STAGES>(later);
            else wait_stages<LPW_LO, STAGES>(later);
            __builtin_amdgcn_s_barrier();     // every wave's loads landed; stage kt-1 fully read
            const bool more = kt + STAGES - 1 < nk;
            const int next = k_first + kt + STAGES - 1;
            const bf16_t* st = sm + ((k_first + kt) % STAGES) * STAGE;
            body(st, [&] {
                if (more) issue(next);
            });
        }
    };
    // the multiply of one stage for 256-row tiles whose fragments all hold rows
    auto body_full256 = [&](const bf16_t* st, auto&& pre) {
        if constexpr (TM == 8 && BK == 64)
            mfma_stage_full256<BNB, BKN>(st, acc, wm, wn, lane, pre);
    };
    // the multiply of one stage in general (fragments past the group's
    // last row skip their reads and MFMAs)
    auto body_general = [&](const bf16_t* st, auto&& pre) {
        pre();
        if (TM <= 4 && wlive == TM) {
            // whole fragments: one straight block (every fragment read, then
            // the MFMAs) the scheduler can overlap freely.  Measured faster
            // with 4 row fragments per wave; with 5 slower and with 8 the
            // doubled fragment registers spill, so larger tiles keep the
            // path below.
            bf16x8 af[BK / 32][TM], bfr[BK / 32][TN];
#pragma unroll
            for (int kk = 0; kk < BK / 32; ++kk) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[kk][i] = *reinterpret_cast<const bf16x8*>(
                        st + swz<BK>(wm * WROWS + 16 * i + fr, kk * 4 + fc));
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (BKN)
                        bfr[kk][j] = kn_fragment<BNB>(st + BM * BK, kk * 32, wn * 64 + 16 * j, lane);
                    else
                        bfr[kk][j] = *reinterpret_cast<const bf16x8*>(
                            st + BM * BK + swz<BK>(wn * 64 + 16 * j + fr, kk * 4 + fc));
                }
            }
#pragma unroll
            for (int kk = 0; kk < BK / 32; ++kk)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[kk][j], af[kk][i],
                                                                            acc[i][j], 0, 0, 0);
            return;
        }
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            if (wlive > 0) {
                bf16x8 af[TM], bfr[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int row = wm * WROWS + 16 * i + fr;
                    if (i < wlive)
                        af[i] = *reinterpret_cast<const bf16x8*>(st + swz<BK>(row, kk * 4 + fc));
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int row = wn * 64 + 16 * j + fr;
                    if constexpr (BKN)
                        bfr[j] = kn_fragment<BNB>(st + BM * BK, kk * 32, wn * 64 + 16 * j, lane);
                    else
                        bfr[j] = *reinterpret_cast<const bf16x8*>(
                            st + BM * BK + swz<BK>(row, kk * 4 + fc));
                }
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if (i < wlive) {
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i],
                                                                                acc[i][j], 0, 0, 0);
                    }
                }
            }
        }
    };
    // wlive is fixed for the whole loop, so the two bodies get loops of
    // their own (in one loop their registers add up and spill)
    if constexpr (TM == 8 && BK == 64) {
        if (wlive == TM) kloop(body_full256);
        else kloop(body_general);
    } else {
        kloop(body_general);
    }

    // Epilogue straight from registers (out_epilogue / dh_epilogue).  Every
    // load has landed by now, so this wait costs nothing; without it the
    // compiler cannot prove that the row weights loaded before the K loop
    // have arrived and waits for all memory operations at each one's first
    // use, which also drains the stores of the previous fragment rows.
    wait_vmcnt<0>();
    if constexpr (EPI == EPI_DH_SWIGLU || EPI == EPI_DH_GELU) {
        dh_epilogue<EPI, TM, TN, WROWS, WN>(g, tl, acc, wlive, wm, wn, n_base, nt, lane);
    } else {
        out_epilogue<EPI, TM, TN, WROWS>(g, tl, acc, wlive, wm, wn, n_base, kg, kc_id, lane,
                                          wpre);
    }
}

// Scalar (wave-uniform) load of p[index] through the constant address
// space: tracked by lgkmcnt, so it never waits for pending vector-memory
// stores or buffer-to-LDS loads.  The data is written by earlier kernels
// only; the caller keeps index in range.
typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
__device__ __forceinline__ int32_t sload(const void* p, int64_t index) {
    return ((const_i32_ptr)p)[index];
}

// Weight-gradient GEMM: C[kg][r, n] = sum over group kg's K range of
// A[r, k] B[n, k] (bf16 in, fp32 out; A [rows, K] and B [N, K] row-major;
// koff gives each group's K range in multiples of 64, or one group covers
// [0, K)).  The general kernel's dense/K-grouped path without its row
// gather, tiled or KN operands, pairing and split-K: 256 x 256 tiles, K = 64
// stages two deep, 170 VGPRs.  Measured against the general kernel on the
// same tiles: GLaM expert weight gradients 8.72 -> 8.23 ms, GLM-4.5 6.54 ->
// 5.97 ms.  Variants that measured slower: two workgroups per CU on
// 128 x 256 tiles of K = 32 stages (one storing while the other multiplies:
// 9.75 ms), a persistent grid loading the next tile before storing the last
// (9.37 ms), non-temporal stores (10.7 ms).  These products are bound by
// their fp32 stores: 17.2 GB per GLaM weight at 6.1 TB/s (the rate a pure
// write of the same tiles in the same order reaches) would be 2.8 ms.
template <int BM, int BNB, int BK, int STAGES>
__global__ __launch_bounds__(NT, 1) void wgrad_bf16(GemmArgs g, int m_tiles, int n_tiles) {
    constexpr int CPR = BK / 8, RPL = 1024 / (BK * 2);   // chunks per row, rows per wave load
    constexpr int A_LOADS = BM / RPL, B_LOADS = BNB / RPL, LOADS = A_LOADS + B_LOADS;
    static_assert(LOADS % 8 == 0 && B_LOADS % 8 == 0, "loads split evenly over the waves");
    constexpr int LPW = LOADS / 8, QB = B_LOADS / 8;
    constexpr int STAGE = (BM + BNB) * BK;
    constexpr int WN = BNB / 64, WM = 8 / WN, WROWS = BM / WM, TM = WROWS / 16, TN = 4;
    static_assert(WM * WN == 8 && WROWS % 16 == 0, "eight waves, whole fragments");
    static_assert(STAGES >= 2 && STAGES <= 4 && (BK == 32 || BK == 64), "ring");
    __shared__ __attribute__((aligned(1024))) bf16_t sm[STAGES * STAGE];

    const int per_group = m_tiles * n_tiles;
    const int kg = (int)blockIdx.x / per_group;
    int mt, nt;
    tile_coords(m_tiles, n_tiles, g.group_m > 0 ? g.group_m : 4,
                (int)blockIdx.x - kg * per_group, mt, nt, 1);
    const int k0 = g.koff ? sload(g.koff, kg) / BK : 0;
    const int nk = g.koff ? sload(g.koff, kg + 1) / BK - k0 : (g.K + BK - 1) / BK;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int K = g.K, N = g.N;
    const int64_t rows = g.dense_rows;
    const i32x4 ra = make_rsrc(g.a, (uint32_t)(rows * K * 2));
    const i32x4 rb = make_rsrc(g.b, (uint32_t)((int64_t)N * K * 2));
    // load q of this wave (ins = wave + 8 q): B rows of block ins for q < QB,
    // else A rows of block ins - B_LOADS; lane -> row lane / CPR of the
    // block, stored chunk lane % CPR (blocks start at multiples of RPL rows,
    // so the swizzle depends on the lane's row only); rows past the end read
    // zeros
    const int lrow = lane / CPR, lchunk = (lane % CPR) ^ swz_chunk<BK>(lrow);
    uint32_t rowoff[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
        const int ins = wave + 8 * q;
        if (q >= QB) {
            const int64_t r = (int64_t)mt * BM + RPL * (ins - B_LOADS) + lrow;
            rowoff[q] = r < rows ? (uint32_t)(r * K * 2) : kOOB;
        } else {
            const int n = nt * BNB + RPL * ins + lrow;
            rowoff[q] = n < N ? (uint32_t)n * (uint32_t)K * 2u : kOOB;
        }
    }
    auto issue = [&](int s) {   // stage s of this tile into ring slot s % STAGES
        bf16_t* st = sm + (s % STAGES) * STAGE;
        const int kc = (k0 + s) * BK + lchunk * 8;
#pragma unroll
        for (int q = 0; q < LPW; ++q) {
            const int ins = wave + 8 * q;
            const uint32_t off = kc < K ? rowoff[q] + (uint32_t)kc * 2u : kOOB;
            if (q < QB)
                llvm_amdgcn_raw_buffer_load_lds(rb, (lds_u32_ptr)(st + BM * BK + ins * 512), 16,
                                                (int)off, 0, 0, 0);
            else
                llvm_amdgcn_raw_buffer_load_lds(ra, (lds_u32_ptr)(st + (ins - B_LOADS) * 512), 16,
                                                (int)off, 0, 0, 0);
        }
    };

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < STAGES - 1; ++s0)
        if (s0 < nk) issue(s0);
    const int fr = lane & 15, fc = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
        wait_stages<LPW, STAGES>(min(nk - 1, kt + STAGES - 2) - kt);
        __builtin_amdgcn_s_barrier();   // every wave's loads landed; stage kt-1 fully read
        if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
        const bf16_t* st = sm + (kt % STAGES) * STAGE;
        if constexpr (BM == 256 && BNB == 256 && BK == 64) {
            mfma_stage_full256<BNB, 0>(st, acc, wm, wn, lane);   // rows past the end read zeros
        } else {
#pragma unroll
            for (int kk = 0; kk < BK / 32; ++kk) {
                bf16x8 af[TM], bfr[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = *reinterpret_cast<const bf16x8*>(
                        st + swz<BK>(wm * WROWS + 16 * i + fr, kk * 4 + fc));
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bfr[j] = *reinterpret_cast<const bf16x8*>(
                        st + BM * BK + swz<BK>(wn * 64 + 16 * j + fr, kk * 4 + fc));
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i],
                                                                            acc[i][j], 0, 0, 0);
            }
        }
    }
    // results straight from the accumulators: lane l holds row 16 i + l % 16
    // of its wave and columns 4 (l / 16) .. +3 of fragment j
    const int lr = lane & 15, lc = 4 * (lane >> 4);
    const bool vec = (N % 4) == 0;
    float* C = static_cast<float*>(g.c) + (int64_t)kg * g.c_group_stride;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t r = (int64_t)mt * BM + wm * WROWS + 16 * i + lr;
        if (r >= rows) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = nt * BNB + 64 * wn + 16 * j + lc;
            if (n >= N) continue;
            float* dst = C + r * N + n;
            if (vec && n + 4 <= N) {
                *reinterpret_cast<floatx4*>(dst) = acc[i][j];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (n + q < N) dst[q] = acc[i][j][q];
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
    const float* B = (g.b_extra && tl.e == g.extra_group)
                         ? static_cast<const float*>(g.b_extra)
                         : static_cast<const float*>(g.b) + (int64_t)tl.e * g.b_stride;

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
            const float wr = (EPI == EPI_DOWN_SCALED && g.row_w) ? g.row_w[r] : 1.f;
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

// Workgroups to launch for m_tiles x n_tiles tiles (m_tiles may bound the
// valid count from above): mode 0 deals whole groups to the eight XCDs in
// turn, so the grid is rounded up to eight groups.
int64_t grid_tiles(const GemmArgs& g, int64_t m_tiles, int64_t n_tiles) {
    if (g.koff) return m_tiles * n_tiles * g.kgroups;
    if (g.k_split > 1) return m_tiles * n_tiles * g.k_split;
    if (g.xcd_mode != 0) return m_tiles * n_tiles;
    const int64_t gm = g.group_m > 0 ? g.group_m : 4;
    const int64_t groups = (m_tiles + gm - 1) / gm;
    return ((groups + 7) / 8) * 8 * gm * n_tiles;
}

template <int EPI, int BMv, int BNv, int STv, int KS = 64, int BKN = 0>
hipError_t launch_bf16(hipStream_t s, const GemmArgs& g, int64_t m_tiles) {
    const int opt = epi_pairs(EPI) ? BNv / 2 : BNv;
    const int n_tiles = (g.N + opt - 1) / opt;
    if (g.k_split > (g.K + BK - 1) / BK) return hipErrorInvalidValue;   // each K chunk needs a stage
    if (g.b_tiled && (KS != kTileK || kTileRows % BNv != 0)) return hipErrorInvalidValue;
    const int64_t total = grid_tiles(g, m_tiles, n_tiles);
    if (BKN && g.b_tiled) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16<EPI, BMv, BNv, STv, KS, BKN>), dim3((unsigned)total), dim3(NT), 0, s,
                       g, (int)m_tiles, n_tiles);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_one(hipStream_t s, int dtype, int bm, const GemmArgs& g, int64_t m_tiles) {
    if (m_tiles <= 0) return hipSuccess;
    if (dtype == 1) {
        if constexpr (EPI == EPI_DH_SWIGLU || EPI == EPI_DH_GELU || EPI == EPI_DOWN_F32) {
            if (g.b_kn) {
                if (bm == 256) return launch_bf16<EPI, 256, 256, 2, 64, 1>(s, g, m_tiles);
                if (bm == 160) return launch_bf16<EPI, 160, 256, 3, 64, 1>(s, g, m_tiles);
                if (bm == 64) return launch_bf16<EPI, 64, 128, 5, 64, 1>(s, g, m_tiles);
                return launch_bf16<EPI, 128, 256, 3, 64, 1>(s, g, m_tiles);
            }
        } else {
            if (g.b_kn) return hipErrorInvalidValue;
        }
        // (256 x 256 with K = 32 stages, 4 or 5 deep, measured slower than 2 x 64)
        if (bm == 256) return launch_bf16<EPI, 256, 256, 2>(s, g, m_tiles);
        if (bm == 160) return launch_bf16<EPI, 160, 256, 3>(s, g, m_tiles);
        if (bm == 64) {   // down projections: 256 B rows, 4 stages (160 KB)
            if constexpr (EPI == EPI_DOWN_SCALED) return launch_bf16<EPI, 64, 256, 4>(s, g, m_tiles);
            else return launch_bf16<EPI, 64, 128, 5>(s, g, m_tiles);
        }
        return launch_bf16<EPI, 128, 256, 3>(s, g, m_tiles);
    }
    if constexpr (EPI > EPI_DOWN_F32) {
        return hipErrorInvalidValue;   // the backward epilogues are bf16 only
    } else {
        const int opt = (EPI == EPI_SWIGLU) ? FBN / 2 : FBN;
        dim3 grid((unsigned)((g.N + opt - 1) / opt), (unsigned)m_tiles);
        hipLaunchKernelGGL(gemm_f32<EPI>, grid, dim3(256), 0, s, g);
        return hipGetLastError();
    }
}

}  // namespace

// Tile height.  A group's weights stream from HBM once per m-tile of the
// group, so when groups hold about a tile of rows (weight-bound: ~2 flops
// per weight byte per row) the tile should cover a whole group with the
// deepest ring that fits: 160-row tiles (3 stages) take groups of up to 160
// rows, enough for a mean of ~128 rows under uniform routing.  Far smaller
// groups leave most of any tile empty, and 128-row tiles waste the least;
// for groups of a few rows (decode) the up projection takes 64 x 128 tiles
// with a 5-stage ring, twice the workgroups over the same weights, which
// evens out the last round of workgroups (GLM-4.5 decode up projection
// 0.29 -> 0.26 ms), and the down projection (K = expert width) 64 x 256
// tiles with a 4-stage ring, three stages of weights in flight (decode
// layer 0.4542-0.4550 -> 0.4524-0.4531 ms against 128 x 256 x 3; 64 x 128
// tiles were slower there).
// Groups of hundreds of rows are MFMA-bound: 256-row tiles halve the LDS
// traffic per MFMA and take the scheduled full-tile K loop, for the down
// projection too (GLM-4.5 prefill down projection 1.51 -> 1.30 ms against
// 128-row tiles, GLM-5 4.62 -> 4.01 ms).  Dense GEMMs take 256-row tiles
// when that still gives every CU a workgroup (GLM-4.5 shared expert: up
// 0.42 -> 0.32 ms, down 0.79 -> 0.39 ms); the router's narrow logit GEMM
// keeps 128-row tiles.  Measured on MI355X over the layer shapes the tests
// use.
int gemm_block_m(int dtype, int64_t rows, int64_t groups, bool down, int64_t b_rows,
                 int request) {
    if (dtype != 1) return FBM;
    if (request == 64 || request == 128 || request == 160 || request == 256) return request;
    if (groups <= 1) {
        const int64_t tiles256 = (rows / 256) * ((b_rows + 255) / 256);
        return tiles256 >= 256 ? 256 : 128;
    }
    const int64_t avg = rows / groups;
    if (avg <= 16) return 64;
    if (avg <= 96) return 128;
    if (avg <= 136) return 160;
    return 256;
}

int gemm_group_m(int64_t rows, int64_t groups, int bm, int request, bool down) {
    if (request >= 1 && request <= 16) return request;
    // Grouped down projections deal whole groups to the XCDs; one m-tile
    // per group spreads the experts' uneven tiles over the XCDs in finer
    // pieces, at the price of more L2 misses (more fabric traffic, the
    // same or lower time): GLM-4.5 prefill down projection 1.150-1.160 ->
    // 1.134 ms, GLM-5 3.63-3.64 -> 3.57 ms against two m-tiles per group
    // (the up projections, in hardware order, lose with one: 1.93 -> 2.07).
    if (down && groups > 1) return 1;
    const int64_t per = (rows / (groups > 0 ? groups : 1) + bm / 2) / bm;
    return per < 1 ? 1 : per > 4 ? 4 : (int)per;
}

// Workgroup order of a GEMM (tile_coords modes).  Grouped up projections
// keep the hardware order: their tiles' cost follows the rows each expert
// received, and dealing single tiles to the XCDs in turn balances them
// best; measured faster than per-XCD groups by ~1% (GLM-4.5 prefill) to 9%
// (GLM-5, Zipf-skewed).  An up projection over one group (a single-expert
// layer) has no such skew and gives each XCD a contiguous eighth of the
// tiles (dense GLM-4.5-shaped prefix layer 3.15 -> 2.92 ms).  The grouped
// down projections and the dense GEMMs deal whole groups to the XCDs, which
// keeps a group's operand slabs in one L2 (GLM-4.5 down projection on
// 128-row tiles 1.34 ms against 1.61 ms in hardware order; on 256-row tiles
// the two orders are within 1%).
int gemm_xcd_mode(bool grouped, bool down, bool one_group, int request) {
    // request: 1 groups dealt to the XCDs (mode 0), 2 hardware order (mode
    // 1), 3 contiguous eighths (mode 2)
    if (request >= 1 && request <= 3) return request - 1;
    if (grouped && !down) return one_group ? 2 : 1;
    return 0;
}

// Weight-gradient GEMM (wgrad_bf16): rows = g.dense_rows, one group per
// g.koff entry (g.kgroups groups, outputs g.c_group_stride apart) or one
// dense group.
hipError_t launch_wgrad(hipStream_t s, const GemmArgs& g) {
    constexpr int BM = 256, BNB = 256;
    const int64_t m_tiles = (g.dense_rows + BM - 1) / BM, n_tiles = ((int64_t)g.N + BNB - 1) / BNB;
    const int64_t groups = g.koff ? g.kgroups : 1;
    const int64_t total = m_tiles * n_tiles * groups;
    if (total <= 0) return hipSuccess;
    if (total >= ((int64_t)1 << 31) || g.dense_rows * g.K * 2 >= ((int64_t)1 << 31) ||
        (int64_t)g.N * g.K * 2 >= ((int64_t)1 << 31) || g.b_tiled || g.b_kn || g.gather ||
        g.k_split > 1 || (g.koff && g.kgroups <= 0))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((wgrad_bf16<BM, BNB, 64, 2>), dim3((unsigned)total), dim3(NT), 0, s, g,
                       (int)m_tiles, (int)n_tiles);
    return hipGetLastError();
}

hipError_t launch_gemm(hipStream_t s, int dtype, int bm, int epi, const GemmArgs& g,
                       int64_t m_tiles) {
    switch (epi) {
        case EPI_SWIGLU: return launch_one<EPI_SWIGLU>(s, dtype, bm, g, m_tiles);
        case EPI_GELU: return launch_one<EPI_GELU>(s, dtype, bm, g, m_tiles);
        case EPI_DOWN_SCALED: return launch_one<EPI_DOWN_SCALED>(s, dtype, bm, g, m_tiles);
        case EPI_SWIGLU_SAVE: return launch_one<EPI_SWIGLU_SAVE>(s, dtype, bm, g, m_tiles);
        case EPI_GELU_SAVE: return launch_one<EPI_GELU_SAVE>(s, dtype, bm, g, m_tiles);
        case EPI_DH_SWIGLU: return launch_one<EPI_DH_SWIGLU>(s, dtype, bm, g, m_tiles);
        case EPI_DH_GELU: return launch_one<EPI_DH_GELU>(s, dtype, bm, g, m_tiles);
        default: return launch_one<EPI_DOWN_F32>(s, dtype, bm, g, m_tiles);
    }
}

int gemm_part_cols(int bm, int64_t N) {
    const int bnb = bm == 64 ? 128 : 256;   // the B rows of that tile height's config
    return (int)((N + bnb - 1) / bnb) * (bnb / 64);
}

}  // namespace moe
