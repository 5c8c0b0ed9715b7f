// C ABI of the MoE layer: descriptor validation, workspace plan, stream
// fork/join and kernel launches.  Every check runs before the first
// launch, so an error leaves the outputs and the streams untouched.
#include <algorithm>
#include <mutex>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "common.hpp"

using namespace moe;

namespace {

thread_local std::string g_detail;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_detail = buf;
    return code;
}

const char* kLabels[L_COUNT] = {"route",      "perm_count", "perm_scan",  "perm_scatter",
                                "tile_table", "ffn_up",     "ffn_down",   "shared_up",
                                "shared_down", "combine",   "b_up",       "b_dh",
                                "b_dx",       "b_wgrad",    "b_transpose", "b_other"};

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// Device workspace layout shared by every entry point.
struct Plan {
    // merged: moe_forward runs the shared expert as one more group (index
    // M, every token once) of the routed GEMMs; its rows follow the S routed
    // rows, so Hsh and Ysh are the tails of H and O, and Sx = S + T.
    bool merged = false;
    // compact: moe_forward hands the expert rows from the down projection to
    // the combine as fp16 values with a scale per 64 (in O's space)
    bool compact = false;
    int64_t Sx = 0;
    int64_t S = 0, nblk = 0, max_tiles_up = 0, max_tiles_dn = 0;
    int bm_up = 0, bm_dn = 0, bm_sh_up = 0, bm_sh_dn = 0;
    size_t esz = 0;
    size_t idx = 0, w = 0, counts = 0, offsets = 0, sorted_token = 0, sorted_slot = 0,
           slot_row = 0, hist = 0, row_scale = 0, tiles_up = 0, tiles_dn = 0, H = 0, O = 0, Hsh = 0, Ysh = 0, route = 0,
           total = 0;
};

Plan make_plan(const moe_desc* d, bool allow_merge = true) {
    Plan p;
    p.esz = d->dtype == MOE_DTYPE_BF16 ? 2 : 4;
    p.S = d->T * d->k;
    p.nblk = (d->T + kPermBlock - 1) / kPermBlock;
    const int64_t G = d->act == MOE_ACT_SWIGLU ? 2 : 1;   // up-projection weight rows per F
    // A shared expert of one routed expert's shape joins the routed GEMMs
    // when the batch is decode-sized: alone its GEMMs have a handful of
    // workgroups and only contend with the router on the second stream.
    // shared_mode 1 keeps it separate, 2 merges it wherever the shape allows.
    const bool can_merge = d->F_shared > 0 && d->F_shared == d->F &&
                           d->act == MOE_ACT_SWIGLU && d->dtype == MOE_DTYPE_BF16 &&
                           d->T <= kSmallT && d->M + 1 <= 1024;
    p.merged = allow_merge && can_merge && d->shared_mode != 1;
    p.compact = !p.merged && d->dtype == MOE_DTYPE_BF16 && d->rows_format != 1;
    const int64_t groups = d->M + (p.merged ? 1 : 0);
    p.Sx = p.S + (p.merged ? d->T : 0);
    p.bm_up = gemm_block_m(d->dtype, p.Sx, groups, false, G * d->F, d->tile_rows[MOE_GEMM_UP]);
    p.bm_dn = gemm_block_m(d->dtype, p.Sx, groups, true, d->D, d->tile_rows[MOE_GEMM_DOWN]);
    p.bm_sh_up = gemm_block_m(d->dtype, d->T, 1, false, 2 * d->F_shared,
                              d->tile_rows[MOE_GEMM_SHARED_UP]);
    p.bm_sh_dn = gemm_block_m(d->dtype, d->T, 1, true, d->D, d->tile_rows[MOE_GEMM_SHARED_DOWN]);
    // ceil(Sx / bm) tiles plus at most one partial tile per non-empty group
    const int64_t partial = groups < p.Sx ? groups : p.Sx;
    p.max_tiles_up = (p.Sx + p.bm_up - 1) / p.bm_up + partial;
    p.max_tiles_dn = (p.Sx + p.bm_dn - 1) / p.bm_dn + partial;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    p.idx = take(p.S * 4);
    p.w = take(p.S * 4);
    p.counts = take(d->M * 4);
    p.offsets = take((d->M + 2) * 4);
    p.sorted_token = take(p.Sx * 4);
    p.sorted_slot = take(p.S * 4);
    p.slot_row = take(p.S * 4);
    p.hist = take((size_t)p.nblk * d->M * 4);
    p.row_scale = take(p.Sx * 4);
    p.tiles_up = take(((size_t)p.max_tiles_up * 2 + 1) * 4);
    p.tiles_dn = p.bm_dn == p.bm_up ? p.tiles_up : take(((size_t)p.max_tiles_dn * 2 + 1) * 4);
    if (p.merged) {
        p.H = take((size_t)p.Sx * d->F * p.esz);
        p.Hsh = p.H + (size_t)p.S * d->F * p.esz;
        p.O = take((size_t)p.Sx * d->D * 4);
        p.Ysh = p.O + (size_t)p.S * d->D * 4;
    } else {
        p.H = take((size_t)p.S * d->F * p.esz);
        // fp32 rows, or the compact rows (smaller except at tiny sizes,
        // where the exponents' 256-byte alignment dominates)
        p.O = take(std::max((size_t)p.S * d->D * 4,
                            (size_t)compact_row_bytes(p.S, d->D)));
        p.Hsh = take((size_t)d->T * d->F_shared * p.esz);
        // fp32 shared rows (the stage entry points), or compact ones
        p.Ysh = take(d->F_shared > 0 ? std::max((size_t)d->T * d->D * 4,
                                                (size_t)compact_row_bytes(d->T, d->D))
                                     : 0);
    }
    p.route = take(route_workspace(d->dtype, d->T, d->D, d->M));
    p.total = off;
    return p;
}

int validate(const moe_desc* d) {
    if (!d) return fail(MOE_ERR_INVALID, "descriptor is NULL");
    if (d->T < 0) return fail(MOE_ERR_INVALID, "T=%lld < 0", (long long)d->T);
    if (d->D <= 0 || d->M <= 0 || d->F <= 0 || d->F_shared < 0)
        return fail(MOE_ERR_INVALID, "D, M, F must be > 0 and F_shared >= 0");
    if (d->k < 1 || d->k > d->M)
        return fail(MOE_ERR_INVALID, "k=%d must be in [1, M=%lld]", d->k, (long long)d->M);
    if (d->scorer != MOE_SCORER_SOFTMAX && d->scorer != MOE_SCORER_SIGMOID)
        return fail(MOE_ERR_INVALID, "unknown scorer %d", d->scorer);
    if (d->act != MOE_ACT_SWIGLU && d->act != MOE_ACT_GELU)
        return fail(MOE_ERR_INVALID, "unknown activation %d", d->act);
    if (d->dtype != MOE_DTYPE_F32 && d->dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (d->out_dtype != MOE_DTYPE_F32 && d->out_dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_INVALID, "unknown out_dtype %d", d->out_dtype);
    if (d->renorm != 0 && d->renorm != 1) return fail(MOE_ERR_INVALID, "renorm must be 0 or 1");
    if (d->n_group < 0 || d->topk_group < 0)
        return fail(MOE_ERR_INVALID, "n_group and topk_group must be >= 0");
    if (d->n_group > 1) {
        if (d->n_group > MOE_MAX_GROUPS)
            return fail(MOE_ERR_UNSUPPORTED, "n_group=%d > %d", d->n_group, MOE_MAX_GROUPS);
        if (d->M % d->n_group)
            return fail(MOE_ERR_INVALID, "M=%lld is not a multiple of n_group=%d",
                        (long long)d->M, d->n_group);
        if (d->topk_group < 1 || d->topk_group > d->n_group ||
            (int64_t)d->topk_group * (d->M / d->n_group) < d->k)
            return fail(MOE_ERR_INVALID, "topk_group=%d must be in [1, n_group] and keep >= k "
                        "experts", d->topk_group);
    }
    for (int i = 0; i < 4; ++i) {
        const int r = d->tile_rows[i], o = d->tile_order[i];
        if (r != 0 && r != 64 && r != 128 && r != 160 && r != 256)
            return fail(MOE_ERR_INVALID, "tile_rows[%d]=%d is not 0, 64, 128, 160 or 256", i, r);
        if (o < 0 || o > 3) return fail(MOE_ERR_INVALID, "tile_order[%d]=%d is not in [0, 3]", i, o);
    }
    if (d->group_m < 0 || d->group_m > 16)
        return fail(MOE_ERR_INVALID, "group_m=%d is not in [0, 16]", d->group_m);
    if (d->shared_mode < 0 || d->shared_mode > 2)
        return fail(MOE_ERR_INVALID, "shared_mode=%d is not in [0, 2]", d->shared_mode);
    if (d->rows_format < 0 || d->rows_format > 2)
        return fail(MOE_ERR_INVALID, "rows_format=%d is not in [0, 2]", d->rows_format);
    if (d->rows_format == 2 && d->dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "compact expert rows need a bf16 layer");
    if (d->weight_layout != MOE_LAYOUT_ROWS && d->weight_layout != MOE_LAYOUT_TILED)
        return fail(MOE_ERR_INVALID, "unknown weight_layout %d", d->weight_layout);
    if (d->weight_layout == MOE_LAYOUT_TILED && d->dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "the tiled weight layout is bf16 only");
    if (!(d->eps >= 0.f) || d->alpha != d->alpha)
        return fail(MOE_ERR_INVALID, "eps must be >= 0 and alpha a number");
    if (d->k > MOE_MAX_K) return fail(MOE_ERR_UNSUPPORTED, "k=%d > %d", d->k, MOE_MAX_K);
    if (d->M > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_UNSUPPORTED, "M=%lld > %d", (long long)d->M, MOE_MAX_EXPERTS);
    if (d->D % 8 || d->F % 8 || d->F_shared % 8)
        return fail(MOE_ERR_UNSUPPORTED, "D, F and F_shared must be multiples of 8");
    const int64_t lim = 0x7fffffffLL;
    if (d->T * (int64_t)d->k > lim || d->T > lim / 2)
        return fail(MOE_ERR_UNSUPPORTED, "T*k exceeds int32 indexing");
    if (d->D > lim / 16 || d->F > lim / 16 || d->F_shared > lim / 16)
        return fail(MOE_ERR_UNSUPPORTED, "D/F too large");
    // bf16 operands are read through 32-bit buffer offsets
    const int64_t G = d->act == MOE_ACT_SWIGLU ? 2 : 1;
    const int64_t S = d->T * (int64_t)d->k;
    if (d->dtype == MOE_DTYPE_BF16 &&
        (d->T * d->D * 2 > lim || S * d->F * 2 > lim || G * d->F * d->D * 2 > lim ||
         d->T * d->F_shared * 2 > lim || 2 * d->F_shared * d->D * 2 > lim))
        return fail(MOE_ERR_UNSUPPORTED, "an operand exceeds 2 GiB");
    if (d->weight_layout == MOE_LAYOUT_TILED &&
        (tiled_elems(d->F, d->D, d->act == MOE_ACT_SWIGLU) * 2 > lim ||
         tiled_elems(d->D, d->F, false) * 2 > lim ||
         tiled_elems(d->F_shared, d->D, true) * 2 > lim ||
         tiled_elems(d->D, d->F_shared, false) * 2 > lim))
        return fail(MOE_ERR_UNSUPPORTED, "a tiled weight matrix exceeds 2 GiB");
    return MOE_OK;
}

// Shape of weight matrix `which`: experts, rows, output columns, K, SwiGLU.
struct WeightShape {
    int64_t E, rows, n_out, K;
    bool swiglu;
};
int weight_shape(const moe_desc* d, int which, WeightShape& ws) {
    const bool sw = d->act == MOE_ACT_SWIGLU;
    switch (which) {
        case MOE_WEIGHT_W1: ws = {d->M, (sw ? 2 : 1) * d->F, d->F, d->D, sw}; return MOE_OK;
        case MOE_WEIGHT_W2: ws = {d->M, d->D, d->D, d->F, false}; return MOE_OK;
        case MOE_WEIGHT_SH_GU: ws = {1, 2 * d->F_shared, d->F_shared, d->D, true}; break;
        case MOE_WEIGHT_SH_DN: ws = {1, d->D, d->D, d->F_shared, false}; break;
        default: return fail(MOE_ERR_INVALID, "unknown weight matrix %d", which);
    }
    if (d->F_shared <= 0) return fail(MOE_ERR_INVALID, "no shared expert (F_shared = 0)");
    return MOE_OK;
}

struct DeviceGuard {
    int prev = -1;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// Fixed device scratch of moe_forward_no_alloc: one copy per GPU, kept until
// the process ends.  Host code never passes the array's name to a kernel or
// a copy (on the host it is only a stand-in for the symbol): it uses the
// device address hipGetSymbolAddress returns, resolved once per device in
// moe_create with that device current.
constexpr size_t kScratchBytes = (size_t)MOE_NO_ALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device `dev` (resolved once).
int scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

struct moe_handle {
    int device = 0;
    void* scratch = nullptr;   // this device's fixed scratch (moe_forward_no_alloc)
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    // profiling
    bool prof_on = false;
    std::string prof_filter;
    std::vector<hipEvent_t> prof_events;   // 2 per record
    std::vector<int> prof_labels;
    int prof_used = 0;
    int64_t launches[L_COUNT] = {};
    double total_ms[L_COUNT] = {};
};

namespace {

// Launch through `fn` with optional timing events around it.
template <class Fn>
int run(moe_handle* h, hipStream_t s, int label, Fn&& fn) {
    const bool rec = h->prof_on && h->prof_used < (int)h->prof_labels.size() &&
                     (h->prof_filter.empty() ||
                      std::strstr(kLabels[label], h->prof_filter.c_str()) != nullptr);
    if (rec) {
        if (hipEventRecord(h->prof_events[2 * h->prof_used], s) != hipSuccess)
            return fail(MOE_ERR_HIP, "hipEventRecord failed");
    }
    const hipError_t e = fn();
    if (e != hipSuccess)
        return fail(MOE_ERR_HIP, "%s launch: %s", kLabels[label], hipGetErrorString(e));
    if (rec) {
        if (hipEventRecord(h->prof_events[2 * h->prof_used + 1], s) != hipSuccess)
            return fail(MOE_ERR_HIP, "hipEventRecord failed");
        h->prof_labels[h->prof_used++] = label;
    }
    return MOE_OK;
}

#define TRY(x)                        \
    do {                              \
        const int _rc = (x);          \
        if (_rc != MOE_OK) return _rc; \
    } while (0)

int check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
    if (ws_bytes < p.total)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, p.total);
    if (p.total > 0 && !ws) return fail(MOE_ERR_INVALID, "workspace pointer is NULL");
    return MOE_OK;
}

template <class T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Stage bodies (no validation).
int do_route(moe_handle* h, const moe_desc* d, const Plan& p, const void* x, const float* W_r,
             const float* bias, int32_t* idx, float* w, void* ws, hipStream_t s) {
    return run(h, s, L_ROUTE, [&] {
        return launch_route(s, d->dtype, d->scorer, x, W_r, bias, idx, w, d->T, d->D, d->M, d->k,
                            d->renorm, d->alpha, d->eps, d->n_group > 1 ? d->n_group : 0,
                            d->topk_group, at<char>(ws, p.route));
    });
}

// The expert GEMMs' tile tables of this plan (up and down tile heights).
TileTables tile_tables(const Plan& p, void* ws, int* ntables) {
    int32_t* tiles_up = at<int32_t>(ws, p.tiles_up);
    int32_t* tiles_dn = at<int32_t>(ws, p.tiles_dn);
    *ntables = tiles_dn == tiles_up ? 1 : 2;
    return TileTables{{p.bm_up, p.bm_dn},
                      {(int)p.max_tiles_up, (int)p.max_tiles_dn},
                      {tiles_up, tiles_dn}};
}

// With w non-null (moe_forward on a batch of at most kSmallT tokens) the
// one-workgroup dispatch also builds the tile tables and row scales that
// do_expert_ffn would otherwise build in a launch of its own (`extra`: the
// merged shared expert's rows); *tables_built reports it.
int do_permute(moe_handle* h, const moe_desc* d, const Plan& p, const int32_t* idx,
               int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* sorted_slot,
               int32_t* slot_row, void* ws, hipStream_t s, const float* w = nullptr,
               int64_t extra = 0, bool* tables_built = nullptr) {
    if (tables_built) *tables_built = false;
    if (d->T <= kSmallT) {
        int ntables = 0;
        TileTables tt{};
        if (w) tt = tile_tables(p, ws, &ntables);
        float* row_scale = w ? at<float>(ws, p.row_scale) : nullptr;
        TRY(run(h, s, L_PERM_SCATTER, [&] {
            return launch_perm_small(s, idx, d->T, d->k, d->M, counts, offsets, sorted_token,
                                     sorted_slot, slot_row, w ? &tt : nullptr, ntables, w,
                                     row_scale, extra);
        }));
        if (tables_built) *tables_built = w != nullptr;
        return MOE_OK;
    }
    int32_t* hist = at<int32_t>(ws, p.hist);
    TRY(run(h, s, L_PERM_COUNT, [&] { return launch_perm_count(s, idx, hist, d->T, d->k, d->M); }));
    TRY(run(h, s, L_PERM_SCAN, [&] {
        return launch_perm_scan(s, hist, p.nblk, d->T, d->k, d->M, counts, offsets, sorted_token,
                                sorted_slot);
    }));
    return run(h, s, L_PERM_SCATTER, [&] {
        return launch_perm_scatter(s, idx, hist, offsets, d->T, d->k, d->M, sorted_token,
                                   sorted_slot, slot_row);
    });
}

// The routed expert GEMMs.  With Wsh_gu / Wsh_dn non-null (a merged plan,
// from moe_forward only, whose sorted_token and offsets live in the
// workspace with room for the extra group) the shared expert runs as group
// M of the same launches, its T rows after the S routed ones.
int do_expert_ffn(moe_handle* h, const moe_desc* d, const Plan& p, const void* x,
                  int32_t* sorted_token, const int32_t* sorted_slot, int32_t* offsets,
                  const float* w, const void* W1, const void* b1, const void* W2, const void* b2,
                  float* O, void* ws, hipStream_t s, const void* Wsh_gu = nullptr,
                  const void* Wsh_dn = nullptr, bool compact = false,
                  bool tables_built = false) {
    const bool merged = Wsh_gu != nullptr;
    const int64_t rows = merged ? p.Sx : p.S;
    int ntables = 0;
    const TileTables tt = tile_tables(p, ws, &ntables);
    int32_t* tiles_up = tt.tiles[0];
    int32_t* tiles_dn = tt.tiles[1];
    void* H = at<char>(ws, p.H);
    float* row_scale = at<float>(ws, p.row_scale);
    if (!tables_built)
        TRY(run(h, s, L_TILE_TABLE, [&] {
            return launch_tile_table(s, offsets, d->M, tt, ntables, sorted_slot, w, p.S,
                                     row_scale, merged ? d->T : 0, sorted_token);
        }));
    const bool swiglu = d->act == MOE_ACT_SWIGLU;
    GemmArgs up{};
    up.a = x;
    up.gather = sorted_token;
    const bool tiled = d->weight_layout == MOE_LAYOUT_TILED;
    up.b = W1;
    up.b_stride = tiled ? tiled_elems(d->F, d->D, swiglu) : (swiglu ? 2 : 1) * d->F * d->D;
    up.b_tiled = tiled;
    up.bias = swiglu ? nullptr : b1;
    up.c = H;
    up.tiles = tiles_up;
    up.dense_rows = rows;
    up.group_m = gemm_group_m(rows, d->M, p.bm_up, d->group_m);
    if (merged) {
        up.b_extra = Wsh_gu;
        up.extra_group = (int)d->M;
    }
    up.xcd_mode = gemm_xcd_mode(true, false, d->M == 1 && !merged, d->tile_order[MOE_GEMM_UP]);
    up.offsets = offsets;
    up.a_rows = d->T;
    up.b_rows = (int)((swiglu ? 2 : 1) * d->F);
    up.K = (int)d->D;
    up.N = (int)d->F;
    up.F_split = (int)d->F;
    TRY(run(h, s, L_FFN_UP, [&] {
        return launch_gemm(s, d->dtype, p.bm_up, swiglu ? EPI_SWIGLU : EPI_GELU, up,
                           p.max_tiles_up);
    }));
    GemmArgs dn{};
    dn.a = H;
    dn.b = W2;
    dn.b_stride = tiled ? tiled_elems(d->D, d->F, false) : d->D * d->F;
    dn.b_tiled = tiled;
    dn.bias = swiglu ? nullptr : b2;
    dn.row_w = row_scale;
    dn.dense_rows = rows;
    dn.c = O;
    if (compact) {   // O's space holds the compact rows instead
        dn.c16 = O;
        dn.cexp = reinterpret_cast<int8_t*>(O) + compact_exp_offset(rows, d->D);
    }
    dn.tiles = tiles_dn;
    dn.group_m = gemm_group_m(rows, d->M, p.bm_dn, d->group_m, true);
    if (merged) {
        dn.b_extra = Wsh_dn;
        dn.extra_group = (int)d->M;
    }
    dn.xcd_mode = gemm_xcd_mode(true, true, false, d->tile_order[MOE_GEMM_DOWN]);
    dn.offsets = offsets;
    dn.a_rows = rows;
    dn.b_rows = (int)d->D;
    dn.K = (int)d->F;
    dn.N = (int)d->D;
    return run(h, s, L_FFN_DOWN,
               [&] { return launch_gemm(s, d->dtype, p.bm_dn, EPI_DOWN_SCALED, dn, p.max_tiles_dn); });
}

// The shared expert; with `compact` its rows go to Ysh's space in the
// compact format of the routed rows (fp16 with a power-of-two scale per 64
// values; moe_forward's combine reads them), else as fp32 rows.
int do_shared(moe_handle* h, const moe_desc* d, const Plan& p, const void* x, const void* Wgu,
              const void* Wdn, float* Ysh, void* ws, hipStream_t s, bool compact = false) {
    void* Hsh = at<char>(ws, p.Hsh);
    const int64_t mt_up = (d->T + p.bm_sh_up - 1) / p.bm_sh_up;
    const int64_t mt_dn = (d->T + p.bm_sh_dn - 1) / p.bm_sh_dn;
    GemmArgs up{};
    up.a = x;
    const bool tiled = d->weight_layout == MOE_LAYOUT_TILED;
    up.b = Wgu;
    up.b_stride = tiled ? tiled_elems(d->F_shared, d->D, true) : 0;
    up.b_tiled = tiled;
    up.c = Hsh;
    up.dense_rows = d->T;
    up.a_rows = d->T;
    up.b_rows = (int)(2 * d->F_shared);
    up.K = (int)d->D;
    up.N = (int)d->F_shared;
    up.F_split = (int)d->F_shared;
    up.xcd_mode = gemm_xcd_mode(false, false, false, d->tile_order[MOE_GEMM_SHARED_UP]);
    TRY(run(h, s, L_SHARED_UP,
            [&] { return launch_gemm(s, d->dtype, p.bm_sh_up, EPI_SWIGLU, up, mt_up); }));
    GemmArgs dn{};
    dn.a = Hsh;
    dn.b = Wdn;
    dn.b_stride = tiled ? tiled_elems(d->D, d->F_shared, false) : 0;
    dn.b_tiled = tiled;
    dn.c = Ysh;
    if (compact) {   // weight 1 (row_w NULL), no bias
        dn.c16 = Ysh;
        dn.cexp = reinterpret_cast<int8_t*>(Ysh) + compact_exp_offset(d->T, d->D);
    }
    dn.dense_rows = d->T;
    dn.a_rows = d->T;
    dn.b_rows = (int)d->D;
    dn.K = (int)d->F_shared;
    dn.N = (int)d->D;
    dn.xcd_mode = gemm_xcd_mode(false, true, false, d->tile_order[MOE_GEMM_SHARED_DOWN]);
    return run(h, s, L_SHARED_DOWN, [&] {
        return launch_gemm(s, d->dtype, p.bm_sh_dn, compact ? EPI_DOWN_SCALED : EPI_DOWN_F32, dn,
                           mt_dn);
    });
}

// With `compact` the expert rows, and the shared rows when present, are in
// the compact format.
int do_combine(moe_handle* h, const moe_desc* d, const float* O, const int32_t* slot_row,
               const float* Ysh, void* y, hipStream_t s, bool compact = false) {
    return run(h, s, L_COMBINE, [&] {
        if (compact)
            return launch_combine_compact(
                s, d->out_dtype, O,
                reinterpret_cast<const int8_t*>(O) + compact_exp_offset(d->T * d->k, d->D),
                slot_row, nullptr, Ysh,
                Ysh ? reinterpret_cast<const int8_t*>(Ysh) + compact_exp_offset(d->T, d->D)
                    : nullptr,
                y, d->T, d->k, d->D);
        return launch_combine(s, d->out_dtype, O, slot_row, Ysh, y, d->T, d->k, d->D);
    });
}

// ------------------------------------------------------------- backward

// Backward workspace: the forward's (unmerged) layout, with H, O, Hsh and
// Ysh reused as H, the expert rows' input gradients dXs [S, D] fp32, Hsh and
// the shared expert's dXsh [T, D] fp32, followed by the backward's own
// regions.  Spad = S + 64 M, rounded up to 64, bounds the per-expert padded
// positions.
struct BwdPlan {
    Plan f;
    int64_t S = 0, G = 1, Spad = 0, Tp = 0;
    int part_ld = 0, bm_w2 = 0, bm_w1 = 0, bm_sh2 = 0, bm_sh1 = 0, bm_r = 0;
    size_t Z = 0, dZ = 0, part = 0, Zsh = 0, dZsh = 0, poff = 0, pad_row = 0, pad_tok = 0, dOT = 0, HT = 0, dZT = 0, XT = 0,
           xT = 0, dyT = 0, HshT = 0, dZshT = 0, dl = 0, gate = 0, dlT3 = 0, C3 = 0, total = 0;
};

BwdPlan make_bwd_plan(const moe_desc* d) {
    BwdPlan b;
    b.f = make_plan(d, false);
    const int64_t T = d->T, D = d->D, M = d->M, F = d->F, Fs = d->F_shared;
    b.S = T * d->k;
    b.G = d->act == MOE_ACT_SWIGLU ? 2 : 1;
    b.Spad = ((b.S + 64 * M + 63) / 64) * 64;
    b.Tp = ((T + 63) / 64) * 64;
    b.part_ld = gemm_part_cols(b.f.bm_up, F);
    b.bm_w2 = gemm_block_m(MOE_DTYPE_BF16, D, 1, false, F);
    b.bm_w1 = gemm_block_m(MOE_DTYPE_BF16, b.G * F, 1, false, D);
    b.bm_sh2 = gemm_block_m(MOE_DTYPE_BF16, D, 1, false, Fs);
    b.bm_sh1 = gemm_block_m(MOE_DTYPE_BF16, 2 * Fs, 1, false, D);
    b.bm_r = gemm_block_m(MOE_DTYPE_BF16, 3 * M, 1, false, D);
    size_t off = b.f.total;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    const size_t GF = b.G * F;
    b.Z = take(b.S * GF * 2);
    b.dZ = take(b.S * GF * 2);
    b.part = take(b.S * b.part_ld * 4);
    b.Zsh = take(T * 2 * Fs * 2);
    b.dZsh = take(T * 2 * Fs * 2);
    b.poff = take((M + 1) * 4);
    b.pad_row = take(b.Spad * 4);
    b.pad_tok = take(b.Spad * 4);
    b.dOT = take(D * b.Spad * 2);
    b.HT = take(F * b.Spad * 2);
    b.dZT = take(GF * b.Spad * 2);
    b.XT = take(D * b.Spad * 2);
    b.xT = take(D * b.Tp * 2);
    b.dyT = take(Fs > 0 ? D * b.Tp * 2 : 0);
    b.HshT = take(Fs * b.Tp * 2);
    b.dZshT = take(2 * Fs * b.Tp * 2);
    b.dl = take(T * M * 4);
    b.gate = take(T * M * 4);
    b.dlT3 = take(3 * M * b.Tp * 2);
    b.C3 = take(std::max(3 * M * D, ((T + 255) / 256) * M) * 4);
    b.total = off;
    return b;
}

int validate_bwd(const moe_desc* d) {
    TRY(validate(d));
    if (d->dtype != MOE_DTYPE_BF16)
        return fail(MOE_ERR_UNSUPPORTED, "the backward runs on bf16 layers only");
    if (d->weight_layout != MOE_LAYOUT_ROWS)
        return fail(MOE_ERR_UNSUPPORTED, "the backward reads row-major weights only");
    const int64_t S = d->T * d->k, Spad = ((S + 64 * d->M + 63) / 64) * 64;
    const int64_t G = d->act == MOE_ACT_SWIGLU ? 2 : 1;
    const int64_t biggest = std::max({d->D * Spad, G * d->F * Spad, d->D * G * d->F});
    if (biggest * 2 > ((int64_t)1 << 31))
        return fail(MOE_ERR_UNSUPPORTED, "a backward operand exceeds 2 GiB");
    return MOE_OK;
}

GemmArgs dense_args(const void* a, const void* b, void* c, int64_t rows, int64_t b_rows,
                    int64_t K, int64_t N) {
    GemmArgs g{};
    g.a = a;
    g.b = b;
    g.c = c;
    g.dense_rows = rows;
    g.a_rows = rows;
    g.b_rows = (int)b_rows;
    g.K = (int)K;
    g.N = (int)N;
    g.xcd_mode = gemm_xcd_mode(false, false);
    return g;
}

int do_backward(moe_handle* h, const moe_desc* d, const BwdPlan& b, const void* x,
                const float* W_r, const float* bias, const void* W1, const void* b1,
                const void* W2, const void* b2, const void* Wsh_gu, const void* Wsh_dn,
                const void* dy,
                float* dx, float* dW_r, float* dW1, float* db1, float* dW2, float* db2,
                float* dWsh_gu, float* dWsh_dn, int32_t* load_count, float* load_score, void* ws,
                hipStream_t s) {
    const Plan& p = b.f;
    const int64_t T = d->T, D = d->D, M = d->M, F = d->F, Fs = d->F_shared, S = b.S;
    const int64_t GF = b.G * F;
    const bool swiglu = d->act == MOE_ACT_SWIGLU;
    int32_t* idx = at<int32_t>(ws, p.idx);
    float* w = at<float>(ws, p.w);
    int32_t* counts = at<int32_t>(ws, p.counts);
    int32_t* offsets = at<int32_t>(ws, p.offsets);
    int32_t* sorted_token = at<int32_t>(ws, p.sorted_token);
    int32_t* sorted_slot = at<int32_t>(ws, p.sorted_slot);
    int32_t* slot_row = at<int32_t>(ws, p.slot_row);
    float* row_scale = at<float>(ws, p.row_scale);
    int32_t* tiles_up = at<int32_t>(ws, p.tiles_up);
    int32_t* tiles_dn = at<int32_t>(ws, p.tiles_dn);
    void* H = at<char>(ws, p.H);
    float* dXs = at<float>(ws, p.O);
    void* Hsh = at<char>(ws, p.Hsh);
    float* dXsh = Fs > 0 ? at<float>(ws, p.Ysh) : nullptr;
    const float* L = reinterpret_cast<const float*>(at<char>(ws, p.route) +
                                                    route_logits_offset(1, T, D, M));
    void* Z = at<char>(ws, b.Z);
    void* dZ = at<char>(ws, b.dZ);
    float* part = at<float>(ws, b.part);
    int32_t* poff = at<int32_t>(ws, b.poff);
    int32_t* pad_row = at<int32_t>(ws, b.pad_row);
    int32_t* pad_tok = at<int32_t>(ws, b.pad_tok);
    void* dOT = at<char>(ws, b.dOT);
    void* HT = at<char>(ws, b.HT);
    void* dZT = at<char>(ws, b.dZT);
    void* XT = at<char>(ws, b.XT);
    void* xT = at<char>(ws, b.xT);
    float* dl = at<float>(ws, b.dl);
    float* gate = at<float>(ws, b.gate);
    void* dlT3 = at<char>(ws, b.dlT3);
    float* C3 = at<float>(ws, b.C3);

    // forward recompute of the routing (the bf16 router leaves its logits)
    TRY(do_route(h, d, p, x, W_r, bias, idx, w, ws, s));
    TRY(do_permute(h, d, p, idx, counts, offsets, sorted_token, sorted_slot, slot_row, ws, s));
    TileTables tt{{p.bm_up, p.bm_dn},
                  {(int)p.max_tiles_up, (int)p.max_tiles_dn},
                  {tiles_up, tiles_dn}};
    const int ntables = tiles_dn == tiles_up ? 1 : 2;
    TRY(run(h, s, L_TILE_TABLE, [&] {
        return launch_tile_table(s, offsets, M, tt, ntables, sorted_slot, w, S, row_scale, 0,
                                 sorted_token);
    }));
    // 1. up projection again, keeping the pre-activations Z (bf16)
    GemmArgs up{};
    up.a = x;
    up.gather = sorted_token;
    up.b = W1;
    up.b_stride = GF * D;
    up.bias = swiglu ? nullptr : b1;
    up.c = H;
    up.c2 = Z;
    up.tiles = tiles_up;
    up.offsets = offsets;
    up.dense_rows = S;
    up.a_rows = T;
    up.b_rows = (int)GF;
    up.K = (int)D;
    up.N = (int)F;
    up.F_split = (int)F;
    up.group_m = gemm_group_m(S, M, p.bm_up, d->group_m);
    up.xcd_mode = gemm_xcd_mode(true, false, M == 1, d->tile_order[MOE_GEMM_UP]);
    TRY(run(h, s, L_B_UP, [&] {
        return launch_gemm(s, 1, p.bm_up, swiglu ? EPI_SWIGLU_SAVE : EPI_GELU_SAVE, up,
                           p.max_tiles_up);
    }));
    // 2. dH_raw = dy W2[e] per sorted row -> dZ (activation derivative, row
    //    weight) and the per-tile dots H . dH_raw for the router
    GemmArgs dh = up;
    dh.a = dy;
    dh.b = W2;             // read in place as [K = D, N = F]
    dh.b_kn = 1;
    dh.b_stride = D * F;
    dh.bias = nullptr;
    dh.c = dZ;
    dh.c2 = Z;
    dh.aux = H;
    dh.row_w = row_scale;
    dh.part = part;
    dh.part_ld = b.part_ld;
    dh.b_rows = (int)F;
    dh.F_split = 0;
    TRY(run(h, s, L_B_DH, [&] {
        return launch_gemm(s, 1, p.bm_up, swiglu ? EPI_DH_SWIGLU : EPI_DH_GELU, dh,
                           p.max_tiles_up);
    }));
    // 3. expert rows' input gradients dXs = dZ W1[e] (fp32, sorted order).
    //    MFMA-bound with full-width K like an up projection: it takes the up
    //    projection's tile height when that is 128 rows or more (GLM-4.5
    //    prefill 256: 3.76 -> 3.24 ms against the down projection's 128)
    const bool dx_up = p.bm_up >= 128;
    const int bm_dx = dx_up ? p.bm_up : p.bm_dn;
    GemmArgs dxg{};
    dxg.a = dZ;
    dxg.b = W1;            // read in place as [K = G F, N = D]
    dxg.b_kn = 1;
    dxg.b_stride = GF * D;
    dxg.c = dXs;
    dxg.tiles = dx_up ? tiles_up : tiles_dn;
    dxg.offsets = offsets;
    dxg.dense_rows = S;
    dxg.a_rows = S;
    dxg.b_rows = (int)D;
    dxg.K = (int)GF;
    dxg.N = (int)D;
    dxg.group_m = gemm_group_m(S, M, bm_dx, d->group_m);
    dxg.xcd_mode = gemm_xcd_mode(true, true, false, d->tile_order[MOE_GEMM_DOWN]);
    TRY(run(h, s, L_B_DX, [&] {
        return launch_gemm(s, 1, bm_dx, EPI_DOWN_F32, dxg,
                           dx_up ? p.max_tiles_up : p.max_tiles_dn);
    }));

    // 4. the shared expert, the same three steps as one dense group
    if (Fs > 0) {
        void* Zsh = at<char>(ws, b.Zsh);
        void* dZsh = at<char>(ws, b.dZsh);
        const int64_t mt_up = (T + p.bm_sh_up - 1) / p.bm_sh_up;
        const int64_t mt_dn = (T + p.bm_sh_dn - 1) / p.bm_sh_dn;
        GemmArgs su = dense_args(x, Wsh_gu, Hsh, T, 2 * Fs, D, Fs);
        su.c2 = Zsh;
        su.F_split = (int)Fs;
        TRY(run(h, s, L_B_UP, [&] {
            return launch_gemm(s, 1, p.bm_sh_up, EPI_SWIGLU_SAVE, su, mt_up);
        }));
        GemmArgs sd = dense_args(dy, Wsh_dn, dZsh, T, Fs, D, Fs);
        sd.b_kn = 1;
        sd.b_stride = D * Fs;
        sd.c2 = Zsh;
        TRY(run(h, s, L_B_DH, [&] {
            return launch_gemm(s, 1, p.bm_sh_up, EPI_DH_SWIGLU, sd, mt_up);
        }));
        GemmArgs sx = dense_args(dZsh, Wsh_gu, dXsh, T, D, 2 * Fs, D);
        sx.b_kn = 1;
        sx.b_stride = 2 * Fs * D;
        TRY(run(h, s, L_B_DX, [&] { return launch_gemm(s, 1, p.bm_sh_dn, EPI_DOWN_F32, sx, mt_dn); }));
    }

    // 5. router: weights -> gate values -> logits; then dx
    TRY(run(h, s, L_B_OTHER, [&] {
        hipError_t e = launch_router_backward(s, L, idx, w, slot_row, part, b.part_ld,
                                              swiglu ? nullptr : b2, dy, D, T, M, d->k, d->scorer,
                                              d->renorm, d->alpha, d->eps, dl, gate);
        if (e != hipSuccess) return e;
        e = launch_bwd_combine(s, dXs, slot_row, dXsh, dl, idx, W_r, T, d->k, M, D,
                               d->scorer == MOE_SCORER_SIGMOID, dx);
        if (e != hipSuccess) return e;
        // the split-plane router product's buffer C3 serves as scratch here
        return launch_load_stats(s, gate, T, M, counts, C3, load_count, load_score);
    }));

    // 6. weight gradients: per-expert padded, transposed operands, one
    //    K-grouped GEMM each (K = the expert's padded rows)
    TRY(run(h, s, L_B_TRANSPOSE, [&] {
        hipError_t e = launch_pad_layout(s, offsets, M, sorted_token, b.Spad, poff, pad_row, pad_tok);
        if (e != hipSuccess) return e;
        // dO = w dy per sorted row (gathered through sorted_token)
        e = launch_transpose(s, dy, D, S, 0, pad_row, sorted_token, row_scale, D, b.Spad, dOT,
                             b.Spad, 0, 1);
        if (e != hipSuccess) return e;
        e = launch_transpose(s, H, F, S, 0, pad_row, nullptr, nullptr, F, b.Spad, HT, b.Spad, 0, 1);
        if (e != hipSuccess) return e;
        e = launch_transpose(s, dZ, GF, S, 0, pad_row, nullptr, nullptr, GF, b.Spad, dZT, b.Spad, 0,
                             1);
        if (e != hipSuccess) return e;
        e = launch_transpose(s, x, D, S, 0, pad_row, sorted_token, nullptr, D, b.Spad, XT, b.Spad,
                             0, 1);
        if (e != hipSuccess) return e;
        return launch_transpose(s, x, D, T, 0, nullptr, nullptr, nullptr, D, b.Tp, xT, b.Tp, 0, 1);
    }));
    GemmArgs w2 = dense_args(dOT, HT, dW2, D, F, b.Spad, F);
    w2.koff = poff;
    w2.kgroups = (int)M;
    w2.c_group_stride = D * F;
    GemmArgs w1 = dense_args(dZT, XT, dW1, GF, D, b.Spad, D);
    w1.koff = poff;
    w1.kgroups = (int)M;
    w1.c_group_stride = GF * D;
    // the weight-gradient kernel (store-bound products)
    auto wgrad = [&](const GemmArgs& g, int, int64_t) { return launch_wgrad(s, g); };
    TRY(run(h, s, L_B_WGRAD, [&] {
        hipError_t e = wgrad(w2, b.bm_w2, D);
        if (e != hipSuccess) return e;
        return wgrad(w1, b.bm_w1, GF);
    }));
    if (Fs > 0) {
        void* dyT = at<char>(ws, b.dyT);
        void* HshT = at<char>(ws, b.HshT);
        void* dZshT = at<char>(ws, b.dZshT);
        void* dZsh = at<char>(ws, b.dZsh);
        TRY(run(h, s, L_B_TRANSPOSE, [&] {
            hipError_t e = launch_transpose(s, dy, D, T, 0, nullptr, nullptr, nullptr, D, b.Tp, dyT,
                                            b.Tp, 0, 1);
            if (e != hipSuccess) return e;
            e = launch_transpose(s, Hsh, Fs, T, 0, nullptr, nullptr, nullptr, Fs, b.Tp, HshT, b.Tp,
                                 0, 1);
            if (e != hipSuccess) return e;
            return launch_transpose(s, dZsh, 2 * Fs, T, 0, nullptr, nullptr, nullptr, 2 * Fs, b.Tp,
                                    dZshT, b.Tp, 0, 1);
        }));
        GemmArgs s2 = dense_args(dyT, HshT, dWsh_dn, D, Fs, b.Tp, Fs);
        GemmArgs s1 = dense_args(dZshT, xT, dWsh_gu, 2 * Fs, D, b.Tp, D);
        TRY(run(h, s, L_B_WGRAD, [&] {
            hipError_t e = wgrad(s2, b.bm_sh2, D);
            if (e != hipSuccess) return e;
            return wgrad(s1, b.bm_sh1, 2 * Fs);
        }));
    }
    // router weight gradient: dl split exactly into three bf16 planes, so the
    // MFMA products with bf16 x are exact; the planes' results are summed
    GemmArgs rw = dense_args(dlT3, xT, C3, 3 * M, D, b.Tp, D);
    TRY(run(h, s, L_B_WGRAD, [&] {
        hipError_t e = launch_split_transpose_dl(s, dl, T, M, b.Tp, dlT3);
        if (e != hipSuccess) return e;
        e = launch_gemm(s, 1, b.bm_r, EPI_DOWN_F32, rw, (3 * M + b.bm_r - 1) / b.bm_r);
        if (e != hipSuccess) return e;
        return launch_sum3(s, C3, C3 + M * D, C3 + 2 * M * D, M * D, dW_r);
    }));
    // bias gradients (GELU experts): db1 = column sums of dz, db2 of w dy
    if (!swiglu && (db1 || db2)) {
        TRY(run(h, s, L_B_OTHER, [&] {
            hipError_t e = hipSuccess;
            if (db1) e = launch_seg_colsum(s, dZ, F, offsets, nullptr, nullptr, M, F, db1);
            if (e != hipSuccess) return e;
            if (db2) e = launch_seg_colsum(s, dy, D, offsets, sorted_token, row_scale, M, D, db2);
            return e;
        }));
    }
    return MOE_OK;
}

#define CHECK_HANDLE(h)                                                      \
    do {                                                                     \
        if (!(h)) return fail(MOE_ERR_INVALID, "handle is NULL");            \
    } while (0)
#define NEED(p, name)                                                        \
    do {                                                                     \
        if (!(p)) return fail(MOE_ERR_INVALID, "%s is NULL", name);          \
    } while (0)

// moe_forward, and moe_forward_no_alloc (fixed: the workspace is this
// device's static scratch, for callers that cannot allocate).
int forward_impl(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
                 const float* bias, const void* W1, const void* b1, const void* W2,
                 const void* b2, const void* Wsh_gu, const void* Wsh_dn, void* y, void* ws,
                 size_t ws_bytes, void* stream, void* aux_stream, bool fixed) {
    CHECK_HANDLE(h);
    TRY(validate(d));
    if (d->T == 0) return MOE_OK;
    NEED(x, "x");
    NEED(W_r, "W_r");
    NEED(W1, "W1");
    NEED(W2, "W2");
    NEED(y, "y");
    if (d->F_shared > 0) {
        NEED(Wsh_gu, "Wsh_gu");
        NEED(Wsh_dn, "Wsh_dn");
    }
    if (y == x) return fail(MOE_ERR_INVALID, "y aliases x");
    const Plan p = make_plan(d);
    if (fixed) {
        if (p.total > kScratchBytes)
            return fail(MOE_ERR_UNSUPPORTED,
                        "the layer needs %zu bytes of workspace; the fixed scratch of "
                        "moe_forward_no_alloc holds %zu (use moe_forward)", p.total,
                        kScratchBytes);
        ws = h->scratch;
        ws_bytes = kScratchBytes;
    }
    TRY(check_ws(p, ws, ws_bytes));
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipStream_t aux = static_cast<hipStream_t>(aux_stream);
    int32_t* idx = at<int32_t>(ws, p.idx);
    float* w = at<float>(ws, p.w);
    int32_t* counts = at<int32_t>(ws, p.counts);
    int32_t* offsets = at<int32_t>(ws, p.offsets);
    int32_t* sorted_token = at<int32_t>(ws, p.sorted_token);
    int32_t* sorted_slot = at<int32_t>(ws, p.sorted_slot);
    int32_t* slot_row = at<int32_t>(ws, p.slot_row);
    float* O = at<float>(ws, p.O);
    float* Ysh = d->F_shared > 0 ? at<float>(ws, p.Ysh) : nullptr;

    if (p.merged) {
        // the shared expert is group M of the routed GEMMs; Ysh is O's tail
        TRY(do_route(h, d, p, x, W_r, bias, idx, w, ws, s));
        bool built = false;
        TRY(do_permute(h, d, p, idx, counts, offsets, sorted_token, sorted_slot, slot_row, ws, s,
                       w, d->T, &built));
        TRY(do_expert_ffn(h, d, p, x, sorted_token, sorted_slot, offsets, w, W1, b1, W2, b2, O,
                          ws, s, Wsh_gu, Wsh_dn, false, built));
        return do_combine(h, d, O, slot_row, Ysh, y, s);
    }
    const bool fork = Ysh && aux && aux != s;
    if (Ysh) {
        if (fork) {
            hipError_t e;
            if ((e = hipEventRecord(h->ev_fork, s)) != hipSuccess ||
                (e = hipStreamWaitEvent(aux, h->ev_fork, 0)) != hipSuccess)
                return fail(MOE_ERR_HIP, "stream fork: %s", hipGetErrorString(e));
            TRY(do_shared(h, d, p, x, Wsh_gu, Wsh_dn, Ysh, ws, aux, p.compact));
            if ((e = hipEventRecord(h->ev_join, aux)) != hipSuccess)
                return fail(MOE_ERR_HIP, "stream join: %s", hipGetErrorString(e));
        } else {
            TRY(do_shared(h, d, p, x, Wsh_gu, Wsh_dn, Ysh, ws, s, p.compact));
        }
    }
    TRY(do_route(h, d, p, x, W_r, bias, idx, w, ws, s));
    bool built = false;
    TRY(do_permute(h, d, p, idx, counts, offsets, sorted_token, sorted_slot, slot_row, ws, s, w,
                   0, &built));
    TRY(do_expert_ffn(h, d, p, x, sorted_token, sorted_slot, offsets, w, W1, b1, W2, b2, O, ws, s,
                      nullptr, nullptr, p.compact, built));
    if (fork) {
        const hipError_t e = hipStreamWaitEvent(s, h->ev_join, 0);
        if (e != hipSuccess) return fail(MOE_ERR_HIP, "stream join: %s", hipGetErrorString(e));
    }
    return do_combine(h, d, O, slot_row, Ysh, y, s, p.compact);
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_last_error_detail(void) { return g_detail.c_str(); }

int moe_create(int device, moe_handle** out) {
    if (!out) return fail(MOE_ERR_INVALID, "out is NULL");
    *out = nullptr;
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceCount: %s", hipGetErrorString(e));
    if (device < 0 || device >= n)
        return fail(MOE_ERR_INVALID, "device %d not in [0, %d)", device, n);
    DeviceGuard g(device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    void* scr = nullptr;
    TRY(scratch_address(device, &scr));
    moe_handle* h = new moe_handle();
    h->device = device;
    h->scratch = scr;
    if ((e = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming)) != hipSuccess) {
        if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
        delete h;
        return fail(MOE_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
    *out = h;
    return MOE_OK;
}

int moe_destroy(moe_handle* h) {
    if (!h) return MOE_OK;
    {
        DeviceGuard g(h->device);
        if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
        if (h->ev_join) (void)hipEventDestroy(h->ev_join);
        for (hipEvent_t ev : h->prof_events) (void)hipEventDestroy(ev);
    }
    delete h;
    return MOE_OK;
}

int moe_workspace_size(const moe_desc* d, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
    TRY(validate(d));
    *bytes = make_plan(d).total;
    return MOE_OK;
}

int moe_route(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
              const float* bias, int32_t* idx, float* w, void* ws, size_t ws_bytes,
              void* stream) {
    CHECK_HANDLE(h);
    TRY(validate(d));
    if (d->T == 0) return MOE_OK;
    NEED(x, "x");
    NEED(W_r, "W_r");
    NEED(idx, "idx");
    NEED(w, "w");
    const Plan p = make_plan(d);
    TRY(check_ws(p, ws, ws_bytes));
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    return do_route(h, d, p, x, W_r, bias, idx, w, ws, static_cast<hipStream_t>(stream));
}

int moe_permute(moe_handle* h, const moe_desc* d, const int32_t* idx, int32_t* counts,
                int32_t* offsets, int32_t* sorted_token, int32_t* sorted_slot, int32_t* slot_row,
                void* ws, size_t ws_bytes, void* stream) {
    CHECK_HANDLE(h);
    TRY(validate(d));
    if (d->T == 0) return MOE_OK;
    NEED(idx, "idx");
    NEED(counts, "counts");
    NEED(offsets, "offsets");
    NEED(sorted_token, "sorted_token");
    NEED(sorted_slot, "sorted_slot");
    NEED(slot_row, "slot_row");
    const Plan p = make_plan(d);
    TRY(check_ws(p, ws, ws_bytes));
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    return do_permute(h, d, p, idx, counts, offsets, sorted_token, sorted_slot, slot_row, ws,
                      static_cast<hipStream_t>(stream));
}

int moe_expert_ffn(moe_handle* h, const moe_desc* d, const void* x, const int32_t* sorted_token,
                   const int32_t* sorted_slot, const int32_t* offsets, const float* w,
                   const void* W1, const void* b1, const void* W2, const void* b2, float* O,
                   void* ws, size_t ws_bytes, void* stream) {
    CHECK_HANDLE(h);
    TRY(validate(d));
    if (d->T == 0) return MOE_OK;
    NEED(x, "x");
    NEED(sorted_token, "sorted_token");
    NEED(sorted_slot, "sorted_slot");
    NEED(offsets, "offsets");
    NEED(w, "w");
    NEED(W1, "W1");
    NEED(W2, "W2");
    NEED(O, "O");
    const Plan p = make_plan(d);
    TRY(check_ws(p, ws, ws_bytes));
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    // not merged: nothing is written through these two
    return do_expert_ffn(h, d, p, x, const_cast<int32_t*>(sorted_token), sorted_slot,
                         const_cast<int32_t*>(offsets), w, W1, b1, W2, b2, O, ws,
                         static_cast<hipStream_t>(stream));
}

int moe_shared_expert(moe_handle* h, const moe_desc* d, const void* x, const void* Wsh_gu,
                      const void* Wsh_dn, float* Ysh, void* ws, size_t ws_bytes, void* stream) {
    CHECK_HANDLE(h);
    TRY(validate(d));
    if (d->F_shared <= 0) return fail(MOE_ERR_INVALID, "F_shared is 0: no shared expert");
    if (d->T == 0) return MOE_OK;
    NEED(x, "x");
    NEED(Wsh_gu, "Wsh_gu");
    NEED(Wsh_dn, "Wsh_dn");
    NEED(Ysh, "Ysh");
    const Plan p = make_plan(d);
    TRY(check_ws(p, ws, ws_bytes));
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    return do_shared(h, d, p, x, Wsh_gu, Wsh_dn, Ysh, ws, static_cast<hipStream_t>(stream));
}

int moe_tiled_weight_size(const moe_desc* d, int which, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
    TRY(validate(d));
    if (d->dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "tiled weights are bf16 only");
    WeightShape w;
    TRY(weight_shape(d, which, w));
    const int64_t per = tiled_elems(w.n_out, w.K, w.swiglu);
    if (per * 2 > 0x7fffffffLL)
        return fail(MOE_ERR_UNSUPPORTED, "a tiled weight matrix exceeds 2 GiB");
    *bytes = (size_t)(w.E * per * 2);
    return MOE_OK;
}

int moe_tile_weights(moe_handle* h, const moe_desc* d, int which, const void* src, void* dst,
                     void* stream) {
    CHECK_HANDLE(h);
    size_t bytes = 0;
    TRY(moe_tiled_weight_size(d, which, &bytes));
    NEED(src, "src");
    NEED(dst, "dst");
    WeightShape w;
    TRY(weight_shape(d, which, w));
    const char* s0 = static_cast<const char*>(src);
    const char* d0 = static_cast<const char*>(dst);
    const size_t src_bytes = (size_t)(w.E * w.rows * w.K * 2);
    if (d0 < s0 + src_bytes && s0 < d0 + bytes) return fail(MOE_ERR_INVALID, "src and dst overlap");
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    const hipError_t e = launch_tile_weights(static_cast<hipStream_t>(stream), src, dst, w.E,
                                             w.rows, w.n_out, w.K, w.swiglu);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "tile_weights launch: %s", hipGetErrorString(e));
    return MOE_OK;
}

int moe_combine(moe_handle* h, const moe_desc* d, const float* O, const int32_t* slot_row,
                const float* Ysh, void* y, void* stream) {
    CHECK_HANDLE(h);
    TRY(validate(d));
    if (d->T == 0) return MOE_OK;
    NEED(O, "O");
    NEED(slot_row, "slot_row");
    NEED(y, "y");
    if (y == static_cast<const void*>(O) || y == static_cast<const void*>(Ysh))
        return fail(MOE_ERR_INVALID, "y aliases O or Ysh");
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    return do_combine(h, d, O, slot_row, Ysh, y, static_cast<hipStream_t>(stream));
}

int moe_forward(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
                const float* bias, const void* W1, const void* b1, const void* W2, const void* b2,
                const void* Wsh_gu, const void* Wsh_dn, void* y, void* ws, size_t ws_bytes,
                void* stream, void* aux_stream) {
    return forward_impl(h, d, x, W_r, bias, W1, b1, W2, b2, Wsh_gu, Wsh_dn, y, ws, ws_bytes,
                        stream, aux_stream, false);
}

int moe_forward_no_alloc(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
                         const float* bias, const void* W1, const void* b1, const void* W2,
                         const void* b2, const void* Wsh_gu, const void* Wsh_dn, void* y,
                         void* stream, void* aux_stream) {
    return forward_impl(h, d, x, W_r, bias, W1, b1, W2, b2, Wsh_gu, Wsh_dn, y, nullptr, 0,
                        stream, aux_stream, true);
}

int moe_backward_workspace_size(const moe_desc* d, size_t* bytes) {
    if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
    TRY(validate_bwd(d));
    *bytes = make_bwd_plan(d).total;
    return MOE_OK;
}

int moe_backward(moe_handle* h, const moe_desc* d, const void* x, const float* W_r,
                 const float* bias, const void* W1, const void* b1, const void* W2,
                 const void* b2, const void* Wsh_gu, const void* Wsh_dn, const void* dy,
                 float* dx, float* dW_r, float* dW1, float* db1, float* dW2, float* db2,
                 float* dWsh_gu, float* dWsh_dn, int32_t* load_count, float* load_score,
                 void* ws, size_t ws_bytes, void* stream) {
    CHECK_HANDLE(h);
    TRY(validate_bwd(d));
    NEED(dW_r, "dW_r");
    NEED(dW1, "dW1");
    NEED(dW2, "dW2");
    NEED(load_count, "load_count");
    NEED(load_score, "load_score");
    if (d->F_shared > 0) {
        NEED(dWsh_gu, "dWsh_gu");
        NEED(dWsh_dn, "dWsh_dn");
    }
    if (d->T > 0) {   // with no tokens only the (zeroed) gradients are touched
        NEED(x, "x");
        NEED(W_r, "W_r");
        NEED(W1, "W1");
        NEED(W2, "W2");
        NEED(dy, "dy");
        NEED(dx, "dx");
        if (d->F_shared > 0) {
            NEED(Wsh_gu, "Wsh_gu");
            NEED(Wsh_dn, "Wsh_dn");
        }
    }
    if (d->act == MOE_ACT_SWIGLU) db1 = db2 = nullptr;   // no biases
    const BwdPlan b = make_bwd_plan(d);
    if (ws_bytes < b.total)
        return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, b.total);
    if (!ws) return fail(MOE_ERR_INVALID, "workspace pointer is NULL");
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (d->T == 0) {   // no tokens: every gradient and statistic is zero
        const int64_t G = d->act == MOE_ACT_SWIGLU ? 2 : 1;
        hipError_t e = hipSuccess;
        const std::pair<float*, int64_t> zs[] = {
            {dW_r, d->M * d->D}, {dW1, d->M * G * d->F * d->D}, {dW2, d->M * d->D * d->F},
            {db1, d->M * d->F}, {db2, d->M * d->D}, {load_score, d->M},
            {reinterpret_cast<float*>(load_count), d->M},
            {d->F_shared > 0 ? dWsh_gu : nullptr, 2 * d->F_shared * d->D},
            {d->F_shared > 0 ? dWsh_dn : nullptr, d->D * d->F_shared}};
        for (const auto& z : zs)
            if (e == hipSuccess) e = launch_fill_zero(s, z.first, z.second);
        if (e != hipSuccess) return fail(MOE_ERR_HIP, "zero fill: %s", hipGetErrorString(e));
        return MOE_OK;
    }
    return do_backward(h, d, b, x, W_r, bias, W1, b1, W2, b2, Wsh_gu, Wsh_dn, dy, dx, dW_r, dW1, db1,
                       dW2, db2, dWsh_gu, dWsh_dn, load_count, load_score, ws, s);
}

int moe_profile_start(moe_handle* h, int capacity, const char* filter) {
    CHECK_HANDLE(h);
    if (capacity < 0) return fail(MOE_ERR_INVALID, "capacity < 0");
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(g.err));
    while ((int)h->prof_events.size() < 2 * capacity) {
        hipEvent_t ev;
        // timing only: no system-scope cache writeback at each record
        const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableSystemFence);
        if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        h->prof_events.push_back(ev);
    }
    h->prof_labels.assign(capacity, 0);
    h->prof_used = 0;
    h->prof_filter = filter ? filter : "";
    for (int i = 0; i < L_COUNT; ++i) {
        h->launches[i] = 0;
        h->total_ms[i] = 0.0;
    }
    h->prof_on = true;
    return MOE_OK;
}

int moe_profile_stop(moe_handle* h) {
    CHECK_HANDLE(h);
    h->prof_on = false;
    DeviceGuard g(h->device);
    for (int i = 0; i < h->prof_used; ++i) {
        hipError_t e = hipEventSynchronize(h->prof_events[2 * i + 1]);
        float ms = 0.f;
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, h->prof_events[2 * i], h->prof_events[2 * i + 1]);
        if (e != hipSuccess) return fail(MOE_ERR_HIP, "profile events: %s", hipGetErrorString(e));
        h->launches[h->prof_labels[i]] += 1;
        h->total_ms[h->prof_labels[i]] += ms;
    }
    h->prof_used = 0;
    return MOE_OK;
}

int moe_profile_results(moe_handle* h, moe_kernel_time* out, int max_entries, int* n_entries) {
    CHECK_HANDLE(h);
    if (!n_entries || (max_entries > 0 && !out)) return fail(MOE_ERR_INVALID, "NULL output");
    int n = 0;
    for (int i = 0; i < L_COUNT; ++i) {
        if (h->launches[i] == 0) continue;
        if (n < max_entries) {
            std::memset(out[n].label, 0, sizeof out[n].label);
            std::strncpy(out[n].label, kLabels[i], sizeof out[n].label - 1);
            out[n].launches = h->launches[i];
            out[n].total_ms = h->total_ms[i];
        }
        ++n;
    }
    *n_entries = n;
    return MOE_OK;
}

}  // extern "C"
