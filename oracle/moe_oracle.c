/*
 * CPU oracle for the sparse MoE feed-forward layer: forward pass and its
 * gradient.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the harness's
 * CPU-baseline leg call this; the HIP library never does and shares no code
 * with it.  It is the layer's plain definition, one token at a time, in fp64.
 *
 * Sources (cited by page title and section):
 *  [GLaM]  GLaM study note, "Sparse MoE Layer": dense FFN
 *          W2 s(W1 x + b1) + b2, router r = softmax(W_r x), S = TopK(r, 2),
 *          MoE(x) = sum over S of the normalised gate weight times E_i(x).
 *  [GLM45] "Shared Expert" (GLM-4.5 study note), "How it works": shared
 *          SwiGLU expert on every token; sigmoid router scores plus a
 *          correction bias that only decides selection; the selected
 *          sigmoid scores renormalised by their sum plus eps = 1e-20, then
 *          scaled by routed_scaling_factor; output = routed sum + shared.
 *  [GLM5]  "Shared expert" (GLM-5 inspector page), "All 5 steps":
 *          g = x W1, u = x W3, a = g sigma(g), h = a (.) u, y = h W2; its
 *          routed-experts code excerpt: gate/up projection split gate first,
 *          expert output scaled by the slot's weight, an extra one-hot class
 *          (index = number of experts) that is skipped.
 *
 * Readings where the pages leave a step open:
 *  - GLaM's "normalized gate weight": the selected softmax probabilities
 *    divided by their sum (plus eps, which cannot change a sum >= k/M).
 *  - The correction bias enters only the selection score; the weights use
 *    the unbiased sigmoid scores.  Without renormalisation w = alpha * g.
 *  - Exactly equal selection scores: the lower expert index wins.
 *  - Slots of a token are stored in ascending expert order.
 *  - GELU is the exact erf form z * Phi(z).
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element i of an array stored as fp32 or bf16, widened exactly to double. */
static double elem(const void* base, int32_t dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* sum_i W[row0 + i] * v[i], i < n, accumulated in order in fp64. */
static double dot(const void* W, int32_t dtype, int64_t row0, int64_t n, const double* v)
{
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i)
        acc += elem(W, dtype, row0 + i) * v[i];
    return acc;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu(double z) { return z / (1.0 + exp(-z)); }
static double gelu_erf(double z) { return 0.5 * z * (1.0 + erf(z / sqrt(2.0))); }

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the oracle's parallel loops use from now on (timing only: the
 * results do not depend on it, every token is computed on its own). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Router for one token [GLaM router and TopK; GLM45 sigmoid router]. */
static void route_token(const moe_oracle_cfg* c, const void* x, const float* W_r,
                        const float* bias, int64_t t, int32_t* idx_out,
                        double* w_out, double* gap_out, double* logit_out,
                        double* sel_out)
{
    const int64_t D = c->D, M = c->M;
    const int32_t k = c->k;
    double* xv = malloc(sizeof(double) * D);
    double* l = malloc(sizeof(double) * M);
    double* g = malloc(sizeof(double) * M);     /* gate value entering the weights */
    double* sel = malloc(sizeof(double) * M);   /* selection score */
    char* taken = calloc((size_t)M, 1);
    int32_t* chosen = malloc(sizeof(int32_t) * k);

    for (int64_t d = 0; d < D; ++d)
        xv[d] = elem(x, c->dtype, t * D + d);

    /* logits l_e = W_r[e,:] . x_t */
    for (int64_t e = 0; e < M; ++e) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += (double)W_r[e * D + d] * xv[d];
        l[e] = acc;
        if (logit_out)
            logit_out[e] = acc;
    }

    if (c->scorer == ORACLE_SOFTMAX) {
        /* r = softmax(l); both the selection score and the gate value */
        double mx = l[0];
        for (int64_t e = 1; e < M; ++e)
            if (l[e] > mx) mx = l[e];
        double Z = 0.0;
        for (int64_t e = 0; e < M; ++e)
            Z += exp(l[e] - mx);
        for (int64_t e = 0; e < M; ++e) {
            g[e] = exp(l[e] - mx) / Z;
            sel[e] = g[e];
        }
    } else {
        /* s = sigmoid(l); selection uses s + bias, the weights use s */
        for (int64_t e = 0; e < M; ++e) {
            g[e] = sigmoid(l[e]);
            sel[e] = g[e] + (bias ? (double)bias[e] : 0.0);
        }
    }

    if (sel_out)
        for (int64_t e = 0; e < M; ++e)
            sel_out[e] = sel[e];

    /* Expert groups [GLM45 "How it works": the router "optionally masks by
     * expert group" before the top-k].  Experts form n_group contiguous
     * groups; a group's score is the largest selection score among its
     * experts; the topk_group best groups are kept (lower group index on an
     * exact tie) and the other groups' experts leave the selection.  Marking
     * them `taken` removes them from the top-k below. */
    double group_gap = INFINITY;
    if (c->n_group > 1) {
        const int32_t ng = c->n_group, gs = (int32_t)(M / ng);
        double* gscore = malloc(sizeof(double) * ng);
        char* kept = calloc((size_t)ng, 1);
        for (int32_t gi = 0; gi < ng; ++gi) {
            gscore[gi] = sel[(int64_t)gi * gs];
            for (int32_t u = 1; u < gs; ++u)
                if (sel[(int64_t)gi * gs + u] > gscore[gi])
                    gscore[gi] = sel[(int64_t)gi * gs + u];
        }
        double last_kept = INFINITY;
        for (int32_t r = 0; r < c->topk_group; ++r) {
            int32_t best = -1;
            for (int32_t gi = 0; gi < ng; ++gi)
                if (!kept[gi] && (best < 0 || gscore[gi] > gscore[best]))
                    best = gi;
            kept[best] = 1;
            last_kept = gscore[best];
        }
        for (int32_t gi = 0; gi < ng; ++gi)
            if (!kept[gi]) {
                if (last_kept - gscore[gi] < group_gap)
                    group_gap = last_kept - gscore[gi];
                for (int32_t u = 0; u < gs; ++u)
                    taken[(int64_t)gi * gs + u] = 1;
            }
        free(gscore);
        free(kept);
    }

    /* TopK: k times, take the not-yet-taken expert with the largest
     * selection score; scanning upward with a strict comparison keeps the
     * lower index on an exact tie. */
    for (int32_t j = 0; j < k; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < M; ++e)
            if (!taken[e] && (best < 0 || sel[e] > sel[best]))
                best = e;
        taken[best] = 1;
        chosen[j] = (int32_t)best;
    }
    /* boundary gap: k-th largest minus (k+1)-th largest selection score
     * among the candidates (and the group boundary's gap) */
    double next = -INFINITY;
    int have_next = 0;
    for (int64_t e = 0; e < M; ++e)
        if (!taken[e] && (!have_next || sel[e] > next)) {
            next = sel[e];
            have_next = 1;
        }
    *gap_out = have_next ? sel[chosen[k - 1]] - next : INFINITY;
    if (group_gap < *gap_out)
        *gap_out = group_gap;

    /* slots in ascending expert order (insertion sort of k values) */
    for (int32_t a = 1; a < k; ++a) {
        int32_t v = chosen[a];
        int32_t b = a - 1;
        while (b >= 0 && chosen[b] > v) {
            chosen[b + 1] = chosen[b];
            --b;
        }
        chosen[b + 1] = v;
    }

    /* weights: alpha * g / (sum of selected g + eps), or alpha * g */
    double gsum = 0.0;
    for (int32_t j = 0; j < k; ++j)
        gsum += g[chosen[j]];
    for (int32_t j = 0; j < k; ++j) {
        idx_out[j] = chosen[j];
        w_out[j] = c->renorm ? c->alpha * g[chosen[j]] / (gsum + c->eps)
                             : c->alpha * g[chosen[j]];
    }

    free(xv); free(l); free(g); free(sel); free(taken); free(chosen);
}

void oracle_route(const moe_oracle_cfg* c, const void* x, const float* W_r,
                  const float* bias, int64_t ntok, const int64_t* tokens,
                  int32_t* idx, double* w, double* gap, double* logits, double* sel)
{
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < ntok; ++i)
        route_token(c, x, W_r, bias, tokens[i], idx + i * c->k, w + i * c->k, gap + i,
                    logits ? logits + i * c->M : NULL, sel ? sel + i * c->M : NULL);
}

/* Dispatch: group the flat slots f = t*k + j by expert, keeping slot order
 * inside each expert (a stable counting sort). */
void oracle_dispatch(int64_t T, int32_t k, int64_t M, const int32_t* idx,
                     int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                     int32_t* sorted_slot, int32_t* slot_row)
{
    const int64_t S = T * k;
    for (int64_t e = 0; e < M; ++e)
        counts[e] = 0;
    for (int64_t f = 0; f < S; ++f)
        if (idx[f] >= 0 && idx[f] < M)
            counts[idx[f]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < M; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t* cursor = malloc(sizeof(int32_t) * (M > 0 ? M : 1));
    for (int64_t e = 0; e < M; ++e)
        cursor[e] = offsets[e];
    for (int64_t r = 0; r < S; ++r) {
        sorted_slot[r] = -1;
        sorted_token[r] = -1;
    }
    for (int64_t f = 0; f < S; ++f) {
        int32_t e = idx[f];
        if (e < 0 || e >= M) {
            slot_row[f] = -1;
            continue;
        }
        int32_t r = cursor[e]++;
        sorted_slot[r] = (int32_t)f;
        sorted_token[r] = (int32_t)(f / k);
        slot_row[f] = r;
    }
    free(cursor);
}

/* SwiGLU of width Fw applied to xv [GLM5 "All 5 steps"; GLM45 shared-expert
 * equation]: Wgu holds the gate rows (0..Fw-1) then the up rows (Fw..2Fw-1),
 * each of length D; Wdn holds D rows of length Fw. */
static void swiglu(int32_t dtype, int64_t D, int64_t Fw, const void* Wgu, int64_t gu0,
                   const void* Wdn, int64_t dn0, const double* xv, double* h, double* out)
{
    for (int64_t f = 0; f < Fw; ++f) {
        double gate = dot(Wgu, dtype, gu0 + f * D, D, xv);
        double up = dot(Wgu, dtype, gu0 + (Fw + f) * D, D, xv);
        h[f] = silu(gate) * up;
    }
    for (int64_t d = 0; d < D; ++d)
        out[d] = dot(Wdn, dtype, dn0 + d * Fw, Fw, h);
}

/* Dense FFN W2 gelu(W1 x + b1) + b2 [GLaM dense FFN equation]; a null bias
 * is zero. */
static void gelu_ffn(int32_t dtype, int64_t D, int64_t Fw, const void* W1, int64_t w10,
                     const void* b1, int64_t b10, const void* W2, int64_t w20,
                     const void* b2, int64_t b20, const double* xv, double* h, double* out)
{
    for (int64_t f = 0; f < Fw; ++f) {
        double a = dot(W1, dtype, w10 + f * D, D, xv);
        if (b1)
            a += elem(b1, dtype, b10 + f);
        h[f] = gelu_erf(a);
    }
    for (int64_t d = 0; d < D; ++d) {
        double o = dot(W2, dtype, w20 + d * Fw, Fw, h);
        if (b2)
            o += elem(b2, dtype, b20 + d);
        out[d] = o;
    }
}

static void load_row(const moe_oracle_cfg* c, const void* x, int64_t t, double* xv)
{
    for (int64_t d = 0; d < c->D; ++d)
        xv[d] = elem(x, c->dtype, t * c->D + d);
}

static void expert_on_row(const moe_oracle_cfg* c, const double* xv, int64_t e,
                          const void* W1, const void* b1, const void* W2,
                          const void* b2, double* h, double* out)
{
    const int64_t D = c->D, F = c->F;
    if (c->act == ORACLE_SWIGLU)
        swiglu(c->dtype, D, F, W1, e * 2 * F * D, W2, e * D * F, xv, h, out);
    else
        gelu_ffn(c->dtype, D, F, W1, e * F * D, b1, e * F, W2, e * D * F, b2, e * D,
                 xv, h, out);
}

void oracle_expert(const moe_oracle_cfg* c, const void* x, int64_t t, int64_t e,
                   const void* W1, const void* b1, const void* W2, const void* b2,
                   double* out)
{
    double* xv = malloc(sizeof(double) * c->D);
    double* h = malloc(sizeof(double) * c->F);
    load_row(c, x, t, xv);
    expert_on_row(c, xv, e, W1, b1, W2, b2, h, out);
    free(xv); free(h);
}

void oracle_shared(const moe_oracle_cfg* c, const void* x, int64_t t,
                   const void* Wsh_gu, const void* Wsh_dn, double* out)
{
    double* xv = malloc(sizeof(double) * c->D);
    double* h = malloc(sizeof(double) * (c->F_shared > 0 ? c->F_shared : 1));
    load_row(c, x, t, xv);
    swiglu(c->dtype, c->D, c->F_shared, Wsh_gu, 0, Wsh_dn, 0, xv, h, out);
    free(xv); free(h);
}

/* y_t = sum_j w_j E_{idx_j}(x_t) + E_sh(x_t) [GLaM MoE output; GLM45 output
 * sum; the shared branch reads the same pre-routing x_t]. */
static void layer_token(const moe_oracle_cfg* c, const void* x, const int32_t* idx_t,
                        const double* w_t, const void* W1, const void* b1,
                        const void* W2, const void* b2, const void* Wsh_gu,
                        const void* Wsh_dn, int64_t t, double* y, double* slot_out,
                        double* shared_out)
{
    const int64_t D = c->D;
    const int64_t hmax = c->F > c->F_shared ? c->F : c->F_shared;
    double* xv = malloc(sizeof(double) * D);
    double* h = malloc(sizeof(double) * (hmax > 0 ? hmax : 1));
    double* o = malloc(sizeof(double) * D);
    load_row(c, x, t, xv);
    for (int64_t d = 0; d < D; ++d)
        y[d] = 0.0;
    for (int32_t j = 0; j < c->k; ++j) {
        int32_t e = idx_t[j];
        if (e < 0 || e >= c->M) {          /* dropped slot: contributes nothing */
            if (slot_out)
                for (int64_t d = 0; d < D; ++d)
                    slot_out[j * D + d] = 0.0;
            continue;
        }
        expert_on_row(c, xv, e, W1, b1, W2, b2, h, o);
        for (int64_t d = 0; d < D; ++d) {
            double v = w_t[j] * o[d];
            y[d] += v;
            if (slot_out)
                slot_out[j * D + d] = v;
        }
    }
    if (c->F_shared > 0) {
        swiglu(c->dtype, D, c->F_shared, Wsh_gu, 0, Wsh_dn, 0, xv, h, o);
        for (int64_t d = 0; d < D; ++d) {
            y[d] += o[d];
            if (shared_out)
                shared_out[d] = o[d];
        }
    } else if (shared_out) {
        for (int64_t d = 0; d < D; ++d)
            shared_out[d] = 0.0;
    }
    free(xv); free(h); free(o);
}

void oracle_layer(const moe_oracle_cfg* c, const void* x, const int32_t* idx,
                  const double* w, const void* W1, const void* b1,
                  const void* W2, const void* b2, const void* Wsh_gu,
                  const void* Wsh_dn, int64_t ntok, const int64_t* tokens,
                  double* y, double* slot_out, double* shared_out)
{
    const int64_t D = c->D;
    const int32_t k = c->k;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < ntok; ++i) {
        int64_t t = tokens[i];
        layer_token(c, x, idx + t * k, w + t * k, W1, b1, W2, b2, Wsh_gu, Wsh_dn, t,
                    y + i * D, slot_out ? slot_out + i * k * D : NULL,
                    shared_out ? shared_out + i * D : NULL);
    }
}

void oracle_forward(const moe_oracle_cfg* c, const void* x, const float* W_r,
                    const float* bias, const void* W1, const void* b1,
                    const void* W2, const void* b2, const void* Wsh_gu,
                    const void* Wsh_dn, int64_t ntok, const int64_t* tokens,
                    int32_t* idx, double* w, double* y)
{
    const int64_t D = c->D;
    const int32_t k = c->k;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < ntok; ++i) {
        double gap;
        route_token(c, x, W_r, bias, tokens[i], idx + i * k, w + i * k, &gap, NULL, NULL);
        layer_token(c, x, idx + i * k, w + i * k, W1, b1, W2, b2, Wsh_gu, Wsh_dn,
                    tokens[i], y + i * D, NULL, NULL);
    }
}

/* ------------------------------------------------------------------ backward
 *
 * Gradient of the forward pass above for an output gradient dy[T,D], by the
 * chain rule through each step of its definition, one token at a time.
 * The selection (top-k, and the correction bias, which only enters the
 * selection) is piecewise constant and passes no gradient; the weights w
 * pass it to the gate values g (softmax probabilities or sigmoid scores)
 * and on to the router logits.  The training objective that produces dy is
 * the GLaM study note's causal LM loss ("training objective"); the pages give
 * no other training term for the layer.
 */

static double silu_grad(double z)
{
    double s = sigmoid(z);
    return s * (1.0 + z * (1.0 - s));
}

/* d/dz of z Phi(z) = Phi(z) + z phi(z). */
static double gelu_erf_grad(double z)
{
    double Phi = 0.5 * (1.0 + erf(z / sqrt(2.0)));
    double phi = exp(-0.5 * z * z) / sqrt(2.0 * 3.14159265358979323846);
    return Phi + z * phi;
}

static void add_outer(double* G, int64_t g0, int64_t rows, int64_t cols, const double* a,
                      const double* b)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t q = 0; q < cols; ++q)
            G[g0 + r * cols + q] += a[r] * b[q];
}

/* SwiGLU of width Fw on xv with output gradient dout: accumulates the weight
 * gradients (same layouts as Wgu / Wdn, at offsets ggu0 / gdn0 of dWgu /
 * dWdn; NULL skips them) and dx; returns the forward output in out. */
static void swiglu_backward(int32_t dtype, int64_t D, int64_t Fw, const void* Wgu, int64_t gu0,
                            const void* Wdn, int64_t dn0, const double* xv, const double* dout,
                            double* out, double* dWgu, int64_t ggu0, double* dWdn, int64_t gdn0,
                            double* dx)
{
    double* a = malloc(sizeof(double) * Fw);
    double* b = malloc(sizeof(double) * Fw);
    double* h = malloc(sizeof(double) * Fw);
    double* dh = malloc(sizeof(double) * Fw);
    double* da = malloc(sizeof(double) * Fw);
    double* db = malloc(sizeof(double) * Fw);
    for (int64_t f = 0; f < Fw; ++f) {
        a[f] = dot(Wgu, dtype, gu0 + f * D, D, xv);
        b[f] = dot(Wgu, dtype, gu0 + (Fw + f) * D, D, xv);
        h[f] = silu(a[f]) * b[f];
    }
    for (int64_t d = 0; d < D; ++d)
        out[d] = dot(Wdn, dtype, dn0 + d * Fw, Fw, h);
    /* dh = Wdn^T dout; dWdn += dout h^T */
    for (int64_t f = 0; f < Fw; ++f) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += elem(Wdn, dtype, dn0 + d * Fw + f) * dout[d];
        dh[f] = acc;
    }
    if (dWdn)
        add_outer(dWdn, gdn0, D, Fw, dout, h);
    for (int64_t f = 0; f < Fw; ++f) {
        da[f] = dh[f] * b[f] * silu_grad(a[f]);
        db[f] = dh[f] * silu(a[f]);
    }
    if (dWgu) {
        add_outer(dWgu, ggu0, Fw, D, da, xv);
        add_outer(dWgu, ggu0 + Fw * D, Fw, D, db, xv);
    }
    for (int64_t f = 0; f < Fw; ++f)
        for (int64_t d = 0; d < D; ++d)
            dx[d] += elem(Wgu, dtype, gu0 + f * D + d) * da[f] +
                     elem(Wgu, dtype, gu0 + (Fw + f) * D + d) * db[f];
    free(a); free(b); free(h); free(dh); free(da); free(db);
}

/* GELU FFN W2 gelu(W1 x + b1) + b2 with output gradient dout (a null bias is
 * zero and gets no gradient).  Weight and bias gradients go to expert slot
 * ge of dW1 / db1 / dW2 / db2; ge < 0 skips them. */
static void gelu_backward(int32_t dtype, int64_t D, int64_t Fw, const void* W1, int64_t w10,
                          const void* b1, int64_t b10, const void* W2, int64_t w20,
                          const void* b2, int64_t b20, const double* xv, const double* dout,
                          double* out, int64_t ge, double* dW1, double* db1, double* dW2,
                          double* db2, double* dx)
{
    double* z = malloc(sizeof(double) * Fw);
    double* h = malloc(sizeof(double) * Fw);
    double* dz = malloc(sizeof(double) * Fw);
    for (int64_t f = 0; f < Fw; ++f) {
        z[f] = dot(W1, dtype, w10 + f * D, D, xv) + (b1 ? elem(b1, dtype, b10 + f) : 0.0);
        h[f] = gelu_erf(z[f]);
    }
    for (int64_t d = 0; d < D; ++d)
        out[d] = dot(W2, dtype, w20 + d * Fw, Fw, h) + (b2 ? elem(b2, dtype, b20 + d) : 0.0);
    for (int64_t f = 0; f < Fw; ++f) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += elem(W2, dtype, w20 + d * Fw + f) * dout[d];
        dz[f] = acc * gelu_erf_grad(z[f]);
    }
    if (ge >= 0) {
        add_outer(dW2, ge * D * Fw, D, Fw, dout, h);
        if (b2)
            for (int64_t d = 0; d < D; ++d)
                db2[ge * D + d] += dout[d];
        add_outer(dW1, ge * Fw * D, Fw, D, dz, xv);
        if (b1)
            for (int64_t f = 0; f < Fw; ++f)
                db1[ge * Fw + f] += dz[f];
    }
    for (int64_t f = 0; f < Fw; ++f)
        for (int64_t d = 0; d < D; ++d)
            dx[d] += elem(W1, dtype, w10 + f * D + d) * dz[f];
    free(z); free(h); free(dz);
}

void oracle_backward(const moe_oracle_cfg* c, const void* x, const float* W_r,
                     const float* bias, const void* W1, const void* b1, const void* W2,
                     const void* b2, const void* Wsh_gu, const void* Wsh_dn, const double* dy,
                     double* dx, double* dW_r, double* dW1, double* db1, double* dW2,
                     double* db2, double* dWsh_gu, double* dWsh_dn, int64_t* load_count,
                     double* load_score, const int32_t* expert_slot, int64_t n_slots)
{
    const int64_t T = c->T, D = c->D, M = c->M, F = c->F, Fs = c->F_shared;
    const int32_t k = c->k;
    const int64_t G = c->act == ORACLE_SWIGLU ? 2 : 1;
    const int64_t Mg = expert_slot ? n_slots : M;   /* experts whose gradients are kept */
    memset(dx, 0, sizeof(double) * T * D);
    memset(dW_r, 0, sizeof(double) * M * D);
    memset(dW1, 0, sizeof(double) * Mg * G * F * D);
    memset(dW2, 0, sizeof(double) * Mg * D * F);
    if (db1) memset(db1, 0, sizeof(double) * Mg * F);
    if (db2) memset(db2, 0, sizeof(double) * Mg * D);
    if (Fs > 0) {
        memset(dWsh_gu, 0, sizeof(double) * 2 * Fs * D);
        memset(dWsh_dn, 0, sizeof(double) * D * Fs);
    }
    memset(load_count, 0, sizeof(int64_t) * M);
    memset(load_score, 0, sizeof(double) * M);

    double* xv = malloc(sizeof(double) * D);
    double* l = malloc(sizeof(double) * M);
    double* g = malloc(sizeof(double) * M);
    double* dg = malloc(sizeof(double) * M);
    double* dl = malloc(sizeof(double) * M);
    double* o = malloc(sizeof(double) * D);
    double* dout = malloc(sizeof(double) * D);
    int32_t* idx = malloc(sizeof(int32_t) * k);
    double* w = malloc(sizeof(double) * k);
    double* dw = malloc(sizeof(double) * k);

    for (int64_t t = 0; t < T; ++t) {
        double gap;
        route_token(c, x, W_r, bias, t, idx, w, &gap, l, NULL);
        load_row(c, x, t, xv);
        const double* dyt = dy + t * D;
        double* dxt = dx + t * D;
        /* gate values g over all experts, as in the router */
        if (c->scorer == ORACLE_SOFTMAX) {
            double mx = l[0], Z = 0.0;
            for (int64_t e = 1; e < M; ++e)
                if (l[e] > mx) mx = l[e];
            for (int64_t e = 0; e < M; ++e)
                Z += exp(l[e] - mx);
            for (int64_t e = 0; e < M; ++e)
                g[e] = exp(l[e] - mx) / Z;
        } else {
            for (int64_t e = 0; e < M; ++e)
                g[e] = sigmoid(l[e]);
        }
        for (int64_t e = 0; e < M; ++e)
            load_score[e] += g[e];

        /* routed experts: dw_j = dy . E_j(x); the expert sees w_j dy */
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = idx[j];
            dw[j] = 0.0;
            if (e < 0 || e >= M)
                continue;
            load_count[e] += 1;
            for (int64_t d = 0; d < D; ++d)
                dout[d] = w[j] * dyt[d];
            const int64_t ge = expert_slot ? expert_slot[e] : e;
            if (c->act == ORACLE_SWIGLU)
                swiglu_backward(c->dtype, D, F, W1, e * 2 * F * D, W2, e * D * F, xv, dout, o,
                                ge >= 0 ? dW1 : NULL, ge * 2 * F * D, ge >= 0 ? dW2 : NULL,
                                ge * D * F, dxt);
            else
                gelu_backward(c->dtype, D, F, W1, e * F * D, b1, e * F, W2, e * D * F, b2,
                              e * D, xv, dout, o, ge, dW1, db1, dW2, db2, dxt);
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d)
                acc += dyt[d] * o[d];
            dw[j] = acc;
        }
        /* shared expert, weight 1 */
        if (Fs > 0)
            swiglu_backward(c->dtype, D, Fs, Wsh_gu, 0, Wsh_dn, 0, xv, dyt, o, dWsh_gu, 0,
                            dWsh_dn, 0, dxt);

        /* weights -> gate values: w_j = alpha g_j / (sum_S g + eps), or alpha g_j */
        for (int64_t e = 0; e < M; ++e)
            dg[e] = 0.0;
        if (c->renorm) {
            double Gs = 0.0, s = 0.0;
            for (int32_t j = 0; j < k; ++j)
                if (idx[j] >= 0 && idx[j] < M)
                    Gs += g[idx[j]];
            const double den = Gs + c->eps;
            for (int32_t j = 0; j < k; ++j)
                if (idx[j] >= 0 && idx[j] < M)
                    s += dw[j] * g[idx[j]];
            for (int32_t j = 0; j < k; ++j)
                if (idx[j] >= 0 && idx[j] < M)
                    dg[idx[j]] = c->alpha * (dw[j] / den - s / (den * den));
        } else {
            for (int32_t j = 0; j < k; ++j)
                if (idx[j] >= 0 && idx[j] < M)
                    dg[idx[j]] = c->alpha * dw[j];
        }
        /* gate values -> logits */
        if (c->scorer == ORACLE_SOFTMAX) {
            double s = 0.0;
            for (int64_t e = 0; e < M; ++e)
                s += dg[e] * g[e];
            for (int64_t e = 0; e < M; ++e)
                dl[e] = g[e] * (dg[e] - s);
        } else {
            for (int64_t e = 0; e < M; ++e)
                dl[e] = dg[e] * g[e] * (1.0 - g[e]);
        }
        /* logits l = W_r x: dW_r += dl x^T, dx += W_r^T dl */
        add_outer(dW_r, 0, M, D, dl, xv);
        for (int64_t e = 0; e < M; ++e)
            for (int64_t d = 0; d < D; ++d)
                dxt[d] += (double)W_r[e * D + d] * dl[e];
    }
    free(xv); free(l); free(g); free(dg); free(dl); free(o); free(dout); free(idx);
    free(w); free(dw);
}
