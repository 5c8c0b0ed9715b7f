/*
 * CPU oracle for the sparse MoE feed-forward layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously correct
 * definition of what the layer computes, used to check the HIP library.
 * Only the tests, the smoke check and the harness's CPU-baseline leg may
 * call it; the library never does, and the two share no code.
 *
 * Every input is widened exactly to double (fp32 and bf16 both embed
 * exactly in fp64) and all arithmetic is fp64 with no intermediate
 * rounding.  Pointers are host memory owned by the caller.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_SOFTMAX = 0, ORACLE_SIGMOID = 1 };
enum { ORACLE_SWIGLU = 0, ORACLE_GELU = 1 };
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

typedef struct {
    int64_t T, D, M, F, F_shared;
    int32_t k;
    int32_t scorer;  /* ORACLE_SOFTMAX | ORACLE_SIGMOID */
    int32_t act;     /* ORACLE_SWIGLU  | ORACLE_GELU    */
    int32_t dtype;   /* storage of x, expert and shared weights: ORACLE_F32 | ORACLE_BF16 */
    int32_t renorm;  /* 1: renormalise the selected gate values */
    double alpha;    /* routed scaling factor */
    double eps;      /* renormalisation epsilon */
    int32_t n_group;     /* expert groups (<= 1: none) */
    int32_t topk_group;  /* groups kept per token */
} moe_oracle_cfg;

/* Router for tokens tokens[0..ntok): logits, scores, top-k, weights.
 * Outputs are indexed by position in the token list:
 *   idx[i*k+j] expert of slot j (ascending expert order), w[i*k+j] weight,
 *   gap[i] = (k-th largest selection score) - ((k+1)-th largest), +inf if k == M;
 *   with expert groups, the smaller of that (among the kept groups' experts)
 *   and the topk_group-th minus the (topk_group+1)-th group score,
 *   logits[i*M+e] and the selection scores sel[i*M+e] (both nullable).
 *   bias is nullable (zero bias). */
void oracle_route(const moe_oracle_cfg* c, const void* x, const float* W_r,
                  const float* bias, int64_t ntok, const int64_t* tokens,
                  int32_t* idx, double* w, double* gap, double* logits, double* sel);

/* Dispatch over all T*k flat slots f = t*k + j: per-expert counts, their
 * exclusive prefix sum offsets[0..M] and a stable counting sort of the slots
 * by expert.  Index value M (and any value outside [0, M)) is a dropped slot:
 * counted nowhere, slot_row = -1.  Entries r >= offsets[M] of sorted_slot
 * and sorted_token are -1. */
void oracle_dispatch(int64_t T, int32_t k, int64_t M, const int32_t* idx,
                     int32_t* counts, int32_t* offsets, int32_t* sorted_token,
                     int32_t* sorted_slot, int32_t* slot_row);

/* One routed expert e applied to token t: out[D] = E_e(x_t). */
void oracle_expert(const moe_oracle_cfg* c, const void* x, int64_t t, int64_t e,
                   const void* W1, const void* b1, const void* W2, const void* b2,
                   double* out);

/* The shared SwiGLU expert applied to token t: out[D] = E_sh(x_t). */
void oracle_shared(const moe_oracle_cfg* c, const void* x, int64_t t,
                   const void* Wsh_gu, const void* Wsh_dn, double* out);

/* Layer output for the listed tokens given their routing (idx, w indexed by
 * token t as idx[t*k+j]):  y[i*D + d] = sum_j w_j E_{idx_j}(x_t) + E_sh(x_t).
 * slot_out (nullable) receives w_j E_{idx_j}(x_t) per slot at
 * slot_out[(i*k+j)*D + d] (zero for a dropped slot); shared_out (nullable)
 * receives E_sh(x_t).  Tokens run in parallel (OpenMP). */
void oracle_layer(const moe_oracle_cfg* c, const void* x, const int32_t* idx,
                  const double* w, const void* W1, const void* b1,
                  const void* W2, const void* b2, const void* Wsh_gu,
                  const void* Wsh_dn, int64_t ntok, const int64_t* tokens,
                  double* y, double* slot_out, double* shared_out);

/* Router followed by the layer for the listed tokens (idx/w/y indexed by
 * list position).  This is the whole per-token forward pass. */
void oracle_forward(const moe_oracle_cfg* c, const void* x, const float* W_r,
                    const float* bias, const void* W1, const void* b1,
                    const void* W2, const void* b2, const void* Wsh_gu,
                    const void* Wsh_dn, int64_t ntok, const int64_t* tokens,
                    int32_t* idx, double* w, double* y);

/* Gradient of oracle_forward over all T tokens for the output gradient
 * dy[T,D] (fp64): dx[T,D]; dW_r[M,D]; dW1, db1, dW2, db2 and dWsh_gu, dWsh_dn
 * in the layouts of the weights they belong to (db1 / db2 nullable: no
 * biases; the shared ones only written when F_shared > 0).  The top-k
 * selection and the correction bias pass no gradient (piecewise constant);
 * the weights pass it through the renormalisation and the gate values to the
 * logits.  Per-expert load statistics of the same pass: load_count[e] slots
 * routed to e, load_score[e] the sum over tokens of e's gate value (softmax
 * probability or sigmoid score).  expert_slot (nullable) keeps the expert
 * weight and bias gradients of some experts only: expert e's go to slot
 * expert_slot[e] of n_slots-expert arrays, none when it is negative (for
 * large layers, where all M would not fit); NULL keeps all M in place.
 * Single-threaded, for small shapes or few tokens. */
void oracle_backward(const moe_oracle_cfg* c, const void* x, const float* W_r,
                     const float* bias, const void* W1, const void* b1, const void* W2,
                     const void* b2, const void* Wsh_gu, const void* Wsh_dn, const double* dy,
                     double* dx, double* dW_r, double* dW1, double* db1, double* dW2,
                     double* db2, double* dWsh_gu, double* dWsh_dn, int64_t* load_count,
                     double* load_score, const int32_t* expert_slot, int64_t n_slots);

/* Number of OpenMP threads the oracle will use. */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
