/*
 * oracle.h -- plain, slow CPU oracle for one decode step through a stack of
 * MoE transformer layers.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * calls it and shares no code, header, table or helper with it.
 *
 * What it computes.  The pages describe a model whose every layer is an MoE
 * block in which a router picks a few experts per token, independently per
 * layer, and whose decode step streams every layer's weights once
 * [P3 "TPU Megakernel Achieves 709 tokens/s on Kimi K3, Outpacing GB200",
 *  explanatory box under "Cross-Layer Weight Prefetching"; P2 myzaker article,
 *  section "把几百个小 kernel，焊成一个大程序"].  The megakernel changes only the
 * schedule of that step, not its mathematics [P4 tanhow.com blog translation,
 * paragraph on the megakernel removing kernel boundaries], so the oracle is
 * the plain layer-by-layer, token-by-token definition:
 *
 *   pre-norm block   h1 = h + Attn(RMSNorm(h; g1))          (attention stacks)
 *                    h2 = h1 + MoE(RMSNorm(h1; g2))
 *   RMSNorm(x; g)_i  = x_i / sqrt(mean_j x_j^2 + eps) * g_i
 *   router           z = Wr x (+ b),  p = softmax(z)
 *   top-k            the k largest p, equal values ranked by lower expert id
 *   renormalise      w_i = p_i / sum_{j in S} p_j
 *   SwiGLU expert    y_e = Wd_e (silu(Wg_e x) * (Wu_e x)),  silu(u) = u/(1+e^-u)
 *   combine          MoE(x) = sum_{e in S} w_e y_e + sum_shared y_s
 *   GQA attention    q = Wq x, k = Wk x, v = Wv x; RoPE (half-split pairs
 *                    (i, i+hd/2), inv_freq_i = theta^(-2i/hd)) on q and k at the
 *                    row's position; k, v rounded to bf16 (round to nearest
 *                    even) and stored in the cache at that position; head h
 *                    reads kv head h / (H/G); scores q.K_j / sqrt(hd) over
 *                    cache positions 0..pos; softmax; o = sum_j a_j V_j;
 *                    Attn(x) = Wo concat_h(o_h).
 *
 * Precision.  Every sum is accumulated in double.  Weights, norms and the KV
 * cache are widened exactly from their stored type (fp32 or bf16).  The hidden
 * state stays in double between layers; only the step's output is rounded to
 * fp32.  The one rounding inside the step is the bf16 rounding of the new k
 * and v rows, since the cache holds bf16.
 *
 * Storage (all row-major, [out][in] as for a linear layer's weight):
 *   g1, g2 [d];  wq [H*hd][d];  wk, wv [G*hd][d];  wo [d][H*hd];
 *   wr [E][d];   br [E] fp32 or NULL;
 *   w_gate[e], w_up[e] [F][d];  w_down[e] [d][F]   (one pointer per expert)
 *   s_gate[s], s_up[s] [F][d];  s_down[s] [d][F]   (one pointer per shared expert)
 *   KV cache per layer: k, v [n_seq][G][capacity][hd] bf16 (uint16 bits)
 *   rows: row r belongs to sequence r / rows_per_seq and sits at positions[r].
 *
 * Errors: functions return 0 on success and a negative code otherwise
 * (ORC_EARG bad argument, ORC_EPTR a needed expert pointer is NULL, ORC_EPOS a
 * position outside the cache).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_OK = 0, ORC_EARG = -1, ORC_EPTR = -2, ORC_EPOS = -3 };

typedef struct orc_dims {
  int d;          /* hidden size */
  int n_experts;  /* E routed experts */
  int top_k;      /* k */
  int d_ff;       /* F expert width */
  int n_shared;   /* always-on shared experts, weight 1 */
  int wdtype;     /* ORC_F32 or ORC_BF16: matrices and norm gains */
  double rms_eps;
  int n_heads;    /* H; 0 = no attention */
  int n_kv_heads; /* G */
  int head_dim;   /* hd */
  double rope_theta;
} orc_dims;

typedef struct orc_layer {
  const void* g1;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* g2;
  const void* wr;
  const float* br;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
  const void* const* s_gate;
  const void* const* s_up;
  const void* const* s_down;
} orc_layer;

typedef struct orc_kv {
  int n_seq;
  int capacity;
  uint16_t* k; /* [n_seq][G][capacity][hd] */
  uint16_t* v;
} orc_kv;

/* ---- building blocks (exported so the tests can pin each one) ---- */
double orc_bf16_to_double(uint16_t b);
uint16_t orc_double_to_bf16(double x);
void orc_rmsnorm(int n, const double* x, const void* g, int gdtype, double eps, double* out);
void orc_matvec(int n_out, int n_in, const void* w, int wdtype, const double* x, double* y);
double orc_silu(double u);
void orc_softmax(int n, const double* z, double* p);
/* top-k of p with lower-id tie-break, weights renormalised over the set;
 * forced (nullable) replaces the selection, weights still come from p. */
void orc_topk(int n, int k, const double* p, const int* forced, int* ids, double* w);
void orc_expert(int d, int F, const void* wg, const void* wu, const void* wdn, int wdtype,
                const double* x, double* y);
void orc_rope(int hd, double theta, int pos, double* x);

/* ---- layer stages ---- */
/* h_out = h + Attn(RMSNorm(h; g1)) for all M rows; writes the new k, v rows. */
int orc_attn_block(const orc_dims* dm, const orc_layer* lw, int M, int rows_per_seq,
                   const int32_t* positions, orc_kv* kv, const double* h, double* h_out);
/* router on RMSNorm(h; g2): logits [M][E], ids [M][k], w [M][k], margin [M]
 * (k-th minus (k+1)-th largest logit; +inf when k == E).  forced [M][k]
 * nullable. */
int orc_route(const orc_dims* dm, const orc_layer* lw, int M, const double* h, const int* forced,
              double* logits, int* ids, double* w, double* margin);
/* h_out = h + MoE(RMSNorm(h; g2)) with the given routing. */
int orc_moe_block(const orc_dims* dm, const orc_layer* lw, int M, const double* h, const int* ids,
                  const double* w, double* h_out);

/* Whole step through L layers from fp32 hidden_in to fp32 hidden_out.
 * kv: array of L per-layer caches (ignored without attention).  Trace
 * outputs are nullable: logits [L][M][E], ids [L][M][k], w [L][M][k],
 * margin [L][M]. */
int orc_forward(const orc_dims* dm, int L, const orc_layer* layers, int M, int rows_per_seq,
                const int32_t* positions, orc_kv* kv, const float* hidden_in, float* hidden_out,
                double* t_logits, int* t_ids, double* t_w, double* t_margin);

/* ---- multi-head latent attention (MLA) at decode, absorbed form ----
 * The pages name MLA as the attention of the model (P4, paragraph on VMEM
 * budgeting: the KV cache MLA uses is short-lived) and define nothing else;
 * the definition followed is the published one (multi-head latent
 * attention, DeepSeek-V2 report, section 2.1): a cache row per position is
 * a compressed latent c (Dc values) and one rotary key k_R (Dr values)
 * shared by all heads; head h's key is (W_UK,h c, k_R) and its value
 * W_UV,h c.  At decode the up-projections fold into the query and the
 * output, so the attention itself runs over the cache rows directly:
 *   q[r][h]  = (W_UK,h^T q_nope, q_rope)   (Dc + Dr values, given)
 *   s_j      = scale * q[r][h] . cache[seq][j],   j = 0 .. positions[r]
 *   a        = softmax(s)
 *   out[r][h][i] = sum_j a_j cache[seq][j][i],   i < Dc
 * (the head's output is then W_UV,h out[r][h]).  Row r belongs to sequence
 * r / rows_per_seq; cache is bf16 [n_seq][capacity][Dc + Dr]. */
int orc_mla_attention(int M, int rows_per_seq, int H, int Dc, int Dr, int n_seq, int capacity, double scale,
                      const double* q, const uint16_t* cache, const int32_t* positions, double* out);

/* threads the oracle's parallel loops use (1 when built without OpenMP) */
int orc_num_threads(void);
int orc_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
