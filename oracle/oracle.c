/*
 * oracle.c -- plain CPU oracle for one decode step through a stack of MoE
 * transformer layers.  TEST INFRASTRUCTURE ONLY: loaded by the test suite,
 * the smoke check and the benchmark's CPU-baseline leg, never by the product
 * path, and sharing no code with it.
 *
 * Every function below is the textbook definition written out with double
 * accumulation, in the order the definition states it.  The pages fix the
 * structure (a deep stack of MoE layers, a router choosing a few experts per
 * token in every layer, attention before the MoE block, the whole step being
 * one forward pass) but print no formula; the formulas are the standard ones
 * for those operators, listed in oracle.h.
 *
 * Sources for the structure:
 *  - P3 "TPU Megakernel Achieves 709 tokens/s on Kimi K3, Outpacing GB200",
 *    section "The Key Innovation: 92 MoE Layers in a Single Pallas Kernel"
 *    (all MoE layers of the model inside one program) and the explanatory box
 *    under "Cross-Layer Weight Prefetching" (router selects a few experts per
 *    token; routing is independent per layer).
 *  - P2 myzaker article, section "把几百个小 kernel，焊成一个大程序" (one call runs
 *    the whole forward; layer N+1's attention weights are fetched during
 *    layer N's MoE, so every layer is attention then MoE).
 *  - P4 tanhow.com translation of the authors' post, paragraph on VMEM
 *    budgeting (activations stay resident for the whole forward, the KV cache
 *    is short-lived): a KV cache is read by the attention of every layer.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of the next parallel loops (timing only: every output is summed
   in the same fixed order whatever the thread count). */
int orc_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16, ties to even, in one step (no detour
 * through binary32).  bf16 has an 8-bit significand (7 stored bits). */
uint16_t orc_double_to_bf16(double x) {
  if (isnan(x)) return 0x7fc0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int e;
  double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  /* normal bf16: exponent field 1..254 means a in [2^-126, 2^128) */
  if (e - 1 < -126) {
    /* subnormal range: quantum is 2^-133 */
    double q = ldexp(1.0, -133);
    double n = a / q;
    double r = nearbyint(n); /* default rounding mode: ties to even */
    uint32_t mant = (uint32_t)r;
    /* mant may reach 2^7 (smallest normal) which encodes naturally */
    return (uint16_t)(sign | mant);
  }
  /* significand with 8 bits: scale m in [0.5,1) to [128, 256) */
  double s = ldexp(m, 8);
  double r = nearbyint(s);
  if (r >= 256.0) {
    r = 128.0;
    e += 1;
  }
  int biased = (e - 1) + 127;
  if (biased >= 255) return (uint16_t)(sign | 0x7f80); /* overflow to inf */
  uint32_t mant7 = (uint32_t)r - 128u;
  return (uint16_t)(sign | ((uint32_t)biased << 7) | mant7);
}

/* element i of a stored tensor, widened exactly */
static double wget(const void* p, int dtype, size_t i) {
  if (dtype == ORC_BF16) return orc_bf16_to_double(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

/* RMSNorm: out_i = x_i / sqrt(mean(x^2) + eps) * g_i  (eps inside the root,
 * multiplicative gain). */
void orc_rmsnorm(int n, const double* x, const void* g, int gdtype, double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * inv * wget(g, gdtype, (size_t)i);
}

/* y_o = sum_i W[o][i] x_i, W stored [n_out][n_in] row-major. */
void orc_matvec(int n_out, int n_in, const void* w, int wdtype, const double* x, double* y) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static) if (n_out >= 256)
#endif
  for (int o = 0; o < n_out; ++o) {
    double s = 0.0;
    size_t base = (size_t)o * n_in;
    for (int i = 0; i < n_in; ++i) s += wget(w, wdtype, base + i) * x[i];
    y[o] = s;
  }
}

/* silu(u) = u * sigmoid(u) = u / (1 + e^-u) */
double orc_silu(double u) { return u / (1.0 + exp(-u)); }

/* p_i = e^{z_i} / sum_j e^{z_j}, shifted by the max for range */
void orc_softmax(int n, const double* z, double* p) {
  double m = z[0];
  for (int i = 1; i < n; ++i)
    if (z[i] > m) m = z[i];
  double s = 0.0;
  for (int i = 0; i < n; ++i) {
    p[i] = exp(z[i] - m);
    s += p[i];
  }
  for (int i = 0; i < n; ++i) p[i] /= s;
}

/* Top-k selection: repeatedly take the largest remaining p, the lower id
 * winning among equal values.  Then w_i = p_i / sum over the chosen set. */
void orc_topk(int n, int k, const double* p, const int* forced, int* ids, double* w) {
  if (forced) {
    for (int j = 0; j < k; ++j) ids[j] = forced[j];
  } else {
    char* taken = (char*)calloc((size_t)n, 1);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int i = 0; i < n; ++i) {
        if (taken[i]) continue;
        if (best < 0 || p[i] > p[best]) best = i; /* strict '>' keeps the lower id on ties */
      }
      ids[j] = best;
      taken[best] = 1;
    }
    free(taken);
  }
  double s = 0.0;
  for (int j = 0; j < k; ++j) s += p[ids[j]];
  for (int j = 0; j < k; ++j) w[j] = p[ids[j]] / s;
}

/* SwiGLU expert: y = Wd (silu(Wg x) * (Wu x)); Wg, Wu [F][d], Wd [d][F]. */
void orc_expert(int d, int F, const void* wg, const void* wu, const void* wdn, int wdtype,
                const double* x, double* y) {
  double* g = (double*)malloc(sizeof(double) * (size_t)F);
  double* u = (double*)malloc(sizeof(double) * (size_t)F);
  orc_matvec(F, d, wg, wdtype, x, g);
  orc_matvec(F, d, wu, wdtype, x, u);
  for (int f = 0; f < F; ++f) g[f] = orc_silu(g[f]) * u[f];
  orc_matvec(d, F, wdn, wdtype, g, y);
  free(g);
  free(u);
}

/* Rotary position embedding, half-split pairing: element i is paired with
 * element i + hd/2 and the pair is rotated by the angle pos * theta^(-2i/hd).
 *   x'_i        = x_i cos(a) - x_{i+hd/2} sin(a)
 *   x'_{i+hd/2} = x_{i+hd/2} cos(a) + x_i sin(a)  */
void orc_rope(int hd, double theta, int pos, double* x) {
  int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = pow(theta, -2.0 * (double)i / (double)hd);
    double a = (double)pos * inv_freq;
    double c = cos(a), s = sin(a);
    double x0 = x[i], x1 = x[i + half];
    x[i] = x0 * c - x1 * s;
    x[i + half] = x1 * c + x0 * s;
  }
}

static size_t kv_index(const orc_dims* dm, const orc_kv* kv, int seq, int g, int pos) {
  return (((size_t)seq * dm->n_kv_heads + g) * kv->capacity + pos) * dm->head_dim;
}

int orc_attn_block(const orc_dims* dm, const orc_layer* lw, int M, int rows_per_seq,
                   const int32_t* positions, orc_kv* kv, const double* h, double* h_out) {
  const int d = dm->d, H = dm->n_heads, G = dm->n_kv_heads, hd = dm->head_dim;
  if (H <= 0 || G <= 0 || H % G != 0 || hd % 2 != 0 || rows_per_seq <= 0) return ORC_EARG;
  const int qd = H * hd, kd = G * hd;
  double* xn = (double*)malloc(sizeof(double) * (size_t)d);
  double* q = (double*)malloc(sizeof(double) * (size_t)M * qd);
  double* kk = (double*)malloc(sizeof(double) * (size_t)kd);
  double* vv = (double*)malloc(sizeof(double) * (size_t)kd);
  double* o = (double*)malloc(sizeof(double) * (size_t)qd);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  int rc = ORC_OK;
  /* 1. projections, RoPE, and the cache write for every row first, so that a
   *    row may attend to the other new rows of its sequence at lower
   *    positions (several rows of one sequence are consecutive positions). */
  for (int r = 0; r < M && rc == ORC_OK; ++r) {
    int seq = r / rows_per_seq, pos = positions[r];
    if (seq >= kv->n_seq || pos < 0 || pos >= kv->capacity) {
      rc = ORC_EPOS;
      break;
    }
    orc_rmsnorm(d, h + (size_t)r * d, lw->g1, dm->wdtype, dm->rms_eps, xn);
    orc_matvec(qd, d, lw->wq, dm->wdtype, xn, q + (size_t)r * qd);
    orc_matvec(kd, d, lw->wk, dm->wdtype, xn, kk);
    orc_matvec(kd, d, lw->wv, dm->wdtype, xn, vv);
    for (int hh = 0; hh < H; ++hh) orc_rope(hd, dm->rope_theta, pos, q + (size_t)r * qd + (size_t)hh * hd);
    for (int g = 0; g < G; ++g) {
      orc_rope(hd, dm->rope_theta, pos, kk + (size_t)g * hd);
      size_t base = kv_index(dm, kv, seq, g, pos);
      for (int i = 0; i < hd; ++i) {
        kv->k[base + i] = orc_double_to_bf16(kk[(size_t)g * hd + i]);
        kv->v[base + i] = orc_double_to_bf16(vv[(size_t)g * hd + i]);
      }
    }
  }
  /* 2. attention per row and head over cache positions 0..pos */
  for (int r = 0; r < M && rc == ORC_OK; ++r) {
    int seq = r / rows_per_seq, pos = positions[r];
    int npos = pos + 1;
    double* s = (double*)malloc(sizeof(double) * (size_t)npos);
    double scale = 1.0 / sqrt((double)hd);
    for (int hh = 0; hh < H; ++hh) {
      int g = hh / (H / G);
      const double* qh = q + (size_t)r * qd + (size_t)hh * hd;
      for (int j = 0; j < npos; ++j) {
        size_t base = kv_index(dm, kv, seq, g, j);
        double dot = 0.0;
        for (int i = 0; i < hd; ++i) dot += qh[i] * orc_bf16_to_double(kv->k[base + i]);
        s[j] = dot * scale;
      }
      orc_softmax(npos, s, s);
      double* oh = o + (size_t)hh * hd;
      for (int i = 0; i < hd; ++i) oh[i] = 0.0;
      for (int j = 0; j < npos; ++j) {
        size_t base = kv_index(dm, kv, seq, g, j);
        for (int i = 0; i < hd; ++i) oh[i] += s[j] * orc_bf16_to_double(kv->v[base + i]);
      }
    }
    free(s);
    orc_matvec(d, qd, lw->wo, dm->wdtype, o, y);
    for (int i = 0; i < d; ++i) h_out[(size_t)r * d + i] = h[(size_t)r * d + i] + y[i];
  }
  free(xn);
  free(q);
  free(kk);
  free(vv);
  free(o);
  free(y);
  return rc;
}

int orc_route(const orc_dims* dm, const orc_layer* lw, int M, const double* h, const int* forced,
              double* logits, int* ids, double* w, double* margin) {
  const int d = dm->d, E = dm->n_experts, k = dm->top_k;
  if (k < 1 || k > E) return ORC_EARG;
  double* xn = (double*)malloc(sizeof(double) * (size_t)d);
  double* p = (double*)malloc(sizeof(double) * (size_t)E);
  double* srt = (double*)malloc(sizeof(double) * (size_t)E);
  for (int r = 0; r < M; ++r) {
    double* z = logits + (size_t)r * E;
    orc_rmsnorm(d, h + (size_t)r * d, lw->g2, dm->wdtype, dm->rms_eps, xn);
    orc_matvec(E, d, lw->wr, dm->wdtype, xn, z);
    if (lw->br)
      for (int e = 0; e < E; ++e) z[e] += (double)lw->br[e];
    orc_softmax(E, z, p);
    orc_topk(E, k, p, forced ? forced + (size_t)r * k : NULL, ids + (size_t)r * k, w + (size_t)r * k);
    if (margin) {
      /* k-th and (k+1)-th largest logits by plain insertion sort */
      for (int e = 0; e < E; ++e) srt[e] = z[e];
      for (int a = 1; a < E; ++a) {
        double v = srt[a];
        int b = a - 1;
        while (b >= 0 && srt[b] < v) {
          srt[b + 1] = srt[b];
          --b;
        }
        srt[b + 1] = v;
      }
      margin[r] = (k == E) ? INFINITY : srt[k - 1] - srt[k];
    }
  }
  free(xn);
  free(p);
  free(srt);
  return ORC_OK;
}

int orc_moe_block(const orc_dims* dm, const orc_layer* lw, int M, const double* h, const int* ids,
                  const double* w, double* h_out) {
  const int d = dm->d, E = dm->n_experts, k = dm->top_k, F = dm->d_ff;
  double* xn = (double*)malloc(sizeof(double) * (size_t)d);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  int rc = ORC_OK;
  for (int r = 0; r < M && rc == ORC_OK; ++r) {
    const double* hr = h + (size_t)r * d;
    double* outr = h_out + (size_t)r * d;
    orc_rmsnorm(d, hr, lw->g2, dm->wdtype, dm->rms_eps, xn);
    for (int i = 0; i < d; ++i) outr[i] = hr[i];
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)r * k + j];
      if (e < 0 || e >= E) { rc = ORC_EARG; break; }
      if (!lw->w_gate || !lw->w_up || !lw->w_down || !lw->w_gate[e] || !lw->w_up[e] || !lw->w_down[e]) {
        rc = ORC_EPTR;
        break;
      }
      orc_expert(d, F, lw->w_gate[e], lw->w_up[e], lw->w_down[e], dm->wdtype, xn, y);
      double we = w[(size_t)r * k + j];
      for (int i = 0; i < d; ++i) outr[i] += we * y[i];
    }
    for (int s = 0; s < dm->n_shared && rc == ORC_OK; ++s) {
      if (!lw->s_gate || !lw->s_up || !lw->s_down || !lw->s_gate[s] || !lw->s_up[s] || !lw->s_down[s]) {
        rc = ORC_EPTR;
        break;
      }
      orc_expert(d, F, lw->s_gate[s], lw->s_up[s], lw->s_down[s], dm->wdtype, xn, y);
      for (int i = 0; i < d; ++i) outr[i] += y[i];
    }
  }
  free(xn);
  free(y);
  return rc;
}

int orc_forward(const orc_dims* dm, int L, const orc_layer* layers, int M, int rows_per_seq,
                const int32_t* positions, orc_kv* kv, const float* hidden_in, float* hidden_out,
                double* t_logits, int* t_ids, double* t_w, double* t_margin) {
  const int d = dm->d, E = dm->n_experts, k = dm->top_k;
  if (L < 0 || M <= 0 || d <= 0 || E <= 0 || k <= 0 || k > E) return ORC_EARG;
  double* h = (double*)malloc(sizeof(double) * (size_t)M * d);
  double* h1 = (double*)malloc(sizeof(double) * (size_t)M * d);
  double* lg = (double*)malloc(sizeof(double) * (size_t)M * E);
  int* ids = (int*)malloc(sizeof(int) * (size_t)M * k);
  double* w = (double*)malloc(sizeof(double) * (size_t)M * k);
  double* mg = (double*)malloc(sizeof(double) * (size_t)M);
  int rc = ORC_OK;
  for (size_t i = 0; i < (size_t)M * d; ++i) h[i] = (double)hidden_in[i];
  for (int l = 0; l < L && rc == ORC_OK; ++l) {
    const orc_layer* lw = &layers[l];
    if (dm->n_heads > 0) {
      rc = orc_attn_block(dm, lw, M, rows_per_seq, positions, &kv[l], h, h1);
      if (rc) break;
    } else {
      memcpy(h1, h, sizeof(double) * (size_t)M * d);
    }
    rc = orc_route(dm, lw, M, h1, NULL, lg, ids, w, mg);
    if (rc) break;
    rc = orc_moe_block(dm, lw, M, h1, ids, w, h);
    if (t_logits) memcpy(t_logits + (size_t)l * M * E, lg, sizeof(double) * (size_t)M * E);
    if (t_ids) memcpy(t_ids + (size_t)l * M * k, ids, sizeof(int) * (size_t)M * k);
    if (t_w) memcpy(t_w + (size_t)l * M * k, w, sizeof(double) * (size_t)M * k);
    if (t_margin) memcpy(t_margin + (size_t)l * M, mg, sizeof(double) * (size_t)M);
  }
  if (rc == ORC_OK)
    for (size_t i = 0; i < (size_t)M * d; ++i) hidden_out[i] = (float)h[i];
  free(h);
  free(h1);
  free(lg);
  free(ids);
  free(w);
  free(mg);
  return rc;
}

/* MLA attention at decode over the latent cache (definition in oracle.h):
 * per row and head, the scores over positions 0..pos, their softmax, and the
 * softmax-weighted sum of the latent part of the cache rows. */
int orc_mla_attention(int M, int rows_per_seq, int H, int Dc, int Dr, int n_seq, int capacity, double scale,
                      const double* q, const uint16_t* cache, const int32_t* positions, double* out) {
  if (M <= 0 || rows_per_seq <= 0 || H <= 0 || Dc <= 0 || Dr < 0 || capacity <= 0) return ORC_EARG;
  const int Dk = Dc + Dr;
  for (int r = 0; r < M; ++r)
    if (r / rows_per_seq >= n_seq || positions[r] < 0 || positions[r] >= capacity) return ORC_EPOS;
#pragma omp parallel for schedule(static)
  for (int rh = 0; rh < M * H; ++rh) {
    const int r = rh / H, h = rh % H;
    const int seq = r / rows_per_seq, npos = positions[r] + 1;
    const double* qv = q + ((size_t)r * H + h) * Dk;
    const uint16_t* rows = cache + (size_t)seq * capacity * Dk;
    double* s = (double*)malloc(sizeof(double) * (size_t)npos);
    for (int j = 0; j < npos; ++j) {
      double dot = 0.0;
      for (int i = 0; i < Dk; ++i) dot += qv[i] * orc_bf16_to_double(rows[(size_t)j * Dk + i]);
      s[j] = scale * dot;
    }
    orc_softmax(npos, s, s);
    double* o = out + ((size_t)r * H + h) * Dc;
    for (int i = 0; i < Dc; ++i) o[i] = 0.0;
    for (int j = 0; j < npos; ++j)
      for (int i = 0; i < Dc; ++i) o[i] += s[j] * orc_bf16_to_double(rows[(size_t)j * Dk + i]);
    free(s);
  }
  return ORC_OK;
}
