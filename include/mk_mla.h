/*
 * mk_mla.h -- multi-head latent attention (MLA) at decode over a latent KV
 * cache, on gfx950.  C ABI (status codes and mk_strerror from mk.h).
 *
 * What it computes.  The pages name MLA as the attention of the model they
 * run (P4, tanhow.com translation of "TPS on Kimi K3 with TPU Megakernels",
 * paragraph on VMEM budgeting: the KV cache MLA uses is short-lived) and
 * give no shapes or formulas.  The definition followed is the published
 * one (multi-head latent attention, DeepSeek-V2 report, section 2.1): the
 * cache holds, per position, a compressed latent c (Dc values) and one
 * rotary key k_R (Dr values) shared by all heads; head h's key is
 * (W_UK,h c, k_R) and its value W_UV,h c.  At decode the up-projections fold
 * into the query and the output (the absorbed form), so the attention runs
 * over the cache rows themselves, every head against the same rows:
 *
 *   q[r][h] = (W_UK,h^T q_nope, q_rope)                       Dc + Dr values
 *   s_j     = scale * q[r][h] . cache[seq(r)][j],  j = 0 .. positions[r]
 *   out[r][h][i] = sum_j softmax(s)_j cache[seq(r)][j][i],    i < Dc
 *
 * and the head's output is W_UV,h out[r][h] (not done here).  Shapes follow
 * that model family: Dc = 512, Dr = 64.
 *
 * How.  Cache tiles of 32 positions through LDS, scores and the weighted
 * sum on the matrix cores, online softmax, the positions split over
 * workgroups whose partials a second launch combines (none with one split).
 * A sequence with few query vectors (decode: the H heads of one row) takes
 * workgroups of 16 vectors, two per CU, the 576 key columns split over the 4
 * waves and summed in a fixed order; a sequence with 128 or more (verify
 * blocks of several rows) takes workgroups of 64 vectors (8 waves, one per
 * CU), so that every tile is read once for 64 vectors.  Queries enter the
 * matrix cores as bf16 high and low parts (about 16 significant bits), the
 * cache as bf16 exactly, with fp32 accumulation.
 */
#ifndef MK_MLA_H
#define MK_MLA_H

#include <stdint.h>

#include "mk.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mk_mla_config {
  int32_t n_heads;      /* H: 16, 32, 64 or 128 query heads */
  int32_t latent_dim;   /* Dc: 512 */
  int32_t rope_dim;     /* Dr: 64 */
  int32_t rows;         /* M: rows per call, 1..64, fixed per handle */
  int32_t rows_per_seq; /* rows of one sequence (1 at decode; 8 for a verify pass); divides rows */
  int32_t n_seq;        /* sequences in the cache, >= rows / rows_per_seq */
  int32_t capacity;     /* positions per sequence in the cache, 1 .. 2^21 */
  float scale;          /* softmax scale, > 0 (1/sqrt(d_nope + Dr) in the published model) */
} mk_mla_config;

typedef struct mk_mla_info {
  int32_t splits;          /* KV splits per (sequence, query group) */
  int32_t workgroups;      /* workgroups of the split launch */
  int64_t workspace_bytes; /* device memory owned by the handle */
} mk_mla_info;

typedef struct mk_mla_handle mk_mla_handle;

/* Validates cfg on the current device (gfx950) and allocates the split
 * partials and an error word (hipMalloc).  MK_ERR_INVALID_ARG for a NULL
 * argument or an inconsistent config, MK_ERR_UNSUPPORTED for shapes outside
 * the ones above, MK_ERR_DEVICE for another device, MK_ERR_HIP when the
 * allocation fails.  *out is set only on MK_OK. */
int mk_mla_create(const mk_mla_config* cfg, mk_mla_handle** out);

/* out[r][h][0..Dc) = MLA attention of row r, head h (definition above).
 *   q         device fp32 [rows][H][Dc + Dr]: absorbed latent query, then
 *             the rotated rotary query; not pre-scaled.
 *   cache     device bf16 bits [n_seq][capacity][Dc + Dr]: per position the
 *             latent then the rotated rotary key; rows up to each row's
 *             position must be written before the call (the step's own row
 *             included); read only.
 *   positions device int32 [rows]: row r of sequence r / rows_per_seq
 *             attends positions 0 .. positions[r] of that sequence.
 *   out       device fp32 [rows][H][Dc]; must not overlap q or cache.
 * Asynchronous on stream (two launches).  A position outside [0, capacity)
 * is not read: the row's outputs are zero and the next mk_mla_sync returns
 * MK_ERR_INVALID_ARG.  Calls on one handle must not overlap (they share the
 * partials).  MK_ERR_INVALID_ARG for NULL arguments, MK_ERR_HIP when a
 * launch fails. */
int mk_mla_attention(mk_mla_handle* h, const float* q, const uint16_t* cache, const int32_t* positions,
                     float* out, void* stream);

/* Waits for the handle's work on stream; MK_ERR_INVALID_ARG when a call
 * since the last sync had a position outside the cache (the flag is then
 * cleared), MK_ERR_HIP on a runtime error. */
int mk_mla_sync(mk_mla_handle* h, void* stream);

int mk_mla_get_info(const mk_mla_handle* h, mk_mla_info* info);

/* Frees the handle and its device memory (after the stream's work on it has
 * finished).  Accepts NULL. */
int mk_mla_destroy(mk_mla_handle* h);

/* The message of the last MK_ERR_* status an mk_mla_* call returned on this
 * thread ("" if none). */
const char* mk_mla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
