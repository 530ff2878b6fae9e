/*
 * mk.h -- C ABI of libmk.so: one decode step through a stack of MoE
 * transformer layers, run on an MI355X (gfx950) as ONE persistent kernel.
 *
 * What a step computes.  For each of L layers, for each of M rows (tokens):
 *     (attention stacks)  h1 = h + Wo . GQA-Attn(RoPE(Wq x), RoPE(Wk x), Wv x),
 *                         x = RMSNorm(h; attn_norm)
 *     h2 = h1 + sum_{e in top-k} w_e . Wd_e (silu(Wg_e y) * Wu_e y)
 *             + sum_shared Wd_s (silu(Wg_s y) * Wu_s y),   y = RMSNorm(h1; moe_norm)
 * with router logits z = Wr y (+ bias), p = softmax(z), the top-k experts by
 * p (equal values: lower expert id first) and w_e = p_e / sum_{top-k} p.
 * The pages describe exactly this shape of work: a deep stack of MoE layers in
 * which a router picks a few experts per token independently per layer, each
 * layer's attention preceding its MoE, and the entire decode step run inside
 * one program so that weight loads are no longer tied to per-operator kernel
 * boundaries [P3 "TPU Megakernel Achieves 709 tokens/s on Kimi K3, Outpacing
 * GB200", sections "The Key Innovation: 92 MoE Layers in a Single Pallas
 * Kernel" and "Cross-Layer Weight Prefetching"; P2 myzaker article, section
 * "把几百个小 kernel，焊成一个大程序"; P4 tanhow.com translation of the authors'
 * post, paragraphs on kernel-boundary bubbles and on the megakernel].
 * Definitions of the operators (RMSNorm with eps inside the root and a
 * multiplicative gain, SwiGLU, half-split RoPE with inv_freq_i =
 * theta^(-2i/hd), GQA head h reading kv head h / (H/G), scale 1/sqrt(hd)) are
 * the standard ones; the pages give none.
 *
 * Storage.  Every matrix is row-major [out][in] (a linear layer's weight):
 *   attn_norm, moe_norm  [d]                 dtype (fp32 or bf16)
 *   wq [H*hd][d], wk [G*hd][d], wv [G*hd][d], wo [d][H*hd]   dtype
 *   w_router [E][d] dtype;  b_router [E] fp32 or NULL
 *   w_gate, w_up [E][F][d];  w_down [E][d][F]        dtype, experts packed
 *   s_gate, s_up [n_shared][F][d];  s_down [n_shared][d][F]
 * bf16 means the upper 16 bits of an IEEE binary32 (round-to-nearest-even
 * from fp32 wherever the library rounds).  Hidden rows are fp32 [M][d].
 * KV cache (bf16): k and v each [L][kv->n_seq][G][capacity][hd], contiguous;
 * a step uses sequences 0 .. rows/rows_per_seq - 1 of it (a cache may hold
 * more sequences than one handle's step, e.g. batch 1 over a batch-8 cache).
 * Row r belongs to sequence r / rows_per_seq and sits at positions[r]; a
 * step writes the row's k, v (RoPE applied to k, rounded to bf16) at that
 * position and attends to cache positions 0..positions[r] of its sequence.
 * Several rows of one sequence (a speculative-verify pass) must hold distinct
 * positions; each row then sees the new rows of its sequence at lower or
 * equal positions (causal).
 *
 * Ownership.  Weights, KV cache, hidden buffers and positions are device
 * memory owned by the caller; the library never copies, repacks or frees
 * them and only reads the weights.  The handle owns its workspace (scratch
 * activations, barrier counters, the device copy of the weight-pointer
 * table), allocated in mk_create and freed in mk_destroy.
 *
 * Errors.  Every call returns MK_OK (0) or a negative mk_status.  Argument
 * checks that need no device data happen at once.  Conditions only the
 * device can see (a position outside [0, capacity), two rows of one
 * sequence at the same position, a grid barrier or an attention split
 * combine that does not complete within the device watchdog) set
 * a device error flag; the step then skips the affected writes and ends, and
 * the next mk_sync returns the error and clears it.  mk_strerror describes a
 * status; mk_last_error describes the most recent failure of this thread.
 *
 * Concurrency.  A handle's workspace is shared by its launches: do not run
 * steps of one handle on two streams at once.  Several handles may share the
 * same weights (e.g. batch 1 and batch 8 over one stack).  A step is a launch
 * of one workgroup per CU, each taking the CU's whole LDS, whose workgroups
 * wait for each other at grid barriers, so two steps must not run at the
 * same time: the library orders the steps of all handles on a device (a step
 * enqueued on another stream than the device's previous step waits for that
 * step on the GPU).  Steps enqueued while their stream captures a graph are
 * not ordered: replays of such graphs on different streams must not overlap.
 * Kernels of other code running beside a step delay its start on the CUs
 * they hold; a step whose workgroups do not all arrive within the watchdog
 * ends with MK_ERR_TIMEOUT.
 */
#ifndef MK_H
#define MK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 1

typedef enum mk_status {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = -1, /* NULL/aliased pointer, inconsistent sizes, bad position (device) */
  MK_ERR_UNSUPPORTED = -2, /* shape or dtype outside what the kernels implement */
  MK_ERR_DEVICE = -3,      /* no suitable gfx950 device, or one workgroup per CU cannot be co-resident */
  MK_ERR_HIP = -4,         /* a HIP runtime call or launch failed */
  MK_ERR_TIMEOUT = -5      /* a grid barrier or split combine did not complete (device watchdog) */
} mk_status;

typedef enum mk_dtype { MK_F32 = 0, MK_BF16 = 1 } mk_dtype;

typedef struct mk_config {
  int32_t n_layers;        /* L >= 1 */
  int32_t d_model;         /* d: row length 1, 2, 4 or 8 KiB in the weight dtype */
  int32_t n_experts;       /* E, 1..64 */
  int32_t top_k;           /* k, 1..min(E, 8) */
  int32_t n_shared;        /* always-on shared experts, weight 1; 0..4, and
                              min(rows, 8) * n_shared * d_ff * 4 <= 39424 bytes */
  int32_t d_ff;            /* F: row length of w_down, 1, 2, 4 or 8 KiB */
  int32_t dtype;           /* mk_dtype of matrices and norm gains */
  int32_t has_router_bias; /* b_router must be non-NULL when set */
  float rms_eps;           /* > 0 */
  int32_t has_attn;        /* 0: MoE-only layers (h1 = h) */
  int32_t n_heads;         /* H (attention stacks); H * head_dim rows of 2, 4 or 8
                              KiB in bf16 (1..8 KiB in fp32) */
  int32_t n_kv_heads;      /* G, H % G == 0.  Q = rows_per_seq * H / G query vectors
                              per (sequence, kv head): Q <= 32, and Q <= 4 for fp32
                              stacks.  Each (sequence, kv head) takes 1 attention
                              task when Q <= 4, else n = ceil(Q / 16) tasks of Q / n
                              queries (n must divide Q); sequences * G * n per
                              launch must not outnumber the CUs */
  int32_t head_dim;        /* hd = 128 */
  float rope_theta;        /* > 0 */
  int32_t rows;            /* M, 1..64, fixed per handle.  Above 8, a multiple of 8 with
                              rows_per_seq dividing 8.  With bf16 weights the step then
                              runs its rows/8 groups of 8 rows (whole sequences) in one
                              launch: each group on an equal share of the CUs for the
                              attention block, the router and the shared expert (the
                              groups stream the same weight tiles in step, so each tile
                              is read from HBM about once), and the routed experts as
                              tasks of one expert and at most 8 of the rows of all groups
                              routed to it, spread over every CU (an expert chosen by n
                              rows is streamed ceil(n/8) times).  With fp32 weights, or
                              where the CUs do not split that way (a power-of-two number
                              per group and XCD), as rows/8 launches of 8 rows on the
                              stream */
  int32_t rows_per_seq;    /* 1 for decode; > 1 for a verify pass; divides M */
  int32_t kv_capacity;     /* positions per sequence in the cache (attention stacks) */
} mk_config;

typedef struct mk_layer_weights {
  const void* attn_norm;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* moe_norm;
  const void* w_router;
  const float* b_router;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* s_gate;
  const void* s_up;
  const void* s_down;
} mk_layer_weights;

typedef struct mk_kv_cache {
  void* k;          /* [L][n_seq][G][capacity][hd] bf16, device */
  void* v;
  int32_t n_seq;    /* >= rows / rows_per_seq */
  int32_t capacity; /* == cfg.kv_capacity */
} mk_kv_cache;

typedef struct mk_info {
  int32_t n_cu;              /* workgroups in the persistent grid (one per CU) */
  int32_t threads;           /* threads per workgroup */
  int32_t lds_bytes;         /* dynamic LDS per workgroup */
  int32_t barriers_per_step; /* grid barriers one launch executes (a step of row groups in
                                one launch has one more per layer, where the groups
                                publish their routing) */
  int32_t attn_splits;       /* KV splits per (sequence, kv head) */
  int32_t launches_per_step; /* kernel launches of one mk_decode_step: 1, or rows/8 when the
                                row groups run one launch each */
  int64_t workspace_bytes;   /* device memory owned by the handle */
} mk_info;

typedef struct mk_handle mk_handle;

/* Validate cfg, bind the weights of all L layers (host array `layers` of
 * device pointers, read at this call only), allocate the workspace.  On
 * success *out receives the handle.  Errors: INVALID_ARG, UNSUPPORTED,
 * DEVICE, HIP. */
int mk_create(const mk_config* cfg, const mk_layer_weights* layers, mk_handle** out);

/* Enqueue one decode step on `stream` (a hipStream_t; NULL = default
 * stream) and return at once.  hidden_in [M][d] fp32, positions [M] int32,
 * hidden_out [M][d] fp32 are device pointers; hidden_out must not overlap
 * hidden_in.  kv may be NULL only for stacks without attention.  Errors:
 * INVALID_ARG, HIP.
 * The call may be captured into a HIP graph and replayed: the launch tag that
 * the attention split combine checks is taken on the device at launch start,
 * so every replay gets a new one. */
int mk_decode_step(mk_handle* h, const float* hidden_in, const int32_t* positions, const mk_kv_cache* kv,
                   float* hidden_out, void* stream);

/* The same step as a sequence of kernel launches, one per phase of every
 * layer (QKV, attention, output projection, router + shared gate/up, routed
 * gate/up, down projection; 6 per layer, 7 with several rows), with no
 * weight prefetch across a launch boundary.  This is the many-small-kernels
 * execution that P4 (the paragraph on kernel-boundary bubbles) measures the
 * megakernel against, kept as a baseline.  It runs the same phase code, so
 * hidden_out, the cache rows and the trace equal those of mk_decode_step
 * bit for bit.  Arguments, ownership and errors as mk_decode_step;
 * mk_set_timing does not apply. */
int mk_decode_step_phased(mk_handle* h, const float* hidden_in, const int32_t* positions, const mk_kv_cache* kv,
                          float* hidden_out, void* stream);

/* Size of the fixed device array that mk_decode_step_noalloc uses as its
 * workspace: one per device, held from the library's load until the process
 * ends. */
#define MK_NOALLOC_SCRATCH_BYTES (64u << 20)

/* mk_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same step, bit for bit, with the step's workspace (activations and
 * barrier counters) in a fixed array of MK_NOALLOC_SCRATCH_BYTES inside the
 * library instead of the handle's workspace.  The call allocates nothing; the
 * array's device address is taken once per device by the first mk_create on
 * that device.  Arguments, layouts and ownership as mk_decode_step.  Errors:
 * as mk_decode_step, and UNSUPPORTED when the handle's workspace
 * (mk_info.workspace_bytes without its barrier block and pointer table) does
 * not fit the array (about 64 MiB: e.g. a 16-layer MoE-only stack, or an
 * attention stack of up to ~50 layers at one row; not the 92-layer stack).
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (nothing a step reads depends on them): calls that overlap
 * on one device (two streams or threads, any handles) race and must not be
 * made.  Device-side errors are reported and cleared by the next mk_sync of
 * the same handle, which then clears the whole array. */
int mk_decode_step_noalloc(mk_handle* h, const float* hidden_in, const int32_t* positions, const mk_kv_cache* kv,
                           float* hidden_out, void* stream);

/* Free the workspace and the handle.  NULL is accepted. */
int mk_destroy(mk_handle* h);

/* Wait for `stream` and report (then clear) any device-side error of this
 * handle's steps: TIMEOUT or INVALID_ARG.  Clearing resets the barrier state
 * and zeroes the handle's workspace. */
int mk_sync(mk_handle* h, void* stream);

/* Record routing per step into device buffers (any may be NULL; all NULL
 * turns tracing off): ids [L][M][k] int32, w [L][M][k] fp32 (renormalised
 * weights, in top-k order), logits [L][M][E] fp32 (after bias). */
int mk_set_trace(mk_handle* h, int32_t* ids, float* w, float* logits);

/* Per-phase timestamps for profiling (NULL turns it off).  stamps is a
 * device buffer of int64 [n_cu][4 * (barriers_per_step + 1)]: workgroup c
 * writes the 100 MHz device realtime counter at four points of each phase
 * i, into slots 4i .. 4i+3: the phase start (after the preceding grid
 * barrier), the start and the end of its weight-tile loop, and the phase end
 * (before the next barrier).  Phases in order per layer: QKV, ATTN, WO
 * (attention stacks), RS, RG, DOWN; with more than one row DOWN is two
 * phases (the expert-major products, then the column sums, which stream no
 * tiles and may leave their loop slots unset).  A step of more than 8 rows
 * leaves the stamps of its last launch. */
int mk_set_timing(mk_handle* h, int64_t* stamps);

/* Device watchdog of the handle's later steps, in ticks of the 100 MHz
 * device realtime counter (default 200,000,000: 2 s); ticks >= 1, else
 * INVALID_ARG.  Every grid-barrier poll and split-combine wait of a step gives
 * up after this long: the step then ends early on every workgroup, its output
 * and cache rows are undefined, and the next mk_sync returns TIMEOUT and
 * resets the handle, which stays usable.  A limit far below a step's barrier
 * latency (a few ticks) forces that path, for tests of error handling. */
int mk_set_watchdog(mk_handle* h, int64_t ticks);

/* Launch geometry and workspace size of a handle. */
int mk_get_info(const mk_handle* h, mk_info* info);

const char* mk_strerror(int status);
const char* mk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
