// mk_internal.h -- structures shared by the host runtime and the persistent
// decode kernel.  Not part of the public ABI (include/mk.h).
#pragma once

#include <cstddef>
#include <cstdint>

namespace mk {

constexpr int kThreads = 256;           // 4 waves of 64 lanes: one wave per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kTileBytes = 8192;        // weight tile streamed through the LDS ring
constexpr int kChunk = 1024;            // one global_load_lds: 64 lanes x 16 B
constexpr int kRing = 12;               // ring slots (tiles in flight per CU)
constexpr int kSlotBytes = kTileBytes + 128;  // slot pitch: four neighbouring slots start in different LDS bank halves
constexpr int kMaxRows = 8;             // M
constexpr int kMaxGroups = 8;           // row groups of one launch (kMaxRows rows each)
constexpr int kMaxExperts = 64;         // E (one lane per expert in top-k)
constexpr int kMaxTopK = 8;
constexpr int kMaxShared = 4;
constexpr int kMaxQ = 32;               // query vectors per (sequence, kv head): rows_per_seq * H / G
constexpr int kMaxQTask = 16;           // query vectors per attention task (one 16-wide MFMA operand)
constexpr int kAttnTile = 32;           // positions per KV tile (hd = 128 bf16 -> 8 KB)
constexpr int kLdsTotal = 160 * 1024;
constexpr int kPartBytes = 16 * 1024;
constexpr int kMiscBytes = 8 * 1024;
constexpr int kXsBytes = kLdsTotal - kRing * kSlotBytes - kPartBytes - kMiscBytes;  // 38.5 KiB
constexpr int kPartStride = 132;        // words per attention partial: m, l, pad, pad, acc[128]
constexpr int kPartAcc = 3072;          // floats of GEMV partial sums in the part region
constexpr int kResFloats = kPartBytes / 4 - kPartAcc;  // epilogue residual slice after them

// device error flag bits
enum : unsigned { kErrTimeout = 1u, kErrPosition = 2u, kErrDupPosition = 4u };

// phases of a layer, in order (attention stacks run all; MoE-only stacks
// start at PH_RS; PH_DOWNB only with several rows)
enum Phase : int { PH_QKV = 0, PH_ATTN, PH_WO, PH_RS, PH_RG, PH_DOWN, PH_DOWNB };

// Device copy of one layer's weight pointers.
struct DevLayer {
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
};

// Byte offsets of one layer's activation scratch (all fp32, 256-byte aligned,
// every location written at most once per launch).
struct ActLayout {
  size_t h1;      // [M][d]
  size_t qkv;     // [M][(H+2G)*hd]   raw projections (RoPE applied by the reader)
  size_t part;    // [n_seq][G][S][Q][kPartStride] 64-bit tag words: attention partials (m, l, -, -, acc[hd])
  size_t o;       // [M][H*hd]
  size_t logits;  // [M][E]
  size_t a_s;     // [M][n_shared][F]  shared SwiGLU activations
  size_t a;       // [M][k][F]         routed SwiGLU activations (slot = top-k rank)
  size_t y_s;     // [M][d]            shared-expert down projection
  size_t yp;      // [M][k][d]         routed down projections per top-k slot, weighted (rows > 1 only)
  size_t h2;      // [M][d]            layer output (next layer's input)
  size_t rtab;    // [n_groups][M][k] i32 top-k ids, then [n_groups][M][k] fp32 weights: every row
                  // group's routing (group 0's workspace only; row-group launches)
  size_t stride;  // bytes per layer
};

// Barrier / counter block (each word on its own 256-byte line).
struct SyncLayout {
  static constexpr int kLine = 64;  // in uint32 words
  static constexpr int kGlobal = 0;
  static constexpr int kEpoch = 1 * kLine;
  static constexpr int kErr = 2 * kLine;
  static constexpr int kTag = 3 * kLine;     // tag epoch: launch-tagged words carry this + 1
  static constexpr int kGroup = 4 * kLine;   // 8 group counters
  static constexpr int kFlag = 12 * kLine;   // 8 group release flags
  static constexpr int kWords = 20 * kLine;
};

struct KParams {
  // shapes
  int L, d, E, k, S, F;
  int H, G, hd, M, rps, n_seq, cap;
  int kv_seqs;               // sequences in the caller's cache (its layer stride); >= n_seq
  int row0, seq0, Mt;        // this launch's first row and sequence within the step; rows of the step
  int attn, has_bias, wide;  // wide: weights are fp32
  float eps, theta;
  int n_splits;              // KV splits per (seq, kv head)
  int q_per_task;            // query vectors per attention task: rps * (H / G) / q_groups
  int q_groups;              // attention tasks per (seq, kv head, split), each with its own queries
  int only_l, only_ph;       // one phase per launch: its layer and Phase; only_ph < 0: the whole step
  // Row groups: n_groups groups of M rows (whole sequences) in one launch,
  // each on vncu = n_cu / n_groups workgroups, 2^cpx_log2 of them per XCD;
  // each group's activations at act + group * act_gstride (1, n_cu, 0, 0 for
  // a launch of one group)
  int n_groups, vncu, cpx_log2;
  size_t act_gstride;
  // launch geometry / LDS carve-up
  int n_cu;
  int ring_tiles;
  int x_bytes;               // LDS x region
  int barriers;              // grid barriers per step
  long long timeout_ticks;   // s_memrealtime ticks (100 MHz) before a barrier gives up
  // pointers
  const DevLayer* layers;
  const float* hidden_in;
  float* hidden_out;
  const int* positions;
  uint16_t* kcache;
  uint16_t* vcache;
  char* act;
  ActLayout al;
  unsigned* sync;            // SyncLayout
  long long* stamps;         // [n_cu][4*(barriers+1)] or null
  int* t_ids;
  float* t_w;
  float* t_logits;
};

}  // namespace mk

// One launch (one workgroup per CU) of the kernel that p selects.  Returns 0, a
// hipError_t of the launch (> 0), -1 (device query or the dynamic-LDS
// attribute failed), -2 (geometry outside the instantiations) or -3 (the
// kernel declares static LDS).
extern "C" int mk_launch_kernel(const mk::KParams* p, void* stream);
