// mk_runtime.hip -- host side of libmk.so: argument validation, workspace,
// the device copy of the weight-pointer table, the launch, and
// device-error reporting.  See include/mk.h for the contract.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_internal.h"

using mk::ActLayout;
using mk::DevLayer;
using mk::KParams;
using mk::SyncLayout;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool is_row_size_ok(long long bytes) {
  return bytes == 1024 || bytes == 2048 || bytes == 4096 || bytes == 8192;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// rows of one launch: a step of more than kMaxRows rows runs as
// rows / kMaxRows launches of whole sequences
int launch_rows(const mk_config& c) { return c.rows < mk::kMaxRows ? c.rows : mk::kMaxRows; }

}  // namespace

// ---- the workspace of mk_decode_step_noalloc
//
// A fixed device array in place of a handle's workspace, for callers that
// cannot allocate: the barrier block first, then the activation workspace.
// Every device that loads the library holds its own copy until the process
// ends.  In host code `scratch` is only a stand-in for the symbol: the device
// address of each device's copy comes from hipGetSymbolAddress, taken once
// per device (at the first mk_create on that device, with it current) and
// kept in g_scratch[device]; kernels get that address, never the symbol.
static __device__ __align__(256) char scratch[MK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchSync = (SyncLayout::kWords * 4 + 255) & ~(size_t)255;  // barrier block, 256-byte aligned
constexpr size_t kScratchAct = MK_NOALLOC_SCRATCH_BYTES - kScratchSync;          // activation workspace
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kScratchDevices] = {};

// Once per device, with that device current: the device address of its copy
// of `scratch`, zeroed (barrier counters and launch tags start at zero).
// Returns MK_OK or an error status.
int scratch_setup(int dev) {
  if (dev < 0 || dev >= kScratchDevices) return MK_OK;  // mk_decode_step_noalloc then refuses this device
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return MK_OK;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) return fail(MK_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
  e = hipMemset(ptr, 0, MK_NOALLOC_SCRATCH_BYTES);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(MK_ERR_HIP, "clearing the no-allocation workspace failed: %s", hipGetErrorString(e));
  g_scratch[dev] = static_cast<char*>(ptr);
  return MK_OK;
}

}  // namespace

struct mk_handle {
  mk_config cfg;
  int device;
  int n_cu;
  int n_groups;   // row groups of kMaxRows rows run in one launch (1: a launch per group of rows)
  int vncu;       // workgroups per row group
  int cpx_log2;   // log2 of a row group's workgroups per XCD
  int n_splits;
  int q_groups;  // attention tasks per (sequence, kv head, split)
  int q_task;    // query vectors per attention task
  int barriers;
  int ring_tiles;
  int x_bytes;
  ActLayout al;
  DevLayer* d_layers = nullptr;
  char* d_act = nullptr;
  unsigned* d_sync = nullptr;
  size_t act_bytes = 0;
  int32_t* t_ids = nullptr;
  float* t_w = nullptr;
  float* t_logits = nullptr;
  int64_t* stamps = nullptr;
  long long watchdog_ticks = 200LL * 1000 * 1000;  // 2 s of the 100 MHz realtime counter
  bool last_scratch = false;  // the last step ran in the no-allocation workspace
};

namespace {

int validate(const mk_config* c) {
  if (!c) return fail(MK_ERR_INVALID_ARG, "cfg is NULL");
  if (c->n_layers < 1) return fail(MK_ERR_INVALID_ARG, "n_layers must be >= 1");
  if (c->dtype != MK_F32 && c->dtype != MK_BF16) return fail(MK_ERR_UNSUPPORTED, "dtype must be MK_F32 or MK_BF16");
  const int es = c->dtype == MK_F32 ? 4 : 2;
  if (c->d_model < 1 || !is_row_size_ok((long long)c->d_model * es))
    return fail(MK_ERR_UNSUPPORTED, "d_model rows must be 1, 2, 4 or 8 KiB (d=%d)", c->d_model);
  if (c->d_ff < 1 || !is_row_size_ok((long long)c->d_ff * es))
    return fail(MK_ERR_UNSUPPORTED, "d_ff rows must be 1, 2, 4 or 8 KiB (F=%d)", c->d_ff);
  // bf16 GEMV tiles merge the two 1 KiB chunks a wave reads before the
  // cross-lane reduction, which needs rows of at least 2 KiB
  if (c->dtype == MK_BF16 && (c->d_model * es < 2048 || c->d_ff * es < 2048 ||
                              (c->has_attn && (long long)c->n_heads * c->head_dim * es < 2048)))
    return fail(MK_ERR_UNSUPPORTED, "bf16 rows (d_model, d_ff, n_heads*head_dim) must be at least 2 KiB");
  const int rpt_d = 8192 / (c->d_model * es);
  if (c->d_ff % rpt_d) return fail(MK_ERR_UNSUPPORTED, "d_ff must be a multiple of %d", rpt_d);
  const int rpt_f = 8192 / (c->d_ff * es);
  if (c->d_model % rpt_f) return fail(MK_ERR_UNSUPPORTED, "d_model must be a multiple of %d", rpt_f);
  if (c->n_experts < 1 || c->n_experts > mk::kMaxExperts) return fail(MK_ERR_UNSUPPORTED, "n_experts must be 1..64");
  if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > mk::kMaxTopK)
    return fail(MK_ERR_UNSUPPORTED, "top_k must be 1..min(n_experts, 8)");
  if (c->n_shared < 0 || c->n_shared > mk::kMaxShared) return fail(MK_ERR_UNSUPPORTED, "n_shared must be 0..4");
  if (!(c->rms_eps > 0.f)) return fail(MK_ERR_INVALID_ARG, "rms_eps must be > 0");
  if (c->rows < 1 || c->rows > 64) return fail(MK_ERR_UNSUPPORTED, "rows must be 1..64");
  if (c->rows > mk::kMaxRows && (c->rows % mk::kMaxRows || c->rows_per_seq < 1 || mk::kMaxRows % c->rows_per_seq))
    return fail(MK_ERR_UNSUPPORTED, "rows above %d must be a multiple of %d with rows_per_seq dividing %d", mk::kMaxRows,
                mk::kMaxRows, mk::kMaxRows);
  if ((size_t)launch_rows(*c) * c->n_shared * c->d_ff * 4 > (size_t)mk::kXsBytes)
    return fail(MK_ERR_UNSUPPORTED, "rows * n_shared * d_ff * 4 must fit %d bytes of LDS", mk::kXsBytes);
  if (c->rows_per_seq < 1 || c->rows % c->rows_per_seq) return fail(MK_ERR_INVALID_ARG, "rows_per_seq must divide rows");
  if (c->has_attn) {
    if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
      return fail(MK_ERR_INVALID_ARG, "n_heads must be a positive multiple of n_kv_heads");
    if (c->head_dim != 128) return fail(MK_ERR_UNSUPPORTED, "head_dim must be 128");
    if (c->rows_per_seq * (c->n_heads / c->n_kv_heads) > mk::kMaxQ)
      return fail(MK_ERR_UNSUPPORTED, "rows_per_seq * n_heads / n_kv_heads must be <= %d", mk::kMaxQ);
    if (c->dtype == MK_F32 && c->rows_per_seq * (c->n_heads / c->n_kv_heads) > 4)
      return fail(MK_ERR_UNSUPPORTED, "fp32 stacks support at most 4 query vectors per kv head and sequence");
    if (!is_row_size_ok((long long)c->n_heads * c->head_dim * es))
      return fail(MK_ERR_UNSUPPORTED, "n_heads*head_dim rows must be 1, 2, 4 or 8 KiB");
    if (c->d_model % (8192 / (c->n_heads * c->head_dim * es)))
      return fail(MK_ERR_UNSUPPORTED, "d_model must be a multiple of the rows per Wo tile");
    if (!(c->rope_theta > 0.f)) return fail(MK_ERR_INVALID_ARG, "rope_theta must be > 0");
    if (c->kv_capacity < 1) return fail(MK_ERR_INVALID_ARG, "kv_capacity must be >= 1");
    if ((long long)c->kv_capacity * c->head_dim * 2 >= (1LL << 31))
      return fail(MK_ERR_UNSUPPORTED, "kv_capacity too large");
  }
  return MK_OK;
}

}  // namespace

extern "C" {

const char* mk_strerror(int status) {
  switch (status) {
    case MK_OK: return "success";
    case MK_ERR_INVALID_ARG: return "invalid argument";
    case MK_ERR_UNSUPPORTED: return "unsupported configuration";
    case MK_ERR_DEVICE: return "no suitable gfx950 device or co-residency not possible";
    case MK_ERR_HIP: return "HIP runtime error";
    case MK_ERR_TIMEOUT: return "grid barrier timed out on the device";
    default: return "unknown status";
  }
}

const char* mk_last_error(void) { return g_last_error.c_str(); }

int mk_create(const mk_config* cfg, const mk_layer_weights* layers, mk_handle** out) {
  if (!out) return fail(MK_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = validate(cfg);
  if (rc) return rc;
  if (!layers) return fail(MK_ERR_INVALID_ARG, "layers is NULL");
  const mk_config& c = *cfg;
  for (int l = 0; l < c.n_layers; ++l) {
    const mk_layer_weights& w = layers[l];
    if (!w.moe_norm || !w.w_router || !w.w_gate || !w.w_up || !w.w_down)
      return fail(MK_ERR_INVALID_ARG, "layer %d: MoE weight pointer is NULL", l);
    if (c.has_router_bias && !w.b_router) return fail(MK_ERR_INVALID_ARG, "layer %d: b_router is NULL", l);
    if (c.n_shared > 0 && (!w.s_gate || !w.s_up || !w.s_down))
      return fail(MK_ERR_INVALID_ARG, "layer %d: shared expert pointer is NULL", l);
    if (c.has_attn && (!w.attn_norm || !w.wq || !w.wk || !w.wv || !w.wo))
      return fail(MK_ERR_INVALID_ARG, "layer %d: attention weight pointer is NULL", l);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MK_ERR_DEVICE, "no HIP device");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MK_ERR_DEVICE, "hipGetDeviceProperties failed");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MK_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  if (prop.maxSharedMemoryPerMultiProcessor < (size_t)mk::kLdsTotal)
    return fail(MK_ERR_DEVICE, "device has %zu bytes of LDS per CU, need %d", prop.maxSharedMemoryPerMultiProcessor,
                mk::kLdsTotal);

  rc = scratch_setup(dev);  // the no-allocation entry point's workspace on this device
  if (rc) return rc;
  mk_handle* h = new (std::nothrow) mk_handle();
  if (!h) return fail(MK_ERR_HIP, "out of host memory");
  h->cfg = c;
  h->device = dev;
  h->n_cu = prop.multiProcessorCount;
  const int M = launch_rows(c);
  const int n_seq = M / c.rows_per_seq;
  // A step of more than kMaxRows rows with bf16 weights runs its groups of
  // kMaxRows rows in one launch when the CUs split into equal groups with the
  // same power-of-two number on every XCD (workgroups are dealt to the 8 XCDs
  // round-robin); otherwise as one launch per group.
  h->n_groups = 1;
  h->vncu = h->n_cu;
  h->cpx_log2 = 0;
  if (c.rows > M && c.dtype == MK_BF16) {
    const int ng = c.rows / M;
    const int per = h->n_cu / ng;
    if (h->n_cu % (8 * ng) == 0 && ((per / 8) & (per / 8 - 1)) == 0) {
      h->n_groups = ng;
      h->vncu = per;
      while ((8 << h->cpx_log2) < per) ++h->cpx_log2;
    }
  }
  const int H = c.has_attn ? c.n_heads : 0, G = c.has_attn ? c.n_kv_heads : 0, hd = c.has_attn ? c.head_dim : 0;
  h->n_splits = 1;
  h->q_groups = 1;
  h->q_task = 0;
  if (c.has_attn) {
    // Up to 4 query vectors share a task (decode); more (several rows of a
    // sequence: verify) are split into groups of at most 16, one MFMA
    // operand each, which read the same cache tiles.
    const int Qall = c.rows_per_seq * (c.n_heads / c.n_kv_heads);
    h->q_groups = Qall <= 4 ? 1 : (Qall + mk::kMaxQTask - 1) / mk::kMaxQTask;
    if (Qall % h->q_groups) {
      delete h;
      return fail(MK_ERR_UNSUPPORTED, "rows_per_seq * n_heads / n_kv_heads = %d does not split into equal query "
                  "groups of at most %d", Qall, mk::kMaxQTask);
    }
    h->q_task = Qall / h->q_groups;
    if (n_seq * G * h->q_groups > h->vncu) {  // one attention task per CU at least
      delete h;
      return fail(MK_ERR_UNSUPPORTED, "%d sequences x %d kv heads x %d query groups exceed the %d CUs", n_seq, G,
                  h->q_groups, h->vncu);
    }
    int s = h->vncu / (n_seq * G * h->q_groups);
    if (s < 1) s = 1;
    int maxs = (c.kv_capacity + mk::kAttnTile - 1) / mk::kAttnTile;
    if (s > maxs) s = maxs;
    h->n_splits = s;
    // the split combine gathers, per split, the (m, l) words of the queries
    // its output slice touches and the slice's acc words into the x region
    const int nout = h->q_task * hd, nper = (nout + s - 1) / s;
    int maxw = 0;
    for (int z = 0; z < s; ++z) {
      const int o0 = z * nper, o1 = std::min(o0 + nper, nout);
      if (o0 >= o1) break;
      maxw = std::max(maxw, 2 * ((o1 - 1) / hd - o0 / hd + 1) + (o1 - o0));
    }
    if ((size_t)s * maxw * 4 > (size_t)mk::kXsBytes) {
      delete h;
      return fail(MK_ERR_UNSUPPORTED, "attention split combine needs %zu bytes of LDS scratch (%d available)",
                  (size_t)s * maxw * 4, mk::kXsBytes);
    }
  }
  {
    // epilogue residual slices (output columns of one CU, every row) live in
    // kResFloats floats of LDS
    const int esz = c.dtype == MK_BF16 ? 2 : 4;
    auto cols = [&](int row_elems) {
      const int rpt = mk::kTileBytes / (row_elems * esz);
      const int units = c.d_model / rpt;
      return ((units + h->vncu - 1) / h->vncu) * rpt;
    };
    int ncol = cols(c.d_ff);
    if (c.has_attn && cols(c.n_heads * c.head_dim) > ncol) ncol = cols(c.n_heads * c.head_dim);
    if (ncol * M > mk::kResFloats) {
      delete h;
      return fail(MK_ERR_UNSUPPORTED, "d_model * rows too large for %d CUs", prop.multiProcessorCount);
    }
  }
  // several rows: the routed down projection runs in two phases (expert-major
  // products, then the per-column sum), one more barrier per layer
  // and row groups in one launch meet at one more barrier per layer, where
  // they publish their routing
  h->barriers = c.n_layers * ((c.has_attn ? 6 : 3) + (M > 1 ? 1 : 0) + (h->n_groups > 1 ? 1 : 0)) - 1;
  // LDS: fixed carve-up (ring, x staging, per-row partial sums, misc)
  h->x_bytes = mk::kXsBytes;
  h->ring_tiles = mk::kRing;
  // activation scratch per layer
  const int E = c.n_experts, k = c.top_k, S = c.n_shared, F = c.d_ff, d = c.d_model;
  const int Q = c.has_attn ? c.rows_per_seq * (H / G) : 0;
  size_t off = 0;
  ActLayout al{};
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  al.h1 = take((size_t)M * d * 4);
  al.qkv = take((size_t)M * (H + 2 * G) * hd * 4);
  al.part = take((size_t)n_seq * G * h->n_splits * Q * mk::kPartStride * 8);
  al.o = take((size_t)M * H * hd * 4);
  al.logits = take((size_t)M * E * 4);
  al.a_s = take((size_t)M * S * F * 4);
  al.a = take((size_t)M * k * F * 4);
  al.y_s = take((size_t)M * d * 4);
  al.yp = take(M > 1 ? (size_t)M * k * d * 4 : 0);
  al.h2 = take((size_t)M * d * 4);
  al.rtab = take(h->n_groups > 1 ? (size_t)h->n_groups * M * c.top_k * 8 : 0);
  al.stride = align256(off);
  h->al = al;
  h->act_bytes = al.stride * c.n_layers * h->n_groups;  // a workspace per row group

  auto cleanup = [&]() {
    if (h->d_layers) (void)hipFree(h->d_layers);
    if (h->d_act) (void)hipFree(h->d_act);
    if (h->d_sync) (void)hipFree(h->d_sync);
    delete h;
  };
  std::vector<DevLayer> hl(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    const mk_layer_weights& w = layers[l];
    hl[l] = DevLayer{w.attn_norm, w.wq, w.wk, w.wv, w.wo, w.moe_norm, w.w_router, w.b_router,
                     w.w_gate, w.w_up, w.w_down, w.s_gate, w.s_up, w.s_down};
  }
  if (hipMalloc(&h->d_layers, sizeof(DevLayer) * c.n_layers) != hipSuccess ||
      hipMalloc(&h->d_act, h->act_bytes) != hipSuccess ||
      hipMalloc(&h->d_sync, SyncLayout::kWords * 4) != hipSuccess) {
    cleanup();
    return fail(MK_ERR_HIP, "workspace allocation failed");
  }
  if (hipMemcpy(h->d_layers, hl.data(), sizeof(DevLayer) * c.n_layers, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(h->d_sync, 0, SyncLayout::kWords * 4) != hipSuccess ||
      hipMemset(h->d_act, 0, h->act_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    cleanup();
    return fail(MK_ERR_HIP, "workspace initialisation failed");
  }
  *out = h;
  return MK_OK;
}

int mk_destroy(mk_handle* h) {
  if (!h) return MK_OK;
  int rc = MK_OK;
  if (h->d_layers && hipFree(h->d_layers) != hipSuccess) rc = MK_ERR_HIP;
  if (h->d_act && hipFree(h->d_act) != hipSuccess) rc = MK_ERR_HIP;
  if (h->d_sync && hipFree(h->d_sync) != hipSuccess) rc = MK_ERR_HIP;
  delete h;
  return rc == MK_OK ? MK_OK : fail(rc, "hipFree failed");
}

int mk_set_trace(mk_handle* h, int32_t* ids, float* w, float* logits) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "handle is NULL");
  h->t_ids = ids;
  h->t_w = w;
  h->t_logits = logits;
  return MK_OK;
}

int mk_set_timing(mk_handle* h, int64_t* stamps) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "handle is NULL");
  h->stamps = stamps;
  return MK_OK;
}

int mk_set_watchdog(mk_handle* h, int64_t ticks) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "handle is NULL");
  if (ticks < 1) return fail(MK_ERR_INVALID_ARG, "watchdog ticks must be >= 1");
  h->watchdog_ticks = ticks;
  return MK_OK;
}

int mk_get_info(const mk_handle* h, mk_info* info) {
  if (!h || !info) return fail(MK_ERR_INVALID_ARG, "NULL argument");
  info->n_cu = h->n_cu;
  info->threads = mk::kThreads;
  info->lds_bytes = h->ring_tiles * mk::kSlotBytes + h->x_bytes + mk::kPartBytes + mk::kMiscBytes;
  info->barriers_per_step = h->barriers;
  info->attn_splits = h->n_splits;
  info->launches_per_step = h->n_groups > 1 ? 1 : h->cfg.rows / launch_rows(h->cfg);
  info->workspace_bytes =
      (int64_t)(h->act_bytes + SyncLayout::kWords * 4 + sizeof(DevLayer) * h->cfg.n_layers);
  return MK_OK;
}

}  // extern "C"

namespace {

// A step needs every CU at once: one workgroup per CU, each holding the CU's
// whole LDS, and grid barriers that wait for all of them.  Two steps running
// at the same time on different streams would each hold part of the CUs and
// wait at their first barrier for workgroups that cannot be placed, until
// the watchdog ends both.  So the steps of all handles on one device are
// ordered: an event is recorded after every step, and a step enqueued on
// another stream than the device's previous step first waits for it.  Steps
// on one stream need no wait.  A stream that is capturing a graph takes no
// part (graph replays on different streams must not overlap).
struct StepOrder {
  std::mutex mu;
  hipEvent_t ev = nullptr;  // created on first use, kept until the process ends
  hipStream_t last = nullptr;
  bool any = false;
};
constexpr int kOrderDevices = 64;
StepOrder g_order[kOrderDevices];

int launch_status(int e) {
  if (e == -2) return fail(MK_ERR_UNSUPPORTED, "launch geometry out of range");
  if (e == -3) return fail(MK_ERR_HIP, "the kernel declares static LDS, which leaves no room for its ring");
  if (e == -1) return fail(MK_ERR_HIP, "querying the device or setting the kernel's dynamic LDS limit failed");
  if (e != 0) return fail(MK_ERR_HIP, "launch failed: %s", hipGetErrorString((hipError_t)e));
  return MK_OK;
}

// One step: per group of up to kMaxRows rows, either one launch of the
// persistent kernel or (phased) one launch per phase of every layer.
// act, sync: the step's workspace (the handle's, or the no-allocation array)
int run_step(mk_handle* h, const float* hidden_in, const int32_t* positions, const mk_kv_cache* kv,
             float* hidden_out, void* stream, bool phased, char* act, unsigned* sync) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "handle is NULL");
  if (!hidden_in || !hidden_out || !positions) return fail(MK_ERR_INVALID_ARG, "NULL device pointer");
  const mk_config& c = h->cfg;
  const size_t hb = (size_t)c.rows * c.d_model * 4;
  const char* a0 = reinterpret_cast<const char*>(hidden_in);
  const char* b0 = reinterpret_cast<const char*>(hidden_out);
  if (a0 < b0 + hb && b0 < a0 + hb) return fail(MK_ERR_INVALID_ARG, "hidden_out overlaps hidden_in");
  const int n_seq = c.rows / c.rows_per_seq;
  if (c.has_attn) {
    if (!kv || !kv->k || !kv->v) return fail(MK_ERR_INVALID_ARG, "kv cache required for attention stacks");
    if (kv->n_seq < n_seq) return fail(MK_ERR_INVALID_ARG, "kv->n_seq (%d) < sequences per step (%d)", kv->n_seq, n_seq);
    if (kv->capacity != c.kv_capacity)
      return fail(MK_ERR_INVALID_ARG, "kv->capacity (%d) != cfg.kv_capacity (%d)", kv->capacity, c.kv_capacity);
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device)
    return fail(MK_ERR_INVALID_ARG, "current device differs from the handle's device");
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(hs, &cap) != hipSuccess) return fail(MK_ERR_HIP, "querying the stream's capture state failed");
  StepOrder* so = (cap == hipStreamCaptureStatusNone && dev < kOrderDevices) ? &g_order[dev] : nullptr;
  std::unique_lock<std::mutex> order_lock;
  if (so) {
    order_lock = std::unique_lock<std::mutex>(so->mu);
    if (!so->ev && hipEventCreateWithFlags(&so->ev, hipEventDisableTiming) != hipSuccess)
      return fail(MK_ERR_HIP, "creating the step-order event failed");
    if (so->any && so->last != hs && hipStreamWaitEvent(hs, so->ev, 0) != hipSuccess)
      return fail(MK_ERR_HIP, "ordering the step after the previous step on another stream failed");
  }
  const int Mg = launch_rows(c);
  // the persistent kernel runs all row groups in one launch when the handle
  // allows it; the phase launches take one row group at a time
  const bool grouped = !phased && h->n_groups > 1;
  const int n_launch = grouped ? 1 : c.rows / Mg;
  int rc = MK_OK;
  for (int gi = 0; gi < n_launch && rc == MK_OK; ++gi) {
    KParams p{};
    p.L = c.n_layers; p.d = c.d_model; p.E = c.n_experts; p.k = c.top_k; p.S = c.n_shared; p.F = c.d_ff;
    p.attn = c.has_attn ? 1 : 0;
    p.H = c.has_attn ? c.n_heads : 0; p.G = c.has_attn ? c.n_kv_heads : 1; p.hd = c.has_attn ? c.head_dim : 0;
    p.M = Mg; p.rps = c.rows_per_seq; p.n_seq = Mg / c.rows_per_seq;
    p.cap = c.has_attn ? kv->capacity : 0;
    p.kv_seqs = c.has_attn ? kv->n_seq : 0;
    p.row0 = gi * Mg; p.seq0 = gi * (Mg / c.rows_per_seq); p.Mt = c.rows;
    p.has_bias = c.has_router_bias ? 1 : 0;
    p.wide = c.dtype == MK_F32 ? 1 : 0;
    p.eps = c.rms_eps; p.theta = c.rope_theta;
    p.n_splits = h->n_splits;
    p.q_per_task = h->q_task;
    p.q_groups = h->q_groups;
    p.n_cu = h->n_cu;
    p.n_groups = grouped ? h->n_groups : 1;
    p.vncu = grouped ? h->vncu : h->n_cu;
    p.cpx_log2 = grouped ? h->cpx_log2 : 0;
    p.act_gstride = grouped ? h->al.stride * c.n_layers : 0;
    p.ring_tiles = h->ring_tiles;
    p.x_bytes = h->x_bytes;
    // barriers of this launch (the row groups' routing exchange only when grouped)
    p.barriers = grouped || h->n_groups == 1 ? h->barriers
                                             : c.n_layers * ((c.has_attn ? 6 : 3) + (Mg > 1 ? 1 : 0)) - 1;
    p.timeout_ticks = h->watchdog_ticks;
    p.layers = h->d_layers;
    p.hidden_in = hidden_in + (size_t)p.row0 * c.d_model;
    p.hidden_out = hidden_out + (size_t)p.row0 * c.d_model;
    p.positions = positions + p.row0;
    p.kcache = c.has_attn ? static_cast<uint16_t*>(kv->k) : nullptr;
    p.vcache = c.has_attn ? static_cast<uint16_t*>(kv->v) : nullptr;
    p.act = act;
    p.al = h->al;
    p.sync = sync;
    p.t_ids = h->t_ids; p.t_w = h->t_w; p.t_logits = h->t_logits;
    if (!phased) {
      p.stamps = reinterpret_cast<long long*>(h->stamps);
      p.only_l = 0;
      p.only_ph = -1;
      rc = launch_status(mk_launch_kernel(&p, stream));
      continue;
    }
    p.stamps = nullptr;
    const int ph0 = c.has_attn ? mk::PH_QKV : mk::PH_RS;
    const int ph1 = Mg > 1 ? mk::PH_DOWNB : mk::PH_DOWN;
    for (int l = 0; l < c.n_layers && rc == MK_OK; ++l) {
      for (int ph = ph0; ph <= ph1 && rc == MK_OK; ++ph) {
        p.only_l = l;
        p.only_ph = ph;
        rc = launch_status(mk_launch_kernel(&p, stream));
      }
    }
  }
  // recorded after a failed launch too: launches before it may be running
  if (so) {
    if (hipEventRecord(so->ev, hs) != hipSuccess)
      return rc != MK_OK ? rc : fail(MK_ERR_HIP, "recording the step-order event failed");
    so->last = hs;
    so->any = true;
  }
  return rc;
}

}  // namespace

extern "C" {

int mk_decode_step(mk_handle* h, const float* hidden_in, const int32_t* positions, const mk_kv_cache* kv,
                   float* hidden_out, void* stream) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "handle is NULL");
  const int rc = run_step(h, hidden_in, positions, kv, hidden_out, stream, false, h->d_act, h->d_sync);
  if (rc == MK_OK) h->last_scratch = false;
  return rc;
}

int mk_decode_step_phased(mk_handle* h, const float* hidden_in, const int32_t* positions, const mk_kv_cache* kv,
                          float* hidden_out, void* stream) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "handle is NULL");
  const int rc = run_step(h, hidden_in, positions, kv, hidden_out, stream, true, h->d_act, h->d_sync);
  if (rc == MK_OK) h->last_scratch = false;
  return rc;
}

int mk_decode_step_noalloc(mk_handle* h, const float* hidden_in, const int32_t* positions, const mk_kv_cache* kv,
                           float* hidden_out, void* stream) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "handle is NULL");
  if (h->act_bytes > kScratchAct)
    return fail(MK_ERR_UNSUPPORTED, "the step needs %zu bytes of workspace; the no-allocation workspace holds %zu",
                h->act_bytes, kScratchAct);
  const int dev = h->device;
  char* base = (dev >= 0 && dev < kScratchDevices) ? g_scratch[dev] : nullptr;  // set once per device by mk_create
  if (!base) return fail(MK_ERR_DEVICE, "no no-allocation workspace on device %d", dev);
  const int rc = run_step(h, hidden_in, positions, kv, hidden_out, stream, false, base + kScratchSync,
                          reinterpret_cast<unsigned*>(base));
  if (rc == MK_OK) h->last_scratch = true;
  return rc;
}

int mk_sync(mk_handle* h, void* stream) {
  if (!h) return fail(MK_ERR_INVALID_ARG, "handle is NULL");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MK_ERR_HIP, "stream synchronize failed: %s", hipGetErrorString(e));
  // the barrier block of the workspace the last step ran in
  char* scr = (h->last_scratch && h->device >= 0 && h->device < kScratchDevices) ? g_scratch[h->device] : nullptr;
  unsigned* sync = scr ? reinterpret_cast<unsigned*>(scr) : h->d_sync;
  unsigned err = 0;
  e = hipMemcpy(&err, sync + SyncLayout::kErr, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MK_ERR_HIP, "reading the device error flag failed: %s", hipGetErrorString(e));
  if (err == 0) return MK_OK;
  // reset barrier state, counters and the tag epoch so the handle can run
  // again; the workspace is cleared with it, so that no word tagged before
  // the reset can carry a tag that the restarted epoch hands out again (the
  // whole no-allocation array: other handles' steps used it too)
  if (scr) {
    if (hipMemset(scr, 0, MK_NOALLOC_SCRATCH_BYTES) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
      return fail(MK_ERR_HIP, "resetting the no-allocation workspace failed");
  } else if (hipMemset(h->d_sync, 0, SyncLayout::kWords * 4) != hipSuccess ||
             hipMemset(h->d_act, 0, h->act_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    return fail(MK_ERR_HIP, "resetting the barrier state failed");
  }
  if (err & mk::kErrTimeout) return fail(MK_ERR_TIMEOUT, "a grid barrier timed out (device flag 0x%x)", err);
  return fail(MK_ERR_INVALID_ARG, "a position was outside the cache or repeated within a sequence (flag 0x%x)", err);
}

}  // extern "C"
