// C ABI of the routed MoE-layer library: context, workspace carving, the
// decode path through the slot cache and the double-buffered prefill
// streamer.  Kernels live in the .hip files; this file only orchestrates
// HIP streams, events, copies and the host thread pool.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <thread>
#include <vector>

#include "moe.h"
#include "common.h"
#include "fwd_ws.h"
#include "host_ffn.h"

extern "C" {
hipError_t moe_launch_router(const uint16_t* x, const float* R, const float* bias, int T, int E, int H, float* z,
                             hipStream_t s);
hipError_t moe_launch_topk(const float* z, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);
hipError_t moe_launch_topk_group(const float* z, int T, int E, int k, int32_t* ids, float* w,
                                 const uint32_t* miss_mask, const int32_t* slot_row, int mb, int32_t* counts,
                                 int32_t* offsets, int32_t* pos, int32_t* perm_tok, WorkList* wl, int* err,
                                 int32_t* pslot, hipStream_t s);
hipError_t moe_launch_group(const int32_t* ids, int T, int k, int E, const uint32_t* miss_mask,
                            const int32_t* slot_row, int mb, int32_t* counts, int32_t* offsets, int32_t* pos,
                            int32_t* perm_tok, int32_t* hist, WorkList* wl, int* err, const TailSplit* tail,
                            hipStream_t s);
hipError_t moe_launch_gemm_dec(int fmt, int gated, int ns, int n_cu, const WorkList* wl, const int32_t* counts,
                               const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0, size_t woff1,
                               size_t soff0, size_t soff1, const void* X, const void* Xs, const int32_t* row_tok,
                               int K, int N, void* out, void* part, size_t part_bytes, int fix, int* err,
                               hipStream_t s);
size_t moe_dec_part_bytes();
int moe_dec_max_ns(int fmt);
int moe_pf_tile_tokens();
int moe_gemv_max_tokens();
hipError_t moe_launch_gemv_down_combine(int fmt, const int32_t* pslot, const float* w, const int32_t* pos,
                                        const uint8_t* pool, size_t S, size_t woff, size_t soff, const void* A, int T,
                                        int k, int K, int N, const float* hp, const int32_t* hp_count, void* out,
                                        float* out_f32, hipStream_t s);
hipError_t moe_launch_gemv_routed(int fmt, int grid, const GemvRoute* rt, const uint8_t* pool, size_t S,
                                  size_t woff0, size_t woff1, size_t soff0, size_t soff1, const void* X, int K, int N,
                                  void* out, hipStream_t s);
hipError_t moe_launch_gemv(int fmt, int max_rows, int gated, int grid, const WorkList* wl, const int32_t* counts,
                           const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0, size_t woff1,
                           size_t soff0, size_t soff1, const void* X, const int32_t* row_tok, int K, int N, void* out,
                           hipStream_t s);
int moe_pf8_tile_tokens(int fmt, int small);
hipError_t moe_launch_gemm_pf8(int fmt, int gated, int small, int n_cu, const WorkList* wl, const int32_t* counts,
                               const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0, size_t woff1,
                               size_t soff0, size_t soff1, const void* X, const void* Xs, int xcap, int K,
                               int N, void* out, int trash_row, hipStream_t s);
hipError_t moe_launch_gemm_pf(int fmt, int gated, int grid, const WorkList* wl, const int32_t* counts,
                              const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0, size_t woff1,
                              size_t soff0, size_t soff1, const void* X, const int32_t* row_tok, int K, int N,
                              void* out, hipStream_t s);
hipError_t moe_launch_combine(const uint16_t* Z, const int32_t* ids, const float* w, const int32_t* pos,
                              const uint32_t* miss_mask, const int32_t* slot_row, const float* hp,
                              const int32_t* hp_count, int T, int k, int H, uint16_t* out, float* out_f32,
                              hipStream_t s);
hipError_t moe_launch_range_mask(int lo, int hi, int E, uint32_t* mask, hipStream_t s);
hipError_t moe_launch_cvt_f16(const void* src, long n, void* dst, hipStream_t s);
hipError_t moe_launch_quant(int fmt, int src_bf16, const void* src, int rows, const int32_t* nrows_dev,
                            const int32_t* row_map, int cols, uint8_t* q, void* scale, int cap,
                            hipStream_t s);
hipError_t moe_launch_plan(const int32_t* ids, int n_assign, int layer, int E, int n_slots, int32_t* slot_table,
                           int32_t* owner, uint32_t* last_use, void* ctl, int policy, double BP, double BH,
                           uint32_t* miss_mask, void* plan, const void* host_stage, hipStream_t s);
hipError_t moe_launch_fill(const void* plan, const uint8_t* host_pool_dev, int layer, int E, size_t S,
                           uint8_t* slot_pool, int grid, hipStream_t s);
hipError_t moe_launch_evict(const int32_t* experts, int n, int layer, int E, int32_t* slot_table, int32_t* owner,
                            uint32_t* last_use, hipStream_t s);
hipError_t moe_launch_install_layer(int layer, int base, int E, void* ctl, int32_t* slot_table, int32_t* owner,
                                    uint32_t* last_use, hipStream_t s);
hipError_t moe_launch_free_slots(const int32_t* slots, int n, int32_t* slot_table, int32_t* owner,
                                 uint32_t* last_use, hipStream_t s);
hipError_t moe_launch_reset(int n_table, int n_slots, int32_t* slot_table, int32_t* owner, uint32_t* last_use,
                            int* err, hipStream_t s);
}

namespace {

thread_local std::string g_err;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte offsets of gate/up/down and of their scale arrays inside one blob.
struct BlobLayout {
  size_t w[3];
  size_t s[3];
  size_t S;
};

BlobLayout blob_layout(const moe_config& c) {
  const size_t n = (size_t)c.H * c.I;
  BlobLayout b{};
  if (c.wfmt == MOE_W_BF16) {
    for (int i = 0; i < 3; ++i) { b.w[i] = i * n * 2; b.s[i] = 0; }
    b.S = 3 * n * 2;
  } else if (c.wfmt == MOE_W_FP8_E4M3_B128) {
    const size_t ns = n / (128 * 128);
    for (int i = 0; i < 3; ++i) { b.w[i] = i * n; b.s[i] = 3 * n + i * ns * 4; }
    b.S = 3 * n + 3 * ns * 4;
  } else if (c.wfmt == MOE_W_NVFP4) {
    // E4M3 block scales per 16 inputs, then the three fp32 tensor scales (16 bytes)
    for (int i = 0; i < 3; ++i) { b.w[i] = i * (n / 2); b.s[i] = 3 * (n / 2) + i * (n / 16); }
    b.S = 3 * (n / 2) + 3 * (n / 16) + 16;
  } else {
    for (int i = 0; i < 3; ++i) { b.w[i] = i * (n / 2); b.s[i] = 3 * (n / 2) + i * (n / 32); }
    b.S = 3 * (n / 2) + 3 * (n / 32);
  }
  return b;
}

// Workspace carving (all offsets 256-byte aligned).
struct WsLayout {
  size_t slot_table, owner, last_use, ctl, err, logits, ids, w, pos, pslot, perm_tok, counts, offsets, hist, wl, wl_tail,
      tail_rows, mask, plan, A,
      Aq, As, Z, Xq, Xs, hp, part, total;
};

// fwd_only: the buffers of a forward alone (no residency table, cache
// state, plan or host partial), with `part_bytes` of partial tiles last.
WsLayout ws_layout(const moe_config& c, bool fwd_only = false, size_t part_bytes = 0) {
  WsLayout L{};
  const size_t Tm = (size_t)std::max(c.max_tokens, 1);
  const size_t R = Tm * c.k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(std::max<size_t>(bytes, 1));
    return at;
  };
  if (!fwd_only) {
    L.slot_table = take((size_t)c.L * c.E * 4);
    // slot metadata sized for the largest pool, so a rebuild can grow it
    L.owner = take((size_t)MOE_MAX_SLOTS * 4);
    L.last_use = take((size_t)MOE_MAX_SLOTS * 4);
    L.ctl = take(sizeof(CacheCtl));
  }
  L.err = take(64);
  L.logits = take(Tm * c.E * 4);
  L.ids = take(R * 4);
  L.w = take(R * 4);
  L.pos = take(R * 4);
  L.pslot = take(R * 4);
  L.perm_tok = take((R + moe_pf_tile_tokens()) * 4);   // + one tile of slack: the prefill GEMM reads whole blocks
  L.counts = take((size_t)c.E * 4);
  L.offsets = take((size_t)(c.E + 1) * 4);
  L.hist = take(((Tm + 255) / 256) * c.E * 4);
  L.wl = take(sizeof(WorkList));
  // large batches: the overflow rows' work list and per-expert row splits
  L.wl_tail = take(sizeof(WorkList));
  L.tail_rows = take((size_t)3 * c.E * 4);
  L.mask = take(64);
  if (!fwd_only) L.plan = take(sizeof(PlanOut));
  const bool q8 = c.wfmt == MOE_W_FP8_E4M3_B128 || c.wfmt == MOE_W_MXFP4;   // quantised activations
  // MXFP4 may take MXFP6 activations: 128-column planes of x6_plane_bytes(R) bytes
  auto qbytes = [&](size_t cols) {
    return c.wfmt == MOE_W_MXFP4 ? std::max(R * cols, cols / 128 * x6_plane_bytes(R)) : (q8 ? R * cols : 0);
  };
  L.A = take((R + 1) * c.I * (q8 ? 4 : 2));   // + a spare row for the 8-bit large-batch GEMM's padding stores
  L.Aq = take(qbytes(c.I));
  L.As = take(c.wfmt == MOE_W_FP8_E4M3_B128 ? R * (c.I / 128) * 4 : (q8 ? R * (c.I / 32) : 0));
  L.Z = take((R + 1) * c.H * 2);
  // quantised activations in grouped order (one row per routed pair)
  L.Xq = take(c.wfmt == MOE_W_NVFP4 ? Tm * c.H * 2 : qbytes(c.H));   // NVFP4: the hidden rows in fp16
  L.Xs = take(c.wfmt == MOE_W_FP8_E4M3_B128 ? R * (c.H / 128) * 4 : (q8 ? R * (c.H / 32) : 0));
  if (!fwd_only) L.hp = take(Tm * c.H * 4);
  // small-batch GEMM: partial tiles of items cut between workgroups
  L.part = take(fwd_only ? part_bytes : moe_dec_part_bytes());
  L.total = o;
  return L;
}

}  // namespace

// Argument of one host-branch callback of the asynchronous decode path.
struct AsyncArg {
  moe_ctx* c;
  int layer, T;
};

struct moe_ctx {
  moe_config cfg;
  BlobLayout bl;
  WsLayout wsl;
  uint8_t* host_pool = nullptr;
  uint8_t* slot_pool = nullptr;
  uint8_t* ws = nullptr;
  int device = 0;
  int n_cu = 256;
  // device buffers (carved)
  int32_t* slot_table;
  int32_t* owner;
  uint32_t* last_use;
  CacheCtl* ctl;
  int* err;
  float* logits;
  int32_t* ids;
  float* w;
  int32_t* pos;
  int32_t* pslot;           // per routed pair: its expert's GPU slot, -1 if not on the GPU (fused grouping)
  int32_t* perm_tok;
  int32_t* counts;
  int32_t* offsets;
  int32_t* hist;
  WorkList* wl;
  WorkList* wl_tail;
  int32_t* tail_rows;       // [3][E]: main rows, overflow rows, first overflow row
  uint32_t* mask;
  PlanOut* plan_dev;
  void* A;
  uint8_t* Aq;
  void* As;
  uint16_t* Z;
  uint8_t* Xq;
  void* Xs;
  float* hp;
  void* part;
  size_t part_bytes = 0;
  // pinned host staging
  PlanOut* plan_host = nullptr;
  uint16_t* hidden_host = nullptr;
  int32_t* ids_host = nullptr;
  float* w_host = nullptr;
  float* hp_host = nullptr;
  int32_t* list_dev_stage = nullptr;   // pinned staging for small int lists sent to the device
  uint8_t* host_pool_dev = nullptr;    // device mapping of the pinned host pool (NULL: not mapped)
  HostStage stage_dev{};                // device mappings of the staging buffers (plan NULL: not mapped)
  float* hp_host_dev = nullptr;
  // policy
  int policy = MOE_POLICY_OFFLOAD;
  double BP = 1.0, BH = 1.0;
  double host_t0_us = 0.0;              // per-call time of the host branch (calibrated)
  int act = MOE_ACT_DEFAULT;              // MXFP4's large-batch activation format
  // asynchronous decode: host-branch callback arguments, one per (layer, T),
  // alive until moe_destroy because captured graphs keep their addresses
  std::map<std::pair<int, int>, std::unique_ptr<AsyncArg>> async_args;
  hipEvent_t async_plan_evt = nullptr, async_host_evt = nullptr;
  int async_err = 0;                    // set by a host-branch callback that failed
  double host_ms = 0.0;                 // time of the host branches (both decode paths), from the pool
  // events
  hipEvent_t plan_evt = nullptr, fill_evt = nullptr, ready[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
  int pf_next = -1;
  HostPool* pool = nullptr;
  std::string err_msg;
  // optional per-stage timing (moe_profile_begin / moe_profile_end)
  bool prof_on = false;
  unsigned prof_mask = 0;               // stages timed (bit per MOE_STAGE_*)
  // the last forward left its down GEMM to the combine (matrix-vector path): its format
  int down_fused = -1;
  bool fills_pending = false;           // fill_evt recorded since the last wait on it
  std::vector<hipEvent_t> prof_ev;      // 2 per record
  std::vector<int> prof_stage;
  size_t prof_used = 0;
};

namespace {

// Device buffers of a context carved out of its workspace w (layout c->wsl;
// the forward-only layout leaves the cache-control buffers null).
void carve(moe_ctx* c, uint8_t* w, bool fwd_only) {
  const WsLayout& L = c->wsl;
  c->ws = w;
  c->slot_table = fwd_only ? nullptr : (int32_t*)(w + L.slot_table);
  c->owner = fwd_only ? nullptr : (int32_t*)(w + L.owner);
  c->last_use = fwd_only ? nullptr : (uint32_t*)(w + L.last_use);
  c->ctl = fwd_only ? nullptr : (CacheCtl*)(w + L.ctl);
  c->err = (int*)(w + L.err);
  c->logits = (float*)(w + L.logits);
  c->ids = (int32_t*)(w + L.ids);
  c->w = (float*)(w + L.w);
  c->pos = (int32_t*)(w + L.pos);
  c->pslot = (int32_t*)(w + L.pslot);
  c->perm_tok = (int32_t*)(w + L.perm_tok);
  c->counts = (int32_t*)(w + L.counts);
  c->offsets = (int32_t*)(w + L.offsets);
  c->hist = (int32_t*)(w + L.hist);
  c->wl = (WorkList*)(w + L.wl);
  c->wl_tail = (WorkList*)(w + L.wl_tail);
  c->tail_rows = (int32_t*)(w + L.tail_rows);
  c->mask = (uint32_t*)(w + L.mask);
  c->plan_dev = fwd_only ? nullptr : (PlanOut*)(w + L.plan);
  c->A = w + L.A;
  c->Aq = w + L.Aq;
  c->As = w + L.As;
  c->Z = (uint16_t*)(w + L.Z);
  c->Xq = w + L.Xq;
  c->Xs = w + L.Xs;
  c->hp = fwd_only ? nullptr : (float*)(w + L.hp);
  c->part = w + L.part;
}

int fail(moe_ctx* c, int code, const std::string& m) {
  if (c) c->err_msg = m;
  g_err = m;
  return code;
}

#define HIPCHK(ctx, expr)                                                                  \
  do {                                                                                     \
    hipError_t _e = (expr);                                                                \
    if (_e != hipSuccess)                                                                  \
      return fail(ctx, MOE_E_HIP, std::string(#expr) + ": " + hipGetErrorString(_e));      \
  } while (0)

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Opens a timed record for one launch of `stage` on stream s (-1 when off).
int prof_open(moe_ctx* c, int stage, hipStream_t s) {
  if (!c->prof_on || !((c->prof_mask >> stage) & 1u) || c->prof_used >= c->prof_stage.size()) return -1;
  const int i = (int)c->prof_used++;
  c->prof_stage[i] = stage;
  if (hipEventRecord(c->prof_ev[2 * i], s) != hipSuccess) return -1;
  return i;
}

void prof_close(moe_ctx* c, int i, hipStream_t s) {
  if (i >= 0) (void)hipEventRecord(c->prof_ev[2 * i + 1], s);
}

// HIP launch `expr` on stream s, timed as `stage` when profiling is on.
#define STAGE(ctx, stage, s, expr)                 \
  do {                                             \
    const int _pi = prof_open(ctx, stage, s);      \
    HIPCHK(ctx, expr);                             \
    prof_close(ctx, _pi, s);                       \
  } while (0)

int check_cfg(const moe_config* c) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null config");
  if (c->L < 1 || c->E < 1 || c->E > 256 || c->k < 1 || c->k > 8 || c->k > c->E)
    return fail(nullptr, MOE_E_INVAL, "need 1 <= k <= 8, k <= E <= 256, L >= 1");
  if (c->H < 256 || c->H % 256 || c->I < 128 || c->I % 128)
    return fail(nullptr, MOE_E_INVAL, "need H % 256 == 0 and I % 128 == 0");
  if (c->wfmt < 0 || c->wfmt > 3) return fail(nullptr, MOE_E_INVAL, "unknown weight format");
  if (c->n_slots < 0 || c->n_slots > MOE_MAX_SLOTS)
    return fail(nullptr, MOE_E_UNSUPPORTED, "n_slots must be in [0, 8192]");
  if (c->max_tokens < 1) return fail(nullptr, MOE_E_INVAL, "max_tokens must be >= 1");
  // the small-batch GEMM numbers its (item, K-chunk) units with 32-bit ints
  const double units = ((double)c->max_tokens * c->k / 16 + 1 + c->E) * (std::max(c->H, c->I) / 64) *
                       (std::max(c->H, c->I) / 128);
  if (units >= 2147483647.0) return fail(nullptr, MOE_E_UNSUPPORTED, "max_tokens * k too large for one call");
  return MOE_OK;
}

int nthreads_of(const moe_config& c) {
  if (c.host_threads > 0) return c.host_threads;
  const unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}

HostFfnShape host_shape(const moe_config& c, size_t S) { return HostFfnShape{c.wfmt, c.E, c.k, c.H, c.I, S}; }

// Idle time before each timed host-branch call of the calibration: about a
// small-batch decode layer's GPU work ahead of its host branch.
constexpr int kHostIdleGapUs = 200;


// Grouping, quantisation and both grouped GEMMs for a routed batch (ids/w in
// the workspace).  slot_row: this layer's device row of the residency table.
// Batches of at most this many tokens run top-k and grouping as one launch
// when nothing sits between them (the resident forward).
constexpr int FUSED_TOPK_T = 16;

int forward_experts(moe_ctx* c, const void* hidden, int T, const int32_t* slot_row, const uint32_t* mask,
                    hipStream_t s, bool fused_topk = false, bool fuse_down = false) {
  const moe_config& g = c->cfg;
  c->down_fused = -1;
  if (c->fills_pending) {                 // weights copied by slot_pool_* / the decode plan
    HIPCHK(c, hipStreamWaitEvent(s, c->fill_evt, 0));
    c->fills_pending = false;
  }
  // many tokens per expert: LDS-tiled MFMA kernels; otherwise weight streaming
  const bool tiled = T > 64 && (long)T * g.k >= 48L * g.E;
  const bool tiled16 = g.wfmt == MOE_W_BF16 || g.wfmt == MOE_W_NVFP4;   // 16-bit tokens in the tiled kernels
  // 8-bit formats with few tokens per expert (at most 160 on average): the
  // 128-token, three-stage variant (a weight stream more than a GEMM)
  const int small8 = (long)T * g.k <= 160L * g.E ? 1 : 0;
  const int tile_mb = tiled16 ? moe_pf_tile_tokens() : moe_pf8_tile_tokens(g.wfmt, small8);
  // weight streaming with 16-bit activations: fp8 and MXFP4 weights are
  // dequantised to bf16 in registers (the small-batch kernels are bound by
  // the weight bytes, so unrounded activations cost nothing)
  const int dfmt = g.wfmt == MOE_W_FP8_E4M3_B128 ? WFMT_FP8_A16 : (g.wfmt == MOE_W_MXFP4 ? WFMT_MXFP4_A16 : g.wfmt);
  // m-blocks of 16 * ns tokens (each m-block reads the expert's weights
  // once; larger blocks cost LDS and idle MFMA rows)
  const int ns = std::min(T <= 16 ? 1 : (T <= 64 ? 2 : 4), moe_dec_max_ns(dfmt));
  // MXFP4 weights with MXFP6 activations when selected (large batches)
  const int qf = g.wfmt == MOE_W_MXFP4 && c->act == MOE_ACT_MXFP6 ? WFMT_MXFP4_A6 : g.wfmt;
  // Large batches: an expert whose last m-tile would hold at most one
  // small-batch m-block of rows keeps one tile fewer and its overflow rows
  // run through the small-batch kernel, so a few such tiles do not add a
  // round of items to the persistent grid (not for MXFP6 rows, which only
  // the tiled kernel reads).
  const bool split = tiled && qf != WFMT_MXFP4_A6;
  const int ns_tail = std::min(4, moe_dec_max_ns(g.wfmt));
  int32_t* mcounts = c->tail_rows;
  int32_t* tcounts = c->tail_rows + g.E;
  int32_t* toffsets = c->tail_rows + 2 * g.E;
  // items per m-tile of GEMM 1: the tiled kernels' 256 weight rows are 128 gate and 128 up rows
  const int ntiles1 = g.I / 128;
  const TailSplit tail{c->wl_tail, mcounts, tcounts, toffsets, 16 * ns_tail, 16 * ns_tail, c->n_cu, ntiles1};
  // one token in the resident forward: the gate/up launch takes the top-k
  // and grouping over (it picks its experts from the logits and writes the
  // routing for the down/combine launch), one launch fewer.  Only where its
  // grid fits one round of workgroups (four per CU): every workgroup repeats
  // the selection before its weight loads, which a second round would wait
  // for (T=1 layer: bf16 decode shape 27.4 -> 26.0 us, NVFP4 26.5 -> 25.0;
  // fp8 49.0 -> 49.8 and MXFP4 67.2 -> 71.8 with their 1536- and
  // 2048-workgroup grids)
  const bool routed = fused_topk && fuse_down && T == 1 && !tiled && g.k <= 8 &&
                      (long)std::min(g.k, g.E) * (g.I / 8) <= 4L * c->n_cu;
  if (fused_topk) {      // the router's logits to top-k and grouping (T <= FUSED_TOPK_T, never tiled)
    if (tiled || T > FUSED_TOPK_T) return fail(c, MOE_E_INVAL, "fused top-k and grouping needs a small batch");
    if (!routed)
      STAGE(c, MOE_STAGE_GROUP, s,
            moe_launch_topk_group(c->logits, T, g.E, g.k, c->ids, c->w, mask, slot_row, 16 * ns, c->counts,
                                  c->offsets, c->pos, c->perm_tok, c->wl, c->err, c->pslot, s));
  } else {
    STAGE(c, MOE_STAGE_GROUP, s,
          moe_launch_group(c->ids, T, g.k, g.E, mask, slot_row, tiled ? tile_mb : 16 * ns, c->counts,
                           c->offsets, c->pos, c->perm_tok, c->hist, c->wl, c->err, split ? &tail : nullptr, s));
  }
  const int ncu = c->n_cu;
  const BlobLayout& b = c->bl;
  const int32_t* tile_counts = split ? mcounts : c->counts;
  // the overflow rows of GEMM 1 (gated) or GEMM 2 through the small-batch
  // kernel, one workgroup per item (an overflow is at most one m-block, so
  // there are at most E times the weight tiles items), after the tiled
  // launch on the same stream (running them beside the tiled kernels on a
  // second stream was slower: they take CUs from the persistent grid's next
  // launch)
  // the grouping splits at most n_cu / (4 * ntiles1) experts, each with at
  // most one m-block of overflow rows, so that many experts times the 64-row
  // weight tiles bound the overflow items
  const int max_split = std::max(1, std::min(g.E, c->n_cu / (4 * ntiles1)));
  auto tail_gemm = [&](int gated, const void* X, const void* Xs, const int32_t* row_tok, void* out) -> int {
    if (!split) return MOE_OK;
    const int N = gated ? g.I : g.H;
    STAGE(c, MOE_STAGE_TAIL, s,
          moe_launch_gemm_dec(g.wfmt, gated, ns_tail, ncu, c->wl_tail, tcounts, toffsets, c->slot_pool, b.S,
                              gated ? b.w[0] : b.w[2], gated ? b.w[1] : 0, gated ? b.s[0] : b.s[2],
                              gated ? b.s[1] : 0, X, Xs, row_tok, gated ? g.H : g.I, N, out, nullptr,
                              0, -(max_split * (N / 64)), c->err, s));
    return MOE_OK;
  };
  if (tiled && !tiled16) {
    const int trash = g.max_tokens * g.k;       // the spare row of A and Z
    // activations quantised straight into grouped order (row p <- token perm_tok[p])
    STAGE(c, MOE_STAGE_QUANT_X, s,
          moe_launch_quant(qf, 1, hidden, T * g.k, c->offsets + g.E, c->perm_tok, g.H, c->Xq, c->Xs, trash, s));
    STAGE(c, MOE_STAGE_GEMM1, s,
          moe_launch_gemm_pf8(qf, 1, small8, c->n_cu, c->wl, tile_counts, c->offsets, c->slot_pool, b.S, b.w[0],
                              b.w[1], b.s[0], b.s[1], c->Xq, c->Xs, trash, g.H, g.I, c->A, trash, s));
    int rc = tail_gemm(1, c->Xq, c->Xs, nullptr, c->A);
    if (rc) return rc;
    STAGE(c, MOE_STAGE_QUANT_A, s,
          moe_launch_quant(qf, 0, c->A, T * g.k, c->offsets + g.E, nullptr, g.I, c->Aq, c->As, trash, s));
    STAGE(c, MOE_STAGE_GEMM2, s,
          moe_launch_gemm_pf8(qf, 0, small8, c->n_cu, c->wl, tile_counts, c->offsets, c->slot_pool, b.S, b.w[2], 0,
                              b.s[2], 0, c->Aq, c->As, trash, g.I, g.H, c->Z, trash, s));
    if ((rc = tail_gemm(0, c->Aq, c->As, nullptr, c->Z))) return rc;
  } else if (tiled) {
    // bf16 tokens, or for NVFP4 the hidden rows converted to fp16 (A in fp16)
    const void* x16 = hidden;
    if (g.wfmt == MOE_W_NVFP4) {
      STAGE(c, MOE_STAGE_QUANT_X, s, moe_launch_cvt_f16(hidden, (long)T * g.H, c->Xq, s));
      x16 = c->Xq;
    }
    STAGE(c, MOE_STAGE_GEMM1, s,
          moe_launch_gemm_pf(g.wfmt, 1, c->n_cu, c->wl, tile_counts, c->offsets, c->slot_pool, b.S, b.w[0],
                             b.w[1], b.s[0], b.s[1], x16, c->perm_tok, g.H, g.I, c->A, s));
    int rc = tail_gemm(1, x16, nullptr, c->perm_tok, c->A);
    if (rc) return rc;
    STAGE(c, MOE_STAGE_GEMM2, s,
          moe_launch_gemm_pf(g.wfmt, 0, c->n_cu, c->wl, tile_counts, c->offsets, c->slot_pool, b.S, b.w[2], 0,
                             b.s[2], 0, c->A, nullptr, g.I, g.H, c->Z, s));
    if ((rc = tail_gemm(0, c->A, nullptr, nullptr, c->Z))) return rc;
  } else {
    // 16-bit tokens gathered through perm_tok for GEMM 1 (bf16, or the
    // hidden rows converted to fp16 for NVFP4's fp16 MFMA), A in the same
    // type; the quantised formats carry their scale offsets
    const void* x16 = hidden;
    if (g.wfmt == MOE_W_NVFP4) {
      STAGE(c, MOE_STAGE_QUANT_X, s, moe_launch_cvt_f16(hidden, (long)T * g.H, c->Xq, s));
      x16 = c->Xq;
    }
    if (T <= moe_gemv_max_tokens()) {
      // at most 8 tokens per expert: matrix-vector products, one weight
      // load per weight, no partial tiles; grids sized by the bound on the
      // active experts (min(T*k, E))
      const long ne = std::min<long>((long)T * g.k, g.E);
      if (routed) {
        const GemvRoute rt{c->logits, g.E,       g.k,       16 * ns,     mask,  slot_row, c->ids, c->w,
                           c->counts, c->offsets, c->pos,  c->perm_tok, c->wl, c->err,   c->pslot};
        STAGE(c, MOE_STAGE_GEMM1, s,
              moe_launch_gemv_routed(dfmt, (int)(ne * (g.I / 8)), &rt, c->slot_pool, b.S, b.w[0], b.w[1], b.s[0],
                                     b.s[1], x16, g.H, g.I, c->A, s));
        c->down_fused = dfmt;
        return MOE_OK;
      }
      STAGE(c, MOE_STAGE_GEMM1, s,
            moe_launch_gemv(dfmt, T, 1, (int)(ne * (g.I / 8)), c->wl, c->counts, c->offsets, c->slot_pool, b.S, b.w[0],
                            b.w[1], b.s[0], b.s[1], x16, c->perm_tok, g.H, g.I, c->A, s));
      // the combine runs the down GEMM (one launch fewer); it reads the
      // per-pair slots the fused top-k/grouping writes
      if (fuse_down && fused_topk && T <= 8 && g.k <= 8) {
        c->down_fused = dfmt;
        return MOE_OK;
      }
      STAGE(c, MOE_STAGE_GEMM2, s,
            moe_launch_gemv(dfmt, T, 0, (int)(ne * (g.H / 16)), c->wl, c->counts, c->offsets, c->slot_pool, b.S, b.w[2],
                            0, b.s[2], 0, c->A, nullptr, g.I, g.H, c->Z, s));
      return MOE_OK;
    }
    // Equal ranges of the weight stream balance the bytes over every CU but
    // cut items, whose partial tiles a second launch adds (6-8 us with its
    // gap).  When every item (expert m-block x 64 weight rows) can have a
    // workgroup of its own in one round (the m-blocks are at most T*k, and
    // at most E plus T*k over the block size), one workgroup per item saves
    // that launch, at the price of one workgroup streaming a whole item.
    // That pays while an item takes at most ~30 us: measured one-workgroup
    // rates per item, with the layer wall times at T=1 (split -> whole):
    // bf16 512 KiB gate/up items ~32 GB/s (decode shape 51 -> 44 us), fp8
    // ~18 GB/s (fp8 shape 67 -> 66 us), NVFP4 ~7.5 GB/s on 128 KiB items
    // (52 -> 43 us), MXFP4 ~8 GB/s on 384 KiB items (78 -> 91 us: 47 us for
    // the gate/up GEMM).
    const long mb_bound = std::min<long>((long)T * g.k, (long)g.E + (long)T * g.k / (16 * ns));
    const long it1 = mb_bound * (g.I / 64), it2 = mb_bound * (g.H / 64);
    const double vb = g.wfmt == MOE_W_BF16 ? 2.0 : (g.wfmt == MOE_W_FP8_E4M3_B128 ? 1.0 : 0.5);   // bytes per weight
    const double wg_GBps = g.wfmt == MOE_W_BF16 ? 32.0 : (g.wfmt == MOE_W_FP8_E4M3_B128 ? 18.0 : (g.wfmt == MOE_W_NVFP4 ? 7.5 : 8.0));
    const double item1_us = 2.0 * 64 * g.H * vb / (wg_GBps * 1e3), item2_us = 64.0 * g.I * vb / (wg_GBps * 1e3);
    const int nc1 = item1_us <= 30.0 && it1 <= ncu ? (int)it1 : 0;
    const int nc2 = item2_us <= 30.0 && it2 <= ncu ? (int)it2 : 0;
    STAGE(c, MOE_STAGE_GEMM1, s,
          moe_launch_gemm_dec(dfmt, 1, ns, ncu, c->wl, c->counts, c->offsets, c->slot_pool, b.S, b.w[0], b.w[1],
                              b.s[0], b.s[1], x16, nullptr, c->perm_tok, g.H, g.I, c->A, c->part, c->part_bytes, -nc1,
                              c->err, s));
    if (!nc1)
      STAGE(c, MOE_STAGE_FIXUP, s,
          moe_launch_gemm_dec(dfmt, 1, ns, ncu, c->wl, c->counts, c->offsets, c->slot_pool, b.S, b.w[0], b.w[1],
                              b.s[0], b.s[1], x16, nullptr, c->perm_tok, g.H, g.I, c->A, c->part, c->part_bytes, 1,
                              c->err, s));
    STAGE(c, MOE_STAGE_GEMM2, s,
          moe_launch_gemm_dec(dfmt, 0, ns, ncu, c->wl, c->counts, c->offsets, c->slot_pool, b.S, b.w[2], 0, b.s[2],
                              0, c->A, nullptr, nullptr, g.I, g.H, c->Z, c->part, c->part_bytes, -nc2, c->err, s));
    if (!nc2)
      STAGE(c, MOE_STAGE_FIXUP, s,
          moe_launch_gemm_dec(dfmt, 0, ns, ncu, c->wl, c->counts, c->offsets, c->slot_pool, b.S, b.w[2], 0, b.s[2],
                              0, c->A, nullptr, nullptr, g.I, g.H, c->Z, c->part, c->part_bytes, 1, c->err, s));
  }
  return MOE_OK;
}

// Router logits, then top-k unless the caller fuses it with the grouping.
int route_only(moe_ctx* c, const void* hidden, const float* R, const float* bias, int T, hipStream_t s,
               bool with_topk = true) {
  const moe_config& g = c->cfg;
  STAGE(c, MOE_STAGE_ROUTE, s, moe_launch_router((const uint16_t*)hidden, R, bias, T, g.E, g.H, c->logits, s));
  if (with_topk) STAGE(c, MOE_STAGE_TOPK, s, moe_launch_topk(c->logits, T, g.E, g.k, c->ids, c->w, s));
  return MOE_OK;
}

int combine(moe_ctx* c, const uint32_t* mask, const int32_t* row, const float* hp, int T, void* out, hipStream_t s,
            const int32_t* hp_count = nullptr, float* out_f32 = nullptr) {
  if (c->down_fused >= 0) {
    const int f = c->down_fused;
    c->down_fused = -1;
    const BlobLayout& b = c->bl;
    STAGE(c, MOE_STAGE_COMBINE, s,
          moe_launch_gemv_down_combine(f, c->pslot, c->w, c->pos, c->slot_pool, b.S, b.w[2], b.s[2], c->A, T,
                                       c->cfg.k, c->cfg.I, c->cfg.H, hp, hp_count, out, out_f32, s));
    return MOE_OK;
  }
  STAGE(c, MOE_STAGE_COMBINE, s,
        moe_launch_combine(c->Z, c->ids, c->w, c->pos, mask, row, hp, hp_count, T, c->cfg.k, c->cfg.H,
                           (uint16_t*)out, out_f32, s));
  return MOE_OK;
}

int check_T(moe_ctx* c, int T) {
  if (T < 0 || T > c->cfg.max_tokens) return fail(c, MOE_E_INVAL, "T outside [0, max_tokens]");
  return MOE_OK;
}

int plan_sync(moe_ctx* c, int layer, const int32_t* ids_dev, int T, uint32_t* mask_dev, int policy, hipStream_t s) {
  const moe_config& g = c->cfg;
  STAGE(c, MOE_STAGE_PLAN, s,
        moe_launch_plan(ids_dev, T * g.k, layer, g.E, g.n_slots, c->slot_table, c->owner, c->last_use, c->ctl, policy,
                        c->BP, c->BH, mask_dev, c->plan_dev, nullptr, s));
  HIPCHK(c, hipMemcpyAsync(c->plan_host, c->plan_dev, sizeof(PlanOut), hipMemcpyDeviceToHost, s));
  return MOE_OK;
}

void fill_info(moe_ctx* c, moe_plan_info* info) {
  if (!info) return;
  const PlanOut& p = *c->plan_host;
  info->n_unique = p.n_unique;
  info->n_hit = p.n_hit;
  info->m = p.m;
  info->q = p.q;
  info->n_host = p.n_host;
  info->n_evict = p.n_evict;
  const double S = (double)c->bl.S;
  info->t_fill_pred_us = p.q * S / (c->BP * 1e9) * 1e6;
  const double BR = c->BH - c->BP;
  info->t_host_pred_us =
      p.n_host == 0 ? 0.0 : (BR > 0 ? c->host_t0_us + p.n_host * S / (BR * 1e9) * 1e6 : INFINITY);
}

int issue_fills(moe_ctx* c, int layer, const int* experts, const int* slots, int n, hipStream_t copy) {
  const size_t S = c->bl.S;
  for (int i = 0; i < n; ++i) {
    const size_t g = (size_t)layer * c->cfg.E + experts[i];
    HIPCHK(c, hipMemcpyAsync(c->slot_pool + (size_t)slots[i] * S, c->host_pool + g * S, S, hipMemcpyHostToDevice,
                             copy));
  }
  HIPCHK(c, hipEventRecord(c->fill_evt, copy));
  c->fills_pending = true;
  return MOE_OK;
}

// Host branch of the asynchronous decode path, run by the HIP runtime when
// the host stream reaches it: the plan and the routed inputs have just been
// copied into the pinned staging buffers; the host set C runs on the thread
// pool into hp_host.  Calls no HIP function.
void host_branch_cb(void* p) {
  const AsyncArg* a = (const AsyncArg*)p;
  moe_ctx* c = a->c;
  const PlanOut& pl = *c->plan_host;
  if (pl.n_host <= 0) return;
  if (pl.n_host > c->cfg.E) {
    c->async_err = 1;
    return;
  }
  HostFfnHandle* h = host_ffn_start(c->pool, host_shape(c->cfg, c->bl.S), c->host_pool, a->layer, a->T,
                                    c->hidden_host, c->ids_host, c->w_host, pl.C, pl.n_host, c->hp_host);
  c->host_ms += host_ffn_wait(c->pool, h);
}

}  // namespace

extern "C" {

size_t moe_expert_bytes(const moe_config* cfg) {
  if (!cfg) return 0;
  return blob_layout(*cfg).S;
}

size_t moe_workspace_bytes(const moe_config* cfg) {
  if (check_cfg(cfg) != MOE_OK) return 0;
  return ws_layout(*cfg).total;
}

const char* moe_last_error(moe_ctx* ctx) { return ctx ? ctx->err_msg.c_str() : g_err.c_str(); }

int moe_host_alloc(size_t bytes, void** out) {
  if (!out) return fail(nullptr, MOE_E_INVAL, "null out");
  *out = nullptr;
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
  if (e != hipSuccess) return fail(nullptr, MOE_E_PIN, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  *out = p;
  return MOE_OK;
}

int moe_host_free(void* p) {
  if (!p) return MOE_OK;
  hipError_t e = hipHostFree(p);
  if (e != hipSuccess) return fail(nullptr, MOE_E_HIP, std::string("hipHostFree: ") + hipGetErrorString(e));
  return MOE_OK;
}

int moe_create(const moe_config* cfg, void* host_pool, size_t host_bytes, void* d_slot_pool, size_t slot_bytes,
               void* d_workspace, size_t ws_bytes, moe_ctx** out) {
  if (!out) return fail(nullptr, MOE_E_INVAL, "null out");
  *out = nullptr;
  int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  moe_ctx* c = new moe_ctx();
  c->cfg = *cfg;
  c->bl = blob_layout(*cfg);
  c->wsl = ws_layout(*cfg);
  const size_t S = c->bl.S;
  auto bad = [&](int code, const std::string& m) {
    delete c;
    return fail(nullptr, code, m);
  };
  if (!host_pool || host_bytes < (size_t)cfg->L * cfg->E * S) return bad(MOE_E_INVAL, "host pool smaller than L*E*S");
  if ((cfg->n_slots > 0 && !d_slot_pool) || slot_bytes < (size_t)cfg->n_slots * S)
    return bad(MOE_E_INVAL, "slot pool smaller than n_slots*S");
  if (!d_workspace || ws_bytes < c->wsl.total) return bad(MOE_E_INVAL, "workspace smaller than moe_workspace_bytes");
  c->host_pool = (uint8_t*)host_pool;
  c->slot_pool = (uint8_t*)d_slot_pool;
  if (hipGetDevice(&c->device) != hipSuccess) return bad(MOE_E_HIP, "hipGetDevice failed");
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, c->device) == hipSuccess && ncu > 0)
    c->n_cu = ncu;
  carve(c, (uint8_t*)d_workspace, false);
  c->part_bytes = moe_dec_part_bytes();
  const size_t Tm = cfg->max_tokens;
  const size_t R = Tm * cfg->k;
  void* p;
  // staging shared with kernels of the asynchronous path: coherent, so the
  // device's stores and loads through the mappings bypass its caches
  const unsigned coh = hipHostMallocCoherent;
  if (hipHostMalloc(&p, sizeof(PlanOut), coh) != hipSuccess) return bad(MOE_E_PIN, "staging");
  c->plan_host = (PlanOut*)p;
  if (hipHostMalloc(&p, Tm * cfg->H * 2, coh) != hipSuccess) return bad(MOE_E_PIN, "staging");
  c->hidden_host = (uint16_t*)p;
  if (hipHostMalloc(&p, R * 4, coh) != hipSuccess) return bad(MOE_E_PIN, "staging");
  c->ids_host = (int32_t*)p;
  if (hipHostMalloc(&p, R * 4, coh) != hipSuccess) return bad(MOE_E_PIN, "staging");
  c->w_host = (float*)p;
  if (hipHostMalloc(&p, Tm * cfg->H * 4, coh) != hipSuccess) return bad(MOE_E_PIN, "staging");
  c->hp_host = (float*)p;
  if (hipHostMalloc(&p, 2 * 8192 * 4, hipHostMallocDefault) != hipSuccess) return bad(MOE_E_PIN, "staging");
  c->list_dev_stage = (int32_t*)p;
  if (hipEventCreateWithFlags(&c->plan_evt, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->fill_evt, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->async_plan_evt, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->async_host_evt, hipEventDisableTiming) != hipSuccess)
    return bad(MOE_E_HIP, "event create");
  // the indexed fill kernel reads the host pool through its device mapping
  // (pinned memory from hipHostMalloc has one; other memory leaves the
  // asynchronous decode path unavailable)
  void* hdev = nullptr;
  if (hipHostGetDevicePointer(&hdev, host_pool, 0) == hipSuccess) c->host_pool_dev = (uint8_t*)hdev;
  (void)hipGetLastError();
  {
    void *a = nullptr, *b = nullptr, *d = nullptr, *e = nullptr, *f = nullptr;
    if (hipHostGetDevicePointer(&a, c->plan_host, 0) == hipSuccess &&
        hipHostGetDevicePointer(&b, c->ids_host, 0) == hipSuccess &&
        hipHostGetDevicePointer(&d, c->w_host, 0) == hipSuccess &&
        hipHostGetDevicePointer(&e, c->hidden_host, 0) == hipSuccess &&
        hipHostGetDevicePointer(&f, c->hp_host, 0) == hipSuccess) {
      c->stage_dev.plan = (PlanOut*)a;
      c->stage_dev.ids = (int32_t*)b;
      c->stage_dev.w = (float*)d;
      c->stage_dev.hidden = (uint16_t*)e;
      c->hp_host_dev = (float*)f;
    } else {
      c->host_pool_dev = nullptr;      // the asynchronous path needs every mapping
    }
    (void)hipGetLastError();
  }
  if (hipMemset(c->ctl, 0, sizeof(CacheCtl)) != hipSuccess) return bad(MOE_E_HIP, "control block clear");
  for (int i = 0; i < 2; ++i)
    if (hipEventCreateWithFlags(&c->ready[i], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->done[i], hipEventDisableTiming) != hipSuccess)
      return bad(MOE_E_HIP, "event create");
  if (moe_launch_reset(cfg->L * cfg->E, cfg->n_slots, c->slot_table, c->owner, c->last_use, c->err, nullptr) !=
      hipSuccess)
    return bad(MOE_E_HIP, "reset kernel launch");
  if (hipEventRecord(c->fill_evt, nullptr) != hipSuccess) return bad(MOE_E_HIP, "event record");
  for (int i = 0; i < 2; ++i)
    if (hipEventRecord(c->done[i], nullptr) != hipSuccess || hipEventRecord(c->ready[i], nullptr) != hipSuccess)
      return bad(MOE_E_HIP, "event record");
  if (hipDeviceSynchronize() != hipSuccess) return bad(MOE_E_HIP, "init sync");
  c->pool = host_pool_create(nthreads_of(*cfg));
  *out = c;
  return MOE_OK;
}

int moe_destroy(moe_ctx* c) {
  if (!c) return MOE_OK;
  (void)hipDeviceSynchronize();
  if (c->pool) host_pool_destroy(c->pool);
  if (c->plan_host) (void)hipHostFree(c->plan_host);
  if (c->hidden_host) (void)hipHostFree(c->hidden_host);
  if (c->ids_host) (void)hipHostFree(c->ids_host);
  if (c->w_host) (void)hipHostFree(c->w_host);
  if (c->hp_host) (void)hipHostFree(c->hp_host);
  if (c->list_dev_stage) (void)hipHostFree(c->list_dev_stage);
  for (hipEvent_t e : {c->plan_evt, c->fill_evt, c->ready[0], c->ready[1], c->done[0], c->done[1],
                       c->async_plan_evt, c->async_host_evt})
    if (e) (void)hipEventDestroy(e);
  delete c;
  return MOE_OK;
}

int moe_set_activations(moe_ctx* c, int act) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  if (act != MOE_ACT_DEFAULT && act != MOE_ACT_MXFP6) return fail(c, MOE_E_INVAL, "unknown activation format");
  if (act == MOE_ACT_MXFP6 && c->cfg.wfmt != MOE_W_MXFP4)
    return fail(c, MOE_E_INVAL, "MXFP6 activations need MXFP4 weights");
  c->act = act;
  return MOE_OK;
}

int moe_set_policy(moe_ctx* c, int policy, double B_P, double B_H) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  if (policy < 0 || policy > 2) return fail(c, MOE_E_INVAL, "unknown policy");
  if (!(B_P > 0) || !(B_H > 0)) return fail(c, MOE_E_INVAL, "bandwidths must be positive");
  c->policy = policy;
  c->BP = B_P;
  c->BH = B_H;
  return MOE_OK;
}

int32_t* moe_slot_table(moe_ctx* c) { return c ? c->slot_table : nullptr; }

int moe_reset_cache(moe_ctx* c, void* stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  HIPCHK(c, moe_launch_reset(c->cfg.L * c->cfg.E, c->cfg.n_slots, c->slot_table, c->owner, c->last_use, c->err,
                             as_stream(stream)));
  c->pf_next = -1;
  return MOE_OK;
}

int moe_route(moe_ctx* c, const void* hidden, const float* R, const float* bias, int T, int32_t* topk_ids,
              float* topk_w, void* stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  int rc = check_T(c, T);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  HIPCHK(c, moe_launch_router((const uint16_t*)hidden, R, bias, T, c->cfg.E, c->cfg.H, c->logits, s));
  HIPCHK(c, moe_launch_topk(c->logits, T, c->cfg.E, c->cfg.k, topk_ids, topk_w, s));
  return MOE_OK;
}

int moe_quantize(int wfmt, int src_bf16, const void* src, int rows, int cols, const int32_t* row_map, uint8_t* q,
                 void* scale, void* stream) {
  if (wfmt != MOE_W_FP8_E4M3_B128 && wfmt != MOE_W_MXFP4 && wfmt != MOE_QUANT_MXFP6)
    return fail(nullptr, MOE_E_INVAL, "format has no quantisation");
  if (rows < 0 || cols <= 0 || cols % (wfmt == MOE_W_MXFP4 ? 32 : 128)) return fail(nullptr, MOE_E_INVAL, "bad shape");
  if (rows == 0) return MOE_OK;
  if (!src || !q || !scale) return fail(nullptr, MOE_E_INVAL, "null argument");
  const int qf = wfmt == MOE_QUANT_MXFP6 ? WFMT_MXFP4_A6 : wfmt;
  hipError_t e = moe_launch_quant(qf, src_bf16 ? 1 : 0, src, rows, nullptr, row_map, cols, q, scale,
                                  rows, as_stream(stream));
  if (e != hipSuccess) return fail(nullptr, MOE_E_HIP, hipGetErrorString(e));
  return MOE_OK;
}

int moe_route_from_logits(moe_ctx* c, const float* logits, int T, int32_t* topk_ids, float* topk_w, int32_t* counts,
                          int32_t* offsets, int32_t* perm_tok, int32_t* pos, void* stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  int rc = check_T(c, T);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  const moe_config& g = c->cfg;
  HIPCHK(c, moe_launch_topk(logits, T, g.E, g.k, topk_ids, topk_w, s));
  HIPCHK(c, moe_launch_group(topk_ids, T, g.k, g.E, nullptr, nullptr, DEC_MB, counts, offsets, pos, perm_tok,
                             c->hist, c->wl, c->err, nullptr, s));
  return MOE_OK;
}

int moe_plan(moe_ctx* c, int layer, const int32_t* topk_ids, int T, uint32_t* miss_mask_out, moe_plan_info* info,
             int32_t* fill_experts, int32_t* fill_slots, void* stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  if (layer < 0 || layer >= c->cfg.L) return fail(c, MOE_E_INVAL, "layer out of range");
  int rc = check_T(c, T);
  if (rc) return rc;
  hipStream_t s = as_stream(stream);
  rc = plan_sync(c, layer, topk_ids, T, miss_mask_out ? miss_mask_out : c->mask, c->policy, s);
  if (rc) return rc;
  HIPCHK(c, hipEventRecord(c->plan_evt, s));
  HIPCHK(c, hipEventSynchronize(c->plan_evt));
  fill_info(c, info);
  const PlanOut& p = *c->plan_host;
  for (int i = 0; i < p.q; ++i) {
    if (fill_experts) fill_experts[i] = p.F[i];
    if (fill_slots) fill_slots[i] = p.F_slot[i];
  }
  return MOE_OK;
}

int slot_pool_fill(moe_ctx* c, int layer, const int32_t* experts, const int32_t* slots, int n, void* copy_stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  if (layer < 0 || layer >= c->cfg.L || n < 0) return fail(c, MOE_E_INVAL, "bad layer or count");
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= c->cfg.E || slots[i] < 0 || slots[i] >= c->cfg.n_slots)
      return fail(c, MOE_E_INVAL, "expert or slot out of range");
  return issue_fills(c, layer, experts, slots, n, as_stream(copy_stream));
}

int slot_pool_admit(moe_ctx* c, int layer, const int32_t* experts, int n, void* copy_stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  const moe_config& g = c->cfg;
  if (layer < 0 || layer >= g.L || n < 0 || n > 8192) return fail(c, MOE_E_INVAL, "bad layer or count");
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= g.E) return fail(c, MOE_E_INVAL, "expert out of range");
  if (n == 0) return MOE_OK;
  hipStream_t s = as_stream(copy_stream);
  // the plan kernel reads the list as routed ids: stage it into the workspace
  std::memcpy(c->list_dev_stage, experts, (size_t)n * 4);
  HIPCHK(c, hipMemcpyAsync(c->ids, c->list_dev_stage, (size_t)n * 4, hipMemcpyHostToDevice, s));
  HIPCHK(c, moe_launch_plan(c->ids, n, layer, g.E, g.n_slots, c->slot_table, c->owner, c->last_use, c->ctl,
                            MOE_POLICY_OFFLOAD, 1.0, 1.0, c->mask, c->plan_dev, nullptr, s));
  HIPCHK(c, hipMemcpyAsync(c->plan_host, c->plan_dev, sizeof(PlanOut), hipMemcpyDeviceToHost, s));
  HIPCHK(c, hipEventRecord(c->plan_evt, s));
  HIPCHK(c, hipEventSynchronize(c->plan_evt));
  const PlanOut& p = *c->plan_host;
  // the experts the plan installed must be copied even when some did not fit
  const int rc = issue_fills(c, layer, p.F, p.F_slot, p.q, s);
  if (rc) return rc;
  if (p.q < p.m) return fail(c, MOE_E_NOSLOTS, "not enough evictable slots to admit every expert");
  return MOE_OK;
}

int slot_pool_resize(moe_ctx* c, void* d_slot_pool, size_t slot_bytes, int n_slots, void* stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  const moe_config& g = c->cfg;
  const size_t S = c->bl.S;
  if (n_slots < 0 || n_slots > MOE_MAX_SLOTS) return fail(c, MOE_E_INVAL, "n_slots outside [0, 8192]");
  if ((n_slots > 0 && !d_slot_pool) || slot_bytes < (size_t)n_slots * S)
    return fail(c, MOE_E_INVAL, "slot pool smaller than n_slots*S");
  hipStream_t s = as_stream(stream);
  HIPCHK(c, hipDeviceSynchronize());            // safe point: no work of the context in flight
  const int n_old = g.n_slots;
  std::vector<int32_t> owner(std::max(n_old, 1));
  std::vector<uint32_t> last(std::max(n_old, 1));
  if (n_old > 0) {
    HIPCHK(c, hipMemcpy(owner.data(), c->owner, (size_t)n_old * 4, hipMemcpyDeviceToHost));
    HIPCHK(c, hipMemcpy(last.data(), c->last_use, (size_t)n_old * 4, hipMemcpyDeviceToHost));
  }
  // survivors: the n_slots most recently used residents (stamp descending,
  // ties to the lower slot), packed into slots 0, 1, ... in old-slot order
  std::vector<int> keep;
  for (int sl = 0; sl < n_old; ++sl)
    if (owner[sl] >= 0) keep.push_back(sl);
  std::stable_sort(keep.begin(), keep.end(), [&](int a, int b) { return last[a] > last[b]; });
  if ((int)keep.size() > n_slots) keep.resize(n_slots);
  std::sort(keep.begin(), keep.end());
  std::vector<int32_t> table((size_t)g.L * g.E, -1), owner_n(std::max(n_slots, 1), -1);
  std::vector<uint32_t> last_n(std::max(n_slots, 1), 0u);
  uint8_t* dst = (uint8_t*)d_slot_pool;
  for (int nw = 0; nw < (int)keep.size(); ++nw) {
    const int old = keep[nw];
    owner_n[nw] = owner[old];
    last_n[nw] = last[old];
    table[owner[old]] = nw;
    // in place, nw <= old and every source above nw is still unmoved
    if (dst != c->slot_pool || nw != old)
      HIPCHK(c, hipMemcpyAsync(dst + (size_t)nw * S, c->slot_pool + (size_t)old * S, S, hipMemcpyDeviceToDevice, s));
  }
  HIPCHK(c, hipMemcpyAsync(c->slot_table, table.data(), table.size() * 4, hipMemcpyHostToDevice, s));
  if (n_slots > 0) {
    HIPCHK(c, hipMemcpyAsync(c->owner, owner_n.data(), (size_t)n_slots * 4, hipMemcpyHostToDevice, s));
    HIPCHK(c, hipMemcpyAsync(c->last_use, last_n.data(), (size_t)n_slots * 4, hipMemcpyHostToDevice, s));
  }
  HIPCHK(c, hipStreamSynchronize(s));
  c->slot_pool = dst;
  c->cfg.n_slots = n_slots;
  c->pf_next = -1;                              // the prefill streamer restarts its buffers
  c->fills_pending = false;
  return MOE_OK;
}

int slot_pool_evict(moe_ctx* c, int layer, const int32_t* experts, int n) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  const moe_config& g = c->cfg;
  if (layer < 0 || layer >= g.L || n < 0 || n > 8192) return fail(c, MOE_E_INVAL, "bad layer or count");
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= g.E) return fail(c, MOE_E_INVAL, "expert out of range");
  if (n == 0) return MOE_OK;
  std::memcpy(c->list_dev_stage, experts, (size_t)n * 4);
  HIPCHK(c, hipMemcpyAsync(c->ids, c->list_dev_stage, (size_t)n * 4, hipMemcpyHostToDevice, nullptr));
  HIPCHK(c, moe_launch_evict(c->ids, n, layer, g.E, c->slot_table, c->owner, c->last_use, nullptr));
  HIPCHK(c, hipStreamSynchronize(nullptr));
  return MOE_OK;
}

int moe_host_partial(moe_ctx* c, int layer, const void* hidden, const int32_t* topk_ids, const float* topk_w, int T,
                     const uint32_t* miss_mask, float* out) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  const moe_config& g = c->cfg;
  if (layer < 0 || layer >= g.L) return fail(c, MOE_E_INVAL, "layer out of range");
  int rc = check_T(c, T);
  if (rc) return rc;
  std::vector<int32_t> C;
  for (int e = 0; e < g.E; ++e)
    if ((miss_mask[e >> 5] >> (e & 31)) & 1u) C.push_back(e);
  HostFfnHandle* h = host_ffn_start(c->pool, host_shape(g, c->bl.S), c->host_pool, layer, T, (const uint16_t*)hidden,
                                    topk_ids, topk_w, C.data(), (int)C.size(), out);
  host_ffn_wait(c->pool, h);
  return MOE_OK;
}

int moe_host_ffn(const moe_config* cfg, const void* host_pool, int layer, const void* hidden, const int32_t* topk_ids,
                 const float* topk_w, int T, const uint32_t* miss_mask, float* out) {
  if (!cfg || !host_pool || !hidden || !topk_ids || !topk_w || !miss_mask || !out)
    return fail(nullptr, MOE_E_INVAL, "null argument");
  if (cfg->E < 1 || cfg->E > 256 || cfg->k < 1 || cfg->k > cfg->E || cfg->H < 1 || cfg->I < 1 || layer < 0 ||
      layer >= cfg->L || T < 0 || cfg->wfmt < 0 || cfg->wfmt > 3)
    return fail(nullptr, MOE_E_INVAL, "bad shape");
  if ((cfg->wfmt == 1 && (cfg->H % 128 || cfg->I % 128)) || (cfg->wfmt == 2 && (cfg->H % 32 || cfg->I % 32)) ||
      (cfg->wfmt == 3 && (cfg->H % 16 || cfg->I % 16)))
    return fail(nullptr, MOE_E_INVAL, "H and I must be multiples of the scale block");
  std::vector<int32_t> C;
  for (int e = 0; e < cfg->E; ++e)
    if ((miss_mask[e >> 5] >> (e & 31)) & 1u) C.push_back(e);
  HostPool* P = host_pool_create(nthreads_of(*cfg));
  HostFfnHandle* h = host_ffn_start(P, host_shape(*cfg, blob_layout(*cfg).S), (const uint8_t*)host_pool, layer, T,
                                    (const uint16_t*)hidden, topk_ids, topk_w, C.data(), (int)C.size(), out);
  host_ffn_wait(P, h);
  host_pool_destroy(P);
  return MOE_OK;
}

int moe_layer_forward(moe_ctx* c, int layer, const void* hidden, const float* R, const float* bias, int T,
                      const int32_t* slot_row, const uint32_t* miss_mask, const float* host_partial, void* out,
                      void* stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  if (layer < 0 || layer >= c->cfg.L) return fail(c, MOE_E_INVAL, "layer out of range");
  if (!slot_row && c->cfg.n_slots > 0) return fail(c, MOE_E_INVAL, "null slot table");
  int rc = check_T(c, T);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  const bool fz = T <= FUSED_TOPK_T;
  rc = route_only(c, hidden, R, bias, T, s, !fz);
  if (rc) return rc;
  rc = forward_experts(c, hidden, T, slot_row, miss_mask, s, fz, true);
  if (rc) return rc;
  return combine(c, miss_mask, slot_row, host_partial, T, out, s);
}

}  // extern "C"

void moe_set_thread_error(const char* msg) { g_err = msg; }

size_t moe_fwd_ws_bytes(const moe_config* cfg, int max_T, size_t part_bytes) {
  moe_config g = *cfg;
  g.max_tokens = max_T;
  return ws_layout(g, true, part_bytes).total;
}

int moe_fwd_on_ws(const moe_config* cfg, int max_T, uint8_t* ws, size_t part_bytes, int n_cu, const void* slot_pool,
                  const int32_t* slot_row, const void* hidden, const float* R, const float* bias, int T,
                  const uint32_t* miss_mask, const float* hp, void* out, int* err, hipStream_t s, const char** msg) {
  // a context on the stack over the given workspace: its containers stay
  // empty, so nothing is allocated
  moe_ctx c;
  c.cfg = *cfg;
  c.cfg.max_tokens = max_T;
  c.cfg.n_slots = 0;
  c.bl = blob_layout(c.cfg);
  c.wsl = ws_layout(c.cfg, true, part_bytes);
  c.slot_pool = (uint8_t*)slot_pool;
  c.n_cu = n_cu;
  carve(&c, ws, true);
  c.err = err;
  c.part_bytes = part_bytes;
  const bool fz = T <= FUSED_TOPK_T;
  int rc = route_only(&c, hidden, R, bias, T, s, !fz);
  if (!rc) rc = forward_experts(&c, hidden, T, slot_row, miss_mask, s, fz, true);
  if (!rc) rc = combine(&c, miss_mask, slot_row, hp, T, out, s);
  if (rc && msg) *msg = "a kernel launch of the forward failed";
  return rc;
}

extern "C" {

int moe_decode_layer(moe_ctx* c, int layer, const void* hidden, const float* R, const float* bias, int T, void* out,
                     moe_plan_info* info, void* compute_stream, void* copy_stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  const moe_config& g = c->cfg;
  if (layer < 0 || layer >= g.L) return fail(c, MOE_E_INVAL, "layer out of range");
  int rc = check_T(c, T);
  if (rc) return rc;
  if (T == 0) return MOE_OK;
  hipStream_t s = as_stream(compute_stream), cs = as_stream(copy_stream);
  rc = route_only(c, hidden, R, bias, T, s);
  if (rc) return rc;
  rc = plan_sync(c, layer, c->ids, T, c->mask, c->policy, s);
  if (rc) return rc;
  const bool may_host = c->policy != MOE_POLICY_OFFLOAD || g.n_slots < g.E;
  if (may_host) {
    HIPCHK(c, hipMemcpyAsync(c->ids_host, c->ids, (size_t)T * g.k * 4, hipMemcpyDeviceToHost, s));
    HIPCHK(c, hipMemcpyAsync(c->w_host, c->w, (size_t)T * g.k * 4, hipMemcpyDeviceToHost, s));
    HIPCHK(c, hipMemcpyAsync(c->hidden_host, hidden, (size_t)T * g.H * 2, hipMemcpyDeviceToHost, s));
  }
  HIPCHK(c, hipEventRecord(c->plan_evt, s));
  HIPCHK(c, hipEventSynchronize(c->plan_evt));
  const PlanOut& p = *c->plan_host;
  fill_info(c, info);
  // host branch first (section 2.5: the CPU branch is launched before the GPU miss path)
  HostFfnHandle* h = nullptr;
  if (p.n_host > 0) {
    if (!may_host) return fail(c, MOE_E_INVAL, "host work planned without staged inputs");
    h = host_ffn_start(c->pool, host_shape(g, c->bl.S), c->host_pool, layer, T, c->hidden_host, c->ids_host,
                       c->w_host, p.C, p.n_host, c->hp_host);
  }
  if (p.q > 0) {
    rc = issue_fills(c, layer, p.F, p.F_slot, p.q, cs);
    if (rc) {
      if (h) host_ffn_wait(c->pool, h);
      return rc;
    }
  }
  const int32_t* row = c->slot_table + (size_t)layer * g.E;
  rc = forward_experts(c, hidden, T, row, c->mask, s);
  if (h) c->host_ms += host_ffn_wait(c->pool, h);
  if (rc) return rc;
  const float* hp = nullptr;
  if (p.n_host > 0) {
    HIPCHK(c, hipMemcpyAsync(c->hp, c->hp_host, (size_t)T * g.H * 4, hipMemcpyHostToDevice, s));
    hp = c->hp;
  }
  return combine(c, c->mask, row, hp, T, out, s);
}

int moe_decode_layer_async(moe_ctx* c, int layer, const void* hidden, const float* R, const float* bias, int T,
                           void* out, void* compute_stream, void* host_stream) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  const moe_config& g = c->cfg;
  if (layer < 0 || layer >= g.L) return fail(c, MOE_E_INVAL, "layer out of range");
  int rc = check_T(c, T);
  if (rc) return rc;
  if (!c->host_pool_dev) return fail(c, MOE_E_UNSUPPORTED, "host pool has no device mapping (use moe_host_alloc)");
  if (T == 0) return MOE_OK;
  hipStream_t s = as_stream(compute_stream), hs = as_stream(host_stream);
  rc = route_only(c, hidden, R, bias, T, s);
  if (rc) return rc;
  // host branch (section 2.5: started before the GPU miss path): the plan
  // kernel writes the plan and the routed inputs into pinned staging; the
  // host stream waits for it, runs C in a host callback into pinned hp, and
  // the combine reads hp through its device mapping
  const bool may_host = c->policy != MOE_POLICY_OFFLOAD || g.n_slots < g.E;
  HostStage hst{};
  if (may_host) {
    hst = c->stage_dev;
    hst.w_src = c->w;
    hst.hidden_src = (const uint16_t*)hidden;
    hst.n_hidden = T * g.H;
  }
  STAGE(c, MOE_STAGE_PLAN, s,
        moe_launch_plan(c->ids, T * g.k, layer, g.E, g.n_slots, c->slot_table, c->owner, c->last_use, c->ctl,
                        c->policy, c->BP, c->BH, c->mask, c->plan_dev, may_host ? &hst : nullptr, s));
  if (may_host) {
    auto& slot = c->async_args[{layer, T}];
    if (!slot) slot.reset(new AsyncArg{c, layer, T});
    HIPCHK(c, hipEventRecord(c->async_plan_evt, s));
    HIPCHK(c, hipStreamWaitEvent(hs, c->async_plan_evt, 0));
    HIPCHK(c, hipLaunchHostFunc(hs, host_branch_cb, slot.get()));
    HIPCHK(c, hipEventRecord(c->async_host_evt, hs));
  }
  // the fill set in one launch, from the device plan (section 2.6)
  if (g.n_slots > 0)
    STAGE(c, MOE_STAGE_FILL, s,
          moe_launch_fill(c->plan_dev, c->host_pool_dev, layer, g.E, c->bl.S, c->slot_pool, 64, s));
  const int32_t* row = c->slot_table + (size_t)layer * g.E;
  rc = forward_experts(c, hidden, T, row, c->mask, s);
  if (rc) return rc;
  if (!may_host) return combine(c, c->mask, row, nullptr, T, out, s);
  HIPCHK(c, hipStreamWaitEvent(s, c->async_host_evt, 0));
  return combine(c, c->mask, row, c->hp_host_dev, T, out, s, &c->plan_dev->n_host);
}

int moe_plan_stats(moe_ctx* c, moe_plan_totals* out, int reset) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  HIPCHK(c, hipDeviceSynchronize());
  CacheCtl v;
  HIPCHK(c, hipMemcpy(&v, c->ctl, sizeof(CacheCtl), hipMemcpyDeviceToHost));
  if (out) {
    out->calls = (long long)v.calls;
    out->n_unique = (long long)v.n_unique;
    out->n_hit = (long long)v.n_hit;
    out->m = (long long)v.m;
    out->q = (long long)v.q;
    out->n_host = (long long)v.n_host;
    out->n_evict = (long long)v.n_evict;
    out->host_ms = c->host_ms;
  }
  if (reset) {
    v.calls = v.n_unique = v.n_hit = v.m = v.q = v.n_host = v.n_evict = 0;
    c->host_ms = 0.0;
    HIPCHK(c, hipMemcpy(c->ctl, &v, sizeof(CacheCtl), hipMemcpyHostToDevice));
  }
  const int e = c->async_err;
  c->async_err = 0;
  if (e) return fail(c, MOE_E_INVAL, "a host-branch callback received an invalid plan");
  return MOE_OK;
}

int prefill_stream_layer(moe_ctx* c, int layer, const void* hidden, const float* R, const float* bias, int T,
                         void* out, void* compute_stream, void* copy_stream, int double_buffer) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  const moe_config& g = c->cfg;
  if (layer < 0 || layer >= g.L) return fail(c, MOE_E_INVAL, "layer out of range");
  int rc = check_T(c, T);
  if (rc) return rc;
  hipStream_t s = as_stream(compute_stream), cs = as_stream(copy_stream);
  const size_t S = c->bl.S;
  const size_t layer_bytes = (size_t)g.E * S;
  if (g.n_slots < g.E && g.n_slots > 0) {
    // not even one full layer fits: the layer in expert ranges of n_slots,
    // each copied in (LRU admission) and evaluated on the GPU; the ranges'
    // weighted sums accumulate unrounded in hp and the last is rounded once
    if (T == 0) return MOE_I_FALLBACK_ONDEMAND;
    const int n = g.n_slots;
    const int32_t* row = c->slot_table + (size_t)layer * g.E;
    std::vector<int32_t> ex((size_t)n);
    for (int lo = 0; lo < g.E; lo += n) {
      const int hi = std::min(g.E, lo + n);
      // the copies overwrite slots the previous range's kernels read
      HIPCHK(c, hipEventRecord(c->done[0], s));
      HIPCHK(c, hipStreamWaitEvent(cs, c->done[0], 0));
      for (int e = lo; e < hi; ++e) ex[e - lo] = e;
      rc = slot_pool_admit(c, layer, ex.data(), hi - lo, cs);
      if (rc) return rc;
      rc = route_only(c, hidden, R, bias, T, s);      // the admission staged its list in the ids buffer
      if (rc) return rc;
      HIPCHK(c, moe_launch_range_mask(lo, hi, g.E, c->mask, s));
      rc = forward_experts(c, hidden, T, row, c->mask, s);
      if (rc) return rc;
      const bool first = lo == 0, last = hi == g.E;
      rc = combine(c, c->mask, row, first ? nullptr : c->hp, T, out, s, nullptr, last ? nullptr : c->hp);
      if (rc) return rc;
    }
    c->pf_next = -1;
    return MOE_I_FALLBACK_ONDEMAND;
  }
  if (g.n_slots == 0) {
    // no slots: every routed expert on the host
    const int saved = c->policy;
    c->policy = MOE_POLICY_OFFLOAD;
    rc = moe_decode_layer(c, layer, hidden, R, bias, T, out, nullptr, compute_stream, copy_stream);
    c->policy = saved;
    return rc ? rc : MOE_I_FALLBACK_ONDEMAND;
  }
  // one full layer fits but not two: the same full-layer copies through a
  // single buffer (copy, then compute; the next copy waits for the compute)
  const bool single = g.n_slots < 2 * g.E;
  if (single) double_buffer = 0;
  auto base_of = [&](int l) { return double_buffer ? (l & 1) * g.E : 0; };
  auto buf_of = [&](int l) { return double_buffer ? (l & 1) : 0; };
  auto issue_copy = [&](int l) -> int {
    const int b = buf_of(l);
    HIPCHK(c, hipStreamWaitEvent(cs, c->done[b], 0));
    HIPCHK(c, moe_launch_install_layer(l, base_of(l), g.E, c->ctl, c->slot_table, c->owner, c->last_use, cs));
    HIPCHK(c, hipMemcpyAsync(c->slot_pool + (size_t)base_of(l) * S, c->host_pool + (size_t)l * layer_bytes,
                             layer_bytes, hipMemcpyHostToDevice, cs));
    HIPCHK(c, hipEventRecord(c->ready[b], cs));
    return MOE_OK;
  };
  if (c->pf_next != layer) {
    rc = issue_copy(layer);
    if (rc) return rc;
  }
  if (double_buffer && layer + 1 < g.L) {
    rc = issue_copy(layer + 1);
    if (rc) return rc;
  }
  HIPCHK(c, hipStreamWaitEvent(s, c->ready[buf_of(layer)], 0));
  if (T > 0) {
    rc = route_only(c, hidden, R, bias, T, s);
    if (rc) return rc;
    const int32_t* row = c->slot_table + (size_t)layer * g.E;
    rc = forward_experts(c, hidden, T, row, nullptr, s);
    if (rc) return rc;
    rc = combine(c, nullptr, row, nullptr, T, out, s);
    if (rc) return rc;
  }
  HIPCHK(c, hipEventRecord(c->done[buf_of(layer)], s));
  if (!double_buffer && layer + 1 < g.L) {
    rc = issue_copy(layer + 1);
    if (rc) return rc;
  }
  c->pf_next = layer + 1 < g.L ? layer + 1 : -1;
  return single ? MOE_I_SINGLE_BUFFER : MOE_OK;
}

int moe_calibrate_ex(moe_ctx* c, int T, moe_calibration* out) {
  if (!c || !out) return fail(c, MOE_E_INVAL, "null argument");
  const moe_config& g = c->cfg;
  if (T < 1 || T > c->cfg.max_tokens) return fail(c, MOE_E_INVAL, "T outside [1, max_tokens]");
  std::memset(out, 0, sizeof(*out));
  const size_t S = c->bl.S;
  const int n_rows = g.L * g.E;
  // statistics of one series of rates: median, min, max
  auto summarise = [](std::vector<double> v, double& med, double& lo, double& hi) {
    if (v.empty()) return;
    std::sort(v.begin(), v.end());
    const size_t n = v.size();
    med = n % 2 ? v[n / 2] : 0.5 * (v[n / 2 - 1] + v[n / 2]);
    lo = v.front();
    hi = v.back();
  };
  // the host branch on a group of G = min(k, E) distinct experts of one
  // layer, each with all T tokens routed to it: at T = 1 the job the decode
  // path hands the host when all of a token's experts miss; and on a single
  // expert, the smallest job.  The two sizes alternate, so both see the same
  // host conditions.  Groups walk (layer, expert) pairs spread over the
  // pool, so no call finds its bytes in the host caches.
  const int G = std::min(g.k, g.E);
  std::vector<uint16_t> hid((size_t)T * g.H, 0x3f80);
  std::vector<int32_t> ids((size_t)T * g.k, -1);
  std::vector<float> w((size_t)T * g.k, 1.0f);
  std::vector<float> outv((size_t)T * g.H);
  std::vector<int32_t> grp(G);
  int pair = 0;
  auto host_call = [&](int n) -> double {      // weight bytes per second of one call on n experts
    const int i = pair++;
    const int l = (int)(((long)i * 5 + 1) % g.L), e0 = (int)(((long)i * 37 + 3) % g.E);
    for (int j = 0; j < n; ++j) grp[j] = (e0 + j) % g.E;
    std::sort(grp.begin(), grp.begin() + n);
    std::fill(ids.begin(), ids.end(), -1);
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < n; ++j) ids[(size_t)t * g.k + j] = grp[j];
    HostFfnHandle* h = host_ffn_start(c->pool, host_shape(g, S), c->host_pool, l, T, hid.data(), ids.data(),
                                      w.data(), grp.data(), n, outv.data());
    const double ms = host_ffn_wait(c->pool, h);
    return (double)n * S / (ms * 1e-3) / 1e9;
  };
  // The decode path calls the host branch once per layer, after the pool
  // has idled through the layer's routing and planning; each timed call
  // follows an idle gap of that order, so the workers' wake-up from idle is
  // part of what is timed.
  const auto idle_gap = std::chrono::microseconds(kHostIdleGapUs);
  auto gapped_call = [&](int n) {
    std::this_thread::sleep_for(idle_gap);
    return host_call(n);
  };
  // warm-up until the pool's threads run at speed: at least 8 calls and
  // 100 ms (right after a large pool fill the first tens of ms run up to a
  // third slower); then 40 timed calls of each size (single calls vary by
  // tens of percent on a shared host, so the medians need many)
  const int n_host = 40;
  {
    const auto w0 = std::chrono::steady_clock::now();
    for (int i = 0; i < 8 || std::chrono::steady_clock::now() - w0 < std::chrono::milliseconds(100); ++i)
      (void)host_call(G);
  }
  std::vector<double> alone, alone1;
  for (int i = 0; i < n_host; ++i) {
    alone.push_back(gapped_call(G));
    alone1.push_back(gapped_call(1));
  }
  double lo1, hi1;
  summarise(alone, out->host_alone, out->host_alone_min, out->host_alone_max);
  summarise(alone1, out->host_alone_1, lo1, hi1);
  out->n_host_alone = (int)alone.size();

  // B_P: whole-expert copies from distinct host rows into the highest slots
  // (freed first, left empty), rounds of n_cp copies
  const int n_cp = std::min(8, g.n_slots);
  if (n_cp > 0) {
    hipStream_t cs;
    HIPCHK(c, hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
    hipEvent_t t0, t1;
    HIPCHK(c, hipEventCreate(&t0));
    HIPCHK(c, hipEventCreate(&t1));
    for (int i = 0; i < n_cp; ++i) c->list_dev_stage[i] = g.n_slots - 1 - i;
    HIPCHK(c, hipMemcpyAsync(c->ids, c->list_dev_stage, (size_t)n_cp * 4, hipMemcpyHostToDevice, cs));
    HIPCHK(c, moe_launch_free_slots(c->ids, n_cp, c->slot_table, c->owner, c->last_use, cs));
    HIPCHK(c, hipStreamSynchronize(cs));
    int row = 0;
    auto copy = [&](int i) -> hipError_t {
      const size_t src = (size_t)(row++ % n_rows) * S;
      return hipMemcpyAsync(c->slot_pool + (size_t)(g.n_slots - 1 - i % n_cp) * S, c->host_pool + src, S,
                            hipMemcpyHostToDevice, cs);
    };
    std::vector<double> rates;
    for (int rep = 0; rep < 6; ++rep) {
      HIPCHK(c, hipEventRecord(t0, cs));
      for (int i = 0; i < n_cp; ++i) HIPCHK(c, copy(i));
      HIPCHK(c, hipEventRecord(t1, cs));
      HIPCHK(c, hipEventSynchronize(t1));
      float ms = 0.f;
      HIPCHK(c, hipEventElapsedTime(&ms, t0, t1));
      if (rep > 0) rates.push_back((double)n_cp * S / (ms * 1e-3) / 1e9);   // the first round warms up
    }
    summarise(rates, out->B_P, out->B_P_min, out->B_P_max);
    out->n_copy = (int)rates.size();
    // the host branch while the link copies: a train of copies long enough
    // to cover the host calls (about three times their expected time); only
    // calls that end before the train does count.  Two trains: the first
    // warms the concurrent regime and is not counted (measured once per
    // calibration, the concurrent rate of a process's first calibration ran
    // up to a fifth below that of its second).
    const double host_s = (n_host + 1) * ((double)G * S / (out->host_alone * 1e9) + (double)S / (out->host_alone_1 * 1e9) +
                                          2e-6 * kHostIdleGapUs);
    const double copy_s = (double)S / (out->B_P * 1e9);
    const int n_train = (int)std::min(1024.0, std::max(4.0 * n_cp, std::ceil(3.0 * host_s / copy_s)));
    std::vector<double> conc, conc1;
    for (int rep = 0; rep < 2; ++rep) {
      for (int i = 0; i < n_train; ++i) HIPCHK(c, copy(i));
      HIPCHK(c, hipEventRecord(t1, cs));
      for (int i = 0; i < n_host + 1; ++i) {
        if (hipEventQuery(t1) != hipErrorNotReady) break;
        const double r = gapped_call(G);
        if (hipEventQuery(t1) != hipErrorNotReady) break;   // the train ended during the call
        const double r1 = gapped_call(1);
        if (hipEventQuery(t1) != hipErrorNotReady) break;
        if (i > 0 && rep == 1) {
          conc.push_back(r);
          conc1.push_back(r1);
        }
      }
      HIPCHK(c, hipEventSynchronize(t1));
    }
    summarise(conc, out->host_conc, out->host_conc_min, out->host_conc_max);
    summarise(conc1, out->host_conc_1, lo1, hi1);
    out->n_host_conc = (int)conc.size();
    (void)hipEventDestroy(t0);
    (void)hipEventDestroy(t1);
    (void)hipStreamDestroy(cs);
  }
  // t(n) = t0 + n S / B_R through the medians at n = 1 and n = G (review
  // section 2.5: B_R = B_H - B_P is the rate the host branch adds); with the
  // link busy when at least 3 pairs of calls ran inside the copy train,
  // else alone.  A single size (G = 1), or medians whose line has no
  // positive intercept, leave t0 = 0 and B_R the rate at G.
  const bool conc_ok = out->n_host_conc >= 3;
  const double rG = conc_ok ? out->host_conc : out->host_alone, r1 = conc_ok ? out->host_conc_1 : out->host_alone_1;
  const double msG = (double)G * S / (rG * 1e9) * 1e3, ms1 = (double)S / (r1 * 1e9) * 1e3;
  double BR = rG, t0_us = 0.0;
  const double tau = G > 1 ? (msG - ms1) / (G - 1) : 0.0;   // ms per further expert
  if (G > 1 && tau > 0 && ms1 > tau) {
    BR = (double)S / (tau * 1e-3) / 1e9;
    t0_us = (ms1 - tau) * 1e3;
  }
  out->B_R = BR;
  out->host_t0_us = t0_us;
  out->B_H = out->B_P + BR;
  c->host_t0_us = t0_us;
  return MOE_OK;
}

int moe_calibrate(moe_ctx* c, double* B_P, double* B_H) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  moe_calibration m;
  const int rc = moe_calibrate_ex(c, 1, &m);
  if (rc) return rc;
  if (B_P) *B_P = m.B_P;
  if (B_H) *B_H = m.B_H;
  return MOE_OK;
}

int moe_check_device_error(moe_ctx* c) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  int v = 0;
  HIPCHK(c, hipDeviceSynchronize());
  HIPCHK(c, hipMemcpy(&v, c->err, sizeof(int), hipMemcpyDeviceToHost));
  HIPCHK(c, hipMemset(c->err, 0, sizeof(int)));
  HIPCHK(c, hipDeviceSynchronize());
  if (v & 1) return fail(c, MOE_E_NOT_RESIDENT, "a routed expert was neither resident nor in the host miss set");
  if (v & 2) return fail(c, MOE_E_UNSUPPORTED, "a one-workgroup-per-item GEMM launch had fewer workgroups than items");
  return MOE_OK;
}

int moe_profile_begin(moe_ctx* c, int max_launches, unsigned stage_mask) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  if (max_launches < 1 || max_launches > (1 << 20)) return fail(c, MOE_E_INVAL, "max_launches out of range");
  c->prof_mask = stage_mask;
  for (hipEvent_t e : c->prof_ev) (void)hipEventDestroy(e);
  c->prof_ev.assign(2 * (size_t)max_launches, nullptr);
  for (auto& e : c->prof_ev) HIPCHK(c, hipEventCreate(&e));
  c->prof_stage.assign(max_launches, -1);
  c->prof_used = 0;
  c->prof_on = true;
  return MOE_OK;
}

int moe_profile_end(moe_ctx* c, moe_profile* out) {
  if (!c) return fail(nullptr, MOE_E_INVAL, "null ctx");
  if (!c->prof_on) return fail(c, MOE_E_INVAL, "profiling was not started");
  c->prof_on = false;
  HIPCHK(c, hipDeviceSynchronize());
  moe_profile p;
  std::memset(&p, 0, sizeof(p));
  for (size_t i = 0; i < c->prof_used; ++i) {
    float ms = 0.f;
    HIPCHK(c, hipEventElapsedTime(&ms, c->prof_ev[2 * i], c->prof_ev[2 * i + 1]));
    const int st = c->prof_stage[i];
    if (st >= 0 && st < MOE_N_STAGES) {
      p.launches[st] += 1;
      p.ms[st] += ms;
    }
  }
  p.dropped = c->prof_used >= c->prof_stage.size() ? 1 : 0;
  for (hipEvent_t e : c->prof_ev) (void)hipEventDestroy(e);
  c->prof_ev.clear();
  c->prof_stage.clear();
  c->prof_used = 0;
  if (out) *out = p;
  return MOE_OK;
}

}  // extern "C"
