/*
 * moe.h - C ABI of the routed MoE-layer library for MI355X (gfx950).
 *
 * One routed MoE layer forward whose expert weights sit in a shared HBM slot
 * pool keyed by (layer, expert), with the full expert pool in pinned host
 * memory as the source of truth.  The method follows the paper.oopus.info
 * review of FreeToken ("论文综述：FreeToken 让个人电脑跑起前沿 MoE 大模型的边缘原生
 * 服务系统"):
 *   section 2    two-level expert memory; one slot holds every tensor of one
 *                (layer, expert); the cache affects speed, never the output;
 *   section 2.2  full-layer double buffering during prefill;
 *   section 2.4  one global LRU over all layers' experts;
 *   section 2.5  the miss set splits into fills (q of m) and host execution,
 *                q* = m B_P / B_H; the two partial sums are added exactly;
 *   section 2.6  device-side cache control in one kernel per layer; the host
 *                branch returns gate-weighted per-token partial outputs;
 *   section 2.7  expert banks indexed by the flattened id l*E + e.
 *
 * Conventions for every call:
 *   - "device" pointers are HIP device memory, "host" pointers are host
 *     memory (pinned where stated).  The caller owns every buffer it passes;
 *     the library keeps no reference beyond the call except for the buffers
 *     given to moe_create (host pool, slot pool, workspace), which must stay
 *     alive until moe_destroy.
 *   - The library allocates no device memory.  It allocates pinned host
 *     staging buffers and a host thread pool inside the context.
 *   - `stream` arguments are hipStream_t values passed as void* (NULL = the
 *     null stream).  Calls taking a stream enqueue their GPU work on it and
 *     return without waiting unless stated otherwise.
 *   - Returns 0 on success, a negative MOE_E_* code on error (message in
 *     moe_last_error), or a positive informational code.  No C++ exception
 *     crosses this interface.  One context must not be used from two host
 *     threads at once.
 *
 * Data layout:
 *   hidden      bf16 [T, H] row-major (device)
 *   router_w    fp32 [E, H] row-major (device); router_bias fp32 [E] or NULL
 *   expert blob (S = moe_expert_bytes bytes; host pool row l*E+e, one slot):
 *     gate [I, H], up [I, H], down [H, I], row-major [out, in], then
 *     - fp8:   fp32 scale per 128x128 block of each matrix ([rows/128][cols/128],
 *              gate, up, down), weight = E4M3FN code * scale;
 *     - mxfp4: E8M0 scale per 32 consecutive inputs of each row ([rows][cols/32],
 *              gate, up, down); two E2M1 codes per byte, even input in the low
 *              nibble; weight = E2M1 value * 2^(scale - 127).
 *     - nvfp4: codes as mxfp4, then an E4M3FN scale per 16 consecutive inputs
 *              of each row ([rows][cols/16], gate, up, down), then three fp32
 *              tensor scales (gate, up, down) and 4 bytes of padding; weight =
 *              E2M1 value * block scale * tensor scale.  The GEMM inputs
 *              (hidden rows, A) are rounded to fp16 and meet the weights,
 *              dequantised exactly to fp16, in the fp16 MFMA (the
 *              large-batch path streams weights as the small one does).
 *   out         bf16 [T, H] (device)
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx;

enum {
  MOE_OK = 0,
  MOE_E_INVAL = -1,          /* bad shape or argument */
  MOE_E_HIP = -2,            /* HIP runtime error (detail in moe_last_error) */
  MOE_E_NOSLOTS = -3,        /* slot pool too small for the request */
  MOE_E_PIN = -4,            /* pinned host allocation failed */
  MOE_E_NOT_RESIDENT = -5,   /* a routed expert neither resident nor masked (device flag) */
  MOE_E_UNSUPPORTED = -6,    /* shape outside the supported range */
  MOE_I_FALLBACK_ONDEMAND = 1, /* prefill ran on demand: fewer than E slots */
  MOE_I_SINGLE_BUFFER = 2      /* prefill streamed full layers through one buffer: E <= slots < 2E */
};

enum { MOE_W_BF16 = 0, MOE_W_FP8_E4M3_B128 = 1, MOE_W_MXFP4 = 2, MOE_W_NVFP4 = 3 };
enum { MOE_ACT_DEFAULT = 0, MOE_ACT_MXFP6 = 1 };   /* moe_set_activations */
enum { MOE_QUANT_MXFP6 = 64 };                      /* moe_quantize format code */

/* Miss policy (paper.oopus.info review, section 5 lists the backend switch
 * offload / cpu / hybrid): OFFLOAD fills every miss (q = m), HOST executes
 * every miss on the host (q = 0), HYBRID uses q* = round(m B_P / B_H),
 * at least 1 (section 2.5). */
enum { MOE_POLICY_OFFLOAD = 0, MOE_POLICY_HOST = 1, MOE_POLICY_HYBRID = 2 };

/* Largest slot pool a context can hold (also the bound of a rebuild). */
enum { MOE_MAX_SLOTS = 8192 };

typedef struct {
  int L, E, k, H, I;   /* layers, experts per layer (<= 256), top-k (<= 8), hidden, expert intermediate */
  int wfmt;            /* MOE_W_* */
  int n_slots;         /* slots in the device slot pool (<= 8192) */
  int max_tokens;      /* largest T of any call */
  int host_threads;    /* host FFN threads (0: hardware concurrency) */
} moe_config;

/* Outcome of one planning call (section 2.5 quantities). */
typedef struct {
  int n_unique;        /* distinct experts routed in this layer */
  int n_hit;           /* resident ones (H) */
  int m;               /* misses */
  int q;               /* filled over the link (F) */
  int n_host;          /* executed on the host (C = m - q) */
  int n_evict;         /* occupied slots overwritten */
  double t_fill_pred_us, t_host_pred_us;  /* qS/B_P and t0 + (m-q)S/(B_H-B_P) (t0 = 0 when m = q) */
} moe_plan_info;

/* Bytes of one expert blob S for the configuration (layout above). */
size_t moe_expert_bytes(const moe_config* cfg);

/* Bytes of device workspace moe_create needs for this configuration. */
size_t moe_workspace_bytes(const moe_config* cfg);

/* Creates a context.  host_pool: host [L*E][S] bytes, pinned (moe_host_alloc)
 * for the copy engines, row l*E+e = expert e of layer l (section 2.7 banks);
 * d_slot_pool: device, n_slots*S bytes; d_workspace: device,
 * moe_workspace_bytes bytes.  Starts with an empty cache (section 2.7: cold
 * start, no warm-up).  Errors: INVAL (shapes: H, I multiples of 128 and H of
 * 256, E <= 256, k <= 8, k <= E, n_slots <= 8192, sizes too small), HIP,
 * PIN (staging), UNSUPPORTED. */
int moe_create(const moe_config* cfg, void* host_pool, size_t host_bytes, void* d_slot_pool, size_t slot_bytes,
               void* d_workspace, size_t ws_bytes, moe_ctx** out);
int moe_destroy(moe_ctx* ctx);

/* Last error message of ctx, or of the calling thread when ctx is NULL. */
const char* moe_last_error(moe_ctx* ctx);

/* Pinned host memory for the host expert pool (hipHostMalloc); the caller
 * fills it and frees it with moe_host_free after moe_destroy. */
int moe_host_alloc(size_t bytes, void** out);
int moe_host_free(void* p);

/* Activation format of the MXFP4 weight path's large-batch GEMMs (the
 * tiled kernels, used when T > 64 and T*k >= 48*E): MOE_ACT_DEFAULT keeps
 * MXFP8 (E4M3 per 32 with an E8M0 scale), MOE_ACT_MXFP6 quantises both GEMM
 * inputs to MXFP6 (E2M3 per 32, see moe_quantize), which the scaled MFMA
 * multiplies with the E2M1 weights at the 6/4-bit rate.  The pages list
 * MXFP4 among the served formats; the activation format is a declared
 * reading.  MOE_E_INVAL for an unknown value or MXFP6 without MXFP4
 * weights.  Small batches keep MXFP8 activations. */
int moe_set_activations(moe_ctx* ctx, int act);

/* Miss policy and the bandwidths (GB/s) q* uses (section 2.5). */
int moe_set_policy(moe_ctx* ctx, int policy, double B_P, double B_H);

/* Startup calibration on the deployed shapes (section 2.5, section 3 Table 1).
 * B_P: rate of whole-expert copies pinned host pool -> slot (median of 5
 * rounds of up to 8 copies from distinct pool rows into the highest slots,
 * which are emptied first and left empty).  The host branch is timed as the
 * decode path calls it, on min(k, E) distinct experts of one layer with all
 * T tokens routed to each (at T = 1, a token whose k experts all miss), the
 * configured threads, weight bytes per second of the call; after a warm-up
 * (at least 8 calls and 100 ms), 40 calls over (layer, expert) groups
 * spread over the pool, so no call finds its bytes in the host caches, first alone
 * (host_alone) and then while a train of copies keeps the link busy
 * (host_conc: calls that end inside the second of two such trains).
 * Single-expert calls (host_alone_1, host_conc_1) are timed beside them, in
 * alternation, each call after a 200 us idle gap (the decode path wakes the
 * pool once per layer, after the layer's GPU work has left it idle): a
 * call on n experts takes t0 + n S / B_R, where t0 is the
 * pool's per-call cost (waking the workers, the phase barriers) and B_R the
 * rate at which further experts stream; the two medians fix both.  Section
 * 2.5 splits the miss set so that the fills, at B_P, and the host branch, on
 * the residual B_R = B_H - B_P, end together; B_R is that marginal rate, from
 * the calls made with the link busy (alone when fewer than 3 calls of each
 * size ran inside the train), and B_H = B_P + B_R.  t0 shifts the balance by
 * t0 B_P B_R / (S (B_P + B_R)) experts (about 0.2 on the decode shape), below
 * the rounding of q*, so q* keeps the closed form; moe_plan_info's host-time
 * prediction adds t0 to every layer that has a host set.  All rates GB/s;
 * medians with min and max.  Synchronous.  INVAL for T outside [1,
 * max_tokens]; HIP. */
typedef struct {
  double B_P, B_P_min, B_P_max;                     /* pinned -> slot copies */
  double B_H;                                       /* B_P + B_R, the value q* uses */
  double host_alone, host_alone_min, host_alone_max;
  double host_conc, host_conc_min, host_conc_max;   /* with the link busy */
  int n_copy, n_host_alone, n_host_conc;            /* timed repeats behind each median */
  double host_alone_1, host_conc_1;                 /* single-expert calls, medians */
  double host_t0_us;                                /* per-call time t0 of the host branch */
  double B_R;                                       /* marginal host rate, B_H - B_P */
} moe_calibration;
int moe_calibrate_ex(moe_ctx* ctx, int T, moe_calibration* out);

/* The same at T = 1 (single-stream decode), returning B_P and B_H. */
int moe_calibrate(moe_ctx* ctx, double* B_P, double* B_H);

/* Device int32 [L*E] residency table: slot of (l, e) or -1.  Review section 2:
 * every slot holds all tensors of one (layer, expert) pair and residency and
 * lookup go by that logical id alone; section 2.6: the control kernel
 * rewrites logical expert ids to physical slot ids.  Owned by the context
 * (inside the workspace); valid until moe_destroy; NULL for a NULL ctx. */
int32_t* moe_slot_table(moe_ctx* ctx);

/* Empties the cache (every slot free, table -1) and clears the device error
 * flag; enqueued on stream. */
int moe_reset_cache(moe_ctx* ctx, void* stream);

/* Router (gpts24, "MoE 模型为什么会造出一个 PCIe 带宽问题": a gate network
 * picks a small subset of experts per incoming token; review section 1: each
 * token activates k of E routed experts).  The pages give no gate formula;
 * the reading taken: logits z = hidden router_w^T + bias (fp32), top-k by
 * logit (larger first, ties to the lower expert id), weights = softmax over
 * the chosen logits (the full softmax renormalised over the k).  hidden
 * device bf16 [T, H]; router_w device fp32 [E, H]; router_bias device fp32
 * [E] or NULL; topk_ids int32 [T, k], topk_w fp32 [T, k] (device,
 * caller-owned).  Asynchronous on stream; INVAL for T outside [0,
 * max_tokens], HIP on a launch failure. */
int moe_route(moe_ctx* ctx, const void* hidden, const float* router_w, const float* router_bias, int T,
              int32_t* topk_ids, float* topk_w, void* stream);

/* Test hook: the activation quantisation that precedes each grouped GEMM
 * of the 8-bit paths (the pages say only that the kernels dequantise in
 * kernel; the rule is a declared reading).  rows x cols values (device),
 * bf16 (src_bf16 = 1) or fp32; output row r quantises source row
 * row_map[r] (device int32 [rows], or NULL for r itself).
 *   wfmt 1 (fp8): per (row, 128 columns) scale = amax/448, q = E4M3(v*448/amax);
 *                 scale fp32 [rows, cols/128]; cols % 128 == 0.
 *   wfmt 2 (mxfp4 weights, MXFP8 activations): per (row, 32 columns) E8M0
 *                 scale 2^x, x = floor(log2 amax) - 8, q = E4M3(v*2^-x);
 *                 scale uint8 [rows, cols/32]; cols % 32 == 0.
 *   MOE_QUANT_MXFP6 (mxfp4 weights, MXFP6 activations): per (row, 32
 *                 columns) E8M0 scale 2^x, x = floor(log2 amax) - 2, codes
 *                 E2M3(v*2^-x) (OCP MX FP6, nearest even, saturating at 7.5);
 *                 cols % 128 == 0.  Chunk-major: q holds cols/128 planes of
 *                 P = round_up(rows*112 + 1024, 256) bytes, rows of 112
 *                 bytes (the last 16 unused); the codes of columns
 *                 128c+32g .. +31 are a 24-byte little-endian string (code
 *                 j at bits 6j..6j+5) whose bytes 0-15 are at
 *                 c*P + r*112 + 24g + 8*(g odd) and bytes 16-23 at
 *                 c*P + r*112 + 24g + 16*(g even); scale uint8
 *                 [cols/128][rows][4], byte g of (c, r) for columns
 *                 128c+32g .. +31.
 * q uint8 [rows, cols] (E4M3 codes) otherwise, caller-owned.  Asynchronous
 * on stream; MOE_E_INVAL for another format or a bad shape. */
int moe_quantize(int wfmt, int src_bf16, const void* src, int rows, int cols, const int32_t* row_map, uint8_t* q,
                 void* scale, void* stream);

/* Same selection from given fp32 logits [T, E] (device), plus the grouping
 * that the grouped evaluation of the GPU set needs (review section 2.5:
 * the GPU evaluates its experts as groups; section 2.6: the routed experts
 * are de-duplicated on the device).  Test hook for bit-exact routing:
 * counts int32 [E], offsets int32 [E+1] (exclusive scan), perm_tok int32 [T*k]
 * (token of each grouped row: experts ascending, tokens ascending within an
 * expert), pos int32 [T, k] (grouped row of each choice).  All device. */
int moe_route_from_logits(moe_ctx* ctx, const float* logits, int T, int32_t* topk_ids, float* topk_w,
                          int32_t* counts, int32_t* offsets, int32_t* perm_tok, int32_t* pos, void* stream);

/* Device-side cache control for one layer (section 2.6): de-duplicate the
 * routed experts in topk_ids (device [T, k]), classify hits and misses,
 * choose q by the policy, pick victims by LRU, rewrite the residency table
 * and write the host-set bits into miss_mask_out (device uint32 [8], bit e
 * set = expert e runs on the host).  Does NOT copy weights: slot_pool_fill
 * or moe_decode_layer does.  Blocks the calling thread until the plan is
 * known; info may be NULL.  The fills it decided are returned through
 * fill_experts / fill_slots (host int32 [E] each, may be NULL). */
int moe_plan(moe_ctx* ctx, int layer, const int32_t* topk_ids, int T, uint32_t* miss_mask_out,
             moe_plan_info* info, int32_t* fill_experts, int32_t* fill_slots, void* stream);

/* Fill of the set F (review section 2.5: the misses chosen for the GPU are
 * copied into their cache slots in one batch; section 2.6: one source /
 * destination table for every bank).  Copies expert (layer, experts[i])
 * from the host pool into slots[i] on copy_stream (n whole-expert DMAs of
 * S bytes) and records the context's fill event, which the next forward
 * on any stream waits for.  experts, slots: host int32 [n]; the residency
 * table is NOT changed (moe_plan already rewrote it).  INVAL for a layer,
 * expert or slot out of range; HIP on a copy failure. */
int slot_pool_fill(moe_ctx* ctx, int layer, const int32_t* experts, const int32_t* slots, int n, void* copy_stream);

/* LRU admission (review section 2.4: one global LRU over every layer's
 * experts; a hit refreshes the expert's recency, a miss installs it in place
 * of the least recently needed one).  experts: host int32 [n] of this
 * layer, n <= 8192: already resident ones are refreshed, the others take
 * the least recently used slots and are copied from the host pool on
 * copy_stream.  Blocks until the admission plan is known (not until the
 * copies end).  NOSLOTS when fewer evictable slots than experts remain
 * (the ones that fit are still installed); INVAL for bad ids. */
int slot_pool_admit(moe_ctx* ctx, int layer, const int32_t* experts, int n, void* copy_stream);

/* Eviction (review section 2.4: the LRU drops what the model needed least
 * recently; section 2.7: the cache is reshaped under a new memory budget).
 * Drops the given experts of a layer (host int32 [n], n <= 8192; absent
 * ones are ignored) from the cache: their slots become free (stamp 0).
 * Synchronous on the null stream; INVAL for bad ids. */
int slot_pool_evict(moe_ctx* ctx, int layer, const int32_t* experts, int n);

/* Rebuilds the expert cache under a new slot budget at a safe point (review
 * section 2.7: no restart, the host pool is not reloaded; section 2: the
 * cache size never changes outputs).  Synchronises the device first, so no
 * work of the context may be in flight on other host threads.  The
 * n_slots (<= MOE_MAX_SLOTS) most recently used residents survive with
 * their recency (stamp descending, ties to the lower slot), packed into
 * slots 0, 1, ... in the order of their old slots; their blobs are copied
 * device-to-device on stream.  d_slot_pool (device, >= n_slots*S bytes,
 * caller-owned) may be the current pool (in place: shrink, or grow within
 * the caller's allocation) or a new one (the old pool may be freed once the
 * call returns).  The prefill streamer restarts its buffers.  HIP graphs
 * captured before the call hold the old pool and slot count and must be
 * captured again.  Errors: INVAL (sizes), HIP. */
int slot_pool_resize(moe_ctx* ctx, void* d_slot_pool, size_t slot_bytes, int n_slots, void* stream);

/* Host branch (section 2.6): host_partial_out[t] = sum over j with
 * topk_ids[t,j] in the mask of topk_w[t,j] * FFN_e(hidden[t]), fp32, computed
 * from the host pool by the context's thread pool.  All pointers host:
 * hidden bf16 [T,H], topk_ids [T,k], topk_w [T,k], miss_mask uint32 [8],
 * host_partial_out fp32 [T,H].  Synchronous. */
int moe_host_partial(moe_ctx* ctx, int layer, const void* hidden, const int32_t* topk_ids, const float* topk_w,
                     int T, const uint32_t* miss_mask, float* host_partial_out);

/* The same computation without a context or GPU: host_pool as in
 * moe_create, host_threads as in moe_config.  Synchronous. */
int moe_host_ffn(const moe_config* cfg, const void* host_pool, int layer, const void* hidden,
                 const int32_t* topk_ids, const float* topk_w, int T, const uint32_t* miss_mask,
                 float* host_partial_out);

/* The routed MoE layer forward on the GPU (review section 2.5: the GPU
 * evaluates its set G = H u F as groups while the host computes C; the two
 * partial sums are added, so the layer output is the plain MoE output;
 * section 2: slot contents change speed, never the result):
 *   out[t] = bf16( sum_{j: e_tj not in mask} w_tj * FFN_e(hidden[t]) + host_partial[t] )
 * routing as moe_route; experts found through slot_table (device int32 [E],
 * this layer's row: slot or -1) in the context's slot pool; miss_mask
 * (device uint32 [8] or NULL) marks experts whose contribution is already in
 * host_partial (device fp32 [T, H] or NULL).  A routed, unmasked expert
 * without a slot sets the device error flag (moe_check_device_error) and is
 * left out.  T <= max_tokens.  Waits for pending fills. */
int moe_layer_forward(moe_ctx* ctx, int layer, const void* hidden, const float* router_w, const float* router_bias,
                      int T, const int32_t* slot_table, const uint32_t* miss_mask, const float* host_partial,
                      void* out, void* stream);

/* Allocation-free moe_layer_forward, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  No context: cfg gives the shape (L,
 * n_slots, max_tokens and host_threads are ignored); slot_pool (device)
 * holds experts in cfg's blob layout; slot_row (device int32 [E]) maps this
 * layer's experts to slots (-1 = absent); the other arguments are those of
 * moe_layer_forward, whose kernels it runs.  Every intermediate lives in one
 * static device array of 40 MiB per GPU, held until the process ends;
 * limits: T <= 64, and a shape whose forward buffers leave at least 4 MiB of
 * the array for the small-batch GEMMs' partial tiles (every shape up to
 * E = 256, k = 8, H = 6144, I = 2048 fits); otherwise MOE_E_UNSUPPORTED,
 * before any device work.  Calls no allocator.  err_flag (device int, may be
 * NULL): error bits are OR-ed into it (bit 0: a routed, unmasked expert
 * without a slot, left out); the caller clears it.  The array keeps the last
 * call's contents; a call writes every part of it that it reads before
 * reading it, so nothing needs clearing between calls.  All calls on one
 * GPU share the array: calls that overlap in time on one GPU (several
 * streams, several host threads) race, so the caller orders them.
 * Asynchronous on stream; errors INVAL, UNSUPPORTED, HIP (message in
 * moe_last_error(NULL)). */
int moe_layer_forward_noalloc(const moe_config* cfg, const void* slot_pool, const int32_t* slot_row,
                              const void* hidden, const float* router_w, const float* router_bias, int T,
                              const uint32_t* miss_mask, const float* host_partial, void* out, int* err_flag,
                              void* stream);

/* One decode-time layer through the cache (sections 2.4-2.6): route, plan
 * (host sync once), start the host branch on C, fill F on copy_stream,
 * grouped GPU evaluation of H u F on compute_stream, add the host partial.
 * Returns after the work is enqueued and the host branch has finished; info
 * may be NULL. */
int moe_decode_layer(moe_ctx* ctx, int layer, const void* hidden, const float* router_w, const float* router_bias,
                     int T, void* out, moe_plan_info* info, void* compute_stream, void* copy_stream);

/* The same layer with no host read of the plan (section 2.6: device-resident
 * cache control, the fill set moved by one fixed-shape launch from a device
 * table with a device valid count, the host branch as a node of the step):
 * every step is enqueued and the call returns at once.
 *   compute_stream: route, plan (the LRU clock advances on the device), the
 *     indexed fill kernel (F from the device plan; reads the pinned host pool
 *     through its device mapping at link speed), grouped GEMMs over H u F,
 *     then, after the host branch, the combine;
 *   host_stream: waits for the plan, copies it and the routed inputs to
 *     pinned staging, runs the host set C on the thread pool in a
 *     hipLaunchHostFunc callback, sends the fp32 partial back.  Used only
 *     when the policy can route misses to the host (not OFFLOAD, or fewer
 *     slots than E); the combine adds the partial only when C is not empty.
 * Both streams may be captured into one HIP graph (fork/join through the
 * context's events; the callback becomes a host node): replays plan afresh.
 * Consecutive calls of one context are ordered through the streams; the
 * staging buffers are shared, so a context runs one asynchronous step
 * sequence at a time and makes no other host-pool call meanwhile.  Results
 * equal moe_decode_layer's.  Errors: INVAL (layer, T), UNSUPPORTED (host pool
 * without a device mapping: allocate it with moe_host_alloc), HIP.  Plan
 * statistics: moe_plan_stats. */
int moe_decode_layer_async(moe_ctx* ctx, int layer, const void* hidden, const float* router_w,
                           const float* router_bias, int T, void* out, void* compute_stream, void* host_stream);

/* Running totals of every plan of the context (device counters, summed by
 * the cache-control kernel): planning calls, routed distinct experts, hits,
 * misses m, fills q, host executions m - q, evictions of a resident expert;
 * host_ms: time the host branches of both decode paths took on the thread
 * pool (from the pool taking the job to its last worker finishing). */
typedef struct moe_plan_totals {
  long long calls, n_unique, n_hit, m, q, n_host, n_evict;
  double host_ms;
} moe_plan_totals;

/* Synchronises the device, reads the totals into out (may be NULL) and clears
 * them when reset != 0.  Also reports (INVAL) a host-branch callback that saw
 * an invalid plan since the last call. */
int moe_plan_stats(moe_ctx* ctx, moe_plan_totals* out, int reset);

/* Prefill with full-layer double buffering (section 2.2): layer l computes
 * from one E-slot buffer while layer l+1's complete expert set is copied into
 * the other on copy_stream.  Buffers are slots [0, E) and [E, 2E) of the
 * pool, entered into the LRU table (survivors warm decode).  Call for
 * l = 0..L-1 in order; layer 0 also issues its own copy.  With E to 2E-1
 * slots the full layers go through one buffer (copy, then compute) and the
 * call returns MOE_I_SINGLE_BUFFER; with fewer than E slots it runs on
 * demand (section 2.2's fallback: the routed experts through the cache,
 * capacity overflow on the host) and returns MOE_I_FALLBACK_ONDEMAND.
 * double_buffer = 0 serialises copy and compute (ablation). */
int prefill_stream_layer(moe_ctx* ctx, int layer, const void* hidden, const float* router_w,
                         const float* router_bias, int T, void* out, void* compute_stream, void* copy_stream,
                         int double_buffer);

/* Reads and clears the device error flag (synchronous): MOE_OK or
 * MOE_E_NOT_RESIDENT.  Review section 2.6: the control kernel maps every
 * routed expert to a slot or to the host marker; a routed expert that a
 * forward finds with neither (a caller that skipped the plan or evicted
 * too early), or a small-batch GEMM launched with fewer workgroups than its
 * items, sets the flag instead of reading a wrong slot. */
int moe_check_device_error(moe_ctx* ctx);

/* Per-stage GPU timing (the pages time stages by wall clock only; this hook
 * brackets each of the context's launches with HIP events on the stream the
 * launch goes to).  Stages: */
enum {
  MOE_STAGE_ROUTE = 0,    /* router logits */
  MOE_STAGE_TOPK = 1,     /* top-k and gate weights */
  MOE_STAGE_GROUP = 2,    /* histogram, scan, permutation, work list */
  MOE_STAGE_QUANT_X = 3,  /* activation quantisation before GEMM 1 (8-bit formats) */
  MOE_STAGE_GEMM1 = 4,    /* grouped gate/up GEMM with SwiGLU */
  MOE_STAGE_QUANT_A = 5,  /* quantisation of A before GEMM 2 (8-bit formats) */
  MOE_STAGE_GEMM2 = 6,    /* grouped down GEMM */
  MOE_STAGE_COMBINE = 7,  /* weighted unpermute-combine */
  MOE_STAGE_PLAN = 8,     /* cache-control kernel */
  MOE_STAGE_FIXUP = 9,    /* small-batch GEMMs: sums of the items cut between workgroups */
  MOE_STAGE_FILL = 10,    /* indexed host-pool -> slot copy of the fill set (asynchronous decode) */
  MOE_STAGE_TAIL = 11,    /* large batches: the overflow rows' small-batch GEMMs and their sums */
  MOE_N_STAGES = 12
};

typedef struct {
  int launches[MOE_N_STAGES];  /* timed launches per stage */
  double ms[MOE_N_STAGES];     /* summed event time per stage, ms */
  int dropped;                 /* 1 if more than max_launches launches happened */
} moe_profile;

/* Starts timing up to max_launches launches of the stages whose bit is set in
 * stage_mask (bit MOE_STAGE_x; allocates 2*max_launches events).  Event
 * records issued while a stream is being captured become graph nodes and
 * time each replay. */
int moe_profile_begin(moe_ctx* ctx, int max_launches, unsigned stage_mask);
/* Synchronises the device, sums the records into out and stops timing. */
int moe_profile_end(moe_ctx* ctx, moe_profile* out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
