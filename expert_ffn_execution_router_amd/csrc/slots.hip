// Device-side cache control over the shared expert slot pool.
//
// Method (paper.oopus.info review of FreeToken):
//  * section 2: one slot holds every tensor of one (layer, expert); the slot
//    table maps the logical id l*E+e to a physical slot;
//  * section 2.4: one global LRU over all layers; a hit refreshes recency, a
//    miss admits the expert and evicts the least recently needed one;
//  * section 2.5: the miss set M of a layer splits into a fill set F
//    (q = |F| experts copied over the link) and a host set C; q* = m B_P/B_H
//    rounded to nearest, at least one fill; C leaves residency untouched;
//  * section 2.6: one kernel per layer de-duplicates the routed experts,
//    classifies hits and misses against the residency table, computes q,
//    picks victims in a single pass that yields K least-recently-used
//    candidates (the miss path takes the first q), and rewrites the table.
// Readings: round half up; B_H <= B_P gives q = m; F = the q misses with the
// smallest ids; victims are slots not stamped in this tick ordered by
// (last-use stamp, slot), empty slots carry stamp 0; the i-th expert of F
// goes to the i-th victim; q is capped by the eligible slot count and the
// remainder joins C.
#include "common.h"

constexpr int PLAN_MAX_SLOTS = 8192;

// Exclusive rank of this lane's predicate among the block's threads, in
// thread order (one call per thread of the block; all threads take part).
// wtot: LDS scratch of one int per wave; returns the block total in *total.
DEV int block_rank(bool pred, int* wtot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint64_t b = __ballot(pred);
  if (lane == 0) wtot[wave] = __popcll(b);
  __syncthreads();
  int off = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int c = wtot[w];
    off += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();                      // wtot may be reused by the next call
  *total = all;
  return off + __popcll(b & ((1ull << lane) - 1ull));
}

__global__ void __launch_bounds__(1024)
plan_kernel(const int32_t* __restrict__ ids, int n_assign, int layer, int E, int n_slots,
            int32_t* __restrict__ slot_table, int32_t* __restrict__ owner, uint32_t* __restrict__ last_use,
            CacheCtl* __restrict__ ctl, int policy, double BP, double BH, uint32_t* __restrict__ miss_mask,
            PlanOut* __restrict__ plan, HostStage hs) {
  __shared__ uint32_t stamp[PLAN_MAX_SLOTS];
  __shared__ int flag[256];
  __shared__ int miss[256];
  __shared__ int hist[256];
  __shared__ int wtot[16];
  __shared__ uint64_t vkey[256];
  __shared__ int vict[256];
  __shared__ int s_digit, s_need, s_nv;
  __shared__ uint32_t mask[8];
  const int tid = threadIdx.x;
  const uint32_t tick = ctl->tick + 1u;   // written back by thread 0 after the last barrier
  if (tid < 256) flag[tid] = 0;
  if (tid < 8) mask[tid] = 0u;
  // stamps before this call (read once; later updates are tracked in LDS)
  for (int s = tid; s < n_slots; s += blockDim.x) stamp[s] = last_use[s];
  __syncthreads();
  for (int i = tid; i < n_assign; i += blockDim.x) flag[ids[i]] = 1;
  __syncthreads();
  // classify: thread e looks up expert e
  const bool routed = tid < E && flag[tid];
  int my_slot = -1;
  if (routed) {
    my_slot = slot_table[layer * E + tid];
    if (my_slot >= 0) {                 // hit: refresh recency
      stamp[my_slot] = tick;
      last_use[my_slot] = tick;
    }
  }
  int m, h, u;
  const int mrank = block_rank(routed && my_slot < 0, wtot, &m);   // misses in ascending expert id
  block_rank(routed && my_slot >= 0, wtot, &h);
  block_rank(routed, wtot, &u);
  if (routed && my_slot < 0) miss[mrank] = tid;
  int q;
  if (m == 0 || policy == 1) q = 0;              // HOST: every miss on the host
  else if (policy == 0 || BH <= BP) q = m;       // OFFLOAD, or no residual host bandwidth
  else {
    q = (int)floor((double)m * BP / BH + 0.5);
    q = max(1, min(m, q));
  }
  int elig = 0;
  if (q > 0) {
    // Victims: the q eligible slots (stamp != tick) with the smallest
    // (stamp, slot).  Radix select of the q-th smallest stamp, one byte per
    // pass from the top, then the lowest-numbered slots holding that stamp.
    int n_elig = 0;
    for (int base = 0; base < n_slots; base += blockDim.x) {
      int c;
      block_rank(base + tid < n_slots && stamp[base + tid] != tick, wtot, &c);
      n_elig += c;
    }
    elig = min(n_elig, 256);
    q = min(q, elig);
  }
  if (q > 0) {
    uint32_t prefix = 0, pmask = 0;
    int need = q;                                 // rank (1-based) still sought among matching stamps
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int s = tid; s < n_slots; s += blockDim.x) {
        const uint32_t st = stamp[s];
        if (st != tick && (st & pmask) == prefix) atomicAdd(&hist[(st >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, d = 0;
        while (cum + hist[d] < need) cum += hist[d++];
        s_digit = d;
        s_need = need - cum;
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      pmask |= 255u << shift;
      need = s_need;
    }
    // prefix = the q-th smallest stamp; every eligible slot below it is a
    // victim, plus the `need` lowest-numbered slots holding it
    if (tid == 0) s_nv = 0;
    __syncthreads();
    int taken = 0;
    for (int base = 0; base < n_slots; base += blockDim.x) {
      const int s = base + tid;
      const uint32_t st = s < n_slots ? stamp[s] : tick;
      const bool below = st != tick && st < prefix;
      const bool at = st != tick && st == prefix;
      int n_at;
      const int r = block_rank(at, wtot, &n_at);
      if (below || (at && taken + r < need)) {
        const int slot_i = atomicAdd(&s_nv, 1);
        vkey[slot_i] = ((uint64_t)st << 32) | (uint32_t)s;
      }
      taken += n_at;
    }
    __syncthreads();
    // order the q victims by (stamp, slot)
    if (tid < q) {
      const uint64_t k = vkey[tid];
      int r = 0;
      for (int j = 0; j < q; ++j) r += vkey[j] < k ? 1 : 0;
      vict[r] = (int)(uint32_t)(k & 0xffffffffull);
    }
    __syncthreads();
  }
  // evict victims' owners, install F
  __shared__ int ev_flag[256];
  if (tid < q) {
    const int e = miss[tid];
    const int s = vict[tid];
    const int old = owner[s];
    ev_flag[tid] = old >= 0 ? 1 : 0;
    if (old >= 0) slot_table[old] = -1;
    owner[s] = layer * E + e;
    slot_table[layer * E + e] = s;
    last_use[s] = tick;
    plan->F[tid] = e;
    plan->F_slot[tid] = s;
    if (hs.plan) {
      hs.plan->F[tid] = e;
      hs.plan->F_slot[tid] = s;
    }
  }
  __syncthreads();
  if (tid >= q && tid < m) {
    const int e = miss[tid];
    atomicOr(&mask[e >> 5], 1u << (e & 31));
    plan->C[tid - q] = e;
    if (hs.plan) hs.plan->C[tid - q] = e;
  }
  __syncthreads();
  if (tid < 8) miss_mask[tid] = mask[tid];
  if (tid == 0) {
    int ne = 0;
    for (int i = 0; i < q; ++i) ne += ev_flag[i];
    plan->n_unique = u;
    plan->n_hit = h;
    plan->m = m;
    plan->q = q;
    plan->n_host = m - q;
    plan->n_evict = ne;
    plan->eligible = elig;
    plan->tick = (int)tick;
    ctl->tick = tick;
    ctl->calls += 1;
    ctl->n_unique += u;
    ctl->n_hit += h;
    ctl->m += m;
    ctl->q += q;
    ctl->n_host += m - q;
    ctl->n_evict += ne;
    if (hs.plan) {
      hs.plan->n_unique = u;
      hs.plan->n_hit = h;
      hs.plan->m = m;
      hs.plan->q = q;
      hs.plan->n_host = m - q;
      hs.plan->n_evict = ne;
      hs.plan->eligible = elig;
      hs.plan->tick = (int)tick;
    }
  }
  // the host branch's inputs, written straight into pinned host memory
  // (visible to the host once the kernel has completed)
  if (hs.plan) {
    for (int i = tid; i < n_assign; i += blockDim.x) {
      hs.ids[i] = ids[i];
      hs.w[i] = hs.w_src[i];
    }
    if ((((uintptr_t)hs.hidden_src | (uintptr_t)hs.hidden) & 15u) == 0 && (hs.n_hidden & 7) == 0) {
      const i32x4_t* src = (const i32x4_t*)hs.hidden_src;
      i32x4_t* dst = (i32x4_t*)hs.hidden;
      for (int i = tid; i < hs.n_hidden / 8; i += blockDim.x) dst[i] = src[i];
    } else {
      for (int i = tid; i < hs.n_hidden; i += blockDim.x) hs.hidden[i] = hs.hidden_src[i];
    }
  }
}

// The fill set of the last plan in one launch (section 2.6: a device-resident
// source/destination table shared by every bank, applied by one fixed-shape
// launch, entries past the device valid count unused): expert F[j] of
// `layer` is read from the pinned host pool through its device mapping and
// written to slot F_slot[j].  Each expert blob is S contiguous bytes in both
// pools, so one table entry moves one blob.  V is the copy word (16, 8 or 4
// bytes, dividing S and both base addresses); four words per thread are in
// flight so a few dozen workgroups keep the link busy.
template <typename V>
__global__ void __launch_bounds__(256)
fill_kernel(const PlanOut* __restrict__ plan, const uint8_t* __restrict__ host_pool, int layer, int E, size_t S,
            uint8_t* __restrict__ slot_pool) {
  const int q = plan->q;
  const size_t n = S / sizeof(V);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (int j = 0; j < q; ++j) {
    const V* __restrict__ src = (const V*)(host_pool + ((size_t)layer * E + plan->F[j]) * S);
    V* __restrict__ dst = (V*)(slot_pool + (size_t)plan->F_slot[j] * S);
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
      const V a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
      dst[i] = a;
      dst[i + stride] = b;
      dst[i + 2 * stride] = c;
      dst[i + 3 * stride] = d;
    }
    for (; i < n; i += stride) dst[i] = src[i];
  }
}

// Drop the given experts of one layer from the cache (slot becomes empty).
__global__ void evict_kernel(const int32_t* __restrict__ experts, int n, int layer, int E,
                             int32_t* __restrict__ slot_table, int32_t* __restrict__ owner,
                             uint32_t* __restrict__ last_use) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int g = layer * E + experts[i];
  const int s = slot_table[g];
  if (s >= 0) {
    slot_table[g] = -1;
    owner[s] = -1;
    last_use[s] = 0u;
  }
}

// Full-layer buffer (section 2.2 of the review): slots [base, base+E) receive
// layer `layer`'s experts in order.  Previous owners of those slots lose
// residency; slots previously holding this layer's experts elsewhere become
// empty.  Two phases separated by a barrier so installs win.
__global__ void __launch_bounds__(256)
install_layer_kernel(int layer, int base, int E, CacheCtl* __restrict__ ctl, int32_t* __restrict__ slot_table,
                     int32_t* __restrict__ owner, uint32_t* __restrict__ last_use) {
  const int e = threadIdx.x;
  const uint32_t tick = ctl->tick + 1u;
  const int g = layer * E + e;
  const int s = base + e;
  if (e < E) {
    const int old = owner[s];
    if (old >= 0 && old != g) slot_table[old] = -1;
    const int prev = slot_table[g];
    if (prev >= 0 && prev != s && (prev < base || prev >= base + E)) {
      owner[prev] = -1;
      last_use[prev] = 0u;
    }
  }
  __threadfence_block();
  __syncthreads();
  if (e < E) {
    owner[s] = g;
    slot_table[g] = s;
    last_use[s] = tick;
  }
  if (e == 0) ctl->tick = tick;
}

// Free the given slots (their owners lose residency).
__global__ void free_slots_kernel(const int32_t* __restrict__ slots, int n, int32_t* __restrict__ slot_table,
                                  int32_t* __restrict__ owner, uint32_t* __restrict__ last_use) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int s = slots[i];
  const int old = owner[s];
  if (old >= 0) slot_table[old] = -1;
  owner[s] = -1;
  last_use[s] = 0u;
}

// Host-set bits of every expert outside [lo, hi) (one round of a layer
// evaluated in expert ranges).
__global__ void range_mask_kernel(int lo, int hi, int E, uint32_t* __restrict__ mask) {
  const int wd = threadIdx.x;           // 8 threads, one 32-expert word each
  uint32_t m = 0u;
  for (int b = 0; b < 32; ++b) {
    const int e = wd * 32 + b;
    if (e < E && (e < lo || e >= hi)) m |= 1u << b;
  }
  mask[wd] = m;
}

// Empty every slot and the whole table.
__global__ void reset_kernel(int n_table, int n_slots, int32_t* slot_table, int32_t* owner, uint32_t* last_use,
                             int* err) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_table) slot_table[i] = -1;
  if (i < n_slots) { owner[i] = -1; last_use[i] = 0u; }
  if (i < 16) err[i] = 0;
}

extern "C" size_t moe_plan_out_bytes() { return sizeof(PlanOut); }

extern "C" hipError_t moe_launch_plan(const int32_t* ids, int n_assign, int layer, int E, int n_slots,
                                      int32_t* slot_table, int32_t* owner, uint32_t* last_use, void* ctl,
                                      int policy, double BP, double BH, uint32_t* miss_mask, void* plan,
                                      const void* host_stage, hipStream_t s) {
  HostStage hs{};
  if (host_stage) hs = *(const HostStage*)host_stage;
  plan_kernel<<<1, 1024, 0, s>>>(ids, n_assign, layer, E, n_slots, slot_table, owner, last_use, (CacheCtl*)ctl,
                                 policy, BP, BH, miss_mask, (PlanOut*)plan, hs);
  return hipGetLastError();
}

// grid: workgroups of the fill launch (the link saturates near 64).
extern "C" hipError_t moe_launch_fill(const void* plan, const uint8_t* host_pool_dev, int layer, int E, size_t S,
                                      uint8_t* slot_pool, int grid, hipStream_t s) {
  const uintptr_t a = (uintptr_t)host_pool_dev | (uintptr_t)slot_pool | (uintptr_t)S;
  const PlanOut* p = (const PlanOut*)plan;
  if ((a & 15u) == 0)
    fill_kernel<i32x4_t><<<grid, 256, 0, s>>>(p, host_pool_dev, layer, E, S, slot_pool);
  else if ((a & 7u) == 0)
    fill_kernel<unsigned long long><<<grid, 256, 0, s>>>(p, host_pool_dev, layer, E, S, slot_pool);
  else if ((a & 3u) == 0)
    fill_kernel<unsigned int><<<grid, 256, 0, s>>>(p, host_pool_dev, layer, E, S, slot_pool);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_range_mask(int lo, int hi, int E, uint32_t* mask, hipStream_t s) {
  range_mask_kernel<<<1, 8, 0, s>>>(lo, hi, E, mask);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_evict(const int32_t* experts, int n, int layer, int E, int32_t* slot_table,
                                       int32_t* owner, uint32_t* last_use, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  evict_kernel<<<(n + 255) / 256, 256, 0, s>>>(experts, n, layer, E, slot_table, owner, last_use);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_install_layer(int layer, int base, int E, void* ctl, int32_t* slot_table,
                                               int32_t* owner, uint32_t* last_use, hipStream_t s) {
  install_layer_kernel<<<1, 256, 0, s>>>(layer, base, E, (CacheCtl*)ctl, slot_table, owner, last_use);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_free_slots(const int32_t* slots, int n, int32_t* slot_table, int32_t* owner,
                                            uint32_t* last_use, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  free_slots_kernel<<<(n + 255) / 256, 256, 0, s>>>(slots, n, slot_table, owner, last_use);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_reset(int n_table, int n_slots, int32_t* slot_table, int32_t* owner,
                                       uint32_t* last_use, int* err, hipStream_t s) {
  const int n = max(max(n_table, n_slots), 16);
  reset_kernel<<<(n + 255) / 256, 256, 0, s>>>(n_table, n_slots, slot_table, owner, last_use, err);
  return hipGetLastError();
}
