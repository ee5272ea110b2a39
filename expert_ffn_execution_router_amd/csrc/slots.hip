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

__global__ void __launch_bounds__(1024)
plan_kernel(const int32_t* __restrict__ ids, int n_assign, int layer, int E, int n_slots,
            int32_t* __restrict__ slot_table, int32_t* __restrict__ owner, uint32_t* __restrict__ last_use,
            uint32_t tick, int policy, double BP, double BH, uint32_t* __restrict__ miss_mask,
            PlanOut* __restrict__ plan) {
  __shared__ uint64_t keys[PLAN_MAX_SLOTS];
  __shared__ int flag[256];
  __shared__ int miss[256];
  __shared__ int s_m, s_q, s_hit, s_uniq, s_npow, s_elig;
  __shared__ uint32_t mask[8];
  const int tid = threadIdx.x;
  if (tid < 256) flag[tid] = 0;
  if (tid < 8) mask[tid] = 0u;
  // stamps before this call (read once; later updates are tracked in LDS)
  for (int s = tid; s < n_slots; s += blockDim.x) keys[s] = last_use[s];
  __syncthreads();
  for (int i = tid; i < n_assign; i += blockDim.x) flag[ids[i]] = 1;
  __syncthreads();
  int my_slot = -1;
  if (tid < E && flag[tid]) {
    my_slot = slot_table[layer * E + tid];
    if (my_slot >= 0) {                 // hit: refresh recency
      keys[my_slot] = tick;
      last_use[my_slot] = tick;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int m = 0, h = 0, u = 0;
    for (int e = 0; e < E; ++e) {
      if (!flag[e]) continue;
      ++u;
      if (slot_table[layer * E + e] >= 0) ++h; else miss[m++] = e;
    }
    int q;
    if (m == 0 || policy == 1) q = 0;              // HOST: every miss on the host
    else if (policy == 0 || BH <= BP) q = m;       // OFFLOAD, or no residual host bandwidth
    else {
      q = (int)floor((double)m * BP / BH + 0.5);
      q = max(1, min(m, q));
    }
    int np = 1;
    while (np < n_slots) np <<= 1;
    s_m = m; s_q = q; s_hit = h; s_uniq = u; s_npow = np;
  }
  __syncthreads();
  const int np = s_npow;
  int q = s_q;
  if (q > 0) {
    // keys: (stamp << 32 | slot); slots stamped this tick are not eligible
    for (int s = tid; s < np; s += blockDim.x) {
      uint64_t k;
      if (s < n_slots) {
        const uint32_t st = (uint32_t)keys[s];
        k = (st == tick) ? ~0ull : (((uint64_t)st << 32) | (uint32_t)s);
      } else {
        k = ~0ull;
      }
      keys[s] = k;
    }
    __syncthreads();
    // bitonic sort, ascending
    for (int kk = 2; kk <= np; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < np; i += blockDim.x) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const uint64_t a = keys[i], b = keys[ixj];
            const bool up = (i & kk) == 0;
            if ((a > b) == up) { keys[i] = b; keys[ixj] = a; }
          }
        }
        __syncthreads();
      }
    }
    if (tid == 0) {
      int el = 0;
      while (el < np && el < 256 && keys[el] != ~0ull) ++el;
      if (el < q) q = el;
      s_q = q;
      s_elig = el;
    }
    __syncthreads();
    q = s_q;
  } else if (tid == 0) {
    s_elig = 0;
  }
  // evict victims' owners, install F
  __shared__ int ev_flag[256];
  if (tid < q) {
    const int e = miss[tid];
    const int s = (int)(uint32_t)(keys[tid] & 0xffffffffull);
    const int old = owner[s];
    ev_flag[tid] = old >= 0 ? 1 : 0;
    if (old >= 0) slot_table[old] = -1;
    owner[s] = layer * E + e;
    slot_table[layer * E + e] = s;
    last_use[s] = tick;
    plan->F[tid] = e;
    plan->F_slot[tid] = s;
  }
  __syncthreads();
  const int m = s_m;
  if (tid >= q && tid < m) {
    const int e = miss[tid];
    atomicOr(&mask[e >> 5], 1u << (e & 31));
    plan->C[tid - q] = e;
  }
  __syncthreads();
  if (tid < 8) miss_mask[tid] = mask[tid];
  if (tid == 0) {
    int ne = 0;
    for (int i = 0; i < q; ++i) ne += ev_flag[i];
    plan->n_unique = s_uniq;
    plan->n_hit = s_hit;
    plan->m = m;
    plan->q = q;
    plan->n_host = m - q;
    plan->n_evict = ne;
    plan->eligible = s_elig;
    plan->tick = (int)tick;
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
install_layer_kernel(int layer, int base, int E, uint32_t tick, int32_t* __restrict__ slot_table,
                     int32_t* __restrict__ owner, uint32_t* __restrict__ last_use) {
  const int e = threadIdx.x;
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
                                      int32_t* slot_table, int32_t* owner, uint32_t* last_use, uint32_t tick,
                                      int policy, double BP, double BH, uint32_t* miss_mask, void* plan,
                                      hipStream_t s) {
  plan_kernel<<<1, 1024, 0, s>>>(ids, n_assign, layer, E, n_slots, slot_table, owner, last_use, tick, policy, BP, BH,
                                 miss_mask, (PlanOut*)plan);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_evict(const int32_t* experts, int n, int layer, int E, int32_t* slot_table,
                                       int32_t* owner, uint32_t* last_use, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  evict_kernel<<<(n + 255) / 256, 256, 0, s>>>(experts, n, layer, E, slot_table, owner, last_use);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_install_layer(int layer, int base, int E, uint32_t tick, int32_t* slot_table,
                                               int32_t* owner, uint32_t* last_use, hipStream_t s) {
  install_layer_kernel<<<1, 256, 0, s>>>(layer, base, E, tick, slot_table, owner, last_use);
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
