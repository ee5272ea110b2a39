// Device code shared by the routing kernels and the matrix-vector kernels
// that route for themselves: top-k of one token per wave and the one-wave
// grouping of at most 64 routed pairs.
//
// Method (paper.oopus.info review of FreeToken, sections 1-2; gpts24
// analysis "FreeToken 重写本地 MoE 推理"): selection on the router logits
// (larger first, equal values -> lower expert index), gate weights = softmax
// over the chosen logits; grouping = the (token, choice) pairs sorted by
// expert, tokens ascending inside an expert.
#pragma once
#include "common.h"

// One wave per token (E <= 256: lane l holds experts l, l+64, l+128, l+192).
// Selection works on an order-preserving 32-bit key of each logit (-0 taken
// as +0, so equal logits have equal keys): the k-th largest key is found by
// bisection on its bits with wave ballots (one compare per expert slot and
// step, the counts in scalar registers), the k winners are the keys above it
// plus the lowest-numbered experts at it, and each winner's output position
// is its rank among the winners (descending logit, ties to the lower expert
// id), counted by lanes 0..k-1 over the k winners staged in LDS.  The gate
// weights are the softmax of the winners, summed in output order.

// Per-wave LDS of topk_row: the winners in expert order, then in output order
// (16-byte aligned arrays of 8, read as two 16-byte vectors).
struct __attribute__((aligned(16))) TopkScratch {
  uint32_t key[8];
  int32_t e[8];
  float v[8];
  int32_t oe[8];
  float ov[8];
};

// LDS written by some lanes of a wave and read by others afterwards: a wave's
// LDS operations complete in order, so the compiler only has to keep them in
// program order.
DEV void wave_lds_order() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// One wave, NS = ceil(E / 64) expert slots per lane (a compile-time count,
// so the bisection loop has no branches besides its own).  k <= 8.  The
// selection: v / key of the lane's experts lane + 64i, and selm[i] the
// ballot of the winners among slot i.
template <int NS>
DEV void topk_select_ns(const float* __restrict__ zr, int E, int k, float (&v)[4], uint32_t (&key)[4],
                        uint64_t (&selm)[4]) {
  const int lane = threadIdx.x & 63;
  constexpr int ns = NS;
  uint64_t vm[4];                               // lanes whose slot i holds an expert
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = 0.0f;
    key[i] = 0u;
    vm[i] = 0ull;
    if (i < ns) {
      const int e = lane + 64 * i;
      const float x = zr[min(e, E - 1)];         // clamped load; entries past E are masked out
      v[i] = x == 0.0f ? 0.0f : x;
      const uint32_t u = __float_as_uint(v[i]);
      key[i] = (u >> 31) ? ~u : (u | 0x80000000u);
      vm[i] = __builtin_amdgcn_ballot_w64(e < E);
    }
  }
  // the k-th largest key
  uint32_t kth = 0;
#pragma unroll 8
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = kth | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < ns) cnt += __popcll(__builtin_amdgcn_ballot_w64(key[i] >= cand) & vm[i]);
    if (cnt >= k) kth = cand;
  }
  // winners: keys above kth, then the lowest-numbered experts at kth
  // (expert ids ascend with the slot, then the lane)
  int need = k;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    selm[i] = i < ns ? __builtin_amdgcn_ballot_w64(key[i] > kth) & vm[i] : 0ull;
    need -= __popcll(selm[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint64_t m = i < ns ? __builtin_amdgcn_ballot_w64(key[i] == kth) & vm[i] : 0ull;
    for (; need > 0 && m; --need) {
      const uint64_t lo = m & (~m + 1ull);
      selm[i] |= lo;
      m ^= lo;
    }
  }
}

template <int NS>
DEV void topk_row_ns(const float* __restrict__ zr, int E, int k, int32_t* __restrict__ ids_r,
                     float* __restrict__ w_r, int32_t* lds_r, TopkScratch* sc) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  float v[4];
  uint32_t key[4];
  uint64_t selm[4];
  topk_select_ns<NS>(zr, E, k, v, key, selm);
  // the winners in expert order
  int at = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if ((selm[i] >> lane) & 1ull) {
      const int p = at + __popcll(selm[i] & below);
      sc->key[p] = key[i];
      sc->e[p] = lane + 64 * i;
      sc->v[p] = v[i];
    }
    at += __popcll(selm[i]);
  }
  wave_lds_order();
  // lane j < k: winner j's output position (all 8 entries read at once;
  // those past k are ignored)
  if (lane < k) {
    const uint32_t kj = sc->key[lane];
    const int ej = sc->e[lane];
    uint32_t kq[8];
    int eq[8];
    __builtin_memcpy(kq, sc->key, sizeof(kq));       // two 16-byte LDS reads each
    __builtin_memcpy(eq, sc->e, sizeof(eq));
    int r = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      r += (int)(q < k) & ((int)(kq[q] > kj) | ((int)(kq[q] == kj) & (int)(eq[q] < ej)));
    sc->oe[r] = ej;
    sc->ov[r] = sc->v[lane];
  }
  wave_lds_order();
  // softmax over the winners in output order (the first is the largest)
  if (lane < k) {
    float ov[8];
    __builtin_memcpy(ov, sc->ov, sizeof(ov));
    const float top = ov[0];
    float ssum = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float eq = expf(ov[q] - top);
      ssum += q < k ? eq : 0.0f;
    }
    const int ej = sc->oe[lane];
    ids_r[lane] = ej;
    w_r[lane] = expf(sc->ov[lane] - top) / ssum;
    if (lds_r) lds_r[lane] = ej;
  }
}

// One wave: the winners of logit row zr as ballots per expert slot (expert
// lane + 64i is a winner iff bit lane of selm[i] is set), any E <= 256.
DEV void topk_select(const float* __restrict__ zr, int E, int k, uint64_t (&selm)[4]) {
  float v[4];
  uint32_t key[4];
  switch ((E + 63) >> 6) {
    case 1: topk_select_ns<1>(zr, E, k, v, key, selm); break;
    case 2: topk_select_ns<2>(zr, E, k, v, key, selm); break;
    case 3: topk_select_ns<3>(zr, E, k, v, key, selm); break;
    default: topk_select_ns<4>(zr, E, k, v, key, selm); break;
  }
}

// One wave: the k winners of logit row zr into ids_r / w_r (and, when
// lds_r is not null, the ids into lds_r too).  sc: this wave's scratch.
DEV void topk_row(const float* __restrict__ zr, int E, int k, int32_t* __restrict__ ids_r, float* __restrict__ w_r,
                  int32_t* lds_r, TopkScratch* sc) {
  switch ((E + 63) >> 6) {
    case 1: topk_row_ns<1>(zr, E, k, ids_r, w_r, lds_r, sc); break;
    case 2: topk_row_ns<2>(zr, E, k, ids_r, w_r, lds_r, sc); break;
    case 3: topk_row_ns<3>(zr, E, k, ids_r, w_r, lds_r, sc); break;
    default: topk_row_ns<4>(zr, E, k, ids_r, w_r, lds_r, sc); break;
  }
}

// Inclusive sum over the wave's lanes in lane order (DPP: shifts by 1, 2, 4
// and 8 within each row of 16 lanes, then rows 1 and 3 add lane 15's total
// of the row before, and rows 2 and 3 lane 31's total of rows 0-1).
DEV int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// The grouping of group_from_lds by wave 0 alone, for at most 64 routed
// pairs (T * k <= 64, so T <= 32 and one presence word per expert): lane p
// takes pair p for the marking and the scatter, and experts lane + 64i for
// the counts; the three scans run over the wave (DPP) in expert order, slot
// by slot, so no workgroup barrier is needed.  Same outputs as
// group_from_lds in route.hip.  bits / off / gsl: LDS [E] each.

// The mask words and slots of experts lane + 64i (0 / 0 without a mask or
// table), loaded at the kernel's start so they overlap the top-k.
struct WaveMeta {
  uint32_t mw[4];
  int sl[4];
};

DEV WaveMeta wave_meta(int E, const uint32_t* miss_mask, const int32_t* slot_row) {
  const int lane = threadIdx.x & 63;
  WaveMeta m;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    m.mw[i] = 0u;
    m.sl[i] = 0;
    if (e < E) {
      if (miss_mask) m.mw[i] = miss_mask[e >> 5];
      if (slot_row) m.sl[i] = slot_row[e];
    }
  }
  return m;
}

DEV void group_wave(const int32_t* s_ids, int T, int k, int E, const WaveMeta& wm, int mb, int32_t* counts,
                    int32_t* offsets, int32_t* __restrict__ pos, int32_t* __restrict__ perm_tok, WorkList* wl,
                    int* err, int32_t* pslot, uint32_t* bits, int* off, int* gsl) {
  const int lane = threadIdx.x & 63;
  const int P = T * k, ns = (E + 63) >> 6;
  const uint32_t* mw = wm.mw;
  const int* sl = wm.sl;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < ns && lane + 64 * i < E) bits[lane + 64 * i] = 0u;
  wave_lds_order();
  const int pe = lane < P ? s_ids[lane] : 0, pt = lane < P ? lane / k : 0;
  if (lane < P) atomicOr(&bits[pe], 1u << pt);
  wave_lds_order();
  int c_off = 0, c_act = 0, c_blk = 0;         // totals of the slots before i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= ns) break;
    const int e = lane + 64 * i;
    const int c = e < E ? __popc(bits[e]) : 0;
    bool act = false;
    int slot = -1;
    if (c > 0 && !((mw[i] >> (e & 31)) & 1u)) {
      slot = sl[i];
      if (slot < 0) atomicOr(err, 1);
      else act = true;
    }
    const int nb = act ? (c + mb - 1) / mb : 0;
    const int io = wave_incl_sum(c), ia = wave_incl_sum(act ? 1 : 0), ib = wave_incl_sum(nb);
    const int o = c_off + io - c, a = c_act + ia - (act ? 1 : 0), pb = c_blk + ib - nb;
    if (e < E) {
      counts[e] = c;
      offsets[e] = o;
      off[e] = o;
      gsl[e] = act ? slot : -1;
    }
    if (act) { wl->act_e[a] = e; wl->act_slot[a] = slot; wl->mblk_prefix[a] = pb; }
    c_off += __builtin_amdgcn_readlane(io, 63);
    c_act += __builtin_amdgcn_readlane(ia, 63);
    c_blk += __builtin_amdgcn_readlane(ib, 63);
  }
  if (lane == 0) {
    offsets[E] = c_off;
    wl->n_act = c_act; wl->n_mblk = c_blk; wl->mb = mb; wl->mblk_prefix[c_act] = c_blk;
  }
  wave_lds_order();
  if (lane < P) {
    const int d = off[pe] + __popc(bits[pe] & ((1u << pt) - 1u));
    pos[lane] = d;
    perm_tok[d] = pt;
    if (pslot) pslot[lane] = gsl[pe];
  }
}
