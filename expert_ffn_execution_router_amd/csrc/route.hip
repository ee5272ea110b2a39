// Routing and grouping kernels: router logits, top-k with renormalised gate
// weights, per-expert histogram, exclusive scan and stable token permutation.
//
// Method (paper.oopus.info review of FreeToken, sections 1-2; gpts24
// analysis "FreeToken 重写本地 MoE 推理"): a gate network picks a few experts
// per token.  The gate is softmax over E router logits; selection uses the
// logits (larger first, equal values -> lower expert index) and the k chosen
// weights are the softmax over the chosen logits, i.e. the full softmax
// renormalised over them.  Grouping sorts the (token, choice) assignments by
// expert, tokens ascending inside an expert (a stable counting sort, so the
// result is a deterministic function of the routing).
#include "route_dev.h"

// ---------------------------------------------------------------------------
// router logits z[t,e] = sum_h x[t,h] R[e,h] + b[e]  (x bf16, R fp32, fp32 sums)
// ---------------------------------------------------------------------------

// Small batches: one wave per (expert, 4 tokens), a workgroup of
// blockDim/64 such waves, grid (E * 64 / blockDim, T/4) so that every CU
// takes part (8 tokens per wave, so that each expert row is read by half as
// many workgroups, ran the 32- and 64-token router 2 us slower).  A lane
// covers 4 consecutive elements of each 256-element chunk of H and issues
// the loads of 8 chunks (2048 elements) at once, so a wave waits for memory
// once per 2048 elements instead of once per chunk.  Loads and sums are unconditional (token rows past T re-read
// row T-1 and are not stored; chunks past H re-read the last one and are
// weighted by zero), so no branch splits the batch.  H % 256 == 0.
constexpr int RT_TOK = 4;
// One wave: the logits of expert e for tokens t0 .. t0 + RT_TOK - 1.
DEV void router_wave(const uint16_t* __restrict__ x, const float* __restrict__ R, const float* __restrict__ bias,
                     int T, int E, int H, float* __restrict__ z, int e, int t0) {
  const int lane = threadIdx.x & 63;
  const float* r = R + (size_t)e * H;
  const uint16_t* xr[RT_TOK];
#pragma unroll
  for (int i = 0; i < RT_TOK; ++i) xr[i] = x + (size_t)min(t0 + i, T - 1) * H;
  float acc[RT_TOK];
#pragma unroll
  for (int i = 0; i < RT_TOK; ++i) acc[i] = 0.0f;
  const int nchunk = H / 256;
  for (int c0 = 0; c0 < nchunk; c0 += 8) {
    float4 rv[8];
    uint2 xv[8][RT_TOK];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int h = min(c0 + c, nchunk - 1) * 256 + lane * 4;
      rv[c] = *(const float4*)(r + h);
#pragma unroll
      for (int i = 0; i < RT_TOK; ++i) xv[c][i] = *(const uint2*)(xr[i] + h);
    }
    __builtin_amdgcn_sched_barrier(0);    // keep every load of the batch ahead of the sums
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // padding chunks (past H) contribute exactly zero; no branch
      const float f = c0 + c < nchunk ? 1.0f : 0.0f;
      const float4 rw = make_float4(rv[c].x * f, rv[c].y * f, rv[c].z * f, rv[c].w * f);
#pragma unroll
      for (int i = 0; i < RT_TOK; ++i) {
        acc[i] += bf16_bits_to_f32(xv[c][i].x & 0xffffu) * rw.x;
        acc[i] += bf16_bits_to_f32(xv[c][i].x >> 16) * rw.y;
        acc[i] += bf16_bits_to_f32(xv[c][i].y & 0xffffu) * rw.z;
        acc[i] += bf16_bits_to_f32(xv[c][i].y >> 16) * rw.w;
      }
    }
  }
  const float b = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < RT_TOK; ++i) {
    const float v = wave_sum(acc[i]);
    if (lane == 0 && t0 + i < T) z[(size_t)(t0 + i) * E + e] = v + b;
  }
}

__global__ void __launch_bounds__(256)
router_small_kernel(const uint16_t* __restrict__ x, const float* __restrict__ R,
                    const float* __restrict__ bias, int T, int E, int H, float* __restrict__ z) {
  const int e = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (e >= E) return;
  router_wave(x, R, bias, T, E, H, z, e, blockIdx.y * RT_TOK);
}

// Large batches on fp32 MFMA: 64 tokens x 64 experts per workgroup, each wave
// 16 tokens x 64 experts with v_mfma_f32_16x16x4f32 (x widened exactly from
// bf16; R fp32; fp32 accumulation).  K is staged through LDS in chunks of 64
// with rows padded to 65 floats so the 16 rows an MFMA operand read touches
// fall in different banks.
__global__ void __launch_bounds__(256)
router_mfma_kernel(const uint16_t* __restrict__ x, const float* __restrict__ R, const float* __restrict__ bias,
                   int T, int E, int H, float* __restrict__ z) {
  __shared__ float xs[64][65];
  __shared__ float rs[64][65];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  f32x4_t acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // staging: thread loads 16 bf16 of one token row and 16 floats of one expert row
  const int sr = tid >> 2, sc = (tid & 3) * 16;
  const uint16_t* xrow = x + (size_t)min(t0 + sr, T - 1) * H + sc;
  const float* rrow = R + (size_t)min(e0 + sr, E - 1) * H + sc;
  for (int k0 = 0; k0 < H; k0 += 64) {
    const i32x4_t xa = ld16(xrow + k0), xb = ld16(xrow + k0 + 8);
    i32x4_t rv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rv[q] = ld16(rrow + k0 + q * 4);
    __syncthreads();                     // previous chunk's reads are done
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = (uint32_t)xa[q], b = (uint32_t)xb[q];
      xs[sr][sc + 2 * q] = bf16_bits_to_f32(a & 0xffffu);
      xs[sr][sc + 2 * q + 1] = bf16_bits_to_f32(a >> 16);
      xs[sr][sc + 8 + 2 * q] = bf16_bits_to_f32(b & 0xffffu);
      xs[sr][sc + 8 + 2 * q + 1] = bf16_bits_to_f32(b >> 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) rs[sr][sc + 4 * q + u] = __int_as_float(rv[q][u]);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const float av = xs[wave * 16 + lr][ks * 4 + lg];
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, rs[n * 16 + lr][ks * 4 + lg], acc[n], 0, 0, 0);
    }
  }
  // lane holds expert column lr of tile n, tokens 4*lg..4*lg+3 of the wave's 16
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = e0 + n * 16 + lr;
    if (e >= E) continue;
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + wave * 16 + lg * 4 + i;
      if (t < T) z[(size_t)t * E + e] = acc[n][i] + b;
    }
  }
}


// ---------------------------------------------------------------------------
// top-k (one wave per token, E <= 256) and renormalised weights
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ z, int T, int E, int k, int32_t* __restrict__ ids,
            float* __restrict__ w) {
  __shared__ TopkScratch sc[4];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * (blockDim.x >> 6) + wave;
  if (t >= T) return;
  topk_row(z + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, nullptr, sc + wave);
}

// ---------------------------------------------------------------------------
// grouping: histogram -> exclusive scan -> stable scatter
// ---------------------------------------------------------------------------
constexpr int GROUP_TOK = 256;   // tokens per grouping block

struct Scan3 {
  int a, b, c;
};

// Exclusive scans of three values per thread over the first 256 threads of
// the block (threads past them, in larger blocks, pass 0 and get no
// result); *tot: the three totals.  Every thread of the block calls it.
__device__ Scan3 block_exclusive_scan256_x3(int a, int b, int c, int* tmp /* >= 12 ints of LDS */, Scan3* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ia = wave_incl_sum(a), ib = wave_incl_sum(b), ic = wave_incl_sum(c);
  if (lane == 63 && wave < 4) {
    tmp[wave] = ia;
    tmp[4 + wave] = ib;
    tmp[8 + wave] = ic;
  }
  __syncthreads();
  Scan3 base{0, 0, 0};
  for (int i = 0; i < wave && i < 4; ++i) {
    base.a += tmp[i];
    base.b += tmp[4 + i];
    base.c += tmp[8 + i];
  }
  tot->a = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  tot->b = tmp[4] + tmp[5] + tmp[6] + tmp[7];
  tot->c = tmp[8] + tmp[9] + tmp[10] + tmp[11];
  __syncthreads();
  return Scan3{base.a + ia - a, base.b + ib - b, base.c + ic - c};
}

// What the grouping needs of expert e = threadIdx.x besides its count: the
// miss-mask word holding its bit (0 without a mask) and its slot (0 without
// a table: grouping only).  Loaded at a kernel's start, so the loads overlap
// the work before the count is known.
struct ExpertMeta {
  uint32_t mword;
  int slot;
};

DEV ExpertMeta expert_meta(int E, const uint32_t* miss_mask, const int32_t* slot_row) {
  const int e = threadIdx.x;
  ExpertMeta m{0u, 0};
  if (e < E) {
    if (miss_mask) m.mword = miss_mask[e >> 5];
    if (slot_row) m.slot = slot_row[e];
  }
  return m;
}

// From per-expert counts (thread e holds counts[e]), write offsets, the list
// of experts that run on the GPU (routed, not in the host miss mask) with
// their slots and m-block prefix.  A routed, unmasked expert without a slot
// raises the device error flag and is skipped.  Returns thread e's offset
// (the first grouped row of expert e); *gslot (may be null): its slot if it
// runs on the GPU, else -1.
__device__ int finish_grouping(int cnt, int E, ExpertMeta em, int32_t* counts, int32_t* offsets, WorkList* wl,
                               int mb, int* err, int* tmp /* >= 12 ints of LDS */, const TailSplit& ts,
                               int* gslot = nullptr) {
  const int e = threadIdx.x;
  const int c = e < E ? cnt : 0;
  bool act = false;
  int slot = -1;
  if (e < E && c > 0) {
    const bool masked = (em.mword >> (e & 31)) & 1u;
    if (!masked) {
      slot = em.slot;
      if (slot < 0) atomicOr(err, 1);
      else act = true;
    }
  }
  int nb = act ? (c + mb - 1) / mb : 0;
  Scan3 tot;
  // offsets, active-expert positions and m-block prefixes in one pass
  const Scan3 x = block_exclusive_scan256_x3(c, act ? 1 : 0, nb, tmp, &tot);
  const int off = x.a, a = x.b, nact = tot.b;
  int pb = x.c, nmblk = tot.c;
  // overflow rows of a last tile of at most tau rows go to the tail list
  // when that removes a round of the tiled grid and the tail items are few
  int tl = 0;
  if (ts.wl) {
    const bool cand = nb >= 2 && c - (nb - 1) * mb <= ts.tau;
    Scan3 t2;
    (void)block_exclusive_scan256_x3(cand ? 1 : 0, 0, 0, tmp, &t2);
    const int n0 = tot.c, ncand = t2.a;
    const long it0 = (long)n0 * ts.ntiles, it1 = (long)(n0 - ncand) * ts.ntiles;
    const bool split = ncand > 0 && (it1 + ts.n_cu - 1) / ts.n_cu < (it0 + ts.n_cu - 1) / ts.n_cu &&
                       (long)ncand * ts.ntiles * 4 <= ts.n_cu;
    if (split && cand) {
      --nb;
      tl = c - nb * mb;
    }
    const int tnb = tl > 0 ? (tl + ts.mb - 1) / ts.mb : 0;
    Scan3 t3;
    const Scan3 y = block_exclusive_scan256_x3(nb, tl > 0 ? 1 : 0, tnb, tmp, &t3);
    pb = y.a;
    nmblk = t3.a;
    const int ta = y.b, tpb = y.c, ntact = t3.b, tnm = t3.c;
    if (e < E) { ts.mcounts[e] = c - tl; ts.tcounts[e] = tl; ts.toffsets[e] = off + c - tl; }
    if (tl > 0) { ts.wl->act_e[ta] = e; ts.wl->act_slot[ta] = slot; ts.wl->mblk_prefix[ta] = tpb; }
    if (e == 0) {
      ts.wl->n_act = ntact; ts.wl->n_mblk = tnm; ts.wl->mb = ts.mb; ts.wl->mblk_prefix[ntact] = tnm;
    }
  }
  if (e < E) { counts[e] = c; offsets[e] = off; }
  if (e == 0) offsets[E] = tot.a;
  if (act) { wl->act_e[a] = e; wl->act_slot[a] = slot; wl->mblk_prefix[a] = pb; }
  if (e == 0) {
    wl->n_act = nact; wl->n_mblk = nmblk; wl->mb = mb; wl->mblk_prefix[nact] = nmblk;
  }
  if (gslot) *gslot = act ? slot : -1;
  return off;
}

// Stable scatter of one block of tokens given per-expert bases for the block.
// bits: LDS [E][8] words, token-major presence bits of the block.
__device__ void scatter_block(const int32_t* __restrict__ ids, int t0, int T, int k, int E,
                              const int* base /* per expert, may be LDS or global */, uint32_t* bits,
                              int32_t* __restrict__ pos, int32_t* __restrict__ perm_tok) {
  const int tl = threadIdx.x, t = t0 + tl;
  const int wi = tl >> 5;
  const uint32_t below = (1u << (tl & 31)) - 1u;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      int r = __popc(bits[e * 8 + wi] & below);
      for (int q = 0; q < wi; ++q) r += __popc(bits[e * 8 + q]);
      const int p = base[e] + r;
      pos[(size_t)t * k + j] = p;
      perm_tok[p] = t;
    }
  }
}

__device__ void mark_block(const int32_t* __restrict__ ids, int t0, int T, int k, int E, uint32_t* bits) {
  for (int i = threadIdx.x; i < E * 8; i += blockDim.x) bits[i] = 0u;
  __syncthreads();
  const int tl = threadIdx.x, t = t0 + tl;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      atomicOr(&bits[e * 8 + (tl >> 5)], 1u << (tl & 31));
    }
  __syncthreads();
}

// One block of T <= 256 tokens, one (token, choice) pair per thread and
// pass: presence bits (token t -> bit t & 31 of word t >> 5 of each of its
// experts' rows; bits is LDS [E][8] of which the first ceil(T / 32) words of
// a row are used) and the stable scatter that reads them.
DEV void mark_pairs(const int32_t* ids, int T, int k, int E, uint32_t* bits) {
  const int nw = (T + 31) >> 5;
  for (int i = threadIdx.x; i < E * nw; i += blockDim.x) bits[(i / nw) * 8 + i % nw] = 0u;
  __syncthreads();
  for (int p = threadIdx.x; p < T * k; p += blockDim.x) {
    const int t = p / k;
    atomicOr(&bits[ids[p] * 8 + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
}

DEV int count_pairs(const uint32_t* bits, int T, int E) {
  const int e = threadIdx.x, nw = (T + 31) >> 5;
  int c = 0;
  if (e < E)
    for (int q = 0; q < nw; ++q) c += __popc(bits[e * 8 + q]);
  return c;
}

// pslot (may be null): per pair, the slot its expert runs from on the GPU,
// -1 where it does not (host-run or without a slot); gslot: those per expert.
DEV void scatter_pairs(const int32_t* ids, int T, int k, const int* base, const uint32_t* bits,
                       int32_t* __restrict__ pos, int32_t* __restrict__ perm_tok, const int* gslot = nullptr,
                       int32_t* __restrict__ pslot = nullptr) {
  for (int p = threadIdx.x; p < T * k; p += blockDim.x) {
    const int t = p / k, e = ids[p], wi = t >> 5;
    int r = __popc(bits[e * 8 + wi] & ((1u << (t & 31)) - 1u));
    for (int q = 0; q < wi; ++q) r += __popc(bits[e * 8 + q]);
    const int d = base[e] + r;
    pos[p] = d;
    perm_tok[d] = t;
    if (pslot) pslot[p] = gslot[e];
  }
}

// T <= 256: histogram, scan, work list and scatter in one workgroup.
__global__ void __launch_bounds__(256)
group_single_kernel(const int32_t* __restrict__ ids, int T, int k, int E, const uint32_t* miss_mask,
                    const int32_t* slot_row, int mb, int32_t* counts, int32_t* offsets,
                    int32_t* __restrict__ pos, int32_t* __restrict__ perm_tok, WorkList* wl, int* err,
                    TailSplit ts) {
  __shared__ uint32_t bits[256 * 8];
  __shared__ int base[256];
  __shared__ int tmp[12];
  const ExpertMeta em = expert_meta(E, miss_mask, slot_row);
  mark_pairs(ids, T, k, E, bits);
  const int off = finish_grouping(count_pairs(bits, T, E), E, em, counts, offsets, wl, mb, err, tmp, ts);
  if ((int)threadIdx.x < E) base[threadIdx.x] = off;
  __syncthreads();
  scatter_pairs(ids, T, k, base, bits, pos, perm_tok);
}

// T <= 16: top-k of every token (wave t takes token t) and the grouping of
// group_single_kernel in one launch; the assignments pass through LDS.
constexpr int TG_MAX_T = 16;

// The grouping of T <= 256 tokens whose k choices each sit in LDS (s_ids,
// written before a barrier), by the first 256 threads of the workgroup.
DEV void group_from_lds(const int32_t* s_ids, int T, int k, int E, ExpertMeta em, int mb, int32_t* counts,
                        int32_t* offsets, int32_t* __restrict__ pos, int32_t* __restrict__ perm_tok, WorkList* wl,
                        int* err, int32_t* pslot, uint32_t* bits, int* base, int* gslot, int* tmp) {
  const TailSplit ts{nullptr, nullptr, nullptr, nullptr, 1, 0};
  mark_pairs(s_ids, T, k, E, bits);
  int gs;
  const int off = finish_grouping(count_pairs(bits, T, E), E, em, counts, offsets, wl, mb, err, tmp, ts, &gs);
  if ((int)threadIdx.x < E) {
    base[threadIdx.x] = off;
    gslot[threadIdx.x] = gs;
  }
  __syncthreads();
  scatter_pairs(s_ids, T, k, base, bits, pos, perm_tok, gslot, pslot);
}

__global__ void __launch_bounds__(1024)
topk_group_kernel(const float* __restrict__ z, int T, int E, int k, int32_t* __restrict__ ids,
                  float* __restrict__ w, const uint32_t* miss_mask, const int32_t* slot_row, int mb,
                  int32_t* counts, int32_t* offsets, int32_t* __restrict__ pos, int32_t* __restrict__ perm_tok,
                  WorkList* wl, int* err, int32_t* pslot) {
  __shared__ uint32_t bits[256 * 8];
  __shared__ int base[256];
  __shared__ int gslot[256];
  __shared__ int tmp[12];
  __shared__ int32_t s_ids[TG_MAX_T * 8];
  __shared__ TopkScratch sc[TG_MAX_T];
  const int wave = threadIdx.x >> 6;
  if (T * k <= 64) {               // one wave groups the at most 64 pairs
    WaveMeta wm{};
    if (wave == 0) wm = wave_meta(E, miss_mask, slot_row);
    if (wave < T)
      topk_row(z + (size_t)wave * E, E, k, ids + (size_t)wave * k, w + (size_t)wave * k, s_ids + wave * k,
               sc + wave);
    __syncthreads();
    if (wave == 0)
      group_wave(s_ids, T, k, E, wm, mb, counts, offsets, pos, perm_tok, wl, err, pslot, bits, base, gslot);
    return;
  }
  const ExpertMeta em = expert_meta(E, miss_mask, slot_row);
  if (wave < T)
    topk_row(z + (size_t)wave * E, E, k, ids + (size_t)wave * k, w + (size_t)wave * k, s_ids + wave * k,
             sc + wave);
  __syncthreads();
  group_from_lds(s_ids, T, k, E, em, mb, counts, offsets, pos, perm_tok, wl, err, pslot, bits, base, gslot, tmp);
}

// General path, pass 1: per-block histograms hist[b][e].
__global__ void __launch_bounds__(256)
group_count_kernel(const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ hist) {
  __shared__ uint32_t bits[256 * 8];
  const int t0 = blockIdx.x * GROUP_TOK;
  mark_block(ids, t0, T, k, E, bits);
  if ((int)threadIdx.x < E) {
    int c = 0;
    for (int q = 0; q < 8; ++q) c += __popc(bits[threadIdx.x * 8 + q]);
    hist[(size_t)blockIdx.x * E + threadIdx.x] = c;
  }
}

// General path, pass 2: counts, offsets, work list; hist[b][e] becomes the
// block's base row for expert e.
__global__ void __launch_bounds__(256)
group_scan_kernel(int nblk, int E, const uint32_t* miss_mask, const int32_t* slot_row, int mb,
                  int32_t* __restrict__ hist, int32_t* counts, int32_t* offsets, WorkList* wl, int* err,
                  TailSplit ts) {
  __shared__ int tmp[12];
  const int e = threadIdx.x;
  const ExpertMeta em = expert_meta(E, miss_mask, slot_row);
  int cnt = 0;
  if (e < E)
    for (int b = 0; b < nblk; ++b) cnt += hist[(size_t)b * E + e];
  const int off = finish_grouping(cnt, E, em, counts, offsets, wl, mb, err, tmp, ts);
  if (e < E) {
    int run = off;
    for (int b = 0; b < nblk; ++b) {
      const int h = hist[(size_t)b * E + e];
      hist[(size_t)b * E + e] = run;
      run += h;
    }
  }
}

// General path, pass 3: stable scatter per block.
__global__ void __launch_bounds__(256)
group_scatter_kernel(const int32_t* __restrict__ ids, int T, int k, int E, const int32_t* __restrict__ hist,
                     int32_t* __restrict__ pos, int32_t* __restrict__ perm_tok) {
  __shared__ uint32_t bits[256 * 8];
  const int t0 = blockIdx.x * GROUP_TOK;
  mark_block(ids, t0, T, k, E, bits);
  scatter_block(ids, t0, T, k, E, hist + (size_t)blockIdx.x * E, bits, pos, perm_tok);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
extern "C" hipError_t moe_launch_router(const uint16_t* x, const float* R, const float* bias, int T, int E, int H,
                                        float* z, hipStream_t s) {
  if (T <= 64) {
    // up to 8 tokens one wave per workgroup, the expert rows spread over E
    // CUs (at T=1 3.2 us per launch against 3.8 with four waves per
    // workgroup on E/4 CUs; at 64 tokens no faster)
    const int wpb = T <= 8 ? 1 : 4;
    router_small_kernel<<<dim3((E + wpb - 1) / wpb, (T + RT_TOK - 1) / RT_TOK), 64 * wpb, 0, s>>>(x, R, bias, T, E,
                                                                                                H, z);
  } else {
    dim3 g((T + 63) / 64, (E + 63) / 64);
    router_mfma_kernel<<<g, 256, 0, s>>>(x, R, bias, T, E, H, z);
  }
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_topk(const float* z, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  // one wave (token) per workgroup
  topk_kernel<<<T, 64, 0, s>>>(z, T, E, k, ids, w);
  return hipGetLastError();
}

// Top-k and grouping in one launch for T <= 16 (same outputs as
// moe_launch_topk followed by moe_launch_group).
// pslot (may be null): [T * k], per (token, choice) the slot its expert runs
// from on the GPU, -1 where it does not.
extern "C" hipError_t moe_launch_topk_group(const float* z, int T, int E, int k, int32_t* ids, float* w,
                                            const uint32_t* miss_mask, const int32_t* slot_row, int mb,
                                            int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* perm_tok,
                                            WorkList* wl, int* err, int32_t* pslot, hipStream_t s) {
  if (T < 1 || T > TG_MAX_T || E > 256 || k > 8) return hipErrorInvalidValue;
  // one wave per token, at least the four waves the grouping needs (fewer
  // waves make its barriers cheaper)
  topk_group_kernel<<<1, 64 * (T < 4 ? 4 : T), 0, s>>>(z, T, E, k, ids, w, miss_mask, slot_row, mb, counts, offsets,
                                                       pos, perm_tok, wl, err, pslot);
  return hipGetLastError();
}

// tail: optional split of the large-batch work (TailSplit); nullptr: none.
extern "C" hipError_t moe_launch_group(const int32_t* ids, int T, int k, int E, const uint32_t* miss_mask,
                                       const int32_t* slot_row, int mb, int32_t* counts, int32_t* offsets,
                                       int32_t* pos, int32_t* perm_tok, int32_t* hist, WorkList* wl, int* err,
                                       const TailSplit* tail, hipStream_t s) {
  const TailSplit ts = tail ? *tail : TailSplit{nullptr, nullptr, nullptr, nullptr, 1, 0};
  if (T <= GROUP_TOK) {
    group_single_kernel<<<1, 256, 0, s>>>(ids, T, k, E, miss_mask, slot_row, mb, counts, offsets, pos, perm_tok,
                                          wl, err, ts);
  } else {
    const int nblk = (T + GROUP_TOK - 1) / GROUP_TOK;
    group_count_kernel<<<nblk, 256, 0, s>>>(ids, T, k, E, hist);
    group_scan_kernel<<<1, 256, 0, s>>>(nblk, E, miss_mask, slot_row, mb, hist, counts, offsets, wl, err, ts);
    group_scatter_kernel<<<nblk, 256, 0, s>>>(ids, T, k, E, hist, pos, perm_tok);
  }
  return hipGetLastError();
}
