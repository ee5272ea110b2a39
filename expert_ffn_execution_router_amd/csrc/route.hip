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
#include "common.h"

// ---------------------------------------------------------------------------
// router logits z[t,e] = sum_h x[t,h] R[e,h] + b[e]  (x bf16, R fp32, fp32 sums)
// ---------------------------------------------------------------------------

// Small batches: one wave per (expert, 4 tokens), grid (E/4, T/4) so that
// every CU takes part.  A lane covers 4 consecutive elements of each
// 256-element chunk of H and issues the loads of 8 chunks (2048 elements) at
// once, so a wave waits for memory once per 2048 elements instead of once
// per chunk.  Loads and sums are unconditional (token rows past T re-read
// row T-1 and are not stored; chunks past H re-read the last one and are
// weighted by zero), so no branch splits the batch.  H % 256 == 0.
constexpr int RT_TOK = 4;
__global__ void __launch_bounds__(256)
router_small_kernel(const uint16_t* __restrict__ x, const float* __restrict__ R,
                    const float* __restrict__ bias, int T, int E, int H, float* __restrict__ z) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  const int t0 = blockIdx.y * RT_TOK;
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
// One wave per token (E <= 256: lane l holds experts l, l+64, l+128, l+192).
// Selection works on an order-preserving 32-bit key of each logit (-0 taken
// as +0, so equal logits have equal keys): the k-th largest key is found by
// bisection on its bits with wave ballots (no data crosses lanes), the k
// winners are the keys above it plus the lowest-numbered experts at it, and
// each winner's output position is its rank among the winners (descending
// logit, ties to the lower expert id).  The gate weights are the softmax of
// the winners, summed in output order.
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ z, int T, int E, int k, int32_t* __restrict__ ids,
            float* __restrict__ w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* zr = z + (size_t)t * E;
  const uint64_t below = (1ull << lane) - 1ull;
  float v[4];
  uint32_t key[4];
  bool valid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    valid[i] = e < E;
    const float x = zr[min(e, E - 1)];           // unconditional load; entries past E are not valid
    v[i] = x == 0.0f ? 0.0f : x;
    const uint32_t u = __float_as_uint(v[i]);
    key[i] = (u >> 31) ? ~u : (u | 0x80000000u);
  }
  // the k-th largest key
  uint32_t kth = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = kth | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt += __popcll(__ballot(valid[i] && key[i] >= cand));
    if (cnt >= k) kth = cand;
  }
  // winners: keys above kth, then the lowest-numbered experts at kth
  int n_gt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) n_gt += __popcll(__ballot(valid[i] && key[i] > kth));
  const int need = k - n_gt;
  bool sel[4];
  int eq_before = 0;                            // experts at kth with a lower id (slots before i, then lanes)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool eq = valid[i] && key[i] == kth;
    const uint64_t m = __ballot(eq);
    sel[i] = (valid[i] && key[i] > kth) || (eq && eq_before + __popcll(m & below) < need);
    eq_before += __popcll(m);
  }
  // rank of each winner among the winners
  int rank[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i2 = 0; i2 < 4; ++i2) {
    uint64_t m = __ballot(sel[i2]);
    while (m) {
      const int L = __builtin_ctzll(m);
      m &= m - 1;
      const uint32_t uk = (uint32_t)__builtin_amdgcn_readlane((int)key[i2], L);   // winner (L, i2)
      const int ue = L + 64 * i2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        rank[i] += (sel[i] && (uk > key[i] || (uk == key[i] && ue < e))) ? 1 : 0;
      }
    }
  }
  // softmax over the winners in output order (the first is the largest)
  float top = 0.0f, ssum = 0.0f;
  for (int j = 0; j < k; ++j) {
    float vj = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t m = __ballot(sel[i] && rank[i] == j);
      if (m) vj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), __builtin_ctzll(m)));
    }
    if (j == 0) top = vj;
    ssum += expf(vj - top);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (sel[i]) {
      ids[(size_t)t * k + rank[i]] = lane + 64 * i;
      w[(size_t)t * k + rank[i]] = expf(v[i] - top) / ssum;
    }
  }
}

// ---------------------------------------------------------------------------
// grouping: histogram -> exclusive scan -> stable scatter
// ---------------------------------------------------------------------------
constexpr int GROUP_TOK = 256;   // tokens per grouping block

// Exclusive scan of one value per thread over a 256-thread block.
__device__ int block_exclusive_scan256(int v, int* tmp /* >= 4 ints of LDS */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wave; ++i) base += tmp[i];
  *total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return base + incl - v;
}

// From per-expert counts (thread e holds counts[e]), write offsets, the list
// of experts that run on the GPU (routed, not in the host miss mask) with
// their slots and m-block prefix.  A routed, unmasked expert without a slot
// raises the device error flag and is skipped.
__device__ void finish_grouping(int cnt, int E, const uint32_t* miss_mask, const int32_t* slot_row,
                                int32_t* counts, int32_t* offsets, WorkList* wl, int mb, int* err,
                                int* tmp, const TailSplit& ts) {
  const int e = threadIdx.x;
  const int c = e < E ? cnt : 0;
  int total;
  const int off = block_exclusive_scan256(c, tmp, &total);
  if (e < E) { counts[e] = c; offsets[e] = off; }
  if (e == 0) offsets[E] = total;
  bool act = false;
  int slot = -1;
  if (e < E && c > 0) {
    const bool masked = miss_mask && ((miss_mask[e >> 5] >> (e & 31)) & 1u);
    if (!masked) {
      slot = slot_row ? slot_row[e] : 0;     // no table: grouping only
      if (slot < 0) atomicOr(err, 1);
      else act = true;
    }
  }
  int nact;
  const int a = block_exclusive_scan256(act ? 1 : 0, tmp, &nact);
  int nb = act ? (c + mb - 1) / mb : 0;
  // overflow rows of a last tile of at most tau rows go to the tail list
  // when that removes a round of the tiled grid and the tail items are few
  int tl = 0;
  if (ts.wl) {
    const bool cand = nb >= 2 && c - (nb - 1) * mb <= ts.tau;
    int n0, ncand;
    (void)block_exclusive_scan256(nb, tmp, &n0);
    (void)block_exclusive_scan256(cand ? 1 : 0, tmp, &ncand);
    const long it0 = (long)n0 * ts.ntiles, it1 = (long)(n0 - ncand) * ts.ntiles;
    const bool split = ncand > 0 && (it1 + ts.n_cu - 1) / ts.n_cu < (it0 + ts.n_cu - 1) / ts.n_cu &&
                       (long)ncand * ts.ntiles * 4 <= ts.n_cu;
    if (split && cand) {
      --nb;
      tl = c - nb * mb;
    }
  }
  int nmblk;
  const int pb = block_exclusive_scan256(nb, tmp, &nmblk);
  if (act) { wl->act_e[a] = e; wl->act_slot[a] = slot; wl->mblk_prefix[a] = pb; }
  if (e == 0) {
    wl->n_act = nact; wl->n_mblk = nmblk; wl->mb = mb; wl->mblk_prefix[nact] = nmblk;
  }
  if (ts.wl) {
    if (e < E) { ts.mcounts[e] = c - tl; ts.tcounts[e] = tl; ts.toffsets[e] = off + c - tl; }
    int ntact;
    const int ta = block_exclusive_scan256(tl > 0 ? 1 : 0, tmp, &ntact);
    const int tnb = tl > 0 ? (tl + ts.mb - 1) / ts.mb : 0;
    int tnm;
    const int tpb = block_exclusive_scan256(tnb, tmp, &tnm);
    if (tl > 0) { ts.wl->act_e[ta] = e; ts.wl->act_slot[ta] = slot; ts.wl->mblk_prefix[ta] = tpb; }
    if (e == 0) {
      ts.wl->n_act = ntact; ts.wl->n_mblk = tnm; ts.wl->mb = ts.mb; ts.wl->mblk_prefix[ntact] = tnm;
    }
  }
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

// T <= 256: histogram, scan, work list and scatter in one workgroup.
__global__ void __launch_bounds__(256)
group_single_kernel(const int32_t* __restrict__ ids, int T, int k, int E, const uint32_t* miss_mask,
                    const int32_t* slot_row, int mb, int32_t* counts, int32_t* offsets,
                    int32_t* __restrict__ pos, int32_t* __restrict__ perm_tok, WorkList* wl, int* err,
                    TailSplit ts) {
  __shared__ uint32_t bits[256 * 8];
  __shared__ int base[256];
  __shared__ int tmp[4];
  mark_block(ids, 0, T, k, E, bits);
  int cnt = 0;
  if ((int)threadIdx.x < E)
    for (int q = 0; q < 8; ++q) cnt += __popc(bits[threadIdx.x * 8 + q]);
  finish_grouping(cnt, E, miss_mask, slot_row, counts, offsets, wl, mb, err, tmp, ts);
  if ((int)threadIdx.x < E) base[threadIdx.x] = offsets[threadIdx.x];
  __syncthreads();
  scatter_block(ids, 0, T, k, E, base, bits, pos, perm_tok);
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
  __shared__ int tmp[4];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E)
    for (int b = 0; b < nblk; ++b) cnt += hist[(size_t)b * E + e];
  finish_grouping(cnt, E, miss_mask, slot_row, counts, offsets, wl, mb, err, tmp, ts);
  if (e < E) {
    int run = offsets[e];
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
    router_small_kernel<<<dim3((E + 3) / 4, (T + RT_TOK - 1) / RT_TOK), 256, 0, s>>>(x, R, bias, T, E, H, z);
  } else {
    dim3 g((T + 63) / 64, (E + 63) / 64);
    router_mfma_kernel<<<g, 256, 0, s>>>(x, R, bias, T, E, H, z);
  }
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_topk(const float* z, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(z, T, E, k, ids, w);
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
