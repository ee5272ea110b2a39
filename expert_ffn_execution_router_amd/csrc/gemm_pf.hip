// Slot-indexed grouped expert GEMMs for large token counts per expert
// (prefill-shaped batches), bf16 weights, fp32 accumulation on MFMA.
//
// Same computation as the small-batch kernels (paper.oopus.info review of
// FreeToken, section 2.5: grouped evaluation of every expert of G for the
// tokens routed to it; SwiGLU expert), but here each expert sees hundreds of
// tokens, so the contraction is MFMA-bound and both operands are reused
// through LDS:
//   * work item = (expert, 256-token m-tile, 256 weight rows); for GEMM 1 the
//     256 rows are 128 gate and 128 up rows of the same 128 features,
//     arranged so that each wave holds gate and up of the same 32 features;
//   * items are ordered expert, then weight tile, then m-tile (the m-tiles
//     sharing a weight tile are neighbours); each XCD (workgroup b runs on
//     XCD b mod 8) takes one eighth of the list and deals it round-robin to
//     its workgroups, so at any time an XCD's CUs work on neighbouring items
//     and share their weight and token tiles in its L2;
//   * one workgroup of 8 waves per CU (two per SIMD, so one wave's LDS waits
//     are covered by the other's MFMAs), in a 2 (tokens) x 4 (weight rows)
//     grid, each computing 64 weight rows x 128 tokens with
//     v_mfma_f32_16x16x32_bf16 (weights as the A operand, tokens as B): 64
//     MFMAs per 64-deep K chunk, 128 accumulators per lane;
//   * K advances in chunks of 64 through two 64 KiB LDS stages filled by
//     direct global->LDS loads (global_load_lds_dwordx4: lane l's 16 bytes
//     land at the instruction's LDS base + 16*l), chunk c+1 in flight while
//     chunk c is multiplied; the stream runs on across item boundaries, so an
//     item's first chunk was requested during the previous item.  Each chunk
//     costs one counter wait and one barrier (everyone's loads have landed,
//     and everyone is done with the stage about to be refilled).  A row
//     segment is 128 bytes (one cache line), which moves twice the bytes per
//     L2 request of a 32-deep chunk;
//   * LDS rows are 128 bytes; their eight 16-byte pieces are XOR-swizzled by
//     ((row / 2) mod 8), so the operand reads of 16 consecutive rows cover all
//     64 banks; the loads pick their source piece so that this layout comes
//     out of the lane-linear placement;
//   * padding rows of a ragged m-tile are loaded clamped to a real row (every
//     chunk issues the same number of loads) and their results are not
//     stored; a wave whose 128-token half holds no routed token skips its
//     MFMAs;
//   * the grid is persistent over the device work list, so the host never
//     reads the routing.
#include "common.h"

namespace {

constexpr int PF_BM = 256;    // tokens per tile
constexpr int PF_BN = 256;    // weight rows per tile
constexpr int PF_BK = 64;     // K per chunk
constexpr int PF_ROWB = PF_BK * 2;                    // bytes per LDS row (128)
constexpr int PF_STAGE = (PF_BM + PF_BN) * PF_ROWB;    // 64 KiB per stage
constexpr int PF_NSTAGE = 2;
constexpr int PF_WAVES = 8;
constexpr int PF_LOADS = (PF_BM + PF_BN) / 8 / PF_WAVES;    // 1 KiB loads of 8 rows per wave per chunk (8)
constexpr int N_XCD = 8;

// byte offset of (row, 16-byte piece) in a stage
DEV int swz(int row, int piece) { return row * PF_ROWB + ((piece ^ ((row >> 1) & 7)) << 4); }

struct PfItem {
  int slot, row0, nrows, f0;
};

}  // namespace

// GATED: out = A (bf16 [rows, N]) with N = I features, weights gate at woff0
// and up at woff1 ([N, K] each).  Otherwise out = Z (bf16 [rows, N]) with
// weights at woff0 ([N, K]).  X rows are gathered through row_tok (GEMM 1) or
// taken in grouped order.  K % 64 == 0; N % 128 (gated) or 256 (not gated).
template <bool GATED>
__global__ void __launch_bounds__(64 * PF_WAVES, 1)
gemm_pf_bf16(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts,
             const int32_t* __restrict__ offsets, const uint8_t* __restrict__ pool, size_t S, size_t woff0,
             size_t woff1, const uint16_t* __restrict__ X, const int32_t* __restrict__ row_tok, int K, int N,
             uint16_t* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int l_pref[257], l_slot[256], l_row0[256], l_cnt[256];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave & 1;        // token half (128 tokens)
  const int wn = wave >> 1;       // weight-row quarter (64 rows)

  const int n_act = wl->n_act;
  for (int i = tid; i <= n_act; i += blockDim.x) {
    l_pref[i] = wl->mblk_prefix[i];
    if (i < n_act) {
      const int e = wl->act_e[i];
      l_slot[i] = wl->act_slot[i];
      l_row0[i] = offsets[e];
      l_cnt[i] = counts[e];
    }
  }
  __syncthreads();

  const int feat = GATED ? PF_BN / 2 : PF_BN;   // output features per item
  const int ntiles = N / feat;
  const int nitems = wl->n_mblk * ntiles;
  const int nchunk = K / PF_BK;
  if (nitems == 0) return;
  // XCD x (workgroups b with b % 8 == x) takes the x-th eighth of the item
  // list and deals it round-robin to its workgroups, so the workgroups of an
  // XCD work on neighbouring items (sharing weight and token tiles in its L2)
  // at the same time
  const int xcd = blockIdx.x % N_XCD, wpx = (gridDim.x + N_XCD - 1 - xcd) / N_XCD, w = blockIdx.x / N_XCD;
  const int xb = (int)((long)xcd * nitems / N_XCD), xe = (int)((long)(xcd + 1) * nitems / N_XCD);
  if (xb + w >= xe) return;
  const int it0 = xb + w, istep = wpx;
  const int my_items = (xe - it0 + istep - 1) / istep;
  const long n_units = (long)my_items * nchunk;

  // item it: m-blocks of active expert a are contiguous in the work list;
  // order inside an expert: weight tile nt, then m-tile mt
  auto decode = [&](int it, PfItem& o) {
    const int p = it / ntiles;                 // some m-block of the expert (any works for the search)
    int a = 0, hi = n_act - 1;
    while (a < hi) {
      const int mid = (a + hi + 1) >> 1;
      if (l_pref[mid] <= p) a = mid; else hi = mid - 1;
    }
    const int pre = l_pref[a], nm = l_pref[a + 1] - pre;
    const int q = it - pre * ntiles;
    const int nt = q / nm, mt = q - nt * nm;
    o.slot = __builtin_amdgcn_readfirstlane(l_slot[a]);
    o.row0 = __builtin_amdgcn_readfirstlane(l_row0[a] + mt * PF_BM);
    o.nrows = __builtin_amdgcn_readfirstlane(min(PF_BM, l_cnt[a] - mt * PF_BM));
    o.f0 = __builtin_amdgcn_readfirstlane(nt * feat);
  };

  // ---- loads: this wave's 8 blocks of 8 stage rows ------------------------
  // stage rows 0..255 are tokens, 256..511 weights; block q of the wave
  // covers rows (8*wave + q)*8 ..+7; lane l writes row r = 8*(8*wave + q) +
  // l/8, physical piece (l&7), so it fetches logical piece (l&7) ^ ((r/2)&7),
  // where (r/2)&7 = 4*(q&1) + (l/8)/2 (waves 0-3 load token rows, waves 4-7
  // weight rows; byte offsets from a uniform base: X, or the slot's blob)
  const int brow = lane >> 3;
  const int bpiece = (lane & 7) ^ (brow >> 1);           // even q; odd q: bpiece ^ 4
  const bool wtok = wave < PF_WAVES / 2;
  uint32_t src[PF_LOADS];
  const uint8_t* sbase = (const uint8_t*)X;
  auto set_sources = [&](const PfItem& t) {
    sbase = wtok ? (const uint8_t*)X : pool + (size_t)t.slot * S;
#pragma unroll
    for (int q = 0; q < PF_LOADS; ++q) {
      const int r = (wave * PF_LOADS + q) * 8 + brow;
      if (wtok) {
        const int rr = min(r, t.nrows - 1);                       // ragged tail: clamped, masked at store
        int xrow = t.row0 + rr;
        if (row_tok) {
          // the block's 8 entries by scalar loads (they do not count on the
          // vector-memory counter the stream waits on), then a per-lane pick;
          // entries past the expert's rows are read but not used (the
          // workspace continues after the permutation)
          const int r0 = (wave * PF_LOADS + q) * 8;
          const int* rp = row_tok + __builtin_amdgcn_readfirstlane(t.row0 + r0);
          int v = __builtin_amdgcn_readfirstlane(row_tok[__builtin_amdgcn_readfirstlane(t.row0 + t.nrows - 1)]);
#pragma unroll
          for (int k2 = 0; k2 < 8; ++k2) {
            const int e = __builtin_amdgcn_readfirstlane(rp[k2]);   // uniform: a scalar load
            v = (brow == k2 && r0 + k2 < t.nrows) ? e : v;
          }
          xrow = v;
        }
        src[q] = (uint32_t)xrow * (uint32_t)(K * 2) + (bpiece ^ ((q & 1) << 2)) * 16;
      } else {
        const int wr = r - PF_BM;                                 // weight tile row 0..255
        if (GATED) {
          // tile rows [64*h + 32*g + j]: h = weight quarter (wave column),
          // g = 0 gate / 1 up, feature f0 + 32*h + j
          const int h = wr >> 6, g = (wr >> 5) & 1, j = wr & 31;
          src[q] = (uint32_t)((g ? woff1 : woff0) + (size_t)(t.f0 + h * 32 + j) * K * 2) +
                   (bpiece ^ ((q & 1) << 2)) * 16;
        } else {
          src[q] = (uint32_t)(woff0 + (size_t)(t.f0 + wr) * K * 2) + (bpiece ^ ((q & 1) << 2)) * 16;
        }
      }
    }
  };
  // issue side: next unit (item iss_it, chunk iss_c)
  int iss_it = it0, iss_c = 0;
  {
    PfItem t;
    decode(iss_it, t);
    set_sources(t);
  }
  auto issue = [&](int stage) {
    if (iss_c == nchunk) {
      iss_c = 0;
      iss_it += istep;
      PfItem t;
      decode(iss_it, t);
      set_sources(t);
    }
    const uint8_t* base = sbase + iss_c * (PF_BK * 2);
    ++iss_c;
#pragma unroll
    for (int q = 0; q < PF_LOADS; ++q)
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(base + src[q]),
                                       (lds_void_t*)((lds_u8_t*)lds + stage * PF_STAGE +
                                                     (wave * PF_LOADS + q) * 1024),
                                       16, 0, 0);
  };

  // operand read offsets inside a stage (K steps 0 and 1 of the chunk): the
  // swizzle of row 16*j + lr depends on lr only, so sub-tile j is a constant
  // 2 KiB step
  const int xoff[2] = {swz(wm * 128 + lr, lg), swz(wm * 128 + lr, 4 + lg)};
  const int woff[2] = {swz(PF_BM + wn * 64 + lr, lg), swz(PF_BM + wn * 64 + lr, 4 + lg)};

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // epilogue: lane holds weight rows 4*lg..+3 of each 16-row sub-tile i for
  // token column lr of each 16-token sub-tile j
  auto store_item = [&](const PfItem& t) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = wm * 128 + j * 16 + lr;
      if (r >= t.nrows) continue;
      uint16_t* orow = out + (size_t)(t.row0 + r) * N;
      if (GATED) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int f = t.f0 + wn * 32 + i * 16 + lg * 4;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = acc[i][j][q], u = acc[2 + i][j][q];
            v[q] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;   // rounded to bf16 below
          }
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          st8(orow + f, pk);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = t.f0 + wn * 64 + i * 16 + lg * 4;
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          st8(orow + f, pk);
        }
      }
    }
  };

  // ---- the stream ----------------------------------------------------------
  // A finished item is stored at the start of the next iteration, ahead of
  // that iteration's loads.  Stores share the memory counter with the loads
  // and may complete before loads issued earlier, so a counter wait is only
  // trusted when the operations it leaves outstanding are all loads issued
  // after everything it must cover; with two stages every wait is vmcnt(0).
#pragma unroll
  for (int s = 0; s < PF_NSTAGE - 1; ++s)
    if (s < n_units) issue(s);
  PfItem ct;
  decode(it0, ct);
  PfItem done{};
  bool pending = false;
  int c = 0, stage = 0;
  for (long v = 0; v < n_units; ++v) {
    wait_vmcnt<0>();                            // this wave's loads of unit v have landed
    barrier_keep_loads();                       // everyone's have; the other stage is free
    if (pending) {
      store_item(done);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pending = false;
    }
    if (v + PF_NSTAGE - 1 < n_units) issue(stage == 0 ? PF_NSTAGE - 1 : stage - 1);
    const uint8_t* cur = lds + stage * PF_STAGE;
    if (ct.nrows > wm * 128) {                  // this wave's token half holds a routed token
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t bx[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bx[j] = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(cur + xoff[ks] + j * 2048));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8_t aw = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(cur + woff[ks] + i * 2048));
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bx[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    stage = stage + 1 == PF_NSTAGE ? 0 : stage + 1;
    if (++c == nchunk) {
      done = ct;
      pending = true;
      c = 0;
      if (v + 1 < n_units) decode(it0 + (int)((v + 1) / nchunk) * istep, ct);
    }
  }
  if (pending) store_item(done);
}

extern "C" size_t moe_pf_lds_bytes() { return PF_NSTAGE * PF_STAGE; }
extern "C" int moe_pf_tile_tokens() { return PF_BM; }

// n_cu: CUs (one workgroup each).
extern "C" hipError_t moe_launch_gemm_pf(int fmt, int gated, int n_cu, const WorkList* wl, const int32_t* counts,
                                         const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0,
                                         size_t woff1, const void* X, const int32_t* row_tok, int K, int N, void* out,
                                         hipStream_t s) {
  const int grid = n_cu;
  if (fmt != WFMT_BF16 || K % PF_BK || N % (gated ? PF_BN / 2 : PF_BN)) return hipErrorInvalidValue;
  const size_t lds = PF_NSTAGE * PF_STAGE;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_pf_bf16<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gemm_pf_bf16<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  if (gated)
    gemm_pf_bf16<true><<<grid, 64 * PF_WAVES, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X, row_tok,
                                              K, N, (uint16_t*)out);
  else
    gemm_pf_bf16<false><<<grid, 64 * PF_WAVES, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X,
                                               row_tok, K, N, (uint16_t*)out);
  return hipGetLastError();
}
