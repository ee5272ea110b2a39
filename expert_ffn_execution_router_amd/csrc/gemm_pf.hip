// Slot-indexed grouped expert GEMMs for large token counts per expert
// (prefill-shaped batches), bf16 weights, fp32 accumulation on MFMA.
//
// Same computation as the small-batch kernels (paper.oopus.info review of
// FreeToken, section 2.5: grouped evaluation of every expert of G for the
// tokens routed to it; SwiGLU expert), but here each expert sees hundreds of
// tokens, so the contraction is MFMA-bound and both operands are reused
// through LDS:
//   * work item = (expert, 128-token m-tile, 256 weight rows); for GEMM 1 the
//     256 rows are 128 gate and 128 up rows of the same 128 features,
//     interleaved in blocks of 64 so that each wave holds gate and up of the
//     same features;
//   * items are ordered expert, then weight tile, then m-tile, and each of
//     the 8 XCDs takes one contiguous eighth of them (workgroup b runs on
//     XCD b mod 8), so the workgroups sharing a weight tile or a token tile
//     share that XCD's L2;
//   * 4 waves in a 2x2 grid, each computing 128 weight rows x 64 tokens with
//     v_mfma_f32_16x16x32_bf16 (weights as the A operand, tokens as B);
//   * K advances in chunks of 32 through a ring of three 24 KiB LDS stages
//     filled by direct global->LDS loads (global_load_lds_dwordx4: lane l's
//     16 bytes land at the instruction's LDS base + 16*l), so no registers
//     stage the tiles; chunk c+2 is requested while chunk c is multiplied,
//     and each chunk costs one counter wait (this wave's loads of chunk c
//     have landed) and one barrier (everyone's have, and everyone is done
//     with the stage about to be refilled); two workgroups share a CU;
//   * LDS rows are 64 bytes; their four 16-byte pieces are XOR-swizzled by
//     ((row / 2) mod 4) so the operand reads of 16 consecutive rows spread
//     over all banks; the loads pick their source piece so that this layout
//     comes out of the lane-linear placement;
//   * the grid is persistent over the device work list, so the host never
//     reads the routing.
#include "common.h"

namespace {

constexpr int PF_BM = 128;    // tokens per tile
constexpr int PF_BN = 256;    // weight rows per tile
constexpr int PF_BK = 32;     // K per chunk
constexpr int PF_ROWB = PF_BK * 2;                    // bytes per LDS row (64)
constexpr int PF_STAGE = (PF_BM + PF_BN) * PF_ROWB;    // 24 KiB per stage
constexpr int PF_NSTAGE = 3;
constexpr int PF_BLOCKS = (PF_BM + PF_BN) / 16;       // 1 KiB blocks of 16 rows per stage (24)
constexpr int PF_BLK_PER_WAVE = PF_BLOCKS / 4;         // 6
constexpr int N_XCD = 8;
constexpr int PF_WG_PER_CU = 2;

DEV int swz(int row, int piece) { return row * PF_ROWB + ((piece ^ ((row >> 1) & 3)) << 4); }

struct PfItem {
  int slot, row0, nrows, f0;
};

// Item order: expert a, then weight tile nt, then m-tile mt.
DEV void pf_decode(const WorkList* wl, const int32_t* counts, const int32_t* offsets, int ntiles, int feat, int it,
                   PfItem& o) {
  const int a = find_active(wl, it / ntiles);
  const int pre = wl->mblk_prefix[a], nm = wl->mblk_prefix[a + 1] - pre;
  const int q = it - pre * ntiles;
  const int nt = q / nm, mt = q - nt * nm;
  const int e = wl->act_e[a];
  o.slot = wl->act_slot[a];
  o.row0 = offsets[e] + mt * PF_BM;
  o.nrows = min(PF_BM, counts[e] - mt * PF_BM);
  o.f0 = nt * feat;
}

}  // namespace

// GATED: out = A (bf16 [rows, N]) with N = I features, weights gate at woff0
// and up at woff1 ([N, K] each).  Otherwise out = Z (bf16 [rows, N]) with
// weights at woff0 ([N, K]).  gridDim.x must be a multiple of 8.
template <bool GATED>
__global__ void __launch_bounds__(256, 2)
gemm_pf_bf16(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts,
             const int32_t* __restrict__ offsets, const uint8_t* __restrict__ pool, size_t S, size_t woff0,
             size_t woff1, const uint16_t* __restrict__ X, const int32_t* __restrict__ row_tok, int K, int N,
             uint16_t* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave & 1;        // token half (64 tokens)
  const int wn = wave >> 1;       // weight-row half (128 rows)
  const int feat = GATED ? PF_BN / 2 : PF_BN;   // output features per item
  const int ntiles = N / feat;
  const int nitems = wl->n_mblk * ntiles;
  const int nchunk = K / PF_BK;
  // XCD-contiguous item ranges
  const int xcd = blockIdx.x % N_XCD, wg_in_xcd = blockIdx.x / N_XCD, wg_per_xcd = gridDim.x / N_XCD;
  const int per_xcd = (nitems + N_XCD - 1) / N_XCD;
  const int it_end = min(nitems, (xcd + 1) * per_xcd);
  // operand read offsets inside a stage (fixed per lane)
  int xoff[4], woff[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) xoff[j] = swz(wm * 64 + j * 16 + lr, lg);
#pragma unroll
  for (int i = 0; i < 8; ++i) woff[i] = PF_BM * PF_ROWB + swz(wn * 128 + i * 16 + lr, lg);
  // direct-load placement: lane l of a block writes row (l/4), physical piece
  // (l&3); it therefore fetches logical piece (l&3) ^ ((l/8)&3) of that row
  const int brow = lane >> 2;
  const int bpiece = (lane & 3) ^ ((lane >> 3) & 3);
  lds_void_t* lds_as = (lds_void_t*)lds;

  for (int it = xcd * per_xcd + wg_in_xcd; it < it_end; it += wg_per_xcd) {
    PfItem t;
    pf_decode(wl, counts, offsets, ntiles, feat, it, t);
    const uint8_t* wbase = pool + (size_t)t.slot * S;
    // source of each of this wave's blocks (tile rows 16*b .. 16*b+15)
    const uint16_t* src[PF_BLK_PER_WAVE];
#pragma unroll
    for (int q = 0; q < PF_BLK_PER_WAVE; ++q) {
      const int b = wave * PF_BLK_PER_WAVE + q;
      const int r = b * 16 + brow;                                // stage row (tokens first)
      if (r < PF_BM) {
        const int rr = min(r, t.nrows - 1);                       // ragged tail: clamped, masked at store
        const int xrow = row_tok ? row_tok[t.row0 + rr] : t.row0 + rr;
        src[q] = X + (size_t)xrow * K + bpiece * 8;
      } else {
        const int wr = r - PF_BM;                                 // weight tile row 0..255
        int wrow;
        const uint16_t* mat;
        if (GATED) {
          const int half = wr >> 7, q2 = wr & 127;
          wrow = t.f0 + half * 64 + (q2 & 63);
          mat = (const uint16_t*)(wbase + (q2 >= 64 ? woff1 : woff0));
        } else {
          wrow = t.f0 + wr;
          mat = (const uint16_t*)(wbase + woff0);
        }
        src[q] = mat + (size_t)wrow * K + bpiece * 8;
      }
    }
    auto issue = [&](int c, int stage) {     // this wave's 6 block loads of chunk c
      const int kb = min(c, nchunk - 1) * PF_BK;
#pragma unroll
      for (int q = 0; q < PF_BLK_PER_WAVE; ++q) {
        const int b = wave * PF_BLK_PER_WAVE + q;
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(src[q] + kb),
                                         (lds_void_t*)((uint8_t __attribute__((address_space(3)))*)lds_as +
                                                       stage * PF_STAGE + b * 1024),
                                         16, 0, 0);
      }
    };

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    issue(1, 1);
    int stage = 0;
    for (int c = 0; c < nchunk; ++c) {
      wait_vmcnt<PF_BLK_PER_WAVE>();           // this wave's loads of chunk c have landed
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // no compiler motion of LDS accesses across
      __builtin_amdgcn_s_barrier();            // everyone's have; stage (c+2)%3 is free
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      int s2 = stage + 2;
      if (s2 >= PF_NSTAGE) s2 -= PF_NSTAGE;
      issue(c + 2, s2);                        // past the end: clamped re-read, never used
      const uint8_t* cur = lds + stage * PF_STAGE;
      bf16x8_t bx[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bx[j] = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(cur + xoff[j]));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8_t aw = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(cur + woff[i]));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bx[j], acc[i][j], 0, 0, 0);
      }
      stage = stage + 1 == PF_NSTAGE ? 0 : stage + 1;
    }
    wait_vmcnt<0>();                           // drain the two spare loads
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();              // nobody reads the ring any more
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    // epilogue: lane holds weight rows 4*lg..+3 of each 16-row sub-tile i for
    // token column lr of each 16-token sub-tile j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wm * 64 + j * 16 + lr;
      if (r >= t.nrows) continue;
      uint16_t* orow = out + (size_t)(t.row0 + r) * N;
      if (GATED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = t.f0 + wn * 64 + i * 16 + lg * 4;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = acc[i][j][q], u = acc[4 + i][j][q];
            v[q] = g / (1.0f + expf(-g)) * u;
          }
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
          st8(orow + f, pk);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int f = t.f0 + wn * 128 + i * 16 + lg * 4;
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16_bits(acc[i][j][0]) | ((uint32_t)f32_to_bf16_bits(acc[i][j][1]) << 16);
          pk.y = (uint32_t)f32_to_bf16_bits(acc[i][j][2]) | ((uint32_t)f32_to_bf16_bits(acc[i][j][3]) << 16);
          st8(orow + f, pk);
        }
      }
    }
    wait_vmcnt<0>();                           // stores done before the next item's counted loads
  }
}

extern "C" size_t moe_pf_lds_bytes() { return PF_NSTAGE * PF_STAGE; }
extern "C" int moe_pf_tile_tokens() { return PF_BM; }

// n_cu: CUs (the launcher runs PF_WG_PER_CU workgroups per CU).
extern "C" hipError_t moe_launch_gemm_pf(int fmt, int gated, int n_cu, const WorkList* wl, const int32_t* counts,
                                         const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0,
                                         size_t woff1, const void* X, const int32_t* row_tok, int K, int N, void* out,
                                         hipStream_t s) {
  const int grid = n_cu * PF_WG_PER_CU;
  if (fmt != WFMT_BF16 || grid % N_XCD) return hipErrorInvalidValue;
  const size_t lds = PF_NSTAGE * PF_STAGE;
  if (gated)
    gemm_pf_bf16<true><<<grid, 256, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X, row_tok,
                                              K, N, (uint16_t*)out);
  else
    gemm_pf_bf16<false><<<grid, 256, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X,
                                               row_tok, K, N, (uint16_t*)out);
  return hipGetLastError();
}
