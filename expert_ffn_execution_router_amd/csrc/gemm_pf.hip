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
//   * 4 waves in a 2x2 grid, each computing 128 weight rows x 64 tokens with
//     v_mfma_f32_16x16x32_bf16 (weights as the A operand, tokens as B);
//   * K advances in chunks of 64; the next chunk's global loads are issued
//     into registers before the current chunk's MFMAs and stored into the
//     other LDS stage afterwards (two stages, one barrier per chunk);
//   * LDS rows are 128 bytes; their eight 16-byte pieces are XOR-swizzled by
//     (row mod 8) so the MFMA operand reads of 16 consecutive rows spread
//     over the banks;
//   * the grid is persistent and walks the device work list, so the host
//     never reads the routing.
#include "common.h"

namespace {

constexpr int PF_BM = 128;    // tokens per tile
constexpr int PF_BN = 256;    // weight rows per tile
constexpr int PF_BK = 64;     // K per chunk
constexpr int PF_ROWB = PF_BK * 2;                    // bytes per LDS row (128)
constexpr int PF_STAGE = (PF_BM + PF_BN) * PF_ROWB;    // 48 KiB per stage

DEV int swz(int row, int piece) { return row * PF_ROWB + ((piece ^ (row & 7)) << 4); }

struct PfItem {
  int e, slot, row0, nrows, n0;
};

DEV void pf_decode(const WorkList* wl, const int32_t* counts, const int32_t* offsets, int ntiles, int it,
                   PfItem& o) {
  const int p = it / ntiles, nt = it - p * ntiles;
  const int a = find_active(wl, p);
  o.e = wl->act_e[a];
  o.slot = wl->act_slot[a];
  const int mb = p - wl->mblk_prefix[a];
  o.row0 = offsets[o.e] + mb * PF_BM;
  o.nrows = min(PF_BM, counts[o.e] - mb * PF_BM);
  o.n0 = nt;
}

}  // namespace

// GATED: out = A (bf16 [rows, N]) with N = I features, weights gate at woff0
// and up at woff1 ([N, K] each).  Otherwise out = Z (bf16 [rows, N]) with
// weights at woff0 ([N, K]).
template <bool GATED>
__global__ void __launch_bounds__(256, 1)
gemm_pf_bf16(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts,
             const int32_t* __restrict__ offsets, const uint8_t* __restrict__ pool, size_t S, size_t woff0,
             size_t woff1, const uint16_t* __restrict__ X, const int32_t* __restrict__ row_tok, int K, int N,
             uint16_t* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave & 1;        // token half (64 tokens)
  const int wn = wave >> 1;       // weight-row half (128 rows)
  // features per item: GATED covers 128 features (256 rows), else 256 rows
  const int feat_per_item = GATED ? PF_BN / 2 : PF_BN;
  const int ntiles = N / feat_per_item;
  const int nitems = wl->n_mblk * ntiles;
  const int nchunk = K / PF_BK;
  // global -> LDS assignment: thread loads 16-byte piece (tid & 7) of rows
  // (tid >> 3) + 32 * j
  const int gp = tid & 7, gr = tid >> 3;

  for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
    PfItem t;
    pf_decode(wl, counts, offsets, ntiles, it, t);
    const int f0 = t.n0 * feat_per_item;
    const uint8_t* wbase = pool + (size_t)t.slot * S;
    // source pointers of the rows this thread stages
    const uint16_t* xsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = gr + 32 * j;
      const int rr = min(r, t.nrows - 1);                      // clamp the ragged tail (masked at store)
      const int src = row_tok ? row_tok[t.row0 + rr] : t.row0 + rr;
      xsrc[j] = X + (size_t)src * K + gp * 8;
    }
    const uint16_t* wsrc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = gr + 32 * j;                               // tile row 0..255
      int wrow;
      const uint16_t* mat;
      if (GATED) {
        const int half = r >> 7, q = r & 127;                  // half = wave column
        const bool up = q >= 64;
        wrow = f0 + half * 64 + (q & 63);
        mat = (const uint16_t*)(wbase + (up ? woff1 : woff0));
      } else {
        wrow = f0 + r;
        mat = (const uint16_t*)(wbase + woff0);
      }
      wsrc[j] = mat + (size_t)wrow * K + gp * 8;
    }
    i32x4_t stg[12];
    auto gload = [&](int c) {
      const int kb = c * PF_BK;
#pragma unroll
      for (int j = 0; j < 4; ++j) stg[j] = ld16(xsrc[j] + kb);
#pragma unroll
      for (int j = 0; j < 8; ++j) stg[4 + j] = ld16(wsrc[j] + kb);
    };
    auto sstore = [&](int stage) {
      uint8_t* base = lds + stage * PF_STAGE;
#pragma unroll
      for (int j = 0; j < 4; ++j) *(i32x4_t*)(base + swz(gr + 32 * j, gp)) = stg[j];
#pragma unroll
      for (int j = 0; j < 8; ++j) *(i32x4_t*)(base + PF_BM * PF_ROWB + swz(gr + 32 * j, gp)) = stg[4 + j];
    };

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    gload(0);
    sstore(0);
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
      const int stage = c & 1;
      if (c + 1 < nchunk) gload(c + 1);
      const uint8_t* xs = lds + stage * PF_STAGE;
      const uint8_t* ws = xs + PF_BM * PF_ROWB;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int piece = ks * 4 + lg;
        bf16x8_t bx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bx[j] = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(xs + swz(wm * 64 + j * 16 + lr, piece)));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bf16x8_t aw =
              __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(ws + swz(wn * 128 + i * 16 + lr, piece)));
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bx[j], acc[i][j], 0, 0, 0);
        }
      }
      if (c + 1 < nchunk) sstore(stage ^ 1);
      __syncthreads();
    }

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
          const int f = f0 + wn * 64 + i * 16 + lg * 4;
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
          const int f = f0 + wn * 128 + i * 16 + lg * 4;
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16_bits(acc[i][j][0]) | ((uint32_t)f32_to_bf16_bits(acc[i][j][1]) << 16);
          pk.y = (uint32_t)f32_to_bf16_bits(acc[i][j][2]) | ((uint32_t)f32_to_bf16_bits(acc[i][j][3]) << 16);
          st8(orow + f, pk);
        }
      }
    }
  }
}

extern "C" size_t moe_pf_lds_bytes() { return 2 * PF_STAGE; }
extern "C" int moe_pf_tile_tokens() { return PF_BM; }

extern "C" hipError_t moe_launch_gemm_pf(int fmt, int gated, int grid, const WorkList* wl, const int32_t* counts,
                                         const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0,
                                         size_t woff1, const void* X, const int32_t* row_tok, int K, int N, void* out,
                                         hipStream_t s) {
  if (fmt != WFMT_BF16) return hipErrorInvalidValue;
  const size_t lds = 2 * PF_STAGE;
  if (gated)
    gemm_pf_bf16<true><<<grid, 256, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X, row_tok,
                                              K, N, (uint16_t*)out);
  else
    gemm_pf_bf16<false><<<grid, 256, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X,
                                               row_tok, K, N, (uint16_t*)out);
  return hipGetLastError();
}
