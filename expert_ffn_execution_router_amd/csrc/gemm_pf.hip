// Slot-indexed grouped expert GEMMs for large token counts per expert
// (prefill-shaped batches), bf16 weights, fp32 accumulation on MFMA.
//
// Same computation as the small-batch kernels (paper.oopus.info review of
// FreeToken, section 2.5: grouped evaluation of every expert of G for the
// tokens routed to it; SwiGLU expert), but here each expert sees hundreds of
// tokens, so the contraction is MFMA-bound and both operands are reused
// through LDS:
//   * work item = (expert, m-tile of up to 288 tokens, 256 weight rows); an
//     expert's c tokens are cut into ceil(c/288) m-tiles of equal size (the
//     weight tiles are streamed once per m-tile, so fewer, fuller m-tiles
//     mean fewer bytes: c = 540 gives two tiles of 270, not 256+256+28); for
//     GEMM 1 the 256 rows are 128 gate and 128 up rows of the same 128
//     features, arranged so that each wave holds gate and up of the same 32
//     features;
//   * items are ordered expert, then weight tile, then m-tile (the m-tiles
//     sharing a weight tile are neighbours); each XCD (workgroup b runs on
//     XCD b mod 8) takes one eighth of the list and deals it round-robin to
//     its workgroups, so at any time an XCD's CUs work on neighbouring items
//     and share their weight and token tiles in its L2;
//   * one workgroup of 8 waves per CU (two per SIMD, so one wave's LDS waits
//     are covered by the other's MFMAs), in a 2 (tokens) x 4 (weight rows)
//     grid, each computing 64 weight rows x 144 tokens with
//     v_mfma_f32_16x16x32_bf16 (weights as the A operand, tokens as B): 72
//     MFMAs per 64-deep K chunk, 144 accumulators per lane;
//   * K advances in chunks of 64 through two 68 KiB LDS stages filled by
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
//   * 8-row blocks of an m-tile that hold no routed token are not loaded
//     (their stale LDS rows only feed result columns that are not stored),
//     padding rows of a partly filled block are loaded clamped to a real row,
//     and a wave whose 144-token half holds no routed token skips its MFMAs;
//   * the grid is persistent over the device work list, so the host never
//     reads the routing.
// NVFP4 experts (E2M1 codes, an E4M3 scale per 16 inputs of a row, an fp32
// scale per matrix) run through the same kernel with fp16 tokens (the hidden
// rows converted to fp16 once per call; A written in fp16): a chunk's weight
// rows are 32 bytes of codes and 4 scale bytes, loaded as they are stored
// (9 KiB a chunk against 32 KiB of bf16 weights), and each wave dequantises
// its operand in registers, element times block scale, exact in fp16 (a
// scaled fp4 -> fp16 pair conversion and a packed fp16 multiply per two
// weights), for v_mfma_f32_16x16x32_f16; the matrix scales multiply the
// fp32 sums in the epilogue (gate and up before SwiGLU, down on Z).  The
// weight operand's 16-byte halves are swapped on rows 8-15 of every 16, so
// the 64 lanes' dword reads of 16 rows hit 64 distinct banks.
#include "common.h"

namespace {

constexpr int PF_BM = 288;    // most tokens per tile (two halves of 144)
constexpr int PF_HALF = PF_BM / 2;
constexpr int PF_SUB = PF_HALF / 16;                  // 16-token sub-tiles per half (9)
constexpr int PF_BN = 256;    // weight rows per tile
constexpr int PF_BK = 64;     // K per chunk
constexpr int PF_ROWB = PF_BK * 2;                    // bytes per LDS row (128)
constexpr int PF_STAGE = (PF_BM + PF_BN) * PF_ROWB;    // 68 KiB per stage
// NVFP4 stage: token rows as above, then 32 code bytes and 4 scale bytes per weight row
constexpr int PF_NV_CODEB = PF_BK / 2;                 // 32
constexpr int PF_NV_CODE_OFF = PF_BM * PF_ROWB;        // 36 KiB
constexpr int PF_NV_SC_OFF = PF_NV_CODE_OFF + PF_BN * PF_NV_CODEB;
constexpr int PF_NV_STAGE = PF_NV_SC_OFF + PF_BN * 4;  // 45 KiB
constexpr int PF_NSTAGE = 2;
constexpr int PF_WAVES = 8;
constexpr int PF_TLOADS = PF_BM / 8 / (PF_WAVES / 2);   // 8-row token blocks per loading wave (9)
constexpr int PF_WLOADS = PF_BN / 8 / (PF_WAVES / 2);   // 8-row weight blocks per loading wave (8)
constexpr int PF_LOADS = PF_TLOADS > PF_WLOADS ? PF_TLOADS : PF_WLOADS;
constexpr int N_XCD = 8;

// byte offset of (row, 16-byte piece) in a stage
DEV int swz(int row, int piece) { return row * PF_ROWB + ((piece ^ ((row >> 1) & 7)) << 4); }

typedef __attribute__((address_space(4))) float cst_f32_t;   // constant memory: scalar loads

struct PfItem {
  int slot, row0, nrows, f0;
};

}  // namespace

// GATED: out = A ([rows, N], bf16; NVFP4: fp16) with N = I features,
// weights gate at woff0 and up at woff1 ([N, K] each).  Otherwise out = Z
// (bf16 [rows, N]) with weights at woff0 ([N, K]).  NV: the weights are
// NVFP4 codes ([N, K/2] bytes) with their E4M3 block scales at soff0 /
// soff1 ([N, K/16] bytes) and the three matrices' fp32 scales after the
// block scales; X is fp16.  X rows are gathered through row_tok (GEMM 1) or
// taken in grouped order.  K % 64 == 0; N % 128 (gated) or 256 (not gated).
// row_tok is read in 8-entry blocks up to 287 entries past a tile's first
// row, so it must hold 288 entries of slack after the last routed row.
template <bool GATED, bool NV>
__global__ void __launch_bounds__(64 * PF_WAVES, 1)
gemm_pf16(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
          const uint8_t* __restrict__ pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
          const uint16_t* __restrict__ X, const int32_t* __restrict__ row_tok, int K, int N,
          uint16_t* __restrict__ out) {
  constexpr int STG = NV ? PF_NV_STAGE : PF_STAGE;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int l_pref[257], l_slot[256], l_row0[256], l_cnt[256];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave & 1;        // token half (144 tokens)
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
    // nm = ceil(c / 288) tiles of ts = ceil(c / nm) <= 288 tokens; the last
    // one is not empty, since (nm - 1) * ts < c while c / nm > nm
    const int c = l_cnt[a], ts = (c + nm - 1) / nm;
    o.slot = __builtin_amdgcn_readfirstlane(l_slot[a]);
    o.row0 = __builtin_amdgcn_readfirstlane(l_row0[a] + mt * ts);
    o.nrows = __builtin_amdgcn_readfirstlane(min(ts, c - mt * ts));
    o.f0 = __builtin_amdgcn_readfirstlane(nt * feat);
  };

  // ---- loads: blocks of 8 stage rows, 1 KiB each ----------------------------
  // stage rows 0..287 are tokens, 288..543 weights.  Waves 0-3 load token
  // blocks 9*wave + q (q < 9), waves 4-7 weight blocks 8*(wave-4) + q (q < 8).
  // Lane l writes row (l/8) of its block, physical piece (l&7), so it fetches
  // logical piece (l&7) ^ ((row/2)&7) of that row.  Byte offsets are 32-bit,
  // from a uniform base: X, or the slot's blob.
  const int brow = lane >> 3;
  const bool wtok = wave < PF_WAVES / 2;
  const int blk0 = wtok ? wave * PF_TLOADS : PF_BM / 8 + (wave - PF_WAVES / 2) * PF_WLOADS;
  uint32_t src[PF_LOADS];
  int tok_blocks = 0;                         // token blocks holding a routed token
  const uint8_t* sbase = (const uint8_t*)X;
  auto set_sources = [&](const PfItem& t) {
    sbase = wtok ? (const uint8_t*)X : pool + (size_t)t.slot * S;
    tok_blocks = (t.nrows + 7) >> 3;
#pragma unroll
    for (int q = 0; q < PF_LOADS; ++q) {
      const int srow = (blk0 + q) * 8 + brow;                     // stage row
      const int piece = (lane & 7) ^ ((srow >> 1) & 7);
      if (wtok) {
        const int r = srow;                                       // token row of the tile
        int xrow = t.row0 + min(r, t.nrows - 1);                  // padding: clamped, not stored
        if (row_tok) {
          // the block's 8 entries by scalar loads (they do not count on the
          // vector-memory counter the stream waits on), then a per-lane pick;
          // entries past the expert's rows are read but not used (the
          // workspace continues after the permutation)
          const int r0 = (blk0 + q) * 8;
          const int* rp = row_tok + __builtin_amdgcn_readfirstlane(t.row0 + r0);
          int v = __builtin_amdgcn_readfirstlane(row_tok[__builtin_amdgcn_readfirstlane(t.row0 + t.nrows - 1)]);
#pragma unroll
          for (int k2 = 0; k2 < 8; ++k2) {
            const int e = __builtin_amdgcn_readfirstlane(rp[k2]);   // uniform: a scalar load
            v = (brow == k2 && r0 + k2 < t.nrows) ? e : v;
          }
          xrow = v;
        }
        src[q] = (uint32_t)xrow * (uint32_t)(K * 2) + piece * 16;
      } else if (NV) {
        // q 0, 1: code rows 32 (2 (wave - 4) + q) + lane/2, 16-byte half
        // lane & 1, swapped on rows 8-15 of every 16; q 2: the scale dword
        // of row 64 (wave - 4) + lane
        const int wq = wave - PF_WAVES / 2;
        if (q < 3) {
          const int wr = q < 2 ? (2 * wq + q) * 32 + (lane >> 1) : 64 * wq + lane;
          size_t f, base;
          if (GATED) {
            const int h = wr >> 6, g = (wr >> 5) & 1, j = wr & 31;
            f = (size_t)(t.f0 + h * 32 + j);
            base = q < 2 ? (g ? woff1 : woff0) : (g ? soff1 : soff0);
          } else {
            f = (size_t)(t.f0 + wr);
            base = q < 2 ? woff0 : soff0;
          }
          src[q] = q < 2 ? (uint32_t)(base + f * (K / 2)) + (((lane & 1) ^ ((wr >> 3) & 1)) << 4)
                         : (uint32_t)(base + f * (K / 16));
        }
      } else if (q < PF_WLOADS) {
        const int wr = srow - PF_BM;                              // weight tile row 0..255
        if (GATED) {
          // tile rows [64*h + 32*g + j]: h = weight quarter (wave column),
          // g = 0 gate / 1 up, feature f0 + 32*h + j
          const int h = wr >> 6, g = (wr >> 5) & 1, j = wr & 31;
          src[q] = (uint32_t)((g ? woff1 : woff0) + (size_t)(t.f0 + h * 32 + j) * K * 2) + piece * 16;
        } else {
          src[q] = (uint32_t)(woff0 + (size_t)(t.f0 + wr) * K * 2) + piece * 16;
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
    const int cc = iss_c++;
    const uint8_t* base = sbase + cc * (PF_BK * 2);
    lds_u8_t* dst = (lds_u8_t*)lds + stage * STG + blk0 * 1024;
    if (wtok) {
#pragma unroll
      for (int q = 0; q < PF_TLOADS; ++q)
        if (blk0 + q < tok_blocks)            // blocks past the tile's rows are skipped
          __builtin_amdgcn_global_load_lds((gbl_void_t*)(base + src[q]), (lds_void_t*)(dst + q * 1024), 16, 0, 0);
    } else if (NV) {
      const int wq = wave - PF_WAVES / 2;
      lds_u8_t* st = (lds_u8_t*)lds + stage * STG;
      const uint8_t* cb = sbase + cc * PF_NV_CODEB;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(cb + src[q]),
                                         (lds_void_t*)(st + PF_NV_CODE_OFF + (2 * wq + q) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void_t*)(sbase + cc * 4 + src[2]),
                                       (lds_void_t*)(st + PF_NV_SC_OFF + wq * 256), 4, 0, 0);
    } else {
#pragma unroll
      for (int q = 0; q < PF_WLOADS; ++q)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(base + src[q]), (lds_void_t*)(dst + q * 1024), 16, 0, 0);
    }
  };

  // operand read offsets inside a stage (K steps 0 and 1 of the chunk): the
  // swizzle of row 16*j + lr depends on lr only, so sub-tile j is a constant
  // 2 KiB step
  const int xoff[2] = {swz(wm * PF_HALF + lr, lg), swz(wm * PF_HALF + lr, 4 + lg)};
  const int woff[2] = {swz(PF_BM + wn * 64 + lr, lg), swz(PF_BM + wn * 64 + lr, 4 + lg)};

  f32x4_t acc[4][PF_SUB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < PF_SUB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // epilogue: lane holds weight rows 4*lg..+3 of each 16-row sub-tile i for
  // token column lr of each 16-token sub-tile j
  auto store_item = [&](const PfItem& t) {
    // NVFP4: the matrices' fp32 scales (gate and up, or down), after the
    // three matrices' codes and block scales
    // (scalar loads through the constant address space: a vector load here
    // would leave its destination registers pending across the loop, and
    // the wait for them would also wait for the next chunk's loads)
    float ts0 = 1.0f, ts1 = 1.0f;
    if (NV) {
      const size_t n = (size_t)K * N;
      const cst_f32_t* ts = (const cst_f32_t*)(pool + (size_t)t.slot * S + 3 * (n / 2) + 3 * (n / 16));
      ts0 = GATED ? ts[0] : ts[2];
      ts1 = GATED ? ts[1] : 1.0f;
    }
#pragma unroll
    for (int j = 0; j < PF_SUB; ++j) {
      const int r = wm * PF_HALF + j * 16 + lr;
      if (r >= t.nrows) continue;
      uint16_t* orow = out + (size_t)(t.row0 + r) * N;
      if (GATED) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int f = t.f0 + wn * 32 + i * 16 + lg * 4;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = acc[i][j][q] * ts0, u = acc[2 + i][j][q] * ts1;
            v[q] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;   // rounded to bf16 (fp16) below
          }
          uint2 pk;
          pk.x = NV ? pack_f16x2(v[0], v[1]) : pack_bf16x2(v[0], v[1]);
          pk.y = NV ? pack_f16x2(v[2], v[3]) : pack_bf16x2(v[2], v[3]);
          st8(orow + f, pk);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = t.f0 + wn * 64 + i * 16 + lg * 4;
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][0] * ts0, acc[i][j][1] * ts0);
          pk.y = pack_bf16x2(acc[i][j][2] * ts0, acc[i][j][3] * ts0);
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
        for (int j = 0; j < PF_SUB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pending = false;
    }
    if (v + PF_NSTAGE - 1 < n_units) issue(stage == 0 ? PF_NSTAGE - 1 : stage - 1);
    const uint8_t* cur = lds + stage * STG;
    if (NV && ct.nrows > wm * PF_HALF) {
      // the four scale bytes (16-input groups 0-3 of the chunk) of row lr of each sub-tile
      uint32_t scd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) scd[i] = *(const uint32_t*)(cur + PF_NV_SC_OFF + (wn * 64 + i * 16 + lr) * 4);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f16x8_t bx[PF_SUB], aw[4];
#pragma unroll
        for (int j = 0; j < PF_SUB; ++j)
          bx[j] = __builtin_bit_cast(f16x8_t, *(const i32x4_t*)(cur + xoff[ks] + j * 2048));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // lane (row lr, group lg): K [32 ks + 8 lg, +8) = code bytes 16 ks + 4 lg of the row, in group 2 ks + lg/2
          const uint32_t cw = *(const uint32_t*)(cur + PF_NV_CODE_OFF + (wn * 64 + i * 16 + lr) * PF_NV_CODEB +
                                                 ((ks ^ ((lr >> 3) & 1)) << 4) + 4 * lg);
          const int scb = (int)(scd[i] >> (8 * (2 * ks + (lg >> 1))));
          const _Float16 sh = (_Float16)__builtin_amdgcn_cvt_f32_fp8(scb, 0);   // E4M3 is exact in fp16
          const f16x2_t s2 = {sh, sh};
          i32x4_t w4;
          w4[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * s2);
          w4[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * s2);
          w4[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * s2);
          w4[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * s2);
          aw[i] = __builtin_bit_cast(f16x8_t, w4);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < PF_SUB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw[i], bx[j], acc[i][j], 0, 0, 0);
      }
    } else if (!NV && ct.nrows > wm * PF_HALF) {   // this wave's token half holds a routed token
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t bx[PF_SUB], aw[4];
#pragma unroll
        for (int j = 0; j < PF_SUB; ++j)
          bx[j] = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(cur + xoff[ks] + j * 2048));
#pragma unroll
        for (int i = 0; i < 4; ++i) aw[i] = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(cur + woff[ks] + i * 2048));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < PF_SUB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[i], bx[j], acc[i][j], 0, 0, 0);
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

extern "C" int moe_pf_tile_tokens() { return PF_BM; }

template <bool GATED, bool NV>
static hipError_t launch_pf16(int grid, const WorkList* wl, const int32_t* counts, const int32_t* offsets,
                              const uint8_t* pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                              const void* X, const int32_t* row_tok, int K, int N, void* out, hipStream_t s) {
  const size_t lds = PF_NSTAGE * (NV ? PF_NV_STAGE : PF_STAGE);
  static bool attr = false;
  if (!attr) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)gemm_pf16<GATED, NV>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  gemm_pf16<GATED, NV><<<grid, 64 * PF_WAVES, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                                         (const uint16_t*)X, row_tok, K, N, (uint16_t*)out);
  return hipGetLastError();
}

// fmt: WFMT_BF16 (X bf16, out bf16) or WFMT_NVFP4 (X fp16; GEMM 1 writes A
// in fp16, GEMM 2 Z in bf16); soff0 / soff1: NVFP4 block-scale offsets.
// n_cu: CUs (one workgroup each).
extern "C" hipError_t moe_launch_gemm_pf(int fmt, int gated, int n_cu, const WorkList* wl, const int32_t* counts,
                                         const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0,
                                         size_t woff1, size_t soff0, size_t soff1, const void* X,
                                         const int32_t* row_tok, int K, int N, void* out, hipStream_t s) {
  if ((fmt != WFMT_BF16 && fmt != WFMT_NVFP4) || K % PF_BK || N % (gated ? PF_BN / 2 : PF_BN))
    return hipErrorInvalidValue;
  if (fmt == WFMT_NVFP4)
    return gated ? launch_pf16<true, true>(n_cu, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X,
                                           row_tok, K, N, out, s)
                 : launch_pf16<false, true>(n_cu, wl, counts, offsets, pool, S, woff0, 0, soff0, 0, X, row_tok, K,
                                            N, out, s);
  return gated ? launch_pf16<true, false>(n_cu, wl, counts, offsets, pool, S, woff0, woff1, 0, 0, X, row_tok, K, N,
                                          out, s)
               : launch_pf16<false, false>(n_cu, wl, counts, offsets, pool, S, woff0, 0, 0, 0, X, row_tok, K, N, out,
                                           s);
}
