// Slot-indexed grouped expert GEMMs for large token counts per expert in the
// 8-bit weight formats: fp8 E4M3 weights with an fp32 scale per 128x128
// block and per-(token, 128 K) fp8 activations, or MXFP4 (E2M1 weights with
// an E8M0 scale per 32 K) with MXFP8 or MXFP6 (E2M3) activations.
//
// Same computation as the small-batch kernels (paper.oopus.info review of
// FreeToken, section 2.5: grouped evaluation of every expert of G for the
// tokens routed to it; SwiGLU expert), laid out like the bf16 large-batch
// kernel:
//   * work item = (expert, m-tile of up to BM tokens, 256 weight rows), BM =
//     256 (fp8) or 288 (MXFP4); an expert's c tokens are cut into ceil(c/BM)
//     equal m-tiles; GEMM 1's 256
//     rows are 128 gate and 128 up rows of the same 128 features (each wave
//     holds gate and up of the same 32 features); items ordered expert ->
//     weight tile -> m-tile, each XCD dealing its eighth of the list
//     round-robin to its workgroups;
//   * one workgroup of 8 waves per CU in a 2 (token halves of BM/2) x 4 (64
//     weight rows) grid; one K chunk is 128 deep (one scale block), moved
//     from global memory into one of two LDS stages by direct global->LDS
//     loads (lane l's bytes land at the instruction's LDS base + size*l):
//     token rows of 128 bytes, weight rows of 128 (fp8) or 64 (E2M1) bytes,
//     and the chunk's scales; one vmcnt(0) wait and one barrier per chunk;
//   * MFMA: v_mfma_scale_f32_16x16x128_f8f6f4, weights as A (16 rows), tokens
//     as B (16 per sub-tile).  fp8: unit E8M0 scales, the 16x16 partial sum
//     of the chunk multiplied by w_scale * x_scale and added to the
//     accumulator (the fp32 block scales are not powers of two).  MXFP4:
//     E2M1 x E4M3 with both operands' E8M0 block scales inside the
//     instruction, accumulated across chunks by the MFMA.  Lane layouts (as
//     measured for the small-batch kernels): an 8-bit operand with uniform
//     scales takes 32 consecutive K bytes per lane group g; an MX 8-bit
//     operand's lane group g holds K [16g, 16g+16) in bytes 0-15 and
//     K [64+16g, 64+16g+16) in bytes 16-31; an E2M1 operand's lane group g
//     holds K [32g, 32g+32) in its low 16 bytes; the E8M0 scale of lane group
//     g covers K block [32g, 32g+32) of that lane's row or column;
//   * LDS rows of 128 bytes have their 16-byte pieces XOR-swizzled by
//     ((row/2) mod 8), rows of 64 bytes by ((row/4) mod 4): 16 consecutive
//     rows read at one logical piece cover all 64 banks;
//   * token rows of a ragged m-tile: blocks past its rows are not loaded,
//     padding rows of a partly filled block are loaded clamped and not
//     stored (to a spare trash row), a wave whose token half is empty skips
//     its MFMAs;
//   * GEMM 1 stores silu(g)*u in fp32 (the next pass quantises it), GEMM 2
//     stores bf16;
//   * MXFP6 activations: the quantisation pass writes each 128-K chunk of
//     the grouped rows as one plane of 112-byte rows (96 bytes of codes), so
//     a tile's rows of a chunk are one contiguous range, moved in 1 KiB
//     blocks; at that stride 16 consecutive rows read at one offset are
//     bank-conflict free wherever the tile starts; the E2M3 operand of lane
//     group g is the 24 bytes of K [32g, 32g+32), one 16-byte and one 8-byte
//     aligned read (x6_off16, x6_off8), and E2M1 x E2M3 issues at the 6/4-bit
//     rate (1.7x the E2M1 x E4M3 rate, measured);
//   * E2M1 weights: the E8M0 scales are stored by row (K/32 bytes a row), so
//     one chunk's 4 bytes of each of 256 rows are 256 separate requests; the
//     weight waves load them 16 bytes a row (four chunks) at the first chunk
//     of each group of four into one of two group buffers outside the stage
//     ring (a group's buffer is reused two groups later, after the chunk
//     barriers), and only chunks past the last whole group of an item load
//     their 4 bytes with the chunk;
//   * few tokens per expert (a weight stream more than a GEMM): tiles of 128
//     tokens and three LDS stages, so two chunks are in flight while one is
//     multiplied; the wait before a chunk counts only loads (the ones this
//     wave issued for the next chunk; loads complete in order, so nothing
//     older can still be outstanding when that many remain), and a finished
//     item's stores go out before the next chunk's loads.
#include "common.h"

namespace {

constexpr int Q_BN = 256;                       // weight rows per tile
constexpr int Q_BK = 128;                       // K per chunk
constexpr int Q_WAVES = 8;
constexpr int N_XCD = 8;

// VAR 0: the largest tiles, two stages; 1: 128-token tiles, three stages
// (few tokens per expert).
template <int FMT, int VAR>
struct QCfg {
  static constexpr bool X6 = FMT == WFMT_MXFP4_A6;                // E2M3 token rows
  static constexpr bool W4 = FMT == WFMT_MXFP4 || X6;             // E2M1 weights, E8M0 scales
  // most tokens per tile: fp8 keeps 32-byte A operands and a scaled partial
  // sum per MFMA, so its tile is 256 tokens (128 accumulators) to stay within
  // 256 registers; MXFP4 takes 288 (144 accumulators)
  static constexpr int BM = VAR == 1 ? 128 : (W4 ? 288 : 256);
  static constexpr int NST = VAR ? 3 : 2;                         // LDS stages
  static constexpr int HALF = BM / 2;
  static constexpr int SUB = HALF / 16;                           // 16-token sub-tiles per half
  // token loads per token wave: 8-row blocks of 128-byte rows, or (E2M3) the
  // 1 KiB blocks of up to BM rows of X6_ROWB bytes
  static constexpr int X6_BLOCKS = (BM * X6_ROWB + 1023) / 1024;
  static constexpr int TLOADS = X6 ? (X6_BLOCKS + 3) / 4 : BM / 8 / (Q_WAVES / 2);
  static constexpr int NXS = (BM + 63) / 64;                      // 4-byte loads of 64 token-scale rows
  static constexpr int WROWB = W4 ? 64 : 128;                     // weight row bytes per chunk
  static constexpr int WRPB = 1024 / WROWB;                       // weight rows per 1 KiB load
  static constexpr int WLOADS = Q_BN / WRPB / (Q_WAVES / 2);      // weight loads per weight wave
  static constexpr int LOADS = TLOADS > WLOADS ? TLOADS : WLOADS;
  static constexpr int T_OFF = 0;
  static constexpr int W_OFF = X6 ? TLOADS * 4 * 1024 : BM * 128;
  static constexpr int XS_OFF = W_OFF + Q_BN * WROWB;
  static constexpr int XS_BYTES = NXS * 256;                      // row r's scale dword at XS_OFF + 4r
  static constexpr int WS_OFF = XS_OFF + XS_BYTES;
  static constexpr int WS_BYTES = W4 ? Q_BN * 4 : 256;
  static constexpr int STAGE = WS_OFF + WS_BYTES;
  // E2M1 weights: two group buffers of 16 scale bytes (four chunks) per row
  static constexpr int GB_BYTES = W4 ? 2 * Q_BN * 16 : 0;
  static constexpr int LDS = NST * STAGE + GB_BYTES;
};

struct QItem {
  int slot, row0, nrows, f0;
};

// offset of (row, 16-byte piece) inside a region of 128- or 64-byte rows
template <int ROWB>
DEV int qswz(int row, int piece) {
  return ROWB == 128 ? row * 128 + ((piece ^ ((row >> 1) & 7)) << 4) : row * 64 + ((piece ^ ((row >> 2) & 3)) << 4);
}

DEV i32x4_t lds16(const uint8_t* p) { return *(const i32x4_t*)p; }

DEV float silu_f(float g) { return g / (1.0f + expf(-g)); }

DEV void dma16(const void* src, lds_u8_t* dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}
DEV void dma4(const void* src, lds_u8_t* dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 4, 0, 0);
}

}  // namespace

// GATED: out = A (fp32 [rows, N], N = I features), weights gate at woff0 and
// up at woff1 ([N, K] codes), their scales at soff0 / soff1.  Otherwise out =
// Z (bf16 [rows, N]), weights at woff0, scales at soff0.  X: quantised rows
// in grouped order ([rows, K] E4M3 codes, or MXFP6 planes sized for xcap
// rows) with scales Xs (fp8: fp32 [rows, K/128]; MXFP4: E8M0 [rows, K/32];
// MXFP6: E8M0 planes [K/128][xcap][4]).  K % 128 == 0; N % 128 (gated) or
// 256 (not gated).  trash_row: a spare row of out for padding stores.
template <int FMT, bool GATED, int VAR>
__global__ void __launch_bounds__(64 * Q_WAVES, 1)
gemm_pf_q8(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts,
           const int32_t* __restrict__ offsets, const uint8_t* __restrict__ pool, size_t S, size_t woff0,
           size_t woff1, size_t soff0, size_t soff1, const uint8_t* __restrict__ X, const uint8_t* __restrict__ Xs,
           int xcap, int K, int N, void* __restrict__ out, int trash_row) {
  using C = QCfg<FMT, VAR>;
  static_assert(C::LDS + 4200 <= 160 * 1024, "LDS budget");
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int l_pref[257], l_slot[256], l_row0[256], l_cnt[256];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int wm = wave & 1;        // token half (BM/2 tokens)
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

  const int feat = GATED ? Q_BN / 2 : Q_BN;
  const int ntiles = N / feat;
  const int nitems = wl->n_mblk * ntiles;
  const int nchunk = K / Q_BK;
  if (nitems == 0) return;
  const int xcd = blockIdx.x % N_XCD, wpx = (gridDim.x + N_XCD - 1 - xcd) / N_XCD, w = blockIdx.x / N_XCD;
  const int xb = (int)((long)xcd * nitems / N_XCD), xe = (int)((long)(xcd + 1) * nitems / N_XCD);
  if (xb + w >= xe) return;
  const int it0 = xb + w, istep = wpx;
  const int my_items = (xe - it0 + istep - 1) / istep;
  const long n_units = (long)my_items * nchunk;

  auto decode = [&](int it, QItem& o) {
    const int p = it / ntiles;
    int a = 0, hi = n_act - 1;
    while (a < hi) {
      const int mid = (a + hi + 1) >> 1;
      if (l_pref[mid] <= p) a = mid; else hi = mid - 1;
    }
    const int pre = l_pref[a], nm = l_pref[a + 1] - pre;
    const int q = it - pre * ntiles;
    const int nt = q / nm, mt = q - nt * nm;
    const int c = l_cnt[a], ts = (c + nm - 1) / nm;   // nm = ceil(c/BM) tiles of ts <= BM
    o.slot = __builtin_amdgcn_readfirstlane(l_slot[a]);
    o.row0 = __builtin_amdgcn_readfirstlane(l_row0[a] + mt * ts);
    o.nrows = __builtin_amdgcn_readfirstlane(min(ts, c - mt * ts));
    o.f0 = __builtin_amdgcn_readfirstlane(nt * feat);
  };

  // ---- loads ------------------------------------------------------------------
  // Waves 0-3: token blocks TLOADS*wave + q (8 rows of 128 bytes), and the
  // token scales of rows 64n .. 64n+63 for n = wave, wave + 4 (< NXS).  Waves 4-7: weight
  // blocks (WRPB rows each) and the weight scales.  Lane l writes row l/8
  // (l/4 for 64-byte rows) of its block, physical piece l&7 (l&3), so it
  // fetches the logical piece that the row's swizzle puts there.
  const bool wtok = wave < Q_WAVES / 2;
  const int kb128 = K / 128, kb32 = K / 32;
  const int xrowb = K;                                    // bytes of a quantised token row
  const int wrowb = C::W4 ? K / 2 : K;                    // bytes of a weight row
  uint32_t src[C::LOADS];
  uint32_t xs_src[2];
  uint32_t ws_src = 0;
  int tok_blocks = 0;
  const uint8_t* wbase = pool;
  auto set_sources = [&](const QItem& t) __attribute__((always_inline)) {
    wbase = pool + (size_t)t.slot * S;
    tok_blocks = (t.nrows + 7) >> 3;
    if (wtok) {
      if (C::X6) {
        // rows row0 .. row0 + nrows - 1 of the chunk's plane, whole 1 KiB blocks
        tok_blocks = (t.nrows * X6_ROWB + 1023) >> 10;
#pragma unroll
        for (int q = 0; q < C::TLOADS; ++q)
          src[q] = (uint32_t)t.row0 * (uint32_t)X6_ROWB + (uint32_t)((wave * C::TLOADS + q) * 1024 + lane * 16);
      } else {
#pragma unroll
        for (int q = 0; q < C::TLOADS; ++q) {
          const int r = (wave * C::TLOADS + q) * 8 + (lane >> 3);
          const int piece = (lane & 7) ^ ((r >> 1) & 7);
          src[q] = (uint32_t)(t.row0 + min(r, t.nrows - 1)) * (uint32_t)xrowb + piece * 16;
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = min(64 * (wave + 4 * i) + lane, C::BM - 1);
        const uint32_t xr = (uint32_t)(t.row0 + min(r, t.nrows - 1));
        xs_src[i] = C::X6 ? xr * 4u : (C::W4 ? xr * (uint32_t)kb32 : xr * (uint32_t)kb128 * 4u);
      }
    } else {
      const int wv = wave - Q_WAVES / 2;
#pragma unroll
      for (int q = 0; q < C::WLOADS; ++q) {
        const int wr = (wv * C::WLOADS + q) * C::WRPB + lane / (64 / C::WRPB);   // weight tile row
        const int piece = C::W4 ? ((lane & 3) ^ ((wr >> 2) & 3)) : ((lane & 7) ^ ((wr >> 1) & 7));
        size_t off;
        if (GATED) {
          const int h = wr >> 6, g = (wr >> 5) & 1, j = wr & 31;
          off = (g ? woff1 : woff0) + (size_t)(t.f0 + h * 32 + j) * wrowb;
        } else {
          off = woff0 + (size_t)(t.f0 + wr) * wrowb;
        }
        src[q] = (uint32_t)off + piece * 16;
      }
      if (C::W4) {
        // E8M0 dword (4 blocks of 32) of weight tile row 64*wv + lane
        const int wr = 64 * wv + lane;
        size_t off;
        if (GATED) {
          const int h = wr >> 6, g = (wr >> 5) & 1, j = wr & 31;
          off = (g ? soff1 : soff0) + (size_t)(t.f0 + h * 32 + j) * kb32;
        } else {
          off = soff0 + (size_t)(t.f0 + wr) * kb32;
        }
        ws_src = (uint32_t)off;
      } else {
        // fp8: two block scales (gated: gate and up of feature block f0/128;
        // otherwise blocks f0/128 and f0/128 + 1), lanes 0 and 1
        const int h = lane & 1;
        const size_t off = GATED ? ((h ? soff1 : soff0) + (size_t)(t.f0 / 128) * kb128 * 4)
                                 : (soff0 + (size_t)(t.f0 / 128 + h) * kb128 * 4);
        ws_src = (uint32_t)off;
      }
    }
  };
  int iss_it = it0, iss_c = 0, iss_g = -1;
  lds_u8_t* const gb = (lds_u8_t*)lds + C::NST * C::STAGE;    // scale group buffers (E2M1 weights)
  {
    QItem t;
    decode(iss_it, t);
    set_sources(t);
  }
  // returns the number of loads this wave issued (uniform per wave)
  auto issue = [&](int stage) __attribute__((always_inline)) {
    if (iss_c == nchunk) {
      iss_c = 0;
      iss_it += istep;
      QItem t;
      decode(iss_it, t);
      set_sources(t);
    }
    const int kc = iss_c++;
    lds_u8_t* sb = (lds_u8_t*)lds + stage * C::STAGE;
    int n = 0;
    if (wtok) {
      const uint8_t* xb_ = C::X6 ? X + (size_t)kc * x6_plane_bytes(xcap) : X + kc * 128;
#pragma unroll
      for (int q = 0; q < C::TLOADS; ++q)
        if (wave * C::TLOADS + q < tok_blocks) {
          dma16(xb_ + src[q], sb + C::T_OFF + (wave * C::TLOADS + q) * 1024);
          ++n;
        }
      // fp32 scale kc, or E8M0 bytes 4kc..4kc+3 (MXFP6: scale plane kc)
      const uint8_t* xsb = C::X6 ? Xs + (size_t)kc * xcap * 4 : Xs + kc * 4;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (wave + 4 * i < C::NXS) {
          dma4(xsb + xs_src[i], sb + C::XS_OFF + (wave + 4 * i) * 256);
          ++n;
        }
    } else {
      const int wv = wave - Q_WAVES / 2;
      const uint8_t* wb_ = wbase + kc * C::WROWB;
#pragma unroll
      for (int q = 0; q < C::WLOADS; ++q) dma16(wb_ + src[q], sb + C::W_OFF + (wv * C::WLOADS + q) * 1024);
      n = C::WLOADS;
      if (C::W4) {
        if ((kc & ~3) + 4 <= nchunk) {                     // in a whole group of four chunks
          if ((kc & 3) == 0) {                             // its first: the group's 16 bytes a row
            ++iss_g;
            dma16(wbase + ws_src + kc * 4, gb + (iss_g & 1) * (Q_BN * 16) + wv * 1024);
            ++n;
          }
        } else {
          dma4(wbase + ws_src + kc * 4, sb + C::WS_OFF + wv * 256);
          ++n;
        }
      } else if (wv == 0) {
        dma4(wbase + ws_src + kc * 4, sb + C::WS_OFF);
        ++n;
      }
    }
    return n;
  };

  // ---- operand reads (bytes inside a stage) -----------------------------------
  // token sub-tile j: rows HALF*wm + 16j + lr; weight sub-tile i: rows 64*wn +
  // 16i + lr of the weight region; the swizzle of such a row depends on lr only
  const int trow = C::HALF * wm + lr, wrow = 64 * wn + lr;
  int x_rd[2], w_rd[2];
  if (C::W4) {
    x_rd[0] = C::T_OFF + qswz<128>(trow, lg);
    x_rd[1] = C::T_OFF + qswz<128>(trow, 4 + lg);
    w_rd[0] = C::W_OFF + qswz<64>(wrow, lg);
    w_rd[1] = 0;
  } else {
    x_rd[0] = C::T_OFF + qswz<128>(trow, 2 * lg);
    x_rd[1] = C::T_OFF + qswz<128>(trow, 2 * lg + 1);
    w_rd[0] = C::W_OFF + qswz<128>(wrow, 2 * lg);
    w_rd[1] = C::W_OFF + qswz<128>(wrow, 2 * lg + 1);
  }
  // LDS offset of the scale dword of token row r of the tile
  auto xs_at = [&](int r) { return C::XS_OFF + 4 * r; };

  f32x4_t acc[4][C::SUB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < C::SUB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // wsb / wss: the E2M1 weight scales of the chunk, row r's byte for lane
  // group g at wsb[r * wss + g]
  auto compute = [&](const uint8_t* sb, const uint8_t* wsb, int wss) __attribute__((always_inline)) {
    i32x8_t wa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x4_t lo = lds16(sb + w_rd[0] + i * 16 * C::WROWB);
      if (C::W4) {
        wa[i] = i32x8_t{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      } else {
        const i32x4_t hi = lds16(sb + w_rd[1] + i * 16 * C::WROWB);
        wa[i] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    }
    if (C::X6) {
      int wsc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wsc[i] = wsb[(wrow + 16 * i) * wss + lg];
      const uint8_t* rb = sb + C::T_OFF + trow * X6_ROWB;
      const int o16 = x6_off16(lg), o8 = x6_off8(lg);
#pragma unroll
      for (int j = 0; j < C::SUB; ++j) {
        const uint8_t* p = rb + j * 16 * X6_ROWB;
        const i32x4_t a = lds16(p + o16);
        // two dword reads, not one 8-byte read: the compiler cannot tell an
        // 8-byte LDS read from the stage the direct loads are filling and
        // puts a wait for every outstanding load (the next chunk's too)
        // before it
        const int b0 = *(const int*)(p + o8), b1 = *(const int*)(p + o8 + 4);
        const i32x8_t xv = i32x8_t{a[0], a[1], a[2], a[3], b0, b1, 0, 0};
        const int xsc = sb[xs_at(trow + 16 * j) + lg];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa[i], xv, acc[i][j], 4, 2, 0, wsc[i], 0, xsc);
      }
    } else if (C::W4) {
      int wsc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wsc[i] = wsb[(wrow + 16 * i) * wss + lg];
#pragma unroll
      for (int j = 0; j < C::SUB; ++j) {
        const i32x4_t lo = lds16(sb + x_rd[0] + j * 16 * 128);
        const i32x4_t hi = lds16(sb + x_rd[1] + j * 16 * 128);
        const i32x8_t xv = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const int xsc = sb[xs_at(trow + 16 * j) + lg];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa[i], xv, acc[i][j], 4, 0, 0, wsc[i], 0, xsc);
      }
    } else {
      // weight block scales of this wave's rows: gated i < 2 gate, i >= 2 up;
      // otherwise the wave's 64 rows lie in block f0/128 + wn/2
      const float* wsp = (const float*)(sb + C::WS_OFF);
      float ws[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ws[i] = GATED ? wsp[i >> 1] : wsp[wn >> 1];
      const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < C::SUB; ++j) {
        const i32x4_t lo = lds16(sb + x_rd[0] + j * 16 * 128);
        const i32x4_t hi = lds16(sb + x_rd[1] + j * 16 * 128);
        const i32x8_t xv = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const float xs = *(const float*)(sb + xs_at(trow + 16 * j));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4_t pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa[i], xv, z4, 0, 0, 0, 127, 0, 127);
          acc[i][j] += pr * (ws[i] * xs);
        }
      }
    }
  };

  // epilogue: lane holds weight rows 4*lg..+3 of sub-tile i for token lr of
  // sub-tile j; padding rows go to the trash row
  auto store_item = [&](const QItem& t) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < C::SUB; ++j) {
      const int r = wm * C::HALF + j * 16 + lr;
      const size_t orow = (size_t)(r < t.nrows ? t.row0 + r : trash_row) * N;
      if (GATED) {
        float* o = (float*)out + orow;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int f = t.f0 + wn * 32 + i * 16 + lg * 4;
          float4 v;
          v.x = silu_f(acc[i][j][0]) * acc[2 + i][j][0];
          v.y = silu_f(acc[i][j][1]) * acc[2 + i][j][1];
          v.z = silu_f(acc[i][j][2]) * acc[2 + i][j][2];
          v.w = silu_f(acc[i][j][3]) * acc[2 + i][j][3];
          *(float4*)(o + f) = v;
        }
      } else {
        uint16_t* o = (uint16_t*)out + orow;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = t.f0 + wn * 64 + i * 16 + lg * 4;
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          st8(o + f, pk);
        }
      }
    }
  };

  // ---- the stream -------------------------------------------------------------
  // A finished item is stored at the start of the next iteration, ahead of
  // that iteration's loads.  Two stages: every wait is vmcnt(0), which also
  // covers stores that complete out of order with the loads.  Three stages:
  // the wait leaves outstanding only the loads issued for unit v+1 (the last
  // issue, `last_n` of them); the stores went out before those loads.
  (void)issue(0);
  int last_n = 0;
  if (C::NST == 3 && n_units > 1) last_n = issue(1);
  QItem ct;
  decode(it0, ct);
  QItem done{};
  bool pending = false;
  int c = 0, stage = 0, cg = -1;
  for (long v = 0; v < n_units; ++v) {
    if (C::NST == 3 && v + 1 < n_units) {
      switch (last_n) {                         // this wave's loads of unit v have landed
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 9: wait_vmcnt<9>(); break;
        default: wait_vmcnt<0>(); break;
      }
    } else {
      wait_vmcnt<0>();
    }
    barrier_keep_loads();                       // everyone's have; the oldest stage is free
    if (pending) {
      store_item(done);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < C::SUB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pending = false;
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);    // the stores stay ahead of the next loads
    __builtin_amdgcn_sched_barrier(0);
    if (C::NST == 2) {
      if (v + 1 < n_units) (void)issue(stage ^ 1);
    } else {
      if (v + 2 < n_units) last_n = issue(stage == 0 ? 2 : stage - 1);
    }
    const uint8_t* sbv = lds + stage * C::STAGE;
    const uint8_t* wsb = sbv + C::WS_OFF;
    int wss = 4;
    if (C::W4 && (c & ~3) + 4 <= nchunk) {
      if ((c & 3) == 0) ++cg;
      wsb = lds + C::NST * C::STAGE + (cg & 1) * (Q_BN * 16) + (c & 3) * 4;
      wss = 16;
    }
    if (ct.nrows > wm * C::HALF) compute(sbv, wsb, wss);
    stage = stage + 1 == C::NST ? 0 : stage + 1;
    if (++c == nchunk) {
      done = ct;
      pending = true;
      c = 0;
      if (v + 1 < n_units) decode(it0 + (int)((v + 1) / nchunk) * istep, ct);
    }
  }
  if (pending) store_item(done);
}

template <int FMT, int VAR>
static size_t lds_of() { return (size_t)QCfg<FMT, VAR>::LDS; }

extern "C" size_t moe_pf8_lds_bytes(int fmt, int small) {
  if (fmt == WFMT_MXFP4_A6) return small ? lds_of<WFMT_MXFP4_A6, 1>() : lds_of<WFMT_MXFP4_A6, 0>();
  if (fmt == WFMT_MXFP4) return small ? lds_of<WFMT_MXFP4, 1>() : lds_of<WFMT_MXFP4, 0>();
  return small ? lds_of<WFMT_FP8, 1>() : lds_of<WFMT_FP8, 0>();
}
// Tokens per m-tile of the large-batch 8-bit kernel (fmt WFMT_MXFP4_A6: MXFP6
// activations); small != 0: the variant for few tokens per expert.
extern "C" int moe_pf8_tile_tokens(int fmt, int small) {
  if (small) return QCfg<WFMT_FP8, 1>::BM;
  return fmt == WFMT_FP8 ? QCfg<WFMT_FP8, 0>::BM : QCfg<WFMT_MXFP4, 0>::BM;
}

template <int FMT, bool GATED, int VAR>
static hipError_t launch_q8(int n_cu, const WorkList* wl, const int32_t* counts, const int32_t* offsets,
                            const uint8_t* pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                            const uint8_t* X, const uint8_t* Xs, int xcap, int K, int N, void* out,
                            int trash_row, hipStream_t s) {
  const size_t lds = lds_of<FMT, VAR>();
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_pf_q8<FMT, GATED, VAR>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  gemm_pf_q8<FMT, GATED, VAR><<<n_cu, 64 * Q_WAVES, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0,
                                                                 soff1, X, Xs, xcap, K, N, out, trash_row);
  return hipGetLastError();
}

// n_cu: CUs (one workgroup each).  The work list must have been built with
// m-blocks of moe_pf8_tile_tokens(fmt, small) tokens.  xcap: the row
// capacity the MXFP6 planes are sized for (fmt WFMT_MXFP4_A6; ignored
// otherwise).
extern "C" hipError_t moe_launch_gemm_pf8(int fmt, int gated, int small, int n_cu, const WorkList* wl,
                                          const int32_t* counts, const int32_t* offsets, const uint8_t* pool,
                                          size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                                          const void* X, const void* Xs, int xcap, int K, int N, void* out,
                                          int trash_row, hipStream_t s) {
  if (K % Q_BK || N % (gated ? Q_BN / 2 : Q_BN)) return hipErrorInvalidValue;
  const uint8_t* x = (const uint8_t*)X;
  const uint8_t* xs = (const uint8_t*)Xs;
#define MOE_Q8_ARGS n_cu, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, x, xs, xcap, K, N, out, \
                    trash_row, s
  if (fmt == WFMT_FP8) {
    if (small) return gated ? launch_q8<WFMT_FP8, true, 1>(MOE_Q8_ARGS) : launch_q8<WFMT_FP8, false, 1>(MOE_Q8_ARGS);
    return gated ? launch_q8<WFMT_FP8, true, 0>(MOE_Q8_ARGS) : launch_q8<WFMT_FP8, false, 0>(MOE_Q8_ARGS);
  }
  if (fmt == WFMT_MXFP4) {
    if (small) return gated ? launch_q8<WFMT_MXFP4, true, 1>(MOE_Q8_ARGS) : launch_q8<WFMT_MXFP4, false, 1>(MOE_Q8_ARGS);
    return gated ? launch_q8<WFMT_MXFP4, true, 0>(MOE_Q8_ARGS) : launch_q8<WFMT_MXFP4, false, 0>(MOE_Q8_ARGS);
  }
  if (fmt == WFMT_MXFP4_A6) {
    if (small)
      return gated ? launch_q8<WFMT_MXFP4_A6, true, 1>(MOE_Q8_ARGS) : launch_q8<WFMT_MXFP4_A6, false, 1>(MOE_Q8_ARGS);
    return gated ? launch_q8<WFMT_MXFP4_A6, true, 0>(MOE_Q8_ARGS) : launch_q8<WFMT_MXFP4_A6, false, 0>(MOE_Q8_ARGS);
  }
#undef MOE_Q8_ARGS
  return hipErrorInvalidValue;
}
