// Slot-indexed grouped expert GEMMs for small token counts per expert.
//
// Method (paper.oopus.info review of FreeToken, section 2.5): the GPU
// evaluates every expert of G = H u F (cache hits and fresh fills) for the
// tokens routed to it, as one grouped evaluation; each expert is found
// through its slot in the shared slot pool (section 2: a slot holds every
// tensor of one (layer, expert)).  The expert is a SwiGLU FFN:
//   GEMM 1: [g | u] = X W_gate^T, X W_up^T   (fp32 accumulate), A = silu(g) * u
//   GEMM 2: Z = A W_down^T                    (fp32 accumulate)
//
// Small batches are bound by HBM: every weight byte of an active expert is
// read once, so the kernel is a weight stream with MFMAs riding on it.
//
// Work.  An item is (expert, m-block of 16*NS tokens, 64 weight rows per
// matrix); its K range is cut into chunks of 256 bytes per weight row (128
// bf16, 256 fp8 or 512 E2M1 values; NVFP4: 128 bytes, 256 values).  The flat
// sequence of (item, chunk)
// units is split into equal contiguous ranges, one per workgroup, so every
// workgroup streams the same number of bytes whatever the expert sizes; the
// ranges of consecutive workgroups of one XCD are contiguous.  An item cut by
// a range boundary leaves fp32 partial tiles, one per workgroup that holds
// part of it; a second small kernel adds them in workgroup order and applies
// the epilogue, so the sum is deterministic for a given set of GPU experts
// and no workgroup waits for another (cross-XCD visibility inside one kernel
// would need an L2 write-back and invalidate per handoff, which costs more
// than the launch).
//
// Memory.  Each chunk goes from HBM into a ring of three LDS stages (two for
// NVFP4 with up to 32 tokens per m-block, which fits more workgroups per CU) by
// direct global->LDS loads (lane l's 16 bytes land at the instruction's LDS
// base + 16*l) with the nontemporal hint: 16 consecutive lanes cover one
// 256-byte row segment, the pattern that streams HBM at 7.0-7.3 TB/s on
// MI355X (weights are read once and must not displace reused lines).  The
// 16-byte pieces of a row are XOR-swizzled by the row index so the MFMA
// operand reads of 16 rows hit distinct banks; the loads pick their source
// piece so the swizzle comes out of the lane-linear placement.  The token
// rows of the chunk, the scales of the 8-bit formats and the weight scales
// go through the same ring, so one counter wait per chunk covers everything
// the chunk needs: chunk c+NST-1 is requested while chunk c is multiplied.
//
// MFMA.  Wave w owns weight rows 16w..16w+15 of the item (of each matrix);
// weights are the A operand (16 rows) and tokens the B operand (16 tokens per
// sub-tile).  Result lane l holds weight rows 4*(l/16)..+3 of token l%16.
//  * bf16: v_mfma_f32_16x16x32_bf16; lane group g of MFMA q takes the K
//    values [32q + 8g, 32q + 8g + 8) of the chunk, i.e. 16-byte piece 4q+g.
//  * fp8 (E4M3, fp32 scale per 128x128 weight block, per token per 128-K
//    activation group): v_mfma_scale_f32_16x16x128_f8f6f4 with unit E8M0
//    scales per 128-K half of the chunk, its partial sum multiplied by
//    w_scale * x_scale.  With uniform scales only the agreement of the A and
//    B byte layouts matters, so lane group g takes 32 consecutive bytes.
//  * MXFP4: the same instruction with E2M1 weights (A) and MXFP8 activations
//    (B) and their E8M0 block scales.  Lane layout of that instruction
//    (measured on gfx950 with one-hot inputs): an E2M1 operand's lane group
//    g holds the 32 K values [32g, 32g+32) in its low 16 bytes; an 8-bit
//    operand's lane group g holds K [16g, 16g+16) in bytes 0-15 and
//    K [64+16g, 64+16g+16) in bytes 16-31; the E8M0 scale of lane group g
//    covers K block [32g, 32g+32) of that lane's row (A) or column (B).
//  * NVFP4 (E2M1 elements, E4M3 scale per 16 inputs, fp32 scale per
//    matrix): gfx950's scaled MFMA takes only power-of-two block scales, so
//    the weights are dequantised in registers to fp16 (element * block
//    scale, exact: at most six significant bits within 2^-10 .. 2688): one
//    scaled fp4 -> fp16 pair conversion and one packed fp16 multiply per
//    two weights (a bf16 product would need fp32 multiplies and packs:
//    gfx950 has no packed bf16 multiply); they meet fp16 tokens (the hidden
//    rows converted once per call, A stored in fp16 by GEMM 1) in the fp16
//    MFMA; the matrix's fp32 scale multiplies the fp32 sums in the epilogue
//    (gate and up before SwiGLU, down on Z).  Chunks are 256 K values: 128
//    bytes of codes and 16 scale bytes per weight row (8 lanes per row
//    segment, pieces XOR-swizzled by row & 7), 512 bytes per token row.
//  * fp8 and MXFP4 weights with bf16 activations (the small-batch default:
//    the stream is bound by the weight bytes, so 16-bit activations cost
//    nothing and keep the activations unrounded): the weights are
//    dequantised in registers to bf16 for v_mfma_f32_16x16x32_bf16.  E4M3
//    codes convert exactly (scale 1) and each 128-K block's partial sum is
//    multiplied by its fp32 block scale; E2M1 codes convert with their E8M0
//    block scale, exactly (a power of two times at most two significant
//    bits).  Chunks are 256 K values: 256 (fp8) or 128 (E2M1) bytes per
//    weight row, 512 bytes per token row.  Within a pair of MFMA steps lane
//    group g takes the 16 consecutive K values [16g, 16g+16) of the pair's
//    64 (8 for each step; the token operand uses the same assignment, so the
//    products pair up), one 16-byte (fp8) or 8-byte (E2M1) weight read and
//    one scale per pair.
#include "common.h"

namespace {

constexpr int NW = 4;                 // waves per workgroup
constexpr int ROWS = 16 * NW;         // weight rows per item and matrix
constexpr int N_XCD = 8;
constexpr int MAX_BLOCKS = 1024;      // capacity of the partial-tile buffer (workgroups)
constexpr int CACHE_NT = 2;           // cache-policy bits of a nontemporal load (gfx94x/gfx950)

template <int FMT, bool GATED, int NS>
struct Cfg {
  static constexpr int NMAT = GATED ? 2 : 1;
  static constexpr bool NV = FMT == WFMT_NVFP4;
  static constexpr bool A16 = FMT == WFMT_FP8_A16 || FMT == WFMT_MXFP4_A16;   // 8/4-bit weights, bf16 tokens
  static constexpr bool F8S = FMT == WFMT_FP8 || FMT == WFMT_FP8_A16;         // fp32 128x128 block scales
  static constexpr bool W4 = NV || FMT == WFMT_MXFP4_A16;     // E2M1 rows of 128 bytes per chunk (256 K)
  static constexpr bool BF_X = FMT == WFMT_BF16 || NV || A16; // 16-bit tokens (bf16, or fp16 for NVFP4)
  static constexpr int CK = FMT == WFMT_BF16 ? 128 : (FMT == WFMT_MXFP4 ? 512 : 256);   // K per chunk
  static constexpr int WB = W4 ? 128 : 256;                   // weight bytes per row per chunk
  static constexpr int WSZ = 16 * WB;                         // one wave's rows of one matrix
  static constexpr int NWL = WSZ / 1024;                      // weight loads per wave and matrix
  static constexpr int XB = (FMT == WFMT_MXFP4 || NV || A16) ? 512 : 256;   // token bytes per chunk
  static constexpr int MB = 16 * NS;                          // tokens per m-block
  static constexpr int NXI = MB * XB / 1024 / NW;             // token loads per wave per chunk
  static constexpr int W_OFF = 0;
  static constexpr int X_OFF = NMAT * NW * WSZ;
  static constexpr int XS_OFF = X_OFF + MB * XB;
  static constexpr int XS_BYTES = BF_X ? 0 : NW * 256;
  static constexpr int WS_OFF = XS_OFF + XS_BYTES;
  static constexpr int WS_BYTES = FMT == WFMT_BF16 ? 0 : (F8S ? NW * 256 : NMAT * NW * 256);
  static constexpr int STAGE = WS_OFF + WS_BYTES;
  // ring stages: E2M1 rows with two stages fit more workgroups per CU
  static constexpr int NST = (W4 && NS <= 2) ? 2 : 3;
  // loads per wave per chunk: weights, tokens, token scales, weight scales
  static constexpr int NI = NWL * NMAT + NXI + (BF_X ? 0 : 1) +
                            (FMT == WFMT_BF16 ? 0 : (F8S ? 1 : NMAT));
  static constexpr int NACC = NMAT * NS;
  static_assert(NXI >= 1 && NXI * NW * 1024 == MB * XB, "token chunk must split evenly over the waves");
  static_assert(FMT != WFMT_FP8 || 2 * MB <= NW * 64, "fp8 token scales: one dword per lane");
  static_assert(FMT != WFMT_MXFP4 || 4 * MB <= NW * 64, "MX token scales: one dword per lane");
};

// weights: read once, streamed with the nontemporal hint
DEV void dma16_nt(const void* src, lds_u8_t* dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 16, 0, CACHE_NT);
}
// token rows: re-read by every tile of the expert, kept in the caches
DEV void dma16(const void* src, lds_u8_t* dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
}
DEV void dma4(const void* src, lds_u8_t* dst) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)dst, 4, 0, 0);
}

DEV int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

DEV float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

DEV i32x4_t lds16(const uint8_t* p) { return *(const i32x4_t*)p; }

// Eight E4M3 codes (bytes of d0 then d1, element order) as bf16, exact.
DEV bf16x8_t fp8x8_bf16(int d0, int d1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)d0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)d0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)d1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)d1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight E2M1 codes (nibbles of w, even element in the low nibble) times the
// block scale s (a power of two) as bf16, exact.
DEV bf16x8_t fp4x8_bf16(uint32_t w, float s) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

struct Item {
  int slot, row0, nrows, n0;
};

// First unit of workgroup b when U units are split over G workgroups.
DEV long range_start(long b, long U, long G) { return b * U / G; }
// Workgroup whose range holds unit u (G <= U, so every range is non-empty).
DEV long owner_of(long u, long U, long G) {
  long b = ((u + 1) * G - 1) / U;
  return b < G - 1 ? b : G - 1;
}

// Partial tile of workgroup bb for item i (its first item: slot 0, else 1),
// [NW waves][NACC][64 lanes] f32x4.
template <int NACC>
DEV f32x4_t* part_tile(f32x4_t* part, long bb, int i, long U, long G, int KC, int wave) {
  const int slot = (range_start(bb, U, G) / KC == i) ? 0 : 1;
  return part + (((size_t)bb * 2 + slot) * NW + wave) * NACC * 64;
}

// Output values of one wave's accumulators of an item (SwiGLU for GEMM 1):
// lane holds weight rows 4*lg..+3 (output columns) of token lr of each
// 16-token sub-tile; gate in acc[ms], up in acc[NS + ms].  SCALED: the
// matrices' fp32 scales s0 (gate, or down) and s1 (up) multiply the sums.
template <bool GATED, int NS, bool SCALED = false>
DEV void activate(const f32x4_t* acc, f32x4_t* val, float s0 = 1.0f, float s1 = 1.0f) {
#pragma unroll
  for (int ms = 0; ms < NS; ++ms) {
    if (GATED) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        val[ms][i] = SCALED ? silu_mul(acc[ms][i] * s0, acc[NS + ms][i] * s1) : silu_mul(acc[ms][i], acc[NS + ms][i]);
    } else {
      val[ms] = SCALED ? acc[ms] * s0 : acc[ms];
    }
  }
}

// NVFP4: the fp32 scales of an expert's matrices, after its block scales
// (gate, up, down); n = K * N elements per matrix.
// Scalar loads through the constant address space: a vector load would
// make the epilogue wait for every load in flight (the next chunks' too).
typedef __attribute__((address_space(4))) float cst_f32_t;
DEV void nv_tensor_scales(const uint8_t* pool, size_t S, int slot, int K, int N, bool gated, float& s0, float& s1) {
  const size_t n = (size_t)K * N;
  const cst_f32_t* t = (const cst_f32_t*)(pool + (size_t)slot * S + 3 * (n / 2) + 3 * (n / 16));
  s0 = gated ? t[0] : t[2];
  s1 = gated ? t[1] : 1.0f;
}

// Store the output values (fp32 for GEMM 1 of the 8-bit formats, fp16 for
// GEMM 1 of NVFP4, else bf16).
template <int FMT, bool GATED, int NS>
DEV void store_out(const f32x4_t* val, const Item& it, int wave, int lane, int N, void* out) {
  const int lr = lane & 15, lg = lane >> 4;
  const int col = it.n0 + 16 * wave + 4 * lg;
#pragma unroll
  for (int ms = 0; ms < NS; ++ms) {
    const int t = ms * 16 + lr;
    if (t >= it.nrows) continue;
    const size_t o = (size_t)(it.row0 + t) * N + col;
    if (GATED && (FMT == WFMT_FP8 || FMT == WFMT_MXFP4)) {
      *(f32x4_t*)((float*)out + o) = val[ms];
    } else if (GATED && FMT == WFMT_NVFP4) {
      uint2 pk;
      pk.x = pack_f16x2(val[ms][0], val[ms][1]);
      pk.y = pack_f16x2(val[ms][2], val[ms][3]);
      st8((uint16_t*)out + o, pk);
    } else {
      uint2 pk;
      pk.x = pack_bf16x2(val[ms][0], val[ms][1]);
      pk.y = pack_bf16x2(val[ms][2], val[ms][3]);
      st8((uint16_t*)out + o, pk);
    }
  }
}

// Item i of the work list (m-block p = i / ntiles, 64-row tile i % ntiles),
// read from global memory.
DEV void decode_global(const WorkList* wl, const int32_t* counts, const int32_t* offsets, int ntiles, int MB, int i,
                       Item& it) {
  const int p = i / ntiles, nt = i - p * ntiles;
  const int a = find_active(wl, p);
  const int e = wl->act_e[a];
  const int mb = p - wl->mblk_prefix[a];
  it.slot = wl->act_slot[a];
  it.row0 = offsets[e] + mb * MB;
  it.nrows = min(MB, counts[e] - mb * MB);
  it.n0 = nt * ROWS;
}

}  // namespace

// FMT: WFMT_*.  GATED: GEMM 1 (gate rows at woff0, up rows at woff1, SwiGLU
// epilogue; out = A: bf16 for WFMT_BF16, fp16 for WFMT_NVFP4, else fp32 for
// the quantisation pass).  Otherwise GEMM 2 (weights at woff0; out = Z
// bf16).  Token rows of X are gathered through row_tok (16-bit GEMM 1: bf16,
// or fp16 for NVFP4) or taken in grouped order; Xs holds the activation
// scales of the 8-bit formats; soff0/soff1 the weight scales.
// part: partial tiles [MAX_BLOCKS][2][NW][NACC][64] of the items cut by a
// range boundary, finished by gemm_dec_fix; part == nullptr: one workgroup
// per item, and a grid smaller than the item count sets bit 1 of *err.
template <int FMT, bool GATED, int NS>
__global__ void __launch_bounds__(256, 1)
gemm_dec(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
         const uint8_t* __restrict__ pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
         const uint8_t* __restrict__ X, const uint8_t* __restrict__ Xs, const int32_t* __restrict__ row_tok, int K,
         int N, void* __restrict__ out, f32x4_t* __restrict__ part, int* __restrict__ err) {
  using C = Cfg<FMT, GATED, NS>;
  extern __shared__ __align__(16) uint8_t ring[];
  __shared__ int l_pref[257], l_slot[256], l_row0[256], l_cnt[256];
  // token row of each grouped row this workgroup touches (16-bit GEMM 1)
  constexpr int ROWTAB = (FMT == WFMT_BF16 && GATED) ? 2048 : (((C::NV || C::A16) && GATED) ? 1024 : 1);
  __shared__ int l_rows[ROWTAB];
  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;

  const int n_act = wl->n_act;
  for (int i = threadIdx.x; i <= n_act; i += blockDim.x) {
    l_pref[i] = wl->mblk_prefix[i];
    if (i < n_act) {
      const int e = wl->act_e[i];
      l_slot[i] = wl->act_slot[i];
      l_row0[i] = offsets[e];
      l_cnt[i] = counts[e];
    }
  }
  __syncthreads();

  const int ntiles = N / ROWS;
  const int KC = (K + C::CK - 1) / C::CK;
  const long U = (long)wl->n_mblk * ntiles * KC;     // < 2^31 for any admissible shape (checked by the host)
  if (U == 0) return;
  // part == nullptr: one workgroup per item (the grid covers every item),
  // so no item is cut and nothing needs summing afterwards
  if (!part && U / KC > (long)gridDim.x) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, 2);   // items would be left unwritten
    return;
  }
  const long G = !part ? U / KC : (U < (long)gridDim.x ? U : (long)gridDim.x);
  long b = blockIdx.x;
  if (G == gridDim.x && (gridDim.x % N_XCD) == 0)       // XCD x takes ranges x*G/8 .. (x+1)*G/8 - 1
    b = (long)(blockIdx.x % N_XCD) * (gridDim.x / N_XCD) + blockIdx.x / N_XCD;
  if (b >= G) return;
  const long u0 = range_start(b, U, G), u1 = range_start(b + 1, U, G);

  // bytes of one weight row and of one token row
  const int wrow = FMT == WFMT_BF16 ? K * 2 : (C::F8S ? K : K / 2);
  const int xrow = C::BF_X ? K * 2 : K;

  // Items are visited in order: a cursor (m-block p, tile nt, active expert
  // a) moves to the next item without searching the work list.
  struct Cur {
    int p, nt, a;
  };
  auto cur_at = [&](int i) {
    Cur c;
    c.p = i / ntiles;
    c.nt = i - c.p * ntiles;
    int a = 0, hi = n_act - 1;
    while (a < hi) {
      const int mid = (a + hi + 1) >> 1;
      if (l_pref[mid] <= c.p) a = mid; else hi = mid - 1;
    }
    c.a = uni(a);
    return c;
  };
  auto cur_next = [&](Cur& c) {
    if (++c.nt == ntiles) {
      c.nt = 0;
      ++c.p;
      if (c.a + 1 < n_act && c.p == uni(l_pref[c.a + 1])) ++c.a;
    }
  };
  auto item_of = [&](const Cur& c, Item& it) {
    const int mb = c.p - uni(l_pref[c.a]);
    it.slot = uni(l_slot[c.a]);
    it.row0 = uni(l_row0[c.a]) + mb * C::MB;
    it.nrows = min(C::MB, uni(l_cnt[c.a]) - mb * C::MB);
    it.n0 = c.nt * ROWS;
  };

  const int i_first = (int)(u0 / KC), kc_first = (int)(u0 - (long)i_first * KC);
  // gathered token rows of the workgroup's grouped-row span, when it fits
  int rbase = 0;
  bool tab = false;
  if (row_tok) {
    Item f, l;
    item_of(cur_at(i_first), f);
    item_of(cur_at((int)((u1 - 1) / KC)), l);
    rbase = f.row0;
    const int rspan = l.row0 + l.nrows - f.row0;
    tab = rspan <= ROWTAB;
    if (tab)
      for (int r = threadIdx.x; r < rspan; r += blockDim.x) l_rows[r] = row_tok[rbase + r];
    __syncthreads();
  }

  // ---- per-lane constants ---------------------------------------------------
  // weight loads: instruction j covers rows 4j..4j+3 of the wave's 16; lane l
  // fetches piece (l&15) ^ row so that the lane-linear LDS placement is the
  // swizzled layout
  // (E2M1 rows of 128 bytes: instruction j covers rows 8j..8j+7, lane l piece (l&7) ^ (row&7))
  uint32_t w_lane[4];
#pragma unroll
  for (int j = 0; j < C::NWL; ++j) {
    if (C::W4) {
      const int r = 8 * j + (lane >> 3);
      w_lane[j] = (uint32_t)(16 * wave + r) * wrow + (((lane & 7) ^ (r & 7)) << 4);
    } else {
      const int r = 4 * j + (lane >> 4);
      w_lane[j] = (uint32_t)(16 * wave + r) * wrow + (((lane & 15) ^ r) << 4);
    }
  }
  // token loads: instruction j of the wave covers tokens (wave*NXI + j)*per + ...
  constexpr int XPER = C::XB == 256 ? 4 : 2;
  const int x_tok_lane = C::XB == 256 ? (lane >> 4) : (lane >> 5);
  const int x_pos = C::XB == 256 ? (lane & 15) : (lane & 31);
  // operand reads (bytes inside a stage)
  uint32_t w_rd[4];   // bf16 / MXFP4: piece 4q+lg of row lr; fp8: piece 2lg (+8h) of row lr
  uint32_t x_rd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int pw = FMT == WFMT_FP8 ? (8 * (q >> 1) + 2 * lg + (q & 1)) : (4 * q + lg);
    w_rd[q] = C::W_OFF + wave * 4096 + lr * 256 + ((pw ^ lr) << 4);
    const int px = FMT == WFMT_MXFP4 ? (8 * q + lg) : pw;
    x_rd[q] = C::X_OFF + lr * C::XB + ((px ^ lr) << 4);
  }

  // ---- issue side: the loads of the next unit into one ring stage ----------
  Cur icur = cur_at(i_first);
  Item ii{};
  int iss_kc = kc_first;
  uint32_t x_lane[C::NXI];    // byte offset of this lane's token piece in X (less the chunk)
  int x_tt[C::NXI];           // the lane's token inside the m-block (clamped to a real one)
  auto set_issue_item = [&]() {
    item_of(icur, ii);
#pragma unroll
    for (int j = 0; j < C::NXI; ++j) {
      const int t0 = (wave * C::NXI + j) * XPER;
      const int t = t0 + x_tok_lane;
      const int tt = t < ii.nrows ? t : 0;
      x_tt[j] = tt;
      int row;
      if (tab) {
        row = l_rows[ii.row0 - rbase + tt];
      } else if (row_tok) {
        // uniform lookups of the instruction's tokens (scalar loads), then a per-lane pick
        int r[4];
#pragma unroll
        for (int q = 0; q < XPER; ++q) r[q] = row_tok[ii.row0 + (t0 + q < ii.nrows ? t0 + q : 0)];
        row = r[0];
#pragma unroll
        for (int q = 1; q < XPER; ++q) row = (x_tok_lane == q && t < ii.nrows) ? r[q] : row;
      } else {
        row = ii.row0 + tt;
      }
      x_lane[j] = (uint32_t)row * xrow + ((x_pos ^ (t & 15)) << 4);
    }
  };
  set_issue_item();

  auto issue = [&](int st) {
    if (iss_kc == KC) {
      iss_kc = 0;
      cur_next(icur);
      set_issue_item();
    }
    const int kc = iss_kc++;
    lds_u8_t* sb = (lds_u8_t*)ring + st * C::STAGE;
    const uint8_t* wb = pool + (size_t)ii.slot * S;
    const bool wpart = kc * C::WB + C::WB > wrow;      // last chunk shorter than WB bytes per row
#pragma unroll
    for (int m = 0; m < C::NMAT; ++m) {
      const uint8_t* mat = wb + (m ? woff1 : woff0) + (size_t)ii.n0 * wrow + (size_t)kc * C::WB;
#pragma unroll
      for (int j = 0; j < C::NWL; ++j) {
        uint32_t o = w_lane[j];
        if (FMT != WFMT_BF16 && wpart) {
          const int r = C::W4 ? 8 * j + (lane >> 3) : 4 * j + (lane >> 4);
          const int p16 = (C::W4 ? ((lane & 7) ^ (r & 7)) : ((lane & 15) ^ r)) << 4;
          o = (uint32_t)(16 * wave + r) * wrow + (p16 < wrow - kc * C::WB ? p16 : 0);
        }
        dma16_nt(mat + o, sb + C::W_OFF + (m * NW + wave) * C::WSZ + j * 1024);
      }
    }
    const bool xpart = kc * C::XB + C::XB > xrow;
    const uint8_t* xb = X + (size_t)kc * C::XB;
#pragma unroll
    for (int j = 0; j < C::NXI; ++j) {
      uint32_t o = x_lane[j];
      if (FMT != WFMT_BF16 && xpart) {
        const int t = (wave * C::NXI + j) * XPER + x_tok_lane;
        const int p16 = (x_pos ^ (t & 15)) << 4;
        o = o - p16 + (p16 < xrow - kc * C::XB ? p16 : 0);
      }
      dma16(xb + o, sb + C::X_OFF + (wave * C::NXI + j) * 1024);
    }
    if (C::F8S) {
      const int kb = K / 128;   // 128-K groups per row
      if (FMT == WFMT_FP8) {
        // token scales: entry e = 64*wave + lane -> token e/2, half e%2 of the chunk
        const int e = wave * 64 + lane, t = e >> 1, h = e & 1;
        const int tt = t < ii.nrows ? t : 0;
        const int g = min(kc * 2 + h, kb - 1);
        dma4(Xs + ((size_t)(ii.row0 + tt) * kb + g) * 4, sb + C::XS_OFF + wave * 256);
      }
      {
        // weight scales of this wave's 16 rows: lane (2m + h) -> matrix m, half h
        const int m = (lane >> 1) & 1, h = lane & 1;
        const size_t so = (m && GATED) ? soff1 : soff0;
        const int g = min(kc * 2 + h, kb - 1);
        dma4(wb + so + ((size_t)((ii.n0 + 16 * wave) / 128) * kb + g) * 4, sb + C::WS_OFF + wave * 256);
      }
    } else if (C::NV) {
      const int kb = K / 16;    // 16-K blocks per row
#pragma unroll
      for (int m = 0; m < C::NMAT; ++m) {
        // weight scales: lane -> row lane/4 of the wave's 16, 4 bytes (16 per row per chunk)
        const int r = lane >> 2, qd = lane & 3;
        const int g = min(kc * 16 + qd * 4, kb - 4);
        dma4(wb + (m ? soff1 : soff0) + (size_t)(ii.n0 + 16 * wave + r) * kb + g,
             sb + C::WS_OFF + (m * NW + wave) * 256);
      }
    } else if (FMT == WFMT_MXFP4_A16) {
      const int kb = K / 32;    // 32-K blocks per row
#pragma unroll
      for (int m = 0; m < C::NMAT; ++m) {
        // weight scales: 8 bytes per row per chunk; lane -> row (lane/2) % 16,
        // bytes 4*(lane%2).. (lanes 32-63 repeat rows 0-15 into unused bytes)
        const int r = (lane >> 1) & 15, qd = lane & 1;
        const int g = min(kc * 8 + qd * 4, kb - 4);
        dma4(wb + (m ? soff1 : soff0) + (size_t)(ii.n0 + 16 * wave + r) * kb + g,
             sb + C::WS_OFF + (m * NW + wave) * 256);
      }
    } else if (FMT == WFMT_MXFP4) {
      const int kb = K / 32;    // 32-K blocks per row
      {
        // token scales: entry e -> token e/4, 4 bytes (blocks 4*(e%4)..+3 of the chunk)
        const int e = wave * 64 + lane, t = e >> 2, qd = e & 3;
        const int tt = t < ii.nrows ? t : 0;
        const int g = min(kc * 16 + qd * 4, kb - 4);
        dma4(Xs + (size_t)(ii.row0 + tt) * kb + g, sb + C::XS_OFF + wave * 256);
      }
#pragma unroll
      for (int m = 0; m < C::NMAT; ++m) {
        // weight scales: lane -> row lane/4 of the wave's 16, 4 bytes
        const int r = lane >> 2, qd = lane & 3;
        const int g = min(kc * 16 + qd * 4, kb - 4);
        dma4(wb + (m ? soff1 : soff0) + (size_t)(ii.n0 + 16 * wave + r) * kb + g,
             sb + C::WS_OFF + (m * NW + wave) * 256);
      }
    }
  };

  // ---- compute side ------------------------------------------------------
  f32x4_t acc[C::NACC];
#pragma unroll
  for (int q = 0; q < C::NACC; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Cur ccur = cur_at(i_first);
  Item ci{};
  item_of(ccur, ci);
  float ts0 = 1.0f, ts1 = 1.0f;             // NVFP4 matrix scales of the current item (epilogue)
  if (C::NV) nv_tensor_scales(pool, S, ci.slot, K, N, GATED, ts0, ts1);

  auto compute = [&](int kc, int st) {
    const uint8_t* sb = ring + st * C::STAGE;
    const int nms = (ci.nrows + 15) >> 4;
    if (FMT == WFMT_BF16) {
      i32x4_t wa[C::NMAT][4];
#pragma unroll
      for (int m = 0; m < C::NMAT; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) wa[m][q] = lds16(sb + w_rd[q] + m * NW * 4096);
#pragma unroll
      for (int ms = 0; ms < NS; ++ms) {
        if (ms >= nms) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x4_t xv = lds16(sb + x_rd[q] + ms * 16 * C::XB);
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m)
            acc[m * NS + ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, wa[m][q]), __builtin_bit_cast(bf16x8_t, xv), acc[m * NS + ms], 0, 0, 0);
        }
      }
    } else if (FMT == WFMT_FP8) {
      const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && kc * 256 + 128 >= K) break;
        i32x8_t wa[C::NMAT];
        float ws[C::NMAT];
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m) {
          const i32x4_t lo = lds16(sb + w_rd[2 * h] + m * NW * 4096);
          const i32x4_t hi = lds16(sb + w_rd[2 * h + 1] + m * NW * 4096);
          wa[m] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          ws[m] = *(const float*)(sb + C::WS_OFF + wave * 256 + (2 * m + h) * 4);
        }
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
          if (ms >= nms) break;
          const int t = ms * 16 + lr;
          const i32x4_t lo = lds16(sb + x_rd[2 * h] + ms * 16 * C::XB);
          const i32x4_t hi = lds16(sb + x_rd[2 * h + 1] + ms * 16 * C::XB);
          const i32x8_t xv = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const float xs = *(const float*)(sb + C::XS_OFF + (2 * t + h) * 4);
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m) {
            const f32x4_t pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa[m], xv, z4, 0, 0, 0, 127, 0, 127);
            acc[m * NS + ms] += pr * (ws[m] * xs);
          }
        }
      }
    } else if (C::A16) {
      // 256 K per chunk in two 128-K halves (one fp8 scale block each), each
      // half two pairs of MFMA steps; lane group lg of pair p takes K
      // [64p + 16lg, +16): 8 values for each step of the pair
      const bool full = kc * 256 + 256 <= K;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && !full) break;
        f32x4_t pa[C::NACC];                    // fp8: this block's sums, scaled below
#pragma unroll
        for (int q = 0; q < C::NACC; ++q) pa[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int p = 2 * h + pp;
          bf16x8_t wa0[C::NMAT], wa1[C::NMAT];
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m) {
            if (C::F8S) {
              const i32x4_t v = lds16(sb + (m * NW + wave) * C::WSZ + lr * 256 + (((4 * p + lg) ^ lr) << 4));
              wa0[m] = fp8x8_bf16(v[0], v[1]);
              wa1[m] = fp8x8_bf16(v[2], v[3]);
            } else {
              // two dword reads: the compiler cannot tell an 8-byte LDS read
              // from the stages the direct loads are filling and would wait
              // for every load in flight before it
              const uint8_t* cp = sb + (m * NW + wave) * C::WSZ + lr * 128 +
                                  (((2 * p + (lg >> 1)) ^ (lr & 7)) << 4) + 8 * (lg & 1);
              const uint32_t c0 = *(const uint32_t*)cp, c1 = *(const uint32_t*)(cp + 4);
              const float sc = e8m0_to_f32(sb[C::WS_OFF + (m * NW + wave) * 256 + lr * 8 + 2 * p + (lg >> 1)]);
              wa0[m] = fp4x8_bf16(c0, sc);
              wa1[m] = fp4x8_bf16(c1, sc);
            }
          }
#pragma unroll
          for (int ms = 0; ms < NS; ++ms) {
            if (ms >= nms) break;
            const uint8_t* xr = sb + C::X_OFF + (ms * 16 + lr) * C::XB;
            const bf16x8_t x0 = __builtin_bit_cast(bf16x8_t, lds16(xr + (((8 * p + 2 * lg) ^ lr) << 4)));
            const bf16x8_t x1 = __builtin_bit_cast(bf16x8_t, lds16(xr + (((8 * p + 2 * lg + 1) ^ lr) << 4)));
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m) {
              f32x4_t& d = C::F8S ? pa[m * NS + ms] : acc[m * NS + ms];
              d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa0[m], x0, d, 0, 0, 0);
              d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa1[m], x1, d, 0, 0, 0);
            }
          }
        }
        if (C::F8S) {
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m) {
            const float ws = *(const float*)(sb + C::WS_OFF + wave * 256 + (2 * m + h) * 4);
#pragma unroll
            for (int ms = 0; ms < NS; ++ms) acc[m * NS + ms] += pa[m * NS + ms] * ws;
          }
        }
      }
    } else if (C::NV) {
      // the 16 block-scale bytes of row lr of each matrix for this chunk
      i32x4_t scv[C::NMAT];
#pragma unroll
      for (int m = 0; m < C::NMAT; ++m) scv[m] = lds16(sb + C::WS_OFF + (m * NW + wave) * 256 + lr * 16);
      // K is a multiple of 128: a chunk holds 4 or 8 MFMA steps of 32; each
      // half is converted in one batch (independent conversions back to
      // back), then multiplied
      const bool full = kc * 256 + 256 <= K;
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        if (hq == 1 && !full) break;
        // lane (row lr, group lg): K [32q + 8lg, +8) = 4 code bytes of piece q, one block scale
        uint32_t cw[4][C::NMAT];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m)
            cw[j][m] = *(const uint32_t*)(sb + C::W_OFF + (m * NW + wave) * C::WSZ + lr * C::WB +
                                          (((4 * hq + j) ^ (lr & 7)) << 4) + 4 * lg);
        i32x4_t wa[4][C::NMAT];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = 4 * hq + j;
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m) {
            // block 2q + lg/2 of the chunk: byte 2(q&1) + lg/2 of dword q/2
            const int scw = (int)((uint32_t)scv[m][q >> 1] >> (8 * (2 * (q & 1) + (lg >> 1))));
            const _Float16 sh = (_Float16)__builtin_amdgcn_cvt_f32_fp8(scw, 0);   // E4M3 is exact in fp16
            const f16x2_t s2 = {sh, sh};
            wa[j][m][0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[j][m], 1.0f, 0) * s2);
            wa[j][m][1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[j][m], 1.0f, 1) * s2);
            wa[j][m][2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[j][m], 1.0f, 2) * s2);
            wa[j][m][3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[j][m], 1.0f, 3) * s2);
          }
        }
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
          if (ms >= nms) break;
          i32x4_t xv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xv[j] = lds16(sb + C::X_OFF + (ms * 16 + lr) * C::XB + (((4 * (4 * hq + j) + lg) ^ lr) << 4));
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int m = 0; m < C::NMAT; ++m)
              acc[m * NS + ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, wa[j][m]),
                                                                       __builtin_bit_cast(f16x8_t, xv[j]),
                                                                       acc[m * NS + ms], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q > 0 && kc * 512 + q * 128 >= K) break;
        i32x8_t wa[C::NMAT];
        int wsc[C::NMAT];
#pragma unroll
        for (int m = 0; m < C::NMAT; ++m) {
          const i32x4_t v = lds16(sb + w_rd[q] + m * NW * 4096);
          wa[m] = i32x8_t{v[0], v[1], v[2], v[3], 0, 0, 0, 0};
          wsc[m] = sb[C::WS_OFF + (m * NW + wave) * 256 + lr * 16 + 4 * q + lg];
        }
#pragma unroll
        for (int ms = 0; ms < NS; ++ms) {
          if (ms >= nms) break;
          const int t = ms * 16 + lr;
          // 8-bit operand: bytes 0-15 = K [16g, 16g+16), bytes 16-31 = K [64+16g, 64+16g+16)
          const i32x4_t lo = lds16(sb + x_rd[q] + ms * 16 * C::XB);
          const i32x4_t hi = lds16(sb + C::X_OFF + t * C::XB + (((8 * q + 4 + lg) ^ lr) << 4));
          const i32x8_t xv = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const int xsc = sb[C::XS_OFF + t * 16 + 4 * q + lg];
#pragma unroll
          for (int m = 0; m < C::NMAT; ++m)
            acc[m * NS + ms] =
                __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa[m], xv, acc[m * NS + ms], 4, 0, 0, wsc[m], 0, xsc);
        }
      }
    }
  };

  // Stores share the memory counter with the loads and may complete before
  // loads issued earlier, so a counter wait is only trusted when everything
  // it leaves outstanding is a load issued after what it must cover.  A
  // finished item's outputs are therefore stored at the start of the next
  // iteration, ahead of that iteration's loads (a compiler and scheduling
  // barrier keeps them there), and the partial tiles of the (at most two)
  // items cut by the range boundaries are kept in registers and stored after
  // the stream.
  f32x4_t pend[NS], first_part[C::NACC], last_part[C::NACC];
  Item pit{};
  bool has_pend = false, has_first = false, has_last = false;
  int last_i = 0;
  auto flush = [&]() {
    if (!has_pend) return;
    has_pend = false;
    store_out<FMT, GATED, NS>(pend, pit, wave, lane, N, out);
  };
  auto finish_item = [&](int i) {
    if ((long)i * KC >= u0 && (long)(i + 1) * KC <= u1) {
      activate<GATED, NS, C::NV>(acc, pend, ts0, ts1);
      pit = ci;
      has_pend = true;
    } else if (i == i_first) {    // cut by a range boundary: gemm_dec_fix adds the parts
#pragma unroll
      for (int q = 0; q < C::NACC; ++q) first_part[q] = acc[q];
      has_first = true;
    } else {
#pragma unroll
      for (int q = 0; q < C::NACC; ++q) last_part[q] = acc[q];
      has_last = true;
      last_i = i;
    }
  };

  // ---- the stream ----------------------------------------------------------
  const int n = (int)(u1 - u0);     // units of this workgroup
  constexpr int NST = C::NST;
  static_assert(NST * C::STAGE + 4 * (257 + 3 * 256 + ROWTAB) <= 160 * 1024, "LDS budget");
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < n) issue(s);
  int st = 0, i = i_first, kc = kc_first;
  for (int v = 0; v < n; ++v) {
    // this wave's loads of unit v have landed: what may still be outstanding
    // is the NI loads each of units v+1 .. v+NST-2, all issued after
    // everything else (loads complete in order)
    if (v + NST - 2 < n) wait_vmcnt<C::NI * (NST - 2)>();
    else wait_vmcnt<0>();
    barrier_keep_loads();                                   // everyone's have; the oldest stage is free
    flush();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);                // the stores stay ahead of the next loads
    __builtin_amdgcn_sched_barrier(0);
    if (v + NST - 1 < n) issue(st == 0 ? NST - 1 : st - 1);
    if (kc == KC) {
      kc = 0;
      ++i;
      cur_next(ccur);
      item_of(ccur, ci);
      if (C::NV) nv_tensor_scales(pool, S, ci.slot, K, N, GATED, ts0, ts1);
    }
    compute(kc, st);
    if (kc == KC - 1 || v == n - 1) {
      finish_item(i);
#pragma unroll
      for (int q = 0; q < C::NACC; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    ++kc;
    st = st + 1 == NST ? 0 : st + 1;
  }
  flush();
  if (has_first) {
    f32x4_t* p = part_tile<C::NACC>(part, b, i_first, U, G, KC, wave);
#pragma unroll
    for (int q = 0; q < C::NACC; ++q) p[q * 64 + lane] = first_part[q];
  }
  if (has_last) {
    f32x4_t* p = part_tile<C::NACC>(part, b, last_i, U, G, KC, wave);
#pragma unroll
    for (int q = 0; q < C::NACC; ++q) p[q * 64 + lane] = last_part[q];
  }
}

// Items cut by range boundaries of a gemm_dec launch of `grid` workgroups:
// workgroup j looks at the boundary between ranges j-1 and j; if it cuts an
// item and is the first boundary inside it, the workgroup adds the item's
// partial tiles in workgroup order and applies the epilogue.
template <int FMT, bool GATED, int NS>
__global__ void __launch_bounds__(256)
gemm_dec_fix(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
             const uint8_t* __restrict__ pool, size_t S, int K, int N, int grid, void* __restrict__ out,
             const f32x4_t* __restrict__ part) {
  using C = Cfg<FMT, GATED, NS>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ntiles = N / ROWS;
  const int KC = (K + C::CK - 1) / C::CK;
  const long U = (long)wl->n_mblk * ntiles * KC;
  const long G = U < (long)grid ? U : (long)grid;
  const long j = blockIdx.x;
  if (j < 1 || j >= G) return;
  const long ub = range_start(j, U, G);
  const int i = (int)(ub / KC);
  if (ub == (long)i * KC) return;                      // boundary between items
  const long bf = owner_of((long)i * KC, U, G);
  if (bf != j - 1) return;                             // an earlier boundary owns the item
  const long bl = owner_of((long)(i + 1) * KC - 1, U, G);
  f32x4_t acc[C::NACC];
#pragma unroll
  for (int q = 0; q < C::NACC; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (long bb = bf; bb <= bl; ++bb) {
    const f32x4_t* src = part_tile<C::NACC>((f32x4_t*)part, bb, i, U, G, KC, wave);
#pragma unroll
    for (int q = 0; q < C::NACC; ++q) acc[q] += src[q * 64 + lane];
  }
  Item it;
  decode_global(wl, counts, offsets, ntiles, C::MB, i, it);
  float ts0 = 1.0f, ts1 = 1.0f;
  if (C::NV) nv_tensor_scales(pool, S, it.slot, K, N, GATED, ts0, ts1);
  f32x4_t val[NS];
  activate<GATED, NS, C::NV>(acc, val, ts0, ts1);
  store_out<FMT, GATED, NS>(val, it, wave, lane, N, out);
}

namespace {

template <int FMT, bool GATED, int NS>
hipError_t launch_dec(int n_cu, const WorkList* wl, const int32_t* counts, const int32_t* offsets,
                      const uint8_t* pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                      const void* X, const void* Xs, const int32_t* row_tok, int K, int N, void* out, f32x4_t* part,
                      size_t part_bytes, int fix, int* err, hipStream_t s) {
  using C = Cfg<FMT, GATED, NS>;
  static int per_cu = 0;     // resident workgroups per CU for this instance
  const size_t lds = (size_t)C::NST * C::STAGE;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_dec<FMT, GATED, NS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, gemm_dec<FMT, GATED, NS>, 256, lds) != hipSuccess || nb < 1)
      nb = 1;
    per_cu = nb;
  }
  int grid = n_cu * per_cu;
  if (grid > MAX_BLOCKS) grid = MAX_BLOCKS - MAX_BLOCKS % N_XCD;
  // the partial tiles of 2 items per workgroup must fit the caller's buffer
  const size_t per_wg = (size_t)2 * NW * C::NACC * 64 * sizeof(f32x4_t);
  if (fix >= 0 && (size_t)grid * per_wg > part_bytes) {
    grid = (int)(part_bytes / per_wg);
    if (grid >= N_XCD) grid -= grid % N_XCD;
    if (grid < 1) return hipErrorInvalidValue;
  }
  if (fix < 0)      // one workgroup per item: a grid of -fix workgroups, no partial tiles
    gemm_dec<FMT, GATED, NS><<<-fix, 256, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                                    (const uint8_t*)X, (const uint8_t*)Xs, row_tok, K, N, out,
                                                    nullptr, err);
  else if (fix)
    gemm_dec_fix<FMT, GATED, NS><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, K, N, grid, out, part);
  else
    gemm_dec<FMT, GATED, NS><<<grid, 256, lds, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                                    (const uint8_t*)X, (const uint8_t*)Xs, row_tok, K, N, out, part,
                                                    err);
  return hipGetLastError();
}

template <int FMT, bool GATED>
hipError_t launch_ns(int ns, int n_cu, const WorkList* wl, const int32_t* counts, const int32_t* offsets,
                     const uint8_t* pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                     const void* X, const void* Xs, const int32_t* row_tok, int K, int N, void* out, f32x4_t* part,
                     size_t part_bytes, int fix, int* err, hipStream_t s) {
#define MOE_DEC_ARGS n_cu, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X, Xs, row_tok, K, N, out, part, part_bytes, fix, err, s
  if (ns == 1) return launch_dec<FMT, GATED, 1>(MOE_DEC_ARGS);
  if (ns == 2) return launch_dec<FMT, GATED, 2>(MOE_DEC_ARGS);
  if constexpr (FMT != WFMT_MXFP4 && FMT != WFMT_FP8_A16) {     // 64-token blocks exceed LDS there
    if (ns == 4) return launch_dec<FMT, GATED, 4>(MOE_DEC_ARGS);
  }
#undef MOE_DEC_ARGS
  return hipErrorInvalidValue;
}

}  // namespace

// Bytes of a partial-tile buffer that never limits the grid.
extern "C" size_t moe_dec_part_bytes() { return (size_t)MAX_BLOCKS * 2 * NW * 8 * 64 * sizeof(f32x4_t); }
// Largest tokens-per-m-block choice (16 * ns) for a weight format.
extern "C" int moe_dec_max_ns(int fmt) { return fmt == WFMT_MXFP4 || fmt == WFMT_FP8_A16 ? 2 : 4; }

// ns: 16-token sub-tiles per m-block (1, 2 or 4; 1 or 2 for MXFP4); the work
// list must have been built with m-blocks of 16*ns tokens.  N must be a
// multiple of 64; K a multiple of 128.  For the 8-bit formats X holds the
// quantised rows in grouped order (row_tok must be null).  The stream leaves
// the items cut between workgroups as partial tiles in `part` (part_bytes
// long: a smaller buffer caps the grid at the workgroups whose tiles fit);
// the same call with fix = 1 (same arguments, next on the stream) adds and
// stores them.
// fix = -n: one workgroup per item on a grid of n workgroups (n at least the
// number of items, else bit 1 of *err is set and nothing is written), no
// partial tiles and no second call.
extern "C" hipError_t moe_launch_gemm_dec(int fmt, int gated, int ns, int n_cu, const WorkList* wl,
                                          const int32_t* counts, const int32_t* offsets, const uint8_t* pool,
                                          size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                                          const void* X, const void* Xs, const int32_t* row_tok, int K, int N,
                                          void* out, void* part, size_t part_bytes, int fix, int* err,
                                          hipStream_t s) {
  const bool x16 = fmt == WFMT_BF16 || fmt == WFMT_NVFP4 || fmt == WFMT_FP8_A16 || fmt == WFMT_MXFP4_A16;
  if (N % ROWS || K % 128 || (!x16 && row_tok)) return hipErrorInvalidValue;
  f32x4_t* p = (f32x4_t*)part;
  const int f = fix;
#define MOE_DEC_ARGS ns, n_cu, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X, Xs, row_tok, K, N, out, p, part_bytes, f, err, s
  if (fmt == WFMT_BF16) return gated ? launch_ns<WFMT_BF16, true>(MOE_DEC_ARGS) : launch_ns<WFMT_BF16, false>(MOE_DEC_ARGS);
  if (fmt == WFMT_FP8) return gated ? launch_ns<WFMT_FP8, true>(MOE_DEC_ARGS) : launch_ns<WFMT_FP8, false>(MOE_DEC_ARGS);
  if (fmt == WFMT_NVFP4)
    return gated ? launch_ns<WFMT_NVFP4, true>(MOE_DEC_ARGS) : launch_ns<WFMT_NVFP4, false>(MOE_DEC_ARGS);
  if (fmt == WFMT_FP8_A16)
    return gated ? launch_ns<WFMT_FP8_A16, true>(MOE_DEC_ARGS) : launch_ns<WFMT_FP8_A16, false>(MOE_DEC_ARGS);
  if (fmt == WFMT_MXFP4_A16)
    return gated ? launch_ns<WFMT_MXFP4_A16, true>(MOE_DEC_ARGS) : launch_ns<WFMT_MXFP4_A16, false>(MOE_DEC_ARGS);
  if (fmt != WFMT_MXFP4) return hipErrorInvalidValue;
  return gated ? launch_ns<WFMT_MXFP4, true>(MOE_DEC_ARGS) : launch_ns<WFMT_MXFP4, false>(MOE_DEC_ARGS);
#undef MOE_DEC_ARGS
}
