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
// read once.  A work item is (expert, m-block of <= 64 tokens, 16*4/SPLIT
// weight rows).  Each 16-row tile is streamed by SPLIT waves that split K
// (chunks of 128 taken round-robin); weights go straight from HBM into MFMA
// operand registers (each weight byte is used by one wave, so no LDS), the
// next chunk's weights are in flight while the current chunk is multiplied,
// and the SPLIT partial sums are added through LDS in a fixed wave order so
// the result does not depend on scheduling.  The grid holds exactly the
// resident workgroups and strides over the device work list, so no host
// synchronisation is needed and no workgroup starts late.
//
// MFMA operand mapping (v_mfma_f32_16x16x32_bf16): lane l feeds row l%16 of
// A (16 weight rows) and column l%16 of B (16 tokens), with the 8 K values of
// lane group l/16.  Because a contraction is invariant under a common
// permutation of K, lane group g takes the 32 consecutive K values
// [chunk + 32g, chunk + 32g + 32) spread over four MFMAs (8 per MFMA): each
// lane then reads 64 contiguous bytes of its weight row per 128-K chunk.
// Result lane l holds rows 4*(l/16)..+3 (weight rows) of column l%16 (token).
//
// fp8 (E4M3, 128x128 fp32 block scales): v_mfma_scale_f32_16x16x128_f8f6f4
// with unit E8M0 scales; one instruction covers one 128-K block, whose
// partial sum is multiplied by w_scale[block] * x_scale[token, block].
// MXFP4: the same instruction with E2M1 weights (A) and MXFP8 activations
// (B).  Lane layout of that instruction (measured on gfx950 with one-hot
// inputs): an E2M1 operand's lane group g = l/16 holds the 32 consecutive K
// values [32g, 32g+32) in its low 16 bytes; an 8-bit operand's lane group g
// holds K [16g, 16g+16) in bytes 0-15 and K [64+16g, 64+16g+16) in bytes
// 16-31; the E8M0 scale of lane group g covers K block [32g, 32g+32) of
// that lane's row (A) or column (B).  With uniform scales (the fp8 path)
// the 8-bit layout only has to agree between A and B, so both take 32
// consecutive bytes there.
#include "common.h"

namespace {

constexpr int NWAVE = 4;

// Gathered row of X for token sub-tile ms, lane column c: returns the source
// row index or -1.
DEV int src_row(const int32_t* row_tok, int row0, int nrows, int ms, int c) {
  const int r = ms * 16 + c;
  if (r >= nrows) return -1;
  return row_tok ? row_tok[row0 + r] : row0 + r;
}

DEV float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

DEV i32x8_t cat(i32x4_t lo, i32x4_t hi) { return i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; }

// Per-format pieces: what one lane loads for one 128-K chunk of one weight
// row, what it loads for one token row, and the MFMA(s) that combine them.
struct Bf16 {
  struct W { i32x4_t v[4]; };
  struct X { i32x4_t v[4]; };
  // row pointer at the weight row; kb = chunk K offset (elements)
  static DEV void load_w(W& w, const uint8_t* row, size_t, int kb, int lg) {
    const uint16_t* p = (const uint16_t*)row + kb + lg * 32;
#pragma unroll
    for (int s = 0; s < 4; ++s) w.v[s] = ld16(p + s * 8);
  }
  static DEV void load_x(X& x, const void* base, const void*, int row, int K, int kb, int, int lg) {
    const uint16_t* p = (const uint16_t*)base + (size_t)row * K + kb + lg * 32;
#pragma unroll
    for (int s = 0; s < 4; ++s) x.v[s] = ld16(p + s * 8);
  }
  static DEV void zero_x(X& x) {
#pragma unroll
    for (int s = 0; s < 4; ++s) x.v[s] = i32x4_t{0, 0, 0, 0};
  }
  static DEV void mma(f32x4_t& acc, const W& w, const X& x, float) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w.v[s]),
                                                    __builtin_bit_cast(bf16x8_t, x.v[s]), acc, 0, 0, 0);
  }
};

struct Fp8 {
  struct W { i32x8_t v; float s; };
  struct X { i32x8_t v; float s; };
  // scale row pointer is passed as `srow` (fp32 [N/128][K/128], row block of the tile)
  static DEV void load_w(W& w, const uint8_t* row, size_t, int kb, int lg) {
    const uint8_t* p = row + kb + lg * 32;
    w.v = cat(ld16(p), ld16(p + 16));
  }
  static DEV void load_x(X& x, const void* base, const void* sbase, int row, int K, int kb, int c, int lg) {
    const uint8_t* p = (const uint8_t*)base + (size_t)row * K + kb + lg * 32;
    x.v = cat(ld16(p), ld16(p + 16));
    x.s = ((const float*)sbase)[(size_t)row * (K / 128) + c];
  }
  static DEV void zero_x(X& x) {
    x.v = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    x.s = 0.0f;
  }
  static DEV void mma(f32x4_t& acc, const W& w, const X& x, float ws) {
    const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.v, x.v, z4, 0, 0, 0, 127, 0, 127);
    const float f = ws * x.s;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += p[i] * f;
  }
};

struct Mxfp4 {
  struct W { i32x4_t v; int s; };
  struct X { i32x8_t v; int s; };
  static DEV void load_w(W& w, const uint8_t* row, size_t, int kb, int lg) { w.v = ld16(row + kb / 2 + lg * 16); }
  static DEV void load_x(X& x, const void* base, const void* sbase, int row, int K, int kb, int c, int lg) {
    // 8-bit operand: bytes 0-15 = K [16g, 16g+16), bytes 16-31 = K [64+16g, 64+16g+16)
    const uint8_t* p = (const uint8_t*)base + (size_t)row * K + kb + lg * 16;
    x.v = cat(ld16(p), ld16(p + 64));
    x.s = ((const uint8_t*)sbase)[(size_t)row * (K / 32) + c * 4 + lg];
  }
  static DEV void zero_x(X& x) {
    x.v = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    x.s = 127;
  }
  static DEV void mma(f32x4_t& acc, const W& w, const X& x, float) {
    const i32x8_t a = i32x8_t{w.v[0], w.v[1], w.v[2], w.v[3], 0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, x.v, acc, 4, 0, 0, w.s, 0, x.s);
  }
};

// Weight-side scale of chunk c for the lane's row.
template <class F>
DEV void load_wscale(typename F::W& w, const uint8_t* srow, int c, int lg);
template <>
DEV void load_wscale<Bf16>(Bf16::W&, const uint8_t*, int, int) {}
template <>
DEV void load_wscale<Fp8>(Fp8::W& w, const uint8_t* srow, int c, int) { w.s = ((const float*)srow)[c]; }
template <>
DEV void load_wscale<Mxfp4>(Mxfp4::W& w, const uint8_t* srow, int c, int lg) { w.s = srow[c * 4 + lg]; }

template <class F>
DEV float wscale(const typename F::W& w);
template <>
DEV float wscale<Bf16>(const Bf16::W&) { return 1.0f; }
template <>
DEV float wscale<Fp8>(const Fp8::W& w) { return w.s; }
template <>
DEV float wscale<Mxfp4>(const Mxfp4::W&) { return 1.0f; }

}  // namespace

// FMT: WFMT_*.  GATED: GEMM 1 (gate rows at woff0, up rows at woff1, SwiGLU
// epilogue; out = A, bf16 for WFMT_BF16 else fp32 for the quantisation pass).
// Otherwise GEMM 2 (weights at woff0; out = Z bf16).  X rows are gathered
// through row_tok (GEMM 1) or taken in grouped order (GEMM 2); Xs holds the
// activation scales of the 8-bit formats.  soff0/soff1: weight scale arrays.
template <int FMT, bool GATED, int SPLIT>
__global__ void __launch_bounds__(256)
gemm_dec(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
         const uint8_t* __restrict__ pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
         const void* __restrict__ X, const void* __restrict__ Xs, const int32_t* __restrict__ row_tok, int K, int N,
         void* __restrict__ out) {
  using F = typename std::conditional<FMT == WFMT_BF16, Bf16,
                                      typename std::conditional<FMT == WFMT_FP8, Fp8, Mxfp4>::type>::type;
  constexpr int TILES = NWAVE / SPLIT;          // 16-row tiles per work item
  constexpr int NACC = GATED ? 8 : 4;
  __shared__ float red[(SPLIT > 1 ? (SPLIT - 1) * TILES : 1) * NACC * 4 * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int tw = wave / SPLIT, ks = wave - tw * SPLIT;
  const int rows_item = 16 * TILES;
  const int ntiles = N / rows_item;
  const int nitems = wl->n_mblk * ntiles;
  const int nchunk = K / 128;
  // bytes per weight row and per scale row of one matrix
  const size_t wrow_bytes = FMT == WFMT_BF16 ? (size_t)K * 2 : (FMT == WFMT_FP8 ? (size_t)K : (size_t)K / 2);
  const int last = nchunk - 1 - ((nchunk - 1 - ks) % SPLIT);   // this wave's last chunk (if ks < nchunk)

  // the work list in LDS: an item's expert is then found without a chain of
  // dependent global loads in front of its first weight load
  __shared__ int l_pref[257], l_slot[256], l_row0[256], l_cnt[256];
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

  for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
    const int p = it / ntiles, nt = it - p * ntiles;
    int a = 0;
    {
      int hi = n_act - 1;
      while (a < hi) {
        const int mid = (a + hi + 1) >> 1;
        if (l_pref[mid] <= p) a = mid; else hi = mid - 1;
      }
    }
    const int slot = l_slot[a];
    const int mb = p - l_pref[a];
    const int row0 = l_row0[a] + mb * DEC_MB;
    const int nrows = min(DEC_MB, l_cnt[a] - mb * DEC_MB);
    const int n0 = nt * rows_item + tw * 16;
    const uint8_t* wbase = pool + (size_t)slot * S;
    const int wr = n0 + lr;                                   // this lane's weight row
    const uint8_t* w0 = wbase + woff0 + (size_t)wr * wrow_bytes;
    const uint8_t* w1 = wbase + woff1 + (size_t)wr * wrow_bytes;
    const uint8_t* s0 = nullptr;
    const uint8_t* s1 = nullptr;
    if (FMT == WFMT_FP8) {
      s0 = wbase + soff0 + (size_t)(n0 / 128) * (K / 128) * 4;
      s1 = wbase + soff1 + (size_t)(n0 / 128) * (K / 128) * 4;
    } else if (FMT == WFMT_MXFP4) {
      s0 = wbase + soff0 + (size_t)wr * (K / 32);
      s1 = wbase + soff1 + (size_t)wr * (K / 32);
    }
    int xr[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) xr[ms] = src_row(row_tok, row0, nrows, ms, lr);
    const int nms = (nrows + 15) >> 4;
    f32x4_t acc[NACC];
#pragma unroll
    for (int q = 0; q < NACC; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // loads are unconditional: past the wave's last chunk they re-read that
    // chunk (a cache hit, unused), so no branch drains the memory counter
    auto loadw = [&](int c, typename F::W& ga, typename F::W& ua) {
      const int cc = min(c, last);
      F::load_w(ga, w0, wrow_bytes, cc * 128, lg);
      load_wscale<F>(ga, s0, cc, lg);
      if (GATED) {
        F::load_w(ua, w1, wrow_bytes, cc * 128, lg);
        load_wscale<F>(ua, s1, cc, lg);
      }
    };
    auto compute = [&](int c, const typename F::W& ga, const typename F::W& ua) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= nms) break;
        typename F::X xb;
        F::load_x(xb, X, Xs, max(xr[ms], 0), K, c * 128, c, lg);
        if (xr[ms] < 0) F::zero_x(xb);
        F::mma(acc[ms], ga, xb, wscale<F>(ga));
        if (GATED) F::mma(acc[4 + ms], ua, xb, wscale<F>(ua));
      }
    };
    if (ks < nchunk) {
      typename F::W g0, u0, g1, u1;
      loadw(ks, g0, u0);
      for (int c = ks; c <= last; c += 2 * SPLIT) {
        loadw(c + SPLIT, g1, u1);
        compute(c, g0, u0);
        if (c + SPLIT > last) break;
        loadw(c + 2 * SPLIT, g0, u0);
        compute(c + SPLIT, g1, u1);
      }
    }

    // partial sums of the SPLIT waves of a tile, added in wave order
    if (SPLIT > 1) {
      if (ks > 0) {
#pragma unroll
        for (int q = 0; q < NACC; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[(((tw * (SPLIT - 1) + ks - 1) * NACC + q) * 4 + i) * 64 + lane] = acc[q][i];
      }
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int w = 1; w < SPLIT; ++w)
#pragma unroll
          for (int q = 0; q < NACC; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[q][i] += red[(((tw * (SPLIT - 1) + w - 1) * NACC + q) * 4 + i) * 64 + lane];
      }
      __syncthreads();
    }
    if (ks == 0) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const int r = ms * 16 + lr;
        if (r >= nrows) continue;
        const size_t o = (size_t)(row0 + r) * N + n0 + lg * 4;
        if (GATED && FMT != WFMT_BF16) {
          float4 v;
          v.x = silu_mul(acc[ms][0], acc[4 + ms][0]);
          v.y = silu_mul(acc[ms][1], acc[4 + ms][1]);
          v.z = silu_mul(acc[ms][2], acc[4 + ms][2]);
          v.w = silu_mul(acc[ms][3], acc[4 + ms][3]);
          *(float4*)((float*)out + o) = v;
        } else {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = GATED ? silu_mul(acc[ms][i], acc[4 + ms][i]) : acc[ms][i];
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
          st8((uint16_t*)out + o, pk);
        }
      }
    }
  }
}

namespace {

template <int FMT, bool GATED, int SPLIT>
hipError_t launch_dec(int n_cu, const WorkList* wl, const int32_t* counts, const int32_t* offsets,
                      const uint8_t* pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                      const void* X, const void* Xs, const int32_t* row_tok, int K, int N, void* out, hipStream_t s) {
  static int per_cu = 0;     // resident workgroups per CU for this instance
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, gemm_dec<FMT, GATED, SPLIT>, 256, 0) != hipSuccess ||
        nb < 1)
      nb = 2;
    per_cu = nb;
  }
  gemm_dec<FMT, GATED, SPLIT><<<n_cu * per_cu, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                                             X, Xs, row_tok, K, N, out);
  return hipGetLastError();
}

template <int FMT, bool GATED>
hipError_t launch_split(int split, int n_cu, const WorkList* wl, const int32_t* counts, const int32_t* offsets,
                        const uint8_t* pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                        const void* X, const void* Xs, const int32_t* row_tok, int K, int N, void* out,
                        hipStream_t s) {
  if (split == 1)
    return launch_dec<FMT, GATED, 1>(n_cu, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X, Xs, row_tok,
                                     K, N, out, s);
  if (split == 2)
    return launch_dec<FMT, GATED, 2>(n_cu, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X, Xs, row_tok,
                                     K, N, out, s);
  return launch_dec<FMT, GATED, 4>(n_cu, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X, Xs, row_tok, K,
                                   N, out, s);
}

}  // namespace

// split: waves sharing one 16-row tile's K (1, 2 or 4); N must be a multiple
// of 16*4/split.
extern "C" hipError_t moe_launch_gemm_dec(int fmt, int gated, int split, int n_cu, const WorkList* wl,
                                          const int32_t* counts, const int32_t* offsets, const uint8_t* pool,
                                          size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                                          const void* X, const void* Xs, const int32_t* row_tok, int K, int N,
                                          void* out, hipStream_t s) {
#define MOE_DEC_ARGS split, n_cu, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X, Xs, row_tok, K, N, out, s
  if (fmt == WFMT_BF16) return gated ? launch_split<WFMT_BF16, true>(MOE_DEC_ARGS) : launch_split<WFMT_BF16, false>(MOE_DEC_ARGS);
  if (fmt == WFMT_FP8) return gated ? launch_split<WFMT_FP8, true>(MOE_DEC_ARGS) : launch_split<WFMT_FP8, false>(MOE_DEC_ARGS);
  return gated ? launch_split<WFMT_MXFP4, true>(MOE_DEC_ARGS) : launch_split<WFMT_MXFP4, false>(MOE_DEC_ARGS);
#undef MOE_DEC_ARGS
}
