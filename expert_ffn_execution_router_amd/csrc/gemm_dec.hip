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
// read once.  A work item is (expert, m-block of <= 64 tokens, 16 weight
// rows); its four waves split K and stream weights straight from HBM into
// MFMA operand registers (no LDS for weights: each byte is used by one wave),
// then reduce their partial sums through LDS in a fixed order so the result
// does not depend on scheduling.  The grid is persistent and reads the item
// count from the device work list, so no host synchronisation is needed.
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

constexpr int NWAVE = 4;

// Gathered row of X for token sub-tile ms, lane column c: returns the source
// row index or -1.
DEV int src_row(const int32_t* row_tok, int row0, int nrows, int ms, int c) {
  const int r = ms * 16 + c;
  if (r >= nrows) return -1;
  return row_tok ? row_tok[row0 + r] : row0 + r;
}

// Cross-wave reduction of NACC f32x4 accumulators per lane: waves 1..3 store,
// wave 0 adds them in wave order.  Returns true on wave 0.
template <int NACC>
DEV bool reduce_waves(f32x4_t (&acc)[NACC], float* red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(((wave - 1) * NACC + a) * 4 + i) * 64 + lane] = acc[a][i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < NWAVE; ++w)
#pragma unroll
      for (int a = 0; a < NACC; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[a][i] += red[(((w - 1) * NACC + a) * 4 + i) * 64 + lane];
  }
  __syncthreads();
  return wave == 0;
}

DEV float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Item decoding shared by all formats.
struct Item {
  int e, slot, row0, nrows, n0;
};

DEV bool decode_item(const WorkList* wl, const int32_t* counts, const int32_t* offsets, int ntiles, int it,
                     Item& o) {
  const int p = it / ntiles, nt = it - p * ntiles;
  const int a = find_active(wl, p);
  o.e = wl->act_e[a];
  o.slot = wl->act_slot[a];
  const int mb = p - wl->mblk_prefix[a];
  o.row0 = offsets[o.e] + mb * DEC_MB;
  o.nrows = min(DEC_MB, counts[o.e] - mb * DEC_MB);
  o.n0 = nt * DEC_NT;
  return true;
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------
// GATED: GEMM 1 (gate and up rows, SwiGLU epilogue, out = A [rows, N]).
// Otherwise GEMM 2 (out = Z [rows, N]).  X rows are gathered through row_tok
// (GEMM 1: token of each grouped row) or taken in grouped order (GEMM 2).
template <bool GATED>
__global__ void __launch_bounds__(256)
gemm_dec_bf16(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts,
              const int32_t* __restrict__ offsets, const uint8_t* __restrict__ pool, size_t S,
              size_t woff0, size_t woff1, const uint16_t* __restrict__ X, const int32_t* __restrict__ row_tok,
              int K, int N, uint16_t* __restrict__ out) {
  constexpr int NACC = GATED ? 8 : 4;
  __shared__ float red[(NWAVE - 1) * NACC * 4 * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int ntiles = N / DEC_NT;
  const int nitems = wl->n_mblk * ntiles;
  const int nchunk = K / 128;
  for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
    Item t;
    decode_item(wl, counts, offsets, ntiles, it, t);
    const uint8_t* wbase = pool + (size_t)t.slot * S;
    const uint16_t* w0 = (const uint16_t*)(wbase + woff0) + (size_t)(t.n0 + lr) * K + lg * 32;
    const uint16_t* w1 = (const uint16_t*)(wbase + woff1) + (size_t)(t.n0 + lr) * K + lg * 32;
    int xr[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) xr[ms] = src_row(row_tok, t.row0, t.nrows, ms, lr);
    const int nms = (t.nrows + 15) >> 4;
    f32x4_t acc[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c = wave; c < nchunk; c += NWAVE) {
      const int kb = c * 128;
      i32x4_t wa[4], wb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) wa[s] = ld16(w0 + kb + s * 8);
      if (GATED) {
#pragma unroll
        for (int s = 0; s < 4; ++s) wb[s] = ld16(w1 + kb + s * 8);
      }
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= nms) break;
        i32x4_t xb[4];
        if (xr[ms] >= 0) {
          const uint16_t* xp = X + (size_t)xr[ms] * K + kb + lg * 32;
#pragma unroll
          for (int s = 0; s < 4; ++s) xb[s] = ld16(xp + s * 8);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) xb[s] = i32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          acc[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wa[s]),
                                                            __builtin_bit_cast(bf16x8_t, xb[s]), acc[ms], 0, 0, 0);
          if (GATED)
            acc[4 + ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wb[s]),
                                                                  __builtin_bit_cast(bf16x8_t, xb[s]), acc[4 + ms],
                                                                  0, 0, 0);
        }
      }
    }
    if (reduce_waves<NACC>(acc, red)) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const int r = ms * 16 + lr;
        if (r < t.nrows) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = GATED ? silu_mul(acc[ms][i], acc[4 + ms][i]) : acc[ms][i];
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
          st8(out + (size_t)(t.row0 + r) * N + t.n0 + lg * 4, pk);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp8 e4m3 weights with fp32 128x128 block scales; activations e4m3 with an
// fp32 scale per (row, 128 K).  GATED writes fp32 A (quantised by a separate
// pass), otherwise bf16 Z.
// ---------------------------------------------------------------------------
template <bool GATED>
__global__ void __launch_bounds__(256)
gemm_dec_fp8(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts,
             const int32_t* __restrict__ offsets, const uint8_t* __restrict__ pool, size_t S,
             size_t woff0, size_t woff1, size_t soff0, size_t soff1, const uint8_t* __restrict__ Xq,
             const float* __restrict__ Xs, const int32_t* __restrict__ row_tok, int K, int N,
             void* __restrict__ out) {
  constexpr int NACC = GATED ? 8 : 4;
  __shared__ float red[(NWAVE - 1) * NACC * 4 * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int ntiles = N / DEC_NT;
  const int nitems = wl->n_mblk * ntiles;
  const int nchunk = K / 128;
  const int kbn = K / 128;   // K blocks per weight row block
  for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
    Item t;
    decode_item(wl, counts, offsets, ntiles, it, t);
    const uint8_t* wbase = pool + (size_t)t.slot * S;
    const uint8_t* w0 = wbase + woff0 + (size_t)(t.n0 + lr) * K + lg * 32;
    const uint8_t* w1 = wbase + woff1 + (size_t)(t.n0 + lr) * K + lg * 32;
    const float* s0 = (const float*)(wbase + soff0) + (size_t)(t.n0 / 128) * kbn;
    const float* s1 = (const float*)(wbase + soff1) + (size_t)(t.n0 / 128) * kbn;
    int xr[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) xr[ms] = src_row(row_tok, t.row0, t.nrows, ms, lr);
    const int nms = (t.nrows + 15) >> 4;
    f32x4_t acc[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c = wave; c < nchunk; c += NWAVE) {
      const int kb = c * 128;
      i32x8_t wa, wb;
      {
        const i32x4_t lo = ld16(w0 + kb), hi = ld16(w0 + kb + 16);
        wa = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      if (GATED) {
        const i32x4_t lo = ld16(w1 + kb), hi = ld16(w1 + kb + 16);
        wb = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      const float ws0 = s0[c];
      const float ws1 = GATED ? s1[c] : 0.0f;
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= nms) break;
        i32x8_t xb = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        float xs = 0.0f;
        if (xr[ms] >= 0) {
          const uint8_t* xp = Xq + (size_t)xr[ms] * K + kb + lg * 32;
          const i32x4_t lo = ld16(xp), hi = ld16(xp + 16);
          xb = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          xs = Xs[(size_t)xr[ms] * kbn + c];
        }
        const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
        const f32x4_t p0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xb, z4, 0, 0, 0, 127, 0, 127);
        const float f0 = ws0 * xs;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ms][i] += p0[i] * f0;
        if (GATED) {
          const f32x4_t p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb, xb, z4, 0, 0, 0, 127, 0, 127);
          const float f1 = ws1 * xs;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[4 + ms][i] += p1[i] * f1;
        }
      }
    }
    if (reduce_waves<NACC>(acc, red)) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const int r = ms * 16 + lr;
        if (r < t.nrows) {
          if (GATED) {
            float4 v;
            v.x = silu_mul(acc[ms][0], acc[4 + ms][0]);
            v.y = silu_mul(acc[ms][1], acc[4 + ms][1]);
            v.z = silu_mul(acc[ms][2], acc[4 + ms][2]);
            v.w = silu_mul(acc[ms][3], acc[4 + ms][3]);
            *(float4*)((float*)out + (size_t)(t.row0 + r) * N + t.n0 + lg * 4) = v;
          } else {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16_bits(acc[ms][0]) | ((uint32_t)f32_to_bf16_bits(acc[ms][1]) << 16);
            pk.y = (uint32_t)f32_to_bf16_bits(acc[ms][2]) | ((uint32_t)f32_to_bf16_bits(acc[ms][3]) << 16);
            st8((uint16_t*)out + (size_t)(t.row0 + r) * N + t.n0 + lg * 4, pk);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP4 weights (E2M1, E8M0 per 32 K) x MXFP8 activations (E4M3, E8M0 per 32)
// ---------------------------------------------------------------------------
template <bool GATED>
__global__ void __launch_bounds__(256)
gemm_dec_mxfp4(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts,
               const int32_t* __restrict__ offsets, const uint8_t* __restrict__ pool, size_t S,
               size_t woff0, size_t woff1, size_t soff0, size_t soff1, const uint8_t* __restrict__ Xq,
               const uint8_t* __restrict__ Xs, const int32_t* __restrict__ row_tok, int K, int N,
               void* __restrict__ out) {
  constexpr int NACC = GATED ? 8 : 4;
  __shared__ float red[(NWAVE - 1) * NACC * 4 * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int ntiles = N / DEC_NT;
  const int nitems = wl->n_mblk * ntiles;
  const int nchunk = K / 128;
  const int nsb = K / 32;     // scale blocks per row
  for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
    Item t;
    decode_item(wl, counts, offsets, ntiles, it, t);
    const uint8_t* wbase = pool + (size_t)t.slot * S;
    const uint8_t* w0 = wbase + woff0 + (size_t)(t.n0 + lr) * (K / 2) + lg * 16;
    const uint8_t* w1 = wbase + woff1 + (size_t)(t.n0 + lr) * (K / 2) + lg * 16;
    const uint8_t* s0 = wbase + soff0 + (size_t)(t.n0 + lr) * nsb + lg;
    const uint8_t* s1 = wbase + soff1 + (size_t)(t.n0 + lr) * nsb + lg;
    int xr[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) xr[ms] = src_row(row_tok, t.row0, t.nrows, ms, lr);
    const int nms = (t.nrows + 15) >> 4;
    f32x4_t acc[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int c = wave; c < nchunk; c += NWAVE) {
      const int kb = c * 128;
      const i32x4_t qa = ld16(w0 + kb / 2);
      const i32x8_t wa = i32x8_t{qa[0], qa[1], qa[2], qa[3], 0, 0, 0, 0};
      const int sa = s0[c * 4];
      i32x8_t wb = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      int sb = 127;
      if (GATED) {
        const i32x4_t qb = ld16(w1 + kb / 2);
        wb = i32x8_t{qb[0], qb[1], qb[2], qb[3], 0, 0, 0, 0};
        sb = s1[c * 4];
      }
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= nms) break;
        i32x8_t xb = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        int sx = 127;
        if (xr[ms] >= 0) {
          // 8-bit operand: bytes 0-15 = K [16g, 16g+16), bytes 16-31 = K [64+16g, 64+16g+16)
          const uint8_t* xp = Xq + (size_t)xr[ms] * K + kb + lg * 16;
          const i32x4_t lo = ld16(xp), hi = ld16(xp + 64);
          xb = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          sx = Xs[(size_t)xr[ms] * nsb + c * 4 + lg];
        }
        acc[ms] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, xb, acc[ms], 4, 0, 0, sa, 0, sx);
        if (GATED)
          acc[4 + ms] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb, xb, acc[4 + ms], 4, 0, 0, sb, 0, sx);
      }
    }
    if (reduce_waves<NACC>(acc, red)) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const int r = ms * 16 + lr;
        if (r < t.nrows) {
          if (GATED) {
            float4 v;
            v.x = silu_mul(acc[ms][0], acc[4 + ms][0]);
            v.y = silu_mul(acc[ms][1], acc[4 + ms][1]);
            v.z = silu_mul(acc[ms][2], acc[4 + ms][2]);
            v.w = silu_mul(acc[ms][3], acc[4 + ms][3]);
            *(float4*)((float*)out + (size_t)(t.row0 + r) * N + t.n0 + lg * 4) = v;
          } else {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16_bits(acc[ms][0]) | ((uint32_t)f32_to_bf16_bits(acc[ms][1]) << 16);
            pk.y = (uint32_t)f32_to_bf16_bits(acc[ms][2]) | ((uint32_t)f32_to_bf16_bits(acc[ms][3]) << 16);
            st8((uint16_t*)out + (size_t)(t.row0 + r) * N + t.n0 + lg * 4, pk);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers (grid: persistent, sized from the device count by the caller)
// ---------------------------------------------------------------------------
extern "C" hipError_t moe_launch_gemm_dec(int fmt, int gated, int grid, const WorkList* wl, const int32_t* counts,
                                          const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0,
                                          size_t woff1, size_t soff0, size_t soff1, const void* X, const void* Xs,
                                          const int32_t* row_tok, int K, int N, void* out, hipStream_t s) {
  if (fmt == WFMT_BF16) {
    if (gated)
      gemm_dec_bf16<true><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X,
                                               row_tok, K, N, (uint16_t*)out);
    else
      gemm_dec_bf16<false><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X,
                                                row_tok, K, N, (uint16_t*)out);
  } else if (fmt == WFMT_FP8) {
    if (gated)
      gemm_dec_fp8<true><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                              (const uint8_t*)X, (const float*)Xs, row_tok, K, N, out);
    else
      gemm_dec_fp8<false><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                               (const uint8_t*)X, (const float*)Xs, row_tok, K, N, out);
  } else {
    if (gated)
      gemm_dec_mxfp4<true><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                                (const uint8_t*)X, (const uint8_t*)Xs, row_tok, K, N, out);
    else
      gemm_dec_mxfp4<false><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                                 (const uint8_t*)X, (const uint8_t*)Xs, row_tok, K, N, out);
  }
  return hipGetLastError();
}
