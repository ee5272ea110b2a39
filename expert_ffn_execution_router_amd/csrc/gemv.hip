// Slot-indexed grouped expert GEMMs for the smallest batches (at most 4
// tokens per expert), bf16 weights, as matrix-vector products on the
// vector ALUs.
//
// Method (paper.oopus.info review of FreeToken, section 2.5: the GPU
// evaluates every expert of G = H u F for the tokens routed to it; SwiGLU
// expert): the same two GEMMs as the small-batch MFMA kernel,
//   GEMM 1: A = silu(x W_gate^T) * (x W_up^T), rounded to bf16,
//   GEMM 2: Z = A W_down^T, rounded to bf16,
// with fp32 products and sums.  With one to four tokens an expert's weight
// rows are each used one to four times: the work is the weight stream.
// The MFMA kernel moves every weight through LDS and multiplies 16-token
// tiles that are almost all padding; here each weight is loaded once into
// registers and multiplied by the token values it meets.
//   * an item is (active expert, 16 weight rows): for GEMM 1 the gate and up
//     rows of 8 features, for GEMM 2 16 output columns; one workgroup of
//     4 waves per item, each wave 4 rows;
//   * a row is read by 16 consecutive lanes, 16 bytes each per step, so one
//     wave instruction covers four 256-byte row segments (the pattern that
//     streams HBM fastest with the nontemporal hint); lane i takes the bytes
//     [256 s + 16 i, +16) of its row at step s, and the same K range of
//     each token row (cached: every item of the expert reads it);
//   * the 16 partial sums of a row are added across the lanes with four
//     DPP moves (xor 1, xor 2, rotate 4, rotate 8 inside the 16-lane row);
//     GEMM 1's up sums move to the gate lanes with one lane shuffle.
#include "common.h"

namespace {

constexpr int GV_MAXT = 4;      // tokens per expert
constexpr int GV_BLK = 8;       // 16-byte steps in flight per lane

DEV float dpp_add(float v, int ctrl_sel) {
  int x = __float_as_int(v);
  int y;
  switch (ctrl_sel) {
    case 0: y = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;    // quad_perm 1,0,3,2
    case 1: y = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;    // quad_perm 2,3,0,1
    case 2: y = __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false); break;   // row_ror:4
    default: y = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false); break;  // row_ror:8
  }
  return v + __int_as_float(y);
}

// Sum over the 16 lanes of a DPP row, in every lane of the row.
DEV float row16_sum(float v) {
  v = dpp_add(v, 0);
  v = dpp_add(v, 1);
  v = dpp_add(v, 2);
  return dpp_add(v, 3);
}

// acc += the 8 products of weights w and tokens x (bf16 pairs, exact fp32
// products, fp32 sums in element order).
DEV float dot8(i32x4_t w, i32x4_t x, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = (uint32_t)w[q], b = (uint32_t)x[q];
    acc = fmaf(__uint_as_float(a << 16), __uint_as_float(b << 16), acc);
    acc = fmaf(__uint_as_float(a & 0xffff0000u), __uint_as_float(b & 0xffff0000u), acc);
  }
  return acc;
}

DEV float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace

// GATED: out = A (bf16 [rows, N], N = I) from X = the hidden rows (bf16
// [T, K]) gathered through row_tok, weights gate at woff0 and up at woff1.
// Otherwise out = Z (bf16 [rows, N], N = H) from X = A in grouped order,
// weights at woff0.  Rows of expert e are offsets[e] .. + counts[e] <= 4.
// K % 128 == 0; N % 8 (gated) or 16.  The grid may exceed the items
// (n_act * N / 8 or N / 16): the extra workgroups leave at once.
template <bool GATED>
__global__ void __launch_bounds__(256)
gemv_bf16(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
          const uint8_t* __restrict__ pool, size_t S, size_t woff0, size_t woff1, const uint16_t* __restrict__ X,
          const int32_t* __restrict__ row_tok, int K, int N, uint16_t* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int per_e = GATED ? N / 8 : N / 16;          // items per expert
  const int it = blockIdx.x;
  if (it >= wl->n_act * per_e) return;
  const int a = it / per_e, blk = it - a * per_e;
  const int e = wl->act_e[a];
  const uint8_t* blob = pool + (size_t)wl->act_slot[a] * S;
  const int row0 = offsets[e], cnt = min(counts[e], GV_MAXT);
  // this lane group's weight row
  int wrow, feat;
  const uint8_t* wbase;
  if (GATED) {
    feat = blk * 8 + 2 * wave + (g & 1);
    wbase = blob + ((g >> 1) ? woff1 : woff0);
    wrow = feat;
  } else {
    feat = blk * 16 + 4 * wave + g;
    wbase = blob + woff0;
    wrow = feat;
  }
  const uint8_t* wr = wbase + (size_t)wrow * K * 2 + li * 16;
  const uint8_t* xr[GV_MAXT];
#pragma unroll
  for (int t = 0; t < GV_MAXT; ++t) {
    const int r = row0 + min(t, cnt - 1);
    const int xrow = GATED ? row_tok[r] : r;
    xr[t] = (const uint8_t*)X + (size_t)xrow * K * 2 + li * 16;
  }
  float acc[GV_MAXT] = {0.f, 0.f, 0.f, 0.f};
  const int nstep = K / 128;                          // 256-byte segments per row
  for (int s0 = 0; s0 < nstep; s0 += GV_BLK) {
    i32x4_t wv[GV_BLK];
#pragma unroll
    for (int j = 0; j < GV_BLK; ++j)
      if (s0 + j < nstep) wv[j] = ld16_nt(wr + (s0 + j) * 256);
#pragma unroll
    for (int t = 0; t < GV_MAXT; ++t) {
      if (t >= cnt) break;
#pragma unroll
      for (int j = 0; j < GV_BLK; ++j)
        if (s0 + j < nstep) acc[t] = dot8(wv[j], ld16(xr[t] + (s0 + j) * 256), acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < GV_MAXT; ++t) acc[t] = row16_sum(acc[t]);
  if (GATED) {
    // lane groups 0/1 hold the gate sums of features 2w, 2w+1; groups 2/3
    // the up sums of the same features, 32 lanes on
#pragma unroll
    for (int t = 0; t < GV_MAXT; ++t) {
      const float u = __shfl_down(acc[t], 32, 64);
      if (t < cnt && g < 2 && li == 0)
        out[(size_t)(row0 + t) * N + feat] = f32_to_bf16_bits(silu_mul(acc[t], u));
    }
  } else {
#pragma unroll
    for (int t = 0; t < GV_MAXT; ++t)
      if (t < cnt && li == 0) out[(size_t)(row0 + t) * N + feat] = f32_to_bf16_bits(acc[t]);
  }
}

// grid: at least the items (active experts x N / 8 for GEMM 1, N / 16 for
// GEMM 2); every expert must have at most 4 routed rows.
extern "C" hipError_t moe_launch_gemv(int gated, int grid, const WorkList* wl, const int32_t* counts,
                                      const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0,
                                      size_t woff1, const void* X, const int32_t* row_tok, int K, int N, void* out,
                                      hipStream_t s) {
  if (grid < 1 || K % 128 || N % (gated ? 8 : 16) || (gated && !row_tok)) return hipErrorInvalidValue;
  if (gated)
    gemv_bf16<true><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X, row_tok,
                                         K, N, (uint16_t*)out);
  else
    gemv_bf16<false><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, (const uint16_t*)X, row_tok,
                                          K, N, (uint16_t*)out);
  return hipGetLastError();
}

extern "C" int moe_gemv_max_tokens() { return GV_MAXT; }
