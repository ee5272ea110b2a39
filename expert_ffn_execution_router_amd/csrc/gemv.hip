// Slot-indexed grouped expert GEMMs for the smallest batches (at most 8
// tokens per expert) as matrix-vector products on the vector ALUs, for
// every weight format.
//
// Method (paper.oopus.info review of FreeToken, section 2.5: the GPU
// evaluates every expert of G = H u F for the tokens routed to it; SwiGLU
// expert): the same two GEMMs as the small-batch MFMA kernel,
//   GEMM 1: A = silu(x W_gate^T) * (x W_up^T), rounded to the A type,
//   GEMM 2: Z = A W_down^T, rounded to bf16,
// with exact fp32 products and fp32 sums, and the same rounding points as
// that kernel: bf16 tokens and A for bf16, fp8 and MXFP4 weights; fp16
// tokens (the hidden rows converted once per call) and fp16 A for NVFP4,
// whose fp32 matrix scales multiply the sums (gate and up before the
// SwiGLU, down before rounding Z).  With one to eight tokens an expert's
// weight rows are each used one to eight times: the work is the weight
// stream.  The MFMA kernel moves every weight through LDS and multiplies
// 16-token tiles that are almost all padding; here each weight is loaded
// once into registers, dequantised exactly and multiplied by the token
// values it meets (one to eight token rows).
//   * an item is (active expert, 16 weight rows): for GEMM 1 the gate and up
//     rows of 8 features, for GEMM 2 16 output columns; one workgroup of
//     4 waves per item, each wave 4 rows;
//   * at step s lane l takes bytes [1024 s + 16 l, +16) of each of its
//     wave's four rows: V = 8 (bf16), 16 (fp8) or 32 (E2M1) weights per row,
//     so one wave instruction reads 1 KiB of one row, four 256-byte
//     segments with the nontemporal hint; the V token values of that K range
//     are loaded once per token (cached: every item of the expert reads
//     them) and serve all four rows;
//   * scales: fp8 - the fp32 scale of the 128x128 block multiplies the
//     lane's 16 products (all in one 128-K block); MXFP4 - the E8M0 scale
//     of the lane's 32 weights (one block) goes into the conversion (a
//     power of two: exact); NVFP4 - the E4M3 scales of the lane's two
//     16-weight blocks multiply their products;
//   * the 64 partial sums of a row are added across the lanes with four
//     DPP moves inside each 16-lane row (xor 1, xor 2, rotate 4, rotate 8)
//     and two lane shuffles across the rows; a wave's four rows of GEMM 1
//     are the gate and up rows of two features, so the SwiGLU needs no
//     exchange.
#include "route_dev.h"

namespace {

constexpr int GV_MAXT = 8;      // tokens per expert (instances for 1, 2, 4 and 8)
constexpr int GV_BLK = 2;       // steps in flight (a step: 16 bytes of each of the wave's 4 rows per lane)

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

DEV float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Eight token values (bf16 or fp16 bits, element order) as fp32, exact.
template <bool F16>
DEV void tok8(i32x4_t x, float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t b = (uint32_t)x[q];
    if (F16) {
      const f16x2_t h = __builtin_bit_cast(f16x2_t, b);
      v[2 * q] = (float)h[0];
      v[2 * q + 1] = (float)h[1];
    } else {
      v[2 * q] = __uint_as_float(b << 16);
      v[2 * q + 1] = __uint_as_float(b & 0xffff0000u);
    }
  }
}

// acc += the 8 E2M1 weights of word w (two per byte, even element in the
// low nibble; the conversion scaled by s, a power of two) times x.
DEV float fp4_dot8(uint32_t w, float s, const float (&x)[8], float acc) {
  // the byte selector must be a literal
  const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 0);
  const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 1);
  const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 2);
  const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, s, 3);
  acc = fmaf(p0[0], x[0], acc);
  acc = fmaf(p0[1], x[1], acc);
  acc = fmaf(p1[0], x[2], acc);
  acc = fmaf(p1[1], x[3], acc);
  acc = fmaf(p2[0], x[4], acc);
  acc = fmaf(p2[1], x[5], acc);
  acc = fmaf(p3[0], x[6], acc);
  return fmaf(p3[1], x[7], acc);
}

// acc += the 4 E4M3 weights of word w (element order) times x[0..3].
DEV float fp8_dot4(uint32_t w, const float* x, float acc) {
  const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
  acc = fmaf(lo[0], x[0], acc);
  acc = fmaf(lo[1], x[1], acc);
  acc = fmaf(hi[0], x[2], acc);
  return fmaf(hi[1], x[3], acc);
}

}  // namespace

// FMT: WFMT_BF16, WFMT_FP8_A16, WFMT_MXFP4_A16 or WFMT_NVFP4.  GATED:
// out = A ([rows, N], N = I; fp16 for NVFP4, else bf16) from X = the token
// rows ([T, K], fp16 for NVFP4, else bf16) gathered through row_tok, weights
// gate at woff0 / soff0 and up at woff1 / soff1.  Otherwise out = Z (bf16
// [rows, N], N = H) from X = A in grouped order, weights at woff0 / soff0.
// Rows of expert e are offsets[e] .. + counts[e], MT (1, 2, 4 or 8) at a time.
// The one-token instance is held to four waves per SIMD (128 registers: the
// grids of the fp8 and MXFP4 shapes need more than one round of workgroups,
// and residency decides their speed).  K is a multiple of
// the values in 16 bytes of a row (8, 16 or 32; a row's last 256-byte
// segment may be partial: lanes past it contribute nothing); N % 8 (gated)
// or 16.  The grid may exceed the items (n_act * N / 8 or N / 16): the extra
// workgroups leave at once.
// ROUTE (GATED, MT = 1, one token): the item's expert is the a-th of the
// token's winners that run on the GPU (expert order), picked by wave 0 from
// the logits (rt.z) with the top-k selection of topk_row, its grouped row
// the number of winners with a lower id; workgroup 0 also writes the routing
// and grouping outputs at the end (topk_row and group_wave).  wl, counts,
// offsets and row_tok are not read.
template <int FMT, bool GATED, int MT, bool ROUTE = false>
__global__ void __launch_bounds__(256, MT == 1 ? 4 : 1)
gemv_dec(const WorkList* __restrict__ wl, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
         const uint8_t* __restrict__ pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
         const uint16_t* __restrict__ X, const int32_t* __restrict__ row_tok, int K, int N, uint16_t* __restrict__ out,
         GemvRoute rt = GemvRoute{}) {
  static_assert(!ROUTE || (GATED && MT == 1), "self-routed launches: gate/up, one token");
  constexpr bool NV = FMT == WFMT_NVFP4;
  constexpr bool W4 = NV || FMT == WFMT_MXFP4_A16;
  constexpr int V = FMT == WFMT_BF16 ? 8 : (W4 ? 32 : 16);       // weights per lane and step
  constexpr int WB2 = FMT == WFMT_BF16 ? 4 : (W4 ? 1 : 2);        // weight bytes per value, times 2
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per_e = GATED ? N / 8 : N / 16;          // items per expert
  const int it = blockIdx.x;
  const int a = it / per_e, blk = it - a * per_e;
  int slot, rbase, ctot;
  if constexpr (ROUTE) {
    __shared__ int s_pick[3];                        // slot, grouped row, found
    if (wave == 0) {
      const WaveMeta wm = wave_meta(rt.E, rt.miss_mask, rt.slot_row);
      uint64_t selm[4];
      topk_select(rt.z, rt.E, rt.k, selm);
      int n_act = 0, n_sel = 0, p_slot = 0, p_row = 0, found = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ee = lane + 64 * i;
        const bool act = ((selm[i] >> lane) & 1ull) && !((wm.mw[i] >> (ee & 31)) & 1u) && wm.sl[i] >= 0;
        const uint64_t am = __builtin_amdgcn_ballot_w64(act);
        const int n = __popcll(am);
        if (!found && a < n_act + n) {
          uint64_t m = am;
          for (int q = 0; q < a - n_act; ++q) m &= m - 1ull;
          const int L = __builtin_ctzll(m);
          p_slot = __builtin_amdgcn_readlane(wm.sl[i], L);
          p_row = n_sel + __popcll(selm[i] & ((1ull << L) - 1ull));
          found = 1;
        }
        n_act += n;
        n_sel += __popcll(selm[i]);
      }
      if (lane == 0) {
        s_pick[0] = p_slot;
        s_pick[1] = p_row;
        s_pick[2] = found;
      }
    }
    __syncthreads();
    if (!s_pick[2] && blockIdx.x != 0) return;
    slot = s_pick[2] ? s_pick[0] : 0;
    rbase = s_pick[1];
    ctot = s_pick[2];                                // one row, or none (workgroup 0 still routes)
  } else {
    // the item's work-list entries are read beside the count (entries past
    // n_act are not used), so the weight addresses wait for one load
    const int ac = min(a, 255);
    const int nact = wl->n_act, e = wl->act_e[ac];
    slot = wl->act_slot[ac];
    if (a >= nact) return;
    rbase = offsets[e];
    ctot = counts[e];
  }
  const uint8_t* blob = pool + (size_t)slot * S;
  const int rowb = K * WB2 / 2;                      // weight bytes per row
  // the expert's rows in chunks of MT (the batch bounds them by MT; a chunk
  // loop keeps the kernel correct for any count)
  for (int tc = 0; tc < ctot; tc += MT) {
    const int row0 = rbase + tc, cnt = min(MT, ctot - tc);
    // the wave's four rows: GATED gate f0, gate f0+1, up f0, up f0+1
    // (f0 = 8 blk + 2 wave); otherwise columns 16 blk + 4 wave + q
    const uint8_t* wr[4];
    const float* s8[4];
    const uint8_t* sb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int feat = GATED ? blk * 8 + 2 * wave + (q & 1) : blk * 16 + 4 * wave + q;
      const int m = GATED ? (q >> 1) : 0;
      const size_t woff = m ? woff1 : woff0, soff = m ? soff1 : soff0;
      wr[q] = blob + woff + (size_t)feat * rowb + lane * 16;
      s8[q] = (const float*)(blob + soff) + (size_t)(feat / 128) * (K / 128);
      sb[q] = blob + soff + (size_t)feat * (K / (NV ? 16 : 32));
    }
    const uint8_t* xr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = row0 + min(t, cnt - 1);
      const int xrow = ROUTE ? 0 : (GATED ? row_tok[r] : r);
      xr[t] = (const uint8_t*)X + (size_t)xrow * K * 2 + lane * (2 * V);
    }
    float acc[4][MT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[q][t] = 0.0f;
    const int nstep = (rowb + 1023) / 1024;            // 1 KiB of each row per step (the last may be partial)
    const i32x4_t z4 = {0, 0, 0, 0};
    for (int s0 = 0; s0 < nstep; s0 += GV_BLK) {
      i32x4_t wv[GV_BLK][4];
      float sc[GV_BLK][4][2];
      bool ok[GV_BLK];
#pragma unroll
      for (int j = 0; j < GV_BLK; ++j) {
        if (s0 + j >= nstep) break;
        const int s = s0 + j;
        const int v0 = V * (64 * s + lane);            // first value of the lane's 16 bytes
        ok[j] = 1024 * s + 16 * lane < rowb;           // they lie in the row
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sc[j][q][0] = sc[j][q][1] = 0.0f;
          wv[j][q] = ok[j] ? ld16_nt(wr[q] + 1024 * s) : z4;
          if (!ok[j]) continue;
          if (FMT == WFMT_FP8_A16) {
            sc[j][q][0] = s8[q][v0 / 128];
          } else if (FMT == WFMT_MXFP4_A16) {
            sc[j][q][0] = e8m0_to_f32(sb[q][v0 / 32]);
          } else if (NV) {
            const f32x2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(*(const uint16_t*)(sb[q] + v0 / 16), 1.0f, false);
            sc[j][q][0] = p[0];
            sc[j][q][1] = p[1];
          }
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t >= cnt) break;
#pragma unroll
        for (int j = 0; j < GV_BLK; ++j) {
          if (s0 + j >= nstep) break;
          if (!ok[j]) continue;                         // past the row: contributes nothing
          const uint8_t* xs = xr[t] + (s0 + j) * (128 * V);
          if (FMT == WFMT_BF16) {
            float xv[8];
            tok8<false>(ld16(xs), xv);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const uint32_t w = (uint32_t)wv[j][q][c];
                acc[q][t] = fmaf(__uint_as_float(w << 16), xv[2 * c], acc[q][t]);
                acc[q][t] = fmaf(__uint_as_float(w & 0xffff0000u), xv[2 * c + 1], acc[q][t]);
              }
          } else if (FMT == WFMT_FP8_A16) {
            float xv[2][8];
            tok8<false>(ld16(xs), xv[0]);
            tok8<false>(ld16(xs + 16), xv[1]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float p = 0.0f;
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                p = fp8_dot4((uint32_t)wv[j][q][2 * h], xv[h], p);
                p = fp8_dot4((uint32_t)wv[j][q][2 * h + 1], xv[h] + 4, p);
              }
              acc[q][t] = fmaf(p, sc[j][q][0], acc[q][t]);
            }
          } else {
            float xv[4][8];
#pragma unroll
            for (int h = 0; h < 4; ++h) tok8<NV>(ld16(xs + 16 * h), xv[h]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (NV) {
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {        // two 16-weight blocks, each with its scale
                  float p = fp4_dot8((uint32_t)wv[j][q][2 * bb], 1.0f, xv[2 * bb], 0.0f);
                  p = fp4_dot8((uint32_t)wv[j][q][2 * bb + 1], 1.0f, xv[2 * bb + 1], p);
                  acc[q][t] = fmaf(p, sc[j][q][bb], acc[q][t]);
                }
              } else {
#pragma unroll
                for (int h = 0; h < 4; ++h) acc[q][t] = fp4_dot8((uint32_t)wv[j][q][h], sc[j][q][0], xv[h], acc[q][t]);
              }
            }
          }
        }
      }
    }
    // sums over the 64 lanes: the 16 of each DPP row, then across the rows
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        float v = row16_sum(acc[q][t]);
        v += __shfl_xor(v, 16, 64);
        acc[q][t] = v + __shfl_xor(v, 32, 64);
      }
    float ts = 1.0f, tsu = 1.0f;                        // NVFP4 matrix scales
    if (NV) {
      const size_t n = (size_t)K * N;
      const float* tsc = (const float*)(blob + 3 * (n / 2) + 3 * (n / 16));
      ts = GATED ? tsc[0] : tsc[2];
      tsu = tsc[1];
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t >= cnt) break;
        if (GATED) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const float v = NV ? silu_mul(acc[c][t] * ts, acc[2 + c][t] * tsu) : silu_mul(acc[c][t], acc[2 + c][t]);
            out[(size_t)(row0 + t) * N + blk * 8 + 2 * wave + c] =
                NV ? (uint16_t)(pack_f16x2(v, 0.0f) & 0xffffu) : f32_to_bf16_bits(v);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            out[(size_t)(row0 + t) * N + blk * 16 + 4 * wave + q] = f32_to_bf16_bits(NV ? acc[q][t] * ts : acc[q][t]);
        }
      }
    }
  }
  if constexpr (ROUTE) {
    // workgroup 0: the token's routing and grouping for the launches after this one
    if (blockIdx.x == 0 && wave == 0) {
      __shared__ TopkScratch r_sc;
      __shared__ int32_t r_ids[8];
      __shared__ uint32_t r_bits[256];
      __shared__ int r_off[256], r_gsl[256];
      const WaveMeta wm = wave_meta(rt.E, rt.miss_mask, rt.slot_row);
      topk_row(rt.z, rt.E, rt.k, rt.ids, rt.w, r_ids, &r_sc);
      wave_lds_order();
      group_wave(r_ids, 1, rt.k, rt.E, wm, rt.mb, rt.counts, rt.offsets, rt.pos, rt.perm_tok, rt.wl, rt.err,
                 rt.pslot, r_bits, r_off, r_gsl);
    }
  }
}

// The down GEMM and the weighted combine in one launch, for the resident
// forward at the smallest batches: workgroup (4 output columns h0..h0+3,
// token t), wave j = the token's choice j.  Wave j computes the 4 columns of
// Z for (t, j) exactly as gemv_dec does for that row (same lane layout,
// steps and sums, the NVFP4 down scale on the sum, rounded to bf16); wave
// 0 then adds w_tj * z_j over j = 0..7 in order, choices that ran on the
// host or past k adding zero, then the host partial, as the combine kernel
// does:
//   out[t, h] = bf16( sum_j w_tj z_tj[h] + host_partial[t, h] ).
// out_f32 (optional): the unrounded sum instead.  A: the GEMM 1 output in
// grouped order (row pos[t, j]); pslot[t, j]: the slot of choice j's expert,
// -1 where it did not run on the GPU (the fused top-k/grouping writes it);
// K = I, N = H, N % 4 == 0.  Held to four waves per SIMD (two workgroups
// per CU; MXFP4 spills a few registers there and still runs as fast).
template <int FMT>
__global__ void __launch_bounds__(512, 4)
gemv_down_combine(const int32_t* __restrict__ pslot, const float* __restrict__ w, const int32_t* __restrict__ pos,
                  const uint8_t* __restrict__ pool, size_t S, size_t woff, size_t soff,
                  const uint16_t* __restrict__ A, int k, int K, int N, const float* hp,
                  const int32_t* __restrict__ hp_count, uint16_t* __restrict__ out, float* out_f32) {
  constexpr bool NV = FMT == WFMT_NVFP4;
  constexpr bool W4 = NV || FMT == WFMT_MXFP4_A16;
  constexpr int V = FMT == WFMT_BF16 ? 8 : (W4 ? 32 : 16);
  constexpr int WB2 = FMT == WFMT_BF16 ? 4 : (W4 ? 1 : 2);
  __shared__ float zs[8][4];
  __shared__ int us[8];
  const int j = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h0 = blockIdx.x * 4, t = blockIdx.y;
  const size_t a = (size_t)t * k + j;
  const int slot = pslot[a];        // -1: computed by the host, or not resident (error flagged by the grouping)
  const bool use = slot >= 0;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (use) {
    const uint8_t* blob = pool + (size_t)slot * S;
    const int rowb = K * WB2 / 2;
    const uint8_t* wr[4];
    const float* s8[4];
    const uint8_t* sb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int feat = h0 + q;
      wr[q] = blob + woff + (size_t)feat * rowb + lane * 16;
      s8[q] = (const float*)(blob + soff) + (size_t)(feat / 128) * (K / 128);
      sb[q] = blob + soff + (size_t)feat * (K / (NV ? 16 : 32));
    }
    const uint8_t* xr = (const uint8_t*)A + (size_t)pos[a] * K * 2 + lane * (2 * V);
    const int nstep = (rowb + 1023) / 1024;
    const i32x4_t z4 = {0, 0, 0, 0};
    for (int s0 = 0; s0 < nstep; s0 += GV_BLK) {
      i32x4_t wv[GV_BLK][4];
      float sc[GV_BLK][4][2];
      bool ok[GV_BLK];
#pragma unroll
      for (int jj = 0; jj < GV_BLK; ++jj) {
        if (s0 + jj >= nstep) break;
        const int st = s0 + jj;
        const int v0 = V * (64 * st + lane);
        ok[jj] = 1024 * st + 16 * lane < rowb;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sc[jj][q][0] = sc[jj][q][1] = 0.0f;
          wv[jj][q] = ok[jj] ? ld16_nt(wr[q] + 1024 * st) : z4;
          if (!ok[jj]) continue;
          if (FMT == WFMT_FP8_A16) {
            sc[jj][q][0] = s8[q][v0 / 128];
          } else if (FMT == WFMT_MXFP4_A16) {
            sc[jj][q][0] = e8m0_to_f32(sb[q][v0 / 32]);
          } else if (NV) {
            const f32x2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(*(const uint16_t*)(sb[q] + v0 / 16), 1.0f, false);
            sc[jj][q][0] = p[0];
            sc[jj][q][1] = p[1];
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < GV_BLK; ++jj) {
        if (s0 + jj >= nstep) break;
        if (!ok[jj]) continue;
        const uint8_t* xs = xr + (s0 + jj) * (128 * V);
        if (FMT == WFMT_BF16) {
          float xv[8];
          tok8<false>(ld16(xs), xv);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint32_t wq = (uint32_t)wv[jj][q][c];
              acc[q] = fmaf(__uint_as_float(wq << 16), xv[2 * c], acc[q]);
              acc[q] = fmaf(__uint_as_float(wq & 0xffff0000u), xv[2 * c + 1], acc[q]);
            }
        } else if (FMT == WFMT_FP8_A16) {
          float xv[2][8];
          tok8<false>(ld16(xs), xv[0]);
          tok8<false>(ld16(xs + 16), xv[1]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float p = 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              p = fp8_dot4((uint32_t)wv[jj][q][2 * h], xv[h], p);
              p = fp8_dot4((uint32_t)wv[jj][q][2 * h + 1], xv[h] + 4, p);
            }
            acc[q] = fmaf(p, sc[jj][q][0], acc[q]);
          }
        } else {
          float xv[4][8];
#pragma unroll
          for (int h = 0; h < 4; ++h) tok8<NV>(ld16(xs + 16 * h), xv[h]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (NV) {
#pragma unroll
              for (int bb = 0; bb < 2; ++bb) {
                float p = fp4_dot8((uint32_t)wv[jj][q][2 * bb], 1.0f, xv[2 * bb], 0.0f);
                p = fp4_dot8((uint32_t)wv[jj][q][2 * bb + 1], 1.0f, xv[2 * bb + 1], p);
                acc[q] = fmaf(p, sc[jj][q][bb], acc[q]);
              }
            } else {
#pragma unroll
              for (int h = 0; h < 4; ++h) acc[q] = fp4_dot8((uint32_t)wv[jj][q][h], sc[jj][q][0], xv[h], acc[q]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v = row16_sum(acc[q]);
      v += __shfl_xor(v, 16, 64);
      acc[q] = v + __shfl_xor(v, 32, 64);
    }
    if (NV) {
      const size_t n = (size_t)K * N;
      const float ts = ((const float*)(blob + 3 * (n / 2) + 3 * (n / 16)))[2];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] *= ts;
    }
  }
  if (lane < 4) {
    float zq = acc[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) zq = lane == q ? acc[q] : zq;
    zs[j][lane] = use ? bf16_bits_to_f32(f32_to_bf16_bits(zq)) : 0.0f;
  }
  if (lane == 0) us[j] = use ? 1 : 0;
  __syncthreads();
  if (j != 0 || lane >= 4) return;
  float o = 0.0f;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const bool u = jj < k && us[jj < k ? jj : 0];
    const float lo = jj < k ? w[(size_t)t * k + jj] * zs[jj < k ? jj : 0][lane] : 0.0f;
    o += u ? lo : 0.0f;
  }
  const int h = h0 + lane;
  if (hp && (!hp_count || *hp_count > 0)) o += hp[(size_t)t * N + h];
  if (out_f32) out_f32[(size_t)t * N + h] = o;
  else out[(size_t)t * N + h] = f32_to_bf16_bits(o);
}

namespace {
template <int FMT>
hipError_t launch_gemv_routed(int grid, const GemvRoute& rt, const uint8_t* pool, size_t S, size_t woff0,
                              size_t woff1, size_t soff0, size_t soff1, const void* X, int K, int N, void* out,
                              hipStream_t s) {
  gemv_dec<FMT, true, 1, true><<<grid, 256, 0, s>>>(nullptr, nullptr, nullptr, pool, S, woff0, woff1, soff0, soff1,
                                                    (const uint16_t*)X, nullptr, K, N, (uint16_t*)out, rt);
  return hipGetLastError();
}

template <int FMT, int MT>
hipError_t launch_gemv_mt(int gated, int grid, const WorkList* wl, const int32_t* counts, const int32_t* offsets,
                          const uint8_t* pool, size_t S, size_t woff0, size_t woff1, size_t soff0, size_t soff1,
                          const void* X, const int32_t* row_tok, int K, int N, void* out, hipStream_t s) {
  if (gated)
    gemv_dec<FMT, true, MT><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                                 (const uint16_t*)X, row_tok, K, N, (uint16_t*)out);
  else
    gemv_dec<FMT, false, MT><<<grid, 256, 0, s>>>(wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1,
                                                  (const uint16_t*)X, row_tok, K, N, (uint16_t*)out);
  return hipGetLastError();
}

// Fewer tokens' accumulators keep more waves per SIMD: each batch takes the
// smallest instance that holds its largest expert's rows.
template <int FMT>
hipError_t launch_gemv(int max_rows, int gated, int grid, const WorkList* wl, const int32_t* counts,
                       const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0, size_t woff1, size_t soff0,
                       size_t soff1, const void* X, const int32_t* row_tok, int K, int N, void* out, hipStream_t s) {
#define MOE_GVM_ARGS gated, grid, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X, row_tok, K, N, out, s
  if (max_rows == 1) return launch_gemv_mt<FMT, 1>(MOE_GVM_ARGS);
  if (max_rows == 2) return launch_gemv_mt<FMT, 2>(MOE_GVM_ARGS);
  if (max_rows <= 4) return launch_gemv_mt<FMT, 4>(MOE_GVM_ARGS);
  return launch_gemv_mt<FMT, 8>(MOE_GVM_ARGS);
#undef MOE_GVM_ARGS
}
}  // namespace

// fmt: WFMT_BF16, WFMT_FP8_A16, WFMT_MXFP4_A16 or WFMT_NVFP4.  grid: at
// least the items (active experts x N / 8 for GEMM 1, N / 16 for GEMM 2);
// max_rows: a bound on the routed rows of any expert (at most 8; the batch
// size bounds it).
extern "C" hipError_t moe_launch_gemv(int fmt, int max_rows, int gated, int grid, const WorkList* wl, const int32_t* counts,
                                      const int32_t* offsets, const uint8_t* pool, size_t S, size_t woff0,
                                      size_t woff1, size_t soff0, size_t soff1, const void* X,
                                      const int32_t* row_tok, int K, int N, void* out, hipStream_t s) {
  const int kq = fmt == WFMT_BF16 ? 8 : (fmt == WFMT_FP8_A16 ? 16 : 32);   // K per 16 bytes of a row
  if (grid < 1 || max_rows < 1 || max_rows > GV_MAXT || K % kq || N % (gated ? 8 : 16) || (gated && !row_tok))
    return hipErrorInvalidValue;
#define MOE_GV_ARGS max_rows, gated, grid, wl, counts, offsets, pool, S, woff0, woff1, soff0, soff1, X, row_tok, K, N, out, s
  switch (fmt) {
    case WFMT_BF16: return launch_gemv<WFMT_BF16>(MOE_GV_ARGS);
    case WFMT_FP8_A16: return launch_gemv<WFMT_FP8_A16>(MOE_GV_ARGS);
    case WFMT_MXFP4_A16: return launch_gemv<WFMT_MXFP4_A16>(MOE_GV_ARGS);
    case WFMT_NVFP4: return launch_gemv<WFMT_NVFP4>(MOE_GV_ARGS);
    default: return hipErrorInvalidValue;
  }
#undef MOE_GV_ARGS
}

// The down GEMM of a matrix-vector forward fused with the combine (see
// gemv_down_combine): fmt as moe_launch_gemv; k <= 8; N % 4 == 0.
extern "C" hipError_t moe_launch_gemv_down_combine(int fmt, const int32_t* pslot, const float* w, const int32_t* pos,
                                                   const uint8_t* pool, size_t S, size_t woff, size_t soff,
                                                   const void* A, int T, int k, int K, int N, const float* hp,
                                                   const int32_t* hp_count, void* out, float* out_f32, hipStream_t s) {
  const int kq = fmt == WFMT_BF16 ? 8 : (fmt == WFMT_FP8_A16 ? 16 : 32);
  if (T < 1 || k < 1 || k > 8 || N % 4 || K % kq) return hipErrorInvalidValue;
  const dim3 grid(N / 4, T);
#define MOE_DC_ARGS pslot, w, pos, pool, S, woff, soff, (const uint16_t*)A, k, K, N, hp, hp_count, \
                    (uint16_t*)out, out_f32
  switch (fmt) {
    case WFMT_BF16: gemv_down_combine<WFMT_BF16><<<grid, 64 * k, 0, s>>>(MOE_DC_ARGS); break;
    case WFMT_FP8_A16: gemv_down_combine<WFMT_FP8_A16><<<grid, 64 * k, 0, s>>>(MOE_DC_ARGS); break;
    case WFMT_MXFP4_A16: gemv_down_combine<WFMT_MXFP4_A16><<<grid, 64 * k, 0, s>>>(MOE_DC_ARGS); break;
    case WFMT_NVFP4: gemv_down_combine<WFMT_NVFP4><<<grid, 64 * k, 0, s>>>(MOE_DC_ARGS); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_DC_ARGS
  return hipGetLastError();
}

extern "C" int moe_gemv_max_tokens() { return GV_MAXT; }

// The gate/up matrix-vector launch of a one-token batch that routes for
// itself (GemvRoute): grid at least min(k, E) * N / 8 workgroups (the
// experts that run on the GPU are at most k); X holds the token's row (bf16,
// or fp16 for NVFP4).
extern "C" hipError_t moe_launch_gemv_routed(int fmt, int grid, const GemvRoute* rt, const uint8_t* pool, size_t S,
                                             size_t woff0, size_t woff1, size_t soff0, size_t soff1, const void* X,
                                             int K, int N, void* out, hipStream_t s) {
  const int kq = fmt == WFMT_BF16 ? 8 : (fmt == WFMT_FP8_A16 ? 16 : 32);
  if (!rt || grid < 1 || K % kq || N % 8 || rt->E < 1 || rt->E > 256 || rt->k < 1 || rt->k > 8 || rt->k > rt->E)
    return hipErrorInvalidValue;
#define MOE_GR_ARGS grid, *rt, pool, S, woff0, woff1, soff0, soff1, X, K, N, out, s
  switch (fmt) {
    case WFMT_BF16: return launch_gemv_routed<WFMT_BF16>(MOE_GR_ARGS);
    case WFMT_FP8_A16: return launch_gemv_routed<WFMT_FP8_A16>(MOE_GR_ARGS);
    case WFMT_MXFP4_A16: return launch_gemv_routed<WFMT_MXFP4_A16>(MOE_GR_ARGS);
    case WFMT_NVFP4: return launch_gemv_routed<WFMT_NVFP4>(MOE_GR_ARGS);
    default: return hipErrorInvalidValue;
  }
#undef MOE_GR_ARGS
}
