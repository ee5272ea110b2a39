// Weighted unpermute-combine and activation quantisation.
//
// Combine (paper.oopus.info review of FreeToken, section 2.5: the GPU and the
// host each compute the partial sum of their own experts and the two are
// added, leaving the MoE output unchanged):
//   out[t] = bf16( sum_{j<k, e_tj on the GPU} w_tj * Z[pos[t,j]]  + host_partial[t] )
// summed in fp32 in the order j = 0..k-1, then the host partial.
//
// Quantisation of GEMM inputs for the 8-bit weight formats (the pages only
// say the kernels dequantise in-kernel; these are the declared readings):
//   * fp8 path: per (row, 128 columns): scale = amax/448, code = E4M3(v*(448/amax));
//   * mxfp4 path: OCP MX rule, E4M3 elements per 32 columns with E8M0 scale
//     2^(floor(log2 amax) - 8);
//   * its MXFP6 variant: OCP MX rule, E2M3 elements per 32 columns with E8M0
//     scale 2^(floor(log2 amax) - 2), round to nearest even, saturating at 7.5.
#include "common.h"

__global__ void __launch_bounds__(256)
combine_kernel(const uint16_t* __restrict__ Z, const int32_t* __restrict__ ids, const float* __restrict__ w,
               const int32_t* __restrict__ pos, const uint32_t* __restrict__ miss_mask,
               const int32_t* __restrict__ slot_row, const float* hp, const int32_t* __restrict__ hp_count, int T,
               int k, int H, uint16_t* __restrict__ out, float* out_f32) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (t >= T || h >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  // all loads unconditional (choices past k repeat choice k-1 and are not
  // used); excluded choices are dropped with a select, never multiplied,
  // because their Z rows were not written
  int p[8];
  bool use[8];
  float wj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const size_t a = (size_t)t * k + min(j, k - 1);
    const int e = ids[a];
    const bool host = miss_mask && ((miss_mask[e >> 5] >> (e & 31)) & 1u);   // computed by the host
    use[j] = j < k && !host && slot_row[e] >= 0;                            // not resident: error flagged
    p[j] = pos[a];
    wj[j] = w[a];
  }
  i32x4_t zv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) zv[j] = ld16(Z + (size_t)p[j] * H + h);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = (uint32_t)zv[j][i];
      const float lo = wj[j] * bf16_bits_to_f32(u & 0xffffu), hi = wj[j] * bf16_bits_to_f32(u >> 16);
      acc[2 * i] += use[j] ? lo : 0.0f;
      acc[2 * i + 1] += use[j] ? hi : 0.0f;
    }
  }
  // hp_count (device, optional): the host partial is used only when the
  // plan sent at least one expert to the host
  if (hp && (!hp_count || *hp_count > 0)) {
    const float4 a = *(const float4*)(hp + (size_t)t * H + h);
    const float4 b = *(const float4*)(hp + (size_t)t * H + h + 4);
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
  if (out_f32) {            // unrounded partial sum (may overwrite hp in place: same thread, read first)
    *(float4*)(out_f32 + (size_t)t * H + h) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)(out_f32 + (size_t)t * H + h + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    return;
  }
  i32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (int)((uint32_t)f32_to_bf16_bits(acc[2 * i]) | ((uint32_t)f32_to_bf16_bits(acc[2 * i + 1]) << 16));
  *(i32x4_t*)(out + (size_t)t * H + h) = o;
}

// 16 consecutive source values of one row as fp32 (bf16: two 16-byte loads;
// fp32: four).
template <bool SRC_BF16>
DEV void load16(const void* src, size_t i, float (&v)[16]) {
  if (SRC_BF16) {
    const i32x4_t a = ld16((const uint16_t*)src + i), b = ld16((const uint16_t*)src + i + 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_bits_to_f32((uint32_t)a[k] & 0xffffu);
      v[2 * k + 1] = bf16_bits_to_f32((uint32_t)a[k] >> 16);
      v[8 + 2 * k] = bf16_bits_to_f32((uint32_t)b[k] & 0xffffu);
      v[8 + 2 * k + 1] = bf16_bits_to_f32((uint32_t)b[k] >> 16);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const i32x4_t a = ld16((const float*)src + i + 4 * k);
#pragma unroll
      for (int m = 0; m < 4; ++m) v[4 * k + m] = __int_as_float(a[m]);
    }
  }
}

// 16 E4M3 codes packed little-endian into 16 bytes.
DEV i32x4_t pack_e4m3x16(const float (&v)[16], float mul) {
  i32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = (int)(f32_to_e4m3(v[4 * k] * mul) | (f32_to_e4m3(v[4 * k + 1] * mul) << 8) |
                 (f32_to_e4m3(v[4 * k + 2] * mul) << 16) | (f32_to_e4m3(v[4 * k + 3] * mul) << 24));
  return o;
}

// One thread per (row, 16 columns); the 8 threads of a 128-column group are
// consecutive lanes.  Rows from *nrows_dev when given.  Output row r
// quantises source row row_map[r] (r itself without a map).
template <bool SRC_BF16>
__global__ void __launch_bounds__(256)
quant_fp8_kernel(const void* __restrict__ src, int rows, const int32_t* __restrict__ nrows_dev,
                 const int32_t* __restrict__ row_map, int cols, uint8_t* __restrict__ q, float* __restrict__ scale) {
  const long g = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = cols / 16;
  const int nrows = nrows_dev ? *nrows_dev : rows;
  const long r = g / per_row;
  const int c0 = (int)(g - r * per_row) * 16;
  if (r >= nrows) return;                     // whole 8-lane groups leave together (cols % 128 == 0)
  float v[16];
  load16<SRC_BF16>(src, (size_t)(row_map ? row_map[r] : r) * cols + c0, v);
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(v[k]));
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
  const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  *(i32x4_t*)(q + (size_t)r * cols + c0) = pack_e4m3x16(v, inv);
  if ((c0 & 127) == 0) scale[(size_t)r * (cols / 128) + c0 / 128] = sc;
}

// One thread per (row, 16 columns); two threads per 32-column MX block.
template <bool SRC_BF16>
__global__ void __launch_bounds__(256)
quant_mxfp8_kernel(const void* __restrict__ src, int rows, const int32_t* __restrict__ nrows_dev,
                   const int32_t* __restrict__ row_map, int cols, uint8_t* __restrict__ q,
                   uint8_t* __restrict__ scale) {
  const long g = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = cols / 16;
  const int nrows = nrows_dev ? *nrows_dev : rows;
  const long r = g / per_row;
  const int c0 = (int)(g - r * per_row) * 16;
  if (r >= nrows) return;                     // lane pairs leave together (cols % 32 == 0)
  float v[16];
  load16<SRC_BF16>(src, (size_t)(row_map ? row_map[r] : r) * cols + c0, v);
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax = fmaxf(amax, fabsf(v[k]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  int x = 0;
  if (amax > 0.0f) {
    int e;
    frexpf(amax, &e);                    // amax = m * 2^e, m in [0.5, 1)
    x = min(127, max(-127, (e - 1) - 8));
  }
  // ldexpf(v, -x) is exact scaling by a power of two (no overflow: |v| <
  // 2^(x+9), and x >= -127 keeps results finite)
  float w[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) w[k] = ldexpf(v[k], -x);
  *(i32x4_t*)(q + (size_t)r * cols + c0) = pack_e4m3x16(w, 1.0f);
  if ((c0 & 31) == 0) scale[(size_t)r * (cols / 32) + c0 / 32] = (uint8_t)(x + 127);
}

// E2M3 code of w (OCP MX FP6: bias 1, max 7.5, subnormal step 1/8), round to
// nearest even, saturating.  The step is 1/8 below 2, 1/4 in [2, 4) and 1/2
// above, and the codes count up through the binades without a gap, so the
// code is an offset plus w divided by its binade's step, rounded (ties to the
// even integer, which is the even code).
DEV uint32_t f32_to_e2m3(float w) {
  const float a = fabsf(w);
  uint32_t c;
  if (a < 2.0f) c = (uint32_t)rintf(a * 8.0f);
  else if (a < 4.0f) c = 8u + (uint32_t)rintf(a * 4.0f);
  else c = min(16u + (uint32_t)rintf(fminf(a, 8.0f) * 2.0f), 31u);
  return c ? (c | ((__float_as_uint(w) >> 26) & 0x20u)) : 0u;
}

// One thread per (row, 32-column block).  Rows from *nrows_dev when given;
// output row r quantises source row row_map[r] (r itself without a map).
template <bool SRC_BF16>
__global__ void __launch_bounds__(256)
quant_mxfp6_kernel(const void* __restrict__ src, int rows, const int32_t* __restrict__ nrows_dev,
                   const int32_t* __restrict__ row_map, int cols, int cap, uint8_t* __restrict__ q,
                   uint8_t* __restrict__ scale) {
  const long gi = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = cols / 32;
  const int nrows = nrows_dev ? *nrows_dev : rows;
  const long r = gi / per_row;
  const int b = (int)(gi - r * per_row);
  if (r >= nrows) return;
  float v[2][16];
  const size_t at = (size_t)(row_map ? row_map[r] : r) * cols + b * 32;
  load16<SRC_BF16>(src, at, v[0]);
  load16<SRC_BF16>(src, at + 16, v[1]);
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(v[k >> 4][k & 15]));
  int x = 0;
  if (amax > 0.0f) {
    int e;
    frexpf(amax, &e);                    // amax = m * 2^e, m in [0.5, 1)
    x = min(127, max(-127, (e - 1) - 2));
  }
  unsigned long long pc[3] = {0ull, 0ull, 0ull};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const unsigned long long c = f32_to_e2m3(ldexpf(v[j >> 4][j & 15], -x));   // exact power-of-two scaling
    const int bit = 6 * j, wd = bit >> 6, off = bit & 63;
    pc[wd] |= c << off;
    if (off > 58) pc[wd + 1] |= c >> (64 - off);
  }
  uint8_t* row = q + (size_t)(b >> 2) * x6_plane_bytes(cap) + (size_t)r * X6_ROWB;
  const int g = b & 3;
  *(i32x4_t*)(row + x6_off16(g)) = i32x4_t{(int)pc[0], (int)(pc[0] >> 32), (int)pc[1], (int)(pc[1] >> 32)};
  st8(row + x6_off8(g), make_uint2((uint32_t)pc[2], (uint32_t)(pc[2] >> 32)));
  scale[(size_t)(b >> 2) * cap * 4 + r * 4 + (b & 3)] = (uint8_t)(x + 127);
}

// bf16 -> IEEE binary16, 8 values a thread (round to nearest even; the NVFP4
// path's fp16 MFMA takes fp16 tokens).  n % 8 == 0.
__global__ void __launch_bounds__(256) cvt_f16_kernel(const uint16_t* __restrict__ src, long n,
                                                      uint16_t* __restrict__ dst) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const i32x4_t v = ld16(src + i);
  i32x4_t o;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = (int)pack_f16x2(bf16_bits_to_f32((uint32_t)v[k] & 0xffffu), bf16_bits_to_f32((uint32_t)v[k] >> 16));
  *(i32x4_t*)(dst + i) = o;
}

extern "C" hipError_t moe_launch_cvt_f16(const void* src, long n, void* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  cvt_f16_kernel<<<(unsigned)((n / 8 + 255) / 256), 256, 0, s>>>((const uint16_t*)src, n, (uint16_t*)dst);
  return hipGetLastError();
}

extern "C" hipError_t moe_launch_combine(const uint16_t* Z, const int32_t* ids, const float* w, const int32_t* pos,
                                         const uint32_t* miss_mask, const int32_t* slot_row, const float* hp,
                                         const int32_t* hp_count, int T, int k, int H, uint16_t* out,
                                         float* out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // one wave per workgroup: a token's H/8 threads spread over H/512 CUs
  dim3 g((H / 8 + 63) / 64, T);
  combine_kernel<<<g, 64, 0, s>>>(Z, ids, w, pos, miss_mask, slot_row, hp, hp_count, T, k, H, out, out_f32);
  return hipGetLastError();
}

// fmt WFMT_MXFP4_A6: MXFP6 codes and scales in 128-column planes sized for
// cap rows (x6_plane_bytes); cols % 128 == 0, rows <= cap.
extern "C" hipError_t moe_launch_quant(int fmt, int src_bf16, const void* src, int rows, const int32_t* nrows_dev,
                                       const int32_t* row_map, int cols, uint8_t* q, void* scale, int cap,
                                       hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (fmt == WFMT_MXFP4_A6) {
    if (cols % 128 || cap < rows) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)(((long)rows * (cols / 32) + 255) / 256);
    if (src_bf16)
      quant_mxfp6_kernel<true><<<blocks, 256, 0, s>>>(src, rows, nrows_dev, row_map, cols, cap, q, (uint8_t*)scale);
    else
      quant_mxfp6_kernel<false><<<blocks, 256, 0, s>>>(src, rows, nrows_dev, row_map, cols, cap, q,
                                                       (uint8_t*)scale);
    return hipGetLastError();
  }
  const long threads = (long)rows * (cols / 16);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (fmt == WFMT_FP8) {
    if (cols % 128) return hipErrorInvalidValue;
    if (src_bf16)
      quant_fp8_kernel<true><<<blocks, 256, 0, s>>>(src, rows, nrows_dev, row_map, cols, q, (float*)scale);
    else
      quant_fp8_kernel<false><<<blocks, 256, 0, s>>>(src, rows, nrows_dev, row_map, cols, q, (float*)scale);
  } else {
    if (cols % 32) return hipErrorInvalidValue;
    if (src_bf16)
      quant_mxfp8_kernel<true><<<blocks, 256, 0, s>>>(src, rows, nrows_dev, row_map, cols, q, (uint8_t*)scale);
    else
      quant_mxfp8_kernel<false><<<blocks, 256, 0, s>>>(src, rows, nrows_dev, row_map, cols, q, (uint8_t*)scale);
  }
  return hipGetLastError();
}
