// Shared device-side definitions of the MoE layer library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <type_traits>

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef int i32x4_t __attribute__((__vector_size__(4 * sizeof(int))));
typedef int i32x8_t __attribute__((__vector_size__(8 * sizeof(int))));

#define DEV __device__ __forceinline__

enum { WFMT_BF16 = 0, WFMT_FP8 = 1, WFMT_MXFP4 = 2, WFMT_NVFP4 = 3 };
// Internal to the large-batch path: MXFP4 weights with MXFP6 (E2M3)
// activations.
enum { WFMT_MXFP4_A6 = 4 };
// Internal to the small-batch path: fp8 or MXFP4 weights met by bf16
// activations, the weights dequantised to bf16 in registers.
enum { WFMT_FP8_A16 = 5, WFMT_MXFP4_A16 = 6 };

// fp32 value of an E8M0 scale byte, 2^(e - 127) (e = 0 is the fp32
// subnormal 2^-127; 255, NaN, is never stored).
DEV float e8m0_to_f32(uint32_t e) { return __uint_as_float(e ? e << 23 : 0x00400000u); }

// MXFP6 activation rows: per 128-column chunk c a plane of 112-byte rows;
// the 32 six-bit codes of column block 4c + g form a 24-byte little-endian
// string (code j at bits 6j..6j+5) at bytes [24g, 24g+24) of the row, its
// bytes 0-15 at the 16-byte aligned offset x6_off16(g) and bytes 16-23 at
// x6_off8(g); bytes 96-111 are padding.  At a 112-byte stride any 16
// consecutive rows read at one offset, 16 bytes a lane (or 8 bytes, two lane
// groups at a time), cover the 64 LDS banks once.
// Their E8M0 scales are chunk-major too: plane c holds 4 bytes per row (the
// scales of column blocks 4c..4c+3), so a tile's scales of one chunk are one
// contiguous range.  Planes are sized for a row capacity: x6_plane_bytes(cap)
// for the codes (plus the 1 KiB the large-batch GEMM may read past the last
// row) and 4 * cap for the scales.
constexpr int X6_ROWB = 112;
DEV int x6_off16(int g) { return 24 * g + ((g & 1) << 3); }
DEV int x6_off8(int g) { return 24 * g + ((g & 1) ? 0 : 16); }
__host__ __device__ inline size_t x6_plane_bytes(size_t cap) {
  return (cap * X6_ROWB + 1024 + 255) / 256 * 256;
}

// m-block size used when only the grouping (not a GEMM) reads the work list.
constexpr int DEC_MB = 64;

// Device-resident description of one forward's grouped work, written by the
// grouping kernels and read by the GEMM kernels (no host round trip).
struct WorkList {
  int n_act;          // experts that run on the GPU this call
  int n_mblk;         // total m-blocks over those experts
  int mb;             // tokens per m-block used to build mblk_prefix
  int pad;
  int act_e[256];     // expert id of active expert a (ascending ids)
  int act_slot[256];  // slot holding it
  int mblk_prefix[257];
};

// A gate/up matrix-vector launch that routes its one token itself (T = 1):
// every workgroup picks its expert from the router logits, and workgroup 0
// also writes the routing and grouping outputs (ids, w, counts, offsets,
// pos, perm_tok, the work list, per-pair slots) for the launches after it.
struct GemvRoute {
  const float* z;                 // logits [E]
  int E, k, mb;
  const uint32_t* miss_mask;      // may be null
  const int32_t* slot_row;        // may be null: grouping only
  int32_t* ids;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* pos;
  int32_t* perm_tok;
  WorkList* wl;
  int* err;
  int32_t* pslot;
};

// Optional split of the large-batch work: an expert whose last m-tile would
// hold at most tau rows keeps one tile fewer, its main rows (mcounts) going
// to the tiled kernels through the main work list and the overflow rows
// (tcounts rows from toffsets) to the small-batch kernel through wl, built
// with m-blocks of mb rows.  The split is taken only when it removes a round
// of the persistent tiled grid (n_cu workgroups, ntiles items per m-tile)
// and its overflow items are few (at most n_cu / 4): re-streaming many
// experts' weights for their overflow rows costs more than the round.
// wl == nullptr: no split.
struct TailSplit {
  WorkList* wl;
  int32_t* mcounts;
  int32_t* tcounts;
  int32_t* toffsets;
  int mb, tau, n_cu, ntiles;
};

// Result of the per-layer cache-control kernel, copied to the host.
struct PlanOut {
  int n_unique, n_hit, m, q, n_host, n_evict, eligible, tick;
  int F[256];       // experts filled over the link, ascending
  int F_slot[256];  // their slots
  int C[256];       // experts executed on the host, ascending
};

// Device-resident cache-control state beside the residency table: the LRU
// clock (one tick per planning or layer-install call, advanced by the kernel
// itself so a captured graph replays with fresh ticks) and running plan
// statistics.
struct CacheCtl {
  uint32_t tick;
  uint32_t pad[3];
  unsigned long long calls, n_unique, n_hit, m, q, n_host, n_evict, pad2;
};

// Pinned host staging (device mappings) that the cache-control kernel fills
// for a host branch: the plan and the routed inputs.  plan == nullptr: none.
struct HostStage {
  PlanOut* plan;
  int32_t* ids;
  float* w;
  uint16_t* hidden;
  const float* w_src;
  const uint16_t* hidden_src;
  int n_hidden;                 // T * H
};

DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

DEV uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two floats to packed bf16 (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
DEV uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Two floats to packed IEEE binary16 (low half = a), round to nearest even,
// overflow to infinity.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((__vector_size__(8 * sizeof(_Float16))));
DEV uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}

// OCP E4M3FN code of v, round to nearest even, saturating at +-448.
DEV uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t s = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  float af = __uint_as_float(a);
  if (af >= 448.0f) return s | 0x7Eu;
  if (af < 0.015625f) {                      // below 2^-6: subnormal step 2^-9
    float q = rintf(af * 512.0f);            // exact scaling, RNE
    return s | (uint32_t)q;                  // q == 8 is the smallest normal code
  }
  int E = (int)(a >> 23) - 127;
  uint32_t m = a & 0x7fffffu;
  uint32_t r = m >> 20, rem = m & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  if (r == 8u) { r = 0u; ++E; }
  uint32_t code = ((uint32_t)(E + 7) << 3) | r;
  if (code > 0x7Eu) code = 0x7Eu;
  return s | code;
}

DEV float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

DEV float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

DEV i32x4_t ld16(const void* p) { return *(const i32x4_t*)p; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;
typedef uint8_t __attribute__((address_space(3))) lds_u8_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that leaves outstanding memory counters alone (a plain
// __syncthreads waits for every load in flight); the signal fences keep the
// compiler from moving LDS accesses across it.
DEV void barrier_keep_loads() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Streaming load for bytes read once (expert weights): the nontemporal hint
// keeps them from displacing reused lines and streams HBM at a higher rate
// (7.0-7.2 TB/s measured for 16-byte loads, against 6.0-6.4 TB/s without).
DEV i32x4_t ld16_nt(const void* p) { return __builtin_nontemporal_load((const i32x4_t*)p); }
DEV void st8(void* p, uint2 v) { *(uint2*)p = v; }

// Locate active expert a holding global m-block p (mblk_prefix ascending).
DEV int find_active(const WorkList* wl, int p) {
  int lo = 0, hi = wl->n_act - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (wl->mblk_prefix[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}
