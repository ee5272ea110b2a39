// Host-side expert execution for the miss set C.
//
// Method (paper.oopus.info review of FreeToken, sections 2.5-2.6): experts in
// C run on the CPU straight from the host expert pool, on a resident thread
// pool, with dequantisation inside the kernel so the path stays bound by host
// memory bandwidth; it returns the gate-weighted per-token partial output,
// which the GPU adds to its own partial sum.
//
// Arithmetic: fp32 throughout (x widened exactly from bf16, weights
// dequantised exactly, g, u, a = silu(g)*u and the down projection in fp32),
// no intermediate rounding.  Experts are processed in ascending id order and
// each output element is owned by one thread, so the result is deterministic.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <immintrin.h>
#include <thread>
#include <type_traits>
#include <vector>
#include <immintrin.h>
#include <mutex>

#include "host_ffn.h"

namespace {

// E4M3FN value of each code, from the bit fields (bias 7, S.1111.111 = NaN).
struct Tables {
  float e4m3[256];
  float e2m1[16];
  float e8m0[256];                    // 2^(c-127); 255 (NaN) is never stored
  Tables() {
    for (int c = 0; c < 256; ++c) {
      const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
      float v;
      if (e == 15 && m == 7) v = NAN;
      else if (e == 0) v = std::ldexp((float)m, -9);
      else v = std::ldexp(1.0f + m / 8.0f, e - 7);
      e4m3[c] = s ? -v : v;
    }
    for (int c = 0; c < 256; ++c) e8m0[c] = std::ldexp(1.0f, c - 127);
    for (int c = 0; c < 16; ++c) {
      const int s = c >> 3, e = (c >> 1) & 3, m = c & 1;
      const float v = e == 0 ? 0.5f * m : std::ldexp(1.0f + 0.5f * m, e - 1);
      e2m1[c] = s ? -v : v;
    }
  }
};
const Tables& tables() {
  static Tables t;
  return t;
}

// ---------------------------------------------------------------------------
// Row kernels.  With AVX-512 a weight row of `cols` inputs meets up to 8
// token vectors per pass: it is dequantised in registers and multiplied with
// no intermediate buffer.  The AVX2 baseline decodes the row once into a
// buffer and dots it with each vector.  Input vectors are stored in the row's
// decode order: natural for bf16 and fp8; for the E2M1 formats, within every
// 32 inputs the 16 even ones then the 16 odd ones (the order in which the low
// and high nibbles of 16 bytes come out).
// ---------------------------------------------------------------------------
// Position of input i of a row in decode order.
inline int arranged(int fmt, int i) {
  if (fmt < 2) return i;
  const int w = i & 31;
  return (i & ~31) + ((w & 1) << 4) + (w >> 1);
}

// One dequantisation row: codes, its scales and the matrix scale.
struct Row {
  int fmt, cols;
  const uint8_t* q;       // bf16 values, E4M3 codes, or packed E2M1 codes
  const float* s8;        // fp8: the row's fp32 block scales, one per 128 inputs
  const uint8_t* sb;      // mxfp4: E8M0 per 32 inputs; nvfp4: E4M3 per 16 inputs
  float t;                // nvfp4: matrix scale
};

Row make_row(const HostFfnShape& sh, const uint8_t* blob, int mat, int r) {
  const int cols = mat < 2 ? sh.H : sh.I;
  const size_t n = (size_t)sh.H * sh.I;
  Row w{sh.fmt, cols, nullptr, nullptr, nullptr, 1.0f};
  if (sh.fmt == 0) {
    w.q = blob + (mat * n + (size_t)r * cols) * 2;
  } else if (sh.fmt == 1) {
    w.q = blob + mat * n + (size_t)r * cols;
    w.s8 = (const float*)(blob + 3 * n) + mat * (n / 16384) + (size_t)(r / 128) * (cols / 128);
  } else {
    w.q = blob + mat * (n / 2) + (size_t)r * (cols / 2);
    if (sh.fmt == 3) {
      w.sb = blob + 3 * (n / 2) + mat * (n / 16) + (size_t)r * (cols / 16);
      std::memcpy(&w.t, blob + 3 * (n / 2) + 3 * (n / 16) + 4 * mat, 4);
    } else {
      w.sb = blob + 3 * (n / 2) + mat * (n / 32) + (size_t)r * (cols / 32);
    }
  }
  return w;
}

// ---- AVX2 (the x86-64-v3 baseline): decode the row, then dot -----------

// Eight E2M1 codes (one per byte of the low 8 bytes of c8) as floats times
// s: magnitude from a register table, sign bit moved to bit 31.
inline __m256 e2m1x8(__m128i c8, __m256 lut, __m256 s) {
  const __m256i idx = _mm256_cvtepu8_epi32(c8);
  const __m256 mag = _mm256_permutevar8x32_ps(lut, idx);               // low 3 bits select
  const __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(idx, _mm256_set1_epi32(8)), 28);
  return _mm256_mul_ps(_mm256_xor_ps(mag, _mm256_castsi256_ps(sgn)), s);
}

// Eight E4M3FN codes as floats times s: the 7 magnitude bits placed at the
// top of an fp32 mantissa/exponent give value * 2^-120 (subnormal codes
// land on fp32 subnormals, exact), so s carries the 2^120; sign to bit 31.
// (The NaN code S.1111.111 is not decoded as NaN; stored pools never hold it.)
inline __m256 e4m3x8(const uint8_t* p, __m256 s120) {
  const __m256i v = _mm256_cvtepu8_epi32(_mm_loadl_epi64((const __m128i*)p));
  const __m256i mag = _mm256_slli_epi32(_mm256_and_si256(v, _mm256_set1_epi32(0x7F)), 20);
  const __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(v, _mm256_set1_epi32(0x80)), 24);
  return _mm256_mul_ps(_mm256_castsi256_ps(_mm256_or_si256(mag, sgn)), s120);
}

// The row's values in decode order into dst[cols].
void decode_row_avx2(const Row& w, float* dst) {
  const Tables& tb = tables();
  if (w.fmt == 0) {
    const uint16_t* v = (const uint16_t*)w.q;
    for (int c = 0; c < w.cols; c += 8) {
      const __m256i x = _mm256_cvtepu16_epi32(_mm_loadu_si128((const __m128i*)(v + c)));
      _mm256_storeu_ps(dst + c, _mm256_castsi256_ps(_mm256_slli_epi32(x, 16)));
    }
  } else if (w.fmt == 1) {
    const float p120 = std::ldexp(1.0f, 120);
    for (int b = 0; b < w.cols / 128; ++b) {
      const __m256 s = _mm256_set1_ps(w.s8[b] * p120);      // exact: a power-of-two factor
      for (int c = b * 128; c < b * 128 + 128; c += 8) _mm256_storeu_ps(dst + c, e4m3x8(w.q + c, s));
    }
  } else {
    // E2M1 magnitudes for codes 0..7
    const __m256 lut = _mm256_setr_ps(0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f);
    const __m128i m4 = _mm_set1_epi8(0x0F);
    for (int b = 0; b < w.cols / 32; ++b) {
      // 16 bytes: low nibbles = the 16 even inputs, high nibbles = the 16 odd ones
      const __m128i x = _mm_loadu_si128((const __m128i*)(w.q + b * 16));
      const __m128i lo = _mm_and_si128(x, m4), hi = _mm_and_si128(_mm_srli_epi16(x, 4), m4);
      __m256 s0, s1;     // scales of inputs 0-15 and 16-31 of the block
      if (w.fmt == 3) {
        s0 = _mm256_set1_ps(tb.e4m3[w.sb[2 * b]] * w.t);
        s1 = _mm256_set1_ps(tb.e4m3[w.sb[2 * b + 1]] * w.t);
      } else {
        s0 = s1 = _mm256_set1_ps(tb.e8m0[w.sb[b]]);
      }
      float* d = dst + b * 32;
      _mm256_storeu_ps(d, e2m1x8(lo, lut, s0));                        // even inputs 0..14
      _mm256_storeu_ps(d + 8, e2m1x8(_mm_srli_si128(lo, 8), lut, s1));  // even inputs 16..30
      _mm256_storeu_ps(d + 16, e2m1x8(hi, lut, s0));
      _mm256_storeu_ps(d + 24, e2m1x8(_mm_srli_si128(hi, 8), lut, s1));
    }
  }
}

inline float dot_avx2(const float* a, const float* b, int n) {
  // n is a multiple of 128 (checked shapes): four independent 8-wide sums
  __m256 s0 = _mm256_setzero_ps(), s1 = _mm256_setzero_ps(), s2 = _mm256_setzero_ps(), s3 = _mm256_setzero_ps();
  for (int i = 0; i < n; i += 32) {
    s0 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i), _mm256_loadu_ps(b + i), s0);
    s1 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i + 8), _mm256_loadu_ps(b + i + 8), s1);
    s2 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i + 16), _mm256_loadu_ps(b + i + 16), s2);
    s3 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i + 24), _mm256_loadu_ps(b + i + 24), s3);
  }
  const __m256 s = _mm256_add_ps(_mm256_add_ps(s0, s1), _mm256_add_ps(s2, s3));
  const __m128 h = _mm_add_ps(_mm256_castps256_ps128(s), _mm256_extractf128_ps(s, 1));
  const __m128 q = _mm_add_ps(h, _mm_movehl_ps(h, h));
  return _mm_cvtss_f32(_mm_add_ss(q, _mm_shuffle_ps(q, q, 1)));
}

// ---- AVX-512 (runtime-selected): 16 values per instruction -------------
#define AVX512 __attribute__((target("avx512f,avx512bw,avx512dq,avx512vl")))

// Sixteen consecutive values of the row in decode order starting at input c
// (c a multiple of 16), fp8 with its block scale s120 (2^120 folded in).
AVX512 inline __m512 fp8x16(const uint8_t* q, __m512 s120) {
  const __m512i v = _mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i*)q));
  const __m512i mag = _mm512_slli_epi32(_mm512_and_si512(v, _mm512_set1_epi32(0x7F)), 20);
  const __m512i sgn = _mm512_slli_epi32(_mm512_and_si512(v, _mm512_set1_epi32(0x80)), 24);
  return _mm512_mul_ps(_mm512_castsi512_ps(_mm512_or_si512(mag, sgn)), s120);
}

// The 32 values of E2M1 block b (16 bytes at q + 16b) in decode order: lo =
// even inputs, hi = odd inputs, times the block's scale vector s (MXFP4: one
// value; NVFP4: lanes 0-7 for inputs 0-15, lanes 8-15 for inputs 16-31); the
// 16-entry table holds every signed E2M1 value.
AVX512 inline void fp4x32(const uint8_t* q, int b, __m512 lut, __m512 s, __m512& lo, __m512& hi) {
  const __m512i v = _mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i*)(q + b * 16)));
  lo = _mm512_mul_ps(_mm512_permutexvar_ps(v, lut), s);                          // index: low 4 bits
  hi = _mm512_mul_ps(_mm512_permutexvar_ps(_mm512_srli_epi32(v, 4), lut), s);
}

// The scale vector of E2M1 block b of the row (see fp4x32).
AVX512 inline __m512 fp4_scale(const float* e4m3, const float* e8m0, const uint8_t* sb, float t, bool nv, int b) {
  if (nv) return _mm512_insertf32x8(_mm512_set1_ps(e4m3[sb[2 * b]] * t), _mm256_set1_ps(e4m3[sb[2 * b + 1]] * t), 1);
  return _mm512_set1_ps(e8m0[sb[b]]);
}

// The E2M1 blocks of a row against N vectors (every invariant in a register).
template <int N, bool NV>
AVX512 inline void fp4_dots(const uint8_t* q, const uint8_t* sb, float t, int nb, __m512 lut, const Tables& tb,
                            const float* const* x, __m512 (*acc)[2]) {
  for (int b = 0; b < nb; ++b) {
    __m512 lo, hi;
    fp4x32(q, b, lut, fp4_scale(tb.e4m3, tb.e8m0, sb, t, NV, b), lo, hi);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      acc[j][0] = _mm512_fmadd_ps(lo, _mm512_loadu_ps(x[j] + b * 32), acc[j][0]);
      acc[j][1] = _mm512_fmadd_ps(hi, _mm512_loadu_ps(x[j] + b * 32 + 16), acc[j][1]);
    }
  }
}

// res[j] = row . xs[j] for j < N <= 8, the row dequantised in registers;
// two accumulators per vector (even and odd halves of a block), so no FMA
// chain waits on the previous one.
template <int N>
AVX512 void row_dots_avx512(const Row& w, const float* const* xs, float* res) {
  __m512 acc[N][2];
#pragma unroll
  for (int j = 0; j < N; ++j) acc[j][0] = acc[j][1] = _mm512_setzero_ps();
  if (w.fmt == 0) {
    const uint16_t* v = (const uint16_t*)w.q;
    for (int c = 0; c < w.cols; c += 32) {
      const __m512i x0 = _mm512_cvtepu16_epi32(_mm256_loadu_si256((const __m256i*)(v + c)));
      const __m512i x1 = _mm512_cvtepu16_epi32(_mm256_loadu_si256((const __m256i*)(v + c + 16)));
      const __m512 f0 = _mm512_castsi512_ps(_mm512_slli_epi32(x0, 16));
      const __m512 f1 = _mm512_castsi512_ps(_mm512_slli_epi32(x1, 16));
#pragma unroll
      for (int j = 0; j < N; ++j) {
        acc[j][0] = _mm512_fmadd_ps(f0, _mm512_loadu_ps(xs[j] + c), acc[j][0]);
        acc[j][1] = _mm512_fmadd_ps(f1, _mm512_loadu_ps(xs[j] + c + 16), acc[j][1]);
      }
    }
  } else if (w.fmt == 1) {
    const float p120 = std::ldexp(1.0f, 120);
    for (int b = 0; b < w.cols / 128; ++b) {
      const __m512 s = _mm512_set1_ps(w.s8[b] * p120);
#pragma unroll 2
      for (int c = b * 128; c < b * 128 + 128; c += 32) {
        const __m512 f0 = fp8x16(w.q + c, s), f1 = fp8x16(w.q + c + 16, s);
#pragma unroll
        for (int j = 0; j < N; ++j) {
          acc[j][0] = _mm512_fmadd_ps(f0, _mm512_loadu_ps(xs[j] + c), acc[j][0]);
          acc[j][1] = _mm512_fmadd_ps(f1, _mm512_loadu_ps(xs[j] + c + 16), acc[j][1]);
        }
      }
    }
  } else {
    // every loop-invariant in a local, so nothing is reloaded per block
    const Tables& tb = tables();
    const __m512 lut = _mm512_loadu_ps(tb.e2m1);
    const uint8_t* q = w.q;
    const uint8_t* sb = w.sb;
    const float t = w.t;
    const int nb = w.cols / 32;
    const bool nv = w.fmt == 3;
    const float* x[N];
#pragma unroll
    for (int j = 0; j < N; ++j) x[j] = xs[j];
    if (nv) fp4_dots<N, true>(q, sb, t, nb, lut, tb, x, acc);
    else fp4_dots<N, false>(q, sb, t, nb, lut, tb, x, acc);
  }
#pragma unroll
  for (int j = 0; j < N; ++j) res[j] = _mm512_reduce_add_ps(_mm512_add_ps(acc[j][0], acc[j][1]));
}

// AVX-512 when the host has it (MOE_HOST_ISA=avx2 forces the baseline).
bool use_avx512() {
  static const bool v = [] {
    const char* e = std::getenv("MOE_HOST_ISA");
    if (e && std::strcmp(e, "avx2") == 0) return false;
    __builtin_cpu_init();
    return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
           __builtin_cpu_supports("avx512dq") && __builtin_cpu_supports("avx512vl");
  }();
  return v;
}

// res[j] = row . xs[j], j < n: with AVX-512 fused in registers, up to 8
// vectors per pass over the row (16 accumulators; the row's 2-4 KB stay in
// L1 between passes); else the row decoded once into buf (cols floats) and
// dotted with each vector.
void row_dots(const Row& w, const float* const* xs, int n, float* res, float* buf) {
  if (use_avx512()) {
    for (int j0 = 0; j0 < n; j0 += 8) {
      const float* const* x = xs + j0;
      float* r = res + j0;
      switch (std::min(8, n - j0)) {
        case 1: row_dots_avx512<1>(w, x, r); break;
        case 2: row_dots_avx512<2>(w, x, r); break;
        case 3: row_dots_avx512<3>(w, x, r); break;
        case 4: row_dots_avx512<4>(w, x, r); break;
        case 5: row_dots_avx512<5>(w, x, r); break;
        case 6: row_dots_avx512<6>(w, x, r); break;
        case 7: row_dots_avx512<7>(w, x, r); break;
        default: row_dots_avx512<8>(w, x, r); break;
      }
    }
    return;
  }
  decode_row_avx2(w, buf);
  for (int j = 0; j < n; ++j) res[j] = dot_avx2(buf, xs[j], w.cols);
}

}  // namespace

// ---------------------------------------------------------------------------
// resident thread pool with a phase barrier
// ---------------------------------------------------------------------------
struct HostFfnWork;
static void host_ffn_worker(HostPool* P, const HostFfnWork* W, int id);

// Buffers of one job, kept by the pool between jobs (the pool runs one job
// at a time) so a job allocates nothing once they have grown to its size.
struct HostScratch {
  std::vector<int> slot;          // [E]: index in C of expert e, or -1
  std::vector<int> begin;         // [nC + 1]: expert ci's pairs are [begin[ci], begin[ci+1])
  std::vector<int> next;          // [nC]: next free pair of expert ci while bucketing
  std::vector<int> tok, jj;       // per pair: token and choice, expert-major, tokens ascending
  std::vector<float> X;           // [T][H]: hidden rows widened to fp32, decode order
  std::vector<float> A;           // [pairs][I]: SwiGLU activations, decode order
};

struct HostFfnWork {
  HostFfnShape sh;
  const uint8_t* pool;
  int layer, T;
  const uint16_t* hidden;
  const float* w;
  const int32_t* C;
  int nC;
  float* out;
  HostScratch* sc;
};

// Workers sleep on a generation word (a futex through std::atomic::wait, so
// a start wakes them all at once with no lock to queue on); the last one to
// finish stamps the end time and wakes the waiter.  Before sleeping, a
// worker polls the word for kSpinUs: the decode path starts one job per
// layer, a few hundred microseconds apart, and a worker woken from the futex
// starts tens of microseconds late (the last of 14 up to ~100 us on a busy
// host) while the job's phase barriers wait for every worker.  (The caller
// sleeps on the end of its job: polling there took a core from the workers
// for the whole job, and jobs of many experts ran up to half again longer.)
constexpr int kSpinUs = 500;

// Polls pred() with a pause between reads until it holds or `us`
// microseconds have passed; returns whether it held.
template <class P>
static bool spin_until(P pred, int us) {
  const auto t_end = std::chrono::steady_clock::now() + std::chrono::microseconds(us);
  for (int i = 0;; ++i) {
    if (pred()) return true;
    _mm_pause();
    if ((i & 63) == 63 && std::chrono::steady_clock::now() >= t_end) return pred();
  }
}

struct HostPool {
  int n;
  std::vector<std::thread> th;
  std::atomic<uint32_t> gen{0};
  std::atomic<uint32_t> done{1};
  std::atomic<int> running{0};
  std::atomic<bool> stop{false};
  const HostFfnWork* work = nullptr;   // published by the release on gen
  // one job at a time: held from host_ffn_start to host_ffn_wait
  std::mutex job_mu;
  HostScratch scratch;
  std::chrono::steady_clock::time_point t_start, t_done;
  // spin barrier for phases inside a job
  std::atomic<int> bar_count{0};
  std::atomic<int> bar_gen{0};

  explicit HostPool(int nthreads) : n(nthreads < 1 ? 1 : nthreads) {
    for (int i = 0; i < n; ++i) th.emplace_back([this, i] { loop(i); });
  }
  ~HostPool() {
    stop.store(true, std::memory_order_release);
    gen.fetch_add(1, std::memory_order_release);
    gen.notify_all();
    for (auto& t : th) t.join();
  }
  void loop(int id) {
    uint32_t seen = 0;
    for (;;) {
      if (!spin_until([&] { return gen.load(std::memory_order_acquire) != seen; }, kSpinUs))
        gen.wait(seen, std::memory_order_acquire);
      const uint32_t g = gen.load(std::memory_order_acquire);
      if (g == seen) continue;                    // spurious wake
      seen = g;
      if (stop.load(std::memory_order_acquire)) return;
      host_ffn_worker(this, work, id);
      if (running.fetch_sub(1, std::memory_order_acq_rel) == 1) {
        t_done = std::chrono::steady_clock::now();
        done.store(1, std::memory_order_release);
        done.notify_one();
      }
    }
  }
  void start(const HostFfnWork* w) {
    work = w;
    running.store(n, std::memory_order_relaxed);
    done.store(0, std::memory_order_relaxed);
    t_start = std::chrono::steady_clock::now();
    gen.fetch_add(1, std::memory_order_release);
    gen.notify_all();
  }
  // duration of the finished job in ms
  double wait() {
    while (done.load(std::memory_order_acquire) == 0) done.wait(0, std::memory_order_acquire);
    return std::chrono::duration<double, std::milli>(t_done - t_start).count();
  }
  void barrier() {
    const int g = bar_gen.load(std::memory_order_acquire);
    if (bar_count.fetch_add(1, std::memory_order_acq_rel) == n - 1) {
      bar_count.store(0, std::memory_order_relaxed);
      bar_gen.fetch_add(1, std::memory_order_acq_rel);
    } else {
      while (bar_gen.load(std::memory_order_acquire) == g) std::this_thread::yield();
    }
  }
};

HostPool* host_pool_create(int nthreads) { return new HostPool(nthreads); }
void host_pool_destroy(HostPool* p) { delete p; }
int host_pool_threads(const HostPool* p) { return p->n; }

// Worker `id` of the pool.  The routed (expert, token) pairs are bucketed
// by the caller.  Phases, separated by the pool's barrier:
//   1: zero this worker's slice of out; its share of the T hidden rows,
//      widened exactly to fp32 in decode order;
//   2: gate and up rows of every expert (the (expert, row) pairs split
//      evenly): a = silu(g) * u per routed token, stored in decode order;
//   3: down rows: each worker owns an H range and takes the experts in
//      ascending order, adding w * y to out (one writer per element, a fixed
//      order: deterministic).
static void host_ffn_worker(HostPool* P, const HostFfnWork* W, int id) {
  const HostFfnShape& sh = W->sh;
  const HostScratch& sc = *W->sc;
  const int nt = P->n, H = sh.H, I = sh.I, k = sh.k, fmt = sh.fmt, nC = W->nC;
  const size_t S = sh.S;
  float* X = W->sc->X.data();
  float* A = W->sc->A.data();
  thread_local std::vector<float> rowbuf;         // AVX2 row buffer, grown once per thread
  if (rowbuf.size() < (size_t)std::max(H, I)) rowbuf.resize((size_t)std::max(H, I));
  float* buf = rowbuf.data();
  const float* ptr[8];
  float r0[8], r1[8];
  {
    const size_t tot = (size_t)W->T * H;
    const size_t a = tot * id / nt, b = tot * (id + 1) / nt;
    std::memset(W->out + a, 0, (b - a) * sizeof(float));
    for (size_t i = a; i < b; ++i) {
      const size_t t = i / H;
      const int h = (int)(i % H);
      const uint32_t u = (uint32_t)W->hidden[i] << 16;
      std::memcpy(X + t * H + arranged(fmt, h), &u, 4);
    }
  }
  P->barrier();
  // phase 2: gate and up rows, up to 8 tokens of an expert per row pass
  {
    const long tot = (long)nC * I;
    const long g0 = tot * id / nt, g1 = tot * (id + 1) / nt;
    for (long g = g0; g < g1; ++g) {
      const int ci = (int)(g / I), i = (int)(g % I);
      const int p0 = sc.begin[ci], p1 = sc.begin[ci + 1];
      if (p0 == p1) continue;
      const uint8_t* blob = W->pool + ((size_t)W->layer * sh.E + W->C[ci]) * S;
      const Row wg = make_row(sh, blob, 0, i), wu = make_row(sh, blob, 1, i);
      const int ai = arranged(fmt, i);
      for (int q0 = p0; q0 < p1; q0 += 8) {
        const int ne = std::min(8, p1 - q0);
        for (int r = 0; r < ne; ++r) ptr[r] = X + (size_t)sc.tok[q0 + r] * H;
        row_dots(wg, ptr, ne, r0, buf);
        row_dots(wu, ptr, ne, r1, buf);
        for (int r = 0; r < ne; ++r) A[(size_t)(q0 + r) * I + ai] = r0[r] / (1.0f + std::exp(-r0[r])) * r1[r];
      }
    }
  }
  P->barrier();
  // phase 3: down rows, this worker's H range, experts ascending
  {
    const int h0 = (int)((long)H * id / nt), h1 = (int)((long)H * (id + 1) / nt);
    for (int ci = 0; ci < nC; ++ci) {
      const int p0 = sc.begin[ci], p1 = sc.begin[ci + 1];
      if (p0 == p1) continue;
      const uint8_t* blob = W->pool + ((size_t)W->layer * sh.E + W->C[ci]) * S;
      for (int q0 = p0; q0 < p1; q0 += 8) {
        const int ne = std::min(8, p1 - q0);
        for (int r = 0; r < ne; ++r) ptr[r] = A + (size_t)(q0 + r) * I;
        for (int h = h0; h < h1; ++h) {
          row_dots(make_row(sh, blob, 2, h), ptr, ne, r0, buf);
          for (int r = 0; r < ne; ++r) {
            const int t = sc.tok[q0 + r];
            W->out[(size_t)t * H + h] += W->w[(size_t)t * k + sc.jj[q0 + r]] * r0[r];
          }
        }
      }
    }
  }
}

struct HostFfnHandle {
  HostFfnWork work;
};

HostFfnHandle* host_ffn_start(HostPool* P, const HostFfnShape& sh, const uint8_t* pool, int layer, int T,
                              const uint16_t* hidden, const int32_t* ids, const float* w, const int32_t* C, int nC,
                              float* out) {
  P->job_mu.lock();                 // released by host_ffn_wait on this thread
  HostScratch& sc = P->scratch;
  nC = nC > 0 ? nC : 0;
  // bucket the routed pairs by expert: one pass over ids
  sc.slot.assign((size_t)sh.E, -1);
  for (int ci = 0; ci < nC; ++ci) sc.slot[C[ci]] = ci;
  sc.begin.assign((size_t)nC + 1, 0);
  for (int q = 0; q < T * sh.k; ++q) {
    const int e = ids[q];
    if (e >= 0 && e < sh.E && sc.slot[e] >= 0) ++sc.begin[sc.slot[e] + 1];
  }
  for (int ci = 0; ci < nC; ++ci) sc.begin[ci + 1] += sc.begin[ci];
  const int np = sc.begin[nC];
  sc.tok.resize((size_t)np);
  sc.jj.resize((size_t)np);
  sc.next.assign(sc.begin.begin(), sc.begin.end() - 1);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < sh.k; ++j) {
      const int e = ids[(size_t)t * sh.k + j];
      if (e < 0 || e >= sh.E || sc.slot[e] < 0) continue;
      const int q = sc.next[sc.slot[e]]++;
      sc.tok[q] = t;
      sc.jj[q] = j;
    }
  if (sc.X.size() < (size_t)T * sh.H) sc.X.resize((size_t)T * sh.H);
  if (sc.A.size() < (size_t)np * sh.I) sc.A.resize((size_t)np * sh.I);
  HostFfnHandle* h = new HostFfnHandle();
  HostFfnWork& W = h->work;
  W.sh = sh;
  W.pool = pool;
  W.layer = layer;
  W.T = T;
  W.hidden = hidden;
  W.w = w;
  W.C = C;
  W.nC = nC;
  W.out = out;
  W.sc = &sc;
  P->start(&W);
  return h;
}

double host_ffn_wait(HostPool* P, HostFfnHandle* h) {
  const double ms = P->wait();
  delete h;
  P->job_mu.unlock();
  return ms;
}
