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
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <immintrin.h>
#include <mutex>
#include <condition_variable>
#include <functional>

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

// Eight E2M1 codes (one per byte of the low 8 bytes of c8) as floats times
// s: magnitude from a register table, sign bit moved to bit 31.
inline __m256 e2m1x8(__m128i c8, __m256 lut, __m256 s) {
  const __m256i idx = _mm256_cvtepu8_epi32(c8);
  const __m256 mag = _mm256_permutevar8x32_ps(lut, idx);               // low 3 bits select
  const __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(idx, _mm256_set1_epi32(8)), 28);
  return _mm256_mul_ps(_mm256_xor_ps(mag, _mm256_castsi256_ps(sgn)), s);
}

// 16 packed bytes = 32 E2M1 codes (even element in the low nibble), in
// element order, into dst[0..32): codes 0-15 times s0, 16-31 times s1.
inline void e2m1x32(const uint8_t* p, __m256 lut, __m256 s0, __m256 s1, float* dst) {
  const __m128i b = _mm_loadu_si128((const __m128i*)p);
  const __m128i m = _mm_set1_epi8(0x0F);
  const __m128i lo = _mm_and_si128(b, m), hi = _mm_and_si128(_mm_srli_epi16(b, 4), m);
  const __m128i e0 = _mm_unpacklo_epi8(lo, hi), e1 = _mm_unpackhi_epi8(lo, hi);   // codes 0-15, 16-31
  _mm256_storeu_ps(dst, e2m1x8(e0, lut, s0));
  _mm256_storeu_ps(dst + 8, e2m1x8(_mm_srli_si128(e0, 8), lut, s0));
  _mm256_storeu_ps(dst + 16, e2m1x8(e1, lut, s1));
  _mm256_storeu_ps(dst + 24, e2m1x8(_mm_srli_si128(e1, 8), lut, s1));
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

// Dequantise row `r` of matrix `mat` (0 gate, 1 up, 2 down) into dst[cols]
// (AVX2; cols is a multiple of 128 for every format the library accepts).
void load_row(const HostFfnShape& sh, const uint8_t* blob, int mat, int r, float* dst) {
  const int cols = mat < 2 ? sh.H : sh.I;
  const size_t n = (size_t)sh.H * sh.I;
  const Tables& tb = tables();
  if (sh.fmt == 0) {
    const uint16_t* w = (const uint16_t*)blob + mat * n + (size_t)r * cols;
    for (int c = 0; c < cols; c += 8) {
      const __m256i v = _mm256_cvtepu16_epi32(_mm_loadu_si128((const __m128i*)(w + c)));
      _mm256_storeu_ps(dst + c, _mm256_castsi256_ps(_mm256_slli_epi32(v, 16)));
    }
  } else if (sh.fmt == 1) {
    const uint8_t* q = blob + mat * n + (size_t)r * cols;
    const float* sc = (const float*)(blob + 3 * n) + mat * (n / 16384) + (size_t)(r / 128) * (cols / 128);
    const float p120 = std::ldexp(1.0f, 120);
    for (int b = 0; b < cols / 128; ++b) {
      const __m256 s = _mm256_set1_ps(sc[b] * p120);      // exact: a power-of-two factor
      for (int c = b * 128; c < b * 128 + 128; c += 8) _mm256_storeu_ps(dst + c, e4m3x8(q + c, s));
    }
  } else {
    // E2M1 magnitudes for codes 0..7
    const __m256 lut = _mm256_setr_ps(0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f);
    const uint8_t* p = blob + mat * (n / 2) + (size_t)r * (cols / 2);
    if (sh.fmt == 3) {
      // NVFP4: E4M3 block scale per 16 inputs and one fp32 scale per matrix
      const uint8_t* sc = blob + 3 * (n / 2) + mat * (n / 16) + (size_t)r * (cols / 16);
      float t;
      std::memcpy(&t, blob + 3 * (n / 2) + 3 * (n / 16) + 4 * mat, 4);
      for (int b = 0; b < cols / 32; ++b)
        e2m1x32(p + b * 16, lut, _mm256_set1_ps(tb.e4m3[sc[2 * b]] * t), _mm256_set1_ps(tb.e4m3[sc[2 * b + 1]] * t),
                dst + b * 32);
    } else {
      const uint8_t* sc = blob + 3 * (n / 2) + mat * (n / 32) + (size_t)r * (cols / 32);
      for (int b = 0; b < cols / 32; ++b) {
        const __m256 s = _mm256_set1_ps(tb.e8m0[sc[b]]);
        e2m1x32(p + b * 16, lut, s, s, dst + b * 32);
      }
    }
  }
}

inline float dot(const float* a, const float* b, int n) {
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

}  // namespace

// ---------------------------------------------------------------------------
// resident thread pool with a phase barrier
// ---------------------------------------------------------------------------
struct HostPool {
  int n;
  std::vector<std::thread> th;
  std::mutex mu;
  std::condition_variable cv, done_cv;
  std::function<void(int)> job;
  uint64_t gen = 0;
  int running = 0;
  bool stop = false;
  // one job at a time: held from host_ffn_start to host_ffn_wait
  std::mutex job_mu;
  std::chrono::steady_clock::time_point t_start, t_done;
  // spin barrier for phases inside a job
  std::atomic<int> bar_count{0};
  std::atomic<int> bar_gen{0};

  explicit HostPool(int nthreads) : n(nthreads < 1 ? 1 : nthreads) {
    for (int i = 0; i < n; ++i) th.emplace_back([this, i] { loop(i); });
  }
  ~HostPool() {
    {
      std::lock_guard<std::mutex> g(mu);
      stop = true;
    }
    cv.notify_all();
    for (auto& t : th) t.join();
  }
  void loop(int id) {
    uint64_t seen = 0;
    for (;;) {
      std::function<void(int)> f;
      {
        std::unique_lock<std::mutex> g(mu);
        cv.wait(g, [&] { return stop || gen != seen; });
        if (stop) return;
        seen = gen;
        f = job;
      }
      f(id);
      {
        std::lock_guard<std::mutex> g(mu);
        if (--running == 0) {
          t_done = std::chrono::steady_clock::now();
          done_cv.notify_all();
        }
      }
    }
  }
  void start(std::function<void(int)> f) {
    {
      std::lock_guard<std::mutex> g(mu);
      job = std::move(f);
      running = n;
      ++gen;
      t_start = std::chrono::steady_clock::now();
    }
    cv.notify_all();
  }
  // duration of the finished job in ms
  double wait() {
    std::unique_lock<std::mutex> g(mu);
    done_cv.wait(g, [&] { return running == 0; });
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

// Body of the host FFN for worker `id` of `nt`.  Shared scratch lives in `ws`.
struct HostFfnWork {
  HostFfnShape sh;
  const uint8_t* pool;
  int layer, T;
  const uint16_t* hidden;
  const int32_t* ids;
  const float* w;
  const int32_t* C;
  int nC;
  float* out;
  // scratch
  std::vector<int> tok, jj;
  std::vector<float> X, A;   // [n_e, H], [n_e, I]
};

static void host_ffn_worker(HostPool* P, HostFfnWork* W, int id) {
  const HostFfnShape& sh = W->sh;
  const int nt = P->n, H = sh.H, I = sh.I, k = sh.k;
  const size_t S = sh.S;
  std::vector<float> row((size_t)(H > I ? H : I)), row2((size_t)H);
  // zero own slice of out
  {
    const size_t tot = (size_t)W->T * H;
    const size_t a = tot * id / nt, b = tot * (id + 1) / nt;
    std::memset(W->out + a, 0, (b - a) * sizeof(float));
  }
  P->barrier();
  for (int ci = 0; ci < W->nC; ++ci) {
    const int e = W->C[ci];
    const uint8_t* blob = W->pool + ((size_t)W->layer * sh.E + e) * S;
    if (id == 0) {
      W->tok.clear();
      W->jj.clear();
      for (int t = 0; t < W->T; ++t)
        for (int j = 0; j < k; ++j)
          if (W->ids[(size_t)t * k + j] == e) { W->tok.push_back(t); W->jj.push_back(j); }
      const int ne = (int)W->tok.size();
      W->X.resize((size_t)ne * H);
      W->A.resize((size_t)ne * I);
      for (int r = 0; r < ne; ++r)
        for (int h = 0; h < H; ++h) {
          const uint32_t u = (uint32_t)W->hidden[(size_t)W->tok[r] * H + h] << 16;
          float f;
          std::memcpy(&f, &u, 4);
          W->X[(size_t)r * H + h] = f;
        }
    }
    P->barrier();
    const int ne = (int)W->tok.size();
    if (ne > 0) {
      // gate / up rows [i0, i1)
      const int i0 = (int)((long)I * id / nt), i1 = (int)((long)I * (id + 1) / nt);
      for (int i = i0; i < i1; ++i) {
        load_row(sh, blob, 0, i, row.data());
        load_row(sh, blob, 1, i, row2.data());
        for (int r = 0; r < ne; ++r) {
          const float* x = &W->X[(size_t)r * H];
          const float g = dot(row.data(), x, H);
          const float u = dot(row2.data(), x, H);
          W->A[(size_t)r * I + i] = g / (1.0f + std::exp(-g)) * u;
        }
      }
    }
    P->barrier();
    if (ne > 0) {
      const int h0 = (int)((long)H * id / nt), h1 = (int)((long)H * (id + 1) / nt);
      for (int h = h0; h < h1; ++h) {
        load_row(sh, blob, 2, h, row.data());
        for (int r = 0; r < ne; ++r) {
          const float y = dot(row.data(), &W->A[(size_t)r * I], I);
          const int t = W->tok[r];
          W->out[(size_t)t * H + h] += W->w[(size_t)t * k + W->jj[r]] * y;
        }
      }
    }
    P->barrier();
  }
}

struct HostFfnHandle {
  HostFfnWork work;
};

HostFfnHandle* host_ffn_start(HostPool* P, const HostFfnShape& sh, const uint8_t* pool, int layer, int T,
                              const uint16_t* hidden, const int32_t* ids, const float* w, const int32_t* C, int nC,
                              float* out) {
  HostFfnHandle* h = new HostFfnHandle();
  HostFfnWork& W = h->work;
  W.sh = sh;
  W.pool = pool;
  W.layer = layer;
  W.T = T;
  W.hidden = hidden;
  W.ids = ids;
  W.w = w;
  W.C = C;
  W.nC = nC;
  W.out = out;
  HostFfnWork* wp = &W;
  P->job_mu.lock();                 // released by host_ffn_wait on this thread
  P->start([P, wp](int id) { host_ffn_worker(P, wp, id); });
  return h;
}

double host_ffn_wait(HostPool* P, HostFfnHandle* h) {
  const double ms = P->wait();
  delete h;
  P->job_mu.unlock();
  return ms;
}
