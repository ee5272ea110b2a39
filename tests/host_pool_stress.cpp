// Two host threads share one host FFN thread pool, as the library's
// synchronous decode calls and the HIP host callbacks of an asynchronous step
// do: each submits jobs back to back; the pool must run them one at a time
// and every result must equal the same job run alone.  Then one thread
// submits jobs after idle gaps shorter and longer than the workers' polling
// window (workers still polling, just asleep, long asleep).  Built with
// ThreadSanitizer by tests/test_host_tsan.py; prints "ok" on success.
#include <algorithm>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "host_ffn.h"

namespace {

// bf16 bits of small normal values from a linear congruential generator
uint16_t next_bf16(uint64_t& s) {
  s = s * 6364136223846793005ull + 1442695040888963407ull;
  const uint32_t m = (uint32_t)(s >> 40) & 0x7f;             // mantissa
  const uint32_t e = 120 + (uint32_t)((s >> 50) & 3);          // 2^-7 .. 2^-4
  const uint32_t sg = (uint32_t)(s >> 63);
  return (uint16_t)((sg << 15) | (e << 7) | m);
}

struct Job {
  std::vector<uint16_t> hidden;
  std::vector<int32_t> ids;
  std::vector<float> w;
  std::vector<int32_t> C;
  std::vector<float> out;
};

}  // namespace

int main() {
  const int E = 4, k = 2, H = 256, I = 128, T = 3, L = 2;
  const size_t S = (size_t)3 * H * I * 2;
  const HostFfnShape sh{0, E, k, H, I, S};
  std::vector<uint8_t> pool((size_t)L * E * S);
  uint64_t seed = 12345;
  for (size_t i = 0; i < pool.size() / 2; ++i) ((uint16_t*)pool.data())[i] = next_bf16(seed);
  auto make_job = [&](int variant) {
    Job j;
    j.hidden.resize((size_t)T * H);
    for (auto& v : j.hidden) v = next_bf16(seed);
    j.ids.resize((size_t)T * k);
    j.w.resize((size_t)T * k);
    for (int t = 0; t < T; ++t)
      for (int q = 0; q < k; ++q) {
        j.ids[(size_t)t * k + q] = (t + q + variant) % E;
        j.w[(size_t)t * k + q] = 0.25f + 0.5f * q;
      }
    j.C = {variant % E, (variant + 1) % E};
    j.out.assign((size_t)T * H, 0.f);
    return j;
  };
  const int n_jobs = 12;
  std::vector<Job> a, b, ref_a, ref_b;
  for (int i = 0; i < n_jobs; ++i) {
    a.push_back(make_job(i));
    b.push_back(make_job(i + 1));
  }
  ref_a = a;
  ref_b = b;
  HostPool* P = host_pool_create(4);
  auto run = [&](std::vector<Job>& jobs, int layer) {
    for (auto& j : jobs) {
      HostFfnHandle* h = host_ffn_start(P, sh, pool.data(), layer, T, j.hidden.data(), j.ids.data(), j.w.data(),
                                        j.C.data(), (int)j.C.size(), j.out.data());
      (void)host_ffn_wait(P, h);
    }
  };
  run(ref_a, 0);                  // alone, one thread after the other
  run(ref_b, 1);
  std::thread t1([&] { run(a, 0); });
  std::thread t2([&] { run(b, 1); });
  t1.join();
  t2.join();
  // one thread again, with idle gaps on both sides of the workers' polling
  // window before each job, so a job finds the workers polling, just gone
  // to sleep, or long asleep
  std::vector<Job> c = ref_a;
  for (auto& j : c) std::fill(j.out.begin(), j.out.end(), 0.f);
  const int gaps_us[] = {0, 100, 450, 550, 1500, 3000};
  for (int i = 0; i < n_jobs; ++i) {
    std::this_thread::sleep_for(std::chrono::microseconds(gaps_us[i % 6]));
    Job& j = c[i];
    HostFfnHandle* h = host_ffn_start(P, sh, pool.data(), 0, T, j.hidden.data(), j.ids.data(), j.w.data(),
                                      j.C.data(), (int)j.C.size(), j.out.data());
    (void)host_ffn_wait(P, h);
  }
  host_pool_destroy(P);
  for (int i = 0; i < n_jobs; ++i)
    if (std::memcmp(a[i].out.data(), ref_a[i].out.data(), a[i].out.size() * 4) ||
        std::memcmp(b[i].out.data(), ref_b[i].out.data(), b[i].out.size() * 4) ||
        std::memcmp(c[i].out.data(), ref_a[i].out.data(), c[i].out.size() * 4)) {
      std::printf("mismatch in job %d\n", i);
      return 1;
    }
  std::printf("ok\n");
  return 0;
}
