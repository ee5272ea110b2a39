// Host FFN path: resident thread pool evaluating the host miss set C.
#pragma once
#include <cstddef>
#include <cstdint>

struct HostFfnShape {
  int fmt, E, k, H, I;
  size_t S;
};

struct HostPool;
struct HostFfnHandle;

HostPool* host_pool_create(int nthreads);
void host_pool_destroy(HostPool* p);
int host_pool_threads(const HostPool* p);

// Starts the job on the pool and returns at once; out[T*H] is overwritten
// with sum over (t, j) with ids[t,j] in C of w[t,j] * FFN_e(x_t).
// The pool runs one job at a time: a start holds the pool until the matching
// wait, so jobs started from different threads (a caller's synchronous call
// and a HIP host callback of an asynchronous step) run one after the other.
// The thread that calls host_ffn_start must call host_ffn_wait.
HostFfnHandle* host_ffn_start(HostPool* P, const HostFfnShape& sh, const uint8_t* pool, int layer, int T,
                              const uint16_t* hidden, const int32_t* ids, const float* w, const int32_t* C, int nC,
                              float* out);
// Waits for the job and returns its duration in ms, from the moment the
// pool took it to the moment its last worker finished.
double host_ffn_wait(HostPool* P, HostFfnHandle* h);
