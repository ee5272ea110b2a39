// Allocation-free variant of moe_layer_forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  Every intermediate of the forward
// (logits, routing, grouping, work lists, A, Z, quantised activations and
// the small-batch GEMMs' partial tiles) lives in one file-scope device
// array; the call computes exactly what moe_layer_forward computes, with the
// same kernels.
#include <mutex>

#include "fwd_ws.h"

namespace {

// Largest T of one call, and the scratch size: the forward's buffers for
// T <= 64 at the largest supported shape (E = 256, k = 8, H = 6144,
// I = 2048) take about 16 MiB, and what is left holds the partial tiles
// (the small-batch GEMMs cap their grid at the tiles that fit).
constexpr int NOALLOC_MAX_T = 64;
constexpr size_t SCRATCH_BYTES = (size_t)40 << 20;
constexpr size_t ERR_BYTES = 256;                    // the unreported error word when the caller passes none
constexpr size_t MIN_PART_BYTES = (size_t)4 << 20;   // below this the grid would be too small to stream well
constexpr int MAX_DEVICES = 64;

// One copy per GPU, held until the process ends.  Host code never uses this
// name as an address: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

std::mutex g_mu;
uint8_t* g_ptr[MAX_DEVICES];       // device address of `scratch`, per device
int g_ncu[MAX_DEVICES];

// the message moe_last_error(NULL) returns on this thread
int fail(int code, const char* m) {
  moe_set_thread_error(m);
  return code;
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(const moe_config* cfg, const void* slot_pool, const int32_t* slot_row,
                                         const void* hidden, const float* router_w, const float* router_bias,
                                         int T, const uint32_t* miss_mask, const float* host_partial, void* out,
                                         int* err_flag, void* stream) {
  if (!cfg) return fail(MOE_E_INVAL, "null config");
  const moe_config& c = *cfg;
  if (c.E < 1 || c.E > 256 || c.k < 1 || c.k > 8 || c.k > c.E)
    return fail(MOE_E_INVAL, "need 1 <= k <= 8, k <= E <= 256");
  if (c.H < 256 || c.H % 256 || c.I < 128 || c.I % 128) return fail(MOE_E_INVAL, "need H % 256 == 0 and I % 128 == 0");
  if (c.wfmt < 0 || c.wfmt > 3) return fail(MOE_E_INVAL, "unknown weight format");
  if (T < 0 || T > NOALLOC_MAX_T) return fail(MOE_E_UNSUPPORTED, "T outside [0, 64] for the allocation-free forward");
  if (T == 0) return MOE_OK;
  if (!hidden || !router_w || !out || !slot_row) return fail(MOE_E_INVAL, "null argument");
  const size_t fixed = ERR_BYTES + moe_fwd_ws_bytes(cfg, NOALLOC_MAX_T, 0);
  if (fixed + MIN_PART_BYTES > SCRATCH_BYTES)
    return fail(MOE_E_UNSUPPORTED, "shape too large for the allocation-free forward's 40 MiB scratch");
  const size_t part_bytes = (SCRATCH_BYTES - fixed) & ~(size_t)255;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return fail(MOE_E_HIP, "hipGetDevice failed");
  uint8_t* base;
  int n_cu;
  {
    // set-up once per device, with that device current
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return fail(MOE_E_HIP, "hipGetSymbolAddress of the scratch array failed");
      int ncu = 0;
      if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
        return fail(MOE_E_HIP, "device attribute query failed");
      g_ncu[dev] = ncu;
      g_ptr[dev] = (uint8_t*)p;
    }
    base = g_ptr[dev];
    n_cu = g_ncu[dev];
  }
  int* err = err_flag ? err_flag : (int*)base;
  const char* msg = "";
  const int rc = moe_fwd_on_ws(cfg, NOALLOC_MAX_T, base + ERR_BYTES, part_bytes, n_cu, slot_pool, slot_row, hidden,
                               router_w, router_bias, T, miss_mask, host_partial, out, err, (hipStream_t)stream, &msg);
  if (rc) return fail(rc, msg);
  return MOE_OK;
}
