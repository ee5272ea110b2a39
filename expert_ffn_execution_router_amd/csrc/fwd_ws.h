// Internal (not part of the C ABI): the routed layer forward over a
// workspace the caller hands in, with no library context.  Used by the
// allocation-free entry point, whose workspace is a static device array.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

// Bytes of the forward-only workspace for cfg at T <= max_T, of which
// part_bytes hold the small-batch GEMMs' partial tiles (the partial-tile
// area comes last).
size_t moe_fwd_ws_bytes(const moe_config* cfg, int max_T, size_t part_bytes);

// moe_layer_forward over ws (device, moe_fwd_ws_bytes bytes, 256-byte
// aligned) for T <= max_T: routing, grouping, both grouped GEMMs and the
// combine, enqueued on s.  err: device flag the kernels OR their error bits
// into (bit 0: a routed unmasked expert without a slot).  Returns a MOE_*
// code; on error *msg (may be NULL) points at a static description.
int moe_fwd_on_ws(const moe_config* cfg, int max_T, uint8_t* ws, size_t part_bytes, int n_cu,
                  const void* slot_pool, const int32_t* slot_row, const void* hidden, const float* router_w,
                  const float* router_bias, int T, const uint32_t* miss_mask, const float* host_partial,
                  void* out, int* err, hipStream_t s, const char** msg);

// Sets the message moe_last_error(NULL) returns on the calling thread.
void moe_set_thread_error(const char* msg);
