// Argument checking and launch of one decode call, shared by the entry points
// that differ only in where the cross-partition partials live (not installed).
#pragma once

#include "pa.h"
#include "pa_internal.h"

namespace pa {

struct DecodeCall {
  DecodeArgs a;           // kernel arguments, partials pointers unset
  int G;                  // query heads per KV head
  bool even;              // the work is split evenly over the resident workgroups
  size_t partials_bytes;  // workspace the call needs (0: one partition covers every sequence)
};

// Checks every argument of pa_decode except the workspace and fills `call`.
// On PA_OK with call->a.S == 0 there is nothing to launch. `fn` names the
// entry point in error details.
pa_status decode_prepare(const char* fn, void* out, const void* query, const void* k_pool,
                         const void* v_pool, const int32_t* block_tables,
                         const int32_t* context_lens, int S, int Hq, int Hkv, int D, int B, int NB,
                         int MB, int max_context_len, float scale, int partition_size,
                         DecodeCall* call);

// Enqueues the partition kernel (and the reduce kernel when partitions need
// merging) with the partials at `partials`, a device buffer of at least
// call.partials_bytes bytes, 16-byte aligned (unused when that is 0).
pa_status decode_enqueue(const char* fn, DecodeCall& call, void* partials, hipStream_t stream);

}  // namespace pa
