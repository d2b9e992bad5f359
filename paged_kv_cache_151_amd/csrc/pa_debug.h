// Bounds checks of the debug build (not installed).
//
// libpa_debug.so is built from the same sources with PA_DEBUG_BOUNDS=1. In it
// every global-memory access a kernel forms (a K/V tile or row inside its
// pool, a query row, a table entry, a length, an output or partial element, a
// slot or a copy pair) is first compared with the extent of the buffer it
// points into, as the call's sizes define it. An access that would leave its
// buffer is not made: a load reads zeros, a store is dropped, a tile's range
// becomes empty. The refusal is counted per check site in a device counter,
// which pa_debug_bounds_violations reads and clears. Nothing traps, so a run
// of the debug build ends normally whatever it finds.
//
// In the release build (PA_DEBUG_BOUNDS unset or 0) PA_IN_BOUNDS is the
// constant true and its condition is never evaluated: the kernels compile to
// the same code as without the checks.
#pragma once

#include <hip/hip_runtime.h>

#ifndef PA_DEBUG_BOUNDS
#define PA_DEBUG_BOUNDS 0
#endif

namespace pa {

// Check sites; each has one counter.
enum BoundsSite : int {
  kBsLength = 0,   // a context length or query start read
  kBsTable,        // a block-table entry read
  kBsQuery,        // a query row read
  kBsPool,         // a K/V tile or row inside its pool (read or written)
  kBsOut,          // an output element written
  kBsPartial,      // a partial result or piece count written or read
  kBsSlot,         // a slot or token index read (mapping, store)
  kBsPair,         // a copy pair read or its blocks inside their pools
  kBsSites
};

#if PA_DEBUG_BOUNDS
// One set of counters per translation unit; each unit exports a collector
// (PA_BOUNDS_COLLECTOR) that adds its counts into a host array and clears them.
static __device__ unsigned int g_bounds[kBsSites];

__device__ __forceinline__ bool bounds_ok(int site, bool ok) {
  if (!ok) atomicAdd(&g_bounds[site], 1u);
  return ok;
}

// Counts one refusal at every site of this unit's counters (no other memory
// is touched): the self-test of the counting path.
static __global__ void bounds_selftest_kernel() {
  if (threadIdx.x < kBsSites) bounds_ok((int)threadIdx.x, false);
}

#define PA_IN_BOUNDS(site, cond) (::pa::bounds_ok((site), (cond)))
#define PA_BOUNDS_COLLECTOR(name)                                                          \
  hipError_t name(unsigned int* acc) {                                                     \
    unsigned int c[kBsSites] = {};                                                         \
    hipError_t e = hipMemcpyFromSymbol(c, HIP_SYMBOL(g_bounds), sizeof(c), 0,              \
                                       hipMemcpyDeviceToHost);                             \
    if (e != hipSuccess) return e;                                                         \
    for (int i = 0; i < kBsSites; ++i) acc[i] += c[i];                                     \
    const unsigned int z[kBsSites] = {};                                                   \
    return hipMemcpyToSymbol(HIP_SYMBOL(g_bounds), z, sizeof(z), 0, hipMemcpyHostToDevice); \
  }                                                                                        \
  hipError_t name##_selftest() {                                                           \
    bounds_selftest_kernel<<<1, 64, 0, 0>>>();                                             \
    return hipGetLastError();                                                              \
  }
#else
#define PA_IN_BOUNDS(site, cond) (true)
#define PA_BOUNDS_COLLECTOR(name)
#endif

// Collectors of the translation units with kernels, and their self-tests
// (debug build only).
hipError_t bounds_take_cache_ops(unsigned int* acc);
hipError_t bounds_take_decode(unsigned int* acc);
hipError_t bounds_take_decode_mfma(unsigned int* acc);
hipError_t bounds_take_prefill(unsigned int* acc);
hipError_t bounds_take_cache_ops_selftest();
hipError_t bounds_take_decode_selftest();
hipError_t bounds_take_decode_mfma_selftest();
hipError_t bounds_take_prefill_selftest();

}  // namespace pa
