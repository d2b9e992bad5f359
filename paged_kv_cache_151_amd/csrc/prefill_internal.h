// Internal declarations of the prefill kernel (not installed).
#pragma once

#include "pa_internal.h"

namespace pa {

// Query row tiles of 16 per prefill wave. More rows per wave read each
// staged key/value chunk from LDS for more rows, but hold more registers: one
// tile fits in about 150 VGPRs (three waves per SIMD); two tiles need about
// 300 (one wave per SIMD), and held to 256 they spill and measured 30 % slower.
#ifndef PA_PREFILL_ROW_TILES
#define PA_PREFILL_ROW_TILES 1
#endif
constexpr int kPrefillRowTiles = PA_PREFILL_ROW_TILES;
// Waves per prefill workgroup: they share each staged key/value chunk. The
// load layout (each wave loads one pool, K or V, of half the units of every
// chunk) is built for four. Eight (one workgroup per CU at two waves per
// SIMD) measured 15 % slower: nothing covers the barrier waits.
constexpr int kPrefillWaves = 4;
// Keys per pipeline step (32 or 64).
#ifndef PA_PREFILL_CHUNK
#define PA_PREFILL_CHUNK 32
#endif
constexpr int kPrefillChunk = PA_PREFILL_CHUNK;

// Arguments of the prefill kernel.
struct PrefillArgs {
  _Float16* out;                     // [T][Hq][D]
  const _Float16* q;                 // [T][Hq][D]
  const _Float16* k_pool;            // [NB][Hkv][B][D]
  const _Float16* v_pool;            // [NB][Hkv][B][D]
  const int32_t* tables;             // [S][MB]
  const int32_t* lens;               // [S]   tokens in the cache, new ones included
  const int32_t* qstart;             // [S+1] first packed query row of each sequence
  int S, T, Hq, Hkv, NB, MB, B;
  float scale_log2;                  // softmax scale times log2(e)
  int n_rank;                        // row blocks per (sequence, head group) in the launch
  int64_t n_work;                    // work items: n_rank * S * head groups * Hkv
  int64_t per_xcd;                   // work items per XCD: ceil(n_work / 8)
};

// Query rows one prefill workgroup covers for a group of G query heads.
int prefill_rows_per_workgroup(int G);

// Work items (workgroups before padding to a multiple of 8) of one launch.
int64_t prefill_work_items(int G, int S, int Hkv, int max_query_len);

// Launches the prefill kernel over ceil(max_query_len / rows) row blocks per
// sequence and head group.
hipError_t launch_prefill(const PrefillArgs& a, int B, int G, int max_query_len,
                          hipStream_t stream);

}  // namespace pa
