// Internal declarations of the prefill kernel (not installed).
#pragma once

#include "pa_internal.h"

namespace pa {

// Query row tiles of 16 per prefill wave. More rows per wave read each
// staged key/value chunk from LDS for more rows, but hold more registers: one
// tile fits in about 150 VGPRs (three waves per SIMD), two in about 235 (two
// waves per SIMD). Measured on MI355X: for groups of 4 query heads (the
// shared-prefix suffixes) two tiles are 5 % faster (289 against 304 us); for
// one head per group (the 16-prompt chat batch) they tied in one session (292
// against 293) and were 2-3 % faster in two others (297-300 against 307-309).
#ifndef PA_PREFILL_ROW_TILES
#define PA_PREFILL_ROW_TILES 2
#endif
#ifndef PA_PREFILL_ROW_TILES_GROUPED
#define PA_PREFILL_ROW_TILES_GROUPED 2
#endif
constexpr int kPrefillRowTiles = PA_PREFILL_ROW_TILES;
// Row tiles per wave for a group of G query heads (4 and 8 take the grouped value).
constexpr int prefill_row_tiles(int G) {
  return G >= 4 ? PA_PREFILL_ROW_TILES_GROUPED : kPrefillRowTiles;
}
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
// LDS stages of the key/value pipeline (3 or 4): chunks are loaded
// kPrefillStages - 1 ahead of the one being computed.
#ifndef PA_PREFILL_STAGES
#define PA_PREFILL_STAGES 3
#endif
constexpr int kPrefillStages = PA_PREFILL_STAGES;

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
