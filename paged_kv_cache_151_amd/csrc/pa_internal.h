// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kHeadDim = 128;        // decode kernels are specialised for D = 128
constexpr int kDecodeWaves = 4;      // waves per decode workgroup
constexpr int kMaxPartitions = 1 << 16;

// Arguments of the decode partition kernel (passed by value in the kernarg segment).
struct DecodeArgs {
  _Float16* out;                     // [S][Hq][D]
  const _Float16* q;                 // [S][Hq][D]
  const _Float16* k_pool;            // [NB][Hkv][B][D]
  const _Float16* v_pool;            // [NB][Hkv][B][D]
  const int32_t* tables;             // [S][MB]
  const int32_t* lens;               // [S]
  float* part_acc;                   // [S][Hq][Pmax][D]   (unused when Pmax == 1)
  float* part_ml;                    // [S][Hq][Pmax][2]   (running max, sum; log2 domain)
  int S, Hq, Hkv, NB, MB;
  int P;                             // partition size in tokens (multiple of B)
  int Pmax;                          // partitions the launch covers
  float scale_log2;                  // softmax scale times log2(e)
};

hipError_t launch_slot_mapping(int64_t* slots, const int32_t* tables, const int32_t* seq_ids,
                               const int32_t* positions, const int32_t* lens, int T, int S,
                               int MB, int B, int NB, hipStream_t stream);

hipError_t launch_write_kv(const void* key, const void* value, void* k_pool, void* v_pool,
                           const int64_t* slots, int T, int Hkv, int D, int B, int NB,
                           hipStream_t stream);

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int n, int Hkv,
                              int D, int B, int NB, hipStream_t stream);

// Launches the partition kernel and, when Pmax > 1, the cross-partition reduce.
hipError_t launch_decode(const DecodeArgs& a, int B, int G, hipStream_t stream);

}  // namespace pa
