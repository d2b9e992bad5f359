// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kHeadDim = 128;        // decode kernels are specialised for D = 128
constexpr int kDecodeUnit = 16;      // tokens per decode work unit; B and P are multiples
// Decode tuning parameters (compile-time): waves per workgroup, software
// prefetch depth in 16-token units, and whether K/V loads carry the
// non-temporal hint. Defaults are the fastest measured on MI355X for the
// batch-128 chat workload: 2 waves, depth 1 (82 VGPRs, 5 waves per SIMD),
// non-temporal loads (K/V bytes are read once; the hint keeps the stream
// from displacing cached lines and lifted a plain streaming read from 5.7 to
// 6.26 TB/s).
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 2
#endif
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 1
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif
// Query heads of one KV group that one wave serves (grouped-query attention).
// Fewer heads per wave means fewer registers but more waves re-reading each
// tile; on MI355X four heads per wave measured fastest for G = 4.
#ifndef PA_DECODE_HEADS_PER_WAVE
#define PA_DECODE_HEADS_PER_WAVE 4
#endif
#ifndef PA_DECODE_MIN_WAVES_PER_EU
#define PA_DECODE_MIN_WAVES_PER_EU 1
#endif
constexpr int kDecodeWaves = PA_DECODE_WAVES;
constexpr int kDecodeDepth = PA_DECODE_DEPTH;
constexpr bool kDecodeNontemporal = PA_DECODE_NT != 0;
constexpr int kDecodeHeadsPerWave = PA_DECODE_HEADS_PER_WAVE;

// Waves per decode workgroup for a query group of G heads: a group's update
// costs G times the arithmetic per tile, so larger groups split each
// partition's units over more waves (measured: 2 for one head, 4 for four).
constexpr int decode_waves(int G) {
  return G >= 8 ? 4 * kDecodeWaves : (G >= 4 ? 2 * kDecodeWaves : kDecodeWaves);
}

// Compute units of one MI355X (8 XCDs x 32).
constexpr int64_t kComputeUnits = 256;

// Launches of at most this many workgroups leave most SIMDs with one wave or
// none; groups of one or two heads then double their waves per workgroup, so
// more tile loads are in flight per compute unit (measured on batch-1 to
// batch-8 decode: 3-9 % faster, one shape 3 % slower).
constexpr int64_t kSmallLaunchWorkgroups = 2 * kComputeUnits;
constexpr int kMaxPartitions = 1 << 16;
// Devices a process may use the library on (per-device caches).
constexpr int kMaxDevices = 64;

// Batches whose sequences span more than one partition split their work
// evenly over the workgroups the GPU holds at once instead of one workgroup
// per partition. Pieces of a sequence are then at least P tokens long, except
// where a run begins or ends, so a sequence has at most ceil(L / P) + 1 of
// them. Each workgroup reads all S lengths first, which bounds S; positions in
// the split are 32-bit. For one or two query heads per KV head the split is
// taken only when the per-partition grid is larger than one round of the
// vector kernel's resident workgroups (8 per CU): with one round every
// partition starts at the launch, there is no late tail to remove, and the
// split measured 0.6-2.3 % slower (16 x 4,096 tokens, 32 heads) against 1.1 %
// faster on the chat lengths (12,288 partitions).
constexpr int kEvenSplitMaxSeqs = 1024;
constexpr int64_t kVecEvenSplitMinPartitions = 8 * kComputeUnits;
#ifndef PA_EVEN_SPLIT_MIN_PARTS
#define PA_EVEN_SPLIT_MIN_PARTS 2
#endif
inline bool decode_even_split(int S, int Hq, int Hkv, int P, int64_t partitions) {
  const int G = Hkv > 0 ? Hq / Hkv : 0;
  if ((G != 1 && G != 2 && G != 4 && G != 8) || partitions < PA_EVEN_SPLIT_MIN_PARTS ||
      partitions < 2 || S > kEvenSplitMaxSeqs)
    return false;
  if (G <= 2 && (int64_t)S * Hkv * partitions <= kVecEvenSplitMinPartitions) return false;
  const int64_t units = (int64_t)S * Hkv * partitions * (P / kDecodeUnit);
  const int64_t runs = (int64_t)S * Hkv * partitions + 8;
  return units + runs + 9 * (int64_t)(P / kDecodeUnit) < ((int64_t)1 << 31);
}

// Arguments of the decode partition kernel (passed by value in the kernarg segment).
struct DecodeArgs {
  _Float16* out;                     // [S][Hq][D]
  const _Float16* q;                 // [S][Hq][D]
  const _Float16* k_pool;            // [NB][Hkv][B][D]
  const _Float16* v_pool;            // [NB][Hkv][B][D]
  const int32_t* tables;             // [S][MB]
  const int32_t* lens;               // [S]
  float* part_acc;                   // [S][Hq][Pmax][D] fp16 rows in the first half of
                                     // this area (unused when Pmax == 1): a piece's
                                     // normalised result (weighted sum of values over
                                     // the sum of weights), row r at _Float16 index r * D
  float* part_ml;                    // [S][Hq][Pmax][2]   (running max, sum; log2 domain)
  int32_t* part_np;                  // [S][Hkv] pieces per sequence and KV head when the work
                                     // is split evenly (nullptr: one per partition)
  int S, Hq, Hkv, NB, MB;
  int B;                             // block size in tokens (multiple of 16)
  int P;                             // partition size in tokens (multiple of 16)
  int Pmax;                          // partial rows per (sequence, query head); lengths are
                                     // clamped to Pmax * P, or (Pmax - 1) * P when split evenly
  float scale_log2;                  // softmax scale times log2(e)
};

hipError_t launch_slot_mapping(int64_t* slots, const int32_t* tables, const int32_t* seq_ids,
                               const int32_t* positions, const int32_t* lens, int T, int S,
                               int MB, int B, int NB, hipStream_t stream);

// The slot mapping and the K/V store in one launch (slots may be nullptr).
hipError_t launch_append_kv(int64_t* slots, const void* key, const void* value, void* k_pool,
                            void* v_pool, const int32_t* tables, const int32_t* seq_ids,
                            const int32_t* positions, const int32_t* lens, int T, int S, int MB,
                            int Hkv, int D, int B, int NB, hipStream_t stream);

hipError_t launch_write_kv(const void* key, const void* value, void* k_pool, void* v_pool,
                           const int64_t* slots, int T, int Hkv, int D, int B, int NB,
                           hipStream_t stream);

// Copies block src of the source pools to block dst of the destination pools
// for each (src, dst) pair; the pools may be the same (copy-on-write).
hipError_t launch_copy_blocks(void* k_dst, void* v_dst, const void* k_src, const void* v_src,
                              const int32_t* pairs, int n, int Hkv, int D, int B, int NB_src,
                              int NB_dst, hipStream_t stream);

// Launches the partition kernel and, when Pmax > 1, the cross-partition reduce.
hipError_t launch_decode(const DecodeArgs& a, int B, int G, hipStream_t stream);

// Partition kernel for groups of G = 4 or 8 query heads on the matrix cores
// (B = 8 or a multiple of 16); same grid, outputs and partials as the vector
// kernel.
hipError_t launch_decode_mfma(const DecodeArgs& a, int B, int G, hipStream_t stream);

}  // namespace pa
