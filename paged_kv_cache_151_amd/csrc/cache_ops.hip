// Cache-maintenance kernels: slot translation, token writes, block copies.
//
// [L] "Paged Attention: OS-Inspired Memory Management for KV Caches",
//     sections "How PagedAttention works" and "Memory sharing across requests".
// All three are bit-level: no arithmetic touches the cached values.
#include "pa_debug.h"
#include "pa_internal.h"

namespace pa {
namespace {

// slot of token i of sequence s = seq_ids[i] (or i) at position t =
// positions[i] (or lens[s] - 1): table entry of logical block t / B, times B,
// plus t % B. -1 when the token cannot be placed (bad sequence, position or
// table entry).
__device__ __forceinline__ int64_t token_slot(int i, const int32_t* __restrict__ tables,
                                              const int32_t* __restrict__ seq_ids,
                                              const int32_t* __restrict__ positions,
                                              const int32_t* __restrict__ lens, int S, int MB,
                                              int B, int NB) {
  const int s = seq_ids ? seq_ids[i] : i;
  int64_t slot = -1;
  if (s >= 0 && s < S) {
    const int t = positions ? positions[i] : (PA_IN_BOUNDS(kBsLength, s < S) ? lens[s] - 1 : -1);
    if (t >= 0) {
      const int j = t / B;
      if (j < MB) {
        const int64_t te = (int64_t)s * MB + j;
        const int phys = PA_IN_BOUNDS(kBsTable, te >= 0 && te < (int64_t)S * MB) ? tables[te] : -1;
        if (phys >= 0 && phys < NB) slot = (int64_t)phys * B + (t - j * B);
      }
    }
  }
  return slot;
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    int64_t* __restrict__ slots, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ lens, int T, int S, int MB, int B, int NB) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T) return;
  slots[i] = token_slot(i, tables, seq_ids, positions, lens, S, MB, B, NB);
}

// The slot mapping and the store in one pass: each thread of the store finds
// its token's slot itself (the token's threads read the same few index words,
// which the caches serve), and the first thread of each token records it.
__global__ __launch_bounds__(256) void append_kv_kernel(
    int64_t* __restrict__ slots_out, const uint4* __restrict__ key,
    const uint4* __restrict__ value, uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_ids,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ lens, int64_t total,
    int Hkv, int chunks, int S, int MB, int B, int NB) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int c = (int)(e % chunks);
  const int64_t ih = e / chunks;           // token * Hkv + head
  const int h = (int)(ih % Hkv);
  const int i = (int)(ih / Hkv);
  const int64_t slot = token_slot(i, tables, seq_ids, positions, lens, S, MB, B, NB);
  if (slots_out && h == 0 && c == 0) slots_out[i] = slot;
  if (slot < 0) return;
  const int64_t blk = slot / B;
  const int off = (int)(slot - blk * B);
  const int64_t dst = ((blk * Hkv + h) * B + off) * chunks + c;
  if (!PA_IN_BOUNDS(kBsPool, dst >= 0 && dst < (int64_t)NB * B * Hkv * chunks)) return;
  k_pool[dst] = key[e];
  v_pool[dst] = value[e];
}

// One thread moves one 16-byte chunk (8 fp16) of one token's row for one head,
// for K and for V. Grid covers T * Hkv * (D / 8) chunks.
__global__ __launch_bounds__(256) void write_kv_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ k_pool,
    uint4* __restrict__ v_pool, const int64_t* __restrict__ slots, int64_t total, int Hkv,
    int chunks, int B, int64_t n_slots) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const int c = (int)(e % chunks);
  const int64_t ih = e / chunks;           // token * Hkv + head
  const int h = (int)(ih % Hkv);
  const int64_t i = ih / Hkv;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= n_slots) return;
  const int64_t blk = slot / B;
  const int off = (int)(slot - blk * B);
  const int64_t dst = ((blk * Hkv + h) * B + off) * chunks + c;
  if (!PA_IN_BOUNDS(kBsPool, dst >= 0 && dst < n_slots * Hkv * chunks)) return;
  k_pool[dst] = key[e];
  v_pool[dst] = value[e];
}

// Grid: (segments, n pairs). Each workgroup copies one contiguous segment of
// a block from the source pools to the destination pools (the same pools for
// copy-on-write; a device pool and a pinned host pool for swapping). A block
// is Hkv * B * D fp16 = `chunks` 16-byte chunks; consecutive threads move
// consecutive chunks, so every wave reads and writes 1 KiB contiguous. (A
// variant issuing four chunks' loads per thread before the stores measured
// 6 % slower device to device and moved 1.37x the bytes.)
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* __restrict__ k_dst, uint4* __restrict__ v_dst, const uint4* __restrict__ k_src,
    const uint4* __restrict__ v_src, const int32_t* __restrict__ pairs, int64_t chunks,
    int seg_chunks, int NB_src, int NB_dst) {
  const int p = blockIdx.y;
  const int src = pairs[2 * p];
  const int dst = pairs[2 * p + 1];
  if (src < 0 || src >= NB_src || dst < 0 || dst >= NB_dst) return;
  const int64_t lo = (int64_t)blockIdx.x * seg_chunks;
  int64_t hi = lo + seg_chunks;
  if (hi > chunks) hi = chunks;
  const uint4* ks = k_src + (int64_t)src * chunks;
  const uint4* vs = v_src + (int64_t)src * chunks;
  uint4* kd = k_dst + (int64_t)dst * chunks;
  uint4* vd = v_dst + (int64_t)dst * chunks;
  if (!PA_IN_BOUNDS(kBsPair, lo >= 0 && hi <= chunks)) return;
  for (int64_t x = lo + threadIdx.x; x < hi; x += blockDim.x) {
    const uint4 a = ks[x];
    const uint4 b = vs[x];
    kd[x] = a;
    vd[x] = b;
  }
}

}  // namespace

PA_BOUNDS_COLLECTOR(bounds_take_cache_ops)

hipError_t launch_slot_mapping(int64_t* slots, const int32_t* tables, const int32_t* seq_ids,
                               const int32_t* positions, const int32_t* lens, int T, int S,
                               int MB, int B, int NB, hipStream_t stream) {
  const int threads = 256;
  const int grid = (T + threads - 1) / threads;
  slot_mapping_kernel<<<grid, threads, 0, stream>>>(slots, tables, seq_ids, positions, lens, T,
                                                    S, MB, B, NB);
  return hipGetLastError();
}

hipError_t launch_append_kv(int64_t* slots, const void* key, const void* value, void* k_pool,
                            void* v_pool, const int32_t* tables, const int32_t* seq_ids,
                            const int32_t* positions, const int32_t* lens, int T, int S, int MB,
                            int Hkv, int D, int B, int NB, hipStream_t stream) {
  const int chunks = D / 8;
  const int64_t total = (int64_t)T * Hkv * chunks;
  const int threads = 256;
  const int64_t grid = (total + threads - 1) / threads;
  append_kv_kernel<<<(unsigned)grid, threads, 0, stream>>>(
      slots, static_cast<const uint4*>(key), static_cast<const uint4*>(value),
      static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), tables, seq_ids, positions, lens,
      total, Hkv, chunks, S, MB, B, NB);
  return hipGetLastError();
}

hipError_t launch_write_kv(const void* key, const void* value, void* k_pool, void* v_pool,
                           const int64_t* slots, int T, int Hkv, int D, int B, int NB,
                           hipStream_t stream) {
  const int chunks = D / 8;
  const int64_t total = (int64_t)T * Hkv * chunks;
  const int threads = 256;
  const int64_t grid = (total + threads - 1) / threads;
  write_kv_kernel<<<(unsigned)grid, threads, 0, stream>>>(
      static_cast<const uint4*>(key), static_cast<const uint4*>(value),
      static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), slots, total, Hkv, chunks, B,
      (int64_t)NB * B);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_dst, void* v_dst, const void* k_src, const void* v_src,
                              const int32_t* pairs, int n, int Hkv, int D, int B, int NB_src,
                              int NB_dst, hipStream_t stream) {
  const int64_t chunks = (int64_t)Hkv * B * D / 8;
  const int seg = 2048;                          // 32 KiB of each pool per workgroup
  const int64_t segs = (chunks + seg - 1) / seg;
  dim3 grid((unsigned)segs, (unsigned)n);
  copy_blocks_kernel<<<grid, 256, 0, stream>>>(
      static_cast<uint4*>(k_dst), static_cast<uint4*>(v_dst), static_cast<const uint4*>(k_src),
      static_cast<const uint4*>(v_src), pairs, chunks, seg, NB_src, NB_dst);
  return hipGetLastError();
}

}  // namespace pa
