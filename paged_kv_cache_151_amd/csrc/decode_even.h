// The equal-work split of a decode batch, shared by the vector and the
// matrix-core decode kernels (not installed).
//
// [L] "Paged Attention: OS-Inspired Memory Management for KV Caches",
//     "How PagedAttention works", step 4: attention walks each sequence's
//     blocks; how that walk is cut into pieces and spread over the GPU is this
//     library's own choice (the result is the same softmax).
//
// The 16-token units of every (KV head, sequence) pair are taken in the order
// (KV head, sequence, position) and cut into runs of q consecutive units, one
// run per workgroup; q is the total over the grid, at least a.P / 16. A
// workgroup walks its run pair by pair, each pair's part being one piece for
// the reduce kernel. Every workgroup of the grid is resident at once (the
// same number on every compute unit), so every run starts at the launch and
// they all end together: no workgroup starts late behind a long one, which
// cost grouped heads about a tenth of a launch, and one or two heads per KV
// head about 1.5 %, in the per-partition grid on the chat lengths. Fewer,
// longer runs cut fewer sequences into pieces: two workgroups per compute
// unit measured best where the kernel leaves the choice (one query head per
// KV head, and the matrix-core kernel). Workgroup b runs on XCD b % 8 and
// takes run (b % 8) * (grid / 8) + b / 8, so each XCD walks one contiguous
// eighth of the order.
#pragma once

#include <atomic>

#include "pa_debug.h"
#include "pa_internal.h"

namespace pa {
namespace {   // each translation unit keeps its own copy (and its own bounds counters)

// Workgroups of `kernel` (`threads` threads each) the current device holds at
// once, rounded down to a multiple of 8; measured once per device and kernel.
template <class K>
int resident_workgroups(K kernel, int threads) {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) !=
          hipSuccess)
    return 0;
  int n = per_cu * cus / 8 * 8;
  if (n < 8) n = 8;
  if (dev >= 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Grid of an evenly split launch: per_cu workgroups per compute unit, at most
// the resident ones, a multiple of 8, and no more runs than the minimum run
// length leaves units for. 0 when a device query fails.
template <class K>
int64_t even_split_grid(const DecodeArgs& a, K kernel, int threads, int per_cu) {
  const int resident = resident_workgroups(kernel, threads);
  if (resident <= 0) return 0;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int64_t want = (int64_t)per_cu * cus / 8 * 8;
  if (want < 8) want = 8;
  if (want > resident) want = resident;
  const int64_t most = ((int64_t)a.S * a.Hkv * (a.Pmax - 1) + 7) / 8 * 8;
  return most < want ? most : want;
}

// Clamped context length of sequence s: within the table and the launch.
__device__ __forceinline__ int even_clamped_len(const DecodeArgs& a, int s, int B, int cap) {
  int L = PA_IN_BOUNDS(kBsLength, s >= 0 && s < a.S) ? a.lens[s] : 0;
  L = L < 0 ? 0 : L;
  L = L > a.MB * B ? a.MB * B : L;
  return L > cap ? cap : L;
}

// The workgroup's run. piece(s, g, L, tok0, len, nparts, p) attends tokens
// [tok0, tok0 + len) of sequence s (clamped length L) and KV head g, piece p
// of nparts; empty(s) zeroes the output of an empty sequence. NTH threads.
template <int NTH, class Piece, class Empty>
__device__ __forceinline__ void even_split_walk(const DecodeArgs& a, int B, Piece&& piece,
                                                Empty&& empty) {
  constexpr int U = kDecodeUnit;
  const int cap = (a.Pmax - 1) * a.P;   // the launch's bound on every length
  const int lane = threadIdx.x & 63;
  const int nwg = gridDim.x;            // a multiple of 8
  const int w = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;

  // every length once, into registers (lane l holds sequences 64c + l), so
  // that the sum below, the empty sequences and the search for the run's
  // first pair need one round trip to memory between them
  constexpr int kChunks = kEvenSplitMaxSeqs / 64;
  int lc[kChunks];
  int acc = 0;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    lc[c] = 64 * c + lane < a.S ? even_clamped_len(a, 64 * c + lane, B, cap) : 0;
    acc += (lc[c] + U - 1) / U;
  }
  // empty sequences (workgroup b serves sequences b, b + grid, ...): zero
  // output and no pieces
  for (int s = blockIdx.x; s < a.S; s += nwg) {
    int lv = lc[0];
#pragma unroll
    for (int c = 1; c < kChunks; ++c) lv = (s >> 6) == c ? lc[c] : lv;
    if (__builtin_amdgcn_readlane(lv, s & 63) == 0) {
      empty(s);
      for (int g = threadIdx.x; g < a.Hkv; g += NTH)
        if (PA_IN_BOUNDS(kBsPartial, s * a.Hkv + g < a.S * a.Hkv)) a.part_np[s * a.Hkv + g] = 0;
    }
  }

  // N = units of one KV head over the batch; the run length q
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d);
  const int N = __builtin_amdgcn_readfirstlane(acc);
  const int total = N * a.Hkv;
  const int qmin = a.P / U;
  const int qe = (total + nwg - 1) / nwg;
  const int q = __builtin_amdgcn_readfirstlane(qe > qmin ? qe : qmin);
  const int begin = w * q;
  if (begin >= total) return;
  const int end = begin + q < total ? begin + q : total;

  // the pair of the run's first unit: KV head g, then the first sequence
  // whose running unit count passes the offset r inside that head
  int g = __builtin_amdgcn_readfirstlane(begin / N);
  const int r = begin - g * N;
  int s = 0, cs = 0, ns = 0, Ls = 0;
  bool found = false;
  int base = 0;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    if (!found && 64 * c < a.S) {
      const int n = (lc[c] + U - 1) / U;
      int incl = n;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d);
        incl += lane >= d ? t : 0;
      }
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(base + incl > r);
      if (hit) {
        const int f = __builtin_ctzll(hit);
        s = 64 * c + f;
        ns = __builtin_amdgcn_readlane(n, f);
        Ls = __builtin_amdgcn_readlane(lc[c], f);
        cs = base + __builtin_amdgcn_readlane(incl, f) - ns;
        found = true;
      } else {
        base += __builtin_amdgcn_readlane(incl, 63);
      }
    }
  }
  s = __builtin_amdgcn_readfirstlane(s);
  ns = __builtin_amdgcn_readfirstlane(ns);
  Ls = __builtin_amdgcn_readfirstlane(Ls);
  cs = __builtin_amdgcn_readfirstlane(cs);
  if (ns == 0) return;   // unreachable: r < N

  int pos = begin;
  for (bool first = true;; first = false) {
    const int pair0 = g * N + cs;                  // order position of the pair's unit 0
    const int j0 = pos - pair0;
    const int j1 = end - pair0 < ns ? end - pair0 : ns;
    const int p = w - pair0 / q;                   // runs are numbered by position / q
    const int nparts = (pair0 + ns - 1) / q - pair0 / q + 1;
    if (!first) __syncthreads();                   // the last piece's merge has read LDS
    const int tok0 = j0 * U;
    const int tok1 = j1 * U < Ls ? j1 * U : Ls;
    piece(s, g, Ls, tok0, tok1 - tok0, nparts, p);
    if (j1 == ns && threadIdx.x == 0 &&
        PA_IN_BOUNDS(kBsPartial, s * a.Hkv + g < a.S * a.Hkv && nparts <= a.Pmax))
      a.part_np[s * a.Hkv + g] = nparts;
    pos = pair0 + j1;
    if (pos >= end) break;
    // the next pair in the order with at least one unit
    do {
      cs += ns;
      if (++s == a.S) {
        s = 0;
        cs = 0;
        if (++g == a.Hkv) return;   // unreachable: pos < end <= total
      }
      // a load after the kernel's stores: the compiler cannot see it uniform
      Ls = __builtin_amdgcn_readfirstlane(even_clamped_len(a, s, B, cap));
      ns = (Ls + U - 1) / U;
    } while (ns == 0);
  }
}

}  // namespace
}  // namespace pa
