// C ABI of the paged KV-cache library: host-side validation, launch sizing,
// error reporting. Declared in include/pa.h.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>

#include "pa.h"
#include "pa_error.h"
#include "decode_call.h"
#include "pa_internal.h"
#include "prefill_internal.h"
#include "pa_debug.h"

namespace pa {
hipError_t launch_stream_read(const void* buf, size_t bytes, void* sink, int workgroups,
                              hipStream_t stream);
}  // namespace pa

namespace pa {

namespace {
thread_local char g_err[512] = "";
}  // namespace

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

pa_status ok() {
  g_err[0] = '\0';
  return PA_OK;
}

const char* last_error() { return g_err; }

}  // namespace pa

namespace {

using pa::fail;
using pa::ok;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

pa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// A dispatch packet holds the grid as a 32-bit count of work-items per
// dimension: `workgroups` of `threads` each must stay within it.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFLL;
bool dispatch_fits(int64_t workgroups, int threads) {
  return workgroups >= 0 && workgroups <= kMaxWorkItems / threads;
}

// 16-byte chunks in one block of one pool (Hkv * B * D fp16), or -1 when that
// exceeds what one copy launch covers: the copy kernel gives each workgroup of
// 256 threads a segment of 2048 chunks, so at most 2^24 - 1 segments (just
// under 512 GiB per block).
int64_t block_chunks(int Hkv, int B, int D) {
  const int64_t max_chunks = (kMaxWorkItems / 256) * 2048;
  const int64_t hb = (int64_t)Hkv * B;
  const int64_t per = D / 8;
  if (hb > max_chunks / per) return -1;
  return hb * per;
}

}  // namespace

namespace pa {

pa_status decode_prepare(const char* fn, void* out, const void* query, const void* k_pool,
                         const void* v_pool, const int32_t* block_tables,
                         const int32_t* context_lens, int S, int Hq, int Hkv, int D, int B, int NB,
                         int MB, int max_context_len, float scale, int partition_size,
                         DecodeCall* call) {
  call->a.S = 0;
  if (S < 0) return fail(PA_ERR_SHAPE, "%s: S=%d must be >= 0", fn, S);
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0 || MB <= 0)
    return fail(PA_ERR_SHAPE, "%s: Hq=%d Hkv=%d D=%d B=%d NB=%d MB=%d must be > 0", fn, Hq, Hkv,
                D, B, NB, MB);
  if (Hq % Hkv) return fail(PA_ERR_SHAPE, "%s: Hq=%d not a multiple of Hkv=%d", fn, Hq, Hkv);
  if ((int64_t)MB * B >= ((int64_t)1 << 31))
    return fail(PA_ERR_SHAPE, "%s: MB*B=%lld exceeds int32", fn, (long long)MB * B);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)MB * B)
    return fail(PA_ERR_SHAPE, "%s: max_context_len=%d outside [0, MB*B=%lld]", fn,
                max_context_len, (long long)MB * B);
  if (partition_size < 0 || (partition_size > 0 && partition_size % kDecodeUnit))
    return fail(PA_ERR_SHAPE, "%s: partition_size=%d must be 0 or a multiple of %d", fn,
                partition_size, kDecodeUnit);
  const int G = Hq / Hkv;
  if (D != kHeadDim) return fail(PA_ERR_UNSUPPORTED, "%s: D=%d (supported: 128)", fn, D);
  if (B != 8 && B % kDecodeUnit)
    return fail(PA_ERR_UNSUPPORTED, "%s: B=%d (supported: 8 and multiples of %d)", fn, B,
                kDecodeUnit);
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_ERR_UNSUPPORTED, "%s: Hq/Hkv=%d (supported: 1, 2, 4, 8)", fn, G);
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "%s: scale is not finite", fn);
  const int P = pa_decode_partition_size(S, Hq, Hkv, B, max_context_len, partition_size);
  const int parts = max_context_len > 0 ? ceil_div(max_context_len, P) : 1;
  const bool even = decode_even_split(S, Hq, Hkv, P, parts);
  const int Pmax = even ? parts + 1 : parts;   // an even split adds at most one piece
  if (Pmax > kMaxPartitions)
    return fail(PA_ERR_SHAPE, "%s: %d partitions exceed %d", fn, Pmax, kMaxPartitions);
  // partition kernel: one workgroup per (partition, sequence, KV head) of
  // max(waves for the group size, heads / heads per wave) waves; reduce
  // kernel: one wave per (sequence, query head)
  const int hpw = G < kDecodeHeadsPerWave ? G : kDecodeHeadsPerWave;
  const int waves = decode_waves(G) > G / hpw ? decode_waves(G) : G / hpw;
  const int64_t wgs = (int64_t)parts * S * Hkv;
  if (!dispatch_fits(wgs, waves * 64) || !dispatch_fits((int64_t)S * Hq, 64))
    return fail(PA_ERR_SHAPE, "%s: launch too large (S=%d Hq=%d, %lld workgroups)", fn, S, Hq,
                (long long)wgs);
  if (S == 0) return ok();
  if (!out || !query || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PA_ERR_NULL, "%s: null pointer argument", fn);
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(PA_ERR_ALIGN, "%s: out/query/pools must be 16-byte aligned", fn);
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_ALIGN, "%s: block_tables/context_lens misaligned", fn);

  DecodeArgs& a = call->a;
  a.out = static_cast<_Float16*>(out);
  a.q = static_cast<const _Float16*>(query);
  a.k_pool = static_cast<const _Float16*>(k_pool);
  a.v_pool = static_cast<const _Float16*>(v_pool);
  a.tables = block_tables;
  a.lens = context_lens;
  a.part_acc = nullptr;
  a.part_ml = nullptr;
  a.part_np = nullptr;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.NB = NB;
  a.MB = MB;
  a.B = B;
  a.P = P;
  a.Pmax = Pmax;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  call->G = G;
  call->even = even;
  call->partials_bytes = pa_decode_workspace_bytes(S, Hq, Hkv, D, B, max_context_len, P);
  if (Pmax > 1 && call->partials_bytes == 0)
    return fail(PA_ERR_SHAPE, "%s: partials of %d partitions do not fit in size_t", fn, Pmax);
  return ok();
}

pa_status decode_enqueue(const char* fn, DecodeCall& call, void* partials, hipStream_t stream) {
  DecodeArgs& a = call.a;
  if (call.partials_bytes > 0) {
    float* ws = static_cast<float*>(partials);
    a.part_acc = ws;
    a.part_ml = ws + (size_t)a.S * a.Hq * a.Pmax * kHeadDim;
    if (call.even) a.part_np = reinterpret_cast<int32_t*>(a.part_ml + (size_t)a.S * a.Hq * a.Pmax * 2);
  }
  const hipError_t e = launch_decode(a, a.B, call.G, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace pa

extern "C" {

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_EXHAUSTED: return "PA_ERR_EXHAUSTED";
    case PA_ERR_STATE: return "PA_ERR_STATE";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error(void) { return pa::last_error(); }

int pa_version(void) { return 200; }

const char* pa_debug_bounds_site(int site) {
  static const char* const names[pa::kBsSites] = {
      "length", "table", "query", "pool", "out", "partial", "slot", "pair"};
  return site >= 0 && site < pa::kBsSites ? names[site] : nullptr;
}

int pa_debug_bounds_selftest(void) {
#if PA_DEBUG_BOUNDS
  if (pa::bounds_take_cache_ops_selftest() != hipSuccess ||
      pa::bounds_take_decode_selftest() != hipSuccess ||
      pa::bounds_take_decode_mfma_selftest() != hipSuccess ||
      pa::bounds_take_prefill_selftest() != hipSuccess)
    return -2;
  return 4;
#else
  return -1;
#endif
}

int pa_debug_bounds_violations(unsigned int* counts, int n) {
#if PA_DEBUG_BOUNDS
  if (hipDeviceSynchronize() != hipSuccess) return -2;
  unsigned int acc[pa::kBsSites] = {};
  if (pa::bounds_take_cache_ops(acc) != hipSuccess || pa::bounds_take_decode(acc) != hipSuccess ||
      pa::bounds_take_decode_mfma(acc) != hipSuccess || pa::bounds_take_prefill(acc) != hipSuccess)
    return -2;
  for (int i = 0; counts && i < n && i < pa::kBsSites; ++i) counts[i] = acc[i];
  return pa::kBsSites;
#else
  (void)counts;
  (void)n;
  return -1;
#endif
}

pa_status pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* seq_ids, const int32_t* positions,
                          const int32_t* context_lens, int T, int S, int MB, int B, int NB,
                          hipStream_t stream) {
  if (T < 0 || S < 0) return fail(PA_ERR_SHAPE, "pa_slot_mapping: T=%d S=%d must be >= 0", T, S);
  if (B <= 0 || NB <= 0 || MB <= 0)
    return fail(PA_ERR_SHAPE, "pa_slot_mapping: B=%d NB=%d MB=%d must be > 0", B, NB, MB);
  if (!seq_ids && T > S)
    return fail(PA_ERR_SHAPE, "pa_slot_mapping: T=%d > S=%d needs seq_ids", T, S);
  if ((int64_t)NB * B > ((int64_t)1 << 62))
    return fail(PA_ERR_SHAPE, "pa_slot_mapping: pool too large");
  if (T == 0) return ok();
  if (!slot_mapping || !block_tables)
    return fail(PA_ERR_NULL, "pa_slot_mapping: slot_mapping and block_tables are required");
  if (!positions && !context_lens)
    return fail(PA_ERR_NULL, "pa_slot_mapping: need positions or context_lens");
  if (!aligned(slot_mapping, 8) || !aligned(block_tables, 4) || !aligned(seq_ids, 4) ||
      !aligned(positions, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_ALIGN, "pa_slot_mapping: misaligned index buffer");
  return hip_status(pa::launch_slot_mapping(slot_mapping, block_tables, seq_ids, positions,
                                            context_lens, T, S, MB, B, NB, stream),
                    "pa_slot_mapping launch");
}

pa_status pa_write_kv(const void* key, const void* value, void* k_pool, void* v_pool,
                      const int64_t* slot_mapping, int T, int Hkv, int D, int B, int NB,
                      hipStream_t stream) {
  if (T < 0) return fail(PA_ERR_SHAPE, "pa_write_kv: T=%d must be >= 0", T);
  if (Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0)
    return fail(PA_ERR_SHAPE, "pa_write_kv: Hkv=%d D=%d B=%d NB=%d must be > 0", Hkv, D, B, NB);
  if (D % 8) return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: D=%d must be a multiple of 8", D);
  // one work-item per 16-byte chunk of every token's row: T * Hkv * D / 8
  if (T > 0 && (int64_t)Hkv * (D / 8) > (kMaxWorkItems - 255) / T)
    return fail(PA_ERR_SHAPE, "pa_write_kv: T=%d tokens of Hkv=%d x D=%d exceed one launch", T,
                Hkv, D);
  if (T == 0) return ok();
  if (!key || !value || !k_pool || !v_pool || !slot_mapping)
    return fail(PA_ERR_NULL, "pa_write_kv: null pointer argument");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(PA_ERR_ALIGN, "pa_write_kv: key/value/pools must be 16-byte aligned");
  if (!aligned(slot_mapping, 8)) return fail(PA_ERR_ALIGN, "pa_write_kv: slot_mapping misaligned");
  return hip_status(pa::launch_write_kv(key, value, k_pool, v_pool, slot_mapping, T, Hkv, D, B,
                                        NB, stream),
                    "pa_write_kv launch");
}

pa_status pa_append_kv(int64_t* slot_mapping, const void* key, const void* value, void* k_pool,
                       void* v_pool, const int32_t* block_tables, const int32_t* seq_ids,
                       const int32_t* positions, const int32_t* context_lens, int T, int S,
                       int MB, int Hkv, int D, int B, int NB, hipStream_t stream) {
  if (T < 0 || S < 0) return fail(PA_ERR_SHAPE, "pa_append_kv: T=%d S=%d must be >= 0", T, S);
  if (Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0 || MB <= 0)
    return fail(PA_ERR_SHAPE, "pa_append_kv: Hkv=%d D=%d B=%d NB=%d MB=%d must be > 0", Hkv, D, B,
                NB, MB);
  if (D % 8) return fail(PA_ERR_UNSUPPORTED, "pa_append_kv: D=%d must be a multiple of 8", D);
  if (!seq_ids && T > S)
    return fail(PA_ERR_SHAPE, "pa_append_kv: T=%d > S=%d needs seq_ids", T, S);
  if ((int64_t)NB * B > ((int64_t)1 << 62))
    return fail(PA_ERR_SHAPE, "pa_append_kv: pool too large");
  if (T > 0 && (int64_t)Hkv * (D / 8) > (kMaxWorkItems - 255) / T)
    return fail(PA_ERR_SHAPE, "pa_append_kv: T=%d tokens of Hkv=%d x D=%d exceed one launch", T,
                Hkv, D);
  if (T == 0) return ok();
  if (!key || !value || !k_pool || !v_pool || !block_tables)
    return fail(PA_ERR_NULL, "pa_append_kv: null pointer argument");
  if (!positions && !context_lens)
    return fail(PA_ERR_NULL, "pa_append_kv: need positions or context_lens");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(PA_ERR_ALIGN, "pa_append_kv: key/value/pools must be 16-byte aligned");
  if (!aligned(slot_mapping, 8) || !aligned(block_tables, 4) || !aligned(seq_ids, 4) ||
      !aligned(positions, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_ALIGN, "pa_append_kv: misaligned index buffer");
  return hip_status(pa::launch_append_kv(slot_mapping, key, value, k_pool, v_pool, block_tables,
                                         seq_ids, positions, context_lens, T, S, MB, Hkv, D, B,
                                         NB, stream),
                    "pa_append_kv launch");
}

pa_status pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_mapping, int n,
                         int Hkv, int D, int B, int NB, hipStream_t stream) {
  if (n < 0) return fail(PA_ERR_SHAPE, "pa_copy_blocks: n=%d must be >= 0", n);
  if (Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0)
    return fail(PA_ERR_SHAPE, "pa_copy_blocks: Hkv=%d D=%d B=%d NB=%d must be > 0", Hkv, D, B,
                NB);
  if (D % 8) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: D=%d must be a multiple of 8", D);
  if (block_chunks(Hkv, B, D) < 0)
    return fail(PA_ERR_SHAPE, "pa_copy_blocks: block of Hkv=%d x B=%d x D=%d too large", Hkv, B, D);
  if (n == 0) return ok();
  if (!k_pool || !v_pool || !block_mapping)
    return fail(PA_ERR_NULL, "pa_copy_blocks: null pointer argument");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(PA_ERR_ALIGN, "pa_copy_blocks: pools must be 16-byte aligned");
  if (!aligned(block_mapping, 4)) return fail(PA_ERR_ALIGN, "pa_copy_blocks: mapping misaligned");
  // the y grid dimension carries the pair index; split very long lists
  const int kMaxY = 65535;
  for (int off = 0; off < n; off += kMaxY) {
    const int cnt = n - off < kMaxY ? n - off : kMaxY;
    hipError_t e = pa::launch_copy_blocks(k_pool, v_pool, k_pool, v_pool,
                                          block_mapping + 2 * (int64_t)off, cnt, Hkv, D, B, NB,
                                          NB, stream);
    if (e != hipSuccess) return hip_status(e, "pa_copy_blocks launch");
  }
  return ok();
}

// The address a kernel uses for `p`: p itself for device memory, the mapped
// device address for pinned host memory; NULL for anything else (pageable
// host memory is never handed to a kernel).
static void* device_view(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return const_cast<void*>(p);
  if (attr.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    return d;
  }
  return nullptr;
}

pa_status pa_swap_blocks(void* dst_k_pool, void* dst_v_pool, const void* src_k_pool,
                         const void* src_v_pool, const int32_t* block_mapping, int n, int Hkv,
                         int D, int B, int NB_dst, int NB_src, hipStream_t stream) {
  if (n < 0) return fail(PA_ERR_SHAPE, "pa_swap_blocks: n=%d must be >= 0", n);
  if (Hkv <= 0 || D <= 0 || B <= 0 || NB_dst <= 0 || NB_src <= 0)
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: Hkv=%d D=%d B=%d NB_dst=%d NB_src=%d must be > 0",
                Hkv, D, B, NB_dst, NB_src);
  if (D % 8) return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: D=%d must be a multiple of 8", D);
  if (block_chunks(Hkv, B, D) < 0)
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: block of Hkv=%d x B=%d x D=%d too large", Hkv, B, D);
  if (n == 0) return ok();
  if (!dst_k_pool || !dst_v_pool || !src_k_pool || !src_v_pool || !block_mapping)
    return fail(PA_ERR_NULL, "pa_swap_blocks: null pointer argument");
  if (!aligned(dst_k_pool, 16) || !aligned(dst_v_pool, 16) || !aligned(src_k_pool, 16) ||
      !aligned(src_v_pool, 16))
    return fail(PA_ERR_ALIGN, "pa_swap_blocks: pools must be 16-byte aligned");
  if (!aligned(block_mapping, 4)) return fail(PA_ERR_ALIGN, "pa_swap_blocks: mapping misaligned");
  void* dk = device_view(dst_k_pool);
  void* dv = device_view(dst_v_pool);
  void* sk = device_view(src_k_pool);
  void* sv = device_view(src_v_pool);
  if (!dk || !dv || !sk || !sv)
    return fail(PA_ERR_UNSUPPORTED,
                "pa_swap_blocks: every pool must be device memory or pinned host memory");
  const int32_t* map = static_cast<const int32_t*>(device_view(block_mapping));
  if (!map)
    return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: block_mapping must be device-accessible");
  const int kMaxY = 65535;
  for (int off = 0; off < n; off += kMaxY) {
    const int cnt = n - off < kMaxY ? n - off : kMaxY;
    hipError_t e = pa::launch_copy_blocks(dk, dv, sk, sv, map + 2 * (int64_t)off, cnt, Hkv, D, B,
                                          NB_src, NB_dst, stream);
    if (e != hipSuccess) return hip_status(e, "pa_swap_blocks launch");
  }
  return ok();
}

// The default decode partition keeps at least one workgroup per compute unit
// (kComputeUnits).

int pa_decode_partition_size(int S, int Hq, int Hkv, int B, int max_context_len,
                             int partition_size) {
  const int U = pa::kDecodeUnit;
  if (B <= 0 || partition_size < 0 || (partition_size > 0 && partition_size % U)) return -1;
  if (partition_size > 0) return partition_size;
  // Default: 1024 tokens (64 blocks of 16, one table chunk), halved while the
  // launch would have fewer workgroups than the MI355X has compute units
  // (256), down to 64 tokens. Splitting a sequence further costs a reduce
  // launch and more partials, which outweighs the extra parallelism once every
  // CU has a workgroup. Measured on MI355X (one call replayed in a HIP graph):
  // for the batch-128 chat workload 1024 beats 512 by 4 %; for the 32/8-head
  // shared-prefix workload one 1024-token partition per sequence (no reduce)
  // beats 512 by 20 %; for 8 sequences of at most 853 tokens x 32 heads one
  // partition takes 19.3 us against 20.6 at 256 tokens; for one sequence of
  // 4000 tokens x 32 heads 512 tokens take 17.5 us against 20.3 at 128.
  // When such a call would not split its work evenly and its partitions fill
  // at least four workgroups per compute unit, P is doubled while they still
  // fill two: fewer, longer partitions, and none at all to merge once P covers
  // every sequence. For 16 sequences of 4096 tokens x 32 heads, one partition
  // per sequence (512 workgroups, no reduce) takes 164.6 us against 168.0 at
  // 1024 tokens and 167.0 at 2048 (one process alternating the sizes).
  int P = 1024;
  const int64_t units = (int64_t)(S > 0 ? S : 1) * (Hkv > 0 ? Hkv : 1);
  const int maxL = max_context_len > 0 ? max_context_len : 1;
  while (P > 4 * U && units * ceil_div(maxL, P) < pa::kComputeUnits) P /= 2;
  const int64_t parts = ceil_div(maxL, P);
  if (!pa::decode_even_split(S, Hq, Hkv, P, parts) && units * parts >= 4 * pa::kComputeUnits) {
    while (P < maxL && P <= (1 << 29) && units * ceil_div(maxL, 2 * P) >= 2 * pa::kComputeUnits)
      P *= 2;
  }
  return P;
}

size_t pa_decode_workspace_bytes(int S, int Hq, int Hkv, int D, int B, int max_context_len,
                                 int partition_size) {
  const int P = pa_decode_partition_size(S, Hq, Hkv, B, max_context_len, partition_size);
  if (P <= 0 || S <= 0 || Hq <= 0 || D <= 0 || max_context_len <= 0) return 0;
  const int64_t parts = ceil_div(max_context_len, P);
  if (parts <= 1) return 0;
  // an even split (groups of 4 and 8 over several partitions) has one more
  // piece per sequence and a piece count per (sequence, KV head)
  const bool even = pa::decode_even_split(S, Hq, Hkv, P, parts);
  const int64_t Pmax = even ? parts + 1 : parts;
  size_t n = 0;   // S * Hq * Pmax * (D + 2) floats (+ S * Hkv int32); 0 when that overflows
  if (__builtin_mul_overflow((size_t)S, (size_t)Hq, &n) ||
      __builtin_mul_overflow(n, (size_t)Pmax, &n) ||
      __builtin_mul_overflow(n, ((size_t)D + 2) * sizeof(float), &n))
    return 0;
  if (even && __builtin_add_overflow(n, (size_t)S * Hkv * sizeof(int32_t), &n)) return 0;
  return n;
}

pa_status pa_decode(void* out, const void* query, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* context_lens, int S, int Hq,
                    int Hkv, int D, int B, int NB, int MB, int max_context_len, float scale,
                    int partition_size, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  pa::DecodeCall call;
  const pa_status st = pa::decode_prepare("pa_decode", out, query, k_pool, v_pool, block_tables,
                                          context_lens, S, Hq, Hkv, D, B, NB, MB, max_context_len,
                                          scale, partition_size, &call);
  if (st != PA_OK || call.a.S == 0) return st;
  const size_t need = call.partials_bytes;
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "pa_decode: workspace %zu bytes < %zu needed", workspace_bytes,
                  need);
    if (!aligned(workspace, 16)) return fail(PA_ERR_ALIGN, "pa_decode: workspace misaligned");
  }
  return pa::decode_enqueue("pa_decode", call, workspace, stream);
}

pa_status pa_prefill(void* out, const void* query, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start, int S, int T, int Hq, int Hkv, int D, int B,
                     int NB, int MB, int max_query_len, float scale, hipStream_t stream) {
  if (S < 0 || T < 0) return fail(PA_ERR_SHAPE, "pa_prefill: S=%d T=%d must be >= 0", S, T);
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0 || MB <= 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: Hq=%d Hkv=%d D=%d B=%d NB=%d MB=%d must be > 0", Hq,
                Hkv, D, B, NB, MB);
  if (Hq % Hkv) return fail(PA_ERR_SHAPE, "pa_prefill: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if ((int64_t)MB * B >= ((int64_t)1 << 31))
    return fail(PA_ERR_SHAPE, "pa_prefill: MB*B=%lld exceeds int32", (long long)MB * B);
  if (max_query_len < 0 || max_query_len > T)
    return fail(PA_ERR_SHAPE, "pa_prefill: max_query_len=%d outside [0, T=%d]", max_query_len, T);
  const int G = Hq / Hkv;
  if (D != pa::kHeadDim) return fail(PA_ERR_UNSUPPORTED, "pa_prefill: D=%d (supported: 128)", D);
  if (B != 8 && B % pa::kDecodeUnit)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: B=%d (supported: 8 or multiples of %d)", B,
                pa::kDecodeUnit);
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: Hq/Hkv=%d (supported: 1, 2, 4, 8)", G);
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "pa_prefill: scale is not finite");
  // workgroups of kPrefillWaves waves, padded to a multiple of 8 at launch
  const int64_t grid = pa::prefill_work_items(G, S, Hkv, max_query_len);
  if (!dispatch_fits(grid + 7, pa::kPrefillWaves * 64))
    return fail(PA_ERR_SHAPE, "pa_prefill: launch too large (%lld workgroups)", (long long)grid);
  if (S == 0 || max_query_len == 0) return ok();
  if (!out || !query || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_NULL, "pa_prefill: null pointer argument");
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(PA_ERR_ALIGN, "pa_prefill: out/query/pools must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
    return fail(PA_ERR_ALIGN, "pa_prefill: index arrays misaligned");

  pa::PrefillArgs a;
  a.out = static_cast<_Float16*>(out);
  a.q = static_cast<const _Float16*>(query);
  a.k_pool = static_cast<const _Float16*>(k_pool);
  a.v_pool = static_cast<const _Float16*>(v_pool);
  a.tables = block_tables;
  a.lens = context_lens;
  a.qstart = query_start;
  a.S = S;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.NB = NB;
  a.MB = MB;
  a.B = B;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return hip_status(pa::launch_prefill(a, B, G, max_query_len, stream), "pa_prefill launch");
}

pa_status pa_stream_read(const void* buffer, size_t bytes, void* sink, int workgroups,
                         hipStream_t stream) {
  if (workgroups <= 0 || workgroups > (1 << 20))
    return fail(PA_ERR_SHAPE, "pa_stream_read: workgroups=%d outside [1, 2^20]", workgroups);
  if (bytes % 16) return fail(PA_ERR_SHAPE, "pa_stream_read: bytes=%zu not a multiple of 16", bytes);
  if (bytes == 0) return ok();
  if (!buffer || !sink) return fail(PA_ERR_NULL, "pa_stream_read: null pointer argument");
  if (!aligned(buffer, 16) || !aligned(sink, 4))
    return fail(PA_ERR_ALIGN, "pa_stream_read: buffer must be 16-byte aligned, sink 4-byte aligned");
  return hip_status(pa::launch_stream_read(buffer, bytes, sink, workgroups, stream),
                    "pa_stream_read launch");
}

}  // extern "C"
