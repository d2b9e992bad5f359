// pa_decode_static: paged decode with the cross-partition partials in a fixed
// device array of the library instead of a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation). The kernels are pa_decode's.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends. In host
// code its name is only a stand-in for the symbol, so the device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept; kernels receive that address. Nothing in the array needs
// to start at zero: the partition kernel writes every partial and piece count
// that the reduce kernel reads in the same call.
#include <mutex>

#include "decode_call.h"
#include "pa_error.h"

namespace {

// 32 MiB per device: the partials of, e.g., 128 sequences x 32 query heads x
// 15 partitions (up to 15,360 tokens at the default 1,024-token partition).
constexpr size_t kScratchBytes = (size_t)32 << 20;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// Address of the current device's copy of the array.
pa_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return pa::fail(PA_ERR_HIP, "pa_decode_static: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode_static: device %d beyond the %d supported", dev,
                    kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pa::fail(PA_ERR_HIP, "pa_decode_static: hipGetSymbolAddress: %s",
                      hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return pa::ok();
}

}  // namespace

extern "C" {

size_t pa_decode_static_scratch_bytes(void) { return kScratchBytes; }

pa_status pa_decode_static(void* out, const void* query, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens, int S,
                           int Hq, int Hkv, int D, int B, int NB, int MB, int max_context_len,
                           float scale, int partition_size, hipStream_t stream) {
  pa::DecodeCall call;
  const pa_status st = pa::decode_prepare("pa_decode_static", out, query, k_pool, v_pool,
                                          block_tables, context_lens, S, Hq, Hkv, D, B, NB, MB,
                                          max_context_len, scale, partition_size, &call);
  if (st != PA_OK || call.a.S == 0) return st;
  void* partials = nullptr;
  if (call.partials_bytes > 0) {
    if (call.partials_bytes > kScratchBytes)
      return pa::fail(PA_ERR_WORKSPACE,
                      "pa_decode_static: the partials need %zu bytes, more than the %zu bytes of "
                      "the static scratch (use pa_decode with a workspace, or larger partitions)",
                      call.partials_bytes, kScratchBytes);
    const pa_status sp = scratch_of_current_device(&partials);
    if (sp != PA_OK) return sp;
  }
  return pa::decode_enqueue("pa_decode_static", call, partials, stream);
}

}  // extern "C"
