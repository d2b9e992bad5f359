// Read-bandwidth probe: one linear pass over a device buffer with 16-byte
// non-temporal loads. Not part of the attention path; the benchmark times it
// on the same GPU, in the same run, as the practical ceiling that decode's
// streaming reads are compared with.
#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Each thread folds its words into one value and stores it only if it equals
// a constant, so the loads cannot be dropped and nothing is written in practice.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                          unsigned* __restrict__ sink) {
  unsigned x = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, void* sink, int workgroups,
                              hipStream_t stream) {
  stream_read_kernel<<<workgroups, 256, 0, stream>>>(static_cast<const u32x4*>(buf),
                                                      (int64_t)(bytes / 16),
                                                      static_cast<unsigned*>(sink));
  return hipGetLastError();
}

}  // namespace pa
