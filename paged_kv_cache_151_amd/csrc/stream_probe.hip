// Read-bandwidth probe: one linear pass over a device buffer. Not part of the
// attention path; the benchmark times it on the same GPU, in the same run, as
// the practical read ceiling that decode's reads are compared with. Each lane
// keeps 8 independent 16-byte loads in flight, with the non-temporal and sc1
// cache-policy bits: of the forms measured on MI355X (1 to 8 loads in flight;
// no hint, nt, sc0, sc1 and their pairs; 2k to 16k workgroups) this one read
// fastest, 7.05 TB/s over 3.5 GB.
#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kInFlight = 8;
constexpr int kPolicy = 2 | 16;           // non-temporal + sc1
constexpr int64_t kWindow = 1 << 26;      // 16-byte words per buffer resource (1 GiB)

__device__ __forceinline__ u32x4 load16(const unsigned char* base, int64_t e) {
  // one buffer resource per 1 GiB window keeps the byte offset in 32 bits
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(base + ((e / kWindow) << 30)), 0, 0x7fffffff, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, (unsigned)((e % kWindow) * 16), 0, kPolicy);
}

// Each thread folds its words into one value and stores it only if it equals
// a constant, so the loads cannot be dropped and nothing is written in practice.
__global__ __launch_bounds__(256) void stream_read_kernel(const unsigned char* __restrict__ p,
                                                          int64_t n16, unsigned* __restrict__ sink) {
  unsigned x = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = load16(p, i + k * stride);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = load16(p, i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, void* sink, int workgroups,
                              hipStream_t stream) {
  stream_read_kernel<<<workgroups, 256, 0, stream>>>(static_cast<const unsigned char*>(buf),
                                                      (int64_t)(bytes / 16),
                                                      static_cast<unsigned*>(sink));
  return hipGetLastError();
}

}  // namespace pa
