// Streaming-read reference: the bandwidth a plain read of a byte range
// reaches on this GPU, with the same 16-byte non-temporal loads the decode
// kernels use for the cached rows.  A decode step's cost is the read of its
// kept rows (H2O review page, main findings: the cache bounds throughput), so
// this is the ceiling its achieved bandwidth is compared with.
#include "common.hpp"

namespace kve {
namespace {

constexpr int kNT = 256;
constexpr int kInFlight = 4;                    // 16-byte loads per thread per round
constexpr size_t kBlockBytes = (size_t)kNT * 16 * kInFlight * 2;   // 32 KiB per workgroup

__device__ inline uint4 ld_stream(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroup b reads bytes [b * kBlockBytes, min((b + 1) * kBlockBytes, n16 * 16))
// in rounds of kInFlight loads per thread; the XOR of everything it read is
// stored only if it equals `magic` (so the loads cannot be dropped and the
// kernel writes nothing in practice).
__global__ __launch_bounds__(kNT) void stream_read_kernel(const uint4* src, size_t n16, uint32_t magic,
                                                          uint32_t* sink) {
  const size_t per = kBlockBytes / 16;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = min(b0 + per, n16);
  uint32_t acc = 0;
  for (size_t i0 = b0 + threadIdx.x; i0 < b1; i0 += (size_t)kNT * kInFlight) {
    uint4 v[kInFlight];
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) {
      const size_t i = i0 + (size_t)j * kNT;
      v[j] = i < b1 ? ld_stream(src + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == magic) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  if (!src || !sink || bytes < 16 || bytes % 16 || (uintptr_t)src % 16) return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const size_t blocks = (bytes + kBlockBytes - 1) / kBlockBytes;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kNT), 0, st, (const uint4*)src, n16,
                     0x9e3779b9u, sink);
  return hipGetLastError();
}

}  // namespace kve
