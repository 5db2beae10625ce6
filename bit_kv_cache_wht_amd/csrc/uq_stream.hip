// A plain streaming read of device memory: the bandwidth reference against which
// the decode kernel's HBM rate is read.  Every 16-byte word is loaded once,
// coalesced, eight nontemporal loads in flight per lane (the fastest plain read
// measured on MI355X: ~7.0 TB/s, against ~6.3 TB/s with ordinary loads); the XOR
// of all 32-bit words leaves the kernel through one atomic per wave, so no load
// can be dropped and the result can be checked.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "uq_device.h"
#include "uq_internal.h"

namespace uq {
namespace {

constexpr int kSrThreads = 256;
constexpr int kSrUnroll = 8;                       // 256 lanes x 8 x 16 B = 32 KiB per block pass
constexpr int kSrBlocksPerCu = 8;

__global__ __launch_bounds__(kSrThreads) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  constexpr int64_t kChunk = (int64_t)kSrThreads * kSrUnroll;
  const int64_t nchunks = n16 / kChunk;
  uint32_t acc = 0;
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const uint4* p = src + c * kChunk + threadIdx.x;        // < (c + 1) * kChunk <= n16
    uint4 v[kSrUnroll];
#pragma unroll
    for (int u = 0; u < kSrUnroll; ++u) v[u] = load16_stream(p + u * kSrThreads);
#pragma unroll
    for (int u = 0; u < kSrUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int64_t i = nchunks * kChunk + (int64_t)blockIdx.x * kSrThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kSrThreads) {
    const uint4 v = load16_stream(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & 63) == 0 && acc != 0u) atomicXor(sink, acc);
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    cus = (hipGetDevice(&dev) == hipSuccess &&
           hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
  }
  return cus;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t want = (n16 + kSrThreads - 1) / kSrThreads;
  const unsigned blocks = (unsigned)std::min<int64_t>(want, (int64_t)device_cus() * kSrBlocksPerCu);
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kSrThreads), 0, s, static_cast<const uint4*>(src), n16,
                     sink);
  return hipGetLastError();
}

}  // namespace uq
