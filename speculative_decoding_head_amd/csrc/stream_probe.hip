// Read-only HBM streaming probe, for measurement only (not part of the C ABI of the cycle):
// the ceiling of the access pattern the tiled LM-head kernels use.  Each wave reads a
// contiguous range of 1 KiB blocks, 16 bytes per lane per block, with the same raw
// non-temporal buffer loads, DEPTH blocks in flight per lane; the loaded words are folded into one XOR per lane and stored only if the fold hits a
// value that a sink check makes practically impossible, so every load is kept and nothing
// is written.  Built into its own library (libmtp_probe.so) that only the benchmark loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lmhead_common.hpp"

namespace {

using namespace mtp::lm;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

template <int DEPTH>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const void* buf, uint32_t nblocks, uint32_t magic,
                                                               uint32_t* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t gw = (uint64_t)blockIdx.x * kWaves + wave, nw = (uint64_t)gridDim.x * kWaves;
  const uint32_t b0 = (uint32_t)(gw * nblocks / nw), b1 = (uint32_t)((gw + 1) * nblocks / nw);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(buf, nblocks * 1024u);
  const uint32_t lo = (uint32_t)lane * 16u;
  auto load = [&](uint4 (&v)[DEPTH], uint32_t b) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const uint32_t blk = b + (uint32_t)u;
      // blocks past this wave's range read out of bounds (zeros): no branch around the load
      v[u] = bload16_stream(r, (blk < b1 ? blk * 1024u : kOOB) + lo);
    }
  };
  uint32_t acc = 0;
  // DEPTH loads in flight per lane, then their fold; other waves on the SIMD cover the wait
  for (uint32_t blk = b0; blk < b1; blk += DEPTH) {
    uint4 v[DEPTH];
    load(v, blk);
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == magic) sink[gw * 64 + lane] = acc;
}

}  // namespace

extern "C" {

// Read nbytes (a multiple of 1024, below 2 GiB) of device memory at buf once with `grid`
// blocks of 512 threads and DEPTH 8, 16 or 32; sink: device uint32 [grid * 512] (written
// only in the practically impossible case that a lane's fold equals magic).  0 on success,
// -1 for bad arguments, -7 for a launch error.
int mtp_probe_stream_read(const void* buf, size_t nbytes, int grid, int depth, uint32_t magic, uint32_t* sink,
                          void* stream) {
  if (!buf || !sink || nbytes == 0 || nbytes % 1024 != 0 || nbytes >= ((size_t)1 << 31) || grid < 1 ||
      grid > 65535)
    return -1;
  const uint32_t nblocks = (uint32_t)(nbytes / 1024);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (depth) {
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(kThreads), 0, s, buf, nblocks, magic, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(grid), dim3(kThreads), 0, s, buf, nblocks, magic, sink); break;
    case 32: hipLaunchKernelGGL(stream_read_kernel<32>, dim3(grid), dim3(kThreads), 0, s, buf, nblocks, magic, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
