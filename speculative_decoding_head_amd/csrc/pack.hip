// One-time repack of a row-major LM head into the tiled layouts (MTP_W_BF16_TILED,
// MTP_W_Q4A32_TILED).  Pure data movement: every output byte is a copy of one source byte
// or a zero pad past the vocabulary.  In the tiled layout one 16-row tile's K-step (bf16)
// or group quad (4-bit) is a contiguous 1 KiB block in the MFMA B-operand lane order, so
// the LM-head kernels read whole contiguous KiB per wave per load.
#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

namespace {

constexpr int kPackThreads = 256;

// bf16: output vector v = ((t * nsteps + s) * 64 + l)  <-  W[16t + l%16][32s + 8(l/16) .. +7]
__global__ __launch_bounds__(kPackThreads) void pack_bf16_kernel(const uint16_t* src, u32x4* dst, int d, int vocab,
                                                                 long long nvec) {
  const long long v = (long long)blockIdx.x * kPackThreads + threadIdx.x;
  if (v >= nvec) return;
  const int nsteps = d / 32;
  const int l = (int)(v & 63);
  const long long blk = v >> 6;
  const int s = (int)(blk % nsteps);
  const long long t = blk / nsteps;
  const long long row = t * 16 + (l & 15);
  u32x4 out = u32x4{0u, 0u, 0u, 0u};
  if (row < vocab) out = *reinterpret_cast<const u32x4*>(src + row * d + 32 * s + 8 * (l >> 4));
  dst[v] = out;
}

// 4-bit nibbles: output vector v = ((t * nquads + q) * 64 + l), word u = source bytes
// [16(4q+u) + 4(l/16), +4) of row 16t + l%16
__global__ __launch_bounds__(kPackThreads) void pack_q4_kernel(const uint8_t* src, u32x4* dst, int d, int vocab,
                                                               long long nvec) {
  const long long v = (long long)blockIdx.x * kPackThreads + threadIdx.x;
  if (v >= nvec) return;
  const int nquads = d / 128;
  const int l = (int)(v & 63);
  const long long blk = v >> 6;
  const int q = (int)(blk % nquads);
  const long long t = blk / nquads;
  const long long row = t * 16 + (l & 15);
  u32x4 out = u32x4{0u, 0u, 0u, 0u};
  if (row < vocab) {
    const uint32_t* rw = reinterpret_cast<const uint32_t*>(src + row * (d / 2));
    const int base = (16 * 4 * q + 4 * (l >> 4)) / 4;   // in words
    out = u32x4{rw[base], rw[base + 4], rw[base + 8], rw[base + 12]};
  }
  dst[v] = out;
}

// scales / mins: output vector v = ((t * nocts + c) * 16 + r)  <-  row 16t + r, groups 8c..8c+7
__global__ __launch_bounds__(kPackThreads) void pack_q4_scales_kernel(const uint16_t* src, u32x4* dst, int d,
                                                                      int vocab, long long nvec) {
  const long long v = (long long)blockIdx.x * kPackThreads + threadIdx.x;
  if (v >= nvec) return;
  const int nocts = d / 256;
  const int r = (int)(v & 15);
  const long long blk = v >> 4;
  const int c = (int)(blk % nocts);
  const long long t = blk / nocts;
  const long long row = t * 16 + r;
  u32x4 out = u32x4{0u, 0u, 0u, 0u};
  if (row < vocab) out = *reinterpret_cast<const u32x4*>(src + row * (d / 32) + 8 * c);
  dst[v] = out;
}

unsigned int blocks_for(long long n) { return (unsigned int)((n + kPackThreads - 1) / kPackThreads); }

}  // namespace

size_t tiled_bytes(int wtype, int d, int vocab, int part) {
  const size_t tiles = (size_t)(vocab + 15) / 16;
  if (wtype == MTP_W_BF16) return part == 0 ? tiles * 16 * (size_t)d * 2 : 0;
  if (wtype == MTP_W_Q4A32) return part == 0 ? tiles * 16 * (size_t)d / 2 : tiles * 16 * (size_t)(d / 32) * 2;
  return 0;
}

// gather: one block per output row; row r <- row ids[r] of the source (zeros for an id
// outside [0, vocab)); for 4-bit heads also the row's scales and mins
__global__ __launch_bounds__(kPackThreads) void gather_rows_kernel(const unsigned char* src, unsigned char* dst,
                                                                  size_t row_bytes, const int32_t* ids, int vocab) {
  const int r = blockIdx.x;
  const int id = ids[r];
  const bool ok = id >= 0 && id < vocab;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + (ok ? (size_t)id : 0) * row_bytes);
  u32x4* o = reinterpret_cast<u32x4*>(dst + (size_t)r * row_bytes);
  for (size_t v = threadIdx.x; v < row_bytes / 16; v += kPackThreads) o[v] = ok ? s[v] : u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_gather(int wtype, const void* w, const void* scale, const void* minv, int d, int vocab,
                         const int32_t* ids, int n, void* dst_w, void* dst_scale, void* dst_minv, hipStream_t stream) {
  const size_t rb = wtype == MTP_W_F32 ? (size_t)d * 4 : (wtype == MTP_W_BF16 ? (size_t)d * 2 : (size_t)d / 2);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(n), dim3(kPackThreads), 0, stream, static_cast<const unsigned char*>(w),
                     static_cast<unsigned char*>(dst_w), rb, ids, vocab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || wtype != MTP_W_Q4A32) return e;
  const size_t sb = (size_t)(d / 32) * 2;   // bf16 per 32-value group
  for (int part = 0; part < 2; ++part) {
    hipLaunchKernelGGL(gather_rows_kernel, dim3(n), dim3(kPackThreads), 0, stream,
                       static_cast<const unsigned char*>(part ? minv : scale),
                       static_cast<unsigned char*>(part ? dst_minv : dst_scale), sb, ids, vocab);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_pack(int wtype, const void* w, const void* scale, const void* minv, int d, int vocab,
                       void* dst_w, void* dst_scale, void* dst_minv, hipStream_t stream) {
  if (wtype == MTP_W_BF16) {
    const long long nvec = (long long)tiled_bytes(wtype, d, vocab, 0) / 16;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3(blocks_for(nvec)), dim3(kPackThreads), 0, stream,
                       static_cast<const uint16_t*>(w), static_cast<u32x4*>(dst_w), d, vocab, nvec);
    return hipGetLastError();
  }
  const long long nw = (long long)tiled_bytes(wtype, d, vocab, 0) / 16;
  hipLaunchKernelGGL(pack_q4_kernel, dim3(blocks_for(nw)), dim3(kPackThreads), 0, stream,
                     static_cast<const uint8_t*>(w), static_cast<u32x4*>(dst_w), d, vocab, nw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long ns = (long long)tiled_bytes(wtype, d, vocab, 1) / 16;
  hipLaunchKernelGGL(pack_q4_scales_kernel, dim3(blocks_for(ns)), dim3(kPackThreads), 0, stream,
                     static_cast<const uint16_t*>(scale), static_cast<u32x4*>(dst_scale), d, vocab, ns);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pack_q4_scales_kernel, dim3(blocks_for(ns)), dim3(kPackThreads), 0, stream,
                     static_cast<const uint16_t*>(minv), static_cast<u32x4*>(dst_minv), d, vocab, ns);
  return hipGetLastError();
}

}  // namespace mtp
