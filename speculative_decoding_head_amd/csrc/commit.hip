// Commit of one speculative cycle: the accepted row's recurrent-state snapshot becomes
// the live state and the KV rows of rejected drafts are trimmed (DS4Server issue "Add
// Qwen3.8 Flash Next native MTP speculation", section "Implementation": capture
// verification-row state, trim rejected rows, commit only accepted rows; lucebox-hub PR
// "feat(qwen4exp): MTP speculative decoding", section "Exactness": rollback restores the
// KV / recurrent state bit-exactly; llama.cpp PR "qwen4exp : port NextN/MTP speculative
// decoding to master", commit "keep speculative checkpoints on device": the state never
// leaves device memory).
//
// Grid (chunks + 1, B).  Blocks 1.. copy 16-byte vectors of snapshots[b][a] into live[b]
// with non-temporal loads and stores (the bytes are streamed once); block 0 of each
// request zero-fills its rejected KV rows and then updates kv_len[b].  Only block 0
// reads or writes kv_len, so the update cannot race with the trim.
#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

namespace {

constexpr int kCommitThreads = 256;
// 16-byte vectors per thread per block: 64 KiB chunks for a copy of tens of MiB, 16 KiB
// chunks for hundreds (more, shorter blocks: reads and writes of different blocks overlap
// better; measured 5.9 vs 5.2 TB/s for 16 x 36 MiB, and the reverse below ~100 MiB)
constexpr int kVecLarge = 16, kVecSmall = 4;
constexpr size_t kSmallChunksFrom = (size_t)256 << 20;   // total bytes copied

template <int VPT>
__global__ __launch_bounds__(kCommitThreads) void mtp_commit_state_kernel(CommitLaunch p) {
  constexpr int kVecPerThread = VPT;
  constexpr size_t kChunkBytes = (size_t)kCommitThreads * kVecPerThread * 16;
  const int b = blockIdx.y;
  int a = p.n_accept[b];
  a = a < 0 ? 0 : (a > p.k ? p.k : a);

  if (blockIdx.x > 0) {
    const size_t chunk = blockIdx.x - 1;
    const size_t nvec = p.state_bytes / 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.snapshots) +
                                                      ((size_t)b * (p.k + 1) + a) * p.state_bytes);
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<unsigned char*>(p.live) + (size_t)b * p.state_bytes);
    const size_t v0 = chunk * (kChunkBytes / 16);
    u32x4 v[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const size_t idx = v0 + (size_t)u * kCommitThreads + threadIdx.x;
      if (idx < nvec) v[u] = __builtin_nontemporal_load(src + idx);
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
      const size_t idx = v0 + (size_t)u * kCommitThreads + threadIdx.x;
      if (idx < nvec) __builtin_nontemporal_store(v[u], dst + idx);
    }
    return;
  }

  // block 0: KV trim, then kv_len
  int len = p.kv_len[b];
  len = len < 0 ? 0 : (len > p.max_rows ? p.max_rows : len);
  if (p.n_layers > 0) {
    const int lo = min(len + a + 1, p.max_rows), hi = min(len + p.k + 1, p.max_rows);
    const size_t row_vecs = p.kv_row_bytes / 16;
    const size_t per_plane = (size_t)(hi > lo ? hi - lo : 0) * row_vecs;   // vectors per (layer, K|V)
    unsigned char* base = static_cast<unsigned char*>(p.kv) +
                          (size_t)b * p.n_layers * 2 * p.max_rows * p.kv_row_bytes;
    // the rejected rows of one plane are contiguous: one plane after the other, no division
    for (int plane = 0; plane < 2 * p.n_layers; ++plane) {
      u32x4* dst = reinterpret_cast<u32x4*>(base + ((size_t)plane * p.max_rows + lo) * p.kv_row_bytes);
      for (size_t off = threadIdx.x; off < per_plane; off += kCommitThreads) dst[off] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) p.kv_len[b] = min(len + a + 1, p.max_rows);
}

}  // namespace

template <int VPT>
static hipError_t launch_commit_t(const CommitLaunch& p, hipStream_t stream) {
  constexpr size_t kChunkBytes = (size_t)kCommitThreads * VPT * 16;
  const size_t chunks = (p.state_bytes + kChunkBytes - 1) / kChunkBytes;
  hipLaunchKernelGGL(mtp_commit_state_kernel<VPT>, dim3((unsigned)chunks + 1, p.B), dim3(kCommitThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitLaunch& p, hipStream_t stream) {
  return (size_t)p.B * p.state_bytes >= kSmallChunksFrom ? launch_commit_t<kVecSmall>(p, stream)
                                                         : launch_commit_t<kVecLarge>(p, stream);
}

}  // namespace mtp
