// Whole-block copies: dst block d = src block s for each (s, d) pair.
//
// Two uses, one kernel. Inside the pool it is the device half of copy-on-write: a
// sequence about to write into a last block it shares with others first gets a fresh
// block holding the same tokens (page "vLLM GitHub 项目 …", section 二, item 4: shared
// prefix blocks). Between the pool and pinned host memory it swaps blocks out and back in
// (the CPU swap space, --swap-space in the flag table of page "vLLM 部署深度指南").
//
// Each workgroup copies one 16 KiB chunk of one pair's block: 256 threads, four 16-byte
// pieces each, loads first, then stores. A pair that names a block outside its buffer is
// skipped. Bound by HBM (pool to pool: every byte read once and written once) or by the
// host link (swaps). Every source byte is read once, so the loads carry the non-temporal
// hint (4096 pairs of 256 KiB blocks after a cache flush: 5.24 -> 5.61 TB/s of reads and
// writes, against 5.42 for torch's contiguous copy of the same bytes; back to back, with
// the last copy's writes still draining, 4.99 -> 4.89); the hint on the stores, or eight
// pieces per thread, was slower (4.98 and 3.87 TB/s after a flush).
#include "pa_device.h"
#include "pa_launch.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kPiecesPerThread = 4;
constexpr int64_t kChunkBytes = (int64_t)kThreads * kPiecesPerThread * 16;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void move_blocks_kernel(
    char* dst, const char* src, const int64_t* __restrict__ pairs,
    int64_t block_bytes, int64_t chunks, int64_t dst_blocks, int64_t src_blocks) {
  const int64_t item = blockIdx.x;
  const int64_t pair = item / chunks;
  const int64_t chunk = item % chunks;
  const int64_t s = pairs[2 * pair];
  const int64_t d = pairs[2 * pair + 1];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;  // uniform per workgroup
  const char* from = src + s * block_bytes + chunk * kChunkBytes;
  char* to = dst + d * block_bytes + chunk * kChunkBytes;
  const int64_t left = block_bytes - chunk * kChunkBytes;
  u32x4 v[kPiecesPerThread];
#pragma unroll
  for (int i = 0; i < kPiecesPerThread; ++i) {
    const int64_t off = ((int64_t)i * kThreads + threadIdx.x) * 16;
    if (off < left) v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(from + off));
  }
#pragma unroll
  for (int i = 0; i < kPiecesPerThread; ++i) {
    const int64_t off = ((int64_t)i * kThreads + threadIdx.x) * 16;
    if (off < left) *reinterpret_cast<u32x4*>(to + off) = v[i];
  }
}

}  // namespace

hipError_t launch_move_blocks(void* dst, const void* src, const int64_t* pairs, int num_pairs,
                              int64_t block_bytes, int64_t dst_blocks, int64_t src_blocks,
                              hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = (block_bytes + kChunkBytes - 1) / kChunkBytes;
  const int64_t items = chunks * num_pairs;
  if (items > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(move_blocks_kernel, dim3((unsigned)items), dim3(kThreads), 0, stream,
                     static_cast<char*>(dst), static_cast<const char*>(src), pairs, block_bytes,
                     chunks, dst_blocks, src_blocks);
  return hipGetLastError();
}

}  // namespace pkv
