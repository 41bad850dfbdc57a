// Byte-moving kernels of the per-block memory: zero fill at creation, the
// record write into Z0 / a RAW slot, and the RAW -> SUM eviction of the
// summary rows in every block at once.
//
// Model card "GTA world model: weights and inference code", section
// "One buffer, no mask": a frame's record is written into its RAW place and,
// when the frame leaves the raw window, only the K/V of its summary rows are
// copied into SUM; that copy is all it costs to move a frame into long-term
// memory.  All of these are HBM-bound copies: 16-byte vector loads and
// stores, four in flight per thread, 64-bit indexing.
#include "sf_internal.h"

namespace sf {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint4* __restrict__ p, size_t n16) {
  size_t i = (size_t)blockIdx.x * kThreads * kVecPerThread + threadIdx.x;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j, i += kThreads)
    if (i < n16) p[i] = z;
}

// Two independent copies of n16 16-byte vectors (K and V) in one launch:
// the first half of the grid copies K, the second half V.
__global__ __launch_bounds__(kThreads) void copy_pair_kernel(uint4* __restrict__ dk, uint4* __restrict__ dv,
                                                             const uint4* __restrict__ sk,
                                                             const uint4* __restrict__ sv, size_t n16,
                                                             unsigned blocks_per_tensor) {
  const bool second = blockIdx.x >= blocks_per_tensor;
  const unsigned b = second ? blockIdx.x - blocks_per_tensor : blockIdx.x;
  uint4* __restrict__ d = second ? dv : dk;
  const uint4* __restrict__ s = second ? sv : sk;
  size_t i = (size_t)b * kThreads * kVecPerThread + threadIdx.x;
  uint4 r[kVecPerThread];
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j)
    if (i + (size_t)j * kThreads < n16) r[j] = s[i + (size_t)j * kThreads];
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j)
    if (i + (size_t)j * kThreads < n16) d[i + (size_t)j * kThreads] = r[j];
}

// Eviction: for every block b and tensor (K, V), copy n16 vectors from
// src_off to dst_off.  Grid: blocks_per_copy workgroups per (block, tensor).
__global__ __launch_bounds__(kThreads) void evict_kernel(char* __restrict__ mem, size_t block_stride,
                                                         size_t v_offset, size_t src_off, size_t dst_off,
                                                         size_t n16, unsigned blocks_per_copy) {
  const unsigned copy = blockIdx.x / blocks_per_copy;  // = 2 * block + tensor
  const unsigned b = blockIdx.x - copy * blocks_per_copy;
  char* base = mem + (size_t)(copy >> 1) * block_stride + ((copy & 1u) ? v_offset : 0);
  const uint4* __restrict__ s = reinterpret_cast<const uint4*>(base + src_off);
  uint4* __restrict__ d = reinterpret_cast<uint4*>(base + dst_off);
  size_t i = (size_t)b * kThreads * kVecPerThread + threadIdx.x;
  uint4 r[kVecPerThread];
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j)
    if (i + (size_t)j * kThreads < n16) r[j] = s[i + (size_t)j * kThreads];
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j)
    if (i + (size_t)j * kThreads < n16) d[i + (size_t)j * kThreads] = r[j];
}

unsigned blocks_for(size_t n16) {
  return (unsigned)((n16 + (size_t)kThreads * kVecPerThread - 1) / ((size_t)kThreads * kVecPerThread));
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15u)) return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const size_t per_launch = (size_t)1 << 28;  // vectors per launch keeps the grid well inside 2^31
  for (size_t off = 0; off < n16; off += per_launch) {
    const size_t n = n16 - off < per_launch ? n16 - off : per_launch;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, stream,
                       reinterpret_cast<uint4*>(p) + off, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_copy_rows(void* dst_k, void* dst_v, const void* src_k, const void* src_v, size_t bytes,
                            hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0) return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const unsigned per = blocks_for(n16);
  if ((size_t)per * 2 >= ((size_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_pair_kernel, dim3(per * 2), dim3(kThreads), 0, stream, reinterpret_cast<uint4*>(dst_k),
                     reinterpret_cast<uint4*>(dst_v), reinterpret_cast<const uint4*>(src_k),
                     reinterpret_cast<const uint4*>(src_v), n16, per);
  return hipGetLastError();
}

hipError_t launch_evict(void* mem, int n_blocks, size_t block_stride, size_t v_offset, size_t src_off,
                        size_t dst_off, size_t bytes, hipStream_t stream) {
  if (bytes == 0 || n_blocks <= 0) return hipSuccess;
  if (bytes % 16 != 0 || src_off % 16 != 0 || dst_off % 16 != 0) return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const unsigned per = blocks_for(n16);
  const size_t grid = (size_t)per * 2 * (size_t)n_blocks;
  if (grid >= ((size_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(evict_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, reinterpret_cast<char*>(mem),
                     block_stride, v_offset, src_off, dst_off, n16, per);
  return hipGetLastError();
}

}  // namespace sf
