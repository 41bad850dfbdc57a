// Byte-moving kernels of the per-block memory: zero fill at creation, the
// record write into Z0 / a RAW slot, and the RAW -> SUM eviction of the
// summary rows in every block at once.
//
// Model card "GTA world model: weights and inference code", section
// "One buffer, no mask": a frame's record is written into its RAW place and,
// when the frame leaves the raw window, only the K/V of its summary rows are
// copied into SUM; that copy is all it costs to move a frame into long-term
// memory.  These are HBM-bound copies.  Each thread moves kVec 16-byte
// vectors; the loads of a thread are all issued before its first store (no
// branches between them), so every wave keeps kVec loads in flight.  Only
// the last workgroup of a copy takes the bounds-checked path.
#include "sf_internal.h"

namespace sf {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kVec = 4;
constexpr size_t kPerBlock = (size_t)kThreads * kVec;  // vectors per workgroup

__device__ __forceinline__ void copy_chunk(u32x4* __restrict__ d, const u32x4* __restrict__ s, size_t first,
                                           size_t n16) {
  const size_t i = first + tid_x();
  if (first + kPerBlock <= n16) {
    // the source is not read again: stream it past the caches
    const u32x4 a0 = __builtin_nontemporal_load(s + i);
    const u32x4 a1 = __builtin_nontemporal_load(s + i + kThreads);
    const u32x4 a2 = __builtin_nontemporal_load(s + i + 2 * kThreads);
    const u32x4 a3 = __builtin_nontemporal_load(s + i + 3 * kThreads);
    d[i] = a0;
    d[i + kThreads] = a1;
    d[i + 2 * kThreads] = a2;
    d[i + 3 * kThreads] = a3;
  } else {
    for (size_t j = i; j < n16; j += kThreads) d[j] = s[j];
  }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(u32x4* __restrict__ p, size_t n16) {
  const size_t first = (size_t)wg_x() * kPerBlock;
  const size_t i = first + tid_x();
  const u32x4 z = {0u, 0u, 0u, 0u};
  if (first + kPerBlock <= n16) {
    p[i] = z;
    p[i + kThreads] = z;
    p[i + 2 * kThreads] = z;
    p[i + 3 * kThreads] = z;
  } else {
    for (size_t j = i; j < n16; j += kThreads) p[j] = z;
  }
}

// Two copies of n16 vectors (K and V) in one launch: workgroups
// [0, per) copy K, [per, 2*per) copy V.
__global__ __launch_bounds__(kThreads) void copy_pair_kernel(u32x4* __restrict__ dk, u32x4* __restrict__ dv,
                                                             const u32x4* __restrict__ sk,
                                                             const u32x4* __restrict__ sv, size_t n16,
                                                             unsigned per) {
  const bool second = wg_x() >= per;
  const unsigned b = second ? wg_x() - per : wg_x();
  copy_chunk(second ? dv : dk, second ? sv : sk, (size_t)b * kPerBlock, n16);
}

// Eviction: for every block and tensor (K, V) copy n16 vectors from src_off
// to dst_off.  Workgroup w serves copy w / per (= 2 * block + tensor).
__global__ __launch_bounds__(kThreads) void evict_kernel(char* __restrict__ mem, size_t block_stride,
                                                         size_t v_offset, size_t src_off, size_t dst_off,
                                                         size_t n16, unsigned per) {
  const unsigned copy = wg_x() / per;
  const unsigned b = wg_x() - copy * per;
  char* base = mem + (size_t)(copy >> 1) * block_stride + ((copy & 1u) ? v_offset : 0);
  copy_chunk(reinterpret_cast<u32x4*>(base + dst_off), reinterpret_cast<const u32x4*>(base + src_off),
             (size_t)b * kPerBlock, n16);
}

unsigned blocks_for(size_t n16) { return (unsigned)((n16 + kPerBlock - 1) / kPerBlock); }

// Measurement aid: a copy through LDS with the transfer the head_dim-64 attention uses
// for its K/V tiles (buffer_load_dwordx4 ... lds), so that hardware traffic counters can
// be calibrated on that path.  Workgroup c moves the 16 KiB chunk c: each wave lands four
// 1 KiB transfers in its own quarter of the LDS buffer, waits for them, reads its own
// bytes back and stores them.
constexpr int kLdsChunk = 16384;
__global__ __launch_bounds__(kThreads) void lds_copy_kernel(char* __restrict__ dst, const char* __restrict__ src) {
  __shared__ __attribute__((aligned(16))) char buf[kLdsChunk];
  const size_t c = wg_x();
  const int wave = __builtin_amdgcn_readfirstlane((int)(tid_x() >> 6));  // uniform: scalar offsets
  const int lane = (int)(tid_x() & 63);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + c * kLdsChunk, (short)0, kLdsChunk, 0x00020000);
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int off = wave * 4096 + m * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(buf + off), 16, (unsigned)(lane * 16), (unsigned)off, 0,
                                             0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's transfers have landed
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int off = wave * 4096 + m * 1024 + lane * 16;
    *reinterpret_cast<u32x4*>(dst + c * kLdsChunk + off) = *reinterpret_cast<const u32x4*>(buf + off);
  }
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15u)) return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  const size_t per_launch = (size_t)1 << 30;  // vectors per launch keeps the grid well inside 2^31
  for (size_t off = 0; off < n16; off += per_launch) {
    const size_t n = n16 - off < per_launch ? n16 - off : per_launch;
    launch(fill_zero_kernel, dim3(blocks_for(n)), dim3(kThreads), stream,
                       reinterpret_cast<u32x4*>(p) + off, n);
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
  launch(copy_pair_kernel, dim3(per * 2), dim3(kThreads), stream, reinterpret_cast<u32x4*>(dst_k),
                     reinterpret_cast<u32x4*>(dst_v), reinterpret_cast<const u32x4*>(src_k),
                     reinterpret_cast<const u32x4*>(src_v), n16, per);
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
  launch(evict_kernel, dim3((unsigned)grid), dim3(kThreads), stream, reinterpret_cast<char*>(mem),
                     block_stride, v_offset, src_off, dst_off, n16, per);
  return hipGetLastError();
}

hipError_t launch_lds_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (bytes % kLdsChunk != 0 || bytes / kLdsChunk >= ((size_t)1 << 31)) return hipErrorInvalidValue;
  launch(lds_copy_kernel, dim3((unsigned)(bytes / kLdsChunk)), dim3(kThreads), stream, reinterpret_cast<char*>(dst),
         reinterpret_cast<const char*>(src));
  return hipGetLastError();
}

}  // namespace sf
