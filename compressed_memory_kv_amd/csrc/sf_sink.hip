// The streaming sink: Z0's stored keys moved forward in time, in place.
//
// Model card "GTA world model: weights and inference code", section "Running for
// a long time: the start image follows the window": rotary keys compose,
// rotation(id + T) = rotation(id) * rotation(T), so when the start image falls too
// far behind the window its cached keys are multiplied by one more rotation; values
// are untouched and nothing is recomputed.  Section "Telling a summary from a pixel:
// level planes" gives 12 temporal planes per head at head_dim 64, which is the
// temporal band of the rotary table the "Positions" item credits (Wan2.1): the
// first hd/2 - 2*floor(hd/6) complex planes of a head (dims 2i, 2i+1).
//
// One thread per (block, Z0 row, head): it loads the head's temporal planes, turns
// plane i by the angle whose cosine and sine the host computed in fp64 (stored as
// fp32), x' = x c - y s, y' = x s + y c in fp32, and stores them rounded to the
// storage type (bf16: nearest even).  The kernel is HBM-bound: the temporal dims
// are the first bytes of each 128- or 256-byte head row.
#include "sf_internal.h"

namespace sf {
namespace {

constexpr int kSinkThreads = 256;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
  return (unsigned)__builtin_bit_cast(unsigned short, a) | ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}

template <bool BF16>
__global__ __launch_bounds__(kSinkThreads) void sink_rotate_kernel(char* __restrict__ mem, size_t block_stride,
                                                                    int n_blocks, int rows, int heads, int head_dim,
                                                                    SinkTable tab) {
  const long long gid = (long long)wg_x() * kSinkThreads + tid_x();
  const long long per_block = (long long)rows * heads;
  if (gid >= per_block * n_blocks) return;
  const int b = (int)(gid / per_block);
  const long long rh = gid - (long long)b * per_block;  // row * heads + head
  const int np = tab.n_planes;
  if (BF16) {
    unsigned* p = reinterpret_cast<unsigned*>(mem + (size_t)b * block_stride + (size_t)rh * head_dim * 2);
    for (int i = 0; i < np; ++i) {
      const unsigned w = p[i];
      const float x = bf16_lo(w), y = bf16_hi(w);
      const float xr = __builtin_fmaf(x, tab.c[i], -(y * tab.s[i]));
      const float yr = __builtin_fmaf(x, tab.s[i], y * tab.c[i]);
      p[i] = pack_bf16(xr, yr);
    }
  } else {
    float2* p = reinterpret_cast<float2*>(mem + (size_t)b * block_stride + (size_t)rh * head_dim * 4);
    for (int i = 0; i < np; ++i) {
      const float2 v = p[i];
      p[i] = make_float2(__builtin_fmaf(v.x, tab.c[i], -(v.y * tab.s[i])), __builtin_fmaf(v.x, tab.s[i], v.y * tab.c[i]));
    }
  }
}

}  // namespace

hipError_t launch_sink_rotate(void* mem, int n_blocks, size_t block_stride, int rows, int heads, int head_dim,
                              bool bf16, const SinkTable& tab, hipStream_t stream) {
  const long long n = (long long)n_blocks * rows * heads;
  if (n == 0) return hipSuccess;
  const long long grid = (n + kSinkThreads - 1) / kSinkThreads;
  if (grid >= (1LL << 31)) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(sink_rotate_kernel<true>, dim3((unsigned)grid), dim3(kSinkThreads), 0, stream,
                       static_cast<char*>(mem), block_stride, n_blocks, rows, heads, head_dim, tab);
  else
    hipLaunchKernelGGL(sink_rotate_kernel<false>, dim3((unsigned)grid), dim3(kSinkThreads), 0, stream,
                       static_cast<char*>(mem), block_stride, n_blocks, rows, heads, head_dim, tab);
  return hipGetLastError();
}

}  // namespace sf
