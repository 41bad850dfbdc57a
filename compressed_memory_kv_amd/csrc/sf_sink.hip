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
// One thread per 16-byte chunk of the temporal planes of a (block, Z0 row, head); it
// turns
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NP temporal planes of one head start its row: NP * (bf16 ? 4 : 8) bytes, 16-byte aligned
// (a head row is 128 or 256 bytes), cut into 16-byte chunks (the last may be 8 bytes).
// One thread per chunk: neighbouring lanes take neighbouring chunks of a head, so a wave
// touches one run of bytes per head instead of one word per lane of 64 heads.
template <bool BF16, int NP>
__global__ __launch_bounds__(kSinkThreads) void sink_rotate_kernel(char* __restrict__ mem, size_t block_stride,
                                                                    int n_blocks, int rows, int heads, int head_dim,
                                                                    SinkTable tab) {
  constexpr int EB = BF16 ? 4 : 8;                     // bytes per plane
  constexpr int BYTES = NP * EB;
  constexpr int NC = (BYTES + 15) / 16;                // chunks per head
  constexpr int PPC = 16 / EB;                         // planes per full chunk
  const unsigned per_block = (unsigned)rows * (unsigned)heads * NC;  // < 2^31 (checked at launch)
  const unsigned idx = wg_x() * kSinkThreads + tid_x();
  if (idx >= per_block) return;
  const unsigned b = wg_y();                           // one grid row per block
  const unsigned rh = idx / NC;                        // row * heads + head
  const int ch = (int)(idx - rh * NC);
  char* p = mem + (size_t)b * block_stride + (size_t)rh * head_dim * (BF16 ? 2 : 4) + 16 * ch;
  const int p0 = ch * PPC;                             // first plane of the chunk
  const bool full = (ch + 1) * 16 <= BYTES;
  unsigned w[4];
  if (full) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  } else {                                             // the 8-byte tail chunk
    const unsigned* q = reinterpret_cast<const unsigned*>(p);
    w[0] = q[0];
    w[1] = q[1];
    w[2] = 0u;
    w[3] = 0u;
  }
  if (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = min(p0 + j, NP - 1);
      const float c = tab.c[i], s = tab.s[i];
      const float a = bf16_lo(w[j]), b2 = bf16_hi(w[j]);
      w[j] = pack_bf16(__builtin_fmaf(a, c, -(b2 * s)), __builtin_fmaf(a, s, b2 * c));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = min(p0 + j, NP - 1);
      const float c = tab.c[i], s = tab.s[i];
      const float a = __builtin_bit_cast(float, w[2 * j]);
      const float b2 = __builtin_bit_cast(float, w[2 * j + 1]);
      const float ra = __builtin_fmaf(a, c, -(b2 * s));
      const float rb = __builtin_fmaf(a, s, b2 * c);
      w[2 * j] = __builtin_bit_cast(unsigned, ra);
      w[2 * j + 1] = __builtin_bit_cast(unsigned, rb);
    }
  }
  if (full) {
    u32x4 v;
    v.x = w[0];
    v.y = w[1];
    v.z = w[2];
    v.w = w[3];
    *reinterpret_cast<u32x4*>(p) = v;
  } else {
    unsigned* q = reinterpret_cast<unsigned*>(p);
    q[0] = w[0];
    q[1] = w[1];
  }
}

}  // namespace

hipError_t launch_sink_rotate(void* mem, int n_blocks, size_t block_stride, int rows, int heads, int head_dim,
                              bool bf16, const SinkTable& tab, hipStream_t stream) {
  const int eb = bf16 ? 4 : 8;
  const long long n = (long long)rows * heads * ((tab.n_planes * eb + 15) / 16);  // threads per block
  if (n == 0 || n_blocks == 0) return hipSuccess;
  if (n >= (1LL << 31) || n_blocks > 65535) return hipErrorInvalidValue;
  const long long grid = (n + kSinkThreads - 1) / kSinkThreads;
  // the temporal band of the two head sizes: 12 planes at 64, 22 at 128
  char* m = static_cast<char*>(mem);
  const dim3 g((unsigned)grid, (unsigned)n_blocks), t(kSinkThreads);
  if (tab.n_planes == 12 && head_dim == 64) {
    if (bf16) hipLaunchKernelGGL((sink_rotate_kernel<true, 12>), g, t, 0, stream, m, block_stride, n_blocks, rows, heads, head_dim, tab);
    else hipLaunchKernelGGL((sink_rotate_kernel<false, 12>), g, t, 0, stream, m, block_stride, n_blocks, rows, heads, head_dim, tab);
  } else if (tab.n_planes == 22 && head_dim == 128) {
    if (bf16) hipLaunchKernelGGL((sink_rotate_kernel<true, 22>), g, t, 0, stream, m, block_stride, n_blocks, rows, heads, head_dim, tab);
    else hipLaunchKernelGGL((sink_rotate_kernel<false, 22>), g, t, 0, stream, m, block_stride, n_blocks, rows, heads, head_dim, tab);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sf
