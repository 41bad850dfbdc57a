// Rotary kernels of the per-block memory: the streaming sink (Z0's stored keys moved
// forward in time, in place) and the rotating record write (a record's keys, or a
// query, turned by its frame id on the temporal planes, with the level planes).
//
// Model card "GTA world model: weights and inference code":
//  * section "Running for a long time: the start image follows the window": rotary
//    keys compose, rotation(id + T) = rotation(id) * rotation(T), so when the start
//    image falls too far behind the window its cached keys are multiplied by one more
//    rotation; values are untouched and nothing is recomputed.
//  * section "Telling a summary from a pixel: level planes": 12 temporal planes per
//    head at head_dim 64; the two slowest carry no usable position and become a level
//    axis: summary tokens take an exact quarter turn on them.
//  * the "Positions" item of "The rest of the model": one rotary table adapted from
//    Wan2.1, whose temporal band is the first hd/2 - 2*floor(hd/6) complex planes of a
//    head (dims 2i, 2i+1).
//
// Plane i turns by the angle whose cosine and sine the host computed in fp64 (stored
// as fp32): x' = x c - y s, y' = x s + y c in fp32, rounded to the storage type (bf16:
// nearest even).  The quarter turn (x, y) -> (-y, x) is exact: a swap and a sign, so
// with the level planes a summary row's bytes on those planes are a pure function of
// its input bytes (replace reading) or of its rotated bytes (add reading).  Both kernels
// are HBM-bound: one thread per 16-byte chunk, neighbouring lanes on neighbouring bytes.
#include "sf_internal.h"

namespace sf {
namespace {

constexpr int kRopeThreads = 256;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
  return (unsigned)__builtin_bit_cast(unsigned short, a) | ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// What happens to one plane of one row.
enum PlaneOp : int { kKeep = 0, kTurn = 1, kQuarter = 2, kTurnQuarter = 3 };

// Temporal planes p0 .. p0 + 16/EB - 1 held in w[4] (bf16: one plane per word; fp32: two
// words per plane).  Plane p < NP turns by (c[p], s[p]) unless `lvl_op` applies (p is one
// of the two slowest planes and the row is a summary row).
template <bool BF16, int NP>
__device__ __forceinline__ void turn_planes(unsigned w[4], int p0, bool summary, int lvl_op, const SinkTable& tab) {
  if (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = p0 + j;
      const int op = p >= NP ? kKeep : (summary && p >= NP - 2) ? lvl_op : kTurn;
      const int i = min(p, NP - 1);
      const float c = tab.c[i], s = tab.s[i];
      const float a = bf16_lo(w[j]), b = bf16_hi(w[j]);
      const float ra = __builtin_fmaf(a, c, -(b * s));
      const float rb = __builtin_fmaf(a, s, b * c);
      if (op == kTurn) w[j] = pack_bf16(ra, rb);
      else if (op == kQuarter) w[j] = ((w[j] >> 16) ^ 0x8000u) | (w[j] << 16);
      else if (op == kTurnQuarter) w[j] = pack_bf16(-rb, ra);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = p0 + j;
      const int op = p >= NP ? kKeep : (summary && p >= NP - 2) ? lvl_op : kTurn;
      const int i = min(p, NP - 1);
      const float c = tab.c[i], s = tab.s[i];
      const unsigned wa = w[2 * j], wb = w[2 * j + 1];
      const float a = __builtin_bit_cast(float, wa);
      const float b = __builtin_bit_cast(float, wb);
      const float ra = __builtin_fmaf(a, c, -(b * s));
      const float rb = __builtin_fmaf(a, s, b * c);
      if (op == kTurn) {
        w[2 * j] = __builtin_bit_cast(unsigned, ra);
        w[2 * j + 1] = __builtin_bit_cast(unsigned, rb);
      } else if (op == kQuarter) {
        w[2 * j] = wb ^ 0x80000000u;
        w[2 * j + 1] = wa;
      } else if (op == kTurnQuarter) {
        w[2 * j] = __builtin_bit_cast(unsigned, rb) ^ 0x80000000u;
        w[2 * j + 1] = __builtin_bit_cast(unsigned, ra);
      }
    }
  }
}

// Sink: NP temporal planes of one head start its row: NP * (bf16 ? 4 : 8) bytes, 16-byte
// aligned (a head row is 128 or 256 bytes), cut into 16-byte chunks (the last may be 8
// bytes).  Chunks of (block, Z0 row, head) are numbered per block; a thread takes
// kSinkPer of them, kRopeThreads apart (each load instruction of a wave covers
// consecutive chunks), and issues all its loads before the first store, so that many
// bytes are in flight: the line size makes the memory system move whole 128-byte head
// rows for the 48 (or 88) bytes the planes hold.  Grid row = block.  Rows from
// `lvl_row0` on keep their two slowest planes (the level axis under the replace reading);
// lvl_row0 >= rows turns every plane of every row.
constexpr int kSinkPer = 4;
template <bool BF16, int NP>
__global__ __launch_bounds__(kRopeThreads) void sink_rotate_kernel(char* __restrict__ mem, size_t block_stride,
                                                                    int lvl_row0, int rows, int heads, int head_dim,
                                                                    SinkTable tab) {
  constexpr int EB = BF16 ? 4 : 8;                     // bytes per plane
  constexpr int BYTES = NP * EB;
  constexpr int NC = (BYTES + 15) / 16;                // chunks per head
  constexpr int PPC = 16 / EB;                         // planes per full chunk
  const unsigned per_block = (unsigned)rows * (unsigned)heads * NC;  // < 2^31 (checked at launch)
  const unsigned first = wg_x() * (kRopeThreads * kSinkPer) + tid_x();
  char* base = mem + (size_t)wg_y() * block_stride;   // one grid row per block
  unsigned w[kSinkPer][4];
  char* p[kSinkPer];
  int ch[kSinkPer];
#pragma unroll
  for (int k = 0; k < kSinkPer; ++k) {
    const unsigned idx = first + k * kRopeThreads;
    const unsigned rh = idx / NC;                      // row * heads + head
    ch[k] = (int)(idx - rh * NC);
    p[k] = base + (size_t)rh * head_dim * (BF16 ? 2 : 4) + 16 * ch[k];
    w[k][0] = w[k][1] = w[k][2] = w[k][3] = 0u;
    if (idx >= per_block) continue;
    if ((ch[k] + 1) * 16 <= BYTES) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(p[k]);
      w[k][0] = v.x;
      w[k][1] = v.y;
      w[k][2] = v.z;
      w[k][3] = v.w;
    } else {                                           // the 8-byte tail chunk
      const unsigned* q = reinterpret_cast<const unsigned*>(p[k]);
      w[k][0] = q[0];
      w[k][1] = q[1];
    }
  }
#pragma unroll
  for (int k = 0; k < kSinkPer; ++k) {
    const unsigned idx = first + k * kRopeThreads;
    if (idx >= per_block) continue;
    const bool keep_level = (int)(idx / NC / (unsigned)heads) >= lvl_row0;
    turn_planes<BF16, NP>(w[k], ch[k] * PPC, keep_level, kKeep, tab);
    if ((ch[k] + 1) * 16 <= BYTES) {
      u32x4 v;
      v.x = w[k][0];
      v.y = w[k][1];
      v.z = w[k][2];
      v.w = w[k][3];
      *reinterpret_cast<u32x4*>(p[k]) = v;
    } else {
      unsigned* q = reinterpret_cast<unsigned*>(p[k]);
      q[0] = w[k][0];
      q[1] = w[k][1];
    }
  }
}

// Rotating write: up to three tensors of `rows` rows [heads][head_dim], each moved from
// src to dst, either with the temporal planes turned (a record's K, a query) or as it is
// (a record's V).  One thread per 16-byte chunk: threads [j*n, (j+1)*n) take tensor j's
// chunks in order.  Rows from hw on are summary rows: their two slowest planes take
// `lvl_op`.  src and dst may be the same rows (in place: each thread reads its chunk
// before it writes it).
struct RopeTensors {
  u32x4* dst[3];
  const u32x4* src[3];
  int turn[3];
};

template <bool BF16, int NP>
__global__ __launch_bounds__(kRopeThreads) void rope_rows_kernel(const RopeTensors r, unsigned n, int n_tensors,
                                                                  int hw, int heads, int chunks_per_head,
                                                                  int lvl_op, SinkTable tab) {
  constexpr int PPC = BF16 ? 4 : 2;                    // planes per 16-byte chunk
  const unsigned gidx = wg_x() * kRopeThreads + tid_x();
  const unsigned j = gidx / n;
  if ((int)j >= n_tensors) return;
  const unsigned idx = gidx - j * n;
  u32x4* dst = r.dst[j];
  const u32x4 v = __builtin_nontemporal_load(r.src[j] + idx);
  const unsigned rh = idx / (unsigned)chunks_per_head;
  const int ch = (int)(idx - rh * (unsigned)chunks_per_head);
  if (!r.turn[j] || ch * PPC >= NP) {                  // a value tensor, or past the temporal band
    dst[idx] = v;
    return;
  }
  unsigned w[4] = {v.x, v.y, v.z, v.w};
  const bool summary = (int)(rh / (unsigned)heads) >= hw;
  turn_planes<BF16, NP>(w, ch * PPC, summary, lvl_op, tab);
  u32x4 o;
  o.x = w[0];
  o.y = w[1];
  o.z = w[2];
  o.w = w[3];
  dst[idx] = o;
}

}  // namespace

hipError_t launch_sink_rotate(void* mem, int n_blocks, size_t block_stride, int lvl_row0, int rows, int heads,
                              int head_dim, bool bf16, const SinkTable& tab, hipStream_t stream) {
  const int eb = bf16 ? 4 : 8;
  const long long n = (long long)rows * heads * ((tab.n_planes * eb + 15) / 16);  // threads per block
  if (n == 0 || n_blocks == 0) return hipSuccess;
  if (n >= (1LL << 31) || n_blocks > 65535) return hipErrorInvalidValue;
  const long long grid = (n + kRopeThreads * kSinkPer - 1) / (kRopeThreads * kSinkPer);
  // the temporal band of the two head sizes: 12 planes at 64, 22 at 128
  char* m = static_cast<char*>(mem);
  const dim3 g((unsigned)grid, (unsigned)n_blocks), t(kRopeThreads);
  if (tab.n_planes == 12 && head_dim == 64) {
    if (bf16) launch((sink_rotate_kernel<true, 12>), g, t, stream, m, block_stride, lvl_row0, rows, heads, head_dim, tab);
    else launch((sink_rotate_kernel<false, 12>), g, t, stream, m, block_stride, lvl_row0, rows, heads, head_dim, tab);
  } else if (tab.n_planes == 22 && head_dim == 128) {
    if (bf16) launch((sink_rotate_kernel<true, 22>), g, t, stream, m, block_stride, lvl_row0, rows, heads, head_dim, tab);
    else launch((sink_rotate_kernel<false, 22>), g, t, stream, m, block_stride, lvl_row0, rows, heads, head_dim, tab);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rope_rows(const RopeJob& job, int rows, int hw, int heads, int head_dim, bool bf16,
                            int level_mode, const SinkTable& tab, hipStream_t stream) {
  RopeTensors r;
  int nt = 0;
  const void* srcs[3] = {job.src_k, job.src_v, job.src_q};
  void* dsts[3] = {job.dst_k, job.dst_v, job.dst_q};
  for (int i = 0; i < 3; ++i) {
    if ((srcs[i] == nullptr) != (dsts[i] == nullptr)) return hipErrorInvalidValue;
    if (!srcs[i]) continue;
    if ((reinterpret_cast<uintptr_t>(srcs[i]) | reinterpret_cast<uintptr_t>(dsts[i])) & 15u) return hipErrorInvalidValue;
    r.src[nt] = static_cast<const u32x4*>(srcs[i]);
    r.dst[nt] = static_cast<u32x4*>(dsts[i]);
    r.turn[nt] = i != 1;
    ++nt;
  }
  for (int i = nt; i < 3; ++i) {
    r.src[i] = nullptr;
    r.dst[i] = nullptr;
    r.turn[i] = 0;
  }
  if (nt == 0 || (level_mode != 1 && level_mode != 2)) return hipErrorInvalidValue;
  const int chunks = head_dim * (bf16 ? 2 : 4) / 16;
  const long long n = (long long)rows * heads * chunks;
  if (n == 0) return hipSuccess;
  if (3 * n >= (1LL << 31)) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((nt * n + kRopeThreads - 1) / kRopeThreads);
  const int lvl_op = level_mode == 1 ? kQuarter : kTurnQuarter;
  const dim3 g(grid), t(kRopeThreads);
  if (tab.n_planes == 12 && head_dim == 64) {
    if (bf16) launch((rope_rows_kernel<true, 12>), g, t, stream, r, (unsigned)n, nt, hw, heads, chunks, lvl_op, tab);
    else launch((rope_rows_kernel<false, 12>), g, t, stream, r, (unsigned)n, nt, hw, heads, chunks, lvl_op, tab);
  } else if (tab.n_planes == 22 && head_dim == 128) {
    if (bf16) launch((rope_rows_kernel<true, 22>), g, t, stream, r, (unsigned)n, nt, hw, heads, chunks, lvl_op, tab);
    else launch((rope_rows_kernel<false, 22>), g, t, stream, r, (unsigned)n, nt, hw, heads, chunks, lvl_op, tab);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sf
