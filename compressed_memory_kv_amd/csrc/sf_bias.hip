// Recency bias on summary keys: the table copy and the per-row biases of a frame.
//
// Model card "GTA world model: weights and inference code": the section "Files" lists an
// optional recency bias on summary keys, and "Credits" says it follows a paper the page
// does not reproduce.  It is taken here as a term added to the scaled scores of summary
// keys that depends on the head and on the age of the key's frame; the caller sets its
// values as a table over ages 0 .. W.  The attention kernels read one fp32 value per
// buffer row and head (log2 units, as their scores are), rebuilt here once per frame from
// the slot formulas of section "One buffer, no mask":
//   RAW slot s holds the frame f <= t with f = s mod (Y+1): age (t - s) mod (Y+1);
//   SUM slot u holds the frame f <= t-Y-1 with f = u mod (W-Y): age Y+1 + (t-Y-1-u) mod (W-Y).
// Only summary rows (record rows from hw on) of RAW and SUM slots take it; Z0 (the start
// image) and raw rows take 0.  A row whose slot is empty is never read.
#include "sf_internal.h"

namespace sf {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kBiasFloor = -1e30f;  // below this a key's weight is exactly 0 in fp32 anyway

__global__ __launch_bounds__(kThreads) void bias_table_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                              int n) {
  const int i = (int)(wg_x() * kThreads + tid_x());
  if (i < n) dst[i] = src[i];
}

__device__ __forceinline__ int64_t pos_mod(int64_t a, int64_t m) {
  const int64_t r = a % m;
  return r < 0 ? r + m : r;
}

__global__ __launch_bounds__(kThreads) void bias_rows_kernel(float* __restrict__ dst, const float* __restrict__ tab,
                                                             const BiasGeo g) {
  const int row = (int)(wg_x() * kThreads + tid_x());
  const int h = (int)wg_y();
  if (row >= g.capacity) return;
  const int sum0 = g.rows * (g.y + 2);
  int age = -1;
  if (row >= sum0) {
    const int u = (row - sum0) / g.x;
    age = g.y + 1 + (int)pos_mod(g.t - g.y - 1 - u, g.w - g.y);
  } else if (row >= g.rows) {
    const int s = (row - g.rows) / g.rows;
    const int within = row - g.rows * (1 + s);
    if (within >= g.hw) age = (int)pos_mod(g.t - s, g.y + 1);
  }
  float b = 0.0f;
  if (age >= 0) {
    b = tab[(size_t)h * (g.w + 1) + age] * kLog2e;
    b = b < kBiasFloor ? kBiasFloor : b;
  }
  dst[(size_t)h * g.capacity + row] = b;
}

}  // namespace

hipError_t launch_bias_table(float* dst, const float* src, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  launch(bias_table_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), stream, dst, src, n);
  return hipGetLastError();
}

hipError_t launch_bias_rows(float* dst, const float* tab, const BiasGeo& g, hipStream_t stream) {
  if (g.capacity <= 0 || g.heads <= 0) return hipSuccess;
  if (g.heads > 65535) return hipErrorInvalidValue;
  launch(bias_rows_kernel, dim3((g.capacity + kThreads - 1) / kThreads, g.heads), dim3(kThreads), stream, dst, tab,
         g);
  return hipGetLastError();
}

}  // namespace sf
