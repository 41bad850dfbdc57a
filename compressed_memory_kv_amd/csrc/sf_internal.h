// Private interface between the host state machine (sf_host.cpp) and the
// gfx950 kernels (sf_copy.hip, sf_attn_bf16.hip, sf_attn_f32.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/sf.h"

namespace sf {

// Most sessions one attention launch covers; sf_attend splits larger batches.
constexpr int kMaxLaunchSessions = 16;
// Most key splits per (session, head, query tile); bounds the scratch region.
constexpr int kMaxSplit = 8;

// One session's share of a batched attention launch.  Device addresses.
struct AttnSession {
  const void* q;        // [rows][H][D] in the session dtype
  float* out;           // [rows][H][D] fp32
  const void* k;        // this block's K [C][H][D]
  const void* v;        // this block's V [C][H][D]
  float* part_o;        // [split][rows][H][D] fp32 partial numerators (split > 1)
  float* part_ml;       // [split][rows][H][2] fp32 (reference max in log2 units, row sum)
  int32_t rows;         // query rows (R)
  int32_t n_keys;       // readable rows
  int32_t n_seg;        // readable row segments (<= SF_MAX_SEGMENTS)
  int32_t split;        // key splits (1 = write out directly)
  int32_t qtiles;       // query tiles of this session
  int32_t unit_begin;   // first work unit of this session in the launch
  int32_t seg_begin[SF_MAX_SEGMENTS];
  int32_t seg_len[SF_MAX_SEGMENTS];
};

struct AttnLaunch {
  int32_t n_sessions;
  int32_t n_heads;
  int32_t head_dim;
  int32_t total_units;
  float scale_log2;     // softmax scale times log2(e)
  int32_t pad[3];
  AttnSession s[kMaxLaunchSessions];
};

// Query rows per workgroup of each attention kernel.
constexpr int kBf16RowsPerTile = 128;
constexpr int kF32RowsPerTile = 256;
// Keys per tile of the bf16 kernel (split boundaries are multiples of it).
constexpr int kBf16KeysPerTile = 64;

// Scratch bytes one session needs for split-key partial results.
size_t attend_scratch_bytes(int64_t rows, int n_heads, int head_dim);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_copy_rows(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                            size_t bytes, hipStream_t stream);
// Copies `bytes` from src_off to dst_off inside K and V of every block:
// block b's K starts at mem + b*block_stride, its V at that + v_offset.
hipError_t launch_evict(void* mem, int n_blocks, size_t block_stride, size_t v_offset,
                        size_t src_off, size_t dst_off, size_t bytes, hipStream_t stream);
hipError_t launch_attend_bf16(const AttnLaunch& a, hipStream_t stream);
hipError_t launch_attend_f32(const AttnLaunch& a, hipStream_t stream);
hipError_t launch_combine(const AttnLaunch& a, hipStream_t stream);

}  // namespace sf
