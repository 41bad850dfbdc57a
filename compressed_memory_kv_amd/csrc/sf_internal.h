// Private interface between the host state machine (sf_host.cpp) and the
// gfx950 kernels (sf_copy.hip, sf_rope.hip, sf_bias.hip, sf_attn.hip, sf_attn_sk.hip).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/sf.h"

namespace sf {

// Work-item and workgroup ids read straight from the hardware.  HIP's threadIdx and
// blockIdx go through device-library functions built with packed fp32 ops on; code built
// with them off cannot inline those (the callee's target features are not a subset of
// the caller's), so each use would be a real call: a stack, saved registers and spills.
__device__ __forceinline__ unsigned tid_x() { return __builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ unsigned wg_x() { return __builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ unsigned wg_y() { return __builtin_amdgcn_workgroup_id_y(); }

// Events that the next kernel launches of this thread have the dispatch itself stamp with
// its start and end (so they bracket the kernel alone, as a profiler's dispatch timestamps
// do); both NULL when tracing is off.  `launched` counts the launches made meanwhile.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
  int launched;
};
LaunchEvents& launch_events();

// Every kernel of the library is launched through here.
template <typename F, typename... Args>
inline void launch(F kernel, const dim3& grid, const dim3& block, hipStream_t stream, Args... args) {
  LaunchEvents& ev = launch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0, args...);
  if (hipPeekAtLastError() == hipSuccess) ++ev.launched;  // a failed launch stamps nothing
}

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
  const float* bias;    // recency bias per buffer row, log2 units, [H][bias_stride]; NULL: none
  int32_t bias_stride;  // rows per head in `bias` (the capacity C)
  int32_t pad_;
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

// ---- persistent stream-K attention (bf16, head_dim 64) ----------------------
// A unit is (session, head, 128-row query tile); a column is (session, head), the
// full 64-key tiles its units share.  The launch's work is the flattened sequence of
// (session, head, tile) column iterations; group g of workgroups takes the iterations
// between costs floor(g*T/NG) and floor((g+1)*T/NG) (see SkLaunch::piece_cost), each
// member of the group the same iterations for its own query tiles.  A unit whose tiles
// span several groups leaves one partial result per group ("piece") in its session's
// scratch; keys past the last full tile (the tail) leave one more, from the unit's tail
// workgroup (launched past the persistent ones, or on its own when the read has no full
// tile), in the unit's last slot; the combine kernel merges them.
constexpr int kSkRows = 128;        // query rows per unit
constexpr int kSkKeys = 64;         // keys per tile
constexpr int kSkMinRange = 8;      // fewest tiles of a column a group range starting inside it holds
constexpr int kSkWgPerCu = 2;       // persistent workgroups per CU
constexpr int kSkPieceCost = 7;     // a piece's fixed overhead, in tiles (tuned: 4, 5, 7, 9, 12 measured)
constexpr int kRecSlot = SF_MAX_SEGMENTS - 1;  // segment slot of a record read from its source
constexpr int kSkGrpTable = 384;    // most groups whose ranges the host tabulates
// Cost weight of a workgroup dispatched first on its CU over one dispatched second, minus
// one: the weighted cut the host tabulates gives the first 1 + skew/2, the second 1 - skew/2
// (measured at the served shape: 0 -> 42.6 us, 0.06 / 0.10 / 0.14 -> 43.0 / 42.2 / 41.9,
// 0.20 to 0.45 -> 40.5 to 41.4); one-session launches only (a batch of sessions measured
// slower weighted).
constexpr double kSkDispatchSkew = 0.20;
struct SkSession {
  const void* q;        // [rows][H][64] bf16
  float* out;           // [rows][H][64] fp32
  const void* k;        // this block's K [C][H][64]
  const void* v;        // this block's V [C][H][64]
  float* part_o;        // [units][ppu][kSkRows][64] unnormalised partial numerators
  float* part_ml;       // [units][ppu][kSkRows][2] (reference max in log2 units, row sum)
  // A record written by this launch (sf_step): its K/V are read from rec_k / rec_v
  // (segment slot kRecSlot, rows counted from the record's first row, keys last) while
  // they are copied into the buffer at row rec_row0 (see SkLaunch::rec_copy_idle).  rec_seg = kRecSlot
  // when present, -1 otherwise.  Unused segment slots have length 0.
  const void* rec_k;    // [rows][H][64] bf16
  const void* rec_v;
  int32_t rec_seg;
  int32_t rec_row0;
  int32_t rows;         // query rows (R)
  int32_t n_keys;       // readable rows
  int32_t n_seg;        // buffer segments in use (slots 0..n_seg-1)
  int32_t qtiles;       // ceil(rows / kSkRows)
  int32_t ntiles;       // full key tiles: n_keys / kSkKeys
  int32_t ppu;          // piece slots per unit in the scratch
  int32_t it_begin;     // first column iteration of this session in the launch
  int32_t cost_begin;   // first cost unit of this session (see SkLaunch::piece_cost)
  int32_t mult;         // units of a column one workgroup of a group takes: ceil(qtiles / grp_size)
  int32_t pad;
  int32_t seg_begin[SF_MAX_SEGMENTS];
  int32_t seg_len[SF_MAX_SEGMENTS];
};
struct SkLaunch {
  int32_t n_sessions;
  int32_t n_heads;
  int32_t n_wg;         // workgroups of the launch
  int32_t n_iters;      // N, column iterations
  float scale_log2;
  // Group ranges are cut in cost units: a column of ntiles full tiles costs
  // mult * (ntiles + piece_cost) (piece_cost: a piece's overhead, in tiles; mult: the
  // units of the column one member takes), a column without full tiles 0; total_cost = T.
  // Tile t of a column sits at cost mult * (piece_cost + t) from the column's start, and
  // group g starts at the first tile at or past cost floor(g*T/NG).
  int32_t piece_cost;
  int32_t total_cost;
  // The tail and combine kernels take a unit on the XCD whose workgroups produced its
  // pieces (xcd_map = 1), so the partials are read from that XCD's L2: workgroup g serves
  // units xcd_first[g & 7] .. xcd_first[(g & 7) + 1] - 1, xcd_per per XCD at most.
  int32_t xcd_map;
  int32_t xcd_per;
  int32_t xcd_first[9];
  // Groups: grp_size workgroups take the same key ranges, one query tile each (tile qt of
  // a column goes to member qt mod grp_size), so a K/V tile is fetched once for the group.
  // n_grp groups; the ranges above are cut per group (n_grp takes the place of G).  With
  // grp_per_xcd > 0 each XCD holds grp_per_xcd whole groups (logical workgroups of an XCD
  // past them take no work); 0: group g is logical workgroups g*grp_size ...
  int32_t n_grp;
  int32_t grp_size;
  int32_t grp_per_xcd;
  // 1 when (T + 1) * NG < 2^31: the range and group formulas then fit 32-bit arithmetic
  // (64-bit divisions cost about 0.7 us at the start of a served read).
  int32_t narrow;
  // 1: the record of a one-session sf_step launch is copied into its buffer rows by the
  // attention kernel's workgroups past the XCDs' whole groups (which have no attention
  // work), while the others read; 0: by combine_sk_kernel.
  int32_t rec_copy_idle;
  // grp_table = 1: entry g of grp_first is group g's first iteration (low 24 bits) and
  // the piece slot of its first piece (high 8 bits), for g <= n_grp (entry n_grp: N), as
  // the formulas above give them; every later piece of a group starts its column, slot 0.
  // The host fills it when n_grp <= kSkGrpTable, N < 2^24 and every slot < 128: the
  // kernel's start-up is bound by the scalar unit, which its CU's 8 waves share.
  int32_t grp_table;
  // H * qtiles when every session of the launch has the same number of query tiles (their
  // units then split evenly: unit ug is unit ug % uni_units of session ug / uni_units),
  // else 0 (the sessions are walked).
  int32_t uni_units;
  // Units whose tails the attention launch takes itself, in workgroups past its n_wg (the
  // launch's units when any session has a tail and the launch has full tiles), else 0.
  int32_t tail_units;
  SkSession s[kMaxLaunchSessions];
  int32_t grp_first[kSkGrpTable + 1];
};
static_assert(sizeof(SkLaunch) <= 4000, "kernel arguments stay under the 4 KB limit");
// Piece slots per unit a session of capacity C needs (bounded because a group range
// that starts inside a column holds at least kSkMinRange of its tiles).
int32_t sk_pieces_per_unit(int64_t capacity_rows);
size_t sk_scratch_bytes(int64_t rows, int n_heads, int64_t capacity_rows);
hipError_t launch_attend_sk(const SkLaunch& a, hipStream_t stream);
hipError_t launch_tail_sk(const SkLaunch& a, int total_units, hipStream_t stream);
hipError_t launch_combine_sk(const SkLaunch& a, int total_units, hipStream_t stream);

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
hipError_t launch_lds_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_evict(void* mem, int n_blocks, size_t block_stride, size_t v_offset,
                        size_t src_off, size_t dst_off, size_t bytes, hipStream_t stream);
// Rotary tables: the first n_planes (dims 2i, 2i+1) planes of a head turn by the angle
// with cosine c[i] and sine s[i].
constexpr int kSinkMaxPlanes = 32;
struct SinkTable {
  int32_t n_planes;
  int32_t pad;
  float c[kSinkMaxPlanes];
  float s[kSinkMaxPlanes];
};
// Streaming sink: turns those planes of every head of the first `rows` K rows of every
// block (K of block b at mem + b*block_stride), in place.  Rows from lvl_row0 on keep
// their two slowest planes.
hipError_t launch_sink_rotate(void* mem, int n_blocks, size_t block_stride, int lvl_row0, int rows, int heads,
                              int head_dim, bool bf16, const SinkTable& tab, hipStream_t stream);
// Rotating write: each present tensor of `rows` rows [heads][head_dim] moved from src to
// dst; K and Q with their temporal planes turned (summary rows, from hw on, take the level
// planes: level_mode 1 = the quarter turn of the input, 2 = turned then the quarter turn),
// V as it is.  A tensor is absent when both its pointers are NULL.  16-byte aligned
// pointers; a dst may equal its src.  One launch.
struct RopeJob {
  void* dst_k;
  void* dst_v;
  void* dst_q;
  const void* src_k;
  const void* src_v;
  const void* src_q;
};
hipError_t launch_rope_rows(const RopeJob& job, int rows, int hw, int heads, int head_dim, bool bf16,
                            int level_mode, const SinkTable& tab, hipStream_t stream);
// Recency bias: copies a caller's table [heads][w+1] (n floats) into the session memory.
hipError_t launch_bias_table(float* dst, const float* src, int n, hipStream_t stream);
// Recency bias per buffer row at frame t: dst[h][row] = log2(e) * tab[h][age] for a
// summary row of a generated frame (age = t - its frame, from the slot formulas), 0 for raw
// rows and for Z0; values below -1e30 are raised to it.
struct BiasGeo {
  int32_t rows;      // R
  int32_t hw;
  int32_t x;
  int32_t y;
  int32_t w;
  int32_t heads;
  int32_t capacity;  // C
  int32_t pad;
  int64_t t;
};
hipError_t launch_bias_rows(float* dst, const float* tab, const BiasGeo& g, hipStream_t stream);
// Workgroups of the bf16 split-key kernel that fit on one compute unit at once.
int attend_bf16_wgs_per_cu(int head_dim, bool bias);
// bias: any session has a recency bias (kernels that read AttnSession::bias).
hipError_t launch_attend_bf16(const AttnLaunch& a, bool bias, hipStream_t stream);
hipError_t launch_attend_f32(const AttnLaunch& a, bool bias, hipStream_t stream);
hipError_t launch_combine(const AttnLaunch& a, hipStream_t stream);

}  // namespace sf
