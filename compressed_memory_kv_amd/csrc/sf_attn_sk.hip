// The dense read of the per-block memory, head_dim 64, bf16, as a persistent
// stream-K kernel for gfx950.
//
// Model card "GTA world model: weights and inference code", sections "What a
// frame attends to" and "One buffer, no mask": every row of frame t's record
// attends, with no mask, to every filled row of the block's K/V buffer:
//     O[i,h] = sum_j softmax_j(scale * <Q[i,h], K[j,h]>) V[j,h]
// The filled rows are at most a few contiguous segments; the kernels walk them
// as one flattened key sequence (addressing, not masking).
//
// Work decomposition.  A unit is (session, head, 128-row query tile).  Its keys
// are floor(keys/64) full 64-key tiles plus, when keys is not a multiple of 64,
// a tail of fewer than 64 keys.  The units of one (session, head), a "column", share
// those tiles.
//   attn_sk_kernel: persistent 4-wave workgroups, two per CU, form groups of as
//     many members as a session has query tiles (9 at 1104 rows), each XCD holding
//     whole groups (the hardware deals workgroups round robin over the 8 XCDs, and
//     the grid is remapped so each XCD owns a contiguous eighth).  The full tiles of
//     all columns of the launch, in order, are cut into one contiguous range per
//     group; every member walks the group's range for its own query tile, so the
//     members read each K/V tile at about the same time and it comes from HBM once
//     (the rest from the XCD's L2), at the start of a range too.  The cut is made in
//     cost units: a column costs its tiles plus a fixed charge for its piece overhead
//     (prologue and stream merge: seven tiles, the best of the charges measured), so
//     a range that crosses into another column holds fewer tiles and every group
//     finishes at about the same time.  The part of a unit inside one group's range
//     is a "piece"; a piece that is the whole unit (and the unit has no tail) writes
//     the output, otherwise it writes an unnormalised partial (O, reference max, row
//     sum) to the session's scratch.  The column's last piece marks the unit's piece
//     slots past its own as empty (reference -inf), and a whole unit marks slot 0
//     (+inf), so the combine needs no count of a unit's pieces.  Workgroups past the
//     persistent ones, one per unit, read the units' tails (a unit's last scratch
//     slot): the hardware dispatches them as attention workgroups finish;
//   attn_tail_kernel: the same tail workgroups as a launch of their own, for reads
//     without a full tile (no attention launch to ride on);
//   combine_sk_kernel: merges every piece slot and the tail of each unit that is not
//     marked whole.
// sf_step launches fold the record write in: the attention kernels read the new
// record's keys from the caller's K/V (segment slot kRecSlot, after the buffer's
// keys) and copy the record into the buffer meanwhile with the workgroups past the XCDs'
// whole groups, which have no attention work (combine_sk_kernel makes the copy when a
// launch has none).
//
// Inside a workgroup of attn_sk_kernel.  Four waves = two key streams x two waves;
// the piece's tiles are cut into two contiguous halves, one per stream.  The two
// waves of a stream hold 64 query rows each (two 32-row MFMA blocks), so every K/V
// operand read from LDS feeds two MFMAs.  K and V tiles go from global memory
// straight into LDS (buffer_load_dwordx4 ... lds: a scalar tile offset plus a lane
// offset fixed for the piece, no staging VGPRs and no VALU address arithmetic),
// double buffered.  Two such workgroups share a CU (256 VGPRs per wave, 2 waves per
// SIMD): one's prologue and merge overlap the other's main loop.  The instruction
// arbiter favours the wave dispatched first, which would leave the later workgroup
// of a CU running alone at the end of the launch; each wave therefore sets its
// priority from its workgroup's progress (3 in the first quarter of its range down
// to 0 in the last), so the workgroup that is behind wins the arbiter.
//
// Softmax with a fixed reference.  Each stream takes one reference per query,
// the max of the scores of its first 32 keys, and keeps it: p = exp2(s*c - mref) may
// exceed 1 but no rescaling of O is ever needed inside the loop, which is
// therefore branch-free.  A lane's largest quarter sum is tracked; if in some
// stream of the workgroup a p could have exceeded 2^40 (or overflowed), the
// workgroup redoes the piece with the exact max over each stream's keys, where
// every p is at most 1.  Exact softmax either way, up to rounding.
//
// Per 64-key tile and wave: four "quarters" (32-key half h, 32-query block qb),
//   S^T (32 keys x 32 queries) = K . Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows
//     from LDS, B = Q in VGPRs): each lane owns one query and 16 of its scores;
//   P = exp2(S * scale*log2e - mref) in fp32, rounded to bf16 (nearest even); the
//     row sum adds the fp32 values;
//   O^T (64 x 32 queries) += V^T . P^T on the same MFMA; V^T comes from the
//     row-major V tile through ds_read_b64_tr_b16.
// The quarters are software pipelined across tiles: in each region the matrix
// core computes one quarter's S^T and an earlier quarter's O^T while the VALU does
// the softmax of a quarter whose S^T is already there.
#include "sf_internal.h"

#include <cmath>

namespace sf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int D = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kStreams = 2;
constexpr int BN = kSkKeys;                           // 64 keys per tile
constexpr int ROW = 2 * D;                            // bytes per K/V row
constexpr int TILE = BN * ROW;                        // 8 KB
constexpr int STAGE = 2 * TILE;                       // K tile then V tile
constexpr int STAGE_ALL = kStreams * STAGE;           // one stage of every stream (32 KB)
constexpr int DMA_ROWS = 8;                           // rows one wave-wide 1 KB transfer covers
constexpr int DMA_PER_WAVE = BN / DMA_ROWS / 2;       // transfers per wave per tensor per tile (4)
constexpr float kOverflowSum = 0x1p40f;               // a lane quarter sum above this asks for exact maxima
// Stream merge: the wave of stream s with query rows hw leaves the other stream the d block
// that one finishes, in stage array hw at slot s (64 lanes x XCHG_FLOATS floats each).
constexpr int XCHG_FLOATS = 36;  // per lane: one d block of both query blocks (32), references, sums
static_assert(kStreams * 64 * XCHG_FLOATS * 4 <= STAGE_ALL, "both streams' exchange slots fit in one stage array");
static_assert(BN == 64, "a tile is two 32-key MFMA blocks");

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Issue priority from the workgroup's progress through its range: 3 in the first quarter
// down to 0 in the last.  The workgroups sharing a CU then stay level with each other:
// the one that is behind wins the instruction arbiter (which otherwise favours the wave
// dispatched first), so neither ends up running alone at the end of the launch.
__device__ __forceinline__ void progress_priority(const int done, const int total) {
  const int q = (4 * done) / total;
  if (q <= 0) __builtin_amdgcn_s_setprio(3);
  else if (q == 1) __builtin_amdgcn_s_setprio(2);
  else if (q == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// p as a wave-uniform value (scalar registers).
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
}

// Raw buffer resource from p with no range limit (gfx9 family dword3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const char* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, -1, 0x00020000);
}

__device__ __forceinline__ int session_of_iter(const SkLaunch& a, int it) {
  int si = 0;
  for (int i = 1; i < a.n_sessions; ++i)
    if (a.s[i].it_begin <= it) si = i;
  return __builtin_amdgcn_readfirstlane(si);
}

// Group ranges are cut in cost units: a column costs mult * (piece_cost + its tiles), and
// tile t of a column sits at cost mult * (piece_cost + t) from the column's start.  Group
// g starts at the first tile at or past cost floor(g*T/NG).
// I: the integer type the formulas run in (unsigned when SkLaunch::narrow holds; each
// kernel that uses them is built for both and the launch picks one).
template <typename I>
__device__ __forceinline__ int range_start_t(const SkLaunch& a, const int g) {
  const I C = (I)g * (I)a.total_cost / (I)a.n_grp;
  int si = 0;
  for (int i = 0; i < a.n_sessions; ++i)
    if (a.s[i].ntiles > 0 && (I)a.s[i].cost_begin <= C) si = i;
  si = __builtin_amdgcn_readfirstlane(si);
  const SkSession& S = a.s[si];
  const I m = (I)S.mult;
  const I per = m * (I)(S.ntiles + a.piece_cost);
  const I r0 = C - (I)S.cost_begin;
  const I col = r0 / per;
  const int t = (int)((r0 - col * per + m - 1) / m) - a.piece_cost;
  return (int)(S.it_begin + (int)col * S.ntiles + (t > 0 ? t : 0));
}
template <typename I>
__device__ __forceinline__ int range_start(const SkLaunch& a, const int g) {
  return g >= a.n_grp ? a.n_iters : range_start_t<I>(a, g);
}

// Group holding column iteration i: the last g whose range starts at or before it.
template <typename I>
__device__ __forceinline__ int grp_of_iter(const SkLaunch& a, const int i) {
  const SkSession& S = a.s[session_of_iter(a, i)];
  const int local = i - S.it_begin;
  const int col = local / S.ntiles;
  const I m = (I)S.mult;
  const I X = (I)S.cost_begin + (I)col * m * (I)(S.ntiles + a.piece_cost) +
              m * (I)(a.piece_cost + (local - col * S.ntiles));
  return (int)(((X + 1) * (I)a.n_grp - 1) / (I)a.total_cost);
}

// Session and unit of a unit index counted over the whole launch.
__device__ __forceinline__ void decode_unit(const SkLaunch& a, int ug, int& si, int& u) {
  if (a.uni_units > 0) {  // sessions of equal size: no walk (one dependent load per session)
    si = __builtin_amdgcn_readfirstlane(ug / a.uni_units);
    u = __builtin_amdgcn_readfirstlane(ug - si * a.uni_units);
    return;
  }
  int s = 0, base = 0, acc = 0;
  for (int i = 0; i < a.n_sessions; ++i) {
    if (ug >= acc) {
      s = i;
      base = acc;
    }
    acc += a.n_heads * a.s[i].qtiles;
  }
  si = __builtin_amdgcn_readfirstlane(s);
  u = __builtin_amdgcn_readfirstlane(ug - base);
}

// Row of flattened key kappa (segments in ascending key order) and its segment.  The
// row counts in the buffer, or in the source of the record written by this launch for
// that record's segment.
__device__ __forceinline__ int key_row(const int* seg_row, const int* seg_key, int kappa, int& seg) {
  int row = seg_row[0] + kappa;
  seg = 0;
#pragma unroll
  for (int i = 1; i < SF_MAX_SEGMENTS; ++i) {
    const bool in = kappa >= seg_key[i];
    row = in ? seg_row[i] + (kappa - seg_key[i]) : row;
    seg = in ? i : seg;
  }
  return row;
}

// Segment i covers keys [seg_key[i], seg_key[i] + seg_len[i]) in slot order; an empty
// slot starts where the next one does, so a lookup of the last slot whose start is at
// or below a key never lands on it.  REC: the last slot holds the record's rows, which
// are read from the caller's record (row 0 = its first row).
template <bool REC>
__device__ __forceinline__ void seg_tables(const SkSession& S, int* seg_row, int* seg_key) {
  int cum = 0;
#pragma unroll
  for (int i = 0; i < SF_MAX_SEGMENTS; ++i) {
    seg_row[i] = (REC && i == kRecSlot) ? 0 : S.seg_begin[i];
    seg_key[i] = cum;
    cum += S.seg_len[i];
  }
}

// ---- MFMA building blocks shared by both attention kernels ---------------------------
// S^T of a quarter: 4 MFMA over the head dimension (A = K rows from LDS, B = Q^T).
#define SK_QK(SD, KOP, QOP)                                                               \
  SD = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KOP[0], QOP[0], zero16, 0, 0, 0);          \
  SD = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KOP[1], QOP[1], SD, 0, 0, 0);              \
  SD = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KOP[2], QOP[2], SD, 0, 0, 0);              \
  SD = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KOP[3], QOP[3], SD, 0, 0, 0);
// O^T += V^T . P^T of a quarter: 2 key steps of 16 x 2 d blocks.
#define SK_PV(O0, O1, VOP, P)                                                             \
  O0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VOP[0], P[0], O0, 0, 0, 0);                \
  O1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VOP[1], P[0], O1, 0, 0, 0);                \
  O0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VOP[2], P[1], O0, 0, 0, 0);                \
  O1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VOP[3], P[1], O1, 0, 0, 0);
// LDS operands of 32 keys starting at row R0 of a stage: K rows (A of S^T) and V^T
// (A of O^T; entry 2*j + db for key step j and d block db).
#define SK_LOAD_K(KOP, ST, R0)                                                            \
  _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) KOP[kk] =                              \
      *reinterpret_cast<const bf16x8*>((ST) + kaddr[kk] + (R0) * ROW);
#define SK_LOAD_V(VOP, ST, R0)                                                            \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                         \
    _Pragma("unroll") for (int db = 0; db < 2; ++db) {                                    \
      const char* vp_ = (ST) + vaddr[db] + ((R0) + 16 * j) * ROW;                         \
      const i16x4 va_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp_));       \
      const i16x4 vb_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp_ + 8 * ROW)); \
      VOP[2 * j + db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va_, vb_, 0, 1, 2, 3, 4, 5, 6, 7)); \
    }                                                                                     \
  }
// Lane addresses of those operands inside a stage (K chunk c of row r at c ^ ((r >> 1) & 7),
// V chunk c at c ^ 2*(r & 3): conflict-free reads).  A 128-byte row is half a line of the
// 64 LDS banks, so the 16 lanes a b128 read serves per cycle (rows r .. r+15, one chunk
// each) cover all 64 banks only if rows of the same parity differ in their swizzle: r >> 1.
#define SK_OPERAND_ADDRESSES(BASE)                                                        \
  int kaddr[4];                                                                           \
  _Pragma("unroll") for (int kk = 0; kk < 4; ++kk) kaddr[kk] =                            \
      (BASE) + l32 * ROW + (((2 * kk + g) ^ ((l32 >> 1) & 7)) << 4);                      \
  int vaddr[2];                                                                           \
  {                                                                                       \
    const int trow_ = (lane >> 2) & 3;                                                    \
    _Pragma("unroll") for (int db = 0; db < 2; ++db) {                                    \
      const int chunk_ = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);              \
      vaddr[db] = (BASE) + TILE + (4 * g + trow_) * ROW + ((chunk_ ^ (2 * trow_)) << 4) + 8 * (lane & 1); \
    }                                                                                     \
  }

// The record of a one-session launch copied into its buffer rows (K then V, 16-byte
// chunks): share j of n workgroups, kCopyBatch loads in flight per lane before their stores.
constexpr int kCopyBatch = 16;
__device__ __forceinline__ void copy_record_share(const SkLaunch& a, const int j, const int n) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const SkSession& S0 = a.s[0];
  const int n16 = S0.rows * a.n_heads * D * 2 / 16;  // chunks per tensor
  const size_t dst0 = (size_t)S0.rec_row0 * a.n_heads * D * 2 / 16;
  const u32x4* __restrict__ sk = reinterpret_cast<const u32x4*>(S0.rec_k);
  const u32x4* __restrict__ sv = reinterpret_cast<const u32x4*>(S0.rec_v);
  u32x4* __restrict__ dk = reinterpret_cast<u32x4*>(const_cast<void*>(S0.k)) + dst0;
  u32x4* __restrict__ dv = reinterpret_cast<u32x4*>(const_cast<void*>(S0.v)) + dst0;
  const int stride = n * kThreads;
  for (int i0 = j * kThreads + (int)tid_x(); i0 < 2 * n16; i0 += stride * kCopyBatch) {
    u32x4 x[kCopyBatch];
#pragma unroll
    for (int b = 0; b < kCopyBatch; ++b) {
      const int i = i0 + b * stride;
      if (i < 2 * n16) x[b] = __builtin_nontemporal_load(i < n16 ? sk + i : sv + (i - n16));
    }
#pragma unroll
    for (int b = 0; b < kCopyBatch; ++b) {
      const int i = i0 + b * stride;
      if (i < 2 * n16) __builtin_nontemporal_store(x[b], i < n16 ? dk + i : dv + (i - n16));
    }
  }
}

// The lane's index, computed where it is used (volatile: never hoisted or kept live
// across the main loop, where every register counts).
__device__ __forceinline__ int fresh_lane() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// The tail of every unit whose key count is not a multiple of 64: the last keys % 64
// keys, exact softmax over them (one tile, so the reference is the true max), written as
// a partial to the unit's last scratch slot.  One workgroup per unit of the launch; wave
// w holds query rows 32*w .. 32*w+31 of the unit.
constexpr int kTailWaves = 4;
// Unit (launch numbering) and part of a tail or combine workgroup: by the unit's producing
// XCD when the launch maps them (the hardware deals workgroup g to XCD g mod 8), else in
// order.  False: no unit for this workgroup.
__device__ __forceinline__ bool unit_of_wg(const SkLaunch& a, int total_units, int split, int& ug, int& part) {
  if (a.xcd_map) {
    const int x = (int)(wg_x() & 7u), j = (int)(wg_x() >> 3);
    ug = a.xcd_first[x] + j / split;
    part = j % split;
    return ug < a.xcd_first[x + 1];
  }
  ug = (int)wg_x() / split;
  part = (int)wg_x() % split;
  return ug < total_units;
}

// The tail of unit ug (launch numbering) by one 4-wave workgroup, staging in st (STAGE bytes).
__device__ __forceinline__ void tail_unit(const SkLaunch& a, const int ug, char* st) {
  int si, u;
  decode_unit(a, ug, si, u);
  const SkSession& S = a.s[si];
  const int nk = S.n_keys & (BN - 1);
  if (nk == 0) return;  // no tail: uniform over the workgroup
  const int key0 = S.n_keys - nk;
  const int H = a.n_heads;
  const float c = a.scale_log2;
  const int qt = u % S.qtiles, h = u / S.qtiles;
  const int tid = tid_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int row_stride = H * D;
  const int row_bytes = 2 * row_stride;
  int seg_row[SF_MAX_SEGMENTS], seg_key[SF_MAX_SEGMENTS];
  seg_tables<false>(S, seg_row, seg_key);

  // the 64-row tile of keys key0 .. key0+63 (past the last key: its row again), wave w
  // moving rows 8w .. 8w+7 and 32+8w .. 32+8w+7 of K and of V (one K chunk per lane for both)
  {
    const int drow = lane >> 3;
    const int kchunk = (lane & 7) ^ (((wave & 1) << 2) | (drow >> 1));
    const int vchunk = (lane & 7) ^ (2 * (drow & 3));
    const char* kg = reinterpret_cast<const char*>(S.k) + 2 * h * D;
    const char* vg = reinterpret_cast<const char*>(S.v) + 2 * h * D;
    const char* krec = reinterpret_cast<const char*>(S.rec_k) + 2 * h * D;
    const char* vrec = reinterpret_cast<const char*>(S.rec_v) + 2 * h * D;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int trow = 8 * wave + 32 * m;
      const int kappa = min(key0 + trow + drow, S.n_keys - 1);
      int sg;
      const unsigned rb = (unsigned)(key_row(seg_row, seg_key, kappa, sg) * row_bytes);
      const char* kb = (S.rec_seg >= 0 && sg == kRecSlot) ? krec : kg;
      const char* vb = (S.rec_seg >= 0 && sg == kRecSlot) ? vrec : vg;
      __builtin_amdgcn_global_load_lds(kb + rb + kchunk * 16, (lds_void*)(st + trow * ROW), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vb + rb + vchunk * 16, (lds_void*)(st + TILE + trow * ROW), 16, 0, 0);
    }
  }
  bf16x8 qop[4];
  const int qrow = qt * kSkRows + 32 * wave + l32;
  {
    const int r = min(qrow, S.rows - 1);
    const __bf16* qp = reinterpret_cast<const __bf16*>(S.q) + r * row_stride + h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qop[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
  }
  __syncthreads();

  SK_OPERAND_ADDRESSES(0);
  const f32x16 zero16 = {};
  f32x16 s[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    bf16x8 kop[4];
    SK_LOAD_K(kop, st, 32 * hh);
    SK_QK(s[hh], kop, qop);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * hh + 8 * (r >> 2) + 4 * g + (r & 3);
      if (key >= nk) s[hh][r] = -INFINITY;
    }
  }
  float mt = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; r += 2) mt = max3(mt, max3(s[0][r], s[0][r + 1], s[1][r]), s[1][r + 1]);
  const float mref = fmaxf(mt, xor32(mt)) * c;  // key 0 of the tail is real, so this is finite
  f32x16 oa = zero16, ob = zero16;
  float l = 0.0f;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    bf16x8 vop[4], p[2];
    SK_LOAD_V(vop, st, 32 * hh);
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hh][8 * b + r], c, -mref));
        p[b][r] = (__bf16)e;
        l += e;
      }
    SK_PV(oa, ob, vop, p);
  }
  const float lt = l + xor32(l);
  if (qrow < S.rows) {
    const size_t slot = (size_t)u * S.ppu + (S.ppu - 1);
    const int rin = qrow - qt * kSkRows;
    float* po = S.part_o + (slot * kSkRows + rin) * D;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      *reinterpret_cast<float4*>(po + 8 * q4 + 4 * g) = make_float4(oa[4 * q4], oa[4 * q4 + 1], oa[4 * q4 + 2], oa[4 * q4 + 3]);
      *reinterpret_cast<float4*>(po + 32 + 8 * q4 + 4 * g) =
          make_float4(ob[4 * q4], ob[4 * q4 + 1], ob[4 * q4 + 2], ob[4 * q4 + 3]);
    }
    if (g == 0) *reinterpret_cast<float2*>(S.part_ml + (slot * kSkRows + rin) * 2) = make_float2(mref, lt);
  }
}

template <bool REC, typename I>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_sk_kernel(const SkLaunch a) {
  __shared__ __attribute__((aligned(16))) char st_a[STAGE_ALL];  // stage 0 of each stream
  __shared__ __attribute__((aligned(16))) char st_b[STAGE_ALL];  // stage 1 of each stream
  __shared__ int redo[kWaves];
  // Workgroups past the attention's (SkLaunch::tail_units of them) take the units' tails:
  // dispatched as attention workgroups finish, they fill the compute units the early
  // finishers leave.
  if ((int)wg_x() >= a.n_wg) {
    tail_unit(a, (int)wg_x() - a.n_wg, st_a);
    return;
  }
  const int G = a.n_wg;
  const int w = (G & 7) == 0 ? (int)(wg_x() & 7u) * (G >> 3) + (int)(wg_x() >> 3) : (int)wg_x();
  // group and member of this workgroup
  const int GS = a.grp_size;
  int grp, mem;
  if (a.grp_per_xcd > 0) {
    const int per = G >> 3, x = w / per, lw = w - x * per;
    const int busy = a.grp_per_xcd * GS;
    if (lw >= busy) {  // past the XCD's whole groups: no attention work
      if (REC && a.rec_copy_idle) copy_record_share(a, x * (per - busy) + (lw - busy), 8 * (per - busy));
      return;
    }
    grp = x * a.grp_per_xcd + lw / GS;
    mem = lw % GS;
  } else {
    grp = w / GS;
    mem = w - grp * GS;
    if (grp >= a.n_grp) return;
  }
  grp = __builtin_amdgcn_readfirstlane(grp);
  mem = __builtin_amdgcn_readfirstlane(mem);
  int it_lo, it_hi, k_first;  // this group's iterations [it_lo, it_hi), its first piece's slot
  if (a.grp_table) {
    const int e0 = a.grp_first[grp], e1 = a.grp_first[grp + 1];
    it_lo = e0 & 0xffffff;
    k_first = e0 >> 24;
    it_hi = e1 & 0xffffff;
  } else {
    it_lo = range_start<I>(a, grp);
    it_hi = range_start<I>(a, grp + 1);
    k_first = -1;
  }
  it_lo = __builtin_amdgcn_readfirstlane(it_lo);
  it_hi = __builtin_amdgcn_readfirstlane(it_hi);
  k_first = __builtin_amdgcn_readfirstlane(k_first);
  const int H = a.n_heads;
  const float c = a.scale_log2;

  const int tid = tid_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int stream = wave >> 1;   // key stream
  const int hw = wave & 1;        // which 64 query rows of the unit
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int soff = stream * STAGE;  // this stream's stage within a stage array

  // A wave-wide transfer fills 1 KB = 8 rows of a stage, lane L landing at row L/8,
  // position L%8, so lane L fetches the logical chunk that belongs there (both
  // swizzles are involutions).  The two waves of a stream take alternate 8-row groups
  // (wave hw: rows 8*hw + 16*m + 0..7), so every transfer of a wave starts at a row
  // with the same (row >> 1) & 4 and the same V phase: one K chunk and one V chunk per
  // lane for all of them.
  const int drow = lane >> 3;
  const int kchunk = (lane & 7) ^ ((hw << 2) | (drow >> 1));
  const int vchunk = (lane & 7) ^ (2 * (drow & 3));
  const int trow0 = hw * DMA_ROWS + drow;  // tile row of transfer 0; transfer m adds 16 m
  SK_OPERAND_ADDRESSES(soff);
  const f32x16 zero16 = {};

  // Q^T operands of query tile qt of head h: query block qb holds rows qrow0 + 32*qb +
  // l32 (rows past R read row R-1).  The next piece's are loaded as soon as the current
  // piece's last S^T is done, so their latency hides behind the merge.
  bf16x8 q0[4], q1[4];
  auto load_q = [&](const SkSession& S, const int h, const int qt) {
    const int qrow0 = qt * kSkRows + hw * 64;
    const int r0 = min(qrow0 + l32, S.rows - 1);
    const int r1 = min(qrow0 + 32 + l32, S.rows - 1);
    const __bf16* qp0 = reinterpret_cast<const __bf16*>(S.q) + r0 * H * D + h * D + 8 * g;
    const __bf16* qp1 = reinterpret_cast<const __bf16*>(S.q) + r1 * H * D + h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      q0[kk] = *reinterpret_cast<const bf16x8*>(qp0 + 16 * kk);
      q1[kk] = *reinterpret_cast<const bf16x8*>(qp1 + 16 * kk);
    }
  };
  // The first query tile this member takes in column iteration it (none: qtiles or more).
  auto first_q = [&](const int it, int& qh) {
    const SkSession& S = a.s[session_of_iter(a, it)];
    qh = __builtin_amdgcn_readfirstlane((it - S.it_begin) / S.ntiles);
    return mem < S.qtiles;
  };
  bool q_ok = false;  // q0 / q1 hold the Q of the next piece
  if (it_lo < it_hi) {
    int qh;
    if (first_q(it_lo, qh)) {
      load_q(a.s[session_of_iter(a, it_lo)], qh, mem);
      q_ok = true;
    }
  }

  for (int it = it_lo; it < it_hi;) {
    // ---- a column piece: tiles [tile0, tile1) of head h inside this group's range, for
    // each of this member's query tiles
    const int si = session_of_iter(a, it);
    const SkSession& S = a.s[si];
    const int nt = S.ntiles;
    const int local = it - S.it_begin;
    const int h = __builtin_amdgcn_readfirstlane(local / nt);
    const int tile0 = __builtin_amdgcn_readfirstlane(local - h * nt);
    const int tile1 = min(nt, tile0 + (it_hi - it));
    const int n = tile1 - tile0;
    const int s_lo = tile0 + (stream * n) / kStreams;   // this stream's tiles [s_lo, s_hi)
    const int s_hi = tile0 + ((stream + 1) * n) / kStreams;
    const int steps = (n + kStreams - 1) / kStreams;
    const int row_stride = H * D;
    const int row_bytes = 2 * row_stride;

    int seg_row[SF_MAX_SEGMENTS], seg_key[SF_MAX_SEGMENTS];
    seg_tables<REC>(S, seg_row, seg_key);

    // Buffer resources over the head's K and V (and the record's source): a transfer is a
    // scalar tile offset plus a lane offset fixed for the piece, so it costs no VALU.
    const char* __restrict__ kg = uniform_ptr(reinterpret_cast<const char*>(S.k) + 2 * h * D);
    const char* __restrict__ vg = uniform_ptr(reinterpret_cast<const char*>(S.v) + 2 * h * D);
    const char* __restrict__ krec = uniform_ptr(reinterpret_cast<const char*>(S.rec_k) + 2 * h * D);
    const char* __restrict__ vrec = uniform_ptr(reinterpret_cast<const char*>(S.rec_v) + 2 * h * D);
    const unsigned lane_k = (unsigned)(trow0 * row_bytes + kchunk * 16);
    const unsigned lane_v = (unsigned)(trow0 * row_bytes + vchunk * 16);

    // Starts the transfer of this stream's tile TL into stage array ST (this wave's
    // half: rows [32*hw, 32*hw+32) of K and of V).  A tile inside one segment is a run
    // of rows (scalar base + fixed lane offsets); otherwise rows are looked up per lane.
    auto dma_tile = [&](const int tl, char* st) {
      const int kap0 = tl * BN;
      int srow = seg_row[0], skey = seg_key[0], send = seg_key[1], sidx = 0;
#pragma unroll
      for (int i = 1; i < SF_MAX_SEGMENTS; ++i) {
        const bool in = kap0 >= seg_key[i];
        srow = in ? seg_row[i] : srow;
        skey = in ? seg_key[i] : skey;
        send = in ? (i + 1 < SF_MAX_SEGMENTS ? seg_key[i + 1 < SF_MAX_SEGMENTS ? i + 1 : i] : 0x7fffffff) : send;
        sidx = in ? i : sidx;
      }
      srow = __builtin_amdgcn_readfirstlane(srow);  // uniform: tiles and segments are per workgroup
      skey = __builtin_amdgcn_readfirstlane(skey);
      send = __builtin_amdgcn_readfirstlane(send);
      sidx = __builtin_amdgcn_readfirstlane(sidx);
      char* kdst = st + soff + (trow0 - drow) * ROW;
      char* vdst = kdst + TILE;
      constexpr int kStep = 2 * DMA_ROWS;  // rows between a wave's transfers
      if (kap0 + BN <= send) {
        const bool rec = REC && sidx == kRecSlot;
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(rec ? krec : kg);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(rec ? vrec : vg);
        const unsigned base = (unsigned)((srow + kap0 - skey) * row_bytes);
#pragma unroll
        for (int m = 0; m < DMA_PER_WAVE; ++m) {
          const unsigned so = base + (unsigned)(m * kStep * row_bytes);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kdst + m * kStep * ROW), 16, lane_k, so, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vdst + m * kStep * ROW), 16, lane_v, so, 0, 0);
        }
      } else {
#pragma unroll
        for (int m = 0; m < DMA_PER_WAVE; ++m) {
          int sg;
          const unsigned rb = (unsigned)(key_row(seg_row, seg_key, kap0 + trow0 + m * kStep, sg) * row_bytes);
          const bool rec = REC && sg == kRecSlot;
          __builtin_amdgcn_global_load_lds((rec ? krec : kg) + rb + kchunk * 16, (lds_void*)(kdst + m * kStep * ROW), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((rec ? vrec : vg) + rb + vchunk * 16, (lds_void*)(vdst + m * kStep * ROW), 16, 0, 0);
        }
      }
    };

    // piece slot of the column's units: the k-th group of the column writes slot k
    const int k = a.grp_table ? (it == it_lo ? k_first : 0) : grp - grp_of_iter<I>(a, S.it_begin + h * nt);
    for (int qt = mem; qt < S.qtiles; qt += GS) {
    const int u = h * S.qtiles + qt;
    if (!q_ok) load_q(S, h, qt);
    const int qrow0 = qt * kSkRows + hw * 64;
    const bool wave_on = qrow0 < S.rows;
    f32x16 o00, o10, o01, o11;  // O^T blocks [d block][query block]
    float mref0, mref1, lsum0, lsum1, tsmax;

    // P = exp2(S*c - mref) rounded to bf16; the lane's sum of the fp32 values goes to the
    // row sum, and the largest such sum is kept to detect a reference that is too low.
#define SK_SOFTMAX(S, MREF, LSUM, P)                                                      \
  {                                                                                       \
    float h_[2];                                                                          \
    _Pragma("unroll") for (int b_ = 0; b_ < 2; ++b_) {                                    \
      float e_[8];                                                                        \
      _Pragma("unroll") for (int r = 0; r < 8; ++r)                                       \
          e_[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * b_ + r], c, -(MREF)));      \
      _Pragma("unroll") for (int r = 0; r < 8; ++r) P[b_][r] = (__bf16)e_[r];             \
      h_[b_] = ((e_[0] + e_[1]) + (e_[2] + e_[3])) + ((e_[4] + e_[5]) + (e_[6] + e_[7]));  \
    }                                                                                     \
    const float ts_ = h_[0] + h_[1];                                                      \
    LSUM += ts_;                                                                          \
    tsmax = fmaxf(tsmax, ts_);                                                            \
  }
    // Scheduling hints for one region: ND LDS reads first, NV0 VALU ops, then NM MFMAs
    // each followed by NV VALU ops; the region ends there.
#define SK_REGION_HINTS(ND, NV0, NM, NV)                                                  \
  __builtin_amdgcn_sched_group_barrier(0x100, (ND), 0);                                   \
  __builtin_amdgcn_sched_group_barrier(0x002, (NV0), 0);                                  \
  _Pragma("unroll") for (int k_ = 0; k_ < (NM); ++k_) {                                   \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                    \
    __builtin_amdgcn_sched_group_barrier(0x002, (NV), 0);                                 \
  }                                                                                       \
  __builtin_amdgcn_sched_barrier(0);

    // Pipeline over full tiles.  Quarters q0 = (h0, qb0), q1 = (h0, qb1), q2 = (h1, qb0),
    // q3 = (h1, qb1).  State carried between steps: K(t) half 0 (kop0), V(t-1) half 1
    // (vop1), S(t, q0) (sa) and P(t-1, q3) (p3).  Per step, tile t in CUR, tile t+1
    // landing in NXT:
    //   A: S(t,q1)    O(t-1,q3) | P(t,q0)
    //   B: S(t,q2)    O(t,q0)   | P(t,q1)
    //   C: S(t,q3)    O(t,q1)   | P(t,q2)
    //   -- barrier: tile t+1 is in NXT for every wave --
    //   D: S(t+1,q0)  O(t,q2)   | P(t,q3)
    //   -- barrier: every wave is done with CUR, which the next step refills --
    bf16x8 kop0[4], vop1[4], p2[2], p3[2];
    f32x16 sa, sb;
#define SK_STEP_ABC(CUR)                                                                  \
  {                                                                                       \
    bf16x8 kop1[4], vop0[4], p0[2], p1[2];                                                \
    SK_QK(sb, kop0, q1);                                                                  \
    SK_PV(o01, o11, vop1, p3);                                                            \
    SK_SOFTMAX(sa, mref0, lsum0, p0);                                                     \
    SK_REGION_HINTS(0, 0, 8, 7);                                                          \
    SK_LOAD_K(kop1, CUR, 32);                                                             \
    SK_LOAD_V(vop0, CUR, 0);                                                              \
    SK_QK(sa, kop1, q0);                                                                  \
    SK_PV(o00, o10, vop0, p0);                                                            \
    SK_SOFTMAX(sb, mref1, lsum1, p1);                                                     \
    SK_REGION_HINTS(12, 16, 8, 5);                                                        \
    SK_QK(sb, kop1, q1);                                                                  \
    SK_PV(o01, o11, vop0, p1);                                                            \
    SK_SOFTMAX(sa, mref0, lsum0, p2);                                                     \
    SK_REGION_HINTS(0, 0, 8, 7);                                                          \
    SK_LOAD_V(vop1, CUR, 32);                                                             \
  }
#define SK_STEP_D(NXT)                                                                    \
  {                                                                                       \
    SK_LOAD_K(kop0, NXT, 0);                                                              \
    SK_QK(sa, kop0, q0);                                                                  \
    SK_PV(o00, o10, vop1, p2);                                                            \
    SK_SOFTMAX(sb, mref1, lsum1, p3);                                                     \
    SK_REGION_HINTS(4, 16, 8, 5);                                                         \
  }

    // Per-lane max of the raw scores of a tile in stage ST, both query blocks.
    auto tile_max = [&](const char* st, float& mt0, float& mt1) {
#pragma unroll 1
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 kop[4];
        f32x16 s0, s1;
        SK_LOAD_K(kop, st, 32 * hh);
        SK_QK(s0, kop, q0);
        SK_QK(s1, kop, q1);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          mt0 = max3(mt0, s0[r], s0[r + 1]);
          mt1 = max3(mt1, s1[r], s1[r + 1]);
        }
      }
    };

    // Softmax with a reference fixed per query for the whole piece.  Attempt 0 takes the
    // max of the stream's first 32 keys; if some p could then have exceeded 2^40 (a lane's
    // quarter sum above it, +inf included) anywhere in the workgroup, attempt 1 redoes the
    // piece with the exact max over each stream's keys, where every p is at most 1.
    for (int attempt = 0;; ++attempt) {
      float mt0 = -INFINITY, mt1 = -INFINITY;
      if (attempt == 1) {
        // exact maxima over the stream's tiles, then the first tile again
        if (s_lo < s_hi) dma_tile(s_lo, st_a);
        __syncthreads();
        for (int i = 0; i < steps; i += 2) {
          const int tl = s_lo + i;
          if (tl + 1 < s_hi) dma_tile(tl + 1, st_b);
          if (tl < s_hi && wave_on) tile_max(st_a, mt0, mt1);
          __syncthreads();
          if (i + 1 >= steps) break;
          if (tl + 2 < s_hi) dma_tile(tl + 2, st_a);
          if (tl + 1 < s_hi && wave_on) tile_max(st_b, mt0, mt1);
          __syncthreads();
        }
      }
      if (s_lo < s_hi) dma_tile(s_lo, st_a);  // the stream's first tile, in stage a
      __syncthreads();
      o00 = zero16;
      o10 = zero16;
      o01 = zero16;
      o11 = zero16;
      lsum0 = lsum1 = 0.0f;
      tsmax = 0.0f;

      // All waves take `steps` steps (uniform barriers); a wave whose stream has no tile
      // at a step only takes part in the barriers.  Attempt 0 takes the reference of each
      // query from the first 32 keys of the stream (the scores the pipeline starts with).
      const bool run = s_lo < s_hi && wave_on;
      // The last quarter's operands start at zero in every wave: the compiler may issue
      // the closing O^T MFMAs below without the stream's guard, and a stream without
      // tiles must then add exactly zero (not whatever the registers held).
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) vop1[q][e] = (__bf16)0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p3[0][e] = (__bf16)0.0f;
        p3[1][e] = (__bf16)0.0f;
      }
      if (run) {
        SK_LOAD_K(kop0, st_a, 0);
        SK_QK(sa, kop0, q0);
        if (attempt == 0) {
          f32x16 s1;
          SK_QK(s1, kop0, q1);
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            mt0 = max3(mt0, sa[r], sa[r + 1]);
            mt1 = max3(mt1, s1[r], s1[r + 1]);
          }
        }
      }
      mref0 = fmaxf(mt0, xor32(mt0)) * c;
      mref1 = fmaxf(mt1, xor32(mt1)) * c;
      for (int i = 0; i < steps; i += 2) {
        progress_priority(it - it_lo + kStreams * i, it_hi - it_lo);
        const int tl = s_lo + i;
        if (tl + 1 < s_hi) dma_tile(tl + 1, st_b);
        if (tl < s_hi && wave_on) SK_STEP_ABC(st_a);
        __syncthreads();
        if (tl < s_hi && wave_on) SK_STEP_D(st_b);
        __syncthreads();
        if (i + 1 >= steps) break;
        if (tl + 2 < s_hi) dma_tile(tl + 2, st_a);
        if (tl + 1 < s_hi && wave_on) SK_STEP_ABC(st_b);
        __syncthreads();
        if (tl + 1 < s_hi && wave_on) SK_STEP_D(st_a);
        __syncthreads();
      }
      if (run) SK_PV(o01, o11, vop1, p3);  // the stream's last quarter

      // Workgroup-wide decision: redo the piece with exact maxima?
      const int bad = __any(tsmax > kOverflowSum) ? 1 : 0;
      if (lane == 0) redo[wave] = bad;
      __syncthreads();
      int any_bad = 0;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) any_bad |= redo[wv];
      __syncthreads();
      if (!__builtin_amdgcn_readfirstlane(any_bad) || attempt == 1) break;
    }

    // the next piece's Q: this member's next query tile of the column, else its first of
    // the next column piece
    q_ok = false;
    if (qt + GS < S.qtiles) {
      load_q(S, h, qt + GS);
      q_ok = true;
    } else if (it + n < it_hi) {
      int qh;
      if (first_q(it + n, qh)) {
        load_q(a.s[session_of_iter(a, it + n)], qh, mem);
        q_ok = true;
      }
    }

    // ---- merge the two streams: stream s finishes d block s (head dims 32s .. 32s+31) of
    // both query blocks.  Each wave hands the wave of the other stream with the same query
    // rows the d block that one finishes, with its references and sums.
    const int mlane = fresh_lane();
    auto xslot = [&](const int sm) -> float* {  // slot of stream sm's wave of this hw
      return reinterpret_cast<float*>(hw == 0 ? st_a : st_b) + (sm * 64 + mlane) * XCHG_FLOATS;
    };
    if (wave_on) {
      float* dst = xslot(stream);
      const f32x16& g0 = stream == 0 ? o10 : o00;
      const f32x16& g1 = stream == 0 ? o11 : o01;
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        *reinterpret_cast<float4*>(dst + r) = make_float4(g0[r], g0[r + 1], g0[r + 2], g0[r + 3]);
        *reinterpret_cast<float4*>(dst + 16 + r) = make_float4(g1[r], g1[r + 1], g1[r + 2], g1[r + 3]);
      }
      *reinterpret_cast<float4*>(dst + 32) = make_float4(mref0, mref1, lsum0, lsum1);
    }
    __syncthreads();
    if (wave_on) {
      const float* src = xslot(1 - stream);
      const float4 ml = *reinterpret_cast<const float4*>(src + 32);
      // a stream without tiles has reference -inf and contributes nothing
      const float mx0 = fmaxf(mref0, ml.x), mx1 = fmaxf(mref1, ml.y);
      const float fa0 = __builtin_amdgcn_exp2f(mref0 - mx0), fa1 = __builtin_amdgcn_exp2f(mref1 - mx1);
      const float fb0 = __builtin_amdgcn_exp2f(ml.x - mx0), fb1 = __builtin_amdgcn_exp2f(ml.y - mx1);
      const float l0 = lsum0 * fa0 + ml.z * fb0, l1 = lsum1 * fa1 + ml.w * fb1;
      const float lt0 = l0 + xor32(l0), lt1 = l1 + xor32(l1);
      const bool has_tail = (S.n_keys & (BN - 1)) != 0;
      const bool whole = tile0 == 0 && tile1 == nt && !has_tail;
      const int el32 = mlane & 31, eg = mlane >> 5;
      const int dofs = 32 * stream;  // this stream's d block
      auto finish = [&](const f32x16& a0, const f32x16& a1) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int row = qrow0 + 32 * qb + el32;
          if (row >= S.rows) continue;
          const f32x16& oa = qb == 0 ? a0 : a1;
          const float fa = qb == 0 ? fa0 : fa1, fb = qb == 0 ? fb0 : fb1;
          const float lt = qb == 0 ? lt0 : lt1;
          const float mx = qb == 0 ? mx0 : mx1;
          const float* xs = src + 16 * qb;
          const float sc = whole ? 1.0f / lt : 1.0f;
          float* dp = whole ? S.out + row * row_stride + h * D + dofs
                            : S.part_o + (((size_t)u * S.ppu + k) * kSkRows + (row - qt * kSkRows)) * D + dofs;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 x = *reinterpret_cast<const float4*>(xs + 4 * q4);
            *reinterpret_cast<float4*>(dp + 8 * q4 + 4 * eg) =
                make_float4((oa[4 * q4] * fa + x.x * fb) * sc, (oa[4 * q4 + 1] * fa + x.y * fb) * sc,
                            (oa[4 * q4 + 2] * fa + x.z * fb) * sc, (oa[4 * q4 + 3] * fa + x.w * fb) * sc);
          }
          if (!whole && stream == 0 && eg == 0)
            *reinterpret_cast<float2*>(S.part_ml + (((size_t)u * S.ppu + k) * kSkRows + (row - qt * kSkRows)) * 2) =
                make_float2(mx, lt);
        }
      };
      if (stream == 0) finish(o00, o01);
      else finish(o10, o11);
      // Marks for the combine, which then merges every piece slot of a unit and needs no
      // count of its pieces: the column's last piece gives the unit's piece slots past its
      // own the reference -inf (no partial this launch); a unit written whole gets +inf in
      // slot 0 (nothing to merge).
      if (stream == 0 && eg == 0 && tile1 == nt) {
        const int ke0 = whole ? 0 : k + 1, ke1 = whole ? 1 : S.ppu - 1;
        const float mark = whole ? INFINITY : -INFINITY;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int row = qrow0 + 32 * qb + el32;
          if (row >= S.rows) continue;
          float2* ml = reinterpret_cast<float2*>(S.part_ml) + (size_t)u * S.ppu * kSkRows + (row - qt * kSkRows);
          for (int ke = ke0; ke < ke1; ++ke) ml[(size_t)ke * kSkRows] = make_float2(mark, 0.0f);
        }
      }
    }
    __syncthreads();  // the merge buffer overlays the stages of the next piece
    }
    it += n;
  }
}

__global__ __launch_bounds__(kTailWaves * 64) void attn_tail_kernel(const SkLaunch a, int total_units) {
  __shared__ __attribute__((aligned(16))) char st[STAGE];
  int ug, part_unused;
  if (!unit_of_wg(a, total_units, 1, ug, part_unused)) return;
  tail_unit(a, ug, st);
}

// Combine tiling: the partials of a unit are its pieces from attn_sk_kernel (slots
// 0 .. last - first workgroup of the unit) and its tail (last slot).  Small workgroups
// (16 rows of a unit each, one float4 per thread) measured faster than 32- or 64-row ones.
constexpr int kCombThreads = 256;
constexpr int kCombRows = 16;                                   // query rows per workgroup
constexpr int kCombSplit = kSkRows / kCombRows;                 // workgroups per unit
constexpr int kCombPer = kCombRows * (D / 4) / kCombThreads;    // rows per thread: 1
constexpr int kCombBatch = 4;                                   // partials loaded at once
static_assert(kCombSplit * kCombRows == kSkRows && kCombPer * kCombThreads == kCombRows * (D / 4), "combine tiling");

// Merges the partials of each unit that has more than one, in slot order (pieces, then
// the tail), and writes the normalised output.  kCombSplit workgroups per unit, each
// owning kCombRows rows; a thread owns 4 columns of kCombPer rows.  Partials are read
// kCombBatch at a time, all loads in flight before the first is used.  ONE: a one-session
// launch, whose session is 0 at compile time (its fields come from fixed argument offsets,
// with no dependent loads to find it).
template <bool ONE>
__global__ __launch_bounds__(kCombThreads) void combine_sk_kernel(const SkLaunch a, int total_units, int n_wg) {
  // A record written by this launch (one session) and not copied by the attention kernel:
  // the attention read its keys from the source, so the copy into the buffer can wait
  // until now; its loads overlap the loads of the partials below.
  if (a.n_sessions == 1 && a.s[0].rec_seg >= 0 && !a.rec_copy_idle) {
    const SkSession& S0 = a.s[0];
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const size_t n16 = (size_t)S0.rows * a.n_heads * D * 2 / 16;
    const size_t dst0 = (size_t)S0.rec_row0 * a.n_heads * D * 2 / 16;
    const u32x4* __restrict__ sk = reinterpret_cast<const u32x4*>(S0.rec_k);
    const u32x4* __restrict__ sv = reinterpret_cast<const u32x4*>(S0.rec_v);
    u32x4* __restrict__ dk = reinterpret_cast<u32x4*>(const_cast<void*>(S0.k)) + dst0;
    u32x4* __restrict__ dv = reinterpret_cast<u32x4*>(const_cast<void*>(S0.v)) + dst0;
    const size_t nthr = (size_t)n_wg * kCombThreads;  // the whole grid
    for (size_t i = (size_t)wg_x() * kCombThreads + tid_x(); i < n16; i += nthr) {
      const u32x4 x = __builtin_nontemporal_load(sk + i);
      const u32x4 y = __builtin_nontemporal_load(sv + i);
      __builtin_nontemporal_store(x, dk + i);
      __builtin_nontemporal_store(y, dv + i);
    }
  }
  int ug, part;
  if (!unit_of_wg(a, total_units, kCombSplit, ug, part)) return;
  int si = 0, u = ug;
  if (!ONE) decode_unit(a, ug, si, u);
  const SkSession& S = a.s[si];
  const bool has_tail = (S.n_keys & (kSkKeys - 1)) != 0;
  const int qt = u % S.qtiles, h = u / S.qtiles;
  // Every piece slot but the last: a partial of this launch, or -inf (none); slot 0 holds
  // +inf when one workgroup wrote the unit whole.  The last slot holds the tail's partial.
  const int pieces = S.ntiles > 0 ? S.ppu - 1 : 0;
  const int total = pieces + (has_tail ? 1 : 0);
  const int H = a.n_heads;
  constexpr int RSTRIDE = kCombThreads / (D / 4);  // 16 rows between a thread's rows
  const int r0 = part * kCombRows + tid_x() / (D / 4);
  const int d4 = (tid_x() % (D / 4)) * 4;
  float mx[kCombPer], l[kCombPer];
  float4 acc[kCombPer];
#pragma unroll
  for (int i = 0; i < kCombPer; ++i) {
    mx[i] = -INFINITY;
    l[i] = 0.0f;
    acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int k0 = 0; k0 < total; k0 += kCombBatch) {
    float2 ml[kCombBatch][kCombPer];
    float4 x[kCombBatch][kCombPer];
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      const int k = k0 + j;
      if (k >= total) break;
      const size_t slot = (size_t)u * S.ppu + (k < pieces ? k : S.ppu - 1);
#pragma unroll
      for (int i = 0; i < kCombPer; ++i) {
        const int rin = r0 + RSTRIDE * i;
        ml[j][i] = *reinterpret_cast<const float2*>(S.part_ml + (slot * kSkRows + rin) * 2);
        x[j][i] = *reinterpret_cast<const float4*>(S.part_o + (slot * kSkRows + rin) * D + d4);
      }
    }
    // written whole by one workgroup (the mark is per unit, so uniform over the workgroup)
    if (k0 == 0 && pieces > 0 && ml[0][0].x == INFINITY) return;
#pragma unroll
    for (int j = 0; j < kCombBatch; ++j) {
      if (k0 + j >= total) break;
#pragma unroll
      for (int i = 0; i < kCombPer; ++i) {
        const float mn = fmaxf(mx[i], ml[j][i].x);
        const float fo = __builtin_amdgcn_exp2f(mx[i] - mn);  // mx = -inf on the first partial: 0
        const float fn = __builtin_amdgcn_exp2f(ml[j][i].x - mn);
        // a slot without a partial (reference -inf) adds nothing, whatever its stale numerators
        const float4 xn = fn > 0.0f ? make_float4(x[j][i].x * fn, x[j][i].y * fn, x[j][i].z * fn, x[j][i].w * fn)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
        l[i] = l[i] * fo + (fn > 0.0f ? ml[j][i].y * fn : 0.0f);
        acc[i] = make_float4(acc[i].x * fo + xn.x, acc[i].y * fo + xn.y, acc[i].z * fo + xn.z, acc[i].w * fo + xn.w);
        mx[i] = mn;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kCombPer; ++i) {
    const int row = qt * kSkRows + r0 + RSTRIDE * i;
    if (row >= S.rows) continue;
    const float inv = 1.0f / l[i];
    *reinterpret_cast<float4*>(S.out + (size_t)row * H * D + h * D + d4) =
        make_float4(acc[i].x * inv, acc[i].y * inv, acc[i].z * inv, acc[i].w * inv);
  }
}

}  // namespace

int32_t sk_pieces_per_unit(int64_t capacity_rows) {
  // pieces of a unit: at most ceil(tiles / kSkMinRange) + 1 (a group range that
  // starts inside a column holds at least kSkMinRange of its tiles); one more slot for
  // the tail
  const int64_t nt = capacity_rows / kSkKeys;
  return (int32_t)((nt + kSkMinRange - 1) / kSkMinRange + 2);
}

size_t sk_scratch_bytes(int64_t rows, int n_heads, int64_t capacity_rows) {
  const int64_t units = (int64_t)n_heads * ((rows + kSkRows - 1) / kSkRows);
  return (size_t)units * sk_pieces_per_unit(capacity_rows) * kSkRows * (D + 2) * sizeof(float);
}

hipError_t launch_attend_sk(const SkLaunch& a, hipStream_t stream) {
  static_assert(kTailWaves == kWaves, "tail workgroups share the attention launch's shape");
  const bool rec = a.n_sessions == 1 && a.s[0].rec_seg >= 0;
  const dim3 grid(a.n_wg + a.tail_units);
  if (rec && a.narrow) launch(attn_sk_kernel<true, unsigned>, grid, dim3(kThreads), stream, a);
  else if (rec) launch(attn_sk_kernel<true, long long>, grid, dim3(kThreads), stream, a);
  else if (a.narrow) launch(attn_sk_kernel<false, unsigned>, grid, dim3(kThreads), stream, a);
  else launch(attn_sk_kernel<false, long long>, grid, dim3(kThreads), stream, a);
  return hipGetLastError();
}

hipError_t launch_tail_sk(const SkLaunch& a, int total_units, hipStream_t stream) {
  const int grid = a.xcd_map ? 8 * a.xcd_per : total_units;
  launch(attn_tail_kernel, dim3(grid), dim3(kTailWaves * 64), stream, a, total_units);
  return hipGetLastError();
}

hipError_t launch_combine_sk(const SkLaunch& a, int total_units, hipStream_t stream) {
  const int grid = (a.xcd_map ? 8 * a.xcd_per : total_units) * kCombSplit;
  if (a.n_sessions == 1) launch(combine_sk_kernel<true>, dim3(grid), dim3(kCombThreads), stream, a, total_units, grid);
  else launch(combine_sk_kernel<false>, dim3(grid), dim3(kCombThreads), stream, a, total_units, grid);
  return hipGetLastError();
}

}  // namespace sf
