// The dense read of the per-block memory on gfx950.
//
// Model card "GTA world model: weights and inference code": section "What a
// frame attends to" lists what frame t's tokens see, and section "One buffer,
// no mask" makes that exactly the filled rows of one preallocated K/V buffer,
// read by one dense attention call with no mask.  Every query row of the
// record (raw and summary rows alike) attends to every filled row:
//     O[i,h] = sum_j softmax_j(scale * <Q[i,h], K[j,h]>) V[j,h]
// The filled rows form at most a few contiguous row segments of the buffer
// (never more than two for this slot map); the kernels walk the segments as
// one flattened key sequence, so a segment boundary is addressing, not a mask.
//
// bf16 kernel (attn_bf16_kernel<D>, D = head_dim 64 or 128)
//   workgroup = 4 waves = 128 query rows of one head; wave = 32 query rows.
//   Keys go in tiles of 64 rows; K and V tiles are staged in LDS (double
//   buffered, XOR-swizzled 16/32-byte chunks so MFMA operand reads are
//   bank-conflict free).  Per tile and wave:
//     S^T (64 keys x 32 queries) = K_tile . Q^T   on v_mfma_f32_32x32x16_bf16
//       (A = K rows from LDS, B = Q held in VGPRs for the whole loop), so each
//       lane owns one query and 32 of its scores: the row max is in-lane plus
//       one exchange with lane^32;
//     online softmax in fp32 with exp2 (scale*log2e folded into one FMA); the
//       reference max is raised only when a tile's max exceeds it by more than
//       2^8, so rescaling the accumulator is rare;
//     P rounded to bf16 (round to nearest even) and its row sum taken from
//       those rounded values (v_dot2_f32_bf16 against ones);
//     O^T (D x 32 queries) += V^T . P^T  on the same MFMA; the V^T operand is
//       read from the row-major V tile with ds_read_b64_tr_b16 (each 16-lane
//       group turns four 8-byte row pieces into four consecutive keys per
//       lane), P^T is the packed score registers as they are.
//   Work units are (session, head, query tile, key split), numbered so that
//   consecutive units share a head; the grid is remapped so each XCD (the
//   hardware deals workgroups to the 8 XCDs round robin) gets a contiguous
//   range of units and the head's K/V stays in that XCD's L2.
//   With split > 1 each unit writes an unnormalised partial (O, reference
//   max, row sum) and combine_kernel merges the splits.
//   Recency bias (BIAS = true; the page's section "Files" lists an optional
//   recency bias on summary keys): each tile also stages its 64 keys' biases
//   (log2 units, one fp32 per buffer row and head) in LDS, and the scores
//   become S*c + bias in one FMA before the softmax.  A session without a
//   bias in such a launch reads zeros.
//
// fp32 kernel (attn_f32_kernel<D>): one thread per query row, K/V tiles of a
//   few keys broadcast from LDS, exact online softmax in fp32 on VALU.
#include "sf_internal.h"

#include <atomic>
#include <cmath>

namespace sf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int BM = kBf16RowsPerTile;  // 128 query rows per workgroup
constexpr int BN = kBf16KeysPerTile;  // 64 keys per tile
static_assert(BM == kWaves * 32, "one 32-row MFMA block per wave");

// Work unit of this workgroup: XCD-aware remap of the workgroup id; the grid is
// total_units rounded up to a multiple of 8.
__device__ __forceinline__ int unit_of_block(int total_units) {
  const int per_xcd = ((total_units + 7) & ~7) >> 3;
  return (int)(wg_x() & 7u) * per_xcd + (int)(wg_x() >> 3);
}

// Everything a workgroup needs about its unit, wave-uniform (held in SGPRs).
struct Unit {
  const char* q;
  float* out;
  const char* k;
  const char* v;
  float* part_o;
  float* part_ml;
  const float* bias;  // recency bias per buffer row, [H][bias_stride] log2 units, or NULL
  int bias_stride;
  int rows, n_keys, split, ks, qt, h;
  int seg_row[SF_MAX_SEGMENTS];  // first buffer row of segment i
  int seg_key[SF_MAX_SEGMENTS];  // first flattened key of segment i (INT_MAX when unused)
};

// Decodes unit -> (session, head, query tile, key split).  Units of one launch are
// numbered session by session, then head, then query tile, then split.
__device__ __forceinline__ Unit decode_unit(const AttnLaunch& a, int unit, bool with_split) {
  int si = 0;
  for (int i = 1; i < a.n_sessions; ++i)
    if (a.s[i].unit_begin <= unit) si = i;
  si = __builtin_amdgcn_readfirstlane(si);
  const AttnSession& S = a.s[si];
  Unit u;
  u.q = reinterpret_cast<const char*>(S.q);
  u.out = S.out;
  u.k = reinterpret_cast<const char*>(S.k);
  u.v = reinterpret_cast<const char*>(S.v);
  u.part_o = S.part_o;
  u.part_ml = S.part_ml;
  u.bias = S.bias;
  u.bias_stride = S.bias_stride;
  u.rows = S.rows;
  u.n_keys = S.n_keys;
  u.split = with_split ? S.split : 1;
  // Integer division is emulated on the VALU; readfirstlane puts the (uniform) results back in SGPRs.
  int local = unit - S.unit_begin;
  u.ks = __builtin_amdgcn_readfirstlane(local % u.split);
  local = __builtin_amdgcn_readfirstlane(local / u.split);
  u.qt = __builtin_amdgcn_readfirstlane(local % S.qtiles);
  u.h = __builtin_amdgcn_readfirstlane(local / S.qtiles);
  int cum = 0;
#pragma unroll
  for (int i = 0; i < SF_MAX_SEGMENTS; ++i) {
    const bool used = i < S.n_seg;
    u.seg_row[i] = used ? S.seg_begin[i] : 0;
    u.seg_key[i] = used ? cum : 0x7fffffff;
    cum += used ? S.seg_len[i] : 0;
  }
  return u;
}

// Flattened key index -> buffer row (branch-free walk over the segments).
__device__ __forceinline__ int key_row(const Unit& u, int kappa) {
  int row = u.seg_row[0] + kappa;
#pragma unroll
  for (int i = 1; i < SF_MAX_SEGMENTS; ++i)
    row = kappa >= u.seg_key[i] ? u.seg_row[i] + (kappa - u.seg_key[i]) : row;
  return row;
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// LDS tile geometry: one stage holds a K tile then a V tile, BN rows of 2D bytes
// each, as 16-byte chunks permuted within each row so that the MFMA operand reads
// are bank-conflict free on the 64 banks (256 bytes per cycle) of gfx950's LDS:
//   K: chunk c of row r sits at c ^ ksw(r).  A ds_read_b128 serves 16 lanes (16
//      consecutive rows at one chunk) per cycle, which must land on 16 distinct
//      16-byte positions of a bank line: D = 128 (a row is one line) needs r & 15;
//      D = 64 (two rows per line) needs (r >> 1) & 7.
//   V: chunk c of row r sits at c ^ vsw(r).  A ds_read_b64_tr_b16 pass (32 lanes:
//      rows 4g .. 4g+3, eight 8-byte words each) must cover the line once: D = 64
//      puts two rows in a line and takes 2 * (r & 3); D = 128 takes 4 * (r & 3).
template <int D>
struct Tile {
  static constexpr int ROW = 2 * D;              // bytes per row
  static constexpr int KBYTES = BN * ROW;
  static constexpr int STAGE = 2 * KBYTES;       // K tile then V tile
  static __device__ __forceinline__ int ksw(int r) { return D == 64 ? ((r >> 1) & 7) : (r & 15); }
  static __device__ __forceinline__ int vsw(int r) { return D == 64 ? 2 * (r & 3) : 4 * (r & 3); }
};

// Probability sums above this make the tile recompute against its true max: every
// p stays <= 2^15 in the accumulators, and p of the first tile (reference -inf) is inf.
constexpr float kSumLimit = 32768.0f;

template <int D, bool BIAS>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(const AttnLaunch a) {
  using T = Tile<D>;
  constexpr int CH = D / 8;                  // 16-byte chunks per K/V row
  constexpr int PER = BN * CH / kThreads;    // chunks per thread per tensor per tile
  constexpr int KSTEPS = D / 16;             // MFMA k-steps over head_dim
  constexpr int DBLK = D / 32;               // 32-row blocks of O^T
  static_assert(PER * kThreads == BN * CH, "tile loads divide evenly");
  static_assert(BN <= kThreads, "one thread stages each key's bias");
  constexpr int BIAS_OFF = 2 * T::STAGE;    // two stages of BN fp32 biases follow the K/V stages
  __shared__ __attribute__((aligned(16))) char sm[2 * T::STAGE + (BIAS ? 2 * BN * 4 : 0)];

  const int unit = unit_of_block(a.total_units);
  if (unit >= a.total_units) return;
  const Unit U = decode_unit(a, unit, true);
  const int H = a.n_heads;
  const int ntiles = (U.n_keys + BN - 1) / BN;
  const int t0 = __builtin_amdgcn_readfirstlane((int)((long long)U.ks * ntiles / U.split));
  const int t1 = __builtin_amdgcn_readfirstlane((int)((long long)(U.ks + 1) * ntiles / U.split));
  const int key_hi = min(t1 * BN, U.n_keys);

  const int tid = tid_x();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5;   // lane half: k-group of MFMA operands
  const int l32 = lane & 31; // query of this lane within the wave's block
  const int qrow = U.qt * BM + wave * 32 + l32;
  const bool row_ok = qrow < U.rows;
  const bool wave_on = U.qt * BM + wave * 32 < U.rows;  // wave-uniform
  const float c = a.scale_log2;
  const int row_stride = H * D;       // elements per buffer row
  const int row_bytes = 2 * row_stride;
  // recency bias of this head's rows (log2 units), NULL when the session has none
  const float* __restrict__ brow = BIAS && U.bias ? U.bias + (size_t)U.h * U.bias_stride : nullptr;

  // Q^T operand: lane holds Q[qrow][16*kk + 8*g .. +7] for every k-step (rows past R read row R-1).
  bf16x8 qreg[KSTEPS];
  {
    const int qoff = min(qrow, U.rows - 1) * row_stride + U.h * D + 8 * g;
    const __bf16* qp = reinterpret_cast<const __bf16*>(U.q) + qoff;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
  }

  // Per-thread tile-load geometry (loop invariant).  Chunk p of this thread is row
  // tid/CH + p*RSTEP, chunk tid%CH; rows p*RSTEP apart share their swizzles (both
  // depend on row & 15 at most), so every chunk's global and LDS offsets are those
  // of chunk 0 plus a constant.
  constexpr int RSTEP = kThreads / CH;
  static_assert(RSTEP % 16 == 0, "chunks of one thread share their swizzle");
  const char* __restrict__ kg = U.k + 2 * U.h * D;
  const char* __restrict__ vg = U.v + 2 * U.h * D;
  const int prow = tid / CH;
  const unsigned goff = (unsigned)(prow * row_bytes + (tid % CH) * 16);
  const unsigned gstep = (unsigned)(RSTEP * row_bytes);
  const int ksoff = prow * T::ROW + (((tid % CH) ^ T::ksw(prow)) << 4);
  const int vsoff = T::KBYTES + prow * T::ROW + (((tid % CH) ^ T::vsw(prow)) << 4);
  // Per-lane LDS operand addresses (bytes within a stage).
  int kaddr[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) kaddr[kk] = l32 * T::ROW + (((2 * kk + g) ^ T::ksw(l32)) << 4);
  const int trow = (lane >> 2) & 3;
  int vaddr[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
    const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    vaddr[db] = T::KBYTES + (4 * g + trow) * T::ROW + ((chunk ^ T::vsw(trow)) << 4) + 8 * (lane & 1);
  }

  // Loads tile TILE into staging registers KR/VR.  A tile inside one segment is a
  // run of rows: a scalar base plus the fixed per-thread offsets.  Otherwise each
  // row is looked up; keys past the unit's range re-read its last key (finite
  // data) and get score -inf.
#define SF_LOAD_TILE(TILE, KR, VR, BR)                                                      \
  {                                                                                         \
    const int kap0_ = (TILE) * BN;                                                          \
    if constexpr (BIAS) {                                                                   \
      if (tid < BN) BR = brow ? brow[key_row(U, min(kap0_ + tid, key_hi - 1))] : 0.0f;      \
    }                                                                                       \
    int srow_ = U.seg_row[0], skey_ = U.seg_key[0], send_ = U.seg_key[1];                   \
    _Pragma("unroll") for (int i = 1; i < SF_MAX_SEGMENTS; ++i) {                           \
      const bool in_ = kap0_ >= U.seg_key[i];                                               \
      srow_ = in_ ? U.seg_row[i] : srow_;                                                   \
      skey_ = in_ ? U.seg_key[i] : skey_;                                                   \
      send_ = in_ ? (i + 1 < SF_MAX_SEGMENTS ? U.seg_key[i + 1 < SF_MAX_SEGMENTS ? i + 1 : i] : 0x7fffffff) : send_; \
    }                                                                                       \
    if (kap0_ + BN <= min(send_, key_hi)) {                                                 \
      const unsigned base_ = (unsigned)((srow_ + kap0_ - skey_) * row_bytes);               \
      _Pragma("unroll") for (int p = 0; p < PER; ++p) {                                     \
        KR[p] = *reinterpret_cast<const u32x4*>(kg + base_ + p * gstep + goff);             \
        VR[p] = *reinterpret_cast<const u32x4*>(vg + base_ + p * gstep + goff);             \
      }                                                                                     \
    } else {                                                                                \
      _Pragma("unroll") for (int p = 0; p < PER; ++p) {                                     \
        const int kappa_ = min(kap0_ + prow + p * RSTEP, key_hi - 1);                       \
        const unsigned off_ = (unsigned)(key_row(U, kappa_) * row_bytes) + (tid % CH) * 16; \
        KR[p] = *reinterpret_cast<const u32x4*>(kg + off_);                                 \
        VR[p] = *reinterpret_cast<const u32x4*>(vg + off_);                                 \
      }                                                                                     \
    }                                                                                       \
  }
#define SF_STORE_TILE(STAGE_BYTES, KR, VR, BR)                                              \
  _Pragma("unroll") for (int p = 0; p < PER; ++p) {                                         \
    *reinterpret_cast<u32x4*>(sm + (STAGE_BYTES) + ksoff + p * RSTEP * T::ROW) = KR[p];     \
    *reinterpret_cast<u32x4*>(sm + (STAGE_BYTES) + vsoff + p * RSTEP * T::ROW) = VR[p];     \
  }                                                                                         \
  if constexpr (BIAS) {                                                                     \
    if (tid < BN) reinterpret_cast<float*>(sm + BIAS_OFF + ((STAGE_BYTES) / T::STAGE) * BN * 4)[tid] = BR; \
  }

  f32x16 o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float mref = -INFINITY;  // reference max, log2 units
  float lsum = 0.0f;       // this lane's share of the row sum
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // One tile of work on the stage at byte offset ST.
  auto compute_tile = [&](const int tile, const int ST) {
    const char* st = sm + ST;
    // ---- S^T = K . Q^T : two 32-key blocks
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(st + kaddr[kk]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(st + kaddr[kk] + 32 * T::ROW);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[kk], s1, 0, 0, 0);
    }
    // ---- keys past the end of this unit's range (ragged last tile) score -inf
    if (tile * BN + BN > key_hi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kb = tile * BN + 8 * (r >> 2) + 4 * g + (r & 3);
        if (kb >= key_hi) s0[r] = -INFINITY;
        if (kb + 32 >= key_hi) s1[r] = -INFINITY;
      }
    }
    // ---- recency bias: scores to log2 units with each key's bias added (register r of
    // block b holds key 32b + 8(r/4) + 4g + r%4); from here on the scale is 1.
    if constexpr (BIAS) {
      const float* bs = reinterpret_cast<const float*>(sm + BIAS_OFF + (ST / T::STAGE) * BN * 4);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 b0 = *reinterpret_cast<const float4*>(bs + 8 * q4 + 4 * g);
        const float4 b1 = *reinterpret_cast<const float4*>(bs + 32 + 8 * q4 + 4 * g);
        s0[4 * q4 + 0] = __builtin_fmaf(s0[4 * q4 + 0], c, b0.x);
        s0[4 * q4 + 1] = __builtin_fmaf(s0[4 * q4 + 1], c, b0.y);
        s0[4 * q4 + 2] = __builtin_fmaf(s0[4 * q4 + 2], c, b0.z);
        s0[4 * q4 + 3] = __builtin_fmaf(s0[4 * q4 + 3], c, b0.w);
        s1[4 * q4 + 0] = __builtin_fmaf(s1[4 * q4 + 0], c, b1.x);
        s1[4 * q4 + 1] = __builtin_fmaf(s1[4 * q4 + 1], c, b1.y);
        s1[4 * q4 + 2] = __builtin_fmaf(s1[4 * q4 + 2], c, b1.z);
        s1[4 * q4 + 3] = __builtin_fmaf(s1[4 * q4 + 3], c, b1.w);
      }
    }
    const float cs = BIAS ? 1.0f : c;
    // ---- P = exp2(S*c - mref) in bf16 and its row sum, against the current reference.
    bf16x8 pb[4];
    float ts;
    auto probs = [&]() {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        pb[0][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], cs, -mref));
        pb[1][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[8 + r], cs, -mref));
        pb[2][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], cs, -mref));
        pb[3][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s1[8 + r], cs, -mref));
      }
      float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pr = {pb[j][2 * e], pb[j][2 * e + 1]};
          part[j] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, part[j], false);
        }
      ts = (part[0] + part[1]) + (part[2] + part[3]);
    };
    probs();
    // ---- the reference moves only when some p left its range, and on the unit's first
    // tile (the reference is -inf before it; masked keys there give NaN p, discarded here).
    if (tile == t0 || __any(ts > kSumLimit)) {
      float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = max3(mt, s0[r], s1[r]);
      mt = fmaxf(mt, xor32(mt)) * cs;
      const float mnew = fmaxf(mref, mt);
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      lsum *= alpha;
      mref = mnew;
      probs();
    }
    lsum += ts;
    // ---- O^T += V^T . P^T ; k-step j covers S^T registers 8*(j&1).. of block j>>1,
    // i.e. keys 32*(j>>1) + 16*(j&1) + {4g..4g+3} then {8+4g..8+4g+3}.
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int roff = (32 * (j >> 1) + 16 * (j & 1)) * T::ROW;
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + vaddr[db] + roff));
        const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + vaddr[db] + roff + 8 * T::ROW));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[j], o[db], 0, 0, 0);
      }
    }
  };

  // Pipeline: tile i is computed from stage i&1 while tile i+2 is in flight in one
  // register set and tile i+1 (the other set) is stored to stage (i+1)&1 after it.
  u32x4 kra[PER], vra[PER], krb[PER], vrb[PER];
  float bra = 0.0f, brb = 0.0f;  // this thread's key bias of each set (BIAS only)
  SF_LOAD_TILE(t0, kra, vra, bra)
  if (t0 + 1 < t1) SF_LOAD_TILE(t0 + 1, krb, vrb, brb)
  SF_STORE_TILE(0, kra, vra, bra)
  __syncthreads();
  for (int tile = t0; tile < t1; tile += 2) {
    // even step: compute stage 0, refill set a with tile+2, store set b (tile+1) to stage 1
    if (tile + 2 < t1) SF_LOAD_TILE(tile + 2, kra, vra, bra)
    if (wave_on) compute_tile(tile, 0);
    if (tile + 1 < t1) SF_STORE_TILE(T::STAGE, krb, vrb, brb)
    __syncthreads();
    if (tile + 1 >= t1) break;
    // odd step: compute stage 1, refill set b with tile+3, store set a (tile+2) to stage 0
    if (tile + 3 < t1) SF_LOAD_TILE(tile + 3, krb, vrb, brb)
    if (wave_on) compute_tile(tile + 1, T::STAGE);
    if (tile + 2 < t1) SF_STORE_TILE(0, kra, vra, bra)
    __syncthreads();
  }
#undef SF_LOAD_TILE
#undef SF_STORE_TILE

  if (!wave_on) return;
  const float ltot = lsum + xor32(lsum);
  const size_t obase = (size_t)qrow * row_stride + (size_t)U.h * D;
  if (!row_ok) return;
  if (U.split == 1) {
    const float inv = 1.0f / ltot;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * g;
        float4 w = make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                               o[db][4 * q4 + 3] * inv);
        *reinterpret_cast<float4*>(U.out + obase + d) = w;
      }
  } else {
    float* po = U.part_o + (size_t)U.ks * U.rows * row_stride + obase;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * g;
        *reinterpret_cast<float4*>(po + d) =
            make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
      }
    if (g == 0) {
      float* pm = U.part_ml + ((size_t)U.ks * U.rows * H + (size_t)qrow * H + U.h) * 2;
      *reinterpret_cast<float2*>(pm) = make_float2(mref, ltot);
    }
  }
}

// Merge key splits: one wave per (row, head); lane covers D/64 output columns.  Every
// split's partial (reference max, row sum, numerators) is loaded before the first use, so
// a wave has all its loads in flight at once.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const AttnLaunch a) {
  const AttnSession& S = a.s[wg_y()];
  if (S.split <= 1) return;
  const int H = a.n_heads;
  const int idx = wg_x() * 4 + (tid_x() >> 6);
  if (idx >= S.rows * H) return;
  const int lane = tid_x() & 63;
  const size_t slice = (size_t)S.rows * H;  // (row, head) pairs per split
  const int split = S.split;                // <= kMaxSplit
  constexpr int PER = D / 64;
  float m[kMaxSplit], l[kMaxSplit], po[kMaxSplit][PER];
#pragma unroll
  for (int k = 0; k < kMaxSplit; ++k) {
    m[k] = -INFINITY;
    l[k] = 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) po[k][j] = 0.0f;
    if (k < split) {
      const float2 ml = *reinterpret_cast<const float2*>(S.part_ml + (k * slice + idx) * 2);
      m[k] = ml.x;
      l[k] = ml.y;
      const float* p = S.part_o + (k * slice + idx) * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) po[k][j] = p[lane + 64 * j];
    }
  }
  float mmax = m[0];
#pragma unroll
  for (int k = 1; k < kMaxSplit; ++k) mmax = fmaxf(mmax, m[k]);
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;
  float lt = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxSplit; ++k) {
    const float wgt = __builtin_amdgcn_exp2f(m[k] - mmax);  // 0 for the splits past `split`
    lt += wgt * l[k];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] += wgt * po[k][j];
  }
  const float inv = 1.0f / lt;
#pragma unroll
  for (int j = 0; j < PER; ++j) S.out[(size_t)idx * D + lane + 64 * j] = acc[j] * inv;
}

// ---------------------------------------------------------------- fp32 path
constexpr int kF32Threads = kF32RowsPerTile;

template <int D, bool BIAS>
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(const AttnLaunch a) {
  constexpr int KT = D <= 64 ? 16 : 8;  // keys per LDS tile
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  __shared__ float bs[KT];  // recency bias of the tile's keys, log2 units (BIAS only)
  const int unit = (int)wg_x();
  if (unit >= a.total_units) return;
  const Unit U = decode_unit(a, unit, false);
  const int H = a.n_heads;
  const int tid = tid_x();
  const int qrow = U.qt * kF32RowsPerTile + tid;
  const bool row_ok = qrow < U.rows;
  const int row_stride = H * D;
  const float* __restrict__ kg = reinterpret_cast<const float*>(U.k) + U.h * D;
  const float* __restrict__ vg = reinterpret_cast<const float*>(U.v) + U.h * D;
  const float c = a.scale_log2;
  const int n_keys = U.n_keys;
  const float* __restrict__ brow = BIAS && U.bias ? U.bias + (size_t)U.h * U.bias_stride : nullptr;

  float q[D], o[D];
  {
    const float* qp = reinterpret_cast<const float*>(U.q) + min(qrow, U.rows - 1) * row_stride + U.h * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      q[d] = qp[d];
      o[d] = 0.0f;
    }
  }
  float m = -INFINITY, l = 0.0f;
  for (int base = 0; base < n_keys; base += KT) {
    for (int e = tid; e < KT * D; e += kF32Threads) {
      const int j = e / D, d = e % D;
      const int off = key_row(U, min(base + j, n_keys - 1)) * row_stride + d;
      ks[j][d] = kg[off];
      vs[j][d] = vg[off];
    }
    if constexpr (BIAS) {
      if (tid < KT) bs[tid] = brow ? brow[key_row(U, min(base + tid, n_keys - 1))] : 0.0f;
    }
    __syncthreads();
    float s[KT];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], ks[j][d], acc);
      s[j] = (base + j < n_keys) ? (BIAS ? __builtin_fmaf(acc, c, bs[j]) : acc * c) : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float mnew = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const float p = __builtin_amdgcn_exp2f(s[j] - mnew);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, vs[j][d], o[d]);
    }
    m = mnew;
    __syncthreads();
  }
  if (!row_ok) return;
  float* op = U.out + qrow * row_stride + U.h * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
}

int round_up8(int n) { return (n + 7) & ~7; }

}  // namespace

size_t attend_scratch_bytes(int64_t rows, int n_heads, int head_dim) {
  return (size_t)kMaxSplit * (size_t)rows * (size_t)n_heads * ((size_t)head_dim + 2) * sizeof(float);
}

hipError_t launch_attend_bf16(const AttnLaunch& a, bool bias, hipStream_t stream) {
  const int grid = round_up8(a.total_units);
  if (a.head_dim == 64 && bias)
    launch(attn_bf16_kernel<64, true>, dim3(grid), dim3(kThreads), stream, a);
  else if (a.head_dim == 64)
    launch(attn_bf16_kernel<64, false>, dim3(grid), dim3(kThreads), stream, a);
  else if (a.head_dim == 128 && bias)
    launch(attn_bf16_kernel<128, true>, dim3(grid), dim3(kThreads), stream, a);
  else if (a.head_dim == 128)
    launch(attn_bf16_kernel<128, false>, dim3(grid), dim3(kThreads), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

int attend_bf16_wgs_per_cu(int head_dim, bool bias) {
  // per device and variant; 0 until asked (every thread that asks stores the same value)
  static std::atomic<int> cache[64][4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  const int v = (head_dim == 128 ? 2 : 0) + (bias ? 1 : 0);
  int cached = cache[dev][v].load(std::memory_order_relaxed);
  if (cached == 0) {
    int n = 0;
    hipError_t e;
    if (v == 0) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<64, false>, kThreads, 0);
    else if (v == 1) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<64, true>, kThreads, 0);
    else if (v == 2) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<128, false>, kThreads, 0);
    else e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<128, true>, kThreads, 0);
    cached = (e == hipSuccess && n > 0) ? n : 1;
    cache[dev][v].store(cached, std::memory_order_relaxed);
  }
  return cached;
}

hipError_t launch_combine(const AttnLaunch& a, hipStream_t stream) {
  int max_pairs = 0;
  bool any = false;
  for (int i = 0; i < a.n_sessions; ++i) {
    if (a.s[i].split > 1) any = true;
    max_pairs = max_pairs > a.s[i].rows * a.n_heads ? max_pairs : a.s[i].rows * a.n_heads;
  }
  if (!any) return hipSuccess;
  const dim3 grid((max_pairs + 3) / 4, a.n_sessions);
  if (a.head_dim == 64)
    launch(combine_kernel<64>, grid, dim3(256), stream, a);
  else if (a.head_dim == 128)
    launch(combine_kernel<128>, grid, dim3(256), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attend_f32(const AttnLaunch& a, bool bias, hipStream_t stream) {
  if (a.head_dim == 64 && bias)
    launch(attn_f32_kernel<64, true>, dim3(a.total_units), dim3(kF32Threads), stream, a);
  else if (a.head_dim == 64)
    launch(attn_f32_kernel<64, false>, dim3(a.total_units), dim3(kF32Threads), stream, a);
  else if (a.head_dim == 128 && bias)
    launch(attn_f32_kernel<128, true>, dim3(a.total_units), dim3(kF32Threads), stream, a);
  else if (a.head_dim == 128)
    launch(attn_f32_kernel<128, false>, dim3(a.total_units), dim3(kF32Threads), stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sf
