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
//   Keys go in tiles of 64 rows (32 at head_dim 128, where three workgroups share
//   a CU); K and V tiles go from global memory straight
//   into LDS (buffer_load_dwordx4 ... lds: a scalar tile offset plus a lane
//   offset fixed for the unit, no staging registers), double buffered in two
//   LDS arrays, as XOR-swizzled 16-byte chunks so MFMA operand reads are
//   bank-conflict free.  Per tile and wave:
//     S^T (tile keys x 32 queries) = K_tile . Q^T on v_mfma_f32_32x32x16_bf16
//       (A = K rows from LDS, B = Q held in VGPRs for the whole loop), so each
//       lane owns one query and 32 of its scores: the row max is in-lane plus
//       one exchange with lane^32;
//     online softmax in fp32 with exp2 (scale*log2e folded into one FMA); the
//       reference max is raised only when a tile's max exceeds it by more than
//       2^8, so rescaling the accumulator is rare;
//     P rounded to bf16 (round to nearest even); the row sum adds the fp32
//       values;
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int BM = kBf16RowsPerTile;  // 128 query rows per workgroup
// Keys per tile: 64 at head_dim 64; 32 at head_dim 128, whose smaller stages (32 KB for
// both) and leaner registers let three workgroups share a CU (three waves per SIMD).
template <int D>
constexpr int kTileKeys = D == 128 ? 32 : kBf16KeysPerTile;
template <int D>
constexpr int kWavesPerEu = D == 128 ? 3 : 1;
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

// LDS tile geometry: one stage holds a K tile then a V tile, kTileKeys rows of 2D bytes
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
  static constexpr int KBYTES = kTileKeys<D> * ROW;
  static constexpr int STAGE = 2 * KBYTES;       // K tile then V tile
  static __device__ __forceinline__ int ksw(int r) { return D == 64 ? ((r >> 1) & 7) : (r & 15); }
  static __device__ __forceinline__ int vsw(int r) { return D == 64 ? 2 * (r & 3) : 4 * (r & 3); }
};

typedef __attribute__((address_space(3))) void lds_void;

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

// Probability sums above this make the tile recompute against its true max: every
// p stays <= 2^15 in the accumulators, and p of the first tile (reference -inf) is inf.
constexpr float kSumLimit = 32768.0f;

template <int D, bool BIAS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEu<D>)))
void attn_bf16_kernel(const AttnLaunch a) {
  constexpr int BN = kTileKeys<D>;
  constexpr int KB = BN / 32;                // 32-key MFMA blocks per tile
  using T = Tile<D>;
  constexpr int CH = D / 8;                  // 16-byte chunks per K/V row
  constexpr int KSTEPS = D / 16;             // MFMA k-steps over head_dim
  constexpr int DBLK = D / 32;               // 32-row blocks of O^T
  constexpr int NQK = KSTEPS * KB;           // MFMAs of S^T per tile
  constexpr int NPV = DBLK * 2 * KB;         // MFMAs of O^T per tile
  constexpr int KPF = D == 128 && BIAS ? 2 : 4;  // K operands read ahead of their MFMA (fits the VGPR budget)
  constexpr int VPF = 2;                     // V^T operands read ahead of their MFMA
  static_assert(BN <= kThreads, "one thread stages each key's bias");
  // Two stages, each in an array of its own: the compiler then knows that transfers into
  // one stage never alias the operand reads of the other (one array would make it wait for
  // every transfer in flight before each LDS read).
  __shared__ __attribute__((aligned(16))) char st_a[T::STAGE + (BIAS ? BN * 4 : 0)];
  __shared__ __attribute__((aligned(16))) char st_b[T::STAGE + (BIAS ? BN * 4 : 0)];
  constexpr int BIAS_OFF = T::STAGE;        // the tile's BN fp32 biases follow its K/V

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

  // K/V tiles go from global memory straight into LDS (buffer_load_dwordx4 ... lds, no
  // staging registers).  One wave-wide transfer fills 1 KB = RPT rows of a stage, lane L
  // landing at row L / CH, chunk position L % CH; lane L therefore fetches the logical
  // chunk that belongs there (the swizzles are involutions).  Wave w takes the transfers
  // starting at rows RPT*w + 4*RPT*m, which all have the same row phase modulo 16, so each
  // lane fetches the same K chunk and the same V chunk in every transfer of the piece.
  constexpr int RPT = 1024 / T::ROW;          // rows per transfer (4 at D = 128, 8 at D = 64)
  constexpr int NTW = BN / RPT / kWaves;      // transfers per wave per tensor per tile
  static_assert(NTW * RPT * kWaves == BN, "transfers divide the tile");
  const char* __restrict__ kg = uniform_ptr(U.k + 2 * U.h * D);
  const char* __restrict__ vg = uniform_ptr(U.v + 2 * U.h * D);
  const int rl = lane / CH;                   // row of this lane within a transfer
  const int r0w = RPT * wave;                 // first row of this wave's transfer 0
  const int kchunk = (lane % CH) ^ T::ksw(r0w + rl);
  const int vchunk = (lane % CH) ^ T::vsw(r0w + rl);
  const unsigned lane_k = (unsigned)(rl * row_bytes + kchunk * 16);
  const unsigned lane_v = (unsigned)(rl * row_bytes + vchunk * 16);
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

  // Starts the transfers of tile TILE into stage ST (this wave's rows of K and V).  A tile
  // inside one segment is a run of rows: a scalar offset plus the fixed lane offsets.
  // Otherwise each row is looked up; keys past the unit's range re-read its last key
  // (finite data) and get score -inf.  The bias of the tile's keys (BIAS) goes through a
  // register: loaded here into BR, stored by store_bias after the stage's compute.
  auto dma_tile = [&](const int tile, char* st, float& br) {
    const int kap0 = tile * BN;
    if constexpr (BIAS) {
      if (tid < BN) br = brow ? brow[key_row(U, min(kap0 + tid, key_hi - 1))] : 0.0f;
    }
    int srow = U.seg_row[0], skey = U.seg_key[0], send = U.seg_key[1];
#pragma unroll
    for (int i = 1; i < SF_MAX_SEGMENTS; ++i) {
      const bool in = kap0 >= U.seg_key[i];
      srow = in ? U.seg_row[i] : srow;
      skey = in ? U.seg_key[i] : skey;
      send = in ? (i + 1 < SF_MAX_SEGMENTS ? U.seg_key[i + 1 < SF_MAX_SEGMENTS ? i + 1 : i] : 0x7fffffff) : send;
    }
    srow = __builtin_amdgcn_readfirstlane(srow);
    skey = __builtin_amdgcn_readfirstlane(skey);
    send = __builtin_amdgcn_readfirstlane(send);
    if (kap0 + BN <= min(send, key_hi)) {
      const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kg);
      const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vg);
      const unsigned base = (unsigned)((srow + kap0 - skey + r0w) * row_bytes);
#pragma unroll
      for (int m = 0; m < NTW; ++m) {
        const unsigned so = base + (unsigned)(m * 4 * RPT * row_bytes);
        char* dk = st + (r0w + m * 4 * RPT) * T::ROW;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)dk, 16, lane_k, so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dk + T::KBYTES), 16, lane_v, so, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NTW; ++m) {
        const int kappa = min(kap0 + r0w + m * 4 * RPT + rl, key_hi - 1);
        const unsigned rb = (unsigned)(key_row(U, kappa) * row_bytes);
        char* dk = st + (r0w + m * 4 * RPT) * T::ROW;
        __builtin_amdgcn_global_load_lds(kg + rb + kchunk * 16, (lds_void*)dk, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vg + rb + vchunk * 16, (lds_void*)(dk + T::KBYTES), 16, 0, 0);
      }
    }
  };
  auto store_bias = [&](char* st, const float br) {
    if constexpr (BIAS) {
      if (tid < BN) reinterpret_cast<float*>(st + BIAS_OFF)[tid] = br;
    }
  };

  f32x16 o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float mref = -INFINITY;  // reference max, log2 units
  float lsum = 0.0f;       // this lane's share of the row sum

  // One tile of work on the stage at byte offset ST.
  auto compute_tile = [&](const int tile, const char* st) {
    // ---- S^T = K . Q^T : KB 32-key blocks
    f32x16 sb[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) sb[b][r] = 0.0f;
    // K operands KPF ahead of their MFMA, so an operand's LDS latency overlaps the MFMAs
    // before it (operand i = k-step i / KB of block i % KB).
    {
      bf16x8 ka[NQK];
#pragma unroll
      for (int i = 0; i < KPF; ++i)
        ka[i] = *reinterpret_cast<const bf16x8*>(st + kaddr[i / KB] + 32 * (i % KB) * T::ROW);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        if (i + KPF < NQK)
          ka[i + KPF] = *reinterpret_cast<const bf16x8*>(st + kaddr[(i + KPF) / KB] + 32 * ((i + KPF) % KB) * T::ROW);
        sb[i % KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qreg[i / KB], sb[i % KB], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, KPF, 0);
#pragma unroll
      for (int i = 0; i < NQK - KPF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KPF, 0);
    }
    // ---- keys past the end of this unit's range (ragged last tile) score -inf
    if (tile * BN + BN > key_hi) {
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kb = tile * BN + 32 * b + 8 * (r >> 2) + 4 * g + (r & 3);
          if (kb >= key_hi) sb[b][r] = -INFINITY;
        }
    }
    // ---- recency bias: scores to log2 units with each key's bias added (register r of
    // block b holds key 32b + 8(r/4) + 4g + r%4); from here on the scale is 1.
    if constexpr (BIAS) {
      const float* bs = reinterpret_cast<const float*>(st + BIAS_OFF);
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 bb = *reinterpret_cast<const float4*>(bs + 32 * b + 8 * q4 + 4 * g);
          sb[b][4 * q4 + 0] = __builtin_fmaf(sb[b][4 * q4 + 0], c, bb.x);
          sb[b][4 * q4 + 1] = __builtin_fmaf(sb[b][4 * q4 + 1], c, bb.y);
          sb[b][4 * q4 + 2] = __builtin_fmaf(sb[b][4 * q4 + 2], c, bb.z);
          sb[b][4 * q4 + 3] = __builtin_fmaf(sb[b][4 * q4 + 3], c, bb.w);
        }
    }
    const float cs = BIAS ? 1.0f : c;
    // ---- P = exp2(S*c - mref) in bf16 and its row sum, against the current reference.
    bf16x8 pb[2 * KB];
    float ts;
    auto probs = [&]() {
      float part[2 * KB];
#pragma unroll
      for (int j = 0; j < 2 * KB; ++j) {
        float e[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb[j >> 1][8 * (j & 1) + r], cs, -mref));
#pragma unroll
        for (int r = 0; r < 8; ++r) pb[j][r] = (__bf16)e[r];
        part[j] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      }
      ts = part[0];
#pragma unroll
      for (int j = 1; j < 2 * KB; ++j) ts += part[j];
    };
    probs();
    // ---- the reference moves only when some p left its range, and on the unit's first
    // tile (the reference is -inf before it; masked keys there give NaN p, discarded here).
    if (tile == t0 || __any(ts > kSumLimit)) {
      float mt = fmaxf(sb[0][0], sb[0][1]);
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mt = max3(mt, sb[b][r], sb[b][r + 1]);
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
    // V^T operands VPF ahead of their MFMA (operand i = d block i / (2 KB), k-step i % (2 KB)).
    {
      auto vload = [&](const int i) {
        const int db = i / (2 * KB), j = i % (2 * KB);
        const int roff = (32 * (j >> 1) + 16 * (j & 1)) * T::ROW;
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + vaddr[db] + roff));
        const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + vaddr[db] + roff + 8 * T::ROW));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 av[NPV];
#pragma unroll
      for (int i = 0; i < VPF; ++i) av[i] = vload(i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i + VPF < NPV) av[i + VPF] = vload(i + VPF);
        o[i / (2 * KB)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], pb[i % (2 * KB)], o[i / (2 * KB)], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * VPF, 0);
#pragma unroll
      for (int i = 0; i < NPV - VPF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, VPF, 0);
    }
  };

  // Pipeline: tile i is computed from stage i&1 while tile i+1 lands in the other stage;
  // the barrier after each compute waits for this wave's transfers (and the stage's bias
  // store) and for every wave to be done with the stage the next step refills.
  float bra = 0.0f, brb = 0.0f;  // this thread's key bias of each stage (BIAS only)
  dma_tile(t0, st_a, bra);
  store_bias(st_a, bra);
  __syncthreads();
  for (int tile = t0; tile < t1; tile += 2) {
    // Issue priority from progress through the unit's tiles, 3 in the first quarter down to
    // 0 in the last: the workgroups sharing a CU then keep level (the arbiter otherwise
    // favours the one dispatched first, and the last one to finish sets the launch's time).
    {
      const int q = (4 * (tile - t0)) / (t1 - t0);
      if (q <= 0) __builtin_amdgcn_s_setprio(3);
      else if (q == 1) __builtin_amdgcn_s_setprio(2);
      else if (q == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    if (tile + 1 < t1) dma_tile(tile + 1, st_b, brb);
    if (wave_on) compute_tile(tile, st_a);
    if (tile + 1 < t1) store_bias(st_b, brb);
    __syncthreads();
    if (tile + 1 >= t1) break;
    if (tile + 2 < t1) dma_tile(tile + 2, st_a, bra);
    if (wave_on) compute_tile(tile + 1, st_b);
    if (tile + 2 < t1) store_bias(st_a, bra);
    __syncthreads();
  }

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

// Merge key splits: D/4 threads per (row, head), one float4 of the output each, so a
// workgroup covers 256/(D/4) (row, head) pairs with 16-byte loads.  Every split's partial
// (reference max, row sum, numerators) is loaded before the first use, so a thread has all
// its loads in flight at once.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const AttnLaunch a) {
  constexpr int TPP = D / 4;        // threads per (row, head) pair
  constexpr int PPW = 256 / TPP;    // pairs per workgroup
  const AttnSession& S = a.s[wg_y()];
  if (S.split <= 1) return;
  const int H = a.n_heads;
  const int idx = wg_x() * PPW + tid_x() / TPP;
  if (idx >= S.rows * H) return;
  const int d4 = (tid_x() % TPP) * 4;
  const size_t slice = (size_t)S.rows * H;  // (row, head) pairs per split
  const int split = S.split;                // <= kMaxSplit
  float m[kMaxSplit], l[kMaxSplit];
  float4 po[kMaxSplit];
#pragma unroll
  for (int k = 0; k < kMaxSplit; ++k) {
    m[k] = -INFINITY;
    l[k] = 0.0f;
    po[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (k < split) {
      const float2 ml = *reinterpret_cast<const float2*>(S.part_ml + (k * slice + idx) * 2);
      m[k] = ml.x;
      l[k] = ml.y;
      po[k] = *reinterpret_cast<const float4*>(S.part_o + (k * slice + idx) * D + d4);
    }
  }
  float mmax = m[0];
#pragma unroll
  for (int k = 1; k < kMaxSplit; ++k) mmax = fmaxf(mmax, m[k]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lt = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxSplit; ++k) {
    const float wgt = __builtin_amdgcn_exp2f(m[k] - mmax);  // 0 for the splits past `split`
    lt += wgt * l[k];
    acc = make_float4(acc.x + wgt * po[k].x, acc.y + wgt * po[k].y, acc.z + wgt * po[k].z, acc.w + wgt * po[k].w);
  }
  const float inv = 1.0f / lt;
  *reinterpret_cast<float4*>(S.out + (size_t)idx * D + d4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
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
  if (a.head_dim == 64)
    launch(combine_kernel<64>, dim3((max_pairs + 15) / 16, a.n_sessions), dim3(256), stream, a);
  else if (a.head_dim == 128)
    launch(combine_kernel<128>, dim3((max_pairs + 7) / 8, a.n_sessions), dim3(256), stream, a);
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
