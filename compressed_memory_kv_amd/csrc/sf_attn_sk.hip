// The dense read of the per-block memory, head_dim 64, as a persistent
// stream-K kernel for gfx950.
//
// Model card "GTA world model: weights and inference code", sections "What a
// frame attends to" and "One buffer, no mask": every row of frame t's record
// attends, with no mask, to every filled row of the block's K/V buffer:
//     O[i,h] = sum_j softmax_j(scale * <Q[i,h], K[j,h]>) V[j,h]
// The filled rows are at most a few contiguous segments; the kernel walks them
// as one flattened key sequence (addressing, not masking).
//
// Work decomposition.  A unit is (session, head, 128-row query tile); its work
// is ceil(keys/64) iterations of 64 keys.  The iterations of all units of the
// launch, in order, are cut into G equal contiguous ranges, one per persistent
// workgroup (G = number of CUs, one 8-wave workgroup per CU).  Consecutive
// ranges share a head, and the grid is remapped so each XCD (the hardware deals
// workgroups round robin over the 8 XCDs) owns a contiguous eighth: a head's K/V
// stays in one XCD's L2.  The part of a unit inside one workgroup's range is a
// "piece".  A piece that is the whole unit writes the output; otherwise it
// writes an unnormalised partial (O, reference max, row sum) to the session's
// scratch and combine_sk_kernel merges the pieces of the unit.
//
// Inside a workgroup.  Eight waves = four key streams x two waves.  The piece's
// tiles are cut into four contiguous quarters, one per stream; the two waves of
// a stream hold 64 query rows each (two 32-row MFMA blocks), so every K/V
// operand read from LDS feeds two MFMAs.  Per stream, K and V tiles go from
// global memory straight into LDS (global_load_lds_dwordx4: no staging VGPRs)
// into two stages, kept as two separate LDS arrays so the compiler can tell the
// tile in flight from the tile being read; the next tile's transfer overlaps
// the current tile's compute and the barrier ending each step waits for it.
// At the end of a piece the four streams are merged through LDS.
//
// Per tile and wave, in two halves of 32 keys:
//   S^T (32 keys x 32 queries, per query block) = K . Q^T on
//     v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q in VGPRs), so each
//     lane owns one query and 16 of its scores;
//   P = exp2(S * scale*log2e - mref) in fp32, rounded to bf16, and its row sum
//     taken from the rounded values (v_dot2_f32_bf16 against ones).  The
//     reference mref moves only when some p of the half would exceed 2^15 (a
//     wave-uniform test on the sums) and on a stream's first half-tile: then
//     the true max of the half is taken and O and the sum are rescaled.  Exact
//     softmax either way, up to rounding;
//   O^T (64 x 32 queries, per query block) += V^T . P^T on the same MFMA; V^T
//     comes from the row-major V tile through ds_read_b64_tr_b16.
#include "sf_internal.h"

#include <cmath>

namespace sf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int D = 64;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStreams = 4;
constexpr int kStreamThreads = kThreads / kStreams;  // 128
constexpr int BN = kSkKeys;
constexpr int ROW = 2 * D;                            // bytes per K/V row
constexpr int TILE = BN * ROW;                        // 8 KB
constexpr int STAGE = 2 * TILE;                       // K tile then V tile
constexpr int STAGE_ALL = kStreams * STAGE;          // one stage of every stream (64 KB)
constexpr int DMA_ROWS = 8;                           // rows one wave-wide 1 KB transfer covers
constexpr int DMA_PER_WAVE = BN / DMA_ROWS / 2;       // transfers per wave per tensor per tile (4)
constexpr float kSumLimit = 32768.0f;
// Stream merge buffer: 3 streams x 2 waves x 64 lanes x (64 O + 2 m + 2 l) floats,
// slots 0-2 in stage array a, 3-5 in stage array b.
constexpr int MERGE_FLOATS = 68;
constexpr int MERGE_SLOT = 64 * MERGE_FLOATS * 4;
static_assert(3 * MERGE_SLOT <= STAGE_ALL, "three merge slots fit in one stage array");

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Workgroup holding iteration i when N iterations are cut into G ranges.
__device__ __forceinline__ int wg_of_iter(long long i, int G, int N) {
  return (int)(((i + 1) * G - 1) / N);
}

__device__ __forceinline__ int session_of_iter(const SkLaunch& a, int it) {
  int si = 0;
  for (int i = 1; i < a.n_sessions; ++i)
    if (a.s[i].it_begin <= it) si = i;
  return __builtin_amdgcn_readfirstlane(si);
}

typedef __attribute__((address_space(3))) void lds_void;

__global__ __launch_bounds__(kThreads) void attn_sk_kernel(const SkLaunch a) {
  __shared__ __attribute__((aligned(16))) char st_a[STAGE_ALL];  // stage 0 of each stream
  __shared__ __attribute__((aligned(16))) char st_b[STAGE_ALL];  // stage 1 of each stream
  const int G = a.n_wg;
  const int N = a.n_iters;
  const int w = (G & 7) == 0 ? (int)(blockIdx.x & 7u) * (G >> 3) + (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int it_lo = __builtin_amdgcn_readfirstlane((int)((long long)w * N / G));
  const int it_hi = __builtin_amdgcn_readfirstlane((int)((long long)(w + 1) * N / G));
  const int H = a.n_heads;
  const float c = a.scale_log2;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int stream = wave >> 1;   // key stream
  const int hw = wave & 1;        // which 64 query rows of the unit
  const int lane = tid & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int soff = stream * STAGE;  // this stream's stage within a stage array

  // Stage layout (as in sf_attn.hip): K chunk c of row r sits at c ^ (r & 7), V chunk c
  // at c ^ 2*(r & 3).  A wave-wide transfer fills 1 KB = 8 rows, lane L landing at
  // row L/8, position L%8, so lane L fetches the logical chunk that belongs there
  // (both swizzles are involutions).  Rows of a tile differ by multiples of 8 between
  // a wave's transfers, so the chunk a lane fetches is the same for all of them.
  const int drow = lane >> 3;                                  // row within a transfer
  const int kchunk = (lane & 7) ^ drow;                        // K: p ^ (r & 7)
  const int vchunk = (lane & 7) ^ (2 * (drow & 3));            // V: p ^ 2*(r & 3)
  const int trow0 = hw * DMA_PER_WAVE * DMA_ROWS + drow;       // tile row of transfer 0
  int kaddr[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) kaddr[kk] = l32 * ROW + (((2 * kk + g) ^ (l32 & 7)) << 4);
  const int trow = (lane >> 2) & 3;
  int vaddr[2];
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    vaddr[db] = TILE + (4 * g + trow) * ROW + ((chunk ^ (2 * trow)) << 4) + 8 * (lane & 1);
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  for (int it = it_lo; it < it_hi;) {
    // ---- the piece: one unit's tiles [tile0, tile1) inside this workgroup's range
    const int si = session_of_iter(a, it);
    const SkSession& S = a.s[si];
    const int nt = S.ntiles;
    const int local = it - S.it_begin;
    const int u = __builtin_amdgcn_readfirstlane(local / nt);
    const int tile0 = __builtin_amdgcn_readfirstlane(local - u * nt);
    const int tile1 = min(nt, tile0 + (it_hi - it));
    const int qt = __builtin_amdgcn_readfirstlane(u % S.qtiles);
    const int h = __builtin_amdgcn_readfirstlane(u / S.qtiles);
    const int key_hi = min(tile1 * BN, S.n_keys);
    const int n = tile1 - tile0;
    const int s_lo = tile0 + (stream * n) / kStreams;
    const int s_hi = tile0 + ((stream + 1) * n) / kStreams;
    const int steps = (n + kStreams - 1) / kStreams;
    const int row_stride = H * D;
    const int row_bytes = 2 * row_stride;
    const int qrow0 = qt * kSkRows + hw * 64;
    const bool wave_on = qrow0 < S.rows;

    int seg_row[SF_MAX_SEGMENTS], seg_key[SF_MAX_SEGMENTS];
    {
      int cum = 0;
#pragma unroll
      for (int i = 0; i < SF_MAX_SEGMENTS; ++i) {
        const bool used = i < S.n_seg;
        seg_row[i] = used ? S.seg_begin[i] : 0;
        seg_key[i] = used ? cum : 0x7fffffff;
        cum += used ? S.seg_len[i] : 0;
      }
    }

    // Q^T operands: query block qb holds rows qrow0 + 32*qb + l32 (rows past R read row R-1).
    bf16x8 qreg[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = min(qrow0 + 32 * qb + l32, S.rows - 1);
      const __bf16* qp = reinterpret_cast<const __bf16*>(S.q) + row * row_stride + h * D + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qreg[qb][kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
    }

    const char* __restrict__ kg = reinterpret_cast<const char*>(S.k) + 2 * h * D;
    const char* __restrict__ vg = reinterpret_cast<const char*>(S.v) + 2 * h * D;

    // Starts the transfer of this stream's tile TL into stage array ST (this wave's
    // half: rows [32*hw, 32*hw+32) of K and of V).  A tile inside one segment is a
    // run of rows (scalar base + fixed lane offsets); otherwise rows are looked up
    // per lane, and keys past the piece's range re-read its last key (finite data
    // that gets score -inf).
    auto dma_tile = [&](const int tl, char* st) {
      const int kap0 = tl * BN;
      int srow = seg_row[0], skey = seg_key[0], send = seg_key[1];
#pragma unroll
      for (int i = 1; i < SF_MAX_SEGMENTS; ++i) {
        const bool in = kap0 >= seg_key[i];
        srow = in ? seg_row[i] : srow;
        skey = in ? seg_key[i] : skey;
        send = in ? (i + 1 < SF_MAX_SEGMENTS ? seg_key[i + 1 < SF_MAX_SEGMENTS ? i + 1 : i] : 0x7fffffff) : send;
      }
      char* kdst = st + soff + (trow0 - drow) * ROW;
      char* vdst = kdst + TILE;
      if (kap0 + BN <= min(send, key_hi)) {
        const unsigned base = (unsigned)((srow + kap0 - skey + trow0) * row_bytes);
#pragma unroll
        for (int m = 0; m < DMA_PER_WAVE; ++m) {
          const unsigned rb = base + (unsigned)(m * DMA_ROWS * row_bytes);
          __builtin_amdgcn_global_load_lds(kg + rb + kchunk * 16, (lds_void*)(kdst + m * DMA_ROWS * ROW), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vg + rb + vchunk * 16, (lds_void*)(vdst + m * DMA_ROWS * ROW), 16, 0, 0);
        }
      } else {
#pragma unroll
        for (int m = 0; m < DMA_PER_WAVE; ++m) {
          const int kappa = min(kap0 + trow0 + m * DMA_ROWS, key_hi - 1);
          int row = seg_row[0] + kappa;
#pragma unroll
          for (int i = 1; i < SF_MAX_SEGMENTS; ++i)
            row = kappa >= seg_key[i] ? seg_row[i] + (kappa - seg_key[i]) : row;
          const unsigned rb = (unsigned)(row * row_bytes);
          __builtin_amdgcn_global_load_lds(kg + rb + kchunk * 16, (lds_void*)(kdst + m * DMA_ROWS * ROW), 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vg + rb + vchunk * 16, (lds_void*)(vdst + m * DMA_ROWS * ROW), 16, 0, 0);
        }
      }
    };

    f32x16 o[2][2];  // [d block][query block]
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][qb][r] = 0.0f;
    float mref[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.0f, 0.0f};

    // One 64-key tile of this stream from stage array STA.
    auto compute_tile = [&](const int tl, const char* sta) {
      const char* st = sta + soff;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        // S^T for keys 32*kh .. 32*kh+31 of the tile, both query blocks
        f32x16 s[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[0][r] = 0.0f; s[1][r] = 0.0f; }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(st + kaddr[kk] + kh * 32 * ROW);
          s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[0][kk], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[1][kk], s[1], 0, 0, 0);
        }
        if (tl * BN + 32 * kh + 32 > key_hi) {  // ragged end of the piece
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = tl * BN + 32 * kh + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= key_hi) { s[0][r] = -INFINITY; s[1][r] = -INFINITY; }
          }
        }
        bf16x8 pb[2][2];
        float ts[2];
        auto probs = [&]() {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              pb[qb][0][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c, -mref[qb]));
              pb[qb][1][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][8 + r], c, -mref[qb]));
            }
            float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bf16x2 a0 = {pb[qb][0][2 * e], pb[qb][0][2 * e + 1]};
              const bf16x2 a1 = {pb[qb][1][2 * e], pb[qb][1][2 * e + 1]};
              p0 = __builtin_amdgcn_fdot2_f32_bf16(a0, ones, p0, false);
              p1 = __builtin_amdgcn_fdot2_f32_bf16(a1, ones, p1, false);
            }
            ts[qb] = p0 + p1;
          }
        };
        probs();
        // The first half-tile of a stream always sets the reference (it is -inf before,
        // so masked keys there give NaN p, which this path discards).  Later sums are
        // finite or +inf, never NaN.
        const bool first = tl == s_lo && kh == 0;
        if (first || __any(ts[0] > kSumLimit || ts[1] > kSumLimit)) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            float mt = fmaxf(s[qb][0], s[qb][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) mt = max3(mt, s[qb][r], s[qb][r + 1]);
            mt = fmaxf(mt, xor32(mt)) * c;
            const float mnew = fmaxf(mref[qb], mt);
            const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mnew);
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
            lsum[qb] *= alpha;
            mref[qb] = mnew;
          }
          probs();
        }
        lsum[0] += ts[0];
        lsum[1] += ts[1];
        // O^T += V^T . P^T over this half's two 16-key k-steps
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int roff = (32 * kh + 16 * j) * ROW;
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + vaddr[db] + roff));
            const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + vaddr[db] + roff + 8 * ROW));
            const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[0][j], o[db][0], 0, 0, 0);
            o[db][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[1][j], o[db][1], 0, 0, 0);
          }
        }
      }
    };

    // ---- pipeline over this stream's tiles [s_lo, s_hi): all waves take `steps` steps.
    // Each step computes one stage while the next tile flows into the other; the
    // barrier that ends the step also waits for that transfer.
    if (s_lo < s_hi) dma_tile(s_lo, st_a);
    __syncthreads();
    for (int i = 0; i < steps; i += 2) {
      const int tl = s_lo + i;
      if (tl + 1 < s_hi) dma_tile(tl + 1, st_b);
      if (tl < s_hi && wave_on) compute_tile(tl, st_a);
      __syncthreads();
      if (i + 1 >= steps) break;
      if (tl + 2 < s_hi) dma_tile(tl + 2, st_a);
      if (tl + 1 < s_hi && wave_on) compute_tile(tl + 1, st_b);
      __syncthreads();
    }

    // ---- merge the four streams (stream 0 collects), then write
    auto merge_slot = [&](const int sl) -> float* {
      return reinterpret_cast<float*>((sl < 3 ? st_a : st_b) + (sl % 3) * MERGE_SLOT) + lane * MERGE_FLOATS;
    };
    if (stream > 0 && wave_on) {
      float* dst = merge_slot((stream - 1) * 2 + hw);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; r += 4)
            *reinterpret_cast<float4*>(dst + (db * 2 + qb) * 16 + r) =
                make_float4(o[db][qb][r], o[db][qb][r + 1], o[db][qb][r + 2], o[db][qb][r + 3]);
      *reinterpret_cast<float4*>(dst + 64) = make_float4(mref[0], mref[1], lsum[0], lsum[1]);
    }
    __syncthreads();
    if (stream == 0 && wave_on) {
      float mx[2] = {mref[0], mref[1]};
#pragma unroll
      for (int s2 = 0; s2 < 3; ++s2) {
        const float4 ml = *reinterpret_cast<const float4*>(merge_slot(s2 * 2 + hw) + 64);
        mx[0] = fmaxf(mx[0], ml.x);
        mx[1] = fmaxf(mx[1], ml.y);
      }
      float sc0[2] = {__builtin_amdgcn_exp2f(mref[0] - mx[0]), __builtin_amdgcn_exp2f(mref[1] - mx[1])};
      float l[2] = {lsum[0] * sc0[0], lsum[1] * sc0[1]};
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][qb][r] *= sc0[qb];
#pragma unroll 1
      for (int s2 = 0; s2 < 3; ++s2) {  // one stream at a time keeps the live set small
        const float* src = merge_slot(s2 * 2 + hw);
        const float4 ml = *reinterpret_cast<const float4*>(src + 64);
        const float f0 = __builtin_amdgcn_exp2f(ml.x - mx[0]);
        const float f1 = __builtin_amdgcn_exp2f(ml.y - mx[1]);
        l[0] += ml.z * f0;
        l[1] += ml.w * f1;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
              const float4 x = *reinterpret_cast<const float4*>(src + (db * 2 + qb) * 16 + r);
              const float f = qb == 0 ? f0 : f1;
              o[db][qb][r] += f * x.x;
              o[db][qb][r + 1] += f * x.y;
              o[db][qb][r + 2] += f * x.z;
              o[db][qb][r + 3] += f * x.w;
            }
      }
      const float lt[2] = {l[0] + xor32(l[0]), l[1] + xor32(l[1])};
      const bool whole = tile0 == 0 && tile1 == nt;
      // piece slot of this unit: its k-th workgroup writes slot k
      const int k = w - wg_of_iter((long long)S.it_begin + (long long)u * nt, G, N);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int row = qrow0 + 32 * qb + l32;
        if (row >= S.rows) continue;
        if (whole) {
          const float inv = 1.0f / lt[qb];
          float* op = S.out + row * row_stride + h * D;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              *reinterpret_cast<float4*>(op + 32 * db + 8 * q4 + 4 * g) =
                  make_float4(o[db][qb][4 * q4] * inv, o[db][qb][4 * q4 + 1] * inv, o[db][qb][4 * q4 + 2] * inv,
                              o[db][qb][4 * q4 + 3] * inv);
        } else {
          const size_t slot = (size_t)u * S.ppu + k;
          const int rin = row - qt * kSkRows;
          float* po = S.part_o + (slot * kSkRows + rin) * D;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              *reinterpret_cast<float4*>(po + 32 * db + 8 * q4 + 4 * g) =
                  make_float4(o[db][qb][4 * q4], o[db][qb][4 * q4 + 1], o[db][qb][4 * q4 + 2], o[db][qb][4 * q4 + 3]);
          if (g == 0) *reinterpret_cast<float2*>(S.part_ml + (slot * kSkRows + rin) * 2) = make_float2(mx[qb], lt[qb]);
        }
      }
    }
    __syncthreads();  // the merge buffer overlays the stages of the next piece
    it += tile1 - tile0;
  }
}

// Merges the pieces of every unit that spans several workgroups.  One workgroup
// per unit; thread t owns 8 float4 of the unit's 128 x 64 output (rows
// t/16 + 16*i, columns 4*(t%16)).  Pieces are folded in one pass with a running
// max, and each piece's loads for all 8 elements are issued together, so a unit
// costs one global round trip per piece.
constexpr int kCombThreads = 256;
constexpr int kCombPer = kSkRows * (D / 4) / kCombThreads;  // 8
__global__ __launch_bounds__(kCombThreads) void combine_sk_kernel(const SkLaunch a, int total_units) {
  const int ug = blockIdx.x;
  if (ug >= total_units) return;
  int si = 0, ubase = 0;
  {
    int acc = 0;
    for (int i = 0; i < a.n_sessions; ++i) {
      if (ug >= acc) { si = i; ubase = acc; }
      acc += a.n_heads * a.s[i].qtiles;
    }
  }
  si = __builtin_amdgcn_readfirstlane(si);
  ubase = __builtin_amdgcn_readfirstlane(ubase);
  const SkSession& S = a.s[si];
  const int u = ug - ubase;
  const int G = a.n_wg, N = a.n_iters;
  const long long first = (long long)S.it_begin + (long long)u * S.ntiles;
  const int wl = wg_of_iter(first, G, N);
  const int wh = wg_of_iter(first + S.ntiles - 1, G, N);
  if (wl == wh) return;  // written whole by one workgroup
  const int pieces = wh - wl + 1;
  const int qt = u % S.qtiles, h = u / S.qtiles;
  const int H = a.n_heads;
  const int r0 = threadIdx.x / (D / 4);
  const int d4 = (threadIdx.x % (D / 4)) * 4;
  constexpr int RSTRIDE = kCombThreads / (D / 4);  // 16 rows between a thread's elements
  float mx[kCombPer], l[kCombPer];
  float4 acc[kCombPer];
#pragma unroll
  for (int i = 0; i < kCombPer; ++i) {
    mx[i] = -INFINITY;
    l[i] = 0.0f;
    acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int k = 0; k < pieces; ++k) {
    const size_t slot = (size_t)u * S.ppu + k;
    float2 ml[kCombPer];
    float4 x[kCombPer];
#pragma unroll
    for (int i = 0; i < kCombPer; ++i) {
      const int rin = r0 + RSTRIDE * i;
      ml[i] = *reinterpret_cast<const float2*>(S.part_ml + (slot * kSkRows + rin) * 2);
      x[i] = *reinterpret_cast<const float4*>(S.part_o + (slot * kSkRows + rin) * D + d4);
    }
#pragma unroll
    for (int i = 0; i < kCombPer; ++i) {
      const float mn = fmaxf(mx[i], ml[i].x);
      const float fo = __builtin_amdgcn_exp2f(mx[i] - mn);  // mx = -inf on the first piece: 0
      const float fn = __builtin_amdgcn_exp2f(ml[i].x - mn);
      l[i] = l[i] * fo + ml[i].y * fn;
      acc[i] = make_float4(acc[i].x * fo + x[i].x * fn, acc[i].y * fo + x[i].y * fn, acc[i].z * fo + x[i].z * fn,
                           acc[i].w * fo + x[i].w * fn);
      mx[i] = mn;
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
  const int64_t nt = (capacity_rows + kSkKeys - 1) / kSkKeys;
  return (int32_t)((nt + kSkMinRange - 1) / kSkMinRange + 2);
}

size_t sk_scratch_bytes(int64_t rows, int n_heads, int64_t capacity_rows) {
  const int64_t units = (int64_t)n_heads * ((rows + kSkRows - 1) / kSkRows);
  return (size_t)units * sk_pieces_per_unit(capacity_rows) * kSkRows * (D + 2) * sizeof(float);
}

hipError_t launch_attend_sk(const SkLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL(attn_sk_kernel, dim3(a.n_wg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine_sk(const SkLaunch& a, int total_units, hipStream_t stream) {
  hipLaunchKernelGGL(combine_sk_kernel, dim3(total_units), dim3(kCombThreads), 0, stream, a, total_units);
  return hipGetLastError();
}

}  // namespace sf
