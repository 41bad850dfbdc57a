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
//
// fp32 kernel (attn_f32_kernel<D>): one thread per query row, K/V tiles of a
//   few keys broadcast from LDS, exact online softmax in fp32 on VALU.
#include "sf_internal.h"

#include <cmath>

namespace sf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int BM = kBf16RowsPerTile;  // 128 query rows per workgroup
constexpr int BN = kBf16KeysPerTile;  // 64 keys per tile
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the reference max moves
static_assert(BM == kWaves * 32, "one 32-row MFMA block per wave");

// Flattened key index -> buffer row, walking the readable segments in order.
__device__ __forceinline__ int key_row(const AttnSession& s, int kappa) {
  int r = kappa;
#pragma unroll
  for (int i = 0; i < SF_MAX_SEGMENTS; ++i) {
    if (i < s.n_seg) {
      if (r < s.seg_len[i]) return s.seg_begin[i] + r;
      r -= s.seg_len[i];
    }
  }
  return 0;  // not reached for kappa < n_keys
}

// Work unit of this workgroup: XCD-aware remap of blockIdx.x.
__device__ __forceinline__ int unit_of_block() {
  const int per_xcd = gridDim.x >> 3;  // grid is a multiple of 8
  return (int)(blockIdx.x & 7u) * per_xcd + (int)(blockIdx.x >> 3);
}

__device__ __forceinline__ int session_of_unit(const AttnLaunch& a, int unit) {
  int si = 0;
  for (int i = 1; i < a.n_sessions; ++i)
    if (a.s[i].unit_begin <= unit) si = i;
  return si;
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

template <int D>
struct Bf16Smem {
  uint4 k[2][BN * D / 8];  // [buffer][row * D/8 + swizzled 16-byte chunk]
  uint4 v[2][BN * D / 8];  // [buffer][row * D/8 + swizzled 16-byte chunk, 32-byte XOR]
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(const AttnLaunch a) {
  constexpr int CH = D / 8;                  // 16-byte chunks per K/V row
  constexpr int PER = BN * CH / kThreads;    // chunks per thread per tensor per tile
  constexpr int KSTEPS = D / 16;             // MFMA k-steps over head_dim
  constexpr int DBLK = D / 32;               // 32-row blocks of O^T
  static_assert(PER * kThreads == BN * CH, "tile loads divide evenly");
  __shared__ Bf16Smem<D> sm;

  const int unit = unit_of_block();
  if (unit >= a.total_units) return;
  const AttnSession& S = a.s[session_of_unit(a, unit)];
  const int H = a.n_heads;
  int local = unit - S.unit_begin;
  const int split = S.split;
  const int ks = local % split;
  local /= split;
  const int qt = local % S.qtiles;
  const int h = local / S.qtiles;
  const int ntiles = (S.n_keys + BN - 1) / BN;
  const int t0 = (int)((long long)ks * ntiles / split);
  const int t1 = (int)((long long)(ks + 1) * ntiles / split);
  const int key_hi = min(t1 * BN, S.n_keys);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 5;   // lane half: k-group of MFMA operands
  const int l32 = lane & 31; // query of this lane within the wave's block
  const int qrow = qt * BM + wave * 32 + l32;
  const bool row_ok = qrow < S.rows;
  const bool wave_on = qt * BM + wave * 32 < S.rows;
  const float c = a.scale_log2;

  const __bf16* __restrict__ kg = reinterpret_cast<const __bf16*>(S.k);
  const __bf16* __restrict__ vg = reinterpret_cast<const __bf16*>(S.v);
  const size_t row_stride = (size_t)H * D;

  // Q^T operand: lane holds Q[qrow][16*kk + 8*g .. +7] for every k-step.
  bf16x8 qreg[KSTEPS];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(S.q) + (size_t)qrow * row_stride + (size_t)h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (row_ok) {
        qreg[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qreg[kk][i] = (__bf16)0.0f;
      }
    }
  }

  uint4 kr[PER], vr[PER];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int ci = tid + p * kThreads;
      const int row = ci / CH;
      const int cc = ci % CH;
      const int kappa = tile * BN + row;
      if (kappa < key_hi) {
        const size_t off = (size_t)key_row(S, kappa) * row_stride + (size_t)h * D + cc * 8;
        kr[p] = *reinterpret_cast<const uint4*>(kg + off);
        vr[p] = *reinterpret_cast<const uint4*>(vg + off);
      } else {
        kr[p] = make_uint4(0u, 0u, 0u, 0u);
        vr[p] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int ci = tid + p * kThreads;
      const int row = ci / CH;
      const int cc = ci % CH;
      sm.k[buf][row * CH + (cc ^ (row & 7))] = kr[p];
      sm.v[buf][row * CH + ((((cc >> 1) ^ (row & 3)) << 1) | (cc & 1))] = vr[p];
    }
  };

  f32x16 o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float mref = -INFINITY;  // reference max, log2 units
  float lsum = 0.0f;       // this lane's share of the row sum

  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  if (t0 < t1) {
    load_tile(t0);
    store_tile(0);
  }
  __syncthreads();

  for (int tile = t0; tile < t1; ++tile) {
    const int buf = (tile - t0) & 1;
    const bool more = tile + 1 < t1;
    if (more) load_tile(tile + 1);

    if (wave_on) {
      const uint4* ks_lds = sm.k[buf];
      // ---- S^T = K . Q^T : two 32-key blocks
      f32x16 s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int ch = 2 * kk + g;
        const int r0 = l32, r1 = 32 + l32;
        const uint4 a0 = ks_lds[r0 * CH + (ch ^ (r0 & 7))];
        const uint4 a1 = ks_lds[r1 * CH + (ch ^ (r1 & 7))];
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), qreg[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), qreg[kk], s1, 0, 0, 0);
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
      // ---- tile max over this query's 64 scores (32 here, 32 in lane^32)
      float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
      mt = fmaxf(mt, xor32(mt)) * c;
      const bool need = mt > mref + kLazyRescale;
      if (__any(need)) {
        const float mnew = fmaxf(mref, mt);
        const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        lsum *= alpha;
        mref = mnew;
      }
      // ---- P = exp2(S*c - mref), rounded to bf16; row sum of the rounded values
      bf16x8 pb[4];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        pb[0][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c, -mref));
        pb[1][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s0[8 + r], c, -mref));
        pb[2][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c, -mref));
        pb[3][r] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s1[8 + r], c, -mref));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pr = {pb[j][2 * e], pb[j][2 * e + 1]};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
        }
      }
      // ---- O^T += V^T . P^T ; k-step j covers S^T registers 8*(j&1).. of block j>>1,
      // i.e. keys 32*(j>>1) + 16*(j&1) + {4g..4g+3} then {8+4g..8+4g+3}.
      const char* vs_lds = reinterpret_cast<const char*>(sm.v[buf]);
      const int trow = (lane >> 2) & 3;           // row within the 4-row group this lane addresses
      const int tcol = 4 * (lane & 3);            // column within the 16-column chunk
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const int chunk32 = 2 * db + ((lane >> 4) & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kb = 32 * (j >> 1) + 16 * (j & 1) + 4 * g;
          const int ra = kb + trow, rb = kb + 8 + trow;
          const int ea = ra * D + (((chunk32 ^ (ra & 3)) << 4) | tcol);
          const int eb = rb * D + (((chunk32 ^ (rb & 3)) << 4) | tcol);
          const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs_lds + 2 * ea));
          const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs_lds + 2 * eb));
          const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[j], o[db], 0, 0, 0);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_on) return;
  const float ltot = lsum + xor32(lsum);
  const size_t obase = (size_t)qrow * row_stride + (size_t)h * D;
  if (split == 1) {
    if (!row_ok) return;
    const float inv = 1.0f / ltot;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * g;
        float4 w = make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                               o[db][4 * q4 + 3] * inv);
        *reinterpret_cast<float4*>(S.out + obase + d) = w;
      }
  } else {
    if (!row_ok) return;
    float* po = S.part_o + (size_t)ks * S.rows * row_stride + obase;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * g;
        *reinterpret_cast<float4*>(po + d) =
            make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
      }
    if (g == 0) {
      float* pm = S.part_ml + ((size_t)ks * S.rows * H + (size_t)qrow * H + h) * 2;
      *reinterpret_cast<float2*>(pm) = make_float2(mref, ltot);
    }
  }
}

// Merge key splits: one wave per (row, head); lane covers D/64 output columns.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const AttnLaunch a) {
  const AttnSession& S = a.s[blockIdx.y];
  if (S.split <= 1) return;
  const int H = a.n_heads;
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (idx >= S.rows * H) return;
  const int lane = threadIdx.x & 63;
  const size_t slice = (size_t)S.rows * H;  // (row, head) pairs per split
  float mmax = -INFINITY;
  for (int k = 0; k < S.split; ++k) mmax = fmaxf(mmax, S.part_ml[(k * slice + idx) * 2]);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;
  float l = 0.0f;
  for (int k = 0; k < S.split; ++k) {
    const float2 ml = *reinterpret_cast<const float2*>(S.part_ml + (k * slice + idx) * 2);
    const float wgt = __builtin_amdgcn_exp2f(ml.x - mmax);
    l += wgt * ml.y;
    const float* po = S.part_o + (k * slice + idx) * D;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] += wgt * po[lane + 64 * j];
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int j = 0; j < PER; ++j) S.out[(size_t)idx * D + lane + 64 * j] = acc[j] * inv;
}

// ---------------------------------------------------------------- fp32 path
constexpr int kF32Threads = kF32RowsPerTile;

template <int D>
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(const AttnLaunch a) {
  constexpr int KT = D <= 64 ? 16 : 8;  // keys per LDS tile
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const int unit = (int)blockIdx.x;
  if (unit >= a.total_units) return;
  const AttnSession& S = a.s[session_of_unit(a, unit)];
  const int H = a.n_heads;
  const int local = unit - S.unit_begin;
  const int qt = local % S.qtiles;
  const int h = local / S.qtiles;
  const int tid = threadIdx.x;
  const int qrow = qt * kF32RowsPerTile + tid;
  const bool row_ok = qrow < S.rows;
  const size_t row_stride = (size_t)H * D;
  const float* __restrict__ kg = reinterpret_cast<const float*>(S.k);
  const float* __restrict__ vg = reinterpret_cast<const float*>(S.v);
  const float c = a.scale_log2;

  float q[D], o[D];
  {
    const float* qp = reinterpret_cast<const float*>(S.q) + (size_t)(row_ok ? qrow : 0) * row_stride + (size_t)h * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      q[d] = row_ok ? qp[d] : 0.0f;
      o[d] = 0.0f;
    }
  }
  float m = -INFINITY, l = 0.0f;
  for (int base = 0; base < S.n_keys; base += KT) {
    for (int e = tid; e < KT * D; e += kF32Threads) {
      const int j = e / D, d = e % D;
      const int kappa = base + j;
      float kv = 0.0f, vv = 0.0f;
      if (kappa < S.n_keys) {
        const size_t off = (size_t)key_row(S, kappa) * row_stride + (size_t)h * D + d;
        kv = kg[off];
        vv = vg[off];
      }
      ks[j][d] = kv;
      vs[j][d] = vv;
    }
    __syncthreads();
    float s[KT];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float acc = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], ks[j][d], acc);
      s[j] = (base + j < S.n_keys) ? acc * c : -INFINITY;
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
  float* op = S.out + (size_t)qrow * row_stride + (size_t)h * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
}

int round_up8(int n) { return (n + 7) & ~7; }

}  // namespace

size_t attend_scratch_bytes(int64_t rows, int n_heads, int head_dim) {
  return (size_t)kMaxSplit * (size_t)rows * (size_t)n_heads * ((size_t)head_dim + 2) * sizeof(float);
}

hipError_t launch_attend_bf16(const AttnLaunch& a, hipStream_t stream) {
  const int grid = round_up8(a.total_units);
  if (a.head_dim == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
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
    hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, stream, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attend_f32(const AttnLaunch& a, hipStream_t stream) {
  if (a.head_dim == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(a.total_units), dim3(kF32Threads), 0, stream, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(a.total_units), dim3(kF32Threads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sf
