// Device pieces shared by the decode kernels: wave reductions, the split
// records and the chunked float32 online-softmax pass.
#pragma once

#include "lrkv_internal.h"

namespace lrkv {

constexpr float kNegInf = -__builtin_huge_valf();

// word 3 of a raw buffer resource on gfx9-family parts (32-bit data format)
constexpr int kBufferWord3 = 0x00020000;

// one element of storage type T at a byte offset of a buffer resource
template <typename T> __device__ __forceinline__ float buffer_elem(__amdgpu_buffer_rsrc_t r, int off);
template <> __device__ __forceinline__ float buffer_elem<float>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <> __device__ __forceinline__ float buffer_elem<bf16_t>(__amdgpu_buffer_rsrc_t r, int off) {
  return to_f32(bf16_t(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)));
}

// 2^x with the hardware exp2 (v_exp_f32): results below 2^-126 flush to zero,
// 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Wave reductions without the LDS crossbar: rotations inside each 16-lane row
// (DPP row_ror), then the four rows' results taken by readlane.  Every lane gets
// the result; the order of the operations is fixed.
template <int N> __device__ __forceinline__ float dpp_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_of(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_ror<8>(v));
  v = fmaxf(v, dpp_ror<4>(v));
  v = fmaxf(v, dpp_ror<2>(v));
  v = fmaxf(v, dpp_ror<1>(v));
  return fmaxf(fmaxf(lane_of(v, 0), lane_of(v, 16)), fmaxf(lane_of(v, 32), lane_of(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_ror<8>(v);
  v += dpp_ror<4>(v);
  v += dpp_ror<2>(v);
  v += dpp_ror<1>(v);
  return (lane_of(v, 0) + lane_of(v, 16)) + (lane_of(v, 32) + lane_of(v, 48));
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48) with this part's row-swapping permutes: permlane16_swap of a value
// with itself leaves each lane holding its own row's value and its row
// partner's (rows 0 <-> 1, 2 <-> 3) in the two results, permlane32_swap the
// same for the wave's halves.  No LDS round trip; every lane gets the same
// bits (the operations are commutative and the association is the same).
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// The work item of stage-1 workgroup (blockIdx.x, blockIdx.y) of a
// (row_items, batch) grid: batch row b, latent group h, split s of its S_h.
// Workgroup i of a launch runs on XCD i % 8, each XCD with its own L2: when the
// items divide by 8, XCD x takes the x-th eighth of the item list, so the splits
// of a (row, group) unit -- which share its query, U_K and anchor rows -- land on
// one XCD (a unit may straddle two eighths).
struct WorkItem {
  int b, h, split, S;
};
// The group is found without a loop of dependent reads: with uniform splits by a
// division, otherwise by counting, over every entry of split0 at once (scalar
// reads that issue together), the groups h >= 1 whose first item is <= r.
__device__ __forceinline__ WorkItem work_item(const LayerArgs &L, const DecodeArgs &d) {
  const int i = blockIdx.x + d.row_items * blockIdx.y;
  const int j = (d.items & 7) == 0 ? (i & 7) * (d.items >> 3) + (i >> 3) : i;
  WorkItem w;
  w.b = j / d.row_items;
  const int r = j - w.b * d.row_items;
  int h = 0;
  if (d.uniform) {
    h = r / d.n_splits;
  } else {
#pragma unroll
    for (int k = 1; k < 16; ++k) h += (k < L.n_lat && d.split0[k] <= r) ? 1 : 0;
    if (L.n_lat > 16) {
#pragma unroll
      for (int k = 16; k < LRKV_MAX_KV_HEADS; ++k) h += (k < L.n_lat && d.split0[k] <= r) ? 1 : 0;
    }
  }
  w.h = h;
  w.split = r - d.split0[h];
  w.S = d.nsplit[h];
  return w;
}

// record of query head qi = b * n_q + i for split s
__device__ __forceinline__ float *split_record(const DecodeArgs &d, int64_t qi, int split) {
  return d.ws + (qi * d.n_splits + split) * d.rec;
}

// anchor rows [lo, hi) of split s out of a anchors: consecutive runs of at
// least 16 rows on the first splits, so most splits carry no anchors at all
constexpr int kMinAnchorRows = 16;
__host__ __device__ __forceinline__ int anchor_rows_per_split(int a, int S) {
  const int even = (a + S - 1) / S;
  return even > kMinAnchorRows ? even : kMinAnchorRows;
}
__device__ __forceinline__ void anchor_share(int a, int split, int S, int &lo, int &hi) {
  const int per = anchor_rows_per_split(a, S);
  lo = min(split * per, a);
  hi = min(lo + per, a);
}

// Basis versions: the code blocks of a row form one segment per version
// (version v owns blocks [B_v, B_v+1), B_v = its first slot / 32, clamped to the
// row's nblk), and the S splits are shared out so that every version has at
// least one: version v's splits start at P_v = v + (S - V) B_v / nblk.
struct SplitSeg {
  int v;        // basis version
  int s, ns;    // split index inside the version, splits of the version
  int lo, hi;   // code blocks [lo, hi) of the version
};
__device__ __forceinline__ SplitSeg split_segment(const LayerArgs &L, int b, int split, int S, int nblk) {
  SplitSeg g{0, split, S, 0, nblk};
  const int V = L.n_versions;
  if (V <= 1) return g;
  const int32_t *vs = L.vstart + int64_t(b) * V;
  auto blk = [&](int v) {  // B_v, non-decreasing, in [0, nblk]
    if (v <= 0) return 0;
    if (v >= V) return nblk;
    int bv = vs[v] / kBlock;
    return bv < 0 ? 0 : (bv > nblk ? nblk : bv);
  };
  auto first = [&](int v) {
    if (v >= V) return S;
    return v + int((int64_t(S - V) * blk(v)) / (nblk > 0 ? nblk : 1));
  };
  int v = 0;
  while (v + 1 < V && first(v + 1) <= split) ++v;
  const int p0 = first(v), p1 = first(v + 1);
  g.v = v;
  g.s = split - p0;
  g.ns = p1 - p0;
  g.lo = blk(v);
  g.hi = max(g.lo, blk(v + 1));
  return g;
}

// code blocks [lo, hi) of split s out of nblk (contiguous ranges)
__device__ __forceinline__ void block_share(int nblk, int split, int S, int &lo, int &hi) {
  lo = int((int64_t(split) * nblk) / S);
  hi = int((int64_t(split + 1) * nblk) / S);
}

// LDS of the chunked (64-row) online-softmax pass
struct ChunkSmem {
  float sq[LRKV_MAX_GROUP][kD];   // query side (scaled into log2 units)
  float sp[LRKV_MAX_GROUP][64];   // scores, then weights, of the current chunk
  float m[LRKV_MAX_GROUP], l[LRKV_MAX_GROUP], alpha[LRKV_MAX_GROUP];
};

// One online-softmax pass over rows [lo, hi) for the g query heads of a group,
// 256 threads: chunks of 64 rows, scores for every head into LDS, then one
// softmax update per head (a wave per head), then the value sums, each thread
// owning up to eight (head, column) accumulators.  kval(t, c) and vval(t, c)
// read row t's key (dk columns) and value (dv columns) as float.  The query
// side must already be in sm.sq, and sm.m / sm.l hold the running state (set
// them to -inf / 0 before a first pass).  acc is zeroed on entry.
template <typename KF, typename VF>
__device__ __forceinline__ void chunked_softmax_pass(ChunkSmem &sm, int g, int lo, int hi, int dk,
                                                     int dv, KF kval, VF vval, float (&acc)[8]) {
  constexpr int CH = 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  __syncthreads();
  for (int base = lo; base < hi; base += CH) {
    const int nv = min(CH, hi - base);
    for (int p = tid; p < g * CH; p += blockDim.x) {
      const int hh = p / CH, j = p % CH;
      float s = kNegInf;
      if (j < nv) {
        float a = 0.f;
        for (int c0 = 0; c0 < dk; c0 += 16) {  // dk is a multiple of 16: 16 loads in flight
          float x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) x[u] = kval(base + j, c0 + u);
#pragma unroll
          for (int u = 0; u < 16; ++u) a = fmaf(sm.sq[hh][c0 + u], x[u], a);
        }
        s = a;
      }
      sm.sp[hh][j] = s;
    }
    __syncthreads();
    for (int hh = wave; hh < g; hh += 4) {
      const float s = sm.sp[hh][lane];
      const float mo = sm.m[hh];
      const float mn = fmaxf(mo, wave_max(s));  // finite: the chunk has nv >= 1 rows
      const float p = exp2f(s - mn);             // s = -inf gives 0
      sm.sp[hh][lane] = p;
      const float ps = wave_sum(p);
      if (lane == 0) {
        const float al = exp2f(mo - mn);  // mo = -inf gives 0
        sm.alpha[hh] = al;
        sm.l[hh] = sm.l[hh] * al + ps;
        sm.m[hh] = mn;
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int o = threadIdx.x + e * 256;
      if (o < g * dv) {
        const int hh = o / dv, c = o % dv;
        float a = acc[e] * sm.alpha[hh];
        for (int j0 = 0; j0 < nv; j0 += 16) {  // 16 loads in flight, rows clamped to the chunk
          float x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) x[u] = vval(base + min(j0 + u, nv - 1), c);
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (j0 + u < nv) a = fmaf(sm.sp[hh][j0 + u], x[u], a);
        }
        acc[e] = a;
      }
    }
    __syncthreads();
  }
}

}  // namespace lrkv
