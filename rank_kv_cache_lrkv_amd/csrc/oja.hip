// Online basis adaptation (OjaKV summary and FAQ: Oja's algorithm for online PCA
// keeps adapting the projection basis during prompt prefill and now and then
// during decoding).  One step of the textbook subspace rule per KV head:
//
//   C  = sum of x x^T over the batch's rows          (matrix cores, float32)
//   U' = U + eta (C U - U (U^T C U)) / N
//   U_new = U' with its columns orthonormalised in order (modified Gram-Schmidt)
//
// Two kernels.  k_oja_gram streams the rows once: each workgroup takes 32-row
// tiles of one head, stages a tile in LDS and accumulates the 36 upper 16x16
// tiles of the 128x128 Gram matrix on the matrix cores (bf16 rows are exact
// operands, float32 accumulation), leaving one partial sum per workgroup.
// k_oja_finish (one workgroup per head) adds the partials in a fixed order, then
// does the small dense steps in LDS in float32 and stores U_new as bf16 U^T rows.

#include "decode_common.h"
#include "mfma_util.h"

namespace lrkv {

constexpr int kOjaTiles = 36;                    // upper 16x16 tiles of a 128x128 matrix
constexpr int kOjaPartial = kOjaTiles * 256;     // floats per partial
constexpr int kXStride = kD + 8;                 // padded LDS row of one staged input row

// workgroups per head for the Gram accumulation
int oja_partials(int n_kv) {
  const int p = (1024 + n_kv - 1) / n_kv;
  return p < 1 ? 1 : (p > 64 ? 64 : p);
}

// tile k -> (a, b), a <= b, enumerating the upper triangle row by row
__device__ __forceinline__ void oja_tile(int k, int &a, int &b) {
  a = 0;
  int first = 0;  // index of tile (a, a)
  while (k >= first + (8 - a)) {
    first += 8 - a;
    ++a;
  }
  b = a + (k - first);
}
__device__ __forceinline__ int oja_tile_index(int a, int b) {  // a <= b
  return a * 8 - (a * (a - 1)) / 2 + (b - a);
}

// ---------------------------------------------------------------------------
// Gram matrix partials.  Grid (P, n_kv), 256 threads.  Wave w accumulates tiles
// w, w + 4, ..., w + 32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_oja_gram(LayerArgs L, const bf16_t *x, int64_t sb, int64_t sh,
                                                  int64_t st, int n_tok, float *part) {
  __shared__ bf16_t sx[2][32][kXStride];
  const int P = gridDim.x, p = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const int tpr = (n_tok + 31) / 32;  // tiles per batch row
  const int ntiles = L.batch * tpr;
  // this thread's share of a tile: row tid / 8, features 16 (tid % 8) .. +15
  const int tk = tid >> 3, f0 = (tid & 7) * 16;

  f32x4 acc[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](int i, u32x4 &a, u32x4 &b2) {
    const int b = i / tpr, t = (i - b * tpr) * 32 + tk;
    const bf16_t *row = x + b * sb + h * sh + int64_t(min(t, n_tok - 1)) * st + f0;
    a = *reinterpret_cast<const u32x4 *>(row);
    b2 = *reinterpret_cast<const u32x4 *>(row + 8);
    if (t >= n_tok) a = b2 = u32x4{0u, 0u, 0u, 0u};  // rows past n_tok add nothing
  };

  int i = p;
  if (i < ntiles) {
    u32x4 na, nb;
    load(i, na, nb);
    int buf = 0;
    for (; i < ntiles; i += P) {
      *reinterpret_cast<u32x4 *>(&sx[buf][tk][f0]) = na;
      *reinterpret_cast<u32x4 *>(&sx[buf][tk][f0 + 8]) = nb;
      __syncthreads();  // also orders the previous reads of sx[buf ^ 1] before its next writes
      if (i + P < ntiles) load(i + P, na, nb);
      // fragment ft: lane (q4, t16) holds feature 16 ft + t16 of rows 8 q4 .. 8 q4 + 7,
      // the K-slice layout of both MFMA operands, so D[m][n] = sum_t x_t[16a + m] x_t[16b + n]
      u32x4 fr[8];
#pragma unroll
      for (int ft = 0; ft < 8; ++ft)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          fr[ft][j] = uint32_t(sx[buf][8 * q4 + 2 * j][16 * ft + t16]) |
                      (uint32_t(sx[buf][8 * q4 + 2 * j + 1][16 * ft + t16]) << 16);
#pragma unroll
      for (int ii = 0; ii < 9; ++ii) {
        int a, b;
        oja_tile(wave + 4 * ii, a, b);
        acc[ii] = mfma16x16x32(fr[a], fr[b], acc[ii]);
      }
      buf ^= 1;
    }
  }
  // tile element (row m, column n) at m * 16 + n; lane (q4, t16) holds rows 4 q4 + v, column t16
  float *out = part + (int64_t(h) * P + p) * kOjaPartial;
#pragma unroll
  for (int ii = 0; ii < 9; ++ii)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(wave + 4 * ii) * 256 + (4 * q4 + v) * 16 + t16] = acc[ii][v];
}

// ---------------------------------------------------------------------------
// The update and the orthonormalisation.  Grid (n_kv), 1024 threads.
// ---------------------------------------------------------------------------
constexpr int kGStride = kD + 1;  // padded LDS row of the 128 x 128 float matrix

__global__ __launch_bounds__(1024) void k_oja_finish(LayerArgs L, int which, const float *part, int P,
                                                     float eta_over_n, int vin, int vout) {
  __shared__ float sg[kD * kGStride];   // C, then G = C U, then A = G - U U^T G, then U', Q
  __shared__ bf16_t su[kD * kD];        // U^T rows [r][128]
  __shared__ float sdot[16 * kD];       // U^T G for 16 columns at a time
  __shared__ float snrm[kD];            // squared column norms during Gram-Schmidt
  const int h = blockIdx.x, tid = threadIdx.x;
  const HeadInfo hd = L.heads[h];
  const int r = which ? hd.rv : hd.rk;
  const int64_t off = which ? hd.u_v : hd.u_k;
  const bf16_t *uin = static_cast<const bf16_t *>(L.bases) + vin * L.version_elems + off;
  bf16_t *uout = const_cast<bf16_t *>(static_cast<const bf16_t *>(L.bases)) + vout * L.version_elems + off;

  // C = sum of the partials in workgroup order; element (i, j) comes from tile
  // (i/16, j/16) or, below the diagonal, from the transposed tile
  const float *ph = part + int64_t(h) * P * kOjaPartial;
  for (int e = tid; e < kD * kD; e += blockDim.x) {
    const int i = e >> 7, j = e & 127;
    const int a = i >> 4, b = j >> 4;
    const int k = a <= b ? oja_tile_index(a, b) : oja_tile_index(b, a);
    const int o = k * 256 + (a <= b ? (i & 15) * 16 + (j & 15) : (j & 15) * 16 + (i & 15));
    float s = 0.f;
    for (int q = 0; q < P; ++q) s += ph[int64_t(q) * kOjaPartial + o];
    sg[i * kGStride + j] = s;
  }
  for (int e = tid; e < r * kD; e += blockDim.x) su[e] = uin[e];
  __syncthreads();

  // G = C U (128 x r): G[f][c] = sum_k C[f][k] U^T[c][k]
  constexpr int kMaxPer = kD * kD / 1024;
  float g[kMaxPer];
#pragma unroll
  for (int n = 0; n < kMaxPer; ++n) {
    const int e = tid + 1024 * n;
    g[n] = 0.f;
    if (e < kD * r) {
      const int f = e / r, c = e - f * r;
      float s = 0.f;
      for (int k = 0; k < kD; ++k) s = fmaf(sg[f * kGStride + k], to_f32(su[c * kD + k]), s);
      g[n] = s;
    }
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < kMaxPer; ++n) {
    const int e = tid + 1024 * n;
    if (e < kD * r) {
      const int f = e / r, c = e - f * r;
      sg[f * kGStride + c] = g[n];
    }
  }
  __syncthreads();

  // A = G - U (U^T G), 16 columns at a time; then U' = U + eta / N * A
  for (int c0 = 0; c0 < r; c0 += 16) {
    for (int e = tid; e < 16 * r; e += blockDim.x) {  // (U^T G)[k][c0 + cc]
      const int cc = e / r, k = e - cc * r;
      float s = 0.f;
      for (int f = 0; f < kD; ++f) s = fmaf(to_f32(su[k * kD + f]), sg[f * kGStride + c0 + cc], s);
      sdot[cc * kD + k] = s;
    }
    __syncthreads();
    for (int e = tid; e < 16 * kD; e += blockDim.x) {
      const int f = e >> 4, cc = e & 15;
      float s = 0.f;
      for (int k = 0; k < r; ++k) s = fmaf(to_f32(su[k * kD + f]), sdot[cc * kD + k], s);
      const int c = c0 + cc;
      sg[f * kGStride + c] = fmaf(eta_over_n, sg[f * kGStride + c] - s, to_f32(su[c * kD + f]));
    }
    __syncthreads();
  }

  // modified Gram-Schmidt on the r columns, unnormalised until the end: step j
  // removes column j's direction from every later column.  Column k is handled by
  // the 8 consecutive threads 8 g .. 8 g + 7 (16 rows each), g = k - j - 1.
  const int grp = tid >> 3, sub = tid & 7;
  auto col_dot = [&](int ca, int cb) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = fmaf(sg[(16 * sub + i) * kGStride + ca], sg[(16 * sub + i) * kGStride + cb], s);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);
    return s;
  };
  if (grp == 0) {
    const float n0 = col_dot(0, 0);
    if (sub == 0) snrm[0] = n0;
  }
  __syncthreads();
  for (int j = 0; j + 1 < r; ++j) {
    const int k = j + 1 + grp;
    if (k < r) {
      const float d = col_dot(j, k) / snrm[j];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float *v = &sg[(16 * sub + i) * kGStride];
        v[k] = fmaf(-d, v[j], v[k]);
      }
      if (k == j + 1) {  // column j + 1 is final now
        const float n1 = col_dot(k, k);
        if (sub == 0) snrm[k] = n1;
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < r * kD; e += blockDim.x) {
    const int c = e >> 7, f = e & 127;
    uout[c * kD + f] = from_f32<bf16_t>(sg[f * kGStride + c] / sqrtf(snrm[c]));
  }
}

hipError_t launch_oja(const LayerArgs &L, int which, const void *x, int64_t sb, int64_t sh, int64_t st,
                      int n_tok, float eta, int vin, int vout, float *ws, hipStream_t s) {
  const int P = oja_partials(L.n_kv);
  hipLaunchKernelGGL(k_oja_gram, dim3(P, L.n_kv), dim3(256), 0, s, L, static_cast<const bf16_t *>(x), sb, sh,
                     st, n_tok, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float eta_over_n = float(double(eta) / (double(L.batch) * double(n_tok)));
  hipLaunchKernelGGL(k_oja_finish, dim3(L.n_kv), dim3(1024), 0, s, L, which, ws, P, eta_over_n, vin, vout);
  return hipGetLastError();
}

size_t oja_workspace_bytes(const LayerArgs &L) {
  return size_t(L.n_kv) * oja_partials(L.n_kv) * kOjaPartial * sizeof(float);
}

}  // namespace lrkv
