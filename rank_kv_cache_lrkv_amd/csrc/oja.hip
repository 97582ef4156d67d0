// Online basis adaptation (OjaKV summary and FAQ: Oja's algorithm for online PCA
// keeps adapting the projection basis during prompt prefill and now and then
// during decoding).  One step of the textbook subspace rule per KV head:
//
//   C  = sum of x x^T over the batch's rows          (matrix cores, float32)
//   U' = U + eta (C U - U (U^T C U)) / N
//   U_new = U' with its columns orthonormalised in order (modified Gram-Schmidt)
//
// Three kernels.  k_oja_gram streams the rows once: each workgroup takes 128-row
// tiles of one head, stages a tile in LDS and accumulates the 36 upper 16x16
// tiles of the 128x128 Gram matrix on the matrix cores (bf16 rows are exact
// operands, float32 accumulation), leaving one partial sum per workgroup.
// k_oja_reduce adds the partials tile by tile in a fixed order (so the result is
// reproducible bit for bit), and k_oja_finish (one workgroup per head) does the
// small dense steps in LDS in float32 and stores U_new as bf16 U^T rows.

#include "decode_common.h"
#include "mfma_util.h"

namespace lrkv {

constexpr int kOjaTiles = 36;                    // upper 16x16 tiles of a 128x128 matrix
constexpr int kOjaPartial = kOjaTiles * 256;     // floats per partial
// LDS row of one staged input row: 65 words, so the four 8-row groups a fragment
// read spans start 8 banks apart
constexpr int kXStride = kD + 2;

// workgroups per head for the Gram accumulation
int oja_partials(int n_kv) {
  const int p = (1024 + n_kv - 1) / n_kv;
  return p < 1 ? 1 : (p > 64 ? 64 : p);
}

// tile (a, b), a <= b, numbered row by row over the upper triangle
__host__ __device__ constexpr int oja_tile_index(int a, int b) { return a * 8 - (a * (a - 1)) / 2 + (b - a); }

// Wave w owns the tile rows w and 7 - w (8 - w plus w + 1 tiles: 9 each); its
// accumulator n holds tile (oja_row(w, n), oja_col(w, n)).  Fixed at compile
// time, so fragments are picked from registers with constant indices.
__host__ __device__ constexpr int oja_row(int w, int n) { return n < 8 - w ? w : 7 - w; }
__host__ __device__ constexpr int oja_col(int w, int n) { return n < 8 - w ? w + n : 7 - w + (n - (8 - w)); }

template <int W>
__device__ __forceinline__ void oja_wave_mfma(const u32x4 (&fr)[8], f32x4 (&acc)[9]) {
#pragma unroll
  for (int n = 0; n < 9; ++n) acc[n] = mfma16x16x32(fr[oja_row(W, n)], fr[oja_col(W, n)], acc[n]);
}

// ---------------------------------------------------------------------------
// Gram matrix partials.  Grid (P, n_kv), 256 threads.  Each iteration stages a
// 128-row tile (four K-steps of 32 rows; every thread has 4 x 32 bytes in
// flight while the previous tile is multiplied).  Wave w accumulates the tiles
// of rows w and 7 - w.
// ---------------------------------------------------------------------------
constexpr int kOjaRows = 128;  // rows per staged tile

__global__ __launch_bounds__(256) void k_oja_gram(LayerArgs L, const bf16_t *x, int64_t sb, int64_t sh,
                                                  int64_t st, int n_tok, float *part) {
  __shared__ bf16_t sx[2][kOjaRows][kXStride];
  const int P = gridDim.x, p = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const int tpr = (n_tok + kOjaRows - 1) / kOjaRows;  // tiles per batch row
  const int ntiles = L.batch * tpr;
  // this thread's share of a tile: rows tid / 8 + 32 u (u < 4), features 16 (tid % 8) .. +15
  const int tk = tid >> 3, f0 = (tid & 7) * 16;

  f32x4 acc[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](int i, u32x4 (&a)[8]) {
    const int b = i / tpr, t0 = (i - b * tpr) * kOjaRows + tk;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + 32 * u;
      const bf16_t *row = x + b * sb + h * sh + int64_t(min(t, n_tok - 1)) * st + f0;
      a[2 * u] = *reinterpret_cast<const u32x4 *>(row);
      a[2 * u + 1] = *reinterpret_cast<const u32x4 *>(row + 8);
      if (t >= n_tok) a[2 * u] = a[2 * u + 1] = u32x4{0u, 0u, 0u, 0u};  // rows past n_tok add nothing
    }
  };

  int i = p;
  if (i < ntiles) {
    u32x4 nx[8];
    load(i, nx);
    int buf = 0;
    for (; i < ntiles; i += P) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // 4-byte aligned rows: word stores
        uint32_t *row = reinterpret_cast<uint32_t *>(&sx[buf][tk + 32 * u][f0]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          row[w] = nx[2 * u][w];
          row[4 + w] = nx[2 * u + 1][w];
        }
      }
      __syncthreads();  // also orders the previous reads of sx[buf ^ 1] before its next writes
      if (i + P < ntiles) load(i + P, nx);
      // fragment ft of K-step ks: lane (q4, t16) holds feature 16 ft + t16 of rows
      // 32 ks + 8 q4 .. +7, the K-slice layout of both MFMA operands, so
      // D[m][n] = sum_t x_t[16a + m] x_t[16b + n]
#pragma unroll
      for (int ks = 0; ks < kOjaRows / 32; ++ks) {
        u32x4 fr[8];
#pragma unroll
        for (int ft = 0; ft < 8; ++ft)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            fr[ft][j] = uint32_t(sx[buf][32 * ks + 8 * q4 + 2 * j][16 * ft + t16]) |
                        (uint32_t(sx[buf][32 * ks + 8 * q4 + 2 * j + 1][16 * ft + t16]) << 16);
        switch (wave) {
          case 0: oja_wave_mfma<0>(fr, acc); break;
          case 1: oja_wave_mfma<1>(fr, acc); break;
          case 2: oja_wave_mfma<2>(fr, acc); break;
          default: oja_wave_mfma<3>(fr, acc); break;
        }
      }
      buf ^= 1;
    }
  }
  // tile element (row m, column n) at m * 16 + n; lane (q4, t16) holds rows 4 q4 + v, column t16
  float *out = part + (int64_t(h) * P + p) * kOjaPartial;
#pragma unroll
  for (int ii = 0; ii < 9; ++ii) {
    const int k = oja_tile_index(oja_row(wave, ii), oja_col(wave, ii));
#pragma unroll
    for (int v = 0; v < 4; ++v) out[k * 256 + (4 * q4 + v) * 16 + t16] = acc[ii][v];
  }
}

// ---------------------------------------------------------------------------
// The partials of one 16x16 tile added in workgroup order.  Grid (36, n_kv),
// 256 threads (one element each).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_oja_reduce(const float *part, int P, float *gram) {
  const int k = blockIdx.x, h = blockIdx.y, e = threadIdx.x;
  const float *src = part + int64_t(h) * P * kOjaPartial + k * 256 + e;
  float s = 0.f;
  for (int q = 0; q < P; ++q) s += src[int64_t(q) * kOjaPartial];
  gram[(int64_t(h) * kOjaTiles + k) * 256 + e] = s;
}

// ---------------------------------------------------------------------------
// The update and the orthonormalisation.  Grid (n_kv), 1024 threads.
// ---------------------------------------------------------------------------
constexpr int kGStride = kD + 1;  // padded LDS row of the 128 x 128 float matrix
constexpr int kUPad = kD + 2;     // padded LDS row of U (128 x r, r <= 128), bf16

__global__ __launch_bounds__(1024) void k_oja_finish(LayerArgs L, int which, const float *gram,
                                                     float eta_over_n, int vin, int vout) {
  __shared__ float sg[kD * kGStride];   // C, then G = C U, then U' (row f, column c)
  __shared__ bf16_t su[kD * kUPad];     // U (row f, column k)
  __shared__ float sdot[kD * 16];       // U^T G for 16 columns at a time, [k][16]
  __shared__ float sq[2][kD];           // the newest orthonormal column, by step parity
  const int h = blockIdx.x, tid = threadIdx.x;
  const HeadInfo hd = L.heads[h];
  const int r = which ? hd.rv : hd.rk;
  const int64_t off = which ? hd.u_v : hd.u_k;
  const bf16_t *uin = static_cast<const bf16_t *>(L.bases) + vin * L.version_elems + off;
  bf16_t *uout = const_cast<bf16_t *>(static_cast<const bf16_t *>(L.bases)) + vout * L.version_elems + off;

  // C: element (i, j) comes from tile (i/16, j/16) or, below the diagonal, from
  // the transposed tile
  const float *gh = gram + int64_t(h) * kOjaTiles * 256;
  for (int e = tid; e < kD * kD; e += blockDim.x) {
    const int i = e >> 7, j = e & 127;
    const int a = i >> 4, b = j >> 4;
    const int k = a <= b ? oja_tile_index(a, b) : oja_tile_index(b, a);
    sg[i * kGStride + j] = gh[k * 256 + (a <= b ? (i & 15) * 16 + (j & 15) : (j & 15) * 16 + (i & 15))];
  }
  for (int e = tid; e < r * kD; e += blockDim.x) {  // U^T rows in memory, U in LDS
    const int c = e >> 7, f = e & 127;
    su[f * kUPad + c] = uin[e];
  }
  __syncthreads();
  auto U = [&](int f, int c) { return to_f32(su[f * kUPad + c]); };

  // G = C U (128 x r); a wave shares one column c (U read as a broadcast)
  constexpr int kMaxPer = kD * kD / 1024;
  float g[kMaxPer];
#pragma unroll
  for (int n = 0; n < kMaxPer; ++n) {
    const int e = tid + 1024 * n;
    g[n] = 0.f;
    if (e < kD * r) {
      const int f = e & 127, c = e >> 7;
      float s = 0.f;
      for (int k = 0; k < kD; ++k) s = fmaf(sg[f * kGStride + k], U(k, c), s);
      g[n] = s;
    }
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < kMaxPer; ++n) {
    const int e = tid + 1024 * n;
    if (e < kD * r) {
      const int f = e & 127, c = e >> 7;
      sg[f * kGStride + c] = g[n];
    }
  }
  __syncthreads();

  // U' = U + eta / N (G - U (U^T G)), 16 columns at a time
  for (int c0 = 0; c0 < r; c0 += 16) {
    for (int e = tid; e < 16 * r; e += blockDim.x) {  // (U^T G)[k][c0 + cc]
      const int cc = e & 15, k = e >> 4;
      float s = 0.f;
      for (int f = 0; f < kD; ++f) s = fmaf(U(f, k), sg[f * kGStride + c0 + cc], s);
      sdot[k * 16 + cc] = s;
    }
    __syncthreads();
    for (int e = tid; e < 16 * kD; e += blockDim.x) {
      const int f = e >> 4, cc = e & 15;
      float s = 0.f;
      for (int k = 0; k < r; ++k) s = fmaf(U(f, k), sdot[k * 16 + cc], s);
      const int c = c0 + cc;
      sg[f * kGStride + c] = fmaf(eta_over_n, sg[f * kGStride + c] - s, U(f, c));
    }
    __syncthreads();
  }

  // modified Gram-Schmidt: the 8 consecutive threads of group c own column c
  // (16 rows each, in registers).  At step j column j is final: it is
  // normalised and published in LDS, and every later column removes its
  // component along it.
  const int grp = tid >> 3, sub = tid & 7;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = grp < r ? sg[(16 * sub + i) * kGStride + grp] : 0.f;
  auto group_sum = [&](float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    return x;
  };
  // sum over i of a[i] b[i] for this thread's 16 rows, as four independent chains
  auto dot16 = [&](const float *a, const float *b) {
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      p0 = fmaf(a[i], b[i], p0);
      p1 = fmaf(a[i + 1], b[i + 1], p1);
      p2 = fmaf(a[i + 2], b[i + 2], p2);
      p3 = fmaf(a[i + 3], b[i + 3], p3);
    }
    return (p0 + p1) + (p2 + p3);
  };
  for (int j = 0; j < r; ++j) {
    float *q = sq[j & 1];
    if (grp == j) {
      const float inv = 1.f / sqrtf(group_sum(dot16(v, v)));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v[i] *= inv;
        q[16 * sub + i] = v[i];
      }
    }
    __syncthreads();  // also: every read of sq[j & 1] at step j - 2 is done
    if (grp > j && grp < r) {
      float qv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) qv[i] = q[16 * sub + i];
      const float d = group_sum(dot16(qv, v));
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = fmaf(-d, qv[i], v[i]);
    }
  }
  if (grp < r) {
#pragma unroll
    for (int i = 0; i < 16; ++i) uout[grp * kD + 16 * sub + i] = from_f32<bf16_t>(v[i]);
  }
}

hipError_t launch_oja(const LayerArgs &L, int which, const void *x, int64_t sb, int64_t sh, int64_t st,
                      int n_tok, float eta, int vin, int vout, float *ws, hipStream_t s) {
  // workspace: the partials, then the summed Gram tiles
  const int P = oja_partials(L.n_kv);
  float *gram = ws + size_t(L.n_kv) * P * kOjaPartial;
  hipLaunchKernelGGL(k_oja_gram, dim3(P, L.n_kv), dim3(256), 0, s, L, static_cast<const bf16_t *>(x), sb, sh,
                     st, n_tok, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_oja_reduce, dim3(kOjaTiles, L.n_kv), dim3(256), 0, s, ws, P, gram);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float eta_over_n = float(double(eta) / (double(L.batch) * double(n_tok)));
  hipLaunchKernelGGL(k_oja_finish, dim3(L.n_kv), dim3(1024), 0, s, L, which, gram, eta_over_n, vin, vout);
  return hipGetLastError();
}

size_t oja_workspace_bytes(const LayerArgs &L) {
  return size_t(L.n_kv) * (oja_partials(L.n_kv) + 1) * kOjaPartial * sizeof(float);
}

}  // namespace lrkv
