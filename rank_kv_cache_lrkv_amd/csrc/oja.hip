// Online basis adaptation (OjaKV summary and FAQ: Oja's algorithm for online PCA
// keeps adapting the projection basis during prompt prefill and now and then
// during decoding).  One step of the textbook subspace rule per KV head:
//
//   C  = sum of x x^T over the batch's rows          (matrix cores, float32)
//   U' = U + eta (C U - U (U^T C U)) / N
//   U_new = U' with its columns orthonormalised in order (modified Gram-Schmidt)
//
// Three kernels.  k_oja_gram streams the rows once: each workgroup takes 128-row
// tiles of one head, stages a tile in LDS transposed (features as rows, tokens
// contiguous) and accumulates the 36 upper 16x16 tiles of the 128x128 Gram
// matrix on the matrix cores (bf16 rows are exact operands, float32
// accumulation), leaving one partial sum per workgroup.  k_oja_reduce adds the
// partials tile by tile in a fixed order (so the result is reproducible bit for
// bit) and writes C in full.  k_oja_finish (one workgroup per head) takes the
// three small products on the float32 matrix cores, then orthonormalises in LDS
// and stores U_new as bf16 U^T rows.

#include "decode_common.h"
#include "mfma_util.h"

namespace lrkv {

constexpr int kOjaTiles = 36;                    // upper 16x16 tiles of a 128x128 matrix
constexpr int kOjaPartial = kOjaTiles * 256;     // floats per partial

// workgroups per head for the Gram accumulation (two per compute unit)
int oja_partials(int n_kv) {
  const int p = (512 + n_kv - 1) / n_kv;
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
// Gram matrix partials.  Grid (P, n_kv), 256 threads, two workgroups per
// compute unit.  The staged tile is transposed: LDS row f holds feature f of the
// tile's 128 tokens as 16 chunks of 8 tokens, chunk c at position c ^ (f / 8)
// (the swizzle spreads both the transposing stores and the operand reads over
// the banks), rows 136 elements apart.  A matrix-core operand (8 tokens of one
// feature) is then one 16-byte read.  Every thread keeps the loads of two tiles
// in flight (16 x 16 bytes) while the workgroup multiplies the staged one.
// ---------------------------------------------------------------------------
constexpr int kOjaRows = 128;            // rows per staged tile
constexpr int kTPitch = kOjaRows + 8;    // bf16 per LDS row (one feature)

__device__ __forceinline__ int oja_lds_pos(int f, int chunk) { return f * kTPitch + 8 * (chunk ^ (f >> 3)); }

__global__ __launch_bounds__(256, 2) void k_oja_gram(LayerArgs L, const bf16_t *x, int64_t sb, int64_t sh,
                                                     int64_t st, int n_tok, float *part) {
  __shared__ __align__(16) bf16_t sx[kD * kTPitch];
  const int P = gridDim.x, p = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const int tpr = (n_tok + kOjaRows - 1) / kOjaRows;  // tiles per batch row
  const int ntiles = L.batch * tpr;
  // this thread's share of a tile: features 8 fb .. 8 fb + 7 of the rows
  // 4 g .. 4 g + 3 and 64 + 4 g .. 64 + 4 g + 3 (a wave's load covers four whole rows)
  const int fb = tid & 15, g = tid >> 4;

  f32x4 acc[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // rows past n_tok are read clamped and zeroed when staged (no wait at the load)
  auto load = [&](int i, u32x4 (&a)[8]) {
    const int b = i / tpr, t0 = (i - b * tpr) * kOjaRows + 4 * g;
    const bf16_t *base = x + b * sb + h * sh + 8 * fb;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + (u >> 2) * 64 + (u & 3);
      a[u] = *reinterpret_cast<const u32x4 *>(base + int64_t(min(t, n_tok - 1)) * st);
    }
  };
  // word w of a load holds features 8 fb + 2 w (low half) and 8 fb + 2 w + 1
  // (high half); four rows of one feature are one 8-byte store
  auto stage = [&](int i, const u32x4 (&a)[8]) {
    const int b = i / tpr, t0 = (i - b * tpr) * kOjaRows + 4 * g;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        r[u] = t0 + 64 * hf + u < n_tok ? a[4 * hf + u] : u32x4{0u, 0u, 0u, 0u};
      const int chunk = 8 * hf + (g >> 1), half = 4 * (g & 1);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 lo = {(r[0][w] & 0xffffu) | (r[1][w] << 16), (r[2][w] & 0xffffu) | (r[3][w] << 16)};
        const u32x2 hi = {(r[0][w] >> 16) | (r[1][w] & 0xffff0000u), (r[2][w] >> 16) | (r[3][w] & 0xffff0000u)};
        const int f = 8 * fb + 2 * w;
        *reinterpret_cast<u32x2 *>(&sx[oja_lds_pos(f, chunk) + half]) = lo;
        *reinterpret_cast<u32x2 *>(&sx[oja_lds_pos(f + 1, chunk) + half]) = hi;
      }
    }
  };
  // fragment ft of K-step ks: lane (q4, t16) holds tokens 32 ks + 8 q4 .. +7 of
  // feature 16 ft + t16, the K-slice layout of both operands, so
  // D[m][n] = sum_t x_t[16a + m] x_t[16b + n]
  auto multiply = [&]() {
#pragma unroll
    for (int ks = 0; ks < kOjaRows / 32; ++ks) {
      u32x4 fr[8];
#pragma unroll
      for (int ft = 0; ft < 8; ++ft)
        fr[ft] = *reinterpret_cast<const u32x4 *>(&sx[oja_lds_pos(16 * ft + t16, 4 * ks + q4)]);
      switch (wave) {
        case 0: oja_wave_mfma<0>(fr, acc); break;
        case 1: oja_wave_mfma<1>(fr, acc); break;
        case 2: oja_wave_mfma<2>(fr, acc); break;
        default: oja_wave_mfma<3>(fr, acc); break;
      }
    }
  };
  // tile i from registers r, which then take tile i + 2P
  auto step = [&](int i, u32x4 (&r)[8]) {
    __syncthreads();  // the previous tile's operand reads are done
    stage(i, r);
    __syncthreads();
    if (i + 2 * P < ntiles) load(i + 2 * P, r);
    multiply();
  };

  u32x4 ra[8], rb[8];
  if (p < ntiles) load(p, ra);
  if (p + P < ntiles) load(p + P, rb);
  for (int i = p; i < ntiles; i += 2 * P) {
    step(i, ra);
    if (i + P < ntiles) step(i + P, rb);
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
// The partials of one 16x16 tile added in workgroup order; C stored in full
// (row-major 128 x 128 per head, the tile and its mirror).  Grid (36, n_kv),
// 256 threads (one element each, eight partials in flight).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_oja_reduce(const float *part, int P, float *gram) {
  const int k = blockIdx.x, h = blockIdx.y, e = threadIdx.x;
  const float *src = part + int64_t(h) * P * kOjaPartial + k * 256 + e;
  float s = 0.f;
  int q = 0;
  for (; q + 8 <= P; q += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[int64_t(q + j) * kOjaPartial];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  for (; q < P; ++q) s += src[int64_t(q) * kOjaPartial];
  int a = 0;  // tile (a, b) of index k
  while (oja_tile_index(a + 1, a + 1) <= k) ++a;
  const int b = a + (k - oja_tile_index(a, a));
  const int m = e >> 4, n = e & 15;
  float *gh = gram + int64_t(h) * kD * kD;
  gh[(16 * a + m) * kD + 16 * b + n] = s;
  if (a != b) gh[(16 * b + n) * kD + 16 * a + m] = s;
}

// ---------------------------------------------------------------------------
// The update and the orthonormalisation.  Grid (n_kv), 1024 threads (16 waves).
// The products are 16x16 tiles on the float32 matrix cores (16x16x4: lane
// (q4, t16) supplies A[t16][q4] and B[q4][t16] and receives D[4 q4 + v][t16]):
//   G = C U             (128 x r; A from C in memory, B from U in LDS)
//   S = U^T G[:, chunk] (r x 64 columns at a time)
//   U' = U + eta / N (G - U S) over the chunk's columns, in place of G
// then modified Gram-Schmidt on the columns of U' (oja_gram_schmidt).
// ---------------------------------------------------------------------------
constexpr int kUPad = kD + 2;     // padded LDS row of U (128 x r, r <= 128), bf16
constexpr int kGPitch = kD + 16;  // LDS row of G / U' (float)
constexpr int kSChunk = 64;       // columns of S per pass
constexpr int kSPitch = kSChunk + 16;

// v + v of another lane of its row of 16, by DPP (no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __uint_as_float(uint32_t(__builtin_amdgcn_update_dpp(0, int(__float_as_uint(v)), CTRL, 0xf, 0xf, false)));
}
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Modified Gram-Schmidt on the r columns of U' (LDS, row f at f * kGPitch) by
// 1024 threads: the 128 / RPL consecutive threads of group c own column c, RPL
// rows each in registers (RPL = 8 while 16-thread groups fit, r <= 64; else 16).
// At step j column j is final: its group normalises it and publishes it in LDS,
// and every later column removes its component along it.  Group sums are DPP
// steps (no LDS round trip).  The result is stored as bf16 U^T rows.
template <int RPL>
__device__ __forceinline__ void oja_gram_schmidt(const float *sg, float (*sq)[kD], int r, int tid, bf16_t *uout) {
  constexpr int kLanes = kD / RPL;  // threads per column: 8 or 16
  const int grp = tid / kLanes, sub = tid % kLanes;
  float v[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) v[i] = grp < r ? sg[(RPL * sub + i) * kGPitch + grp] : 0.f;
  auto group_sum = [&](float x) {
    x = dpp_add<0xb1>(x);                     // quad_perm [1,0,3,2]
    x = dpp_add<0x4e>(x);                     // quad_perm [2,3,0,1]
    x = dpp_add<0x141>(x);                    // row_half_mirror: the other quad of each eight
    if constexpr (kLanes == 16) x = dpp_add<0x140>(x);  // row_mirror: the other eight of the row
    return x;
  };
  // sum over i of a[i] b[i] for this thread's rows, as four independent chains
  auto dot = [&](const float *a, const float *b) {
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; i += 4) {
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
      const float inv = __builtin_amdgcn_rsqf(group_sum(dot(v, v)));  // hardware 1/sqrt (about 1 ulp)
#pragma unroll
      for (int i = 0; i < RPL; ++i) v[i] *= inv;
#pragma unroll
      for (int i = 0; i < RPL; i += 4)
        *reinterpret_cast<f32x4 *>(&q[RPL * sub + i]) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
    }
    __syncthreads();  // also: every read of sq[j & 1] at step j - 2 is done
    if (grp > j && grp < r) {
      float qv[RPL];
#pragma unroll
      for (int i = 0; i < RPL; i += 4) {
        const f32x4 t = *reinterpret_cast<const f32x4 *>(&q[RPL * sub + i]);
        qv[i] = t[0];
        qv[i + 1] = t[1];
        qv[i + 2] = t[2];
        qv[i + 3] = t[3];
      }
      const float d = group_sum(dot(qv, v));
#pragma unroll
      for (int i = 0; i < RPL; ++i) v[i] = fmaf(-d, qv[i], v[i]);
    }
  }
  if (grp < r) {
#pragma unroll
    for (int i = 0; i < RPL; i += 2)
      *reinterpret_cast<uint32_t *>(uout + grp * kD + RPL * sub + i) =
          uint32_t(from_f32<bf16_t>(v[i])) | (uint32_t(from_f32<bf16_t>(v[i + 1])) << 16);
  }
}

__global__ __launch_bounds__(1024) void k_oja_finish(LayerArgs L, int which, const float *gram,
                                                     float eta_over_n, int vin, int vout) {
  __shared__ float sg[kD * kGPitch];     // G, then U' (row f, column c)
  __shared__ float ss[kD * kSPitch];     // S for one chunk of columns (row k, column n)
  __shared__ bf16_t su[kD * kUPad];      // U (row f, column k)
  __shared__ __align__(16) float sq[2][kD];  // the newest orthonormal column, by step parity
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const HeadInfo hd = L.heads[h];
  const int r = which ? hd.rv : hd.rk;
  const int nr = r >> 4;  // 16-column tiles of U
  const int64_t off = which ? hd.u_v : hd.u_k;
  const bf16_t *uin = static_cast<const bf16_t *>(L.bases) + vin * L.version_elems + off;
  bf16_t *uout = const_cast<bf16_t *>(static_cast<const bf16_t *>(L.bases)) + vout * L.version_elems + off;
  const float *gh = gram + int64_t(h) * kD * kD;

  // U^T rows in memory, U in LDS: 8 features of one column per 16-byte load, at
  // most two per thread (both issued before either is stored)
  {
    u32x4 w[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int e = min(tid + 1024 * n, r * 16 - 1);  // 16-byte piece: column e / 16, features 8 (e % 16) ..
      w[n] = *reinterpret_cast<const u32x4 *>(uin + 8 * e);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int e = tid + 1024 * n;
      if (e < r * 16) {
        const int c = e >> 4, f0 = 8 * (e & 15);
#pragma unroll
        for (int i = 0; i < 8; ++i) su[(f0 + i) * kUPad + c] = bf16_t(w[n][i >> 1] >> (16 * (i & 1)));
      }
    }
  }
  auto U = [&](int f, int c) { return to_f32(su[f * kUPad + c]); };

  // G: wave w takes the tiles (w mod 8, w / 8 + 2 j); its 32 A operands (a
  // 16-row strip of C, read as columns since C is symmetric) are loaded once
  {
    const int mt = wave & 7;
    float a[32];
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) a[ks] = gh[(4 * ks + q4) * kD + 16 * mt + t16];
    __syncthreads();  // U staged
    for (int nt = wave >> 3; nt < nr; nt += 2) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;  // two chains: even and odd K-steps
#pragma unroll
      for (int ks = 0; ks < 32; ks += 2) {
        acc0 = mfma16x16x4(a[ks], U(4 * ks + q4, 16 * nt + t16), acc0);
        acc1 = mfma16x16x4(a[ks + 1], U(4 * ks + 4 + q4, 16 * nt + t16), acc1);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) sg[(16 * mt + 4 * q4 + v) * kGPitch + 16 * nt + t16] = acc0[v] + acc1[v];
    }
  }
  __syncthreads();

  for (int c0 = 0; c0 < r; c0 += kSChunk) {
    const int nc = min(kSChunk, r - c0) >> 4;  // 16-column tiles in this chunk
    // S[k][n] = sum_f U[f][k] G[f][c0 + n]
    for (int t = wave; t < nr * nc; t += 16) {
      const int kt = t / nc, nt = t - kt * nc;
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll 8
      for (int ks = 0; ks < 32; ks += 2) {
        acc0 = mfma16x16x4(U(4 * ks + q4, 16 * kt + t16), sg[(4 * ks + q4) * kGPitch + c0 + 16 * nt + t16], acc0);
        acc1 = mfma16x16x4(U(4 * ks + 4 + q4, 16 * kt + t16), sg[(4 * ks + 4 + q4) * kGPitch + c0 + 16 * nt + t16],
                           acc1);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) ss[(16 * kt + 4 * q4 + v) * kSPitch + 16 * nt + t16] = acc0[v] + acc1[v];
    }
    __syncthreads();
    // U'[f][c0 + n] = U[f][c0 + n] + eta / N (G[f][c0 + n] - sum_k U[f][k] S[k][n])
    for (int t = wave; t < 8 * nc; t += 16) {
      const int mt = t / nc, nt = t - mt * nc;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < 4 * nr; k0 += 4) {  // operands of four K-steps read together
        float a4[4], b4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a4[u] = U(16 * mt + t16, 4 * (k0 + u) + q4);
          b4[u] = ss[(4 * (k0 + u) + q4) * kSPitch + 16 * nt + t16];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = mfma16x16x4(a4[u], b4[u], acc);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int f = 16 * mt + 4 * q4 + v, c = c0 + 16 * nt + t16;
        float &gv = sg[f * kGPitch + c];
        gv = fmaf(eta_over_n, gv - acc[v], U(f, c));
      }
    }
    __syncthreads();
  }

  if (r <= 64)
    oja_gram_schmidt<8>(sg, sq, r, tid, uout);
  else
    oja_gram_schmidt<16>(sg, sq, r, tid, uout);
}

hipError_t launch_oja(const LayerArgs &L, int which, const void *x, int64_t sb, int64_t sh, int64_t st,
                      int n_tok, float eta, int vin, int vout, float *ws, hipStream_t s) {
  // workspace: the partials, then the summed Gram tiles
  const int P = oja_partials(L.n_kv);
  float *gram = ws + size_t(L.n_kv) * P * kOjaPartial;  // C in full: 128 x 128 floats per head
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
  return size_t(L.n_kv) * (size_t(oja_partials(L.n_kv)) * kOjaPartial + size_t(kD) * kD) * sizeof(float);
}

}  // namespace lrkv
