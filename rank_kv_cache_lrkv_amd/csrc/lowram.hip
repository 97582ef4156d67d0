// LowRAM value amortisation, prefill side (LowRAM abstract: inside a head the
// values are largely predictable from the keys; a light per-head predictor is
// fitted at test time and residuals are kept only for the tokens it reconstructs
// worst).  The page gives no predictor form or selection rule; this one is a
// linear map from the stored key codes, one per (batch row, KV head):
//
//   M   = (C^T C + lam I)^-1 C^T V,  lam = 1e-6 tr(C^T C) / r_k
//   e_t = V_t - C_t M                 (M as stored, bf16)
//
// and every 32-slot block keeps the residual rows of its R tokens with the
// largest ||e_t||^2.  Three kernels:
//
//   k_lowram_gram   C^T [C | V] on the matrix cores, one partial sum per
//                   workgroup: each 32-token tile is staged in LDS column by
//                   column (the MFMA contracts over tokens, so every operand
//                   fragment is 8 consecutive tokens of one column)
//   k_lowram_solve  one workgroup per (row, head): the partials summed in a
//                   fixed order, Cholesky of C^T C + lam I and the two triangular
//                   solves in LDS (float32), M stored as bf16
//   k_lowram_resid  per block: C M on the matrix cores against the staged M^T,
//                   e = V - C M, squared norms, the block's top R by rank
//                   counting, residual rows, slots and norms stored

#include "decode_common.h"
#include "mfma_util.h"

namespace lrkv {

constexpr int kZStride = 40;  // LDS column of a staged tile: 32 tokens + 8 pad (80 bytes)

int lowram_partials(const LayerArgs &L) {
  const int units = L.batch * L.n_kv;
  const int p = (1024 + units - 1) / units;
  return p < 1 ? 1 : (p > 16 ? 16 : p);
}

static int lowram_rk_max(const LayerArgs &L) {
  int m = 0;
  for (int h = 0; h < L.n_kv; ++h) m = L.heads[h].rk > m ? L.heads[h].rk : m;
  return m;
}

// floats of one partial: the r_k x (r_k + 128) product at the layer's largest rank
static int64_t lowram_partial_floats(const LayerArgs &L) {
  const int64_t r = lowram_rk_max(L);
  return r * (r + kD);
}

size_t lowram_workspace_bytes(const LayerArgs &L) {
  return size_t(L.batch) * L.n_kv * lowram_partials(L) * lowram_partial_floats(L) * sizeof(float);
}

// ---------------------------------------------------------------------------
// C^T [C | V] partials.  Grid (P, batch * n_kv), 256 threads.  Partial p takes the
// blocks [p nb / P, (p + 1) nb / P).  Wave w owns the column tiles jt = w, w + 4,
// ... of the product and every row tile.
// ---------------------------------------------------------------------------
template <int RKMAX>
__global__ __launch_bounds__(256) void k_lowram_gram(LayerArgs L, const bf16_t *v, int64_t sb, int64_t sh,
                                                     int64_t st, int n_tok, int64_t pfloats, float *ws) {
  constexpr int NZ = RKMAX + kD;
  constexpr int NIT = RKMAX / 16, NJT = (NZ / 16 + 3) / 4;
  __shared__ bf16_t sz[NZ * kZStride];
  const int P = gridDim.x, p = blockIdx.x, unit = blockIdx.y;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const HeadInfo hd = L.heads[h];
  const int rk = hd.rk, nz = rk + kD;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const int nb = (n_tok + kBlock - 1) / kBlock;
  const int blo = int(int64_t(p) * nb / P), bhi = int(int64_t(p + 1) * nb / P);
  const bf16_t *codes = static_cast<const bf16_t *>(L.codes_k) + hd.ck + int64_t(b) * L.cap * rk;
  const bf16_t *vb = v + b * sb + h * sh;

  f32x4 acc[NIT][NJT];
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int jj = 0; jj < NJT; ++jj) acc[it][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int blk = blo; blk < bhi; ++blk) {
    __syncthreads();  // the previous tile's readers are done
    // key codes: 32 tokens x rk / 8 pieces of 8 columns; slots past n_tok are zero
    for (int pc = tid; pc < 4 * rk; pc += 256) {
      const int t = pc / (rk / 8), cg = pc - t * (rk / 8);
      const int slot = blk * kBlock + t;
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (slot < n_tok) x = *reinterpret_cast<const u32x4 *>(codes + kslot(slot, 8 * cg, rk));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sz[(8 * cg + 2 * i) * kZStride + t] = bf16_t(x[i] & 0xffffu);
        sz[(8 * cg + 2 * i + 1) * kZStride + t] = bf16_t(x[i] >> 16);
      }
    }
    // values: 32 tokens x 16 pieces of 8 features
    for (int pc = tid; pc < 32 * 16; pc += 256) {
      const int t = pc >> 4, fg = pc & 15;
      const int slot = blk * kBlock + t;
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (slot < n_tok) x = *reinterpret_cast<const u32x4 *>(vb + int64_t(slot) * st + 8 * fg);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sz[(rk + 8 * fg + 2 * i) * kZStride + t] = bf16_t(x[i] & 0xffffu);
        sz[(rk + 8 * fg + 2 * i + 1) * kZStride + t] = bf16_t(x[i] >> 16);
      }
    }
    __syncthreads();
    // D[i][j] += sum over the tile's tokens of C[t][i] Z[t][j]: lane (q4, t16) feeds
    // tokens 8 q4 .. 8 q4 + 7 of column 16 it + t16 (A) and of column 16 jt + t16 (B)
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (it < rk / 16) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(&sz[(16 * it + t16) * kZStride + 8 * q4]);
#pragma unroll
        for (int jj = 0; jj < NJT; ++jj) {
          const int jt = wave + 4 * jj;
          if (jt < nz / 16) {
            const u32x4 bb = *reinterpret_cast<const u32x4 *>(&sz[(16 * jt + t16) * kZStride + 8 * q4]);
            acc[it][jj] = mfma16x16x32(a, bb, acc[it][jj]);
          }
        }
      }
    }
  }
  // lane (q4, t16) holds D[16 it + 4 q4 + v][16 jt + t16]; rows of nz floats
  float *out = ws + (int64_t(unit) * P + p) * pfloats;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (it < rk / 16) {
#pragma unroll
      for (int jj = 0; jj < NJT; ++jj) {
        const int jt = wave + 4 * jj;
        if (jt < nz / 16) {
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) out[(16 * it + 4 * q4 + v4) * nz + 16 * jt + t16] = acc[it][jj][v4];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The solve.  One workgroup of 256 threads per (row, head); everything in LDS,
// float32.  A = C^T C + lam I is factored as L L^T in place (lower triangle,
// right-looking, one column per step), then L Y = C^T V and L^T M = Y are solved
// with one thread per output feature.
// ---------------------------------------------------------------------------
constexpr int kSolveStride = 129;  // LDS row of the 128 x 128 matrices (odd: no bank conflicts down a column)

__global__ __launch_bounds__(256) void k_lowram_solve(LayerArgs L, int P, int64_t pfloats, const float *ws) {
  __shared__ float sa[128 * kSolveStride];
  __shared__ float sbm[128 * kSolveStride];
  __shared__ float s_lam;
  const int unit = blockIdx.x;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const HeadInfo hd = L.heads[h];
  const int rk = hd.rk, nz = rk + kD;
  const int tid = threadIdx.x;
  const float *part = ws + int64_t(unit) * P * pfloats;
  for (int e = tid; e < rk * nz; e += 256) {
    float x = 0.f;
    for (int p = 0; p < P; ++p) x += part[int64_t(p) * pfloats + e];  // fixed order
    const int i = e / nz, j = e - i * nz;
    if (j < rk) sa[i * kSolveStride + j] = x;
    else sbm[i * kSolveStride + (j - rk)] = x;
  }
  __syncthreads();
  if (tid == 0) {
    float tr = 0.f;
    for (int i = 0; i < rk; ++i) tr += sa[i * kSolveStride + i];
    s_lam = 1e-6f * tr / float(rk) + 1e-30f;
  }
  __syncthreads();
  if (tid < rk) sa[tid * kSolveStride + tid] += s_lam;
  __syncthreads();
  for (int k = 0; k < rk; ++k) {
    if (tid == 0) sa[k * kSolveStride + k] = sqrtf(fmaxf(sa[k * kSolveStride + k], 1e-30f));
    __syncthreads();
    const float dk = sa[k * kSolveStride + k];
    for (int i = k + 1 + tid; i < rk; i += 256) sa[i * kSolveStride + k] /= dk;
    __syncthreads();
    const int m = rk - k - 1;
    for (int e = tid; e < m * m; e += 256) {
      const int i = k + 1 + e / m, j = k + 1 + e % m;
      if (j <= i) sa[i * kSolveStride + j] -= sa[i * kSolveStride + k] * sa[j * kSolveStride + k];
    }
    __syncthreads();
  }
  if (tid < kD) {
    const int f = tid;
    for (int i = 0; i < rk; ++i) {  // L Y = B
      float y = sbm[i * kSolveStride + f];
      for (int k = 0; k < i; ++k) y -= sa[i * kSolveStride + k] * sbm[k * kSolveStride + f];
      sbm[i * kSolveStride + f] = y / sa[i * kSolveStride + i];
    }
    for (int i = rk - 1; i >= 0; --i) {  // L^T M = Y
      float y = sbm[i * kSolveStride + f];
      for (int k = i + 1; k < rk; ++k) y -= sa[k * kSolveStride + i] * sbm[k * kSolveStride + f];
      sbm[i * kSolveStride + f] = y / sa[i * kSolveStride + i];
    }
  }
  __syncthreads();
  bf16_t *m = static_cast<bf16_t *>(L.pred) + hd.pred + int64_t(b) * rk * kD;
  for (int e = tid; e < rk * kD; e += 256) m[e] = from_f32<bf16_t>(sbm[(e / kD) * kSolveStride + e % kD]);
}

// ---------------------------------------------------------------------------
// Residuals and the per-block choice.  Grid (ceil(nb / kResidBlocks), batch *
// n_kv), 256 threads.  M^T (feature-major) is staged once per workgroup; per
// block, wave w computes D[f][t] = sum_c M[c][f] C[t][c] for the feature tiles
// 2w and 2w + 1 and both 16-token halves (A = M^T rows from LDS, B = the key
// codes as loaded: 8 columns of one token per lane), so lane (q4, t16) ends with
// 4 consecutive features of token 16 h2 + t16 and reads the matching 8 bytes of
// V.  Squared norms are summed over the features (lanes, then waves), each
// token's rank among the block's valid tokens is counted (equal norms: the lower
// slot first), and the tokens ranked below R write their rows to entry = rank.
// ---------------------------------------------------------------------------
constexpr int kResidBlocks = 4;  // blocks per workgroup (M^T staged once)

template <int RKMAX>
__global__ __launch_bounds__(256) void k_lowram_resid(LayerArgs L, const bf16_t *v, int64_t sb, int64_t sh,
                                                      int64_t st, int n_tok) {
  constexpr int MS = RKMAX + 8;  // LDS row of M^T (a multiple of 8 elements: 16-byte fragments)
  constexpr int NKC = (RKMAX + 31) / 32;
  __shared__ bf16_t smt[kD * MS];
  __shared__ float sq_w[4][kBlock];
  __shared__ float sq[kBlock];
  __shared__ int srank[kBlock];
  const int unit = blockIdx.y;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const HeadInfo hd = L.heads[h];
  const int rk = hd.rk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const int nb = (n_tok + kBlock - 1) / kBlock;
  const bf16_t *m = static_cast<const bf16_t *>(L.pred) + hd.pred + int64_t(b) * rk * kD;
  for (int e = tid; e < rk * kD; e += 256) smt[(e % kD) * MS + e / kD] = m[e];  // M[c][f] -> M^T[f][c]
  for (int e = tid; e < kD * (MS - rk); e += 256) smt[(e / (MS - rk)) * MS + rk + e % (MS - rk)] = 0;
  __syncthreads();
  const bf16_t *codes = static_cast<const bf16_t *>(L.codes_k) + hd.ck + int64_t(b) * L.cap * rk;
  const bf16_t *vb = v + b * sb + h * sh;
  bf16_t *rrow = static_cast<bf16_t *>(L.resid);
  const int nkg = rk >> 3;

  for (int bi = 0; bi < kResidBlocks; ++bi) {
    const int blk = blockIdx.x * kResidBlocks + bi;
    if (blk >= nb) break;  // uniform over the workgroup
    f32x4 e[2][2];         // [feature tile 2 wave + i][h2]
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int tok = blk * kBlock + 16 * h2 + t16;
      const bool valid = tok < n_tok;
      u32x4 bc[NKC];  // B = key codes of token tok, columns 32 kc + 8 q4 .. + 7
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int kg = 4 * kc + q4;
        bc[kc] = u32x4{0u, 0u, 0u, 0u};
        if (valid && kg < nkg) bc[kc] = *reinterpret_cast<const u32x4 *>(codes + kslot(tok, 8 * kg, rk));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ft = 2 * wave + i;
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const u32x4 a = *reinterpret_cast<const u32x4 *>(&smt[(16 * ft + t16) * MS + 32 * kc + 8 * q4]);
          d = mfma16x16x32(a, bc[kc], d);
        }
        // lane (q4, t16) holds D[16 ft + 4 q4 + v][token 16 h2 + t16]... as produced by
        // the MFMA the rows are features and the columns tokens
        uint2 vv = uint2{0u, 0u};
        if (valid) vv = *reinterpret_cast<const uint2 *>(vb + int64_t(tok) * st + 16 * ft + 4 * q4);
        const float x0 = __uint_as_float(vv.x << 16), x1 = __uint_as_float(vv.x & 0xffff0000u);
        const float x2 = __uint_as_float(vv.y << 16), x3 = __uint_as_float(vv.y & 0xffff0000u);
        e[i][h2] = valid ? f32x4{x0 - d[0], x1 - d[1], x2 - d[2], x3 - d[3]} : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // squared norms: this lane's 8 features of each of its two tokens, then the
    // four lanes q4 of the token, then the four waves
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) s = fmaf(e[i][h2][v4], e[i][h2][v4], s);
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      if (q4 == 0) sq_w[wave][16 * h2 + t16] = s;
    }
    __syncthreads();
    if (tid < kBlock) sq[tid] = (sq_w[0][tid] + sq_w[1][tid]) + (sq_w[2][tid] + sq_w[3][tid]);
    __syncthreads();
    if (tid < kBlock) {
      const int nvalid = min(kBlock, n_tok - blk * kBlock);
      int rank = kBlock;
      if (tid < nvalid) {
        rank = 0;
        const float mine = sq[tid];
        for (int u = 0; u < nvalid; ++u) rank += (sq[u] > mine || (sq[u] == mine && u < tid)) ? 1 : 0;
      }
      srank[tid] = rank;
    }
    __syncthreads();
    if (tid < L.R) {  // entry tid: the token of rank tid, if any
      int slot = -1;
      for (int u = 0; u < kBlock; ++u) slot = srank[u] == tid ? u : slot;
      const int64_t ei = resid_entry(L, h, b, blk, tid);
      L.rslot[ei] = slot;
      L.rnorm[ei] = slot >= 0 ? sq[slot] : 0.f;
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int r = srank[16 * h2 + t16];
      if (r < L.R) {
        bf16_t *row = rrow + resid_entry(L, h, b, blk, r) * kD;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int f = 16 * (2 * wave + i) + 4 * q4;
          uint2 o;
          o.x = pack_rne(e[i][h2][0], e[i][h2][1]);
          o.y = pack_rne(e[i][h2][2], e[i][h2][3]);
          *reinterpret_cast<uint2 *>(row + f) = o;
        }
      }
    }
    __syncthreads();  // sq, srank reused by the next block
  }
}

template <int RKMAX>
static void launch_fit_rk(const LayerArgs &L, const bf16_t *v, int64_t sb, int64_t sh, int64_t st, int n_tok,
                          float *ws, hipStream_t s) {
  const int P = lowram_partials(L);
  const int64_t pf = lowram_partial_floats(L);
  const int units = L.batch * L.n_kv;
  hipLaunchKernelGGL(k_lowram_gram<RKMAX>, dim3(P, units), dim3(256), 0, s, L, v, sb, sh, st, n_tok, pf, ws);
  hipLaunchKernelGGL(k_lowram_solve, dim3(units), dim3(256), 0, s, L, P, pf, static_cast<const float *>(ws));
  const int nb = (n_tok + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(k_lowram_resid<RKMAX>, dim3((nb + kResidBlocks - 1) / kResidBlocks, units), dim3(256), 0, s,
                     L, v, sb, sh, st, n_tok);
}

hipError_t launch_lowram_fit(const LayerArgs &L, const bf16_t *v, int64_t sb, int64_t sh, int64_t st, int n_tok,
                             float *ws, hipStream_t s) {
  const int r = lowram_rk_max(L);
  if (r <= 32) launch_fit_rk<32>(L, v, sb, sh, st, n_tok, ws, s);
  else if (r <= 64) launch_fit_rk<64>(L, v, sb, sh, st, n_tok, ws, s);
  else if (r <= 96) launch_fit_rk<96>(L, v, sb, sh, st, n_tok, ws, s);
  else launch_fit_rk<128>(L, v, sb, sh, st, n_tok, ws, s);
  return hipGetLastError();
}

}  // namespace lrkv
