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
//                   workgroup: each 64-token tile is staged in LDS column by
//                   column (the MFMA contracts over tokens, so every operand
//                   fragment is 8 consecutive tokens of one column)
//   k_lowram_solve  one workgroup per (row, head): the partials summed in a
//                   fixed order, C^T C + lam I eliminated (Cholesky with
//                   unscaled columns) and the two triangular solves in LDS
//                   (float32), M stored as bf16
//   k_lowram_resid  per block: C M on the matrix cores against the staged M^T,
//                   e = V - C M, squared norms, the block's top R by rank
//                   counting, residual rows, slots and norms stored

#include "decode_common.h"
#include "mfma_util.h"

namespace lrkv {

constexpr int kMaxPartials = 16;  // Gram partials per unit (the solve keeps them all in flight)

int lowram_partials(const LayerArgs &L) {
  const int units = L.batch * L.n_kv;
  const int p = (1024 + units - 1) / units;
  return p < 1 ? 1 : (p > kMaxPartials ? kMaxPartials : p);
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
// 64-token tiles [p nt / P, (p + 1) nt / P).  A tile is staged in LDS transposed
// (row = one column of C or of V, its 64 tokens contiguous; rows 144 bytes apart,
// so the 16 rows a fragment read spans fall on distinct banks): thread (tg, grp)
// loads tokens 4 tg .. 4 tg + 3 of code column group grp (8 columns; one 64-byte
// run of the blocked layout) and of value feature group grp, and stores each
// column's four tokens as one 8-byte write.  Every thread keeps the loads of two
// tiles in flight while the staged one is multiplied.  Wave w owns the column
// tiles jt = w, w + 4, ... of the product and every row tile.
// ---------------------------------------------------------------------------
constexpr int kGTile = 64;               // tokens per staged tile
constexpr int kGPitch = kGTile + 8;      // bf16 per LDS row (144 bytes)

template <int RKMAX>
__global__ __launch_bounds__(256) void k_lowram_gram(LayerArgs L, const bf16_t *v, int64_t sb, int64_t sh,
                                                     int64_t st, int n_tok, int64_t pfloats, float *ws) {
  constexpr int NZ = RKMAX + kD;
  constexpr int NIT = RKMAX / 16, NJT = (NZ / 16 + 3) / 4;
  __shared__ __align__(16) bf16_t sz[NZ * kGPitch];
  const int P = gridDim.x, p = blockIdx.x, unit = blockIdx.y;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const HeadInfo hd = L.heads[h];
  const int rk = hd.rk, nz = rk + kD;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const int nt = (n_tok + kGTile - 1) / kGTile;
  const int tlo = int(int64_t(p) * nt / P), thi = int(int64_t(p + 1) * nt / P);
  const bf16_t *codes = static_cast<const bf16_t *>(L.codes_k) + hd.ck + int64_t(b) * L.cap * rk;
  const bf16_t *vb = v + b * sb + h * sh;
  const int tg = tid & 15, grp = tid >> 4;  // tokens 4 tg .. 4 tg + 3; column / feature group grp
  const bool has_code = grp < rk / 8;

  f32x4 acc[NIT][NJT];
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int jj = 0; jj < NJT; ++jj) acc[it][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Tile {
    u32x4 k[4], v[4];
  };
  // tokens past n_tok are read clamped and zeroed when staged (no wait at the load)
  auto load = [&](int tile, Tile &t) {
    const int cg = has_code ? grp : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tok = min(tile * kGTile + 4 * tg + u, n_tok - 1);
      t.k[u] = *reinterpret_cast<const u32x4 *>(codes + kslot(tok, 8 * cg, rk));
      t.v[u] = *reinterpret_cast<const u32x4 *>(vb + int64_t(tok) * st + 8 * grp);
    }
  };
  // word w of a piece holds columns 2 w (low half) and 2 w + 1 (high half)
  auto put = [&](int row0, const u32x4 (&x)[4], bool valid0, bool valid1, bool valid2, bool valid3) {
    u32x4 r[4];
    r[0] = valid0 ? x[0] : u32x4{0u, 0u, 0u, 0u};
    r[1] = valid1 ? x[1] : u32x4{0u, 0u, 0u, 0u};
    r[2] = valid2 ? x[2] : u32x4{0u, 0u, 0u, 0u};
    r[3] = valid3 ? x[3] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x2 lo = {(r[0][w] & 0xffffu) | (r[1][w] << 16), (r[2][w] & 0xffffu) | (r[3][w] << 16)};
      const u32x2 hi = {(r[0][w] >> 16) | (r[1][w] & 0xffff0000u), (r[2][w] >> 16) | (r[3][w] & 0xffff0000u)};
      *reinterpret_cast<u32x2 *>(&sz[(row0 + 2 * w) * kGPitch + 4 * tg]) = lo;
      *reinterpret_cast<u32x2 *>(&sz[(row0 + 2 * w + 1) * kGPitch + 4 * tg]) = hi;
    }
  };
  auto stage = [&](int tile, const Tile &t) {
    const int t0 = tile * kGTile + 4 * tg;
    const bool v0 = t0 < n_tok, v1 = t0 + 1 < n_tok, v2 = t0 + 2 < n_tok, v3 = t0 + 3 < n_tok;
    if (has_code) put(8 * grp, t.k, v0, v1, v2, v3);
    put(rk + 8 * grp, t.v, v0, v1, v2, v3);
  };
  // D[i][j] += sum over the tile's tokens of C[t][i] Z[t][j]: lane (q4, t16) feeds
  // tokens 32 ks + 8 q4 .. +7 of column 16 it + t16 (A) and of column 16 jt + t16 (B)
  auto multiply = [&]() {
#pragma unroll
    for (int ks = 0; ks < kGTile / 32; ++ks) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (it < rk / 16) {
          const u32x4 a = *reinterpret_cast<const u32x4 *>(&sz[(16 * it + t16) * kGPitch + 32 * ks + 8 * q4]);
#pragma unroll
          for (int jj = 0; jj < NJT; ++jj) {
            const int jt = wave + 4 * jj;
            if (jt < nz / 16) {
              const u32x4 bb = *reinterpret_cast<const u32x4 *>(&sz[(16 * jt + t16) * kGPitch + 32 * ks + 8 * q4]);
              acc[it][jj] = mfma16x16x32(a, bb, acc[it][jj]);
            }
          }
        }
      }
    }
  };
  auto step = [&](int tile, Tile &t) {
    __syncthreads();  // the previous tile's readers are done
    stage(tile, t);
    __syncthreads();
    if (tile + 2 < thi) load(tile + 2, t);
    multiply();
  };
  Tile ta, tb;
  if (tlo < thi) load(tlo, ta);
  if (tlo + 1 < thi) load(tlo + 1, tb);
  for (int tile = tlo; tile < thi; tile += 2) {
    step(tile, ta);
    if (tile + 1 < thi) step(tile + 1, tb);
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
// The solve.  One workgroup of 1024 threads per (row, head), float32.  The
// partials are summed in a fixed order (all of them in flight).  A = C^T C +
// lam I is eliminated in LDS right-looking with unscaled columns, one column and
// one barrier per step: a_ij -= a_ik a_jk / a_kk for k < j <= i (threads as a
// 32 x 32 grid over the pairs), which leaves A = K diag(1/d) K^T with K the
// lower triangle (column k as it stood at step k, d_k = K_kk; the Cholesky
// factor is K diag(d)^-1/2).  B = C^T V sits in registers, row i with the eight
// threads 8 i .. 8 i + 7 (16 columns each); in the same steps row k is
// published and every later row takes b_i -= a_ik b_k / a_kk, which leaves
// B = diag(d) Z with K diag(1/d) Z = C^T V.  The backward sweep solves
// K^T M = B the same way: row k of M = b_k / d_k published, b_i -= K_ki m_k for
// i < k, one barrier per row.
// ---------------------------------------------------------------------------
constexpr int kSolveStride = 129;  // LDS row of the 128 x 128 matrices (odd: no bank conflicts down a column)
constexpr int kSolveThreads = 1024;

__global__ __launch_bounds__(kSolveThreads) void k_lowram_solve(LayerArgs L, int P, int64_t pfloats,
                                                                 const float *ws) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  __shared__ float sa[128 * kSolveStride];   // A, then the factor K in its lower triangle
  __shared__ float sbm[128 * kSolveStride];  // B as summed
  __shared__ __align__(16) float srow[2][kD];  // the published row of B (or of M), by step parity
  __shared__ float s_lam;
  const int unit = blockIdx.x;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const HeadInfo hd = L.heads[h];
  const int rk = hd.rk, nz = rk + kD;
  const int tid = threadIdx.x;
  const float *part = ws + int64_t(unit) * P * pfloats;
  // 4 consecutive elements of a row per piece (nz is a multiple of 16)
  for (int e4 = tid; e4 < rk * nz / 4; e4 += kSolveThreads) {
    f4 v[kMaxPartials];
#pragma unroll
    for (int p = 0; p < kMaxPartials; ++p)
      v[p] = *reinterpret_cast<const f4 *>(part + int64_t(min(p, P - 1)) * pfloats + 4 * e4);
    f4 x = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kMaxPartials; ++p)
      if (p < P) x += v[p];  // fixed order
    const int e = 4 * e4, i = e / nz, j = e - i * nz;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (j + c < rk) sa[i * kSolveStride + j + c] = x[c];
      else sbm[i * kSolveStride + (j + c - rk)] = x[c];
    }
  }
  __syncthreads();
  if (tid < 64) {  // lam from the trace (one wave)
    float tr = 0.f;
    for (int i = tid; i < rk; i += 64) tr += sa[i * kSolveStride + i];
    tr = wave_sum(tr);
    if (tid == 0) s_lam = 1e-6f * tr / float(rk) + 1e-30f;
  }
  __syncthreads();
  if (tid < rk) sa[tid * kSolveStride + tid] += s_lam;
  const int ti = tid >> 5, tj = tid & 31;  // A: the 32 x 32 grid
  const int bi = tid >> 3, bc = tid & 7;   // B: row bi, columns bc + 8 q
  float br[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) br[q] = bi < rk ? sbm[bi * kSolveStride + bc + 8 * q] : 0.f;
  __syncthreads();
  auto rcp_d = [&](int k) { return __builtin_amdgcn_rcpf(fmaxf(sa[k * kSolveStride + k], 1e-30f)); };
  auto publish = [&](float *row) {
#pragma unroll
    for (int q = 0; q < 16; ++q) row[bc + 8 * q] = br[q];
  };
  if (bi == 0) publish(srow[0]);
  __syncthreads();
  for (int k = 0; k < rk; ++k) {
    const float inv = __builtin_amdgcn_rcpf(fmaxf(sa[k * kSolveStride + k], 1e-30f));  // hardware reciprocal
    for (int i = k + 1 + ti; i < rk; i += 32) {
      const float aik = sa[i * kSolveStride + k] * inv;
      for (int j = k + 1 + tj; j <= i; j += 32)
        sa[i * kSolveStride + j] = fmaf(-aik, sa[j * kSolveStride + k], sa[i * kSolveStride + j]);
    }
    if (bi > k && bi < rk) {
      const float* row = srow[k & 1];
      const float aik = sa[bi * kSolveStride + k] * inv;
#pragma unroll
      for (int q = 0; q < 16; ++q) br[q] = fmaf(-aik, row[bc + 8 * q], br[q]);
      if (bi == k + 1) publish(srow[(k + 1) & 1]);  // row k + 1 is final now
    }
    __syncthreads();  // also: every read of the other parity's row is done
  }
  // backward
  if (bi == rk - 1) {
    const float r = rcp_d(rk - 1);
#pragma unroll
    for (int q = 0; q < 16; ++q) br[q] *= r;
    publish(srow[(rk - 1) & 1]);
  }
  __syncthreads();
  for (int k = rk - 1; k > 0; --k) {
    if (bi < k) {
      const float* row = srow[k & 1];
      const float kki = sa[k * kSolveStride + bi];
#pragma unroll
      for (int q = 0; q < 16; ++q) br[q] = fmaf(-kki, row[bc + 8 * q], br[q]);
      if (bi == k - 1) {  // row k - 1 is final now: m_{k-1} = b_{k-1} / d_{k-1}
        const float r = rcp_d(k - 1);
#pragma unroll
        for (int q = 0; q < 16; ++q) br[q] *= r;
        publish(srow[(k - 1) & 1]);
      }
    }
    __syncthreads();
  }
  if (bi < rk) {
    bf16_t *mo = static_cast<bf16_t *>(L.pred) + hd.pred + int64_t(b) * rk * kD + bi * kD;
#pragma unroll
    for (int q = 0; q < 16; ++q) mo[bc + 8 * q] = from_f32<bf16_t>(br[q]);
  }
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
  hipLaunchKernelGGL(k_lowram_solve, dim3(units), dim3(kSolveThreads), 0, s, L, P, pf, static_cast<const float *>(ws));
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
