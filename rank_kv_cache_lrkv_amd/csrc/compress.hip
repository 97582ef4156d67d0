// Cache writers: prefill projection into codes, full-rank anchor stores and the
// per-step maintenance that moves the token leaving the recent window into the
// code region.
//
// Prefill projection follows the blog "Half the Memory, None of the Answers
// Lost", section 04 (one projection per (layer, head), keys after RoPE); the
// anchor policy follows the OjaKV article's FAQ (first token and the most recent
// tokens stay at full rank).

#include "decode_common.h"

namespace lrkv {

// ---------------------------------------------------------------------------
// Generic projection (float32 storage, which has no head groups; bf16 and
// quantised codes run on the matrix cores, see compress_mfma.hip).
// One workgroup per (64-token tile, batch row, KV head).  The 64x128 input tile
// is staged in LDS as float32; each thread produces code columns with a float32
// dot product over the 128 features against a basis row (read through the cache).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_compress_generic(LayerArgs L, int which, const T *x,
                                                          int64_t sb, int64_t sh, int64_t st,
                                                          int n_tok, int slot0) {
  constexpr int TT = 64;
  __shared__ float sx[TT][kD + 1];
  const int unit = blockIdx.y;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const HeadInfo hd = L.heads[h];
  const int r = which ? hd.rv : hd.rk;
  const T *U = static_cast<const T *>(L.bases) + (which ? hd.u_v : hd.u_k);
  T *codes = static_cast<T *>(which ? L.codes_v : L.codes_k) + (which ? hd.cv : hd.ck) +
             int64_t(b) * L.cap * r;
  const int t0 = blockIdx.x * TT;
  const int nt = min(TT, n_tok - t0);
  const T *xb = x + b * sb + h * sh + int64_t(t0) * st;
  for (int i = threadIdx.x; i < nt * kD; i += blockDim.x) {
    const int t = i / kD, k = i % kD;
    sx[t][k] = to_f32(xb[int64_t(t) * st + k]);
  }
  __syncthreads();
  for (int o = threadIdx.x; o < nt * r; o += blockDim.x) {
    const int t = o / r, c = o % r;
    float acc = 0.f;
    for (int k = 0; k < kD; ++k) acc = fmaf(sx[t][k], to_f32(U[c * kD + k]), acc);
    const int j = slot0 + t0 + t;
    codes[which ? vslot(j, c, r) : kslot(j, c, r)] = from_f32<T>(acc);
  }
}

// ---------------------------------------------------------------------------
// Anchor store: one workgroup (128 threads, one per feature) per (token, row, head).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(128) void k_store_anchors(LayerArgs L, const T *k, const T *v,
                                                       int64_t sb, int64_t sh, int64_t st,
                                                       int pos0) {
  const int t = blockIdx.x;
  const int unit = blockIdx.y;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const int slot = anchor_slot(pos0 + t, L.window);
  const int64_t src = b * sb + h * sh + int64_t(t) * st + threadIdx.x;
  const int64_t dst = (int64_t(unit) * (1 + L.window) + slot) * kD + threadIdx.x;
  static_cast<T *>(L.anchor_k)[dst] = k[src];
  static_cast<T *>(L.anchor_v)[dst] = v[src];
}

// ---------------------------------------------------------------------------
// Decode-step maintenance: one workgroup (128 threads) per (row, latent group),
// that is per (row, KV head) without head groups.  The rows to compress (one per
// KV head of the group) are staged in LDS before the anchor slots are
// overwritten, so the read of a leaving token and the write of the new one
// cannot overlap.  Thread t makes code column t from the concatenated rows: the
// sum over the group's KV heads j of row_j . (slice j of basis row t).
// ---------------------------------------------------------------------------
// largest |x| over the 128 threads of the workgroup (every thread calls it)
__device__ __forceinline__ float block_absmax(float x, float *red) {
  const float w = wave_max(fabsf(x));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  const float a = fmaxf(red[0], red[1]);
  __syncthreads();
  return a;
}

// sum over the 128 threads of the workgroup (every thread calls it)
__device__ __forceinline__ float block_sum(float x, float *red) {
  float w = x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) w += __shfl_xor(w, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  const float a = red[0] + red[1];
  __syncthreads();
  return a;
}

// LowRAM (values from the key codes, residuals kept for the worst-predicted
// tokens of each block): the value of code slot j enters its block.  Thread t
// holds column t of the stored key code (0 past rank_k) and feature t of the
// value.  e = v - code M (float32); a slot opening a block empties the block's
// entries first; the residual takes an empty entry, else replaces the entry of
// smallest squared norm (among equal ones the highest slot) if its own norm is
// strictly larger.  Inserting a block's slots in order this way keeps its R
// largest norms (equal norms: the lower slots).
__device__ void lowram_insert(const LayerArgs &L, int h, int b, int j, float code_t, float v_t, float *red) {
  __shared__ float s_code[kD];
  __shared__ int s_take;
  const int tid = threadIdx.x;
  const HeadInfo hd = L.heads[h];
  s_code[tid] = code_t;
  __syncthreads();
  const bf16_t *m = static_cast<const bf16_t *>(L.pred) + hd.pred + int64_t(b) * hd.rk * kD;
  float pr = 0.f;
  for (int c = 0; c < hd.rk; ++c) pr = fmaf(s_code[c], to_f32(m[c * kD + tid]), pr);
  const float e = v_t - pr;
  const float sq = block_sum(e * e, red);
  const int blk = j / kBlock, sl = j % kBlock;
  const int64_t e0 = resid_entry(L, h, b, blk, 0);
  if (tid == 0) {
    if (sl == 0)
      for (int i = 0; i < L.R; ++i) L.rslot[e0 + i] = -1;
    int take = -1, low = -1;
    float lown = 0.f;
    for (int i = 0; i < L.R; ++i) {
      const int si = L.rslot[e0 + i];
      if (si < 0) {
        if (take < 0) take = i;
      } else {
        const float ni = L.rnorm[e0 + i];
        if (low < 0 || ni < lown || (ni == lown && si > L.rslot[e0 + low])) {
          low = i;
          lown = ni;
        }
      }
    }
    if (take < 0 && low >= 0 && sq > lown) take = low;
    if (take >= 0) {
      L.rslot[e0 + take] = sl;
      L.rnorm[e0 + take] = sq;
    }
    s_take = take;
  }
  __syncthreads();
  if (s_take >= 0) static_cast<bf16_t *>(L.resid)[(e0 + s_take) * kD + tid] = from_f32<bf16_t>(e);
}

// Eight consecutive elements of a basis row: one 16-byte piece of a bf16 row,
// two of a float32 row.
template <typename T> struct Piece;
template <> struct Piece<bf16_t> { uint4 a; };
template <> struct Piece<float> { float4 a, b; };
__device__ __forceinline__ Piece<bf16_t> load_piece(const bf16_t *p, int off) {
  return Piece<bf16_t>{*reinterpret_cast<const uint4 *>(p + off)};
}
__device__ __forceinline__ Piece<float> load_piece(const float *p, int off) {
  return Piece<float>{*reinterpret_cast<const float4 *>(p + off), *reinterpret_cast<const float4 *>(p + off + 4)};
}
__device__ __forceinline__ void unpack_piece(const Piece<bf16_t> &w, float (&u)[8]) {
  const uint32_t ww[4] = {w.a.x, w.a.y, w.a.z, w.a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u[2 * i] = __uint_as_float(ww[i] << 16);
    u[2 * i + 1] = __uint_as_float(ww[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack_piece(const Piece<float> &w, float (&u)[8]) {
  u[0] = w.a.x, u[1] = w.a.y, u[2] = w.a.z, u[3] = w.a.w;
  u[4] = w.b.x, u[5] = w.b.y, u[6] = w.b.z, u[7] = w.b.w;
}
// column steps (8 code columns each) of the append whose basis loads are in
// flight together
constexpr int kSteps = 16;

// QMAX: 0 for bf16 / f32 codes, 127 for int8 codes, 7 for 4-bit codes
template <typename T, int QMAX>
__global__ __launch_bounds__(128) void k_append(LayerArgs L, const T *knew, const T *vnew, int pos) {
  __shared__ float rk_row[LRKV_MAX_HEAD_GROUP][kD], rv_row[LRKV_MAX_HEAD_GROUP][kD];
  __shared__ float red[2];
  // setup reads in two rounds: the kernel-argument scalars (taken together by
  // the empty asm; the divisor passes through it, so the division cannot start,
  // and wait, before every load is issued), then the group's row of the head table
  int nlat = L.n_lat;
  __asm__ volatile("" : "+s"(nlat)
                   : "s"(L.hg), "s"(L.window), "s"(L.n_kv), "s"(L.n_versions), "s"(L.vstart), "s"(L.version_elems),
                     "s"(L.bases), "s"(L.lowram), "s"(L.anchor_k), "s"(L.anchor_v), "s"(L.rope), "s"(L.cap),
                     "s"(L.codes_k), "s"(L.codes_v));
  const int unit = blockIdx.x;
  const int b = unit / nlat, h = unit % nlat;
  const int hg = L.hg;
  const int W = L.window;
  const int tid = threadIdx.x;
  const HeadInfo hd = L.heads[h];
  __asm__ volatile("" ::"s"(hd.rk), "s"(hd.rv), "s"(hd.u_k), "s"(hd.u_v));
  const int64_t kv0 = int64_t(b) * L.n_kv + int64_t(h) * hg;  // the group's first (row, KV head)
  auto ak = [&](int j) { return static_cast<T *>(L.anchor_k) + (kv0 + j) * (1 + W) * kD; };
  auto av = [&](int j) { return static_cast<T *>(L.anchor_v) + (kv0 + j) * (1 + W) * kD; };
  auto kn = [&](int j) { return knew + (kv0 + j) * kD; };
  auto vn = [&](int j) { return vnew + (kv0 + j) * kD; };

  int slot = -1, code_slot = -1;
  if (W >= 1 && pos > W) {
    slot = 1 + (pos - 1) % W;  // holds token pos - W, which now leaves the window
    code_slot = pos - W - 1;
  } else if (W == 0 && pos >= 1) {
    code_slot = pos - 1;
  } else {
    slot = anchor_slot(pos, W);
  }
  // basis version of the code slot: the last one starting at or before it
  int ver = 0;
  if (code_slot >= 0)
    for (int v = 1; v < L.n_versions; ++v)
      if (L.vstart[int64_t(b) * L.n_versions + v] <= code_slot) ver = v;
  const T *Uk = static_cast<const T *>(L.bases) + ver * L.version_elems + hd.u_k;
  const T *Uv = static_cast<const T *>(L.bases) + ver * L.version_elems + hd.u_v;
  const int urow = hg * kD;  // elements of a basis row (U^T row)
  const int lane = tid & 63, q = lane >> 4, f8 = lane & 15, wave = tid >> 6;
  const int ncol = hd.rk + (L.lowram ? 0 : hd.rv);  // LowRAM layers have no value codes
  auto basis_piece = [&](int e00, int k, int j) {  // this lane's piece of step k of a chunk
    const int ec = min(e00 + 8 * k + 4 * wave + q, ncol - 1);
    return load_piece(ec < hd.rk ? Uk + ec * urow : Uv + (ec - hd.rk) * urow, j * kD + 8 * f8);
  };
  // the first chunk's basis pieces of the first KV head are requested before the
  // leaving row, so the two round trips overlap
  Piece<T> w0[kSteps];
  if (code_slot >= 0) {
#pragma unroll
    for (int k = 0; k < kSteps; ++k) w0[k] = basis_piece(0, k, 0);
  }
  // the new token's key and value (stored into the ring at the end), requested now
  T kx[LRKV_MAX_HEAD_GROUP], vx[LRKV_MAX_HEAD_GROUP];
  if (slot >= 0) {
#pragma unroll
    for (int j = 0; j < LRKV_MAX_HEAD_GROUP; ++j) {
      if (j < hg) {
        kx[j] = kn(j)[tid];
        vx[j] = vn(j)[tid];
      }
    }
  }
  if (W >= 1 && pos > W) {
    for (int j = 0; j < hg; ++j) {
      rk_row[j][tid] = to_f32(ak(j)[slot * kD + tid]);
      rv_row[j][tid] = to_f32(av(j)[slot * kD + tid]);
    }
  } else if (W == 0 && pos >= 1) {
    for (int j = 0; j < hg; ++j) {
      rk_row[j][tid] = to_f32(kn(j)[tid]);
      rv_row[j][tid] = to_f32(vn(j)[tid]);
    }
  }
  __syncthreads();
  if (L.rope && code_slot >= 0) {  // keys compressed before RoPE: the leaving (post-RoPE)
                                   // key turned back by its position's angle
    if (tid < kD / 2) {
      const float p = float(W >= 1 ? pos - W : pos);
      const float rev = rope_rev(L.rope_a[tid][0], L.rope_a[tid][1], p);
      const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
      const float x = rk_row[0][tid], y = rk_row[0][tid + kD / 2];
      rk_row[0][tid] = fmaf(x, cs, y * sn);
      rk_row[0][tid + kD / 2] = fmaf(y, cs, -(x * sn));
    }
    __syncthreads();
  }
  __shared__ float res[2 * kD];
  if (code_slot >= 0) {  // uniform over the workgroup
    // Column e of the codes (key columns 0 .. rk - 1, then value columns) is the
    // dot product of the leaving row(s) with basis row e: 16 lanes share a
    // column, lane f8 taking features 8 f8 .. 8 f8 + 7 of every 128-slice, four
    // columns per wave and step, the lanes' partial sums added by shuffles inside
    // each 16-lane group.  The basis pieces of kSteps steps (a chunk) are loaded
    // together, every load from a clamped in-range row, before any is used: one
    // round trip per chunk (one for ranks up to 128 columns in all) instead of
    // one per step.
    for (int e00 = 0; e00 < ncol; e00 += 8 * kSteps) {
      float acc[kSteps];
#pragma unroll
      for (int k = 0; k < kSteps; ++k) acc[k] = 0.f;
      for (int j = 0; j < hg; ++j) {
        Piece<T> w[kSteps];
        if (e00 == 0 && j == 0) {
#pragma unroll
          for (int k = 0; k < kSteps; ++k) w[k] = w0[k];
        } else {
#pragma unroll
          for (int k = 0; k < kSteps; ++k) w[k] = basis_piece(e00, k, j);
        }
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
          const int ec = min(e00 + 8 * k + 4 * wave + q, ncol - 1);
          const float *xr = (ec < hd.rk ? rk_row[j] : rv_row[j]) + 8 * f8;
          float u[8];
          unpack_piece(w[k], u);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[k] = fmaf(u[i], xr[i], acc[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < kSteps; ++k) {
        float a = acc[k];
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
        const int e = e00 + 8 * k + 4 * wave + q;
        if (f8 == 0 && e < ncol) res[e] = a;
      }
    }
    __syncthreads();
    const float acck = tid < hd.rk ? res[tid] : 0.f;
    const float accv = tid < hd.rv && !L.lowram ? res[hd.rk + tid] : 0.f;
    if constexpr (QMAX > 0) {
      const float sk = qn_scale<QMAX>(block_absmax(tid < hd.rk ? acck : 0.f, red));
      const float sv = qn_scale<QMAX>(block_absmax(tid < hd.rv ? accv : 0.f, red));
      const int64_t rgk = hd.ck + int64_t(b) * L.cap * hd.rk, rgv = hd.cv + int64_t(b) * L.cap * hd.rv;
      if constexpr (QMAX == 127) {
        int8_t *ck = static_cast<int8_t *>(L.codes_k) + rgk;
        int8_t *cv = static_cast<int8_t *>(L.codes_v) + rgv;
        if (tid < hd.rk) ck[kslot(code_slot, tid, hd.rk)] = int8_t(qn_value<QMAX>(acck, sk));
        if (tid < hd.rv) cv[vslot(code_slot, tid, hd.rv)] = int8_t(qn_value<QMAX>(accv, sv));
      } else {  // two elements per byte: regions start on even elements
        uint8_t *ck = static_cast<uint8_t *>(L.codes_k) + rgk / 2;
        uint8_t *cv = static_cast<uint8_t *>(L.codes_v) + rgv / 2;
        if (tid < hd.rk) store_q4(ck, kslot(code_slot, tid, hd.rk), qn_value<QMAX>(acck, sk));
        if (tid < hd.rv) store_q4(cv, vslot(code_slot, tid, hd.rv), qn_value<QMAX>(accv, sv));
      }
      if (tid == 0) {
        L.scales_k[scale_index(L, h, b, code_slot)] = sk;
        L.scales_v[scale_index(L, h, b, code_slot)] = sv;
      }
    } else {
      T *ck = static_cast<T *>(L.codes_k) + hd.ck + int64_t(b) * L.cap * hd.rk;
      if (tid < hd.rk) ck[kslot(code_slot, tid, hd.rk)] = from_f32<T>(acck);
      if (!L.lowram) {
        T *cv = static_cast<T *>(L.codes_v) + hd.cv + int64_t(b) * L.cap * hd.rv;
        if (tid < hd.rv) cv[vslot(code_slot, tid, hd.rv)] = from_f32<T>(accv);
      } else {
        lowram_insert(L, h, b, code_slot, tid < hd.rk ? to_f32(from_f32<T>(acck)) : 0.f, rv_row[0][tid], red);
      }
    }
  }
  if (slot >= 0) {
#pragma unroll
    for (int j = 0; j < LRKV_MAX_HEAD_GROUP; ++j) {
      if (j < hg) {
        ak(j)[slot * kD + tid] = kx[j];
        av(j)[slot * kD + tid] = vx[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Quantisation of given float32 code rows (QMAX 127: int8, 7: 4 bits): one wave
// per (token, row, head or latent group), lane l holding columns l and l + 64.
// ---------------------------------------------------------------------------
template <int QMAX>
__global__ __launch_bounds__(256) void k_quantize(LayerArgs L, int which, const float *x, int64_t sb,
                                                  int64_t sh, int64_t st, int n_tok, int slot0) {
  const int t = blockIdx.x * 4 + int(threadIdx.x >> 6);
  const int unit = blockIdx.y;
  const int b = unit / L.n_lat, h = unit % L.n_lat;
  if (t >= n_tok) return;  // no barrier follows
  const HeadInfo hd = L.heads[h];
  const int r = which ? hd.rv : hd.rk;
  const int lane = threadIdx.x & 63;
  const float *row = x + b * sb + h * sh + int64_t(t) * st;
  const float v0 = lane < r ? row[lane] : 0.f;
  const float v1 = lane + 64 < r ? row[lane + 64] : 0.f;
  const float s = qn_scale<QMAX>(wave_max(fmaxf(fabsf(v0), fabsf(v1))));
  const int64_t region = (which ? hd.cv : hd.ck) + int64_t(b) * L.cap * r;
  const int j = slot0 + t;
  auto pos = [&](int c) { return which ? vslot(j, c, r) : kslot(j, c, r); };
  if constexpr (QMAX == 127) {
    int8_t *codes = static_cast<int8_t *>(which ? L.codes_v : L.codes_k) + region;
    if (lane < r) codes[pos(lane)] = int8_t(qn_value<QMAX>(v0, s));
    if (lane + 64 < r) codes[pos(lane + 64)] = int8_t(qn_value<QMAX>(v1, s));
  } else {
    uint8_t *codes = static_cast<uint8_t *>(which ? L.codes_v : L.codes_k) + region / 2;
    if (lane < r) store_q4(codes, pos(lane), qn_value<QMAX>(v0, s));
    if (lane + 64 < r) store_q4(codes, pos(lane + 64), qn_value<QMAX>(v1, s));
  }
  if (lane == 0) (which ? L.scales_v : L.scales_k)[scale_index(L, h, b, j)] = s;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quantize(const LayerArgs &L, int which, const float *x, int64_t sb, int64_t sh,
                           int64_t st, int n_tok, int slot0, hipStream_t s) {
  dim3 grid((n_tok + 3) / 4, L.batch * L.n_lat);
  if (L.dtype == LRKV_BF16_Q8)
    hipLaunchKernelGGL(k_quantize<127>, grid, dim3(256), 0, s, L, which, x, sb, sh, st, n_tok, slot0);
  else
    hipLaunchKernelGGL(k_quantize<7>, grid, dim3(256), 0, s, L, which, x, sb, sh, st, n_tok, slot0);
  return hipGetLastError();
}

hipError_t launch_compress(const LayerArgs &L, int which, const void *x, int64_t sb, int64_t sh,
                           int64_t st, int n_tok, int slot0, hipStream_t s) {
  if (L.dtype != LRKV_F32) return launch_compress_mfma(L, which, x, sb, sh, st, n_tok, slot0, s);
  dim3 grid((n_tok + 63) / 64, L.batch * L.n_kv);
  hipLaunchKernelGGL(k_compress_generic<float>, grid, dim3(256), 0, s, L, which,
                     static_cast<const float *>(x), sb, sh, st, n_tok, slot0);
  return hipGetLastError();
}

hipError_t launch_store_anchors(const LayerArgs &L, const void *k, const void *v, int64_t sb,
                                int64_t sh, int64_t st, int pos0, int n_tok, hipStream_t s) {
  dim3 grid(n_tok, L.batch * L.n_kv);
  if (L.dtype == LRKV_F32)
    hipLaunchKernelGGL(k_store_anchors<float>, grid, dim3(kD), 0, s, L,
                       static_cast<const float *>(k), static_cast<const float *>(v), sb, sh, st, pos0);
  else
    hipLaunchKernelGGL(k_store_anchors<bf16_t>, grid, dim3(kD), 0, s, L,
                       static_cast<const bf16_t *>(k), static_cast<const bf16_t *>(v), sb, sh, st, pos0);
  return hipGetLastError();
}

hipError_t launch_append(const LayerArgs &L, const void *k, const void *v, int pos, hipStream_t s) {
  dim3 grid(L.batch * L.n_lat);
  const bf16_t *kb = static_cast<const bf16_t *>(k), *vb = static_cast<const bf16_t *>(v);
  if (L.dtype == LRKV_F32)
    hipLaunchKernelGGL((k_append<float, 0>), grid, dim3(kD), 0, s, L, static_cast<const float *>(k),
                       static_cast<const float *>(v), pos);
  else if (L.dtype == LRKV_BF16)
    hipLaunchKernelGGL((k_append<bf16_t, 0>), grid, dim3(kD), 0, s, L, kb, vb, pos);
  else if (L.dtype == LRKV_BF16_Q8)
    hipLaunchKernelGGL((k_append<bf16_t, 127>), grid, dim3(kD), 0, s, L, kb, vb, pos);
  else
    hipLaunchKernelGGL((k_append<bf16_t, 7>), grid, dim3(kD), 0, s, L, kb, vb, pos);
  return hipGetLastError();
}

}  // namespace lrkv
