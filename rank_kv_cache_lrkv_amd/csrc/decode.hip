// Decode attention read directly from the compressed cache (blog "Half the
// Memory, None of the Answers Lost", section 08: scores against the codes, one
// up-projection per head, the full tensors never rebuilt), with the first token
// and the recent window at full rank (OjaKV article, FAQ on hybrid storage).
//
// Stage 1 (partials) runs one workgroup per (split, batch row, KV head) over the
// codes, plus one workgroup per (batch row, KV head) over the anchors; all g
// query heads of a GQA group share every code row read.  Stage 2 (combine) merges
// the partials of each query head and up-projects once.
//
// Scores are kept in log2 units (scale * log2 e folded into the query), so every
// exponential is a hardware exp2.

#include "lrkv_internal.h"

namespace lrkv {

constexpr float kNegInf = -__builtin_huge_valf();

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

// ---------------------------------------------------------------------------
// Generic stage 1: float32 storage (and the plain path for any storage type).
// Chunks of 64 tokens: scores for all g heads into LDS, one online-softmax
// update per head (a wave per head), then the value sums, each thread owning a
// few (head, column) accumulators.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_partials_generic(LayerArgs L, DecodeArgs d) {
  constexpr int CH = 64;
  constexpr int NACC = LRKV_MAX_GROUP * kD / 256;
  __shared__ float sq[LRKV_MAX_GROUP][kD];
  __shared__ float sp[LRKV_MAX_GROUP][CH];
  __shared__ float s_m[LRKV_MAX_GROUP], s_l[LRKV_MAX_GROUP], s_alpha[LRKV_MAX_GROUP];

  const int S = d.n_splits;
  const int split = blockIdx.x;
  const bool anchors = split == S;
  const int unit = blockIdx.y;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const int g = L.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = row_ctx(d, b);
  const int W = L.window;
  const HeadInfo hd = L.heads[h];
  const T *qb = static_cast<const T *>(d.q) + (int64_t(b) * L.n_q + h * g) * kD;

  int lo, hi, dk, dv;
  const T *krows, *vrows;
  if (anchors) {
    lo = 0;
    hi = min(n, 1 + W);
    dk = dv = kD;
    krows = static_cast<const T *>(L.anchor_k) + int64_t(unit) * (1 + W) * kD;
    vrows = static_cast<const T *>(L.anchor_v) + int64_t(unit) * (1 + W) * kD;
  } else {
    const int c = max(0, n - 1 - W);
    const int nblk = (c + kBlock - 1) / kBlock;
    lo = int((int64_t(split) * nblk) / S) * kBlock;
    hi = min(int((int64_t(split + 1) * nblk) / S) * kBlock, c);
    dk = hd.rk;
    dv = hd.rv;
    krows = static_cast<const T *>(L.codes_k) + hd.ck + int64_t(b) * L.cap * hd.rk;
    vrows = static_cast<const T *>(L.codes_v) + hd.cv + int64_t(b) * L.cap * hd.rv;
  }
  auto kval = [&](int t, int c) -> float {
    return anchors ? to_f32(krows[t * kD + c]) : to_f32(krows[kslot(t, c, dk)]);
  };
  auto vval = [&](int t, int c) -> float {
    return anchors ? to_f32(vrows[t * kD + c]) : to_f32(vrows[vslot(t, c, dv)]);
  };

  // the query side: q itself for the anchors, q~ = U_K^T q for the codes
  if (anchors) {
    for (int i = tid; i < g * kD; i += blockDim.x) sq[i / kD][i % kD] = to_f32(qb[i]) * d.scale_log2;
  } else {
    const T *Uk = static_cast<const T *>(L.bases) + hd.u_k;
    for (int i = tid; i < g * dk; i += blockDim.x) {
      const int hh = i / dk, c = i % dk;
      float acc = 0.f;
      for (int k = 0; k < kD; ++k) acc = fmaf(to_f32(qb[hh * kD + k]), to_f32(Uk[k * dk + c]), acc);
      sq[hh][c] = acc * d.scale_log2;
    }
  }
  if (tid < g) {
    s_m[tid] = kNegInf;
    s_l[tid] = 0.f;
  }
  float acc[NACC];
#pragma unroll
  for (int e = 0; e < NACC; ++e) acc[e] = 0.f;
  __syncthreads();

  for (int base = lo; base < hi; base += CH) {
    const int nv = min(CH, hi - base);
    for (int p = tid; p < g * CH; p += blockDim.x) {
      const int hh = p / CH, j = p % CH;
      float s = kNegInf;
      if (j < nv) {
        float a = 0.f;
        for (int c = 0; c < dk; ++c) a = fmaf(sq[hh][c], kval(base + j, c), a);
        s = a;
      }
      sp[hh][j] = s;
    }
    __syncthreads();
    for (int hh = wave; hh < g; hh += 4) {
      const float s = sp[hh][lane];
      const float mo = s_m[hh];
      const float mn = fmaxf(mo, wave_max(s));
      const float p = exp2f(s - mn);  // s = -inf -> 0; mn is finite (nv >= 1)
      sp[hh][lane] = p;
      const float ps = wave_sum(p);
      if (lane == 0) {
        const float al = exp2f(mo - mn);  // mo = -inf -> 0
        s_alpha[hh] = al;
        s_l[hh] = s_l[hh] * al + ps;
        s_m[hh] = mn;
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NACC; ++e) {
      const int o = tid + e * 256;
      if (o < g * dv) {
        const int hh = o / dv, c = o % dv;
        float a = acc[e] * s_alpha[hh];
        for (int j = 0; j < nv; ++j) a = fmaf(sp[hh][j], vval(base + j, c), a);
        acc[e] = a;
      }
    }
    __syncthreads();
  }

  // write the partial record of each query head of the group
  for (int hh = 0; hh < g; ++hh) {
    const int64_t qi = int64_t(b) * L.n_q + h * g + hh;
    float *rec = anchors ? d.ws_anchor + qi * kAnchorRec : d.ws_codes + (qi * S + split) * d.rec;
    if (tid == 0) {
      rec[0] = s_m[hh];
      rec[1] = s_l[hh];
    }
  }
#pragma unroll
  for (int e = 0; e < NACC; ++e) {
    const int o = tid + e * 256;
    if (o < g * dv) {
      const int hh = o / dv, c = o % dv;
      const int64_t qi = int64_t(b) * L.n_q + h * g + hh;
      float *rec = anchors ? d.ws_anchor + qi * kAnchorRec : d.ws_codes + (qi * S + split) * d.rec;
      rec[4 + c] = acc[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 2: one workgroup (128 threads = the 128 output features) per
// (query head, batch row).  M = max of all partial maxima (the anchor partial is
// never empty, so M is finite); weights 2^(m - M); the rank-space sums are merged,
// up-projected once with U_V, added to the anchor sum and normalised.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(128) void k_combine(LayerArgs L, DecodeArgs d, float *out) {
  __shared__ float s_w[LRKV_MAX_SPLITS];
  __shared__ float s_o[kD];
  __shared__ float s_red[2][2];
  const int i = blockIdx.x, b = blockIdx.y;
  const int h = i / L.group;
  const HeadInfo hd = L.heads[h];
  const int rv = hd.rv;
  const int S = d.n_splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t qi = int64_t(b) * L.n_q + i;
  const float *rc = d.ws_codes + qi * S * d.rec;
  const float *ra = d.ws_anchor + qi * kAnchorRec;

  const float ma = ra[0];
  float m = ma;
  for (int s = tid; s < S; s += blockDim.x) m = fmaxf(m, rc[int64_t(s) * d.rec]);
  m = wave_max(m);
  if (lane == 0) s_red[0][wave] = m;
  __syncthreads();
  const float M = fmaxf(s_red[0][0], s_red[0][1]);
  float l = 0.f;
  for (int s = tid; s < S; s += blockDim.x) {
    const float w = exp2f(rc[int64_t(s) * d.rec] - M);
    s_w[s] = w;
    l = fmaf(w, rc[int64_t(s) * d.rec + 1], l);
  }
  l = wave_sum(l);
  if (lane == 0) s_red[1][wave] = l;
  __syncthreads();
  const float wa = exp2f(ma - M);
  const float Ltot = s_red[1][0] + s_red[1][1] + wa * ra[1];
  if (tid < rv) {
    float o = 0.f;
    for (int s = 0; s < S; ++s) o = fmaf(s_w[s], rc[int64_t(s) * d.rec + 4 + tid], o);
    s_o[tid] = o;
  }
  __syncthreads();
  const T *Uv = static_cast<const T *>(L.bases) + hd.u_v + tid * rv;
  float y = 0.f;
  for (int c = 0; c < rv; ++c) y = fmaf(to_f32(Uv[c]), s_o[c], y);
  out[qi * kD + tid] = (y + wa * ra[4 + tid]) / Ltot;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_decode_partials(const LayerArgs &L, const DecodeArgs &d, hipStream_t s) {
  dim3 grid(d.n_splits + 1, L.batch * L.n_kv);
  if (L.dtype == LRKV_F32)
    hipLaunchKernelGGL(k_partials_generic<float>, grid, dim3(256), 0, s, L, d);
  else
    hipLaunchKernelGGL(k_partials_generic<bf16_t>, grid, dim3(256), 0, s, L, d);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const LayerArgs &L, const DecodeArgs &d, float *out, hipStream_t s) {
  dim3 grid(L.n_q, L.batch);
  if (L.dtype == LRKV_F32)
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(kD), 0, s, L, d, out);
  else
    hipLaunchKernelGGL(k_combine<bf16_t>, grid, dim3(kD), 0, s, L, d, out);
  return hipGetLastError();
}

}  // namespace lrkv
