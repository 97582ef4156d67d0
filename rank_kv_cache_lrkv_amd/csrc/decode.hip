// Decode attention read directly from the compressed cache (blog "Half the
// Memory, None of the Answers Lost", section 08: scores against the codes, one
// up-projection per head, the full tensors never rebuilt), with the first token
// and the recent window at full rank (OjaKV article, FAQ on hybrid storage).
//
// Stage 1 (partials) runs one workgroup per (split, batch row, KV head).  A split
// covers a share of the row's code blocks and a share of its anchor rows, and
// all g query heads of the GQA group share every row read.  Stage 2 (combine)
// merges the split records of each query head, up-projects the rank-space sum
// once with U_V, adds the anchor sum and normalises.
//
// Scores are kept in log2 units (scale * log2 e folded into the query), so every
// exponential is a hardware exp2.
//
// This file holds the float32-arithmetic stage 1 (used for float32 storage), the
// combine, and the launchers; the bfloat16 stage 1 on the matrix cores is in
// decode_mfma.hip.

#include "decode_common.h"

namespace lrkv {

// ---------------------------------------------------------------------------
// Stage 1, float32 arithmetic on the vector ALUs, any storage type: a pass over
// the split's codes (query side q~ = U_K^T q), then a pass over its anchor rows
// (query side q) continuing the same running max and denominator.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_partials_generic(LayerArgs L, DecodeArgs d) {
  __shared__ ChunkSmem sm;
  const int S = d.n_splits;
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const int g = L.group;
  const int W = L.window;
  const int tid = threadIdx.x;
  const int n = row_ctx(d, b);
  const HeadInfo hd = L.heads[h];
  const int dk = hd.rk, dv = hd.rv;
  const T *qb = static_cast<const T *>(d.q) + (int64_t(b) * L.n_q + h * g) * kD;
  const int c = max(0, n - 1 - W);
  int blo, bhi, alo, ahi;
  block_share((c + kBlock - 1) / kBlock, split, S, blo, bhi);
  anchor_share(min(n, 1 + W), split, S, alo, ahi);
  const int lo = blo * kBlock, hi = min(bhi * kBlock, c);
  const T *krows = static_cast<const T *>(L.codes_k) + hd.ck + int64_t(b) * L.cap * dk;
  const T *vrows = static_cast<const T *>(L.codes_v) + hd.cv + int64_t(b) * L.cap * dv;
  const T *ak = static_cast<const T *>(L.anchor_k) + int64_t(unit) * (1 + W) * kD;
  const T *av = static_cast<const T *>(L.anchor_v) + int64_t(unit) * (1 + W) * kD;

  // q~ = U_K^T q (U_K^T rows are the key basis directions), scaled into log2 units
  const T *Uk = static_cast<const T *>(L.bases) + hd.u_k;
  for (int i = tid; i < g * dk; i += blockDim.x) {
    const int hh = i / dk, cc = i % dk;
    float acc = 0.f;
    for (int k = 0; k < kD; ++k) acc = fmaf(to_f32(qb[hh * kD + k]), to_f32(Uk[cc * kD + k]), acc);
    sm.sq[hh][cc] = acc * d.scale_log2;
  }
  if (tid < g) {
    sm.m[tid] = kNegInf;
    sm.l[tid] = 0.f;
  }
  float oc[8], oa[8];
  chunked_softmax_pass(
      sm, g, lo, hi, dk, dv, [&](int t, int cc) { return to_f32(krows[kslot(t, cc, dk)]); },
      [&](int t, int cc) { return to_f32(vrows[vslot(t, cc, dv)]); }, oc);
  // the code sums are relative to the max reached after the codes; remember it
  // so they can follow the final max once the anchors are in
  __shared__ float s_mc[LRKV_MAX_GROUP];
  if (tid < g) s_mc[tid] = sm.m[tid];
  for (int i = tid; i < g * kD; i += blockDim.x) sm.sq[i / kD][i % kD] = to_f32(qb[i]) * d.scale_log2;
  chunked_softmax_pass(
      sm, g, alo, ahi, kD, kD, [&](int t, int cc) { return to_f32(ak[t * kD + cc]); },
      [&](int t, int cc) { return to_f32(av[t * kD + cc]); }, oa);

  const int64_t q0 = int64_t(b) * L.n_q + h * g;
  if (tid < g) {
    float *rec = split_record(d, q0 + tid, split);
    rec[0] = sm.m[tid];
    rec[1] = sm.l[tid];
    rec[2] = rec[3] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int o = tid + e * 256;
    if (o < g * dv) {
      const int hh = o / dv;
      // rescale from the max after the codes to the final max (no-op if equal)
      const float mc = s_mc[hh], mf = sm.m[hh];
      split_record(d, q0 + hh, split)[4 + o % dv] = mc == kNegInf ? 0.f : oc[e] * exp2f(mc - mf);
    }
    if (o < g * kD) split_record(d, q0 + o / kD, split)[d.oa + o % kD] = oa[e];
  }
}

// ---------------------------------------------------------------------------
// Stage 2: one workgroup (128 threads = the 128 output features) per
// (query head, batch row), two dependent rounds of loads.  Round 1: the split
// maxima and denominators, and the U_V column of this thread's output feature.
// Round 2: every weighted sum at once.  M = max of the split maxima (finite:
// token 0 is an anchor of every row); weights 2^(m - M); the rank-space sums are
// merged and up-projected once with U_V, the anchor sums (present on the first
// splits only) are merged in the 128-dim space, and the total is normalised.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(128) void k_combine(LayerArgs L, DecodeArgs d, float *out) {
  constexpr int UPRE = 32;  // U_V columns loaded in round 1 (the rest, if any, later)
  constexpr int PRE = 16;   // weighted-sum terms per thread loaded in one go
  __shared__ float s_w[LRKV_MAX_SPLITS];
  __shared__ float s_l[LRKV_MAX_SPLITS];
  __shared__ float s_part[128];
  __shared__ float s_o[kD];
  __shared__ float s_red[2][2];
  const int i = blockIdx.x, b = blockIdx.y;
  const int h = i / L.group;
  const HeadInfo hd = L.heads[h];
  const int rv = hd.rv;
  const int S = d.n_splits;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t qi = int64_t(b) * L.n_q + i;
  const float *rc = split_record(d, qi, 0);
  const int a = min(row_ctx(d, b), 1 + L.window);
  const int per = anchor_rows_per_split(a, S);
  const int sa = min(S, (a + per - 1) / per);  // splits 0 .. sa-1 carry anchor sums
  const T *Uv = static_cast<const T *>(L.bases) + hd.u_v + tid;  // column tid of the U_V^T rows

  // round 1
  float upre[UPRE];
#pragma unroll
  for (int c = 0; c < UPRE; ++c) upre[c] = to_f32(Uv[min(c, rv - 1) * kD]);  // masked at use
  float m = kNegInf;
  for (int s = tid; s < S; s += blockDim.x) {
    const float ms = rc[int64_t(s) * d.rec];
    s_w[s] = ms;
    s_l[s] = rc[int64_t(s) * d.rec + 1];
    m = fmaxf(m, ms);
  }
  m = wave_max(m);
  if (lane == 0) s_red[0][wave] = m;
  __syncthreads();
  const float M = fmaxf(s_red[0][0], s_red[0][1]);
  float l = 0.f;
  for (int s = tid; s < S; s += blockDim.x) {
    const float w = exp2f(s_w[s] - M);  // empty splits: 2^-inf = 0
    s_w[s] = w;
    l = fmaf(w, s_l[s], l);
  }
  l = wave_sum(l);
  if (lane == 0) s_red[1][wave] = l;
  __syncthreads();
  const float Ltot = s_red[1][0] + s_red[1][1];

  // round 2: rank-space sums in `groups` groups of rv threads (group g takes
  // splits g, g + groups, ...) and the anchor sums.  The loads are issued first,
  // unconditionally from clamped in-bounds indices (masked when summed), so that
  // none waits on another.
  const int groups = int(blockDim.x) / rv;
  const int col = tid % rv, grp = tid / rv;
  const int grp_c = min(grp, groups - 1);
  float ov[PRE], av[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int s = min(grp_c + k * groups, S - 1);
    ov[k] = rc[int64_t(s) * d.rec + 4 + col];
    av[k] = rc[int64_t(min(k, sa - 1)) * d.rec + d.oa + tid];
  }
  float oc = 0.f, oa = 0.f;
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int s = grp + k * groups;
    if (grp < groups && s < S) oc = fmaf(s_w[s], ov[k], oc);
    if (k < sa) oa = fmaf(s_w[k], av[k], oa);
  }
  if (grp < groups)
    for (int s = grp + PRE * groups; s < S; s += groups) oc = fmaf(s_w[s], rc[int64_t(s) * d.rec + 4 + col], oc);
  for (int s = PRE; s < sa; ++s) oa = fmaf(s_w[s], rc[int64_t(s) * d.rec + d.oa + tid], oa);
  s_part[tid] = oc;
  __syncthreads();
  if (tid < rv) {
    float o = 0.f;
    for (int g = 0; g < groups; ++g) o += s_part[g * rv + tid];
    s_o[tid] = o;
  }
  __syncthreads();
  float y = 0.f;
#pragma unroll
  for (int c = 0; c < UPRE; ++c) y = fmaf(upre[c], c < rv ? s_o[c] : 0.f, y);
  for (int c = UPRE; c < rv; ++c) y = fmaf(to_f32(Uv[c * kD]), s_o[c], y);
  out[qi * kD + tid] = (y + oa) / Ltot;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_decode_partials(const LayerArgs &L, const DecodeArgs &d, hipStream_t s) {
  if (L.dtype == LRKV_BF16) return launch_partials_mfma(L, d, s);
  dim3 grid(d.n_splits, L.batch * L.n_kv);
  hipLaunchKernelGGL(k_partials_generic<float>, grid, dim3(256), 0, s, L, d);
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
