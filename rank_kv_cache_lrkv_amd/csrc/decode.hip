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
// Stage 2: one workgroup of 128 threads (t = the output features) per (query
// head i, batch row b) merges that head's split records, with a single
// round of loads: every term a thread needs (split maxima and denominators,
// rank-space sums, anchor sums, its U_V column) is loaded at once from clamped
// in-bounds indices and masked when used.  The threads form `groups` groups of
// rv threads; group g merges splits g, g + groups, ... under its own max, then
// the groups are merged under the common max M (finite: token 0 is an anchor
// of every row, held by split 0).  The merged rank-space sum is up-projected
// once with U_V, the anchor sums (on the first splits only) are added in the
// 128-dim space, and the total is normalised.
// Loads go through buffer resources (32-bit offsets).
// ---------------------------------------------------------------------------
struct CombineSmem {
  float m[128 / 16], l[128 / 16];  // per group of rv threads
  float o[128];                    // per thread: its group's rank-space sum
  float ot[128];                   // the merged rank-space sum
};

template <typename T>
__global__ __launch_bounds__(128) void k_combine(LayerArgs L, DecodeArgs d, float *out) {
  constexpr int UPRE = 32;  // U_V columns loaded up front (the rest, if any, later)
  constexpr int PRE = 16;   // terms per thread loaded up front (the rest, if any, later)
  __shared__ CombineSmem cs;
  const int i = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int kvh = i / L.group;                 // KV head; its latent group and slice
  const int h = kvh / L.hg, j = kvh % L.hg;
  const HeadInfo hd = L.heads[h];
  const int rv = hd.rv;
  const int S = d.n_splits;
  const int64_t qi = int64_t(b) * L.n_q + i;
  const float *rc = split_record(d, qi, 0);
  const __amdgpu_buffer_rsrc_t rr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(rc), 0, S * d.rec * 4, kBufferWord3);
  auto rec = [&](int s, int f) {  // float f of split s's record
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, (s * d.rec + f) * 4, 0, 0));
  };
  const int a1 = min(row_ctx(d, b), 1 + L.window);  // anchor rows per KV head
  const int per = anchor_rows_per_split(a1 * L.hg, S);
  // splits s_a0 .. s_a1 - 1 hold this KV head's anchor rows j a1 .. (j + 1) a1 - 1
  // (the unit's rows, KV head after KV head, cut into runs of per rows); LowRAM:
  // every split holds residual sums there
  const int s_a0 = L.lowram ? 0 : (j * a1) / per;
  const int s_a1 = L.lowram ? S : min(S, ((j + 1) * a1 + per - 1) / per);
  // U_V^T rows (hg * 128 elements, this KV head's slice at j * 128), or for LowRAM
  // the row's predictor M (rank_k rows of 128): element (c, t) of the slice is
  // column c of output feature t
  const int urow = L.hg * kD;
  const T *ubase = L.lowram ? static_cast<const T *>(L.pred) + hd.pred + int64_t(b) * rv * kD
                            : static_cast<const T *>(L.bases) + hd.u_v;
  const __amdgpu_buffer_rsrc_t ur =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(ubase), 0, rv * urow * int(sizeof(T)), kBufferWord3);
  auto uv = [&](int c) { return buffer_elem<T>(ur, (c * urow + j * kD + t) * int(sizeof(T))); };
  const int groups = 128 / rv;
  const int col = t % rv, grp = t / rv;
  const int grp_c = min(grp, groups - 1);

  float upre[UPRE];
  float2 ml[PRE];
  float ov[PRE], ma[PRE], av[PRE];
  float mg = kNegInf, lg = 0.f, og = 0.f;
#pragma unroll
  for (int c = 0; c < UPRE; ++c) upre[c] = uv(min(c, rv - 1));
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int s = min(grp_c + k * groups, S - 1);
    ml[k] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rr, s * d.rec * 4, 0, 0));
    ov[k] = rec(s, 4 + col);
    const int sk = min(s_a0 + k, s_a1 - 1);
    ma[k] = rec(sk, 0);
    av[k] = rec(sk, d.oa + t);
  }
  // this group's splits under the group's own max
#pragma unroll
  for (int k = 0; k < PRE; ++k)
    if (grp_c + k * groups < S) mg = fmaxf(mg, ml[k].x);
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    if (grp_c + k * groups < S && ml[k].x != kNegInf) {  // empty splits hold nothing
      const float w = fast_exp2(ml[k].x - mg);
      lg = fmaf(w, ml[k].y, lg);
      og = fmaf(w, ov[k], og);
    }
  }
  // more splits than loaded up front: 8 at a time, all loads issued before the merge
  for (int s0 = grp_c + PRE * groups; s0 < S; s0 += 8 * groups) {
    float2 mlx[8];
    float ovx[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u * groups, S - 1);
      mlx[u] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rr, s * d.rec * 4, 0, 0));
      ovx[u] = rec(s, 4 + col);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float ms = mlx[u].x;
      if (s0 + u * groups >= S || ms == kNegInf) continue;
      const float mn = fmaxf(mg, ms);
      const float a0 = fast_exp2(mg - mn), a1 = fast_exp2(ms - mn);  // mg = -inf gives a0 = 0
      lg = fmaf(a1, mlx[u].y, lg * a0);
      og = fmaf(a1, ovx[u], og * a0);
      mg = mn;
    }
  }
  if (grp < groups) {
    cs.o[t] = og;
    if (col == 0) {
      cs.m[grp] = mg;
      cs.l[grp] = lg;
    }
  }
  __syncthreads();

  float M = kNegInf, Ltot = 0.f, oa = 0.f;
  for (int g = 0; g < groups; ++g) M = fmaxf(M, cs.m[g]);
  for (int g = 0; g < groups; ++g)
    if (cs.m[g] != kNegInf) Ltot = fmaf(fast_exp2(cs.m[g] - M), cs.l[g], Ltot);
  if (t < rv) {
    float o = 0.f;
    for (int g = 0; g < groups; ++g)
      if (cs.m[g] != kNegInf) o = fmaf(fast_exp2(cs.m[g] - M), cs.o[g * rv + t], o);
    cs.ot[t] = o;
  }
  // anchor sums of output feature t (a split without rows of this head has m = -inf: weight 0)
#pragma unroll
  for (int k = 0; k < PRE; ++k)
    if (s_a0 + k < s_a1 && ma[k] != kNegInf) oa = fmaf(fast_exp2(ma[k] - M), av[k], oa);
  for (int s0 = s_a0 + PRE; s0 < s_a1; s0 += 8) {  // 8 at a time, loads first
    float mx[8], ax[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = min(s0 + u, s_a1 - 1);
      mx[u] = rec(s, 0);
      ax[u] = rec(s, d.oa + t);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < s_a1 && mx[u] != kNegInf) oa = fmaf(fast_exp2(mx[u] - M), ax[u], oa);
  }
  __syncthreads();

  float y = 0.f;
#pragma unroll
  for (int c = 0; c < UPRE; ++c) y = fmaf(upre[c], c < rv ? cs.ot[c] : 0.f, y);
  for (int c = UPRE; c < rv; ++c) y = fmaf(uv(c), cs.ot[c], y);
  out[qi * kD + t] = (y + oa) / Ltot;
}

// ---------------------------------------------------------------------------
// Stage 2 with basis versions (codes made under several bases, OjaKV): each
// version's rank-space sum is merged from that version's splits and
// up-projected with that version's U_V; the rest is as in k_combine.  One
// workgroup of 128 threads per (query head, batch row), thread t = output
// feature t.  The splits' maxima, sums and versions (each record carries its
// split's version) are read once into LDS (a thread per split); every later loop runs over LDS or issues its record
// loads eight at a time ahead of the arithmetic.  Sums run split by split in
// index order, as the records are laid out.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(128) void k_combine_versions(LayerArgs L, DecodeArgs d, float *out) {
  __shared__ float sm[LRKV_MAX_SPLITS], sl[LRKV_MAX_SPLITS];  // split maxima, sums
  __shared__ int sv[LRKV_MAX_SPLITS];                         // split versions
  __shared__ float sot[LRKV_MAX_VERSIONS][128];               // per-version rank-space sums
  const int i = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int kvh = i / L.group;
  const int h = kvh / L.hg, j = kvh % L.hg;
  const HeadInfo hd = L.heads[h];
  const int rv = hd.rv;
  const int S = d.n_splits, V = L.n_versions;
  const int64_t qi = int64_t(b) * L.n_q + i;
  const int n = row_ctx(d, b);
  const int a1 = min(n, 1 + L.window);  // anchor rows per KV head
  const int per = anchor_rows_per_split(a1 * L.hg, S);
  const int s_a0 = (j * a1) / per, s_a1 = min(S, ((j + 1) * a1 + per - 1) / per);  // as in k_combine

  // the anchor sums of output feature t from the first 8 splits holding this KV
  // head's anchor rows, requested before anything else (as k_combine does)
  float ax0[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) ax0[u] = split_record(d, qi, min(s_a0 + u, s_a1 - 1))[d.oa + t];
  for (int s = t; s < S; s += blockDim.x) {  // m, l and the version the partials kernel wrote
    const float4 r = *reinterpret_cast<const float4 *>(split_record(d, qi, s));
    sm[s] = r.x;
    sl[s] = r.y;
    sv[s] = min(max(int(r.z), 0), V - 1);
  }
  for (int e = t; e < V * kD; e += blockDim.x) sot[e / kD][e % kD] = 0.f;
  __syncthreads();

  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, sm[s]);  // finite: token 0 is an anchor
  float Ltot = 0.f;
  for (int s = 0; s < S; ++s)
    if (sm[s] != kNegInf) Ltot = fmaf(fast_exp2(sm[s] - M), sl[s], Ltot);
  // each version's merged rank-space sum (the splits of a version are consecutive)
  if (t < rv) {
    float o = 0.f;
    int cur = sv[0];
    for (int s0 = 0; s0 < S; s0 += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = split_record(d, qi, min(s0 + u, S - 1))[4 + t];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u;
        if (s >= S) break;
        if (sv[s] != cur) {
          sot[cur][t] = o;
          o = 0.f;
          cur = sv[s];
        }
        if (sm[s] != kNegInf) o = fmaf(fast_exp2(sm[s] - M), x[u], o);
      }
    }
    sot[cur][t] = o;
  }
  __syncthreads();
  float y = 0.f;
  for (int v = 0; v < V; ++v) {
    const T *uvt = static_cast<const T *>(L.bases) + v * L.version_elems + hd.u_v;  // U_V^T rows
#pragma unroll 8
    for (int cc = 0; cc < rv; ++cc) y = fmaf(to_f32(uvt[cc * L.hg * kD + j * kD + t]), sot[v][cc], y);
  }
  float oa = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int s = s_a0 + u;
    if (s < s_a1 && sm[s] != kNegInf) oa = fmaf(fast_exp2(sm[s] - M), ax0[u], oa);
  }
  for (int s0 = s_a0 + 8; s0 < s_a1; s0 += 8) {  // more anchor splits: 8 at a time, loads first
    float ax[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) ax[u] = split_record(d, qi, min(s0 + u, s_a1 - 1))[d.oa + t];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u;
      if (s < s_a1 && sm[s] != kNegInf) oa = fmaf(fast_exp2(sm[s] - M), ax[u], oa);
    }
  }
  out[qi * kD + t] = (y + oa) / Ltot;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_decode_partials(const LayerArgs &L, const DecodeArgs &d, hipStream_t s) {
  if (L.dtype != LRKV_F32) return launch_partials_mfma(L, d, s);
  dim3 grid(d.n_splits, L.batch * L.n_kv);
  hipLaunchKernelGGL(k_partials_generic<float>, grid, dim3(256), 0, s, L, d);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const LayerArgs &L, const DecodeArgs &d, float *out, hipStream_t s) {
  dim3 grid(L.n_q, L.batch);
  if (L.n_versions > 1)  // float32 layers have one version
    hipLaunchKernelGGL(k_combine_versions<bf16_t>, grid, dim3(kD), 0, s, L, d, out);
  else if (L.dtype == LRKV_F32)
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(kD), 0, s, L, d, out);
  else
    hipLaunchKernelGGL(k_combine<bf16_t>, grid, dim3(kD), 0, s, L, d, out);
  return hipGetLastError();
}

}  // namespace lrkv
