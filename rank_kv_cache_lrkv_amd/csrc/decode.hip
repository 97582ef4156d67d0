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
// combine (with or without basis versions), and the launchers; the bfloat16 stage
// 1 on the matrix cores is in decode_mfma.hip.

#include <algorithm>

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
  const WorkItem wi = work_item(L, d);
  const int S = wi.S, split = wi.split;
  const int b = wi.b, h = wi.h;
  const int unit = b * L.n_kv + h;
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
  // four consecutive threads per element, a quarter of the features each (all
  // 64 of a thread's loads in flight), summed by two lane exchanges
  for (int i0 = 0; i0 < g * dk; i0 += blockDim.x / 4) {
    const int i = min(i0 + (tid >> 2), g * dk - 1), k0 = 32 * (tid & 3);
    const int hh = i / dk, cc = i % dk;
    float x[32], y[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      x[u] = to_f32(qb[hh * kD + k0 + u]);
      y[u] = to_f32(Uk[cc * kD + k0 + u]);
    }
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u) acc = fmaf(x[u], y[u], acc);
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    if ((tid & 3) == 0 && i0 + (tid >> 2) < g * dk) sm.sq[hh][cc] = acc * d.scale_log2;
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
// Stage 2: one workgroup of 128 threads per (query head i, batch row b), thread t
// = output feature t, merges the S_h split records of the head's group.
//
// Everything it reads is cut into 16-byte pieces of three kinds: the splits'
// rank-space sums (rv / 4 pieces per split), the anchor sums of the splits that
// hold this KV head's anchor rows (32 per split), and the U_V rows (128
// elements each, one row per (version, column) pair).  Each thread takes P
// pieces of every kind (P a compile-time instance, chosen on the host from the
// call's sizes), all loaded in one round before any is used, every load
// unconditional from a clamped in-range index (threads whose index was clamped
// write the same data to the same LDS slot as the thread they duplicate);
// pieces past a round's capacity are taken in further rounds.  Then:
//  - every wave finds the common max M (finite: token 0 is an anchor of every
//    row) from the split headers in LDS, and the denominator L;
//  - thread e < V rv sums 2^(m_s - M) o~_s[c] over the splits of version
//    v = e / rv, c = e % rv, in index order (the splits of a version are
//    consecutive; each record carries its version);
//  - thread t sums 2^(m_s - M) o_A,s[t] over the anchor splits in index order,
//    up-projects the merged sums with column t of every U_V row, adds and
//    divides by L.
// U_V is U_V(version)^T of the head's KV head (rows of hg * 128 elements, the
// slice at 128 j), or for LowRAM layers the row's predictor M (rank_k rows of
// 128).  All orders are fixed, so a call is bitwise reproducible.
// ---------------------------------------------------------------------------
constexpr int kCT = 128;  // threads of a combine workgroup

// per-launch geometry of the combine (host-computed): slots per thread, round
// capacities and the LDS layout (byte offsets)
struct CombineArgs {
  int P;                  // pieces of each kind per thread and round
  int na;                 // most anchor splits of any KV head
  int so, sa;             // splits of rank-space sums / anchor sums per round
  int urows;              // U_V rows per round
  int m, l, v, o, a, ov, u, bytes;
};

template <typename T, int P>
__global__ __launch_bounds__(128) void k_combine(LayerArgs L, DecodeArgs d, CombineArgs g, float *out) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  constexpr int kEP = 16 / sizeof(T);          // U_V elements per 16-byte piece
  constexpr int kPPR = kD / kEP;               // pieces per U_V row
  extern __shared__ __align__(16) char lds[];
  // Setup reads in two rounds: every kernel-argument scalar first (the empty asm
  // takes them as operands, so their loads issue together and are waited for
  // once), then the head's row of the head table, its split count and the row
  // length; left to itself the compiler spreads them over six dependent rounds.
  // (The group sizes pass through the first asm, so the divisions by them cannot
  // start, and wait, before every load of the round is issued.)
  int grp = L.group, hgs = L.hg;
  __asm__ volatile("" : "+s"(grp), "+s"(hgs)
                   : "s"(L.n_q), "s"(L.n_versions), "s"(L.window), "s"(L.lowram), "s"(L.pred), "s"(L.bases),
                     "s"(L.version_elems), "s"(d.ws), "s"(d.n_splits), "s"(d.rec), "s"(d.oa), "s"(d.ctx_lens),
                     "s"(d.n_ctx), "s"(g.so), "s"(g.sa), "s"(g.urows), "s"(out), "s"(g.m), "s"(g.l), "s"(g.v),
                     "s"(g.o), "s"(g.a), "s"(g.ov), "s"(g.u));
  const int i = blockIdx.x, b = blockIdx.y, t = threadIdx.x, lane = t & 63;
  const int kvh = i / grp;                     // KV head; its latent group and slice
  const int h = kvh / hgs, j = kvh % hgs;
  const HeadInfo hd = L.heads[h];
  const int n_row = row_ctx(d, b);
  __asm__ volatile("" ::"s"(hd.rv), "s"(hd.u_v), "s"(hd.pred), "s"(d.nsplit[h]), "s"(n_row));
  const int rv = hd.rv;
  const int S = d.nsplit[h], V = L.n_versions;
  float *sm = reinterpret_cast<float *>(lds + g.m);
  float *sl = reinterpret_cast<float *>(lds + g.l);
  int *sv = reinterpret_cast<int *>(lds + g.v);
  float *so = reinterpret_cast<float *>(lds + g.o);   // [split of the round][rv]
  float *sa = reinterpret_cast<float *>(lds + g.a);   // [anchor split of the round][128]
  float *sov = reinterpret_cast<float *>(lds + g.ov); // [version][rv]
  T *su = reinterpret_cast<T *>(lds + g.u);           // [row of the round][128]
  const int64_t qi = int64_t(b) * L.n_q + i;
  const __amdgpu_buffer_rsrc_t rr =
      __builtin_amdgcn_make_buffer_rsrc(split_record(d, qi, 0), 0, S * d.rec * 4, kBufferWord3);
  auto rec4 = [&](int s, int f) {  // floats f .. f + 3 of split s's record
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rr, (s * d.rec + f) * 4, 0, 0));
  };
  const int a1 = min(n_row, 1 + L.window);  // anchor rows per KV head
  const int per = anchor_rows_per_split(a1 * L.hg, S);
  // splits s_a0 .. s_a1 - 1 hold this KV head's anchor rows j a1 .. (j + 1) a1 - 1
  // (the unit's rows, KV head after KV head, cut into runs of per rows); LowRAM:
  // every split holds residual sums there
  const int s_a0 = L.lowram ? 0 : (j * a1) / per;
  const int s_a1 = L.lowram ? S : min(S, ((j + 1) * a1 + per - 1) / per);
  const int na = s_a1 - s_a0;              // >= 1
  const int urow = L.hg * kD;
  const int rows = V * rv;                 // U_V rows: (version, column) pairs
  // U^T row e = (version e / rv, column e % rv) of this KV head's slice, through a
  // buffer resource over every version's rows
  const T *ubase = L.lowram ? static_cast<const T *>(L.pred) + hd.pred + int64_t(b) * rv * kD
                            : static_cast<const T *>(L.bases) + hd.u_v;
  const int vstride = L.lowram ? 0 : int(L.version_elems);
  const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(ubase), 0, ((V - 1) * vstride + rv * urow) * int(sizeof(T)), kBufferWord3);
  // piece k of this thread: sums piece pc of split s_t + s_step k (npc divides
  // 128); anchor piece ac of anchor split a_t + 4 k; U_V piece uc of row
  // u_t + (128 / kPPR) k
  const int npc = rv >> 2, pc = t % npc, s_t = t / npc, s_step = kCT / npc;
  const int ac = t & 31, a_t = t >> 5;
  // this thread's anchor-sum float in a record, held in a register from here: the
  // compiler would otherwise read d.oa from the arguments again just before the
  // anchor loads and wait for it there
  int a_f = d.oa + 4 * ac;
  __asm__ volatile("" : "+v"(a_f));
  const int uc = t % kPPR, u_t = t / kPPR;
  const int sr = min(S, g.so), ar = min(na, g.sa), ur_rows = min(rows, g.urows);
  f4 op[P], ap[P];
  u4 up[P];
  auto load_o = [&](int r0, int nr) {
#pragma unroll
    for (int k = 0; k < P; ++k) op[k] = rec4(r0 + min(s_t + s_step * k, nr - 1), 4 + 4 * pc);
  };
  auto store_o = [&](int nr) {
#pragma unroll
    for (int k = 0; k < P; ++k) *reinterpret_cast<f4 *>(&so[min(s_t + s_step * k, nr - 1) * rv + 4 * pc]) = op[k];
  };
  auto load_a = [&](int r0, int nr) {
#pragma unroll
    for (int k = 0; k < P; ++k) ap[k] = rec4(s_a0 + r0 + min(a_t + 4 * k, nr - 1), a_f);
  };
  auto store_a = [&](int nr) {
#pragma unroll
    for (int k = 0; k < P; ++k) *reinterpret_cast<f4 *>(&sa[min(a_t + 4 * k, nr - 1) * kD + 4 * ac]) = ap[k];
  };
  auto load_u = [&](int e0, int nr) {
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int e = e0 + min(u_t + (kCT / kPPR) * k, nr - 1);
      const int v = e / rv, c = e - v * rv;
      up[k] = __builtin_amdgcn_raw_buffer_load_b128(ur, (v * vstride + c * urow + j * kD + uc * kEP) * int(sizeof(T)),
                                                    0, 0);
    }
  };
  auto store_u = [&](int nr) {
#pragma unroll
    for (int k = 0; k < P; ++k)
      *reinterpret_cast<u4 *>(&su[(min(u_t + (kCT / kPPR) * k, nr - 1) * kPPR + uc) * kEP]) = up[k];
  };

  // ---- one round of loads, then everything to LDS
  const f4 hdr = rec4(min(t, S - 1), 0);
  load_o(0, sr);
  load_u(0, ur_rows);
  load_a(0, ar);
  __asm__ volatile("" ::: "memory");  // the loads stay ahead of every store below
  sm[min(t, S - 1)] = hdr.x;
  sl[min(t, S - 1)] = hdr.y;
  sv[min(t, S - 1)] = min(max(int(hdr.z), 0), V - 1);
  for (int s = t + kCT; s < S; s += kCT) {  // more than 128 splits
    const f4 x = rec4(s, 0);
    sm[s] = x.x;
    sl[s] = x.y;
    sv[s] = min(max(int(x.z), 0), V - 1);
  }
  store_o(sr);
  store_u(ur_rows);
  store_a(ar);
  __syncthreads();

  float M = kNegInf;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, sm[s]);
  M = wave_max(M);
  auto wgt = [&](int s) {  // a split that saw nothing (m = -inf) weighs 0
    const float m = sm[s];
    return m == kNegInf ? 0.f : fast_exp2(m - M);
  };
  float Ltot = 0.f;
  for (int s = lane; s < S; s += 64) Ltot = fmaf(wgt(s), sl[s], Ltot);
  Ltot = wave_sum(Ltot);

  // ---- merged rank-space sums, round by round of sr splits
  for (int r0 = 0; r0 < S; r0 += sr) {
    const int nr = min(sr, S - r0);
    if (r0 > 0) {
      __syncthreads();  // the previous round is summed
      load_o(r0, nr);
      __asm__ volatile("" ::: "memory");
      store_o(nr);
      __syncthreads();
    }
    for (int e = t; e < rows; e += kCT) {
      const int v = e / rv, c = e - v * rv;
      float a = r0 > 0 ? sov[e] : 0.f;
      if (V == 1) {
#pragma unroll 8
        for (int s = 0; s < nr; ++s) a = fmaf(wgt(r0 + s), so[s * rv + c], a);
      } else {
        for (int s = 0; s < nr; ++s) a = fmaf(sv[r0 + s] == v ? wgt(r0 + s) : 0.f, so[s * rv + c], a);
      }
      sov[e] = a;
    }
  }
  // ---- anchor sums of feature t, round by round of ar anchor splits
  float oa = 0.f;
  for (int r0 = 0; r0 < na; r0 += ar) {
    const int nr = min(ar, na - r0);
    if (r0 > 0) {
      __syncthreads();
      load_a(r0, nr);
      __asm__ volatile("" ::: "memory");
      store_a(nr);
      __syncthreads();
    }
    for (int s = 0; s < nr; ++s) {
      const float w = wgt(s_a0 + r0 + s);
      oa = w != 0.f ? fmaf(w, sa[s * kD + t], oa) : oa;
    }
  }
  __syncthreads();  // sov complete

  // ---- up-projection: column t of every U_V row against the merged sums
  float y = 0.f;
  for (int e0 = 0; e0 < rows; e0 += ur_rows) {
    const int nr = min(ur_rows, rows - e0);
    if (e0 > 0) {
      __syncthreads();
      load_u(e0, nr);
      __asm__ volatile("" ::: "memory");
      store_u(nr);
      __syncthreads();
    }
#pragma unroll 8
    for (int e = 0; e < nr; ++e) y = fmaf(to_f32(su[e * kD + t]), sov[e0 + e], y);
  }
  out[qi * kD + t] = (y + oa) / Ltot;
}

// ---------------------------------------------------------------------------
// Stage 2 in one round, for calls whose pieces of every kind fit one round of P
// per thread and whose heads have at most 128 splits: the same loads as above,
// then
//  - each wave finds M and L itself from the split headers it loaded (split s
//    in lane s % 64, register s / 64), with DPP row rotations and four
//    readlanes instead of LDS round trips, and each lane turns its split's max
//    into that split's weight 2^(m_s - M) once;
//  - every thread scales the rank-space pieces it loaded by their splits'
//    weights (fetched from the owning lanes) and adds them in registers, and
//    likewise the anchor pieces, so LDS receives partial sums, not records;
//  - after one barrier thread c < rv adds the partial sums of column c, thread
//    t the four anchor partials of feature t; after a second, thread t
//    up-projects;
//  - with several basis versions the weighted pieces go to LDS split by split
//    with each split's version, row e = (version v, column c) adds the splits of
//    version v in index order, and the up-projection runs over every version's
//    U_V rows.
// Every order is fixed, so a call is bitwise reproducible.
// ---------------------------------------------------------------------------
struct Combine1Lds {
  // byte offsets: partial sums ([s_step][rv]; with several versions every split's
  // weighted sums [S][rv]), anchor partials [4][128], split versions [S], o~ [V rv],
  // U rows [V rv][128]
  int red, anc, ver, ov, u, bytes;
};

template <typename T, int P, int PU>
__global__ __launch_bounds__(128) void k_combine1(LayerArgs L, DecodeArgs d, Combine1Lds g, float *out) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  constexpr int kEP = 16 / sizeof(T);          // U elements per 16-byte piece
  constexpr int kPPR = kD / kEP;               // pieces per U row
  extern __shared__ __align__(16) char lds[];
  int grp = L.group, hgs = L.hg;
  __asm__ volatile("" : "+s"(grp), "+s"(hgs)
                   : "s"(L.n_q), "s"(L.window), "s"(L.lowram), "s"(L.pred), "s"(L.bases), "s"(d.ws),
                     "s"(d.n_splits), "s"(d.rec), "s"(d.oa), "s"(d.ctx_lens), "s"(d.n_ctx), "s"(out), "s"(g.red),
                     "s"(g.anc), "s"(g.ver), "s"(g.ov), "s"(g.u), "s"(L.n_versions), "s"(L.version_elems));
  const int i = blockIdx.x, b = blockIdx.y, t = threadIdx.x, lane = t & 63;
  const int kvh = i / grp;                     // KV head; its latent group and slice
  const int h = kvh / hgs, j = kvh % hgs;
  const HeadInfo hd = L.heads[h];
  const int n_row = row_ctx(d, b);
  __asm__ volatile("" ::"s"(hd.rv), "s"(hd.u_v), "s"(hd.pred), "s"(d.nsplit[h]), "s"(n_row));
  const int rv = hd.rv;
  const int S = d.nsplit[h], V = L.n_versions;
  const int rows = V * rv;                     // U rows: (version, column) pairs
  float *sred = reinterpret_cast<float *>(lds + g.red);
  float *sanc = reinterpret_cast<float *>(lds + g.anc);
  int *sver = reinterpret_cast<int *>(lds + g.ver);
  float *sov = reinterpret_cast<float *>(lds + g.ov);
  T *su = reinterpret_cast<T *>(lds + g.u);
  const int64_t qi = int64_t(b) * L.n_q + i;
  const __amdgpu_buffer_rsrc_t rr =
      __builtin_amdgcn_make_buffer_rsrc(split_record(d, qi, 0), 0, S * d.rec * 4, kBufferWord3);
  auto rec4 = [&](int s, int f) {  // floats f .. f + 3 of split s's record
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rr, (s * d.rec + f) * 4, 0, 0));
  };
  const int a1 = min(n_row, 1 + L.window);     // anchor rows per KV head
  const int per = anchor_rows_per_split(a1 * L.hg, S);
  const int s_a0 = L.lowram ? 0 : (j * a1) / per;
  const int s_a1 = L.lowram ? S : min(S, ((j + 1) * a1 + per - 1) / per);
  const int na = s_a1 - s_a0;                  // >= 1
  const int urow = L.hg * kD;
  const T *ubase = L.lowram ? static_cast<const T *>(L.pred) + hd.pred + int64_t(b) * rv * kD
                            : static_cast<const T *>(L.bases) + hd.u_v;
  const int vstride = L.lowram ? 0 : int(L.version_elems);  // elements between versions' bases
  const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(ubase), 0, ((V - 1) * vstride + rv * urow) * int(sizeof(T)), kBufferWord3);
  // piece k of this thread: sums piece pc of split s_t + s_step k (threads past
  // npc s_step, when npc does not divide 128, take none); anchor piece ac of
  // anchor split a_t + 4 k; U piece uc of row u_t + (128 / kPPR) k
  const int npc = rv >> 2, pc = t % npc, s_t = t / npc, s_step = kCT / npc;
  const bool sact = s_t < s_step;
  const int ac = t & 31, a_t = t >> 5;
  const int uc = t % kPPR, u_t = t / kPPR;
  int a_f = d.oa + 4 * ac;
  __asm__ volatile("" : "+v"(a_f));

  // ---- one round of loads
  const f4 h0 = rec4(min(lane, S - 1), 0), h1 = rec4(min(lane + 64, S - 1), 0);
  f4 op[P], ap[P];
  u4 up[PU];
#pragma unroll
  for (int k = 0; k < P; ++k) op[k] = rec4(min(s_t + s_step * k, S - 1), 4 + 4 * pc);
#pragma unroll
  for (int k = 0; k < PU; ++k) {
    const int e = min(u_t + (kCT / kPPR) * k, rows - 1);  // U row (version e / rv, column e % rv)
    const int v = e / rv, cc = e - v * rv;
    up[k] = __builtin_amdgcn_raw_buffer_load_b128(ur, (v * vstride + cc * urow + j * kD + uc * kEP) * int(sizeof(T)),
                                                  0, 0);
  }
#pragma unroll
  for (int k = 0; k < P; ++k) ap[k] = rec4(s_a0 + min(a_t + 4 * k, na - 1), a_f);

  // ---- the common max, the denominator and each split's weight (per wave)
  const float m0 = lane < S ? h0.x : kNegInf, m1 = lane + 64 < S ? h1.x : kNegInf;
  const float M = wave_max_dpp(fmaxf(m0, m1));  // finite: token 0 is an anchor of every row
  const float w0 = m0 == kNegInf ? 0.f : fast_exp2(m0 - M);  // a split that saw nothing weighs 0
  const float w1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - M);
  const float Ltot = wave_sum_dpp(fmaf(w0, h0.y, w1 * h1.y));
  auto weight = [&](int s) {  // the weight of split s < 128, from the lane that holds it
    const float x = __shfl(w0, s & 63, 64), y = __shfl(w1, s & 63, 64);
    return s < 64 ? x : y;
  };

  // ---- partial sums into LDS: with one version each thread's splits added in
  // registers; with several, every split's weighted sums by split, and its version
  {
    if (V == 1) {
      f4 part = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < P; ++k) {
        const int s = s_t + s_step * k;
        const float w = weight(s);
        part += (sact && s < S ? w : 0.f) * op[k];
      }
      if (sact) *reinterpret_cast<f4 *>(&sred[s_t * rv + 4 * pc]) = part;
    } else {
#pragma unroll
      for (int k = 0; k < P; ++k) {
        const int s = s_t + s_step * k;
        const float w = weight(s);
        if (sact && s < S) *reinterpret_cast<f4 *>(&sred[s * rv + 4 * pc]) = w * op[k];
      }
      if (t < 64) {  // wave 0: lane s holds split s's header (and s + 64's)
        if (lane < S) sver[lane] = min(max(int(h0.z), 0), V - 1);
        if (lane + 64 < S) sver[lane + 64] = min(max(int(h1.z), 0), V - 1);
      }
    }
    f4 pa = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int r = a_t + 4 * k;
      const float w = weight(s_a0 + min(r, na - 1));
      pa += (r < na ? w : 0.f) * ap[k];
    }
    *reinterpret_cast<f4 *>(&sanc[a_t * kD + 4 * ac]) = pa;
#pragma unroll
    for (int k = 0; k < PU; ++k)
      *reinterpret_cast<u4 *>(&su[(min(u_t + (kCT / kPPR) * k, rows - 1) * kPPR + uc) * kEP]) = up[k];
  }
  __syncthreads();
  if (V == 1) {
    if (t < rv) {
      float a = 0.f;
      for (int r = 0; r < s_step; ++r) a += sred[r * rv + t];
      sov[t] = a;
    }
  } else {
    for (int e = t; e < rows; e += kCT) {  // row e: version e / rv, column e % rv, its splits in order
      const int v = e / rv, cc = e - v * rv;
      float a = 0.f;
      for (int s = 0; s < S; ++s) a += sver[s] == v ? sred[s * rv + cc] : 0.f;
      sov[e] = a;
    }
  }
  const float oa = (sanc[t] + sanc[kD + t]) + (sanc[2 * kD + t] + sanc[3 * kD + t]);
  __syncthreads();

  // ---- up-projection: column t of every U row against the merged sums
  float y = 0.f;
#pragma unroll 8
  for (int e = 0; e < rows; ++e) y = fmaf(to_f32(su[e * kD + t]), sov[e], y);
  out[qi * kD + t] = (y + oa) / Ltot;
}

// the combine geometry of a call: P from the largest piece count of any kind
// (rounded up to 2, 4, 8 or 16), round capacities, LDS layout
static CombineArgs combine_args(const LayerArgs &L, const DecodeArgs &d) {
  const int esize = L.dtype == LRKV_F32 ? 4 : 2;
  const int S = d.n_splits, rv = L.rv_max, V = L.n_versions;
  const int rows = V * rv;
  int na = S;  // anchor splits of one KV head (all splits for LowRAM layers)
  if (!L.lowram) {
    const int a1 = d.n_ctx < 1 + L.window ? d.n_ctx : 1 + L.window;
    na = 0;
    for (int h = 0; h < L.n_lat; ++h) {
      const int Sh = d.nsplit[h], per = anchor_rows_per_split(a1 * L.hg, Sh);
      for (int jj = 0; jj < L.hg; ++jj) {
        const int s0 = (jj * a1) / per, s1 = std::min(Sh, ((jj + 1) * a1 + per - 1) / per);
        na = std::max(na, s1 - s0);
      }
    }
    na = std::max(na, 1);
  }
  // a round covers P splits per thread row: kCT / (rv / 4) rows of threads take
  // pieces of the sums (when rv / 4 does not divide kCT the remaining threads
  // take none, so the capacity is P times the whole rows, not P kCT / (rv / 4))
  const int srow = kCT / (rv / 4);
  const int need = std::max({(S + srow - 1) / srow, (rows * (kD * esize / 16) + kCT - 1) / kCT,
                             (na * 32 + kCT - 1) / kCT});
  CombineArgs g{};
  g.P = need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
  g.na = na;
  g.so = g.P * srow;
  g.sa = g.P * kCT / 32;
  g.urows = g.P * kCT / (kD * esize / 16);
  const int so_n = std::min(S, g.so), sa_n = std::min(na, g.sa), u_n = std::min(rows, g.urows);
  g.m = 0;
  g.l = g.m + 4 * S;
  g.v = g.l + 4 * S;
  g.o = (g.v + 4 * S + 15) / 16 * 16;
  g.a = g.o + 4 * so_n * rv;
  g.ov = g.a + 4 * sa_n * kD;
  g.u = (g.ov + 4 * rows + 15) / 16 * 16;
  g.bytes = g.u + u_n * kD * esize;
  return g;
}

int generic_blocks_per_cu() { return kernel_blocks_per_cu(reinterpret_cast<const void *>(k_partials_generic<float>)); }

hipError_t launch_decode_partials(const LayerArgs &L, const DecodeArgs &d, hipStream_t s) {
  if (L.dtype != LRKV_F32) return launch_partials_mfma(L, d, s);
  hipLaunchKernelGGL(k_partials_generic<float>, dim3(d.row_items, L.batch), dim3(256), 0, s, L, d);
  return hipGetLastError();
}

template <typename T>
static void launch_combine_t(const LayerArgs &L, const DecodeArgs &d, const CombineArgs &g, float *out,
                             hipStream_t s) {
  dim3 grid(L.n_q, L.batch);
  switch (g.P) {
    case 2: hipLaunchKernelGGL((k_combine<T, 2>), grid, dim3(kCT), g.bytes, s, L, d, g, out); break;
    case 4: hipLaunchKernelGGL((k_combine<T, 4>), grid, dim3(kCT), g.bytes, s, L, d, g, out); break;
    case 8: hipLaunchKernelGGL((k_combine<T, 8>), grid, dim3(kCT), g.bytes, s, L, d, g, out); break;
    default: hipLaunchKernelGGL((k_combine<T, 16>), grid, dim3(kCT), g.bytes, s, L, d, g, out); break;
  }
}

static Combine1Lds combine1_lds(const LayerArgs &L, const DecodeArgs &d, int esize) {
  const int V = L.n_versions, rows = V * L.rv_max;
  Combine1Lds g{};
  g.red = 0;
  g.anc = g.red + 4 * (V == 1 ? 512 : d.n_splits * L.rv_max);
  g.ver = g.anc + 4 * 4 * kD;
  g.ov = g.ver + 4 * ((d.n_splits + 3) / 4 * 4);
  g.u = g.ov + 4 * ((rows + 3) / 4 * 4);
  g.bytes = g.u + rows * kD * esize;
  return g;
}

template <typename T, int P>
static void launch_combine1_pu(const LayerArgs &L, const DecodeArgs &d, const Combine1Lds &g, int PU, float *out,
                               hipStream_t s) {
  dim3 grid(L.n_q, L.batch);
  switch (PU) {
    case 2: hipLaunchKernelGGL((k_combine1<T, P, 2>), grid, dim3(kCT), g.bytes, s, L, d, g, out); break;
    case 4: hipLaunchKernelGGL((k_combine1<T, P, 4>), grid, dim3(kCT), g.bytes, s, L, d, g, out); break;
    case 8: hipLaunchKernelGGL((k_combine1<T, P, 8>), grid, dim3(kCT), g.bytes, s, L, d, g, out); break;
    default: hipLaunchKernelGGL((k_combine1<T, P, 16>), grid, dim3(kCT), g.bytes, s, L, d, g, out); break;
  }
}

// P: pieces of the split sums and anchor sums per thread, PU: of the U rows
template <typename T>
static void launch_combine1_t(const LayerArgs &L, const DecodeArgs &d, int P, int PU, float *out, hipStream_t s) {
  const Combine1Lds g = combine1_lds(L, d, int(sizeof(T)));
  switch (P) {
    case 2: launch_combine1_pu<T, 2>(L, d, g, PU, out, s); break;
    case 4: launch_combine1_pu<T, 4>(L, d, g, PU, out, s); break;
    case 8: launch_combine1_pu<T, 8>(L, d, g, PU, out, s); break;
    default: launch_combine1_pu<T, 16>(L, d, g, PU, out, s); break;
  }
}

hipError_t launch_decode_combine(const LayerArgs &L, const DecodeArgs &d, float *out, hipStream_t s) {
  const CombineArgs g = combine_args(L, d);
  // one round of loads holds every piece when the round capacities cover the
  // splits, the anchor splits and the U rows
  const bool one_round = g.so >= d.n_splits && g.sa >= g.na && g.urows >= L.n_versions * L.rv_max;
  // (and its LDS, with several versions a record slice per split, within 64 KB)
  const bool fits = combine1_lds(L, d, L.dtype == LRKV_F32 ? 4 : 2).bytes <= 65536;
  if (d.n_splits <= 128 && one_round && fits) {
    // separate piece counts for the sums and anchors and for the U rows (with
    // several versions the U rows alone may need many)
    const int esize = L.dtype == LRKV_F32 ? 4 : 2;
    const int srow = kCT / (L.rv_max / 4);
    const int need = std::max((d.n_splits + srow - 1) / srow, (g.na * 32 + kCT - 1) / kCT);
    const int need_u = (L.n_versions * L.rv_max * (kD * esize / 16) + kCT - 1) / kCT;
    auto round_p = [](int n) { return n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : 16; };
    if (L.dtype == LRKV_F32)
      launch_combine1_t<float>(L, d, round_p(need), round_p(need_u), out, s);
    else
      launch_combine1_t<bf16_t>(L, d, round_p(need), round_p(need_u), out, s);
    return hipGetLastError();
  }
  if (L.dtype == LRKV_F32)  // float32 layers have one version
    launch_combine_t<float>(L, d, g, out, s);
  else
    launch_combine_t<bf16_t>(L, d, g, out, s);
  return hipGetLastError();
}

}  // namespace lrkv
