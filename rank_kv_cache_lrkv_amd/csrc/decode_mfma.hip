// Stage 1 of decode attention for bfloat16 caches (and int8 or 4-bit codes with
// per-token scales, converted to bf16 on the way in) on the gfx950 matrix cores.
//
// One workgroup of four waves per (split, batch row, KV head).  For one 32-slot
// code block a wave computes
//
//   scores   S[t][h] = C_K[t] . q~_h   two 16-token tiles, K = 32 rank columns
//            per MFMA; q~ is split into a bf16 hi + lo pair (two MFMAs) so the
//            projected query keeps ~16 significant bits
//   softmax  block max per head across the wave, running max and denominator,
//            exp2 of scores already in log2 units
//   values   o~[h][c] += sum_t p[h][t] C_V[t][c]   16 columns per MFMA, K = the
//            32 tokens, the weights split into bf16 hi + lo (two MFMAs)
//
// The code layout (lrkv.h) puts the 16 bytes each lane feeds a matrix core next
// to each other, so a key block is read as one contiguous 1 KiB per 32 rank
// columns and a value block as four contiguous 256-byte runs per 16 columns.
// The score result lands, with no lane exchange, where the value MFMA takes its
// weights: lane (q, t) holds head t's weights of tokens 16 h + 4 q + v, which
// the value layout files as k-slot 4 h + v of lane group q.
//
// Memory schedule.  Split s, wave w streams blocks 4 s + w + k 4S, so all the
// waves of a (row, head) sweep its codes together as one moving front (DRAM rows
// stay open), and every wave keeps the next block in flight while it computes
// the current one (double buffering keeps the kernel at four waves per SIMD, so
// all workgroups of a 32-split, 32-unit decode are resident at once).  Loads are
// raw buffer loads: a per-lane constant offset plus a scalar block offset.  The first splits also take the anchor rows (token 0 and the
// recent window, full rank) in runs of at least 16; they are staged in LDS in the
// prologue together with the group's queries and the query projection
// q~ = U_K^T q, and wave 0 folds them in before its code blocks while the other
// waves already stream.

#include <map>
#include <mutex>

#include "decode_common.h"
#include "mfma_util.h"

namespace lrkv {

// LDS traffic of one wave is processed in order: a wave-scope fence orders it
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete
// (lgkmcnt 0; vmcnt and expcnt left at their maxima, i.e. not waited for), then
// all waves meet.  Global loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

constexpr int kAnchorChunk = kMinAnchorRows;  // anchor rows staged in LDS at a time

template <int RKMAX, int RVMAX, bool RP = false>
struct MfmaSmem {
  union {
    float qt[LRKV_MAX_GROUP][RKMAX];  // prologue: projected queries (log2 units)
    float oa[LRKV_MAX_GROUP][kD];     // epilogue: anchor value sums
  } u;
  u32x4 bq[(RKMAX + 31) / 32][2][64];       // score B operands of each lane (hi, lo)
  uint32_t ak[kAnchorChunk][kD / 2];        // anchor rows (bf16 pairs)
  uint32_t av[kAnchorChunk][kD / 2];
  uint32_t sq[LRKV_MAX_GROUP][kD / 2];      // the group's queries (bf16 pairs), zero rows past G
  float qs[LRKV_MAX_GROUP];                 // quantised codes: scale of a head's int8 q~ parts
  float m[5][LRKV_MAX_GROUP];               // per wave; [4] = the anchors
  float l[5][LRKV_MAX_GROUP];
  union {
    float o[4][LRKV_MAX_GROUP][RVMAX];      // epilogue: per-wave rank-space sums
    struct {                                // pre-RoPE codes, during the block loop:
      bf16_t su[RP ? kD * (RKMAX + 8) : 1]; //   U_K feature-major (rows of RKMAX + 8)
      u32x4 rq[RP ? 4 : 1][2][64];          //   score B operands (q permuted, hi / lo)
    } r;
  } w;
};

// CB: bits per code element (16 bf16, 8 int8, 4 four-bit)
template <int NKC, int NVC, int CB>
struct BlockRegs {
  u32x4 k[2][NKC];
  u32x4 v[NVC];
  uint32_t e[LRKV_MAX_RESID];  // LowRAM: features 2 lane, 2 lane + 1 of the block's residual rows
  uint32_t es;                 // LowRAM: lane i < R holds the in-block slot of entry i
};
// int8 codes: 8 bytes per lane and operand, and one key and one value scale per
// lane: lane (q4, t16) of the 16-lane row q4 holds those of token
// 16 ((t16 >> 2) & 1) + 4 q4 + (t16 & 3), so lanes 0 .. 7 of the row hold the
// row's 8 tokens 16 h2 + 4 q4 + v in the order 4 h2 + v
template <int NKC, int NVC>
struct BlockRegs<NKC, NVC, 8> {
  u32x2 k[2][NKC];
  u32x2 v[NVC];
  uint32_t sk, sv;
};
// 4-bit codes: 4 bytes per lane and operand, scales as for int8
template <int NKC, int NVC>
struct BlockRegs<NKC, NVC, 4> {
  uint32_t k[2][NKC];
  uint32_t v[NVC];
  uint32_t sk, sv;
};

// lane N of this lane's 16-lane row (DPP row_newbcast)
template <int N>
__device__ __forceinline__ float row_lane(uint32_t x) {
  return __uint_as_float(uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x150 + N, 0xf, 0xf, false)));
}
// the 8 scales of the row's tokens, in the order 4 h2 + v
__device__ __forceinline__ void row_scales(uint32_t x, float (&o)[8]) {
  o[0] = row_lane<0>(x);
  o[1] = row_lane<1>(x);
  o[2] = row_lane<2>(x);
  o[3] = row_lane<3>(x);
  o[4] = row_lane<4>(x);
  o[5] = row_lane<5>(x);
  o[6] = row_lane<6>(x);
  o[7] = row_lane<7>(x);
}

// 8 int8 values (low byte first) as the 8 bf16 values of an MFMA operand: exact,
// every integer of [-128, 127] has a bfloat16 representation
__device__ __forceinline__ u32x4 i8x8_to_bf16(u32x2 w) {
  auto pair = [](float a, float b) {  // the high halves of two float32 values
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
  };
  u32x4 r;
  r[0] = pair(float(int8_t(w[0])), float(int8_t(w[0] >> 8)));
  r[1] = pair(float(int8_t(w[0] >> 16)), float(int32_t(w[0]) >> 24));
  r[2] = pair(float(int8_t(w[1])), float(int8_t(w[1] >> 8)));
  r[3] = pair(float(int8_t(w[1] >> 16)), float(int32_t(w[1]) >> 24));
  return r;
}

// 8 four-bit values (lowest nibble first) as 8 bf16 values of 16 times their
// value: each nibble is moved to the top of a byte and converted with the
// sign-extending byte select (the factor 16 is taken out of the scales)
__device__ __forceinline__ u32x4 i4x8_to_bf16_x16(uint32_t w) {
  auto pair = [](float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
  };
  const uint32_t ev = (w << 4) & 0xf0f0f0f0u;  // elements 0, 2, 4, 6
  const uint32_t od = w & 0xf0f0f0f0u;         // elements 1, 3, 5, 7
  u32x4 r;
  r[0] = pair(float(int8_t(ev)), float(int8_t(od)));
  r[1] = pair(float(int8_t(ev >> 8)), float(int8_t(od >> 8)));
  r[2] = pair(float(int8_t(ev >> 16)), float(int8_t(od >> 16)));
  r[3] = pair(float(int32_t(ev) >> 24), float(int32_t(od) >> 24));
  return r;
}

// EXACT: every head of the layer has rank_k == RKMAX and rank_v == RVMAX, so all
// rank tests fold at compile time; otherwise ranks are read per head (<= the max).
// CB = 8 or 4: quantised codes with a float32 scale per token (keys and values):
// key codes are scored on the int8 matrix cores as loaded (4-bit codes as 16
// times their value, the 16 taken out of q~), against q~ held as two int8 parts
// per head; value codes enter the bf16 MFMAs converted exactly (4-bit: 16 times
// their value, the 16 taken out of the value sums).  A score is the product
// times the key scale, and a token's weight is multiplied by its value scale
// before it becomes the value MFMA's A operand (the denominator keeps the plain
// weight).
//
// LR: LowRAM value amortisation (bf16 codes, RVMAX == RKMAX).  No value codes are
// read: the value operand of a block is its key codes transposed (8 tokens of one
// column per lane), made on the matrix cores as the product with a 0/1 selector,
// which lands the codes exactly in the layout the value MFMA takes; the rank-space
// sum over the key codes is up-projected by the combine with the row's predictor
// M.  The block's kept residual rows (R entries: slot, 128 bf16) are loaded with
// the block and added as p[t][h] e_t into 128-dim sums per head (each lane two
// features), which leave the split with the anchor sums.
// LR > 0 is the most query heads per KV head the instance handles (4 or 16), LRR
// the most residual entries per block (4 or 8): both size register arrays.
//
// RP: keys compressed before RoPE (Palu's on-the-fly reconstruction; bf16 codes).
// Codes cannot be scored in code space: per block the wave reconstructs its 32
// keys on the matrix cores, D[f][t] = sum_c U_K[f][c] C[t][c] (A = U_K staged in
// LDS feature by feature, B = the key fragments as loaded), which leaves lane
// (q4, t16) features 16 ft + 4 q4 + v of token 16 h2 + t16 -- so the pair
// (f, f + 64) of a rotation sits in the same lane (tiles ft and ft + 4).  Each
// pair is turned by its position's angle (hardware sin/cos of the angle in
// revolutions).  A lane keeps the angles of its 16 pairs at its first token,
// reduced exactly from the position on the wave's first block and every 16th
// after, and in between advanced by the angle of the wave's block stride (one
// add and a fraction, error a few units of 2^-24 revolutions); its second
// token, 16 positions on, is turned by the angle-addition formula from the
// first one's sin and cos.  The rotated keys, split into bf16 hi + lo,
// are scored against q whose features are permuted to the order the lanes hold
// (k = 8 q4 + i <-> feature 32 kc + 16 (i / 4) + 4 q4 + i % 4).
template <int RKMAX, int RVMAX, bool EXACT, int CB, int LR = 0, int LRR = 0, bool RP = false>
__device__ __forceinline__ void partials_body(const LayerArgs &L, const DecodeArgs &d, MfmaSmem<RKMAX, RVMAX, RP> &sm) {
  constexpr int NKC = (RKMAX + 31) / 32;  // score MFMAs per 16-token tile (K = 32 each)
  constexpr int NVC = RVMAX / 16;         // value MFMAs per block (16 columns each)
  constexpr bool QC = CB < 16;            // quantised codes with per-token scales
  constexpr float kX16 = CB == 4 ? 0.0625f : 1.f;  // undoes the x16 of 4-bit operands
  constexpr int RS = RKMAX + 8;           // RP: LDS row of U_K (one feature, RKMAX + 8 bf16)
  static_assert(LR == 0 || LRKV_MAX_GROUP * RVMAX >= kBlock * 16, "a wave's epilogue slice holds a block's weights");
  __shared__ float sra[RP ? kD / 2 : 1][2];      // RP: angle per position of each pair (revolutions)
  __shared__ float srd[RP ? kD / 2 : 1][3];      // RP: the angle over a wave's block stride; cos, sin over 16 positions
  bf16_t *const su = sm.w.r.su;
  auto &rq = sm.w.r.rq;

  // Setup reads.  Every kernel-argument scalar the setup needs is taken at once
  // (the empty asm takes them all as operands, so their scalar loads issue
  // together and are waited for once); otherwise each branch on a loaded value
  // would wait for its own round trip, a dozen of them before the first load.
  __asm__ volatile("" ::"s"(d.row_items), "s"(d.items), "s"(d.uniform), "s"(d.n_splits), "s"(d.balance),
                   "s"(d.ctx_lens), "s"(d.n_ctx), "s"(d.q), "s"(L.n_lat), "s"(L.window), "s"(L.hg), "s"(L.group),
                   "s"(L.n_versions), "s"(L.cap), "s"(L.n_kv), "s"(L.n_q), "s"(L.codes_k), "s"(L.codes_v),
                   "s"(L.anchor_k), "s"(L.anchor_v), "s"(L.bases));
  // (batch row b, latent group h) and split `split` of the group's S; the G
  // query heads are those of the hg KV heads h hg .. h hg + hg - 1 (GK each),
  // which share the group's codes
  const WorkItem wi = work_item(L, d);
  const int S = wi.S, split = wi.split;
  const int b = wi.b, h = wi.h;
  const int GK = L.group, G = GK * L.hg;
  const int W = L.window;
  const HeadInfo hd = L.heads[h];
  // the group's row of the head table and the row's length: the second (and
  // last) round of setup reads
  const int n = row_ctx(d, b);
  __asm__ volatile("" ::"s"(hd.rk), "s"(hd.rv), "s"(hd.u_k), "s"(hd.ck), "s"(hd.cv), "s"(wi.S), "s"(n));
  const int rk = EXACT ? RKMAX : hd.rk, rv = EXACT ? RVMAX : hd.rv;
  const int nkg = rk >> 3;   // 8-column groups of a key code
  const int nvt = rv >> 4;   // 16-column tiles of a value code
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const int c = max(0, n - 1 - W);
  const int nblk = (c + kBlock - 1) / kBlock;
  // the unit's anchor rows: a1 per KV head, KV head after KV head
  const int a1 = min(n, 1 + W);
  int alo, ahi;
  anchor_share(a1 * L.hg, split, S, alo, ahi);
  const int na = ahi - alo;
  auto anchor_row = [&](int rho) {  // element row of anchor row rho of the unit
    return (int64_t(b) * L.n_kv + h * L.hg + rho / a1) * (1 + W) + rho % a1;
  };
  const int64_t q0 = int64_t(b) * L.n_q + h * G;
  // with basis versions the split sweeps its version's blocks [sg.lo, sg.hi)
  const SplitSeg sg = split_segment(L, b, split, S, nblk);
  const int bhi = sg.hi;
  const int first = sg.lo + 4 * sg.s + wave, step = 4 * sg.ns;
  // When every workgroup is resident at once, the older workgroups on a compute unit
  // get their loads served first and the youngest would stream alone at the end;
  // the waves with the larger share of their blocks still to read get the higher
  // issue priority instead, so all of them finish together.
  // The priority of a request for block blk is floor(4 left / (total + 1)) with
  // left = ceil((bhi - blk) / step) this wave's blocks from blk on: it is at least
  // k exactly when left >= ceil(k (total + 1) / 4), i.e. when blk < bk[k] -- three
  // thresholds taken once, so a request costs scalar compares, no division.
  const int total = first < bhi ? (bhi - first + step - 1) / step : 0;  // this wave's blocks
  auto threshold = [&](int k) { return bhi - ((k * (total + 1) + 3) / 4 - 1) * step; };
  const int bk1 = __builtin_amdgcn_readfirstlane(threshold(1));
  const int bk2 = __builtin_amdgcn_readfirstlane(threshold(2));
  const int bk3 = __builtin_amdgcn_readfirstlane(threshold(3));
  auto set_priority = [&](int blk) {
    if (!d.balance) return;
    blk = __builtin_amdgcn_readfirstlane(blk);
    if (blk < bk3) __builtin_amdgcn_s_setprio(3);
    else if (blk < bk2) __builtin_amdgcn_s_setprio(2);
    else if (blk < bk1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  };
  if (d.balance) __builtin_amdgcn_s_setprio(3);

  if (4 * sg.s >= bhi - sg.lo && na == 0) {  // nothing for this split
    for (int i = tid; i < G; i += blockDim.x) {
      float *rec = split_record(d, q0 + i, split);
      rec[0] = kNegInf;
      rec[1] = rec[3] = 0.f;
      rec[2] = float(sg.v);
    }
    for (int i = tid; i < G * rv; i += blockDim.x) split_record(d, q0 + i / rv, split)[4 + i % rv] = 0.f;
    return;
  }

  // this (row, head)'s key and value code regions (and int8 scales) as buffer
  // resources; byte offsets are element offsets * CB / 8 (regions start on even
  // elements).  The extents are cap times the bytes of one code row (r * CB / 8,
  // an integer for ranks that are multiples of 16), which the host bounds below
  // 2^31; forming cap * r * CB first could overflow 32 bits.
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<char *>(L.codes_k) + (hd.ck + int64_t(b) * L.cap * rk) * CB / 8, 0, L.cap * (rk * CB / 8),
      kBufferWord3);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<char *>(L.codes_v) + (hd.cv + int64_t(b) * L.cap * rv) * CB / 8, 0, L.cap * (rv * CB / 8),
      kBufferWord3);
  __amdgpu_buffer_rsrc_t skres = kres, svres = vres;
  if constexpr (QC) {
    skres = __builtin_amdgcn_make_buffer_rsrc(L.scales_k + scale_index(L, h, b, 0), 0, L.cap * 4, kBufferWord3);
    svres = __builtin_amdgcn_make_buffer_rsrc(L.scales_v + scale_index(L, h, b, 0), 0, L.cap * 4, kBufferWord3);
  }
  const int soff = (16 * ((t16 >> 2) & 1) + 4 * q4 + (t16 & 3)) * 4;  // this lane's scale in a block
  // LowRAM: this (row, head)'s residual entries, R per block
  __amdgpu_buffer_rsrc_t eres = kres, esres = kres;
  if constexpr (LR > 0) {
    const int64_t e0 = resid_entry(L, h, b, 0, 0);
    eres = __builtin_amdgcn_make_buffer_rsrc(static_cast<bf16_t *>(L.resid) + e0 * kD, 0,
                                             (L.cap / kBlock) * L.R * kD * 2, kBufferWord3);
    esres = __builtin_amdgcn_make_buffer_rsrc(L.rslot + e0, 0, (L.cap / kBlock) * L.R * 4, kBufferWord3);
  }
  // the same regions with no extent: a request with nothing left to fetch (the
  // prefetch after a wave's last block, the first block of a wave without any)
  // goes to these, so it stays an unconditional load yet the buffer unit returns
  // zeros without touching memory
  const __amdgpu_buffer_rsrc_t kres0 = __builtin_amdgcn_make_buffer_rsrc(L.codes_k, 0, 0, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vres0 = __builtin_amdgcn_make_buffer_rsrc(L.codes_v, 0, 0, kBufferWord3);
  const int kblk_bytes = kBlock * rk * CB / 8, vblk_bytes = kBlock * rv * CB / 8;
  // Code blocks (and their scales and residual rows) are read exactly once per
  // call: their loads carry the streaming (non-temporal) cache policy, which
  // keeps them from displacing the query, U_K and anchor lines the splits of a
  // unit share in L2, and measurably raises the read rate on this part.
  constexpr int kStream = 2;
  // column groups past the head's rank (instances wider than the head) read from
  // an offset past the region's extent: the buffer unit returns zeros for them
  // without touching memory
  constexpr int kAbsent = 0x40000000;
  int koff[2][NKC];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int kg = 4 * kc + q4;
      koff[h2][kc] = kg < nkg ? ((h2 * nkg + kg) * 16 + t16) * CB : kAbsent;
    }
  int voff[NVC];
#pragma unroll
  for (int ni = 0; ni < NVC; ++ni) voff[ni] = ni < nvt ? (q4 * rv + 16 * ni + t16) * CB : kAbsent;

  auto load = [&](int blk, bool live, BlockRegs<NKC, NVC, CB> &r) {
    set_priority(blk);
    const __amdgpu_buffer_rsrc_t kr = live ? kres : kres0, vr = live ? vres : vres0;
    const __amdgpu_buffer_rsrc_t skr = live ? skres : kres0, svr = live ? svres : kres0;
    const __amdgpu_buffer_rsrc_t er = live ? eres : kres0, esr = live ? esres : kres0;
    // the block offsets are wave-uniform: keep them in scalar registers
    const int ks = __builtin_amdgcn_readfirstlane(blk * kblk_bytes);
    const int vs = __builtin_amdgcn_readfirstlane(blk * vblk_bytes);
    if constexpr (QC) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          if constexpr (CB == 8) r.k[h2][kc] = __builtin_amdgcn_raw_buffer_load_b64(kr, koff[h2][kc], ks, kStream);
          else r.k[h2][kc] = __builtin_amdgcn_raw_buffer_load_b32(kr, koff[h2][kc], ks, kStream);
        }
#pragma unroll
      for (int ni = 0; ni < NVC; ++ni) {
        if constexpr (CB == 8) r.v[ni] = __builtin_amdgcn_raw_buffer_load_b64(vr, voff[ni], vs, kStream);
        else r.v[ni] = __builtin_amdgcn_raw_buffer_load_b32(vr, voff[ni], vs, kStream);
      }
      const int ss = __builtin_amdgcn_readfirstlane(blk * kBlock * 4);
      r.sk = __builtin_amdgcn_raw_buffer_load_b32(skr, soff, ss, kStream);
      r.sv = __builtin_amdgcn_raw_buffer_load_b32(svr, soff, ss, kStream);
    } else {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
          r.k[h2][kc] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[h2][kc], ks, kStream);
      if constexpr (LR == 0) {
#pragma unroll
        for (int ni = 0; ni < NVC; ++ni) r.v[ni] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[ni], vs, kStream);
      }
    }
    if constexpr (LR > 0) {
      const int es = __builtin_amdgcn_readfirstlane(blk * L.R * kD * 2);
#pragma unroll
      for (int i = 0; i < LRR; ++i)
        if (i < L.R) r.e[i] = __builtin_amdgcn_raw_buffer_load_b32(er, lane * 4 + i * kD * 2, es, kStream);
      r.es = __builtin_amdgcn_raw_buffer_load_b32(esr, min(lane, L.R - 1) * 4,
                                                  __builtin_amdgcn_readfirstlane(blk * L.R * 4), kStream);
    }
  };

  // ---- prologue.  Loads are issued in this order: the operands of q~ (q and
  // this wave's share of the U_K^T rows), the queries and first anchor rows for
  // LDS, and only then the wave's first code block.  Vector-memory loads
  // complete in order, so waiting for the prologue operands never waits for the
  // code blocks, and the barriers below wait for LDS traffic only.
  const bf16_t *qb = static_cast<const bf16_t *>(d.q) + q0 * kD;
  const bf16_t *ut = static_cast<const bf16_t *>(L.bases) + sg.v * L.version_elems + hd.u_k;
  constexpr int NT = RKMAX / 16;
  constexpr int NTW = (NT + 3) / 4;  // column tiles of q~ per wave
  // every load below is unconditional, from a clamped in-bounds address; what is
  // absent is zeroed afterwards (no divergent branches around the loads)
  const int urow = L.hg * kD;        // elements per U^T row (one 128-slice per KV head of the group)
  u32x4 bu[NTW][4];                  // B = rows of U_K^T, the slice of the group's first KV head
  auto load_bu = [&](int j) {
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int nt = min(wave + 4 * i, rk / 16 - 1);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        bu[i][kc] = *reinterpret_cast<const u32x4 *>(ut + (16 * nt + t16) * urow + j * kD + 32 * kc + 8 * q4);
    }
  };
  // pre-RoPE codes: U_K^T rows in 16-byte pieces (row c, features 8 p .. 8 p + 7),
  // all requested now and written to LDS feature-major below
  constexpr int NUP = RP ? (RKMAX * 16 + 255) / 256 : 1;
  u32x4 upc[NUP];
  if constexpr (RP) {
#pragma unroll
    for (int i = 0; i < NUP; ++i) {
      const int pc = min(tid + 256 * i, rk * 16 - 1);
      upc[i] = *reinterpret_cast<const u32x4 *>(ut + (pc >> 4) * kD + (pc & 15) * 8);
    }
  } else {
    load_bu(0);
  }
  const int r16 = tid >> 4, piece = tid & 15;  // 16 rows x 16 pieces of 16 bytes
  u32x4 qq = *reinterpret_cast<const u32x4 *>(qb + min(r16, G - 1) * kD + piece * 8);
  const int64_t arow = na > 0 ? anchor_row(alo + min(r16, na - 1)) : anchor_row(0);
  u32x4 kk = *reinterpret_cast<const u32x4 *>(static_cast<const bf16_t *>(L.anchor_k) + arow * kD + piece * 8);
  u32x4 vv = *reinterpret_cast<const u32x4 *>(static_cast<const bf16_t *>(L.anchor_v) + arow * kD + piece * 8);
  __builtin_amdgcn_sched_barrier(0);
  // the wave's first block (a wave with no blocks at all requests nothing)
  BlockRegs<NKC, NVC, CB> r0, r1;
  {
    const int last = max(nblk - 1, 0);
    load(min(first, last), first < bhi, r0);
  }
  __builtin_amdgcn_sched_barrier(0);

  const u32x4 zero4 = u32x4{0u, 0u, 0u, 0u};
  if (r16 >= G) qq = zero4;
  if (r16 >= min(na, kAnchorChunk)) kk = vv = zero4;
  *reinterpret_cast<u32x4 *>(&sm.sq[r16][piece * 4]) = qq;
  *reinterpret_cast<u32x4 *>(&sm.ak[r16][piece * 4]) = kk;
  *reinterpret_cast<u32x4 *>(&sm.av[r16][piece * 4]) = vv;
  lds_barrier();
  if constexpr (RP) {
    // U_K feature-major (columns past rk zero), the pair angles, and q's score
    // operands in the permuted feature order, hi and lo parts (zero past G)
#pragma unroll
    for (int i = 0; i < NUP; ++i) {
      const int pc = tid + 256 * i;
      if (pc < rk * 16) {
        const int c = pc >> 4, f0 = (pc & 15) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          su[(f0 + 2 * e) * RS + c] = bf16_t(upc[i][e] & 0xffffu);
          su[(f0 + 2 * e + 1) * RS + c] = bf16_t(upc[i][e] >> 16);
        }
      }
    }
    for (int e = tid; e < kD * (RS - rk); e += blockDim.x)  // columns past rk: zero
      su[(e % kD) * RS + rk + e / kD] = bf16_t(0);
    if (tid < kD / 2) {
      const float ahi = L.rope_a[tid][0], alo = L.rope_a[tid][1];
      sra[tid][0] = ahi;
      sra[tid][1] = alo;
      srd[tid][0] = rope_rev(ahi, alo, float(kBlock * step));  // exact: kBlock * step < 2^24
      const float r16 = rope_rev(ahi, alo, 16.f);
      srd[tid][1] = __builtin_amdgcn_cosf(r16);
      srd[tid][2] = __builtin_amdgcn_sinf(r16);
    }
    if (wave == 0) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int f = 32 * kc + 16 * (i >> 2) + 4 * q4 + (i & 3);
          const uint32_t wd = sm.sq[t16][f >> 1];
          const float qv = __uint_as_float((f & 1) ? (wd & 0xffff0000u) : (wd << 16));
          x[i] = t16 < G ? qv * d.scale_log2 : 0.f;
        }
        u32x4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = pack_hi(x[2 * i], x[2 * i + 1]);
          lo[i] = pack_rne(x[2 * i] - bf16_trunc(x[2 * i]), x[2 * i + 1] - bf16_trunc(x[2 * i + 1]));
        }
        rq[kc][0][lane] = hi;
        rq[kc][1][lane] = lo;
      }
    }
    lds_barrier();
  } else {
  // A = q from LDS: lane (q4, t16) holds head t16, features 32 kc + 8 q4 .. (zero past G)
  u32x4 aq[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) aq[kc] = *reinterpret_cast<const u32x4 *>(&sm.sq[t16][16 * kc + 4 * q4]);
  // D[head][col] = sum_k q[head][k] U_K[k][col], with U_K the slice of the head's
  // own KV head: one pass per KV head of the group, the other heads' q zeroed;
  // the waves share the column tiles
  f32x4 qacc[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) qacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < L.hg; ++j) {
    if (j > 0) load_bu(j);
    u32x4 aj[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) aj[kc] = t16 / GK == j ? aq[kc] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qacc[i] = mfma16x16x32(aj[kc], bu[i][kc], qacc[i]);
  }
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int nt = wave + 4 * i;
    if (nt < rk / 16) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int head = 4 * q4 + v;
        if (head < G) sm.u.qt[head][16 * nt + t16] = qacc[i][v] * (d.scale_log2 * kX16);
      }
    }
  }
  lds_barrier();
  // score B operands: lane (q4, t16) holds head t16's columns 8 (4 kc + q4) .. +7
  // as bf16 hi and lo parts, zero for absent heads/columns.
  // Quantised codes are scored on the int8 matrix cores instead: q~ of head h is
  // held as S (a + b / 254) with int8 a, b (|a|, |b| <= 127) and S = max |q~| / 127
  // over the head's columns (an error below S / 508 per element); the B operand of
  // MFMA pair pp has, in k-slot i of lane (q4, t16), the column that the A
  // operand's slot i holds: chunk kc = 2 pp + i / 8, group 4 kc + q4, element j =
  // i % 8 of it (4-bit codes: the even elements of the group in slots 0 .. 3, the
  // odd ones in 4 .. 7, as the nibble split below lays them out).
  if (wave == 0 && QC) {
    constexpr int NP = (NKC + 1) / 2;
    auto col_of = [&](int pp, int i) {  // column of k-slot i of pair pp, -1 if absent
      const int kc = 2 * pp + (i >> 3), kg = 4 * kc + q4, j = i & 7;
      const int e = CB == 4 ? (j < 4 ? 2 * j : 2 * (j - 4) + 1) : j;
      return (kc < NKC && kg < nkg) ? kg * 8 + e : -1;
    };
    auto qval = [&](int pp, int i) {
      const int cidx = col_of(pp, i);
      return (t16 < G && cidx >= 0) ? sm.u.qt[t16][cidx] : 0.f;
    };
    float mx = 0.f;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(qval(pp, i)));
    mx = rows_max(mx);  // over the four rows: every column of the head
    const float S = mx / 127.f;  // 0 for an absent head
    const float inv = S > 0.f ? 1.f / S : 0.f, inv2 = S > 0.f ? 254.f / S : 0.f;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      u32x4 bh, bl;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        uint32_t hw = 0u, lw = 0u;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const float x = qval(pp, 4 * w4 + bb);
          const float hf = fminf(fmaxf(__builtin_rintf(x * inv), -127.f), 127.f);
          const float lf = fminf(fmaxf(__builtin_rintf((x - S * hf) * inv2), -127.f), 127.f);
          hw |= (uint32_t(int(hf)) & 0xffu) << (8 * bb);
          lw |= (uint32_t(int(lf)) & 0xffu) << (8 * bb);
        }
        bh[w4] = hw;
        bl[w4] = lw;
      }
      sm.bq[pp][0][lane] = bh;
      sm.bq[pp][1][lane] = bl;
    }
    if (q4 == 0) sm.qs[t16] = S / 254.f;
  } else if (wave == 0) {
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int kg = 4 * kc + q4;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (t16 < G && kg < nkg) ? sm.u.qt[t16][kg * 8 + i] : 0.f;
      u32x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = pack_hi(x[2 * i], x[2 * i + 1]);
        lo[i] = pack_rne(x[2 * i] - bf16_trunc(x[2 * i]), x[2 * i + 1] - bf16_trunc(x[2 * i + 1]));
      }
      sm.bq[kc][0][lane] = hi;
      sm.bq[kc][1][lane] = lo;
    }
  }
  lds_barrier();
  }
  // quantised codes: this lane's head's scale of its int8 q~ parts
  float qsc = 0.f;
  if constexpr (QC) qsc = sm.qs[t16];

  // ---- the split's anchor rows (wave 0, before its code blocks, while the other
  // waves already stream): scores on the matrix cores against q; the 128-dim
  // value sums are accumulated in LDS (slot 4 of the merge), one head at a time,
  // every lane taking features 2 lane and 2 lane + 1.  Head hh's weight of row r
  // sits in lane 16 (r / 4) + hh, register r % 4, and its rescale factor in lane
  // hh: both are read as scalars.
  if (wave == 0) {
    float mA = kNegInf, lA = 0.f;
    for (int r0 = 0; r0 < na; r0 += kAnchorChunk) {
      const int nr = min(kAnchorChunk, na - r0);
      if (r0 > 0) {  // rows past the first chunk: stage them now
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int idx = lane + 64 * i, r = idx >> 4, piece = idx & 15;
          const int64_t row = anchor_row(alo + r0 + min(r, nr - 1));
          const u32x4 kk = *reinterpret_cast<const u32x4 *>(static_cast<const bf16_t *>(L.anchor_k) + row * kD + piece * 8);
          const u32x4 vv = *reinterpret_cast<const u32x4 *>(static_cast<const bf16_t *>(L.anchor_v) + row * kD + piece * 8);
          *reinterpret_cast<u32x4 *>(&sm.ak[r][piece * 4]) = kk;
          *reinterpret_cast<u32x4 *>(&sm.av[r][piece * 4]) = vv;
        }
        wave_lds_fence();
      }
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        s = mfma16x16x32(*reinterpret_cast<const u32x4 *>(&sm.ak[t16][16 * kc + 4 * q4]),
                         *reinterpret_cast<const u32x4 *>(&sm.sq[t16][16 * kc + 4 * q4]), s);
      // row 4 q4 + v (of KV head (alo + r0 + row) / a1) scores only that KV head's query heads
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * q4 + v;
        s[v] = row < nr && (alo + r0 + row) / a1 == t16 / GK ? s[v] * d.scale_log2 : kNegInf;
      }
      float cm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      cm = rows_max(cm);
      // a head may have no row in this chunk (rows of another KV head, or an absent head)
      const float mn = fmaxf(mA, cm);
      const bool none = mn == kNegInf;
      const float al = none ? 1.f : fast_exp2(mA - mn);
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v] = none ? 0.f : fast_exp2(s[v] - mn);
      float ps = (p[0] + p[1]) + (p[2] + p[3]);
      ps = rows_sum(ps);
      lA = lA * al + ps;
      mA = mn;
      uint32_t vrow[kAnchorChunk];
#pragma unroll
      for (int r = 0; r < kAnchorChunk; ++r) vrow[r] = sm.av[r][lane];
      for (int hh = 0; hh < G; ++hh) {
        float a0 = 0.f, a1 = 0.f;
        if (r0 > 0) {
          const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, al), hh));
          a0 = sm.u.oa[hh][2 * lane] * a;
          a1 = sm.u.oa[hh][2 * lane + 1] * a;
        }
#pragma unroll
        for (int r = 0; r < kAnchorChunk; ++r) {
          if (r < nr) {
            const float pw = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[r & 3]), 16 * (r >> 2) + hh));
            a0 = fmaf(pw, __uint_as_float(vrow[r] << 16), a0);
            a1 = fmaf(pw, __uint_as_float(vrow[r] & 0xffff0000u), a1);
          }
        }
        sm.u.oa[hh][2 * lane] = a0;
        sm.u.oa[hh][2 * lane + 1] = a1;
      }
      wave_lds_fence();
    }
    if (q4 == 0 && t16 < G) {
      sm.m[4][t16] = mA;
      sm.l[4][t16] = lA;
    }
  }

  // ---- the code blocks
  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[NVC];
#pragma unroll
  for (int ni = 0; ni < NVC; ++ni) o[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  // LowRAM: residual sums (lane: features 2 lane, 2 lane + 1 of every head), and the
  // selectors B[k][n] = (k == 16 half + n) that pick 16 of a fragment's 32 columns
  float res[LR > 0 ? LR : 1][2];
  if constexpr (LR > 0) {
#pragma unroll
    for (int hh = 0; hh < LR; ++hh) res[hh][0] = res[hh][1] = 0.f;
  }
  auto selector = [&](int half) {
    const int idx = 16 * half + t16 - 8 * q4;  // the element of this lane's 8 that is 1, if any
    u32x4 sv;
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (idx == 2 * i ? 0x3f80u : 0u) | (idx == 2 * i + 1 ? 0x3f800000u : 0u);
    return sv;
  };

  // RP: the lane's pair angles (revolutions) at its first token of the block being
  // processed, and the blocks left before they are reduced from the position again
  // (ranks up to 64 + 32 only: wider ones have no registers to spare for them and
  // reduce every angle from its position)
  constexpr bool kLean = RKMAX + RVMAX <= 96;
  constexpr int kReseed = 16;
  float rang[RP && kLean ? 4 : 1][4];
  int rseed = 0;
  auto process = [&](int blk, BlockRegs<NKC, NVC, CB> &r) {
    if constexpr (LR > 0) {  // slots past c may hold any bits: their codes become 0 (the
                         // transposes below mix a token's columns; scores are masked anyway)
      if (blk * kBlock + kBlock > c) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          if (blk * kBlock + 16 * h2 + t16 >= c)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) r.k[h2][kc] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    f32x4 s[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) s[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (RP && kLean) {
      // angles of the lane's pairs at its first token, position blk * 32 + t16 + 1
      // (code slot j holds token j + 1)
      if (rseed == 0) {
        const float pos = float(blk * kBlock + t16 + 1);
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int f = 16 * ft + 4 * q4 + v;
            rang[ft][v] = rope_rev(sra[f][0], sra[f][1], pos);
          }
        rseed = kReseed;
      } else {
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            rang[ft][v] = __builtin_amdgcn_fractf(rang[ft][v] + srd[16 * ft + 4 * q4 + v][0]);
      }
      --rseed;
    }
    if constexpr (RP) {
      // feature tiles {2 hf, 2 hf + 1} and their rotation partners {2 hf + 4, 2 hf + 5}
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 kr[4][2];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int ft = 2 * hf + (tt & 1) + 4 * (tt >> 1);
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) kr[tt][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          // U_K columns past rk are zero in LDS (and the code lanes of absent
          // groups read zeros), so chunks past a head's rank add nothing: for
          // narrow ranks they run unconditionally, sparing the branches
          for (int kc = 0; kc < NKC; ++kc) {
            if (kLean || 4 * kc < nkg) {
              const u32x4 a = *reinterpret_cast<const u32x4 *>(&su[(16 * ft + t16) * RS + 32 * kc + 8 * q4]);
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) kr[tt][h2] = mfma16x16x32(a, r.k[h2][kc], kr[tt][h2]);
            }
          }
        }
        // rotate pair (f, f + 64), f = 16 ft + 4 q4 + v, at the token's position
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int ft = 2 * hf + tt;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int f = 16 * ft + 4 * q4 + v;
            float sn2[2], cs2[2];
            if constexpr (kLean) {
              // the second token (16 positions on) by the angle-addition formula
              const float rev0 = rang[ft][v];
              sn2[0] = __builtin_amdgcn_sinf(rev0);
              cs2[0] = __builtin_amdgcn_cosf(rev0);
              const float c16 = srd[f][1], s16 = srd[f][2];
              cs2[1] = fmaf(cs2[0], c16, -sn2[0] * s16);
              sn2[1] = fmaf(sn2[0], c16, cs2[0] * s16);
            } else {
              const float pos = float(blk * kBlock + t16 + 1);
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                const float rev = rope_rev(sra[f][0], sra[f][1], pos + 16.f * h2);
                sn2[h2] = __builtin_amdgcn_sinf(rev);
                cs2[h2] = __builtin_amdgcn_cosf(rev);
              }
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const float sn = sn2[h2], cs = cs2[h2];
              const float x = kr[tt][h2][v], y = kr[tt + 2][h2][v];
              kr[tt][h2][v] = x * cs - y * sn;
              kr[tt + 2][h2][v] = fmaf(x, sn, y * cs);
            }
          }
        }
        // score chunks hf (tiles 2 hf, 2 hf + 1) and hf + 2 (tiles 2 hf + 4, 2 hf + 5)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int kcq = hf + 2 * cc;
          const u32x4 bh = rq[kcq][0][lane], bl = rq[kcq][1][lane];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[i] = kr[2 * cc][h2][i];
              x[4 + i] = kr[2 * cc + 1][h2][i];
            }
            u32x4 ah, al;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              ah[i] = pack_hi(x[2 * i], x[2 * i + 1]);
              al[i] = pack_rne(x[2 * i] - bf16_trunc(x[2 * i]), x[2 * i + 1] - bf16_trunc(x[2 * i + 1]));
            }
            s[h2] = mfma16x16x32(ah, bh, s[h2]);
            s[h2] = mfma16x16x32(ah, bl, s[h2]);
            s[h2] = mfma16x16x32(al, bh, s[h2]);
          }
        }
      }
    } else if constexpr (QC) {
      // int8 matrix cores: 16 columns (two 8-column chunks) per product; the
      // int8 codes are the A operand as loaded, 4-bit codes become 16 times their
      // value by moving each nibble to the top of a byte (even and odd elements of
      // a chunk in separate words); D = 254 D_a + D_b is exact in int32
      constexpr int NP = (NKC + 1) / 2;
      auto nib_even = [](uint32_t w) { return (w << 4) & 0xf0f0f0f0u; };
      auto nib_odd = [](uint32_t w) { return w & 0xf0f0f0f0u; };
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        i32x4 dh = i32x4{0, 0, 0, 0}, dl = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          if (8 * pp < nkg) {
            u32x4 a;
            if constexpr (CB == 8) {
              const u32x2 k0 = r.k[h2][2 * pp];
              const u32x2 k1 = 2 * pp + 1 < NKC ? r.k[h2][2 * pp + 1] : u32x2{0u, 0u};
              a = u32x4{k0[0], k0[1], k1[0], k1[1]};
            } else {
              const uint32_t k0 = r.k[h2][2 * pp];
              const uint32_t k1 = 2 * pp + 1 < NKC ? r.k[h2][2 * pp + 1] : 0u;
              a = u32x4{nib_even(k0), nib_odd(k0), nib_even(k1), nib_odd(k1)};
            }
            dh = mfma16x16x64_i8(a, sm.bq[pp][0][lane], dh);
            dl = mfma16x16x64_i8(a, sm.bq[pp][1][lane], dl);
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) s[h2][v] = float(dh[v] * 254 + dl[v]) * qsc;
      }
    } else {
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      if (4 * kc < nkg) {
        const u32x4 bh = sm.bq[kc][0][lane], bl = sm.bq[kc][1][lane];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u32x4 a = r.k[h2][kc];
          if (4 * kc + q4 >= nkg) a = u32x4{0u, 0u, 0u, 0u};
          s[h2] = mfma16x16x32(a, bh, s[h2]);
          s[h2] = mfma16x16x32(a, bl, s[h2]);
        }
      }
    }
    }
    if constexpr (QC) {
      float ksc[8];
      row_scales(r.sk, ksc);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[h2][v] *= ksc[4 * h2 + v];
    }
    const int tok0 = blk * kBlock;
    const bool ragged = tok0 + kBlock > c;
    if (ragged) {  // the ragged last block: mask slots >= c
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (tok0 + 16 * h2 + 4 * q4 + v >= c) s[h2][v] = kNegInf;
    }
    if constexpr (!QC) {
    if (tok0 + kBlock > c) {  // bf16 slots past c may hold any bits: zero them
      uint32_t keep[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j0 = 2 * i, j1 = 2 * i + 1;
        const bool v0 = tok0 + 16 * (j0 >> 2) + 4 * q4 + (j0 & 3) < c;
        const bool v1 = tok0 + 16 * (j1 >> 2) + 4 * q4 + (j1 & 3) < c;
        keep[i] = (v0 ? 0x0000ffffu : 0u) | (v1 ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int ni = 0; ni < NVC; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[ni][i] &= keep[i];
    }
    }
    // online softmax of head t16 over its 8 scores in this lane, 32 per block
    float bm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    bm = rows_max(bm);
    const float mn = fmaxf(m_run, bm);  // finite: a block holds at least one slot < c
    const float m_prev = m_run;
    const float alpha = fast_exp2(m_run - mn);
    // lanes of absent heads (t16 >= G) score 0 against zero queries: their weights
    // stay finite and only feed accumulator rows that are never read
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = fast_exp2(s[j >> 2][j & 3] - mn);
    l_run = l_run * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
    m_run = mn;
    // rescale the sums (lane (q4, t16) holds heads 4 q4 + v) unless no head's
    // maximum moved: then every factor is exactly 1
    if (__builtin_amdgcn_ballot_w64(mn != m_prev) != 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float a = __shfl(alpha, 4 * q4 + v, 64);
#pragma unroll
        for (int ni = 0; ni < NVC; ++ni) o[ni][v] *= a;
      }
      if constexpr (LR > 0) {  // head hh's factor sits in lane hh
#pragma unroll
        for (int hh = 0; hh < LR; ++hh) {
          if (hh < G) {
            const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), hh));
            res[hh][0] *= a;
            res[hh][1] *= a;
          }
        }
      }
    }
    if constexpr (LR > 0) {
      // kept residual rows: entry i holds slot t of this block (wave-uniform).  The
      // block's weights go to this wave's slice of the epilogue's LDS (free until
      // the wave leaves its loop) as [token][head]: lane (q4, t16) holds head t16's
      // weights of tokens 16 (j / 4) + 4 q4 + j % 4; an entry then reads its
      // token's weights of four heads at a time with one broadcast 16-byte load,
      // instead of selecting the register and reading each head's lane
      float *pw = &sm.w.o[wave][0][0];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pw[(16 * (jj >> 2) + 4 * q4 + (jj & 3)) * 16 + t16] = p[jj];
      wave_lds_fence();
#pragma unroll
      for (int i = 0; i < LRR; ++i) {
        if (i < L.R) {
          const int t = __builtin_amdgcn_readlane(int(r.es), i);
          if (t >= 0 && blk * kBlock + t < c) {
            const float e0 = __uint_as_float(r.e[i] << 16), e1 = __uint_as_float(r.e[i] & 0xffff0000u);
#pragma unroll
            for (int h4 = 0; h4 < LR; h4 += 4) {
              if (h4 < G) {
                const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&pw[t * 16 + h4]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  if (h4 + v < G) {
                    res[h4 + v][0] = fmaf(w4[v], e0, res[h4 + v][0]);
                    res[h4 + v][1] = fmaf(w4[v], e1, res[h4 + v][1]);
                  }
                }
              }
            }
          }
        }
      }
      wave_lds_fence();  // this block's reads are done before the next block's writes
    }
    // weights as the A operand (k-slot j = 4 h + v), hi and lo parts
    if constexpr (QC) {
      float vsc[8];
      row_scales(r.sv, vsc);
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] *= vsc[j];
      if (ragged) {  // slots past c: weight 0 whatever their scale holds (quantised codes are finite)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (tok0 + 16 * (j >> 2) + 4 * q4 + (j & 3) >= c) p[j] = 0.f;
      }
    }
    u32x4 a_hi, a_lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a_hi[i] = pack_hi(p[2 * i], p[2 * i + 1]);
      a_lo[i] = pack_rne(p[2 * i] - bf16_trunc(p[2 * i]), p[2 * i + 1] - bf16_trunc(p[2 * i + 1]));
    }
#pragma unroll
    for (int ni = 0; ni < NVC; ++ni) {
      if (ni < nvt) {
        u32x4 bv;
        if constexpr (CB == 8) bv = i8x8_to_bf16(r.v[ni]);
        else if constexpr (CB == 4) bv = i4x8_to_bf16_x16(r.v[ni]);
        else if constexpr (LR > 0) {
          // the key codes of columns 16 ni .. 16 ni + 15 as the value operand:
          // D[token][n] = C[token][32 kc + 16 half + n], lane (q4, t16) gets tokens
          // 16 h2 + 4 q4 + v of column 16 ni + t16, exact in float32
          const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
          const u32x4 sl = selector(ni & 1);
          const f32x4 d0 = mfma16x16x32(r.k[0][ni >> 1], sl, z);
          const f32x4 d1 = mfma16x16x32(r.k[1][ni >> 1], sl, z);
          bv = u32x4{pack_hi(d0[0], d0[1]), pack_hi(d0[2], d0[3]), pack_hi(d1[0], d1[1]), pack_hi(d1[2], d1[3])};
        } else bv = r.v[ni];
        o[ni] = mfma16x16x32(a_hi, bv, o[ni]);
        o[ni] = mfma16x16x32(a_lo, bv, o[ni]);
      }
    }
  };

  // double-buffered sweep.  The scheduling barriers keep the next block's loads
  // ahead of the current block's work: hoisting that work above them would make
  // the wave wait for the current block with nothing else in flight.
  // The block indices are wave-uniform; taken as scalars, the clamped index of
  // the next request is a scalar select, so nothing at the top of the loop writes
  // a vector register (such a write made the compiler wait there for every load
  // in flight, the next block's included, on every other block).  After the
  // wave's last block the request goes to the regions without extent.
  int j = __builtin_amdgcn_readfirstlane(first);
  const int jstep = __builtin_amdgcn_readfirstlane(step), jend = __builtin_amdgcn_readfirstlane(bhi);
  if (j < jend) {
    while (true) {
      load(j + jstep < jend ? j + jstep : j, j + jstep < jend, r1);
      __builtin_amdgcn_sched_barrier(0);
      process(j, r0);
      j += jstep;
      if (j >= jend) break;
      load(j + jstep < jend ? j + jstep : j, j + jstep < jend, r0);
      __builtin_amdgcn_sched_barrier(0);
      process(j, r1);
      j += jstep;
      if (j >= jend) break;
    }
  }

  // ---- per-wave state to LDS (pre-RoPE codes: U_K and q's operands share the
  // space of the rank-space sums, so every wave must be done with its blocks)
  if constexpr (RP) __syncthreads();
  l_run = rows_sum(l_run);
  if (q4 == 0 && t16 < G) {
    sm.m[wave][t16] = m_run;
    sm.l[wave][t16] = l_run;
  }
#pragma unroll
  for (int ni = 0; ni < NVC; ++ni) {
    if (ni < nvt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int head = 4 * q4 + v;
        if (head < G) sm.w.o[wave][head][16 * ni + t16] = o[ni][v];
      }
    }
  }

  __syncthreads();

  // ---- merge the four waves and the anchors into the split's records
  auto weight = [&](int w, int hh, float M) {
    const float mw = sm.m[w][hh];
    return mw == kNegInf ? 0.f : fast_exp2(mw - M);
  };
  auto head_max = [&](int hh) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 5; ++w) M = fmaxf(M, sm.m[w][hh]);
    return M;
  };
  for (int i = tid; i < G * rv; i += blockDim.x) {
    const int hh = i / rv, cc = i - hh * rv;
    const float M = head_max(hh);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = fmaf(weight(w, hh, M), sm.w.o[w][hh][cc], acc);
    split_record(d, q0 + hh, split)[4 + cc] = acc * kX16;
  }
  // o_A of the heads whose KV head has anchor rows in this split; the combine
  // reads it from exactly these splits and skips the others
  if constexpr (LR > 0) {
    // every split: the waves' residual sums and the anchor sums under the head's
    // common max, added into sm.u.oa wave by wave (wave 0 first, over its anchors)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (wave == w) {
#pragma unroll
        for (int hh = 0; hh < LR; ++hh) {
          if (hh < G) {
            const float M = head_max(hh);
            const float f = weight(w, hh, M);
            float x0 = f * res[hh][0], x1 = f * res[hh][1];
            if (w > 0) {
              x0 += sm.u.oa[hh][2 * lane];
              x1 += sm.u.oa[hh][2 * lane + 1];
            } else if (na > 0) {
              const float fa = weight(4, hh, M);
              x0 = fmaf(fa, sm.u.oa[hh][2 * lane], x0);
              x1 = fmaf(fa, sm.u.oa[hh][2 * lane + 1], x1);
            }
            sm.u.oa[hh][2 * lane] = x0;
            sm.u.oa[hh][2 * lane + 1] = x1;
          }
        }
      }
      __syncthreads();
    }
    for (int i = tid; i < G * kD; i += blockDim.x) {
      const int hh = i / kD, cc = i - hh * kD;
      split_record(d, q0 + hh, split)[d.oa + cc] = sm.u.oa[hh][cc];
    }
  } else if (na > 0) {
    for (int i = tid; i < G * kD; i += blockDim.x) {
      const int hh = i / kD, cc = i - hh * kD;
      const int jj = hh / GK;
      if (jj * a1 < ahi && (jj + 1) * a1 > alo)
        split_record(d, q0 + hh, split)[d.oa + cc] = weight(4, hh, head_max(hh)) * sm.u.oa[hh][cc];
    }
  }
  for (int hh = tid; hh < G; hh += blockDim.x) {
    const float M = head_max(hh);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < 5; ++w) l = fmaf(weight(w, hh, M), sm.l[w][hh], l);
    float *rec = split_record(d, q0 + hh, split);
    rec[0] = M;
    rec[1] = l;
    rec[2] = float(sg.v);
    rec[3] = 0.f;
  }
}

// The kernels.  Code-space instances whose value width is at most 32 are asked
// to fit four workgroups per compute unit (128 registers a lane): every such
// instance does so without spilling, except the 128-wide key body with bf16 codes
// and the LowRAM bodies with 16 residual rows, which keep the compiler's own
// choice, as do the wider value bodies (they cannot fit four).  The pre-RoPE
// instances are asked for three where that needs no spill (their LDS is sized for
// three), else for two (the 128/128 body keeps the compiler's choice: it spills
// at two).
template <int RKMAX, int RVMAX, int CB, int LR>
constexpr int partials_min_blocks() {
  return (RVMAX <= 32 && LR != 16 && !(RKMAX == 128 && CB == 16)) ? 4 : 1;
}
//
// With mixed ranks (not EXACT, code-space values) a workgroup whose group's key
// width fits a narrower body (64 columns; 32 in the 64-wide instances) runs that
// body, so narrow groups do not carry the widest group's score MFMAs and operand
// slots; the two bodies share one LDS allocation (the wider layout; the narrower
// one is no larger).  (A third body made the compiler copy the kernel arguments
// to scratch.)
template <int RKMAX, int RVMAX, bool EXACT, int CB, int LR = 0, int LRR = 0>
__global__ __launch_bounds__(256, (partials_min_blocks<RKMAX, RVMAX, CB, LR>())) void k_partials_mfma(LayerArgs L, DecodeArgs d) {
  __shared__ MfmaSmem<RKMAX, RVMAX, false> sm;
  if constexpr (!EXACT && LR == 0 && RKMAX > 32) {
    constexpr int NARROW = RKMAX > 64 ? 64 : 32;
    if (L.heads[work_item(L, d).h].rk <= NARROW) {
      partials_body<NARROW, RVMAX, false, CB>(L, d, reinterpret_cast<MfmaSmem<NARROW, RVMAX, false> &>(sm));
      return;
    }
  }
  partials_body<RKMAX, RVMAX, EXACT, CB, LR, LRR, false>(L, d, sm);
}
template <int RKMAX, int RVMAX>
constexpr int rope_min_blocks() {
  return (RKMAX == 128 && RVMAX == 128) ? 1 : (RVMAX <= 32 && RKMAX <= 64 && !(RKMAX == 64 && RVMAX == 32)) ? 3 : 2;
}
template <int RKMAX, int RVMAX>
__global__ __launch_bounds__(256, (rope_min_blocks<RKMAX, RVMAX>())) void k_partials_rope(LayerArgs L, DecodeArgs d) {
  __shared__ MfmaSmem<RKMAX, RVMAX, true> sm;
  partials_body<RKMAX, RVMAX, false, 16, 0, 0, true>(L, d, sm);
}

// ---------------------------------------------------------------------------
// instance selection (the same choice for the launch and for the occupancy the
// host sizes grids by)
// ---------------------------------------------------------------------------
typedef void (*PartialsFn)(LayerArgs, DecodeArgs);

template <int RKMAX, int RVMAX, bool EXACT>
static PartialsFn pick_cb(const LayerArgs &L) {
  if (L.dtype == LRKV_BF16_Q8) return k_partials_mfma<RKMAX, RVMAX, EXACT, 8>;
  if (L.dtype == LRKV_BF16_Q4) return k_partials_mfma<RKMAX, RVMAX, EXACT, 4>;
  return k_partials_mfma<RKMAX, RVMAX, EXACT, 16>;
}

template <int RKMAX, int RVMAX>
static PartialsFn pick_rv(const LayerArgs &L) {
  bool exact = true;
  for (int h = 0; h < L.n_lat; ++h) exact = exact && L.heads[h].rk == RKMAX && L.heads[h].rv == RVMAX;
  return exact ? pick_cb<RKMAX, RVMAX, true>(L) : pick_cb<RKMAX, RVMAX, false>(L);
}

template <int RKMAX>
static PartialsFn pick_rk(const LayerArgs &L) {
  if (L.rv_max <= 16) return pick_rv<RKMAX, 16>(L);
  if (L.rv_max <= 32) return pick_rv<RKMAX, 32>(L);
  if (L.rv_max <= 64) return pick_rv<RKMAX, 64>(L);
  return pick_rv<RKMAX, 128>(L);
}

// LowRAM layers: value sums over the key codes (RVMAX = RKMAX), bf16 codes; ranks
// are read per head (no exact-rank instances); register arrays sized for at most
// 4 query heads per KV head and 4 residual entries where that suffices
template <int RKMAX>
static PartialsFn pick_lr(const LayerArgs &L) {
  const bool g4 = L.group <= 4, r4 = L.R <= 4;
  if (g4 && r4) return k_partials_mfma<RKMAX, RKMAX, false, 16, 4, 4>;
  if (g4) return k_partials_mfma<RKMAX, RKMAX, false, 16, 4, 8>;
  if (r4) return k_partials_mfma<RKMAX, RKMAX, false, 16, 16, 4>;
  return k_partials_mfma<RKMAX, RKMAX, false, 16, 16, 8>;
}

// keys compressed before RoPE (bf16 codes, per-head ranks read at run time)
template <int RKMAX>
static PartialsFn pick_rp(const LayerArgs &L) {
  if (L.rv_max <= 16) return k_partials_rope<RKMAX, 16>;
  if (L.rv_max <= 32) return k_partials_rope<RKMAX, 32>;
  if (L.rv_max <= 64) return k_partials_rope<RKMAX, 64>;
  return k_partials_rope<RKMAX, 128>;
}

static PartialsFn pick_partials(const LayerArgs &L) {
  int rk_max = 0;
  for (int h = 0; h < L.n_lat; ++h) rk_max = L.heads[h].rk > rk_max ? L.heads[h].rk : rk_max;
  if (L.rope) {
    if (rk_max <= 32) return pick_rp<32>(L);
    if (rk_max <= 64) return pick_rp<64>(L);
    if (rk_max <= 96) return pick_rp<96>(L);
    return pick_rp<128>(L);
  }
  if (L.lowram) {
    if (rk_max <= 32) return pick_lr<32>(L);
    if (rk_max <= 64) return pick_lr<64>(L);
    if (rk_max <= 96) return pick_lr<96>(L);
    return pick_lr<128>(L);
  }
  if (rk_max <= 32) return pick_rk<32>(L);
  if (rk_max <= 64) return pick_rk<64>(L);
  if (rk_max <= 96) return pick_rk<96>(L);
  return pick_rk<128>(L);
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// resident workgroups of 256 threads per compute unit for a kernel, asked of the
// runtime once per (kernel, device) and remembered
int kernel_blocks_per_cu(const void *fn) {
  static std::mutex mu;
  static std::map<std::pair<const void *, int>, int> known;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const auto key = std::make_pair(fn, dev);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = known.find(key);
    if (it != known.end()) return it->second;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 256, 0) != hipSuccess) return 0;
  std::lock_guard<std::mutex> g(mu);
  known[key] = n;
  return n;
}

int partials_blocks_per_cu(const LayerArgs &L) {
  if (L.dtype == LRKV_F32) return generic_blocks_per_cu();
  return kernel_blocks_per_cu(reinterpret_cast<const void *>(pick_partials(L)));
}

hipError_t launch_partials_mfma(const LayerArgs &L, const DecodeArgs &d0, hipStream_t s) {
  DecodeArgs d = d0;
  // balancing pays when the whole grid is resident at once
  const int per_cu = partials_blocks_per_cu(L), cus = device_cu_count();
  d.balance = per_cu > 0 && cus > 0 && int64_t(d.items) <= int64_t(per_cu) * cus;
  PartialsFn fn = pick_partials(L);
  LayerArgs la = L;
  void *args[] = {&la, &d};
  return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(d.row_items, L.batch), dim3(256), args, 0, s);
}

}  // namespace lrkv
