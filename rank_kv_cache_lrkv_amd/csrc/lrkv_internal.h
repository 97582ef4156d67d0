// Internal definitions shared by the kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrkv.h"

namespace lrkv {

constexpr int kD = LRKV_HEAD_DIM;
constexpr int kBlock = LRKV_BLOCK;
constexpr float kLog2e = 1.4426950408889634f;

// Per-KV-head geometry, element offsets precomputed on the host.
struct HeadInfo {
  int32_t rk, rv;
  int32_t u_k, u_v;  // offsets of U_K(h), U_V(h) in the bases buffer (rows of hg * 128)
  int64_t ck, cv;    // offsets of head h's [batch][cap][r] code region
  int64_t pred;      // LowRAM: element offset of M(0, h) in the predictor buffer
};

// With group-head latents (hg > 1) the hg consecutive KV heads of latent group g
// share one code stream; HeadInfo and the code / scale regions are per latent
// group (n_lat of them), anchors per KV head.  hg = 1: a group is one KV head.
struct LayerArgs {
  int32_t dtype, batch, n_q, n_kv, group, window, cap, rv_max;
  int32_t hg, n_lat;           // KV heads per latent group, latent groups
  const void *bases;
  void *codes_k, *codes_v, *anchor_k, *anchor_v;
  float *scales_k, *scales_v;  // quantised codes: one scale per (head, row, slot)
  int32_t n_versions;          // basis versions (>= 1)
  const int32_t *vstart;       // [batch][n_versions] first code slot of each version (n_versions > 1)
  int64_t version_elems;       // elements of one version of the bases
  // LowRAM value amortisation: values are C_K M(b, h) plus kept residual rows;
  // for these layers heads[h].rv == heads[h].rk (the value sums are rank_k wide)
  int32_t lowram, R;           // the mode, residual entries per 32-slot block
  void *pred;                  // bf16 M(b, h) rows (rank_k x 128)
  void *resid;                 // bf16 residual rows, [h][b][cap / 32][R][128]
  int32_t *rslot;              // in-block slot of each entry, -1 empty
  float *rnorm;                // squared norm of each entry
  // keys compressed before RoPE: rope_a[i] = theta_i / (2 pi) as a float32 pair
  // (hi, lo), theta_i = base^(-2 i / 128), so angles in revolutions come out
  // exact to float32 at any position
  int32_t rope;
  float rope_a[kD / 2][2];
  HeadInfo heads[LRKV_MAX_KV_HEADS];
};

// the RoPE angle of pair i at position pos, in revolutions reduced to about
// [-0.5, 0.5]: pos * (hi + lo) with the product's rounding error recovered by an FMA
__device__ __forceinline__ float rope_rev(float hi, float lo, float pos) {
  const float p = pos * hi;
  const float e = fmaf(pos, hi, -p);
  return (p - __builtin_rintf(p)) + fmaf(pos, lo, e);
}

// LowRAM: index of entry i of block j of (head h, row b)
__host__ __device__ __forceinline__ int64_t resid_entry(const LayerArgs &L, int h, int b, int j, int i) {
  return ((int64_t(h) * L.batch + b) * (L.cap / kBlock) + j) * L.R + i;
}

// Split s of a (batch row, KV head) covers a share of its code blocks and a
// share of its a anchors (runs of at least 16 rows on the first splits); per
// query head it leaves one record in the workspace:
//   [m, l, v, 0, o~[rvp], o_A[128]]
// m: running max of the scores (log2 units, -inf if the split saw nothing),
// v: the split's basis version (a float32 integer; 0 with one version),
// l: sum of 2^(s - m), o~: rank-space value sum of the codes (rvp = rv_max
// rounded up to 4), o_A: 128-dim value sum of the anchors (written only by
// splits that hold anchors).
//
// Splits per latent group.  n_splits = S is the split count of the group with
// the most code bytes per token; group h gets S_h = nsplit[h] <= S splits, in
// proportion to its own code bytes per token (all S with uniform ranks), so the
// workgroups of a layer with mixed ranks stream about the same bytes each.
// Stage 1 runs one workgroup per work item (batch row b, group h, split s < S_h),
// items ordered by b, then h, then s: row_items = sum_h S_h per row, group h's
// first item of a row at split0[h].  The launch grid is (row_items, batch).
struct DecodeArgs {
  int32_t n_ctx;
  int32_t n_splits;      // S: record stride, and S_h of the widest groups
  int32_t rec;           // floats per record: 4 + rvp + 128
  int32_t oa;            // offset of o_A in a record: 4 + rvp
  float scale_log2;      // sm_scale * log2(e): scores are kept in log2 units
  const int32_t *ctx_lens;
  const void *q;
  float *ws;             // [batch][n_q][n_splits][rec]
  int32_t balance;       // stage 1: raise the wave priority of the waves with more work left
  int32_t uniform;       // every group has S_h = S
  int32_t row_items;     // sum over groups of S_h
  int32_t items;         // batch * row_items: the stage-1 workgroups
  int32_t nsplit[LRKV_MAX_KV_HEADS];      // S_h
  int32_t split0[LRKV_MAX_KV_HEADS + 1];  // first item of group h within a row
};

// host: the workgroups of one stage-1 launch that are resident on one compute
// unit at once, for the kernel instance the layer would launch (0 if unknown)
int partials_blocks_per_cu(const LayerArgs &L);
// host: compute units of the current device (0 if unknown)
int device_cu_count();
// host: resident workgroups of 256 threads per compute unit of a kernel, and of
// the float32 stage-1 kernel (0 if unknown)
int kernel_blocks_per_cu(const void *fn);
int generic_blocks_per_cu();

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  // gfx950 converts with round-to-nearest-even in hardware (v_cvt_pk_bf16_f32)
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(bf16_t, b);
}

// ---------------------------------------------------------------------------
// code layout: in-block element positions (see lrkv.h)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kpos(int t, int c, int r) {
  return ((t >> 4) * (r >> 3) + (c >> 3)) * 128 + (t & 15) * 8 + (c & 7);
}
__device__ __forceinline__ int vpos(int t, int c, int r) {
  return (((t & 15) >> 2) * r + c) * 8 + ((t >> 4) << 2) + (t & 3);
}
// element offset of code slot j, column c, inside one (row, head) region
__device__ __forceinline__ int64_t kslot(int j, int c, int r) {
  return int64_t(j >> 5) * (kBlock * r) + kpos(j & 31, c, r);
}
__device__ __forceinline__ int64_t vslot(int j, int c, int r) {
  return int64_t(j >> 5) * (kBlock * r) + vpos(j & 31, c, r);
}

__device__ __forceinline__ int anchor_slot(int p, int window) {
  return p == 0 ? 0 : 1 + (p - 1) % window;
}

// quantised codes: element of the scale of slot j of (latent group h, batch row b)
__device__ __forceinline__ int64_t scale_index(const LayerArgs &L, int h, int b, int j) {
  return (int64_t(h) * L.batch + b) * L.cap + j;
}
// QMAX = 127 (int8 codes) or 7 (4-bit codes): the scale of a code row with
// largest magnitude a, and one quantised value, x / s rounded to nearest even
// and clipped to [-QMAX, QMAX] (float32 divisions, correctly rounded); a zero
// row (s = 0) quantises to 0
template <int QMAX> __device__ __forceinline__ float qn_scale(float absmax) { return absmax / float(QMAX); }
template <int QMAX> __device__ __forceinline__ int qn_value(float x, float s) {
  if (!(s > 0.f)) return 0;
  const float t = __builtin_rintf(x / s);
  return int(fminf(fmaxf(t, -float(QMAX)), float(QMAX)));
}
__device__ __forceinline__ float q8_scale(float absmax) { return qn_scale<127>(absmax); }
__device__ __forceinline__ int q8_value(float x, float s) { return qn_value<127>(x, s); }

// 4-bit codes: store value q of element position p of a region (two per byte,
// even p in the low half).  Neighbouring elements share bytes, so the update is
// two word-wide atomics on disjoint bits: any number of threads may store
// different elements of one word concurrently.
__device__ __forceinline__ void store_q4(uint8_t *region, int64_t p, int q) {
  const int64_t byte = p >> 1;
  uint32_t *word = reinterpret_cast<uint32_t *>(region + (byte & ~int64_t(3)));
  const int shift = int(byte & 3) * 8 + int(p & 1) * 4;
  atomicAnd(word, ~(0xfu << shift));
  atomicOr(word, (uint32_t(q) & 0xfu) << shift);
}

// bits per code element: 16 (bf16), 32 (f32), 8 or 4 (quantised)
__device__ __host__ __forceinline__ int code_bits(int dtype) {
  return dtype == LRKV_F32 ? 32 : dtype == LRKV_BF16 ? 16 : dtype == LRKV_BF16_Q8 ? 8 : 4;
}

// context length of batch row b
__device__ __forceinline__ int row_ctx(const DecodeArgs &d, int b) {
  if (!d.ctx_lens) return d.n_ctx;
  int n = d.ctx_lens[b];
  return n < 1 ? 1 : (n > d.n_ctx ? d.n_ctx : n);
}

// ---------------------------------------------------------------------------
// host-side launchers (defined in the .hip files)
// ---------------------------------------------------------------------------
hipError_t launch_compress(const LayerArgs &L, int which, const void *x, int64_t sb, int64_t sh,
                           int64_t st, int n_tok, int slot0, hipStream_t s);
hipError_t launch_compress_mfma(const LayerArgs &L, int which, const void *x, int64_t sb,
                                int64_t sh, int64_t st, int n_tok, int slot0, hipStream_t s);
hipError_t launch_quantize(const LayerArgs &L, int which, const float *x, int64_t sb, int64_t sh,
                           int64_t st, int n_tok, int slot0, hipStream_t s);
hipError_t launch_store_anchors(const LayerArgs &L, const void *k, const void *v, int64_t sb,
                                int64_t sh, int64_t st, int pos0, int n_tok, hipStream_t s);
hipError_t launch_append(const LayerArgs &L, const void *k, const void *v, int pos, hipStream_t s);
hipError_t launch_decode_partials(const LayerArgs &L, const DecodeArgs &d, hipStream_t s);
hipError_t launch_partials_mfma(const LayerArgs &L, const DecodeArgs &d, hipStream_t s);
hipError_t launch_decode_combine(const LayerArgs &L, const DecodeArgs &d, float *out, hipStream_t s);
// the decode step with its split records in the library's per-device array
// (noalloc.hip); D.ws is set there
size_t noalloc_scratch_bytes();
lrkv_status decode_attn_noalloc(const LayerArgs &A, DecodeArgs &D, float *out, hipStream_t s);
hipError_t launch_oja(const LayerArgs &L, int which, const void *x, int64_t sb, int64_t sh, int64_t st,
                      int n_tok, float eta, int vin, int vout, float *ws, hipStream_t s);
size_t oja_workspace_bytes(const LayerArgs &L);
hipError_t launch_lowram_fit(const LayerArgs &L, const bf16_t *v, int64_t sb, int64_t sh, int64_t st, int n_tok,
                             float *ws, hipStream_t s);
size_t lowram_workspace_bytes(const LayerArgs &L);

}  // namespace lrkv
