// Prefill projection of bfloat16 keys or values into codes on the gfx950 matrix
// cores (blog "Half the Memory, None of the Answers Lost", section 04: one
// projection per (layer, head), keys taken after RoPE): code[t][c] = x_t . u_c for
// the rank-many basis directions u_c (the rows of U^T), float32 accumulation,
// rounded to nearest even bf16.
//
// One workgroup of four waves per (128-token tile, batch row, KV head).  The
// head's U^T rows are staged once in LDS (rows padded to 136 elements so the 16
// lanes of a fragment read 16 different bank groups); each wave takes 32 tokens
// as two 16-token tiles, loads their rows once (16 bytes per lane per 32
// features) and sweeps the 16-column tiles of the code:
//
//   keys    D[col][token]: A = U^T rows, B = x; a lane ends with 4 consecutive
//           columns of one token, 8 contiguous bytes of the key layout
//   values  D[token][col]: A = x, B = U^T rows; a lane ends with 4 consecutive
//           tokens of one column, 8 contiguous bytes of the value layout (when the
//           4 slots are 4-aligned and present; single elements otherwise)
//
// The work is bound by reading the 256-byte input rows: 16 MFMAs per 32 tokens
// and 16 columns keep the matrix cores a small fraction busy.

#include "mfma_util.h"

namespace lrkv {

constexpr int kUStride = kD + 8;  // padded LDS row of one basis direction

__global__ __launch_bounds__(256) void k_compress_mfma(LayerArgs L, int which, const bf16_t *x,
                                                       int64_t sb, int64_t sh, int64_t st,
                                                       int n_tok, int slot0) {
  __shared__ bf16_t su[kD * kUStride];
  const int unit = blockIdx.y;
  const int b = unit / L.n_kv, h = unit % L.n_kv;
  const HeadInfo hd = L.heads[h];
  const int r = which ? hd.rv : hd.rk;
  const bf16_t *ut = static_cast<const bf16_t *>(L.bases) + (which ? hd.u_v : hd.u_k);
  bf16_t *codes = static_cast<bf16_t *>(which ? L.codes_v : L.codes_k) + (which ? hd.cv : hd.ck) +
                  int64_t(b) * L.cap * r;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;

  // this wave's input rows first (their HBM latency overlaps the staging of U^T):
  // lane (q4, t16) holds token t16's features 32 kc + 8 q4 .. +7 of the two 16-token
  // tiles; rows past n_tok re-read the last one and are not stored
  const int t_base = blockIdx.x * 128 + wave * 32;
  const bf16_t *xb = x + b * sb + h * sh;
  u32x4 xo[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tok = min(t_base + 16 * tt + t16, n_tok - 1);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      xo[tt][kc] = *reinterpret_cast<const u32x4 *>(xb + int64_t(tok) * st + 32 * kc + 8 * q4);
  }
  // U^T rows, r x 16 pieces of 16 bytes, all requested before any is stored
  u32x4 uu[kD * 16 / 256];
#pragma unroll
  for (int k = 0; k < kD * 16 / 256; ++k) {
    const int p = min(tid + 256 * k, r * 16 - 1);
    uu[k] = *reinterpret_cast<const u32x4 *>(ut + (p >> 4) * kD + (p & 15) * 8);
  }
#pragma unroll
  for (int k = 0; k < kD * 16 / 256; ++k) {
    const int p = tid + 256 * k;
    if (p < r * 16) *reinterpret_cast<u32x4 *>(&su[(p >> 4) * kUStride + (p & 15) * 8]) = uu[k];
  }
  __syncthreads();
  if (t_base >= n_tok) return;  // no barrier follows
  for (int nt = 0; nt < r / 16; ++nt) {
    u32x4 uo[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      uo[kc] = *reinterpret_cast<const u32x4 *>(&su[(16 * nt + t16) * kUStride + 32 * kc + 8 * q4]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (which == 0) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) acc = mfma16x16x32(uo[kc], xo[tt][kc], acc);
        // lane (q4, t16): columns 16 nt + 4 q4 + v of token t16
        const int tok = t_base + 16 * tt + t16;
        if (tok < n_tok) {
          uint2 v2;
          v2.x = pack_rne(acc[0], acc[1]);
          v2.y = pack_rne(acc[2], acc[3]);
          *reinterpret_cast<uint2 *>(codes + kslot(slot0 + tok, 16 * nt + 4 * q4, r)) = v2;
        }
      } else {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) acc = mfma16x16x32(xo[tt][kc], uo[kc], acc);
        // lane (q4, t16): tokens 4 q4 + v of column 16 nt + t16
        const int tok0 = t_base + 16 * tt + 4 * q4;
        const int col = 16 * nt + t16;
        const int j0 = slot0 + tok0;
        if (tok0 + 3 < n_tok && (j0 & 3) == 0) {
          uint2 v2;
          v2.x = pack_rne(acc[0], acc[1]);
          v2.y = pack_rne(acc[2], acc[3]);
          *reinterpret_cast<uint2 *>(codes + vslot(j0, col, r)) = v2;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (tok0 + v < n_tok) codes[vslot(j0 + v, col, r)] = from_f32<bf16_t>(acc[v]);
        }
      }
    }
  }
}

hipError_t launch_compress_mfma(const LayerArgs &L, int which, const void *x, int64_t sb,
                                int64_t sh, int64_t st, int n_tok, int slot0, hipStream_t s) {
  dim3 grid((n_tok + 127) / 128, L.batch * L.n_kv);
  hipLaunchKernelGGL(k_compress_mfma, grid, dim3(256), 0, s, L, which,
                     static_cast<const bf16_t *>(x), sb, sh, st, n_tok, slot0);
  return hipGetLastError();
}

}  // namespace lrkv
