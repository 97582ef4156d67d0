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
//
// Quantised codes (LRKV_BF16_Q8, LRKV_BF16_Q4) take the same products; each
// token's row is then quantised with its own scale (largest |code| / 127 or / 7).

#include "mfma_util.h"

namespace lrkv {

constexpr int kUStride = kD + 8;  // padded LDS row of one basis direction

// 4 quantised values, first value lowest: int8 in the bytes of a word (QMAX 127)
// or 4-bit in the nibbles of a half word (QMAX 7)
template <int QMAX>
__device__ __forceinline__ uint32_t pack_qn(f32x4 v, float s0, float s1, float s2, float s3) {
  constexpr int B = QMAX == 127 ? 8 : 4;
  constexpr uint32_t M = (1u << B) - 1;
  return (uint32_t(qn_value<QMAX>(v[0], s0)) & M) | ((uint32_t(qn_value<QMAX>(v[1], s1)) & M) << B) |
         ((uint32_t(qn_value<QMAX>(v[2], s2)) & M) << (2 * B)) |
         ((uint32_t(qn_value<QMAX>(v[3], s3)) & M) << (3 * B));
}

// QMAX > 0: quantised codes (127: int8, 7: 4 bits) with one float32 scale per
// token and matrix.  The largest |code| of a token is known only once every
// column tile is done, so the tiles are swept twice (the products are cheap next
// to reading the rows): the first sweep takes the maxima and writes the scales,
// the second quantises.
template <int QMAX>
__global__ __launch_bounds__(256) void k_compress_mfma(LayerArgs L, int which, const bf16_t *x,
                                                       int64_t sb, int64_t sh, int64_t st,
                                                       int n_tok, int slot0) {
  __shared__ bf16_t su[kD * kUStride];
  const int unit = blockIdx.y;
  const int b = unit / L.n_lat, h = unit % L.n_lat;
  const HeadInfo hd = L.heads[h];
  const int r = which ? hd.rv : hd.rk;
  // the latest basis version (prefill compresses before later versions appear)
  const bf16_t *ut = static_cast<const bf16_t *>(L.bases) + (L.n_versions - 1) * L.version_elems +
                     (which ? hd.u_v : hd.u_k);
  const int64_t region = (which ? hd.cv : hd.ck) + int64_t(b) * L.cap * r;
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

  // column tile nt of the basis, then the 16 x 16 product with token tile tt
  // (keys: lane (q4, t16) gets columns 16 nt + 4 q4 + v of token t16; values:
  // tokens 4 q4 + v of column 16 nt + t16)
  auto basis_tile = [&](int nt, u32x4 (&uo)[4]) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      uo[kc] = *reinterpret_cast<const u32x4 *>(&su[(16 * nt + t16) * kUStride + 32 * kc + 8 * q4]);
  };
  auto product = [&](const u32x4 (&uo)[4], int tt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (which == 0) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) acc = mfma16x16x32(uo[kc], xo[tt][kc], acc);
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) acc = mfma16x16x32(xo[tt][kc], uo[kc], acc);
    }
    return acc;
  };

  if constexpr (QMAX == 0) {
    bf16_t *codes = static_cast<bf16_t *>(which ? L.codes_v : L.codes_k) + region;
    for (int nt = 0; nt < r / 16; ++nt) {
      u32x4 uo[4];
      basis_tile(nt, uo);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 acc = product(uo, tt);
        if (which == 0) {
          const int tok = t_base + 16 * tt + t16;
          if (tok < n_tok) {
            uint2 v2;
            v2.x = pack_rne(acc[0], acc[1]);
            v2.y = pack_rne(acc[2], acc[3]);
            *reinterpret_cast<uint2 *>(codes + kslot(slot0 + tok, 16 * nt + 4 * q4, r)) = v2;
          }
        } else {
          // 8 contiguous bytes when the 4 slots are 4-aligned and present
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
  } else {
    // int8: one byte per element; 4 bits: regions start on even elements
    uint8_t *codes = static_cast<uint8_t *>(which ? L.codes_v : L.codes_k) + (QMAX == 127 ? region : region / 2);
    // 4 consecutive elements from element position p (a multiple of 4)
    auto store4 = [&](int64_t p, uint32_t packed) {
      if constexpr (QMAX == 127) *reinterpret_cast<uint32_t *>(codes + p) = packed;
      else *reinterpret_cast<uint16_t *>(codes + p / 2) = uint16_t(packed);
    };
    auto store1 = [&](int64_t p, int q) {
      if constexpr (QMAX == 127) codes[p] = uint8_t(q);
      else store_q4(codes, p, q);
    };
    float *scales = (which ? L.scales_v : L.scales_k) + scale_index(L, h, b, 0);
    // sweep 1: amax[tt][v] = largest |code| of this lane's token(s) (keys: v = 0 only)
    float amax[2][4] = {};
    for (int nt = 0; nt < r / 16; ++nt) {
      u32x4 uo[4];
      basis_tile(nt, uo);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 acc = product(uo, tt);
        if (which == 0) {
          amax[tt][0] = fmaxf(amax[tt][0], fmaxf(fmaxf(fabsf(acc[0]), fabsf(acc[1])),
                                                 fmaxf(fabsf(acc[2]), fabsf(acc[3]))));
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) amax[tt][v] = fmaxf(amax[tt][v], fabsf(acc[v]));
        }
      }
    }
    // keys: a token's columns are spread over the 4 lanes q4 (xor 16, 32);
    // values: over the 16 lanes t16 (xor 1 .. 8)
    float sc[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (which == 0) {
        float a = amax[tt][0];
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        sc[tt][0] = sc[tt][1] = sc[tt][2] = sc[tt][3] = qn_scale<QMAX>(a);
        const int tok = t_base + 16 * tt + t16;
        if (q4 == 0 && tok < n_tok) scales[slot0 + tok] = sc[tt][0];
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float a = amax[tt][v];
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
          sc[tt][v] = qn_scale<QMAX>(a);
          const int tok = t_base + 16 * tt + 4 * q4 + v;
          if (t16 == 0 && tok < n_tok) scales[slot0 + tok] = sc[tt][v];
        }
      }
    }
    // sweep 2: quantise and store (4 bytes of one word where they are contiguous)
    for (int nt = 0; nt < r / 16; ++nt) {
      u32x4 uo[4];
      basis_tile(nt, uo);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 acc = product(uo, tt);
        if (which == 0) {
          const int tok = t_base + 16 * tt + t16;
          if (tok < n_tok)
            store4(kslot(slot0 + tok, 16 * nt + 4 * q4, r),
                   pack_qn<QMAX>(acc, sc[tt][0], sc[tt][0], sc[tt][0], sc[tt][0]));
        } else {
          const int tok0 = t_base + 16 * tt + 4 * q4;
          const int col = 16 * nt + t16;
          const int j0 = slot0 + tok0;
          if (tok0 + 3 < n_tok && (j0 & 3) == 0) {
            store4(vslot(j0, col, r), pack_qn<QMAX>(acc, sc[tt][0], sc[tt][1], sc[tt][2], sc[tt][3]));
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (tok0 + v < n_tok) store1(vslot(j0 + v, col, r), qn_value<QMAX>(acc[v], sc[tt][v]));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Head groups (Palu's group-head latents): one workgroup per (128-token tile,
// batch row, latent group).  A token's code is the product of its concatenated
// rows (the group's KV heads one after another) with U(g), so the kernel walks
// the KV heads j of the group: it loads that head's rows, stages slice j of the
// U^T rows (columns 128 j .. 128 j + 127) in LDS and adds the products into
// accumulators that hold every column tile of the wave's 32 tokens.  The codes
// are stored (or quantised from the accumulators: the row maxima need no second
// sweep) once all heads are in.
// ---------------------------------------------------------------------------
template <int QMAX>
__global__ __launch_bounds__(256) void k_compress_group(LayerArgs L, int which, const bf16_t *x,
                                                        int64_t sb, int64_t sh, int64_t st,
                                                        int n_tok, int slot0) {
  __shared__ bf16_t su[kD * kUStride];
  const int unit = blockIdx.y;
  const int b = unit / L.n_lat, h = unit % L.n_lat;
  const HeadInfo hd = L.heads[h];
  const int r = which ? hd.rv : hd.rk;
  const int ntr = r / 16;
  const int urow = L.hg * kD;
  const bf16_t *ut = static_cast<const bf16_t *>(L.bases) + (L.n_versions - 1) * L.version_elems +
                     (which ? hd.u_v : hd.u_k);
  const int64_t region = (which ? hd.cv : hd.ck) + int64_t(b) * L.cap * r;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, t16 = lane & 15;
  const int t_base = blockIdx.x * 128 + wave * 32;

  f32x4 acc[kD / 16][2];
#pragma unroll
  for (int nt = 0; nt < kD / 16; ++nt) acc[nt][0] = acc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < L.hg; ++j) {
    const bf16_t *xb = x + b * sb + (int64_t(h) * L.hg + j) * sh;
    u32x4 xo[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = min(t_base + 16 * tt + t16, n_tok - 1);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        xo[tt][kc] = *reinterpret_cast<const u32x4 *>(xb + int64_t(tok) * st + 32 * kc + 8 * q4);
    }
    u32x4 uu[kD * 16 / 256];
#pragma unroll
    for (int k = 0; k < kD * 16 / 256; ++k) {
      const int p = min(tid + 256 * k, r * 16 - 1);
      uu[k] = *reinterpret_cast<const u32x4 *>(ut + (p >> 4) * urow + j * kD + (p & 15) * 8);
    }
    if (j > 0) __syncthreads();  // every wave is done with slice j - 1
#pragma unroll
    for (int k = 0; k < kD * 16 / 256; ++k) {
      const int p = tid + 256 * k;
      if (p < r * 16) *reinterpret_cast<u32x4 *>(&su[(p >> 4) * kUStride + (p & 15) * 8]) = uu[k];
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < kD / 16; ++nt) {
      if (nt < ntr) {
        u32x4 uo[4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          uo[kc] = *reinterpret_cast<const u32x4 *>(&su[(16 * nt + t16) * kUStride + 32 * kc + 8 * q4]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          if (which == 0) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) acc[nt][tt] = mfma16x16x32(uo[kc], xo[tt][kc], acc[nt][tt]);
          } else {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) acc[nt][tt] = mfma16x16x32(xo[tt][kc], uo[kc], acc[nt][tt]);
          }
        }
      }
    }
  }
  if (t_base >= n_tok) return;  // no barrier follows

  // keys: lane (q4, t16) holds columns 16 nt + 4 q4 + v of token t16; values:
  // tokens 4 q4 + v of column 16 nt + t16 (as in k_compress_mfma)
  float sc[2][4] = {};
  if constexpr (QMAX > 0) {
    float *scales = (which ? L.scales_v : L.scales_k) + scale_index(L, h, b, 0);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float am[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < kD / 16; ++nt)
        if (nt < ntr)
#pragma unroll
          for (int v = 0; v < 4; ++v) am[v] = fmaxf(am[v], fabsf(acc[nt][tt][v]));
      if (which == 0) {
        float a = fmaxf(fmaxf(am[0], am[1]), fmaxf(am[2], am[3]));
        a = fmaxf(a, __shfl_xor(a, 16, 64));
        a = fmaxf(a, __shfl_xor(a, 32, 64));
        sc[tt][0] = sc[tt][1] = sc[tt][2] = sc[tt][3] = qn_scale<QMAX>(a);
        const int tok = t_base + 16 * tt + t16;
        if (q4 == 0 && tok < n_tok) scales[slot0 + tok] = sc[tt][0];
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float a = am[v];
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
          sc[tt][v] = qn_scale<QMAX>(a);
          const int tok = t_base + 16 * tt + 4 * q4 + v;
          if (t16 == 0 && tok < n_tok) scales[slot0 + tok] = sc[tt][v];
        }
      }
    }
  }
  // 4 consecutive elements from position p (a multiple of 4), or one element at
  // p: bf16, int8 or 4-bit, quantised with the scales sc
  char *base = static_cast<char *>(which ? L.codes_v : L.codes_k);
  auto store4 = [&](int64_t p, f32x4 v, float s0, float s1, float s2, float s3) {
    if constexpr (QMAX == 0) {
      uint2 v2;
      v2.x = pack_rne(v[0], v[1]);
      v2.y = pack_rne(v[2], v[3]);
      *reinterpret_cast<uint2 *>(reinterpret_cast<bf16_t *>(base) + region + p) = v2;
    } else if constexpr (QMAX == 127) {
      *reinterpret_cast<uint32_t *>(base + region + p) = pack_qn<QMAX>(v, s0, s1, s2, s3);
    } else {
      *reinterpret_cast<uint16_t *>(base + (region + p) / 2) = uint16_t(pack_qn<QMAX>(v, s0, s1, s2, s3));
    }
  };
  auto store1 = [&](int64_t p, float val, float s) {
    if constexpr (QMAX == 0) reinterpret_cast<bf16_t *>(base)[region + p] = from_f32<bf16_t>(val);
    else if constexpr (QMAX == 127) reinterpret_cast<int8_t *>(base)[region + p] = int8_t(qn_value<QMAX>(val, s));
    else store_q4(reinterpret_cast<uint8_t *>(base) + region / 2, p, qn_value<QMAX>(val, s));
  };
#pragma unroll
  for (int nt = 0; nt < kD / 16; ++nt) {
    if (nt < ntr) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const f32x4 a = acc[nt][tt];
        if (which == 0) {  // 4 consecutive columns of one token: contiguous
          const int tok = t_base + 16 * tt + t16;
          if (tok < n_tok) store4(kslot(slot0 + tok, 16 * nt + 4 * q4, r), a, sc[tt][0], sc[tt][0], sc[tt][0], sc[tt][0]);
        } else {  // 4 tokens of one column: contiguous when 4-aligned and present
          const int tok0 = t_base + 16 * tt + 4 * q4;
          const int j0 = slot0 + tok0, col = 16 * nt + t16;
          if (tok0 + 3 < n_tok && (j0 & 3) == 0) {
            store4(vslot(j0, col, r), a, sc[tt][0], sc[tt][1], sc[tt][2], sc[tt][3]);
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (tok0 + v < n_tok) store1(vslot(j0 + v, col, r), a[v], sc[tt][v]);
          }
        }
      }
    }
  }
}

hipError_t launch_compress_mfma(const LayerArgs &L, int which, const void *x, int64_t sb,
                                int64_t sh, int64_t st, int n_tok, int slot0, hipStream_t s) {
  dim3 grid((n_tok + 127) / 128, L.batch * L.n_lat);
  const bf16_t *xb = static_cast<const bf16_t *>(x);
  if (L.hg > 1) {
    if (L.dtype == LRKV_BF16_Q8)
      hipLaunchKernelGGL(k_compress_group<127>, grid, dim3(256), 0, s, L, which, xb, sb, sh, st, n_tok, slot0);
    else if (L.dtype == LRKV_BF16_Q4)
      hipLaunchKernelGGL(k_compress_group<7>, grid, dim3(256), 0, s, L, which, xb, sb, sh, st, n_tok, slot0);
    else
      hipLaunchKernelGGL(k_compress_group<0>, grid, dim3(256), 0, s, L, which, xb, sb, sh, st, n_tok, slot0);
  } else if (L.dtype == LRKV_BF16_Q8)
    hipLaunchKernelGGL(k_compress_mfma<127>, grid, dim3(256), 0, s, L, which, xb, sb, sh, st, n_tok, slot0);
  else if (L.dtype == LRKV_BF16_Q4)
    hipLaunchKernelGGL(k_compress_mfma<7>, grid, dim3(256), 0, s, L, which, xb, sb, sh, st, n_tok, slot0);
  else
    hipLaunchKernelGGL(k_compress_mfma<0>, grid, dim3(256), 0, s, L, which, xb, sb, sh, st, n_tok, slot0);
  return hipGetLastError();
}

}  // namespace lrkv
