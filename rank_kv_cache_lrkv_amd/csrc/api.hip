// C entry points: argument checks on the host (before any HIP call), layout
// offsets, then the launches.  No device memory is allocated here.

#include <algorithm>
#include <cmath>
#include <cstring>

#include "lrkv_internal.h"

using namespace lrkv;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_rank(int32_t r) { return r >= 16 && r <= 128 && r % 16 == 0; }
int elem_bytes(int32_t dtype) { return dtype == LRKV_F32 ? 4 : 2; }
bool quantised(int32_t dtype) { return dtype == LRKV_BF16_Q8 || dtype == LRKV_BF16_Q4; }

// Checks the layer description and fills the kernel-side copy.
lrkv_status make_layer(const lrkv_layer *L, LayerArgs *A) {
  if (!L) return LRKV_ERR_NULL;
  if (L->dtype != LRKV_F32 && L->dtype != LRKV_BF16 && L->dtype != LRKV_BF16_Q8 &&
      L->dtype != LRKV_BF16_Q4)
    return LRKV_ERR_DTYPE;
  if (L->batch < 1 || L->n_kv_heads < 1 || L->n_kv_heads > LRKV_MAX_KV_HEADS) return LRKV_ERR_SHAPE;
  // (row, head) units are the second launch dimension
  if (int64_t(L->batch) * L->n_kv_heads > 65535) return LRKV_ERR_SHAPE;
  if (L->n_q_heads < L->n_kv_heads || L->n_q_heads % L->n_kv_heads) return LRKV_ERR_SHAPE;
  if (L->n_q_heads / L->n_kv_heads > LRKV_MAX_GROUP) return LRKV_ERR_SHAPE;
  if (L->window < 0 || L->cap < 0 || L->cap % LRKV_BLOCK) return LRKV_ERR_SHAPE;
  // one (row, head) code region is addressed with 32-bit byte offsets
  if (int64_t(L->cap) * kD * elem_bytes(L->dtype) > INT32_MAX) return LRKV_ERR_SHAPE;
  if (L->value_mode != LRKV_VALUES_CODES && L->value_mode != LRKV_VALUES_LOWRAM) return LRKV_ERR_DTYPE;
  const bool lr = L->value_mode == LRKV_VALUES_LOWRAM;  // no value codes
  if (!L->rank_k || !L->rank_v || !L->bases || !L->codes_k || (!lr && !L->codes_v) || !L->anchor_k ||
      !L->anchor_v)
    return LRKV_ERR_NULL;
  if (!aligned16(L->bases) || !aligned16(L->codes_k) || (!lr && !aligned16(L->codes_v)) ||
      !aligned16(L->anchor_k) || !aligned16(L->anchor_v))
    return LRKV_ERR_ALIGN;
  const int32_t nver = L->n_versions == 0 ? 1 : L->n_versions;
  if (nver < 1 || nver > LRKV_MAX_VERSIONS) return LRKV_ERR_SHAPE;
  if (nver > 1 && L->dtype == LRKV_F32) return LRKV_ERR_DTYPE;
  if (nver > 1 && !L->version_start) return LRKV_ERR_NULL;
  if (nver > 1 && (reinterpret_cast<uintptr_t>(L->version_start) & 3u)) return LRKV_ERR_ALIGN;
  const int32_t hg = L->head_group <= 1 ? 1 : L->head_group;
  if (hg > LRKV_MAX_HEAD_GROUP || L->n_kv_heads % hg) return LRKV_ERR_SHAPE;
  if (hg > 1 && int64_t(hg) * (L->n_q_heads / L->n_kv_heads) > LRKV_MAX_GROUP) return LRKV_ERR_SHAPE;
  if (hg > 1 && L->dtype == LRKV_F32) return LRKV_ERR_DTYPE;
  if (quantised(L->dtype)) {
    if (!L->scales_k || !L->scales_v) return LRKV_ERR_NULL;
    if (!aligned16(L->scales_k) || !aligned16(L->scales_v)) return LRKV_ERR_ALIGN;
  }
  if (L->rope_base != 0.f) {
    if (!(L->rope_base > 1.f) || !(L->rope_base < 3.0e38f)) return LRKV_ERR_SHAPE;
    if (L->dtype != LRKV_BF16 || nver > 1 || hg > 1 || lr) return LRKV_ERR_DTYPE;
  }
  if (lr) {
    if (L->dtype != LRKV_BF16 || nver > 1 || hg > 1) return LRKV_ERR_DTYPE;
    if (L->resid_per_block < 1 || L->resid_per_block > LRKV_MAX_RESID) return LRKV_ERR_SHAPE;
    if (!L->predictor || !L->resid || !L->resid_slot || !L->resid_norm) return LRKV_ERR_NULL;
    if (!aligned16(L->predictor) || !aligned16(L->resid) || !aligned16(L->resid_slot) ||
        !aligned16(L->resid_norm))
      return LRKV_ERR_ALIGN;
  }
  std::memset(A, 0, sizeof(*A));
  A->dtype = L->dtype;
  A->batch = L->batch;
  A->n_q = L->n_q_heads;
  A->n_kv = L->n_kv_heads;
  A->group = L->n_q_heads / L->n_kv_heads;
  A->hg = hg;
  A->n_lat = L->n_kv_heads / hg;
  A->window = L->window;
  A->cap = L->cap;
  A->bases = L->bases;
  A->codes_k = L->codes_k;
  A->codes_v = L->codes_v;
  A->anchor_k = L->anchor_k;
  A->anchor_v = L->anchor_v;
  A->scales_k = quantised(L->dtype) ? L->scales_k : nullptr;
  A->scales_v = quantised(L->dtype) ? L->scales_v : nullptr;
  int64_t ub = 0, ck = 0, cv = 0, pr = 0;
  int rv_max = 0;
  for (int h = 0; h < A->n_lat; ++h) {
    const int32_t rk = L->rank_k[h], rv = L->rank_v[h];
    if (!valid_rank(rk) || !valid_rank(rv)) return LRKV_ERR_RANK;
    HeadInfo &hd = A->heads[h];
    hd.rk = rk;
    hd.rv = lr ? rk : rv;  // LowRAM value sums run over the key codes
    hd.pred = pr;
    pr += int64_t(L->batch) * rk * kD;
    hd.u_k = int32_t(ub);
    hd.u_v = int32_t(ub + int64_t(hg) * kD * rk);
    hd.ck = ck;
    hd.cv = cv;
    ub += int64_t(hg) * kD * (rk + rv);
    ck += int64_t(L->batch) * L->cap * rk;
    cv += int64_t(L->batch) * L->cap * rv;
    rv_max = hd.rv > rv_max ? hd.rv : rv_max;
  }
  A->rv_max = rv_max;
  A->n_versions = nver;
  A->vstart = nver > 1 ? L->version_start : nullptr;
  A->version_elems = ub;
  if (L->rope_base != 0.f) {
    // theta_i / (2 pi) with theta_i = base^(-2 i / 128): one pow, then a running
    // product in double (relative error ~1e-14, far below float32), so a decode
    // call spends well under a microsecond here
    A->rope = 1;
    const double step = std::pow(double(L->rope_base), -2.0 / kD);
    double theta = 1.0;
    for (int i = 0; i < kD / 2; ++i, theta *= step) {
      const double a = theta / (2.0 * 3.14159265358979323846);
      A->rope_a[i][0] = float(a);
      A->rope_a[i][1] = float(a - double(float(a)));
    }
  }
  if (lr) {
    A->lowram = 1;
    A->R = L->resid_per_block;
    A->pred = L->predictor;
    A->resid = L->resid;
    A->rslot = L->resid_slot;
    A->rnorm = L->resid_norm;
  }
  return LRKV_OK;
}

int32_t rvp_floats(const LayerArgs &A) { return ((A.rv_max + 3) / 4) * 4; }
int32_t rec_floats(const LayerArgs &A) { return 4 + rvp_floats(A) + kD; }

// code bytes per compressed token of latent group h (codes, scales, LowRAM
// residual records): what one of its splits streams per token
double token_bytes(const LayerArgs &A, int h) {
  const HeadInfo &hd = A.heads[h];
  if (A.lowram) return hd.rk * 2.0 + A.R * (kD * 2.0 + 4.0) / kBlock;
  switch (A.dtype) {
    case LRKV_F32: return (hd.rk + hd.rv) * 4.0;
    case LRKV_BF16: return (hd.rk + hd.rv) * 2.0;
    case LRKV_BF16_Q8: return (hd.rk + hd.rv) + 8.0;
    default: return (hd.rk + hd.rv) * 0.5 + 8.0;
  }
}

// S_h of every group for S splits of the widest group: in proportion to the
// group's bytes per token, rounded, at least the basis versions (and 1)
void group_splits(const LayerArgs &A, int32_t S, int32_t *nsplit) {
  double wmax = 0.0;
  for (int h = 0; h < A.n_lat; ++h) wmax = std::max(wmax, token_bytes(A, h));
  for (int h = 0; h < A.n_lat; ++h) {
    int64_t sh = std::llround(double(S) * token_bytes(A, h) / wmax);
    sh = std::max<int64_t>(sh, A.n_versions);
    sh = std::max<int64_t>(sh, 1);
    nsplit[h] = int32_t(std::min<int64_t>(sh, S));
  }
}

int32_t auto_splits(const LayerArgs &A, int32_t n_ctx) {
  const int64_t c = n_ctx - 1 - A.window;
  const int64_t nblk = c > 0 ? (c + LRKV_BLOCK - 1) / LRKV_BLOCK : 0;
  // about as many workgroups as the launched kernel keeps resident at once on
  // the device (its occupancy per compute unit times the compute units); without
  // a device to ask, the figures of MI355X (256 compute units, four workgroups
  // per unit, three for the LowRAM kernels and the narrower pre-RoPE ones).  The groups' splits
  // follow their bytes per token, so the widest group's count is scaled by
  // (widest bytes) / (mean bytes).  At least sixteen 32-slot blocks per split
  // on the matrix-core kernels (four per wave: with fewer, the per-workgroup setup
  // outweighs the streaming it starts), four on the float32 one.
  const int per_cu = partials_blocks_per_cu(A), cus = device_cu_count();
  const int64_t target = (per_cu > 0 && cus > 0) ? int64_t(per_cu) * cus : ((A.rope || A.lowram) ? 768 : 1024);
  double wsum = 0.0, wmax = 0.0;
  for (int h = 0; h < A.n_lat; ++h) {
    wsum += token_bytes(A, h);
    wmax = std::max(wmax, token_bytes(A, h));
  }
  int64_t s = int64_t(std::floor(double(target) * wmax / (double(A.batch) * wsum) + 1e-9));
  const int64_t min_blocks = A.dtype == LRKV_F32 ? 4 : 16;
  const int64_t most = std::max<int64_t>(1, (nblk + min_blocks / 2) / min_blocks);
  if (s > most) s = most;
  if (s < 1) s = 1;
  if (s > LRKV_MAX_SPLITS) s = LRKV_MAX_SPLITS;
  // the groups' rounded split counts must not add up to more workgroups than are
  // resident at once: a second, nearly empty round would double the tail
  int32_t ns[LRKV_MAX_KV_HEADS];
  while (s > 1) {
    group_splits(A, int32_t(s), ns);
    int64_t items = 0;
    for (int h = 0; h < A.n_lat; ++h) items += ns[h];
    if (items * A.batch <= target) break;
    --s;
  }
  if (s < A.n_versions) s = A.n_versions;  // every basis version needs a split
  return int32_t(s);
}

size_t ws_bytes(const LayerArgs &A, int32_t S) {
  const size_t rows = size_t(A.batch) * A.n_q;
  return rows * S * rec_floats(A) * sizeof(float);
}

lrkv_status check_strides(const lrkv_layer *L, const void *x, int64_t sb, int64_t sh, int64_t st) {
  if (sb < 0 || sh < 0 || st < 0) return LRKV_ERR_SHAPE;
  const int64_t eb = elem_bytes(L->dtype);
  if (!aligned16(x) || (sb * eb) % 16 || (sh * eb) % 16 || (st * eb) % 16) return LRKV_ERR_ALIGN;
  return LRKV_OK;
}

// Builds the decode arguments; shared by the three decode entry points.
lrkv_status make_decode(const lrkv_layer *L, const LayerArgs &A, int32_t n_ctx,
                        const int32_t *ctx_lens, const void *q, float sm_scale, int32_t n_splits,
                        void *ws, size_t ws_len, DecodeArgs *D) {
  if (n_ctx < 1) return LRKV_ERR_SHAPE;
  const int64_t c = int64_t(n_ctx) - 1 - A.window;
  if (c > A.cap) return LRKV_ERR_CAPACITY;
  if (n_splits < 0 || n_splits > LRKV_MAX_SPLITS) return LRKV_ERR_SHAPE;
  if (!(sm_scale > 0.f) || sm_scale != sm_scale) return LRKV_ERR_SHAPE;
  const int32_t S = n_splits ? n_splits : auto_splits(A, n_ctx);
  if (S < A.n_versions) return LRKV_ERR_SHAPE;
  if (!ws) return LRKV_ERR_WORKSPACE;
  if (ws_len < ws_bytes(A, S)) return LRKV_ERR_WORKSPACE;
  if (!aligned16(ws) || (ctx_lens && (reinterpret_cast<uintptr_t>(ctx_lens) & 3u)))
    return LRKV_ERR_ALIGN;
  if (q && !aligned16(q)) return LRKV_ERR_ALIGN;
  (void)L;
  std::memset(D, 0, sizeof(*D));
  D->n_ctx = n_ctx;
  D->n_splits = S;
  group_splits(A, S, D->nsplit);
  D->uniform = 1;
  int32_t acc = 0;
  for (int h = 0; h < A.n_lat; ++h) {
    D->split0[h] = acc;
    acc += D->nsplit[h];
    D->uniform = D->uniform && D->nsplit[h] == S;
  }
  D->split0[A.n_lat] = acc;
  D->row_items = acc;
  D->items = acc * A.batch;
  D->rec = rec_floats(A);
  D->oa = 4 + rvp_floats(A);
  D->scale_log2 = sm_scale * kLog2e;
  D->ctx_lens = ctx_lens;
  D->q = q;
  D->ws = static_cast<float *>(ws);
  return LRKV_OK;
}

lrkv_status hip_status(hipError_t e) { return e == hipSuccess ? LRKV_OK : LRKV_ERR_HIP; }

}  // namespace

extern "C" {

lrkv_status lrkv_compress(const lrkv_layer *L, int32_t which, const void *x, int64_t stride_b,
                          int64_t stride_h, int64_t stride_t, int32_t n_tok, int32_t slot0,
                          lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (which != 0 && which != 1) return LRKV_ERR_SHAPE;
  if (which == 1 && A.lowram) return LRKV_ERR_DTYPE;  // no value codes
  if (n_tok < 0 || slot0 < 0) return LRKV_ERR_SHAPE;
  if (int64_t(slot0) + n_tok > L->cap) return LRKV_ERR_CAPACITY;
  if (n_tok == 0) return LRKV_OK;
  if (!x) return LRKV_ERR_NULL;
  st = check_strides(L, x, stride_b, stride_h, stride_t);
  if (st != LRKV_OK) return st;
  return hip_status(launch_compress(A, which, x, stride_b, stride_h, stride_t, n_tok, slot0,
                                    reinterpret_cast<hipStream_t>(stream)));
}

lrkv_status lrkv_quantize(const lrkv_layer *L, int32_t which, const float *x, int64_t stride_b,
                          int64_t stride_h, int64_t stride_t, int32_t n_tok, int32_t slot0,
                          lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (!quantised(L->dtype)) return LRKV_ERR_DTYPE;
  if (which != 0 && which != 1) return LRKV_ERR_SHAPE;
  if (n_tok < 0 || slot0 < 0) return LRKV_ERR_SHAPE;
  if (int64_t(slot0) + n_tok > L->cap) return LRKV_ERR_CAPACITY;
  if (n_tok == 0) return LRKV_OK;
  if (!x) return LRKV_ERR_NULL;
  if (stride_b < 0 || stride_h < 0 || stride_t < 0) return LRKV_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(x) & 3u) return LRKV_ERR_ALIGN;
  return hip_status(launch_quantize(A, which, x, stride_b, stride_h, stride_t, n_tok, slot0,
                                    reinterpret_cast<hipStream_t>(stream)));
}

size_t lrkv_oja_workspace_size(const lrkv_layer *L) {
  LayerArgs A;
  if (make_layer(L, &A) != LRKV_OK) return 0;
  return oja_workspace_bytes(A);
}

lrkv_status lrkv_oja_update(const lrkv_layer *L, int32_t which, const void *x, int64_t stride_b,
                            int64_t stride_h, int64_t stride_t, int32_t n_tok, float eta,
                            int32_t version_in, int32_t version_out, void *workspace,
                            size_t workspace_bytes, lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (L->dtype == LRKV_F32) return LRKV_ERR_DTYPE;
  if (A.hg != 1) return LRKV_ERR_SHAPE;  // the step is per KV head
  if (which != 0 && which != 1) return LRKV_ERR_SHAPE;
  if (n_tok < 1 || !(eta == eta) || eta > 3.4e38f || eta < -3.4e38f) return LRKV_ERR_SHAPE;
  if (version_in < 0 || version_in >= A.n_versions || version_out < 0 || version_out >= A.n_versions)
    return LRKV_ERR_SHAPE;
  if (!x) return LRKV_ERR_NULL;
  st = check_strides(L, x, stride_b, stride_h, stride_t);
  if (st != LRKV_OK) return st;
  if (!workspace || workspace_bytes < oja_workspace_bytes(A)) return LRKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LRKV_ERR_ALIGN;
  return hip_status(launch_oja(A, which, x, stride_b, stride_h, stride_t, n_tok, eta, version_in,
                               version_out, static_cast<float *>(workspace),
                               reinterpret_cast<hipStream_t>(stream)));
}

size_t lrkv_lowram_workspace_size(const lrkv_layer *L) {
  LayerArgs A;
  if (make_layer(L, &A) != LRKV_OK || !A.lowram) return 0;
  return lowram_workspace_bytes(A);
}

lrkv_status lrkv_lowram_fit(const lrkv_layer *L, const void *v, int64_t stride_b, int64_t stride_h,
                            int64_t stride_t, int32_t n_tok, void *workspace, size_t workspace_bytes,
                            lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (!A.lowram) return LRKV_ERR_DTYPE;
  if (n_tok < 1) return LRKV_ERR_SHAPE;
  if (n_tok > L->cap) return LRKV_ERR_CAPACITY;
  if (!v) return LRKV_ERR_NULL;
  st = check_strides(L, v, stride_b, stride_h, stride_t);
  if (st != LRKV_OK) return st;
  if (!workspace || workspace_bytes < lowram_workspace_bytes(A)) return LRKV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LRKV_ERR_ALIGN;
  return hip_status(launch_lowram_fit(A, static_cast<const bf16_t *>(v), stride_b, stride_h, stride_t, n_tok,
                                      static_cast<float *>(workspace), reinterpret_cast<hipStream_t>(stream)));
}

lrkv_status lrkv_store_anchors(const lrkv_layer *L, const void *k, const void *v, int64_t stride_b,
                               int64_t stride_h, int64_t stride_t, int32_t pos0, int32_t n_tok,
                               lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (n_tok < 0 || pos0 < 0) return LRKV_ERR_SHAPE;
  const int64_t most = pos0 == 0 ? int64_t(1) + L->window : L->window;
  if (n_tok > most) return LRKV_ERR_SHAPE;
  if (n_tok == 0) return LRKV_OK;
  if (!k || !v) return LRKV_ERR_NULL;
  st = check_strides(L, k, stride_b, stride_h, stride_t);
  if (st == LRKV_OK) st = check_strides(L, v, stride_b, stride_h, stride_t);
  if (st != LRKV_OK) return st;
  return hip_status(launch_store_anchors(A, k, v, stride_b, stride_h, stride_t, pos0, n_tok,
                                         reinterpret_cast<hipStream_t>(stream)));
}

lrkv_status lrkv_append(const lrkv_layer *L, const void *k_new, const void *v_new, int32_t pos,
                        lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (pos < 0) return LRKV_ERR_SHAPE;
  if (!k_new || !v_new) return LRKV_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return LRKV_ERR_ALIGN;
  const int64_t code_slot = L->window >= 1 ? int64_t(pos) - L->window - 1 : int64_t(pos) - 1;
  if (code_slot >= L->cap) return LRKV_ERR_CAPACITY;
  return hip_status(launch_append(A, k_new, v_new, pos, reinterpret_cast<hipStream_t>(stream)));
}

size_t lrkv_decode_workspace_size(const lrkv_layer *L, int32_t n_splits) {
  LayerArgs A;
  if (make_layer(L, &A) != LRKV_OK) return 0;
  if (n_splits < 1 || n_splits > LRKV_MAX_SPLITS) return 0;
  return ws_bytes(A, n_splits);
}

int32_t lrkv_decode_auto_splits(const lrkv_layer *L, int32_t n_ctx) {
  LayerArgs A;
  if (make_layer(L, &A) != LRKV_OK || n_ctx < 1) return 0;
  return auto_splits(A, n_ctx);
}

lrkv_status lrkv_decode_partials(const lrkv_layer *L, int32_t n_ctx, const int32_t *ctx_lens,
                                 const void *q, float sm_scale, int32_t n_splits, void *workspace,
                                 size_t workspace_bytes, lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (!q) return LRKV_ERR_NULL;
  DecodeArgs D;
  st = make_decode(L, A, n_ctx, ctx_lens, q, sm_scale, n_splits, workspace, workspace_bytes, &D);
  if (st != LRKV_OK) return st;
  return hip_status(launch_decode_partials(A, D, reinterpret_cast<hipStream_t>(stream)));
}

lrkv_status lrkv_decode_combine(const lrkv_layer *L, int32_t n_ctx, const int32_t *ctx_lens,
                                int32_t n_splits, const void *workspace, size_t workspace_bytes,
                                float *out, lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (!out) return LRKV_ERR_NULL;
  if (!aligned16(out)) return LRKV_ERR_ALIGN;
  if (n_splits < 1 || n_splits > LRKV_MAX_SPLITS) return LRKV_ERR_SHAPE;
  DecodeArgs D;
  st = make_decode(L, A, n_ctx, ctx_lens, nullptr, 1.f, n_splits, const_cast<void *>(workspace),
                   workspace_bytes, &D);
  if (st != LRKV_OK) return st;
  return hip_status(launch_decode_combine(A, D, out, reinterpret_cast<hipStream_t>(stream)));
}

lrkv_status lrkv_decode_attn(const lrkv_layer *L, int32_t n_ctx, const int32_t *ctx_lens,
                             const void *q, float *out, float sm_scale, int32_t n_splits,
                             void *workspace, size_t workspace_bytes, lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (!q || !out) return LRKV_ERR_NULL;
  if (!aligned16(out)) return LRKV_ERR_ALIGN;
  DecodeArgs D;
  st = make_decode(L, A, n_ctx, ctx_lens, q, sm_scale, n_splits, workspace, workspace_bytes, &D);
  if (st != LRKV_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = hip_status(launch_decode_partials(A, D, s));
  if (st != LRKV_OK) return st;
  return hip_status(launch_decode_combine(A, D, out, s));
}

lrkv_status lrkv_decode_attn_noalloc(const lrkv_layer *L, int32_t n_ctx, const int32_t *ctx_lens,
                                     const void *q, float *out, float sm_scale, int32_t n_splits,
                                     lrkv_stream_t stream) {
  LayerArgs A;
  lrkv_status st = make_layer(L, &A);
  if (st != LRKV_OK) return st;
  if (!q || !out) return LRKV_ERR_NULL;
  if (!aligned16(out)) return LRKV_ERR_ALIGN;
  // every check first, with a stand-in for the array's address: the records of
  // this call must fit in it (LRKV_ERR_WORKSPACE otherwise)
  DecodeArgs D;
  st = make_decode(L, A, n_ctx, ctx_lens, q, sm_scale, n_splits, reinterpret_cast<void *>(uintptr_t(256)),
                   noalloc_scratch_bytes(), &D);
  if (st != LRKV_OK) return st;
  return decode_attn_noalloc(A, D, out, reinterpret_cast<hipStream_t>(stream));
}

const char *lrkv_status_string(lrkv_status s) {
  switch (s) {
    case LRKV_OK: return "ok";
    case LRKV_ERR_NULL: return "a required pointer is NULL";
    case LRKV_ERR_SHAPE: return "a size, count, position or stride is out of range";
    case LRKV_ERR_RANK: return "a rank is not a multiple of 16 in [16, 128]";
    case LRKV_ERR_DTYPE: return "unknown storage type";
    case LRKV_ERR_ALIGN: return "a device pointer or stride is not 16-byte aligned";
    case LRKV_ERR_CAPACITY: return "the code slots needed exceed the capacity";
    case LRKV_ERR_WORKSPACE: return "workspace missing or too small";
    case LRKV_ERR_HIP: return "a HIP kernel launch failed";
  }
  return "unknown status";
}

int32_t lrkv_version(void) { return 100; }

}  // extern "C"
