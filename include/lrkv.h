/*
 * lrkv.h - decode attention read directly from a low-rank-compressed KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The method.  Per (layer, KV head) the keys (taken after RoPE) and the values
 * are stored as r-dim codes under fixed bases with orthonormal columns,
 * C_K = K U_K and C_V = V U_V (blog "Half the Memory, None of the Answers Lost",
 * section 04).  The first token and the most recent `window` tokens stay at full
 * rank as anchors (OjaKV article, FAQ on which tokens are compressed).  A decode
 * step scores the codes in code space with the projected query q~ = U_K^T q, the
 * anchors with q itself, runs one softmax over both, sums the values of the codes
 * in the r_v-dim code space and up-projects that sum once (blog section 08: the
 * compressed form is algebraically the attention over the reconstructed cache,
 * so the full tensors are never rebuilt).
 *
 * Conventions for every entry point:
 *  - head_dim is fixed at 128.  Query head i reads KV head i / g, g = n_q_heads / n_kv_heads.
 *  - All tensors are caller-owned.  The library allocates no device memory and keeps
 *    no per-call state; device pointers are plain HIP device addresses.
 *  - Every argument is checked on the host before any HIP call; on an error
 *    nothing is launched and no buffer is touched.  Launch failures return
 *    LRKV_ERR_HIP; faults inside a kernel surface at the caller's next stream sync.
 *  - Work is enqueued on `stream` (0 = the null stream) and returns at once.
 *    Calls on different streams that write the same buffers race.
 *  - Device pointers must be 16-byte aligned.
 */
#ifndef LRKV_H
#define LRKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *lrkv_stream_t; /* same object as hipStream_t */

typedef enum lrkv_status {
  LRKV_OK = 0,
  LRKV_ERR_NULL = 1,      /* a required pointer is NULL */
  LRKV_ERR_SHAPE = 2,     /* a size, count, position or stride is out of range */
  LRKV_ERR_RANK = 3,      /* a rank is not a multiple of 16 in [16, 128] */
  LRKV_ERR_DTYPE = 4,     /* unknown storage type */
  LRKV_ERR_ALIGN = 5,     /* a device pointer or row stride is not 16-byte aligned */
  LRKV_ERR_CAPACITY = 6,  /* the code slots needed exceed `cap` */
  LRKV_ERR_WORKSPACE = 7, /* workspace missing or smaller than lrkv_decode_workspace_size */
  LRKV_ERR_HIP = 8        /* a kernel launch failed */
} lrkv_status;

typedef enum lrkv_dtype {
  LRKV_F32 = 0,     /* float32 storage and float32 arithmetic */
  LRKV_BF16 = 1,    /* bfloat16 storage, float32 accumulation */
  LRKV_BF16_Q8 = 2, /* bfloat16 bases, anchors, queries and compress/append inputs;
                       int8 codes with one float32 scale per code slot (see below) */
  LRKV_BF16_Q4 = 3  /* as LRKV_BF16_Q8 with 4-bit codes, two per byte (see below) */
} lrkv_dtype;

#define LRKV_HEAD_DIM 128
#define LRKV_BLOCK 32         /* code slots per layout block */
#define LRKV_MAX_KV_HEADS 64  /* per layer */
#define LRKV_MAX_GROUP 16     /* query heads per KV head */
#define LRKV_MAX_SPLITS 1024
#define LRKV_MAX_VERSIONS 16  /* basis versions per layer */
#define LRKV_MAX_HEAD_GROUP 8 /* KV heads sharing one code stream */
#define LRKV_MAX_RESID 8      /* LowRAM residual rows kept per 32-slot block */

typedef enum lrkv_value_mode {
  LRKV_VALUES_CODES = 0,  /* values stored as codes C_V = V U_V */
  LRKV_VALUES_LOWRAM = 1  /* values predicted from the key codes, with residuals (see below) */
} lrkv_value_mode;

/*
 * One layer of compressed cache.  Storage type `dtype` applies to the bases, the
 * codes, the anchors, the queries and the compress/append inputs; the decode
 * output is always float32.
 *
 * rank_k[h], rank_v[h] (host arrays of n_kv_heads): multiples of 16 in [16, 128].
 *
 * bases (device): the heads in order; head h holds the rank_k[h] key basis
 *   directions (the columns of U_K(h)) as rows of 128 contiguous elements, i.e.
 *   U_K(h)^T as [rank_k[h]][128], and right after it U_V(h)^T as [rank_v[h]][128];
 *   U_K(h) starts at element 128 * sum_{h' < h} (rank_k[h'] + rank_v[h']).  A code
 *   is x U: column c of a code is the dot product of x with basis row c.
 *   With basis versions (n_versions > 1, see below) `bases` holds n_versions
 *   copies of this layout back to back: version v starts at element
 *   v * 128 * sum_h (rank_k[h] + rank_v[h]).
 *
 * codes_k, codes_v (device): the heads in order; head h owns `batch * cap * r`
 *   elements (r = rank_k[h] resp. rank_v[h]), starting at element
 *   batch * cap * sum_{h' < h} r(h').  Inside, batch row b owns cap * r elements
 *   (cap a multiple of 32), grouped in blocks of 32 slots (32 * r elements each).
 *   Code slot j holds token j + 1 (the tokens between the first one and the
 *   window).  Slot j lives in block j / 32 at in-block position t = j % 32, and
 *   column c of its code sits at in-block element
 *     keys:   ((t / 16) * (r / 8) + c / 8) * 128 + (t % 16) * 8 + c % 8
 *     values: ((t % 16) / 4 * r + c) * 8 + 4 * (t / 16) + t % 4
 *   i.e. 8 consecutive columns of 16 tokens (keys), or 8 tokens of one column
 *   (values), are 8 consecutive elements: the order the matrix cores consume.
 *
 * anchor_k, anchor_v (device): [batch][n_kv_heads][1 + window][128].  Slot 0 is
 *   token 0; a token p >= 1 inside the window sits in slot 1 + (p - 1) % window.
 *   At context n the valid slots are the prefix [0, min(n, 1 + window)).
 *
 * Int8 codes (dtype LRKV_BF16_Q8).  The pages pair low-rank caches with
 * quantisation (LowRAM and Palu abstracts) but fix no quantiser; this one is a
 * design choice.  A code row x (the float32 projection of one token, r columns)
 * is stored as q = x / s rounded to nearest even and clipped to [-127, 127], with
 * s = max_c |x_c| / 127, all in float32 (a zero row: s = 0, q = 0); the code it
 * stands for is s q.  codes_k / codes_v keep the blocked positions above with
 * one-byte elements; the scales are float32:
 *   scales_k, scales_v (device): slot j of batch row b, KV head h (latent group
 *   h with head groups) at element (h * batch + b) * cap + j.
 *
 * Group-head latents (head_group = n_g > 1; Palu abstract: a medium-grained
 * decomposition between one latent per head and one for all heads).  The n_g
 * consecutive KV heads of a group (g = h / n_g) share one code per token: the
 * projection of their concatenated rows [x_{g n_g}, ..., x_{g n_g + n_g - 1}]
 * (n_g * 128 features, head by head) onto one basis U(g) of n_g * 128 rows; KV
 * head h reads its 128-row slice (rows 128 (h % n_g) ..) of U(g).  Everything
 * "per head" above is then per group: rank_k / rank_v have n_kv_heads / n_g
 * entries, bases hold per group U_K(g)^T as [rank_k[g]][n_g * 128] then
 * U_V(g)^T, codes and scales regions are per group.  Anchors stay per KV head.
 * n_kv_heads must be a multiple of n_g, n_g * (n_q_heads / n_kv_heads) <=
 * LRKV_MAX_GROUP, n_g <= LRKV_MAX_HEAD_GROUP, and the storage is bf16 (or
 * quantised codes); lrkv_oja_update needs n_g = 1.  Errors: LRKV_ERR_SHAPE for
 * a group size that breaks these limits, LRKV_ERR_DTYPE for float32 storage.
 *
 * LowRAM value amortisation (value_mode = LRKV_VALUES_LOWRAM; LowRAM abstract:
 * inside a head the values are largely predictable from the keys, a light
 * per-head predictor is fitted at test time and residuals are kept only for the
 * worst-predicted tokens).  No value codes are stored.  Per (batch row b, KV
 * head h) a predictor M(b, h) of rank_k[h] x 128 maps key codes to values; the
 * value the decode reads for compressed token t is C_K[t] M + e_t, where e_t is
 * the residual row V_t - C_K[t] M kept for R = resid_per_block tokens of each
 * 32-slot block (those with the largest squared norm), and 0 for the others.
 * lrkv_lowram_fit fits M on the prompt and makes the residuals; lrkv_append
 * keeps them up to date.  codes_v and the U_V rows of `bases` are not read
 * (codes_v may be NULL; rank_v still lays out `bases`).  Buffers (nb = cap / 32
 * blocks per row):
 *   predictor  bf16, M(b, h) row c (128 values) at element
 *              (batch * P_h + b * rank_k[h] + c) * 128, P_h = sum of rank_k[h'] for h' < h;
 *   resid      bf16, entry i of block j of (h, b) at row ((h * batch + b) * nb + j) * R + i,
 *              128 elements per row;
 *   resid_slot int32, same entry index: the entry's slot inside its block (0 .. 31),
 *              or -1 for an empty entry;
 *   resid_norm float32, same entry index: the squared norm of the entry's residual
 *              (float32), which decides replacements.
 * Requires dtype LRKV_BF16, one basis version and head_group <= 1
 * (LRKV_ERR_DTYPE otherwise) and 1 <= R <= LRKV_MAX_RESID (LRKV_ERR_SHAPE).
 *
 * Keys compressed before RoPE (rope_base > 1; Palu abstract: the full keys are
 * reconstructed on the fly).  The key codes hold projections of the keys before
 * the rotary position embedding, so they cannot be scored in code space: the
 * decode reconstructs every compressed key (U_K c), rotates it to its position
 * (code slot j holds token j + 1) with rotate-half RoPE -- feature pair
 * (i, i + 64), i < 64, turned by position * rope_base^(-2 i / 128) -- and scores
 * it against q.  q, the anchors and the keys given to lrkv_store_anchors and
 * lrkv_append are post-RoPE (as attention uses them); lrkv_compress takes
 * pre-RoPE keys; values are never rotated.  Requires dtype LRKV_BF16, one basis
 * version, head_group <= 1 and value codes (LRKV_ERR_DTYPE otherwise); rope_base
 * must be finite and > 1 (LRKV_ERR_SHAPE).
 *
 * 4-bit codes (dtype LRKV_BF16_Q4): the same rule with 7 in place of 127
 * (s = max_c |x_c| / 7, q in [-7, 7]), the same scales.  Element position p of
 * the blocked layout above sits in byte p / 2 of the region, in the low four
 * bits for even p and the high four bits for odd p, two's complement; a
 * (row, head) region of r-column codes is cap * r / 2 bytes.
 */
typedef struct lrkv_layer {
  int32_t dtype;          /* lrkv_dtype */
  int32_t batch;          /* >= 1, batch * n_kv_heads <= 65535 */
  int32_t n_q_heads;      /* multiple of n_kv_heads, group <= LRKV_MAX_GROUP */
  int32_t n_kv_heads;     /* 1 .. LRKV_MAX_KV_HEADS */
  int32_t window;         /* W >= 0 recent tokens kept at full rank */
  int32_t cap;            /* code slots per (batch row, KV head); multiple of 32, >= 0,
                             cap * 128 * element size < 2^31 */
  const int32_t *rank_k;  /* host [n_kv_heads] */
  const int32_t *rank_v;  /* host [n_kv_heads] */
  const void *bases;      /* device, see above */
  void *codes_k;          /* device */
  void *codes_v;          /* device */
  void *anchor_k;         /* device [batch][n_kv_heads][1 + window][128] */
  void *anchor_v;         /* device */
  float *scales_k;        /* device, LRKV_BF16_Q8 and _Q4 only (may be NULL otherwise) */
  float *scales_v;        /* device, LRKV_BF16_Q8 and _Q4 only */
  int32_t n_versions;     /* basis versions held in `bases`, 1 .. LRKV_MAX_VERSIONS
                             (0 is read as 1; more than 1 needs bf16 bases:
                             LRKV_ERR_DTYPE for float32 layers) */
  const int32_t *version_start; /* device [batch][n_versions] when n_versions > 1 (else
                             ignored): the first code slot of each version in row b;
                             version 0 starts at 0, starts are multiples of 32 and
                             non-decreasing.  Code slot j of row b was made with the
                             last version whose start is <= j. */
  int32_t head_group;     /* KV heads sharing one code stream (Palu's group-head
                             latents, see below); 0 or 1: one per KV head */
  int32_t value_mode;     /* lrkv_value_mode (0: value codes) */
  int32_t resid_per_block;/* LowRAM: R, residual rows kept per 32-slot block */
  void *predictor;        /* LowRAM, device, see above (NULL otherwise) */
  void *resid;            /* LowRAM, device */
  int32_t *resid_slot;    /* LowRAM, device */
  float *resid_norm;      /* LowRAM, device */
  float rope_base;        /* 0: keys compressed after RoPE (scored in code space);
                             > 1: keys compressed before RoPE, see below */
} lrkv_layer;

/*
 * Prefill compression (blog section 04: one projection per (layer, head), keys
 * after RoPE).  For every (batch row b, KV head h) and t in [0, n_tok): code slot
 * slot0 + t of `which` (0 = keys with U_K, 1 = values with U_V) receives
 * x[b, h, t, :] U, rounded to the storage type (with head groups: group g's slot
 * receives the concatenated rows of its KV heads times U(g)) (bf16: round to nearest even of
 * the float32 accumulation; LRKV_BF16_Q8 / _Q4: the float32 accumulation
 * quantised to int8 / 4 bits with its scale, as described above).  With basis
 * versions the latest version (n_versions - 1) is used.
 *   x: device, element (b, h, t, i) at x + b*stride_b + h*stride_h + t*stride_t + i
 *      (strides in elements of the storage type; the 128 features contiguous).
 * Errors: LRKV_ERR_SHAPE if n_tok < 0, slot0 < 0 or a stride is negative;
 * LRKV_ERR_CAPACITY if slot0 + n_tok > cap; LRKV_ERR_ALIGN if x or a stride is
 * not 16-byte aligned; LRKV_ERR_DTYPE for which = 1 on a LowRAM layer (it has no
 * value codes).  n_tok == 0 is a no-op.
 */
lrkv_status lrkv_compress(const lrkv_layer *L, int32_t which, const void *x,
                          int64_t stride_b, int64_t stride_h, int64_t stride_t,
                          int32_t n_tok, int32_t slot0, lrkv_stream_t stream);

/*
 * The quantising step of lrkv_compress on given float32 code rows (LRKV_BF16_Q8
 * and LRKV_BF16_Q4 layers only): slot slot0 + t of head h (of latent group h
 * with head groups), row b receives the quantisation of
 * x[b, h, t, 0 .. r-1] (r = the head's rank for `which`) and its scale.
 *   x: device float32, element (b, h, t, c) at x + b*stride_b + h*stride_h + t*stride_t + c.
 * Errors: LRKV_ERR_DTYPE for other layer types; otherwise as lrkv_compress
 * (strides and x need only 4-byte alignment).
 */
lrkv_status lrkv_quantize(const lrkv_layer *L, int32_t which, const float *x,
                          int64_t stride_b, int64_t stride_h, int64_t stride_t,
                          int32_t n_tok, int32_t slot0, lrkv_stream_t stream);

/*
 * LowRAM prefill (LowRAM abstract: the per-head predictor is fitted at test
 * time; the page gives neither its form nor the selection rule, so both are
 * stated here).  For every (b, h), with C the stored key codes of slots
 * 0 .. n_tok - 1 (made by lrkv_compress) and V the rows v[b, h, t, :] of the
 * same tokens (row t = the token in code slot t):
 *   M = (C^T C + lam I)^-1 C^T V, lam = 1e-6 tr(C^T C) / rank_k[h]   (float32,
 *       Cholesky), stored as bfloat16 into `predictor`;
 *   e_t = V_t - C[t] M with M as stored (float32), and for each 32-slot block of
 *       slots below n_tok the R slots with the largest ||e_t||^2 (float32; equal
 *       norms: the lower slot) keep e_t (bfloat16, in order of decreasing norm)
 *       with its slot and norm; the block's other entries are made empty.
 *   v: device bfloat16, element (b, h, t, i) at v + b*stride_b + h*stride_h + t*stride_t + i.
 * workspace: device, >= lrkv_lowram_workspace_size(L) bytes, no initialisation.
 * Errors: LRKV_ERR_DTYPE unless value_mode is LRKV_VALUES_LOWRAM; LRKV_ERR_SHAPE if
 * n_tok < 1 or a stride is negative; LRKV_ERR_CAPACITY if n_tok > cap;
 * LRKV_ERR_ALIGN; LRKV_ERR_WORKSPACE.
 */
size_t lrkv_lowram_workspace_size(const lrkv_layer *L);
lrkv_status lrkv_lowram_fit(const lrkv_layer *L, const void *v, int64_t stride_b, int64_t stride_h,
                            int64_t stride_t, int32_t n_tok, void *workspace, size_t workspace_bytes,
                            lrkv_stream_t stream);

/*
 * Online basis adaptation (OjaKV summary and FAQ: Oja's algorithm for online PCA
 * keeps adapting the projection basis, thoroughly during prompt prefill and now
 * and then during decoding; the page gives no update rule, so this is the
 * textbook subspace rule).  For every KV head h, with U = U_K(h) (which = 0) or
 * U_V(h) (which = 1) of basis version `version_in` and the rows x[b, h, t, :] for
 * b < batch, t < n_tok (N = batch * n_tok rows):
 *   C  = sum over the rows of x x^T                      (float32)
 *   U' = U + eta (C U - U (U^T C U)) / N
 *   U_new = the columns of U' orthonormalised in order (modified Gram-Schmidt,
 *           float32), stored as bfloat16 U^T rows into version `version_out`
 *           (which may equal version_in).  The other matrix of version_out is
 *           left as it is.
 *   x: device bfloat16, element (b, h, t, i) at x + b*stride_b + h*stride_h + t*stride_t + i.
 *   workspace: device, >= lrkv_oja_workspace_size(L) bytes, needs no initialisation.
 * The kernels write into `bases` (version_out) although the layer describes it
 * as const for every other call.
 * Errors: LRKV_ERR_DTYPE for float32 layers; LRKV_ERR_SHAPE if n_tok < 1, a stride
 * is negative, eta is not finite or a version is outside [0, n_versions);
 * LRKV_ERR_ALIGN as lrkv_compress; LRKV_ERR_WORKSPACE if the workspace is short.
 */
size_t lrkv_oja_workspace_size(const lrkv_layer *L);
lrkv_status lrkv_oja_update(const lrkv_layer *L, int32_t which, const void *x,
                            int64_t stride_b, int64_t stride_h, int64_t stride_t,
                            int32_t n_tok, float eta, int32_t version_in,
                            int32_t version_out, void *workspace, size_t workspace_bytes,
                            lrkv_stream_t stream);

/*
 * Full-rank anchors (OjaKV FAQ: the first token and the most recent tokens are
 * kept uncompressed).  Copies tokens [pos0, pos0 + n_tok) of k and v into their
 * anchor slots (slot 0 for token 0, 1 + (p - 1) % window otherwise).
 *   k, v: device, element (b, h, t, i) at base + b*stride_b + h*stride_h + t*stride_t + i,
 *         where t = p - pos0.
 * Errors: LRKV_ERR_SHAPE unless n_tok >= 0, pos0 >= 0 and the range maps to
 * distinct slots (pos0 == 0: n_tok <= 1 + window; pos0 >= 1: n_tok <= window).
 */
lrkv_status lrkv_store_anchors(const lrkv_layer *L, const void *k, const void *v,
                               int64_t stride_b, int64_t stride_h, int64_t stride_t,
                               int32_t pos0, int32_t n_tok, lrkv_stream_t stream);

/*
 * Cache maintenance of one decode step, the same for every batch row: the new
 * token at position `pos` (k_new, v_new: device [batch][n_kv_heads][128]).
 *  - window >= 1 and pos > window: token pos - window leaves the window; its anchor
 *    slot is compressed into code slot pos - window - 1 (keys and values; quantised
 *    with its scale for LRKV_BF16_Q8 / _Q4), then the new token takes over that slot.
 *  - window == 0 and pos >= 1: the new token is compressed into code slot pos - 1.
 *  - otherwise the new token is stored into its anchor slot.
 * With basis versions the code is made with the version the code slot belongs
 * to (version_start of the row).  Keys compressed before RoPE: the leaving key
 * (post-RoPE, from its anchor slot, or k_new when window = 0) is turned back to
 * its pre-RoPE form at its position before projection.  LowRAM layers: the key is compressed as usual
 * and the value's residual e = V - C_K M (float32, C_K the stored code) enters the
 * slot's block: a slot opening a block (slot % 32 == 0) first empties the block's
 * entries; the residual takes an empty entry if there is one, else replaces the
 * entry of smallest norm (among equal ones the highest slot) if its own squared
 * norm is strictly larger.  The block then keeps the same slots lrkv_lowram_fit
 * would choose.  With head groups the group's code is made from
 * the leaving rows of all its KV heads, and each KV head's anchor slot is updated.
 * Errors: LRKV_ERR_SHAPE if pos < 0; LRKV_ERR_CAPACITY if the code slot >= cap.
 */
lrkv_status lrkv_append(const lrkv_layer *L, const void *k_new, const void *v_new,
                        int32_t pos, lrkv_stream_t stream);

/*
 * Decode attention (blog section 08) in two stages that lrkv_decode_attn runs
 * back to back.
 *
 * n_ctx: cached tokens including the decode token (>= 1); codes cover tokens
 *   1 .. n_ctx - window - 1 and need cap >= max(0, n_ctx - 1 - window).
 * ctx_lens: optional device int32 [batch] of per-row lengths (ragged batches);
 *   each is clamped into [1, n_ctx].  NULL: every row has n_ctx tokens.
 * q: device [batch][n_q_heads][128] in the storage type (bfloat16 for the
 *    quantised-code types).
 * sm_scale: score scale, normally 1/sqrt(128).
 * n_splits: the compressed tokens of each (row, KV head) are cut into this many
 *   contiguous ranges of 32-slot blocks, each scored by its own workgroup
 *   (1 .. LRKV_MAX_SPLITS; 0 = lrkv_decode_auto_splits).  Results agree across
 *   n_splits to rounding; a fixed n_splits is bitwise reproducible.  With basis
 *   versions (OjaKV: codes keep the basis they were made with) every version
 *   gets its own splits, so n_splits >= n_versions (else LRKV_ERR_SHAPE); a
 *   code token is scored against the query projected with its version's U_K
 *   and its value sum is up-projected with its version's U_V.
 * workspace: device, >= lrkv_decode_workspace_size(L, n_splits) bytes, float32
 *   split records; needs no initialisation, and lrkv_decode_partials rewrites
 *   every record lrkv_decode_combine reads.
 * out: device float32 [batch][n_q_heads][128].
 */
size_t lrkv_decode_workspace_size(const lrkv_layer *L, int32_t n_splits);
int32_t lrkv_decode_auto_splits(const lrkv_layer *L, int32_t n_ctx);

/* Stage 1: one workgroup per (split, row, KV head) scores its share of the code
 * blocks and its share of the anchors (runs of at least 16 anchor rows on the
 * first splits, none on the rest) for the g query heads of the group, and writes
 * per (row, query head, split) one float32 record: the running max (log2 units),
 * the softmax denominator, the rank-space value sum of its codes and, on splits
 * that hold anchors, the 128-dim value sum of its anchors, all relative to that
 * max.  The workspace is private to the library between the two stages. */
lrkv_status lrkv_decode_partials(const lrkv_layer *L, int32_t n_ctx, const int32_t *ctx_lens,
                                 const void *q, float sm_scale, int32_t n_splits,
                                 void *workspace, size_t workspace_bytes, lrkv_stream_t stream);

/* Stage 2: merge the split records of each (row, query head) under their common
 * max, up-project the merged rank-space sum once with U_V, add the merged anchor
 * sum and normalise by the merged denominator.  n_ctx, ctx_lens and n_splits
 * must be the values the partials call used (n_splits after resolving 0): they
 * fix which splits hold anchor sums. */
lrkv_status lrkv_decode_combine(const lrkv_layer *L, int32_t n_ctx, const int32_t *ctx_lens,
                                int32_t n_splits, const void *workspace, size_t workspace_bytes,
                                float *out, lrkv_stream_t stream);

/* The whole decode step: stage 1 then stage 2 on `stream`. */
lrkv_status lrkv_decode_attn(const lrkv_layer *L, int32_t n_ctx, const int32_t *ctx_lens,
                             const void *q, float *out, float sm_scale, int32_t n_splits,
                             void *workspace, size_t workspace_bytes, lrkv_stream_t stream);

/*
 * The decode step without a caller workspace, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): as lrkv_decode_attn, with the split records in an array the
 * library holds in device memory, one per GPU, of 16 MiB (16777216 bytes), set
 * up on the first call on each device and kept until the process ends.  The
 * call allocates nothing.  Every call on one GPU shares the array: calls that
 * overlap on a GPU (other streams, other threads) race, so serialise them.  The same kernels run as for lrkv_decode_attn with the same
 * n_splits, so the output is bitwise the same.
 * Errors: as lrkv_decode_attn; LRKV_ERR_WORKSPACE when
 * lrkv_decode_workspace_size(L, n_splits) (n_splits after resolving 0) exceeds
 * 16 MiB; LRKV_ERR_HIP if the array's address cannot be obtained.
 */
lrkv_status lrkv_decode_attn_noalloc(const lrkv_layer *L, int32_t n_ctx, const int32_t *ctx_lens,
                                     const void *q, float *out, float sm_scale, int32_t n_splits,
                                     lrkv_stream_t stream);

const char *lrkv_status_string(lrkv_status s);

/* Library version as 10000*major + 100*minor + patch. */
int32_t lrkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LRKV_H */
