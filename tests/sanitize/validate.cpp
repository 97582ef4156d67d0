// Drives every entry point of include/lrkv.h through its host-side argument
// checks (built with AddressSanitizer and UndefinedBehaviorSanitizer, the
// launchers replaced by counting stand-ins): each bad argument must give its
// status with no launch, each good call must reach the launchers.  Prints
// "validate: N checks passed" and exits 0, or names the first failing check.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "lrkv.h"

extern int g_launches;

static int checks = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    ++checks;                                                            \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                      \
    }                                                                    \
  } while (0)

// a 16-byte aligned non-null address the checks never dereference
static void *const F = reinterpret_cast<void *>(uintptr_t(1) << 20);

struct Layer {
  std::vector<int32_t> rk, rv;
  lrkv_layer L{};
  Layer(int dtype, int batch, int hq, int hkv, int window, int cap, std::vector<int32_t> k,
        std::vector<int32_t> v)
      : rk(k), rv(v) {
    L.dtype = dtype;
    L.batch = batch;
    L.n_q_heads = hq;
    L.n_kv_heads = hkv;
    L.window = window;
    L.cap = cap;
    L.rank_k = rk.data();
    L.rank_v = rv.data();
    L.bases = F;
    L.codes_k = F;
    L.codes_v = F;
    L.anchor_k = F;
    L.anchor_v = F;
    L.scales_k = static_cast<float *>(F);
    L.scales_v = static_cast<float *>(F);
  }
};

// status of a call and whether it launched nothing
#define ERR(call, st)                    \
  do {                                   \
    const int before = g_launches;       \
    EXPECT((call) == (st));              \
    EXPECT(g_launches == before);        \
  } while (0)
#define OK(call)                         \
  do {                                   \
    const int before = g_launches;       \
    EXPECT((call) == LRKV_OK);           \
    EXPECT(g_launches > before);         \
  } while (0)

int main() {
  float *out = static_cast<float *>(F);
  // layer checks, through the decode entry point
  {
    Layer a(LRKV_BF16, 4, 32, 8, 128, 32768, std::vector<int32_t>(8, 64), std::vector<int32_t>(8, 32));
    const size_t ws = lrkv_decode_workspace_size(&a.L, 32);
    EXPECT(ws == size_t(4) * 32 * 32 * (4 + 32 + 128) * 4);
    OK(lrkv_decode_attn(&a.L, 32768, nullptr, F, out, 0.088f, 32, F, ws, nullptr));
    OK(lrkv_decode_attn_noalloc(&a.L, 32768, nullptr, F, out, 0.088f, 32, nullptr));
    ERR(lrkv_decode_attn(nullptr, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_NULL);
    ERR(lrkv_decode_attn(&a.L, 0, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    ERR(lrkv_decode_attn(&a.L, 40000, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_CAPACITY);
    ERR(lrkv_decode_attn(&a.L, 100, nullptr, F, out, -1.f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    ERR(lrkv_decode_attn(&a.L, 100, nullptr, F, out, 0.088f, 2000, F, ws, nullptr), LRKV_ERR_SHAPE);
    ERR(lrkv_decode_attn(&a.L, 32768, nullptr, F, out, 0.088f, 32, F, ws - 4, nullptr), LRKV_ERR_WORKSPACE);
    ERR(lrkv_decode_attn(&a.L, 100, nullptr, F, out + 1, 0.088f, 2, F, ws, nullptr), LRKV_ERR_ALIGN);
    ERR(lrkv_decode_attn(&a.L, 100, nullptr, nullptr, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_NULL);
    ERR(lrkv_decode_attn_noalloc(&a.L, 32768, nullptr, F, out, 0.088f, 1024, nullptr), LRKV_ERR_WORKSPACE);
    EXPECT(lrkv_decode_auto_splits(&a.L, 32768) == 32);  // no device: 1024 workgroups
    // every field of the description
    lrkv_layer b = a.L;
    b.dtype = 9;
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_DTYPE);
    b = a.L;
    b.n_q_heads = 31;
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    b = a.L;
    b.cap = 33;
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    b = a.L;
    b.cap = (1 << 30);  // one code region past 2^31 bytes
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    b = a.L;
    b.codes_v = reinterpret_cast<char *>(F) + 8;
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_ALIGN);
    b = a.L;
    b.n_versions = 17;
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    b = a.L;
    b.head_group = 3;
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    b = a.L;
    b.rope_base = 0.5f;
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    b = a.L;
    b.value_mode = LRKV_VALUES_LOWRAM;
    b.resid_per_block = 9;
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_SHAPE);
    std::vector<int32_t> bad(8, 64);
    bad[7] = 72;
    b = a.L;
    b.rank_k = bad.data();
    ERR(lrkv_decode_attn(&b, 100, nullptr, F, out, 0.088f, 2, F, ws, nullptr), LRKV_ERR_RANK);
  }
  // the widest layer description: 64 KV heads, 16 query heads each, mixed ranks
  {
    std::vector<int32_t> k(64), v(64);
    for (int h = 0; h < 64; ++h) {
      k[h] = 16 * (1 + h % 8);
      v[h] = 16 * (1 + (h * 3) % 8);
    }
    Layer w(LRKV_BF16, 2, 1024, 64, 4, 4096, k, v);
    const int32_t S = lrkv_decode_auto_splits(&w.L, 4000);
    EXPECT(S >= 1);
    const size_t ws = lrkv_decode_workspace_size(&w.L, S);
    OK(lrkv_decode_attn(&w.L, 4000, nullptr, F, out, 0.088f, 0, F, ws, nullptr));
    OK(lrkv_decode_attn(&w.L, 4000, nullptr, F, out, 0.088f, 1024,
                        F, lrkv_decode_workspace_size(&w.L, 1024), nullptr));
  }
  // compress, quantise, anchors, append
  {
    Layer a(LRKV_BF16, 2, 8, 2, 4, 64, {64, 32}, {32, 16});
    OK(lrkv_compress(&a.L, 0, F, 1024, 512, 128, 10, 0, nullptr));
    ERR(lrkv_compress(&a.L, 2, F, 1024, 512, 128, 10, 0, nullptr), LRKV_ERR_SHAPE);
    ERR(lrkv_compress(&a.L, 0, F, 1024, 512, 128, 60, 10, nullptr), LRKV_ERR_CAPACITY);
    ERR(lrkv_compress(&a.L, 0, F, 1024, 512, 127, 10, 0, nullptr), LRKV_ERR_ALIGN);
    ERR(lrkv_compress(&a.L, 0, F, -1, 512, 128, 10, 0, nullptr), LRKV_ERR_SHAPE);
    ERR(lrkv_compress(&a.L, 0, nullptr, 1024, 512, 128, 10, 0, nullptr), LRKV_ERR_NULL);
    EXPECT(lrkv_compress(&a.L, 0, F, 1024, 512, 128, 0, 0, nullptr) == LRKV_OK);  // no-op
    ERR(lrkv_quantize(&a.L, 0, static_cast<float *>(F), 1024, 512, 128, 10, 0, nullptr), LRKV_ERR_DTYPE);
    OK(lrkv_store_anchors(&a.L, F, F, 1024, 512, 128, 0, 5, nullptr));
    ERR(lrkv_store_anchors(&a.L, F, F, 1024, 512, 128, 0, 6, nullptr), LRKV_ERR_SHAPE);
    ERR(lrkv_store_anchors(&a.L, F, F, 1024, 512, 128, 3, 5, nullptr), LRKV_ERR_SHAPE);
    OK(lrkv_append(&a.L, F, F, 10, nullptr));
    ERR(lrkv_append(&a.L, F, F, -1, nullptr), LRKV_ERR_SHAPE);
    ERR(lrkv_append(&a.L, F, F, 100, nullptr), LRKV_ERR_CAPACITY);
    Layer q(LRKV_BF16_Q8, 2, 8, 2, 4, 64, {64, 32}, {32, 16});
    OK(lrkv_quantize(&q.L, 1, static_cast<float *>(F), 1024, 512, 128, 10, 0, nullptr));
    q.L.scales_k = nullptr;
    ERR(lrkv_quantize(&q.L, 1, static_cast<float *>(F), 1024, 512, 128, 10, 0, nullptr), LRKV_ERR_NULL);
  }
  // Oja and LowRAM fit
  {
    Layer a(LRKV_BF16, 2, 8, 2, 4, 64, {64, 32}, {32, 16});
    a.L.n_versions = 2;
    a.L.version_start = static_cast<const int32_t *>(F);
    const size_t ows = lrkv_oja_workspace_size(&a.L);
    OK(lrkv_oja_update(&a.L, 0, F, 1024, 512, 128, 10, 0.5f, 0, 1, F, ows, nullptr));
    ERR(lrkv_oja_update(&a.L, 0, F, 1024, 512, 128, 10, 0.5f, 0, 2, F, ows, nullptr), LRKV_ERR_SHAPE);
    ERR(lrkv_oja_update(&a.L, 0, F, 1024, 512, 128, 10, 0.5f, 0, 1, F, ows - 1, nullptr), LRKV_ERR_WORKSPACE);
    Layer r(LRKV_BF16, 2, 8, 2, 4, 64, {64, 32}, {32, 16});
    r.L.value_mode = LRKV_VALUES_LOWRAM;
    r.L.resid_per_block = 4;
    r.L.codes_v = nullptr;
    r.L.predictor = F;
    r.L.resid = F;
    r.L.resid_slot = static_cast<int32_t *>(F);
    r.L.resid_norm = static_cast<float *>(F);
    const size_t lws = lrkv_lowram_workspace_size(&r.L);
    OK(lrkv_lowram_fit(&r.L, F, 1024, 512, 128, 40, F, lws, nullptr));
    ERR(lrkv_lowram_fit(&r.L, F, 1024, 512, 128, 65, F, lws, nullptr), LRKV_ERR_CAPACITY);
    ERR(lrkv_compress(&r.L, 1, F, 1024, 512, 128, 10, 0, nullptr), LRKV_ERR_DTYPE);
  }
  for (int s = 0; s <= 9; ++s) EXPECT(lrkv_status_string(lrkv_status(s)) != nullptr);
  std::printf("validate: %d checks passed\n", checks);
  return 0;
}
