// Host-only stand-ins for the library's launchers and device queries, so the
// argument checks of the C entry points (api.hip) can run under AddressSanitizer
// and UndefinedBehaviorSanitizer with no GPU and no device code.  Every
// stand-in counts as one launch.
#include "lrkv_internal.h"

int g_launches = 0;

namespace lrkv {
static hipError_t launched() {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_compress(const LayerArgs &, int, const void *, int64_t, int64_t, int64_t, int, int, hipStream_t) {
  return launched();
}
hipError_t launch_compress_mfma(const LayerArgs &, int, const void *, int64_t, int64_t, int64_t, int, int,
                                hipStream_t) {
  return launched();
}
hipError_t launch_quantize(const LayerArgs &, int, const float *, int64_t, int64_t, int64_t, int, int, hipStream_t) {
  return launched();
}
hipError_t launch_store_anchors(const LayerArgs &, const void *, const void *, int64_t, int64_t, int64_t, int, int,
                                hipStream_t) {
  return launched();
}
hipError_t launch_append(const LayerArgs &, const void *, const void *, int, hipStream_t) { return launched(); }
hipError_t launch_decode_partials(const LayerArgs &, const DecodeArgs &, hipStream_t) { return launched(); }
hipError_t launch_partials_mfma(const LayerArgs &, const DecodeArgs &, hipStream_t) { return launched(); }
hipError_t launch_decode_combine(const LayerArgs &, const DecodeArgs &, float *, hipStream_t) { return launched(); }
size_t noalloc_scratch_bytes() { return size_t(16) << 20; }
lrkv_status decode_attn_noalloc(const LayerArgs &, DecodeArgs &, float *, hipStream_t) {
  launched();
  return LRKV_OK;
}
hipError_t launch_oja(const LayerArgs &, int, const void *, int64_t, int64_t, int64_t, int, float, int, int, float *,
                      hipStream_t) {
  return launched();
}
size_t oja_workspace_bytes(const LayerArgs &) { return size_t(1) << 20; }
hipError_t launch_lowram_fit(const LayerArgs &, const bf16_t *, int64_t, int64_t, int64_t, int, float *,
                             hipStream_t) {
  return launched();
}
size_t lowram_workspace_bytes(const LayerArgs &) { return size_t(1) << 20; }
int partials_blocks_per_cu(const LayerArgs &) { return 0; }
int device_cu_count() { return 0; }
int kernel_blocks_per_cu(const void *) { return 0; }
int generic_blocks_per_cu() { return 0; }
}  // namespace lrkv
