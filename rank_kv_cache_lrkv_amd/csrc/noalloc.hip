// lrkv_decode_attn_noalloc: the decode step with its split records in a
// file-scope device array instead of a caller workspace, for callers that cannot
// allocate (code under graph capture, tight serving loops).  Same kernels as
// lrkv_decode_attn.
//
// The array's name is a host-side stand-in in host code: its device address is
// asked of the runtime once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels.  Each GPU holds its own
// copy until the process ends; every call on a GPU shares it, so calls that
// overlap on one GPU (different streams, or different host threads) race.  The
// records need no clearing: stage 1 writes every record stage 2 reads.

#include <mutex>

#include "lrkv_internal.h"

namespace lrkv {
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex scratch_mu;
void *scratch_dev[kMaxDevices] = {};

// the device address of `scratch` on the current device (looked up once per device)
lrkv_status scratch_address(void **p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LRKV_ERR_HIP;
  std::lock_guard<std::mutex> g(scratch_mu);
  if (!scratch_dev[dev]) {
    void *a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return LRKV_ERR_HIP;
    scratch_dev[dev] = a;
  }
  *p = scratch_dev[dev];
  return LRKV_OK;
}

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

lrkv_status decode_attn_noalloc(const LayerArgs &A, DecodeArgs &D, float *out, hipStream_t s) {
  void *ws = nullptr;
  lrkv_status st = scratch_address(&ws);
  if (st != LRKV_OK) return st;
  D.ws = static_cast<float *>(ws);
  if (launch_decode_partials(A, D, s) != hipSuccess) return LRKV_ERR_HIP;
  return launch_decode_combine(A, D, out, s) == hipSuccess ? LRKV_OK : LRKV_ERR_HIP;
}

}  // namespace lrkv
