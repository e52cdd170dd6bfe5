// Allocation-free batched rotation: ckks_rotate_noalloc.
//
// The key switch needs a workspace (ModUp inputs, raised digits,
// accumulators, ModDown output).  ckks_rotate grows a context-owned buffer
// with hipMalloc on demand and spreads chunks over internal streams; this
// entry point instead takes its workspace from one file-scope device array,
// `scratch`, and runs every chunk on the caller's stream, so the call
// allocates nothing and can be recorded into a HIP graph or run in a loop that
// forbids allocation.
//
// Each GPU that loads the library holds its own copy of `scratch` (128 MiB)
// until the process ends.  Its device address is resolved once per device,
// with that device current, when a context is created there
// (noalloc_init_device, called by ckks_ctx_create) and kept per device; the
// kernels take that address as an ordinary workspace pointer.  On the host
// the array's name is only a stand-in for the symbol, never passed to a
// kernel.
//
// Every call on one GPU shares that GPU's array: two calls that overlap in
// time on one GPU (on different streams, or from different threads) race on
// it.  The pipeline writes every workspace word before it reads it, so
// nothing needs clearing between calls.
#include <mutex>

#include "kernels.h"

namespace ckks {

namespace {

constexpr uint64_t kScratchWords = 1ull << 24;  // 128 MiB of 64-bit words
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint64_t scratch[kScratchWords];

std::mutex g_scratch_mu;
uint64_t* g_scratch_ptr[kMaxDevices] = {};

uint64_t* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

}  // namespace

int noalloc_init_device(int device) {
  if (device < 0 || device >= kMaxDevices) return set_error(CKKS_EINVAL, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return CKKS_OK;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p)
    return set_error(CKKS_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  g_scratch_ptr[device] = static_cast<uint64_t*>(p);
  return CKKS_OK;
}

}  // namespace ckks

using namespace ckks;

extern "C" {

int ckks_rotate_noalloc(ckks_ctx* ctx, const uint64_t* d_ct_in, uint64_t* d_ct_out, int batch, int level,
                        const uint32_t* galois_elts, const uint64_t* const* d_evks, unsigned flags,
                        ckks_stream_t stream) {
  if (!ctx) return set_error(CKKS_EINVAL, "ctx is NULL");
  if (hipSetDevice(ctx->device) != hipSuccess) return set_error(CKKS_EHIP, "hipSetDevice failed");
  int rc = rotate_check(ctx, d_ct_in, d_ct_out, batch, level, galois_elts, d_evks, flags);
  if (rc) return rc;
  uint64_t* ws = scratch_ptr(ctx->device);
  if (!ws) return set_error(CKKS_EINTERNAL, "scratch address not resolved for this device");
  const uint64_t per = ks_ws_words(ctx, level);
  if (per > kScratchWords)
    return set_error(CKKS_ERANGE, "one ciphertext's key-switch workspace at this level (" +
                                      std::to_string(per * 8 >> 20) + " MiB) exceeds the " +
                                      std::to_string(kScratchWords * 8 >> 20) +
                                      " MiB scratch of the allocation-free rotation");
  ctx->no_alloc = true;
  rc = rotate_fixed_ws(ctx, stream, d_ct_in, d_ct_out, batch, level, galois_elts, d_evks, flags, ws, kScratchWords);
  ctx->no_alloc = false;
  return rc;
}

}  // extern "C"
