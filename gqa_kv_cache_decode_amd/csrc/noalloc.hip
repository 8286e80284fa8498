// gqa_attend_decode for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the same kernels, with the library's own scratch array in
// place of the caller's workspace.
//
// `scratch` is a file-scope device array of kScratchBytes that every GPU the
// library runs on holds from the module's load until the process ends.  In
// host code its name is only a stand-in, so the array's device address is
// resolved once per device, on that device's first call (hipGetSymbolAddress
// with the device current), and kept; the kernels get that address, never
// the name.  Every call on a GPU shares its array: calls that overlap on one
// GPU (two streams, or two host threads) race.  attend_decode's workspace
// needs no initialisation (every partial is written before it is read), so
// nothing is cleared between calls.
#include <mutex>

#include "gqa_decode.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device

// The scratch array's address on the stream's device, which must be the
// current one (resolved there on its first call).
gqa_status scratch_for(hipStream_t stream, void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_DEVICE;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return GQA_ERR_DEVICE;
    if (sdev != dev) return GQA_ERR_INVALID_ARGUMENT;
  }
  if (dev < 0 || dev >= kMaxDevices) return GQA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return GQA_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_attend_decode_noalloc(const void *q, int32_t num_q_heads,
                                     const gqa_cache *cache,
                                     const int32_t *lens, float scale,
                                     const float *bias, int64_t bias_stride,
                                     const gqa_carry *carry_in,
                                     const gqa_carry *carry_out, float *out,
                                     hipStream_t stream) {
  size_t need = 0;
  gqa_status st = gqa::attend_decode_check(q, num_q_heads, cache, lens, scale,
                                           bias, bias_stride, carry_in,
                                           carry_out, out, &need);
  if (st != GQA_OK) return st;
  if (need > kScratchBytes) return GQA_ERR_WORKSPACE_TOO_SMALL;
  void *ws = nullptr;
  if ((st = scratch_for(stream, &ws)) != GQA_OK) return st;
  return gqa_attend_decode(q, num_q_heads, cache, lens, scale, bias,
                           bias_stride, carry_in, carry_out, out, ws,
                           kScratchBytes, stream);
}

}  // extern "C"
