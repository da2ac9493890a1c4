// wa_decode_attn_noalloc: one-token decode attention for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).  It runs the kernels of wa_decode_attn;
// the split-key partials, the one buffer those kernels need beyond their
// inputs and outputs, live in `scratch`, a file-scope device array of
// kScratchBytes that each GPU holds until the process ends.
//
// Host code never passes the array's name to a kernel: on the host that name
// is a stand-in, not a device address.  The first call on a device, with
// that device current, asks the runtime for the address of that device's
// copy (hipGetSymbolAddress) and keeps it; every later call uses that
// address.
//
// Every call on a GPU shares its array and finds the last call's contents
// there.  The array begins with the split-key calls' per-(b, h) counters,
// which must start at zero: a device array is zero when the code object is
// loaded, and every call leaves its counters zero again.  The partials after
// them need no initialisation (the merge reads only what blocks of the same
// call wrote).  Two calls in flight at once on one GPU (two streams, two host
// threads) race on the array.
#include <mutex>

#include "wa_internal.h"

namespace {

// The largest scratch a call can need: the planner splits the keys only
// for fewer than 640 (b, h) pairs, into at most ceil(1024 / (B*H)) chunks,
// so n_split * B * H < 1024 + 640 and the partials stay below 1664 * 272 B
// (452 KB), after at most 2.5 KB of counters.  The check below stays, in
// case the planner changes.
constexpr size_t kScratchBytes = WA_DECODE_NOALLOC_SCRATCH_BYTES;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];

// The device address of the current device's `scratch`, looked up once per
// device (with that device current) and kept.
wa_status scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return WA_ERR_HIP;
  if (dev >= kMaxDevices) return WA_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  if (!g_ptr[dev]) return WA_ERR_HIP;
  *out = g_ptr[dev];
  return WA_OK;
}

}  // namespace

extern "C" {

wa_status wa_decode_attn_noalloc(const uint16_t *q, wa_strides qs, const uint8_t *k_cache,
                                 const uint8_t *v_cache, wa_strides cs, int cache_len,
                                 const float *k_scale, const float *v_scale, wa_scale_gran gran,
                                 const int32_t *lens, int B, int H, int head_dim,
                                 float softmax_scale, uint16_t *o, wa_strides os,
                                 hipStream_t stream) {
  wa::DecodeArgs a;
  wa_status st = wa::decode_args(q, qs, k_cache, v_cache, cs, cache_len, k_scale, v_scale, gran, lens,
                                 B, H, head_dim, softmax_scale, o, os, nullptr, nullptr,
                                 wa_strides{0, 0, 0}, &a);
  if (st != WA_OK) return st;
  if (a.need > kScratchBytes) return WA_ERR_TOO_LARGE;
  st = wa::check_device();
  if (st != WA_OK) return st;
  void *ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != WA_OK) return st;
  const hipError_t e = wa::launch_decode(q, a.qs, k_cache, v_cache, cs, cache_len, k_scale, v_scale,
                                         gran == WA_SCALE_PER_HEAD, lens, B, H, softmax_scale, o, a.os,
                                         static_cast<float *>(ws), a.plan, stream);
  return e == hipSuccess ? WA_OK : WA_ERR_HIP;
}

}  // extern "C"
