// iq_decode_attention_noalloc: iq_decode_attention for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The split
// plan and the split-K partials live in this file's device array `scratch`, of a fixed size, instead
// of a caller's workspace; the kernels are the ones iq_decode_attention launches.
//
// `scratch` is a host-side stand-in in host code: its device address is looked up once per device
// with hipGetSymbolAddress (the device current) and only that address is passed to the kernels.
// Every call on a device shares that device's array.  Nothing in it has to start at zero: the split
// kernel writes the plan and every partial row before the combine kernel of the same call reads
// them.  Calls that overlap on one device (other streams, other host threads) race on it.
#include <mutex>

#include "iq.h"
#include "iq_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[IQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (nullptr: not looked up yet)

// The device address of the current device's `scratch`, looked up on the first call there.
int scratch_on_current_device(const char* fn, void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) {
    iq::set_error("%s: hipGetDevice failed: %s", fn, hipGetErrorString(err));
    return IQ_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    iq::set_error("%s: device %d is beyond the %d devices the library tracks", fn, dev, kMaxDevices);
    return IQ_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr) {
      iq::set_error("%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(err));
      return IQ_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return IQ_OK;
}

}  // namespace

extern "C" int iq_decode_attention_noalloc(const void* q, int32_t q_dtype, const uint8_t* k_codes,
                                           const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                                           const float* rot, int64_t rot_stride_batch, const int32_t* seq_lens,
                                           int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_cap,
                                           float sm_scale, float* out, int32_t head_dim, int32_t bits,
                                           void* stream) {
  static const char* fn = "iq_decode_attention_noalloc";
  iq::clear_error();
  if (head_dim != IQ_HEAD_DIM || bits != IQ_BITS) {
    iq::set_error("%s: head_dim must be 128 and bits 3 (got %d, %d)", fn, head_dim, bits);
    return IQ_EUNSUPPORTED;
  }
  void* ws = nullptr;
  const int rc = scratch_on_current_device(fn, &ws);
  if (rc) return rc;
  return iq::decode_entry(fn, q, q_dtype, 1, k_codes, k_scales, v_codes, v_scales, rot, rot_stride_batch, seq_lens,
                          batch, n_q_heads, n_kv_heads, cache_cap, sm_scale, out, ws, IQ_NOALLOC_SCRATCH_BYTES,
                          IQ_FMT_U3, stream, true);
}
