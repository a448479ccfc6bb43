// moe_decode_stack_noalloc: moe_decode_stack without a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).  Its scratch is
// the file-scope device array below, one copy per GPU that loads the
// library, held until the process ends.  Host code never passes the array's
// name to a kernel: it is a host-side stand-in there, not a device address.
// Each device's address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that pointer is used.
#include <mutex>

#include "moe_common.h"
#include "moe_sizes.h"
#include "moe_kernels.h"

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WS_BYTES];

#define MOE_NOALLOC_MAX_DEVICES 64

// The device address of this device's `scratch`, or NULL with the error
// recorded.
static void* noalloc_scratch(int dev) {
  static std::mutex mu;
  static void* ptr[MOE_NOALLOC_MAX_DEVICES] = {};
  if (dev < 0 || dev >= MOE_NOALLOC_MAX_DEVICES) {
    moe_fail(MOE_EUNSUPPORTED, "decode stack (no-alloc): device %d out of [0, %d)", dev, MOE_NOALLOC_MAX_DEVICES);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      moe_fail(MOE_EHIP, "decode stack (no-alloc): hipGetSymbolAddress failed on device %d: %s", dev,
               hipGetErrorString(e));
      (void)hipGetLastError();
      return nullptr;
    }
    ptr[dev] = p;
  }
  return ptr[dev];
}

extern "C" int moe_decode_stack_noalloc(const float* x_in, int T, int H, int F, int E, int k, int L,
                                        const uint16_t* w_router, const float* bias, const int32_t* slot_table,
                                        const void* pool, int64_t record_bytes, int qfmt, float* x_out,
                                        int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* stream) {
  int rc = moe_decode_stack_check(x_in, T, H, F, E, k, L, w_router, slot_table, pool, record_bytes, qfmt, x_out,
                                  x_hist);
  if (rc) return rc;
  const size_t need = moe_ws_decode_stack(T, k, E, H, F, qfmt);
  MOE_REQUIRE(need <= (size_t)MOE_NOALLOC_WS_BYTES, MOE_EWORKSPACE,
              "decode stack (no-alloc): these sizes need %zu bytes of scratch, more than the %d reserved", need,
              MOE_NOALLOC_WS_BYTES);
  int dev = 0;
  MOE_REQUIRE(hipGetDevice(&dev) == hipSuccess, MOE_EHIP, "decode stack (no-alloc): no current device");
  void* ws = noalloc_scratch(dev);
  if (!ws) return dev < 0 || dev >= MOE_NOALLOC_MAX_DEVICES ? MOE_EUNSUPPORTED : MOE_EHIP;
  return moe_decode_stack_run(x_in, T, H, F, E, k, L, w_router, bias, slot_table, pool, record_bytes, qfmt, x_out,
                              topk_idx_out, topk_w_out, x_hist, ws, (size_t)MOE_NOALLOC_WS_BYTES, moe_stream(stream));
}
