// One decode / verify step through L layers as ONE persistent kernel: the
// buffer set-up kernels and the host launcher.  The kernel and its design are
// in decode_persistent_kernel.h; its instances in decode_persistent_mt*.hip.
#include "decode_persistent_kernel.h"

#include <mutex>

// Tags.  Every call takes the tags base+1 .. base+L, where base is the tag
// count reserved so far on this workspace (hdr[1]); the reservation is made
// by the set-up kernel before the step starts, so a call's tags are larger
// than every tag any earlier call on the workspace wrote, whatever its layer
// count, token count or outcome.  A stale word therefore never matches.
// The tagged region is zeroed (and the count restarted) when the header is
// not a valid one (first use, or memory that held something else), after a
// call that timed out, and before the 32-bit count would wrap.
__device__ __forceinline__ bool pt_ws_needs_reset(const uint32_t* hdr, int L) {
  return hdr[0] != PT_MAGIC || hdr[2] != 0u || hdr[3] != (hdr[1] ^ PT_CHECK) ||
         hdr[1] > 0xFFFFFFFFu - 2u * (uint32_t)L;
}
// Zeroes every word of the workspace after the header when a reset is due.
// No header word is written here (every workgroup tests the same values);
// the reserve kernel after it does that.
__global__ void decode_persistent_init_kernel(const uint32_t* hdr, u64* buf, size_t nwords, int L) {
  if (!pt_ws_needs_reset(hdr, L)) return;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (size_t)gridDim.x * blockDim.x)
    buf[i] = 0ull;
}
// Restarts the count after a reset, then reserves this call's L tags:
// hdr[4] = this call's base, hdr[1] = the new count (with its check word).
__global__ void decode_persistent_reserve_kernel(uint32_t* hdr, int L) {
  if (threadIdx.x == 0) {
    const uint32_t base = pt_ws_needs_reset(hdr, L) ? 0u : hdr[1];
    hdr[4] = base;
    hdr[1] = base + (uint32_t)L;
    hdr[3] = (base + (uint32_t)L) ^ PT_CHECK;
    hdr[2] = 0u;
    hdr[0] = PT_MAGIC;
  }
}

// ---------------------------------------------------------------- host side
struct PtLayout {
  size_t hdr, xbuf, lbuf, pbuf, total;
  int G, nfs, rpw;
  size_t prep_bytes, lds;
};

static int pt_grid(int H, int E) {
  static int ncu = 0;
  if (!ncu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      ncu = 0;
    if (ncu <= 0) ncu = 256;
  }
  int lim = ncu < E ? ncu : E;
  if (H / 8 < lim) lim = H / 8;
  int G = 1;
  while (G * 2 <= lim && H % (G * 2) == 0) G *= 2;
  return G;
}

static PtLayout pt_layout(int T, int k, int E, int H, int F, int qfmt, int G) {
  PtLayout P;
  P.G = G;
  P.nfs = F / 32;
  P.rpw = H / G;
  P.prep_bytes = moe_prep_bytes(H, qfmt);
  P.hdr = 0;
  P.xbuf = 256;
  P.lbuf = P.xbuf + moe_ws_up((size_t)PT_REPL * T * H * 8);  // one copy of x per XCD
  P.pbuf = P.lbuf + moe_ws_up((size_t)PT_REPL * T * E * 8);  // one copy of the logits per XCD
  P.total = P.pbuf + moe_ws_up((size_t)G * T * H * 8);  // one partial vector per (workgroup, token)
  P.lds = pt_lds(qfmt, T, k, E, H, P.prep_bytes).total;
  return P;
}

size_t moe_ws_stack_persistent(int T, int k, int E, int H, int F, int qfmt) {
  return pt_layout(T, k, E, H, F, qfmt, pt_grid(H, E)).total;
}

// LDS one workgroup may reserve (the device's opt-in limit; 64 KB if unknown)
static size_t pt_lds_limit() {
  static size_t lim = 0;
  if (!lim) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeSharedMemPerBlockOptin, dev) == hipSuccess && v > 0)
      lim = (size_t)v;
    else
      lim = 64 * 1024;
  }
  return lim;
}

// The instance with the fewest token slots >= T (unused slots cost registers
// and instructions: T=3 on 3 slots 2.21 -> 2.11 ms, T=5 and 6 on 6 slots instead
// of 8 3.84 -> 3.39 and 4.23 -> 3.71 ms per 48-layer step), or NULL.
static const void* pt_instance(int qfmt, int T, int E) {
  const int mt = T <= 4 ? T : T <= 6 ? 6 : 8;
  const int slots = E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
  const void* fn = pt_kernel_mt12(qfmt, mt, slots);
  if (!fn) fn = pt_kernel_mt34(qfmt, mt, slots);
  if (!fn) fn = pt_kernel_mt68(qfmt, mt, slots);
  return fn;
}

// Whether the device can hold all G workgroups of the instance at once (the
// kernel's waits assume every workgroup is running).  The answer of the
// occupancy query is cached per (instance, LDS bytes, device).
bool moe_persistent_coresident(int T, int k, int E, int H, int F, int qfmt) {
  const void* fn = pt_instance(qfmt, T, E);
  if (!fn) return false;
  const int G = pt_grid(H, E);
  const PtLayout P = pt_layout(T, k, E, H, F, qfmt, G);
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    return false;
  struct Entry { const void* fn; size_t lds; int dev; bool ok; };
  static std::mutex mu;
  static Entry cache[64];
  static int n = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (cache[i].fn == fn && cache[i].lds == P.lds && cache[i].dev == dev) return cache[i].ok;
  int per_cu = 0;
  bool ok = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)P.lds) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, PT_THREADS, P.lds) == hipSuccess &&
            (int64_t)per_cu * ncu >= G;
  (void)hipGetLastError();  // a failed query leaves no sticky error behind
  if (n < 64) cache[n++] = Entry{fn, P.lds, dev, ok};
  return ok;
}

bool moe_persistent_supported(int T, int k, int E, int H, int F, int qfmt) {
  if (T < 1 || T > 8 || k > MOE_MAX_K) return false;
  const PtLayout P = pt_layout(T, k, E, H, F, qfmt, pt_grid(H, E));
  // x words per thread (T * H / 512), router chunks (H / 512) and down rows
  // per thread (H / 512) are unrolled up to 4 * MT, 4 and 4; gate/up K units
  // of 128 per wave up to 2: 256 <= H <= 2048
  return P.lds <= pt_lds_limit() && H <= 2048 && H % 256 == 0 && T * k <= 128;
}

#ifdef MOE_PT_STAMPS
// the phase timestamps of the last step (instrumented builds only)
static unsigned long long* g_stamps = nullptr;
extern "C" int moe_pt_read_stamps(void* dst) {
  if (!g_stamps) return -1;
  return (int)hipMemcpy(dst, g_stamps, sizeof(unsigned long long) * 64 * 256 * 16, hipMemcpyDeviceToHost);
}
#endif

int moe_launch_decode_persistent(const float* x_in, int T, int H, int F, int E, int k, int L,
                                 const uint16_t* w_router, const float* bias, const int32_t* slot_table,
                                 const void* pool, int64_t record_bytes, int qfmt, float* x_out,
                                 int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* ws,
                                 size_t ws_bytes, hipStream_t st) {
  const int G = pt_grid(H, E);
  const PtLayout P = pt_layout(T, k, E, H, F, qfmt, G);
  uint8_t* w = (uint8_t*)ws;
  PtArgs a;
  a.x_in = x_in; a.T = T; a.H = H; a.F = F; a.E = E; a.k = k; a.L = L; a.qfmt = qfmt;
  a.w_router = w_router; a.bias = bias; a.slot_table = slot_table; a.pool = (const uint8_t*)pool;
  a.record_bytes = record_bytes; a.x_out = x_out; a.topk_idx_out = topk_idx_out; a.topk_w_out = topk_w_out;
  a.x_hist = x_hist; a.hdr = (uint32_t*)(w + P.hdr); a.xbuf = (u64*)(w + P.xbuf); a.lbuf = (u64*)(w + P.lbuf);
  a.stamps = nullptr;
#ifdef MOE_PT_STAMPS
  if (!g_stamps && hipMalloc(&g_stamps, sizeof(unsigned long long) * 64 * 256 * 16) != hipSuccess) g_stamps = nullptr;
  a.stamps = g_stamps;
#endif
  a.pbuf = (u64*)(w + P.pbuf); a.G = G; a.nfs = P.nfs; a.rpw = P.rpw; a.prep_bytes = P.prep_bytes;
  {  // threads per output row in the final sum: a power of two <= 32 (with 256
     // workgroups, 8 partials a thread: one load each of the NQ in flight;
     // 64 threads per row measured 2.4% slower at one token)
    int tpo = 32;
    while (tpo > 1 && (size_t)T * P.rpw * tpo > PT_THREADS) tpo >>= 1;
    a.tpo = tpo;
  }
  // a reset zeroes all of ws (not only this layout): a larger layout of an
  // earlier call may have left tagged words further in
  const size_t nwords = (ws_bytes - P.xbuf) / 8;
  decode_persistent_init_kernel<<<256, 256, 0, st>>>(a.hdr, a.xbuf, nwords, L);
  decode_persistent_reserve_kernel<<<1, 64, 0, st>>>(a.hdr, L);
  const void* fn = pt_instance(qfmt, T, E);
  if (!fn) return moe_fail(MOE_EUNSUPPORTED, "decode persistent: no kernel for this shape");
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)P.lds) != hipSuccess)
    return moe_fail(MOE_EHIP, "decode persistent: cannot reserve %zu bytes of LDS", P.lds);
  void* args[] = {&a};
  if (hipLaunchKernel(fn, dim3(G), dim3(PT_THREADS), args, P.lds, st) != hipSuccess)
    return moe_fail(MOE_EHIP, "decode persistent: launch failed");
  return moe_check_launch("decode persistent");
}
