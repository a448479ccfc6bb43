// One decode / verify step through L layers as ONE persistent kernel: the
// buffer set-up kernels and the host launcher.  The kernel and its design are
// in decode_persistent_kernel.h; its instances in decode_persistent_mt*.hip.
#include "decode_persistent_kernel.h"

// Zeroes the tagged buffers once per workspace (recognised by a magic word),
// and again after a call that set the error word (its words carry a tag that
// the next call would reuse); restarts the call count.  Neither header word it
// tests is written while it runs: the mark kernel after it sets the magic and
// clears the error word.
__global__ void decode_persistent_init_kernel(uint32_t* hdr, u64* buf, size_t nwords) {
  if (hdr[0] == PT_MAGIC && hdr[2] == 0u) return;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (size_t)gridDim.x * blockDim.x)
    buf[i] = 0ull;
  if (blockIdx.x == 0 && threadIdx.x == 0) hdr[1] = 0;
}
__global__ void decode_persistent_mark_kernel(uint32_t* hdr) {
  if (threadIdx.x == 0) {
    hdr[0] = PT_MAGIC;
    hdr[2] = 0u;
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
  P.lbuf = P.xbuf + moe_ws_up((size_t)T * H * 8);
  P.pbuf = P.lbuf + moe_ws_up((size_t)T * E * 8);
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

bool moe_persistent_supported(int T, int k, int E, int H, int F, int qfmt) {
  if (T < 1 || T > 8 || k > MOE_MAX_K) return false;
  const PtLayout P = pt_layout(T, k, E, H, F, qfmt, pt_grid(H, E));
  // x words per thread (T * H / 512), router chunks (H / 512) and down rows
  // per thread (H / 512) are unrolled up to 4 * MT, 4 and 4; gate/up K units
  // of 128 per wave up to 2: 256 <= H <= 2048
  return P.lds <= pt_lds_limit() && H <= 2048 && H % 256 == 0 && T * k <= 64;
}

int moe_launch_decode_persistent(const float* x_in, int T, int H, int F, int E, int k, int L,
                                 const uint16_t* w_router, const float* bias, const int32_t* slot_table,
                                 const void* pool, int64_t record_bytes, int qfmt, float* x_out,
                                 int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* ws,
                                 hipStream_t st) {
  const int G = pt_grid(H, E);
  const PtLayout P = pt_layout(T, k, E, H, F, qfmt, G);
  uint8_t* w = (uint8_t*)ws;
  PtArgs a;
  a.x_in = x_in; a.T = T; a.H = H; a.F = F; a.E = E; a.k = k; a.L = L; a.qfmt = qfmt;
  a.w_router = w_router; a.bias = bias; a.slot_table = slot_table; a.pool = (const uint8_t*)pool;
  a.record_bytes = record_bytes; a.x_out = x_out; a.topk_idx_out = topk_idx_out; a.topk_w_out = topk_w_out;
  a.x_hist = x_hist; a.hdr = (uint32_t*)(w + P.hdr); a.xbuf = (u64*)(w + P.xbuf); a.lbuf = (u64*)(w + P.lbuf);
  a.pbuf = (u64*)(w + P.pbuf); a.G = G; a.nfs = P.nfs; a.rpw = P.rpw; a.prep_bytes = P.prep_bytes;
  {  // threads per output row in the final sum: a power of two <= 32 (with 256
     // workgroups, 8 partials a thread: one load each of the NQ in flight;
     // 64 threads per row measured 2.4% slower at one token)
    int tpo = 32;
    while (tpo > 1 && (size_t)T * P.rpw * tpo > PT_THREADS) tpo >>= 1;
    a.tpo = tpo;
  }
  const size_t nwords = (P.total - P.xbuf) / 8;
  decode_persistent_init_kernel<<<256, 256, 0, st>>>(a.hdr, a.xbuf, nwords);
  decode_persistent_mark_kernel<<<1, 64, 0, st>>>(a.hdr);
  // the instance with the fewest token slots >= T (unused slots cost registers
  // and instructions: T=3 on 3 slots 2.21 -> 2.11 ms, T=5 and 6 on 6 slots instead
  // of 8 3.84 -> 3.39 and 4.23 -> 3.71 ms per 48-layer step)
  const int mt = T <= 4 ? T : T <= 6 ? 6 : 8;
  const int slots = E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
  const void* fn = pt_kernel_mt12(qfmt, mt, slots);
  if (!fn) fn = pt_kernel_mt34(qfmt, mt, slots);
  if (!fn) fn = pt_kernel_mt68(qfmt, mt, slots);
  if (!fn) return moe_fail(MOE_EUNSUPPORTED, "decode persistent: no kernel for this shape");
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)P.lds) != hipSuccess)
    return moe_fail(MOE_EHIP, "decode persistent: cannot reserve %zu bytes of LDS", P.lds);
  void* args[] = {&a};
  if (hipLaunchKernel(fn, dim3(G), dim3(PT_THREADS), args, P.lds, st) != hipSuccess)
    return moe_fail(MOE_EHIP, "decode persistent: launch failed");
  return moe_check_launch("decode persistent");
}
