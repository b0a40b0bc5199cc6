// lf_attn_forward_noalloc: lf_attn_forward for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that forbid
// allocation).  Its scratch (split tickets, global-row partials; fp32: the preprocessed
// masks) lives in one file-scope device array instead of stream-ordered allocations.
//
// Each device the library runs on holds its own copy of the array until the process
// ends.  Host code never passes the array's name to a kernel (on the host it stands for
// a host-side shadow, not a device address): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and only that address is
// used.  Every call on a device shares the array, so calls that overlap in time on one
// device (on different streams, or from different threads) race; the array keeps the
// last call's contents.  The tickets must be zero when a call starts: they are
// zero-filled on the first call on each device, and every call leaves them zero.
#include <mutex>

#include "../../include/lf.h"
#include "lf_internal.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kNoallocTickets = 16384;   // (batch, head) pairs with global rows
constexpr size_t kTicketBytes = (size_t)kNoallocTickets * sizeof(int);
constexpr size_t kScratchBytes = (size_t)32 << 20;   // tickets, then the partials

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
unsigned char* g_ptr[kMaxDevices];   // device address of `scratch`, per device (nullptr: not yet)

// The device address of this device's array; on the first call per device it is
// looked up and the ticket region zero-filled on `st` (ahead of the call's kernels).
int scratch_ptr(hipStream_t st, unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return lf::set_error(LF_ERR_HIP, "lf_attn_forward_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return lf::set_error(LF_ERR_UNSUPPORTED, "lf_attn_forward_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    unsigned char* p = nullptr;
    e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return lf::set_error(LF_ERR_HIP, "lf_attn_forward_noalloc: hipGetSymbolAddress failed");
    e = lf::launch_fill_i32((int*)p, kNoallocTickets, 0, st);
    if (e != hipSuccess)
      return lf::set_error(LF_ERR_HIP, "lf_attn_forward_noalloc: ticket zero-fill failed");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return LF_OK;
}

}  // namespace

extern "C" {

size_t lf_attn_forward_noalloc_max_scratch(void) { return kScratchBytes - kTicketBytes; }

int lf_attn_forward_noalloc(int dtype, const void* q, const void* k, const void* v,
                            const void* qg, const void* kg, const void* vg,
                            const void* local_mask, const void* global_mask, int B, int H, int S,
                            int W, int G, void* out, void* stream) {
  // the shape rules first: a rejected call enqueues nothing
  if (int e = lf::attn_forward_validate(dtype, q, k, v, qg, kg, vg, local_mask, global_mask, B, H,
                                        S, W, G, out, kScratchBytes - kTicketBytes,
                                        kNoallocTickets, "lf_attn_forward_noalloc"))
    return e;
  unsigned char* p = nullptr;
  if (int e = scratch_ptr((hipStream_t)stream, &p)) return e;
  return lf::attn_forward_in(dtype, q, k, v, qg, kg, vg, local_mask, global_mask, B, H, S, W, G,
                             out, stream, (char*)p + kTicketBytes, kScratchBytes - kTicketBytes,
                             (int*)p, kNoallocTickets, "lf_attn_forward_noalloc");
}

}  // extern "C"
