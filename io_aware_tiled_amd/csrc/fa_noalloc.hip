// Fixed device scratch of the allocation-free backward (fa_bwd_noalloc).
//
// The backward keeps one float32 per query row between its stages: D_i, the
// row dot product dO_i . O_i written by the preprocessing kernel and read by
// the dK/dV and dQ kernels.  fa_bwd takes that buffer from the caller;
// fa_bwd_noalloc takes it from the file-scope array below instead, so that a
// caller that cannot allocate device memory (code under stream capture, a
// serving loop, a harness that forbids allocation) needs no workspace.
//
// Every GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  In host code the array's name is only a
// host-side stand-in, never a device address: the device address is looked
// up once per device with hipGetSymbolAddress (with that device current) and
// kept here; only that address is handed to kernels.  All calls on one GPU
// share the array, so calls that overlap on one GPU (different streams, no
// ordering between them) race on it.  Nothing in it has to start at zero:
// the preprocessing kernel writes every row it covers before the other two
// kernels read it.
#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace fa {

static_assert((size_t)FA_BWD_NOALLOC_MAX_ROWS * sizeof(float) % 256 == 0,
              "scratch is a whole number of 256-byte lines");

static __device__ __align__(256) float scratch[FA_BWD_NOALLOC_MAX_ROWS];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];

}  // namespace

int noalloc_scratch(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return -6;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess)
      g_addr[dev] = p;
  });
  if (g_addr[dev] == nullptr) return -6;
  *addr = g_addr[dev];
  return 0;
}

}  // namespace fa
