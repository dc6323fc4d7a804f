// noalloc.hip -- attn_bwd_noalloc: the dense backward of attn_bwd with its row
// statistics in a static device array instead of a caller's workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` exists once per GPU: each device holds its own copy from the moment
// the library's code is loaded there until the process ends.  Host code reaches
// it only through the address hipGetSymbolAddress reports for the current
// device (looked up once per device, kept in g_scratch_addr); the array's name
// in host code is a host-side stand-in, never a device address.  The kernels
// take that address as their workspace, exactly as they take a caller's.
//
// Every call on a GPU uses the same array, which keeps the last call's
// contents: calls that overlap on one GPU race on it.  Nothing in it needs
// clearing first: the statistics pass writes every row (m, l, delta and the
// row offset) that the dK / dV and dQ passes then read.
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "attn_bwd.h"
#include "launch.hpp"

namespace {

// Four statistics planes of B * H * Sq rows each (256-byte aligned), as
// attn_bwd_workspace_bytes sizes them: 16 MiB for 2^20 rows.
constexpr int64_t kNoAllocRows = (int64_t)1 << 20;
constexpr size_t kPlaneBytes = ((size_t)kNoAllocRows * sizeof(float) + 255) & ~(size_t)255;
constexpr size_t kScratchBytes = 4 * kPlaneBytes;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};  // device address of `scratch`, per device

int err(int code, const char *msg) {
  attn::set_last_error(msg);
  return code;
}

// The device address of `scratch` on the calling thread's current device,
// looked up on the first call on that device.
int scratch_address(void **addr) {
  char msg[256];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(msg, sizeof msg, "attn_bwd_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    return err(ATTN_E_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, sizeof msg, "attn_bwd_noalloc: device index %d out of range", dev);
    return err(ATTN_E_HIP, msg);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(msg, sizeof msg, "attn_bwd_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s",
               dev, hipGetErrorString(e));
      return err(ATTN_E_HIP, msg);
    }
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd_noalloc(const attn_bwd_args *a, void *stream) {
  char msg[256];
  if (!a) return err(ATTN_E_INVALID, "args is NULL");
  // The size limit first, before any HIP call.
  if (a->B < 0 || a->H < 0 || a->Sq < 0) {
    snprintf(msg, sizeof msg, "negative size (B=%lld H=%lld Sq=%lld)", (long long)a->B,
             (long long)a->H, (long long)a->Sq);
    return err(ATTN_E_INVALID, msg);
  }
  int64_t rows;
  if (__builtin_mul_overflow(a->B, a->H, &rows) || __builtin_mul_overflow(rows, a->Sq, &rows) ||
      rows > kNoAllocRows) {
    snprintf(msg, sizeof msg,
             "attn_bwd_noalloc: B * H * Sq must be at most %lld rows (its static statistics scratch "
             "holds %zu bytes per GPU); use attn_bwd with a workspace",
             (long long)kNoAllocRows, kScratchBytes);
    return err(ATTN_E_WORKSPACE, msg);
  }
  void *ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != ATTN_OK) return rc;
  attn_bwd_args b = *a;
  b.workspace = ws;
  // exactly the statistics planes: the one-workgroup-per-block form, the one
  // attn_bwd takes with a workspace of attn_bwd_workspace_bytes()
  b.workspace_bytes = attn_bwd_workspace_bytes(a->B, a->H, a->Sq);
  return attn::run_dense_all(&b, stream);
}
