// w4a4_linear_glu_quant_noalloc (declared in include/w4a4.h): the quantized
// gated output with its workspace taken from a library-owned device array
// instead of the caller, for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` is file-scope device memory: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Host
// code never passes the array's name to a kernel or a copy (on the host it is
// only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, on
// the entry point's first call there.  Nothing here allocates; the
// workspace's contents are scratch (no call needs them cleared).  Calls that
// overlap on one GPU -- on different streams, or from different host threads
// -- share that GPU's array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "w4a4.h"
#include "w4a4_internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;   // W4A4_NOALLOC_SCRATCH_BYTES

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (nullptr on a HIP error).
void* scratch_on_current_device(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = W4A4_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = W4A4_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

static_assert(kScratchBytes == W4A4_NOALLOC_SCRATCH_BYTES, "the header states the array's size");

extern "C" int w4a4_linear_glu_quant_noalloc(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate,
                                             const void* act, const void* wblob, int32_t R_down,
                                             const void* down_wblob, void* act_out, void* stream) {
  // every argument check first, on the host, as the entry point it varies
  int st = w4a4::glu_quant_call(M, N, K, R, r_gate, act, wblob, R_down, down_wblob, act_out, nullptr, stream,
                                true);
  if (st || M == 0) return st;
  size_t need = 0;
  if ((st = w4a4_glu_quant_workspace(M, N, R_down, &need))) return st;
  if (need > kScratchBytes) return W4A4_ERR_SHAPE;   // beyond the array: a caller-provided workspace is needed
  void* ws = scratch_on_current_device(&st);
  if (!ws) return st;
  return w4a4::glu_quant_call(M, N, K, R, r_gate, act, wblob, R_down, down_wblob, act_out, ws, stream, false);
}
