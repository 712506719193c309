// gsa_fwd_noalloc: the chunkwise GSA forward with its scratch space (the
// segment state maps and start states of the chunk-state scan, and the
// segment decay products) taken from a fixed device array of this library
// instead of a caller-provided workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in this code object; every GPU the library runs on holds
// its own copy (allocated when the code object is loaded there, held until
// the process ends).  Host code never names the array directly: its host
// symbol is only a stand-in, so its device address is looked up once per
// device with hipGetSymbolAddress and that address is what the kernels get.
// The forward writes every word of its scratch before reading it, so nothing
// is cleared between calls.  All calls on one GPU share the array: calls that
// overlap on one GPU (different streams, or different host threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gsa.h"

static __device__ __align__(256) unsigned char scratch[GSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::once_flag g_once[kMaxDevices];
hipError_t g_status[kMaxDevices];

// The array's address on device dev, looked up with dev current (once per
// device and process); nullptr if the lookup failed.
void* scratch_on(int dev) {
  std::call_once(g_once[dev], [dev] {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != dev) (void)hipSetDevice(prev);
    g_status[dev] = e;
    g_scratch[dev] = e == hipSuccess ? p : nullptr;
  });
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t gsa_fwd_noalloc_scratch_bytes(void) { return GSA_NOALLOC_SCRATCH_BYTES; }

int gsa_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const float* k0,
                    const float* v0, void* o, float* k_final, float* v_final, int B, int H, int T,
                    int dk, int dv, int m, int C, float tau, int dtype, int chunks_per_segment,
                    int nonlinearity, void* stream, void* const* events) {
  // size first, on the host: nothing touches the device for a rejected call
  const size_t need = gsa_fwd_workspace_bytes(B, H, T, dk, dv, m, C, dtype, chunks_per_segment);
  if (need == (size_t)-1) return GSA_ERR_SHAPE;
  if (need > GSA_NOALLOC_SCRATCH_BYTES) return GSA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return GSA_ERR_HIP;
    ws = scratch_on(dev);
    if (!ws) return GSA_ERR_HIP;
  }
  return gsa_fwd_ex(q, k, v, g, k0, v0, o, k_final, v_final, B, H, T, dk, dv, m, C, tau, dtype, ws,
                    ws ? (size_t)GSA_NOALLOC_SCRATCH_BYTES : 0, chunks_per_segment, nonlinearity,
                    stream, events);
}

}  // extern "C"
