// LM head with argmax for callers that cannot allocate device memory (code
// under stream capture, tight serving loops, harnesses that forbid
// allocation): tv_lmhead_argmax_noalloc runs exactly the kernels of
// tv_lmhead_argmax, with their scratch (the zeroed argmax keys and
// completion counter, and the per-tile partial keys of more than 64 rows)
// taken from one file-scope device array instead of a caller's workspace.
//
// The array is a host-side stand-in in host code: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever handed to kernels.  Every call on a device
// shares the device's one array, so calls that overlap on one device race;
// each call clears the region that must start at zero (a fill kernel on the
// call's stream, which also serves under capture).
#include <mutex>

#include "tv_internal.h"

namespace tv {
namespace {

constexpr size_t kScratchBytes = (size_t)TV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (nullptr on failure).
void* scratch_address(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}

// Zero n16 16-byte pieces.
__global__ __launch_bounds__(256) void zero_kernel(u32x4_t* __restrict__ p, size_t n16) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = z;
}

}  // namespace
}  // namespace tv

extern "C" {

int tv_lmhead_argmax_noalloc(const void* hidden, const void* w, int32_t* argmax, float* logits,
                             int M, int K, int V, int dtype, int w_layout, void* stream) {
  const int st = tv::lmhead_check(hidden, w, argmax, M, K, V, dtype, w_layout);
  if (st != TV_OK) return st;
  const size_t need = tv::lmhead_ws_bytes(M, K, V, dtype);
  if (need > tv::kScratchBytes) return TV_ESCRATCH;
  hipError_t e = hipSuccess;
  void* ptr = tv::scratch_address(&e);
  if (ptr == nullptr) return tv::hip_status(e);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t z16 = (tv::lmhead_zero_bytes(M) + 15) / 16;
  hipLaunchKernelGGL(tv::zero_kernel, dim3((unsigned)((z16 + 255) / 256 < 1024 ? (z16 + 255) / 256 : 1024)),
                     dim3(256), 0, s, static_cast<tv::u32x4_t*>(ptr), z16);
  e = hipGetLastError();
  if (e != hipSuccess) return tv::hip_status(e);
  return tv::hip_status(
      tv::launch_lmhead_argmax(hidden, w, argmax, logits, M, K, V, dtype, w_layout, ptr, need, s));
}

}  // extern "C"
