// The verification's scratch memory for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops): a file-scope
// device array of SV_STATIC_SCRATCH_BYTES that sv_spec_verify_static uses in
// place of a caller's workspace, laid out exactly as a workspace.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address of each
// GPU's copy is looked up once, with that GPU current, by
// hipGetSymbolAddress, and that address is what the kernels receive.
#include <mutex>

#include "sv_device.hpp"

namespace sv {

namespace {

static __device__ __align__(256) unsigned char scratch[SV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices];  // device address of `scratch`, per device, once looked up
bool g_cleared[kMaxDevices];  // the zero fill has run outside a graph capture

// Zero-fill n16 16-byte words with kernel stores (no memset node inside a
// captured graph).
__global__ __launch_bounds__(kThreads) void clear_kernel(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += size_t(gridDim.x) * kThreads)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  if (!g_cleared[dev]) {
    // The workspace contract: zero-filled before the first call.  Under
    // capture the fill becomes part of the graph (every replay clears the
    // scratch first, which is harmless); the first call outside a capture
    // clears it once for all later calls.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return e;
    const size_t n16 = SV_STATIC_SCRATCH_BYTES / 16;
    hipLaunchKernelGGL(clear_kernel, dim3(256), dim3(kThreads), 0, stream, static_cast<uint4*>(g_addr[dev]), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (cs == hipStreamCaptureStatusNone) g_cleared[dev] = true;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace sv
