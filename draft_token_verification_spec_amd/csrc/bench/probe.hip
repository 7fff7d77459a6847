// libsvbench.so: measurement aids for bench.py, not part of the verification
// library's interface.
//
// svb_read_probe reads a device buffer with the access pattern of the
// verification's statistics kernel - one 256-thread workgroup per 32 KiB,
// eight 16-byte non-temporal loads per thread issued together - and does no
// arithmetic beyond an XOR of what it read, so that its rate is the ceiling a
// streaming read of that shape reaches on the device.  Each wave writes the
// XOR of the 16-byte vectors it read (as four 32-bit words) to the sink, word
// 4 * workgroup + wave, so that no load can be optimised away and a test can
// check that every byte was read.
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kNV = 8;  // 16-byte vectors per thread: 32 KiB per workgroup
constexpr size_t kBytesPerBlock = size_t(kThreads) * kNV * 16;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void read_probe_kernel(
    const u32x4* data, size_t n16, uint32_t* sink) {
  const int tid = threadIdx.x;
  const size_t base = size_t(blockIdx.x) * kThreads * kNV;
  u32x4 v[kNV];
#pragma unroll
  for (int k = 0; k < kNV; ++k) {
    const size_t i = base + size_t(k) * kThreads + tid;
    v[k] = i < n16 ? __builtin_nontemporal_load(data + i) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < kNV; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((tid & 63) == 0) sink[size_t(blockIdx.x) * kWaves + (tid >> 6)] = x;
}

}  // namespace

extern "C" {

// Sink words a probe of `bytes` writes: one per wave of each 32 KiB workgroup.
size_t svb_read_probe_sink_words(size_t bytes) {
  return (bytes / 16 * 16 + kBytesPerBlock - 1) / kBytesPerBlock * kWaves;
}

// Read `bytes` at `data` (device, 16-byte aligned, a multiple of 16 bytes)
// on `stream`; 0 on success, -1 for invalid arguments (nothing launched),
// -2 for a buffer too large for one grid, -4 for a launch error.
int svb_read_probe(void* stream, const void* data, size_t bytes, uint32_t* sink, size_t sink_words) {
  if (bytes == 0) return 0;
  if (!data || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(data) & 15u) != 0) return -1;
  const size_t blocks = (bytes + kBytesPerBlock - 1) / kBytesPerBlock;
  if (blocks >= (size_t(1) << 31)) return -2;
  if (sink_words < svb_read_probe_sink_words(bytes)) return -1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(data), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
