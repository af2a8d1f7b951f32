// read_probe.hip -- a streaming-read kernel for the bench's achievable HBM
// read rate (measurement only: no part of the layer uses it; built into its
// own library, libmoe_probe.so).
//
// Every lane keeps 16 loads of 16 bytes in flight, non-temporal, over a
// grid-stride pass of the buffer: the access that the weight-streaming GEMM
// kernels aim at, without their arithmetic. The values read are folded into
// one word that is stored only if it matches a constant, so that the loads
// stay.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kLoads = 16;   // loads in flight per lane
constexpr int kGrid = 8192;  // work-groups
constexpr int kNt = 2;       // cache policy: non-temporal

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint8_t* src, int64_t bytes,
                                                              uint32_t* sink) {
  const int64_t nthreads = (int64_t)gridDim.x * kThreads;
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t step = nthreads * 16 * kLoads;  // bytes per grid step
  uint32_t acc = 0;
  for (int64_t base = 0; base + step <= bytes; base += step) {
    // one buffer resource per step (its offsets are 32-bit)
    const __amdgpu_buffer_rsrc_t res =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + base), 0, (int)step, 0x00020000);
    u32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           res, (uint32_t)((u * nthreads + tid) * 16), 0, kNt));
#pragma unroll
    for (int u = 0; u < kLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

}  // namespace

// Bytes one pass reads: the largest multiple of the grid step not above
// `bytes` (the step is 8192 x 256 x 16 x 16 bytes = 512 MiB).
extern "C" int64_t moe_probe_stream_read_bytes(int64_t bytes) {
  const int64_t step = (int64_t)kGrid * kThreads * 16 * kLoads;
  return bytes / step * step;
}

// One pass over src (device, `bytes` long) on `stream`; sink: device, at least
// 256 uint32. Returns a hipError_t value (0 on success); no host sync.
extern "C" int moe_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                                     void* stream) {
  if (!src || !sink || bytes <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kGrid), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const uint8_t*>(src), bytes, sink);
  return (int)hipGetLastError();
}
