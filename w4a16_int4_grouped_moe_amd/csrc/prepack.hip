// prepack.hip -- one-time repack of the int4 expert weights and their bf16
// scales into the chunk-contiguous layout described in internal.h (gfx950).
//
// The prefill kernel reads each 512-row tile of an expert 128 inputs at a
// time: 64 bytes of every row, half of a 128-byte line, and the scales 16
// groups at a time, 32 bytes of a row's line. In the checkpoint layout (rows
// of K/8 words) the other half of each line is needed one chunk later and has
// often left the cache by then, so lines are fetched twice. In the repacked
// layout a chunk of a tile is one contiguous 32 KB run (and a scale period one
// 16 KB run), so every fetched line is used whole. The arithmetic is the same
// in both layouts, and so are the results, bit for bit.
//
// The repack is a plain copy: one thread per 16-byte group of codes, one
// thread per (row, 16-group period) of scales.
#include "internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void prepack_codes_kernel(const int32_t* __restrict__ packed,
                                                                 int64_t units, int32_t Nw,
                                                                 int32_t K, bool w13, int32_t I,
                                                                 uint8_t* __restrict__ out) {
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (u >= units) return;
  const int32_t ng = K / 32;
  const int32_t g = (int32_t)(u % ng);
  const int64_t row = u / ng;  // e * Nw + n
  const int32_t n = (int32_t)(row % Nw);
  const int64_t e = row / Nw;
  const u32x4 v = *reinterpret_cast<const u32x4*>(packed + row * (K / 8) + 4 * g);
  *reinterpret_cast<u32x4*>(out + e * pack_code_bytes(Nw, K) + pack_code_offset(w13, I, K, n, g)) =
      v;
}

__global__ __launch_bounds__(kThreads) void prepack_scales_kernel(
    const uint16_t* __restrict__ scales, int64_t items, int32_t Nw, int32_t K, bool w13, int32_t I,
    uint8_t* __restrict__ out) {
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (u >= items) return;
  const int32_t ng = K / 32;  // a multiple of 4: pairs of groups never straddle the end
  const int32_t nper = pack_periods(K);
  const int32_t per = (int32_t)(u % nper);
  const int64_t row = u / nper;
  const int32_t n = (int32_t)(row % Nw);
  const int64_t e = row / Nw;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(scales + row * ng);
  uint32_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int32_t g = 16 * per + 2 * i;
    v[i] = g < ng ? src[g / 2] : 0u;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(out + e * pack_scale_bytes(Nw, K) +
                                        pack_scale_offset(w13, I, K, n, 16 * per));
  dst[0] = u32x4{v[0], v[1], v[2], v[3]};
  dst[1] = u32x4{v[4], v[5], v[6], v[7]};
}

}  // namespace

hipError_t launch_prepack(const int32_t* packed, const uint16_t* scales, int32_t E, int32_t Nw,
                          int32_t K, bool w13, int32_t I, uint8_t* codes_out,
                          uint8_t* scales_out, hipStream_t stream) {
  if (Nw % kPackRows || K % kPackChunk) return hipErrorInvalidValue;
  const int64_t units = (int64_t)E * Nw * (K / 32);
  const int64_t items = (int64_t)E * Nw * pack_periods(K);
  const int64_t gc = (units + kThreads - 1) / kThreads, gs = (items + kThreads - 1) / kThreads;
  if (gc > 0x7fffffff || gs > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (gc == 0) return hipSuccess;
  hipLaunchKernelGGL(prepack_codes_kernel, dim3((unsigned)gc), dim3(kThreads), 0, stream, packed,
                     units, Nw, K, w13, I, codes_out);
  hipLaunchKernelGGL(prepack_scales_kernel, dim3((unsigned)gs), dim3(kThreads), 0, stream, scales,
                     items, Nw, K, w13, I, scales_out);
  return hipGetLastError();
}

}  // namespace moe
