// combine.hip -- top-k weighted combine with the shared-expert add (gfx950).
//
//   out[t, n] = bf16( s[t, n] + sum_{j < k, id_tj local} w_tj * y[t*k + j, n] )
//
// summed in fp32 in slot order j = 0..k-1 and rounded once to bf16 (nearest
// even). The shared expert enters with weight 1 (Kimi-K2.6 catalog entry, MoE
// paragraph: one always-on shared expert); routing weights are applied as
// given. One work-group per token and 1024-column slab, four columns per thread
// (16-byte loads of y and s, 8-byte stores).
#include "internal.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float* __restrict__ y, const float* __restrict__ s, const int32_t* __restrict__ ids,
    const float* __restrict__ w, uint16_t* __restrict__ out, int H, int k, int E, int base) {
  const int64_t t = blockIdx.x;
  const int n = (blockIdx.y * kThreads + threadIdx.x) * 4;
  if (n >= H) return;
  f32x4 acc = s ? *reinterpret_cast<const f32x4*>(s + t * H + n) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int e = ids[t * k + j] - base;
    if ((unsigned)e >= (unsigned)E) continue;
    const float wt = w[t * k + j];
    const f32x4 v = *reinterpret_cast<const f32x4*>(y + (t * k + j) * H + n);
    acc.x = fmaf(wt, v.x, acc.x);
    acc.y = fmaf(wt, v.y, acc.y);
    acc.z = fmaf(wt, v.z, acc.z);
    acc.w = fmaf(wt, v.w, acc.w);
  }
  uint2 o;
  o.x = pack_bf16x2(acc.x, acc.y);
  o.y = pack_bf16x2(acc.z, acc.w);
  *reinterpret_cast<uint2*>(out + t * H + n) = o;
}

}  // namespace

hipError_t launch_combine(const float* y, const float* s, const int32_t* topk_ids,
                          const float* topk_weights, uint16_t* out, int64_t T, int32_t H,
                          int32_t k, int32_t E, int32_t base, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)T, (unsigned)((H / 4 + kThreads - 1) / kThreads));
  void* kargs[] = {&y, &s, &topk_ids, &topk_weights, &out, &H, &k, &E, &base};
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel), grid, dim3(kThreads),
                         kargs, 0, stream);
}

}  // namespace moe
