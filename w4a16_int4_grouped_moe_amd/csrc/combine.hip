// combine.hip -- top-k weighted combine with the shared-expert add (gfx950).
//
//   out[t, n] = bf16( s[t, n] + sum_{j < k, id_tj local} w_tj * y[t*k + j, n] )
//
// summed in fp32 in slot order j = 0..k-1 and rounded once to bf16 (nearest
// even). The shared expert enters with weight 1 (Kimi-K2.6 catalog entry, MoE
// paragraph: one always-on shared expert); routing weights are applied as
// given. One work-group per token and 1024-column slab, four columns per thread
// (16-byte loads of y and s, 8-byte stores); the loads of eight slots are in
// flight together.
#include "internal.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

constexpr int kBufferFlags = 0x00020000;       // raw buffer resource, dword 3
constexpr int kOutOfRange = (int)0x80000000u;  // buffer offset past any resource: reads 0
constexpr int kSlotBatch = 8;                  // slots whose loads are in flight together
#ifndef MOE_Y_AUX
#define MOE_Y_AUX 2
#endif
constexpr int kYAux = MOE_Y_AUX;  // cache policy of the y loads (read once)

// The loads of slots j0 .. j0 + kSlotBatch - 1 (all of them inside k when
// FULL: their ids and weights are then read with unconditional scalar loads)
// are issued before any is used; slots past k or not local read out of range,
// i.e. zeros (their rows of y were never written), and are skipped.
template <bool FULL>
__device__ __forceinline__ void combine_slots(f32x4& acc, __amdgpu_buffer_rsrc_t yres,
                                              const int32_t* ids, const float* w, int j0, int k,
                                              int H, int n, int E, int base) {
  bool ok[kSlotBatch];
  float wt[kSlotBatch];
  f32x4 v[kSlotBatch];
#pragma unroll
  for (int u = 0; u < kSlotBatch; ++u) {
    const int j = j0 + u;
    const bool in = FULL || j < k;
    const int e = in ? ids[j] - base : -1;
    ok[u] = (unsigned)e < (unsigned)E;
    wt[u] = in ? w[j] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < kSlotBatch; ++u)
    v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         yres, ok[u] ? ((j0 + u) * H + n) * 4 : kOutOfRange, 0,
                                         kYAux));
#pragma unroll
  for (int u = 0; u < kSlotBatch; ++u) {
    if (!ok[u]) continue;
    acc.x = fmaf(wt[u], v[u].x, acc.x);
    acc.y = fmaf(wt[u], v[u].y, acc.y);
    acc.z = fmaf(wt[u], v[u].z, acc.z);
    acc.w = fmaf(wt[u], v[u].w, acc.w);
  }
}

__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float* __restrict__ y, const float* __restrict__ s, const int32_t* __restrict__ ids,
    const float* __restrict__ w, uint16_t* __restrict__ out, int H, int k, int E, int base) {
  const int64_t t = blockIdx.x;
  const int n = (blockIdx.y * kThreads + threadIdx.x) * 4;
  if (n >= H) return;
  // the token's k rows of y are contiguous (row = pair id = t * k + j); without
  // a shared expert the s resource is empty and reads zeros
  const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(y + t * k * H), 0, k * H * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(s ? s + t * H : y), 0, s ? H * 4 : 0, kBufferFlags);
  f32x4 acc = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sres, n * 4, 0, 0));
  for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
    if (j0 + kSlotBatch <= k)
      combine_slots<true>(acc, yres, ids + t * k, w + t * k, j0, k, H, n, E, base);
    else
      combine_slots<false>(acc, yres, ids + t * k, w + t * k, j0, k, H, n, E, base);
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

