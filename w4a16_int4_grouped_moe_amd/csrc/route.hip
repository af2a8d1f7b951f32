// route.hip -- the router step in front of the layer (gfx950): for each token
// the top-k experts by fp32 score, in descending score order with equal scores
// in ascending expert id, and weights = softmax over the selected scores.
//
// The lmdeploy "support Kimi K2.6" pull request (Runtime Validation) lists MoE
// routing among the validated paths but gives no formula; the plainest rule
// is taken (softmax over all experts renormalised over the k selected equals
// the softmax over the selected scores).
//
// One wave per token, four tokens per work-group. Each score becomes a 64-bit
// key, (order-preserving image of the float) << 32 | ~expert, so one unsigned
// maximum picks the largest score and, among equal scores, the lowest expert
// (-0.0 is mapped to +0.0 first). k rounds of a wave-wide maximum select the
// experts; the owner lane retires the winner's key. Lane j keeps round j's
// score, and lanes j < k then form the softmax in fp32 (expf, IEEE division),
// summed by a fixed butterfly, so the result does not depend on timing.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPerLane = kMaxScored / 64;

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ uint64_t wave_max(uint64_t v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = __shfl_xor(v, d);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

__global__ __launch_bounds__(kThreads) void route_kernel(const float* __restrict__ scores,
                                                         int64_t T, int S, int k,
                                                         int32_t* __restrict__ topk_ids,
                                                         float* __restrict__ topk_weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = scores + t * S;

  // lane l holds experts l, l + 64, ...; a retired or absent entry is 0, below
  // every real key (the key of -inf is 0x007FFFFF)
  uint32_t key[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < S ? order_key(row[e]) : 0u;
  }

  uint32_t mine = 0;  // lane j: the key of round j
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const uint64_t c =
          key[i] ? ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(lane + 64 * i) : 0ull;
      best = c > best ? c : best;
    }
    best = wave_max(best);
    const int e = (int)~(uint32_t)best;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
      if (lane + 64 * i == e) key[i] = 0u;
    if (lane == j) {
      mine = (uint32_t)(best >> 32);
      my_id = e;
    }
  }

  // softmax over the k selected scores; round 0 holds the largest
  const float top = key_value(__builtin_amdgcn_readfirstlane(mine));
  const float z = lane < k ? expf(key_value(mine) - top) : 0.f;
  const float sum = wave_sum(z);
  if (lane < k) {
    topk_ids[t * k + lane] = my_id;
    topk_weights[t * k + lane] = z / sum;
  }
}

}  // namespace

hipError_t launch_route(const float* scores, int64_t T, int32_t S, int32_t k, int32_t* topk_ids,
                        float* topk_weights, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (S < 1 || S > kMaxScored || k < 1 || k > S || k > 64) return hipErrorInvalidValue;
  const int64_t groups = (T + kWaves - 1) / kWaves;
  if (groups > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)groups), dim3(kThreads), 0, stream, scores, T,
                     S, k, topk_ids, topk_weights);
  return hipGetLastError();
}

}  // namespace moe
