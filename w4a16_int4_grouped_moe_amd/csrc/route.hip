// route.hip -- the router step in front of the layer (gfx950): for each token
// the top-k experts by fp32 score, in descending score order with equal scores
// in ascending expert id, and weights = softmax over the selected scores.
//
// The lmdeploy "support Kimi K2.6" pull request (Runtime Validation) lists MoE
// routing among the validated paths but gives no formula; the plainest rule
// is taken (softmax over all experts renormalised over the k selected equals
// the softmax over the selected scores).
//
// One wave per token, four tokens per work-group. Each score becomes a 32-bit
// key, an order-preserving image of the float (-0.0 mapped to +0.0 first), so
// that an unsigned maximum picks the largest score. Each of k rounds takes the
// wave-wide maximum key (DPP row shifts and row broadcasts, no LDS), then the
// lowest expert holding it (a ballot per register, lowest register first:
// expert = lane + 64 * register), and the owner lane retires that key. Lane j
// keeps round j's score, and lanes j < k then form the softmax in fp32
// (expf, IEEE division) with a fixed DPP summation order.
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

// x moved across lanes by a DPP control; lanes without a source, or outside
// ROW_MASK, read 0 (the identity of both reductions below)
template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp(T x) {
  const int i = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, i, CTRL, ROW_MASK, 0xF, false));
}

// op (an unsigned max or a float sum) over the wave in a fixed order,
// returned to every lane
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp<0x111, 0xF>(v));  // row_shr:1
  v = op(v, dpp<0x112, 0xF>(v));  // row_shr:2
  v = op(v, dpp<0x114, 0xF>(v));  // row_shr:4
  v = op(v, dpp<0x118, 0xF>(v));  // row_shr:8: lane 15 of each row holds the row
  v = op(v, dpp<0x142, 0xA>(v));  // row_bcast:15 into rows 1 and 3
  v = op(v, dpp<0x143, 0xC>(v));  // row_bcast:31 into rows 2 and 3: lane 63 holds all
  return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
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

  auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  uint32_t mine = 0;  // lane j: the key of round j
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < kPerLane; ++i) best = umax(best, key[i]);
    const uint32_t m = wave_reduce(best, umax);
    int e = 0;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const uint64_t b = __ballot(key[i] == m);
      if (b) {
        e = 64 * i + __builtin_ctzll(b);
        break;
      }
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
      if (lane + 64 * i == e) key[i] = 0u;
    if (lane == j) {
      mine = m;
      my_id = e;
    }
  }

  // softmax over the k selected scores; round 0 holds the largest
  const float top = key_value(__builtin_amdgcn_readfirstlane(mine));
  const float z = lane < k ? expf(key_value(mine) - top) : 0.f;
  const float sum = wave_reduce(z, [](float a, float b) { return a + b; });
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
