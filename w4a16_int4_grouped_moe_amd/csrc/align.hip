// align.hip -- token/expert bucketing for the grouped W4A16 GEMMs (gfx950).
//
// A stable counting sort of the valid (token, slot) pairs p = t*k + j by local
// expert e = id - base, each expert's bucket padded with the sentinel P = T*k to
// a multiple of block_m, buckets in expert order, plus the block -> expert map.
// The grouped MoE kernels named in the lmdeploy "support Kimi K2.6" pull request
// (Changes list) need such a bucketing; the pages leave its form open, and this
// ordering (ascending p inside a bucket) is the one the library fixes.
//
// One work-group of 16 waves does everything in a single launch:
//   1. each wave histograms a contiguous chunk of pairs (LDS atomics; counts
//      do not depend on order);
//   2. per expert: prefix of the wave counts, padded size, block-wide scan of
//      the padded sizes -> bucket offsets and n_padded;
//   3. each wave walks its chunk 64 pairs at a time in pair order; equal
//      experts inside the 64 are ranked by lane with ballots, so positions are
//      exactly the stable order (no order-dependent atomics);
//   4. sentinel padding and block_expert.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void align_kernel(
    const int32_t* __restrict__ ids, int64_t P, int E, int base, int bm,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ n_padded_out) {
  extern __shared__ int32_t smem[];
  volatile int32_t* hist = smem;             // [kWaves][E]: counts, then write cursors
  int32_t* off = smem + kWaves * E;          // [E] bucket start
  int32_t* cnt = off + E;                    // [E] valid pairs per expert
  int32_t* wsum = cnt + E;                   // [kWaves] scan partials

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int i = tid; i < kWaves * E; i += kThreads) hist[i] = 0;
  __syncthreads();

  // contiguous chunk of this wave, a multiple of 64 pairs long
  const int64_t per = ((P + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t c0 = min(P, per * wave);
  const int64_t c1 = min(P, c0 + per);

  // 1. histogram
  for (int64_t p = c0 + lane; p < c1; p += 64) {
    const int e = ids[p] - base;
    if ((unsigned)e < (unsigned)E) atomicAdd((int32_t*)&hist[wave * E + e], 1);
  }
  __syncthreads();

  // 2. totals, per-wave prefixes and the bucket offsets
  int pad = 0;
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = hist[w * E + tid];
      hist[w * E + tid] = run;
      run += c;
    }
    cnt[tid] = run;
    pad = (run + bm - 1) / bm * bm;
  }
  int incl = pad;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int s = lane < kWaves ? wsum[lane] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(s, d);
      if (lane >= d) s += u;
    }
    if (lane < kWaves) wsum[lane] = s;
  }
  __syncthreads();
  const int excl = incl - pad + (wave > 0 ? wsum[wave - 1] : 0);
  if (tid < E) off[tid] = excl;
  if (tid == kThreads - 1) *n_padded_out = excl + pad;
  __syncthreads();
  for (int i = tid; i < kWaves * E; i += kThreads) hist[i] += off[i % E];
  __syncthreads();

  // 3. stable scatter, 64 pairs at a time in pair order
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t p0 = c0; p0 < c1; p0 += 64) {
    const int64_t p = p0 + lane;
    int e = -1;
    if (p < c1) {
      const int t = ids[p] - base;
      if ((unsigned)t < (unsigned)E) e = t;
    }
    uint64_t active = __ballot(e >= 0);
    int rank = 0, group = 0;
    while (active) {
      const int leader = __builtin_ctzll(active);
      const int key = __builtin_amdgcn_readlane(e, leader);
      const uint64_t m = __ballot(e == key);
      if (e == key) {
        rank = __popcll(m & lt_mask);
        group = __popcll(m);
      }
      active &= ~m;
    }
    if (e >= 0) {
      const int cursor = hist[wave * E + e];
      sorted_ids[cursor + rank] = (int32_t)p;
      if (rank == 0) hist[wave * E + e] = cursor + group;
    }
  }
  __syncthreads();

  // 4. padding and the block map
  if (tid < E) {
    const int o = off[tid];
    const int c = cnt[tid];
    const int pd = (c + bm - 1) / bm * bm;
    for (int r = c; r < pd; ++r) sorted_ids[o + r] = (int32_t)P;
    for (int b = o / bm; b < (o + pd) / bm; ++b) block_expert[b] = tid;
  }
}

}  // namespace

hipError_t launch_align(const int32_t* topk_ids, int64_t P, int32_t E, int32_t base,
                        int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                        int32_t* n_padded, hipStream_t stream) {
  const size_t lds = sizeof(int32_t) * (size_t)(kWaves * E + 2 * E + kWaves);
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), lds, stream, topk_ids, P, E, base,
                     block_m, sorted_ids, block_expert, n_padded);
  return hipGetLastError();
}

}  // namespace moe
