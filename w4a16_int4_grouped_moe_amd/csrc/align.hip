// align.hip -- token/expert bucketing for the grouped W4A16 GEMMs (gfx950).
//
// A stable counting sort of the valid (token, slot) pairs p = t*k + j by local
// expert e = id - base, each expert's bucket padded with the sentinel P = T*k to
// a multiple of block_m, buckets in expert order, plus the block -> expert map.
// The grouped MoE kernels named in the lmdeploy "support Kimi K2.6" pull request
// (Changes list) need such a bucketing; the pages leave its form open, and this
// ordering (ascending p inside a bucket) is the one the library fixes.
//
// Small P: one work-group of 8 waves does everything in a single launch:
//   1. each wave histograms a contiguous chunk of pairs (LDS atomics; counts
//      do not depend on order);
//   2. per expert: prefix of the wave counts, padded size, block-wide scan of
//      the padded sizes -> bucket offsets and n_padded;
//   3. sentinel padding and block_expert (the scatter never writes these
//      positions);
//   4. each wave walks its chunk 64 pairs at a time in pair order; the lanes
//      of a step that share an expert are ranked by lane: each lane ORs its
//      bit into the expert's 64-bit lane mask in a per-wave LDS table (an OR
//      does not depend on order), reads the mask back and counts the lower
//      lanes, so positions are exactly the stable order.
// Split form (small P only): experts with at most `tau` pairs get their
// buckets in a second set of arrays with a second block size (bm2); the
// others keep the first. Each set is the bucketing of its own experts alone
// (buckets in expert order, padded to its block size), and every valid pair
// lands in exactly one of them.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = kMaxExperts;  // thread e owns expert e in the scans
constexpr int kWaves = kThreads / 64;

// The lanes of this wave that hold expert e (e < 0: none), as a lane mask:
// each lane ORs its bit into the expert's entry of the wave's own LDS table (an
// OR does not depend on order) and reads the entry back (a wave's LDS
// operations complete in issue order). The caller's lowest lane of the group
// clears the entry before the table is used again.
__device__ __forceinline__ uint64_t lane_group(uint64_t* wmask, int e, int lane) {
  if (e < 0) return 0;
  __hip_atomic_fetch_or(&wmask[e], 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __hip_atomic_load(&wmask[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void clear_lane_group(uint64_t* wmask, int e) {
  __hip_atomic_store(&wmask[e], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Sentinel padding of each bucket and the block -> expert map, by all the
// work-group's threads (tid of nthreads = 64 nwaves; E <= nthreads).
// off/cnt: bucket start (a multiple of bm) and valid pairs, in LDS.
// sorted_ids must be 16-byte aligned.
//
// Blocks of at most kPadPerThread rows: thread e pads its own bucket (at most
// bm - 1 entries) and writes its blocks.
// Larger blocks: a padding of up to bm - 1 entries per thread would take as
// many serial stores, each to a cache line per lane. Instead a wave splits
// into 8 groups of 8 lanes; group g takes the wave's experts g, g + 8, ...
// (expert wave + nwaves (8 i + g)), and its lanes cover the padding in
// aligned 4-entry windows, lane j windows j, j + 8, ...: a whole window with
// one 16-byte store, the (at most two) partial ones entry by entry.
constexpr int kPadPerThread = 16;

__device__ __forceinline__ void pad_buckets(const int32_t* off, const int32_t* cnt, int E, int bm,
                                            int32_t sentinel, int tid, int nwaves,
                                            int32_t* __restrict__ sorted_ids,
                                            int32_t* __restrict__ block_expert) {
  if (bm <= kPadPerThread) {
    if (tid < E) {
      const int o = off[tid];
      const int c = cnt[tid];
      const int nb = (c + bm - 1) / bm;
      for (int r = c; r < nb * bm; ++r) sorted_ids[o + r] = sentinel;
      const int b0 = o / bm;
      for (int b = 0; b < nb; ++b) block_expert[b0 + b] = tid;
    }
    return;
  }
  const int wave = tid >> 6, g = (tid >> 3) & 7, j = tid & 7;
  const int4 fill = make_int4(sentinel, sentinel, sentinel, sentinel);
  for (int i = 0; wave + nwaves * 8 * i < E; ++i) {
    const int e = wave + nwaves * (8 * i + g);
    if (e >= E) continue;
    const int o = off[e];
    const int c = cnt[e];
    const int nb = (c + bm - 1) / bm;
    const int start = o + c, end = o + nb * bm;
    for (int w = (start >> 2) + j; 4 * w < end; w += 8) {
      const int a = 4 * w;
      if (a >= start && a + 4 <= end) {
        *reinterpret_cast<int4*>(sorted_ids + a) = fill;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (a + u >= start && a + u < end) sorted_ids[a + u] = sentinel;
      }
    }
    const int b0 = o / bm;
    for (int b = j; b < nb; b += 8) block_expert[b0 + b] = e;
  }
}

// Exclusive prefix of v over the work-group's threads (thread order), and the
// total in *total; wsum: kWaves ints of LDS. Ends with a barrier.
__device__ __forceinline__ int block_exclusive_scan(int v, int32_t* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
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
  const int excl = incl - v + (wave > 0 ? wsum[wave - 1] : 0);
  *total = wsum[kWaves - 1];
  __syncthreads();
  return excl;
}

__global__ __launch_bounds__(kThreads) void align_kernel(
    const int32_t* __restrict__ ids, int64_t P, int E, int base, int bm,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ n_padded_out, int tau, int bm2, int32_t* __restrict__ sorted2,
    int32_t* __restrict__ block_expert2, int32_t* __restrict__ n_padded2_out) {
  extern __shared__ int32_t smem[];
  int32_t* hist = smem;                      // [kWaves][E]: counts, then write cursors
  int32_t* off = smem + kWaves * E;          // [E] bucket start (first set)
  int32_t* cnt = off + E;                    // [E] valid pairs per expert (first set)
  int32_t* wsum = cnt + E;                   // [kWaves] scan partials
  // [kWaves][E] lane masks; the offset, 4 (18 E + 16) bytes, is a multiple of 8
  uint64_t* masks = reinterpret_cast<uint64_t*>(smem + kWaves * E + 2 * E + kWaves);
  // split form: [E] bucket start and pairs in the second set
  int32_t* off2 = reinterpret_cast<int32_t*>(masks + kWaves * E);
  int32_t* cnt2 = off2 + E;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool split = tau >= 0;

  for (int i = tid; i < kWaves * E; i += kThreads) {
    hist[i] = 0;
    masks[i] = 0;
  }
  __syncthreads();

  // contiguous chunk of this wave, a multiple of 64 pairs long
  const int64_t per = ((P + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t c0 = min(P, per * wave);
  const int64_t c1 = min(P, c0 + per);

  // 1. histogram
  for (int64_t p = c0 + lane; p < c1; p += 64) {
    const int e = ids[p] - base;
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[wave * E + e], 1);
  }
  __syncthreads();

  // 2. totals, per-wave prefixes and the bucket offsets (per set)
  int run = 0;
  bool first = true;  // the expert's buckets are in the first set
  if (tid < E) {
    for (int w = 0; w < kWaves; ++w) {
      const int c = hist[w * E + tid];
      hist[w * E + tid] = run;
      run += c;
    }
    first = !split || run > tau;
  }
  const int pad = tid < E && first ? (run + bm - 1) / bm * bm : 0;
  int total;
  const int excl = block_exclusive_scan(pad, wsum, &total);
  if (tid < E) {
    off[tid] = excl;
    cnt[tid] = first ? run : 0;
  }
  if (tid == 0) *n_padded_out = total;
  int excl2 = 0;
  if (split) {
    const int pad2 = tid < E && !first ? (run + bm2 - 1) / bm2 * bm2 : 0;
    int total2;
    excl2 = block_exclusive_scan(pad2, wsum, &total2);
    if (tid < E) {
      off2[tid] = excl2;
      cnt2[tid] = first ? 0 : run;
    }
    if (tid == 0) *n_padded2_out = total2;
  }
  __syncthreads();
  // write cursors: bucket start + the pairs of earlier waves; the set is
  // told apart by the cursor's sign bit (second set: ~cursor)
  for (int i = tid; i < kWaves * E; i += kThreads) {
    const int e = i % E;
    hist[i] = (!split || cnt2[e] == 0) ? off[e] + hist[i] : ~(off2[e] + hist[i]);
  }
  __syncthreads();

  // 3. sentinel padding and the block map (positions the scatter never writes)
  pad_buckets(off, cnt, E, bm, (int32_t)P, tid, kWaves, sorted_ids, block_expert);
  if (split) pad_buckets(off2, cnt2, E, bm2, (int32_t)P, tid, kWaves, sorted2, block_expert2);

  // 4. stable scatter, 64 pairs at a time in pair order
  uint64_t* const wmask = masks + wave * E;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t p0 = c0; p0 < c1; p0 += 64) {
    const int64_t p = p0 + lane;
    int e = -1;
    if (p < c1) {
      const int t = ids[p] - base;
      if ((unsigned)t < (unsigned)E) e = t;
    }
    const uint64_t m = lane_group(wmask, e, lane);
    const int rank = __popcll(m & lt_mask);
    const int group = __popcll(m);
    if (e >= 0) {
      const int cursor = hist[wave * E + e];
      if (cursor >= 0) sorted_ids[cursor + rank] = (int32_t)p;
      else sorted2[~cursor + rank] = (int32_t)p;
      if (rank == 0) {
        hist[wave * E + e] = cursor >= 0 ? cursor + group : cursor - group;
        clear_lane_group(wmask, e);
      }
    }
  }
}

// ---- many work-groups (large P): count, scan, scatter ----------------------
// The pairs are cut into chunks of kChunk consecutive pairs, one per wave.
// count: each wave histograms its chunk into counts[chunk][E] (plain stores).
// scan:  one work-group turns the counts into each chunk's pairs of that
//        expert in earlier chunks (in place), stores the bucket offsets after
//        them (scratch[nq * E + e]), and writes n_padded, the padding and the
//        block map.
// scatter: each wave places its chunk's pairs exactly as the single-group
//        kernel does (ranks from LDS lane masks), from its own cursors
//        (bucket offset + earlier pairs).
// The result is identical to the single-group kernel's.
constexpr int kMultiThreads = 256;
constexpr int kMultiWaves = kMultiThreads / 64;
constexpr int kChunk = 256;  // pairs per wave

__global__ __launch_bounds__(kMultiThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int64_t P, int E, int base, int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];  // [kMultiWaves][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kMultiWaves * E; i += kMultiThreads) hist[i] = 0;
  __syncthreads();
  const int64_t q = (int64_t)blockIdx.x * kMultiWaves + wave;  // chunk
  const int64_t c0 = q * kChunk;
  const int64_t c1 = c0 + kChunk < P ? c0 + kChunk : P;
  for (int64_t p = c0 + lane; p < c1; p += 64) {
    const int e = ids[p] - base;
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[wave * E + e], 1);
  }
  __syncthreads();
  const int64_t nq = (P + kChunk - 1) / kChunk;
  for (int i = tid; i < kMultiWaves * E; i += kMultiThreads) {
    const int64_t qq = (int64_t)blockIdx.x * kMultiWaves + i / E;
    if (qq < nq) counts[qq * E + i % E] = hist[i];
  }
}

__global__ __launch_bounds__(1024) void align_scan_kernel(
    int64_t P, int E, int bm, int32_t* __restrict__ counts, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ n_padded_out) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t off_s[kMaxExperts], cnt_s[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nq = (P + kChunk - 1) / kChunk;
  // per expert: exclusive prefix over the chunks (in place), total; sixteen
  // independent loads at a time
  int run = 0;
  if (tid < E) {
    for (int64_t q0 = 0; q0 < nq; q0 += 16) {
      int c[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) c[u] = q0 + u < nq ? counts[(q0 + u) * E + tid] : 0;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (q0 + u < nq) counts[(q0 + u) * E + tid] = run;
        run += c[u];
      }
    }
  }
  const int pad = tid < E ? (run + bm - 1) / bm * bm : 0;
  int incl = pad;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int s = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int u = __shfl_up(s, d);
      if (lane >= d) s += u;
    }
    if (lane < 16) wsum[lane] = s;
  }
  __syncthreads();
  const int off = incl - pad + (wave > 0 ? wsum[wave - 1] : 0);
  if (tid == 1023) *n_padded_out = off + pad;
  if (tid < E) {
    counts[nq * E + tid] = off;
    off_s[tid] = off;
    cnt_s[tid] = run;
  }
  __syncthreads();
  pad_buckets(off_s, cnt_s, E, bm, (int32_t)P, tid, 16, sorted_ids, block_expert);
}

__global__ __launch_bounds__(kMultiThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t P, int E, int base,
    const int32_t* __restrict__ cursors, int32_t* __restrict__ sorted_ids) {
  extern __shared__ int32_t cur_lds[];  // [kMultiWaves][E] cursors, then lane masks
  int32_t* cur = cur_lds;
  // [kMultiWaves][E] lane masks; the offset, 16 E bytes, is a multiple of 8
  uint64_t* masks = reinterpret_cast<uint64_t*>(cur_lds + kMultiWaves * E);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nq = (P + kChunk - 1) / kChunk;
  for (int i = tid; i < kMultiWaves * E; i += kMultiThreads) {
    const int64_t qq = (int64_t)blockIdx.x * kMultiWaves + i / E;
    cur[i] = qq < nq ? cursors[nq * E + i % E] + cursors[qq * E + i % E] : 0;
    masks[i] = 0;
  }
  __syncthreads();
  uint64_t* const wmask = masks + wave * E;
  const int64_t q = (int64_t)blockIdx.x * kMultiWaves + wave;
  const int64_t c0 = q * kChunk;
  const int64_t c1 = c0 + kChunk < P ? c0 + kChunk : P;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t p0 = c0; p0 < c1; p0 += 64) {
    const int64_t p = p0 + lane;
    int e = -1;
    if (p < c1) {
      const int t = ids[p] - base;
      if ((unsigned)t < (unsigned)E) e = t;
    }
    const uint64_t m = lane_group(wmask, e, lane);
    const int rank = __popcll(m & lt_mask);
    const int group = __popcll(m);
    if (e >= 0) {
      const int cursor = cur[wave * E + e];
      sorted_ids[cursor + rank] = (int32_t)p;
      if (rank == 0) {
        cur[wave * E + e] = cursor + group;
        clear_lane_group(wmask, e);
      }
    }
  }
}

}  // namespace

int64_t align_scratch_ints(int64_t P, int32_t E) {
  return ((P + kChunk - 1) / kChunk + 1) * E;
}

hipError_t launch_align_multi(const int32_t* topk_ids, int64_t P, int32_t E, int32_t base,
                              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* n_padded, int32_t* scratch, hipStream_t stream) {
  if (P == 0) return launch_align(topk_ids, P, E, base, block_m, sorted_ids, block_expert,
                                  n_padded, stream);
  const int64_t nq = (P + kChunk - 1) / kChunk;
  const int64_t groups = (nq + kMultiWaves - 1) / kMultiWaves;
  if (groups > 0x7fffffff) return hipErrorInvalidConfiguration;
  const size_t lds = sizeof(int32_t) * (size_t)kMultiWaves * E;
  hipLaunchKernelGGL(align_count_kernel, dim3((unsigned)groups), dim3(kMultiThreads), lds,
                     stream, topk_ids, P, E, base, scratch);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, stream, P, E, block_m, scratch,
                     sorted_ids, block_expert, n_padded);
  hipLaunchKernelGGL(align_scatter_kernel, dim3((unsigned)groups), dim3(kMultiThreads),
                     lds + sizeof(uint64_t) * (size_t)kMultiWaves * E,
                     stream, topk_ids, P, E, base, scratch, sorted_ids);
  return hipGetLastError();
}

hipError_t launch_align_split(const int32_t* topk_ids, int64_t P, int32_t E, int32_t base,
                              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* n_padded, int32_t tau, int32_t block_m2,
                              int32_t* sorted2, int32_t* block_expert2, int32_t* n_padded2,
                              hipStream_t stream) {
  if (E > kMaxExperts || P > 0x3fffffff) return hipErrorInvalidValue;
  const size_t lds = sizeof(int32_t) * (size_t)(kWaves * E + 2 * E + kWaves) +
                     sizeof(uint64_t) * kWaves * E + (tau >= 0 ? sizeof(int32_t) * 2 * E : 0);
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), lds, stream, topk_ids, P, E, base,
                     block_m, sorted_ids, block_expert, n_padded, tau, block_m2, sorted2,
                     block_expert2, n_padded2);
  return hipGetLastError();
}

hipError_t launch_align(const int32_t* topk_ids, int64_t P, int32_t E, int32_t base,
                        int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
                        int32_t* n_padded, hipStream_t stream) {
  return launch_align_split(topk_ids, P, E, base, block_m, sorted_ids, block_expert, n_padded, -1,
                            1, nullptr, nullptr, nullptr, stream);
}

}  // namespace moe
